"""The allocation-free expert entry point against the ordinary one, through
the C ABI: bit-identical accumulated outputs on two calls in a row (the
second with a smaller input, so the fixed activation buffer holds the first
call's values), and shape errors reported before any launch."""

import numpy as np
import pytest

from moe_inputs import CONFIGS, expert_arrays, tokens_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _case(torch, name, H, I, T, seed):
    from int4_group_quantized_router_amd.weights import upload_blob
    cfg = CONFIGS[name].replace(hidden=H, inter=I)
    arr = expert_arrays(cfg, 0, seed)
    blob = upload_blob(H, I, cfg.bits, arr)
    x = torch.from_numpy(tokens_x(cfg, seed, T).view(np.int16)).cuda()
    rng = np.random.default_rng(seed)
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    coef = torch.from_numpy(rng.uniform(0.1, 1.0, T).astype(np.float32)).cuda()
    return cfg, blob, x, y0, coef


@pytest.mark.parametrize("first,second", [
    (("decode35b", 2048, 512, 8), ("tiny", 256, 64, 3)),
    (("decode35b", 2048, 512, 8), ("decode35b", 2048, 512, 1)),
    (("decode80b_int8", 2048, 512, 2), ("decode80b_int8", 2048, 512, 1)),
    (("decode80b_int8", 512, 256, 5), ("tiny", 256, 64, 3)),
])
def test_noalloc_matches_expert_forward(torch, first, second):
    import int4_group_quantized_router_amd as m
    for i, (name, H, I, T) in enumerate((first, second)):
        print("noalloc", name, H, I, T, flush=True)
        cfg, blob, x, y0, coef = _case(torch, name, H, I, T, 5 + i)
        y_ref = torch.from_numpy(y0.copy()).cuda()
        y_new = torch.from_numpy(y0.copy()).cuda()
        m.moe_expert_forward(x, H, I, cfg.bits, blob, coef, y_ref)
        m.moe_expert_forward_noalloc(x, H, I, cfg.bits, blob, coef, y_new)
        torch.cuda.synchronize()
        a, b = y_ref.cpu().numpy(), y_new.cpu().numpy()
        assert np.all(np.isfinite(b))
        assert not np.array_equal(b, y0)  # the expert added something
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, H, I, T)


def test_noalloc_rejects_unsupported_shapes(torch):
    import int4_group_quantized_router_amd as m
    from int4_group_quantized_router_amd import _lib
    cfg, blob, x, y0, coef = _case(torch, "tiny", 256, 64, 2, 1)
    y = torch.from_numpy(y0.copy()).cuda()
    with pytest.raises(m.MoEError) as ei:  # intermediate beyond the supported 2048
        m.moe_expert_forward_noalloc(x, 256, 4096, 4, blob, coef, y)
    assert ei.value.status == _lib.MOE_E_INVAL
    x9 = torch.zeros((9, 256), dtype=torch.int16, device="cuda")
    with pytest.raises(m.MoEError) as ei:  # more tokens than the per-token path takes
        m.moe_expert_forward_noalloc(x9, 256, 64, 4, blob, coef, torch.zeros((9, 256), device="cuda"))
    assert ei.value.status == _lib.MOE_E_INVAL
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y0)  # nothing was launched
