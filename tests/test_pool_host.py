"""The slot pool's own code (csrc/pool.cpp) on the CPU: built with g++ against
a host stand-in of the HIP runtime (tests/host_pool: "device" memory is host
memory, a copy is a memcpy), driven by scripted acquire / release / evict /
flush sequences and compared with the oracle's replay of the pool policy.

Three builds: plain, AddressSanitizer + UndefinedBehaviorSanitizer (host
code only; any report fails the test), and the debug build that overwrites
evicted slots with 0xFF bytes."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.pool_replay import PoolExhausted, PoolReplay, SlotBusy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "host_pool", "pool_driver.cpp"),
       os.path.join(ROOT, "int4_group_quantized_router_amd", "csrc", "pool.cpp"),
       os.path.join(ROOT, "int4_group_quantized_router_amd", "csrc", "layout.cpp"),
       os.path.join(ROOT, "tests", "host_pool", "fake_hip.cpp")]
FLAGS = {
    "plain": ["-O1"],
    "asan": ["-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
             "-fno-sanitize-recover=undefined"],
    "poison": ["-O1", "-DMOE_POOL_POISON"],
}
E_EXHAUSTED, E_BUSY = -5, -6


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("pool_host")
    exe = {}
    for name, flags in FLAGS.items():
        path = str(out / f"pool_driver_{name}")
        cmd = [gxx, "-std=c++17", "-g", "-Wall", *flags,
               "-I" + os.path.join(ROOT, "tests", "host_pool"), "-I" + os.path.join(ROOT, "include"),
               *SRC, "-o", path, "-lpthread"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        exe[name] = path
    return exe


def run(exe, script):
    r = subprocess.run([exe], input="\n".join(script) + "\n", capture_output=True, text=True,
                       timeout=120)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    return r.stdout.splitlines()


def random_trace(seed, L, E, cap, n_ops, k_max):
    """A script and the oracle's expected output for it."""
    rng = np.random.default_rng(seed)
    stride = 8192
    rep = PoolReplay(cap, stride)
    script, want = [], []
    held = []  # acquired, not yet released: (layer, experts)
    for _ in range(n_ops):
        r = rng.random()
        if (r < 0.55 and len(held) < 4) or not held:
            layer = int(rng.integers(0, L))
            # skewed choice, like Zipf-biased routing
            p = 1.0 / np.arange(1, E + 1) ** 1.1
            k = int(rng.integers(1, k_max + 1))
            ex = rng.choice(E, size=min(k, E), replace=False, p=p / p.sum()).tolist()
            script.append("A %d %s" % (layer, " ".join(map(str, ex))))
            try:
                out = rep.acquire(layer, ex)
                want.append("A ok " + " ".join(f"{s} {int(m)}" for s, m in out))
                held.append((layer, ex))
            except PoolExhausted:
                want.append(f"A err {E_EXHAUSTED}")
        elif r < 0.62:
            # prefetch a few experts, some of them maybe resident
            layer = int(rng.integers(0, L))
            ex = rng.choice(E, size=int(rng.integers(1, min(E, 6) + 1)), replace=False).tolist()
            script.append("H %d %s" % (layer, " ".join(map(str, ex))))
            want.append(f"H ok {rep.prefetch(layer, ex)}")
        elif r < 0.85:
            layer, ex = held.pop(int(rng.integers(0, len(held))))
            script.append("R %d %s" % (layer, " ".join(map(str, ex))))
            rep.release(layer, ex)
            want.append("R ok")
        elif r < 0.95:
            layer, e = int(rng.integers(0, L)), int(rng.integers(0, E))
            script.append(f"E {layer} {e}")
            try:
                rep.evict(layer, e)
                want.append("E ok")
            except SlotBusy:
                want.append(f"E err {E_BUSY}")
        else:
            if rng.random() < 0.7:  # release everything first: the flush succeeds
                for layer, ex in held:
                    script.append("R %d %s" % (layer, " ".join(map(str, ex))))
                    rep.release(layer, ex)
                    want.append("R ok")
                held = []
            script.append("F")
            try:
                rep.flush()
                want.append("F ok")
            except SlotBusy:
                want.append(f"F err {E_BUSY}")
        if rng.random() < 0.1:
            st = rep.stats()
            script.append("S")
            want.append(f"S {st['hits']} {st['misses']} {st['evictions']} {st['prefetched']} "
                        f"{st['bytes_h2d']} {st['misses'] + st['prefetched']}")  # one copy per load
        if rng.random() < 0.1 and rep.slot_of:
            keys = sorted(rep.slot_of)
            l, e = keys[int(rng.integers(0, len(keys)))]
            script += [f"X {l} {e}", f"C {l} {e}"]
            want += [f"X {rep.slot_of[(l, e)]}", "C 1"]
    # every key's slot at the end
    for l in range(L):
        for e in range(E):
            script.append(f"X {l} {e}")
            want.append(f"X {rep.slot_of.get((l, e), -1)}")
    st = rep.stats()
    script.append("S")
    want.append(f"S {st['hits']} {st['misses']} {st['evictions']} {st['prefetched']} "
                f"{st['bytes_h2d']} {st['misses'] + st['prefetched']}")
    return stride, script, want


@pytest.mark.parametrize("build", ["plain", "asan"])
@pytest.mark.parametrize("seed,L,E,cap,k_max", [(0, 2, 8, 3, 3), (1, 3, 16, 12, 5),
                                                (2, 4, 32, 40, 10), (3, 1, 6, 6, 6)])
def test_pool_code_matches_oracle_replay(drivers, build, seed, L, E, cap, k_max):
    """Hits, misses, slots, evictions, exhaustion (every slot pinned), busy
    evict and flush, prefetches (free slots only, count 0, no tick),
    counters, one copy per load, slot bytes equal the store's after each
    fill: the pool's C++ code and the replay agree on every operation of a
    random 400-operation script."""
    stride, script, want = random_trace(seed, L, E, cap, 400, k_max)
    got = run(drivers[build], [f"init {L} {E} {stride} {cap}"] + script)
    assert got[0] == "init ok"
    assert len(got) - 1 == len(want)
    for i, (g, w) in enumerate(zip(got[1:], want)):
        assert g == w, (i, script[i], g, w)


def test_file_store_pool_code_matches_oracle_replay(drivers, tmp_path):
    """The same over a container file: every miss one pread (through the
    pinned staging buffers) and one copy; slot bytes equal the file's."""
    stride, script, want = random_trace(7, 3, 12, 10, 300, 6)
    path = str(tmp_path / "experts.qpack")
    got = run(drivers["asan"], [f"file {path} 3 12 {stride} 10"] + script)
    assert got[0] == "file ok"
    for i, (g, w) in enumerate(zip(got[1:], want)):
        assert g == w, (i, script[i], g, w)


def test_evicted_slots_are_poisoned_in_debug_builds(drivers):
    """Debug build: a slot dropped by eviction, explicit evict or flush holds
    only 0xFF bytes (NaN as f32 and bf16) until its next fill; a fill
    replaces them with the blob."""
    s = ["init 1 6 8192 2",
         "A 0 1", "R 0 1", "A 0 2", "R 0 2",   # slots 0, 1
         "A 0 1", "R 0 1",                     # (0,1) used twice
         "A 0 3", "R 0 3",                     # evicts (0,2) from slot 1, refills it
         "P 1", "C 0 3",
         "E 0 3", "P 1", "X 0 3",              # explicit evict: slot 1 poisoned
         "F", "P 0", "P 1",                    # flush: both poisoned
         "A 0 4", "C 0 4", "P 0"]              # refill slot 0
    got = run(drivers["poison"], s)
    assert got == ["init ok", "A ok 0 1", "R ok", "A ok 1 1", "R ok", "A ok 0 0", "R ok",
                   "A ok 1 1", "R ok", "P 0", "C 1", "E ok", "P 1", "X -1", "F ok", "P 1", "P 1",
                   "A ok 0 1", "C 1", "P 0"]
