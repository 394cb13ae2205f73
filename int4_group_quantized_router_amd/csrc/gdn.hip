// One Gated DeltaNet recurrent decode step.
//
// Three of every four layers of the hybrid stack are Gated DeltaNet linear
// attention with a fixed-size recurrent state ([xix] paragraph on Metal and
// DeltaNet; [lens] "エキスパートストリーミングの仕組み").  The pages print
// no recurrence; the step here is the published gated delta rule, per
// sequence b and value head h (key / query head g = h / (Hv / Hk)):
//
//   k^ = k / sqrt(|k|^2 + eps),  q^ = q / sqrt(|q|^2 + eps)
//   S  <- alpha (S - beta (S k^) k^T) + beta v k^T     (S: [dv][dk], f32)
//   o   = scale S q^                                   (with the new S)
//
// At decode this is pure state traffic: the state is read and written once
// (2 x dv x dk x 4 bytes per head) against ~6 dv dk flops, so the kernel is
// bound by HBM bandwidth.  A head's rows are split over SPLIT workgroups
// (ROWS each); TPR adjacent lanes share a state row, each holding CPT
// consecutive columns in registers, so every row of S is read and written
// with 16-byte accesses in one pass:
//
//   1. |k|^2, |q|^2 of this thread's columns, summed over the row's lanes
//      (every row recomputes them; the key and query rows come from cache);
//   2. (S k^)_r over the row's lanes;
//   3. S[r][c] <- alpha S[r][c] + w_r k^_c with w_r = beta (v_r - alpha (S k^)_r);
//   4. o_r = scale sum_c S[r][c] q^_c over the row's lanes.
#include "common.h"
#include "device.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace dev;

struct GdnArgs {
  const uint16_t* q;    // bf16 [B][Hk][DK]
  const uint16_t* k;    // bf16 [B][Hk][DK]
  const uint16_t* v;    // bf16 [B][Hv][DV]
  const float* alpha;   // [B][Hv]
  const float* beta;    // [B][Hv]
  float* state;         // [B][Hv][DV][DK], updated in place
  float* out;           // [B][Hv][DV]
  int Hk, Hv;
  float scale, eps;
};

template <int DK, int DV, int NT, int SPLIT>
__global__ __launch_bounds__(NT) void gdn_step_kernel(GdnArgs a) {
  constexpr int ROWS = DV / SPLIT;  // state rows per workgroup
  constexpr int TPR = NT / ROWS;    // lanes per state row
  constexpr int CPT = DK / TPR;     // columns per lane
  static_assert(ROWS * SPLIT == DV && TPR * ROWS == NT && CPT * TPR == DK && CPT % 8 == 0,
                "state tiling");
  static_assert(TPR == 2 || TPR == 4 || TPR == 8, "row lanes inside a quad or row half");
  const int bh = blockIdx.x / SPLIT;  // b * Hv + h
  const int b = bh / a.Hv, h = bh % a.Hv;
  const int g = h / (a.Hv / a.Hk);
  const int t = threadIdx.x, r = (blockIdx.x % SPLIT) * ROWS + t / TPR, c0 = (t % TPR) * CPT;

  // key and query of this lane's columns (16-byte loads of 8 bf16 each)
  const uint16_t* kp = a.k + ((size_t)b * a.Hk + g) * DK + c0;
  const uint16_t* qp = a.q + ((size_t)b * a.Hk + g) * DK + c0;
  float kc[CPT], qc[CPT];
#pragma unroll
  for (int i = 0; i < CPT / 8; ++i) {
    const uint4 kw = ld16(kp + 8 * i), qw = ld16(qp + 8 * i);
    const uint32_t ku[4] = {kw.x, kw.y, kw.z, kw.w}, qu[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kc[8 * i + 2 * j] = bf16_lo(ku[j]);
      kc[8 * i + 2 * j + 1] = bf16_hi(ku[j]);
      qc[8 * i + 2 * j] = bf16_lo(qu[j]);
      qc[8 * i + 2 * j + 1] = bf16_hi(qu[j]);
    }
  }
  // this lane's slice of state row r
  float* sp = a.state + ((size_t)bh * DV + r) * DK + c0;
  float s[CPT];
#pragma unroll
  for (int i = 0; i < CPT / 4; ++i) {
    const float4 v4 = *reinterpret_cast<const float4*>(sp + 4 * i);
    s[4 * i] = v4.x;
    s[4 * i + 1] = v4.y;
    s[4 * i + 2] = v4.z;
    s[4 * i + 3] = v4.w;
  }
  const float alpha = a.alpha[bh], beta = a.beta[bh];
  const float vr = bf16_to_f32(a.v[(size_t)bh * DV + r]);

  // 1. normalisers
  float kk = 0.f, qq = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    kk = fmaf(kc[i], kc[i], kk);
    qq = fmaf(qc[i], qc[i], qq);
  }
  kk = group_sum(kk, TPR);
  qq = group_sum(qq, TPR);
  const float rk = 1.0f / sqrtf(kk + a.eps), rq = 1.0f / sqrtf(qq + a.eps);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    kc[i] *= rk;
    qc[i] *= rq;
  }
  // 2. (S k^)_r
  float sk = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) sk = fmaf(s[i], kc[i], sk);
  sk = group_sum(sk, TPR);
  // 3. update, 4. output from the new state
  const float w = beta * (vr - alpha * sk);
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    s[i] = fmaf(alpha, s[i], w * kc[i]);
    o = fmaf(s[i], qc[i], o);
  }
  o = group_sum(o, TPR);
#pragma unroll
  for (int i = 0; i < CPT / 4; ++i)
    *reinterpret_cast<float4*>(sp + 4 * i) = make_float4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
  if (t % TPR == 0) a.out[(size_t)bh * DV + r] = a.scale * o;
}

template <int DK, int DV, int NT, int SPLIT>
hipError_t launch_gdn(const GdnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((gdn_step_kernel<DK, DV, NT, SPLIT>), dim3((unsigned)(B * a.Hv * SPLIT)),
                     dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int32_t moe_gdn_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* alpha, const float* beta, float* state, float* out,
                                int32_t B, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                                float scale, float eps, hipStream_t stream) {
  clear_error();
  MOE_REQUIRE(B >= 0 && Hk >= 1 && Hv >= 1 && Hv % Hk == 0,
              "bad heads: B=%d Hk=%d Hv=%d (Hv must be a multiple of Hk)", B, Hk, Hv);
  MOE_REQUIRE((dk == 128 && dv == 128) || (dk == 64 && dv == 64),
              "unsupported head dims dk=%d dv=%d (128x128 or 64x64)", dk, dv);
  MOE_REQUIRE(eps >= 0.f && scale == scale, "bad eps / scale");
  MOE_REQUIRE((int64_t)B * Hv * 2 < (1ll << 31), "B * Hv too large");
  if (B == 0) return MOE_OK;
  MOE_REQUIRE(q && k && v && alpha && beta && state && out, "null argument");
  MOE_REQUIRE((((uintptr_t)q | (uintptr_t)k | (uintptr_t)state) & 15) == 0,
              "q, k and state must be 16-byte aligned");
  GdnArgs a{q, k, v, alpha, beta, state, out, Hk, Hv, scale, eps};
  hipError_t e = dk == 128 ? launch_gdn<128, 128, 512, 2>(a, B, stream)
                           : launch_gdn<64, 64, 256, 1>(a, B, stream);
  MOE_HIP_TRY(e);
  return MOE_OK;
}
