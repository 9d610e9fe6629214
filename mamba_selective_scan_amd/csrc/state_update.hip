// state_update.hip -- one-token selective state update (decode step), gfx950.
//
// For every channel (b, d), with the state held by the caller:
//   delta  = softplus(delta_raw + dt_bias)
//   h[n]   = exp(delta * A[n]) * h[n] + delta * u * B[b, n]     (in place)
//   out    = (sum_n h[n] * C[b, n] + D[d] * u) * silu(z)
// ("mamba-metal: Apple Silicon で Mamba を動かす", section
// "O(L) インクリメンタルデコード": an elementwise step on the carried state,
// closed by the z gate).
//
// One lane per channel, one wave per 64 channels of one batch row, so B and C
// are wave-uniform scalar loads; the dstate entries are walked in registers.
// The step moves a few hundred kilobytes at decode shapes and is bound by
// launch latency, not bandwidth.
#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {

template <typename IO>
__global__ __launch_bounds__(64) void state_update_kernel(
    StepShape s, float* __restrict__ state, const IO* __restrict__ u,
    const IO* __restrict__ delta_raw, const float* __restrict__ A_log,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ dt_bias, IO* __restrict__ out) {
  const int groups = (s.dim + 63) / 64;
  const int b = blockIdx.x / groups;
  const int d = (blockIdx.x - b * groups) * 64 + static_cast<int>(threadIdx.x);
  if (d >= s.dim) return;
  const float x = io_traits<IO>::load(delta_raw + b * s.sd[0] + d * s.sd[1]) +
                  (dt_bias != nullptr ? dt_bias[d] : 0.0f);
  const float dl = s.softplus ? softplus(x) : x;
  const float uv = io_traits<IO>::load(u + b * s.su[0] + d * s.su[1]);
  const float du = dl * uv;
  float* hp = state + (static_cast<int64_t>(b) * s.dim + d) * s.dstate;
  float y = 0.0f;
  for (int n = 0; n < s.dstate; ++n) {
    const float a2 = -expf(A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e;
    const float bn = load_uniform(Bm + b * s.sB[0] + n * s.sB[1]);
    const float cn = load_uniform(Cm + b * s.sC[0] + n * s.sC[1]);
    const float hn = fmaf(fast_exp2(dl * a2), hp[n], du * bn);
    hp[n] = hn;
    y = fmaf(cn, hn, y);
  }
  y = fmaf(Dskip != nullptr ? Dskip[d] : 0.0f, uv, y);
  if (z != nullptr) y *= silu(io_traits<IO>::load(z + b * s.sz[0] + d * s.sz[1]));
  io_traits<IO>::store(out + b * s.so[0] + d * s.so[1], y);
}

template <typename IO>
static hipError_t launch_step_t(const StepShape& s, const StepPtrs& p, hipStream_t stream) {
  const unsigned groups = static_cast<unsigned>((s.dim + 63) / 64);
  state_update_kernel<IO><<<dim3(groups * static_cast<unsigned>(s.batch)), dim3(64), 0, stream>>>(
      s, p.state, static_cast<const IO*>(p.u), static_cast<const IO*>(p.delta_raw), p.A_log,
      static_cast<const IO*>(p.B), static_cast<const IO*>(p.C), p.D, static_cast<const IO*>(p.z),
      p.dt_bias, static_cast<IO*>(p.out));
  return hipGetLastError();
}

hipError_t launch_step(const StepShape& s, const StepPtrs& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_step_t<bf16_t>(s, p, stream) : launch_step_t<float>(s, p, stream);
}

}  // namespace mss
