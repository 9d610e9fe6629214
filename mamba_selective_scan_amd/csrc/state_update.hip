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
// One lane per (channel, state): a 16-lane row of a wave holds one channel's
// 16 states, so the state, A_log, B and C loads are contiguous across the
// row, and y = sum_n C[n] h[n] is a 4-step DPP rotation sum inside the row.
// Lanes past dstate carry zeros.  Every row computes its channel's delta (the
// same value in all 16 lanes); lane 0 of the row adds the skip term, applies
// the gate and stores.  The step moves a few megabytes at most and is bound
// by launch latency at decode shapes.
#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {

constexpr int kStepThreads = 256;                   // 16 channels per workgroup
constexpr int kStepChannels = kStepThreads / kMaxState;

template <typename IO>
__global__ __launch_bounds__(kStepThreads) void state_update_kernel(
    StepShape s, float* __restrict__ state, const IO* __restrict__ u,
    const IO* __restrict__ delta_raw, const float* __restrict__ A_log,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ dt_bias, IO* __restrict__ out) {
  const int n = threadIdx.x % kMaxState;
  const int64_t nch = static_cast<int64_t>(s.batch) * s.dim;
  const int64_t ch_lane = static_cast<int64_t>(blockIdx.x) * kStepChannels + threadIdx.x / kMaxState;
  const bool cvalid = ch_lane < nch;
  const bool active = cvalid && n < s.dstate;
  // Indices clamped into range so that every load below is in bounds and all
  // of them leave before any arithmetic: one memory round trip, not three
  // (the inputs, then A_log, B, C and the state, then z).
  const int64_t ch = cvalid ? ch_lane : 0;
  const int b = static_cast<int>(ch / s.dim);
  const int d = static_cast<int>(ch % s.dim);
  const int nn = n < s.dstate ? n : 0;
  const float xr = io_traits<IO>::load(delta_raw + b * s.sd[0] + d * s.sd[1]);
  const float uv = io_traits<IO>::load(u + b * s.su[0] + d * s.su[1]);
  const float alog = A_log[d * s.sA[0] + nn * s.sA[1]];
  const float bn = io_traits<IO>::load(Bm + b * s.sB[0] + nn * s.sB[1]);
  const float cn = io_traits<IO>::load(Cm + b * s.sC[0] + nn * s.sC[1]);
  float* hp = state + ch * s.dstate + nn;
  const float h_old = *hp;
  const float bias = dt_bias != nullptr ? dt_bias[d] : 0.0f;
  const float skip = Dskip != nullptr ? Dskip[d] : 0.0f;
  const float zv = z != nullptr ? io_traits<IO>::load(z + b * s.sz[0] + d * s.sz[1]) : 0.0f;

  const float x = xr + bias;
  const float dl = s.softplus ? softplus(x) : x;
  const float a2 = -expf(alog) * kLog2e;
  const float hn = fmaf(fast_exp2(dl * a2), h_old, dl * uv * bn);
  if (active) *hp = hn;
  float y = active ? cn * hn : 0.0f;
  y = row_sum16(y);  // every lane of the row takes part
  if (cvalid && n == 0) {
    y = fmaf(skip, uv, y);
    if (z != nullptr) y *= silu(zv);
    io_traits<IO>::store(out + b * s.so[0] + d * s.so[1], y);
  }
}

template <typename IO>
static hipError_t launch_step_t(const StepShape& s, const StepPtrs& p, hipStream_t stream) {
  const int64_t nch = static_cast<int64_t>(s.batch) * s.dim;
  const unsigned blocks = static_cast<unsigned>((nch + kStepChannels - 1) / kStepChannels);
  state_update_kernel<IO><<<dim3(blocks), dim3(kStepThreads), 0, stream>>>(
      s, p.state, static_cast<const IO*>(p.u), static_cast<const IO*>(p.delta_raw), p.A_log,
      static_cast<const IO*>(p.B), static_cast<const IO*>(p.C), p.D, static_cast<const IO*>(p.z),
      p.dt_bias, static_cast<IO*>(p.out));
  return hipGetLastError();
}

hipError_t launch_step(const StepShape& s, const StepPtrs& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_step_t<bf16_t>(s, p, stream) : launch_step_t<float>(s, p, stream);
}

}  // namespace mss
