// conv1d.hip -- causal depthwise conv1d with optional SiLU, and its one-token
// decode step, for gfx950 (wave64).
//
// What is computed, per channel (b, d) and step t, with W taps:
//   pre[b,d,t] = bias[d] + sum_k w[d,k] * x~[b,d,t-(W-1)+k]
//   out[b,d,t] = silu(pre) or pre
// where x~ extends x to the left with the carried window (or zeros): the
// causal depthwise conv of the SpeechLens kernel-optimization notes (causal
// depthwise convolution section, contract table: kernel size 4, three zero
// samples on the causal left edge), followed by the SiLU of the Mamba block
// ("mamba-metal: Apple Silicon で Mamba を動かす", section "カーネルから推論まで").
// The decode step slides the window by one sample ("mamba-metal", section
// "O(L) インクリメンタルデコード").
//
// The op is a stream: every input sample is read once and every output
// written once, with W FMAs and a SiLU per element in between, so it is bound
// by HBM bandwidth.  The kernels keep the taps in registers, move 16-byte
// vectors (4 fp32 or 8 bf16 elements) along the unit-stride axis, and take
// the W-1 samples before each thread's first step from a neighbouring lane or
// from a few extra loads that hit in L2:
//   * channel-fast data ([B,L,D]): a lane owns a vector of adjacent channels
//     and walks a time segment, sliding the window in registers (the walk the
//     SpeechLens notes describe, with a vector of channels per lane so one
//     wave reads 1 KB rows);
//   * time-fast data ([B,D,L]): a lane owns a vector of consecutive steps of
//     one channel and gets the 3 samples before them from the lane below;
//   * any other strides, or vectors that would be misaligned: one element per
//     thread, each tap read directly.
#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kXcdsConv = 8;  // MI355X: 8 accelerator dies

// 16-byte vectors: 4 fp32 or 8 bf16 elements, converted to fp32 on load and
// rounded to nearest even on a bf16 store.
template <typename IO>
struct vec16;
template <>
struct vec16<float> {
  static constexpr int N = 4;
  __device__ static inline void load(const float* p, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static inline void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static inline void load(const bf16_t* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline void store(bf16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = bf16x2_bits(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

__device__ inline float activate(float v, int silu_on) { return silu_on ? silu(v) : v; }

// Workgroups are dispatched round-robin over the XCDs (linear id mod 8).
// Renumber them so that each XCD gets a contiguous range of logical ids:
// neighbouring time blocks of one channel, which read each other's edge
// samples, then share that XCD's L2.
__device__ inline int64_t xcd_contiguous(int64_t lin, int64_t nwg) {
  const int64_t xcd = lin % kXcdsConv;
  const int64_t per = nwg / kXcdsConv, extra = nwg % kXcdsConv;
  return xcd * per + (xcd < extra ? xcd : extra) + lin / kXcdsConv;
}

// The carried sample x~[tau] for tau < 0 of channel row `row` (b * dim + d):
// the initial window when given, else zero.
template <typename IO, int W>
__device__ inline float window_sample(const IO* init, int64_t row, int tau) {
  if (init == nullptr || tau < -(W - 1)) return 0.0f;
  return io_traits<IO>::load(init + row * (W - 1) + (W - 1) + tau);
}

// One element per thread, any strides.
template <typename IO, int W>
__global__ __launch_bounds__(256) void conv_elem_kernel(ConvShape s, ConvPtrs p) {
  const int64_t n = static_cast<int64_t>(s.batch) * s.dim * s.seqlen;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int t = static_cast<int>(i % s.seqlen);
  const int64_t row = i / s.seqlen;
  const int d = static_cast<int>(row % s.dim);
  const int b = static_cast<int>(row / s.dim);
  const IO* x = static_cast<const IO*>(p.x) + b * s.sx[0] + d * s.sx[1];
  const IO* init = static_cast<const IO*>(p.init);
  float win[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const int tau = t - (W - 1) + k;
    win[k] = tau >= 0 ? io_traits<IO>::load(x + tau * s.sx[2]) : window_sample<IO, W>(init, row, tau);
  }
  float acc = p.bias != nullptr ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k) acc = fmaf(p.weight[d * s.sw[0] + k * s.sw[1]], win[k], acc);
  IO* out = static_cast<IO*>(p.out) + b * s.so[0] + d * s.so[1] + t * s.so[2];
  io_traits<IO>::store(out, activate(acc, s.silu));
  if (p.fin != nullptr && t == s.seqlen - 1) {
    IO* fin = static_cast<IO*>(p.fin) + row * (W - 1);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) io_traits<IO>::store(fin + j, win[j + 1]);
  }
}

// Time-fast ([B,D,L]): one wave covers kTfSpan consecutive steps of one
// channel as kTfSpan / (64 VE) blocks; in a block, lane l owns the VE steps
// starting at VE l (VE = 4 fp32 or 8 bf16 elements: 16 bytes).  All of a
// lane's loads are issued before any is used.  The 3 samples before a lane's
// first step are the last ones of the lane below; lane 0 takes them from lane
// 63 of the previous block, and in the first block from memory or the window.
constexpr int kTfSpan = 2048;

template <typename IO, int W>
__global__ __launch_bounds__(64) void conv_tfast_kernel(ConvShape s, ConvPtrs p) {
  constexpr int VE = vec16<IO>::N;
  constexpr int NB = kTfSpan / (64 * VE);
  const int64_t wblocks = (s.seqlen + kTfSpan - 1) / kTfSpan;
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t row = logical / wblocks;
  const int t_base = static_cast<int>(logical % wblocks) * kTfSpan;
  const int d = static_cast<int>(row % s.dim);
  const int b = static_cast<int>(row / s.dim);
  const int lane = threadIdx.x;
  const IO* x = static_cast<const IO*>(p.x) + b * s.sx[0] + d * s.sx[1];
  const IO* init = static_cast<const IO*>(p.init);

  float v[NB][VE];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int t = t_base + j * 64 * VE + lane * VE;
    if (t + VE <= s.seqlen) {
      vec16<IO>::load(x + t, v[j]);
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) v[j][e] = t + e < s.seqlen ? io_traits<IO>::load(x + t + e) : 0.0f;
    }
  }
  float before[3];  // the 3 samples before t_base
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    const int tau = t_base - 3 + e;
    before[e] = lane != 0 ? 0.0f
              : tau >= 0 ? io_traits<IO>::load(x + tau) : window_sample<IO, W>(init, row, tau);
  }
  float wk[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wk[k] = p.weight[d * s.sw[0] + k * s.sw[1]];
  const float bias = p.bias != nullptr ? p.bias[d] : 0.0f;
  IO* out = static_cast<IO*>(p.out) + b * s.so[0] + d * s.so[1];

#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int t = t_base + j * 64 * VE + lane * VE;
    // ext[i] = x~[t - 3 + i]; every lane takes part in the shuffles.
    float ext[3 + VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) ext[3 + e] = v[j][e];
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      const float below = __shfl_up(v[j][VE - 3 + e], 1, 64);
      const float prev = j > 0 ? __shfl(v[j > 0 ? j - 1 : 0][VE - 3 + e], 63, 64) : before[e];
      ext[e] = lane == 0 ? prev : below;
    }
    if (t < s.seqlen) {
      float y[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) {
        float acc = bias;
#pragma unroll
        for (int k = 0; k < W; ++k) acc = fmaf(wk[k], ext[i + 4 - W + k], acc);
        y[i] = activate(acc, s.silu);
      }
      if (t + VE <= s.seqlen) {
        vec16<IO>::store(out + t, y);
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e)
          if (t + e < s.seqlen) io_traits<IO>::store(out + t + e, y[e]);
      }
      // The lane holding step L-1 exports the window x~[L-(W-1) .. L-1].
      if (p.fin != nullptr && s.seqlen - 1 - t < VE) {
        IO* fin = static_cast<IO*>(p.fin) + row * (W - 1);
        const int last = s.seqlen - 1 - t + 3;  // ext index of step L-1
#pragma unroll
        for (int e = 0; e < W - 1; ++e) io_traits<IO>::store(fin + e, ext[last - (W - 2) + e]);
      }
    }
  }
}

// Channel-fast ([B,L,D]): a lane owns VE adjacent channels (16 bytes: 4 fp32
// or 8 bf16) and walks a time segment of s.seg_len steps with the window in
// registers.  A wave is 64 / s.cf_lanes lane groups of s.cf_lanes lanes; each
// group covers s.cf_lanes * VE channels of its own segment, so that rows
// narrower than 64 vectors still keep every lane busy.  Loads are issued
// kCfUnroll steps ahead of use.
constexpr int kCfUnroll = 8;

template <typename IO, int W>
__global__ __launch_bounds__(64) void conv_cfast_kernel(ConvShape s, ConvPtrs p) {
  constexpr int VE = vec16<IO>::N;
  const int lanes = s.cf_lanes;
  const int per_wave = 64 / lanes;  // segments per wave
  const int chans = lanes * VE;     // channels per lane group
  const int groups = (s.dim + chans - 1) / chans;
  const int wsegs = (s.nseg + per_wave - 1) / per_wave;
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int seg = static_cast<int>(logical % wsegs) * per_wave + threadIdx.x / lanes;
  const int64_t rest = logical / wsegs;
  const int cg = static_cast<int>(rest % groups);
  const int b = static_cast<int>(rest / groups);
  const int c = cg * chans + (threadIdx.x % lanes) * VE;
  if (c >= s.dim || seg >= s.nseg) return;
  const int t0 = seg * s.seg_len;
  const int t1 = min(s.seqlen, t0 + s.seg_len);
  const IO* x = static_cast<const IO*>(p.x) + b * s.sx[0] + c;
  const IO* init = static_cast<const IO*>(p.init);
  const int64_t row0 = static_cast<int64_t>(b) * s.dim + c;

  float wk[W][VE], bias[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k][i] = p.weight[(c + i) * s.sw[0] + k * s.sw[1]];
    bias[i] = p.bias != nullptr ? p.bias[c + i] : 0.0f;
  }
  // win[j] = x~[t - (W-1) + j] for the next step t to compute.
  float win[W > 1 ? W - 1 : 1][VE];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int tau = t0 - (W - 1) + j;
    if (tau >= 0) {
      vec16<IO>::load(x + tau * s.sx[2], win[j]);
    } else {
#pragma unroll
      for (int i = 0; i < VE; ++i) win[j][i] = window_sample<IO, W>(init, row0 + i, tau);
    }
  }
  IO* out = static_cast<IO*>(p.out) + b * s.so[0] + c;
  auto step = [&](const float* xv, int t) __attribute__((always_inline)) {
    float y[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      float acc = bias[i];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) acc = fmaf(wk[k][i], win[k][i], acc);
      acc = fmaf(wk[W - 1][i], xv[i], acc);
      y[i] = activate(acc, s.silu);
    }
    vec16<IO>::store(out + t * s.so[2], y);
#pragma unroll
    for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
      for (int i = 0; i < VE; ++i) win[k][i] = win[k + 1][i];
    if constexpr (W > 1) {
#pragma unroll
      for (int i = 0; i < VE; ++i) win[W - 2][i] = xv[i];
    }
  };
  int t = t0;
  for (; t + kCfUnroll <= t1; t += kCfUnroll) {
    float xv[kCfUnroll][VE];
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) vec16<IO>::load(x + (t + u) * s.sx[2], xv[u]);
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) step(xv[u], t + u);
  }
  for (; t < t1; ++t) {
    float xv[VE];
    vec16<IO>::load(x + t * s.sx[2], xv);
    step(xv, t);
  }
  if (p.fin != nullptr && t1 == s.seqlen) {
    IO* fin = static_cast<IO*>(p.fin) + row0 * (W - 1);
#pragma unroll
    for (int i = 0; i < VE; ++i)
#pragma unroll
      for (int j = 0; j < W - 1; ++j) io_traits<IO>::store(fin + i * (W - 1) + j, win[j][i]);
  }
}

// Decode: one thread per channel; the window is read, filtered with the new
// sample and written back shifted by one.
template <typename IO, int W>
__global__ __launch_bounds__(256) void conv_step_kernel(ConvStepShape s, ConvStepPtrs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(s.batch) * s.dim) return;
  const int b = static_cast<int>(i / s.dim);
  const int d = static_cast<int>(i % s.dim);
  IO* st = static_cast<IO*>(p.state) + i * (W - 1);
  float win[W];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) win[k] = io_traits<IO>::load(st + k);
  win[W - 1] = io_traits<IO>::load(static_cast<const IO*>(p.x) + b * s.sx[0] + d * s.sx[1]);
  float acc = p.bias != nullptr ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k) acc = fmaf(p.weight[d * s.sw[0] + k * s.sw[1]], win[k], acc);
  io_traits<IO>::store(static_cast<IO*>(p.out) + b * s.so[0] + d * s.so[1], activate(acc, s.silu));
#pragma unroll
  for (int k = 0; k < W - 1; ++k) io_traits<IO>::store(st + k, win[k + 1]);
}

template <typename IO, int W>
hipError_t launch_conv_w(const ConvShape& s, const ConvPtrs& p, hipStream_t stream) {
  if (s.path == kConvChanFast) {
    const int64_t per_wave = 64 / s.cf_lanes;
    const int64_t groups = (s.dim + s.cf_lanes * vec16<IO>::N - 1) / (s.cf_lanes * vec16<IO>::N);
    const int64_t nwg = s.batch * groups * ((s.nseg + per_wave - 1) / per_wave);
    conv_cfast_kernel<IO, W><<<dim3(static_cast<unsigned>(nwg)), dim3(64), 0, stream>>>(s, p);
  } else if (s.path == kConvTimeFast) {
    const int64_t nwg = static_cast<int64_t>(s.batch) * s.dim * ((s.seqlen + kTfSpan - 1) / kTfSpan);
    conv_tfast_kernel<IO, W><<<dim3(static_cast<unsigned>(nwg)), dim3(64), 0, stream>>>(s, p);
  } else {
    const int64_t n = static_cast<int64_t>(s.batch) * s.dim * s.seqlen;
    conv_elem_kernel<IO, W><<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(s, p);
  }
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_conv_t(const ConvShape& s, const ConvPtrs& p, hipStream_t stream) {
  switch (s.width) {
    case 1: return launch_conv_w<IO, 1>(s, p, stream);
    case 2: return launch_conv_w<IO, 2>(s, p, stream);
    case 3: return launch_conv_w<IO, 3>(s, p, stream);
    default: return launch_conv_w<IO, 4>(s, p, stream);
  }
}

template <typename IO>
hipError_t launch_conv_step_t(const ConvStepShape& s, const ConvStepPtrs& p, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(s.batch) * s.dim;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  switch (s.width) {
    case 1: conv_step_kernel<IO, 1><<<grid, block, 0, stream>>>(s, p); break;
    case 2: conv_step_kernel<IO, 2><<<grid, block, 0, stream>>>(s, p); break;
    case 3: conv_step_kernel<IO, 3><<<grid, block, 0, stream>>>(s, p); break;
    default: conv_step_kernel<IO, 4><<<grid, block, 0, stream>>>(s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvShape& s, const ConvPtrs& p, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_conv_t<bf16_t>(s, p, stream) : launch_conv_t<float>(s, p, stream);
}

hipError_t launch_conv_step(const ConvStepShape& s, const ConvStepPtrs& p, bool io_bf16,
                            hipStream_t stream) {
  return io_bf16 ? launch_conv_step_t<bf16_t>(s, p, stream)
                 : launch_conv_step_t<float>(s, p, stream);
}

}  // namespace mss
