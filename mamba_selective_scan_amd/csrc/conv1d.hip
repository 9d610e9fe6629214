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
// by HBM bandwidth.  The kernels keep the taps in registers, move 4-element
// vectors along the unit-stride axis, and take the W-1 samples before each
// thread's first step from a neighbouring lane or from a few extra loads that
// hit in L2:
//   * channel-fast data ([B,L,D]): a lane owns 4 adjacent channels and walks a
//     time segment, sliding the window in registers (the walk the SpeechLens
//     notes describe, with 4 channels per lane so one wave reads 1 KB rows);
//   * time-fast data ([B,D,L]): a lane owns 4 consecutive steps of one
//     channel and gets the 3 samples before them from the lane below;
//   * any other strides, or vectors that would be misaligned: one element per
//     thread, each tap read directly.
#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kXcdsConv = 8;  // MI355X: 8 accelerator dies

template <typename IO>
struct vec4_io;
template <>
struct vec4_io<float> {
  __device__ static inline void load(const float* p, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static inline void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <>
struct vec4_io<bf16_t> {
  __device__ static inline void load(const bf16_t* p, float* v) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  __device__ static inline void store(bf16_t* p, const float* v) {
    uint2 q;
    q.x = static_cast<uint32_t>(bf16_bits(v[0])) | (static_cast<uint32_t>(bf16_bits(v[1])) << 16);
    q.y = static_cast<uint32_t>(bf16_bits(v[2])) | (static_cast<uint32_t>(bf16_bits(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = q;
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

// Time-fast ([B,D,L]): thread = 4 consecutive steps of one channel, one
// workgroup = 1024 steps.  The W-1 samples before a lane's first step are the
// last ones of the lane below; lane 0 of each wave loads its own.
constexpr int kTfThreads = 256;
constexpr int kTfSteps = kTfThreads * kConvVec;

template <typename IO, int W>
__global__ __launch_bounds__(kTfThreads) void conv_tfast_kernel(ConvShape s, ConvPtrs p) {
  const int64_t tblocks = (s.seqlen + kTfSteps - 1) / kTfSteps;
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t row = logical / tblocks;
  const int t = static_cast<int>(logical % tblocks) * kTfSteps + threadIdx.x * kConvVec;
  const int d = static_cast<int>(row % s.dim);
  const int b = static_cast<int>(row / s.dim);
  const int lane = threadIdx.x & 63;
  const IO* x = static_cast<const IO*>(p.x) + b * s.sx[0] + d * s.sx[1];
  const IO* init = static_cast<const IO*>(p.init);

  // ext[j] = x~[t - 3 + j], j = 0..6: three earlier samples, then this lane's four.
  float ext[3 + kConvVec];
  float* v = ext + 3;
  const bool full = t + kConvVec <= s.seqlen;
  if (full) {
    vec4_io<IO>::load(x + t, v);
  } else {
#pragma unroll
    for (int j = 0; j < kConvVec; ++j) v[j] = t + j < s.seqlen ? io_traits<IO>::load(x + t + j) : 0.0f;
  }
  // Every lane takes part in the shuffles (lanes past the end included).
#pragma unroll
  for (int j = 0; j < 3; ++j) ext[j] = __shfl_up(v[j + 1], 1, 64);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int tau = t - 3 + j;
      ext[j] = tau >= 0 ? io_traits<IO>::load(x + tau) : window_sample<IO, W>(init, row, tau);
    }
  }
  if (t >= s.seqlen) return;

  float wk[W];
#pragma unroll
  for (int k = 0; k < W; ++k) wk[k] = p.weight[d * s.sw[0] + k * s.sw[1]];
  const float bias = p.bias != nullptr ? p.bias[d] : 0.0f;
  float y[kConvVec];
#pragma unroll
  for (int i = 0; i < kConvVec; ++i) {
    float acc = bias;
#pragma unroll
    for (int k = 0; k < W; ++k) acc = fmaf(wk[k], ext[i + 4 - W + k], acc);
    y[i] = activate(acc, s.silu);
  }
  IO* out = static_cast<IO*>(p.out) + b * s.so[0] + d * s.so[1];
  if (full) {
    vec4_io<IO>::store(out + t, y);
  } else {
#pragma unroll
    for (int j = 0; j < kConvVec; ++j)
      if (t + j < s.seqlen) io_traits<IO>::store(out + t + j, y[j]);
  }
  // The lane holding step L-1 exports the window x~[L-(W-1) .. L-1].
  if (p.fin != nullptr && s.seqlen - 1 - t < kConvVec) {
    IO* fin = static_cast<IO*>(p.fin) + row * (W - 1);
    const int last = s.seqlen - 1 - t + 3;  // ext index of step L-1
#pragma unroll
    for (int j = 0; j < W - 1; ++j) io_traits<IO>::store(fin + j, ext[last - (W - 2) + j]);
  }
}

// Channel-fast ([B,L,D]): thread = 4 adjacent channels, one wave = 256
// channels, walking a time segment of s.seg_len steps with the window in
// registers.  Loads are issued kCfUnroll steps ahead of use.
constexpr int kCfThreads = 64;
constexpr int kCfChannels = kCfThreads * kConvVec;
constexpr int kCfUnroll = 8;

template <typename IO, int W>
__global__ __launch_bounds__(kCfThreads) void conv_cfast_kernel(ConvShape s, ConvPtrs p) {
  const int groups = (s.dim + kCfChannels - 1) / kCfChannels;
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int seg = static_cast<int>(logical % s.nseg);
  const int64_t rest = logical / s.nseg;
  const int cg = static_cast<int>(rest % groups);
  const int b = static_cast<int>(rest / groups);
  const int c = cg * kCfChannels + threadIdx.x * kConvVec;
  if (c >= s.dim) return;
  const int t0 = seg * s.seg_len;
  const int t1 = min(s.seqlen, t0 + s.seg_len);
  const IO* x = static_cast<const IO*>(p.x) + b * s.sx[0] + c;
  const IO* init = static_cast<const IO*>(p.init);
  const int64_t row0 = static_cast<int64_t>(b) * s.dim + c;

  float wk[W][kConvVec], bias[kConvVec];
#pragma unroll
  for (int i = 0; i < kConvVec; ++i) {
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k][i] = p.weight[(c + i) * s.sw[0] + k * s.sw[1]];
    bias[i] = p.bias != nullptr ? p.bias[c + i] : 0.0f;
  }
  // win[j] = x~[t - (W-1) + j] for the next step t to compute.
  float win[W > 1 ? W - 1 : 1][kConvVec];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int tau = t0 - (W - 1) + j;
    if (tau >= 0) {
      vec4_io<IO>::load(x + tau * s.sx[2], win[j]);
    } else {
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) win[j][i] = window_sample<IO, W>(init, row0 + i, tau);
    }
  }
  IO* out = static_cast<IO*>(p.out) + b * s.so[0] + c;
  auto step = [&](const float* xv, int t) __attribute__((always_inline)) {
    float y[kConvVec];
#pragma unroll
    for (int i = 0; i < kConvVec; ++i) {
      float acc = bias[i];
#pragma unroll
      for (int k = 0; k < W - 1; ++k) acc = fmaf(wk[k][i], win[k][i], acc);
      acc = fmaf(wk[W - 1][i], xv[i], acc);
      y[i] = activate(acc, s.silu);
    }
    vec4_io<IO>::store(out + t * s.so[2], y);
#pragma unroll
    for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) win[k][i] = win[k + 1][i];
    if constexpr (W > 1) {
#pragma unroll
      for (int i = 0; i < kConvVec; ++i) win[W - 2][i] = xv[i];
    }
  };
  int t = t0;
  for (; t + kCfUnroll <= t1; t += kCfUnroll) {
    float xv[kCfUnroll][kConvVec];
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) vec4_io<IO>::load(x + (t + u) * s.sx[2], xv[u]);
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) step(xv[u], t + u);
  }
  for (; t < t1; ++t) {
    float xv[kConvVec];
    vec4_io<IO>::load(x + t * s.sx[2], xv);
    step(xv, t);
  }
  if (p.fin != nullptr && t1 == s.seqlen) {
    IO* fin = static_cast<IO*>(p.fin) + row0 * (W - 1);
#pragma unroll
    for (int i = 0; i < kConvVec; ++i)
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
    const int64_t groups = (s.dim + kCfChannels - 1) / kCfChannels;
    const int64_t nwg = s.batch * groups * s.nseg;
    conv_cfast_kernel<IO, W><<<dim3(static_cast<unsigned>(nwg)), dim3(kCfThreads), 0, stream>>>(s, p);
  } else if (s.path == kConvTimeFast) {
    const int64_t nwg = static_cast<int64_t>(s.batch) * s.dim * ((s.seqlen + kTfSteps - 1) / kTfSteps);
    conv_tfast_kernel<IO, W><<<dim3(static_cast<unsigned>(nwg)), dim3(kTfThreads), 0, stream>>>(s, p);
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
