// mss_internal.hpp -- parameter blocks and launch entry points shared by the
// host layer (mss_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mss {

// Scan tiling.  One wave owns kCh consecutive channels of one batch row and
// one time segment (the waves of a workgroup are independent).  In the scan, lane (g, c) =
// (lane / kCh, lane % kCh) runs states [g*kStatesPerLane, (g+1)*kStatesPerLane)
// of channel c, and the segment is walked in chunks of kT time steps.  Loads
// and stores move kVec-element vectors along the unit-stride axis.
constexpr int kCh = 8;
constexpr int kGroups = 8;
constexpr int kStatesPerLane = 2;
constexpr int kMaxState = kGroups * kStatesPerLane;  // 16
constexpr int kT = 32;
constexpr int kThreads = 64;                         // one wave
constexpr int kVec = 4;
constexpr int kPerThread = kCh * kT / kThreads;      // 4 tile elements per lane

// Carry kernels (time segments): aggregates loaded per batch of segments.
constexpr int kCarryBatch = 16;
// The forward's carry workgroup cuts the chain of nseg - 1 aggregates into
// ranges of at most kCarryBatch segments (when that takes at most kCarryWaves
// waves), one wave each.
constexpr int kCarryWaves = 16;
inline int carry_waves(int nseg) {
  const int w = (nseg - 1 + kCarryBatch - 1) / kCarryBatch;
  return w < 1 ? 1 : (w > kCarryWaves ? kCarryWaves : w);
}

// Links of a linear chain c_{k+1} = P_k c_k + H_k: a real link is (P, H)
// acting on a float, a complex one (Re P, Im P, Re H, Im H) acting on
// (Re c, Im c).  link_then(acc, a) is the link acc followed by a.
__device__ inline float link_apply(float2 a, float c) { return fmaf(a.x, c, a.y); }
__device__ inline float2 link_then(float2 acc, float2 a) {
  return make_float2(acc.x * a.x, fmaf(a.x, acc.y, a.y));
}
__device__ inline float2 link_identity(float2) { return make_float2(1.0f, 0.0f); }
__device__ inline float2 link_apply(float4 a, float2 c) {
  return make_float2(fmaf(a.x, c.x, fmaf(-a.y, c.y, a.z)), fmaf(a.x, c.y, fmaf(a.y, c.x, a.w)));
}
__device__ inline float4 link_then(float4 acc, float4 a) {
  const float2 P = link_apply(make_float4(a.x, a.y, 0.0f, 0.0f), make_float2(acc.x, acc.y));
  const float2 H = link_apply(a, make_float2(acc.z, acc.w));
  return make_float4(P.x, P.y, H.x, H.y);
}
__device__ inline float4 link_identity(float4) { return make_float4(1.0f, 0.0f, 0.0f, 0.0f); }

// A chain c_{k+1} = link_k(c_k) over links k = 0 .. nlink - 1 from c_0,
// walked by the waves of one workgroup in ranges (the links compose
// associatively), one lane per chain in every wave: a wave composes its range
// into one link, loading its links kCarryBatch at a time ahead of the
// arithmetic; the ranges' links meet in LDS (xch, a slot per wave and lane);
// each wave walks its range again from the value entering it.  link(k)
// returns link k for any k in [0, nlink), also in a lane whose chain is not
// valid (its loads must stay in bounds there); put(k, c) receives c_{k+1}
// and is called in valid lanes only.  nlink >= 1.  Every thread of the
// workgroup calls it (it holds a barrier), in a workgroup of
// 64 x carry_waves(nlink + 1) threads.
template <typename Pair, typename Val, typename Link, typename Put>
__device__ inline void walk_chain_in_ranges(int nlink, Val c, bool valid, Pair (*xch)[64],
                                            Link link, Put put) {
  const int lane = static_cast<int>(threadIdx.x) % 64;
  const int w = static_cast<int>(threadIdx.x) / 64;
  const int nw = static_cast<int>(blockDim.x) / 64;
  const int per = (nlink + nw - 1) / nw;
  const int s0 = min(w * per, nlink);
  const int s1 = min(s0 + per, nlink);
  const Pair one = link_identity(Pair{});
  auto load_batch = [&](Pair (&a)[kCarryBatch], int base) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kCarryBatch; ++j) {  // past the range: the identity
      const bool in = base + j < s1;
      const Pair v = link(in ? base + j : 0);
      a[j] = in ? v : one;
    }
  };
  Pair first[kCarryBatch];
  load_batch(first, s0);
  Pair acc = one;
#pragma unroll
  for (int j = 0; j < kCarryBatch; ++j) acc = link_then(acc, first[j]);
  for (int base = s0 + kCarryBatch; base < s1; base += kCarryBatch) {
    Pair a[kCarryBatch];
    load_batch(a, base);
#pragma unroll
    for (int j = 0; j < kCarryBatch; ++j) acc = link_then(acc, a[j]);
  }
  xch[w][lane] = acc;
  __syncthreads();
  for (int k = 0; k < w; ++k) c = link_apply(xch[k][lane], c);
  if (!valid) return;
#pragma unroll
  for (int j = 0; j < kCarryBatch; ++j) {
    c = link_apply(first[j], c);
    if (s0 + j < s1) put(s0 + j, c);
  }
  for (int base = s0 + kCarryBatch; base < s1; base += kCarryBatch) {
    Pair a[kCarryBatch];
    load_batch(a, base);
#pragma unroll
    for (int j = 0; j < kCarryBatch; ++j) {
      c = link_apply(a[j], c);
      if (base + j < s1) put(base + j, c);
    }
  }
}

// Sizes and element strides (logical order) of one scan call.  Pointers are
// passed as separate kernel arguments so they can carry __restrict__.
struct ScanShape {
  int batch, dim, seqlen, dstate;
  int groups;           // ceil(dim / kCh)
  int nseg, seg_len;    // time segments (seg_len is a multiple of kT)
  int agg_split;        // AGG pass: parts per segment, 1..kMaxAggSplit (the carry pass composes them)
  int part_len;         // AGG pass: steps per part, a multiple of kT
  int64_t nchan_pad;    // batch * groups * kCh: rows of the workspace arrays
  int64_t su[3], sd[3], sz[3], so[3];  // u, delta_raw, z, out: (b, d, t)
  int64_t sB[3], sC[3];                // B, C: (b, n, t)
  int64_t sA[2];                       // A_log: (d, n)
  int softplus;
  int vec_ok;           // every kVec-element vector of u/delta_raw/z/out/B/C is 4-byte aligned
  int use_vec;          // the vector pass runs (else everything is element-wise)
  int t_first, t_stop;  // this pass covers time steps [t_first, t_stop)
  int reverse;          // logical step tau is storage step seqlen-1-tau
  int bc_const;         // B and C have time stride 0 (time-invariant)
};

constexpr int kMaxAggSplit = 2;

struct StepShape {
  int batch, dim, dstate;
  int64_t su[2], sd[2], sz[2], so[2];  // (b, d)
  int64_t sB[2], sC[2];                // (b, n)
  int64_t sA[2];
  int softplus;
};

// Chunk states: the state entering every kStateChunk-step chunk of logical
// time, [ceil(L / kStateChunk)][batch][dim][kMaxState] fp32.  The forward can
// record them; the backward reads them as its checkpoints.
constexpr int kStateChunk = 16;

struct ScanPtrs {
  const void* u;
  const void* delta_raw;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  const float* h0;
  void* out;
  float* final_state;
  float* tail_h0;  // [batch][dim][dstate] state handed from the vector pass to the tail
  float2* agg;    // [nseg-1][nchan_pad][kMaxState] segment (prod a, h from 0)
  float* carry;   // [nseg][nchan_pad][kMaxState] state entering each segment
  float* chunk_states;  // optional output, see kStateChunk
};

struct StepPtrs {
  float* state;
  const void* u;
  const void* delta_raw;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* out;
};

// Causal depthwise conv1d.  Loads and stores move 16-byte vectors (4 fp32 or
// 8 bf16 elements) along the unit-stride axis when the layout allows it.
constexpr int kConvVecBytes = 16;
constexpr int kConvMaxWidth = 4;

enum ConvPath : int { kConvElementwise = 0, kConvTimeFast = 1, kConvChanFast = 2 };

struct ConvShape {
  int batch, dim, seqlen, width;
  int64_t sx[3], so[3];  // x, out: (b, d, t) element strides
  int64_t sw[2];         // weight: (d, k)
  int silu;
  int path;              // ConvPath
  int seg_len;           // channel-fast path: steps per thread
  int nseg;
  int cf_lanes;          // channel-fast path: lanes per row of channels (power of 2, <= 64)
};

struct ConvPtrs {
  const void* x;
  const float* weight;
  const float* bias;
  const void* init;  // [batch][dim][width-1] or null
  void* out;
  void* fin;         // [batch][dim][width-1] or null
};

struct ConvStepShape {
  int batch, dim, width;
  int64_t sx[2], so[2];  // (b, d)
  int64_t sw[2];
  int silu;
};

struct ConvStepPtrs {
  void* state;
  const void* x;
  const float* weight;
  const float* bias;
  void* out;
};

hipError_t launch_conv(const ConvShape& s, const ConvPtrs& p, bool io_bf16, hipStream_t stream);
hipError_t launch_conv_step(const ConvStepShape& s, const ConvStepPtrs& p, bool io_bf16,
                            hipStream_t stream);

// Selective-scan backward.  A workgroup of kBwdWaves waves owns kBwdCh
// channels of one batch row (kCh per wave, lanes as in the forward scan:
// lane (g, c) runs states 2g, 2g+1 of channel c) and walks the sequence in
// chunks of kBwdT steps, the last chunk first.  Four-wave workgroups at up
// to 168 VGPRs and 46 KB of LDS put three workgroups on a CU.
constexpr int kBwdT = kStateChunk;  // a backward chunk is one chunk-state interval
constexpr int kBcSteps = 4;          // dB/dC sum: consecutive steps per thread
constexpr int kBwdWaves = 4;
constexpr int kBwdCh = kCh * kBwdWaves;  // 32
constexpr int kBwdThreads = 64 * kBwdWaves;

struct BwdShape {
  int batch, dim, seqlen, dstate;
  int softplus;
  int nchunk;         // ceil(seqlen / kBwdT)
  int npair;          // ceil(nchunk / 2)
  int tiles;          // ceil(dim / kBwdCh) workgroups per batch row
  int nseg;           // time segments (each seg_chunks chunks; the last may be shorter)
  int seg_chunks;
  int agg_split;      // the aggregate pass cuts each segment into this many parts (a power of 2)
  int64_t nchan_pad;  // batch * tiles * kBwdCh: rows of the checkpoint array
  int64_t su[3], sd[3], sz[3], sdo[3];      // u, delta_raw, z, dout: (b, d, t)
  int64_t sdu[3], sddr[3], sdz[3];          // du, ddelta_raw, dz
  int64_t sB[3], sC[3], sdB[3], sdC[3];     // (b, n, t)
  int64_t sA[2];                            // A_log: (d, n)
  int reverse;                              // logical step tau is storage step seqlen-1-tau
  int pairs;  // the reverse walk moves u, delta_raw, dout, z, du, ddelta_raw, dz
              // as pairs of adjacent steps (unit time stride, even length and strides)
  int quads;  // the checkpoint pass reads u, delta_raw as 4-step vectors
              // (unit time stride, length and strides multiples of 4)
  int bquads;  // ... and B too (the same conditions on B)
  int bcquads;  // B and C both meet them: the segment aggregates read B, C as 4-step vectors
  int dpairs;   // channel-last data: the segment aggregate and checkpoint passes run in
                // 4-wave workgroups per 32-channel tile and read u, delta_raw, dout, z as
                // pairs of adjacent channels (unit channel stride, even dim and strides)
  int nquads;   // the one-wave segment aggregate pass reads B, C as 4-state vectors (unit
                // state stride, dstate and strides multiples of 4)
  int states_given;  // ckpt holds chunk states recorded by the forward: no checkpoint pass
};

struct BwdPtrs {
  const void* u;
  const void* delta_raw;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  const float* h0;
  const void* dout;
  const float* dfinal;
  void* du;
  void* ddelta_raw;
  float* dA_log;
  void* dB;
  void* dC;
  float* dD;
  void* dz;
  float* ddt_bias;
  float* dh0;
  // workspace
  float* ckpt;       // [nchunk][batch][dim][kMaxState] state entering each chunk (chunk states)
  float* part_bc;    // [batch][npair][tiles][2 * kMaxState][2 kBwdT] per-workgroup dB, dC sums:
                     // a workgroup's two chunks of a pair fill 128-byte row pieces, 4 KB in one place
  float* part_chan;  // [nseg][batch][dim][kMaxState + 2] per-row dA_log, dD, ddt_bias
  float4* agg;       // [nseg * agg_split][nchan_pad][kMaxState] per segment part
                     // (prod a, h from 0, g from 0, -)
  float* carry_h;    // [nseg][nchan_pad][kMaxState] state entering each segment
  float* carry_g;    // [nseg][nchan_pad][kMaxState] adjoint reaching each segment's last state
};

hipError_t launch_scan_bwd(const BwdShape& s, const BwdPtrs& p, bool io_bf16, hipStream_t stream);

// Enqueue the scan (segment aggregates, carry propagation when nseg > 1, then
// the main pass).  io_bf16 selects the bf16 storage type; x_tfast says that
// u/delta_raw/z/out have unit stride along t (else along d), bc_tfast that B
// and C have unit stride along t (else along n).
hipError_t launch_scan(const ScanShape& s, const ScanPtrs& p, bool io_bf16, bool x_tfast,
                       bool bc_tfast, hipStream_t stream);

hipError_t launch_step(const StepShape& s, const StepPtrs& p, bool io_bf16, hipStream_t stream);

}  // namespace mss
