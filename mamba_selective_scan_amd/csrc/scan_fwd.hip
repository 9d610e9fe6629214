// scan_fwd.hip -- selective-scan forward kernels for gfx950 (wave64).
//
// What is computed, per channel (b, d), time t and diagonal state n:
//   delta_t = softplus(delta_raw + dt_bias)   A[n] = -exp(A_log[d, n])
//   h_t[n]  = exp(delta_t A[n]) h_{t-1}[n] + delta_t B[b, n, t] u_t
//   out_t   = (sum_n C[b, n, t] h_t[n] + D[d] u_t) * silu(z_t)
// (the recurrence of "mamba-metal: Apple Silicon で Mamba を動かす", section
// "Selective scan の本質", with the diagonal discretisation and the chunk flow
// described in createcentury's reading of the official CUDA kernel, sections
// "なぜ「scan」か" and "1チャンク内の処理フロー").
//
// Mapping.  A is diagonal, so the dstate entries are independent recurrences
// that only meet in the sum over C.  One wave owns 8 channels of one batch
// row for one time segment (a workgroup is that one wave, or the four waves
// of a 32-channel block for d-fast data: kWavesPerWg).  In the scan, lane
// (g, c) = (lane / 8, lane % 8) runs states 2g and 2g+1 of channel c
// sequentially in time, in registers; A_log becomes exp2 multipliers with
// log2(e) folded in, once per lane.  Small waves keep several per SIMD: the
// SIMD's VALU switches to another wave while one waits for memory, and the
// work spreads evenly over the SIMDs.  The segment is walked in chunks of kT
// steps, each in three phases:
//   E  loads of u, delta_raw, B and C (issued ahead of use) with 4-element
//      vectors along the unit-stride axis; softplus, delta*u and D*u per
//      element; (delta, delta*u) and B/C go to LDS;
//   S  per step and state one exp2, two multiplies and two FMAs, all on plain
//      VGPR operands: each lane reads the B and C of its two states from LDS
//      four steps at a time.  The partial sums C.h of the eight state groups
//      of a channel meet through v_permlane32_swap and v_permlane16_swap:
//      two swap-and-add levels reduce four steps at once to two half sums
//      (over the groups of each parity);
//   O  the half sums go through LDS back to the load layout, where they are
//      added, the skip term and the gate are applied and the output is
//      stored.
// For t-fast data every phase is wave-local: there is no workgroup barrier,
// so waves drift apart and memory waits of one wave overlap the recurrence
// of others.  The d-fast vector path exchanges its loads and stores between
// the four waves of a workgroup through LDS, with two barriers per chunk.
//
// Reverse time (REV): logical step tau reads and writes storage step L-1-tau,
// so a backward-direction scan (one half of a bidirectional layer) runs on
// the caller's buffers without a flipped copy.  A chunk's descriptor then
// sits at storage step L-kT-t0 and every time offset inside the chunk is
// mirrored; a 4-step vector along t is loaded whole and its elements taken in
// the opposite order.
//
// Long sequences with few channels are split into time segments so that the
// grid covers the GPU.  Segment s needs the state entering it.  A first pass
// (AGG) runs every segment but the last from a zero state and records, per
// (channel, state), the segment's pair aggregate (prod_t a_t, h_end): the
// product is exp2(A2 * sum_t delta_t) since all a_t share A.  Its waves need
// fewer registers than the main pass's, so it cuts each segment into
// agg_split parts and records one aggregate per part.  A carry pass
// composes the aggregates in order with (a2, b2) o (a1, b1) = (a2 a1,
// a2 b1 + b2) ("mamba-metal", sections "Selective scan の本質" and
// "チャンク間 running prefix"), and the main pass starts each segment from
// its carry.
#include <algorithm>
#include <type_traits>

#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {

using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

// 4-element vectors (16 bytes of fp32, 8 bytes of bf16) and single-element
// buffer access, per storage type.
template <typename IO>
struct vec_io;
template <>
struct vec_io<float> {
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                     float* o) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __uint_as_float(w[j]);
  }
  __device__ static inline void store(const float* y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                      uint32_t soff) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __float_as_uint(y[j]);
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, soff, 0);
  }
  __device__ static inline float load_one(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return buf_one<float>::load(r, off, soff);
  }
  __device__ static inline void store_one(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          uint32_t soff) {
    buf_one<float>::store(y, r, off, soff);
  }
};
template <>
struct vec_io<bf16_t> {
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff,
                                     float* o) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o[2 * j] = __uint_as_float(w[j] << 16);
      o[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ static inline void store(const float* y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                      uint32_t soff) {
    u32x2 w;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[j] = bf16x2_bits(y[2 * j], y[2 * j + 1]);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, soff, 0);
  }
  __device__ static inline float load_one(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return buf_one<bf16_t>::load(r, off, soff);
  }
  __device__ static inline void store_one(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          uint32_t soff) {
    buf_one<bf16_t>::store(y, r, off, soff);
  }
};

constexpr int kXcds = 8;                // MI355X: 8 accelerator dies, 32 CUs each
constexpr int kBcRows = 2 * kMaxState;  // B0..B15, C0..C15
// LDS layouts (floats).  Rows are 16-byte aligned for 128-bit accesses, and
// the eight distinct rows that one S-phase instruction reads fall in distinct
// bank groups: s_dd rows are padded; s_bc rows are not (the LDS budget allows
// five waves per SIMD only without the padding) and instead store the
// 4-step group q of row r at position q ^ ((r / 2) % 8).
constexpr int kDdPitch = 2 * kT + 4;  // s_dd[channel][t] as (delta, delta*u) pairs
__device__ inline int bc_index(int row, int t) {
  return row * kT + ((((t >> 2) ^ (row >> 1)) & 7) << 2) + (t & 3);
}
constexpr int kSkipPitch = kT + 4;    // s_skip[channel][t]

struct f4 {
  float x, y, z, w;
};
__device__ inline f4 lds_f4(const float* p) { return *reinterpret_cast<const f4*>(p); }

// Five waves per SIMD (at most 96 VGPRs) for the vector paths; the
// element-wise paths (ragged tails, unaligned views) and the fp32 d-fast
// n-fast path need more registers and run four.
template <typename IO, bool VEC, bool XT, bool BT>
constexpr int kWavesPerSimd = (VEC && (XT || BT || sizeof(IO) == 2)) ? 5 : 4;

// Waves per workgroup.  For t-fast data a workgroup is one wave.  For d-fast
// data a tile's row of 8 channels is 32 bytes, a quarter of a 128-byte line,
// so a workgroup holds the four tiles of a 32-channel block: on the vector
// path they load and store whole rows together (COOP in the kernel); on the
// element-wise path they stay independent and only share the CU's L1.
template <bool XT>
constexpr int kWavesPerWg = XT ? 1 : 4;

// LTI: B and C do not depend on t (time stride 0, the time-invariant case of
// createcentury's reading, "主要な最適化テクニック": the kIsVariableB/C
// switches).  Each lane then holds the B and C of its two states in registers
// for the whole segment: no B/C loads, LDS stores or LDS reads per chunk.
template <typename IO, bool XT, bool BT, bool AGG, bool VEC, bool REV, bool LTI>
__global__ __launch_bounds__(kThreads * kWavesPerWg<XT>) __attribute__((amdgpu_waves_per_eu(
    kWavesPerSimd<IO, VEC, XT, BT || LTI>, 8))) void scan_kernel(
    ScanShape s, const IO* __restrict__ u, const IO* __restrict__ delta_raw,
    const float* __restrict__ A_log, const IO* __restrict__ Bm, const IO* __restrict__ Cm,
    const float* __restrict__ Dskip, const IO* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ h0, IO* __restrict__ out,
    float* __restrict__ final_state, float2* __restrict__ agg,
    const float* __restrict__ carry, float* __restrict__ chunk_states) {
  constexpr int kWg = kWavesPerWg<XT>;
  // COOP (the d-fast vector path): the waves of a workgroup own the four
  // 8-channel tiles of one 32-channel block (same batch row and segment) and
  // move its data together.  Each wave loads and stores 8 whole 128-byte rows
  // (8 steps x 32 channels) per tensor and chunk, and every value goes to the
  // LDS slice of the wave that scans it; B and C are loaded once per
  // workgroup.  The exchange takes two workgroup barriers per chunk, and the
  // LDS buffers alternate with the chunk's parity.
  constexpr bool COOP = !XT && VEC;
  // The AGG pass has no output phase: a chunk's second barrier already orders
  // every read of its buffer before the next chunk's E phase writes it, so one
  // buffer serves (half the LDS, which leaves room for eight waves per SIMD).
  constexpr int kBufs = (COOP && !AGG) ? 2 : 1;
  constexpr int kBcSize = LTI ? 4 : (AGG ? kMaxState : kBcRows) * kT;
  constexpr int kDdSize = kCh * kDdPitch;
  constexpr int kSkipSize = (AGG || COOP) ? 4 : kCh * kSkipPitch;  // COOP keeps D*u in registers
  constexpr int kChanSpan = COOP ? kWg * kCh : kCh;  // channels whose dt_bias, D sit in s_chan
  __shared__ __attribute__((aligned(16))) float s_bc_all[(COOP ? kBufs : kWg) * kBcSize];
  __shared__ __attribute__((aligned(16))) float s_dd_all[kBufs * kWg * kDdSize];
  __shared__ __attribute__((aligned(16))) float s_skip_all[kBufs * kWg * kSkipSize];
  __shared__ __attribute__((aligned(16))) float s_chan_all[kWg * 2 * kCh];  // dt_bias, D (d-fast)

  const int lane = threadIdx.x & 63;
  const int wave = kWg == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wave's slices (buffer 0; COOP buffer nb adds nb * kBcSize, nb * kWg * kDdSize, ...)
  float* const s_bc = s_bc_all + (COOP ? 0 : wave * kBcSize);
  float* const s_dd = s_dd_all + wave * kDdSize;
  float* const s_skip = s_skip_all + wave * kSkipSize;
  float* const s_chan = s_chan_all + (COOP ? 0 : wave * 2 * kCh);
  // Workgroups are dispatched round-robin over the XCDs (linear id mod 8).
  // Renumber them so that each XCD receives a contiguous range of tiles:
  // tiles of one batch row share B and C, which then stay in that XCD's L2.
  // Tile i of the pass is channel group i % G, time segment i / G (COOP:
  // workgroup i is 32-channel block i % GQ, segment i / GQ).
  const int nwg = gridDim.x;
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  const int per_xcd = nwg / kXcds, extra = nwg % kXcds;
  const int logical = xcd * per_xcd + min(xcd, extra) + lin / kXcds;
  // The AGG pass walks part `link % agg_split` of segment `link / agg_split`.
  const int pass_links = AGG ? (s.nseg - 1) * s.agg_split : s.nseg;
  int b, d0, link, dx0;  // dx0: first channel of the x data the lane loads and stores
  bool tile_ok = true;  // COOP: the wave's tile lies inside the channel groups
  if constexpr (COOP) {
    const int quads = (s.groups + kWg - 1) / kWg;
    const int GQ = s.batch * quads;
    if (logical >= GQ * pass_links) return;  // uniform over the workgroup
    const int gq = logical % GQ;
    link = logical / GQ;
    b = gq / quads;
    const int group = (gq - b * quads) * kWg + wave;
    tile_ok = group < s.groups;
    d0 = group * kCh;
    dx0 = (gq - b * quads) * kWg * kCh;
  } else {
    const int G = s.batch * s.groups;
    const int tile = logical * kWg + wave;
    if (tile >= G * pass_links) return;  // the last workgroup's spare waves
    const int g = tile % G;
    link = tile / G;
    b = g / s.groups;
    d0 = (g - b * s.groups) * kCh;
    dx0 = d0;
  }
  const int seg = AGG ? link / s.agg_split : link;
  const int seg_begin = s.t_first + seg * s.seg_len;
  const int seg_end = min(s.t_stop, seg_begin + s.seg_len);
  // (a trailing part may be empty: it walks no chunk and records (1, 0))
  const int t_begin = AGG ? seg_begin + (link - seg * s.agg_split) * s.part_len : seg_begin;
  const int t_end = AGG ? min(seg_end, t_begin + s.part_len) : seg_end;
  constexpr int64_t es = sizeof(IO);

  // ---- S-phase constants: lane = (state group sg, channel sc) ----
  const int sg = lane >> 3;
  const int sc = lane & 7;
  const int d = d0 + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.groups * kCh + sc + d0;  // workspace row
  float A2[kStatesPerLane], h[kStatesPerLane];
#pragma unroll
  for (int k = 0; k < kStatesPerLane; ++k) {
    const int n = sg * kStatesPerLane + k;
    const bool active = dvalid && n < s.dstate;
    A2[k] = active ? -expf(A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e : 0.0f;
    float h_init = 0.0f;
    if (!AGG && active) {
      if (seg > 0)
        h_init = carry[(static_cast<int64_t>(seg) * s.nchan_pad + chan_row) * kMaxState + n];
      else if (h0 != nullptr)
        h_init = h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n];
    }
    h[k] = h_init;
  }
  float sum_delta = 0.0f;
  // LTI: B (and C outside the AGG pass) of the lane's two states
  float b_lti[kStatesPerLane] = {}, c_lti[kStatesPerLane] = {};
  if constexpr (LTI) {
#pragma unroll
    for (int k = 0; k < kStatesPerLane; ++k) {
      const int n = sg * kStatesPerLane + k;
      if (n < s.dstate) {
        b_lti[k] = io_traits<IO>::load(Bm + static_cast<int64_t>(b) * s.sB[0] + n * s.sB[1]);
        if constexpr (!AGG)
          c_lti[k] = io_traits<IO>::load(Cm + static_cast<int64_t>(b) * s.sC[0] + n * s.sC[1]);
      }
    }
  }

  // ---- chunk memory access ------------------------------------------------
  // All global traffic uses raw buffer loads/stores: a per-chunk descriptor
  // whose base is the tile corner, a 32-bit per-lane offset and a scalar
  // offset per vector.  An element or vector that lies outside the tensor gets
  // an offset beyond the descriptor's range, so the hardware returns 0 (or
  // drops the store) without a branch: every chunk issues the same
  // instruction stream and the compiler counts outstanding loads exactly.
  // Each lane moves one 4-element vector per x-tensor and chunk along the
  // unit-stride axis: for t-fast data lane (xa, xb) = (lane / 8, lane % 8)
  // covers channel xa, steps 4xb..4xb+3 (8 rows of 128 fp32 bytes); for
  // d-fast data lane (lane / 2, lane % 2) covers step lane / 2, channels
  // 4(lane % 2)..+3.  A chunk whose vectors would straddle a tensor edge (a
  // ragged tail) takes the element-wise instantiation instead.
  using VIO = vec_io<IO>;
  // COOP: lane (lane / 8, lane % 8) of wave w covers step 8w + lane / 8,
  // channels 4(lane % 8)..+3 of the 32-channel block.
  const int xa = XT ? lane >> 3 : (COOP ? kCh * wave + (lane >> 3) : lane >> 1);
  const int xb = XT ? lane & 7 : (COOP ? lane & 7 : lane & 1);
  auto x_c = [&](int j) __attribute__((always_inline)) { return XT ? xa : 4 * xb + j; };
  auto x_t = [&](int j) __attribute__((always_inline)) { return XT ? 4 * xb + j : xa; };
  // Time offset of a lane's first x element inside a chunk (mirrored in
  // reverse time: for t-fast vectors the storage start of the vector).
  const int x_toff = REV ? (XT ? kT - kVec - 4 * xb : kT - 1 - xa) : x_t(0);
  auto x_voff = [&](const int64_t* st) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>((x_c(0) * st[1] + x_toff * st[2]) * es);
  };
  // Offset of element j from the lane's first element, for element-wise access.
  auto x_eoff = [&](const int64_t* st, int j) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>((XT ? (REV ? kVec - 1 - j : j) * st[2] : j * st[1]) * es);
  };
  // A t-fast vector read in reverse time holds its steps in the opposite order.
  auto mirror4 = [&](float* v) __attribute__((always_inline)) {
    if constexpr (REV) {
      const float a0 = v[0], a1 = v[1];
      v[0] = v[3];
      v[1] = v[2];
      v[2] = a1;
      v[3] = a0;
    }
  };
  // B/C: instruction i (0, 1: B; 2, 3: C) of a lane covers, for t-fast B/C,
  // state (lane / 8) + 8(i % 2) at steps 4(lane % 8)..+3, and for n-fast B/C
  // step (lane / 4) + 16(i % 2) at states 4(lane % 4)..+3.
  const int ba = BT ? lane >> 3 : lane >> 2;
  const int bb = BT ? lane & 7 : lane & 3;
  auto bc_n = [&](int i, int j) __attribute__((always_inline)) {
    return BT ? ba + 8 * (i & 1) : 4 * bb + j;
  };
  auto bc_tt = [&](int i, int j) __attribute__((always_inline)) {
    return BT ? 4 * bb + j : ba + 16 * (i & 1);
  };
  // In reverse time the n-fast lanes' steps ba and ba + 16 sit at storage
  // offsets kT-1-ba and kT-17-ba: the vector offset takes the latter and the
  // scalar offset adds 16 steps for the even instructions.
  const int bc_toff = REV ? (BT ? kT - kVec - 4 * bb : kT - 17 - ba) : (BT ? 4 * bb : ba);
  auto bc_voff = [&](const int64_t* st) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(((BT ? ba : 4 * bb) * st[1] + bc_toff * st[2]) * es);
  };
  auto bc_soff = [&](const int64_t* st, int i) __attribute__((always_inline)) -> uint32_t {
    if constexpr (BT) return static_cast<uint32_t>((i & 1) * 8 * st[1] * es);
    return static_cast<uint32_t>((REV ? 1 - (i & 1) : (i & 1)) * 16 * st[2] * es);
  };
  auto bc_eoff = [&](const int64_t* st, int j) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>((BT ? (REV ? kVec - 1 - j : j) * st[2] : j * st[1]) * es);
  };

  // Channel constants (dt_bias, D).  With t-fast data each lane's elements
  // share one channel and the pair stays in registers; with d-fast data a
  // lane's four elements are four channels, and the pairs of the tile's 8
  // channels sit in LDS (s_chan) to keep registers for the loads in flight.
  float bias_t = 0.0f, skip_t = 0.0f;
  if constexpr (XT) {
    const int dc = d0 + xa;
    bias_t = (dc < s.dim && dt_bias != nullptr) ? dt_bias[dc] : 0.0f;
    skip_t = (dc < s.dim && Dskip != nullptr) ? Dskip[dc] : 0.0f;
  } else if constexpr (COOP) {
    if (wave == 0) {
      const int dc = dx0 + (lane & (kChanSpan - 1));
      const float* src = lane < kChanSpan ? dt_bias : Dskip;
      s_chan[lane] = (dc < s.dim && src != nullptr) ? src[dc] : 0.0f;
    }
    __syncthreads();
  } else if (lane < 2 * kCh) {
    const int dc = d0 + (lane & (kCh - 1));
    const float* src = lane < kCh ? dt_bias : Dskip;
    s_chan[lane] = (dc < s.dim && src != nullptr) ? src[dc] : 0.0f;
  }
  const bool has_z = z != nullptr;

  // Chunk descriptor base: storage step t0, or L-kT-t0 in reverse time (it may
  // lie before the tensor; only in-range offsets are ever used).
  auto rsrc = [&](const void* ptr, const int64_t* st, int dd0, int t0,
                  int range = kRsrcRange) __attribute__((always_inline)) {
    const int64_t ts = REV ? static_cast<int64_t>(s.seqlen) - kT - t0 : t0;
    const char* base = reinterpret_cast<const char*>(ptr) +
                       (static_cast<int64_t>(b) * st[0] + static_cast<int64_t>(dd0) * st[1] +
                        ts * st[2]) * es;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, range, kRsrcFlags);
  };
  // x_ok / b_ok: element j / B-C value (i, j) lies inside the tensors and the
  // chunk is one this loop loads (lim: first chunk start not loaded).
  auto x_ok = [&](int j, int t0, int lim) __attribute__((always_inline)) {
    return (t0 < lim) && (dx0 + x_c(j) < s.dim) && (t0 + x_t(j) < t_end);
  };
  auto b_ok = [&](int i, int j, int t0, int lim) __attribute__((always_inline)) {
    return (t0 < lim) && (bc_n(i, j) < s.dstate) && (t0 + bc_tt(i, j) < t_end);
  };

  // Chunk inputs live in registers from issue to use: u, delta_raw and B/C
  // one chunk ahead of the chunk being scanned, z from the end of the
  // previous chunk's output phase.
  struct InBuf {
    float u[kPerThread], d[kPerThread];
  };
  struct ZBuf {
    float z[kPerThread];
  };
  constexpr int kBcLoads = LTI ? 0 : (COOP ? 1 : (AGG ? 2 : 4));  // the AGG pass needs no C
  float bcb[kBcLoads > 0 ? kBcLoads * kVec : 1];  // B/C of the next chunk

  // Loads of one x-tensor.  VEC: one vector (wholly in or out of the valid
  // region); else element by element.
  auto load_x = [&](float (&dst)[kPerThread], const IO* ptr, const int64_t* st, int t0, int lim,
                    int range = kRsrcRange) __attribute__((always_inline)) {
    const auto rs = rsrc(ptr, st, dx0, t0, range);
    const uint32_t vo = x_voff(st);
    if constexpr (VEC) {
      VIO::load(rs, x_ok(0, t0, lim) ? vo : kOffNone, 0, dst);
      if constexpr (XT) mirror4(dst);
    } else {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const uint32_t off = x_ok(j, t0, lim) ? vo + x_eoff(st, j) : kOffNone;
        dst[j] = VIO::load_one(rs, off, 0);
      }
    }
  };
  // Without z the descriptor has an empty range and the loads return 0: the
  // instruction stream stays the same, so no branch splits the loop body
  // (a load under a branch makes the compiler drain every outstanding load).
  const IO* z_ptr = has_z ? z : u;
  const int z_range = has_z ? kRsrcRange : 0;
  auto issue_z_loads = [&](ZBuf& zb, int t0, int lim) __attribute__((always_inline)) {
    if constexpr (!AGG) load_x(zb.z, z_ptr, s.sz, t0, lim, z_range);
  };
  auto issue_x_loads = [&](InBuf& ib, int t0, int lim) __attribute__((always_inline)) {
    load_x(ib.u, u, s.su, t0, lim);
    load_x(ib.d, delta_raw, s.sd, t0, lim);
  };
  // COOP B/C: waves 0, 1 load B and waves 2, 3 load C, one vector per lane:
  // t-fast, state 8(w % 2) + lane / 8 at steps 4(lane % 8)..+3; n-fast, step
  // 16(w % 2) + lane / 4 at states 4(lane % 4)..+3.
  const bool cb_c = COOP && wave >= 2;
  const int cb_n = BT ? kCh * (wave & 1) + (lane >> 3) : 4 * (lane & 3);
  const int cb_t = BT ? 4 * (lane & 7) : 16 * (wave & 1) + (lane >> 2);
  auto issue_bc_loads = [&](int t0, int lim) __attribute__((always_inline)) {
    if constexpr (LTI) {
      return;
    } else if constexpr (COOP) {
      const int64_t* st = cb_c ? s.sC : s.sB;
      const auto rs = rsrc(cb_c ? Cm : Bm, st, 0, t0);
      const int ts = REV ? (BT ? kT - kVec - cb_t : kT - 1 - cb_t) : cb_t;
      const bool ok = (t0 < lim) && !(AGG && cb_c) && cb_n < s.dstate && t0 + cb_t < t_end;
      VIO::load(rs, ok ? static_cast<uint32_t>((cb_n * st[1] + ts * st[2]) * es) : kOffNone, 0, bcb);
      if constexpr (BT) mirror4(bcb);
      return;
    }
    const auto rb = rsrc(Bm, s.sB, 0, t0);
    const auto rcm = rsrc(Cm, s.sC, 0, t0);
#pragma unroll
    for (int i = 0; i < kBcLoads; ++i) {
      const bool is_c = i >= 2;
      const auto& rs = is_c ? rcm : rb;
      const int64_t* st = is_c ? s.sC : s.sB;
      const uint32_t vo = bc_voff(st);
      float* dst = bcb + i * kVec;
      if constexpr (VEC) {
        VIO::load(rs, b_ok(i, 0, t0, lim) ? vo : kOffNone, bc_soff(st, i), dst);
        if constexpr (BT) mirror4(dst);
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const uint32_t off = b_ok(i, j, t0, lim) ? vo + bc_eoff(st, j) : kOffNone;
          dst[j] = VIO::load_one(rs, off, bc_soff(st, i));
        }
      }
    }
  };

  // E: (delta, delta*u) and D*u of the chunk go to LDS (s_dd, s_skip), B/C
  // from registers to s_bc.
  // d-fast (delta, delta*u) and D*u slots of the lane's element j in LDS
  // buffer nb: COOP sends channel 4xb+j of the block to wave (4xb+j) / 8.
  auto e_dd = [&](int nb, int j) __attribute__((always_inline)) -> float* {
    if constexpr (COOP)
      return s_dd_all + nb * kWg * kDdSize + (xb >> 1) * kDdSize +
             (4 * (xb & 1) + j) * kDdPitch + 2 * xa;
    return s_dd + (4 * xb + j) * kDdPitch + 2 * xa;
  };
  auto e_sk = [&](int nb, int j) __attribute__((always_inline)) -> float* {
    return s_skip + nb * kSkipSize + (4 * xb + j) * kSkipPitch + xa;  // not COOP: nb = 0
  };
  // COOP: a lane's E and O phases cover the same elements, so D*u of the
  // next chunk waits in registers (skr) instead of LDS.
  float skr[kPerThread];
  auto phase_e = [&](const InBuf& ib, int t0, int nb) __attribute__((always_inline)) {
    float dl[kPerThread], du[kPerThread], sk[kPerThread], bias[kPerThread], skip[kPerThread];
    if constexpr (XT) {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        bias[j] = bias_t;
        skip[j] = skip_t;
      }
    } else {
      const f4 bv = lds_f4(s_chan + 4 * xb), sv = lds_f4(s_chan + kChanSpan + 4 * xb);
      bias[0] = bv.x; bias[1] = bv.y; bias[2] = bv.z; bias[3] = bv.w;
      skip[0] = sv.x; skip[1] = sv.y; skip[2] = sv.z; skip[3] = sv.w;
    }
    // Outside the tensors u reads 0, so delta*u and D*u are 0 already; delta
    // itself is zeroed there so that the state passes through unchanged.  A
    // vector is wholly inside or outside.
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const bool ok = x_ok(VEC ? 0 : j, t0, t_end);
      const float x = ib.d[j] + bias[j];
      const float sp = s.softplus ? softplus(x) : x;
      dl[j] = ok ? sp : 0.0f;
      du[j] = dl[j] * ib.u[j];
      sk[j] = skip[j] * ib.u[j];
    }
    if constexpr (XT) {
      // 4 consecutive steps of one channel: two 16-byte (delta, delta*u) pairs
      float* p = s_dd + xa * kDdPitch + 8 * xb;
      *reinterpret_cast<f4*>(p) = f4{dl[0], du[0], dl[1], du[1]};
      *reinterpret_cast<f4*>(p + 4) = f4{dl[2], du[2], dl[3], du[3]};
      if constexpr (!AGG)
        *reinterpret_cast<f4*>(s_skip + xa * kSkipPitch + 4 * xb) = f4{sk[0], sk[1], sk[2], sk[3]};
    } else {
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        *reinterpret_cast<float2*>(e_dd(nb, j)) = make_float2(dl[j], du[j]);
        if constexpr (COOP)
          skr[j] = sk[j];
        else if constexpr (!AGG)
          *e_sk(nb, j) = sk[j];
      }
    }
    if constexpr (LTI) {
      // B and C stay in registers
    } else if constexpr (COOP) {
      // one vector per lane into the workgroup's shared B/C buffer (n-fast:
      // the two-index form of the non-cooperative path below)
      float* const sbc = s_bc_all + nb * kBcSize;
      const int c_rows = cb_c ? kMaxState * kT : 0;
      if (!(AGG && cb_c)) {
        if constexpr (BT) {
          *reinterpret_cast<f4*>(sbc + c_rows + bc_index(cb_n, cb_t)) =
              f4{bcb[0], bcb[1], bcb[2], bcb[3]};
        } else {
          const int f0 = bc_index(cb_n, cb_t) + c_rows;
          const int f2 = bc_index(cb_n + 2, cb_t) + c_rows;
          sbc[f0] = bcb[0];
          sbc[f0 + kT] = bcb[1];
          sbc[f2] = bcb[2];
          sbc[f2 + kT] = bcb[3];
        }
      }
    } else if constexpr (BT) {
#pragma unroll
      for (int i = 0; i < kBcLoads; ++i) {
        const int row0 = (i >= 2 ? kMaxState : 0);
        *reinterpret_cast<f4*>(s_bc + bc_index(row0 + bc_n(i, 0), bc_tt(i, 0))) =
            f4{bcb[i * kVec], bcb[i * kVec + 1], bcb[i * kVec + 2], bcb[i * kVec + 3]};
      }
    } else {
      // n-fast: value (i, j) is state 4bb+j (+16 rows for C) at step ba+16(i%2).
      // Its swizzled position follows from two computed ones: rows 4bb+1 and
      // 4bb+3 share the key of rows 4bb and 4bb+2 (one row further on), step
      // ba+16 flips bit 2 of the 4-step group (index ^ 16), and C rows keep
      // the key of the B rows 16 rows before.  Four address registers instead
      // of one per value.
      const int e0 = bc_index(bc_n(0, 0), bc_tt(0, 0));
      const int e2 = bc_index(bc_n(0, 2), bc_tt(0, 0));
#pragma unroll
      for (int i = 0; i < kBcLoads; ++i) {
        const int c_rows = i >= 2 ? kMaxState * kT : 0;
        const int f0 = ((i & 1) ? e0 ^ 16 : e0) + c_rows;
        const int f2 = ((i & 1) ? e2 ^ 16 : e2) + c_rows;
        s_bc[f0] = bcb[i * kVec];
        s_bc[f0 + kT] = bcb[i * kVec + 1];
        s_bc[f2] = bcb[i * kVec + 2];
        s_bc[f2 + kT] = bcb[i * kVec + 3];
      }
    }
  };

  // S-phase LDS addresses of this lane: B and C rows of states 2sg, 2sg+1 and
  // the (delta, delta*u) row of channel sc.
  // (all four rows share the swizzle key sg)
  const float* p_b0 = s_bc + (2 * sg) * kT;
  const float* p_c0 = s_bc + (AGG ? 0 : (kMaxState + 2 * sg) * kT);
  const float* p_dd = s_dd + sc * kDdPitch;
  // The same B rows as byte offsets from the buffer start, for the AGG pass's
  // rolled block loop: rows 2sg, 2sg+1 start 256 sg bytes in (bits 4..6 clear)
  // and the swizzled column of block t4 / 4 flips bits 4..6 only, so one XOR
  // per block gives the address: 256 sg + 16 ((t4 / 4) ^ (sg % 8)).
  const uint32_t b_key = static_cast<uint32_t>(2 * sg * kT * 4 + ((sg & 7) << 4));
  // The group reduction leaves step {0, 2, 1, 3}[row] of each block in row
  // `row` = lane / 16, as two sums over four state groups each: lane c + 8h
  // of the row holds the sum over the groups of parity h.  The two sums of
  // step t replace (delta_t, delta_t * u_t) in s_dd -- the block has read
  // them, and later blocks read other steps -- and the output phase adds
  // them (the same sum, in the same order, as a cross-lane add here).
  const int row = lane >> 4;
  const int y_step = row == 1 ? 2 : (row == 2 ? 1 : row);
  float* p_y = s_dd + sc * kDdPitch + 2 * y_step + ((lane >> 3) & 1);

  // Chunk states (main pass only): the state entering logical step t when t
  // is a multiple of kStateChunk, written by the lane for its two states.
  // Vector passes start every chunk on a multiple of kT, so only the blocks
  // at t4 = 0 and t4 = kStateChunk can record, and there the record is one
  // buffer store whose offset falls outside the range when the state is not
  // wanted: no branch in the block, so the next block's LDS reads can be
  // issued ahead.
  const int64_t cs_row = static_cast<int64_t>(b) * s.dim + d;
  const int64_t cs_plane = static_cast<int64_t>(s.batch) * s.dim;
  const bool has_cs = !AGG && chunk_states != nullptr;
  const uint32_t cs_off = static_cast<uint32_t>((sc * kMaxState + sg * kStatesPerLane) * 4);
  auto record_state = [&](int t, int t4) __attribute__((always_inline)) {
    if constexpr (AGG) {
      return;
    } else if constexpr (VEC) {
      static_assert(kT % kStateChunk == 0, "chunks start on chunk-state boundaries");
      if (t4 % kStateChunk != 0) return;
      const int64_t tile0 =
          (static_cast<int64_t>(t / kStateChunk) * cs_plane + static_cast<int64_t>(b) * s.dim +
           d0) * kMaxState;
      void* base = has_cs ? static_cast<void*>(chunk_states + tile0) : static_cast<void*>(out);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, has_cs ? kRsrcRange : 0,
                                                        kRsrcFlags);
      const u32x2 w = {__float_as_uint(h[0]), __float_as_uint(h[1])};
      __builtin_amdgcn_raw_buffer_store_b64(w, rs, (dvalid && t < t_end) ? cs_off : kOffNone, 0,
                                            0);
    } else {
      if (has_cs && (t & (kStateChunk - 1)) == 0 && t < t_end && dvalid)
        *reinterpret_cast<float2*>(chunk_states +
                                   ((t / kStateChunk) * cs_plane + cs_row) * kMaxState +
                                   sg * kStatesPerLane) = make_float2(h[0], h[1]);
    }
  };

  // One block of 4 steps: the scan of this lane's two states and, outside
  // the AGG pass, one state-group reduction of C.h.
  auto scan_block = [&](int t4, int t0, int nb) __attribute__((always_inline)) {
    record_state(t0 + t4, t4);
    const int col = (((t4 >> 2) ^ sg) & 7) << 2;
    const float* pb = AGG ? reinterpret_cast<const float*>(
                                reinterpret_cast<const char*>(s_bc + nb * kBcSize) +
                                (b_key ^ static_cast<uint32_t>(t4 << 2)))
                          : p_b0 + nb * kBcSize + col;
    const float* pd = p_dd + nb * kWg * kDdSize;
    const f4 b0 = LTI ? f4{b_lti[0], b_lti[0], b_lti[0], b_lti[0]} : lds_f4(pb);
    const f4 b1 = LTI ? f4{b_lti[1], b_lti[1], b_lti[1], b_lti[1]} : lds_f4(pb + kT);
    const f4 dd01 = lds_f4(pd + 2 * t4);
    const f4 dd23 = lds_f4(pd + 2 * t4 + 4);
    const float dls[4] = {dd01.x, dd01.z, dd23.x, dd23.z};
    const float dus[4] = {dd01.y, dd01.w, dd23.y, dd23.w};
    const float bs0[4] = {b0.x, b0.y, b0.z, b0.w};
    const float bs1[4] = {b1.x, b1.y, b1.z, b1.w};
    if constexpr (AGG) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[0] = fmaf(fast_exp2(dls[k] * A2[0]), h[0], dus[k] * bs0[k]);
        h[1] = fmaf(fast_exp2(dls[k] * A2[1]), h[1], dus[k] * bs1[k]);
      }
    } else {
      const float* pc = p_c0 + nb * kBcSize;
      const f4 c0 = LTI ? f4{c_lti[0], c_lti[0], c_lti[0], c_lti[0]} : lds_f4(pc + col);
      const f4 c1 = LTI ? f4{c_lti[1], c_lti[1], c_lti[1], c_lti[1]} : lds_f4(pc + kT + col);
      const float cs0[4] = {c0.x, c0.y, c0.z, c0.w};
      const float cs1[4] = {c1.x, c1.y, c1.z, c1.w};
      float y[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[0] = fmaf(fast_exp2(dls[k] * A2[0]), h[0], dus[k] * bs0[k]);
        h[1] = fmaf(fast_exp2(dls[k] * A2[1]), h[1], dus[k] * bs1[k]);
        y[k] = fmaf(cs1[k], h[1], cs0[k] * h[0]);
      }
      p_y[nb * kWg * kDdSize + 2 * t4] = reduce_groups_half(y[0], y[1], y[2], y[3]);
    }
  };
  // The blocks are unrolled: the swizzled B/C offsets become loop-invariant
  // registers and the other LDS offsets immediates.  In the AGG pass a
  // scheduling barrier keeps each block's LDS reads inside the block (hoisted
  // together, they would hold eight blocks of operands in registers), and the
  // segment's sum of delta is split over the lanes of a channel: lane (g, c)
  // adds the four deltas of block g of every chunk (a lane reads them from
  // s_dd like its scan does), and the eight partial sums meet once, at the
  // segment end (sum_over_groups), instead of every lane adding all 32.
  auto phase_s = [&](int t0, int nb) __attribute__((always_inline)) {
    if constexpr (AGG) {
#pragma unroll 1
      for (int t4 = 0; t4 < kT; t4 += 4) scan_block(t4, t0, nb);
    } else {
#pragma unroll
      for (int t4 = 0; t4 < kT; t4 += 4) scan_block(t4, t0, nb);
    }
    if constexpr (AGG) {
      const float* pg = p_dd + nb * kWg * kDdSize + 8 * sg;
      const f4 d01 = lds_f4(pg), d23 = lds_f4(pg + 4);
      sum_delta += (d01.x + d01.z) + (d23.x + d23.z);
    }
  };

  auto phase_o = [&](const ZBuf& zb, int t0, int nb) __attribute__((always_inline)) {
    if constexpr (!AGG) {
      float y[kPerThread];
      if constexpr (XT) {
        const float* p = s_dd + xa * kDdPitch + 8 * xb;
        const f4 v0 = lds_f4(p), v1 = lds_f4(p + 4);
        const f4 sk = lds_f4(s_skip + xa * kSkipPitch + 4 * xb);
        y[0] = (v0.x + v0.y) + sk.x;
        y[1] = (v0.z + v0.w) + sk.y;
        y[2] = (v1.x + v1.y) + sk.z;
        y[3] = (v1.z + v1.w) + sk.w;
      } else {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          const float2 pair = *reinterpret_cast<const float2*>(e_dd(nb, j));
          y[j] = (pair.x + pair.y) + (COOP ? skr[j] : *e_sk(nb, j));
        }
      }
      if (has_z) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) y[j] *= silu(zb.z[j]);
      }
      const auto rs = rsrc(out, s.so, dx0, t0);
      const uint32_t vo_o = x_voff(s.so);
      if constexpr (VEC) {
        if constexpr (XT) mirror4(y);
        VIO::store(y, rs, x_ok(0, t0, t_end) ? vo_o : kOffNone, 0);
      } else {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          const uint32_t off = x_ok(j, t0, t_end) ? vo_o + x_eoff(s.so, j) : kOffNone;
          VIO::store_one(y[j], rs, off, 0);
        }
      }
    }
  };

  // ---- chunk loop (wave-local: LDS traffic is ordered within the wave) ----
  // One iteration scans chunk c.  Loads are issued in every iteration (past
  // the end they are out-of-range no-ops), so the loop body is branch-free and
  // the compiler counts outstanding loads exactly.  B/C and u/delta_raw of
  // chunk c+1 are issued before the scan of chunk c and z of chunk c+1 once
  // O(c) has consumed z(c); E(c+1) then waits for the loads issued before the
  // scan and O(c+1) for z(c+1), the oldest loads in flight at each point.
  // With several waves per SIMD, the scans of the other waves cover the
  // latency.
  const int nchunks = (t_end - t_begin + kT - 1) / kT;
  InBuf in;
  ZBuf zb;
  issue_bc_loads(t_begin, t_end);
  issue_x_loads(in, t_begin, t_end);
  issue_z_loads(zb, t_begin, t_end);
  phase_e(in, t_begin, 0);
  // Priorities: the SIMD issues from the oldest wave among those of the
  // highest priority.  A wave scans at priority 0 and raises itself to 2 for
  // the output and input phases, so a wave whose scan is done gets to its
  // memory waits and load issue at once instead of queueing behind the scans
  // of older waves: loads leave earlier and have longer to arrive.
  // COOP: chunk c uses LDS buffer nb = c % 2 (the AGG pass: buffer 0).  The
  // first barrier publishes every wave's E(c) before any wave scans c; the
  // second publishes every wave's totals of c before any wave reads them in
  // O(c).  E(c+1) writes the other buffer, whose last readers (S(c-1),
  // O(c-1)) all finished before the first barrier of c; with one buffer
  // (AGG: no O phase) its last readers, S(c), finished before the second.
  auto chunk = [&](int c, int nb) __attribute__((always_inline)) {
    const int t0 = t_begin + c * kT;
    issue_bc_loads(t0 + kT, t_end);
    issue_x_loads(in, t0 + kT, t_end);
    if constexpr (COOP) __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    phase_s(t0, nb);
    __builtin_amdgcn_s_setprio(2);
    if constexpr (COOP) __syncthreads();
    phase_o(zb, t0, nb);
    issue_z_loads(zb, t0 + kT, t_end);
    phase_e(in, t0 + kT, kBufs == 2 ? nb ^ 1 : 0);
  };
  if constexpr (COOP) {
    // Two chunks per iteration, so that the buffer index is a constant in
    // the LDS offsets.  An odd count runs one chunk past the segment: its
    // loads are out of range (zeros), delta is 0 so the state passes through
    // unchanged, and its stores and chunk states are masked by t_end.
    for (int c = 0; c < nchunks; c += 2) {
      chunk(c, 0);
      chunk(c + 1, kBufs == 2 ? 1 : 0);
    }
  } else {
    for (int c = 0; c < nchunks; ++c) chunk(c, 0);
  }

  // ---- segment end ----
  if constexpr (AGG) {
    const float seg_delta = sum_over_groups(sum_delta);
#pragma unroll
    for (int k = 0; k < kStatesPerLane; ++k) {
      const int n = sg * kStatesPerLane + k;
      const float prod_a = fast_exp2(A2[k] * seg_delta);
      if (tile_ok)
        agg[(static_cast<int64_t>(link) * s.nchan_pad + chan_row) * kMaxState + n] =
            make_float2(prod_a, h[k]);
    }
  } else {
    if (final_state != nullptr && seg == s.nseg - 1) {
#pragma unroll
      for (int k = 0; k < kStatesPerLane; ++k) {
        const int n = sg * kStatesPerLane + k;
        if (dvalid && n < s.dstate)
          final_state[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] = h[k];
      }
    }
  }
}

// carry[s] = state entering segment s, from the segment aggregates:
//   carry[0] = h0 (or 0),  carry[s+1] = P[s] * carry[s] + H[s],
// where (P[s], H[s]) composes the agg_split part aggregates of segment s in
// order.  One lane per (channel, state); the chain of nseg - 1 aggregates is
// walked in ranges of at most kCarryBatch segments, one wave each (walk_chain_in_ranges):
// one memory latency per call.  (A 256-channel sequence in 128 segments has
// only 4096 chains, and had walked its 127 aggregates in eight dependent
// batches.)
template <int SPLIT>
__global__ __launch_bounds__(kThreads * kCarryWaves) void carry_kernel(
    ScanShape s, const float2* __restrict__ agg, const float* __restrict__ h0,
    float* __restrict__ carry) {
  __shared__ float2 xch[kCarryWaves][kThreads];
  const int64_t sstride = s.nchan_pad * kMaxState;  // idx = row * kMaxState + n
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x % kThreads;
  const bool valid = idx < sstride;
  const int64_t ic = valid ? idx : 0;
  float c = 0.0f;
  if (valid && h0 != nullptr) {
    const int n = static_cast<int>(idx % kMaxState);
    const int64_t row = idx / kMaxState;
    const int64_t per_b = static_cast<int64_t>(s.groups) * kCh;
    const int b = static_cast<int>(row / per_b);
    const int d = static_cast<int>(row % per_b);
    if (d < s.dim && n < s.dstate) c = h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n];
  }
  // Link k of the chain is segment k: its SPLIT (= agg_split) parts composed
  // in order.  (SPLIT is a template argument: with a runtime count the
  // compiler put each further part's load under a branch and waited for it
  // there, one memory latency per link.)
  walk_chain_in_ranges(
      s.nseg - 1, c, valid, xch,
      [&](int k) {
        const float2* a = agg + static_cast<int64_t>(k) * SPLIT * sstride + ic;
        float2 l = a[0];
#pragma unroll
        for (int j = 1; j < SPLIT; ++j) l = link_then(l, a[j * sstride]);
        return l;
      },
      [&](int k, float v) { carry[(k + 1) * sstride + idx] = v; });
}

template <typename IO, bool XT, bool BT, bool VEC, bool REV, bool LTI>
static void launch_pass(const ScanShape& s, const ScanPtrs& p, const float* h0, float* final_state,
                        hipStream_t stream) {
  constexpr int kWg = kWavesPerWg<XT>;
  const dim3 block(kThreads * kWg);
  const unsigned G = static_cast<unsigned>(s.batch) * static_cast<unsigned>(s.groups);
  // COOP (d-fast vector path): one workgroup per 32-channel block and segment
  auto wgs = [&](int nseg) {
    if constexpr (!XT && VEC)
      return dim3(static_cast<unsigned>(s.batch) *
                  static_cast<unsigned>((s.groups + kWg - 1) / kWg) * static_cast<unsigned>(nseg));
    return dim3((G * static_cast<unsigned>(nseg) + kWg - 1) / kWg);
  };
  const IO* u = static_cast<const IO*>(p.u);
  const IO* dr = static_cast<const IO*>(p.delta_raw);
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* z = static_cast<const IO*>(p.z);
  IO* out = static_cast<IO*>(p.out);
  if (s.nseg > 1) {
    const int links = (s.nseg - 1) * s.agg_split;
    scan_kernel<IO, XT, BT, true, VEC, REV, LTI><<<wgs(links), block, 0, stream>>>(
        s, u, dr, p.A_log, Bm, Cm, p.D, z, p.dt_bias, h0, out, final_state, p.agg, p.carry,
        nullptr);
    const int64_t n = s.nchan_pad * kMaxState;
    const dim3 cgrid(static_cast<unsigned>((n + kThreads - 1) / kThreads));
    const dim3 cblock(kThreads * carry_waves(s.nseg));
    static_assert(kMaxAggSplit == 2, "one carry instantiation per part count");
    if (s.agg_split == 2)
      carry_kernel<2><<<cgrid, cblock, 0, stream>>>(s, p.agg, h0, p.carry);
    else
      carry_kernel<1><<<cgrid, cblock, 0, stream>>>(s, p.agg, h0, p.carry);
  }
  scan_kernel<IO, XT, BT, false, VEC, REV, LTI><<<wgs(s.nseg), block, 0, stream>>>(
      s, u, dr, p.A_log, Bm, Cm, p.D, z, p.dt_bias, h0, out, final_state, p.agg, p.carry,
      p.chunk_states);
}

// The vector pass covers [0, s.t_stop); when s.t_stop < seqlen it exports its
// state to p.tail_h0 and an element-wise pass covers the remaining steps.
// Time-invariant B/C (s.bc_const) take the LTI instantiation on the vector
// pass; the element-wise passes read them through their zero time stride.
template <typename IO, bool XT, bool BT, bool REV>
static hipError_t launch_dir(const ScanShape& s, const ScanPtrs& p, hipStream_t stream) {
  if (!s.use_vec) {
    launch_pass<IO, XT, BT, false, REV, false>(s, p, p.h0, p.final_state, stream);
    return hipGetLastError();
  }
  const bool tail = s.t_stop < s.seqlen;
  float* const vec_final = tail ? p.tail_h0 : p.final_state;
  if (s.t_stop > 0) {
    if (s.bc_const && !BT)
      launch_pass<IO, XT, false, true, REV, true>(s, p, p.h0, vec_final, stream);
    else
      launch_pass<IO, XT, BT, true, REV, false>(s, p, p.h0, vec_final, stream);
  }
  if (tail) {
    ScanShape t = s;
    t.t_first = s.t_stop;
    t.t_stop = s.seqlen;
    t.nseg = 1;
    t.seg_len = s.seqlen - s.t_stop;
    launch_pass<IO, XT, BT, false, REV, false>(t, p, s.t_stop > 0 ? p.tail_h0 : p.h0,
                                               p.final_state, stream);
  }
  return hipGetLastError();
}

template <typename IO, bool XT, bool BT>
static hipError_t launch_scan_t(const ScanShape& s, const ScanPtrs& p, hipStream_t stream) {
  return s.reverse ? launch_dir<IO, XT, BT, true>(s, p, stream)
                   : launch_dir<IO, XT, BT, false>(s, p, stream);
}

hipError_t launch_scan(const ScanShape& s, const ScanPtrs& p, bool io_bf16, bool x_tfast,
                       bool bc_tfast, hipStream_t stream) {
  if (io_bf16) {
    if (x_tfast)
      return bc_tfast ? launch_scan_t<bf16_t, true, true>(s, p, stream)
                      : launch_scan_t<bf16_t, true, false>(s, p, stream);
    return bc_tfast ? launch_scan_t<bf16_t, false, true>(s, p, stream)
                    : launch_scan_t<bf16_t, false, false>(s, p, stream);
  }
  if (x_tfast)
    return bc_tfast ? launch_scan_t<float, true, true>(s, p, stream)
                    : launch_scan_t<float, true, false>(s, p, stream);
  return bc_tfast ? launch_scan_t<float, false, true>(s, p, stream)
                  : launch_scan_t<float, false, false>(s, p, stream);
}

}  // namespace mss
