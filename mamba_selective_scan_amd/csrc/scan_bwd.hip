// scan_bwd.hip -- backward of the selective-scan forward, for gfx950 (wave64).
//
// Given dout (and optionally dfinal, the gradient reaching the exported final
// state) the chain rule through the forward (see scan_fwd.hip), taken step by
// step in reverse time, gives with G_tn the total adjoint of h_tn:
//   dy_t = dout_t silu(z_t)            dz_t = dout_t y_t silu'(z_t)
//   G_tn = g_n + dy_t C_tn             g_n <- G_tn a_tn   (adjoint reaching h_(t-1))
//   dC_tn = sum_d dy_t h_tn            dB_tn = sum_d G_tn delta_t u_t
//   du_t = dy_t D + delta_t sum_n G_tn B_tn
//   ddelta_t = u_t sum_n G_tn B_tn + sum_n G_tn h_(t-1)n a_tn A_n
//   ddelta_raw_t = ddelta_t sigmoid(x_t)  (softplus' = sigmoid)
//   dA_log_n = A_n sum_(b,t) G_tn h_(t-1)n a_tn delta_t
//   dD = sum dy u,  ddt_bias = sum ddelta_raw,  dh0 = g after the first step.
// The training backward is what the pages list as not yet written
// ("mamba-metal: Apple Silicon で Mamba を動かす", section "残り課題").
// Every kernel works in logical time; in reverse time (s.reverse) logical
// step t reads and writes storage step L-1-t.  The aggregate, checkpoint and
// reverse-walk passes take the direction as a template argument (REV ==
// s.reverse), so that the order of the steps inside a loaded vector is fixed
// at compile time rather than chosen per element.
//
// Passes:
//   0. (few channels, long sequences) the sequence is cut into time segments
//      so that the grid fills the GPU.  agg_kernel walks every segment forward
//      from zero and records per (channel, state) the product P of its decays,
//      the state H it reaches and the adjoint Z it sends back to its first
//      step's predecessor, Z = sum_t (prod_(r<=t) a_r) dy_t C_t; carry_kernel
//      composes them, forward for the state entering each segment
//      (h_in[s+1] = P_s h_in[s] + H_s) and backward for the adjoint reaching
//      each segment's end (g_in[s-1] = P_s g_in[s] + Z_s): the pair operator
//      of "mamba-metal", sections "Selective scan の本質" and "チャンク間
//      running prefix", applied in both directions.
//   1. ckpt_kernel: the forward recurrence (no outputs) recording the state
//      entering every kBwdT-step chunk.  One wave per 8 channels, lanes as in
//      the forward: lane (g, c) runs states 2g, 2g+1 of channel c.
//   2. bwd_kernel: a workgroup of kBwdWaves waves owns kBwdCh channels of
//      one batch row and walks the chunks from the last to the first.  Per
//      chunk:
//        E  inputs of the chunk: B and C into LDS (shared by the workgroup),
//           per element delta, delta*u and dy into LDS (per wave);
//        F  the chunk's states recomputed forward from its checkpoint, kept
//           in registers (16 steps x 2 states per lane); C.h summed over the
//           state groups gives y for dz;
//        R  the reverse walk above.  Sums over states (for du and ddelta) go
//           through the same cross-lane tree as the forward's C.h; sums over
//           the wave's 8 channels (for dB and dC) through a DPP tree inside
//           each 8-lane group, then over the workgroup's waves through LDS,
//           into one partial per workgroup and step;
//        O  du and ddelta_raw per element.
//   3. reduce_bc_kernel: dB and dC as sums of the workgroup partials, in a
//      fixed order (deterministic); the same launch's last blocks sum
//      dA_log, dD and ddt_bias over the batch rows and segments.
#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {
namespace {

constexpr int kXcdsBwd = 8;
// LDS row pitches (floats), padded so that the rows one instruction reads
// fall in distinct bank groups.
constexpr int kElPitch = kBwdT * 4 + 4;  // s_el[c][t] = (delta, delta*u, dy, y_ssm)
constexpr int kBcPitch = kBwdT + 4;      // s_bc[r][t]: r < 16 B_r, r >= 16 C_(r-16)
constexpr int kGrPitch = kBwdT * 8 + 4;  // s_gr[c][t] = (u, sigmoid(x), dout, z, d(delta*u), ddelta via a, -, -)
// checkpoint pass, staged in blocks of two chunks
constexpr int kCkSpan = 2 * kBwdT;
constexpr int kCkBPitch = kCkSpan + 4;    // s_b[n][t]
constexpr int kCkDdPitch = kCkSpan * 2 + 4;  // s_dd[c][t] = (delta, delta*u)

struct f4 {
  float x, y, z, w;
};
__device__ inline f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ inline float f4_at(const f4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <typename IO>
__device__ inline float ld(const IO* p) { return io_traits<IO>::load(p); }

__device__ inline float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// Storage step of logical step t: mirrored when the scan runs in reverse time.
__device__ inline int64_t tstore(const BwdShape& s, int t) {
  return s.reverse ? static_cast<int64_t>(s.seqlen) - 1 - t : t;
}

// Buffer descriptor of one chunk tile of a [b][row][t] tensor: based at
// (b, row0) and the chunk's lowest storage step, t0 in forward time and
// L - kBwdT - t0 in reverse time (that base may lie before the tensor; only
// in-range offsets are used).  An absent tensor gets an empty range based at
// `fallback`, so that its loads read 0 and its stores are dropped.
template <int SPAN = kBwdT>
__device__ inline __amdgpu_buffer_rsrc_t chunk_rsrc(const BwdShape& s, const void* ptr,
                                                    const int64_t* st, int64_t es, int b, int row0,
                                                    int t0, bool present, const void* fallback) {
  const int64_t ts = s.reverse ? static_cast<int64_t>(s.seqlen) - SPAN - t0 : t0;
  const char* base = static_cast<const char*>(present ? ptr : fallback) +
                     (present ? (b * st[0] + static_cast<int64_t>(row0) * st[1] + ts * st[2]) * es : 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, present ? kRsrcRange : 0,
                                           kRsrcFlags);
}

// Byte offset of (row, logical step tt of the chunk) inside a chunk tile of
// SPAN steps (loop-invariant; the host checks that tiles span less than
// 2 GiB).
template <int SPAN = kBwdT>
__device__ inline uint32_t chunk_off(const BwdShape& s, const int64_t* st, int64_t es, int row,
                                     int tt) {
  const int tl = s.reverse ? SPAN - 1 - tt : tt;
  return static_cast<uint32_t>((row * st[1] + tl * st[2]) * es);
}

// Cache policy of buffer accesses to data that this pass writes or reads
// exactly once (its gradient outputs, the dB/dC partials, the checkpoints):
// the non-temporal bit, so that these lines leave L2 first and the input lines
// that the next chunk reuses (a 16-step chunk is half of a 128-byte line of
// [B,D,L] data) stay.
constexpr int kStream = 2;

// Two adjacent elements of one row through a buffer descriptor, the one at
// the lower address first (stores are streaming).
template <typename IO>
struct pair_io;
template <>
struct pair_io<float> {
  using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float& lo, float& hi) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    lo = __uint_as_float(v[0]);
    hi = __uint_as_float(v[1]);
  }
  __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float lo, float hi) {
    u32x2 v;
    v[0] = __float_as_uint(lo);
    v[1] = __float_as_uint(hi);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStream);
  }
};
template <>
struct pair_io<bf16_t> {
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float& lo, float& hi) {
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    lo = __uint_as_float(v << 16);
    hi = __uint_as_float(v & 0xffff0000u);
  }
  __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float lo, float hi) {
    __builtin_amdgcn_raw_buffer_store_b32(bf16x2_bits(lo, hi), r, off, 0, kStream);
  }
};

// One element, streaming (stores of once-written outputs, loads of
// once-read checkpoints).
template <typename IO>
__device__ inline void store_stream(float y, __amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ inline void store_stream<float>(float y, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), r, off, 0, kStream);
}
template <>
__device__ inline void store_stream<bf16_t>(float y, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(y), r, off, 0, kStream);
}
__device__ inline float load_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStream));
}

// A tensor's row (b, row0) as the loop keeps it: its base address and the
// bytes per time step (32-bit: tiles span less than 2 GiB), three scalar
// registers; each chunk's descriptor is built from them with one multiply-add.
struct RowBase {
  const char* row;
  int32_t step;
};
__device__ inline RowBase row_base(const void* ptr, const int64_t* st, int64_t es, int b, int row0,
                                   bool present, const void* fallback) {
  if (!present) return RowBase{static_cast<const char*>(fallback), 0};
  return RowBase{static_cast<const char*>(ptr) + (b * st[0] + static_cast<int64_t>(row0) * st[1]) * es,
                 static_cast<int32_t>(st[2] * es)};
}
// Descriptor of the chunk whose lowest storage step is ts (an absent tensor:
// empty range).
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const RowBase& r, int64_t ts, bool present) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(r.row + ts * r.step), 0,
                                           present ? kRsrcRange : 0, kRsrcFlags);
}

// Four adjacent elements of one row, the one at the lower address first.
template <typename IO>
struct quad_io;
template <>
struct quad_io<float> {
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[4]) {
    using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
  }
};
template <>
struct quad_io<bf16_t> {
  __device__ static inline void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[4]) {
    using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
  }
};

__device__ inline void store2(float a, float b, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
  u32x2 v;
  v[0] = __float_as_uint(a);
  v[1] = __float_as_uint(b);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ inline int64_t xcd_order(int64_t lin, int64_t nwg) {
  const int64_t xcd = lin % kXcdsBwd;
  const int64_t per = nwg / kXcdsBwd, extra = nwg % kXcdsBwd;
  return xcd * per + (xcd < extra ? xcd : extra) + lin / kXcdsBwd;
}

// Sum over the 8 lanes of a half row (the 8 channels of one state group) of
// one state's per-lane terms, for a pair of states held in a lane-dependent
// order: lanes 0-3 of the half hold (keep, give) = (state 2g, state 2g+1),
// lanes 4-7 hold (state 2g+1, state 2g).  The first level adds each lane's
// keep term to its mirror partner's give term (row_half_mirror pairs i with
// 7 - i, which holds the same state in its give slot), so one DPP add
// reduces both states at once; two quad permutations finish the sum.  Lanes
// 0-3 end with state 2g's total, lanes 4-7 with state 2g+1's.
__device__ inline float sum_pair_half_rows(float keep, float give) {
  float v = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0x141, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  return v;
}

// The reduce_groups tree leaves step {0, 2, 1, 3}[row] of a 4-step block in
// 16-lane row `row`.
__device__ inline int group_step(int lane) {
  const int row = lane >> 4;
  return row == 1 ? 2 : (row == 2 ? 1 : row);
}

// ---------------------------------------------------------------- pass 0 ---
// Segment aggregates, walking each part of a segment (s.agg_split parts of
// ceil(seg_chunks / agg_split) chunks; trailing parts may be empty) forward
// from zero: per state P = prod a_t, H = the state reached,
// Z = sum_t (prod_(r<=t) a_r) dy_t C_t.
// WITH_H: also the forward aggregate H, which only the checkpoint pass
// needs (forward chunk states given: no checkpoint pass, H is skipped).
// XM: how u, delta_raw, dout, z are read: kXScalar element by element,
// kXStepPairs as pairs of adjacent steps (s.pairs); channel-last data takes
// agg_coop_kernel.  BM: B and C element by element (kBScalar), as 4-step
// vectors (kBStepQuads, s.bcquads) or as 4-state vectors (kBStateQuads,
// s.nquads).
enum { kXScalar = 0, kXStepPairs = 1 };
enum { kBScalar = 0, kBStepQuads = 1, kBStateQuads = 2 };
template <typename IO, bool WITH_H, int XM, int BM, bool REV>
__global__ __launch_bounds__(64) void agg_kernel(BwdShape s, BwdPtrs p) {
  __shared__ __attribute__((aligned(16))) float s_bc[2 * kMaxState * kBcPitch];
  __shared__ __attribute__((aligned(16))) float s_el[kCh * kElPitch];
  const int lane = threadIdx.x;
  const int64_t groups8 = static_cast<int64_t>(s.tiles) * kBwdWaves;
  const int64_t logical = xcd_order(blockIdx.x, gridDim.x);
  const int64_t row_part = logical / groups8;
  const int nparts = s.nseg * s.agg_split;
  const int b = static_cast<int>(row_part / nparts);
  const int part = static_cast<int>(row_part % nparts);
  const int dg = static_cast<int>(logical % groups8) * kCh;
  const int sg = lane >> 3, sc = lane & 7;
  const int d = dg + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.tiles * kBwdCh + d;
  const bool has_z = p.z != nullptr;
  float A2[2], H[2] = {0.0f, 0.0f}, P[2] = {1.0f, 1.0f}, Z[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = 2 * sg + k;
    A2[k] = (dvalid && n < s.dstate) ? -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e : 0.0f;
  }
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* u = static_cast<const IO*>(p.u);
  const IO* dr = static_cast<const IO*>(p.delta_raw);
  const IO* zz = static_cast<const IO*>(p.z);
  const IO* dout = static_cast<const IO*>(p.dout);
  const int part_chunks = (s.seg_chunks + s.agg_split - 1) / s.agg_split;
  const int seg_begin = part / s.agg_split * s.seg_chunks;
  const int seg_end = min(s.nchunk, seg_begin + s.seg_chunks);
  const int q_begin = min(seg_end, seg_begin + part % s.agg_split * part_chunks);
  const int q_end = min(seg_end, q_begin + part_chunks);
  constexpr int64_t es = sizeof(IO);
  // Raw inputs go through buffer descriptors with loop-invariant offsets
  // (out-of-range ones read 0), one chunk ahead of use.  B and C: lane
  // covers rows lane / 4 and 16 + lane / 4 at steps 4 (lane % 4) .. + 3, or
  // (kBStateQuads) states 4 (lane % 4) .. + 3 of step lane / 4.  u,
  // delta_raw, dout, z: lane (c, j) covers steps 2j, 2j+1 of channel c.
  const int bn = BM == kBStateQuads ? (lane & 3) * 4 : lane >> 2;  // first state
  const int bt0 = BM == kBStateQuads ? lane >> 2 : (lane & 3) * 4;  // first step
  uint32_t o_b[4], o_c[4], o_u[2], o_dr[2], o_do[2], o_z[2];
  // (the vector and pair forms use slot 0 only: the lower address, which
  // holds a step vector's first step in forward time and its last in reverse
  // time)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = BM == kBStepQuads ? bt0 + (REV ? 3 : 0) : (BM == kBStateQuads ? bt0 : bt0 + i);
    o_b[i] = chunk_off(s, s.sB, es, bn, tt);
    o_c[i] = chunk_off(s, s.sC, es, bn, tt);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int tt = XM == kXStepPairs ? 2 * sg + (REV ? 1 : 0) : 2 * sg + e;
    o_u[e] = chunk_off(s, s.su, es, sc, tt);
    o_dr[e] = chunk_off(s, s.sd, es, sc, tt);
    o_do[e] = chunk_off(s, s.sdo, es, sc, tt);
    o_z[e] = chunk_off(s, s.sz, es, sc, tt);
  }
  const float bias = (dvalid && p.dt_bias != nullptr) ? p.dt_bias[d] : 0.0f;
  float rb[4], rc[4], ru[2], rx[2], rgo[2], rz[2];
  auto load_chunk = [&](int q) __attribute__((always_inline)) {
    const int t0 = q * kBwdT;
    const bool qin = q < q_end;
    const auto rs_b = chunk_rsrc(s, Bm, s.sB, es, b, 0, t0, true, Bm);
    const auto rs_c = chunk_rsrc(s, Cm, s.sC, es, b, 0, t0, true, Cm);
    if constexpr (BM == kBStepQuads) {
      // length a multiple of 4: a vector is wholly inside or past the sequence
      const bool ok = qin && bn < s.dstate && t0 + bt0 < s.seqlen;
      float vb[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vc[4];
      if constexpr (WITH_H) quad_io<IO>::load(rs_b, ok ? o_b[0] : kOffNone, vb);
      quad_io<IO>::load(rs_c, ok ? o_c[0] : kOffNone, vc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rb[i] = REV ? vb[3 - i] : vb[i];
        rc[i] = REV ? vc[3 - i] : vc[i];
      }
    } else if constexpr (BM == kBStateQuads) {
      // dstate a multiple of 4: a vector is wholly inside or past the states
      const bool ok = qin && bn < s.dstate && t0 + bt0 < s.seqlen;
      float vb[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vc[4];
      if constexpr (WITH_H) quad_io<IO>::load(rs_b, ok ? o_b[0] : kOffNone, vb);
      quad_io<IO>::load(rs_c, ok ? o_c[0] : kOffNone, vc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rb[i] = vb[i];
        rc[i] = vc[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = qin && bn < s.dstate && t0 + bt0 + i < s.seqlen;
        rb[i] = WITH_H ? buf_one<IO>::load(rs_b, ok ? o_b[i] : kOffNone, 0) : 0.0f;
        rc[i] = buf_one<IO>::load(rs_c, ok ? o_c[i] : kOffNone, 0);
      }
    }
    const auto rs_u = chunk_rsrc(s, u, s.su, es, b, dg, t0, true, u);
    const auto rs_dr = chunk_rsrc(s, dr, s.sd, es, b, dg, t0, true, u);
    const auto rs_do = chunk_rsrc(s, dout, s.sdo, es, b, dg, t0, true, u);
    const auto rs_z = chunk_rsrc(s, zz, s.sz, es, b, dg, t0, has_z, u);
    if constexpr (XM == kXStepPairs) {
      // even length: a pair is wholly inside or past the sequence
      const bool ok = qin && dvalid && t0 + 2 * sg < s.seqlen;
      auto pair = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[2]) {
        float lo, hi;
        pair_io<IO>::load(r, ok ? off : kOffNone, lo, hi);
        v[0] = REV ? hi : lo;
        v[1] = REV ? lo : hi;
      };
      pair(rs_u, o_u[0], ru);
      pair(rs_dr, o_dr[0], rx);
      pair(rs_do, o_do[0], rgo);
      pair(rs_z, o_z[0], rz);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = qin && dvalid && t0 + 2 * sg + e < s.seqlen;
        ru[e] = buf_one<IO>::load(rs_u, ok ? o_u[e] : kOffNone, 0);
        rx[e] = buf_one<IO>::load(rs_dr, ok ? o_dr[e] : kOffNone, 0);
        rgo[e] = buf_one<IO>::load(rs_do, ok ? o_do[e] : kOffNone, 0);
        rz[e] = buf_one<IO>::load(rs_z, ok ? o_z[e] : kOffNone, 0);
      }
    }
  };
  load_chunk(q_begin);
  for (int q = q_begin; q < q_end; ++q) {
    const int t0 = q * kBwdT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = BM == kBStateQuads ? bn + i : bn;
      const int t = BM == kBStateQuads ? bt0 : bt0 + i;
      s_bc[r * kBcPitch + t] = rb[i];
      s_bc[(kMaxState + r) * kBcPitch + t] = rc[i];
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tt = 2 * sg + e;
      const bool ok = dvalid && t0 + tt < s.seqlen;
      const float x = rx[e] + bias;
      const float dl = ok ? (s.softplus ? softplus(x) : x) : 0.0f;
      const float dy = has_z ? rgo[e] * silu(rz[e]) : rgo[e];
      *reinterpret_cast<f4*>(s_el + sc * kElPitch + 4 * tt) = f4{dl, dl * ru[e], dy, 0.0f};
    }
    load_chunk(q + 1);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t4 = 0; t4 < kBwdT; t4 += 4) {
      const f4 b0 = ld4(s_bc + (2 * sg) * kBcPitch + t4);
      const f4 b1 = ld4(s_bc + (2 * sg + 1) * kBcPitch + t4);
      const f4 c0 = ld4(s_bc + (kMaxState + 2 * sg) * kBcPitch + t4);
      const f4 c1 = ld4(s_bc + (kMaxState + 2 * sg + 1) * kBcPitch + t4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f4 dd = ld4(s_el + sc * kElPitch + 4 * (t4 + i));
        const float bk[2] = {f4_at(b0, i), f4_at(b1, i)};
        const float ck[2] = {f4_at(c0, i), f4_at(c1, i)};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float a = fast_exp2(dd.x * A2[k]);
          if constexpr (WITH_H) H[k] = fmaf(a, H[k], dd.y * bk[k]);
          P[k] *= a;
          Z[k] = fmaf(P[k], dd.z * ck[k], Z[k]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
    p.agg[(static_cast<int64_t>(part) * s.nchan_pad + chan_row) * kMaxState + 2 * sg + k] =
        make_float4(P[k], H[k], Z[k], 0.0f);
}

// The aggregate pass for channel-last u, delta_raw, dout, z (s.dpairs): one
// workgroup of kBwdWaves waves per (row, segment part, 32-channel tile),
// with the scan roles of agg_kernel in each wave.  The workgroup loads the
// tile's inputs together: thread (t, j) = (tid / 16, tid % 16) reads
// channels 2j, 2j+1 of step t of each tensor, so that 16 threads cover one
// 128-byte row of 32 channels, and B and C once for the tile (thread
// (t, n) = (tid / 16, tid % 16)).  The inputs are staged in LDS,
// double-buffered by chunk parity, so that one barrier per chunk orders every
// shared access.  (One wave per 8 channels read a quarter of each row, and
// the four waves that share a row ran in workgroups on different CUs.)
template <typename IO, bool WITH_H>
__global__ __launch_bounds__(kBwdThreads) void agg_coop_kernel(BwdShape s, BwdPtrs p) {
  __shared__ __attribute__((aligned(16))) float s_bc[2][2 * kMaxState * kBcPitch];
  __shared__ __attribute__((aligned(16))) float s_el[2][kBwdCh * kElPitch];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int64_t logical = xcd_order(blockIdx.x, gridDim.x);
  const int tile = static_cast<int>(logical % s.tiles);
  const int64_t row_part = logical / s.tiles;
  const int nparts = s.nseg * s.agg_split;
  const int b = static_cast<int>(row_part / nparts);
  const int part = static_cast<int>(row_part % nparts);
  // scan role: lane (c, g) of wave w, states 2g, 2g+1 of channel 8w + c of the tile
  const int sg = lane >> 3, sc = lane & 7;
  const int d0 = tile * kBwdCh;
  const int d = d0 + w * kCh + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.tiles * kBwdCh + d;
  const bool has_z = p.z != nullptr;
  float A2[2], H[2] = {0.0f, 0.0f}, P[2] = {1.0f, 1.0f}, Z[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = 2 * sg + k;
    A2[k] = (dvalid && n < s.dstate) ? -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e : 0.0f;
  }
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* u = static_cast<const IO*>(p.u);
  const IO* dr = static_cast<const IO*>(p.delta_raw);
  const IO* zz = static_cast<const IO*>(p.z);
  const IO* dout = static_cast<const IO*>(p.dout);
  const int part_chunks = (s.seg_chunks + s.agg_split - 1) / s.agg_split;
  const int seg_begin = part / s.agg_split * s.seg_chunks;
  const int seg_end = min(s.nchunk, seg_begin + s.seg_chunks);
  const int q_begin = min(seg_end, seg_begin + part % s.agg_split * part_chunks);
  const int q_end = min(seg_end, q_begin + part_chunks);
  constexpr int64_t es = sizeof(IO);
  // load role: step lt of the chunk, channels lc, lc + 1 of the tile, state ln
  const int lt = tid >> 4, lc = 2 * (tid & 15), ln = tid & 15;
  const bool xv = d0 + lc < s.dim;  // dim is even: the pair is wholly in or out
  const uint32_t o_u = chunk_off(s, s.su, es, lc, lt);
  const uint32_t o_dr = chunk_off(s, s.sd, es, lc, lt);
  const uint32_t o_do = chunk_off(s, s.sdo, es, lc, lt);
  const uint32_t o_z = chunk_off(s, s.sz, es, lc, lt);
  const uint32_t o_b = chunk_off(s, s.sB, es, ln, lt);
  const uint32_t o_c = chunk_off(s, s.sC, es, ln, lt);
  float bias[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) bias[e] = (xv && p.dt_bias != nullptr) ? p.dt_bias[d0 + lc + e] : 0.0f;
  float ru[2], rx[2], rgo[2], rz[2], rb = 0.0f, rc = 0.0f;
  auto load_chunk = [&](int q) __attribute__((always_inline)) {
    const int t0 = q * kBwdT;
    const bool tin = q < q_end && t0 + lt < s.seqlen;
    const bool ok = tin && xv;
    pair_io<IO>::load(chunk_rsrc(s, u, s.su, es, b, d0, t0, true, u), ok ? o_u : kOffNone, ru[0], ru[1]);
    pair_io<IO>::load(chunk_rsrc(s, dr, s.sd, es, b, d0, t0, true, u), ok ? o_dr : kOffNone, rx[0],
                      rx[1]);
    pair_io<IO>::load(chunk_rsrc(s, dout, s.sdo, es, b, d0, t0, true, u), ok ? o_do : kOffNone,
                      rgo[0], rgo[1]);
    pair_io<IO>::load(chunk_rsrc(s, zz, s.sz, es, b, d0, t0, has_z, u), ok ? o_z : kOffNone, rz[0],
                      rz[1]);
    const bool bok = tin && ln < s.dstate;
    if constexpr (WITH_H)
      rb = buf_one<IO>::load(chunk_rsrc(s, Bm, s.sB, es, b, 0, t0, true, Bm), bok ? o_b : kOffNone, 0);
    rc = buf_one<IO>::load(chunk_rsrc(s, Cm, s.sC, es, b, 0, t0, true, Cm), bok ? o_c : kOffNone, 0);
  };
  load_chunk(q_begin);
  for (int q = q_begin; q < q_end; ++q) {
    const int t0 = q * kBwdT;
    float* bc = s_bc[(q - q_begin) & 1];
    float* el = s_el[(q - q_begin) & 1];
    bc[ln * kBcPitch + lt] = rb;
    bc[(kMaxState + ln) * kBcPitch + lt] = rc;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool ok = xv && t0 + lt < s.seqlen;
      const float x = rx[e] + bias[e];
      const float dl = ok ? (s.softplus ? softplus(x) : x) : 0.0f;
      const float dy = has_z ? rgo[e] * silu(rz[e]) : rgo[e];
      *reinterpret_cast<f4*>(el + (lc + e) * kElPitch + 4 * lt) = f4{dl, dl * ru[e], dy, 0.0f};
    }
    load_chunk(q + 1);
    __syncthreads();
    const float* wel = el + w * kCh * kElPitch;
#pragma unroll
    for (int t4 = 0; t4 < kBwdT; t4 += 4) {
      const f4 b0 = ld4(bc + (2 * sg) * kBcPitch + t4);
      const f4 b1 = ld4(bc + (2 * sg + 1) * kBcPitch + t4);
      const f4 c0 = ld4(bc + (kMaxState + 2 * sg) * kBcPitch + t4);
      const f4 c1 = ld4(bc + (kMaxState + 2 * sg + 1) * kBcPitch + t4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f4 dd = ld4(wel + sc * kElPitch + 4 * (t4 + i));
        const float bk[2] = {f4_at(b0, i), f4_at(b1, i)};
        const float ck[2] = {f4_at(c0, i), f4_at(c1, i)};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float a = fast_exp2(dd.x * A2[k]);
          if constexpr (WITH_H) H[k] = fmaf(a, H[k], dd.y * bk[k]);
          P[k] *= a;
          Z[k] = fmaf(P[k], dd.z * ck[k], Z[k]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
    p.agg[(static_cast<int64_t>(part) * s.nchan_pad + chan_row) * kMaxState + 2 * sg + k] =
        make_float4(P[k], H[k], Z[k], 0.0f);
}

// State entering each segment (forward) and adjoint reaching each segment's
// last state (backward), one lane per (padded channel row, state).  Each
// chain runs over the segment parts of the aggregate pass and is walked in
// ranges, one wave each (walk_chain_in_ranges); the values at segment
// boundaries are kept.
template <bool SPLIT>  // s.agg_split > 1
__global__ __launch_bounds__(64 * kCarryWaves) void carry_bwd_kernel(BwdShape s, BwdPtrs p) {
  __shared__ float2 xch[kCarryWaves][64];
  const int64_t sstride = s.nchan_pad * kMaxState;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x % 64;
  const bool valid = idx < sstride;
  const int64_t ic = valid ? idx : 0;
  const int n = static_cast<int>(ic % kMaxState);
  const int64_t row = ic / kMaxState;
  const int64_t per_b = static_cast<int64_t>(s.tiles) * kBwdCh;
  const int b = static_cast<int>(row / per_b);
  const int d = static_cast<int>(row % per_b);
  const bool active = valid && d < s.dim && n < s.dstate;
  const int64_t ch = (static_cast<int64_t>(b) * s.dim + d) * s.dstate + n;
  const int ks = SPLIT ? s.agg_split : 1;  // a power of two: boundaries by mask and shift
  const int ks_log2 = SPLIT ? __builtin_ctz(static_cast<unsigned>(ks)) : 0;
  const int nparts = s.nseg * ks;
  // the state entering each part, forward over the parts: link k is part k
  const float h = (active && p.h0 != nullptr) ? p.h0[ch] : 0.0f;
  if (valid) p.carry_h[idx] = h;
  walk_chain_in_ranges(
      nparts - 1, h, valid, xch,
      [&](int k) {
        const float4 v = p.agg[k * sstride + ic];
        return make_float2(v.x, v.y);
      },
      [&](int k, float c) {  // c enters part k + 1
        if (!SPLIT || ((k + 1) & (ks - 1)) == 0)
          p.carry_h[((k + 1) >> ks_log2) * sstride + idx] = c;
      });
  __syncthreads();  // xch is used again
  // the adjoint reaching each part's end, backward over the parts: link k is
  // part nparts - 1 - k
  const float g = (active && p.dfinal != nullptr) ? p.dfinal[ch] : 0.0f;
  if (valid) p.carry_g[(s.nseg - 1) * sstride + idx] = g;
  walk_chain_in_ranges(
      nparts - 1, g, valid, xch,
      [&](int k) {
        const float4 v = p.agg[(nparts - 1 - k) * sstride + ic];
        return make_float2(v.x, v.z);
      },
      [&](int k, float c) {  // c reaches the end of part nparts - 2 - k
        const int q = nparts - 2 - k;
        if (!SPLIT || (q & (ks - 1)) == ks - 1) p.carry_g[(q >> ks_log2) * sstride + idx] = c;
      });
}

// ---------------------------------------------------------------- pass 1 ---
// QUAD: u and delta_raw are read as 4-step vectors (s.quads); BQUAD: B as
// well (s.bquads).
template <typename IO, bool QUAD, bool BQUAD, bool REV>
__global__ __launch_bounds__(64) void ckpt_kernel(BwdShape s, BwdPtrs p) {
  __shared__ __attribute__((aligned(16))) float s_b[kMaxState * kCkBPitch];
  __shared__ __attribute__((aligned(16))) float s_dd[kCh * kCkDdPitch];
  const int lane = threadIdx.x;
  const int64_t groups8 = static_cast<int64_t>(s.tiles) * kBwdWaves;  // 8-channel groups per row
  const int64_t logical = xcd_order(blockIdx.x, gridDim.x);
  const int64_t row_seg = logical / groups8;
  const int b = static_cast<int>(row_seg / s.nseg);
  const int seg = static_cast<int>(row_seg % s.nseg);
  const int dg = static_cast<int>(logical % groups8) * kCh;  // first channel of the wave
  const int sg = lane >> 3, sc = lane & 7;
  const int d = dg + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.tiles * kBwdCh + d;
  float A2[2], h[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = 2 * sg + k;
    const bool active = dvalid && n < s.dstate;
    A2[k] = active ? -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e : 0.0f;
    if (s.nseg > 1)
      h[k] = p.carry_h[(static_cast<int64_t>(seg) * s.nchan_pad + chan_row) * kMaxState + n];
    else
      h[k] = (active && p.h0 != nullptr) ? p.h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] : 0.0f;
  }
  const int q_begin = seg * s.seg_chunks;
  const int q_end = min(s.nchunk, q_begin + s.seg_chunks);
  const float bias = (dvalid && p.dt_bias != nullptr) ? p.dt_bias[d] : 0.0f;
  // The inputs are staged in blocks of two chunks (32 steps), so that a
  // wave's loads cover whole 128-byte rows of [B, D, L] data: B (lane covers
  // row lane / 4, steps 8 (lane % 4) .. + 7) and u, delta_raw (lane (c, j)
  // covers steps 4j .. 4j+3 of channel c, one vector when QUAD).  Loads go
  // through buffer descriptors (chunk_rsrc) with loop-invariant lane offsets
  // and are issued one block ahead of use.
  constexpr int64_t es = sizeof(IO);
  const int bn = lane >> 2;
  uint32_t o_b[8], o_u[4], o_dr[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // BQUAD: slots 0 and 4 hold the two vectors' lower addresses (steps
    // 8k and 8k+4 forward, 8k+3 and 8k+7 reversed)
    const int tt = BQUAD ? (lane & 3) * 8 + (i & 4) + (REV ? 3 : 0) : (lane & 3) * 8 + i;
    o_b[i] = bn < s.dstate ? chunk_off<kCkSpan>(s, s.sB, es, bn, tt) : kOffNone;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // QUAD: slot 0 holds the vector's lower address: step 4j forward, 4j+3 reversed
    const int tt = QUAD ? 4 * sg + (REV ? 3 : 0) : 4 * sg + e;
    o_u[e] = dvalid ? chunk_off<kCkSpan>(s, s.su, es, sc, tt) : kOffNone;
    o_dr[e] = dvalid ? chunk_off<kCkSpan>(s, s.sd, es, sc, tt) : kOffNone;
  }
  // checkpoints in the chunk-state layout [q][batch][dim][kMaxState]
  const uint32_t o_ck =
      dvalid ? static_cast<uint32_t>((sc * kMaxState + 2 * sg) * sizeof(float)) : kOffNone;
  const int64_t ck_row0 = static_cast<int64_t>(b) * s.dim + dg;  // wave-uniform
  const int64_t ck_plane = static_cast<int64_t>(s.batch) * s.dim;
  float rb[8], ru[4], rx[4];
  auto load_block = [&](int q) __attribute__((always_inline)) {
    const int t0 = q * kBwdT;
    const bool qok = q < q_end;
    const auto r_b = chunk_rsrc<kCkSpan>(s, p.B, s.sB, es, b, 0, t0, true, p.u);
    const auto r_u = chunk_rsrc<kCkSpan>(s, p.u, s.su, es, b, dg, t0, true, p.u);
    const auto r_dr = chunk_rsrc<kCkSpan>(s, p.delta_raw, s.sd, es, b, dg, t0, true, p.u);
    if constexpr (BQUAD) {
      // length a multiple of 4: a vector is wholly inside or past the sequence
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        float vb[4];
        const bool ok = qok && t0 + (lane & 3) * 8 + 4 * v < s.seqlen;
        quad_io<IO>::load(r_b, ok ? o_b[4 * v] : kOffNone, vb);
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[4 * v + e] = REV ? vb[3 - e] : vb[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rb[i] = buf_one<IO>::load(r_b, (qok && t0 + (lane & 3) * 8 + i < s.seqlen) ? o_b[i] : kOffNone, 0);
    }
    if constexpr (QUAD) {
      // length a multiple of 4: a vector is wholly inside or past the sequence
      const bool ok = qok && t0 + 4 * sg < s.seqlen;
      float vu[4], vx[4];
      quad_io<IO>::load(r_u, ok ? o_u[0] : kOffNone, vu);
      quad_io<IO>::load(r_dr, ok ? o_dr[0] : kOffNone, vx);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ru[e] = REV ? vu[3 - e] : vu[e];
        rx[e] = REV ? vx[3 - e] : vx[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = qok && t0 + 4 * sg + e < s.seqlen;
        ru[e] = buf_one<IO>::load(r_u, ok ? o_u[e] : kOffNone, 0);
        rx[e] = buf_one<IO>::load(r_dr, ok ? o_dr[e] : kOffNone, 0);
      }
    }
  };
  // Walk the 16 steps of chunk q from LDS step c0 of the block, recording the
  // state entering it.
  auto walk_chunk = [&](int q, int c0) __attribute__((always_inline)) {
    store2(h[0], h[1],
           __builtin_amdgcn_make_buffer_rsrc(
               p.ckpt + (static_cast<int64_t>(q) * ck_plane + ck_row0) * kMaxState, 0,
               kRsrcRange, kRsrcFlags),
           o_ck);
#pragma unroll
    for (int t4 = 0; t4 < kBwdT; t4 += 4) {
      const f4 b0 = ld4(s_b + (2 * sg) * kCkBPitch + c0 + t4);
      const f4 b1 = ld4(s_b + (2 * sg + 1) * kCkBPitch + c0 + t4);
      const f4 dd01 = ld4(s_dd + sc * kCkDdPitch + 2 * (c0 + t4));
      const f4 dd23 = ld4(s_dd + sc * kCkDdPitch + 2 * (c0 + t4) + 4);
      const float dl[4] = {dd01.x, dd01.z, dd23.x, dd23.z};
      const float du[4] = {dd01.y, dd01.w, dd23.y, dd23.w};
      // the block's decays and inputs first, then the two dependent chains
      float a0[4], a1[4], x0[4], x1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a0[i] = fast_exp2(dl[i] * A2[0]);
        a1[i] = fast_exp2(dl[i] * A2[1]);
        x0[i] = du[i] * f4_at(b0, i);
        x1[i] = du[i] * f4_at(b1, i);
      }
      asm volatile("" : "+v"(a0[0]), "+v"(a0[1]), "+v"(a0[2]), "+v"(a0[3]),
                        "+v"(a1[0]), "+v"(a1[1]), "+v"(a1[2]), "+v"(a1[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[0] = fmaf(a0[i], h[0], x0[i]);
        h[1] = fmaf(a1[i], h[1], x1[i]);
      }
    }
  };
  load_block(q_begin);
  for (int q = q_begin; q < q_end; q += 2) {
    const int t0 = q * kBwdT;
#pragma unroll
    for (int i = 0; i < 8; ++i) s_b[bn * kCkBPitch + (lane & 3) * 8 + i] = rb[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = 4 * sg + e, t = t0 + tt;
      const bool ok = dvalid && t < s.seqlen;
      const float x = rx[e] + bias;
      const float sp = s.softplus ? softplus(x) : x;
      const float dl = ok ? sp : 0.0f;
      *reinterpret_cast<float2*>(s_dd + sc * kCkDdPitch + 2 * tt) = make_float2(dl, dl * ru[e]);
    }
    load_block(q + 2);
    __builtin_amdgcn_wave_barrier();
    walk_chunk(q, 0);
    if (q + 1 < q_end) walk_chunk(q + 1, kBwdT);
    __builtin_amdgcn_wave_barrier();
  }
}

// The checkpoint pass for channel-last data (s.dpairs): one workgroup of
// kBwdWaves waves per (row, segment, 32-channel tile), each wave walking its
// 8 channels as in ckpt_kernel.  The workgroup loads a block of two chunks
// together: thread (t, j) = (tid / 16, tid % 16) reads channels 2j, 2j+1 of
// steps t and t + 16 of u and delta_raw (16 threads per 128-byte row of 32
// channels), and B at states tid % 16 of the same steps.  The block is staged
// in LDS, double-buffered by block parity, one barrier per block.
template <typename IO>
__global__ __launch_bounds__(kBwdThreads) void ckpt_coop_kernel(BwdShape s, BwdPtrs p) {
  __shared__ __attribute__((aligned(16))) float s_b[2][kMaxState * kCkBPitch];
  __shared__ __attribute__((aligned(16))) float s_dd[2][kBwdCh * kCkDdPitch];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int64_t logical = xcd_order(blockIdx.x, gridDim.x);
  const int tile = static_cast<int>(logical % s.tiles);
  const int64_t row_seg = logical / s.tiles;
  const int b = static_cast<int>(row_seg / s.nseg);
  const int seg = static_cast<int>(row_seg % s.nseg);
  // walk role: lane (c, g) of wave w, states 2g, 2g+1 of channel 8w + c of the tile
  const int sg = lane >> 3, sc = lane & 7;
  const int d0 = tile * kBwdCh;
  const int dg = d0 + w * kCh;
  const int d = dg + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.tiles * kBwdCh + d;
  float A2[2], h[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = 2 * sg + k;
    const bool active = dvalid && n < s.dstate;
    A2[k] = active ? -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e : 0.0f;
    if (s.nseg > 1)
      h[k] = p.carry_h[(static_cast<int64_t>(seg) * s.nchan_pad + chan_row) * kMaxState + n];
    else
      h[k] = (active && p.h0 != nullptr) ? p.h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] : 0.0f;
  }
  const int q_begin = seg * s.seg_chunks;
  const int q_end = min(s.nchunk, q_begin + s.seg_chunks);
  constexpr int64_t es = sizeof(IO);
  // load role: steps lt, lt + 16 of the block, channels lc, lc + 1, state ln
  const int lt = tid >> 4, lc = 2 * (tid & 15), ln = tid & 15;
  const bool xv = d0 + lc < s.dim;  // dim is even: the pair is wholly in or out
  uint32_t o_u[2], o_dr[2], o_b[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    o_u[v] = chunk_off<kCkSpan>(s, s.su, es, lc, lt + 16 * v);
    o_dr[v] = chunk_off<kCkSpan>(s, s.sd, es, lc, lt + 16 * v);
    o_b[v] = chunk_off<kCkSpan>(s, s.sB, es, ln, lt + 16 * v);
  }
  float bias[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) bias[e] = (xv && p.dt_bias != nullptr) ? p.dt_bias[d0 + lc + e] : 0.0f;
  // checkpoints in the chunk-state layout [q][batch][dim][kMaxState]
  const uint32_t o_ck =
      dvalid ? static_cast<uint32_t>((sc * kMaxState + 2 * sg) * sizeof(float)) : kOffNone;
  const int64_t ck_row0 = static_cast<int64_t>(b) * s.dim + dg;  // wave-uniform
  const int64_t ck_plane = static_cast<int64_t>(s.batch) * s.dim;
  float ru[2][2], rx[2][2], rb[2];
  auto load_block = [&](int q) __attribute__((always_inline)) {
    const int t0 = q * kBwdT;
    const auto r_b = chunk_rsrc<kCkSpan>(s, p.B, s.sB, es, b, 0, t0, true, p.u);
    const auto r_u = chunk_rsrc<kCkSpan>(s, p.u, s.su, es, b, d0, t0, true, p.u);
    const auto r_dr = chunk_rsrc<kCkSpan>(s, p.delta_raw, s.sd, es, b, d0, t0, true, p.u);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const bool tin = q < q_end && t0 + lt + 16 * v < s.seqlen;
      pair_io<IO>::load(r_u, (tin && xv) ? o_u[v] : kOffNone, ru[v][0], ru[v][1]);
      pair_io<IO>::load(r_dr, (tin && xv) ? o_dr[v] : kOffNone, rx[v][0], rx[v][1]);
      rb[v] = buf_one<IO>::load(r_b, (tin && ln < s.dstate) ? o_b[v] : kOffNone, 0);
    }
  };
  // Walk the 16 steps of chunk q from LDS step c0 of the block, recording the
  // state entering it.
  auto walk_chunk = [&](const float* sb, const float* sdd, int q, int c0)
      __attribute__((always_inline)) {
    store2(h[0], h[1],
           __builtin_amdgcn_make_buffer_rsrc(
               p.ckpt + (static_cast<int64_t>(q) * ck_plane + ck_row0) * kMaxState, 0,
               kRsrcRange, kRsrcFlags),
           o_ck);
#pragma unroll
    for (int t4 = 0; t4 < kBwdT; t4 += 4) {
      const f4 b0 = ld4(sb + (2 * sg) * kCkBPitch + c0 + t4);
      const f4 b1 = ld4(sb + (2 * sg + 1) * kCkBPitch + c0 + t4);
      const f4 dd01 = ld4(sdd + sc * kCkDdPitch + 2 * (c0 + t4));
      const f4 dd23 = ld4(sdd + sc * kCkDdPitch + 2 * (c0 + t4) + 4);
      const float dl[4] = {dd01.x, dd01.z, dd23.x, dd23.z};
      const float du[4] = {dd01.y, dd01.w, dd23.y, dd23.w};
      float a0[4], a1[4], x0[4], x1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a0[i] = fast_exp2(dl[i] * A2[0]);
        a1[i] = fast_exp2(dl[i] * A2[1]);
        x0[i] = du[i] * f4_at(b0, i);
        x1[i] = du[i] * f4_at(b1, i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[0] = fmaf(a0[i], h[0], x0[i]);
        h[1] = fmaf(a1[i], h[1], x1[i]);
      }
    }
  };
  load_block(q_begin);
  for (int q = q_begin; q < q_end; q += 2) {
    const int t0 = q * kBwdT;
    float* sb = s_b[((q - q_begin) >> 1) & 1];
    float* sdd = s_dd[((q - q_begin) >> 1) & 1];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int tt = lt + 16 * v;
      sb[ln * kCkBPitch + tt] = rb[v];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = xv && t0 + tt < s.seqlen;
        const float x = rx[v][e] + bias[e];
        const float sp = s.softplus ? softplus(x) : x;
        const float dl = ok ? sp : 0.0f;
        *reinterpret_cast<float2*>(sdd + (lc + e) * kCkDdPitch + 2 * tt) =
            make_float2(dl, dl * ru[v][e]);
      }
    }
    load_block(q + 2);
    __syncthreads();
    const float* wdd = sdd + w * kCh * kCkDdPitch;
    walk_chunk(sb, wdd, q, 0);
    if (q + 1 < q_end) walk_chunk(sb, wdd, q + 1, kBwdT);
  }
}

// ---------------------------------------------------------------- pass 2 ---
// PAIR: the lane's two elements (steps 2j, 2j+1 of its channel) are one
// 2-element access per tensor (s.pairs).
template <typename IO, bool PAIR, bool REV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_kernel(BwdShape s, BwdPtrs p) {
  // One LDS block, B/C first and the reduction rows next, so that the rows
  // addressed with per-lane bases plus a step offset stay within reach of the
  // 16-bit DS instruction offset.  B/C and the reduction rows are double
  // buffered by chunk parity, so that one workgroup barrier per chunk orders
  // every shared access (see the loop).
  constexpr int kRedSize = 2 * kMaxState * kBwdT;
  constexpr int kBcSize = 2 * kMaxState * kBcPitch;
  __shared__ __attribute__((aligned(16)))
  float smem[2 * kBcSize + kBwdWaves * (2 * kRedSize + kCh * kElPitch + kCh * kGrPitch)];
  float* const s_bc2 = smem;
  float* const s_red2 = smem + 2 * kBcSize;
  float* const s_el = s_red2 + 2 * kBwdWaves * kRedSize;
  float* const s_gr = s_el + kBwdWaves * kCh * kElPitch;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t logical = xcd_order(blockIdx.x, gridDim.x);
  const int tile = static_cast<int>(logical % s.tiles);
  const int64_t row_seg = logical / s.tiles;
  const int b = static_cast<int>(row_seg / s.nseg);
  const int seg = static_cast<int>(row_seg % s.nseg);
  const int d0 = tile * kBwdCh + w * kCh;  // this wave's first channel
  const int sg = lane >> 3, sc = lane & 7;
  const int d = d0 + sc;
  const bool dvalid = d < s.dim;
  const int64_t chan_row = static_cast<int64_t>(b) * s.tiles * kBwdCh + d;
  const bool has_z = p.z != nullptr;
  const bool has_dz = has_z && p.dz != nullptr;
  // lane (c, g) runs states 2g, 2g+1 of channel c, in the order that
  // sum_pair_half_rows expects: slot k holds state nk[k]
  const int swap = sc >> 2;
  const int nk[2] = {2 * sg + swap, 2 * sg + (swap ^ 1)};

  const IO* u = static_cast<const IO*>(p.u);
  const IO* dr = static_cast<const IO*>(p.delta_raw);
  const IO* zz = static_cast<const IO*>(p.z);
  const IO* dout = static_cast<const IO*>(p.dout);
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  IO* du_out = static_cast<IO*>(p.du);
  IO* ddr_out = static_cast<IO*>(p.ddelta_raw);
  IO* dz_out = static_cast<IO*>(p.dz);

  float A2[2], An[2], g[2], dA[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = nk[k];
    const bool active = dvalid && n < s.dstate;
    An[k] = active ? -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) : 0.0f;
    A2[k] = An[k] * kLog2e;
    if (s.nseg > 1)
      g[k] = p.carry_g[(static_cast<int64_t>(seg) * s.nchan_pad + chan_row) * kMaxState + n];
    else
      g[k] = (active && p.dfinal != nullptr)
                 ? p.dfinal[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] : 0.0f;
    dA[k] = 0.0f;
  }
  const int q_begin = seg * s.seg_chunks;
  const int q_end = min(s.nchunk, q_begin + s.seg_chunks);
  // element roles: lane (c, j) = (lane % 8, lane / 8) owns steps 2j, 2j+1 of
  // channel c (the same channel as its scan role)
  const float bias = (dvalid && p.dt_bias != nullptr) ? p.dt_bias[d] : 0.0f;
  const float skip = (dvalid && p.D != nullptr) ? p.D[d] : 0.0f;
  float acc_dD = 0.0f, acc_db = 0.0f;

  float* el = s_el + w * (kCh * kElPitch);
  float* gr = s_gr + w * (kCh * kGrPitch);
  // Chunk tiles are read and written through buffer descriptors (chunk_rsrc)
  // with loop-invariant 32-bit lane offsets; kOffNone reads 0 or drops the
  // store.
  constexpr int64_t es = sizeof(IO);
  const RowBase rb_u = row_base(u, s.su, es, b, d0, true, u);
  const RowBase rb_dr = row_base(dr, s.sd, es, b, d0, true, u);
  const RowBase rb_do = row_base(dout, s.sdo, es, b, d0, true, u);
  const RowBase rb_z = row_base(zz, s.sz, es, b, d0, has_z, u);
  const RowBase rb_du = row_base(du_out, s.sdu, es, b, d0, true, u);
  const RowBase rb_ddr = row_base(ddr_out, s.sddr, es, b, d0, true, u);
  const RowBase rb_dz = row_base(dz_out, s.sdz, es, b, d0, has_dz, u);
  const RowBase rb_B = row_base(Bm, s.sB, es, b, 0, true, u);
  const RowBase rb_C = row_base(Cm, s.sC, es, b, 0, true, u);
  // lowest storage step of the chunk starting at logical step t0
  auto chunk_ts = [&](int t0) __attribute__((always_inline)) {
    return REV ? static_cast<int64_t>(s.seqlen) - kBwdT - t0 : static_cast<int64_t>(t0);
  };
  auto tile_off = [&](const int64_t* st, int row, int tt) __attribute__((always_inline)) {
    return chunk_off(s, st, es, row, tt);
  };
  // lane (c, j) owns steps 2j, 2j+1 of channel c; thread (r, i) = (tid / 16,
  // tid % 16) loads row r of B (r < 16) or C (r >= 16, the upper four waves)
  // at step i
  // With PAIR only slot 0 is used: the offset of the pair's lower address,
  // which holds step 2j in forward time and step 2j+1 in reverse time.
  uint32_t o_u[2], o_dr[2], o_do[2], o_z[2], o_du[2], o_ddr[2], o_dz[2], o_ck[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int tt = PAIR ? 2 * sg + (REV ? 1 : 0) : 2 * sg + e;
    o_u[e] = dvalid ? tile_off(s.su, sc, tt) : kOffNone;
    o_dr[e] = dvalid ? tile_off(s.sd, sc, tt) : kOffNone;
    o_do[e] = dvalid ? tile_off(s.sdo, sc, tt) : kOffNone;
    o_z[e] = dvalid ? tile_off(s.sz, sc, tt) : kOffNone;
    o_du[e] = dvalid ? tile_off(s.sdu, sc, tt) : kOffNone;
    o_ddr[e] = dvalid ? tile_off(s.sddr, sc, tt) : kOffNone;
    o_dz[e] = dvalid ? tile_off(s.sdz, sc, tt) : kOffNone;
    o_ck[e] = dvalid ? static_cast<uint32_t>((sc * kMaxState + nk[e]) * sizeof(float)) : kOffNone;
  }
  // B/C rows of a chunk: thread (r, i) = (tid / 16, tid % 16) covers step i of
  // rows r + j kBcRowStep, j < kBcPerThread; rows r < 16 are B, the others C
  // (which tensor is wave-uniform)
  constexpr int kBcPerThread = 2 * kMaxState * kBwdT / kBwdThreads;
  constexpr int kBcRowStep = kBwdThreads / kBwdT;
  static_assert(kBcPerThread * kBwdThreads == 2 * kMaxState * kBwdT, "B/C tile split");
  const int bc_t = tid & 15;
  uint32_t o_bc[kBcPerThread];
  auto bc_row = [&](int j) __attribute__((always_inline)) { return (tid >> 4) + j * kBcRowStep; };
  auto bc_is_c = [&](int j) __attribute__((always_inline)) {
    return kBcPerThread == 1 ? w >= kBwdWaves / 2 : j >= kBcPerThread / 2;
  };
#pragma unroll
  for (int j = 0; j < kBcPerThread; ++j) {
    const int n = bc_row(j) & (kMaxState - 1);
    const int64_t st[3] = {0, bc_is_c(j) ? s.sC[1] : s.sB[1], bc_is_c(j) ? s.sC[2] : s.sB[2]};
    o_bc[j] = n < s.dstate ? tile_off(st, n, bc_t) : kOffNone;
  }
  const int64_t ck_row0 = static_cast<int64_t>(b) * s.dim + d0;  // chunk-state layout
  const int64_t ck_plane = static_cast<int64_t>(s.batch) * s.dim;

  // Raw inputs of a chunk, issued one chunk ahead of use: one B or C value
  // per thread, u, delta_raw, dout and z for the lane's two elements, and the
  // checkpoint of the lane's two states.  A chunk before the segment loads
  // nothing.
  float rbc[kBcPerThread], ru[2], rx[2], rgo[2], rz[2], rck[2];
  auto load_chunk = [&](int q) __attribute__((always_inline)) {
    const int t0 = q * kBwdT;
    const int64_t ts = chunk_ts(t0);
    const bool qok = q >= q_begin;
#pragma unroll
    for (int j = 0; j < kBcPerThread; ++j) {
      const auto r_bc = row_rsrc(bc_is_c(j) ? rb_C : rb_B, ts, true);
      rbc[j] = buf_one<IO>::load(r_bc, (qok && t0 + bc_t < s.seqlen) ? o_bc[j] : kOffNone, 0);
    }
    const auto r_u = row_rsrc(rb_u, ts, true);
    const auto r_dr = row_rsrc(rb_dr, ts, true);
    const auto r_do = row_rsrc(rb_do, ts, true);
    const auto r_z = row_rsrc(rb_z, ts, has_z);
    if constexpr (PAIR) {
      // even length: a pair is wholly inside or wholly past the sequence
      const bool ok = qok && t0 + 2 * sg < s.seqlen;
      auto ld2 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, float (&x)[2])
          __attribute__((always_inline)) {
        float lo, hi;
        pair_io<IO>::load(r, ok ? off : kOffNone, lo, hi);
        x[0] = REV ? hi : lo;
        x[1] = REV ? lo : hi;
      };
      ld2(r_u, o_u[0], ru);
      ld2(r_dr, o_dr[0], rx);
      ld2(r_do, o_do[0], rgo);
      ld2(r_z, o_z[0], rz);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = qok && t0 + 2 * sg + e < s.seqlen;
        ru[e] = buf_one<IO>::load(r_u, ok ? o_u[e] : kOffNone, 0);
        rx[e] = buf_one<IO>::load(r_dr, ok ? o_dr[e] : kOffNone, 0);
        rgo[e] = buf_one<IO>::load(r_do, ok ? o_do[e] : kOffNone, 0);
        rz[e] = buf_one<IO>::load(r_z, ok ? o_z[e] : kOffNone, 0);
      }
    }
    const auto r_ck = __builtin_amdgcn_make_buffer_rsrc(
        p.ckpt + (static_cast<int64_t>(q) * ck_plane + ck_row0) * kMaxState, 0, kRsrcRange,
        kRsrcFlags);
#pragma unroll
    for (int k = 0; k < 2; ++k) rck[k] = load_stream(r_ck, qok ? o_ck[k] : kOffNone);
  };
  // The workgroup's dB / dC partial of chunk q (the thread's B/C tile
  // positions): the sum over the waves of their reduction rows.
  auto chunk_partial = [&](int q) __attribute__((always_inline)) {
    const float* red = s_red2 + (q & 1) * (kBwdWaves * kRedSize);
    const int tt = tid & 15, t = q * kBwdT + tt;
#pragma unroll
    for (int j = 0; j < kBcPerThread; ++j) {
      const int r = bc_row(j);
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kBwdWaves; ++ww) sum += red[ww * kRedSize + r * kBwdT + tt];
      if ((r & 15) < s.dstate && t < s.seqlen)
        __builtin_nontemporal_store(
            sum, &p.part_bc[(((static_cast<int64_t>(b) * s.npair + (q >> 1)) * s.tiles + tile) *
                                 2 * kMaxState + r) * (2 * kBwdT) + (q & 1) * kBwdT + tt]);
    }
  };

  // One barrier per chunk.  Iteration q writes B/C buffer q & 1 before it and
  // reduction buffer q & 1 after it, and sums reduction buffer (q + 1) & 1
  // (chunk q + 1) right after it.  Every wave that passes the barrier of
  // iteration q has seen all waves finish iteration q + 1, the last to read
  // B/C buffer q & 1 (chunk q + 2) or to sum reduction buffer q & 1 (chunk
  // q + 2), and to write reduction buffer (q + 1) & 1.
  load_chunk(q_end - 1);
  for (int q = q_end - 1; q >= q_begin; --q) {
    const int t0 = q * kBwdT;
    float* const s_bc = s_bc2 + (q & 1) * kBcSize;
    // ---- E: B and C into LDS; per element, the scan's inputs into s_el and
    // the values the output phase needs into s_gr ----
#pragma unroll
    for (int j = 0; j < kBcPerThread; ++j) s_bc[bc_row(j) * kBcPitch + bc_t] = rbc[j];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tt = 2 * sg + e, t = t0 + tt;
      const bool ok = dvalid && t < s.seqlen;
      const float x = rx[e] + bias;
      const float dl = ok ? (s.softplus ? softplus(x) : x) : 0.0f;
      const float sig = s.softplus ? sigmoid(x) : 1.0f;
      const float dy = has_z ? rgo[e] * silu(rz[e]) : rgo[e];
      *reinterpret_cast<f4*>(el + sc * kElPitch + 4 * tt) = f4{dl, dl * ru[e], dy, 0.0f};
      *reinterpret_cast<f4*>(gr + sc * kGrPitch + 8 * tt) = f4{ru[e], sig, rgo[e], rz[e]};
    }
    float hs[2], h[2], hh[kBwdT][2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      hs[k] = rck[k];
      h[k] = hs[k];
    }
    load_chunk(q - 1);
    __syncthreads();
    if (q + 1 < q_end) chunk_partial(q + 1);

    // ---- F: the chunk's states from its checkpoint ----
    const float* rb0 = s_bc + nk[0] * kBcPitch;
    const float* rb1 = s_bc + nk[1] * kBcPitch;
    const float* rc0 = s_bc + (kMaxState + nk[0]) * kBcPitch;
    const float* rc1 = s_bc + (kMaxState + nk[1]) * kBcPitch;
    const float* rdd = el + sc * kElPitch;
    const int ystep = group_step(lane);
#pragma unroll
    for (int t4 = 0; t4 < kBwdT; t4 += 4) {
      float yp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t4 + i;
        const f4 dd = ld4(rdd + 4 * t);
        h[0] = fmaf(fast_exp2(dd.x * A2[0]), h[0], dd.y * rb0[t]);
        h[1] = fmaf(fast_exp2(dd.x * A2[1]), h[1], dd.y * rb1[t]);
        hh[t][0] = h[0];
        hh[t][1] = h[1];
        yp[i] = fmaf(rc1[t], h[1], rc0[t] * h[0]);
      }
      el[sc * kElPitch + 4 * (t4 + ystep) + 3] = reduce_groups(yp[0], yp[1], yp[2], yp[3]);
    }
    __builtin_amdgcn_wave_barrier();
    // ---- R: reverse walk ----
    // Per step the sums over the wave's 8 channels of the dB and dC terms are
    // finished at once (one DPP tree each for the lane's two states); lanes
    // c = 0 and c = 4 of each state group write them for 4 steps at a time,
    // so that the 4 steps stay one branch-free block.  The sums over states
    // collect 4 steps for one cross-lane tree.
    float* red = s_red2 + (q & 1) * (kBwdWaves * kRedSize) + w * kRedSize;
    const bool writer = (sc & 3) == 0;
#pragma unroll
    for (int t4 = kBwdT - 4; t4 >= 0; t4 -= 4) {
      float qb[4], qa[4], vb[4], vc[4];
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const int t = t4 + i;
        const f4 dd = ld4(rdd + 4 * t);
        float G[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) G[k] = fmaf(dd.z, k == 0 ? rc0[t] : rc1[t], g[k]);
        vb[i] = sum_pair_half_rows(G[0] * dd.y, G[1] * dd.y);
        vc[i] = sum_pair_half_rows(dd.z * hh[t][0], dd.z * hh[t][1]);
        float sb = G[0] * rb0[t];
        sb = fmaf(G[1], rb1[t], sb);
        float sa = 0.0f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float ga = G[k] * fast_exp2(dd.x * A2[k]);
          const float r = ga * (t > 0 ? hh[t > 0 ? t - 1 : 0][k] : hs[k]);
          dA[k] = fmaf(r, dd.x, dA[k]);
          sa = fmaf(r, An[k], sa);
          g[k] = ga;
        }
        qb[i] = sb;
        qa[i] = sa;
      }
      // finish the sums in every lane (one DPP add each) rather than let the
      // compiler move the last add into the writers' branch as a move plus
      // an add
      asm volatile("" : "+v"(vb[0]), "+v"(vb[1]), "+v"(vb[2]), "+v"(vb[3]));
      asm volatile("" : "+v"(vc[0]), "+v"(vc[1]), "+v"(vc[2]), "+v"(vc[3]));
      if (writer) {
        *reinterpret_cast<f4*>(red + nk[0] * kBwdT + t4) = f4{vb[0], vb[1], vb[2], vb[3]};
        *reinterpret_cast<f4*>(red + (kMaxState + nk[0]) * kBwdT + t4) = f4{vc[0], vc[1], vc[2], vc[3]};
      }
      const float gb = reduce_groups(qb[0], qb[1], qb[2], qb[3]);
      const float ga = reduce_groups(qa[0], qa[1], qa[2], qa[3]);
      *reinterpret_cast<float2*>(gr + sc * kGrPitch + 8 * (t4 + ystep) + 4) = make_float2(gb, ga);
    }
    __builtin_amdgcn_wave_barrier();  // R's per-element sums, written by other lanes

    // ---- O: du, ddelta_raw and dz per element ----
    const auto r_du = row_rsrc(rb_du, chunk_ts(t0), true);
    const auto r_ddr = row_rsrc(rb_ddr, chunk_ts(t0), true);
    const auto r_dz = row_rsrc(rb_dz, chunk_ts(t0), has_dz);
    float o_du_v[2], o_ddr_v[2], o_dz_v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int tt = 2 * sg + e, t = t0 + tt;
      const f4 sv = ld4(el + sc * kElPitch + 4 * tt);      // delta, delta*u, dy, C.h
      const f4 ev = ld4(gr + sc * kGrPitch + 8 * tt);      // u, sigmoid(x), dout, z
      const float2 gv = *reinterpret_cast<const float2*>(gr + sc * kGrPitch + 8 * tt + 4);
      o_du_v[e] = fmaf(sv.z, skip, sv.x * gv.x);
      o_ddr_v[e] = fmaf(ev.x, gv.x, gv.y) * ev.y;
      // dz = dout * (C.h + D u) * silu'(z), silu'(z) = sig(z) (1 + z (1 - sig(z)))
      const float y = fmaf(skip, ev.x, sv.w);
      const float sz = sigmoid(ev.w);
      o_dz_v[e] = ev.z * y * (sz * fmaf(ev.w, 1.0f - sz, 1.0f));
      if (dvalid && t < s.seqlen) {
        acc_db += o_ddr_v[e];
        acc_dD = fmaf(sv.z, ev.x, acc_dD);
      }
    }
    if constexpr (PAIR) {
      const bool ok = t0 + 2 * sg < s.seqlen;
      auto st2 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&x)[2])
          __attribute__((always_inline)) {
        pair_io<IO>::store(r, ok ? off : kOffNone, REV ? x[1] : x[0], REV ? x[0] : x[1]);
      };
      st2(r_du, o_du[0], o_du_v);
      st2(r_ddr, o_ddr[0], o_ddr_v);
      if (has_dz) st2(r_dz, o_dz[0], o_dz_v);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = t0 + 2 * sg + e < s.seqlen;
        store_stream<IO>(o_du_v[e], r_du, ok ? o_du[e] : kOffNone);
        store_stream<IO>(o_ddr_v[e], r_ddr, ok ? o_ddr[e] : kOffNone);
        if (has_dz) store_stream<IO>(o_dz_v[e], r_dz, ok ? o_dz[e] : kOffNone);
      }
    }
  }

  // ---- per (row, channel) results ----
  const int64_t prow = ((static_cast<int64_t>(seg) * s.batch + b) * s.dim + d) * (kMaxState + 2);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int n = nk[k];
    if (dvalid && n < s.dstate) {
      p.part_chan[prow + n] = dA[k] * An[k];
      if (p.dh0 != nullptr && seg == 0)
        p.dh0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] = g[k];
    }
  }
  // dD and ddt_bias: the 8 lanes of a channel (lanes c + 8j) meet in LDS
  __syncthreads();
  chunk_partial(q_begin);
  // the other reduction buffer is free: its last reader (chunk q_begin + 1's
  // sum) ran before the barrier
  float* tmp = s_red2 + ((q_begin & 1) ^ 1) * (kBwdWaves * kRedSize) + w * kRedSize;
  tmp[lane] = acc_dD;
  tmp[64 + lane] = acc_db;
  __builtin_amdgcn_wave_barrier();
  if (sg == 0 && dvalid) {
    float sD = 0.0f, sb = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sD += tmp[sc + 8 * j];
      sb += tmp[64 + sc + 8 * j];
    }
    p.part_chan[prow + kMaxState] = sD;
    p.part_chan[prow + kMaxState + 1] = sb;
  }
}

// ---------------------------------------------------------------- pass 3 ---
// sum_(r < n) f(r) added in order of r (the result is bitwise repeatable);
// the terms are loaded kSumBatch at a time ahead of the adds, so the chain
// waits for one memory latency per batch, not per term.
constexpr int kSumBatch = 8;
template <typename F>
__device__ inline float ordered_sum(int n, F f) {
  float sum = 0.0f;
  for (int r0 = 0; r0 < n; r0 += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j) v[j] = f(min(r0 + j, n - 1));
#pragma unroll
    for (int j = 0; j < kSumBatch; ++j)
      if (r0 + j < n) sum += v[j];
  }
  return sum;
}

// dB / dC[b, n, t] = sum over the row's workgroups of their partials, added
// in tile order.  A thread sums four consecutive steps of one state: they are
// adjacent in a partial row (a pair of chunks holds 2 kBwdT steps), so each
// tile's terms arrive as one 16-byte load, and the four sums keep the order
// of a one-step sum.  NF (outputs with unit state stride, as channel-last B
// and C give them): a wave takes 8 states x 32 steps (8 lanes per state,
// each loading 16 bytes of the state's 128-byte partial row), and the two
// waves of a state-half pair cover all 16 states of those steps, so that the
// stores fill whole runs of the output instead of one 4-byte word per 64
// bytes, and every load still reads whole partial rows.
static_assert((2 * kBwdT) % kBcSteps == 0, "a thread's steps lie in one partial row");
// dA_log, dD and ddt_bias: element i of [dim][kMaxState + 2], the sum over
// batch rows and segments of the reverse walk's per-channel partials.
__device__ inline void finalize_sums(const BwdShape& s, const BwdPtrs& p, int64_t i) {
  if (i >= static_cast<int64_t>(s.dim) * (kMaxState + 2)) return;
  const int d = static_cast<int>(i / (kMaxState + 2));
  const int j = static_cast<int>(i % (kMaxState + 2));
  if (j < kMaxState && j >= s.dstate) return;
  const float sum = ordered_sum(s.nseg * s.batch, [&](int r) {
    return p.part_chan[(static_cast<int64_t>(r) * s.dim + d) * (kMaxState + 2) + j];
  });
  if (j < kMaxState)
    p.dA_log[static_cast<int64_t>(d) * s.dstate + j] = sum;
  else if (j == kMaxState) {
    if (p.dD != nullptr) p.dD[d] = sum;
  } else if (p.ddt_bias != nullptr) {
    p.ddt_bias[d] = sum;
  }
}

// Blocks [0, bc_blocks) sum dB and dC; the blocks after them run
// finalize_sums (one launch for both, which read only the reverse walk's
// partials).
template <typename IO, bool NF>
__global__ __launch_bounds__(256) void reduce_bc_kernel(BwdShape s, BwdPtrs p, unsigned bc_blocks) {
  if (blockIdx.x >= bc_blocks) {
    finalize_sums(s, p, static_cast<int64_t>(blockIdx.x - bc_blocks) * blockDim.x + threadIdx.x);
    return;
  }
  const int nq = (s.seqlen + kBcSteps - 1) / kBcSteps;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int t0, n, b;
  bool is_c;
  if constexpr (NF) {  // i = (((b * 2 + is_c) * nqb + qb) * 2 + n_hi) * 64 + q_lo * 8 + n_lo
    constexpr int kQ = 2 * kBwdT / kBcSteps;  // step quads per partial row: 8
    const int nqb = (nq + kQ - 1) / kQ;
    if (i >= static_cast<int64_t>(s.batch) * 2 * nqb * 2 * 64) return;
    const int lane = static_cast<int>(i % 64);
    const int64_t rest = i / 64;
    n = (lane % 8) + 8 * static_cast<int>(rest % 2);
    const int q = static_cast<int>((rest / 2) % nqb) * kQ + lane / 8;
    if (n >= s.dstate || q >= nq) return;
    t0 = q * kBcSteps;
    is_c = (rest / 2 / nqb) % 2 != 0;
    b = static_cast<int>(rest / 2 / nqb / 2);
  } else {  // i = ((b * 2 * dstate) + j) * nq + q
    if (i >= static_cast<int64_t>(s.batch) * 2 * s.dstate * nq) return;
    t0 = static_cast<int>(i % nq) * kBcSteps;
    const int64_t rest = i / nq;
    const int j = static_cast<int>(rest % (2 * s.dstate));
    b = static_cast<int>(rest / (2 * s.dstate));
    is_c = j >= s.dstate;
    n = is_c ? j - s.dstate : j;
  }
  const int r = is_c ? kMaxState + n : n;
  using v4 = float __attribute__((ext_vector_type(4)));
  constexpr int64_t kTileStride = 2 * kMaxState * 2 * kBwdT;  // floats between tiles
  const float* row = p.part_bc +
      (((static_cast<int64_t>(b) * s.npair + t0 / (2 * kBwdT)) * s.tiles) * 2 * kMaxState + r) *
          (2 * kBwdT) + t0 % (2 * kBwdT);
  v4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0b = 0; t0b < s.tiles; t0b += kSumBatch) {
    v4 v[kSumBatch];
#pragma unroll
    for (int k = 0; k < kSumBatch; ++k)
      v[k] = __builtin_nontemporal_load(
          reinterpret_cast<const v4*>(row + min(t0b + k, s.tiles - 1) * kTileStride));
#pragma unroll
    for (int k = 0; k < kSumBatch; ++k)
      if (t0b + k < s.tiles) sum += v[k];
  }
  IO* out = static_cast<IO*>(is_c ? p.dC : p.dB) + b * (is_c ? s.sdC[0] : s.sdB[0]) +
            n * (is_c ? s.sdC[1] : s.sdB[1]);
  const int64_t st = is_c ? s.sdC[2] : s.sdB[2];
#pragma unroll
  for (int e = 0; e < kBcSteps; ++e)
    if (t0 + e < s.seqlen) io_traits<IO>::store(out + tstore(s, t0 + e) * st, sum[e]);
}

template <typename IO, bool WITH_H, int XM, bool REV>
void launch_agg_b(const BwdShape& s, const BwdPtrs& p, hipStream_t stream, unsigned waves) {
  if (s.nquads)
    agg_kernel<IO, WITH_H, XM, kBStateQuads, REV><<<dim3(waves), dim3(64), 0, stream>>>(s, p);
  else if (s.bcquads)
    agg_kernel<IO, WITH_H, XM, kBStepQuads, REV><<<dim3(waves), dim3(64), 0, stream>>>(s, p);
  else
    agg_kernel<IO, WITH_H, XM, kBScalar, REV><<<dim3(waves), dim3(64), 0, stream>>>(s, p);
}

template <typename IO, bool WITH_H, bool REV>
void launch_agg_p(const BwdShape& s, const BwdPtrs& p, hipStream_t stream, unsigned waves) {
  if (s.pairs)
    launch_agg_b<IO, WITH_H, kXStepPairs, REV>(s, p, stream, waves);
  else if (s.dpairs)
    agg_coop_kernel<IO, WITH_H><<<dim3(waves / kBwdWaves), dim3(kBwdThreads), 0, stream>>>(s, p);
  else
    launch_agg_b<IO, WITH_H, kXScalar, REV>(s, p, stream, waves);
}

// Forward aggregate H only without the forward's chunk states.
template <typename IO, bool REV>
void launch_agg(const BwdShape& s, const BwdPtrs& p, hipStream_t stream, unsigned waves) {
  if (s.states_given)
    launch_agg_p<IO, false, REV>(s, p, stream, waves);
  else
    launch_agg_p<IO, true, REV>(s, p, stream, waves);
}

template <typename IO, bool REV>
hipError_t launch_bwd_t(const BwdShape& s, const BwdPtrs& p, hipStream_t stream) {
  const int64_t waves = static_cast<int64_t>(s.batch) * s.nseg * s.tiles * kBwdWaves;
  if (s.nseg > 1) {
    launch_agg<IO, REV>(s, p, stream, static_cast<unsigned>(waves * s.agg_split));
    const int64_t nc = s.nchan_pad * kMaxState;
    const dim3 grid(static_cast<unsigned>((nc + 63) / 64));
    const dim3 block(64 * carry_waves(s.nseg * s.agg_split));
    if (s.agg_split > 1)
      carry_bwd_kernel<true><<<grid, block, 0, stream>>>(s, p);
    else
      carry_bwd_kernel<false><<<grid, block, 0, stream>>>(s, p);
  }
  // chunk states recorded by the forward replace the checkpoint pass
  if (s.states_given == 0) {
    const dim3 grid(static_cast<unsigned>(waves));
    if (s.dpairs)
      ckpt_coop_kernel<IO><<<dim3(static_cast<unsigned>(waves / kBwdWaves)), dim3(kBwdThreads), 0,
                             stream>>>(s, p);
    else if (s.quads && s.bquads)
      ckpt_kernel<IO, true, true, REV><<<grid, dim3(64), 0, stream>>>(s, p);
    else if (s.quads)
      ckpt_kernel<IO, true, false, REV><<<grid, dim3(64), 0, stream>>>(s, p);
    else if (s.bquads)
      ckpt_kernel<IO, false, true, REV><<<grid, dim3(64), 0, stream>>>(s, p);
    else
      ckpt_kernel<IO, false, false, REV><<<grid, dim3(64), 0, stream>>>(s, p);
  }
  const int64_t wgs = static_cast<int64_t>(s.batch) * s.nseg * s.tiles;
  if (s.pairs)
    bwd_kernel<IO, true, REV><<<dim3(static_cast<unsigned>(wgs)), dim3(kBwdThreads), 0, stream>>>(s, p);
  else
    bwd_kernel<IO, false, REV><<<dim3(static_cast<unsigned>(wgs)), dim3(kBwdThreads), 0, stream>>>(s, p);
  const int64_t nq = (s.seqlen + kBcSteps - 1) / kBcSteps;
  const int64_t fin_blocks = (static_cast<int64_t>(s.dim) * (kMaxState + 2) + 255) / 256;
  if (s.sdB[1] == 1 && s.sdB[2] != 1) {
    constexpr int kQ = 2 * kBwdT / kBcSteps;
    const int64_t nbc = static_cast<int64_t>(s.batch) * 2 * ((nq + kQ - 1) / kQ) * 2 * 64;
    const unsigned bc_blocks = static_cast<unsigned>((nbc + 255) / 256);
    reduce_bc_kernel<IO, true><<<dim3(static_cast<unsigned>(bc_blocks + fin_blocks)), dim3(256), 0,
                                 stream>>>(s, p, bc_blocks);
  } else {
    const int64_t nbc = static_cast<int64_t>(s.batch) * 2 * s.dstate * nq;
    const unsigned bc_blocks = static_cast<unsigned>((nbc + 255) / 256);
    reduce_bc_kernel<IO, false><<<dim3(static_cast<unsigned>(bc_blocks + fin_blocks)), dim3(256), 0,
                                  stream>>>(s, p, bc_blocks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd(const BwdShape& s, const BwdPtrs& p, bool io_bf16, hipStream_t stream) {
  if (s.reverse)
    return io_bf16 ? launch_bwd_t<bf16_t, true>(s, p, stream) : launch_bwd_t<float, true>(s, p, stream);
  return io_bf16 ? launch_bwd_t<bf16_t, false>(s, p, stream) : launch_bwd_t<float, false>(s, p, stream);
}

}  // namespace mss
