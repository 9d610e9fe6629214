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
// that only meet in the sum over C.  One wave (the whole workgroup) owns 16
// channels of one batch row for one time segment.  Lane (g, c) = (lane / 16,
// lane % 16) runs states 4g..4g+3 of channel c sequentially in time, in
// registers; A_log becomes exp2 multipliers with log2(e) folded in, once per
// lane.  The segment is walked in chunks of kT steps, each in three phases:
//   E  loads of u, delta_raw, B, C (issued one chunk ahead) with time across
//      lanes for [B,D,L] data (channels across lanes for [B,L,D]); softplus,
//      delta*u and D*u per element; (delta, delta*u) and B/C go to LDS;
//   S  per step and state one exp2, two multiplies and two FMAs.  B and C are
//      the same for all channels: one LDS load gives each 16-lane row the 16
//      coefficients its state group needs for two steps, and the multiplies
//      read them through a DPP row broadcast (row_newbcast).  The partial sums
//      C.h of the four state groups meet through v_permlane32_swap and
//      v_permlane16_swap: two swap-and-add levels reduce four steps at once
//      and leave the totals of those steps in the four rows;
//   O  the totals go through LDS back to the load layout, where the skip term
//      and the gate are applied and the output is stored.
// Every phase is wave-local: there is no workgroup barrier, so waves drift
// apart and memory waits of one wave overlap the recurrence of others.
//
// Long sequences with few channels are split into time segments so that the
// grid covers the GPU.  Segment s needs the state entering it.  A first pass
// (AGG) runs every segment but the last from a zero state and records, per
// (channel, state), the segment's pair aggregate (prod_t a_t, h_end): the
// product is exp2(A2 * sum_t delta_t) since all a_t share A.  A carry pass
// composes the aggregates in order with (a2, b2) o (a1, b1) = (a2 a1,
// a2 b1 + b2) ("mamba-metal", sections "Selective scan の本質" and
// "チャンク間 running prefix"), and the main pass starts each segment from
// its carry.
#include <algorithm>
#include <type_traits>

#include "mss_device.hpp"
#include "mss_internal.hpp"

namespace mss {

// Raw buffer descriptors: the range keeps every valid 32-bit tile offset in
// bounds; kOffNone is past it, so accesses with that offset read 0 / write
// nothing.  Flags: the gfx9 raw-buffer data format word.
constexpr int kRsrcRange = 0x7FFFFFF0;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOffNone = 0x80000000u;

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

// 16-byte vector <-> elements, and single-element buffer access, per type.
template <typename IO>
struct vec_io;
template <>
struct vec_io<float> {
  static constexpr int V = 4;
  __device__ static inline void unpack(u32x4 w, float* o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __uint_as_float(w[j]);
  }
  __device__ static inline u32x4 pack(const float* y) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __float_as_uint(y[j]);
    return w;
  }
  __device__ static inline float load_one(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
  }
  __device__ static inline void store_one(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), r, off, soff, 0);
  }
};
template <>
struct vec_io<bf16_t> {
  static constexpr int V = 8;
  __device__ static inline void unpack(u32x4 w, float* o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __uint_as_float(w[j] << 16);
      o[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 pack(const float* y) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(bf16_bits(y[2 * j])) |
             (static_cast<uint32_t>(bf16_bits(y[2 * j + 1])) << 16);
    return w;
  }
  __device__ static inline float load_one(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0))
                           << 16);
  }
  __device__ static inline void store_one(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                          uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(y), r, off, soff, 0);
  }
};

constexpr int kXcds = 8;                          // MI355X: 8 accelerator dies, 32 CUs each
constexpr int kDdPitch = kCh + 1;                 // float2 per step row of (delta, delta*u)
constexpr int kYPitch = kCh + 1;                  // floats per step row of the totals
constexpr int kBcPitch = kGroups * 8 + 1;         // floats per step row of the B/C tile
constexpr int kBcPerLane = 2 * kMaxState * kT / kThreads;  // 16 B/C values per lane per chunk

// Value held by lane K of this lane's 16-lane row (DPP row_newbcast).
template <int K>
__device__ inline float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xF, 0xF, false));
}

// acc += (lane K of bc's row) * x, in one v_fmac_f32 with a DPP source.  bc is
// always an LDS load result, never written by a VALU instruction, so the DPP
// read needs no wait states.
template <int K>
__device__ inline void fmac_row_bcast(float& acc, float bc, float x) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(acc)
      : "v"(bc), "v"(x), "n"(K));
}

// One time step of a lane's 4 states.  bc holds, per 16-lane row, B0..B3 and
// C0..C3 of the row's state group for step 2p in lanes 0..7 and for step 2p+1
// in lanes 8..15; S selects the half.  Returns the partial sum of C.h.
template <int S, bool AGG>
__device__ inline float scan_step(float dl, float du, float bc, const float (&A2)[kStatesPerLane],
                                  float (&h)[kStatesPerLane]) {
  const float a0 = fast_exp2(dl * A2[0]);
  const float a1 = fast_exp2(dl * A2[1]);
  const float a2 = fast_exp2(dl * A2[2]);
  const float a3 = fast_exp2(dl * A2[3]);
  h[0] = fmaf(a0, h[0], du * row_bcast<8 * S + 0>(bc));
  h[1] = fmaf(a1, h[1], du * row_bcast<8 * S + 1>(bc));
  h[2] = fmaf(a2, h[2], du * row_bcast<8 * S + 2>(bc));
  h[3] = fmaf(a3, h[3], du * row_bcast<8 * S + 3>(bc));
  if constexpr (AGG) {
    return 0.0f;
  } else {
    float y = row_bcast<8 * S + 4>(bc) * h[0];
    fmac_row_bcast<8 * S + 5>(y, bc, h[1]);
    fmac_row_bcast<8 * S + 6>(y, bc, h[2]);
    fmac_row_bcast<8 * S + 7>(y, bc, h[3]);
    return y;
  }
}

// Sum over the four rows (state groups) of four per-step partial sums.  Row r
// of the result holds the total of step {0, 2, 1, 3}[r].
__device__ inline float reduce_groups(float y0, float y1, float y2, float y3) {
  const auto s01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y0), __float_as_uint(y1),
                                                    false, false);
  const auto s23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y2), __float_as_uint(y3),
                                                    false, false);
  // rows 0,1: y0 (resp. y2) summed over groups {0,2} and {1,3}; rows 2,3: y1 (resp. y3)
  const float p01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
  const float p23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(p01), __float_as_uint(p23),
                                                  false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <typename IO, bool XT, bool BT, bool AGG, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void scan_kernel(
    ScanShape s, const IO* __restrict__ u, const IO* __restrict__ delta_raw,
    const float* __restrict__ A_log, const IO* __restrict__ Bm, const IO* __restrict__ Cm,
    const float* __restrict__ Dskip, const IO* __restrict__ z,
    const float* __restrict__ dt_bias, const float* __restrict__ h0, IO* __restrict__ out,
    float* __restrict__ final_state, float2* __restrict__ agg,
    const float* __restrict__ carry) {
  __shared__ float2 s_dd[kT * kDdPitch];            // (delta, delta*u) by [t][channel]
  __shared__ float s_bc[kT * kBcPitch];             // B/C by [t][group][B0..3, C0..3]
  __shared__ float s_y[AGG ? 1 : kT * kYPitch];     // step totals by [t][channel]

  const int lane = threadIdx.x;
  // Workgroups are dispatched round-robin over the XCDs (linear id mod 8).
  // Renumber them so that each XCD receives a contiguous range of tiles:
  // tiles of one batch row share B and C, which then stay in that XCD's L2.
  const int nwg = gridDim.x * gridDim.y;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int xcd = lin % kXcds;
  const int per_xcd = nwg / kXcds, extra = nwg % kXcds;
  const int logical = xcd * per_xcd + min(xcd, extra) + lin / kXcds;
  const int g = logical % gridDim.x;
  const int seg = logical / gridDim.x;
  const int b = g / s.groups;
  const int d0 = (g - b * s.groups) * kCh;
  const int t_begin = s.t_first + seg * s.seg_len;
  const int t_end = min(s.t_stop, t_begin + s.seg_len);
  constexpr int64_t es = sizeof(IO);

  // ---- S-phase constants: lane = (state group sg, channel sc) ----
  const int sg = lane >> 4;
  const int sc = lane & 15;
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

  // ---- chunk memory access ------------------------------------------------
  // All global traffic uses raw buffer loads/stores: a per-chunk descriptor
  // whose base is the tile corner, a 32-bit per-lane offset and a scalar
  // offset per vector.  An element or vector that lies outside the tensor gets
  // an offset beyond the descriptor's range, so the hardware returns 0 (or
  // drops the store) without a branch: every chunk issues the same
  // instruction stream and the compiler counts outstanding loads exactly.
  // Loads and stores move 16-byte vectors (4 fp32 or 8 bf16) along the
  // unit-stride axis; a chunk whose vectors would straddle a tensor edge (a
  // ragged tail) takes an element-wise path instead.
  using VIO = vec_io<IO>;
  constexpr int V = VIO::V;                 // elements per 16-byte vector
  constexpr int NV = kPerThread / V;        // vectors per lane per x-tensor
  constexpr int XL = XT ? kT / V : kCh / V; // lanes per row of vectors
  constexpr int XR = kThreads / XL;         // rows per load instruction
  constexpr int NBV = kBcPerLane / V;       // B/C vectors per lane
  constexpr int BL = BT ? kT / V : kMaxState / V;
  constexpr int BR = kThreads / BL;
  const int xr = lane / XL, xv = lane % XL;
  const int br = lane / BL, bv = lane % BL;
  // x-tensors: vector v of this lane covers elements e = v*V + j
  auto x_c = [&](int v, int j) __attribute__((always_inline)) { return XT ? xr + XR * v : xv * V + j; };
  auto x_t = [&](int v, int j) __attribute__((always_inline)) { return XT ? xv * V + j : xr + XR * v; };
  auto x_voff = [&](const int64_t* st) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(((XT ? xr : xv * V) * st[1] + (XT ? xv * V : xr) * st[2]) * es);
  };
  auto x_soff = [&](const int64_t* st, int v) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(XR * v * (XT ? st[1] : st[2]) * es);
  };
  const uint32_t vo_u = x_voff(s.su), vo_d = x_voff(s.sd), vo_z = x_voff(s.sz), vo_o = x_voff(s.so);
  // B/C: vector i covers (matrix, state, step) with steps (BT) or states along the vector
  auto bc_sel = [&](int i) __attribute__((always_inline)) { return (BR * i) / (BT ? kMaxState : kT); };
  auto bc_n = [&](int i, int j) __attribute__((always_inline)) { return BT ? br + (BR * i) % kMaxState : bv * V + j; };
  auto bc_tt = [&](int i, int j) __attribute__((always_inline)) { return BT ? bv * V + j : br + (BR * i) % kT; };
  auto bc_voff = [&](const int64_t* st) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(((BT ? br : bv * V) * st[1] + (BT ? bv * V : br) * st[2]) * es);
  };
  const uint32_t vo_b = bc_voff(s.sB), vo_c = bc_voff(s.sC);
  auto bc_soff = [&](const int64_t* st, int i) __attribute__((always_inline)) -> uint32_t {
    return static_cast<uint32_t>(((BR * i) % (BT ? kMaxState : kT)) * (BT ? st[1] : st[2]) * es);
  };

  // per-element channel constants
  float bias[kPerThread], skip[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int dc = d0 + x_c(e / V, e % V);
    const bool ok = dc < s.dim;
    bias[e] = (ok && dt_bias != nullptr) ? dt_bias[dc] : 0.0f;
    skip[e] = (ok && Dskip != nullptr) ? Dskip[dc] : 0.0f;
  }
  const bool has_z = z != nullptr;

  auto rsrc = [&](const void* ptr, const int64_t* st, int dd0, int t0) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(ptr) +
                       (static_cast<int64_t>(b) * st[0] + static_cast<int64_t>(dd0) * st[1] +
                        static_cast<int64_t>(t0) * st[2]) * es;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, kRsrcRange, kRsrcFlags);
  };
  // x_ok / b_ok: element (v, j) / B-C value (i, j) lies inside the tensors
  // and the chunk is one this loop loads (lim: first chunk start not loaded).
  auto x_ok = [&](int v, int j, int t0, int lim) __attribute__((always_inline)) {
    return (t0 < lim) && (d0 + x_c(v, j) < s.dim) && (t0 + x_t(v, j) < t_end);
  };
  auto b_ok = [&](int i, int j, int t0, int lim) __attribute__((always_inline)) {
    return (t0 < lim) && (bc_n(i, j) < s.dstate) && (t0 + bc_tt(i, j) < t_end);
  };

  // Chunk inputs live in registers from issue to use: u, delta_raw, B and C
  // two chunks ahead of the chunk being scanned, z one chunk ahead.
  struct InBuf {
    float u[kPerThread], d[kPerThread], bc[kBcPerLane];
  };
  struct ZBuf {
    float z[kPerThread];
  };
  InBuf in0, in1;
  ZBuf zb0, zb1;

  // Loads of one x-tensor.  VEC: 16-byte vectors (each wholly in or out of
  // the valid region); else element by element.
  auto load_x = [&](auto vec, float (&dst)[kPerThread], const IO* ptr, const int64_t* st,
                    uint32_t vo, int t0, int lim) {
    const auto rs = rsrc(ptr, st, d0, t0);
    if constexpr (VEC) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const uint32_t off = x_ok(v, 0, t0, lim) ? vo : kOffNone;
        VIO::unpack(__builtin_amdgcn_raw_buffer_load_b128(rs, off, x_soff(st, v), 0), dst + v * V);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int v = e / V, j = e % V;
        const uint32_t off = x_ok(v, j, t0, lim)
            ? vo + static_cast<uint32_t>(j * (XT ? st[2] : st[1]) * es) : kOffNone;
        dst[e] = VIO::load_one(rs, off, x_soff(st, v));
      }
    }
  };
  auto issue_z_loads = [&](auto vec, ZBuf& zb, int t0, int lim) __attribute__((always_inline)) {
    if constexpr (!AGG) {
      if (has_z) {
        load_x(vec, zb.z, z, s.sz, vo_z, t0, lim);
      } else {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) zb.z[e] = 0.0f;
      }
    }
  };
  auto issue_loads = [&](auto vec, InBuf& ib, int t0, int lim) __attribute__((always_inline)) {
    load_x(vec, ib.u, u, s.su, vo_u, t0, lim);
    load_x(vec, ib.d, delta_raw, s.sd, vo_d, t0, lim);
    const auto rb = rsrc(Bm, s.sB, 0, t0);
    const auto rcm = rsrc(Cm, s.sC, 0, t0);
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const bool is_c = bc_sel(i) == 1;
      float* dst = ib.bc + i * V;
      if (AGG && is_c) {
#pragma unroll
        for (int j = 0; j < V; ++j) dst[j] = 0.0f;
        continue;
      }
      const auto& rs = is_c ? rcm : rb;
      const int64_t* st = is_c ? s.sC : s.sB;
      const uint32_t vo = is_c ? vo_c : vo_b;
      if constexpr (VEC) {
        const uint32_t off = b_ok(i, 0, t0, lim) ? vo : kOffNone;
        VIO::unpack(__builtin_amdgcn_raw_buffer_load_b128(rs, off, bc_soff(st, i), 0), dst);
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const uint32_t off = b_ok(i, j, t0, lim)
              ? vo + static_cast<uint32_t>(j * (BT ? st[2] : st[1]) * es) : kOffNone;
          dst[j] = VIO::load_one(rs, off, bc_soff(st, i));
        }
      }
    }
  };

  float cur_du_skip[kPerThread];
  auto phase_e = [&](const InBuf& ib, int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int v = e / V, j = e % V;
      const bool ok = x_ok(v, j, t0, t_end);
      const float x = ib.d[e] + bias[e];
      float dl = s.softplus ? softplus(x) : x;
      float du = dl * ib.u[e];
      if (!ok) {
        dl = 0.0f;
        du = 0.0f;
      }
      s_dd[x_t(v, j) * kDdPitch + x_c(v, j)] = make_float2(dl, du);
      if constexpr (!AGG) cur_du_skip[e] = skip[e] * ib.u[e];
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int n = bc_n(i, j);
        s_bc[bc_tt(i, j) * kBcPitch + (n >> 2) * 8 + bc_sel(i) * 4 + (n & 3)] = ib.bc[i * V + j];
      }
    }
  };

  const int bc_read = ((sc >> 3) * kBcPitch) + sg * 8 + (sc & 7);

  // The group reduction leaves step {0, 2, 1, 3}[sg] of each block in row sg.
  const int y_row_step = sg == 1 ? 2 : (sg == 2 ? 1 : sg);
  auto phase_s = [&]() __attribute__((always_inline)) {
    // blocks of 4 steps, one state-group reduction each
#pragma unroll 1
    for (int q = 0; q < kT / 4; ++q) {
      const int t4 = 4 * q;
      const float bcA = s_bc[t4 * kBcPitch + bc_read];
      const float bcB = s_bc[(t4 + 2) * kBcPitch + bc_read];
      const float2 dd0 = s_dd[(t4 + 0) * kDdPitch + sc];
      const float2 dd1 = s_dd[(t4 + 1) * kDdPitch + sc];
      const float2 dd2 = s_dd[(t4 + 2) * kDdPitch + sc];
      const float2 dd3 = s_dd[(t4 + 3) * kDdPitch + sc];
      const float y0 = scan_step<0, AGG>(dd0.x, dd0.y, bcA, A2, h);
      const float y1 = scan_step<1, AGG>(dd1.x, dd1.y, bcA, A2, h);
      const float y2 = scan_step<0, AGG>(dd2.x, dd2.y, bcB, A2, h);
      const float y3 = scan_step<1, AGG>(dd3.x, dd3.y, bcB, A2, h);
      if constexpr (!AGG) {
        s_y[(t4 + y_row_step) * kYPitch + sc] = reduce_groups(y0, y1, y2, y3);
      } else {
        sum_delta += (dd0.x + dd1.x) + (dd2.x + dd3.x);
      }
    }
  };

  auto phase_o = [&](auto vec, const ZBuf& zb, int t0) __attribute__((always_inline)) {
    if constexpr (!AGG) {
      float y[kPerThread];
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) {
        const int v = e / V, j = e % V;
        y[e] = cur_du_skip[e] + s_y[x_t(v, j) * kYPitch + x_c(v, j)];
        if (has_z) y[e] *= silu(zb.z[e]);
      }
      const auto rs = rsrc(out, s.so, d0, t0);
      if constexpr (VEC) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint32_t off = x_ok(v, 0, t0, t_end) ? vo_o : kOffNone;
          __builtin_amdgcn_raw_buffer_store_b128(VIO::pack(y + v * V), rs, off, x_soff(s.so, v), 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          const int v = e / V, j = e % V;
          const uint32_t off = x_ok(v, j, t0, t_end)
              ? vo_o + static_cast<uint32_t>(j * (XT ? s.so[2] : s.so[1]) * es) : kOffNone;
          VIO::store_one(y[e], rs, off, x_soff(s.so, v));
        }
      }
    }
  };

  // ---- chunk loop (wave-local: LDS traffic is ordered within the wave) ----
  // One iteration scans chunk c.  Loads are issued in every iteration (past
  // the end they are out-of-range no-ops), so the loop body is branch-free and
  // the compiler counts outstanding loads exactly.  Issue order keeps every
  // wait on the oldest loads: z(c+1), then u/delta_raw/B/C(c+2); O(c) waits
  // for z(c) and E(c+1) for the inputs of c+1, both issued an iteration
  // earlier.  The body is written twice so that the two register buffers swap
  // roles.  VEC kernels move 16-byte vectors, so the host only gives them time
  // ranges and channel tiles in which no vector straddles an edge; the rest
  // (a tail of fewer steps than a vector, or layouts that cannot vectorise)
  // runs through the element-wise instantiation.
  const int nchunks = (t_end - t_begin + kT - 1) / kT;
  constexpr std::integral_constant<bool, VEC> vec{};
  issue_z_loads(vec, zb0, t_begin, t_end);
  issue_loads(vec, in0, t_begin, t_end);
  issue_loads(vec, in1, t_begin + kT, t_end);
  phase_e(in0, t_begin);
  auto iteration = [&](int c, InBuf& in_c, InBuf& in_next, ZBuf& z_c, ZBuf& z_next)
      __attribute__((always_inline)) {
    const int t0 = t_begin + c * kT;
    issue_z_loads(vec, z_next, t0 + kT, t_end);
    issue_loads(vec, in_c, t0 + 2 * kT, t_end);
    phase_s();
    phase_o(vec, z_c, t0);
    phase_e(in_next, t0 + kT);
  };
  for (int c = 0; c < nchunks; c += 2) {
    iteration(c, in0, in1, zb0, zb1);
    if (c + 1 < nchunks) iteration(c + 1, in1, in0, zb1, zb0);
  }

  // ---- segment end ----
  if constexpr (AGG) {
#pragma unroll
    for (int k = 0; k < kStatesPerLane; ++k) {
      const int n = sg * kStatesPerLane + k;
      const float prod_a = fast_exp2(A2[k] * sum_delta);
      agg[(static_cast<int64_t>(seg) * s.nchan_pad + chan_row) * kMaxState + n] =
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
//   carry[0] = h0 (or 0),  carry[s+1] = P[s] * carry[s] + H[s].
__global__ __launch_bounds__(256) void carry_kernel(ScanShape s, const float2* __restrict__ agg,
                                                    const float* __restrict__ h0,
                                                    float* __restrict__ carry) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= s.nchan_pad * kMaxState) return;
  const int n = static_cast<int>(idx % kMaxState);
  const int64_t row = idx / kMaxState;
  const int64_t per_b = static_cast<int64_t>(s.groups) * kCh;
  const int b = static_cast<int>(row / per_b);
  const int d = static_cast<int>(row % per_b);
  float c = 0.0f;
  if (h0 != nullptr && d < s.dim && n < s.dstate)
    c = h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n];
  for (int sgm = 0; sgm + 1 < s.nseg; ++sgm) {
    const float2 a = agg[(static_cast<int64_t>(sgm) * s.nchan_pad + row) * kMaxState + n];
    c = fmaf(a.x, c, a.y);
    carry[(static_cast<int64_t>(sgm + 1) * s.nchan_pad + row) * kMaxState + n] = c;
  }
}

template <typename IO, bool XT, bool BT, bool VEC>
static void launch_pass(const ScanShape& s, const ScanPtrs& p, const float* h0, float* final_state,
                        hipStream_t stream) {
  const dim3 block(kThreads);
  const unsigned G = static_cast<unsigned>(s.batch) * static_cast<unsigned>(s.groups);
  const IO* u = static_cast<const IO*>(p.u);
  const IO* dr = static_cast<const IO*>(p.delta_raw);
  const IO* Bm = static_cast<const IO*>(p.B);
  const IO* Cm = static_cast<const IO*>(p.C);
  const IO* z = static_cast<const IO*>(p.z);
  IO* out = static_cast<IO*>(p.out);
  if (s.nseg > 1) {
    scan_kernel<IO, XT, BT, true, VEC><<<dim3(G, s.nseg - 1), block, 0, stream>>>(
        s, u, dr, p.A_log, Bm, Cm, p.D, z, p.dt_bias, h0, out, final_state, p.agg, p.carry);
    const int64_t n = s.nchan_pad * kMaxState;
    carry_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(
        s, p.agg, h0, p.carry);
  }
  scan_kernel<IO, XT, BT, false, VEC><<<dim3(G, s.nseg), block, 0, stream>>>(
      s, u, dr, p.A_log, Bm, Cm, p.D, z, p.dt_bias, h0, out, final_state, p.agg, p.carry);
}

// The vector pass covers [0, s.t_stop); when s.t_stop < seqlen it exports its
// state to p.tail_h0 and an element-wise pass covers the remaining steps.
template <typename IO, bool XT, bool BT>
static hipError_t launch_scan_t(const ScanShape& s, const ScanPtrs& p, hipStream_t stream) {
  if (!s.use_vec) {
    launch_pass<IO, XT, BT, false>(s, p, p.h0, p.final_state, stream);
    return hipGetLastError();
  }
  const bool tail = s.t_stop < s.seqlen;
  if (s.t_stop > 0)
    launch_pass<IO, XT, BT, true>(s, p, p.h0, tail ? p.tail_h0 : p.final_state, stream);
  if (tail) {
    ScanShape t = s;
    t.t_first = s.t_stop;
    t.t_stop = s.seqlen;
    t.nseg = 1;
    t.seg_len = s.seqlen - s.t_stop;
    launch_pass<IO, XT, BT, false>(t, p, s.t_stop > 0 ? p.tail_h0 : p.h0, p.final_state, stream);
  }
  return hipGetLastError();
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
