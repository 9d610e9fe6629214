// scan_cplx.hip -- selective-scan forward with a complex diagonal A, gfx950.
//
// Per channel (b, d), time t and state n, in complex arithmetic:
//   A[n]  = -exp(A_log[d,n]) + i A_imag[d,n]
//   a_t   = exp(delta_t A[n])
//         = 2^(delta_t Re(A) log2 e) (cos(delta_t Im A) + i sin(delta_t Im A))
//   h_t   = a_t h_(t-1) + delta_t u_t B_t[n]
//   out_t = (Re(sum_n C_t[n] h_t[n]) + D u_t) silu(z_t)
// The pages note that the official CUDA kernel carries a complex-A variant
// with its own complex exp2 ("createcentury" post on the kernel, section
// "主要な最適化テクニック"); delta, the skip term and the gate are the real
// forward's (see scan_fwd.hip).
//
// Mapping: a workgroup of 256 lanes covers 16 channels of one batch row, one
// lane per (channel, state): a 16-lane DPP row holds one channel, and
// Re(C . h) is a DPP reduction inside the row, four time steps at a time
// (row_sum16_x4).  Time is walked in
// chunks of kCxT steps:
//   E  B and C of the chunk (16 states x kCxT steps, shared by the 16
//      channels) and, per element, (delta, delta u) into LDS, from registers
//      loaded during the previous chunk (u, delta_raw, z, B and C of chunk
//      c+1 are in flight while chunk c is scanned);
//   S  each lane walks the chunk: the complex decay from exp2, and from the
//      hardware sin / cos of the fractional turns delta Im(A) / 2 pi (the
//      fraction keeps v_sin / v_cos inside their input range); one complex
//      multiply-add; the row sums of Re(C h), four steps per reduction,
//      land in LDS;
//   O  out = (y + D u) silu(z), one store per element.
// The state never leaves the registers.  Lanes past dstate hold zeros.
//
// Few channels with a long sequence leave most of the GPU idle (16 channels
// per workgroup), so such shapes are cut into time segments, as the real
// forward does ("mamba-metal", section "チャンク間 running prefix"): an
// aggregate pass (AGG) walks every segment but the last from a zero state
// and records, per (channel, state), the segment's pair (prod_t a_t, h_end);
// carry_cplx_kernel composes the pairs in order with the pair operator
// (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2) in complex arithmetic; the main
// pass starts every segment from its carry.  The product of the decays is
// exp(A sum_t delta_t): its modulus comes from the sum of the deltas, and its
// phase from the per-step turns accumulated modulo one turn (a sum of the
// deltas times Im(A) would lose the phase to rounding over long segments).
#include <algorithm>

#include "mss_device.hpp"
#include "mss_internal.hpp"
#include "mss_cplx.hpp"

namespace mss {
namespace {

constexpr float kInv2Pi = 0.15915494309189535f;

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Totals over a 16-lane DPP row of four values per lane, for four steps at
// once: lanes 4q..4q+3 of the row (rl = lane within the row) receive the
// total of v_q.  Level 1, row_ror:8 (lane l meets l ^ 8): the lower half
// keeps (v0, v1) and sends (v2, v3), the upper half the reverse; level 2,
// row_half_mirror (l meets l ^ 7): lanes with l % 8 < 4 keep the first of
// their pair; levels 3 and 4: butterflies inside each quad.  Six selects
// and five adds, against sixteen adds for four separate row sums.
__device__ inline float row_sum16_x4(float v0, float v1, float v2, float v3, int rl) {
  const bool up = (rl & 8) != 0;
  const float w0 = (up ? v2 : v0) + dpp<0x128>(up ? v0 : v2);
  const float w1 = (up ? v3 : v1) + dpp<0x128>(up ? v1 : v3);
  const bool second = (rl & 4) != 0;
  float x = (second ? w1 : w0) + dpp<0x141>(second ? w0 : w1);
  x += dpp<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  x += dpp<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  return x;
}
constexpr int kCxPer = kCxCh * kCxT / kCxThreads;  // elements per lane in E and O (2)

constexpr int kXcds = 8;  // MI355X: 8 accelerator dies

// XR / BR: u, delta_raw (z, out) / B, C have unit stride along their rows
// (channels / states), and their elements are read rows-fastest.
template <bool AGG, bool XR, bool BR>
__global__ __launch_bounds__(kCxThreads) void scan_cplx_kernel(CplxShape s, CplxPtrs p) {
  __shared__ float2 s_B[kMaxState][kCxT + 1];
  __shared__ float2 s_C[AGG ? 1 : kMaxState][kCxT + 1];
  __shared__ float2 s_dd[kCxCh][kCxT + 1];  // (delta, delta * u)
  __shared__ float s_y[AGG ? 1 : kCxCh][kCxT + 1];

  const int tid = threadIdx.x;
  // Workgroups are dispatched round-robin over the XCDs; renumber them so
  // that each XCD takes a contiguous range of tiles (tiles of one batch row
  // share B and C in that XCD's L2).  Tile i of a pass is channel tile i % T
  // of time segment i / T.
  const int nwg = static_cast<int>(gridDim.x), lin = static_cast<int>(blockIdx.x);
  const int xcd = lin % kXcds, per_xcd = nwg / kXcds, extra = nwg % kXcds;
  const int logical = xcd * per_xcd + min(xcd, extra) + lin / kXcds;
  const int T = s.batch * s.tiles;
  const int tile = logical % T, seg = logical / T;
  const int b = tile / s.tiles;
  const int d0 = (tile % s.tiles) * kCxCh;
  const int t_begin = seg * s.seg_len;
  const int t_end = min(s.seqlen, t_begin + s.seg_len);

  // scan role: lane (c, n) = (tid / 16, tid % 16)
  const int c = tid >> 4, n = tid & (kMaxState - 1);
  const int d = d0 + c;
  const bool active = d < s.dim && n < s.dstate;
  const int64_t ws_row = (static_cast<int64_t>(tile) * kCxCh + c) * kMaxState + n;
  float ar2 = 0.0f, ai = 0.0f, hr = 0.0f, hi = 0.0f;
  if (active) {
    ar2 = -expf(p.A_log[d * s.sA[0] + n * s.sA[1]]) * kLog2e;  // Re(A) log2 e
    ai = p.A_imag[d * s.sAi[0] + n * s.sAi[1]] * kInv2Pi;      // Im(A) in turns
    if (!AGG) {
      if (seg > 0) {
        const float2 v = p.carry[static_cast<int64_t>(seg) * s.nchan_pad * kMaxState + ws_row];
        hr = v.x;
        hi = v.y;
      } else if (p.h0 != nullptr) {
        const float2 v = p.h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n];
        hr = v.x;
        hi = v.y;
      }
    }
  }
  float sum_delta = 0.0f, turns_acc = 0.0f;  // AGG: the segment's sum of delta, turns mod 1

  // element roles: element e = tid + kCxThreads j of the 16-row x kCxT-step
  // tile; rows are channels for u, delta, z, out and states for B, C.  Steps
  // run fastest over the lanes when the data has unit stride along time;
  // rows run fastest when it has unit stride along them (channel-last
  // activations, n-fast B/C), so that 16 lanes read one step's 16 adjacent
  // channels or states instead of 16 separate lines.
  int erow[kCxPer], estep[kCxPer], brow[kCxPer], bstep[kCxPer];
  float ebias[kCxPer], eskip[kCxPer];
#pragma unroll
  for (int j = 0; j < kCxPer; ++j) {
    const int e = tid + kCxThreads * j;
    erow[j] = XR ? e % kCxCh : e / kCxT;
    estep[j] = XR ? e / kCxCh : e % kCxT;
    brow[j] = BR ? e % kMaxState : e / kCxT;
    bstep[j] = BR ? e / kMaxState : e % kCxT;
    const int dd = d0 + erow[j];
    const bool ok = dd < s.dim;
    ebias[j] = (ok && p.dt_bias != nullptr) ? p.dt_bias[dd] : 0.0f;
    eskip[j] = (ok && p.D != nullptr) ? p.D[dd] : 0.0f;
  }

  // The raw inputs of a chunk, loaded one chunk ahead of use: the loads of
  // chunk c+1 are in flight while chunk c is scanned.
  float2 rb[kCxPer], rc[kCxPer];
  float rx[kCxPer], ru[kCxPer], rz[kCxPer];
  auto load_chunk = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kCxPer; ++j) {
      const int tb = t0 + bstep[j];
      const int ns = brow[j];
      const bool bok = tb < t_end && ns < s.dstate;
      rb[j] = bok ? p.B[b * s.sB[0] + ns * s.sB[1] + tb * s.sB[2]] : make_float2(0.0f, 0.0f);
      rc[j] = (!AGG && bok) ? p.C[b * s.sC[0] + ns * s.sC[1] + tb * s.sC[2]]
                            : make_float2(0.0f, 0.0f);
      const int t = t0 + estep[j];
      const int dd = d0 + erow[j];
      const bool xok = t < t_end && dd < s.dim;
      rx[j] = xok ? p.delta_raw[b * s.sd[0] + dd * s.sd[1] + t * s.sd[2]] : 0.0f;
      ru[j] = xok ? p.u[b * s.su[0] + dd * s.su[1] + t * s.su[2]] : 0.0f;
      rz[j] = (!AGG && xok && p.z != nullptr) ? p.z[b * s.sz[0] + dd * s.sz[1] + t * s.sz[2]]
                                             : 0.0f;
    }
  };
  load_chunk(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kCxT) {
    float eu[kCxPer], ez[kCxPer];
    // ---- E ----
#pragma unroll
    for (int j = 0; j < kCxPer; ++j) {
      ez[j] = rz[j];
      s_B[brow[j]][bstep[j]] = rb[j];
      if constexpr (!AGG) s_C[brow[j]][bstep[j]] = rc[j];
      const int t = t0 + estep[j];
      const bool xok = t < t_end && d0 + erow[j] < s.dim;
      const float x = rx[j] + ebias[j];
      const float dl = xok ? (s.softplus ? softplus(x) : x) : 0.0f;
      eu[j] = ru[j];
      s_dd[erow[j]][estep[j]] = make_float2(dl, dl * ru[j]);
    }
    load_chunk(t0 + kCxT);
    __syncthreads();
    // ---- S ----
#pragma unroll 2
    for (int t4 = 0; t4 < kCxT; t4 += 4) {
      float yv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 dd = s_dd[c][t4 + i];
        const float2 bb = s_B[n][t4 + i];
        const float turns = __builtin_amdgcn_fractf(dd.x * ai);
        const float m = fast_exp2(dd.x * ar2);
        const float a_r = m * __builtin_amdgcn_cosf(turns);
        const float a_i = m * __builtin_amdgcn_sinf(turns);
        const float nr = fmaf(a_r, hr, fmaf(-a_i, hi, dd.y * bb.x));
        const float ni = fmaf(a_r, hi, fmaf(a_i, hr, dd.y * bb.y));
        hr = nr;
        hi = ni;
        if constexpr (AGG) {
          turns_acc = __builtin_amdgcn_fractf(turns_acc + turns);
        } else {
          const float2 cc = s_C[n][t4 + i];
          yv[i] = fmaf(cc.x, hr, -cc.y * hi);
        }
      }
      if constexpr (!AGG) {
        const float y = row_sum16_x4(yv[0], yv[1], yv[2], yv[3], n);
        if ((n & 3) == 0) s_y[c][t4 + (n >> 2)] = y;
      }
    }
    if constexpr (AGG) {
      // The segment's sum of delta, split over the channel's 16 lanes: lane n
      // adds steps n and n + 16 of each chunk, and the row sums the partial
      // sums at the segment end (every lane had added all 32 steps).
      static_assert(kCxT == 2 * kMaxState, "two steps per lane and chunk");
      sum_delta += s_dd[c][n].x + s_dd[c][n + kMaxState].x;
    }
    __syncthreads();
    if constexpr (AGG) continue;  // the next chunk's E phase follows the barrier
    // ---- O ----
#pragma unroll
    for (int j = 0; j < kCxPer; ++j) {
      const int t = t0 + estep[j];
      const int dd = d0 + erow[j];
      if (t < t_end && dd < s.dim) {
        float y = fmaf(eskip[j], eu[j], s_y[erow[j]][estep[j]]);
        if (p.z != nullptr) y *= silu(ez[j]);
        p.out[b * s.so[0] + dd * s.so[1] + t * s.so[2]] = y;
      }
    }
  }
  if constexpr (AGG) {
    // (prod_t a_t, h from zero) of the segment; lanes outside the tensors
    // record the identity pair ((1, 0), (0, 0))
    const float m = fast_exp2(ar2 * row_sum16(sum_delta));
    p.agg[static_cast<int64_t>(seg) * s.nchan_pad * kMaxState + ws_row] =
        make_float4(m * __builtin_amdgcn_cosf(turns_acc), m * __builtin_amdgcn_sinf(turns_acc),
                    hr, hi);
  } else if (active && p.final_state != nullptr && seg == s.nseg - 1) {
    p.final_state[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n] = make_float2(hr, hi);
  }
}

// carry[k] = complex state entering segment k: carry[0] = h0 (or 0),
// carry[k+1] = P[k] carry[k] + H[k].  One lane per (channel, state); the
// chain is walked in ranges of segments, one wave each
// (walk_chain_in_ranges), at most kCarryWavesCx waves: a range held in
// registers is kCarryBatch complex links, 64 registers, and 16 waves per
// workgroup would leave 128 registers per lane.
constexpr int kCarryWavesCx = 8;
__global__ __launch_bounds__(64 * kCarryWavesCx) void carry_cplx_kernel(
    CplxShape s, const float4* __restrict__ agg, const float2* __restrict__ h0,
    float2* __restrict__ carry) {
  __shared__ float4 xch[kCarryWavesCx][64];
  const int64_t sstride = s.nchan_pad * kMaxState;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x % 64;
  const bool valid = idx < sstride;
  const int64_t ic = valid ? idx : 0;
  float2 c = make_float2(0.0f, 0.0f);
  if (valid && h0 != nullptr) {
    const int n = static_cast<int>(idx % kMaxState);
    const int64_t row = idx / kMaxState;
    const int64_t per_b = static_cast<int64_t>(s.tiles) * kCxCh;
    const int b = static_cast<int>(row / per_b);
    const int d = static_cast<int>(row % per_b);
    if (d < s.dim && n < s.dstate) c = h0[(static_cast<int64_t>(b) * s.dim + d) * s.dstate + n];
  }
  walk_chain_in_ranges(
      s.nseg - 1, c, valid, xch, [&](int k) { return agg[k * sstride + ic]; },
      [&](int k, float2 v) { carry[(k + 1) * sstride + idx] = v; });
}

template <bool XR, bool BR>
void launch_complex_passes(const CplxShape& s, const CplxPtrs& p, hipStream_t stream) {
  const unsigned tiles = static_cast<unsigned>(static_cast<int64_t>(s.batch) * s.tiles);
  if (s.nseg > 1) {
    scan_cplx_kernel<true, XR, BR><<<dim3(tiles * static_cast<unsigned>(s.nseg - 1)),
                                     dim3(kCxThreads), 0, stream>>>(s, p);
    const int64_t lanes = s.nchan_pad * kMaxState;
    carry_cplx_kernel<<<dim3(static_cast<unsigned>((lanes + 63) / 64)),
                        dim3(64 * std::min(carry_waves(s.nseg), kCarryWavesCx)), 0, stream>>>(
        s, p.agg, p.h0, p.carry);
  }
  scan_cplx_kernel<false, XR, BR><<<dim3(tiles * static_cast<unsigned>(s.nseg)), dim3(kCxThreads),
                                    0, stream>>>(s, p);
}

}  // namespace

hipError_t launch_scan_complex(const CplxShape& s, const CplxPtrs& p, hipStream_t stream) {
  const bool xr = s.su[1] == 1 && s.sd[1] == 1;
  const bool br = s.sB[1] == 1 && s.sC[1] == 1;
  if (xr && br) launch_complex_passes<true, true>(s, p, stream);
  else if (xr) launch_complex_passes<true, false>(s, p, stream);
  else if (br) launch_complex_passes<false, true>(s, p, stream);
  else launch_complex_passes<false, false>(s, p, stream);
  return hipGetLastError();
}

}  // namespace mss
