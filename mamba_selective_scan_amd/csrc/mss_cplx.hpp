// mss_cplx.hpp -- parameter blocks and the launch entry point of the
// complex-A forward, shared by the host layer (mss_api.hip) and its kernel
// translation unit (scan_cplx.hip).
#pragma once

#include "mss_internal.hpp"

namespace mss {

// Selective-scan forward with complex diagonal A (fp32 activations, complex64
// B, C and states).  A workgroup of kCxThreads lanes covers kCxCh channels of
// one batch row, one lane per (channel, state), and walks time in chunks of
// kCxT steps.
constexpr int kCxT = 32;
constexpr int kCxThreads = 256;
constexpr int kCxCh = kCxThreads / kMaxState;  // 16

struct CplxShape {
  int batch, dim, seqlen, dstate;
  int softplus;
  int tiles;                               // ceil(dim / kCxCh)
  int nseg, seg_len;                       // time segments (seg_len a multiple of kCxT)
  int64_t nchan_pad;                       // batch * tiles * kCxCh: rows of the workspace arrays
  int64_t su[3], sd[3], sz[3], so[3];      // (b, d, t), fp32 elements
  int64_t sB[3], sC[3];                    // (b, n, t), complex elements
  int64_t sA[2], sAi[2];                   // A_log, A_imag: (d, n)
};

struct CplxPtrs {
  const float* u;
  const float* delta_raw;
  const float* A_log;
  const float* A_imag;
  const float2* B;
  const float2* C;
  const float* D;
  const float* z;
  const float* dt_bias;
  const float2* h0;
  float* out;
  float2* final_state;
  // workspace (time segments only)
  float4* agg;    // [nseg-1][nchan_pad][kMaxState] per segment (prod a: re, im; h from 0: re, im)
  float2* carry;  // [nseg][nchan_pad][kMaxState] complex state entering each segment
};

hipError_t launch_scan_complex(const CplxShape& s, const CplxPtrs& p, hipStream_t stream);

}  // namespace mss
