// mss_api.hip -- the C ABI of libmss: argument checks, launch planning and
// stream-ordered enqueue.  Every check runs on the host before any HIP call,
// so an invalid call launches nothing and touches no memory.  There is one
// execution path per operation and no fallback.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mss.h"
#include "mss_internal.hpp"
#include "mss_cplx.hpp"

namespace {

using mss::kCh;
using mss::kMaxState;
using mss::kT;

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxSeqlen = int64_t{1} << 30;  // time indices, padded, stay in int32
// Time segments: a shape whose channel tiles alone give fewer than
// kSplitBelowTiles waves is split along time into as many segments as keep
// the waves at or below kTargetTiles, four per SIMD: rounding up instead
// would leave a few SIMDs with a fifth wave and the rest waiting on them.
// The plan depends only on the shape, so results do not depend on the device.
constexpr int64_t kSplitBelowTiles = 2048;
constexpr int64_t kTargetTiles = 4096;
// The aggregate pass (every segment but the last, no C, z or output) needs
// about 60 VGPRs, so eight of its waves fit a SIMD where the main pass holds
// four or five.  It cuts every segment into parts, as many as bring its grid
// to at most kAggWaves waves (counting whole 32-channel blocks, so that both
// layouts get the same plan), with parts of at least kAggMinPartChunks
// chunks and at most mss::kMaxAggSplit parts; the carry pass composes the
// parts.
constexpr int64_t kAggWaves = 8 * 1024;
constexpr int64_t kAggMinPartChunks = 4;

struct Extent {
  uintptr_t lo = 0, hi = 0;  // byte range [lo, hi)
  bool valid = false;
};

Extent extent_of(const void* p, const int64_t* sizes, const int64_t* strides, int rank,
                 int64_t elem) {
  Extent e;
  if (p == nullptr) return e;
  int64_t span = 0;
  for (int i = 0; i < rank; ++i) span += (sizes[i] - 1) * strides[i];
  e.lo = reinterpret_cast<uintptr_t>(p);
  e.hi = e.lo + static_cast<uintptr_t>((span + 1) * elem);
  e.valid = true;
  return e;
}

// Bytes of the chunk-state array: [ceil(L / 16)][batch][dim][16] fp32.
Extent chunk_states_extent(const void* p, int64_t batch, int64_t dim, int64_t seqlen) {
  Extent e;
  if (p == nullptr) return e;
  const int64_t nq = (seqlen + mss::kStateChunk - 1) / mss::kStateChunk;
  e.lo = reinterpret_cast<uintptr_t>(p);
  e.hi = e.lo + static_cast<uintptr_t>(nq * batch * dim * kMaxState * 4);
  e.valid = true;
  return e;
}

bool overlaps(const Extent& a, const Extent& b) {
  return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, int64_t a) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(a)) == 0;
}

void norm_strides(int64_t* out, const int64_t* st, const int64_t* sizes) {
  for (int i = 0; i < 3; ++i) out[i] = sizes[i] == 1 ? 1 : st[i];
}

bool strides_nonneg(const int64_t* st, int rank) {
  for (int i = 0; i < rank; ++i)
    if (st[i] < 0) return false;
  return true;
}

// Distinct indices map to distinct elements (needed for outputs only).
bool non_overlapping(const int64_t* sizes, const int64_t* strides, int rank) {
  int idx[3] = {0, 1, 2};
  std::sort(idx, idx + rank, [&](int a, int b) { return strides[a] < strides[b]; });
  int64_t need = 1;
  for (int k = 0; k < rank; ++k) {
    const int i = idx[k];
    if (sizes[i] == 1) continue;
    if (strides[i] < need) return false;
    need = strides[i] * sizes[i];
  }
  return true;
}

// Each kCh-channel x kT-step tile (16-state x kT-step for B and C) is
// addressed with 32-bit byte offsets from a per-tile base.
bool tile_offsets_fit(const int64_t* st, int64_t elem, int64_t rows = kCh) {
  const int64_t span = ((rows - 1) * st[1] + (kT - 1) * st[2] + 1) * elem;
  return span < (int64_t{1} << 31);
}

struct ScanPlan {
  mss::ScanShape shape;
  size_t agg_bytes = 0, carry_bytes = 0, tail_bytes = 0, workspace = 0;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// elements per load/store vector (16 bytes of fp32, 8 bytes of bf16)
int vec_elems(int32_t) { return mss::kVec; }

mss_status check_shape(const mss_scan_args* a) {
  if (a == nullptr || a->struct_size != sizeof(mss_scan_args) || (a->reverse & ~1) != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->io_dtype != MSS_F32 && a->io_dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED_DTYPE;
  if (a->batch < 1 || a->dim < 1 || a->seqlen < 1) return MSS_ERR_BAD_SHAPE;
  if (a->batch > kMaxDim || a->dim > kMaxDim || a->seqlen > kMaxSeqlen) return MSS_ERR_BAD_SHAPE;
  if (a->dstate < 1 || a->dstate > MSS_MAX_DSTATE) return MSS_ERR_UNSUPPORTED_DSTATE;
  // batch * ceil(dim/kCh) workgroups in grid x; batch * dim * dstate states
  const int64_t groups = (a->dim + kCh - 1) / kCh;
  if (a->batch * groups > kMaxDim) return MSS_ERR_BAD_SHAPE;
  if (a->batch * a->dim > kMaxDim) return MSS_ERR_BAD_SHAPE;
  return MSS_OK;
}

ScanPlan make_plan(const mss_scan_args* a) {
  ScanPlan p;
  mss::ScanShape& s = p.shape;
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.seqlen = static_cast<int>(a->seqlen);
  s.dstate = static_cast<int>(a->dstate);
  s.groups = static_cast<int>((a->dim + kCh - 1) / kCh);
  const int64_t tiles = a->batch * s.groups;
  const int64_t chunks = (a->seqlen + kT - 1) / kT;
  int64_t nseg = 1;
  if (tiles < kSplitBelowTiles) nseg = std::max<int64_t>(1, std::min<int64_t>(kTargetTiles / tiles, chunks));
  nseg = std::min<int64_t>(nseg, 65535);
  const int64_t seg_chunks = (chunks + nseg - 1) / nseg;
  s.seg_len = static_cast<int>(seg_chunks * kT);
  s.nseg = static_cast<int>((a->seqlen + s.seg_len - 1) / s.seg_len);
  s.agg_split = 1;
  if (s.nseg > 1) {
    const int64_t blocks = a->batch * ((s.groups + 3) / 4) * 4 * (s.nseg - 1);
    s.agg_split = static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>({kAggWaves / blocks, seg_chunks / kAggMinPartChunks,
                              int64_t{mss::kMaxAggSplit}})));
  }
  s.part_len = static_cast<int>((seg_chunks + s.agg_split - 1) / s.agg_split * kT);
  s.nchan_pad = tiles * kCh;
  s.softplus = a->delta_softplus ? 1 : 0;
  s.reverse = a->reverse;
  s.t_first = 0;
  s.t_stop = s.seqlen;
  if (s.nseg > 1) {
    p.agg_bytes = round_up(static_cast<size_t>(s.nseg - 1) * s.agg_split * s.nchan_pad *
                               kMaxState * sizeof(float2), 256);
    p.carry_bytes = round_up(static_cast<size_t>(s.nseg) * s.nchan_pad * kMaxState * sizeof(float), 256);
  }
  // a sequence that does not end on a vector boundary ends with an
  // element-wise pass that starts from a state handed over in the workspace
  if (a->seqlen % vec_elems(a->io_dtype) != 0)
    p.tail_bytes = round_up(static_cast<size_t>(a->batch * a->dim * a->dstate) * sizeof(float), 256);
  p.workspace = p.agg_bytes + p.carry_bytes + p.tail_bytes;
  return p;
}

// Conv strides with every size-1 dimension's stride set to 0: such a dimension
// is never stepped, so its stride must not decide the path.
void conv_strides(int64_t* out, const int64_t* st, const int64_t* sizes, int rank) {
  for (int i = 0; i < rank; ++i) out[i] = sizes[i] == 1 ? 0 : st[i];
}

bool all_mult(const int64_t* st, int rank, int64_t m, int skip) {
  for (int i = 0; i < rank; ++i)
    if (i != skip && st[i] % m != 0) return false;
  return true;
}

// Backward plan: workspace = checkpoints, dB/dC partials, per-row sums.
struct BwdPlan {
  mss::BwdShape shape;
  size_t ckpt_bytes = 0, bc_bytes = 0, chan_bytes = 0, agg_bytes = 0, carry_bytes = 0;
  size_t workspace = 0;
};

// Backward time segments: a shape with fewer (row, channel tile) pairs than
// the reverse walk's resident workgroups (three per CU on 256 CUs) is split
// along time until it fills them, with segments of at least kBwdMinSegChunks
// chunks.
constexpr int64_t kBwdSplitBelow = 768;
constexpr int64_t kBwdMinSegChunks = 8;
// The segment aggregate pass runs one wave per (row, 8 channels, segment),
// three per SIMD at the split above, where its registers (about 80 with the
// forward's chunk states given, 100 without) leave room for six or five: it
// then cuts every segment into parts, as many as bring its grid to that many
// waves (the carry pass composes the parts), with parts of at least
// kBwdMinSegChunks chunks (shorter ones lost more to the longer carry chain
// than they gained: the 130m-layer shape, 8-chunk segments).  The count is a
// power of two, so that the carry pass finds segment boundaries with a mask.
constexpr int64_t kBwdAggWavesGiven = 6 * 1024;
constexpr int64_t kBwdAggWavesFull = 5 * 1024;
int bwd_agg_split(const mss::BwdShape& s, bool states_given) {
  const int64_t base = static_cast<int64_t>(s.batch) * s.tiles * mss::kBwdWaves * s.nseg;
  const int64_t k = std::min<int64_t>((states_given ? kBwdAggWavesGiven : kBwdAggWavesFull) / base,
                                      s.seg_chunks / kBwdMinSegChunks);
  int split = 1;
  while (2 * split <= k) split *= 2;
  return split;
}

mss_status check_bwd_shape(const mss_scan_bwd_args* a) {
  if (a == nullptr || a->struct_size != sizeof(mss_scan_bwd_args) || (a->reverse & ~1) != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->io_dtype != MSS_F32 && a->io_dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED_DTYPE;
  if (a->batch < 1 || a->dim < 1 || a->seqlen < 1 || a->batch > kMaxDim || a->dim > kMaxDim ||
      a->seqlen > kMaxSeqlen || a->batch * a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->dstate < 1 || a->dstate > MSS_MAX_DSTATE) return MSS_ERR_UNSUPPORTED_DSTATE;
  const int64_t tiles = (a->dim + mss::kBwdCh - 1) / mss::kBwdCh;
  if (a->batch * tiles * mss::kBwdWaves > 0xFFFFFFFFll) return MSS_ERR_BAD_SHAPE;
  // the dB/dC sum's grid: 256-thread blocks over batch x 2 x 16 states x
  // the step quads of whole partial rows, then the parameter sums' blocks
  // (written as a division: the product of the largest allowed sizes
  // overflows)
  const int64_t row_steps = 2 * mss::kBwdT;
  const int64_t quads = (a->seqlen + row_steps - 1) / row_steps * (row_steps / mss::kBcSteps);
  const int64_t fin_blocks = (a->dim * (mss::kMaxState + 2) + 255) / 256;
  if (a->batch > ((int64_t{0xFFFFFFFF} - fin_blocks) * 256) / (2 * mss::kMaxState * quads))
    return MSS_ERR_BAD_SHAPE;
  return MSS_OK;
}

BwdPlan make_bwd_plan(const mss_scan_bwd_args* a) {
  BwdPlan p;
  mss::BwdShape& s = p.shape;
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.seqlen = static_cast<int>(a->seqlen);
  s.dstate = static_cast<int>(a->dstate);
  s.softplus = a->delta_softplus ? 1 : 0;
  s.nchunk = static_cast<int>((a->seqlen + mss::kBwdT - 1) / mss::kBwdT);
  s.npair = (s.nchunk + 1) / 2;
  s.tiles = static_cast<int>((a->dim + mss::kBwdCh - 1) / mss::kBwdCh);
  s.nchan_pad = a->batch * s.tiles * mss::kBwdCh;
  s.reverse = a->reverse;
  const int64_t pairs = a->batch * s.tiles;
  int64_t nseg = 1;
  if (pairs < kBwdSplitBelow)
    nseg = std::min<int64_t>((kBwdSplitBelow + pairs - 1) / pairs,
                             std::max<int64_t>(1, s.nchunk / kBwdMinSegChunks));
  s.seg_chunks = static_cast<int>((s.nchunk + nseg - 1) / nseg);
  s.nseg = (s.nchunk + s.seg_chunks - 1) / s.seg_chunks;
  // checkpoints in the chunk-state layout (unused when the caller passes them)
  p.ckpt_bytes = round_up(static_cast<size_t>(s.nchunk) * a->batch * a->dim * kMaxState * sizeof(float), 256);
  p.bc_bytes = round_up(static_cast<size_t>(a->batch) * s.tiles * 2 * kMaxState * s.npair * 2 *
                            mss::kBwdT * sizeof(float), 256);
  p.chan_bytes = round_up(static_cast<size_t>(s.nseg) * a->batch * a->dim * (kMaxState + 2) * sizeof(float), 256);
  s.agg_split = 1;
  if (s.nseg > 1) {
    // sized for the larger split, so that the workspace does not depend on
    // whether the forward's chunk states are passed
    const int split = std::max(bwd_agg_split(s, true), bwd_agg_split(s, false));
    p.agg_bytes = round_up(static_cast<size_t>(s.nseg) * split * s.nchan_pad * kMaxState * sizeof(float4), 256);
    p.carry_bytes = round_up(static_cast<size_t>(s.nseg) * s.nchan_pad * kMaxState * sizeof(float), 256);
  }
  p.workspace = p.ckpt_bytes + p.bc_bytes + p.chan_bytes + p.agg_bytes + 2 * p.carry_bytes;
  return p;
}

// Channel-fast conv: time segments per 256-channel group so that the grid
// holds about this many waves.
constexpr int64_t kConvTargetWaves = 4096;
constexpr int64_t kConvMinSeg = 64;

// Complex-A forward: shapes with fewer channel tiles (16 channels each) than
// kCxSplitBelow are cut into time segments, as many as bring the grid to about
// kCxTargetWgs workgroups: five 4-wave workgroups per CU, as many as the
// kernel's registers (up to 100 with the chunk loads in flight) let a CU hold.
constexpr int64_t kCxSplitBelow = 512;
constexpr int64_t kCxTargetWgs = 1280;

mss_status check_cplx_shape(const mss_scan_complex_args* a) {
  if (a == nullptr || a->struct_size != sizeof(mss_scan_complex_args) || a->reserved0 != 0 ||
      a->reserved1 != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->batch < 1 || a->dim < 1 || a->seqlen < 1 || a->batch > kMaxDim || a->dim > kMaxDim ||
      a->seqlen > kMaxSeqlen || a->batch * a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->dstate < 1 || a->dstate > MSS_MAX_DSTATE) return MSS_ERR_UNSUPPORTED_DSTATE;
  const int64_t tiles = (a->dim + mss::kCxCh - 1) / mss::kCxCh;
  if (a->batch * tiles > 0x7FFFFFFFll) return MSS_ERR_BAD_SHAPE;
  return MSS_OK;
}

struct CplxPlan {
  mss::CplxShape shape;
  size_t agg_bytes = 0, carry_bytes = 0, workspace = 0;
};

CplxPlan make_cplx_plan(const mss_scan_complex_args* a) {
  CplxPlan p;
  mss::CplxShape& s = p.shape;
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.seqlen = static_cast<int>(a->seqlen);
  s.dstate = static_cast<int>(a->dstate);
  s.softplus = a->delta_softplus ? 1 : 0;
  s.tiles = static_cast<int>((a->dim + mss::kCxCh - 1) / mss::kCxCh);
  const int64_t total = a->batch * s.tiles;
  const int64_t chunks = (a->seqlen + mss::kCxT - 1) / mss::kCxT;
  int64_t nseg = 1;
  if (total < kCxSplitBelow) nseg = std::max<int64_t>(1, std::min<int64_t>(kCxTargetWgs / total, chunks));
  const int64_t seg_chunks = (chunks + nseg - 1) / nseg;
  s.seg_len = static_cast<int>(seg_chunks * mss::kCxT);
  s.nseg = static_cast<int>((a->seqlen + s.seg_len - 1) / s.seg_len);
  s.nchan_pad = total * mss::kCxCh;
  if (s.nseg > 1) {
    p.agg_bytes = round_up(static_cast<size_t>(s.nseg - 1) * s.nchan_pad * kMaxState * sizeof(float4), 256);
    p.carry_bytes = round_up(static_cast<size_t>(s.nseg) * s.nchan_pad * kMaxState * sizeof(float2), 256);
  }
  p.workspace = p.agg_bytes + p.carry_bytes;
  return p;
}

// ---- device scratch of the no-allocation forward --------------------------
// mss_selective_scan_fwd_noalloc keeps its time-segment carries and ragged-tail
// hand-off in this array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy from the first call on it until the
// process ends, and every call on that GPU shares it.  In host code `scratch`
// only names the symbol: its device address comes from hipGetSymbolAddress,
// once per device, and that address is what the kernels receive.
constexpr size_t kScratchBytes = MSS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the device that `stream` belongs to.
mss_status scratch_address(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return MSS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MSS_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MSS_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MSS_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return MSS_ERR_HIP;
    g_scratch_addr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_addr[dev];
  return MSS_OK;
}

// The scan forward.  noalloc: the workspace is this library's device array
// `scratch` instead of the caller's (args->workspace must then be NULL).
mss_status scan_fwd(const mss_scan_args* a, void* stream, bool noalloc) {
  mss_status st = check_shape(a);
  if (st != MSS_OK) return st;
  if (a->u == nullptr || a->delta_raw == nullptr || a->A_log == nullptr || a->B == nullptr ||
      a->C == nullptr || a->out == nullptr)
    return MSS_ERR_NULL_POINTER;
  const int64_t es = a->io_dtype == MSS_BF16 ? 2 : 4;
  const int64_t xs[3] = {a->batch, a->dim, a->seqlen};
  const int64_t bcs[3] = {a->batch, a->dstate, a->seqlen};
  const int64_t as[2] = {a->dim, a->dstate};
  const int64_t vs[1] = {a->dim};
  const int64_t ss[3] = {a->batch, a->dim, a->dstate};
  const int64_t unit[3] = {a->dim * a->dstate, a->dstate, 1};
  const int64_t one[1] = {1};
  // strides
  if (!strides_nonneg(a->u_stride, 3) || !strides_nonneg(a->delta_stride, 3) ||
      !strides_nonneg(a->B_stride, 3) || !strides_nonneg(a->C_stride, 3) ||
      !strides_nonneg(a->out_stride, 3) || !strides_nonneg(a->A_log_stride, 2) ||
      (a->z != nullptr && !strides_nonneg(a->z_stride, 3)))
    return MSS_ERR_BAD_STRIDE;
  if (!non_overlapping(xs, a->out_stride, 3)) return MSS_ERR_BAD_STRIDE;
  if (!tile_offsets_fit(a->u_stride, es) || !tile_offsets_fit(a->delta_stride, es) ||
      !tile_offsets_fit(a->out_stride, es) || (a->z != nullptr && !tile_offsets_fit(a->z_stride, es)) ||
      !tile_offsets_fit(a->B_stride, es, kMaxState) || !tile_offsets_fit(a->C_stride, es, kMaxState))
    return MSS_ERR_BAD_STRIDE;
  // alignment
  if (!aligned(a->u, es) || !aligned(a->delta_raw, es) || !aligned(a->B, es) ||
      !aligned(a->C, es) || !aligned(a->z, es) || !aligned(a->out, es) || !aligned(a->A_log, 4) ||
      !aligned(a->D, 4) || !aligned(a->dt_bias, 4) || !aligned(a->initial_state, 4) ||
      !aligned(a->final_state, 4) || !aligned(a->chunk_states, 8))
    return MSS_ERR_MISALIGNED;
  // aliasing: outputs against every input and each other
  const Extent ins[] = {
      extent_of(a->u, xs, a->u_stride, 3, es),
      extent_of(a->delta_raw, xs, a->delta_stride, 3, es),
      extent_of(a->z, xs, a->z_stride, 3, es),
      extent_of(a->B, bcs, a->B_stride, 3, es),
      extent_of(a->C, bcs, a->C_stride, 3, es),
      extent_of(a->A_log, as, a->A_log_stride, 2, 4),
      extent_of(a->D, vs, one, 1, 4),
      extent_of(a->dt_bias, vs, one, 1, 4),
      extent_of(a->initial_state, ss, unit, 3, 4),
  };
  const Extent eo = extent_of(a->out, xs, a->out_stride, 3, es);
  const Extent ef = extent_of(a->final_state, ss, unit, 3, 4);
  const Extent ecs = chunk_states_extent(a->chunk_states, a->batch, a->dim, a->seqlen);
  for (const Extent& e : ins)
    if (overlaps(eo, e) || overlaps(ef, e) || overlaps(ecs, e)) return MSS_ERR_ALIASING;
  if (overlaps(eo, ef) || overlaps(ecs, eo) || overlaps(ecs, ef)) return MSS_ERR_ALIASING;

  const ScanPlan plan = make_plan(a);
  mss::ScanPtrs p{};
  if (noalloc) {
    if (a->workspace != nullptr || a->workspace_bytes != 0) return MSS_ERR_BAD_STRUCT;
    if (plan.workspace > kScratchBytes) return MSS_ERR_SCRATCH_LIMIT;
  } else if (plan.workspace > 0) {
    if (a->workspace == nullptr || a->workspace_bytes < plan.workspace)
      return MSS_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(a->workspace, 256)) return MSS_ERR_MISALIGNED;
    const Extent ew{reinterpret_cast<uintptr_t>(a->workspace),
                    reinterpret_cast<uintptr_t>(a->workspace) + plan.workspace, true};
    for (const Extent& e : ins)
      if (overlaps(ew, e)) return MSS_ERR_ALIASING;
    if (overlaps(ew, eo) || overlaps(ew, ef) || overlaps(ew, ecs)) return MSS_ERR_ALIASING;
  }
  mss::ScanShape s = plan.shape;
  // A dimension of size 1 is never stepped, so its stride is free: use 1.
  norm_strides(s.su, a->u_stride, xs);
  norm_strides(s.sd, a->delta_stride, xs);
  norm_strides(s.so, a->out_stride, xs);
  norm_strides(s.sB, a->B_stride, bcs);
  norm_strides(s.sC, a->C_stride, bcs);
  std::memcpy(s.sA, a->A_log_stride, sizeof(s.sA));
  if (a->z != nullptr) norm_strides(s.sz, a->z_stride, xs);
  else std::memcpy(s.sz, s.su, sizeof(s.sz));
  // Layouts: u/delta_raw/z/out share a unit-stride axis (t or d), and so do
  // B and C (t or n); loads move kVec-element vectors along that axis.
  const bool x_tfast = s.su[2] == 1 && s.sd[2] == 1 && s.sz[2] == 1 && s.so[2] == 1;
  const bool x_dfast = s.su[1] == 1 && s.sd[1] == 1 && s.sz[1] == 1 && s.so[1] == 1;
  const bool bc_tfast = s.sB[2] == 1 && s.sC[2] == 1;
  const bool bc_nfast = s.sB[1] == 1 && s.sC[1] == 1;
  // Time-invariant B/C (time stride 0; a length-1 time axis has stride 1
  // after norm_strides): the vector pass holds them in registers, so their
  // state stride is free.
  s.bc_const = s.sB[2] == 0 && s.sC[2] == 0;
  if (!(x_tfast || x_dfast) || !(bc_tfast || bc_nfast || s.bc_const)) return MSS_ERR_BAD_STRIDE;
  const bool xt = x_tfast;
  const bool bt = bc_tfast;
  const int V = vec_elems(a->io_dtype);
  // bf16 vectors (8 bytes) start at 4-byte aligned addresses only if every
  // base pointer is 4-byte aligned and every stride other than the unit one is
  // even.
  s.vec_ok = 1;
  if (es == 2) {
    // (a dimension of size 1 is never stepped: its stride does not count)
    auto even = [](int64_t v, int64_t size) { return size == 1 || (v % 2) == 0; };
    const int64_t* xsts[4] = {s.su, s.sd, s.sz, s.so};
    const void* xps[4] = {a->u, a->delta_raw, a->z != nullptr ? a->z : a->u, a->out};
    for (int i = 0; i < 4; ++i)
      if (!aligned(xps[i], 4) || !even(xsts[i][0], a->batch) ||
          !(xt ? even(xsts[i][1], a->dim) : even(xsts[i][2], a->seqlen)))
        s.vec_ok = 0;
    const int64_t* bsts[2] = {s.sB, s.sC};
    const void* bps[2] = {a->B, a->C};
    for (int i = 0; i < 2; ++i)
      if (!aligned(bps[i], 4) || !even(bsts[i][0], a->batch) ||
          !(bt ? even(bsts[i][1], a->dstate) : even(bsts[i][2], a->seqlen)))
        s.vec_ok = 0;
    // in reverse time a t-fast vector starts at storage step seqlen-4-tau:
    // 4-byte aligned only for an even length
    if (a->reverse && (xt || bt) && (a->seqlen % 2) != 0) s.vec_ok = 0;
  }
  p.u = a->u;
  p.delta_raw = a->delta_raw;
  p.A_log = a->A_log;
  p.B = a->B;
  p.C = a->C;
  p.D = a->D;
  p.z = a->z;
  p.dt_bias = a->dt_bias;
  p.h0 = a->initial_state;
  p.out = a->out;
  p.final_state = a->final_state;
  p.chunk_states = a->chunk_states;
  // Vectors along the unit-stride axes need the channel count (for
  // d-fast data) and dstate (for n-fast B/C) to be whole vectors; a time axis
  // that is not a whole number of vectors gets an element-wise tail pass.
  s.use_vec = s.vec_ok && (xt || a->dim % V == 0) && (bt || s.bc_const || a->dstate % V == 0);
  if (s.use_vec && (xt || bt)) s.t_stop = static_cast<int>(a->seqlen / V * V);
  if (s.use_vec) s.nseg = std::max(1, (s.t_stop + s.seg_len - 1) / s.seg_len);
  // Every argument check has passed: the first HIP call of this entry point
  // may come next (the scratch array's address, once per device).
  if (plan.workspace > 0) {
    char* ws = static_cast<char*>(a->workspace);
    if (noalloc) {
      const mss_status sst = scratch_address(static_cast<hipStream_t>(stream), &ws);
      if (sst != MSS_OK) return sst;
    }
    if (plan.agg_bytes > 0) {
      p.agg = reinterpret_cast<float2*>(ws);
      p.carry = reinterpret_cast<float*>(ws + plan.agg_bytes);
    }
    if (plan.tail_bytes > 0)
      p.tail_h0 = reinterpret_cast<float*>(ws + plan.agg_bytes + plan.carry_bytes);
  }
  if (s.use_vec && s.t_stop < s.seqlen && s.t_stop > 0 && p.tail_h0 == nullptr)
    return MSS_ERR_WORKSPACE_TOO_SMALL;  // unreachable: the plan reserves it
  const hipError_t e = mss::launch_scan(s, p, a->io_dtype == MSS_BF16, xt, bt,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

}  // namespace

extern "C" {

int mss_abi_version(void) { return MSS_ABI_VERSION; }

const char* mss_status_string(mss_status status) {
  switch (status) {
    case MSS_OK: return "ok";
    case MSS_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MSS_ERR_BAD_SHAPE: return "invalid shape (sizes must be >= 1 and fit the grid; conv width 1..4)";
    case MSS_ERR_BAD_STRIDE: return "invalid stride (negative, overlapping output, or a tile spans >= 2 GiB)";
    case MSS_ERR_UNSUPPORTED_DTYPE: return "unsupported io dtype (expected MSS_F32 or MSS_BF16)";
    case MSS_ERR_UNSUPPORTED_DSTATE: return "dstate must be between 1 and 16";
    case MSS_ERR_MISALIGNED: return "a pointer is not aligned to its element size";
    case MSS_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or smaller than mss_selective_scan_workspace_size";
    case MSS_ERR_ALIASING: return "an output overlaps an input";
    case MSS_ERR_BAD_STRUCT: return "arguments struct is NULL, of the wrong size, or has reserved fields set";
    case MSS_ERR_HIP: return "the HIP runtime reported an error while enqueuing";
    case MSS_ERR_SCRATCH_LIMIT:
      return "the shape needs more device scratch than the no-allocation forward holds "
             "(MSS_NOALLOC_SCRATCH_BYTES); use mss_selective_scan_fwd with a workspace";
  }
  return "unknown status";
}

size_t mss_selective_scan_workspace_size(const mss_scan_args* a, mss_status* status) {
  const mss_status st = check_shape(a);
  if (status != nullptr) *status = st;
  if (st != MSS_OK) return 0;
  return make_plan(a).workspace;
}

mss_status mss_selective_scan_fwd(const mss_scan_args* a, void* stream) {
  return scan_fwd(a, stream, /*noalloc=*/false);
}

mss_status mss_selective_scan_fwd_noalloc(const mss_scan_args* a, void* stream) {
  return scan_fwd(a, stream, /*noalloc=*/true);
}

mss_status mss_selective_state_update(const mss_step_args* a, void* stream) {
  if (a == nullptr || a->struct_size != sizeof(mss_step_args) || a->reserved0 != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->io_dtype != MSS_F32 && a->io_dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED_DTYPE;
  if (a->batch < 1 || a->dim < 1 || a->batch > kMaxDim || a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->batch * a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->dstate < 1 || a->dstate > MSS_MAX_DSTATE) return MSS_ERR_UNSUPPORTED_DSTATE;
  if (a->state == nullptr || a->u == nullptr || a->delta_raw == nullptr || a->A_log == nullptr ||
      a->B == nullptr || a->C == nullptr || a->out == nullptr)
    return MSS_ERR_NULL_POINTER;
  const int64_t es = a->io_dtype == MSS_BF16 ? 2 : 4;
  if (!strides_nonneg(a->u_stride, 2) || !strides_nonneg(a->delta_stride, 2) ||
      !strides_nonneg(a->B_stride, 2) || !strides_nonneg(a->C_stride, 2) ||
      !strides_nonneg(a->out_stride, 2) || !strides_nonneg(a->A_log_stride, 2) ||
      (a->z != nullptr && !strides_nonneg(a->z_stride, 2)))
    return MSS_ERR_BAD_STRIDE;
  const int64_t xs[2] = {a->batch, a->dim};
  if (!non_overlapping(xs, a->out_stride, 2)) return MSS_ERR_BAD_STRIDE;
  if (!aligned(a->state, 4) || !aligned(a->u, es) || !aligned(a->delta_raw, es) ||
      !aligned(a->B, es) || !aligned(a->C, es) || !aligned(a->z, es) || !aligned(a->out, es) ||
      !aligned(a->A_log, 4) || !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return MSS_ERR_MISALIGNED;
  const int64_t bcs[2] = {a->batch, a->dstate};
  const int64_t as[2] = {a->dim, a->dstate};
  const int64_t vs[1] = {a->dim};
  const int64_t one[1] = {1};
  const int64_t ss[3] = {a->batch, a->dim, a->dstate};
  const int64_t unit[3] = {a->dim * a->dstate, a->dstate, 1};
  const Extent ins[] = {
      extent_of(a->u, xs, a->u_stride, 2, es),      extent_of(a->delta_raw, xs, a->delta_stride, 2, es),
      extent_of(a->z, xs, a->z_stride, 2, es),      extent_of(a->B, bcs, a->B_stride, 2, es),
      extent_of(a->C, bcs, a->C_stride, 2, es),     extent_of(a->A_log, as, a->A_log_stride, 2, 4),
      extent_of(a->D, vs, one, 1, 4),               extent_of(a->dt_bias, vs, one, 1, 4),
  };
  const Extent eo = extent_of(a->out, xs, a->out_stride, 2, es);
  const Extent est = extent_of(a->state, ss, unit, 3, 4);
  for (const Extent& e : ins)
    if (overlaps(eo, e) || overlaps(est, e)) return MSS_ERR_ALIASING;
  if (overlaps(eo, est)) return MSS_ERR_ALIASING;

  mss::StepShape s{};
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.dstate = static_cast<int>(a->dstate);
  std::memcpy(s.su, a->u_stride, sizeof(s.su));
  std::memcpy(s.sd, a->delta_stride, sizeof(s.sd));
  std::memcpy(s.sz, a->z_stride, sizeof(s.sz));
  std::memcpy(s.so, a->out_stride, sizeof(s.so));
  std::memcpy(s.sB, a->B_stride, sizeof(s.sB));
  std::memcpy(s.sC, a->C_stride, sizeof(s.sC));
  std::memcpy(s.sA, a->A_log_stride, sizeof(s.sA));
  if (a->z == nullptr) std::memset(s.sz, 0, sizeof(s.sz));
  s.softplus = a->delta_softplus ? 1 : 0;
  mss::StepPtrs p{a->state, a->u, a->delta_raw, a->A_log, a->B, a->C, a->D, a->z, a->dt_bias, a->out};
  const hipError_t e = mss::launch_step(s, p, a->io_dtype == MSS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

size_t mss_selective_scan_bwd_workspace_size(const mss_scan_bwd_args* a, mss_status* status) {
  const mss_status st = check_bwd_shape(a);
  if (status != nullptr) *status = st;
  if (st != MSS_OK) return 0;
  return make_bwd_plan(a).workspace;
}

mss_status mss_selective_scan_bwd(const mss_scan_bwd_args* a, void* stream) {
  const mss_status st = check_bwd_shape(a);
  if (st != MSS_OK) return st;
  if (a->u == nullptr || a->delta_raw == nullptr || a->A_log == nullptr || a->B == nullptr ||
      a->C == nullptr || a->dout == nullptr || a->du == nullptr || a->ddelta_raw == nullptr ||
      a->dA_log == nullptr || a->dB == nullptr || a->dC == nullptr)
    return MSS_ERR_NULL_POINTER;
  if (a->z == nullptr && a->dz != nullptr) return MSS_ERR_NULL_POINTER;
  const int64_t es = a->io_dtype == MSS_BF16 ? 2 : 4;
  const int64_t xs[3] = {a->batch, a->dim, a->seqlen};
  const int64_t bcs[3] = {a->batch, a->dstate, a->seqlen};
  const int64_t as[2] = {a->dim, a->dstate};
  const int64_t vs[1] = {a->dim};
  const int64_t ss[3] = {a->batch, a->dim, a->dstate};
  const int64_t unit[3] = {a->dim * a->dstate, a->dstate, 1};
  const int64_t aunit[2] = {a->dstate, 1};
  const int64_t one[1] = {1};
  const int64_t* x_strides[] = {a->u_stride, a->delta_stride, a->dout_stride, a->du_stride,
                                a->ddelta_stride};
  for (const int64_t* st3 : x_strides)
    if (!strides_nonneg(st3, 3) || !tile_offsets_fit(st3, es)) return MSS_ERR_BAD_STRIDE;
  if (!strides_nonneg(a->B_stride, 3) || !strides_nonneg(a->C_stride, 3) ||
      !strides_nonneg(a->dB_stride, 3) || !strides_nonneg(a->dC_stride, 3) ||
      !strides_nonneg(a->A_log_stride, 2) || (a->z != nullptr && !strides_nonneg(a->z_stride, 3)) ||
      (a->dz != nullptr && !strides_nonneg(a->dz_stride, 3)))
    return MSS_ERR_BAD_STRIDE;
  // the reverse walk addresses its tiles with 32-bit offsets, as the forward
  if (!tile_offsets_fit(a->B_stride, es, kMaxState) || !tile_offsets_fit(a->C_stride, es, kMaxState) ||
      (a->z != nullptr && !tile_offsets_fit(a->z_stride, es)) ||
      (a->dz != nullptr && !tile_offsets_fit(a->dz_stride, es)))
    return MSS_ERR_BAD_STRIDE;
  if (!non_overlapping(xs, a->du_stride, 3) || !non_overlapping(xs, a->ddelta_stride, 3) ||
      (a->dz != nullptr && !non_overlapping(xs, a->dz_stride, 3)) ||
      !non_overlapping(bcs, a->dB_stride, 3) || !non_overlapping(bcs, a->dC_stride, 3))
    return MSS_ERR_BAD_STRIDE;
  const void* io_ptrs[] = {a->u, a->delta_raw, a->B, a->C, a->z, a->dout, a->du, a->ddelta_raw,
                           a->dB, a->dC, a->dz};
  for (const void* q : io_ptrs)
    if (!aligned(q, es)) return MSS_ERR_MISALIGNED;
  const void* f32_ptrs[] = {a->A_log, a->D, a->dt_bias, a->initial_state, a->dfinal_state,
                            a->dA_log, a->dD, a->ddt_bias, a->dinitial_state, a->workspace};
  for (const void* q : f32_ptrs)
    if (!aligned(q, 4)) return MSS_ERR_MISALIGNED;
  if (!aligned(a->chunk_states, 8)) return MSS_ERR_MISALIGNED;
  const Extent ins[] = {
      chunk_states_extent(a->chunk_states, a->batch, a->dim, a->seqlen),
      extent_of(a->u, xs, a->u_stride, 3, es),
      extent_of(a->delta_raw, xs, a->delta_stride, 3, es),
      extent_of(a->z, xs, a->z_stride, 3, es),
      extent_of(a->B, bcs, a->B_stride, 3, es),
      extent_of(a->C, bcs, a->C_stride, 3, es),
      extent_of(a->A_log, as, a->A_log_stride, 2, 4),
      extent_of(a->D, vs, one, 1, 4),
      extent_of(a->dt_bias, vs, one, 1, 4),
      extent_of(a->initial_state, ss, unit, 3, 4),
      extent_of(a->dout, xs, a->dout_stride, 3, es),
      extent_of(a->dfinal_state, ss, unit, 3, 4),
  };
  const Extent outs[] = {
      extent_of(a->du, xs, a->du_stride, 3, es),
      extent_of(a->ddelta_raw, xs, a->ddelta_stride, 3, es),
      extent_of(a->dA_log, as, aunit, 2, 4),
      extent_of(a->dB, bcs, a->dB_stride, 3, es),
      extent_of(a->dC, bcs, a->dC_stride, 3, es),
      extent_of(a->dD, vs, one, 1, 4),
      extent_of(a->dz, xs, a->dz_stride, 3, es),
      extent_of(a->ddt_bias, vs, one, 1, 4),
      extent_of(a->dinitial_state, ss, unit, 3, 4),
  };
  constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < kOuts; ++i) {
    for (const Extent& e : ins)
      if (overlaps(outs[i], e)) return MSS_ERR_ALIASING;
    for (int j = i + 1; j < kOuts; ++j)
      if (overlaps(outs[i], outs[j])) return MSS_ERR_ALIASING;
  }
  const BwdPlan plan = make_bwd_plan(a);
  if (a->workspace == nullptr || a->workspace_bytes < plan.workspace)
    return MSS_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned(a->workspace, 256)) return MSS_ERR_MISALIGNED;
  const Extent ew{reinterpret_cast<uintptr_t>(a->workspace),
                  reinterpret_cast<uintptr_t>(a->workspace) + plan.workspace, true};
  for (const Extent& e : ins)
    if (overlaps(ew, e)) return MSS_ERR_ALIASING;
  for (const Extent& e : outs)
    if (overlaps(ew, e)) return MSS_ERR_ALIASING;

  mss::BwdShape s = plan.shape;
  std::memcpy(s.su, a->u_stride, sizeof(s.su));
  std::memcpy(s.sd, a->delta_stride, sizeof(s.sd));
  std::memcpy(s.sdo, a->dout_stride, sizeof(s.sdo));
  std::memcpy(s.sdu, a->du_stride, sizeof(s.sdu));
  std::memcpy(s.sddr, a->ddelta_stride, sizeof(s.sddr));
  std::memcpy(s.sB, a->B_stride, sizeof(s.sB));
  std::memcpy(s.sC, a->C_stride, sizeof(s.sC));
  std::memcpy(s.sdB, a->dB_stride, sizeof(s.sdB));
  std::memcpy(s.sdC, a->dC_stride, sizeof(s.sdC));
  std::memcpy(s.sA, a->A_log_stride, sizeof(s.sA));
  if (a->z != nullptr) std::memcpy(s.sz, a->z_stride, sizeof(s.sz));
  else std::memset(s.sz, 0, sizeof(s.sz));
  if (a->dz != nullptr) std::memcpy(s.sdz, a->dz_stride, sizeof(s.sdz));
  else std::memset(s.sdz, 0, sizeof(s.sdz));
  // Step pairs: every (b, d) row starts on a pair boundary and holds whole
  // pairs, so that a 2-element access never straddles a row or the tensor.
  {
    const void* xp[] = {a->u, a->delta_raw, a->dout, a->z, a->du, a->ddelta_raw, a->dz};
    const int64_t* xst[] = {a->u_stride, a->delta_stride, a->dout_stride, a->z_stride,
                            a->du_stride, a->ddelta_stride, a->dz_stride};
    bool ok = a->seqlen % 2 == 0;
    for (int i = 0; i < 7 && ok; ++i) {
      if (xp[i] == nullptr) continue;
      ok = xst[i][2] == 1 && aligned(xp[i], 2 * es) && (a->batch == 1 || xst[i][0] % 2 == 0) &&
           (a->dim == 1 || xst[i][1] % 2 == 0);
    }
    s.pairs = ok ? 1 : 0;
  }
  {
    const void* xp[] = {a->u, a->delta_raw};
    const int64_t* xst[] = {a->u_stride, a->delta_stride};
    bool ok = a->seqlen % 4 == 0;
    for (int i = 0; i < 2 && ok; ++i)
      ok = xst[i][2] == 1 && aligned(xp[i], 4 * es) && (a->batch == 1 || xst[i][0] % 4 == 0) &&
           (a->dim == 1 || xst[i][1] % 4 == 0);
    s.quads = ok ? 1 : 0;
    auto quad_rows = [&](const void* ptr, const int64_t* st) {
      return a->seqlen % 4 == 0 && st[2] == 1 && aligned(ptr, 4 * es) &&
             (a->batch == 1 || st[0] % 4 == 0) && (a->dstate == 1 || st[1] % 4 == 0);
    };
    s.bquads = quad_rows(a->B, a->B_stride) ? 1 : 0;
    s.bcquads = (s.bquads && quad_rows(a->C, a->C_stride)) ? 1 : 0;
  }
  // Channel pairs and state quads (channel-last data) for the segment
  // aggregates: every (b, t) row starts on a pair (quad) boundary and holds
  // whole pairs (quads).
  {
    const void* xp[] = {a->u, a->delta_raw, a->dout, a->z};
    const int64_t* xst[] = {a->u_stride, a->delta_stride, a->dout_stride, a->z_stride};
    bool ok = a->dim % 2 == 0;
    for (int i = 0; i < 4 && ok; ++i) {
      if (xp[i] == nullptr) continue;
      ok = xst[i][1] == 1 && aligned(xp[i], 2 * es) && (a->batch == 1 || xst[i][0] % 2 == 0) &&
           xst[i][2] % 2 == 0;
    }
    s.dpairs = ok ? 1 : 0;
    auto nquad_rows = [&](const void* ptr, const int64_t* st) {
      return a->dstate % 4 == 0 && st[1] == 1 && aligned(ptr, 4 * es) &&
             (a->batch == 1 || st[0] % 4 == 0) && st[2] % 4 == 0;
    };
    s.nquads = (nquad_rows(a->B, a->B_stride) && nquad_rows(a->C, a->C_stride)) ? 1 : 0;
  }
  char* ws = static_cast<char*>(a->workspace);
  mss::BwdPtrs p{};
  p.u = a->u;
  p.delta_raw = a->delta_raw;
  p.A_log = a->A_log;
  p.B = a->B;
  p.C = a->C;
  p.D = a->D;
  p.z = a->z;
  p.dt_bias = a->dt_bias;
  p.h0 = a->initial_state;
  p.dout = a->dout;
  p.dfinal = a->dfinal_state;
  p.du = a->du;
  p.ddelta_raw = a->ddelta_raw;
  p.dA_log = a->dA_log;
  p.dB = a->dB;
  p.dC = a->dC;
  p.dD = a->dD;
  p.dz = a->dz;
  p.ddt_bias = a->ddt_bias;
  p.dh0 = a->dinitial_state;
  p.ckpt = reinterpret_cast<float*>(ws);
  s.states_given = 0;
  if (a->chunk_states != nullptr) {
    // read only: the checkpoint pass that would write it does not run
    p.ckpt = const_cast<float*>(a->chunk_states);
    s.states_given = 1;
  }
  if (s.nseg > 1) s.agg_split = bwd_agg_split(s, s.states_given != 0);
  p.part_bc = reinterpret_cast<float*>(ws + plan.ckpt_bytes);
  p.part_chan = reinterpret_cast<float*>(ws + plan.ckpt_bytes + plan.bc_bytes);
  if (plan.agg_bytes > 0) {
    char* q = ws + plan.ckpt_bytes + plan.bc_bytes + plan.chan_bytes;
    p.agg = reinterpret_cast<float4*>(q);
    p.carry_h = reinterpret_cast<float*>(q + plan.agg_bytes);
    p.carry_g = reinterpret_cast<float*>(q + plan.agg_bytes + plan.carry_bytes);
  }
  const hipError_t e = mss::launch_scan_bwd(s, p, a->io_dtype == MSS_BF16,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

size_t mss_selective_scan_fwd_complex_workspace_size(const mss_scan_complex_args* a,
                                                     mss_status* status) {
  const mss_status st = check_cplx_shape(a);
  if (status != nullptr) *status = st;
  if (st != MSS_OK) return 0;
  return make_cplx_plan(a).workspace;
}

mss_status mss_selective_scan_fwd_complex(const mss_scan_complex_args* a, void* stream) {
  const mss_status sst = check_cplx_shape(a);
  if (sst != MSS_OK) return sst;
  if (a->u == nullptr || a->delta_raw == nullptr || a->A_log == nullptr || a->A_imag == nullptr ||
      a->B == nullptr || a->C == nullptr || a->out == nullptr)
    return MSS_ERR_NULL_POINTER;
  if (!strides_nonneg(a->u_stride, 3) || !strides_nonneg(a->delta_stride, 3) ||
      !strides_nonneg(a->B_stride, 3) || !strides_nonneg(a->C_stride, 3) ||
      !strides_nonneg(a->out_stride, 3) || !strides_nonneg(a->A_log_stride, 2) ||
      !strides_nonneg(a->A_imag_stride, 2) || (a->z != nullptr && !strides_nonneg(a->z_stride, 3)))
    return MSS_ERR_BAD_STRIDE;
  const int64_t xs[3] = {a->batch, a->dim, a->seqlen};
  const int64_t bcs[3] = {a->batch, a->dstate, a->seqlen};
  const int64_t as[2] = {a->dim, a->dstate};
  const int64_t vs[1] = {a->dim};
  const int64_t ss[3] = {a->batch, a->dim, a->dstate};
  const int64_t unit[3] = {a->dim * a->dstate, a->dstate, 1};
  const int64_t one[1] = {1};
  if (!non_overlapping(xs, a->out_stride, 3)) return MSS_ERR_BAD_STRIDE;
  if (!aligned(a->u, 4) || !aligned(a->delta_raw, 4) || !aligned(a->A_log, 4) ||
      !aligned(a->A_imag, 4) || !aligned(a->D, 4) || !aligned(a->z, 4) || !aligned(a->dt_bias, 4) ||
      !aligned(a->out, 4) || !aligned(a->B, 8) || !aligned(a->C, 8) ||
      !aligned(a->initial_state, 8) || !aligned(a->final_state, 8))
    return MSS_ERR_MISALIGNED;
  const Extent ins[] = {
      extent_of(a->u, xs, a->u_stride, 3, 4),
      extent_of(a->delta_raw, xs, a->delta_stride, 3, 4),
      extent_of(a->z, xs, a->z_stride, 3, 4),
      extent_of(a->B, bcs, a->B_stride, 3, 8),
      extent_of(a->C, bcs, a->C_stride, 3, 8),
      extent_of(a->A_log, as, a->A_log_stride, 2, 4),
      extent_of(a->A_imag, as, a->A_imag_stride, 2, 4),
      extent_of(a->D, vs, one, 1, 4),
      extent_of(a->dt_bias, vs, one, 1, 4),
      extent_of(a->initial_state, ss, unit, 3, 8),
  };
  const Extent eo = extent_of(a->out, xs, a->out_stride, 3, 4);
  const Extent ef = extent_of(a->final_state, ss, unit, 3, 8);
  for (const Extent& e : ins)
    if (overlaps(eo, e) || overlaps(ef, e)) return MSS_ERR_ALIASING;
  if (overlaps(eo, ef)) return MSS_ERR_ALIASING;
  const CplxPlan plan = make_cplx_plan(a);
  if (plan.workspace > 0) {
    if (a->workspace == nullptr || a->workspace_bytes < plan.workspace)
      return MSS_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(a->workspace, 256)) return MSS_ERR_MISALIGNED;
    const Extent ew{reinterpret_cast<uintptr_t>(a->workspace),
                    reinterpret_cast<uintptr_t>(a->workspace) + plan.workspace, true};
    for (const Extent& e : ins)
      if (overlaps(ew, e)) return MSS_ERR_ALIASING;
    if (overlaps(ew, eo) || overlaps(ew, ef)) return MSS_ERR_ALIASING;
  }

  mss::CplxShape s = plan.shape;
  std::memcpy(s.su, a->u_stride, sizeof(s.su));
  std::memcpy(s.sd, a->delta_stride, sizeof(s.sd));
  std::memcpy(s.so, a->out_stride, sizeof(s.so));
  std::memcpy(s.sB, a->B_stride, sizeof(s.sB));
  std::memcpy(s.sC, a->C_stride, sizeof(s.sC));
  std::memcpy(s.sA, a->A_log_stride, sizeof(s.sA));
  std::memcpy(s.sAi, a->A_imag_stride, sizeof(s.sAi));
  if (a->z != nullptr) std::memcpy(s.sz, a->z_stride, sizeof(s.sz));
  mss::CplxPtrs p{};
  p.u = a->u;
  p.delta_raw = a->delta_raw;
  p.A_log = a->A_log;
  p.A_imag = a->A_imag;
  p.B = static_cast<const float2*>(a->B);
  p.C = static_cast<const float2*>(a->C);
  p.D = a->D;
  p.z = a->z;
  p.dt_bias = a->dt_bias;
  p.h0 = static_cast<const float2*>(a->initial_state);
  p.out = a->out;
  p.final_state = static_cast<float2*>(a->final_state);
  if (plan.workspace > 0) {
    char* ws = static_cast<char*>(a->workspace);
    p.agg = reinterpret_cast<float4*>(ws);
    p.carry = reinterpret_cast<float2*>(ws + plan.agg_bytes);
  }
  const hipError_t e = mss::launch_scan_complex(s, p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

mss_status mss_causal_conv1d_fwd(const mss_conv_args* a, void* stream) {
  if (a == nullptr || a->struct_size != sizeof(mss_conv_args) || a->reserved0 != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->io_dtype != MSS_F32 && a->io_dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED_DTYPE;
  if (a->batch < 1 || a->dim < 1 || a->seqlen < 1 || a->width < 1 ||
      a->width > MSS_MAX_CONV_WIDTH || a->batch > kMaxDim || a->dim > kMaxDim ||
      a->seqlen > kMaxSeqlen || a->batch * a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->activation != MSS_ACT_NONE && a->activation != MSS_ACT_SILU) return MSS_ERR_BAD_STRUCT;
  if (a->x == nullptr || a->weight == nullptr || a->out == nullptr) return MSS_ERR_NULL_POINTER;
  const int64_t es = a->io_dtype == MSS_BF16 ? 2 : 4;
  const int64_t W = a->width;
  const int64_t xs[3] = {a->batch, a->dim, a->seqlen};
  const int64_t ws[2] = {a->dim, W};
  const int64_t vs[1] = {a->dim};
  const int64_t win[3] = {a->batch, a->dim, W - 1};
  const int64_t unit[3] = {a->dim * (W - 1), W - 1, 1};
  const int64_t one[1] = {1};
  if (!strides_nonneg(a->x_stride, 3) || !strides_nonneg(a->out_stride, 3) ||
      !strides_nonneg(a->weight_stride, 2))
    return MSS_ERR_BAD_STRIDE;
  if (!non_overlapping(xs, a->out_stride, 3)) return MSS_ERR_BAD_STRIDE;
  if (!aligned(a->x, es) || !aligned(a->out, es) || !aligned(a->initial_state, es) ||
      !aligned(a->final_state, es) || !aligned(a->weight, 4) || !aligned(a->bias, 4))
    return MSS_ERR_MISALIGNED;
  // The windows are empty for width 1: nothing to read or write.
  const void* init = W > 1 ? a->initial_state : nullptr;
  void* fin = W > 1 ? a->final_state : nullptr;
  const Extent ins[] = {
      extent_of(a->x, xs, a->x_stride, 3, es),
      extent_of(a->weight, ws, a->weight_stride, 2, 4),
      extent_of(a->bias, vs, one, 1, 4),
      extent_of(init, win, unit, 3, es),
  };
  const Extent eo = extent_of(a->out, xs, a->out_stride, 3, es);
  const Extent ef = extent_of(fin, win, unit, 3, es);
  for (const Extent& e : ins)
    if (overlaps(eo, e) || overlaps(ef, e)) return MSS_ERR_ALIASING;
  if (overlaps(eo, ef)) return MSS_ERR_ALIASING;

  mss::ConvShape s{};
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.seqlen = static_cast<int>(a->seqlen);
  s.width = static_cast<int>(W);
  conv_strides(s.sx, a->x_stride, xs, 3);
  conv_strides(s.so, a->out_stride, xs, 3);
  std::memcpy(s.sw, a->weight_stride, sizeof(s.sw));
  s.silu = a->activation == MSS_ACT_SILU ? 1 : 0;
  s.path = mss::kConvElementwise;
  s.nseg = 1;
  s.seg_len = s.seqlen;
  s.cf_lanes = 64;
  // 16-byte vectors along the unit-stride axis (V = 4 fp32 or 8 bf16
  // elements) need every vector start aligned: the base pointers to 16 bytes
  // and every other stride a multiple of V elements.
  const int64_t V = mss::kConvVecBytes / es;
  const bool vec_aligned = aligned(a->x, mss::kConvVecBytes) && aligned(a->out, mss::kConvVecBytes);
  if (vec_aligned && a->seqlen > 1 && s.sx[2] == 1 && s.so[2] == 1 && all_mult(s.sx, 3, V, 2) &&
      all_mult(s.so, 3, V, 2)) {
    s.path = mss::kConvTimeFast;
    const int64_t nwg = a->batch * a->dim * ((a->seqlen + 2047) / 2048);
    if (nwg > 0xFFFFFFFFll) s.path = mss::kConvElementwise;
  } else if (vec_aligned && a->dim % V == 0 && a->dim > 1 && s.sx[1] == 1 && s.so[1] == 1 &&
             all_mult(s.sx, 3, V, 1) && all_mult(s.so, 3, V, 1)) {
    s.path = mss::kConvChanFast;
    // lanes per row of channels: enough vectors to cover dim, at most a wave
    int64_t lanes = 1;
    while (lanes < 64 && lanes * V < a->dim) lanes *= 2;
    s.cf_lanes = static_cast<int>(lanes);
    const int64_t per_wave = 64 / lanes;
    const int64_t groups = (a->dim + lanes * V - 1) / (lanes * V);
    const int64_t base = a->batch * groups;
    int64_t nseg = std::max<int64_t>(1, (kConvTargetWaves * per_wave + base - 1) / base);
    nseg = std::min<int64_t>(nseg, std::max<int64_t>(1, a->seqlen / kConvMinSeg));
    int64_t seg = (a->seqlen + nseg - 1) / nseg;
    seg = (seg + 7) / 8 * 8;
    s.seg_len = static_cast<int>(seg);
    s.nseg = static_cast<int>((a->seqlen + seg - 1) / seg);
    if (base * ((s.nseg + per_wave - 1) / per_wave) > 0xFFFFFFFFll) s.path = mss::kConvElementwise;
  }
  if (s.path == mss::kConvElementwise && (a->batch * a->dim * a->seqlen + 255) / 256 > 0xFFFFFFFFll)
    return MSS_ERR_BAD_SHAPE;
  const mss::ConvPtrs p{a->x, a->weight, a->bias, init, a->out, fin};
  const hipError_t e = mss::launch_conv(s, p, a->io_dtype == MSS_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

mss_status mss_causal_conv1d_update(const mss_conv_step_args* a, void* stream) {
  if (a == nullptr || a->struct_size != sizeof(mss_conv_step_args) || a->reserved0 != 0)
    return MSS_ERR_BAD_STRUCT;
  if (a->io_dtype != MSS_F32 && a->io_dtype != MSS_BF16) return MSS_ERR_UNSUPPORTED_DTYPE;
  if (a->batch < 1 || a->dim < 1 || a->width < 1 || a->width > MSS_MAX_CONV_WIDTH ||
      a->batch > kMaxDim || a->dim > kMaxDim || a->batch * a->dim > kMaxDim)
    return MSS_ERR_BAD_SHAPE;
  if (a->activation != MSS_ACT_NONE && a->activation != MSS_ACT_SILU) return MSS_ERR_BAD_STRUCT;
  const int64_t W = a->width;
  if (a->x == nullptr || a->weight == nullptr || a->out == nullptr ||
      (W > 1 && a->state == nullptr))
    return MSS_ERR_NULL_POINTER;
  const int64_t es = a->io_dtype == MSS_BF16 ? 2 : 4;
  if (!strides_nonneg(a->x_stride, 2) || !strides_nonneg(a->out_stride, 2) ||
      !strides_nonneg(a->weight_stride, 2))
    return MSS_ERR_BAD_STRIDE;
  const int64_t xs[2] = {a->batch, a->dim};
  if (!non_overlapping(xs, a->out_stride, 2)) return MSS_ERR_BAD_STRIDE;
  if (!aligned(a->x, es) || !aligned(a->out, es) || !aligned(a->state, es) ||
      !aligned(a->weight, 4) || !aligned(a->bias, 4))
    return MSS_ERR_MISALIGNED;
  const int64_t ws[2] = {a->dim, W};
  const int64_t vs[1] = {a->dim};
  const int64_t one[1] = {1};
  const int64_t win[3] = {a->batch, a->dim, W - 1};
  const int64_t unit[3] = {a->dim * (W - 1), W - 1, 1};
  void* state = W > 1 ? a->state : nullptr;
  const Extent ins[] = {
      extent_of(a->x, xs, a->x_stride, 2, es),
      extent_of(a->weight, ws, a->weight_stride, 2, 4),
      extent_of(a->bias, vs, one, 1, 4),
  };
  const Extent eo = extent_of(a->out, xs, a->out_stride, 2, es);
  const Extent est = extent_of(state, win, unit, 3, es);
  for (const Extent& e : ins)
    if (overlaps(eo, e) || overlaps(est, e)) return MSS_ERR_ALIASING;
  if (overlaps(eo, est)) return MSS_ERR_ALIASING;
  mss::ConvStepShape s{};
  s.batch = static_cast<int>(a->batch);
  s.dim = static_cast<int>(a->dim);
  s.width = static_cast<int>(W);
  std::memcpy(s.sx, a->x_stride, sizeof(s.sx));
  std::memcpy(s.so, a->out_stride, sizeof(s.so));
  std::memcpy(s.sw, a->weight_stride, sizeof(s.sw));
  s.silu = a->activation == MSS_ACT_SILU ? 1 : 0;
  const mss::ConvStepPtrs p{state, a->x, a->weight, a->bias, a->out};
  const hipError_t e = mss::launch_conv_step(s, p, a->io_dtype == MSS_BF16,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSS_OK : MSS_ERR_HIP;
}

}  // extern "C"
