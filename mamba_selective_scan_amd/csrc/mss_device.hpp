// mss_device.hpp -- device-side helpers shared by the libmss kernels (gfx950).
//
// Element conversion, the stable softplus, the SiLU gate and the hardware
// exp2.  Everything here is fp32 arithmetic on wave64 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage types: fp32 and bf16 (raw 16-bit pattern; the kernels convert on
// load and round to nearest even on store).
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct io_traits;

template <>
struct io_traits<float> {
  __device__ static inline float load(const float* p) { return *p; }
  __device__ static inline void store(float* p, float v) { *p = v; }
};

// fp32 -> bf16 bit patterns on gfx950's conversion instruction
// (v_cvt_pk_bf16_f32): round to nearest with ties to even (the default
// rounding mode), subnormals kept, a NaN stays a NaN.  The pair form converts
// two values with one instruction.
__device__ static inline uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ static inline uint32_t bf16x2_bits(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <>
struct io_traits<bf16_t> {
  __device__ static inline float load(const bf16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(p->bits) << 16);
  }
  __device__ static inline void store(bf16_t* p, float v) { p->bits = bf16_bits(v); }
};

// 2^x on the transcendental unit (v_exp_f32).  Arguments far below -126 give
// 0, which is the correct limit for the decays it is used for.
__device__ static inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(x) on the transcendental unit (v_log_f32), for x in [1, 2].
__device__ static inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|), in fp32.
// With e = e^-|x| in (0, 1] and w = fl(1 + e), log1p(e) = log(w) + (e - (w - 1))
// up to a relative 2^-24: the bracket is the exact rounding error of w
// (Fast2Sum, valid as e <= 1) and dividing it by w would change the sum by less
// than 2^-25.  The hardware log2 is accurate to a few ulp of its result for w
// near 1, so the sum keeps full relative precision even when e is tiny.
// The last step uses max(x, 0) + v = max(x + v, v) for v = log1p(e) >= 0,
// which holds exactly in floating point as well.
__device__ static inline float softplus(float x) {
  const float e = fast_exp2(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float corr = e - (w - 1.0f);
  const float v = fmaf(fast_log2(w), kLn2, corr);
  return fmaxf(x + v, v);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ static inline float silu(float z) {
  const float den = 1.0f + fast_exp2(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(den);
}

// Sum over four of the eight state groups of one channel (lanes c + 8g) of
// four per-step partial sums.  The two swap-and-add levels sum over lane bits
// 5 and 4 and leave step {0, 2, 1, 3}[row] in 16-lane row `row`: lane c + 8h
// of the row holds the sum over the groups g with g % 2 == h.
__device__ inline float reduce_groups_half(float y0, float y1, float y2, float y3) {
  const auto s01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y0), __float_as_uint(y1),
                                                    false, false);
  const auto s23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y2), __float_as_uint(y3),
                                                    false, false);
  const float p01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
  const float p23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(p01), __float_as_uint(p23),
                                                  false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// The same over all eight groups: a DPP rotation by 8 within the row adds the
// two halves, so lanes c and c + 8 of a row end with the same total.
__device__ inline float reduce_groups(float y0, float y1, float y2, float y3) {
  const float w = reduce_groups_half(y0, y1, y2, y3);
  // row_ror:8 -- lane i of a row reads lane (i + 8) mod 16
  return w + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w), 0x128, 0xF, 0xF,
                                                        false));
}

// Sum over the eight state groups of one channel (lanes c + 8g) of one value
// per lane, left in all eight lanes: a butterfly over lane bits 5, 4 and 3,
// so every lane adds the same pairs (up to order) and ends with the same sum.
__device__ inline float sum_over_groups(float v) {
  v += __shfl_xor(v, 32, 64);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

// Sum over the 16 lanes of a DPP row, left in every lane of the row (every
// source lane of a row rotation is valid, so bound_ctrl changes nothing).
__device__ inline float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, true));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, true));  // row_ror:1
  return v;
}

// Raw buffer descriptors: a range that keeps every valid 32-bit tile offset
// in bounds; kOffNone lies past it, so an access with that offset reads 0 or
// writes nothing.  Flags: the gfx9 raw-buffer data format word.
constexpr int kRsrcRange = 0x7FFFFFF0;
constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOffNone = 0x80000000u;

// One element through a buffer descriptor, per storage type.
template <typename IO>
struct buf_one;
template <>
struct buf_one<float> {
  __device__ static inline float load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
  }
  __device__ static inline void store(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), r, off, soff, 0);
  }
};
template <>
struct buf_one<bf16_t> {
  __device__ static inline float load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0))
                           << 16);
  }
  __device__ static inline void store(float y, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(y), r, off, soff, 0);
  }
};

// Wave-uniform value (lane 0's), kept in a scalar register.
__device__ static inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace mss
