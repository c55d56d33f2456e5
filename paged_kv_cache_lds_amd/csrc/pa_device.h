// Device-side building blocks for the gfx950 paged-attention kernels:
// 16-bit element traits, MFMA wrappers, page addressing and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kF16 = 0;
constexpr int kBF16 = 1;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Element traits: round-to-nearest-even conversion from fp32 and the 16x16x32
// MFMA (fp32 accumulate) on 8-element operands held as four dwords per lane.
// ---------------------------------------------------------------------------
template <int DT> struct Elt;

template <> struct Elt<kF16> {
  __device__ static inline uint16_t from_f32(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

template <> struct Elt<kBF16> {
  __device__ static inline uint16_t from_f32(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
  __device__ static inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// Two fp32 values rounded to nearest even and packed (lo in bits 0-15): one
// packed-convert instruction on gfx950.
template <int DT>
__device__ inline uint32_t pack2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, h2));
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
  }
}

__device__ inline u32x4 load16(const uint16_t *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ inline void store16(uint16_t *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48)
__device__ inline float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ inline float group4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Cache addressing.  The physical token row of logical key `key` of sequence
// `b` is resolved from the block table by its absolute logical page index on
// every use - never by stepping from a previous page - which is the fix the
// small-page-size flash-attention thread settled on after relative page steps
// ran past the end of the table.  Out-of-range entries yield -1 (absent key).
// ---------------------------------------------------------------------------
struct CacheGeom {
  const int32_t *table;  // [batch, mpp] or nullptr (contiguous)
  int page_shift;        // log2(page_size), paged mode
  int mpp;               // table width
  int num_pages;
  int contig_alloc;      // contiguous mode
};

__device__ inline long physical_row(const CacheGeom &c, int b, int key) {
  if (key < 0) return -1L;
  if (c.table == nullptr) {
    return key < c.contig_alloc ? (long)b * c.contig_alloc + key : -1L;
  }
  int lp = key >> c.page_shift;
  if (lp >= c.mpp) return -1L;
  int page = c.table[(long)b * c.mpp + lp];
  if ((unsigned)page >= (unsigned)c.num_pages) return -1L;
  return ((long)page << c.page_shift) | (long)(key & ((1 << c.page_shift) - 1));
}

}  // namespace pa
