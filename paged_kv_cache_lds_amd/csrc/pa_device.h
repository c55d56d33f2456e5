// Device-side building blocks for the gfx950 paged-attention kernels:
// 16-bit element traits, MFMA wrappers, page addressing and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
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
  // 16x16x16: 4-element operands (two dwords per lane)
  __device__ static inline f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
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
  __device__ static inline f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// Rotary position embedding (RoPE), fused into the loads of q and of the new
// keys - the fusion the small-page-size flash-attention thread reports for
// its paged-cache kernel.  Pair i of a head row at position m turns by the
// angle with cosine cos[m][i] and sine sin[m][i] (tables in the element type):
// a' = a cos - b sin, b' = b cos + a sin.  Half-split pairing puts element i
// with i + rdim/2, interleaved pairing puts 2i with 2i + 1; elements from rdim
// on are untouched.  Both products of 16-bit values are exact in fp32, so the
// fp32 result is the exact value rounded once, whatever the compiler contracts;
// it is then rounded to the element type (nearest even).
// ---------------------------------------------------------------------------
struct Rotary {
  const uint16_t *cos;   // [rows, rdim / 2], nullptr: no rotation
  const uint16_t *sin;
  int rows;              // positions 0 .. rows - 1
  int rdim;              // multiple of 16, <= head_dim
  int interleaved;
};

// What the rotation of N chunks of one head row needs, fetched in one batch
// so that a single memory round trip covers every chunk: chunk k holds the
// row's elements e0 = e_base + k * e_step .. e0 + 7 (e0 a multiple of 8).
// Half-split pairing: the partner chunk (elements e0 +- rdim/2) and the eight
// cos / sin entries of the chunk's pairs; interleaved pairing: the four cos /
// sin entries of its pairs (twice over).
template <int N>
struct RotFetch {
  u32x4 pw[N], cw[N], sw[N];
};

// Every load is issued unconditionally, without a branch between the two
// pairings, and stays in bounds: a chunk that is not rotated (e0 >= rdim, or
// a position outside the table) reads table row 0 and itself instead.
template <int N>
__device__ inline void rot_fetch(const Rotary &r, const uint16_t *row, int e_base, int e_step,
                                 int pos, RotFetch<N> &f) {
  const int half = r.rdim >> 1;
  const bool inter = r.interleaved != 0;
  const long t0 = (unsigned)pos < (unsigned)r.rows ? (long)pos * half : 0L;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int e0 = e_base + k * e_step;
    const bool rot = e0 < r.rdim;
    const bool first = e0 < half;
    // partner offset (half-split only) and first table entry of the chunk
    const int dp = (rot & !inter) ? (first ? half : -half) : 0;
    const int ti = rot ? (inter ? (e0 >> 1) : (first ? e0 : e0 - half)) : 0;
    const int t4 = inter ? 0 : 4;   // second 8 bytes: entries 4..7, or 0..3 again
    f.pw[k] = load16(row + e0 + dp);
    const u32x2 c0 = *reinterpret_cast<const u32x2 *>(r.cos + t0 + ti);
    const u32x2 c1 = *reinterpret_cast<const u32x2 *>(r.cos + t0 + ti + t4);
    const u32x2 s0 = *reinterpret_cast<const u32x2 *>(r.sin + t0 + ti);
    const u32x2 s1 = *reinterpret_cast<const u32x2 *>(r.sin + t0 + ti + t4);
    f.cw[k] = u32x4{c0[0], c0[1], c1[0], c1[1]};
    f.sw[k] = u32x4{s0[0], s0[1], s1[0], s1[1]};
  }
}

// Rotates the chunks x[k] (as loaded) for position `pos` with the fetched
// operands; chunks past rdim, and every chunk of a position outside the table,
// keep their bits.
template <int DT, int N>
__device__ inline void rot_apply(const Rotary &r, int e_base, int e_step, int pos, u32x4 (&x)[N],
                                 const RotFetch<N> &f) {
  if ((unsigned)pos >= (unsigned)r.rows) return;
  const int half = r.rdim >> 1;
  auto h = [](uint32_t w, int j) -> uint16_t { return (uint16_t)((j & 1) ? w >> 16 : w & 0xffffu); };
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int e0 = e_base + k * e_step;
    float xv[8], ov[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = Elt<DT>::to_f32(h(x[k][j >> 1], j));
    if (r.interleaved) {
      // pairs (e0 + 2j, e0 + 2j + 1), angle index e0 / 2 + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c = Elt<DT>::to_f32(h(f.cw[k][j >> 1], j));
        const float s = Elt<DT>::to_f32(h(f.sw[k][j >> 1], j));
        ov[2 * j] = xv[2 * j] * c - xv[2 * j + 1] * s;
        ov[2 * j + 1] = xv[2 * j + 1] * c + xv[2 * j] * s;
      }
    } else {
      // first half a' = a c - b s; second half b' = b c + a s (b, a: partner)
      const bool first = e0 < half;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = Elt<DT>::to_f32(h(f.pw[k][j >> 1], j));
        const float c = Elt<DT>::to_f32(h(f.cw[k][j >> 1], j));
        const float s = Elt<DT>::to_f32(h(f.sw[k][j >> 1], j));
        ov[j] = first ? xv[j] * c - pv * s : xv[j] * c + pv * s;
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2<DT>(ov[2 * j], ov[2 * j + 1]);
    x[k] = e0 < r.rdim ? o : x[k];
  }
}

// ---------------------------------------------------------------------------
// Rotary embedding of a query row split between the two halves of a wave, as
// the 32x32 MFMA operand holds it: lane (n, hh) (hh = lane / 32) holds chunks
// c = 2 ds + hh (elements 8c .. 8c+7) of row n for ds < NQ.  With h8 =
// rdim / 16, a half-split pair joins chunks c and c + h8 and uses table chunk
// c (entries 8c .. 8c+7); an interleaved chunk c uses entries 4c .. 4c+3,
// i.e. half of table chunk c / 2.  Each lane loads table chunks j = 2m + hh
// (m < NQ/2): every table entry the row needs is loaded once per row, with
// one 16-byte load per table and per two chunks; partners and the other
// half's table chunks come across the wave with permlane32 swaps.  Chunks of
// tables past rdim / 2 entries read entry 0 instead (in bounds, unused).
// ---------------------------------------------------------------------------

// the value lane l ^ 32 holds
__device__ inline uint32_t other_half(uint32_t v, bool upper) {
  const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  // sw[0]: the lower half's value on every lane, sw[1]: the upper half's.
  // The empty asm keeps the compiler from taking one for a copy of the other.
  uint32_t lo = sw[0], hi = sw[1];
  asm volatile("" : "+v"(lo), "+v"(hi));
  return upper ? lo : hi;
}
__device__ inline u32x4 other_half4(u32x4 v, bool upper) {
  return u32x4{other_half(v[0], upper), other_half(v[1], upper), other_half(v[2], upper),
               other_half(v[3], upper)};
}

template <int NQ>
__device__ inline void rot_fetch_split(const Rotary &r, int pos, int hh, u32x4 (&tc)[NQ / 2],
                                       u32x4 (&ts)[NQ / 2]) {
  const int half = r.rdim >> 1;
  const long t0 = (unsigned)pos < (unsigned)r.rows ? (long)pos * half : 0L;
#pragma unroll
  for (int m = 0; m < NQ / 2; ++m) {
    const int j = 2 * m + hh;
    const long ti = t0 + (8 * j + 8 <= half ? 8 * j : 0);
    tc[m] = load16(r.cos + ti);
    ts[m] = load16(r.sin + ti);
  }
}

// out = x c - p s (first of a pair) or x c + p s (second), element-wise over a
// chunk; x, p, c, s hold eight 16-bit values each
template <int DT>
__device__ inline u32x4 rot_pair_chunk(u32x4 x, u32x4 pw, u32x4 cw, u32x4 sw, bool first) {
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int sh = 16 * e;
      const float xv = Elt<DT>::to_f32((uint16_t)(x[w] >> sh));
      const float pv = Elt<DT>::to_f32((uint16_t)(pw[w] >> sh));
      const float c = Elt<DT>::to_f32((uint16_t)(cw[w] >> sh));
      const float s = Elt<DT>::to_f32((uint16_t)(sw[w] >> sh));
      r[e] = first ? xv * c - pv * s : xv * c + pv * s;
    }
    o[w] = pack2<DT>(r[0], r[1]);
  }
  return o;
}

// half-split pairing with h8 = H8 known at compile time
template <int DT, int NQ, int H8>
__device__ inline void rot_apply_split_half(u32x4 (&q)[NQ], const u32x4 (&tc)[NQ / 2],
                                            const u32x4 (&ts)[NQ / 2], int hh, bool ok) {
  const bool up = hh != 0;
  u32x4 oq[NQ], otc[NQ / 2], ots[NQ / 2];   // the other half's (only the odd case uses them)
  if constexpr (H8 % 2 == 1) {
#pragma unroll
    for (int k = 0; k < NQ; ++k) oq[k] = other_half4(q[k], up);
#pragma unroll
    for (int k = 0; k < NQ / 2; ++k) {
      otc[k] = other_half4(tc[k], up);
      ots[k] = other_half4(ts[k], up);
    }
  }
  u32x4 res[NQ];
#pragma unroll
  for (int ds = 0; ds < NQ; ++ds) {
    if (ds >= H8) {          // chunks 2 ds + hh >= 2 h8: past rdim
      res[ds] = q[ds];
      continue;
    }
    if constexpr (H8 % 2 == 0) {
      constexpr int kh = H8 / 2;
      const bool first = 2 * ds < H8;
      const int pd = first ? ds + kh : ds - kh;   // compile-time after unrolling
      const int m = first ? ds : ds - kh;
      res[ds] = rot_pair_chunk<DT>(q[ds], q[pd], tc[m], ts[m], first);
    } else {
      // lane half h: chunk c = 2 ds + h; first iff c < H8; partner c +- H8 and,
      // for the second of a pair, table chunk c - H8 sit in the other half
      const bool f0 = 2 * ds < H8, f1 = 2 * ds + 1 < H8;
      const int p0 = ((2 * ds + (f0 ? H8 : -H8)) >> 1);
      const int p1 = ((2 * ds + 1 + (f1 ? H8 : -H8)) >> 1);
      const int j0 = f0 ? 2 * ds : 2 * ds - H8;
      const int j1 = f1 ? 2 * ds + 1 : 2 * ds + 1 - H8;
      const u32x4 pw = up ? oq[p1] : oq[p0];
      const u32x4 cw0 = f0 ? tc[j0 >> 1] : otc[j0 >> 1];
      const u32x4 sw0 = f0 ? ts[j0 >> 1] : ots[j0 >> 1];
      const u32x4 cw1 = f1 ? tc[j1 >> 1] : otc[j1 >> 1];
      const u32x4 sw1 = f1 ? ts[j1 >> 1] : ots[j1 >> 1];
      res[ds] = rot_pair_chunk<DT>(q[ds], pw, up ? cw1 : cw0, up ? sw1 : sw0, up ? f1 : f0);
    }
  }
#pragma unroll
  for (int ds = 0; ds < NQ; ++ds) q[ds] = ok ? res[ds] : q[ds];
}

// interleaved pairing: chunk c = 2 ds + hh takes words 2 hh, 2 hh + 1 of
// table chunk ds
template <int DT, int NQ>
__device__ inline void rot_apply_split_inter(u32x4 (&q)[NQ], const u32x4 (&tc)[NQ / 2],
                                             const u32x4 (&ts)[NQ / 2], int hh, int h8, bool ok) {
  const bool up = hh != 0;
  u32x4 otc[NQ / 2], ots[NQ / 2];
#pragma unroll
  for (int k = 0; k < NQ / 2; ++k) {
    otc[k] = other_half4(tc[k], up);
    ots[k] = other_half4(ts[k], up);
  }
#pragma unroll
  for (int ds = 0; ds < NQ; ++ds) {
    const bool own = (ds & 1) == hh;
    const u32x4 cj = own ? tc[ds >> 1] : otc[ds >> 1];
    const u32x4 sj = own ? ts[ds >> 1] : ots[ds >> 1];
    const uint32_t c2[2] = {up ? cj[2] : cj[0], up ? cj[3] : cj[1]};
    const uint32_t s2[2] = {up ? sj[2] : sj[0], up ? sj[3] : sj[1]};
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // the pair (2w, 2w + 1) of the chunk is dword w; its angle is entry w
      const float a = Elt<DT>::to_f32((uint16_t)(q[ds][w] & 0xffffu));
      const float b = Elt<DT>::to_f32((uint16_t)(q[ds][w] >> 16));
      const float c = Elt<DT>::to_f32((uint16_t)(c2[w >> 1] >> (16 * (w & 1))));
      const float s = Elt<DT>::to_f32((uint16_t)(s2[w >> 1] >> (16 * (w & 1))));
      o[w] = pack2<DT>(a * c - b * s, b * c + a * s);
    }
    q[ds] = (ok && ds < h8) ? o : q[ds];
  }
}

template <int DT, int NQ>
__device__ inline void rot_apply_split(const Rotary &r, int pos, int hh, u32x4 (&q)[NQ],
                                       const u32x4 (&tc)[NQ / 2], const u32x4 (&ts)[NQ / 2]) {
  const bool ok = (unsigned)pos < (unsigned)r.rows;
  const int h8 = r.rdim >> 4;
  if (r.interleaved) {
    rot_apply_split_inter<DT, NQ>(q, tc, ts, hh, h8, ok);
    return;
  }
  switch (h8) {
    case 1: rot_apply_split_half<DT, NQ, 1>(q, tc, ts, hh, ok); break;
    case 2: rot_apply_split_half<DT, NQ, 2>(q, tc, ts, hh, ok); break;
    case 3: rot_apply_split_half<DT, NQ, 3>(q, tc, ts, hh, ok); break;
    case 4: rot_apply_split_half<DT, NQ, 4>(q, tc, ts, hh, ok); break;
    default:
      if constexpr (NQ == 8) {
        switch (h8) {
          case 5: rot_apply_split_half<DT, NQ, 5>(q, tc, ts, hh, ok); break;
          case 6: rot_apply_split_half<DT, NQ, 6>(q, tc, ts, hh, ok); break;
          case 7: rot_apply_split_half<DT, NQ, 7>(q, tc, ts, hh, ok); break;
          case 8: rot_apply_split_half<DT, NQ, 8>(q, tc, ts, hh, ok); break;
          default: break;
        }
      }
      break;
  }
}

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
