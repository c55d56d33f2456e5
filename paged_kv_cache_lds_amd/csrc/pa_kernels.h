// gfx950 kernels of the paged KV-cache attention forward pass.
//
//   kv_append_kernel   new K/V rows -> their page slots (bit copy)
//   attn_fwd_kernel    one unified varlen kernel: decode rows and prefill tiles
//                      in one grid; QK^T and PV on MFMA with fp32 accumulation,
//                      online softmax, split-KV partial or final epilogue
//   combine_kernel     log-sum-exp merge of split-KV partials
#pragma once

#include "pa_device.h"

namespace pa {

// Work decomposition constants.
constexpr int kThreads = 256;   // four wave64 per workgroup
constexpr int kWaves = 4;
constexpr int kKeyTile = 32;    // keys per wave main-loop iteration (two 16-key MFMA blocks)
constexpr int kDecodeRows = 16; // packed (token, q-head) rows of a decode work unit
constexpr int kPrefillRows = 64;// rows of a prefill work unit: 16 per wave

struct FwdParams {
  const uint16_t *q;
  const uint16_t *k_cache;
  const uint16_t *v_cache;
  CacheGeom geom;
  const int32_t *cache_seqlens;
  const int32_t *cu_seqlens_q;
  uint16_t *out;
  float *lse;
  float *o_part;     // [S, total_q, hq, D] fp32 (S > 1)
  float *lse_part;   // [S, total_q, hq]
  int batch, total_q, hq, hkv, group;
  int appended, causal, num_splits;
  float scale_log2;  // softmax scale * log2(e)
  int all_decode;    // host knows every sequence has q_len * group <= 16
};

struct AppendParams {
  uint16_t *k_cache;
  uint16_t *v_cache;
  CacheGeom geom;
  const int32_t *cache_seqlens;
  const int32_t *cu_seqlens_q;
  const uint16_t *k_new;
  const uint16_t *v_new;
  int batch, total_q, hkv, head_dim, tokens_per_block;
};

// ---------------------------------------------------------------------------
// Append (vLLM's reshape_and_cache; the in-call k=/v= of flash-attention's
// paged cache): new row i of sequence b goes to logical position
// cache_seqlens[b] + i.  Grid (cdiv(max_seqlen_q, tokens_per_block), batch);
// each thread moves 16-byte vectors.  Targets whose page id is outside the
// pool (a caller precondition violation) are skipped, never written.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.y;
  const int cu_b = p.cu_seqlens_q[b];
  // rows past total_q (malformed cu_seqlens_q) are never touched
  const int q_len = max(0, min(p.cu_seqlens_q[b + 1], p.total_q) - cu_b);
  const int tok0 = blockIdx.x * p.tokens_per_block;
  if (tok0 >= q_len) return;
  const int ntok = min(p.tokens_per_block, q_len - tok0);
  const int vec_per_row = p.hkv * p.head_dim / 8;   // 16-byte vectors per token row
  const int L = p.cache_seqlens[b];
  const int work = ntok * vec_per_row * 2;
  for (int idx = threadIdx.x; idx < work; idx += kThreads) {
    const int which = idx / (ntok * vec_per_row);     // 0: K, 1: V
    const int rem = idx - which * ntok * vec_per_row;
    const int t = rem / vec_per_row;
    const int v = rem - t * vec_per_row;
    const int i = tok0 + t;
    const long prow = physical_row(p.geom, b, L + i);
    if (prow < 0) continue;
    const long src = ((long)(cu_b + i) * vec_per_row + v) * 8;
    const long dst = (prow * vec_per_row + v) * 8;
    if (which == 0) {
      store16(p.k_cache + dst, load16(p.k_new + src));
    } else {
      store16(p.v_cache + dst, load16(p.v_new + src));
    }
  }
}

// ---------------------------------------------------------------------------
// Unified work mapping.  Work units per kv head: a sequence whose packed rows
// (q_len * group) fit one 16-row decode unit gets num_splits units (its keys
// split across workgroups); a longer one gets cdiv(rows, 64) prefill units of
// one split each.  The host sizes the grid from static maxima only; each
// workgroup finds its (sequence, unit) by a block-wide scan of the device
// cu_seqlens_q, and surplus workgroups return at once.  Zero-length
// sequences own no unit.
// ---------------------------------------------------------------------------
__device__ inline int units_of_sequence(int rows, int num_splits) {
  if (rows <= 0) return 0;
  return rows <= kDecodeRows ? num_splits : (rows + kPrefillRows - 1) / kPrefillRows;
}

__device__ inline bool locate_unit(const FwdParams &p, int unit, int &b_out, int &off_out,
                                   int *s_wsum, int *s_found) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_found[0] = -1;
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < p.batch; c0 += kThreads) {
    const int bb = c0 + tid;
    int units = 0;
    if (bb < p.batch) {
      const int ql = p.cu_seqlens_q[bb + 1] - p.cu_seqlens_q[bb];
      units = units_of_sequence(ql * p.group, p.num_splits);
    }
    int x = units;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = s_wsum[w];
      before += (w < wave) ? v : 0;
      total += v;
    }
    const int incl = carry + before + x;
    const int excl = incl - units;
    if (units > 0 && unit >= excl && unit < incl) {
      s_found[0] = bb;
      s_found[1] = unit - excl;
    }
    carry += total;
    __syncthreads();
    if (s_found[0] >= 0) break;
  }
  b_out = s_found[0];
  off_out = s_found[1];
  return b_out >= 0;
}

// ---------------------------------------------------------------------------
// Unified attention kernel.
//
// One workgroup = one work unit (sequence b, kv head g, query tile, key
// split).  Each wave owns 16 packed query rows (row r = token r / group,
// q head g * group + r % group: the group's q heads share every K/V fetch)
// and runs the main loop over 32-key tiles:
//
//   page gather   every lane resolves the physical page of its own key from
//                 the block table by absolute index, once per tile, and loads
//                 16-byte K and V vectors straight from HBM (the next tile's
//                 loads are issued before the current tile is computed);
//   S^T = K Q^T   v_mfma_f32_16x16x32 with keys on M and query rows on N, so
//                 the softmax probabilities come out already in the layout
//                 the PV product takes as its B operand;
//   softmax       online: running max in log2 units (scale * log2 e folded
//                 into one multiply), rescale of the accumulator, per-lane
//                 partial row sums reduced once at the end;
//   O^T += V^T P^T v_mfma_f32_16x16x32, V transposed through the wave's own
//                 LDS region (no workgroup barrier in the loop).
//
// Decode units (<= 16 rows): the four waves share the rows and interleave the
// unit's key tiles; their states merge through LDS.  Prefill units (64 rows):
// each wave has its own 16 rows and walks every key tile its rows can see.
// Key tiles are 32 keys whatever the page size, so results do not depend on
// the page size or on which physical pages hold the keys.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdParams p) {
  constexpr int DS = D / 32;       // k-steps of S^T (32 dims each)
  constexpr int DB = D / 16;       // 16-dim blocks of O^T
  constexpr int VSTR = D + 8;      // padded LDS row (halves) of the V tile
  constexpr int REGION = kKeyTile * VSTR;
  static_assert(REGION * 2 >= kDecodeRows * D * 4, "wave region must hold its O staging");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * REGION];
  __shared__ float sm_m[kWaves][kDecodeRows];
  __shared__ float sm_l[kWaves][kDecodeRows];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_found[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;        // MFMA row/col index within a 16 block
  const int lg = lane >> 4;        // 16-lane group
  const int g = blockIdx.x % p.hkv;
  const int unit = blockIdx.x / p.hkv;
  const int S = p.num_splits;

  int b, off;
  if (p.all_decode) {
    b = unit / S;
    off = unit - b * S;
    if (b >= p.batch) return;
  } else if (!locate_unit(p, unit, b, off, s_wsum, s_found)) {
    return;
  }

  const int cu_b = p.cu_seqlens_q[b];
  const int q_len = max(0, min(p.cu_seqlens_q[b + 1], p.total_q) - cu_b);
  const int group = p.group;
  const int rows_b = q_len * group;
  if (rows_b <= 0) return;
  const bool prefill = !p.all_decode && rows_b > kDecodeRows;
  const int split = prefill ? 0 : off;
  const int S_b = prefill ? 1 : S;
  const int qtile = prefill ? off : 0;
  const int K_b = max(0, p.cache_seqlens[b]) + (p.appended ? q_len : 0);

  // keys visible to packed row r (bottom-right causal alignment)
  auto key_bound = [&](int r) -> int {
    if (!p.causal) return K_b;
    const int lim = K_b - q_len + r / group + 1;
    return max(0, min(lim, K_b));
  };

  const int row0 = prefill ? qtile * kPrefillRows + wave * 16 : 0;
  const int rows_here = min(kDecodeRows, rows_b - row0);   // may be <= 0 (idle wave)
  const int wave_bound = rows_here > 0 ? key_bound(row0 + rows_here - 1) : 0;

  // key-tile range: this unit's split of the visible keys, tile aligned
  const int n_t = (wave_bound + kKeyTile - 1) / kKeyTile;
  const int chunk = (n_t + S_b - 1) / S_b;
  const int t_begin = split * chunk;
  const int t_end = min(t_begin + chunk, n_t);
  const int key_end = min(t_end * kKeyTile, wave_bound);
  const int t_first = prefill ? t_begin : t_begin + wave;
  const int t_step = prefill ? 1 : kWaves;

  // this lane's query row (N index of the MFMAs)
  const int my_row = row0 + lr;
  const bool row_ok = lr < rows_here;
  const int tok = row_ok ? my_row / group : 0;
  const int h = g * group + (row_ok ? my_row - tok * group : 0);
  const int row_lim = row_ok ? min(key_bound(my_row), key_end) : 0;

  u32x4 qf[DS];
  {
    const uint16_t *qrow = p.q + ((long)(cu_b + tok) * p.hq + h) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = row_ok ? load16(qrow + (ds * 4 + lg) * 8) : u32x4{0u, 0u, 0u, 0u};
  }

  auto load_tile = [&](int t, u32x4 (&kf)[2][DS], u32x4 (&vf)[2][DS]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = t * kKeyTile + kb * 16 + lr;
      const long prow = key < key_end ? physical_row(p.geom, b, key) : -1L;
      if (prow >= 0) {
        const long base = (prow * p.hkv + g) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          kf[kb][ds] = load16(p.k_cache + base + (ds * 4 + lg) * 8);
          vf[kb][ds] = load16(p.v_cache + base + (ds * 4 + lg) * 8);
        }
      } else {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          kf[kb][ds] = u32x4{0u, 0u, 0u, 0u};
          vf[kb][ds] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  float m_run = kNegInf;   // running max of scaled scores (log2 units), per row
  float l_part = 0.f;      // this lane's share of the row sum
  f32x4 o_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t *vs = smem + wave * REGION;
  u32x4 kf[2][DS], vf[2][DS];
  if (t_first < t_end) load_tile(t_first, kf, vf);

  for (int t = t_first; t < t_end; t += t_step) {
    u32x4 kn[2][DS], vn[2][DS];
    const int tn = t + t_step;
    if (tn < t_end) load_tile(tn, kn, vn);

    // S^T block per 16 keys: lane holds keys kb*16 + 4*lg + i of row lr
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) sc[kb] = Elt<DT>::mfma16(kf[kb][ds], qf[ds], sc[kb]);
    }

    float s[8];
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t * kKeyTile + kb * 16 + lg * 4 + i;
        const float v = key < row_lim ? sc[kb][i] * p.scale_log2 : kNegInf;
        s[kb * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = group4_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ps[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = fast_exp2(s[e] - m_use);
      psum += ps[e];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o_acc[db] *= alpha;

    // V tile -> this wave's LDS region, row-major [key][dim]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        store16(vs + (kb * 16 + lr) * VSTR + (ds * 4 + lg) * 8, vf[kb][ds]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // P^T operand: element e <-> key (e / 4) * 16 + 4 * lg + e % 4
    u32x4 pb, pb_lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) pb[e] = pack2<DT>(ps[2 * e], ps[2 * e + 1]);
    if constexpr (DT == kBF16) {
      // bf16 keeps 8 bits of each probability; a second (hi, lo) term restores
      // the remainder so the product is accurate to ~16 bits.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float h0 = Elt<DT>::to_f32((uint16_t)(pb[e] & 0xffffu));
        const float h1 = Elt<DT>::to_f32((uint16_t)(pb[e] >> 16));
        pb_lo[e] = pack2<DT>(ps[2 * e] - h0, ps[2 * e + 1] - h1);
      }
    }

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x4 va;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k0 = ((2 * e) >> 2) * 16 + 4 * lg + ((2 * e) & 3);
        const int k1 = ((2 * e + 1) >> 2) * 16 + 4 * lg + ((2 * e + 1) & 3);
        const uint32_t v0 = vs[k0 * VSTR + db * 16 + lr];
        const uint32_t v1 = vs[k1 * VSTR + db * 16 + lr];
        va[e] = v0 | (v1 << 16);
      }
      o_acc[db] = Elt<DT>::mfma16(va, pb, o_acc[db]);
      if constexpr (DT == kBF16) o_acc[db] = Elt<DT>::mfma16(va, pb_lo, o_acc[db]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        kf[kb][ds] = kn[kb][ds];
        vf[kb][ds] = vn[kb][ds];
      }
  }

  const float l_row = group4_sum(l_part);

  // ---- epilogue: stage each wave's (m, l, O) in LDS, then write rows ----
  float *stage = reinterpret_cast<float *>(vs);   // [16 rows][D] fp32, own region
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<f32x4 *>(stage + lr * D + db * 16 + lg * 4) = o_acc[db];
  if (lg == 0) {
    sm_m[wave][lr] = m_run;
    sm_l[wave][lr] = l_row;
  }
  __syncthreads();

  constexpr int CH = D / 16;       // dims per thread in the write-out
  const int orow = tid >> 4;       // 0..15
  const int oc = tid & 15;
  const int nblk = prefill ? kWaves : 1;
  for (int rb = 0; rb < nblk; ++rb) {
    const int prow = (prefill ? qtile * kPrefillRows + rb * 16 : 0) + orow;
    if (prow >= rows_b) continue;
    const int w_lo = prefill ? rb : 0;
    const int w_hi = prefill ? rb + 1 : kWaves;
    float M = kNegInf;
    for (int w = w_lo; w < w_hi; ++w) M = fmaxf(M, sm_m[w][orow]);
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = 0.f;
    float L = 0.f;
    if (M != kNegInf) {
      for (int w = w_lo; w < w_hi; ++w) {
        const float mw = sm_m[w][orow];
        const float wt = fast_exp2(mw - M);   // 0 for waves that saw nothing
        L += wt * sm_l[w][orow];
        const float *src = reinterpret_cast<const float *>(smem + w * REGION) + orow * D + oc * CH;
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] += wt * src[c];
      }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const float lse_val = empty ? kNegInf : (M + __builtin_log2f(L)) * kLn2;
    const int tk = prow / group;
    const int hp = g * group + (prow - tk * group);
    const long ridx = (long)(cu_b + tk) * p.hq + hp;
    if (S_b == 1) {
      uint16_t *dst = p.out + ridx * D + oc * CH;
      if constexpr (CH == 8) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = pack2<DT>(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        store16(dst, pk);
      } else {
        u32x2 pk;
#pragma unroll
        for (int e = 0; e < 2; ++e) pk[e] = pack2<DT>(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        *reinterpret_cast<u32x2 *>(dst) = pk;
      }
      if (oc == 0) p.lse[ridx] = lse_val;
    } else {
      const long pidx = (long)split * p.total_q * p.hq + ridx;
      float *dst = p.o_part + pidx * D + oc * CH;
#pragma unroll
      for (int c = 0; c < CH; c += 4)
        *reinterpret_cast<f32x4 *>(dst + c) =
            f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
      if (oc == 0) p.lse_part[pidx] = lse_val;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV combine: per (token, q head) row, lse = log(sum_s exp(lse_s)) and
// out = sum_s exp(lse_s - lse) * o_s over the splits that saw a key; a row
// whose splits were all empty gets out = 0, lse = -inf.  Only rows of decode
// units carry partials; rows of prefill units were written directly and are
// skipped.  One wave per row.
// ---------------------------------------------------------------------------
struct CombineParams {
  const float *o_part;
  const float *lse_part;
  const int32_t *cu_seqlens_q;
  uint16_t *out;
  float *lse;
  int batch, total_q, hq, group, num_splits, all_decode;
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long)p.total_q * p.hq) return;
  const int token = (int)(row / p.hq);
  if (!p.all_decode) {
    int lo = 0, hi = p.batch;   // largest b with cu[b] <= token
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_seqlens_q[mid] <= token) lo = mid; else hi = mid;
    }
    const int q_len = p.cu_seqlens_q[lo + 1] - p.cu_seqlens_q[lo];
    if (token >= p.cu_seqlens_q[lo + 1]) return;   // past cu[batch]
    if (q_len * p.group > kDecodeRows) return;     // prefill row: already final
  } else if (token >= p.cu_seqlens_q[p.batch]) {
    return;
  }
  const long stride = (long)p.total_q * p.hq;
  const int S = p.num_splits;
  float M = kNegInf;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, p.lse_part[s * stride + row]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  float total = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float ls = p.lse_part[s * stride + row];
      if (ls == kNegInf) continue;
      const float w = fast_exp2((ls - M) * kLog2e);
      total += w;
      const float *src = p.o_part + (s * stride + row) * D + lane * PER;
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] += w * src[c];
    }
  }
  const bool empty = !(total > 0.f);
  const float inv = empty ? 0.f : 1.f / total;
  uint16_t *dst = p.out + row * D + lane * PER;
#pragma unroll
  for (int c = 0; c < PER; ++c) dst[c] = Elt<DT>::from_f32(acc[c] * inv);
  if (lane == 0) p.lse[row] = empty ? kNegInf : M + __builtin_logf(total);
}

}  // namespace pa
