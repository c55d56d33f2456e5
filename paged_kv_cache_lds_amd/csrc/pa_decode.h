// Decode unit of the gfx950 paged KV-cache attention forward pass.
#pragma once

#include "pa_common.h"

namespace pa {

// ---------------------------------------------------------------------------
// Decode unit: <= 16 packed rows (the G q heads of one kv head for one or a
// few tokens), one split of the sequence's keys, on four waves (a workgroup of
// the decode-only kernel, or one half of a unified-kernel workgroup).  The
// waves share the rows and each walks a contiguous share of the split's 32-key
// tiles:
//
//   page ids     a tile's one or two page ids are fetched four tiles ahead
//                with one vector load (lane i holds the page of load
//                instruction i) and moved to scalar registers with lane
//                reads; ids are resolved by absolute logical index, and
//                entries past the last visible page are never read;
//   row loads    every load instruction fetches whole K (V) rows: D*2 bytes
//                per key, 64*16/(D*2) keys per instruction, which streams
//                HBM faster than MFMA-shaped partial-row loads; two tiles are
//                in flight per wave (tile t + 2 is issued as soon as tile t's
//                registers are staged);
//   LDS staging  K and V land in the wave's own LDS slots, rows with their
//                16-byte chunks XOR-swizzled by key; no workgroup barrier in
//                the loop;
//   S^T = K Q^T  16x16x32 MFMA, keys on M: each lane's probabilities are
//                already the B operand of the PV product;
//   O^T += V^T P^T 16x16x32 MFMA on key-contiguous V^T from transposing reads.
// The waves' (max, sum, O) states merge through LDS at the end, after the
// unit's only workgroup barrier (a half without a unit meets it on its own).
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, class Lds>
__device__ __forceinline__ void decode_unit(const FwdParams &p, const int b, const int g,
                                            const int split, const int S_b, const SeqInfo si,
                                            const Lds &lds, float (*sm_m)[kDecodeRows],
                                            float (*sm_l)[kDecodeRows]) {
  constexpr int DS = D / 32;       // k-steps of S^T (32 dims each)
  constexpr int DB = D / 16;       // 16-dim blocks of O^T
  constexpr int CPR = D / 8;       // 16-byte chunks per K/V row
  constexpr int KPI = 64 / CPR;    // keys per row-load instruction
  constexpr int NLD = kKeyTile / KPI;
  constexpr int ROWH = D;          // halves per staged row (no padding: swizzled)
  constexpr int TILEH = kKeyTile * ROWH;          // halves per staged tile (one LDS slot)
  static_assert(TILEH * 2 >= kDecodeRows * D * 4, "a K slot must hold the wave's O staging");
  const int tid = threadIdx.x & (NW * 64 - 1);   // within the unit's waves
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int group = p.group;
  const int rows_b = si.q_len * group;
  const int bound = row_key_bound(rows_b - 1, group, si.q_len, si.K_b, p.causal);

  // this split's tiles, then this wave's contiguous share
  const int n_t = (bound + kKeyTile - 1) / kKeyTile;
  const int t_begin = (int)((long)split * n_t / S_b);
  const int t_end = (int)((long)(split + 1) * n_t / S_b);
  const int key_end = min(t_end * kKeyTile, bound);
  const int n_w = t_end - t_begin;
  const int w_begin = t_begin + wave * (n_w / NW) + min(wave, n_w % NW);
  const int w_end = w_begin + n_w / NW + (wave < n_w % NW ? 1 : 0);
  // keys of this wave: [w_begin * 32, key_end_w); tiles past w_end (the
  // pipeline's tail) read nothing and are fully masked
  const int key_end_w = min(w_end * kKeyTile, key_end);

  const bool row_ok = lr < rows_b;
  const int tok = row_ok ? lr / group : 0;
  const int h = g * group + (row_ok ? lr - tok * group : 0);
  const int row_lim =
      row_ok ? min(row_key_bound(lr, group, si.q_len, si.K_b, p.causal), key_end_w) : 0;

  u32x4 qf[DS];
  {
    const uint16_t *qrow = p.q + (long)(si.cu_b + tok) * p.q_stride + (long)h * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = row_ok ? load16(qrow + (ds * 4 + lg) * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  // fused rotary embedding of the query row, at the token's position
  // K_b - q_len + tok: its operands are fetched with the row, and applied once
  // the first tile's loads are out (see below)
  const bool rot_q = p.rot.cos != nullptr;
  const int rot_pos = row_ok ? si.K_b - si.q_len + tok : -1;
  RotFetch<DS> rotf;
  if (rot_q)
    rot_fetch(p.rot, p.q + (long)(si.cu_b + tok) * p.q_stride + (long)h * D, lg * 8, 32, rot_pos,
              rotf);

  const CacheGeom &cg = p.geom;
  const bool paged = cg.table != nullptr;
  const int shift = cg.page_shift;
  const Slab slab = paged ? Slab{(uint32_t)(p.hkv * D * 2) << shift, (long)(p.hkv * D) << shift}
                          : Slab{(uint32_t)cg.contig_alloc * p.hkv * D * 2,
                                 (long)cg.contig_alloc * p.hkv * D};

  // load role of this lane: key ld_key of each group of KPI keys, chunk ld_chunk
  const int ld_key = lane / CPR;
  const int ld_chunk = lane % CPR;
  // Page ids of tile t: lane i < NLD reads the table entry of load
  // instruction i's keys (KPI consecutive keys never straddle a page).  The
  // read is unconditional; lanes with nothing to read load a harmless word.
  auto load_ids = [&](int t) -> int {
    const int key = t * kKeyTile + (lane % NLD) * KPI;
    // bitwise conditions and one unconditional load: no branch around it
    const bool ok = paged & (lane < NLD) & (key < key_end_w) & ((key >> shift) < cg.mpp);
    const int32_t *src = ok ? cg.table + (long)b * cg.mpp + (key >> shift) : p.cu_seqlens_q;
    return *src;
  };
  // Loop-invariant part of each load's byte offset: the key's row within its
  // page (a 32-key tile never wraps inside a page of >= 32 keys; with 16-key
  // pages its upper half starts a new page), kv head g, 16-byte chunk.
  const uint32_t row_bytes = (uint32_t)p.hkv * D * 2;
  const int in_page_mask = paged ? min((1 << shift), kKeyTile) - 1 : kKeyTile - 1;
  const int upper_lane = in_page_mask < kKeyTile - 1 ? (in_page_mask + 1) / KPI : 0;
  uint32_t lane_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i)
    lane_off[i] = (uint32_t)((i * KPI + ld_key) & in_page_mask) * row_bytes +
                  (uint32_t)(g * D + ld_chunk * 8) * 2;
  auto issue = [&](int t, u32x4 (&kf)[NLD], u32x4 (&vf)[NLD], int ids) {
    const int key0 = t * kKeyTile;
    // first row of the tile inside its page (wave-uniform)
    const uint32_t uni = (uint32_t)(paged ? (key0 & ((1 << shift) - 1)) : key0) * row_bytes;
    // the tile's one or two pages: those of the first load instruction and of
    // the first instruction of the tile's upper half (keys 16.., which start a
    // new page only when pages hold 16 keys)
    const int rl_a = __builtin_amdgcn_readlane(ids, 0);
    const int rl_b = __builtin_amdgcn_readlane(ids, upper_lane);
    int pg_a = paged ? rl_a : b;
    int pg_b = paged ? rl_b : b;
    const bool ok_a = !paged || (unsigned)pg_a < (unsigned)cg.num_pages;
    const bool ok_b = !paged || (unsigned)pg_b < (unsigned)cg.num_pages;
    pg_a = ok_a ? pg_a : 0;
    pg_b = ok_b ? pg_b : 0;
    const __amdgpu_buffer_rsrc_t rk_a = page_rsrc(p.k_cache + pg_a * slab.elems, slab.bytes);
    const __amdgpu_buffer_rsrc_t rv_a = page_rsrc(p.v_cache + pg_a * slab.elems, slab.bytes);
    const __amdgpu_buffer_rsrc_t rk_b = page_rsrc(p.k_cache + pg_b * slab.elems, slab.bytes);
    const __amdgpu_buffer_rsrc_t rv_b = page_rsrc(p.v_cache + pg_b * slab.elems, slab.bytes);
    const int limit = paged ? key_end_w : min(key_end_w, cg.contig_alloc);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const bool second = paged && (i * KPI) > in_page_mask;   // upper half of a 16-key-page tile
      const bool ok = (second ? ok_b : ok_a) && key0 + i * KPI + ld_key < limit;
      const uint32_t off = ok ? lane_off[i] : kOOB;
      kf[i] = buf_load16_stream(second ? rk_b : rk_a, off, uni);
      vf[i] = buf_load16_stream(second ? rv_b : rv_a, off, uni);
    }
  };

  float m_run = kNegInf;   // running max of scaled scores (log2 units), per row
  float l_part = 0.f;      // this lane's share of the row sum
  f32x4 o_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t *ks_ = lds.k(wave);   // K tile [32][D], chunk-swizzled rows
  uint16_t *vs_ = lds.v(wave);   // V tile [32][D], chunk-swizzled rows
  // element offset of (key, 16-byte chunk) in a swizzled tile
  auto soff = [&](int key, int chunk) { return key * ROWH + ((chunk ^ (key & (CPR - 1))) << 3); };

  // per-lane constants of the operand reads
  const uint16_t *k_rd[2][DS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) k_rd[kb][ds] = ks_ + soff(kb * 16 + lr, ds * 4 + lg);

  auto step = [&](int t, u32x4 (&kf)[NLD], u32x4 (&vf)[NLD], int &ids) {
    // stage the tile's rows into LDS
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int o = soff(i * KPI + ld_key, ld_chunk);
      store16(ks_ + o, kf[i]);
      store16(vs_ + o, vf[i]);
    }
    // registers of tile t are free: start tile t + 2 (its page ids arrived two
    // steps ago) and fetch the page ids of tile t + 4
    issue(t + 2, kf, vf, ids);
    ids = load_ids(t + 4);

    // S^T block per 16 keys: lane holds keys kb*16 + 4*lg + i of row lr
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) sc[kb] = Elt<DT>::mfma16(load16(k_rd[kb][ds]), qf[ds], sc[kb]);
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
    const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_use);
    float ps[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ps[e] = fast_exp2(s[e] - m_use);
      psum += ps[e];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {   // rescale only when some row's maximum moved
#pragma unroll
      for (int db = 0; db < DB; ++db) o_acc[db] *= alpha;
    }

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
    // V^T operand: keys 4*lg .. +3 and 16 + 4*lg .. +3 of dim db*16 + lr; lane
    // lr addresses row k0 + lr/4, dims db*16 + 4*(lr%4) .. +3 (8 bytes)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r0 = 4 * lg + (lr >> 2);
      const int r1 = r0 + 16;
      const int ch = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 4;
      const u32x2 a0 = lds_read_tr16(vs_ + soff(r0, ch) + half);
      const u32x2 a1 = lds_read_tr16(vs_ + soff(r1, ch) + half);
      const u32x4 va = u32x4{a0[0], a0[1], a1[0], a1[1]};
      o_acc[db] = Elt<DT>::mfma16(va, pb, o_acc[db]);
      if constexpr (DT == kBF16) o_acc[db] = Elt<DT>::mfma16(va, pb_lo, o_acc[db]);
    }
  };

  // Every load below is issued unconditionally (masked lanes read nothing),
  // so two tiles stay in flight per wave with exact waits.
  if (w_begin < w_end) {
    u32x4 ka[NLD], va_[NLD], kb_[NLD], vb_[NLD];
    int ids_a = load_ids(w_begin);
    int ids_b = load_ids(w_begin + 1);
    issue(w_begin, ka, va_, ids_a);
    if (rot_q) rot_apply<DT>(p.rot, lg * 8, 32, rot_pos, qf, rotf);
    ids_a = load_ids(w_begin + 2);
    issue(w_begin + 1, kb_, vb_, ids_b);
    ids_b = load_ids(w_begin + 3);
    for (int t = w_begin; t < w_end; t += 2) {
      step(t, ka, va_, ids_a);
      step(t + 1, kb_, vb_, ids_b);   // past w_end: an empty, fully masked tile
    }
  }

  const float l_row = group4_sum(l_part);

  // ---- epilogue: stage each wave's (m, l, O) in LDS, merge, write ----
  float *stage = reinterpret_cast<float *>(ks_);   // [16 rows][D] fp32, own region
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
  if (orow >= rows_b) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][orow]);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(sm_m[w][orow] - M);   // 0 for waves that saw nothing
      L += wt * sm_l[w][orow];
      const float *src = reinterpret_cast<const float *>(lds.k_const(w)) + orow * D + oc * CH;
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[c] += wt * src[c];
    }
  }
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  const float lse_val = empty ? kNegInf : (M + __builtin_log2f(L)) * kLn2;
  const int tk = orow / group;
  const int hp = g * group + (orow - tk * group);
  const long ridx = (long)(si.cu_b + tk) * p.hq + hp;
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
  // the row's split count, for the combine (split 0 of every decode sequence)
  if (p.row_splits != nullptr && split == 0 && oc == 0) p.row_splits[ridx] = S_b;
}

}  // namespace pa
