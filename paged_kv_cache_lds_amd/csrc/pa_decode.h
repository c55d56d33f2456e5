// Decode unit of the gfx950 paged KV-cache attention forward pass.
#pragma once

#include "pa_common.h"

namespace pa {

// ---------------------------------------------------------------------------
// Epilogue of a decode unit: each wave stages its (max, sum, O) for the 16
// MFMA columns in LDS (O in its own K slot), then after the unit's workgroup
// barrier 16 threads per row merge the four waves and write the row - out and
// lse for a single split, partial row and lse otherwise - to the packed row
// ridx_of(row).  A half of the unified kernel without a unit meets the barrier
// on its own.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, class Lds, class RowIdx>
__device__ __forceinline__ void decode_epilogue(const FwdParams &p, const Lds &lds,
                                                float (*sm_m)[kDecodeRows],
                                                float (*sm_l)[kDecodeRows],
                                                const f32x4 (&o_acc)[D / 16], float m_run,
                                                float l_part, int rows_b, int split, int S_b,
                                                RowIdx ridx_of) {
  constexpr int DB = D / 16;
  const int tid = threadIdx.x & (NW * 64 - 1);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const float l_row = group4_sum(l_part);
  float *stage = reinterpret_cast<float *>(lds.k(wave));   // [16 rows][D] fp32, own region
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
  const long ridx = ridx_of(orow);
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

  // The query rows (and the fused rotary embedding's operands, at the
  // token's position K_b - q_len + tok) are fetched after the first page ids
  // (below): loads retire in order, so the first tile's loads then wait for
  // the page ids only; the rows are needed only once that tile has landed.
  u32x4 qf[DS];
  const bool rot_q = p.rot.cos != nullptr;
  const int rot_pos = row_ok ? si.K_b - si.q_len + tok : -1;
  RotFetch<DS> rotf;
  auto fetch_q = [&]() {
    // a lane without a row reads the unit's first row (token 0 of the
    // sequence, head g * group: always there) and drops it, so that no load
    // sits behind a branch and the first tile waits for the page ids only
    const uint16_t *qrow = p.q + (long)(si.cu_b + tok) * p.q_stride + (long)h * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 v = load16(qrow + (ds * 4 + lg) * 8);
      qf[ds] = row_ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
    if (rot_q) rot_fetch(p.rot, qrow, lg * 8, 32, rot_pos, rotf);
  };

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
    fetch_q();
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

  decode_epilogue<DT, D, NW>(p, lds, sm_m, sm_l, o_acc, m_run, l_part, rows_b, split, S_b,
                             [&](int orow) {
                               const int tk = orow / group;
                               const int hp = g * group + (orow - tk * group);
                               return (long)(si.cu_b + tk) * p.hq + hp;
                             });
}


// ---------------------------------------------------------------------------
// Decode unit over a pair of adjacent kv heads (2 gp, 2 gp + 1), for batches
// whose decode rows fit twice into the 16 MFMA columns (2 * q_len * group <=
// 16): columns 0 .. rph - 1 are the first head's rows, rph .. 2 rph - 1 the
// second's.  The two heads' slices of a token row are adjacent in the pool
// (512 contiguous bytes at head_dim 128, against 256 for one head), and a
// development read probe streamed 512-byte row slices at 7.1-7.2 TB/s against
// 6.5 for 256-byte ones, so every load instruction fetches both heads of its
// keys.  Inner tiles hold 16 keys of both heads (the slot size of the
// one-head unit); per tile and head S^T = K Q^T on 16x16x32 MFMAs (only the
// head's own columns are kept), and O^T += V^T P^T on 16x16x16 MFMAs with the
// other head's columns of P^T zeroed, so each lane's O is its own column's.
// Splits, page-id prefetch, loads, LDS swizzle and epilogue follow the
// one-head unit; a 16-key tile never straddles a page (pages hold >= 16
// keys), so one page id serves a tile.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, class Lds>
__device__ __forceinline__ void decode_unit_pair(const FwdParams &p, const int b, const int gp,
                                                 const int split, const int S_b, const SeqInfo si,
                                                 const Lds &lds, float (*sm_m)[kDecodeRows],
                                                 float (*sm_l)[kDecodeRows]) {
  constexpr int NH = 2;
  constexpr int TK = kKeyTile / NH;   // keys per inner tile
  constexpr int DS = D / 32;          // k-steps of S^T (32 dims each)
  constexpr int DB = D / 16;          // 16-dim blocks of O^T
  constexpr int CPH = D / 8;          // 16-byte chunks per head row
  constexpr int CPR = NH * CPH;       // per staged row (both heads)
  constexpr int KPI = 64 / CPR;       // keys per row-load instruction
  constexpr int NLD = TK / KPI;
  constexpr int ROWH = NH * D;        // halves per staged row
  static_assert(TK * ROWH == kKeyTile * D, "a pair tile fills one slot of the one-head unit");
  static_assert(KPI >= 1 && NLD * KPI == TK, "whole rows per load instruction");
  const int tid = threadIdx.x & (NW * 64 - 1);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int group = p.group;
  const int rph = si.q_len * group;   // rows per head
  const int rows_b = NH * rph;
  const int bound = row_key_bound(rph - 1, group, si.q_len, si.K_b, p.causal);

  // this split's 32-key tiles and this wave's contiguous share (as the
  // one-head unit), walked as 16-key inner tiles
  const int n_t = (bound + kKeyTile - 1) / kKeyTile;
  const int t_begin = (int)((long)split * n_t / S_b);
  const int t_end = (int)((long)(split + 1) * n_t / S_b);
  const int key_end = min(t_end * kKeyTile, bound);
  const int n_w = t_end - t_begin;
  const int w_begin = t_begin + wave * (n_w / NW) + min(wave, n_w % NW);
  const int w_end = w_begin + n_w / NW + (wave < n_w % NW ? 1 : 0);
  const int key_end_w = min(w_end * kKeyTile, key_end);

  // this lane's column: head hr of the pair, row ri of that head
  const bool row_ok = lr < rows_b;
  const int hr = row_ok ? lr / rph : 0;
  const int ri = row_ok ? lr - hr * rph : 0;
  const int tok = ri / group;
  const int h = (gp * NH + hr) * group + (ri - tok * group);
  const int row_lim =
      row_ok ? min(row_key_bound(ri, group, si.q_len, si.K_b, p.causal), key_end_w) : 0;

  u32x4 qf[DS];
  {
    const uint16_t *qrow = p.q + (long)(si.cu_b + tok) * p.q_stride + (long)h * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = row_ok ? load16(qrow + (ds * 4 + lg) * 8) : u32x4{0u, 0u, 0u, 0u};
  }
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
  const int ld_key = lane / CPR;
  const int ld_chunk = lane % CPR;
  // page id of inner tile tt (every lane reads the same entry; lanes read a
  // harmless word where there is nothing to read)
  auto load_ids = [&](int tt) -> int {
    const int key = tt * TK;
    const bool ok = paged & (key < key_end_w) & ((key >> shift) < cg.mpp);
    const int32_t *src = ok ? cg.table + (long)b * cg.mpp + (key >> shift) : p.cu_seqlens_q;
    return *src;
  };
  const uint32_t row_bytes = (uint32_t)p.hkv * D * 2;
  uint32_t lane_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i)
    lane_off[i] = (uint32_t)(i * KPI + ld_key) * row_bytes +
                  (uint32_t)(gp * NH * D + ld_chunk * 8) * 2;
  auto issue = [&](int tt, u32x4 (&kf)[NLD], u32x4 (&vf)[NLD], int ids) {
    const int key0 = tt * TK;
    const uint32_t uni = (uint32_t)(paged ? (key0 & ((1 << shift) - 1)) : key0) * row_bytes;
    int pg = paged ? __builtin_amdgcn_readlane(ids, 0) : b;
    const bool ok_pg = !paged || (unsigned)pg < (unsigned)cg.num_pages;
    pg = ok_pg ? pg : 0;
    const __amdgpu_buffer_rsrc_t rk = page_rsrc(p.k_cache + pg * slab.elems, slab.bytes);
    const __amdgpu_buffer_rsrc_t rv = page_rsrc(p.v_cache + pg * slab.elems, slab.bytes);
    const int limit = paged ? key_end_w : min(key_end_w, cg.contig_alloc);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const bool ok = ok_pg && key0 + i * KPI + ld_key < limit;
      const uint32_t off = ok ? lane_off[i] : kOOB;
      kf[i] = buf_load16_stream(rk, off, uni);
      vf[i] = buf_load16_stream(rv, off, uni);
    }
  };

  float m_run = kNegInf;
  float l_part = 0.f;
  f32x4 o_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o_acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t *ks_ = lds.k(wave);   // K tile [16 keys][both heads' D], chunk-swizzled rows
  uint16_t *vs_ = lds.v(wave);
  // 16-byte chunk c of key `key` at chunk c ^ key: the 16 rows one MFMA read
  // touches fall on 16 different bank groups
  auto soff = [&](int key, int chunk) { return key * ROWH + ((chunk ^ (key & (TK - 1))) << 3); };
  const uint16_t *k_rd[NH][DS];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) k_rd[hh][ds] = ks_ + soff(lr, hh * CPH + ds * 4 + lg);

  auto step = [&](int tt, u32x4 (&kf)[NLD], u32x4 (&vf)[NLD], int &ids) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int o = soff(i * KPI + ld_key, ld_chunk);
      store16(ks_ + o, kf[i]);
      store16(vs_ + o, vf[i]);
    }
    issue(tt + 2, kf, vf, ids);
    ids = load_ids(tt + 4);

    // S^T of each head (keys 4 lg + i of column lr); the lane keeps its head's
    f32x4 sc[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      sc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) sc[hh] = Elt<DT>::mfma16(load16(k_rd[hh][ds]), qf[ds], sc[hh]);
    }
    const f32x4 sv = hr ? sc[1] : sc[0];
    float s[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = tt * TK + lg * 4 + i;
      const float v = key < row_lim ? sv[i] * p.scale_log2 : kNegInf;
      s[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = group4_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_use);
    float ps[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ps[e] = fast_exp2(s[e] - m_use);
      psum += ps[e];
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o_acc[db] *= alpha;
    }
    // P^T operand of the lane's column (keys 4 lg .. 4 lg + 3), zero in the
    // product with the other head's V
    u32x2 pb{pack2<DT>(ps[0], ps[1]), pack2<DT>(ps[2], ps[3])};
    u32x2 pb_lo{0u, 0u};
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float h0 = Elt<DT>::to_f32((uint16_t)(pb[e] & 0xffffu));
        const float h1 = Elt<DT>::to_f32((uint16_t)(pb[e] >> 16));
        pb_lo[e] = pack2<DT>(ps[2 * e] - h0, ps[2 * e + 1] - h1);
      }
    }
    const u32x2 zero{0u, 0u};
    const u32x2 ph0 = hr == 0 ? pb : zero, ph1 = hr == 0 ? zero : pb;
    const u32x2 pl0 = hr == 0 ? pb_lo : zero, pl1 = hr == 0 ? zero : pb_lo;
    // V^T: keys 4 lg .. 4 lg + 3 of dim db * 16 + lr, both heads per block
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int r0 = 4 * lg + (lr >> 2);
      const int ch = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 4;
      const u32x2 v0 = lds_read_tr16(vs_ + soff(r0, ch) + half);
      const u32x2 v1 = lds_read_tr16(vs_ + soff(r0, CPH + ch) + half);
      o_acc[db] = Elt<DT>::mfma16k16(v0, ph0, o_acc[db]);
      o_acc[db] = Elt<DT>::mfma16k16(v1, ph1, o_acc[db]);
      if constexpr (DT == kBF16) {
        o_acc[db] = Elt<DT>::mfma16k16(v0, pl0, o_acc[db]);
        o_acc[db] = Elt<DT>::mfma16k16(v1, pl1, o_acc[db]);
      }
    }
  };

  const int tt_begin = w_begin * NH, tt_end = w_end * NH;
  if (tt_begin < tt_end) {
    u32x4 ka[NLD], va_[NLD], kb_[NLD], vb_[NLD];
    int ids_a = load_ids(tt_begin);
    int ids_b = load_ids(tt_begin + 1);
    issue(tt_begin, ka, va_, ids_a);
    if (rot_q) rot_apply<DT>(p.rot, lg * 8, 32, rot_pos, qf, rotf);
    ids_a = load_ids(tt_begin + 2);
    issue(tt_begin + 1, kb_, vb_, ids_b);
    ids_b = load_ids(tt_begin + 3);
    for (int tt = tt_begin; tt < tt_end; tt += 2) {
      step(tt, ka, va_, ids_a);
      step(tt + 1, kb_, vb_, ids_b);
    }
  }

  decode_epilogue<DT, D, NW>(p, lds, sm_m, sm_l, o_acc, m_run, l_part, rows_b, split, S_b,
                             [&](int orow) {
                               const int ohr = orow / rph;
                               const int ori = orow - ohr * rph;
                               const int tk = ori / group;
                               const int hp = (gp * NH + ohr) * group + (ori - tk * group);
                               return (long)(si.cu_b + tk) * p.hq + hp;
                             });
}

}  // namespace pa
