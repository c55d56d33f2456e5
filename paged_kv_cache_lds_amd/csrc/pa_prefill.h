// Prefill unit of the gfx950 paged KV-cache attention forward pass.
#pragma once

#include "pa_common.h"

namespace pa {

// ---------------------------------------------------------------------------
// Prefill unit: 128 packed rows (32 per wave) of one sequence and kv head,
// every key those rows can see, one split, in 32-key tiles:
//   loads        each wave moves its share of a tile's K and V rows from the
//                page straight into LDS (buffer loads with an LDS destination:
//                lane l of an instruction fills bytes 16 l .. 16 l + 15 of one
//                1 KiB block, and the lane chooses which 16-byte chunk of which
//                row it fetches, so the swizzles below are free); keys past the
//                visible range and pages outside the pool load as zeros; page
//                ids are fetched one tile ahead by absolute logical index;
//   LDS          two K slots and two V slots, separate LDS objects; K rows keep
//                chunk c at c ^ (row & 7), V rows at c ^ 2 (row & 3), which
//                makes both the 32x32 MFMA K reads and the transposing V reads
//                bank-conflict free with every read a lane base plus an
//                immediate offset; one barrier per tile;
//   iteration t  K of tile t+2 and V of tile t+1 stream in while each wave
//                computes S^T(t+1) = K Q^T (32x32x16 MFMA, keys on M) beside
//                the online softmax of tile t (log2 units, one fma + exp2 per
//                score) and O^T += V^T P^T(t) (32x32x16 MFMA, V^T from
//                transposing LDS reads).
// Tiles every row of the unit sees in full run in a branch-free, mask-free
// loop; the tiles on the causal diagonal follow in a masked loop.  The running
// maximum only moves when it grows by more than 2^8: the stale maximum stays
// an exact common reference for the row sum and the accumulator, and
// probabilities stay <= 256, so rescaling is rare.
// ---------------------------------------------------------------------------
constexpr float kRescaleThreshold = 8.f;   // log2 units

// acc + x.lo + x.hi for two packed 16-bit floats (one dot-product instruction
// against (1, 1); the products are exact, the sum is fp32)
template <int DT>
__device__ inline float add_pair(uint32_t x, float acc) {
  if constexpr (DT == kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, x), h2{(_Float16)1.f, (_Float16)1.f}, acc,
                                  false);
  } else {
    typedef short s2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s2, x), s2{0x3f80, 0x3f80}, acc,
                                           false);
  }
}

template <int DT, int D, bool kPaged>
__device__ __forceinline__ void prefill_unit(const FwdParams &p, const int b, const int g,
                                             const int qtile, const SeqInfo si,
                                             const LdsPool &pool) {
  constexpr int QS = D / 16;        // k-steps over D (16 dims each)
  constexpr int DBP = D / 32;       // 32-dim blocks of O^T
  constexpr int RB = kPrefillRB;    // 32-row blocks per wave
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPB = 64 / CPR;     // rows per 1 KiB load block (4 or 8)
  constexpr int NI = kPTile / (kWaves * RPB);   // load instructions per wave, tile and matrix
  static_assert(NI >= 1 && NI * kWaves * RPB == kPTile, "a tile must split into load blocks");
  static_assert(RPB == 4 || RPB == 8, "swizzle bookkeeping assumes 4 or 8 rows per block");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int n32 = lane & 31;       // MFMA column (row within a 32-row block)
  const int hh = lane >> 5;        // k half
  const int group = p.group;
  const int rows_b = si.q_len * group;
  const int wg_row0 = qtile * kPrefillRows;
  const int wg_rows = min(kPrefillRows, rows_b - wg_row0);
  const int wg_bound = row_key_bound(wg_row0 + wg_rows - 1, group, si.q_len, si.K_b, p.causal);
  const int wg_first = row_key_bound(wg_row0, group, si.q_len, si.K_b, p.causal);
  const int n_t = (wg_bound + kPTile - 1) / kPTile;
  const int n_full = min(wg_first / kPTile, n_t);   // tiles every row sees in full

  const int row0 = wg_row0 + wave * 32 * RB;
  const int rows_here = min(32 * RB, rows_b - row0);   // <= 0: idle wave
  const int wave_bound =
      rows_here > 0 ? row_key_bound(row0 + rows_here - 1, group, si.q_len, si.K_b, p.causal) : 0;
  bool row_ok[RB];
  int tok[RB], hq_[RB], row_lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 32 + n32;
    row_ok[rb] = rb * 32 + n32 < rows_here;
    tok[rb] = row_ok[rb] ? r / group : 0;
    hq_[rb] = g * group + (row_ok[rb] ? r - tok[rb] * group : 0);
    row_lim[rb] = row_ok[rb] ? row_key_bound(r, group, si.q_len, si.K_b, p.causal) : 0;
  }

  u32x4 qf[RB][QS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint16_t *qrow = p.q + ((long)(si.cu_b + tok[rb]) * p.hq + hq_[rb]) * D;
#pragma unroll
    for (int ds = 0; ds < QS; ++ds)
      qf[rb][ds] = row_ok[rb] ? load16(qrow + ds * 16 + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- LDS layout ----
  // LDS serves 256 bytes a clock in 64 four-byte banks: 16 lanes of a 16-byte
  // read, or 32 lanes of an 8-byte read, at a time.  Rows of 2 D bytes all
  // start on the same bank (D = 128) or on one of two (D = 64), so chunks are
  // XOR-swizzled per row:
  //   K, D = 128: chunk c at c ^ (row & 7), and the 1 KiB blocks of rows 8-15
  //               and 24-31 sit 128 bytes later - the 16 rows one 16-byte MFMA
  //               read touches fall on 16 different bank groups;
  //   K, D = 64:  chunk c at c ^ ((row / 2) & 7), same effect;
  //   V:          the 64-byte segment of chunk c moves by the row, c ^ 4 (row & 3)
  //               (D = 128) or c ^ 4 ((row / 2) & 1) (D = 64), so the four rows
  //               one transposing read touches fall on four different quarters.
  // ---- loads ----
  // Instruction r of wave w fills block bb = r * 4 + w of a slot: rows
  // bb * RPB + lane / CPR, physical chunk lane % CPR, i.e. the logical chunk
  // that the row's swizzle puts there.  bb * RPB is a multiple of 4, and of 8
  // when RPB is 8 or w is even, so the swizzles are fixed per lane and the
  // lane part of every byte offset is loop-invariant.
  const CacheGeom &cg = p.geom;
  constexpr bool paged = kPaged;   // block table (else one contiguous allocation per sequence)
  const int shift = cg.page_shift;
  const uint32_t row_bytes = (uint32_t)p.hkv * D * 2;
  const uint32_t slab_bytes = paged ? row_bytes << shift : (uint32_t)cg.contig_alloc * row_bytes;
  const int limit = paged ? wg_bound : min(wg_bound, cg.contig_alloc);
  const int lrow = lane / CPR;
  const int pch = lane % CPR;
  // row & 7 (D = 128) or (row / 2) & 7 (D = 64) of this lane's row, and the
  // V segment swizzle of that row
  const int kx = D == 128 ? ((4 * (wave & 1) + lrow) & 7) : ((4 * wave + (lrow >> 1)) & 7);
  const int vx = D == 128 ? ((lrow & 3) << 2) : (((lrow >> 1) & 1) << 2);
  const uint32_t k_lane = (uint32_t)lrow * row_bytes + (uint32_t)(g * D + ((pch ^ kx) << 3)) * 2;
  const uint32_t v_lane = (uint32_t)lrow * row_bytes + (uint32_t)(g * D + ((pch ^ vx) << 3)) * 2;
  // halves from a slot's start to block bb (K slots carry the D = 128 padding)
  auto k_block = [](int bb) { return bb * 512 + (D == 128 ? 64 * (bb >> 1) : 0); };
  auto v_block = [](int bb) { return bb * 512; };
  // page ids of tile t, one per load instruction of this wave, read with
  // wave-uniform loads through the constant address space (the table is
  // read-only during the call), so they land in scalar registers.  The index
  // is clamped to the last entry the unit may read; a block past that range
  // loads nothing anyway (its lanes are out of range).
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  struct PageIds {
    int v[NI];
  };
  c_i32 *trow = nullptr;
  int last_pg = 0;
  if constexpr (kPaged) {
    trow = (c_i32 *)(cg.table + (long)b * cg.mpp);
    last_pg = max(0, min(cg.mpp, (wg_bound + (1 << shift) - 1) >> shift) - 1);
  }
  auto load_ids = [&](int t) -> PageIds {
    PageIds ids;
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      if constexpr (kPaged)
        ids.v[r] = trow[min((t * kPTile + (r * kWaves + wave) * RPB) >> shift, last_pg)];
      else
        ids.v[r] = b;
    }
    return ids;
  };
  // What a tile's loads need, kept in scalar registers from the K load of the
  // tile to its V load one iteration later: per instruction, the page's byte
  // offset in the pool, the descriptor's record count (the slab size, or 0
  // for a page outside the pool, whose loads then all read zeros) and the
  // block's first row inside the page (capped at the slab size so that an
  // out-of-range lane offset cannot wrap back into range).
  const uint32_t pmask = paged ? (1u << shift) - 1u : 0xffffffffu;
  struct TileInfo {
    uint32_t off_lo[NI], off_hi[NI], nrec[NI], uni[NI];
  };
  auto tile_info = [&](int t, const PageIds &ids) -> TileInfo {
    TileInfo ti;
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const uint32_t pg = (uint32_t)ids.v[r];
      const uint64_t off = (uint64_t)pg * slab_bytes;
      ti.off_lo[r] = (uint32_t)off;
      ti.off_hi[r] = (uint32_t)(off >> 32);
      ti.nrec[r] = (!paged || pg < (uint32_t)cg.num_pages) ? slab_bytes : 0u;
      const int key0 = t * kPTile + (r * kWaves + wave) * RPB;
      ti.uni[r] = min(((uint32_t)key0 & pmask) * row_bytes, slab_bytes);
    }
    return ti;
  };
  // one matrix (K or V) of tile t into an LDS slot
  auto load_tile = [&](const uint16_t *cache, uint16_t *slot, uint32_t lane_part, auto block,
                       int t, const TileInfo &ti) {
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const int bb = r * kWaves + wave;
      const int key0 = t * kPTile + bb * RPB;   // first row of the block (wave-uniform)
      const uint16_t *base = (const uint16_t *)((uintptr_t)cache +
                                                (((uint64_t)ti.off_hi[r] << 32) | ti.off_lo[r]));
      const bool ok = key0 + lrow < limit;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(base, ti.nrec[r]),
                                               (lds_void *)(slot + block(bb)), 16,
                                               ok ? lane_part : kOOB, ti.uni[r], 0, 0);
    }
  };
  // rings of four: K of tile t in slot t % 4, V of tile t in slot 4 + t % 4
  uint16_t *const k_slot[4] = {pool.s0, pool.s1, pool.s2, pool.s3};
  uint16_t *const v_slot[4] = {pool.s4, pool.s5, pool.s6, pool.s7};

  // operand reads.  K: lane (n32, hh) reads logical chunk 2 ds + hh of row n32;
  // with ds = 4 j + i that is stored at 8 j + ((2 i + hh) ^ x), x the row's
  // swizzle, so four lane bases and immediate offsets cover every ds.
  int k_rd[4];
  {
    const int x = D == 128 ? (n32 & 7) : ((n32 >> 1) & 7);
    const int row_base = n32 * D + (D == 128 ? 64 * (n32 >> 3) : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) k_rd[i] = row_base + (((2 * i + hh) ^ x) << 3);
  }
  // V^T: lane s of 16-lane group G reads row 4 (G / 2) + s / 4 (+ 16 ks, + 8),
  // dims 32 db + 16 (G & 1) + 4 (s % 4) .. + 3, i.e. logical chunk
  // 4 db + 2 (G & 1) + (s % 4) / 2; its segment db is stored at db ^ y, y the
  // row's segment swizzle (+ 16 and + 8 rows keep it).
  const int G = lane >> 4;
  const int s16 = lane & 15;
  int v_rd[DBP];
  {
    const int y = D == 128 ? (s16 >> 2) : ((s16 >> 3) & 1);
#pragma unroll
    for (int db = 0; db < DBP; ++db)
      v_rd[db] = (4 * (G >> 1) + (s16 >> 2)) * D +
                 ((4 * (db ^ y) + 2 * (G & 1) + ((s16 & 3) >> 1)) << 3) + 4 * (s16 & 1);
  }

  // S^T blocks of one tile: sc[rb], key m of rows rb*32 + n32
  auto qk = [&](const uint16_t *ks, f32x16 (&sc)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sc[rb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < QS; ++ds) {
      const u32x4 a = load16(ks + k_rd[ds & 3] + (ds >> 2) * 64);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sc[rb] = Elt<DT>::mfma32(a, qf[rb][ds], sc[rb]);
    }
  };

  f32x16 o_acc[DBP][RB];
#pragma unroll
  for (int db = 0; db < DBP; ++db)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o_acc[db][rb] = f32x16{};
  float m_run[RB], l_part[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegInf;   // reference maximum of raw scores (possibly stale by < 2^8)
    l_part[rb] = 0.f;
  }
  const float c2 = p.scale_log2;

  float m_sc[RB];   // m_run * c2, 0 for an empty reference
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) m_sc[rb] = 0.f;

  // The online softmax is split around the MFMA work.  tile_max(t) runs as
  // soon as tile t's scores exist (beside the PV product of the previous
  // tile): mask, row maximum, and - when the maximum grew by more than 2^8 -
  // a new reference, with the row sum and the accumulator rescaled to it.
  // exp_pv(t) then runs one iteration later beside the next tile's QK^T:
  // probabilities against the reference, row sums, O^T += V^T P^T.
  // The row sums add the probabilities as rounded for the PV product (so a
  // constant V comes back exactly), and each tile's sum is pinned to its
  // iteration: left alone, the compiler defers the sums of a whole unrolled
  // group to the loop latch and keeps every probability live until then.
  // Lane (n32, hh) element i of sc[rb] is key t*32 + (i/4)*8 + 4*hh + i%4.
  auto tile_max = [&](int t, f32x16 (&sc)[RB], bool masked) {
    float alpha[RB];
    bool moved = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (masked) {
          const int key = t * kPTile + (i >> 2) * 8 + 4 * hh + (i & 3);
          sc[rb][i] = key < row_lim[rb] ? sc[rb][i] : kNegInf;
        }
        tmax = fmaxf(tmax, sc[rb][i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const bool move = (tmax - m_run[rb]) * c2 > kRescaleThreshold;
      const float m_ref = move ? tmax : m_run[rb];
      alpha[rb] = move ? fast_exp2((m_run[rb] - m_ref) * c2) : 1.f;
      moved |= move;
      m_run[rb] = m_ref;
      m_sc[rb] = m_ref == kNegInf ? 0.f : m_ref * c2;
      l_part[rb] *= alpha[rb];
    }
    if (__any(moved)) {
#pragma unroll
      for (int db = 0; db < DBP; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o_acc[db][rb] *= alpha[rb];
    }
  };
  auto exp_pv = [&](const uint16_t *vs, const f32x16 (&sc)[RB]) {
    // P^T operands: k-step ks (16 keys) takes elements ks*8 .. ks*8+7
    u32x4 pb[RB][2], pb_lo[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float l = l_part[rb];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(sc[rb][ks * 8 + 2 * e], c2, -m_sc[rb]));
          const float p1 = fast_exp2(__builtin_fmaf(sc[rb][ks * 8 + 2 * e + 1], c2, -m_sc[rb]));
          pb[rb][ks][e] = pack2<DT>(p0, p1);
          l = add_pair<DT>(pb[rb][ks][e], l);
          if constexpr (DT == kBF16) {
            pb_lo[rb][ks][e] = pack2<DT>(p0 - Elt<DT>::to_f32((uint16_t)(pb[rb][ks][e] & 0xffffu)),
                                         p1 - Elt<DT>::to_f32((uint16_t)(pb[rb][ks][e] >> 16)));
            l = add_pair<DT>(pb_lo[rb][ks][e], l);
          }
        }
      }
      asm volatile("" : "+v"(l));
      l_part[rb] = l;
    }
    // PV: lane group G reads dims db*32 + 16*(G&1) + 0..15, keys of k half G>>1
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < DBP; ++db) {
        const uint16_t *vt = vs + v_rd[db] + ks * 16 * D;
        const u32x2 a0 = lds_read_tr16(vt);
        const u32x2 a1 = lds_read_tr16(vt + 8 * D);
        const u32x4 va = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          o_acc[db][rb] = Elt<DT>::mfma32(va, pb[rb][ks], o_acc[db][rb]);
          if constexpr (DT == kBF16) o_acc[db][rb] = Elt<DT>::mfma32(va, pb_lo[rb][ks], o_acc[db][rb]);
        }
      }
    }
  };

  // prologue: K of tiles 0-3 and V of tiles 0-2 into LDS, S^T of tile 0; the
  // second barrier lets every wave finish reading K(0) before its slot is
  // refilled.  Loads past the bound are zeros, so nothing here is conditional.
  f32x16 s_a[RB], s_b[RB];
  TileInfo ti_v;    // loads of tile t+3 at the start of iteration t (its K is in flight)
  PageIds ids_k;    // page ids of tile t+4
  {
    const TileInfo ti_0 = tile_info(0, load_ids(0));
    const TileInfo ti_1 = tile_info(1, load_ids(1));
    const TileInfo ti_2 = tile_info(2, load_ids(2));
    ti_v = tile_info(3, load_ids(3));
    ids_k = load_ids(4);
    load_tile(p.k_cache, k_slot[0], k_lane, k_block, 0, ti_0);
    load_tile(p.v_cache, v_slot[0], v_lane, v_block, 0, ti_0);
    load_tile(p.k_cache, k_slot[1], k_lane, k_block, 1, ti_1);
    load_tile(p.v_cache, v_slot[1], v_lane, v_block, 1, ti_1);
    load_tile(p.k_cache, k_slot[2], k_lane, k_block, 2, ti_2);
    load_tile(p.v_cache, v_slot[2], v_lane, v_block, 2, ti_2);
    load_tile(p.k_cache, k_slot[3], k_lane, k_block, 3, ti_v);
  }
  wait_then_barrier<0>();
  qk(k_slot[0], s_a);
  tile_max(0, s_a, n_full == 0);
  wait_then_barrier<0>();

  // iteration t (ph = t % 4): page ids of tile t+5, then K(t+4) into the slot
  // K(t) used and V(t+3) into the slot V(t-1) used; QK^T of tile t+1 beside
  // the probabilities of tile t, the PV product of tile t, and tile t+1's
  // maximum beside that.  At the barrier the loads issued two iterations
  // earlier - K(t+2) and V(t+1), read next iteration - must have landed; the
  // newest two iterations' loads stay in flight.  Full tiles: every wave
  // computes, no mask, and no branch before the rare rescale.  Tail tiles:
  // waves whose rows see nothing of a tile skip it.
  constexpr int kLoadsPerIter = 2 * NI;   // vector loads (the page ids are scalar)
  auto iter = [&](int t, int ph, f32x16 (&cur)[RB], f32x16 (&nxt)[RB], bool tail) {
    const PageIds ids_new = load_ids(t + 5);
    const TileInfo ti_k = tile_info(t + 4, ids_k);
    load_tile(p.k_cache, k_slot[ph], k_lane, k_block, t + 4, ti_k);
    load_tile(p.v_cache, v_slot[(ph + 3) & 3], v_lane, v_block, t + 3, ti_v);
    if (!tail) {
      qk(k_slot[(ph + 1) & 3], nxt);
      exp_pv(v_slot[ph], cur);
      tile_max(t + 1, nxt, false);
    } else {
      const bool next_seen = (t + 1) * kPTile < wave_bound;
      if (next_seen) qk(k_slot[(ph + 1) & 3], nxt);
      if (t * kPTile < wave_bound) exp_pv(v_slot[ph], cur);
      if (next_seen) tile_max(t + 1, nxt, true);
    }
    wait_then_barrier<2 * kLoadsPerIter>();
    ti_v = ti_k;
    ids_k = ids_new;
  };
  // the branch-free loop takes a multiple of four tiles whose successors are
  // full as well (so its unmasked maxima are right), every slot index is a
  // constant, and the masked loop starts on the same registers
  const int n_main = max(n_full - 1, 0) & ~3;
  int t = 0;
  for (; t < n_main; t += 4) {
    iter(t, 0, s_a, s_b, false);
    iter(t + 1, 1, s_b, s_a, false);
    iter(t + 2, 2, s_a, s_b, false);
    iter(t + 3, 3, s_b, s_a, false);
  }
  for (; t < n_t; t += 4) {
    iter(t, 0, s_a, s_b, true);
    if (t + 1 < n_t) iter(t + 1, 1, s_b, s_a, true);
    if (t + 2 < n_t) iter(t + 2, 2, s_a, s_b, true);
    if (t + 3 < n_t) iter(t + 3, 3, s_b, s_a, true);
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!row_ok[rb]) continue;
    const float L = l_part[rb] + __shfl_xor(l_part[rb], 32, 64);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const long ridx = (long)(si.cu_b + tok[rb]) * p.hq + hq_[rb];
    uint16_t *dst = p.out + ridx * D;
#pragma unroll
    for (int db = 0; db < DBP; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 pk;
        pk[0] = pack2<DT>(o_acc[db][rb][q4 * 4 + 0] * inv, o_acc[db][rb][q4 * 4 + 1] * inv);
        pk[1] = pack2<DT>(o_acc[db][rb][q4 * 4 + 2] * inv, o_acc[db][rb][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2 *>(dst + db * 32 + q4 * 8 + 4 * hh) = pk;
      }
    }
    if (hh == 0) p.lse[ridx] = empty ? kNegInf : (m_run[rb] * c2 + __builtin_log2f(L)) * kLn2;
  }
}

}  // namespace pa
