// Prefill unit of the gfx950 paged KV-cache attention forward pass.
#pragma once

#include <type_traits>

#include "pa_common.h"

namespace pa {

// ---------------------------------------------------------------------------
// Prefill unit: 256 packed rows (32 per wave, eight waves) of one sequence and
// kv head, every key those rows can see, one split, in 32-key tiles.
//   ping-pong    the waves form two groups of four, A (waves 0-3) and B (waves
//                4-7), one wave of each on every SIMD.  For every tile a wave
//                runs an MFMA phase - S^T(t+1) = K Q^T and O^T += V^T P^T(t),
//                32x32x16 MFMAs with keys on M, all operand reads issued up
//                front - and a softmax phase.  A starts each tile with its
//                MFMA phase, B with its softmax phase, so every SIMD overlaps
//                one wave's matrix work with the other's vector work.  Both
//                waves keep the default issue priority: raising the MFMA
//                phase's starves the other wave's softmax.
//   loads        the K and V rows of a tile move from the page straight into
//                LDS (buffer loads with an LDS destination: lane l of an
//                instruction fills bytes 16 l .. 16 l + 15 of one 1 KiB block,
//                and the lane picks which 16-byte chunk of which row it
//                fetches, so the swizzles below are free); at D = 128 wave w
//                fills block w of both, at D = 64 waves 0-3 the K blocks and
//                waves 4-7 the V blocks; keys past the visible range and pages outside the
//                pool load as zeros; page ids come through scalar loads by
//                absolute logical index;
//   LDS          rings of four K and four V slots (separate LDS objects), one
//                barrier per tile; the loads of the next two tiles stay in
//                flight across it;
//   softmax      online, log2 units, against a reference maximum that only
//                moves when needed (see below), so rescaling is rare; row sums
//                add the fp32 probabilities with plain adds (the packed
//                dot-product instruction does not overlap with MFMAs).
// Tiles every row of the unit sees in full run in a mask-free loop; the tiles
// on the causal diagonal follow in a masked loop.
// ---------------------------------------------------------------------------
constexpr float kRescaleThreshold = 8.f;   // log2 units
constexpr float kSumBound = 16384.f;       // 2^14

template <int DT, int D, bool kPaged>
__device__ __forceinline__ void prefill_unit(const FwdParams &p, const int b, const int g,
                                             const int qtile, const SeqInfo si,
                                             const LdsPool &pool) {
  constexpr int NW = kUWaves;
  constexpr int QS = D / 16;        // k-steps over D (16 dims each)
  constexpr int DBP = D / 32;       // 32-dim blocks of O^T
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPB = 64 / CPR;     // rows per 1 KiB load block (4 or 8)
  constexpr int BPM = kPTile / RPB; // 1 KiB blocks per tile and matrix: waves 0 .. BPM-1 load
  static_assert(BPM <= NW && BPM * RPB == kPTile, "a tile must split into the waves' blocks");
  static_assert(RPB == 4 || RPB == 8, "swizzle bookkeeping assumes 4 or 8 rows per block");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const bool grp_b = wave >= NW / 2;
  const int n32 = lane & 31;       // MFMA column (row within the wave's 32 rows)
  const int hh = lane >> 5;        // k half
  const int group = p.group;
  const int rows_b = si.q_len * group;
  const int wg_row0 = qtile * kPrefillRows;
  const int wg_rows = min(kPrefillRows, rows_b - wg_row0);
  const int wg_bound = row_key_bound(wg_row0 + wg_rows - 1, group, si.q_len, si.K_b, p.causal);
  const int wg_first = row_key_bound(wg_row0, group, si.q_len, si.K_b, p.causal);
  const int n_t = (wg_bound + kPTile - 1) / kPTile;
  const int n_full = min(wg_first / kPTile, n_t);   // tiles every row sees in full

  const int row0 = wg_row0 + wave * 32;
  const int rows_here = min(32, rows_b - row0);     // <= 0: idle wave
  const int wave_bound =
      rows_here > 0 ? row_key_bound(row0 + rows_here - 1, group, si.q_len, si.K_b, p.causal) : 0;
  const bool row_ok = n32 < rows_here;
  const int tok = row_ok ? (row0 + n32) / group : 0;
  const int hq = g * group + (row_ok ? row0 + n32 - tok * group : 0);
  const int row_lim = row_ok ? row_key_bound(row0 + n32, group, si.q_len, si.K_b, p.causal) : 0;

  u32x4 qf[QS];
  {
    const uint16_t *qrow = p.q + (long)(si.cu_b + tok) * p.q_stride + (long)hq * D;
#pragma unroll
    for (int ds = 0; ds < QS; ++ds)
      qf[ds] = row_ok ? load16(qrow + ds * 16 + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
  }
  // fused rotary embedding of the query row, at the token's position
  // K_b - q_len + tok: its table entries are fetched with the row and applied
  // after the prologue's wait, so their latency hides behind the first tiles'
  // loads
  const bool rot_q = p.rot.cos != nullptr;
  const int rot_pos = row_ok ? si.K_b - si.q_len + tok : -1;
  u32x4 rot_c[QS / 2], rot_s[QS / 2];
  if (rot_q) rot_fetch_split<QS>(p.rot, rot_pos, hh, rot_c, rot_s);

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
  // Loading wave w fills block w of a K and a V slot: rows w * RPB + lane / CPR,
  // physical chunk lane % CPR, i.e. the logical chunk that the row's swizzle
  // puts there; the lane part of every byte offset is loop-invariant.
  const CacheGeom &cg = p.geom;
  constexpr bool paged = kPaged;   // block table (else one contiguous allocation per sequence)
  // Every wave issues the same tile loads at the same program points: at
  // D = 128 (eight blocks per tile) wave w fills block w of a K and of a V
  // tile, at D = 64 (four blocks) waves 0-3 fill the K blocks and waves 4-7
  // the V blocks.
  constexpr bool kSplitKV = 2 * BPM == NW;
  static_assert(BPM == NW || kSplitKV, "blocks per tile: one or two per wave");
  const int bb = wave % BPM;
  const bool k_wave = !kSplitKV || wave < BPM;
  const int shift = cg.page_shift;
  const uint32_t row_bytes = (uint32_t)p.hkv * D * 2;
  const uint32_t slab_bytes = paged ? row_bytes << shift : (uint32_t)cg.contig_alloc * row_bytes;
  const int limit = paged ? wg_bound : min(wg_bound, cg.contig_alloc);
  const int lrow = lane / CPR;
  const int pch = lane % CPR;
  const int kx = D == 128 ? ((4 * (bb & 1) + lrow) & 7) : ((4 * bb + (lrow >> 1)) & 7);
  const int vx = D == 128 ? ((lrow & 3) << 2) : (((lrow >> 1) & 1) << 2);
  const uint32_t k_lane = (uint32_t)lrow * row_bytes + (uint32_t)(g * D + ((pch ^ kx) << 3)) * 2;
  const uint32_t v_lane = (uint32_t)lrow * row_bytes + (uint32_t)(g * D + ((pch ^ vx) << 3)) * 2;
  // halves from a slot's start to this wave's block (K slots carry the D = 128
  // padding)
  const int k_blk = bb * 512 + (D == 128 ? 64 * (bb >> 1) : 0);
  const int v_blk = bb * 512;
  // page id of this wave's block of tile t, read with a wave-uniform load
  // through the constant address space (the table is read-only during the
  // call), so it lands in a scalar register.  The index is clamped to the last
  // entry the unit may read; a block past that range loads nothing anyway.
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  c_i32 *trow = nullptr;
  int last_pg = 0;
  if constexpr (kPaged) {
    trow = (c_i32 *)(cg.table + (long)b * cg.mpp);
    last_pg = max(0, min(cg.mpp, (wg_bound + (1 << shift) - 1) >> shift) - 1);
  }
  auto load_id = [&](int t) -> int {
    if constexpr (kPaged)
      return trow[min((t * kPTile + bb * RPB) >> shift, last_pg)];
    else
      return b;
  };
  // What a tile's loads need, kept in scalar registers from the K load of the
  // tile to its V load one iteration later: the page's byte offset in the
  // pool, the descriptor's record count (the slab size, or 0 for a page
  // outside the pool, whose loads then all read zeros) and the block's first
  // row inside the page (capped at the slab size so that an out-of-range lane
  // offset cannot wrap back into range).
  const uint32_t pmask = paged ? (1u << shift) - 1u : 0xffffffffu;
  struct TileInfo {
    uint32_t off_lo, off_hi, nrec, uni;
  };
  auto tile_info = [&](int t, int id) -> TileInfo {
    const uint32_t pg = (uint32_t)id;
    const uint64_t off = (uint64_t)pg * slab_bytes;
    TileInfo ti;
    ti.off_lo = (uint32_t)off;
    ti.off_hi = (uint32_t)(off >> 32);
    ti.nrec = (!paged || pg < (uint32_t)cg.num_pages) ? slab_bytes : 0u;
    ti.uni = min(((uint32_t)(t * kPTile + bb * RPB) & pmask) * row_bytes, slab_bytes);
    return ti;
  };
  // this wave's block of one matrix (K or V) of tile t into an LDS slot
  auto load_block = [&](const uint16_t *cache, uint16_t *slot, uint32_t lane_part, int blk, int t,
                        const TileInfo &ti) {
    const uint16_t *base =
        (const uint16_t *)((uintptr_t)cache + (((uint64_t)ti.off_hi << 32) | ti.off_lo));
    const bool ok = t * kPTile + bb * RPB + lrow < limit;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(base, ti.nrec), (lds_void *)(slot + blk), 16,
                                             ok ? lane_part : kOOB, ti.uni, 0, 0);
  };
  // rings of four: K of tile t in slot t % 4, V of tile t in slot 4 + t % 4
  uint16_t *const k_slot[4] = {pool.s(0), pool.s(1), pool.s(2), pool.s(3)};
  uint16_t *const v_slot[4] = {pool.s(4), pool.s(5), pool.s(6), pool.s(7)};

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

  f32x16 o_acc[DBP];
#pragma unroll
  for (int db = 0; db < DBP; ++db) o_acc[db] = f32x16{};
  float m_run = kNegInf;   // reference maximum of raw scores (possibly stale by < 2^8)
  float m_sc = 0.f;        // m_run * c2, 0 for an empty reference
  float l_part = 0.f;      // this lane's share of the row sum
  const float c2 = p.scale_log2;

  // S^T of one tile: lane (n32, hh) element i is key (i/4)*8 + 4*hh + i%4 of row n32
  auto qk = [&](const uint16_t *ks, f32x16 &sc) {
    sc = f32x16{};
#pragma unroll
    for (int ds = 0; ds < QS; ++ds)
      sc = Elt<DT>::mfma32(load16(ks + k_rd[ds & 3] + (ds >> 2) * 64), qf[ds], sc);
  };
  // The reference only needs to move when probabilities against it would
  // grow too large, so a tile first takes its probabilities against the
  // reference it has and checks them: while every lane's sum of its sixteen
  // stays within 2^14 (each probability then fits both 16-bit formats with
  // room to spare), nothing else is needed - no row maximum at all.  Otherwise
  // (and for a wave's first tile, which has no reference yet) the exact row
  // maximum is taken, the reference moves to it where it grew by more than
  // 2^8 - rescaling the row sum and the accumulator - and the probabilities
  // are taken again.  A reference is always a maximum the row has seen, so
  // the row sum never falls below 1.
  struct Probs {
    u32x4 hi[2], lo[2];
  };
  // probabilities against the reference, packed as the PV B operand (k-step
  // ks takes elements ks*8 .. ks*8+7; bf16 keeps a low part as well, so the
  // product sees ~16 bits of each probability); returns the lane's sum of the
  // fp32 probabilities (plain adds: a packed dot-product instruction would
  // wait behind the other wave's MFMAs on this SIMD)
  auto make_p = [&](const f32x16 &sc, Probs &pr) -> float {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float &l = ks == 0 ? l0 : l1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(__builtin_fmaf(sc[ks * 8 + 2 * e], c2, -m_sc));
        const float p1 = fast_exp2(__builtin_fmaf(sc[ks * 8 + 2 * e + 1], c2, -m_sc));
        pr.hi[ks][e] = pack2<DT>(p0, p1);
        l += p0 + p1;
        if constexpr (DT == kBF16) {
          pr.lo[ks][e] = pack2<DT>(p0 - Elt<DT>::to_f32((uint16_t)(pr.hi[ks][e] & 0xffffu)),
                                   p1 - Elt<DT>::to_f32((uint16_t)(pr.hi[ks][e] >> 16)));
        } else {
          pr.lo[ks][e] = 0u;
        }
      }
    }
    return l0 + l1;
  };
  // exact row maximum (both k halves: lanes l and l ^ 32 hold the two halves
  // of a row) and, where it grew by more than 2^8, a new reference
  bool have_ref = false;   // wave-uniform: every valid row of the wave has a reference
  auto move_ref = [&](const f32x16 &sc) {
    float tmax = fmaxf(__builtin_fmaxf(sc[0], sc[1]), sc[2]);
    float t1 = fmaxf(__builtin_fmaxf(sc[3], sc[4]), sc[5]);
    float t2 = fmaxf(__builtin_fmaxf(sc[6], sc[7]), sc[8]);
    float t3 = fmaxf(__builtin_fmaxf(sc[9], sc[10]), sc[11]);
    float t4 = fmaxf(__builtin_fmaxf(sc[12], sc[13]), sc[14]);
    tmax = fmaxf(fmaxf(tmax, t1), t2);
    t3 = fmaxf(fmaxf(t3, t4), sc[15]);
    tmax = fmaxf(tmax, t3);
    // one swap leaves the lower half's value in the first result and the
    // upper half's in the second, on every lane.  The results pass through an
    // empty asm: left visible, the compiler takes the second result for a copy
    // of the first and drops it.
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, tmax),
                                                     __builtin_bit_cast(uint32_t, tmax), false, false);
    uint32_t lo_half = sw[0], hi_half = sw[1];
    asm volatile("" : "+v"(lo_half), "+v"(hi_half));
    tmax = fmaxf(__builtin_bit_cast(float, lo_half), __builtin_bit_cast(float, hi_half));
    const bool move = (tmax - m_run) * c2 > kRescaleThreshold;
    const float m_ref = move ? tmax : m_run;
    const float alpha = move ? fast_exp2((m_run - m_ref) * c2) : 1.f;
    m_run = m_ref;
    m_sc = m_ref == kNegInf ? 0.f : m_ref * c2;
    l_part *= alpha;
    if (__any(move)) {
#pragma unroll
      for (int db = 0; db < DBP; ++db) o_acc[db] *= alpha;
    }
    have_ref = !__any(row_ok && m_run == kNegInf);
  };
  // softmax of tile t: mask (diagonal tiles), probabilities, row sum
  auto softmax = [&](int t, f32x16 &sc, bool masked) -> Probs {
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t * kPTile + (i >> 2) * 8 + 4 * hh + (i & 3);
        sc[i] = key < row_lim ? sc[i] : kNegInf;
      }
    }
    Probs pr;
    float ls = make_p(sc, pr);
    if (!have_ref || __any(!(ls <= kSumBound))) {
      move_ref(sc);
      ls = make_p(sc, pr);
    }
    l_part += ls;
    return pr;
  };
  // The MFMA phase: S^T of the next tile (K Q^T) and O^T += V^T P^T of this
  // one (lane group G reads dims db*32 + 16*(G&1) + 0..15 of the keys of k
  // half G>>1).  Every operand read goes out before the MFMAs that need it
  // have started - K first, then V - so that the phase waits for LDS once
  // rather than at every MFMA; in full tiles the order is pinned: K reads,
  // V reads of the first k-step, half of the S^T MFMAs, V reads of the second
  // k-step, the remaining MFMAs.
  constexpr int kPvMfma = 2 * DBP * (DT == kBF16 ? 2 : 1);
  auto mfma_phase = [&](const uint16_t *ks, const uint16_t *vs, const Probs &pr, f32x16 &sn,
                        bool do_qk, bool do_pv, bool pin) {
    u32x4 kop[QS];
    u32x4 vop[2][DBP];
    if (do_qk) {
#pragma unroll
      for (int ds = 0; ds < QS; ++ds) kop[ds] = load16(ks + k_rd[ds & 3] + (ds >> 2) * 64);
    }
    if (do_pv) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int db = 0; db < DBP; ++db) {
          const uint16_t *vt = vs + v_rd[db] + kk * 16 * D;
          const u32x2 a0 = lds_read_tr16(vt);
          const u32x2 a1 = lds_read_tr16(vt + 8 * D);
          vop[kk][db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
        }
      }
    }
    if (do_qk) {
      sn = f32x16{};
#pragma unroll
      for (int ds = 0; ds < QS; ++ds) sn = Elt<DT>::mfma32(kop[ds], qf[ds], sn);
    }
    if (do_pv) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int db = 0; db < DBP; ++db) {
          o_acc[db] = Elt<DT>::mfma32(vop[kk][db], pr.hi[kk], o_acc[db]);
          if constexpr (DT == kBF16) o_acc[db] = Elt<DT>::mfma32(vop[kk][db], pr.lo[kk], o_acc[db]);
        }
      }
    }
    if (pin) {
      __builtin_amdgcn_sched_group_barrier(0x100, QS, 0);            // K reads
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DBP, 0);       // V reads, k-step 0
      __builtin_amdgcn_sched_group_barrier(0x008, QS / 2, 0);        // S^T MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DBP, 0);       // V reads, k-step 1
      __builtin_amdgcn_sched_group_barrier(0x008, QS / 2 + kPvMfma, 0);
    }
  };
  // What a wave carries from one tile to the next, in sixteen integer
  // registers: group A the packed probabilities of its next tile, group B the
  // bits of the scores of its next tile.  The carry must stay an integer
  // vector: the same bits carried inside a float vector (bit-cast in and out)
  // gave wrong outputs for group A's rows with the ROCm 7.2 compiler, while
  // the integer carry is bit-exact; the assertions below keep it that way.
  typedef uint32_t carry_word;
  typedef carry_word u32x16 __attribute__((ext_vector_type(16)));
  static_assert(std::is_integral<carry_word>::value && sizeof(u32x16) == 64,
                "the ping-pong carry is sixteen integer words");
  auto put_p = [](const Probs &pr) -> u32x16 {
    u32x16 c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = pr.hi[0][e];
      c[4 + e] = pr.hi[1][e];
      c[8 + e] = pr.lo[0][e];
      c[12 + e] = pr.lo[1][e];
    }
    return c;
  };
  static_assert(std::is_same<decltype(put_p(Probs{})), u32x16>::value,
                "probabilities are carried in the integer vector");
  auto get_p = [](const u32x16 &c) -> Probs {
    Probs pr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr.hi[0][e] = c[e];
      pr.hi[1][e] = c[4 + e];
      pr.lo[0][e] = c[8 + e];
      pr.lo[1][e] = c[12 + e];
    }
    return pr;
  };
  // prologue: K of tiles 0-3 and V of tiles 0-2 into LDS; S^T of tile 0, and
  // for group A its probabilities as well; the second barrier lets every wave
  // finish reading K(0) before its slot is refilled.  Loads past the bound are
  // zeros, so nothing here is conditional on the unit's length.
  u32x16 carry;
  TileInfo ti_v;   // loads of tile t+3 at the start of iteration t (its K is in flight)
  int id_k;        // page id of tile t+4
  {
    const TileInfo ti_0 = tile_info(0, load_id(0));
    const TileInfo ti_1 = tile_info(1, load_id(1));
    const TileInfo ti_2 = tile_info(2, load_id(2));
    ti_v = tile_info(3, load_id(3));
    id_k = load_id(4);
    if (k_wave) {
      load_block(p.k_cache, k_slot[0], k_lane, k_blk, 0, ti_0);
      load_block(p.k_cache, k_slot[1], k_lane, k_blk, 1, ti_1);
      load_block(p.k_cache, k_slot[2], k_lane, k_blk, 2, ti_2);
      load_block(p.k_cache, k_slot[3], k_lane, k_blk, 3, ti_v);
    }
    if (!kSplitKV || !k_wave) {
      load_block(p.v_cache, v_slot[0], v_lane, v_blk, 0, ti_0);
      load_block(p.v_cache, v_slot[1], v_lane, v_blk, 1, ti_1);
      load_block(p.v_cache, v_slot[2], v_lane, v_blk, 2, ti_2);
    }
  }
  wait_then_barrier<0>();
  if (rot_q) rot_apply_split<DT, QS>(p.rot, rot_pos, hh, qf, rot_c, rot_s);
  {
    f32x16 s0;
    qk(k_slot[0], s0);
    if (!grp_b) {
      carry = put_p(softmax(0, s0, n_full == 0));
    } else {
      carry = __builtin_bit_cast(u32x16, s0);
    }
  }
  wait_then_barrier<0>();

  // iteration t (ph = t % 4): page id of tile t+5, then K(t+4) into the slot
  // K(t) used and V(t+3) into the slot V(t-1) used; both groups read K(t+1)
  // and V(t).  At the barrier the loads issued two iterations earlier - K(t+2)
  // and V(t+1), read next iteration - must have landed; the newest two
  // iterations' loads stay in flight.  Full tiles: no mask.  Tail tiles: a
  // wave skips the tiles its rows cannot see.
  constexpr int kLoadsPerIter = kSplitKV ? 1 : 2;   // vector loads of a wave (page ids are scalar)
  auto iter = [&](int t, int ph, bool tail) {
    // After its MFMA phase every wave reads the page id of tile t+5 and
    // issues its tile loads, at one program point for both groups and every
    // iteration.  Both placements are pinned for the compiler's waits:
    //  - a scalar load still in flight during the MFMA phase would turn each
    //    LDS wait of the phase into a full drain (scalar and LDS loads share a
    //    counter, and scalar loads may return out of order);
    //  - the waits the compiler adds for LDS-destination loads follow every
    //    path through the loop, not just the ones a wave can take; with loads
    //    issued at group-dependent points, or in iterations that may be
    //    skipped, a path with fewer loads makes the explicit wait before the
    //    barrier look too weak, and the compiler then drains every load in
    //    flight before the reads of a slot filled three iterations earlier.
    TileInfo ti_k;
    auto issue_loads = [&]() {
      ti_k = tile_info(t + 4, id_k);
      if (!kSplitKV) {
        load_block(p.k_cache, k_slot[ph], k_lane, k_blk, t + 4, ti_k);
        load_block(p.v_cache, v_slot[(ph + 3) & 3], v_lane, v_blk, t + 3, ti_v);
      } else if (k_wave) {
        load_block(p.k_cache, k_slot[ph], k_lane, k_blk, t + 4, ti_k);
      } else {
        load_block(p.v_cache, v_slot[(ph + 3) & 3], v_lane, v_blk, t + 3, ti_v);
      }
    };
    const uint16_t *ks = k_slot[(ph + 1) & 3];
    const uint16_t *vs = v_slot[ph];
    const bool seen_t = !tail || t * kPTile < wave_bound;
    const bool seen_n = !tail || (t + 1) * kPTile < wave_bound;
    // B: the softmax of t from its carried scores; A: the probabilities it
    // carried.  Then the MFMA phase, common to both groups (one program
    // point updates the accumulator, which keeps it in one set of
    // registers), and A's softmax of t+1.
    Probs pr;
    if (grp_b) {
      if (seen_t) {
        f32x16 sc = __builtin_bit_cast(f32x16, carry);
        pr = softmax(t, sc, tail);
      }
    } else {
      pr = get_p(carry);
    }
    f32x16 sn;
    asm volatile("" ::"s"(id_k));   // the id read an iteration ago has landed
    mfma_phase(ks, vs, pr, sn, seen_n, seen_t, !tail);
    __builtin_amdgcn_sched_barrier(0);
    const int id_new = load_id(t + 5);
    issue_loads();
    if (seen_n) {
      if (!grp_b) {
        carry = put_p(softmax(t + 1, sn, tail));
      } else {
        carry = __builtin_bit_cast(u32x16, sn);
      }
    }
    wait_then_barrier<2 * kLoadsPerIter>();
    ti_v = ti_k;
    id_k = id_new;
  };
  // the mask-free loop takes a multiple of four tiles whose successors are
  // full as well (so its unmasked maxima are right), and every slot index is
  // a constant
  const int n_main = max(n_full - 1, 0) & ~3;
  int t = 0;
  for (; t < n_main; t += 4) {
    iter(t, 0, false);
    iter(t + 1, 1, false);
    iter(t + 2, 2, false);
    iter(t + 3, 3, false);
  }
  // the masked loop runs whole groups of four (iterations past the last tile
  // see no tile: they only load zeros and meet the barrier)
  for (; t < n_t; t += 4) {
    iter(t, 0, true);
    iter(t + 1, 1, true);
    iter(t + 2, 2, true);
    iter(t + 3, 3, true);
  }

  if (!row_ok) return;
  const float L = l_part + __shfl_xor(l_part, 32, 64);
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.f / L;
  const long ridx = (long)(si.cu_b + tok) * p.hq + hq;
  uint16_t *dst = p.out + ridx * D;
#pragma unroll
  for (int db = 0; db < DBP; ++db) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 pk;
      pk[0] = pack2<DT>(o_acc[db][q4 * 4 + 0] * inv, o_acc[db][q4 * 4 + 1] * inv);
      pk[1] = pack2<DT>(o_acc[db][q4 * 4 + 2] * inv, o_acc[db][q4 * 4 + 3] * inv);
      *reinterpret_cast<u32x2 *>(dst + db * 32 + q4 * 8 + 4 * hh) = pk;
    }
  }
  if (hh == 0) p.lse[ridx] = empty ? kNegInf : (m_run * c2 + __builtin_log2f(L)) * kLn2;
  // written directly: the combine that follows a split batch skips the row
  if (hh == 0 && p.row_splits != nullptr) p.row_splits[ridx] = 1;
}

}  // namespace pa
