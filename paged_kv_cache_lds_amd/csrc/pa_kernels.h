// gfx950 kernels of the paged KV-cache attention forward pass.
//
//   kv_append_kernel   new K/V rows -> their page slots (bit copy)
//   attn_fwd_kernel    one unified varlen kernel: decode units and prefill
//                      tiles in one grid; QK^T and PV on MFMA with fp32
//                      accumulation, online softmax, split-KV partial or final
//                      epilogue
//   combine_kernel     log-sum-exp merge of split-KV partials
#pragma once

#include "pa_device.h"

namespace pa {

// Work decomposition constants.
constexpr int kThreads = 256;     // four wave64 per workgroup
constexpr int kWaves = 4;
constexpr int kKeyTile = 32;      // decode: keys per wave main-loop iteration
constexpr int kDecodeRows = 16;   // packed (token, q-head) rows of a decode unit
constexpr int kPrefillRB = 1;     // 32-row MFMA blocks per wave in a prefill unit
constexpr int kPrefillRows = 32 * kPrefillRB * kWaves;   // rows of a prefill unit
constexpr int kPTile = 32;        // prefill: keys per workgroup main-loop iteration
constexpr int kMaxSplits = 128;
constexpr int kWindow = 64;       // block-table entries a wave holds at once (one per lane)

struct FwdParams {
  const uint16_t *q;
  const uint16_t *k_cache;
  const uint16_t *v_cache;
  CacheGeom geom;
  const int32_t *cache_seqlens;
  const int32_t *cu_seqlens_q;
  uint16_t *out;
  float *lse;
  float *o_part;       // [max_splits, total_q, hq, D] fp32 (num_splits > 1)
  float *lse_part;     // [max_splits, total_q, hq]
  int32_t *split_count;// [batch]: splits given to each decode-mode sequence
  int batch, total_q, hq, hkv, group;
  int appended, causal, num_splits;
  float scale_log2;    // softmax scale * log2(e)
  int all_decode;      // host knows every sequence has q_len * group <= 16
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
// Per-sequence bookkeeping shared by every workgroup (and by the combine).
// ---------------------------------------------------------------------------
struct SeqInfo {
  int cu_b, q_len, K_b;
};

__device__ inline SeqInfo seq_info(const FwdParams &p, int b) {
  SeqInfo s;
  s.cu_b = p.cu_seqlens_q[b];
  s.q_len = max(0, min(p.cu_seqlens_q[b + 1], p.total_q) - s.cu_b);
  s.K_b = max(0, p.cache_seqlens[b]) + (p.appended ? s.q_len : 0);
  return s;
}

// Splits of a decode-mode sequence.  The host fixes the unit budget per kv
// head (num_splits per decode sequence on average) from static sizes only;
// here, with the real lengths in hand, every decode sequence keeps one unit
// and the remaining budget is shared in proportion to its key tiles, so long
// sequences get more splits than short ones (cache_seqlens never travels to
// the host).  A pure function of the lengths: every workgroup agrees on it.
__device__ inline int seq_splits(long extra_budget, long tiles_b, long total_tiles) {
  if (extra_budget <= 0 || total_tiles <= 0) return 1;
  const long s = 1 + (extra_budget * tiles_b) / total_tiles;
  return (int)min(s, (long)kMaxSplits);
}

__device__ inline int decode_tiles(int K_b) { return (K_b + kKeyTile - 1) / kKeyTile; }

// inclusive prefix sum over the workgroup (every thread contributes x);
// `total` receives the workgroup sum
__device__ inline int block_inclusive_scan(int x, int *s_wsum, int &total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wsum[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int v = s_wsum[w];
    before += (w < wave) ? v : 0;
    total += v;
  }
  __syncthreads();
  return before + x;
}

// Unified work mapping.  Units per kv head: a sequence whose packed rows
// (q_len * group) fit one 16-row decode unit gets seq_splits() units (its
// keys split across workgroups); a longer one gets cdiv(rows, 128) prefill
// units, heaviest (last, under the causal mask) first.  The host sizes the
// grid from static maxima; each workgroup finds its (sequence, unit) by
// block-wide scans over the device metadata, and surplus workgroups return.
struct UnitInfo {
  int b, off, splits;   // off = split (decode) or query tile (prefill)
};

__device__ inline bool locate_unit(const FwdParams &p, int unit, UnitInfo &u, int *s_wsum,
                                   int *s_found) {
  const int tid = threadIdx.x;
  const int S = p.num_splits;
  // pass 1: decode-mode sequence count and their key tiles
  long extra = 0, total_tiles = 0;
  if (S > 1) {
    long n_dec = 0, tiles = 0;
    for (int c0 = 0; c0 < p.batch; c0 += kThreads) {
      const int bb = c0 + tid;
      int dec = 0, t = 0;
      if (bb < p.batch) {
        const SeqInfo si = seq_info(p, bb);
        const int rows = si.q_len * p.group;
        if (rows > 0 && (p.all_decode || rows <= kDecodeRows)) {
          dec = 1;
          t = decode_tiles(si.K_b);
        }
      }
      int tot_d, tot_t;
      block_inclusive_scan(dec, s_wsum, tot_d);
      block_inclusive_scan(t, s_wsum, tot_t);
      n_dec += tot_d;
      tiles += tot_t;
    }
    extra = n_dec * (S - 1);
    total_tiles = tiles;
  }
  // pass 2: prefix of units, find ours
  if (tid == 0) s_found[0] = -1;
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < p.batch; c0 += kThreads) {
    const int bb = c0 + tid;
    int units = 0, splits = 1;
    if (bb < p.batch) {
      const SeqInfo si = seq_info(p, bb);
      const int rows = si.q_len * p.group;
      if (rows > 0) {
        if (p.all_decode || rows <= kDecodeRows) {
          splits = seq_splits(extra, decode_tiles(si.K_b), total_tiles);
          units = splits;
        } else {
          units = (rows + kPrefillRows - 1) / kPrefillRows;
        }
      }
    }
    int total;
    const int incl = carry + block_inclusive_scan(units, s_wsum, total);
    const int excl = incl - units;
    if (units > 0 && unit >= excl && unit < incl) {
      s_found[0] = bb;
      s_found[1] = unit - excl;
      s_found[2] = splits;
    }
    carry += total;
    __syncthreads();
    if (s_found[0] >= 0) break;
  }
  u.b = s_found[0];
  u.off = s_found[1];
  u.splits = s_found[2];
  return u.b >= 0;
}

// keys visible to packed row r of a sequence (bottom-right causal alignment)
__device__ inline int row_key_bound(int r, int group, int q_len, int K_b, int causal) {
  if (!causal) return K_b;
  const int lim = K_b - q_len + r / group + 1;
  return max(0, min(lim, K_b));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Raw buffer loads over one page (or one contiguous sequence) of the pool:
// 32-bit per-lane byte offsets against a wave-uniform base, and any offset at
// or past the range returns zeros without touching memory.  Masked lanes use
// kOOB, so no load sits behind a branch and the compiler can count
// outstanding loads exactly (keeping several tiles in flight).
constexpr uint32_t kOOB = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// Streaming variant (nt: the rows are read once and should not displace
// cached data): lane offset plus a wave-uniform offset.
__device__ inline u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t lane_off,
                                          uint32_t uniform_off) {
  return __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)lane_off, (int)uniform_off, 2));
}

// Geometry of one "slab" the buffer loads address: a physical page in paged
// mode, a sequence's whole allocation in contiguous mode.  A key's row within
// the slab is key % page_size (paged) or key (contiguous).
struct Slab {
  uint32_t bytes;        // bytes per slab (host checks < 2^31)
  long elems;            // halves per slab
};

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i % 4 of the 8-byte rows addressed by lanes i / 4 + 4 j,
// j = 0..3.  Lane s addressing row k0 + s / 4, columns c0 + 4 (s % 4) .. +3 of
// a row-major [key][dim] tile therefore hands lane i the four keys k0 .. k0+3
// of dim c0 + i: the key-contiguous operand layout the PV product needs.
__device__ inline u32x2 lds_read_tr16(const uint16_t *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

// The eight LDS slots of a workgroup, one 32-row [key][D] tile each.  They
// are separate LDS objects so that the compiler can tell a slot being filled
// by LDS-destination loads from one being read, and keep those loads in
// flight across the reads.
constexpr int kSlots = 8;
struct LdsPool {
  uint16_t *s0, *s1, *s2, *s3, *s4, *s5, *s6, *s7;
  // slot i for a constant i
  __device__ uint16_t *s(int i) const {
    return i < 4 ? (i < 2 ? (i == 0 ? s0 : s1) : (i == 2 ? s2 : s3))
                 : (i < 6 ? (i == 4 ? s4 : s5) : (i == 6 ? s6 : s7));
  }
  // slot i for a run-time i.  The empty asm makes the candidates opaque, so
  // the selection stays a few scalar selects instead of becoming a table of
  // LDS addresses (which a static initializer cannot hold).
  __device__ uint16_t *pick(int i) const {
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    lds_u16 *a0 = (lds_u16 *)s0, *a1 = (lds_u16 *)s1, *a2 = (lds_u16 *)s2, *a3 = (lds_u16 *)s3;
    lds_u16 *a4 = (lds_u16 *)s4, *a5 = (lds_u16 *)s5, *a6 = (lds_u16 *)s6, *a7 = (lds_u16 *)s7;
    asm volatile("" : "+s"(a0), "+s"(a1), "+s"(a2), "+s"(a3), "+s"(a4), "+s"(a5), "+s"(a6),
                      "+s"(a7));
    lds_u16 *r = i < 4 ? (i < 2 ? (i == 0 ? a0 : a1) : (i == 2 ? a2 : a3))
                       : (i < 6 ? (i == 4 ? a4 : a5) : (i == 6 ? a6 : a7));
    return (uint16_t *)r;   // still known to be LDS to the address-space inference
  }
};
typedef __attribute__((address_space(3))) void lds_void;

// Where a decode unit stages wave w's K and V tiles (and, at the end, its
// fp32 output rows in the K tile).  One contiguous array when the kernel runs
// decode units only: the V tile is the K tile plus a constant, which keeps
// the operand addresses in few registers.  The eight-slot pool when decode
// and prefill units share a kernel.
template <int TILEH>
struct ContigDecodeLds {
  uint16_t *base;
  __device__ uint16_t *k(int w) const { return base + w * 2 * TILEH; }
  __device__ uint16_t *v(int w) const { return k(w) + TILEH; }
  __device__ uint16_t *k_const(int w) const { return k(w); }
};
struct PoolDecodeLds {
  LdsPool pool;
  __device__ uint16_t *k(int w) const { return pool.pick(2 * w); }
  __device__ uint16_t *v(int w) const { return pool.pick(2 * w + 1); }
  __device__ uint16_t *k_const(int w) const { return pool.s(2 * w); }
};

// s_waitcnt immediate (gfx9 fields): vmcnt (bits 3:0 and 15:14), expcnt 7 (no
// wait, bits 6:4), lgkmcnt (bits 11:8).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// All but the newest `VM` of this wave's loads (LDS-destination loads
// included; loads complete in issue order) and all its LDS operations
// complete, then a workgroup barrier: afterwards every wave sees whatever any
// wave loaded into LDS before those VM, and no wave still reads a slot that is
// about to be refilled.  The signal fences keep the compiler from moving
// memory accesses across the barrier.
template <int VM>
__device__ inline void wait_then_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// Decode unit: <= 16 packed rows (the G q heads of one kv head for one or a
// few tokens), one split of the sequence's keys.  The four waves share the
// rows and each walks a contiguous quarter of the split's 32-key tiles:
//
//   page window  each lane holds the physical id of one of the next 64
//                logical pages (one table load per 64 pages); the one or two
//                pages a tile touches are read out of the window with scalar
//                lane reads, so no table access sits between tiles; ids are
//                resolved by absolute logical index, and entries past the
//                last visible page are never read;
//   row loads    every load instruction fetches whole K (V) rows: D*2 bytes
//                per key, 64*16/(D*2) keys per instruction, which streams
//                HBM faster than MFMA-shaped partial-row loads; two tiles are
//                in flight per wave (tile t + 2 is issued as soon as tile t's
//                registers are staged);
//   LDS staging  K and V land in the wave's own LDS region, rows with their
//                16-byte chunks XOR-swizzled by key, so both the MFMA-layout
//                K reads and the transposing V reads are bank-conflict free;
//                no workgroup barrier in the loop;
//   S^T = K Q^T  16x16x32 MFMA, keys on M: each lane's probabilities are
//                already the B operand of the PV product;
//   O^T += V^T P^T 16x16x32 MFMA on key-contiguous V^T from transposing reads.
// The waves' (max, sum, O) states merge through LDS at the end.
// ---------------------------------------------------------------------------
template <int DT, int D, class Lds>
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
  const int tid = threadIdx.x;
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
  const int w_begin = t_begin + wave * (n_w >> 2) + min(wave, n_w & 3);
  const int w_end = w_begin + (n_w >> 2) + (wave < (n_w & 3) ? 1 : 0);
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
    const uint16_t *qrow = p.q + ((long)(si.cu_b + tok) * p.hq + h) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = row_ok ? load16(qrow + (ds * 4 + lg) * 8) : u32x4{0u, 0u, 0u, 0u};
  }

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
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][orow]);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
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
}

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

template <int DT, int D, bool kUnified>
__device__ __forceinline__ void attn_fwd_body(const FwdParams &p) {
  // decode-only kernel: one contiguous array, a K and a V tile per wave;
  // unified kernel: eight separate 32-row slots (four K and four V slots of a
  // prefill unit; a K/V pair per wave of a decode unit)
  // (K slots of a prefill unit at D = 128 carry 64 halves of padding per two
  // 1 KiB blocks)
  constexpr int kSlotH = kKeyTile * D + (D == 128 ? 4 * 64 : 0);
  static_assert(kPTile == kKeyTile, "prefill and decode tiles share the slots");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s0[kUnified ? kSlotH : kSlots * kKeyTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s1[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s2[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s3[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s4[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s5[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s6[kUnified ? kSlotH : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s7[kUnified ? kSlotH : 8];
  const LdsPool pool{lds_s0, lds_s1, lds_s2, lds_s3, lds_s4, lds_s5, lds_s6, lds_s7};
  __shared__ float sm_m[kWaves][kDecodeRows];
  __shared__ float sm_l[kWaves][kDecodeRows];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_found[3];

  const int g = blockIdx.x % p.hkv;
  const int unit = blockIdx.x / p.hkv;
  UnitInfo u;
  if (p.all_decode && p.num_splits == 1) {
    u.b = unit;
    u.off = 0;
    u.splits = 1;
    if (u.b >= p.batch) return;
  } else if (!locate_unit(p, unit, u, s_wsum, s_found)) {
    return;
  }
  // the unit and its sequence are the same for every lane: keep them in SGPRs
  // (page indices, buffer descriptors and uniform offsets derive from them)
  u.b = __builtin_amdgcn_readfirstlane(u.b);
  u.off = __builtin_amdgcn_readfirstlane(u.off);
  u.splits = __builtin_amdgcn_readfirstlane(u.splits);
  SeqInfo si = seq_info(p, u.b);
  si.cu_b = __builtin_amdgcn_readfirstlane(si.cu_b);
  si.q_len = __builtin_amdgcn_readfirstlane(si.q_len);
  si.K_b = __builtin_amdgcn_readfirstlane(si.K_b);
  const int rows_b = si.q_len * p.group;
  if (rows_b <= 0) return;
  if (!kUnified || p.all_decode || rows_b <= kDecodeRows) {
    if (g == 0 && u.off == 0 && p.split_count != nullptr && threadIdx.x == 0)
      p.split_count[u.b] = u.splits;
    if constexpr (kUnified)
      decode_unit<DT, D>(p, u.b, g, u.off, u.splits, si, PoolDecodeLds{pool}, sm_m, sm_l);
    else
      decode_unit<DT, D>(p, u.b, g, u.off, u.splits, si, ContigDecodeLds<kKeyTile * D>{lds_s0}, sm_m,
                         sm_l);
  } else if constexpr (kUnified) {
    const int n_qt = (rows_b + kPrefillRows - 1) / kPrefillRows;
    if (p.geom.table != nullptr)
      prefill_unit<DT, D, true>(p, u.b, g, n_qt - 1 - u.off, si, pool);
    else
      prefill_unit<DT, D, false>(p, u.b, g, n_qt - 1 - u.off, si, pool);
  }
}

// Decode-only batches (every sequence fits a decode unit, known on the host):
// two waves per SIMD.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_decode_kernel(FwdParams p) {
  attn_fwd_body<DT, D, false>(p);
}

// Unified kernel for any mix of prefill and decode sequences: two waves per
// SIMD as well.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  attn_fwd_body<DT, D, true>(p);
}

// ---------------------------------------------------------------------------
// Split-KV combine: per (token, q head) row of a decode-mode sequence with
// more than one split, lse = log(sum_s exp(lse_s)) and
// out = sum_s exp(lse_s - lse) * o_s over the splits that saw a key; a row
// whose splits were all empty gets out = 0, lse = -inf.  Rows of prefill
// units and of single-split sequences were written directly and are skipped.
// One wave per row.
// ---------------------------------------------------------------------------
struct CombineParams {
  const float *o_part;
  const float *lse_part;
  const int32_t *split_count;
  const int32_t *cu_seqlens_q;
  uint16_t *out;
  float *lse;
  int batch, total_q, hq, group, all_decode;
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long)p.total_q * p.hq) return;
  const int token = (int)(row / p.hq);
  int lo = 0, hi = p.batch;   // largest b with cu[b] <= token
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.cu_seqlens_q[mid] <= token) lo = mid; else hi = mid;
  }
  const int end = min(p.cu_seqlens_q[lo + 1], p.total_q);
  if (token >= end) return;
  const int q_len = end - p.cu_seqlens_q[lo];
  if (!p.all_decode && q_len * p.group > kDecodeRows) return;   // prefill row: already final
  const int S = p.split_count[lo];
  if (S <= 1) return;                                            // written directly
  const long stride = (long)p.total_q * p.hq;
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
