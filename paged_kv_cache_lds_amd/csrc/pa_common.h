// Shared pieces of the gfx950 paged KV-cache attention kernels: work
// decomposition constants, kernel parameters, the KV append kernel,
// sequence and unit bookkeeping, buffer-load and LDS helpers.
#pragma once

#include "pa_device.h"

namespace pa {


// Work decomposition constants.
constexpr int kThreads = 256;     // decode-only kernel (and append, combine): four wave64
constexpr int kWaves = 4;
constexpr int kUThreads = 512;    // unified kernel: eight wave64, two per SIMD
constexpr int kUWaves = 8;
constexpr int kKeyTile = 32;      // decode: keys per wave main-loop iteration
constexpr int kDecodeRows = 16;   // packed (token, q-head) rows of a decode unit
constexpr int kPrefillRows = 32 * kUWaves;   // rows of a prefill unit (32 per wave)
constexpr int kPTile = 32;        // prefill: keys per workgroup main-loop iteration
constexpr int kMaxSplits = 128;

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
  int32_t *row_splits; // [total_q, hq] (num_splits > 1): splits that wrote partials for
                       // the row, 1 for a row written directly (single split, prefill)
  int batch, total_q, hq, hkv, group;
  int appended, causal, num_splits;
  float scale_log2;    // softmax scale * log2(e)
  int all_decode;      // host knows every sequence has q_len * group <= 16
  Rotary rot;          // rotary embedding of q (rot.cos == nullptr: none)
  long q_stride;       // elements between consecutive tokens' q rows
  int unit_mode;       // 0: every unit; 1: prefill units only; 2: decode units only
                       // (a mixed batch split over two concurrent launches)
  int uniform_q_tiles; // > 0: every sequence has the same query length, of this many
                       // prefill units (query tiles); units map by block index
  int full_search;     // 1: units always from the workgroup-wide search (no shortcut
                       // for one sequence or for a few)
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
  int seq_mode, group; // 0: every sequence; 1: prefill-mode only; 2: decode-mode only
                       // (q_len * group <= kDecodeRows)
  Rotary rot;          // rotary embedding of the new keys (rot.cos == nullptr: none)
  long kn_stride, vn_stride;   // elements between consecutive tokens' k_new / v_new rows
};

// ---------------------------------------------------------------------------
// Append (vLLM's reshape_and_cache; the in-call k=/v= of flash-attention's
// paged cache): new row i of sequence b goes to logical position
// cache_seqlens[b] + i, its key rotated for that position when a rotary table
// is given.  Grid (cdiv(max_seqlen_q, tokens_per_block), batch); each thread
// moves 16-byte vectors.  Targets whose page id is outside the pool (a caller
// precondition violation) are skipped, never written.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.y;
  const int cu_b = p.cu_seqlens_q[b];
  // rows past total_q (malformed cu_seqlens_q) are never touched
  const int q_len = max(0, min(p.cu_seqlens_q[b + 1], p.total_q) - cu_b);
  const int tok0 = blockIdx.x * p.tokens_per_block;
  if (tok0 >= q_len) return;
  if (p.seq_mode != 0 && (p.seq_mode == 2) != (q_len * p.group <= kDecodeRows)) return;
  const int ntok = min(p.tokens_per_block, q_len - tok0);
  const int vec_per_row = p.hkv * p.head_dim / 8;   // 16-byte vectors per token row
  const int L = p.cache_seqlens[b];
  const int work = ntok * vec_per_row * 2;
  if (p.rot.cos == nullptr) {
    // Plain copy: a thread first loads all its vectors of a batch (their
    // sources do not depend on the pages), then finds each target and stores
    // - loads and stores to possibly aliasing buffers would otherwise
    // alternate, one load in flight per thread.
    constexpr int kPer = 4;
    for (int base = 0; base < work; base += kPer * kThreads) {
      u32x4 buf[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int idx = base + j * kThreads + threadIdx.x;
        if (idx < work) {
          const int which = idx / (ntok * vec_per_row);
          const int rem = idx - which * ntok * vec_per_row;
          const int t = rem / vec_per_row;
          const int v = rem - t * vec_per_row;
          const long src = (long)(cu_b + tok0 + t) * (which ? p.vn_stride : p.kn_stride) + v * 8;
          buf[j] = load16((which ? p.v_new : p.k_new) + src);
        }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int idx = base + j * kThreads + threadIdx.x;
        if (idx < work) {
          const int which = idx / (ntok * vec_per_row);
          const int rem = idx - which * ntok * vec_per_row;
          const int t = rem / vec_per_row;
          const int v = rem - t * vec_per_row;
          const long prow = physical_row(p.geom, b, L + tok0 + t);
          if (prow >= 0) store16((which ? p.v_cache : p.k_cache) + (prow * vec_per_row + v) * 8, buf[j]);
        }
      }
    }
    return;
  }
  for (int idx = threadIdx.x; idx < work; idx += kThreads) {
    const int which = idx / (ntok * vec_per_row);     // 0: K, 1: V
    const int rem = idx - which * ntok * vec_per_row;
    const int t = rem / vec_per_row;
    const int v = rem - t * vec_per_row;
    const int i = tok0 + t;
    const long prow = physical_row(p.geom, b, L + i);
    if (prow < 0) continue;
    const long dst = (prow * vec_per_row + v) * 8;
    if (which == 0) {
      const long src = (long)(cu_b + i) * p.kn_stride + v * 8;
      u32x4 k[1] = {load16(p.k_new + src)};
      if (p.rot.cos != nullptr) {
        const int e0 = (v % (p.head_dim >> 3)) * 8;   // offset inside the head row
        RotFetch<1> f;
        rot_fetch(p.rot, p.k_new + src - e0, e0, 0, L + i, f);
        rot_apply<DT>(p.rot, e0, 0, L + i, k, f);
      }
      store16(p.k_cache + dst, k[0]);
    } else {
      store16(p.v_cache + dst, load16(p.v_new + (long)(cu_b + i) * p.vn_stride + v * 8));
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
// the host).  No split gets fewer than kMinSplitTiles key tiles (two per
// wave): a cache allocated far beyond its live length, or a forced budget
// larger than the keys can use, leaves the rest of the budget unused instead
// of paying partial results for near-empty splits.  A pure function of the
// lengths: every workgroup agrees on it.
constexpr long kMinSplitTiles = 8;
__device__ inline int seq_splits(long extra_budget, long tiles_b, long total_tiles) {
  if (extra_budget <= 0 || total_tiles <= 0) return 1;
  long s = 1 + (extra_budget * tiles_b) / total_tiles;
  s = min(s, max(1L, tiles_b / kMinSplitTiles));
  return (int)min(s, (long)kMaxSplits);
}

__device__ inline int decode_tiles(int K_b) { return (K_b + kKeyTile - 1) / kKeyTile; }

// Split budget of a batch of at most kFewSeqs sequences, one lane of wave 0
// per sequence (dec: a decode-mode sequence, t: its key tiles).  The floors of
// seq_splits() drop up to one unit per decode sequence; with few sequences
// that is a large share of the budget, and the longest split, which bounds a
// launch whose units all run at once, stays long.  The dropped units go out
// in rounds, each to every sequence tied for the longest split (most key
// tiles per split) that can still take one; the hand-out stops when a round
// cannot serve its whole tie, since serving part of it would not shorten the
// longest split.  A function of the lengths alone (not of the order of the
// sequences), so every workgroup agrees; the total never exceeds the budget.
constexpr int kFewSeqs = 64;
__device__ inline int few_splits(int dec, int t, long n_dec, long extra, long total_tiles) {
  int s = 1, cap = 1, f = 0;
  if (dec && extra > 0 && total_tiles > 0) {
    f = (int)(1 + extra * t / total_tiles);
    cap = min(max(1, t / (int)kMinSplitTiles), kMaxSplits);
    s = min(f, cap);
  }
  int sum_f = f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum_f += __shfl_xor(sum_f, o, 64);
  long left = (extra > 0 && total_tiles > 0) ? n_dec + extra - sum_f : 0;
  while (left > 0) {
    const int key = (dec && s < cap) ? (t + s - 1) / s : 0;
    int km = key;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) km = max(km, __shfl_xor(km, o, 64));
    if (km == 0) break;
    const long c = __popcll(__ballot(key == km));
    if (c > left) break;
    if (key == km) ++s;
    left -= c;
  }
  return s;
}
__device__ inline void share_splits_few(int dec, int t, long n_dec, long extra,
                                        long total_tiles, int *s_split) {
  const int s = few_splits(dec, t, n_dec, extra, total_tiles);
  if (threadIdx.x < kFewSeqs) s_split[threadIdx.x] = s;
}

// inclusive prefix sum over the workgroup (every thread contributes x);
// `total` receives the workgroup sum
template <int NW>
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
  for (int w = 0; w < NW; ++w) {
    const int v = s_wsum[w];
    before += (w < wave) ? v : 0;
    total += v;
  }
  __syncthreads();
  return before + x;
}

// Decode units in longest-first order.  Workgroups are dispatched in grid
// order and a free slot takes the next one, so the order of the units is the
// schedule: with sequences of mixed lengths, the long ones' units should go
// first, or they start late and finish last (the tail of a varlen batch).
// Decode units are therefore enumerated by decreasing key tiles per unit
// (ties by sequence index), the splits of one sequence consecutive.  Ranks
// come from comparing every decode sequence with every other in LDS; batches
// beyond kOrderMax sequences keep index order.  Already ordered batches
// (equal lengths included) skip the comparisons.  The caller decides where
// this applies (a null order keeps index order).
constexpr int kOrderMax = 1024;
struct DecodeOrder {
  int key[kOrderMax];   // by sequence: key tiles per decode unit, -1 without decode units
  int seq[kOrderMax];   // by rank: the sequence
  int cnt[kOrderMax];   // by rank: its decode units (splits); 0 past the last rank
};

// ints per unit sought in the search's shared slots: sequence, split or
// query tile, splits, and the sequence's cu_b, q_len, K_b
constexpr int kFound = 6;

// The decode unit(s) `first` .. `first + kDecPerWg - 1` (per kv head, in the
// order above) into s_found, as in locate_unit's second pass.  Every thread of
// the workgroup takes part; barriers are uniform.
template <int NT, int kDecPerWg>
__device__ inline void find_decode_ordered(const FwdParams &p, long first, long extra,
                                           long total_tiles, DecodeOrder &o, int *s_wsum,
                                           int *s_found) {
  constexpr int PER = kOrderMax / NT;
  const int tid = threadIdx.x;
  int my_key[PER], my_cnt[PER];
  SeqInfo my_si[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = tid + i * NT;
    int key = -1, cnt = 0;
    my_si[i] = SeqInfo{0, 0, 0};
    if (s < p.batch) {
      const SeqInfo si = seq_info(p, s);
      my_si[i] = si;
      const int rows = si.q_len * p.group;
      if (rows > 0 && (p.all_decode || rows <= kDecodeRows)) {
        const long tiles = decode_tiles(si.K_b);
        cnt = seq_splits(extra, tiles, total_tiles);
        key = (int)((tiles + cnt - 1) / cnt);
      }
      o.key[s] = key;
      o.cnt[s] = 0;
    }
    my_key[i] = key;
    my_cnt[i] = cnt;
  }
  if (tid < kFound * kDecPerWg) s_found[tid] = -1;
  __syncthreads();
  bool unordered = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = tid + i * NT;
    if (s + 1 < p.batch && my_key[i] < o.key[s + 1]) unordered = true;
  }
  unordered = __syncthreads_or(unordered);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = tid + i * NT;
    if (my_key[i] < 0) continue;
    int r = s;   // ordered: decode sequences first, in index order
    if (unordered) {
      r = 0;
      for (int s2 = 0; s2 < p.batch; ++s2) {
        const int k2 = o.key[s2];
        r += (k2 > my_key[i]) | ((k2 == my_key[i]) & (s2 < s));
      }
    }
    o.seq[r] = s;
    o.cnt[r] = my_cnt[i];
  }
  __syncthreads();
  long carry = 0;
  for (int c0 = 0; c0 < p.batch; c0 += NT) {
    const int r = c0 + tid;
    const int units = r < p.batch ? o.cnt[r] : 0;
    int total;
    const long incl = carry + block_inclusive_scan<NT / 64>(units, s_wsum, total);
    const long excl = incl - units;
    for (int h = 0; h < kDecPerWg; ++h) {
      const long want = first + h;
      if (units > 0 && want >= excl && want < incl) {
        s_found[kFound * h] = o.seq[r];
        s_found[kFound * h + 1] = (int)(want - excl);
        s_found[kFound * h + 2] = units;
      }
    }
    carry += total;
    __syncthreads();
    if (s_found[kFound * (kDecPerWg - 1)] >= 0) break;   // the last one sought is found
  }
  // the thread that read a found sequence's metadata passes it on, sparing the
  // workgroup a dependent reload before the unit can start
#pragma unroll
  for (int h = 0; h < kDecPerWg; ++h) {
    const int sq = s_found[kFound * h];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (sq >= 0 && sq == tid + i * NT) {
        s_found[kFound * h + 3] = my_si[i].cu_b;
        s_found[kFound * h + 4] = my_si[i].q_len;
        s_found[kFound * h + 5] = my_si[i].K_b;
      }
    }
  }
  __syncthreads();
}

// Decode unit `first` of a decode-only launch over at most kFewSeqs
// sequences, found by wave 0 alone: one lane per sequence, wave shuffles in
// place of the workgroup scans and barriers of locate_unit and
// find_decode_ordered, with the same units in the same order (longest first
// with one unit per sequence, index order with a split budget) and the same
// split counts.  The result goes to s_found (kFound ints; sequence -1: no
// unit) for the caller to publish with one barrier.
__device__ inline int wave_excl_scan(int x) {
  const int lane = threadIdx.x & 63;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  return incl - x;
}
__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline void find_decode_few(const FwdParams &p, long first, bool longest_first,
                                       int *s_found) {
  const int lane = threadIdx.x;   // wave 0
  const int S = p.num_splits;
  SeqInfo si{0, 0, 0};
  int dec = 0, t = 0;
  if (lane < p.batch) {
    si = seq_info(p, lane);
    const int rows = si.q_len * p.group;
    if (rows > 0 && (p.all_decode || rows <= kDecodeRows)) {
      dec = 1;
      t = decode_tiles(si.K_b);
    }
  }
  int cnt = dec;
  if (S > 1) {
    const long n_dec = wave_sum(dec);
    const long tiles = wave_sum(t);
    const int s = few_splits(dec, t, n_dec, n_dec * (S - 1), tiles);
    cnt = dec ? s : 0;
  }
  int excl;   // units before this sequence's first
  if (S == 1 && longest_first) {
    // one unit per decode sequence, by rank: most key tiles first, ties by
    // index (every decode sequence ranks before every other one)
    const int key = dec ? t : -1;
    const int next = __shfl_down(key, 1, 64);
    if (!__any(lane + 1 < p.batch && key < next)) {
      excl = lane;
    } else {
      excl = 0;
      for (int s2 = 0; s2 < p.batch; ++s2) {
        const int k2 = __shfl(key, s2, 64);
        excl += (k2 > key) | ((k2 == key) & (s2 < lane));
      }
    }
  } else {
    excl = wave_excl_scan(cnt);
  }
  const bool found = cnt > 0 && first >= excl && first < excl + cnt;
  if (found) {
    s_found[0] = lane;
    s_found[1] = (int)(first - excl);
    s_found[2] = cnt;
    s_found[3] = si.cu_b;
    s_found[4] = si.q_len;
    s_found[5] = si.K_b;
  }
  if (__ballot(found) == 0 && lane == 0) s_found[0] = -1;
}

// Work mapping.  Units per kv head, prefill units first: a sequence whose
// packed rows (q_len * group) exceed one 16-row decode unit gets
// cdiv(rows, kPrefillRows) prefill units, heaviest (last, under the causal
// mask) first; then every other sequence gets seq_splits() decode units (its
// keys split across units).  A workgroup of the decode-only kernel takes one
// decode unit; one of the unified kernel takes one prefill unit or two
// consecutive decode units, one per four-wave half, so that a decode unit
// runs the same four-wave code in either kernel.  The host sizes the grid
// from static maxima; every workgroup finds its units by block-wide scans
// over the device metadata, and a workgroup or half without a unit returns.
struct UnitInfo {
  int b, off, splits;   // off = split (decode) or query tile (prefill)
  SeqInfo si;           // the sequence's metadata when the search read it (si.q_len < 0: not read)
};

template <int NT, int kDecPerWg>
__device__ inline bool locate_unit(const FwdParams &p, int wg, UnitInfo &u, bool &decode,
                                   int *s_wsum, int *s_found, int *s_split,
                                   DecodeOrder *order) {
  const int tid = threadIdx.x;
  const int half = kDecPerWg == 2 ? tid / (NT / 2) : 0;
  const int S = p.num_splits;
  auto is_decode = [&](int rows) { return p.all_decode || rows <= kDecodeRows; };
  // pass 1: prefill units, and (split budget) decode-mode sequences and their
  // key tiles.  A prefill-only launch needs neither; a decode-only launch over
  // a mixed batch needs the key tiles only.
  long extra = 0, total_tiles = 0, n_pre = 0;
  const bool count_pre = !p.all_decode && p.unit_mode == 0;
  const bool few = S > 1 && p.unit_mode != 1 && p.batch <= kFewSeqs;
  // a batch of at most NT sequences: pass 2 reuses what pass 1 read
  const bool pass1 = p.unit_mode != 1 && (S > 1 || count_pre);
  const bool reuse = pass1 && p.batch <= NT;
  SeqInfo my_si{0, 0, 0};
  if (pass1) {
    long n_dec = 0, tiles = 0;
    int my_dec = 0, my_t = 0;   // this thread's sequence in the first chunk
    for (int c0 = 0; c0 < p.batch; c0 += NT) {
      const int bb = c0 + tid;
      int dec = 0, t = 0, pre = 0;
      if (bb < p.batch) {
        const SeqInfo si = seq_info(p, bb);
        if (c0 == 0) my_si = si;
        const int rows = si.q_len * p.group;
        if (rows > 0) {
          if (is_decode(rows)) {
            dec = 1;
            t = decode_tiles(si.K_b);
          } else {
            pre = (rows + kPrefillRows - 1) / kPrefillRows;
          }
        }
      }
      int tot_d = 0, tot_t = 0, tot_p = 0;
      if (S > 1) {
        block_inclusive_scan<NT / 64>(dec, s_wsum, tot_d);
        block_inclusive_scan<NT / 64>(t, s_wsum, tot_t);
      }
      if (count_pre) block_inclusive_scan<NT / 64>(pre, s_wsum, tot_p);
      n_dec += tot_d;
      tiles += tot_t;
      n_pre += tot_p;
      if (c0 == 0) {
        my_dec = dec;
        my_t = t;
      }
    }
    extra = n_dec * (S - 1);
    total_tiles = tiles;
    if (few && tid < 64) share_splits_few(my_dec, my_t, n_dec, extra, total_tiles, s_split);
  }
  // pass 2: prefix over the units of our kind, find ours (one per half).  A
  // launch limited to one kind numbers its workgroups within that kind.
  const bool pre_wg = p.unit_mode == 0 ? wg < n_pre : p.unit_mode == 1;
  const long first = pre_wg ? wg : (p.unit_mode == 2 ? wg : wg - n_pre) * kDecPerWg;
  if (!pre_wg && p.batch <= kOrderMax && order != nullptr) {
    find_decode_ordered<NT, kDecPerWg>(p, first, extra, total_tiles, *order, s_wsum, s_found);
    const int slot = kFound * half;
    u.b = s_found[slot];
    u.off = s_found[slot + 1];
    u.splits = s_found[slot + 2];
    u.si.cu_b = s_found[slot + 3];
    u.si.q_len = u.b >= 0 ? s_found[slot + 4] : -1;
    u.si.K_b = s_found[slot + 5];
    decode = true;
    return u.b >= 0;
  }
  if (tid < 2 * kFound) s_found[tid] = -1;
  __syncthreads();
  long carry = 0;
  for (int c0 = 0; c0 < p.batch; c0 += NT) {
    const int bb = c0 + tid;
    int units = 0, splits = 1;
    SeqInfo si{0, 0, 0};
    if (bb < p.batch) {
      si = reuse ? my_si : seq_info(p, bb);
      const int rows = si.q_len * p.group;
      if (rows > 0) {
        if (is_decode(rows)) {
          splits = few ? s_split[bb] : seq_splits(extra, decode_tiles(si.K_b), total_tiles);
          if (!pre_wg) units = splits;
        } else if (pre_wg) {
          units = (rows + kPrefillRows - 1) / kPrefillRows;
        }
      }
    }
    int total;
    const long incl = carry + block_inclusive_scan<NT / 64>(units, s_wsum, total);
    const long excl = incl - units;
    const int n_sought = pre_wg ? 1 : kDecPerWg;
    for (int h = 0; h < n_sought; ++h) {
      const long want = first + h;
      if (units > 0 && want >= excl && want < incl) {
        // the finder passes on what it read of the sequence, sparing the
        // workgroup a dependent reload before the unit can start
        s_found[kFound * h] = bb;
        s_found[kFound * h + 1] = (int)(want - excl);
        s_found[kFound * h + 2] = splits;
        s_found[kFound * h + 3] = si.cu_b;
        s_found[kFound * h + 4] = si.q_len;
        s_found[kFound * h + 5] = si.K_b;
      }
    }
    carry += total;
    __syncthreads();
    if (s_found[kFound * (n_sought - 1)] >= 0) break;   // the last one sought is found
  }
  const int slot = pre_wg ? 0 : kFound * half;
  u.b = s_found[slot];
  u.off = s_found[slot + 1];
  u.splits = s_found[slot + 2];
  u.si.cu_b = s_found[slot + 3];
  u.si.q_len = u.b >= 0 ? s_found[slot + 4] : -1;
  u.si.K_b = s_found[slot + 5];
  decode = !pre_wg;
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

// The LDS slots of a workgroup, one 32-row [key][D] tile each (sixteen in the
// unified kernel).  They are separate LDS objects so that the compiler can
// tell a slot being filled by LDS-destination loads from one being read, and
// keep those loads in flight across the reads.
constexpr int kSlots = 16;
struct LdsPool {
  uint16_t *sl[kSlots];
  // slot i for a constant i
  __device__ uint16_t *s(int i) const { return sl[i]; }
  // slot i for a run-time i.  The empty asm makes the candidates opaque, so
  // the selection stays a few scalar selects instead of becoming a table of
  // LDS addresses (which a static initializer cannot hold); the pointers stay
  // in the LDS address space, so accesses through the result are LDS accesses.
  __device__ uint16_t *pick(int i) const {
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    lds_u16 *a[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      a[k] = (lds_u16 *)sl[k];
      asm volatile("" : "+s"(a[k]));
    }
    lds_u16 *r = a[0];
#pragma unroll
    for (int k = 1; k < kSlots; ++k) r = i == k ? a[k] : r;
    return (uint16_t *)r;
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
template <int H>   // a four-wave half of the unified kernel: slots 8 H .. 8 H + 7
struct PoolDecodeLds {
  LdsPool pool;
  __device__ uint16_t *k(int w) const { return pool.pick(2 * w + 8 * H); }
  __device__ uint16_t *v(int w) const { return pool.pick(2 * w + 1 + 8 * H); }
  __device__ uint16_t *k_const(int w) const { return pool.s(2 * w + 8 * H); }
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

}  // namespace pa
