// Host dispatch and C ABI of libpaged_attn.so (declarations and contracts in
// include/paged_attn.h).  Validates arguments, plans the launch from
// host-static sizes only, carves the caller's workspace and queues
// append -> attention on the caller's stream (a mixed batch given a second
// stream forks its decode units onto it and joins back before the split-KV
// combine).  Never allocates device memory, frees or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <vector>

#include "paged_attn.h"
#include "pa_kernels.h"

// Device scratch of paged_attn_fwd_noalloc: the split-KV partials of calls
// whose caller cannot allocate.  One array per device, held from the
// library's load on that device until the process ends.  In host code its name
// is only a stand-in: its device address comes from hipGetSymbolAddress.
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using pa::kThreads;

constexpr int kMaxSplits = pa::kMaxSplits;

struct Plan {
  int pair = 1;           // kv heads per decode unit of an all-decode batch (1 or 2)
  int splits = 1;         // split budget: average splits per decode sequence
  int max_splits = 1;     // most splits one sequence can receive
  bool all_decode = true;
  bool may_mix = false;   // the batch can hold both decode-mode and prefill-mode sequences
  long grid = 0;          // attention workgroups (one launch)
  long grid_dec = 0;      // decode-only kernel over a mixed batch's decode units
  long grid_pre = 0;      // unified kernel over its prefill units
  size_t ws_bytes = 0;
  size_t o_part_off = 0, lse_part_off = 0, rsplit_off = 0;
  int max_seqlen_k = 0;
  int uniform_q_tiles = 0;   // > 0: equal query lengths, prefill units by block index
};

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
inline int ilog2(int x) { int s = 0; while ((1 << s) < x) ++s; return s; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline long cdiv(long a, long b) { return (a + b - 1) / b; }

// PAGED_ATTN_FULL_SEARCH=1: every unit found by the workgroup-wide search of
// the metadata (no block-index mapping for equal query lengths or a single
// sequence, no one-wave search for a few sequences); the same results
bool full_search_forced() {
  const char *e = std::getenv("PAGED_ATTN_FULL_SEARCH");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

// PAGED_ATTN_HEAD_PAIRS=0: decode units over one kv head only; =2: over
// pairs of kv heads wherever a pair's rows fit one unit (the size rules of
// make_plan skipped); otherwise those rules decide
int pair_mode() {
  const char *e = std::getenv("PAGED_ATTN_HEAD_PAIRS");
  if (e != nullptr && std::strcmp(e, "0") == 0) return 0;
  if (e != nullptr && std::strcmp(e, "2") == 0) return 2;
  return 1;
}


// Argument checks shared by every entry point.  `append_only` relaxes the
// fields the append step does not read; `sizes_only` skips the data pointers
// (used by the host-only sizing queries).
pa_status validate(const pa_fwd_args *a, bool append_only, bool sizes_only = false) {
  if (a == nullptr) return PA_ERR_NULL;
  if (a->dtype != PA_F16 && a->dtype != PA_BF16) return PA_ERR_DTYPE;
  if (a->reserved0 != 0) return PA_ERR_SHAPE;
  if (a->batch < 1 || a->total_q < 0 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
    return PA_ERR_SHAPE;
  // the append grid holds one row of blocks per sequence (grid.y <= 65535)
  if (a->k_new != nullptr && a->batch > 65535) return PA_ERR_SHAPE;
  if (a->total_q > 0 && a->max_seqlen_q < 1) return PA_ERR_SHAPE;
  if (a->num_heads_kv < 1) return PA_ERR_SHAPE;
  if (a->head_dim != 64 && a->head_dim != 128) return PA_ERR_UNSUPPORTED;
  // kernels address one page (or one contiguous sequence) with 32-bit byte
  // offsets: it must span less than 2 GiB
  const long row_bytes = (long)a->num_heads_kv * a->head_dim * 2;
  if (a->block_table != nullptr) {
    if (!is_pow2(a->page_size) || a->page_size < 16 || a->page_size > 256)
      return PA_ERR_UNSUPPORTED;
    if (a->num_pages < 1 || a->max_pages_per_seq < 1) return PA_ERR_SHAPE;
    if (row_bytes * a->page_size >= (1L << 31)) return PA_ERR_UNSUPPORTED;
  } else {
    if (a->contig_alloc < 1) return PA_ERR_SHAPE;
    if (row_bytes * a->contig_alloc >= (1L << 31)) return PA_ERR_UNSUPPORTED;
  }
  if (!sizes_only && (a->k_cache == nullptr || a->v_cache == nullptr ||
                     a->cache_seqlens == nullptr || a->cu_seqlens_q == nullptr))
    return PA_ERR_NULL;
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return PA_ERR_NULL;
  // rotary embedding: both tables or neither; the pairs must fill whole
  // 16-byte chunks (rotary_dim a multiple of 16)
  if (a->reserved1 != 0) return PA_ERR_SHAPE;
  if ((a->rotary_cos == nullptr) != (a->rotary_sin == nullptr)) return PA_ERR_NULL;
  if (a->rotary_cos == nullptr) {
    if (a->rotary_dim != 0 || a->rotary_rows != 0 || a->rotary_interleaved != 0)
      return PA_ERR_SHAPE;
  } else {
    if (a->rotary_dim < 16 || a->rotary_dim > a->head_dim || a->rotary_dim % 16 != 0)
      return PA_ERR_SHAPE;
    if (a->rotary_rows < 1 || (a->rotary_interleaved != 0 && a->rotary_interleaved != 1))
      return PA_ERR_SHAPE;
  }
  // row strides of q / k_new / v_new: 0 (dense) or >= the row, 16-byte aligned
  const long qrow = (long)a->num_heads_q * a->head_dim, kvrow = (long)a->num_heads_kv * a->head_dim;
  if (a->q_row_stride < 0 || a->k_new_row_stride < 0 || a->v_new_row_stride < 0) return PA_ERR_SHAPE;
  if ((a->q_row_stride != 0 && (!append_only && a->q_row_stride < qrow)) ||
      (a->k_new_row_stride != 0 && a->k_new_row_stride < kvrow) ||
      (a->v_new_row_stride != 0 && a->v_new_row_stride < kvrow))
    return PA_ERR_SHAPE;
  if ((a->q_row_stride | a->k_new_row_stride | a->v_new_row_stride) % 8 != 0) return PA_ERR_ALIGN;
  if (!sizes_only) {
    // every buffer the kernels move in 16-byte vectors
    const void *vec[] = {a->k_cache, a->v_cache, a->k_new, a->v_new, a->rotary_cos,
                         a->rotary_sin, append_only ? nullptr : a->q,
                         append_only ? nullptr : a->out};
    for (const void *v : vec)
      if ((reinterpret_cast<uintptr_t>(v) & 15u) != 0) return PA_ERR_ALIGN;
  }
  if (!sizes_only && a->k_new != nullptr) {
    // new rows must not overlap the pools they are appended to
    const long rows = std::max(0, a->total_q);
    const size_t pool_bytes =
        (a->block_table != nullptr ? (size_t)a->num_pages * a->page_size
                                   : (size_t)a->batch * a->contig_alloc) * (size_t)kvrow * 2;
    auto span = [&](const void *p, long stride) {
      const size_t n = rows == 0 ? 0
                                 : ((size_t)(rows - 1) * (size_t)(stride ? stride : kvrow) +
                                    (size_t)kvrow) * 2;
      return std::pair<uintptr_t, uintptr_t>((uintptr_t)p, (uintptr_t)p + n);
    };
    auto overlap = [](std::pair<uintptr_t, uintptr_t> x, const void *pool, size_t bytes) {
      const uintptr_t lo = (uintptr_t)pool, hi = lo + bytes;
      return x.first < hi && lo < x.second;
    };
    const auto kn = span(a->k_new, a->k_new_row_stride), vn = span(a->v_new, a->v_new_row_stride);
    if (overlap(kn, a->k_cache, pool_bytes) || overlap(kn, a->v_cache, pool_bytes) ||
        overlap(vn, a->k_cache, pool_bytes) || overlap(vn, a->v_cache, pool_bytes))
      return PA_ERR_SHAPE;
  }
  if (append_only) {
    if (a->k_new == nullptr) return PA_ERR_NULL;
    return PA_OK;
  }
  if (a->num_heads_q < 1 || a->num_heads_q % a->num_heads_kv != 0) return PA_ERR_SHAPE;
  if (a->causal != 0 && a->causal != 1) return PA_ERR_SHAPE;
  if (a->num_splits < 0 || a->num_splits > kMaxSplits) return PA_ERR_SHAPE;
  if (!(a->softmax_scale == a->softmax_scale)) return PA_ERR_SHAPE;   // NaN
  if (!sizes_only && (a->q == nullptr || a->out == nullptr || a->softmax_lse == nullptr))
    return PA_ERR_NULL;
  return PA_OK;
}

// Compute units of the current device, queried once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int key_bound(const pa_fwd_args *a) {
  if (a->max_seqlen_k > 0) return a->max_seqlen_k;
  if (a->block_table != nullptr) {
    const long cap = (long)a->max_pages_per_seq * a->page_size;
    return cap > INT32_MAX ? INT32_MAX : (int)cap;
  }
  return a->contig_alloc;
}

Plan make_plan(const pa_fwd_args *a, int num_cus) {
  Plan pl;
  const int group = a->num_heads_q / a->num_heads_kv;
  pl.max_seqlen_k = key_bound(a);
  pl.all_decode = (long)a->max_seqlen_q * group <= pa::kDecodeRows;
  // Decode units over pairs of adjacent kv heads read row slices twice as
  // wide (512 bytes at head_dim 128, 256 at 64): when every sequence's rows
  // fit twice into a unit, the kv heads pair up, provided that the batch
  // still gives every compute unit at least two pair units and that the pair
  // units leave no partial round of workgroups the one-head units would not.
  // A CU holds two one-head decode workgroups, so those run in rounds of
  // 2 x CUs, and a pair unit takes two one-head units' time: pairs pay only where
  // 2 * rounds(pairs) <= rounds(one-head units).  Measured (one-head -> pair
  // units): +2 to +5% at head_dim 128 and +9 to +13% at 64 where both fill
  // whole rounds (e.g. 256 x 4096 MHA, 64 x 2048 with 32 heads of 64), but
  // 5-18% slower at 128 where pairs end on a part-filled round (48, 100 and
  // 40 sequences x 32 heads; 160 x 8 kv heads) and 7-23% slower at 64 (96,
  // 128 and 200 sequences x 12 heads).
  const long units1 = (long)a->batch * a->num_heads_kv;
  const long per_round = 2L * num_cus;
  const bool pair_fits = pl.all_decode && a->num_heads_kv % 2 == 0 &&
                         2L * a->max_seqlen_q * group <= pa::kDecodeRows;
  const bool pair_pays =
      units1 >= 4L * num_cus && 2 * cdiv(units1 / 2, per_round) <= cdiv(units1, per_round);
  const int pm = pair_mode();
  pl.pair = pair_fits && (pm == 2 || (pm == 1 && pair_pays)) ? 2 : 1;
  // Pair units that give every CU one keep their key ranges whole: the
  // heuristic's two splits for uneven unit counts made them 7-10% slower (50
  // and 52 sequences x 32 heads, 200 x 8 kv heads).  Fewer pair units (only
  // with PAGED_ATTN_HEAD_PAIRS=2) take the heuristic over the pairs.
  if (a->num_splits > 0)
    pl.splits = a->num_splits;
  else if (pl.pair == 2 && units1 / 2 >= num_cus)
    pl.splits = 1;
  else
    pl.splits = paged_attn_num_splits(a->batch, a->total_q, a->num_heads_q / pl.pair,
                                      a->num_heads_kv / pl.pair, a->head_dim, a->max_seqlen_q,
                                      pl.max_seqlen_k, num_cus);
  // workgroups per kv head: one per decode unit (decode-only kernel); one per
  // prefill unit plus one per two decode units (unified kernel).  Decode
  // units number at most batch * splits; prefill units, the sum over the n_p
  // prefill-mode sequences of cdiv(rows_b, kPrefillRows), at most
  // cdiv(total rows, kPrefillRows) + n_p - 1, where each such sequence has
  // more than kDecodeRows rows.
  long units_per_head = (long)a->batch * pl.splits;
  const long total_rows = (long)a->total_q * group;
  const long n_p = std::max(1L, std::min<long>(a->batch, total_rows / (pa::kDecodeRows + 1)));
  const long pre_per_head = cdiv(total_rows, pa::kPrefillRows) + n_p - 1;
  if (!pl.all_decode) units_per_head = cdiv(units_per_head, 2) + pre_per_head;
  pl.grid = units_per_head * (a->num_heads_kv / pl.pair);
  // Every sequence holds max_seqlen_q new tokens (their sum is total_q and
  // none exceeds max_seqlen_q) and more rows than a decode unit: the unified
  // kernel's prefill units follow from the block index, one per query tile.
  if (!pl.all_decode && (long)a->total_q == (long)a->batch * a->max_seqlen_q &&
      (long)a->max_seqlen_q * group > pa::kDecodeRows && !full_search_forced()) {
    pl.uniform_q_tiles = (int)cdiv((long)a->max_seqlen_q * group, pa::kPrefillRows);
    pl.grid = (long)a->batch * pl.uniform_q_tiles * a->num_heads_kv;
  }
  // A decode-mode sequence has 1 .. kDecodeRows / group new tokens.  The
  // shortest sequence has at least total_q - (batch - 1) * max_seqlen_q; if
  // that already exceeds a decode unit, every sequence is prefill-mode.
  const long shortest = (long)a->total_q - (long)(a->batch - 1) * a->max_seqlen_q;
  pl.may_mix = !pl.all_decode && group <= pa::kDecodeRows &&
               std::max(1L, shortest) * group <= pa::kDecodeRows;
  pl.grid_dec = (long)a->batch * pl.splits * a->num_heads_kv;
  pl.grid_pre = pre_per_head * a->num_heads_kv;
  if (pl.splits > 1) {
    // the device shares the budget by sequence length (one split each, the
    // rest in proportion to key tiles): one sequence can get up to
    // 1 + batch * (splits - 1), capped at kMaxSplits
    const long most = 1 + (long)a->batch * (pl.splits - 1);
    pl.max_splits = (int)std::min<long>(most, kMaxSplits);
    const size_t rows = (size_t)a->total_q * a->num_heads_q;
    pl.o_part_off = 0;
    pl.lse_part_off = align_up((size_t)pl.max_splits * rows * a->head_dim * sizeof(float), 256);
    pl.rsplit_off = align_up(pl.lse_part_off + (size_t)pl.max_splits * rows * sizeof(float), 256);
    pl.ws_bytes = align_up(pl.rsplit_off + rows * sizeof(int32_t), 256);
  }
  return pl;
}

// PAGED_ATTN_DEBUG=1: read the device metadata back (synchronising the
// stream) and check the preconditions the kernels rely on.
bool debug_checks() {
  const char *e = std::getenv("PAGED_ATTN_DEBUG");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

pa_status check_preconditions(const pa_fwd_args *a, bool append_only, hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_HIP;
  const int B = a->batch;
  std::vector<int32_t> seq(B), cu(B + 1);
  if (hipMemcpy(seq.data(), a->cache_seqlens, sizeof(int32_t) * B, hipMemcpyDeviceToHost) !=
          hipSuccess ||
      hipMemcpy(cu.data(), a->cu_seqlens_q, sizeof(int32_t) * (B + 1), hipMemcpyDeviceToHost) !=
          hipSuccess)
    return PA_ERR_HIP;
  const bool paged = a->block_table != nullptr;
  std::vector<int32_t> table;
  if (paged) {
    table.resize((size_t)B * a->max_pages_per_seq);
    if (hipMemcpy(table.data(), a->block_table, sizeof(int32_t) * table.size(),
                  hipMemcpyDeviceToHost) != hipSuccess)
      return PA_ERR_HIP;
  }
  if (cu[0] != 0 || cu[B] > a->total_q) return PA_ERR_PRECONDITION;
  const bool appends = a->k_new != nullptr;
  const long cap = paged ? (long)a->max_pages_per_seq * a->page_size : (long)a->contig_alloc;
  std::vector<long> targets;
  for (int b = 0; b < B; ++b) {
    const long n = (long)cu[b + 1] - cu[b];
    if (n < 0 || n > a->max_seqlen_q || seq[b] < 0) return PA_ERR_PRECONDITION;
    const long K = seq[b] + (appends ? n : 0);
    if (K > cap) return PA_ERR_PRECONDITION;
    if (!append_only && a->max_seqlen_k > 0 && K > a->max_seqlen_k) return PA_ERR_PRECONDITION;
    if (paged) {
      for (long j = 0; j < (K + a->page_size - 1) / a->page_size; ++j) {
        const int32_t pg = table[(size_t)b * a->max_pages_per_seq + j];
        if (pg < 0 || pg >= a->num_pages) return PA_ERR_PRECONDITION;
      }
    }
    if (appends) {
      for (long i = 0; i < n; ++i) {
        const long pos = seq[b] + i;
        targets.push_back(paged ? (long)table[(size_t)b * a->max_pages_per_seq + pos / a->page_size] *
                                          a->page_size + pos % a->page_size
                                : (long)b * a->contig_alloc + pos);
      }
    }
  }
  std::sort(targets.begin(), targets.end());
  if (std::adjacent_find(targets.begin(), targets.end()) != targets.end())
    return PA_ERR_PRECONDITION;
  return PA_OK;
}

bool single_kernel_forced() {
  const char *e = std::getenv("PAGED_ATTN_SINGLE_KERNEL");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

pa::Rotary rotary_of(const pa_fwd_args *a) {
  pa::Rotary r;
  r.cos = static_cast<const uint16_t *>(a->rotary_cos);
  r.sin = static_cast<const uint16_t *>(a->rotary_sin);
  r.rows = a->rotary_rows;
  r.rdim = a->rotary_cos != nullptr ? a->rotary_dim : 0;
  r.interleaved = a->rotary_interleaved;
  return r;
}

pa::CacheGeom geom_of(const pa_fwd_args *a) {
  pa::CacheGeom g;
  g.table = a->block_table;
  g.page_shift = a->block_table ? ilog2(a->page_size) : 0;
  g.mpp = a->max_pages_per_seq;
  g.num_pages = a->num_pages;
  g.contig_alloc = a->block_table ? 0 : a->contig_alloc;
  return g;
}

// seq_mode: 0 every sequence, 1 prefill-mode sequences only, 2 decode-mode
// sequences only
pa_status launch_append(const pa_fwd_args *a, hipStream_t stream, int seq_mode = 0) {
  if (a->total_q == 0 || a->max_seqlen_q == 0) return PA_OK;
  pa::AppendParams p;
  p.k_cache = static_cast<uint16_t *>(a->k_cache);
  p.v_cache = static_cast<uint16_t *>(a->v_cache);
  p.geom = geom_of(a);
  p.cache_seqlens = a->cache_seqlens;
  p.cu_seqlens_q = a->cu_seqlens_q;
  p.k_new = static_cast<const uint16_t *>(a->k_new);
  p.v_new = static_cast<const uint16_t *>(a->v_new);
  p.batch = a->batch;
  p.total_q = a->total_q;
  p.hkv = a->num_heads_kv;
  p.head_dim = a->head_dim;
  p.rot = rotary_of(a);
  const long kvrow = (long)a->num_heads_kv * a->head_dim;
  p.kn_stride = a->k_new_row_stride ? a->k_new_row_stride : kvrow;
  p.vn_stride = a->v_new_row_stride ? a->v_new_row_stride : kvrow;
  const int vec_per_row = a->num_heads_kv * a->head_dim / 8;
  p.tokens_per_block = std::max(1, 1024 / (2 * vec_per_row));
  p.seq_mode = seq_mode;
  p.group = a->num_heads_q / a->num_heads_kv;
  const int rows = seq_mode == 2 ? std::min(a->max_seqlen_q, std::max(1, pa::kDecodeRows / p.group))
                                 : a->max_seqlen_q;
  dim3 grid((unsigned)cdiv(rows, p.tokens_per_block), (unsigned)a->batch);
  if (grid.y > 65535u) return PA_ERR_SHAPE;
  if (a->dtype == PA_BF16)
    hipLaunchKernelGGL(pa::kv_append_kernel<pa::kBF16>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(pa::kv_append_kernel<pa::kF16>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// A mixed batch (decode-mode and prefill-mode sequences) runs its prefill
// units in the unified kernel and then its decode units in the decode-only
// kernel (four-wave workgroups, two per CU, longest first), both on `stream`.
// Measured on one prefill chunk + 64 decode sequences (32 x 128 and 12 x 64,
// chunks of 100 / 500 / 1000 tokens): faster than the same work as two calls
// at every point, 2-8% faster than one unified launch (whose 8-wave
// workgroups pair two decode units and hold the CU until the longer ends),
// and faster than the two kernels on concurrent streams except at 12 x 64
// with 500 / 1000-token chunks: a prefill workgroup needs a whole CU, and
// while the decode launch keeps refilling the CUs it frees, the prefill
// launch waits for CUs to drain.  Given a second stream (aux_stream) the
// concurrent plan is used: an event recorded on `stream` after the append
// forks aux_stream off for the decode units, a second one recorded on
// aux_stream after its launch joins it back.  Those events are created for
// the call and released right after the join is queued (the runtime keeps
// them until they complete).
struct Fork {
  hipEvent_t fork = nullptr, join = nullptr;
  ~Fork() {
    if (join != nullptr) (void)hipEventDestroy(join);
    if (fork != nullptr) (void)hipEventDestroy(fork);
  }
};

// append (if k_new), attention, and with split-KV the combine of the partials
template <int DT, int D>
pa_status launch_attention(const pa_fwd_args *a, const Plan &pl, hipStream_t stream,
                           hipStream_t aux, bool may_fork) {
  const int group = a->num_heads_q / a->num_heads_kv;
  pa::FwdParams p;
  p.q = static_cast<const uint16_t *>(a->q);
  p.q_stride = a->q_row_stride ? a->q_row_stride : (long)a->num_heads_q * a->head_dim;
  p.k_cache = static_cast<const uint16_t *>(a->k_cache);
  p.v_cache = static_cast<const uint16_t *>(a->v_cache);
  p.geom = geom_of(a);
  p.cache_seqlens = a->cache_seqlens;
  p.cu_seqlens_q = a->cu_seqlens_q;
  p.out = static_cast<uint16_t *>(a->out);
  p.lse = a->softmax_lse;
  char *ws = static_cast<char *>(a->workspace);
  const bool split = pl.splits > 1;
  p.o_part = split ? reinterpret_cast<float *>(ws + pl.o_part_off) : nullptr;
  p.lse_part = split ? reinterpret_cast<float *>(ws + pl.lse_part_off) : nullptr;
  p.row_splits = split ? reinterpret_cast<int32_t *>(ws + pl.rsplit_off) : nullptr;
  p.batch = a->batch;
  p.total_q = a->total_q;
  p.hq = a->num_heads_q;
  p.hkv = a->num_heads_kv;
  p.group = group;
  p.appended = a->k_new != nullptr;
  p.causal = a->causal;
  p.num_splits = pl.splits;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale
                                             : 1.0f / std::sqrt((float)a->head_dim);
  p.scale_log2 = scale * pa::kLog2e;
  p.all_decode = pl.all_decode;
  p.rot = rotary_of(a);
  p.unit_mode = 0;
  p.uniform_q_tiles = 0;
  p.full_search = full_search_forced() ? 1 : 0;
  if (pl.grid > 0x7fffffffL || pl.grid_dec > 0x7fffffffL || pl.grid_pre > 0x7fffffffL)
    return PA_ERR_SHAPE;
  // every row is appended before any attention launch, on either stream,
  // reads the pages
  if (a->k_new != nullptr) {
    const pa_status st = launch_append(a, stream);
    if (st != PA_OK) return st;
  }
  if (pl.all_decode) {
    if (pl.pair == 2)
      hipLaunchKernelGGL((pa::attn_decode_kernel<DT, D, 2>), dim3((unsigned)pl.grid),
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((pa::attn_decode_kernel<DT, D, 1>), dim3((unsigned)pl.grid),
                         dim3(kThreads), 0, stream, p);
  } else if (pl.may_mix && !single_kernel_forced() &&
             !(may_fork && aux != nullptr && aux != stream)) {
    p.unit_mode = 1;
    hipLaunchKernelGGL((pa::attn_fwd_kernel<DT, D>), dim3((unsigned)pl.grid_pre),
                       dim3(pa::kUThreads), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    p.unit_mode = 2;
    hipLaunchKernelGGL((pa::attn_decode_kernel<DT, D, 1>), dim3((unsigned)pl.grid_dec),
                       dim3(kThreads), 0, stream, p);
  } else if (pl.may_mix && !single_kernel_forced()) {
    Fork f;
    if (hipEventCreateWithFlags(&f.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&f.join, hipEventDisableTiming) != hipSuccess ||
        hipEventRecord(f.fork, stream) != hipSuccess ||
        hipStreamWaitEvent(aux, f.fork, 0) != hipSuccess)
      return PA_ERR_HIP;
    p.unit_mode = 2;
    hipLaunchKernelGGL((pa::attn_decode_kernel<DT, D, 1>), dim3((unsigned)pl.grid_dec),
                       dim3(kThreads), 0, aux, p);
    if (hipGetLastError() != hipSuccess || hipEventRecord(f.join, aux) != hipSuccess)
      return PA_ERR_HIP;
    p.unit_mode = 1;
    hipLaunchKernelGGL((pa::attn_fwd_kernel<DT, D>), dim3((unsigned)pl.grid_pre),
                       dim3(pa::kUThreads), 0, stream, p);
    // join even when the launch failed, so aux_stream is never left forked
    const bool launched = hipGetLastError() == hipSuccess;
    if (hipStreamWaitEvent(stream, f.join, 0) != hipSuccess || !launched) return PA_ERR_HIP;
  } else {
    p.uniform_q_tiles = pl.uniform_q_tiles;
    hipLaunchKernelGGL((pa::attn_fwd_kernel<DT, D>), dim3((unsigned)pl.grid), dim3(pa::kUThreads), 0,
                       stream, p);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (split) {
    pa::CombineParams c;
    c.o_part = p.o_part;
    c.lse_part = p.lse_part;
    c.row_splits = p.row_splits;
    c.cu_seqlens_q = a->cu_seqlens_q;
    c.out = p.out;
    c.lse = p.lse;
    c.batch = a->batch;
    c.total_q = a->total_q;
    c.hq = a->num_heads_q;
    c.max_splits = pl.max_splits;
    const long rows = (long)a->total_q * a->num_heads_q;
    const long blocks = cdiv(rows, pa::kWaves);
    if (blocks > 0x7fffffffL) return PA_ERR_SHAPE;
    hipLaunchKernelGGL((pa::combine_kernel<DT, D>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, c);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
pa_status scratch_address(void **out) {
  static std::atomic<void *> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= 64) return PA_ERR_UNSUPPORTED;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PA_OK;
}

template <class F>
pa_status dispatch(const pa_fwd_args *a, F &&launch) {
  const bool bf16 = a->dtype == PA_BF16;
  if (a->head_dim == 128)
    return bf16 ? launch(std::integral_constant<int, pa::kBF16>{}, std::integral_constant<int, 128>{})
                : launch(std::integral_constant<int, pa::kF16>{}, std::integral_constant<int, 128>{});
  return bf16 ? launch(std::integral_constant<int, pa::kBF16>{}, std::integral_constant<int, 64>{})
              : launch(std::integral_constant<int, pa::kF16>{}, std::integral_constant<int, 64>{});
}

}  // namespace

extern "C" {

int32_t paged_attn_num_splits(int32_t batch, int32_t total_q, int32_t num_heads_q,
                              int32_t num_heads_kv, int32_t head_dim, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, int32_t num_cus) {
  // Host-only cost model (no device length is read).  Work units without any
  // split: one per (sequence, kv head) plus the prefill tiles.  Once they give
  // every compute unit a workgroup, splitting mostly adds only partial-result
  // traffic and a combine (the exception, uneven units, follows).  Otherwise
  // split each key range so the units reach
  // one per compute unit, but keep at least 8 key tiles of 32 per split (two
  // per wave) so a split's fixed cost stays amortised, and stay within the
  // cap of 128.  A key range that allows only two such splits is halved only
  // while the units fill at most a quarter of the compute units (context 512:
  // halving took batch 1 from 19.8 to 18.0 us, left batch 2 at 18.4-18.6 and
  // took batch 4 from 19.0 to 20.8 - there the combine launch costs more than
  // the halved range saves).  (Measured
  // over MHA decode, 32 x 128, batch 1-256 x context 512-4096: with this
  // target the chosen budget is the fastest of 1/2/4/8 or within a few
  // percent of it at every point; targeting two workgroups per compute unit
  // split 256-unit batches and made them up to 19% slower.)
  (void)head_dim;
  if (batch < 1 || num_heads_q < 1 || num_heads_kv < 1 || max_seqlen_k < 1) return 1;
  if (num_cus < 1) num_cus = 256;
  const long group = num_heads_q / num_heads_kv > 0 ? num_heads_q / num_heads_kv : 1;
  long units = (long)batch * num_heads_kv;
  if ((long)max_seqlen_q * group > pa::kDecodeRows && total_q > 0)
    units += cdiv((long)total_q * group, pa::kPrefillRows) * num_heads_kv;
  const long target = num_cus;
  const long tiles = cdiv(max_seqlen_k, pa::kKeyTile);
  if (units >= target) {
    // An all-decode batch of one to four units per compute unit that leaves
    // some compute units a unit more than others (1.5 or 2.5 per CU) runs two
    // splits per key range when that evens the load by a tenth or more and
    // each split keeps 32 key tiles.  Measured (one split -> two, MHA 32 x 128
    // and 64 q / 8 kv heads): 384 units 2% faster at 2048 keys, 5-7% at 4096
    // and 8192; 640 units 1-4%; 768, 1280, 1536 and 2560 units (whole units
    // per CU) 1-2% slower split, so they stay whole.
    const bool decode_only = (long)max_seqlen_q * group <= pa::kDecodeRows;
    auto balance = [&](long n) { return (double)n / (double)(target * cdiv(n, target)); };
    if (decode_only && units < 4 * target && tiles >= 64 && balance(2 * units) >= balance(units) + 0.1)
      return 2;
    return 1;
  }
  long s = cdiv(target, units);
  const long cap = std::max(1L, tiles / 8);
  if (cap == 2 && s < 4) return 1;
  // With grouped heads the rows of a unit share its keys, so a unit computes
  // more per byte read, and a second workgroup per compute unit hides that
  // compute behind the other's loads: up to two units per CU while every
  // split keeps at least 64 key tiles (measured, 64 q / 8 kv heads x 128:
  // 16 sequences of 4096-12288 keys, budget 4 instead of 2, 105 -> 96 us;
  // the long split of 8 sequences, 8 instead of 4, 85.5 -> 84.0 us; MHA at
  // the same sizes within 1% either way, so it keeps one unit per CU).
  if (group > 1) s = std::max(s, std::min(cdiv(2 * target, units), tiles / 64));
  s = std::min(s, cap);
  s = std::max(1L, std::min(s, (long)kMaxSplits));
  return (int32_t)s;
}

int32_t paged_attn_splits_for(const pa_fwd_args *args) {
  if (validate(args, false, true) != PA_OK) return -1;
  return make_plan(args, device_cus()).splits;
}

size_t paged_attn_workspace_size(const pa_fwd_args *args) {
  if (validate(args, false, true) != PA_OK) return 0;
  return make_plan(args, device_cus()).ws_bytes;
}

pa_status paged_kv_append(const pa_fwd_args *args, void *stream) {
  pa_status st = validate(args, true);
  if (st != PA_OK) return st;
  if (debug_checks()) {
    st = check_preconditions(args, true, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  return launch_append(args, static_cast<hipStream_t>(stream));
}

pa_status paged_attn_fwd(const pa_fwd_args *args, void *stream) {
  pa_status st = validate(args, false);
  if (st != PA_OK) return st;
  if (args->total_q == 0) return PA_OK;
  if (debug_checks()) {
    st = check_preconditions(args, false, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  const Plan pl = make_plan(args, device_cus());
  if (pl.ws_bytes > 0 && (args->workspace == nullptr || args->workspace_bytes < pl.ws_bytes))
    return PA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t aux = static_cast<hipStream_t>(args->aux_stream);
  return dispatch(args, [&](auto dt, auto d) {
    return launch_attention<decltype(dt)::value, decltype(d)::value>(args, pl, s, aux, true);
  });
}

pa_status paged_attn_fwd_noalloc(const pa_fwd_args *args, void *stream) {
  pa_status st = validate(args, false);
  if (st != PA_OK) return st;
  if (args->total_q == 0) return PA_OK;
  const Plan pl = make_plan(args, device_cus());
  if (pl.ws_bytes > kScratchBytes) return PA_ERR_SCRATCH;
  pa_fwd_args a = *args;   // the caller's workspace and aux_stream are not used
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  a.aux_stream = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_address(&a.workspace);
    if (st != PA_OK) return st;
    a.workspace_bytes = kScratchBytes;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dispatch(&a, [&](auto dt, auto d) {
    return launch_attention<decltype(dt)::value, decltype(d)::value>(&a, pl, s, nullptr, false);
  });
}

const char *paged_attn_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case PA_ERR_DTYPE: return "dtype must be PA_F16 or PA_BF16";
    case PA_ERR_UNSUPPORTED: return "head_dim or page size not supported (head_dim 64/128, page size a power of two in [16, 256])";
    case PA_ERR_WORKSPACE: return "workspace missing or smaller than paged_attn_workspace_size";
    case PA_ERR_HIP: return "a HIP launch or runtime call failed";
    case PA_ERR_ALIGN: return "a buffer moved in 16-byte vectors is not 16-byte aligned";
    case PA_ERR_PRECONDITION: return "device metadata breaks a precondition (PAGED_ATTN_DEBUG=1)";
    case PA_ERR_SCRATCH: return "the call needs more split-KV scratch than paged_attn_fwd_noalloc's static 64 MiB array holds";
    default: return "unknown status";
  }
}

}  // extern "C"
