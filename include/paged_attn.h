/*
 * paged_attn.h - C ABI of the MI355X (gfx950) paged KV-cache attention library
 * (libpaged_attn.so).
 *
 * The operation is the paged KV-cache attention forward pass that the
 * flash-attention thread "Add support for small page sizes" exercises in its
 * reproduction script (a block_table maps each sequence's logical pages, 16 to
 * 256 tokens each, onto a shared physical K/V pool; new K/V rows are appended
 * at cache_seqlens and then attended to, causally), generalised to the packed
 * variable-length batches of the vLLM thread "Unify the kernel used in flash
 * attention backend" (prefill chunks and decode tokens in one call) and to the
 * MQA/GQA head layouts of the vLLM pull request "Introduce flash-attn
 * (>= 2.5.0)".
 *
 * Conventions shared by every entry point
 *  - Pure C: no HIP or C++ types cross this boundary.  A stream is passed as
 *    `void *` holding a hipStream_t (NULL = the legacy default stream).
 *  - Every device buffer is owned by the caller.  The library never allocates
 *    device memory, frees or synchronises inside paged_attn_fwd /
 *    paged_kv_append (the reproduction-script thread notes the call reaches
 *    memory only through the block table; the determine_num_splits issue rules
 *    out reading device lengths back to the host).  Scratch space comes in
 *    through `workspace`; the only runtime objects the library creates are the
 *    two events of a forked call described at paged_attn_fwd, released by
 *    the call.
 *  - Launch shape and kernel choice depend only on host-side fields, so a call
 *    can be captured in a HIP graph; the CUDA-graph comment of the "Unify the
 *    kernel" thread sets the rule: static maxima, static metadata buffers,
 *    padded batch slots with zero lengths.
 *  - Errors the host can see are returned before anything is launched.  A
 *    launch failure returns PA_ERR_HIP.  Device-side faults are asynchronous
 *    and surface at the caller's next synchronisation.  No exception crosses
 *    the ABI.  The library keeps no mutable global state except a per-device
 *    cache of the compute-unit count and, for paged_attn_fwd_noalloc only,
 *    its static scratch array and that array's per-device address.
 *  - Element types: q, caches, k_new, v_new and out share one 16-bit float
 *    type (fp16 or bf16).  Accumulation is fp32; out is rounded to nearest
 *    even once; softmax_lse is fp32, natural log.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  PA_ERR_DTYPE = 3,       /* dtype is not PA_F16 / PA_BF16 */
  PA_ERR_UNSUPPORTED = 4, /* head_dim or page size the library does not serve, or one
                             page (contiguous mode: one sequence's allocation) spans
                             2 GiB or more */
  PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than paged_attn_workspace_size */
  PA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_ALIGN = 7,       /* a buffer read or written in 16-byte vectors (q, caches,
                             k_new, v_new, out, rotary tables) is not 16-byte aligned */
  PA_ERR_PRECONDITION = 8,/* device metadata breaks a precondition; only reported when
                             the environment sets PAGED_ATTN_DEBUG=1 (see below) */
  PA_ERR_SCRATCH = 9      /* paged_attn_fwd_noalloc: the call's split-KV scratch exceeds
                             the library's static 64 MiB array */
} pa_status;

typedef enum pa_dtype { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * Arguments of one forward call.  All sizes are host integers; every pointer
 * except workspace-less cases must be a device pointer.
 *
 * Shapes (row-major, dense):
 *   q            [total_q, num_heads_q, head_dim]                dtype
 *   k_cache,     paged:      [num_pages, page_size, num_heads_kv, head_dim]
 *   v_cache      contiguous: [batch, contig_alloc, num_heads_kv, head_dim]
 *   block_table  [batch, max_pages_per_seq] int32, or NULL for contiguous mode
 *   cache_seqlens[batch] int32: tokens already in the cache; NOT modified
 *   cu_seqlens_q [batch + 1] int32: cu[0] = 0, non-decreasing, cu[batch] =
 *                total_q; sequence b owns packed rows cu[b] .. cu[b+1]-1
 *   k_new, v_new [total_q, num_heads_kv, head_dim] dtype, or both NULL
 *   out          [total_q, num_heads_q, head_dim] dtype (written)
 *   softmax_lse  [total_q, num_heads_q] float (written)
 *
 * Semantics (the plainest reading of the pages, where they are silent):
 *   - With k_new/v_new, new row i of sequence b is first written to logical
 *     position cache_seqlens[b] + i (page block_table[b][pos / page_size],
 *     slot pos % page_size), then attended to: K_b = cache_seqlens[b] + q_len_b.
 *     Without them K_b = cache_seqlens[b].
 *   - Causal masking is bottom-right aligned: new token i of sequence b sits at
 *     position K_b - q_len_b + i and sees keys 0 .. K_b - q_len_b + i.
 *   - q head h reads kv head h / (num_heads_q / num_heads_kv).
 *   - A row with no visible key gets out = 0 and softmax_lse = -inf.
 *   - Sequences with q_len_b = 0 (e.g. padded graph slots) write nothing.
 *   - Only the first cdiv(K_b, page_size) entries of a table row are read.
 *   - Rotary embedding (rotary_cos != NULL): the small-page-size thread's
 *     kernel fuses a rotary position embedding into the call; here it is the
 *     standard RoPE rotation.  Every new token has the position K_b - q_len_b
 *     + i (cache_seqlens[b] + i when k_new is given).  Its query row and its
 *     new key row are rotated at that position before anything else; values
 *     never are.  Pair j of a head row (elements (j, j + rotary_dim/2), or
 *     (2j, 2j+1) when rotary_interleaved) becomes
 *         (a cos - b sin, b cos + a sin),  cos = rotary_cos[pos][j],
 *                                         sin = rotary_sin[pos][j];
 *     elements from rotary_dim on are kept.  Arithmetic: the exact value
 *     rounded to fp32, then to the element type (nearest even), so the stored
 *     keys are bit-reproducible.  A position outside [0, rotary_rows) leaves
 *     the row unrotated.
 *
 * Preconditions the host cannot check (device-resident metadata):
 *   q_len_b <= max_seqlen_q; K_b <= max_pages_per_seq * page_size (contiguous
 *   mode: K_b <= contig_alloc); the page ids read lie in [0, num_pages);
 *   append targets of different sequences are distinct slots.  (k_new/v_new
 *   overlapping the caches is host-checkable: PA_ERR_SHAPE.)  With the
 *   environment variable PAGED_ATTN_DEBUG=1, paged_attn_fwd and
 *   paged_kv_append first synchronise the stream, copy cache_seqlens,
 *   cu_seqlens_q and block_table to the host and check these (and that
 *   cu_seqlens_q starts at 0, does not decrease and ends within total_q, and
 *   K_b <= max_seqlen_k when given), returning PA_ERR_PRECONDITION before any
 *   launch if one fails; that mode syncs, so such a call cannot be captured
 *   in a graph.  Otherwise device code never reads outside the table row or
 *   the pool: a key whose page id is out of range is read as a zero K row and
 *   a zero V row (no error is raised; the result is then unspecified beyond
 *   being finite), and an append to such a slot is dropped.
 */
typedef struct pa_fwd_args {
  int32_t dtype;             /* pa_dtype */
  int32_t batch;             /* >= 1 */
  int32_t total_q;           /* rows of q (host-static upper bound allowed: >= cu[batch]) */
  int32_t max_seqlen_q;      /* >= every q_len_b (host-static) */
  int32_t max_seqlen_k;      /* host bound on K_b; 0 -> max_pages_per_seq*page_size (or contig_alloc) */
  int32_t num_heads_q;
  int32_t num_heads_kv;      /* num_heads_q % num_heads_kv == 0 */
  int32_t head_dim;          /* 64 or 128 */
  int32_t page_size;         /* paged mode: power of two in [16, 256] */
  int32_t num_pages;         /* paged mode: pool size */
  int32_t max_pages_per_seq; /* paged mode: block_table width */
  int32_t contig_alloc;      /* contiguous mode: tokens allocated per sequence */
  int32_t causal;            /* 0 / 1 */
  int32_t num_splits;        /* 0 = heuristic; 1..128 = forced split-KV count */
  float softmax_scale;       /* <= 0 -> 1/sqrt(head_dim) */
  int32_t reserved0;         /* must be 0 */
  const void *q;
  void *k_cache;
  void *v_cache;
  const int32_t *block_table;
  const int32_t *cache_seqlens;
  const int32_t *cu_seqlens_q;
  const void *k_new;
  const void *v_new;
  void *out;
  float *softmax_lse;
  void *workspace;           /* device scratch, caller-owned; may be NULL if size is 0 */
  size_t workspace_bytes;
  const void *rotary_cos;    /* [rotary_rows, rotary_dim / 2] dtype, or NULL: no rotary */
  const void *rotary_sin;    /* same shape and type; NULL exactly when rotary_cos is */
  int32_t rotary_dim;        /* with tables: a multiple of 16 in [16, head_dim]; else 0 */
  int32_t rotary_interleaved;/* 0: pairs (j, j + rotary_dim / 2); 1: pairs (2j, 2j + 1) */
  int32_t rotary_rows;       /* with tables: rows (positions) they hold, >= 1; else 0 */
  int32_t reserved1;         /* must be 0 */
  /* Row strides, in elements, between consecutive tokens of q, k_new and
   * v_new (0: dense, num_heads * head_dim).  The heads and head_dim of a row
   * stay dense; a stride lets the three be views into one fused QKV
   * projection output.  A nonzero stride is at least the row size and a
   * multiple of 8 (16-byte aligned rows). */
  int64_t q_row_stride;
  int64_t k_new_row_stride;
  int64_t v_new_row_stride;
  /* Optional second stream (hipStream_t; NULL: none) for a batch that mixes
   * decode-mode and prefill-mode sequences: its decode units then run on it,
   * concurrently with the prefill units on the call's stream (see
   * paged_attn_fwd; measured faster than the one-stream plan only when the
   * prefill part is large).  Owned by the caller; the library only queues
   * work on it. */
  void *aux_stream;
} pa_fwd_args;

/*
 * paged_attn_fwd - the whole forward call on `stream`: append k_new/v_new into
 * the pages (if given), attend over each sequence's cache, and - when the
 * split-KV count is above one - merge the per-split partial rows with a
 * log-sum-exp combine.  Kernels run in that order; the call returns as soon
 * as they are queued.
 * A batch whose sizes allow both decode-mode sequences (q_len * group <= 16)
 * and prefill-mode ones runs its attention as two launches on `stream`: the
 * prefill units (8-wave workgroups), then the decode units (4-wave
 * workgroups).  Called with an aux_stream, the two run concurrently instead:
 * after the append on `stream`, an event forks aux_stream off to run the
 * decode units, the prefill units run on `stream`, and `stream` then waits on
 * a second event recorded on aux_stream before the combine.  Work queued on
 * `stream` afterwards therefore sees the whole call, and a capture of
 * `stream` takes in both launches.  The two events are created for the call
 * and released once the join is queued.  With the environment variable
 * PAGED_ATTN_SINGLE_KERNEL=1 the attention is one unified launch on `stream`.
 * Every plan gives the same results, bit for bit.
 * Returns PA_OK or the first host-detected error (nothing launched then);
 * PA_ERR_HIP if a launch or an event operation fails.
 */
pa_status paged_attn_fwd(const pa_fwd_args *args, void *stream);

/*
 * paged_attn_fwd_noalloc - paged_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels and results (bit for bit)
 * as paged_attn_fwd, except that args->workspace / workspace_bytes and
 * args->aux_stream are ignored: the split-KV scratch is a static device array
 * of the library (64 MiB = 67108864 bytes), one per device, held from the
 * library's load on the device until the process ends, and a mixed batch
 * never forks onto a second stream: all of its launches (by default the
 * prefill units, then the decode units) run on `stream`.  The call makes no
 * allocation of any kind (it creates no events either) and never
 * synchronises; PAGED_ATTN_DEBUG is not honoured here.  A call whose plan
 * needs more scratch than the array holds returns PA_ERR_SCRATCH before any
 * launch (paged_attn_workspace_size gives the need).  Every call on a device
 * shares that device's array, and the array keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap on one device
 * (concurrent streams, or several host threads) race on it and must be
 * serialised by the caller.
 */
pa_status paged_attn_fwd_noalloc(const pa_fwd_args *args, void *stream);

/*
 * paged_kv_append - the append step alone (vLLM's reshape_and_cache): writes
 * k_new/v_new rows to positions cache_seqlens[b] + i through the block table
 * (or the contiguous cache).  Reads only the fields the append needs
 * (dtype, batch, total_q, max_seqlen_q, num_heads_kv, head_dim, page_size,
 * num_pages, max_pages_per_seq, contig_alloc, k_cache, v_cache, block_table,
 * cache_seqlens, cu_seqlens_q, k_new, v_new and the rotary fields).  A bit
 * copy, except that with rotary tables each key row is first rotated at its
 * position cache_seqlens[b] + i, as in paged_attn_fwd.
 */
pa_status paged_kv_append(const pa_fwd_args *args, void *stream);

/*
 * paged_attn_workspace_size - bytes of device workspace paged_attn_fwd needs
 * for these arguments (0 when no split-KV partials are kept): the partial
 * rows and log-sum-exps of every split and each row's split count.  Its
 * contents need no initialisation and are scratch after the call.  Basis: the
 * small-page-size thread notes the paged call allocates nothing itself, so
 * the split-KV partials of the determine_num_splits issue's split path live
 * in caller-owned memory sized by this query.  Host only; no
 * device access.  Only sizes and flags are read (data pointers may still be
 * NULL; k_new/v_new only matter through being NULL or not).  Returns 0 for
 * invalid sizes as well.
 */
size_t paged_attn_workspace_size(const pa_fwd_args *args);

/*
 * paged_attn_splits_for - the split-KV count paged_attn_fwd will use for these
 * arguments (the forced value; else 1 when the plan runs decode units over
 * pairs of kv heads, and paged_attn_num_splits on this device otherwise), or
 * -1 for invalid sizes.  Reads sizes and flags only, like paged_attn_workspace_size;
 * host only apart from one cached device-attribute query.
 */
int32_t paged_attn_splits_for(const pa_fwd_args *args);

/*
 * paged_attn_num_splits - the split-count heuristic (host only, pure function
 * of its arguments).  The determine_num_splits issue fixes its inputs to
 * host-known sizes (batch, heads, head size, query and key lengths, compute
 * unit count) and caps it below 128; lengths on the device are never read.
 * Returns a value in [1, 128].
 */
int32_t paged_attn_num_splits(int32_t batch, int32_t total_q, int32_t num_heads_q,
                              int32_t num_heads_kv, int32_t head_dim,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_cus);

/* paged_attn_status_string - static, human-readable text for a status code.
 * Basis: the pages report failures only as asynchronous CUDA errors far from
 * their cause (the small-page-size thread's illegal-memory-access trace);
 * here every host-detectable error is a status returned before any launch,
 * and this names it. */
const char *paged_attn_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
