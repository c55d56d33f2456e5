/*
 * Paged KV-cache attention forward pass: plain CPU oracle in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference the HIP
 * library is checked against.  Only the test suite, the smoke entry point and
 * the benchmark's CPU-baseline leg load it; the product library never links,
 * calls or shares code with it, and it includes none of the product's headers.
 *
 * It is deliberately slow and literal: every step is the definition written
 * out, in the order the pages describe it, with no tiling, fusion or online
 * rescaling.  Pins (tests that tie it to something other than itself) live in
 * the test suite: brute-force dense attention, closed forms and invariants.
 *
 * Sources followed (page titles; the pages are GitHub threads):
 *  [FA-824]  "flash-attention: Add support for small page sizes"
 *            - reproduction script: cache layout [num_blocks, block_size,
 *              num_heads, head_dim], block_table [batch, cdiv(seq_len,
 *              block_size)] int32, cache_seqlens int32, new k/v appended at
 *              the cache_seqlens position, causal attention over the result.
 *            - follow-up comments: the call allocates nothing and reaches
 *              memory only through block_table; the fix reads each page id by
 *              its absolute logical index and copies only rows below seqlen.
 *  [VLLM-6052] "vllm: [Kernel] Unify the kernel used in flash attention
 *              backend" - one varlen call for prefill and decode tokens;
 *              CUDA-graph comment: padded batch slots with (0, 0) lengths must
 *              be no-ops.
 *  [VLLM-3010] "Introduce flash-attn (>= 2.5.0)" - MHA and MQA/GQA, prefill
 *              over a cached prefix.
 * Readings where the pages are silent (softmax scale 1/sqrt(D), bottom-right
 * causal alignment, q head h reads kv head h / (Hq/Hkv), empty key set gives
 * out = 0 and lse = -inf, lse in natural log) are stated next to the code
 * that takes them.
 *
 * Element storage: fp16 / bf16 values are passed as their raw 16-bit patterns
 * and widened exactly to double here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* IEEE binary16 -> double, exact (every binary16 value is a double). */
static double f16_bits_to_double(uint16_t h) {
  int sign = h >> 15;
  int expo = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)mant, -24);                 /* zero / subnormal */
  } else if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = ldexp((double)(mant | 0x400), expo - 25); /* (1.m) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double bits_to_double(int dtype, uint16_t x) {
  return dtype == ORACLE_BF16 ? bf16_bits_to_double(x) : f16_bits_to_double(x);
}

/* Exposed so the test suite can check the widening against numpy / torch. */
double oracle_bits_to_double(int dtype, uint16_t x) { return bits_to_double(dtype, x); }

/*
 * Physical row of logical key position `pos` of sequence `b`, or -1 when the
 * page id read from the table is outside the pool.  Paged mode follows the
 * reproduction script of [FA-824]: page = block_table[b][pos / page_size],
 * slot = pos % page_size, row = page * page_size + slot.  Contiguous mode
 * (no block table) is the pre-allocated per-sequence cache of the
 * determine_num_splits issue: row = b * alloc + pos.
 */
static long physical_row(int b, long pos, int page_size, int num_pages,
                         int max_pages_per_seq, int contig_alloc,
                         const int32_t *block_table) {
  if (block_table == NULL) {
    if (pos >= contig_alloc) return -1;
    return (long)b * contig_alloc + pos;
  }
  long logical_page = pos / page_size;
  if (logical_page >= max_pages_per_seq) return -1;
  int32_t page = block_table[(long)b * max_pages_per_seq + logical_page];
  if (page < 0 || page >= num_pages) return -1;
  return (long)page * page_size + pos % page_size;
}

/*
 * Step 1, append (the in-call k=, v= of the reproduction script, and vLLM's
 * reshape_and_cache): new token i of sequence b lands at logical position
 * cache_seqlens[b] + i.  A bit copy; cache_seqlens itself is not advanced.
 * Returns 0, or -1 if a target row is outside the pool (a precondition
 * violation the caller must not commit).
 */
int oracle_kv_append(int batch, int num_heads_kv, int head_dim, int page_size,
                     int num_pages, int max_pages_per_seq, int contig_alloc,
                     uint16_t *k_cache, uint16_t *v_cache,
                     const int32_t *block_table, const int32_t *cache_seqlens,
                     const int32_t *cu_seqlens_q, const uint16_t *k_new,
                     const uint16_t *v_new) {
  long row_elems = (long)num_heads_kv * head_dim;
  for (int b = 0; b < batch; ++b) {
    int q_len = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    for (int i = 0; i < q_len; ++i) {
      long pos = (long)cache_seqlens[b] + i;
      long row = physical_row(b, pos, page_size, num_pages, max_pages_per_seq,
                              contig_alloc, block_table);
      if (row < 0) return -1;
      long src = (long)(cu_seqlens_q[b] + i) * row_elems;
      memcpy(k_cache + row * row_elems, k_new + src, row_elems * sizeof(uint16_t));
      memcpy(v_cache + row * row_elems, v_new + src, row_elems * sizeof(uint16_t));
    }
  }
  return 0;
}

/*
 * Steps 2-6: gather, scores, mask, softmax, output.
 *
 *  K_b   = cache_seqlens[b] (+ q_len_b when the call appended new tokens).
 *  Visible keys of new token i of sequence b: j < K_b, and when causal
 *  j <= K_b - q_len_b + i (reading: bottom-right alignment, so token i sits at
 *  absolute position K_b - q_len_b + i; a single decode token then sees the
 *  whole cache, which is how [VLLM-6052] sends decode tokens through the same
 *  causal varlen call).
 *  q head h reads kv head h / (Hq / Hkv) (reading: contiguous groups).
 *  key_begin / key_end (optional, per sequence) restrict the visible keys to a
 *  window; they exist so the split-KV combine can be checked against the
 *  unsplit result.  NULL means no restriction.
 *  Outputs, unrounded fp64: out [total_q, Hq, D]; lse [total_q, Hq] natural
 *  log; an empty visible set gives out = 0, lse = -inf.
 * Returns 0, or -1 when a key row that must be read lies outside the pool.
 */
int oracle_attention(int dtype, int batch, int num_heads_q, int num_heads_kv,
                     int head_dim, int page_size, int num_pages,
                     int max_pages_per_seq, int contig_alloc,
                     const uint16_t *q, const uint16_t *k_cache,
                     const uint16_t *v_cache, const int32_t *block_table,
                     const int32_t *cache_seqlens, const int32_t *cu_seqlens_q,
                     int appended, int causal, double scale,
                     const int32_t *key_begin, const int32_t *key_end,
                     double *out, double *lse, int num_threads) {
  const int group = num_heads_q / num_heads_kv;
  const int D = head_dim;
  int status = 0;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif

  /* One work item per (sequence, kv head): gather that head's keys and
   * values once, then answer every query row that reads them. */
#pragma omp parallel for schedule(dynamic, 1)
  for (long item = 0; item < (long)batch * num_heads_kv; ++item) {
    int b = (int)(item / num_heads_kv);
    int g = (int)(item % num_heads_kv);
    int q_start = cu_seqlens_q[b];
    int q_len = cu_seqlens_q[b + 1] - q_start;
    if (q_len <= 0) continue; /* padded (0, 0) slot: writes nothing */
    long K_b = (long)cache_seqlens[b] + (appended ? q_len : 0);

    double *Kg = (double *)malloc(sizeof(double) * (size_t)(K_b > 0 ? K_b : 1) * D);
    double *Vg = (double *)malloc(sizeof(double) * (size_t)(K_b > 0 ? K_b : 1) * D);
    double *s = (double *)malloc(sizeof(double) * (size_t)(K_b > 0 ? K_b : 1));
    int bad = 0;

    /* Step 2, gather: logical key j of this sequence through the table.  Only
     * the first cdiv(K_b, page_size) table entries are ever read. */
    for (long j = 0; j < K_b && !bad; ++j) {
      long row = physical_row(b, j, page_size, num_pages, max_pages_per_seq,
                              contig_alloc, block_table);
      if (row < 0) { bad = 1; break; }
      const uint16_t *kr = k_cache + (row * num_heads_kv + g) * D;
      const uint16_t *vr = v_cache + (row * num_heads_kv + g) * D;
      for (int c = 0; c < D; ++c) {
        Kg[j * D + c] = bits_to_double(dtype, kr[c]);
        Vg[j * D + c] = bits_to_double(dtype, vr[c]);
      }
    }
    if (bad) {
#pragma omp atomic write
      status = -1;
      free(Kg); free(Vg); free(s);
      continue;
    }

    for (int i = 0; i < q_len; ++i) {
      /* Visible window [lo, hi) of this query token. */
      long hi = K_b;
      if (causal) {
        long lim = K_b - q_len + i + 1;
        if (lim < hi) hi = lim;
      }
      long lo = 0;
      if (key_begin && key_begin[b] > lo) lo = key_begin[b];
      if (key_end && key_end[b] < hi) hi = key_end[b];

      for (int hh = 0; hh < group; ++hh) {
        int h = g * group + hh;
        long row_q = (long)(q_start + i) * num_heads_q + h;
        double *o = out + row_q * D;
        if (hi <= lo) {
          for (int c = 0; c < D; ++c) o[c] = 0.0;
          lse[row_q] = -INFINITY;
          continue;
        }
        double qv[512];
        for (int c = 0; c < D; ++c) qv[c] = bits_to_double(dtype, q[row_q * D + c]);

        /* Step 3, scores. */
        for (long j = lo; j < hi; ++j) {
          double acc = 0.0;
          for (int c = 0; c < D; ++c) acc += qv[c] * Kg[j * D + c];
          s[j] = scale * acc;
        }
        /* Step 4, softmax with the maximum subtracted. */
        double m = -INFINITY;
        for (long j = lo; j < hi; ++j) if (s[j] > m) m = s[j];
        double l = 0.0;
        for (long j = lo; j < hi; ++j) l += exp(s[j] - m);
        /* Step 5, weighted sum of values. */
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        for (long j = lo; j < hi; ++j) {
          double p = exp(s[j] - m) / l;
          for (int c = 0; c < D; ++c) o[c] += p * Vg[j * D + c];
        }
        lse[row_q] = m + log(l);
      }
    }
    free(Kg); free(Vg); free(s);
  }
  return status;
}

/*
 * Split-KV combine (the merge that follows a split-KV launch): partial
 * results o_s (each normalised over its own key window) with log-sum-exp
 * lse_s merge to lse = log(sum_s exp(lse_s)) and out = sum_s exp(lse_s - lse)
 * * o_s.  Splits with lse_s = -inf saw no keys and contribute nothing; if
 * every split is empty, out = 0 and lse = -inf.
 * o_parts [S][rows][D], lse_parts [S][rows].
 */
void oracle_combine(int num_splits, long rows, int head_dim,
                    const double *o_parts, const double *lse_parts,
                    double *out, double *lse) {
  for (long r = 0; r < rows; ++r) {
    double m = -INFINITY;
    for (int s = 0; s < num_splits; ++s) {
      double v = lse_parts[(long)s * rows + r];
      if (v > m) m = v;
    }
    double *o = out + r * head_dim;
    for (int c = 0; c < head_dim; ++c) o[c] = 0.0;
    if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
    double total = 0.0;
    for (int s = 0; s < num_splits; ++s) {
      double v = lse_parts[(long)s * rows + r];
      if (v == -INFINITY) continue;
      total += exp(v - m);
    }
    double L = m + log(total);
    for (int s = 0; s < num_splits; ++s) {
      double v = lse_parts[(long)s * rows + r];
      if (v == -INFINITY) continue;
      double w = exp(v - L);
      const double *os = o_parts + ((long)s * rows + r) * head_dim;
      for (int c = 0; c < head_dim; ++c) o[c] += w * os[c];
    }
    lse[r] = L;
  }
}
