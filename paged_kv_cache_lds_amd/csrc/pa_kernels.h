// gfx950 kernels of the paged KV-cache attention forward pass.
//
//   kv_append_kernel   new K/V rows -> their page slots (bit copy)
//   attn_fwd_kernel    one unified varlen kernel: decode units and prefill
//                      tiles in one grid; QK^T and PV on MFMA with fp32
//                      accumulation, online softmax, split-KV partial or final
//                      epilogue
//   combine_kernel     log-sum-exp merge of split-KV partials
#pragma once

#include "pa_common.h"
#include "pa_decode.h"
#include "pa_prefill.h"

namespace pa {

// NH: kv heads per decode unit in the decode-only kernel (1, or 2 for a pair
// of adjacent heads, see decode_unit_pair); workgroups number units per
// group of NH kv heads.
template <int DT, int D, bool kUnified, int NH = 1>
__device__ __forceinline__ void attn_fwd_body(const FwdParams &p) {
  constexpr int NW = kUnified ? kUWaves : kWaves;   // waves of the workgroup
  __shared__ float sm_m[NW][kDecodeRows];           // per-wave decode states (two halves
  __shared__ float sm_l[NW][kDecodeRows];           // of four in the unified kernel)
  __shared__ int s_wsum[NW];
  __shared__ int s_found[2 * kFound];
  __shared__ int s_split[kFewSeqs];

  static_assert(NH == 1 || !kUnified, "pairs of heads only in the decode-only kernel");
  const int hgroups = p.hkv / NH;
  const int g = blockIdx.x % hgroups;   // kv head (NH = 1) or pair of kv heads (NH = 2)
  const int wg = blockIdx.x / hgroups;
  UnitInfo u;
  bool decode = true;
  bool have = true;
  if constexpr (!kUnified) {
    // decode units with one unit per sequence: longest first (a varlen decode
    // batch of 64 sequences x 32 heads ran 4% faster); past kOrderMax
    // sequences of an all-decode batch, unit = sequence.  With a split budget the device
    // share already evens the units out, and ordering would only add its
    // barriers.
    if (p.num_splits == 1 && p.batch > kOrderMax && p.unit_mode == 0) {
      u.b = wg;
      u.off = 0;
      u.splits = 1;
      u.si.q_len = -1;
      have = u.b < p.batch;
    } else if (p.batch == 1 && p.all_decode && !p.full_search) {
      // one sequence: the whole split budget is its own, so its split count
      // follows from its length alone (what the search below would find) and
      // workgroup wg takes split wg
      const SeqInfo si = seq_info(p, 0);
      const int t = decode_tiles(si.K_b);
      u.b = 0;
      u.off = wg;
      u.splits = si.q_len > 0 ? seq_splits(p.num_splits - 1, t, t) : 0;
      u.si = si;
      have = wg < u.splits;
    } else if (p.batch <= kFewSeqs && (p.all_decode || p.unit_mode == 2) && !p.full_search) {
      // a few sequences: the search in one wave, published with one barrier
      if (threadIdx.x < 64) find_decode_few(p, wg, p.num_splits == 1, s_found);
      __syncthreads();
      u.b = s_found[0];
      u.off = s_found[1];
      u.splits = s_found[2];
      u.si.cu_b = s_found[3];
      u.si.q_len = u.b >= 0 ? s_found[4] : -1;
      u.si.K_b = s_found[5];
      have = u.b >= 0;
    } else if (p.num_splits == 1) {
      __shared__ DecodeOrder s_order;
      have = locate_unit<NW * 64, 1>(p, wg, u, decode, s_wsum, s_found, s_split, &s_order);
    } else {
      have = locate_unit<NW * 64, 1>(p, wg, u, decode, s_wsum, s_found, s_split, nullptr);
    }
  } else if (p.uniform_q_tiles > 0) {
    // Every sequence has the same query length (more rows than a decode
    // unit): the units follow from the block index in the order the search
    // below would give them (sequence by sequence, a sequence's last and
    // heaviest query tile first), without its passes over the metadata.
    // Measured, attention only: causal prefill 4x2048 197 -> 187 us, 4x8192
    // 2181 -> 2079 us.  The heaviest tiles of every sequence first instead
    // ran 1-5% slower than this order, under which the query tiles of one
    // sequence run at the same time and can share its K/V in L2.
    have = wg < p.batch * p.uniform_q_tiles;
    u.b = wg / p.uniform_q_tiles;
    u.off = wg % p.uniform_q_tiles;
    u.splits = 1;
    u.si.q_len = -1;
    decode = false;
  } else {
    // the unified kernel keeps index order: measured, longest-first made a
    // mixed batch with 12 heads x 64 7% faster but one with 32 heads x 128 4%
    // slower (there, short units mixed with long ones keep HBM busy to the end)
    have = locate_unit<NW * 64, 2>(p, wg, u, decode, s_wsum, s_found, s_split, nullptr);
  }
  // A half of the unified kernel without a decode unit still meets the one
  // workgroup barrier of the other half's decode unit.
  auto idle_half = [&]() {
    if (kUnified && decode) __syncthreads();
  };
  if (!have) {
    idle_half();
    return;
  }
  // the unit and its sequence are the same for every lane of a wave: keep
  // them in SGPRs (page indices, buffer descriptors and uniform offsets derive
  // from them)
  u.b = __builtin_amdgcn_readfirstlane(u.b);
  u.off = __builtin_amdgcn_readfirstlane(u.off);
  u.splits = __builtin_amdgcn_readfirstlane(u.splits);
  SeqInfo si = __builtin_amdgcn_readfirstlane(u.si.q_len) >= 0 ? u.si : seq_info(p, u.b);
  si.cu_b = __builtin_amdgcn_readfirstlane(si.cu_b);
  si.q_len = __builtin_amdgcn_readfirstlane(si.q_len);
  si.K_b = __builtin_amdgcn_readfirstlane(si.K_b);
  const int rows_b = si.q_len * p.group;
  if (rows_b <= 0) {   // only in the single-split decode-only mapping
    idle_half();
    return;
  }

  if constexpr (!kUnified) {
    // decode-only kernel: one contiguous array, a K and a V tile per wave
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kWaves * 2 * kKeyTile * D];
    if constexpr (NH == 2)
      decode_unit_pair<DT, D, kWaves>(p, u.b, g, u.off, u.splits, si,
                                      ContigDecodeLds<kKeyTile * D>{lds}, sm_m, sm_l);
    else
      decode_unit<DT, D, kWaves>(p, u.b, g, u.off, u.splits, si,
                                 ContigDecodeLds<kKeyTile * D>{lds}, sm_m, sm_l);
  } else {
    // unified kernel: sixteen separate 32-row slots - a K/V pair per wave of a
    // decode unit, four K and four V slots of a prefill unit (K slots at
    // D = 128 carry 64 halves of padding per two 1 KiB blocks)
    constexpr int kSlotH = kKeyTile * D + (D == 128 ? 3 * 64 : 0);
    static_assert(kPTile == kKeyTile, "prefill and decode tiles share the slots");
    __shared__ __attribute__((aligned(256))) uint16_t lds_s0[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s1[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s2[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s3[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s4[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s5[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s6[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s7[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s8[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s9[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s10[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s11[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s12[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s13[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s14[kSlotH];
    __shared__ __attribute__((aligned(256))) uint16_t lds_s15[kSlotH];
    LdsPool pool;
    pool.sl[0] = lds_s0;
    pool.sl[1] = lds_s1;
    pool.sl[2] = lds_s2;
    pool.sl[3] = lds_s3;
    pool.sl[4] = lds_s4;
    pool.sl[5] = lds_s5;
    pool.sl[6] = lds_s6;
    pool.sl[7] = lds_s7;
    pool.sl[8] = lds_s8;
    pool.sl[9] = lds_s9;
    pool.sl[10] = lds_s10;
    pool.sl[11] = lds_s11;
    pool.sl[12] = lds_s12;
    pool.sl[13] = lds_s13;
    pool.sl[14] = lds_s14;
    pool.sl[15] = lds_s15;
    if (decode) {
      if (threadIdx.x < kWaves * 64)
        decode_unit<DT, D, kWaves>(p, u.b, g, u.off, u.splits, si, PoolDecodeLds<0>{pool}, sm_m,
                                   sm_l);
      else
        decode_unit<DT, D, kWaves>(p, u.b, g, u.off, u.splits, si, PoolDecodeLds<1>{pool},
                                   sm_m + kWaves, sm_l + kWaves);
    } else {
      const int n_qt = (rows_b + kPrefillRows - 1) / kPrefillRows;
      // a query tile past the sequence's rows: only when some sequence broke
      // the q_len <= max_seqlen_q bound, so that this one is shorter than the
      // equal-length mapping assumed
      if (u.off >= n_qt) return;
      if (p.geom.table != nullptr)
        prefill_unit<DT, D, true>(p, u.b, g, n_qt - 1 - u.off, si, pool);
      else
        prefill_unit<DT, D, false>(p, u.b, g, n_qt - 1 - u.off, si, pool);
    }
  }
}

// Decode-only batches (every sequence fits a decode unit, known on the host),
// and the decode units of a mixed batch launched beside its prefill units:
// four waves, two workgroups per CU.
template <int DT, int D, int NH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_decode_kernel(FwdParams p) {
  attn_fwd_body<DT, D, false, NH>(p);
}

// Unified kernel for any mix of prefill and decode sequences: eight waves,
// two per SIMD, one workgroup per CU.
template <int DT, int D>
__global__ __launch_bounds__(kUThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  attn_fwd_body<DT, D, true>(p);
}

// ---------------------------------------------------------------------------
// Split-KV combine: per (token, q head) row written as partials by more than
// one split, lse = log(sum_s exp(lse_s)) and out = sum_s exp(lse_s - lse) *
// o_s over the splits that saw a key; a row whose splits were all empty gets
// out = 0, lse = -inf.  One wave per row.  The attention kernel recorded each
// row's split count (1 for rows it wrote directly), so a wave needs two
// rounds of loads: that count with cu_seqlens_q[batch] (rows past it belong
// to no sequence), then every split's partial row at once.
// ---------------------------------------------------------------------------
struct CombineParams {
  const float *o_part;
  const float *lse_part;
  const int32_t *row_splits;
  const int32_t *cu_seqlens_q;
  uint16_t *out;
  float *lse;
  int batch, total_q, hq, max_splits;
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long)p.total_q * p.hq) return;
  const int rows_end = min(p.cu_seqlens_q[p.batch], p.total_q);
  const int S = min(p.row_splits[row], p.max_splits);   // clamped: never past the partials
  if (row / p.hq >= rows_end || S <= 1) return;          // no sequence, or written directly
  const long stride = (long)p.total_q * p.hq;
  constexpr int PER = D / 64;
  // chunks of eight splits: their lses and partial rows (PER dims per lane)
  // are all loaded before any is used, and chunks merge by a running maximum
  constexpr int CK = 8;
  float M = kNegInf, total = 0.f;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  for (int s0 = 0; s0 < S; s0 += CK) {
    float ls[CK], v[CK][PER];
#pragma unroll
    for (int j = 0; j < CK; ++j) {
      const long sj = min(s0 + j, S - 1);   // past the last split: re-read it, unused
      ls[j] = p.lse_part[sj * stride + row];
      const float *src = p.o_part + (sj * stride + row) * D + lane * PER;
#pragma unroll
      for (int c = 0; c < PER; ++c) v[j][c] = src[c];
    }
    float cm = M;
#pragma unroll
    for (int j = 0; j < CK; ++j)
      if (s0 + j < S) cm = fmaxf(cm, ls[j]);
    if (cm == kNegInf) continue;   // every split so far saw no key
    const float r = M == kNegInf ? 0.f : fast_exp2((M - cm) * kLog2e);
    total *= r;
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] *= r;
#pragma unroll
    for (int j = 0; j < CK; ++j) {
      if (s0 + j >= S || ls[j] == kNegInf) continue;   // a split that saw no key
      const float w = fast_exp2((ls[j] - cm) * kLog2e);
      total += w;
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] += w * v[j][c];
    }
    M = cm;
  }
  const bool empty = !(total > 0.f);
  const float inv = empty ? 0.f : 1.f / total;
  uint16_t *dst = p.out + row * D + lane * PER;
#pragma unroll
  for (int c = 0; c < PER; ++c) dst[c] = Elt<DT>::from_f32(acc[c] * inv);
  if (lane == 0) p.lse[row] = empty ? kNegInf : M + __builtin_logf(total);
}

}  // namespace pa
