"""GPU parity at the workloads' full sizes, in the launch configurations that
bench.py times, on sampled rows the oracle computes one token at a time.

For a sampled new token i of sequence b (q_len n, cache length L, K_b keys
visible to the call), the oracle gets that token's query rows alone, over the
sequence's first K_b - n + i + 1 keys (bottom-right causal alignment) laid
out as one contiguous sequence: cached keys are read from the pool before the
call through the sequence's page list, new keys straight from k_new.  So the
oracle shares nothing with the GPU's append or page walk.  The GPU call is
the whole call (append, heuristic split budget, combine); its appended slots
of the sampled sequences are checked bit-exactly against k_new / v_new.
Bars as in the other parity tests: max |out - oracle| <= 2e-3, |lse - oracle|
<= 1e-4 |oracle| + 1e-6.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_lds_amd as pa
import workloads as wl
from workloads import host, make_inputs

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_REL = 1e-4
LSE_ABS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    assert pa._lib() is not None


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def pages_of(inp, b, n_keys):
    """Physical page ids holding keys 0 .. n_keys-1 of sequence b."""
    P = inp.case.page_size
    return np.asarray(inp.pages_of[b][: -(-n_keys // P)], dtype=np.int64)


def cached_rows(inp, b, L):
    """K and V rows 0 .. L-1 of sequence b as [L, Hkv, D] uint16, read from the
    pool through its page list (paged) or its allocation (contiguous)."""
    if L == 0:
        shape = (0,) + tuple(inp.k_cache.shape[2:])
        return np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
    if inp.block_table is None:
        return host(inp.k_cache[b, :L]), host(inp.v_cache[b, :L])
    P = inp.case.page_size
    idx = torch.from_numpy(pages_of(inp, b, L)).to(inp.k_cache.device)
    k = host(inp.k_cache.index_select(0, idx)).reshape((-1,) + tuple(inp.k_cache.shape[2:]))
    v = host(inp.v_cache.index_select(0, idx)).reshape((-1,) + tuple(inp.v_cache.shape[2:]))
    return k[:L], v[:L]


def run_fullsize(case, samples, num_splits=0, max_seqlen_k=None, causal=None):
    """samples: {sequence: [token indices]}; one whole GPU call, then the
    oracle per sampled token."""
    say(f"case {case.name} seed {case.seed} (full size)")
    inp = make_inputs(case, "cuda")
    causal = case.causal if causal is None else causal
    cu = host(inp.cu_seqlens_q)
    # everything the oracle needs, taken before the call
    before = {b: cached_rows(inp, b, case.cache_seqlens[b]) for b in samples}
    qh = {b: host(inp.q[int(cu[b]):int(cu[b + 1])]) for b in samples}
    knh = {b: host(inp.k_new[int(cu[b]):int(cu[b + 1])]) for b in samples} if case.append else {}
    vnh = {b: host(inp.v_new[int(cu[b]):int(cu[b + 1])]) for b in samples} if case.append else {}
    say("  gpu call")
    out, lse = pa.paged_attn_fwd(
        inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q,
        max_seqlen_k=inp.max_seqlen_k if max_seqlen_k is None else max_seqlen_k,
        k_new=inp.k_new, v_new=inp.v_new, causal=causal, num_splits=num_splits)
    torch.cuda.synchronize()
    worst = 0.0
    for b, toks in samples.items():
        L = case.cache_seqlens[b]
        n = int(cu[b + 1] - cu[b])
        kb, vb = before[b]
        if case.append:
            # appended slots, bit for bit
            ka, va = cached_rows(inp, b, L + n)
            assert np.array_equal(ka[:L], kb) and np.array_equal(va[:L], vb), "cached rows changed"
            assert np.array_equal(ka[L:], knh[b]) and np.array_equal(va[L:], vnh[b]), \
                f"sequence {b}: appended rows differ"
            kb = np.concatenate([kb, knh[b]])
            vb = np.concatenate([vb, vnh[b]])
        K_b = L + (n if case.append else 0)
        for i in toks:
            vis = (K_b - n + i + 1) if causal else K_b
            vis = max(0, min(vis, K_b))
            kc = np.zeros((1, max(vis, 1)) + kb.shape[1:], np.uint16)
            vc = np.zeros((1, max(vis, 1)) + vb.shape[1:], np.uint16)
            kc[0, :vis] = kb[:vis]
            vc[0, :vis] = vb[:vis]
            ref_o, ref_l = oracle.attention(qh[b][i:i + 1], kc, vc, None, np.array([vis], np.int32),
                                            np.array([0, 1], np.int32), dtype=case.dtype,
                                            appended=False, causal=False)
            row = int(cu[b]) + i
            o = out[row].float().cpu().numpy().astype(np.float64)
            l = lse[row].cpu().numpy().astype(np.float64)
            err = np.abs(o - ref_o[0]).max()
            worst = max(worst, err)
            assert err <= OUT_TOL, f"seq {b} token {i}: out err {err}"
            fin = ~np.isneginf(ref_l[0])
            assert np.array_equal(np.isneginf(l), ~fin), f"seq {b} token {i}: -inf pattern"
            assert (np.abs(l[fin] - ref_l[0][fin]) <= LSE_REL * np.abs(ref_l[0][fin]) + LSE_ABS).all(), \
                f"seq {b} token {i}: lse"
    say(f"  max out err {worst:.3g}")
    del inp
    torch.cuda.empty_cache()


def test_mha_decode_b256_ctx4096_with_append():
    # the bench step: append one token per sequence, heuristic split budget
    c = wl.mha_decode(256, 4096, append=True)
    run_fullsize(c, {0: [0], 77: [0], 255: [0]}, causal=False)


@pytest.mark.parametrize("P", [16, 256])
def test_mha_decode_batch_sweep_corner(P):
    # the decode sweep's largest point at both page sizes (attention only)
    c = wl.mha_decode(256, 4096, page_size=P)
    run_fullsize(c, {3: [0], 200: [0]}, causal=False)


@pytest.mark.parametrize("batch", [12, 20])
def test_mha_decode_uneven_units_split_in_two(batch):
    # 384 and 640 one-head units (1.5 and 2.5 per compute unit of an MI355X):
    # the heuristic gives every key range two splits; the bench step's shape
    # otherwise (one appended token, 4096 cached)
    assert pa.paged_attn_num_splits(batch, batch, 32, 32, 128, 1, 4097, 256) == 2
    c = wl.mha_decode(batch, 4096, append=True)
    run_fullsize(c, {0: [0], batch // 2: [0], batch - 1: [0]}, causal=False)


def test_causal_prefill_gqa_bf16_4x2048():
    # grouped heads (32 q / 8 kv, four query heads packed per kv head, so a
    # 256-row unit covers 64 tokens) in bf16 (probabilities split into high
    # and low parts for the PV product), at the prefill bench size
    c = wl.Case(name="prefill_gqa_bf16", q_lens=[2048] * 4, cache_seqlens=[0, 100, 511, 2048],
                num_heads_q=32, num_heads_kv=8, head_dim=128, dtype="bf16", page_size=16,
                append=True, causal=True, seed=7103)
    run_fullsize(c, {0: [0, 63, 64, 2047], 2: [1000], 3: [0, 2047]})


def test_causal_prefill_d64_page256_4x2048():
    # head_dim 64 (waves 0-3 load a tile's K blocks, waves 4-7 its V blocks),
    # pages of 256 keys, cached prefixes of 0-511 keys, at the bench size
    c = wl.Case(name="prefill_d64_p256", q_lens=[2048] * 4, cache_seqlens=[0, 17, 256, 511],
                num_heads_q=16, num_heads_kv=16, head_dim=64, dtype="f16", page_size=256,
                append=True, causal=True, seed=7104)
    run_fullsize(c, {0: [0, 255, 256, 2047], 1: [1500], 3: [0, 2047]})


def test_causal_prefill_one_sequence_of_32768_tokens():
    # one 32768-token chunk with an empty cache, 32 heads x 128, fp16, page
    # 16, appended in the call: query tiles of up to 1024 key tiles
    c = wl.Case(name="prefill_32k", q_lens=[32768], cache_seqlens=[0], num_heads_q=32,
                num_heads_kv=32, head_dim=128, dtype="f16", page_size=16, append=True,
                causal=True, seed=7102)
    run_fullsize(c, {0: [0, 255, 256, 16383, 32766, 32767]})


def test_one_sequence_of_262144_keys():
    # one sequence at 262143 cached keys plus one appended, 64 q / 8 kv heads,
    # bf16, pages of 256: the one-sequence decode path with the heuristic's
    # split budget over a quarter-million keys
    c = wl.Case(name="one_seq_256k", q_lens=[1], cache_seqlens=[262143], num_heads_q=64,
                num_heads_kv=8, head_dim=128, dtype="bf16", page_size=256, append=True,
                causal=True, seed=7100)
    run_fullsize(c, {0: [0]})


def test_contiguous_allocation_at_the_2gib_limit():
    # contiguous allocations of 2^20 - 32 rows of 8 kv heads x 128 (2 GiB less
    # 64 KiB per sequence, under the 2^31-byte bound of 32-bit in-slab
    # offsets); the first sequence fills its allocation after the append
    alloc = (1 << 20) - 32
    c = wl.Case(name="contig_2gib", q_lens=[1, 1], cache_seqlens=[alloc - 1, 1000], num_heads_q=8,
                num_heads_kv=8, head_dim=128, dtype="f16", page_size=None, contig_alloc=alloc,
                append=True, causal=True, seed=7101)
    run_fullsize(c, {0: [0], 1: [0]})


@pytest.mark.parametrize("paged", [True, False])
def test_gqa_long_split_allocation_bound(paged):
    # batch 8, 64/8 heads, lengths in [2048, 32768] inside a 131072-token
    # allocation; heuristic split budget from the allocation bound
    c = wl.gqa_long_split(paged=paged)
    longest = int(np.argmax(c.cache_seqlens))
    run_fullsize(c, {longest: [0], 0: [0]})


@pytest.mark.parametrize("prefix", ["zero", "uniform"])
def test_causal_prefill_4x2048(prefix):
    c = wl.causal_prefill_append(2048, prefix)
    run_fullsize(c, {0: [0, 255, 256, 1000, 2047], 3: [31, 2046]})


def test_causal_prefill_4x170():
    c = wl.causal_prefill_append(170, "uniform")
    run_fullsize(c, {1: [0, 100, 169]})


@pytest.mark.parametrize("prefix", ["zero", "uniform"])
def test_causal_prefill_4x8192(prefix):
    # the "and beyond" prefill size the prefill sweep times: early, middle and
    # late rows, and both sides of two 256-row unit boundaries in sequence 0
    c = wl.causal_prefill_append(8192, prefix)
    run_fullsize(c, {0: [0, 255, 256, 4095, 4096, 8191], 2: [5000], 3: [31, 8190]})


def sharp(c, seed_offset=77):
    """The same shapes with q and keys ~ 3 N(0, 1): scores spread over tens of
    units, so the softmax is dominated by a few keys and every rescaling path
    of the kernels (running maximum, reference moves, bounded sums) is taken."""
    return wl.Case(**{**c.__dict__, "values": "normal3", "seed": c.seed + seed_offset,
                      "name": c.name + "_normal3"})


@pytest.mark.parametrize("nq,prefix", [(2048, "zero"), (2048, "uniform"), (8192, "zero")])
def test_causal_prefill_sharp_softmax_full_size(nq, prefix):
    c = sharp(wl.causal_prefill_append(nq, prefix))
    last = nq - 1
    run_fullsize(c, {0: [0, 1, 300, nq // 2, last], 1: [last - 1], 3: [257, last]})


@pytest.mark.parametrize("paged", [True, False])
def test_gqa_long_split_sharp_softmax_full_size(paged):
    c = sharp(wl.gqa_long_split(paged=paged))
    run_fullsize(c, {b: [0] for b in range(c.batch)})


def run_every_sequence(case, chunk=16):
    """One whole GPU call, then EVERY sequence's rows against the oracle, in
    chunks: the pools are copied on the GPU before the call; per chunk the
    sequences' pages are gathered from that copy into a compact pool with a
    fresh table, and the oracle appends and attends on it by itself."""
    say(f"case {case.name} seed {case.seed} (full size, every sequence)")
    inp = make_inputs(case, "cuda")
    k0, v0 = inp.k_cache.clone(), inp.v_cache.clone()
    cu = host(inp.cu_seqlens_q)
    say("  gpu call")
    out, lse = pa.paged_attn_fwd(
        inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new,
        v_new=inp.v_new, causal=case.causal)
    torch.cuda.synchronize()
    P = case.page_size
    worst = 0.0
    for c0 in range(0, case.batch, chunk):
        bs = list(range(c0, min(case.batch, c0 + chunk)))
        pages = [np.asarray(inp.pages_of[b], np.int64) for b in bs]
        idx = torch.from_numpy(np.concatenate(pages)).to("cuda")
        kc, vc = host(k0.index_select(0, idx)), host(v0.index_select(0, idx))
        width = max(len(p) for p in pages)
        table = np.full((len(bs), width), -1, np.int32)
        off = 0
        for i, p in enumerate(pages):
            table[i, :len(p)] = np.arange(off, off + len(p))
            off += len(p)
        r0, r1 = int(cu[bs[0]]), int(cu[bs[-1] + 1])
        cu_c = (cu[bs[0]:bs[-1] + 2] - cu[bs[0]]).astype(np.int32)
        seq = np.asarray([case.cache_seqlens[b] for b in bs], np.int32)
        kn = host(inp.k_new[r0:r1]) if case.append else None
        vn = host(inp.v_new[r0:r1]) if case.append else None
        ref_o, ref_l, ref_kc, ref_vc = oracle.paged_attention(
            host(inp.q[r0:r1]), kc, vc, table, seq, cu_c, kn, vn, dtype=case.dtype,
            causal=case.causal)
        o = out[r0:r1].float().cpu().numpy().astype(np.float64)
        l = lse[r0:r1].cpu().numpy().astype(np.float64)
        err = np.abs(o - ref_o).max()
        worst = max(worst, err)
        assert err <= OUT_TOL, f"sequences {bs[0]}..{bs[-1]}: out err {err}"
        fin = ~np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(l), ~fin), f"sequences {bs[0]}..{bs[-1]}: -inf pattern"
        assert (np.abs(l[fin] - ref_l[fin]) <= LSE_REL * np.abs(ref_l[fin]) + LSE_ABS).all(), \
            f"sequences {bs[0]}..{bs[-1]}: lse"
        if case.append:
            # the pages after the call hold what the oracle's own append wrote
            kg = host(inp.k_cache.index_select(0, idx))
            vg = host(inp.v_cache.index_select(0, idx))
            for i, b in enumerate(bs):
                rows = np.arange(table[i, 0] * P, table[i, 0] * P + len(pages[i]) * P)
                K_b = case.cache_seqlens[b] + case.q_lens[b]
                a = kg.reshape((-1,) + kg.shape[2:])[rows[:K_b]]
                e = ref_kc.reshape((-1,) + ref_kc.shape[2:])[rows[:K_b]]
                assert np.array_equal(a, e), f"sequence {b}: K pages after the call"
                a = vg.reshape((-1,) + vg.shape[2:])[rows[:K_b]]
                e = ref_vc.reshape((-1,) + ref_vc.shape[2:])[rows[:K_b]]
                assert np.array_equal(a, e), f"sequence {b}: V pages after the call"
    say(f"  {case.batch} sequences, max out err {worst:.3g}")
    del inp, k0, v0
    torch.cuda.empty_cache()


def test_mha_decode_b256_ctx4096_every_sequence():
    # the bench step (append one token, heuristic budget), all 256 x 32 rows
    run_every_sequence(wl.mha_decode(256, 4096, append=True))


@pytest.mark.parametrize("nq,heads,hd", [(100, 32, 128), (500, 32, 128), (1000, 32, 128),
                                         (100, 12, 64), (1000, 12, 64)])
def test_unified_varlen_full(nq, heads, hd):
    c = wl.unified_varlen(nq, heads=heads, head_dim=hd)
    run_fullsize(c, {0: [0, nq // 2, nq - 1], 1: [0], 40: [0], 64: [0]})
