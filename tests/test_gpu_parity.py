"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Bars (the same in every test):
  * cache contents after append: bit-exact;
  * out: max |gpu - oracle| <= 2e-3 (oracle unrounded fp64);
  * softmax_lse: |gpu - oracle| <= 1e-4 * |oracle| + 1e-6 (the additive 1e-6 is
    the fp32 floor for lse values near zero); -inf exactly where the oracle has
    -inf;
  * invariants that hold by construction of the kernels (page size, page
    relabelling, poisoned table tails, GQA packing) are checked bit-exactly.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_lds_amd as pa
import workloads as wl
from workloads import Case, host, make_inputs

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


def gpu_call(inp, num_splits=None, stream=None, **kw):
    c = inp.case
    out, lse = pa.paged_attn_fwd(
        inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=kw.pop("max_seqlen_k", inp.max_seqlen_k),
        k_new=inp.k_new, v_new=inp.v_new, causal=c.causal,
        num_splits=c.num_splits if num_splits is None else num_splits, stream=stream, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_call(inp, kc_host, vc_host):
    c = inp.case
    return oracle.paged_attention(host(inp.q), kc_host, vc_host, host(inp.block_table),
                                  host(inp.cache_seqlens), host(inp.cu_seqlens_q),
                                  host(inp.k_new), host(inp.v_new), dtype=c.dtype,
                                  causal=c.causal)


def check_against_oracle(out, lse, ref_out, ref_lse, what=""):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    err = np.abs(o - ref_out).max(initial=0.0)
    assert err <= OUT_TOL, f"{what}: out max abs err {err}"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), ninf), f"{what}: -inf pattern differs"
    fin = ~ninf
    if fin.any():
        lerr = np.abs(l[fin] - ref_lse[fin]) - (LSE_REL * np.abs(ref_lse[fin]) + LSE_ABS)
        assert lerr.max() <= 0, f"{what}: lse err over bound by {lerr.max()}"
    return err


def run_parity(case, splits=(None,), check_pools=True):
    say(f"case {case.name} seed {case.seed}")
    inp = make_inputs(case, "cuda")
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    ref_out, ref_lse, ref_kc, ref_vc = oracle_call(inp, kc0, vc0)
    errs = []
    for s in splits:
        # restore the pools so every call appends onto the same starting state
        inp.k_cache.copy_(torch.from_numpy(kc0.view(np.int16)).view(inp.k_cache.dtype))
        inp.v_cache.copy_(torch.from_numpy(vc0.view(np.int16)).view(inp.v_cache.dtype))
        say(f"  gpu call num_splits={s}")
        out, lse = gpu_call(inp, num_splits=s)
        errs.append(check_against_oracle(out, lse, ref_out, ref_lse, f"{case.name} S={s}"))
        if check_pools and case.append:
            assert np.array_equal(host(inp.k_cache), ref_kc), "k_cache after append differs"
            assert np.array_equal(host(inp.v_cache), ref_vc), "v_cache after append differs"
    return inp, errs


# ---------------------------------------------------------------------------
# The five workload families at oracle-sized points.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("poison", ["neg1", "intmax"])
def test_tiny_decode(poison):
    run_parity(wl.tiny_decode(poison=poison), splits=(0, 1, 2, 3, 7))


@pytest.mark.parametrize("batch,ctx,P", [(1, 512, 16), (3, 1000, 16), (4, 515, 256), (2, 17, 16),
                                         (5, 1, 32), (2, 2048, 64)])
def test_mha_decode(batch, ctx, P):
    run_parity(wl.mha_decode(batch, ctx, page_size=P), splits=(None, 1, 3))


def test_mha_decode_with_one_token_append():
    run_parity(wl.mha_decode(4, 700, append=True))


def reduced_gqa(paged=True, values="uniform01", seed=2100):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(100, 3000, 8, endpoint=True)]
    return Case(name="gqa_split" + ("_paged" if paged else "_contig"), q_lens=[1] * 8,
                cache_seqlens=lens, num_heads_q=64, num_heads_kv=8, head_dim=128, dtype="bf16",
                page_size=16 if paged else None, contig_alloc=0 if paged else 4096,
                table_width=4096 // 16 if paged else None, causal=True, values=values, seed=seed,
                max_seqlen_k_hint=4096)


@pytest.mark.parametrize("paged", [True, False])
def test_gqa_split_sweep(paged):
    run_parity(reduced_gqa(paged), splits=(None, 1, 2, 4, 8, 16, 32, 64, 128))


@pytest.mark.parametrize("lo,hi", [(1, 300), (64, 512)])
def test_gqa_short_lengths_in_a_large_allocation(lo, hi):
    # live lengths far below the 131072-token allocation the host sizes from:
    # the device keeps every split at >= 8 key tiles, so forced budgets far
    # above what the keys can use leave units empty instead of near-empty
    rng = np.random.default_rng(2400 + lo)
    lens = [int(x) for x in rng.integers(lo, hi, 8, endpoint=True)]
    c = Case(name=f"gqa_short_{lo}_{hi}", q_lens=[1] * 8, cache_seqlens=lens, num_heads_q=64,
             num_heads_kv=8, head_dim=128, dtype="bf16", page_size=16, table_width=131072 // 16,
             causal=True, seed=2400 + lo, max_seqlen_k_hint=131072)
    run_parity(c, splits=(None, 1, 8, 32, 128))


def test_gqa_split_sharp_softmax():
    run_parity(reduced_gqa(True, values="normal3", seed=2200), splits=(None, 1, 5))


@pytest.mark.parametrize("nq,prefix", [(170, "zero"), (170, "uniform"), (33, "uniform")])
def test_causal_prefill_append(nq, prefix):
    run_parity(wl.causal_prefill_append(nq, prefix))


@pytest.mark.parametrize("dtype,P,hq,hkv,hd,prefix", [
    ("bf16", 16, 32, 32, 128, "uniform"),     # bf16 prefill (probabilities as hi + lo)
    ("f16", 256, 32, 32, 128, "uniform"),     # one page holds a whole tile row range
    ("f16", None, 32, 32, 128, "uniform"),    # contiguous cache
    ("bf16", 16, 64, 8, 128, "uniform"),      # GQA prefill: 8 q heads per kv head
    ("f16", 16, 12, 12, 64, "zero"),          # head_dim 64 prefill
    ("bf16", 32, 48, 16, 64, "uniform"),      # GQA group 3: a token's rows straddle units
])
def test_causal_prefill_variants(dtype, P, hq, hkv, hd, prefix):
    rng = np.random.default_rng(3100 + hq + hd)
    L = [0] * 3 if prefix == "zero" else [int(x) for x in rng.integers(0, 300, 3, endpoint=True)]
    nq = [130, 77, 301]
    c = Case(name=f"prefill_{dtype}_P{P}_{hq}x{hkv}x{hd}", q_lens=nq, cache_seqlens=L,
             num_heads_q=hq, num_heads_kv=hkv, head_dim=hd, dtype=dtype, page_size=P,
             contig_alloc=0 if P else max(a + b for a, b in zip(L, nq)) + 5, append=True,
             causal=True, seed=3100 + hq + hd)
    run_parity(c)


@pytest.mark.parametrize("kind", ["prefill", "unified", "decode"])
def test_non_causal_and_softmax_scale(kind):
    # non-causal attention over every key (new rows included) and a caller
    # softmax scale, through each kernel
    if kind == "prefill":
        c = Case(name="noncausal_prefill", q_lens=[130, 40], cache_seqlens=[50, 260], num_heads_q=16,
                 num_heads_kv=4, head_dim=128, dtype="f16", page_size=16, append=True,
                 causal=False, seed=3300)
    elif kind == "unified":
        c = Case(name="noncausal_unified", q_lens=[90, 1, 1, 3], cache_seqlens=[17, 400, 0, 33],
                 num_heads_q=8, num_heads_kv=8, head_dim=64, dtype="bf16", page_size=32,
                 append=True, causal=False, seed=3301)
    else:
        c = Case(name="noncausal_decode", q_lens=[2, 1, 4], cache_seqlens=[300, 45, 1000],
                 num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="f16", page_size=16,
                 append=True, causal=False, seed=3302)
    say(f"case {c.name} seed {c.seed}")
    inp = make_inputs(c, "cuda")
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    scale = 0.37
    ref_out, ref_lse, ref_kc, ref_vc = oracle.paged_attention(
        host(inp.q), kc0, vc0, host(inp.block_table), host(inp.cache_seqlens),
        host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new), dtype=c.dtype, causal=False,
        scale=scale)
    for s in (None, 3):
        inp.k_cache.copy_(torch.from_numpy(kc0.view(np.int16)).view(inp.k_cache.dtype))
        inp.v_cache.copy_(torch.from_numpy(vc0.view(np.int16)).view(inp.v_cache.dtype))
        out, lse = gpu_call(inp, num_splits=s, softmax_scale=scale)
        check_against_oracle(out, lse, ref_out, ref_lse, f"{c.name} S={s}")
        assert np.array_equal(host(inp.k_cache), ref_kc) and np.array_equal(host(inp.v_cache), ref_vc)


def test_causal_prefill_sharp_softmax():
    c = wl.causal_prefill_append(100, "uniform")
    c.values = "normal3"
    run_parity(c)


@pytest.mark.parametrize("nq,heads,hd", [(100, 32, 128), (500, 32, 128), (100, 12, 64),
                                         (1000, 12, 64)])
def test_unified_varlen(nq, heads, hd):
    run_parity(wl.unified_varlen(nq, heads=heads, head_dim=hd), splits=(None, 2))


@pytest.mark.parametrize("q_len,hq,hkv,dtype", [(2, 32, 32, "f16"), (7, 32, 32, "f16"),
                                                (16, 32, 32, "f16"), (2, 64, 8, "bf16")])
def test_multi_token_decode(q_len, hq, hkv, dtype):
    # q_len new tokens per sequence, q_len * G <= 16 packed rows: one decode unit
    # per (sequence, split), causal over the appended tokens
    c = wl.multi_token_decode(3, 700, q_len, heads_q=hq, heads_kv=hkv, dtype=dtype)
    c.cache_seqlens = [700, 41, 1500]
    run_parity(c, splits=(None, 3))


def test_unified_varlen_with_prefix():
    run_parity(wl.unified_varlen(300, prefix=777))


# A batch that can mix decode-mode and prefill-mode sequences runs as two
# launches on the call's stream (prefill units, then decode units); with a
# second stream the two run concurrently (decode units on aux_stream); with
# PAGED_ATTN_SINGLE_KERNEL=1 it is one unified launch.  Every plan runs the
# same unit code, so they must agree bit for bit, and the one-launch plan
# keeps its oracle parity.
@pytest.mark.parametrize("nq,heads,hd", [(100, 32, 128), (1000, 12, 64)])
def test_unified_varlen_one_launch(nq, heads, hd, monkeypatch):
    monkeypatch.setenv("PAGED_ATTN_SINGLE_KERNEL", "1")
    run_parity(wl.unified_varlen(nq, heads=heads, head_dim=hd), splits=(None, 2))


@pytest.mark.parametrize("case", [wl.unified_varlen(300, prefix=777),
                                  wl.unified_varlen(100, heads=12, head_dim=64),
                                  wl.multi_token_decode(3, 700, 2)],
                         ids=lambda c: c.name)
def test_mixed_batch_plans_agree(case, monkeypatch):
    if case.name.startswith("multi_token"):
        # one prefill-mode sequence among decode-mode ones
        case.q_lens = [2, 40, 2]
    say(f"case {case.name} seed {case.seed}")
    inp = make_inputs(case, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    for s in (None, 2):
        got = {}
        for plan in ("sequential", "concurrent", "one"):
            inp.k_cache.copy_(kc0)
            inp.v_cache.copy_(vc0)
            if plan == "one":
                monkeypatch.setenv("PAGED_ATTN_SINGLE_KERNEL", "1")
            out, lse = gpu_call(inp, num_splits=s,
                                aux_stream="auto" if plan == "concurrent" else None)
            monkeypatch.delenv("PAGED_ATTN_SINGLE_KERNEL", raising=False)
            got[plan] = (out.clone(), lse.clone(), inp.k_cache.clone(), inp.v_cache.clone())
        for other in ("concurrent", "one"):
            for name, a, b in zip(("out", "lse", "k_cache", "v_cache"), got["sequential"],
                                  got[other]):
                bits = torch.int16 if a.element_size() == 2 else torch.int32
                assert torch.equal(a.view(bits), b.view(bits)), \
                    f"{case.name} S={s}: {name} differs between the sequential and {other} plans"


# ---------------------------------------------------------------------------
# Invariants that the kernels guarantee bit-exactly.
# ---------------------------------------------------------------------------

def _same_logical(case_a, case_b):
    """Two inputs holding the same logical data in different physical layouts."""
    a = make_inputs(case_a, "cuda")
    b = make_inputs(case_b, "cuda")
    return a, b


def _copy_logical(src, dst):
    """Copy every sequence's keys/values and q/k_new/v_new from src to dst."""
    P_s = src.case.page_size
    P_d = dst.case.page_size
    Kb = src.case.keys_visible()
    for bb, K in enumerate(Kb):
        L = src.case.cache_seqlens[bb]
        for j0 in range(0, L, 16):
            n = min(16, L - j0)
            for j in range(j0, j0 + n):
                if P_s is None:
                    ks, vs = src.k_cache[bb, j], src.v_cache[bb, j]
                else:
                    pg = int(src.pages_of[bb][j // P_s])
                    ks, vs = src.k_cache[pg, j % P_s], src.v_cache[pg, j % P_s]
                if P_d is None:
                    dst.k_cache[bb, j].copy_(ks)
                    dst.v_cache[bb, j].copy_(vs)
                else:
                    pg = int(dst.pages_of[bb][j // P_d])
                    dst.k_cache[pg, j % P_d].copy_(ks)
                    dst.v_cache[pg, j % P_d].copy_(vs)
    dst.q.copy_(src.q)
    if src.k_new is not None:
        dst.k_new.copy_(src.k_new)
        dst.v_new.copy_(src.v_new)


@pytest.mark.parametrize("splits", [1, 3])
def test_page_size_and_contiguous_bit_identical(splits):
    base = dict(q_lens=[1, 5, 1], cache_seqlens=[100, 37, 300], num_heads_q=8, num_heads_kv=2,
                head_dim=128, dtype="f16", append=True, causal=True, seed=77, num_splits=splits)
    say("page-size invariance")
    ref = make_inputs(Case(name="p16", page_size=16, **base), "cuda")
    o_ref, l_ref = gpu_call(ref)
    for P in (32, 64, 128, 256, None):
        c = Case(name=f"p{P}", page_size=P, contig_alloc=400 if P is None else 0, **base)
        other = make_inputs(c, "cuda")
        # re-create ref's starting pools: regenerate to undo its append
        ref0 = make_inputs(Case(name="p16", page_size=16, **base), "cuda")
        _copy_logical(ref0, other)
        o, l = gpu_call(other)
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), f"P={P} differs"


def test_page_relabelling_bit_identical():
    c = wl.causal_prefill_append(40, "uniform")
    a = make_inputs(c, "cuda")
    b = make_inputs(c, "cuda")
    n = a.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5)).cuda()
    b.k_cache[perm] = a.k_cache
    b.v_cache[perm] = a.v_cache
    t = a.block_table.clone()
    live = t >= 0
    t[live] = perm.int()[t[live].long()]
    b.block_table = t
    oa, la = gpu_call(a)
    ob, lb = gpu_call(b)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(b.k_cache[perm], a.k_cache) and torch.equal(b.v_cache[perm], a.v_cache)


def test_poisoned_tails_bit_identical():
    outs = []
    for poison in ("neg1", "intmax", "big", "zero"):
        inp = make_inputs(wl.tiny_decode(num_splits=3, poison=poison), "cuda")
        outs.append(gpu_call(inp))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_gqa_equals_mha_with_repeated_kv_bit_identical():
    # every sequence is a decode unit on both sides (GQA packs 8 q heads x up to
    # 2 tokens = 16 rows; MHA has 1-2 rows per kv head), so both get the same
    # length-proportional split counts and the per-row arithmetic is identical
    G = 8
    c = Case(name="gqa", q_lens=[1, 1, 2], cache_seqlens=[300, 55, 1000], num_heads_q=16,
             num_heads_kv=2, head_dim=128, dtype="bf16", page_size=16, causal=True, seed=99,
             num_splits=2)
    a = make_inputs(c, "cuda")
    m = make_inputs(Case(**{**c.__dict__, "name": "mha", "num_heads_kv": 16}), "cuda")
    m.k_cache.copy_(a.k_cache.repeat_interleave(G, dim=2))
    m.v_cache.copy_(a.v_cache.repeat_interleave(G, dim=2))
    m.q.copy_(a.q)
    m.block_table.copy_(a.block_table)
    oa, la = gpu_call(a)
    om, lm = gpu_call(m)
    assert torch.equal(oa, om) and torch.equal(la, lm)


def test_varlen_equals_one_call_per_sequence():
    c = wl.unified_varlen(120, heads=12, head_dim=64)
    c.q_lens = c.q_lens[:9]
    c.cache_seqlens = c.cache_seqlens[:9]
    inp = make_inputs(c, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    out, lse = gpu_call(inp, num_splits=1)
    cu = inp.cu_seqlens_q.cpu().tolist()
    for b in range(c.batch):
        inp.k_cache.copy_(kc0)
        inp.v_cache.copy_(vc0)
        s, e = cu[b], cu[b + 1]
        o1, l1 = pa.paged_attn_fwd(
            inp.q[s:e].contiguous(), inp.k_cache, inp.v_cache, inp.block_table[b:b + 1].contiguous(),
            inp.cache_seqlens[b:b + 1].contiguous(),
            torch.tensor([0, e - s], dtype=torch.int32, device="cuda"), max_seqlen_q=e - s,
            k_new=inp.k_new[s:e].contiguous(), v_new=inp.v_new[s:e].contiguous(), causal=True,
            num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o1, out[s:e]) and torch.equal(l1, lse[s:e]), f"sequence {b}"


@pytest.mark.parametrize("batch", [40, 1024, 1030])
def test_decode_varlen_unit_order(batch, monkeypatch):
    # decode-only batches with one unit per sequence run their units longest
    # first (up to 1024 sequences; index order past that): unsorted lengths
    # with ties and (0, 0) padding slots; results must not depend on the order
    rng = np.random.default_rng(5200 + batch)
    lens = [int(x) for x in rng.integers(0, 400, batch)]
    lens[3] = lens[7] = lens[11] = 250                      # ties
    q_lens = [1] * batch
    for i in (5, batch - 2):                                # padding slots
        q_lens[i], lens[i] = 0, 0
    c = Case(name=f"decode_varlen_order_b{batch}", q_lens=q_lens, cache_seqlens=lens,
             num_heads_q=8, num_heads_kv=2, head_dim=64, dtype="f16", page_size=16, append=True,
             causal=True, seed=5200 + batch)
    inp, _ = run_parity(c, splits=(1,))
    kc_after, vc_after = inp.k_cache.clone(), inp.v_cache.clone()
    cu = inp.cu_seqlens_q.cpu().tolist()
    seq_after = (inp.cache_seqlens + torch.tensor(q_lens, dtype=torch.int32, device="cuda")).contiguous()

    def whole(order):
        """The batch with its sequences in `order` (a permutation): per-sequence results."""
        q = torch.cat([inp.q[cu[b]:cu[b + 1]] for b in order])
        cu_o = torch.tensor(np.concatenate([[0], np.cumsum([q_lens[b] for b in order])]),
                            dtype=torch.int32, device="cuda")
        o, l = pa.paged_attn_fwd(q, kc_after, vc_after, inp.block_table[order].contiguous(),
                                 seq_after[order].contiguous(), cu_o, max_seqlen_q=1, causal=True,
                                 num_splits=1)
        torch.cuda.synchronize()
        cu_h = cu_o.cpu().tolist()
        return {b: (o[cu_h[i]:cu_h[i + 1]], l[cu_h[i]:cu_h[i + 1]]) for i, b in enumerate(order)}

    # the batch in reverse order runs its units in another order (and, at 1024
    # sequences and more x 2 kv heads, as pair units): the same bits
    fwd, rev = whole(list(range(batch))), whole(list(range(batch))[::-1])
    for b in range(batch):
        assert torch.equal(fwd[b][0], rev[b][0]) and torch.equal(fwd[b][1], rev[b][1]), f"seq {b}"
    # bit-exact against calls over a few single sequences, one-head units in both
    monkeypatch.setenv("PAGED_ATTN_HEAD_PAIRS", "0")
    full_out, full_lse = pa.paged_attn_fwd(inp.q, kc_after, vc_after, inp.block_table, seq_after,
                                           inp.cu_seqlens_q, max_seqlen_q=1, causal=True, num_splits=1)
    torch.cuda.synchronize()
    for b in (0, 3, 7, int(np.argmax(lens)), batch - 1):
        s_, e_ = cu[b], cu[b + 1]
        if e_ == s_:
            continue
        o1, l1 = pa.paged_attn_fwd(
            inp.q[s_:e_].contiguous(), kc_after, vc_after, inp.block_table[b:b + 1].contiguous(),
            seq_after[b:b + 1].contiguous(), torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
            max_seqlen_q=1, causal=True, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o1, full_out[s_:e_]) and torch.equal(l1, full_lse[s_:e_]), f"sequence {b}"


@pytest.mark.parametrize("nq,hq,hkv,hd,dtype,P", [
    (300, 48, 16, 64, "bf16", 32),     # group 3: a token's rows straddle query tiles
    (1000, 32, 32, 128, "f16", None),  # contiguous cache
    (5, 64, 8, 128, "bf16", 16),       # 40 rows: one query tile per sequence
])
def test_equal_query_lengths_map_like_the_search(nq, hq, hkv, hd, dtype, P, monkeypatch):
    # with every sequence at max_seqlen_q new tokens the unified kernel maps
    # its prefill units by block index instead of searching the metadata: the
    # bits must be those of the searched mapping (and the oracle's to the bar)
    rng = np.random.default_rng(5400 + nq)
    lens = [nq + int(x) for x in rng.integers(0, 600, 5)]   # every query row sees keys
    c = Case(name=f"equal_q_{nq}_{hq}x{hkv}x{hd}", q_lens=[nq] * 5, cache_seqlens=lens,
             num_heads_q=hq, num_heads_kv=hkv, head_dim=hd, dtype=dtype, page_size=P,
             contig_alloc=0 if P else 2048, append=False, causal=True, seed=5400 + nq)
    inp, _ = run_parity(c)
    direct = gpu_call(inp)
    monkeypatch.setenv("PAGED_ATTN_FULL_SEARCH", "1")
    searched = gpu_call(inp)
    assert torch.equal(direct[0], searched[0]) and torch.equal(direct[1], searched[1])


def test_single_sequence_decode_matches_a_padded_batch():
    # a one-sequence decode batch maps its splits by block index (no unit
    # search); the same sequence beside a (0, 0) padding slot goes through the
    # search with the same budget per decode sequence: the same bits
    rng = np.random.default_rng(5500)
    for ctx in (1, 300, 513, 4097):
        c = Case(name=f"single_seq_{ctx}", q_lens=[1, 0], cache_seqlens=[ctx, 0], num_heads_q=32,
                 num_heads_kv=8, head_dim=128, dtype="bf16", page_size=16, append=True,
                 causal=True, seed=int(rng.integers(1 << 30)))
        inp = make_inputs(c, "cuda")
        kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
        for s in (1, 2, 3, 8, 64):
            say(f"  ctx {ctx} num_splits {s}")
            inp.k_cache.copy_(kc0); inp.v_cache.copy_(vc0)
            two = gpu_call(inp, num_splits=s)
            inp.k_cache.copy_(kc0); inp.v_cache.copy_(vc0)
            one = pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table[:1].contiguous(),
                                    inp.cache_seqlens[:1].contiguous(), inp.cu_seqlens_q[:2].contiguous(),
                                    max_seqlen_q=1, k_new=inp.k_new, v_new=inp.v_new, causal=True,
                                    num_splits=s)
            torch.cuda.synchronize()
            assert torch.equal(one[0], two[0]) and torch.equal(one[1], two[1]), f"ctx {ctx} S {s}"
        ref_out, ref_lse, _, _ = oracle_call(inp, host(kc0), host(vc0))
        check_against_oracle(one[0], one[1], ref_out, ref_lse, f"single sequence ctx {ctx}")


@pytest.mark.parametrize("splits", [1, 2, 4, 16])
def test_few_sequence_search_matches_the_block_search(splits, monkeypatch):
    # up to 64 sequences, the decode kernel finds its units in one wave; with
    # PAGED_ATTN_FULL_SEARCH=1 the workgroup-wide search runs instead: the
    # same units and split counts, so the same bits (unsorted lengths with
    # ties, a q_len-0 slot inside)
    rng = np.random.default_rng(5600 + splits)
    lens = [int(x) for x in rng.integers(0, 3000, 40)]
    lens[5] = lens[9] = lens[30] = 1500                     # ties
    q_lens = [1] * 40
    q_lens[12], lens[12] = 0, 0                               # a padding slot inside
    c = Case(name=f"few_seq_search_S{splits}", q_lens=q_lens, cache_seqlens=lens, num_heads_q=32,
             num_heads_kv=8, head_dim=128, dtype="f16", page_size=16, append=False, causal=True,
             num_splits=splits, seed=5600 + splits)
    inp, _ = run_parity(c, splits=(splits,))
    wave = gpu_call(inp, num_splits=splits)
    monkeypatch.setenv("PAGED_ATTN_FULL_SEARCH", "1")
    block = gpu_call(inp, num_splits=splits)
    assert torch.equal(wave[0], block[0]) and torch.equal(wave[1], block[1])


def test_zero_length_padding_slots():
    c = wl.unified_varlen(50, heads=12, head_dim=64)
    c.q_lens = c.q_lens[:5]
    c.cache_seqlens = c.cache_seqlens[:5]
    inp = make_inputs(c, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    out, lse = gpu_call(inp, num_splits=2)
    kc1, vc1 = inp.k_cache.clone(), inp.v_cache.clone()
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    pad = 4
    cu = torch.cat([inp.cu_seqlens_q, inp.cu_seqlens_q[-1:].repeat(pad)])
    seq = torch.cat([inp.cache_seqlens, torch.zeros(pad, dtype=torch.int32, device="cuda")])
    bt = torch.cat([inp.block_table, torch.full((pad, inp.block_table.shape[1]), -1,
                                                dtype=torch.int32, device="cuda")])
    o2, l2 = pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, bt, seq, cu,
                               max_seqlen_q=inp.max_seqlen_q, k_new=inp.k_new, v_new=inp.v_new,
                               causal=True, num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(o2, out) and torch.equal(l2, lse)
    assert torch.equal(inp.k_cache, kc1) and torch.equal(inp.v_cache, vc1)


def test_empty_cache_without_append_gives_zero_and_neg_inf():
    c = Case(name="empty", q_lens=[1, 2], cache_seqlens=[0, 5], num_heads_q=4, num_heads_kv=4,
             head_dim=64, page_size=16, causal=True, seed=3, num_pages=8, table_width=2)
    inp = make_inputs(c, "cuda")
    out, lse = gpu_call(inp)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    # causal, 2 new tokens over 5 keys: both rows see keys
    assert torch.all(torch.isfinite(lse[1:]))
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    ref_out, ref_lse, _, _ = oracle_call(inp, kc0, vc0)
    check_against_oracle(out, lse, ref_out, ref_lse, "empty")


def test_single_visible_key_is_exact():
    # first causal row of a fresh sequence sees only key 0: out == v_0 bit-exactly
    c = Case(name="first_row", q_lens=[5, 1], cache_seqlens=[0, 0], num_heads_q=4, num_heads_kv=2,
             head_dim=128, dtype="bf16", page_size=16, append=True, causal=True, seed=8)
    inp = make_inputs(c, "cuda")
    out, lse = gpu_call(inp)
    assert torch.equal(out[0], inp.v_new[0].repeat_interleave(2, dim=0))
    assert torch.equal(out[5], inp.v_new[5].repeat_interleave(2, dim=0))


def test_append_only_entry_point_bit_exact():
    c = wl.causal_prefill_append(70, "uniform")
    inp = make_inputs(c, "cuda")
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    pa.paged_kv_append(inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                       inp.cu_seqlens_q, inp.k_new, inp.v_new, max_seqlen_q=inp.max_seqlen_q)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_append(kc0, vc0, host(inp.block_table), host(inp.cache_seqlens),
                              host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new))
    assert np.array_equal(host(inp.k_cache), ek) and np.array_equal(host(inp.v_cache), ev)


@pytest.mark.parametrize("P", [16, 32])
def test_every_tail_position_of_a_tile(P):
    # cache lengths 1..40: the visible range ends at every key of a 32-key tile,
    # including inside the upper half that starts a second 16-key page
    n = 40
    c = Case(name=f"tails_p{P}", q_lens=[1] * n, cache_seqlens=list(range(1, n + 1)),
             num_heads_q=8, num_heads_kv=2, head_dim=128, dtype="f16", page_size=P,
             causal=False, seed=41 + P)
    run_parity(c, splits=(1, 2, None))
    c2 = Case(**{**c.__dict__, "name": f"tails_append_p{P}", "append": True, "causal": True,
                 "q_lens": [1, 2] * (n // 2), "head_dim": 64, "dtype": "bf16"})
    run_parity(c2, splits=(1, None))


@pytest.mark.parametrize("aux", [None, "auto"])
def test_mixed_batch_on_a_user_stream(aux):
    # a mixed batch queued on a stream of the caller's (both plans: two
    # launches on that stream, or forked onto a second one and joined back):
    # work queued on that stream right after the call (no synchronisation)
    # sees the whole result, which equals the same call on the default stream
    # bit for bit
    c = wl.unified_varlen(100, heads=8, head_dim=128)
    say(f"case {c.name} seed {c.seed} on a user stream")
    inp = make_inputs(c, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    ref_out, ref_lse = gpu_call(inp)
    ref_kc, ref_vc = inp.k_cache.clone(), inp.v_cache.clone()
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, lse = pa.paged_attn_fwd(
            inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
            max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new,
            v_new=inp.v_new, causal=c.causal, stream=s, aux_stream=aux)
        out_copy, lse_copy = out.clone(), lse.clone()
        kc_copy, vc_copy = inp.k_cache.clone(), inp.v_cache.clone()
    torch.cuda.synchronize()
    for name, a, b in (("out", out_copy, ref_out), ("lse", lse_copy, ref_lse),
                       ("k_cache", kc_copy, ref_kc), ("v_cache", vc_copy, ref_vc)):
        bits = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(bits), b.view(bits)), f"{name} differs on the user stream"


def test_allocations_follow_the_call_stream():
    # stream= given without entering torch.cuda.stream(): the binding allocates
    # out, softmax_lse and the split workspace on that stream, so allocations
    # made on the current stream right after the call (filled while the call
    # may still run) cannot take their blocks.  The result equals the same call
    # on the current stream bit for bit.
    c = wl.Case(name="gqa_split_stream", q_lens=[1] * 8, cache_seqlens=[4096 + 37 * i for i in range(8)],
                num_heads_q=32, num_heads_kv=4, head_dim=128, dtype="bf16", page_size=16,
                causal=True, num_splits=16, seed=7101)
    say(f"case {c.name} seed {c.seed}: library allocations on a user stream")
    inp = make_inputs(c, "cuda")
    ref_out, ref_lse = gpu_call(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out, lse = pa.paged_attn_fwd(
        inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, causal=c.causal,
        num_splits=c.num_splits, stream=s)
    # churn the current stream's pool with blocks of the workspace's size
    args = pa.make_args(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                        inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q, causal=c.causal,
                        num_splits=c.num_splits)
    need = pa.paged_attn_workspace_size(args)
    assert need > 0
    junk = []
    for _ in range(4):
        j = torch.empty(need, dtype=torch.uint8, device="cuda")
        j.fill_(0xFF)
        junk.append(j)
        o2 = torch.empty_like(inp.q)
        o2.fill_(float("nan"))
        junk.append(o2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse differs"


# All-decode batches large enough to give every compute unit two units of a
# pair of kv heads, in whole rounds of two workgroups per compute unit, run
# decode units over pairs of adjacent kv heads (one load fetches both heads'
# slices of a key's row); PAGED_ATTN_HEAD_PAIRS=0 keeps one-head units.  Both against the oracle, and within a few output ulps of
# each other (different tile sizes and MFMA shapes round differently).
PAIR_CASES = [
    Case(name="pairs_mha_f16", q_lens=[1] * 64, cache_seqlens=[37 + 11 * i for i in range(64)],
         num_heads_q=16, num_heads_kv=16, head_dim=128, dtype="f16", page_size=16, append=True,
         causal=True, seed=7501),
    Case(name="pairs_gqa8_bf16", q_lens=[1] * 112, cache_seqlens=[300 - 2 * i for i in range(112)],
         num_heads_q=112, num_heads_kv=14, head_dim=128, dtype="bf16", page_size=32,
         causal=True, seed=7502),
    Case(name="pairs_q2_g2_d64", q_lens=[2] * 64, cache_seqlens=[90 + (7 * i) % 50 for i in range(64)],
         num_heads_q=32, num_heads_kv=16, head_dim=64, dtype="f16", page_size=256, append=True,
         causal=True, seed=7503),
    Case(name="pairs_contiguous_bf16", q_lens=[1] * 64, cache_seqlens=[5 + 9 * i for i in range(64)],
         num_heads_q=16, num_heads_kv=16, head_dim=128, dtype="bf16", page_size=None,
         contig_alloc=640, causal=False, seed=7504),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: c.name)
def test_decode_units_over_head_pairs(case, monkeypatch):
    # batch x kv heads >= 4 x 256 compute units, and the pair units end on no
    # part-filled round of 512 workgroups that one-head units would not
    units = case.batch * case.num_heads_kv
    assert units >= 1024 and 2 * -(-(units // 2) // 512) <= -(-units // 512)
    inp, errs = run_parity(case, splits=(None, 3))
    say(f"  pair units: max out err {max(errs):.3g}")
    monkeypatch.setenv("PAGED_ATTN_HEAD_PAIRS", "0")
    inp1, errs1 = run_parity(case, splits=(None,))
    monkeypatch.delenv("PAGED_ATTN_HEAD_PAIRS")
    say(f"  one-head units: max out err {max(errs1):.3g}")
