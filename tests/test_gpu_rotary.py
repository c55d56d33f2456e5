"""GPU parity of the fused rotary embedding (queries in the attention kernels,
new keys in the append kernel) against the CPU oracle.

Bars: the cache after the append is bit-exact (the rotated key is the exact
value rounded to fp32 and then to the element type on both sides); out and
softmax_lse meet the bars of the other parity tests.  A second, bit-exact check
pins the query rotation itself: the fused call returns exactly what the same
kernels return without rotary on queries and keys the oracle rotated.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import rotary as orot
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


def to_dev(bits_np, like):
    return torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(like.dtype).to(
        like.device)


def check(out, lse, ref_out, ref_lse, what):
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


def run_rotary(case, rotary_dim, interleaved, rows=None, kind="angles", splits=(None,)):
    say(f"case {case.name} seed {case.seed} rotary_dim {rotary_dim} interleaved {interleaved} "
        f"rows {rows} kind {kind}")
    inp = make_inputs(case, "cuda")
    Kb = case.keys_visible()
    if rows is None:
        rows = max(Kb) + 1
    cos, sin = wl.rotary_tables(rows, rotary_dim, case.dtype, kind=kind, seed=case.seed)
    tab = (host(cos), host(sin), interleaved)
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    ref_out, ref_lse, ref_kc, ref_vc = oracle.paged_attention(
        host(inp.q), kc0, vc0, host(inp.block_table), host(inp.cache_seqlens),
        host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new), dtype=case.dtype,
        causal=case.causal, rotary=tab)
    # queries and new keys as the oracle rotates them, for the bit-exact check
    pos = orot.token_positions(host(inp.cache_seqlens), host(inp.cu_seqlens_q),
                               appended=case.append, total=inp.q.shape[0])
    q_rot = to_dev(orot.rotate_bits(host(inp.q), tab[0], tab[1], pos, dtype=case.dtype,
                                    interleaved=interleaved), inp.q)
    kn_rot = None
    if case.append:
        kn_rot = to_dev(orot.rotate_bits(host(inp.k_new), tab[0], tab[1], pos, dtype=case.dtype,
                                         interleaved=interleaved), inp.k_new)
    for s in splits:
        inp.k_cache.copy_(to_dev(kc0, inp.k_cache))
        inp.v_cache.copy_(to_dev(vc0, inp.v_cache))
        say(f"  fused call num_splits={s}")
        out, lse = pa.paged_attn_fwd(
            inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
            inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k,
            k_new=inp.k_new, v_new=inp.v_new, causal=case.causal,
            num_splits=case.num_splits if s is None else s, rotary_cos=cos, rotary_sin=sin,
            rotary_interleaved=interleaved)
        torch.cuda.synchronize()
        check(out, lse, ref_out, ref_lse, f"{case.name} S={s}")
        if case.append:
            assert np.array_equal(host(inp.k_cache), ref_kc), "k_cache after rotary append"
            assert np.array_equal(host(inp.v_cache), ref_vc), "v_cache after rotary append"
        # the same kernels without rotary on the oracle-rotated inputs
        inp.k_cache.copy_(to_dev(kc0, inp.k_cache))
        inp.v_cache.copy_(to_dev(vc0, inp.v_cache))
        say(f"  plain call on pre-rotated inputs num_splits={s}")
        out2, lse2 = pa.paged_attn_fwd(
            q_rot, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
            inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k,
            k_new=kn_rot, v_new=inp.v_new, causal=case.causal,
            num_splits=case.num_splits if s is None else s)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), f"{case.name}: fused rotary out differs from pre-rotated"
        assert torch.equal(lse, lse2), f"{case.name}: fused rotary lse differs from pre-rotated"


@pytest.mark.parametrize("make", [lambda: wl.causal_prefill_append(2048, "zero"),
                                  lambda: wl.mha_decode(256, 4096, append=True)],
                         ids=["prefill_4x2048", "decode_256x4096"])
def test_rotary_full_size_equals_pre_rotated(make):
    # the rotary sweep's prefill and decode points at full size: the fused
    # call equals the plain kernels on queries and new keys the oracle
    # rotated, bit for bit, and leaves the same pools (the appended keys are
    # the oracle's rotated bits); the plain path itself is checked against
    # the oracle at these sizes in test_gpu_fullsize.py
    case = make()
    say(f"case {case.name} seed {case.seed} full size, rotary_dim 128")
    inp = make_inputs(case, "cuda")
    cos, sin = wl.rotary_tables(max(case.keys_visible()) + 1, 128, case.dtype, kind="angles",
                                seed=case.seed)
    pos = orot.token_positions(host(inp.cache_seqlens), host(inp.cu_seqlens_q), appended=True,
                               total=inp.q.shape[0])
    q_rot = to_dev(orot.rotate_bits(host(inp.q), host(cos), host(sin), pos, dtype=case.dtype,
                                    interleaved=False), inp.q)
    kn_rot = to_dev(orot.rotate_bits(host(inp.k_new), host(cos), host(sin), pos, dtype=case.dtype,
                                     interleaved=False), inp.k_new)
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    out, lse = pa.paged_attn_fwd(
        inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new,
        v_new=inp.v_new, causal=case.causal, rotary_cos=cos, rotary_sin=sin)
    torch.cuda.synchronize()
    kc1, vc1 = inp.k_cache.clone(), inp.v_cache.clone()
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    out2, lse2 = pa.paged_attn_fwd(
        q_rot, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens, inp.cu_seqlens_q,
        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, k_new=kn_rot,
        v_new=inp.v_new, causal=case.causal)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "fused rotary differs from pre-rotated"
    assert torch.equal(kc1, inp.k_cache) and torch.equal(vc1, inp.v_cache), "pools differ"
    del inp, kc0, vc0, kc1, vc1
    torch.cuda.empty_cache()


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotary_mha_decode_append(interleaved):
    run_rotary(wl.mha_decode(3, 700, append=True), 128, interleaved, splits=(None, 3))


@pytest.mark.parametrize("rotary_dim,interleaved", [(64, False), (32, True), (128, True)])
def test_rotary_gqa_decode_no_append_bf16(rotary_dim, interleaved):
    rng = np.random.default_rng(2300)
    lens = [int(x) for x in rng.integers(100, 3000, 8, endpoint=True)]
    c = Case(name="gqa_rotary", q_lens=[1] * 8, cache_seqlens=lens, num_heads_q=64,
             num_heads_kv=8, head_dim=128, dtype="bf16", page_size=16, table_width=4096 // 16,
             causal=True, seed=2300, max_seqlen_k_hint=4096)
    run_rotary(c, rotary_dim, interleaved, splits=(None, 1, 4))


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotary_causal_prefill_append(interleaved):
    run_rotary(wl.causal_prefill_append(170, "uniform"), 128, interleaved)


@pytest.mark.parametrize("rotary_dim,interleaved", [(64, False), (32, True), (16, False)])
def test_rotary_unified_varlen_d64(rotary_dim, interleaved):
    run_rotary(wl.unified_varlen(100, heads=12, head_dim=64), rotary_dim, interleaved,
               splits=(None, 2))


def test_rotary_unified_varlen_d128_random_tables():
    run_rotary(wl.unified_varlen(300, prefix=77), 96, False, kind="random")


@pytest.mark.parametrize("q_len,hq,hkv,dtype", [(4, 32, 32, "f16"), (2, 64, 8, "bf16")])
def test_rotary_multi_token_decode(q_len, hq, hkv, dtype):
    c = wl.multi_token_decode(3, 700, q_len, heads_q=hq, heads_kv=hkv, dtype=dtype)
    c.cache_seqlens = [700, 41, 1500]
    run_rotary(c, 128, True, splits=(None, 3))


def test_rotary_positions_past_the_table_stay_unrotated():
    # table of 600 rows: sequences past position 600 are left as they are
    c = wl.unified_varlen(100, heads=8, head_dim=128)
    run_rotary(c, 128, False, rows=600)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotary_append_only_entry_point_bit_exact(interleaved):
    c = wl.causal_prefill_append(70, "uniform")
    say(f"append-only rotary interleaved={interleaved}")
    inp = make_inputs(c, "cuda")
    cos, sin = wl.rotary_tables(max(c.keys_visible()) + 1, 64, c.dtype)
    kc0, vc0 = host(inp.k_cache), host(inp.v_cache)
    pa.paged_kv_append(inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                       inp.cu_seqlens_q, inp.k_new, inp.v_new, max_seqlen_q=inp.max_seqlen_q,
                       rotary_cos=cos, rotary_sin=sin, rotary_interleaved=interleaved)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_append(kc0, vc0, host(inp.block_table), host(inp.cache_seqlens),
                              host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new),
                              rotary=(host(cos), host(sin), interleaved), dtype=c.dtype)
    assert np.array_equal(host(inp.k_cache), ek) and np.array_equal(host(inp.v_cache), ev)
    assert not np.array_equal(ek, oracle.kv_append(kc0, vc0, host(inp.block_table),
                                                   host(inp.cache_seqlens),
                                                   host(inp.cu_seqlens_q), host(inp.k_new),
                                                   host(inp.v_new))[0])


def test_rotary_call_replays_from_a_graph():
    # the fused rotary path under graph capture: one capture, replays with new
    # queries and keys loaded into the same buffers equal eager calls bit for bit
    c = wl.unified_varlen(60, heads=8, head_dim=128)
    say(f"case {c.name} (graph)")
    inp = make_inputs(c, "cuda")
    cos, sin = wl.rotary_tables(max(c.keys_visible()) + 1, 128, c.dtype)
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    out = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device="cuda")

    def call():
        pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                          inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                          max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new, v_new=inp.v_new,
                          causal=True, out=out, softmax_lse=lse, rotary_cos=cos, rotary_sin=sin)

    def load(seed):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        for t in (inp.q, inp.k_new, inp.v_new):
            t.copy_(torch.rand(t.shape, generator=g, device="cuda").to(t.dtype))
        inp.k_cache.copy_(kc0)
        inp.v_cache.copy_(vc0)

    eager = []
    for seed in (11, 12):
        load(seed)
        call()
        torch.cuda.synchronize()
        eager.append((out.clone(), lse.clone(), inp.k_cache.clone()))
    load(11)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, seed in enumerate((11, 12)):
            load(seed)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[i][0]) and torch.equal(lse, eager[i][1]), f"replay {rep}/{i}"
            assert torch.equal(inp.k_cache, eager[i][2]), f"replay {rep}/{i}: rotated keys"
