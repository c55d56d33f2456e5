"""Boundary features on the GPU: q / k_new / v_new as row-strided views of one
fused QKV buffer, and the PAGED_ATTN_DEBUG=1 precondition checks."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_lds_amd as pa
import workloads as wl
from workloads import Case, host, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    assert pa._lib() is not None


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kind", ["decode", "unified"])
def test_fused_qkv_views_equal_dense_tensors(kind):
    if kind == "decode":
        c = Case(name="qkv_views_decode", q_lens=[1, 2, 1], cache_seqlens=[300, 77, 1000],
                 num_heads_q=16, num_heads_kv=4, head_dim=128, dtype="bf16", page_size=16,
                 append=True, causal=True, seed=6100)
    else:
        c = Case(name="qkv_views_unified", q_lens=[150, 1, 1], cache_seqlens=[40, 500, 3],
                 num_heads_q=8, num_heads_kv=8, head_dim=64, dtype="f16", page_size=32,
                 append=True, causal=True, seed=6101)
    say(f"case {c.name}")
    inp = make_inputs(c, "cuda")
    T, hq, hkv, d = c.total_q, c.num_heads_q, c.num_heads_kv, c.head_dim
    # one fused buffer [T, (hq + 2 hkv) * d + 8]: q | k | v | 8 elements of padding
    width = (hq + 2 * hkv) * d + 8
    qkv = torch.zeros(T, width, dtype=inp.q.dtype, device="cuda")
    qkv[:, :hq * d] = inp.q.reshape(T, -1)
    qkv[:, hq * d:(hq + hkv) * d] = inp.k_new.reshape(T, -1)
    qkv[:, (hq + hkv) * d:(hq + 2 * hkv) * d] = inp.v_new.reshape(T, -1)
    qv = qkv[:, :hq * d].view(T, hq, d)
    kv = qkv[:, hq * d:(hq + hkv) * d].view(T, hkv, d)
    vv = qkv[:, (hq + hkv) * d:(hq + 2 * hkv) * d].view(T, hkv, d)
    assert not qv.is_contiguous() and qv.stride(0) == width
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    outs = []
    for q, k, v in ((inp.q, inp.k_new, inp.v_new), (qv, kv, vv)):
        inp.k_cache.copy_(kc0)
        inp.v_cache.copy_(vc0)
        o, l = pa.paged_attn_fwd(q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                                 inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q, k_new=k, v_new=v,
                                 causal=True, num_splits=2)
        torch.cuda.synchronize()
        outs.append((o, l, inp.k_cache.clone(), inp.v_cache.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    ref_out, ref_lse, ref_kc, ref_vc = oracle.paged_attention(
        host(inp.q), host(kc0), host(vc0), host(inp.block_table), host(inp.cache_seqlens),
        host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new), dtype=c.dtype, causal=True)
    assert np.abs(outs[1][0].float().cpu().numpy() - ref_out).max() <= 2e-3
    assert np.array_equal(host(outs[1][2]), ref_kc) and np.array_equal(host(outs[1][3]), ref_vc)
    # the append-only entry point takes the views too
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    pa.paged_kv_append(inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                       inp.cu_seqlens_q, kv, vv, max_seqlen_q=inp.max_seqlen_q)
    torch.cuda.synchronize()
    assert np.array_equal(host(inp.k_cache), ref_kc) and np.array_equal(host(inp.v_cache), ref_vc)


def _debug_call(inp, **kw):
    os.environ["PAGED_ATTN_DEBUG"] = "1"
    try:
        return pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                 kw.pop("seqlens", inp.cache_seqlens), kw.pop("cu", inp.cu_seqlens_q),
                                 max_seqlen_q=kw.pop("max_seqlen_q", inp.max_seqlen_q),
                                 k_new=inp.k_new, v_new=inp.v_new, causal=True, **kw)
    finally:
        del os.environ["PAGED_ATTN_DEBUG"]


def test_debug_mode_checks_device_metadata():
    c = Case(name="debug_checks", q_lens=[1, 3, 1], cache_seqlens=[40, 17, 100], num_heads_q=8,
             num_heads_kv=2, head_dim=64, dtype="f16", page_size=16, append=True, causal=True,
             table_width=12, seed=6200)
    say(f"case {c.name}")
    inp = make_inputs(c, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    # valid metadata: the same result as without the checks
    o1, l1 = _debug_call(inp)
    torch.cuda.synchronize()
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    o2, l2 = pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                               inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q, k_new=inp.k_new,
                               v_new=inp.v_new, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

    def expect_precondition(**kw):
        inp.k_cache.copy_(kc0)
        inp.v_cache.copy_(vc0)
        with pytest.raises(pa.PagedAttnError) as e:
            _debug_call(inp, **kw)
        assert e.value.status == 8
        # nothing was launched: the pools are untouched
        torch.cuda.synchronize()
        assert torch.equal(inp.k_cache, kc0) and torch.equal(inp.v_cache, vc0)

    # keys beyond the table row (12 pages of 16)
    expect_precondition(seqlens=torch.tensor([40, 190, 100], dtype=torch.int32, device="cuda"))
    # q_len above max_seqlen_q
    expect_precondition(max_seqlen_q=2)
    # cu_seqlens_q not starting at 0
    expect_precondition(cu=torch.tensor([1, 2, 5, 5], dtype=torch.int32, device="cuda"))
    # a page id outside the pool inside a live range
    bt = inp.block_table.clone()
    bt[2, 1] = inp.k_cache.shape[0] + 5
    saved = inp.block_table
    inp.block_table = bt
    expect_precondition()
    # two sequences appending into the same slot: sequence 0 writes position 40
    # (page 2, slot 8); with cache 24, sequence 1 writes positions 24..26 (page
    # 1, slots 8..10) - made the same physical page
    bt2 = saved.clone()
    bt2[1, 1] = bt2[0, 2]
    inp.block_table = bt2
    expect_precondition(seqlens=torch.tensor([40, 24, 100], dtype=torch.int32, device="cuda"))
    inp.block_table = saved
