"""The allocation-free entry point paged_attn_fwd_noalloc against
paged_attn_fwd, through the C ABI: the same kernels on the same inputs, with
the library's static device scratch in place of the caller's workspace, so
the outputs and the pools after the append must agree bit for bit.  Two calls
in a row, the second smaller than the first (the scratch keeps the first
call's contents), each with a forced split budget so the scratch carries
split-KV partials; the second batch also mixes a prefill sequence in (one
launch: this entry point never forks)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_lds_amd as pa
import workloads as wl
from workloads import Case, host, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both_entry_points(case, splits):
    say(f"case {case.name} seed {case.seed} splits {splits}: noalloc vs workspace entry point")
    inp = make_inputs(case, "cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()
    kw = dict(max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new,
              v_new=inp.v_new, causal=case.causal, num_splits=splits)
    args = pa.make_args(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                        inp.cu_seqlens_q, **kw)
    need = pa.paged_attn_workspace_size(args)
    assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES, need
    ref_out, ref_lse = pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                         inp.cache_seqlens, inp.cu_seqlens_q, **kw)
    torch.cuda.synchronize()
    ref_kc, ref_vc = inp.k_cache.clone(), inp.v_cache.clone()
    inp.k_cache.copy_(kc0)
    inp.v_cache.copy_(vc0)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full(inp.q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    pa.paged_attn_fwd_noalloc(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                              inp.cache_seqlens, inp.cu_seqlens_q, out=out, softmax_lse=lse, **kw)
    torch.cuda.synchronize()
    for name, a, b in (("out", out, ref_out), ("lse", lse, ref_lse),
                       ("k_cache", inp.k_cache, ref_kc), ("v_cache", inp.v_cache, ref_vc)):
        bits = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(bits), b.view(bits)), f"{case.name}: {name} differs"
    # and both against the oracle, within the usual bars
    r_out, r_lse, _, _ = oracle.paged_attention(
        host(inp.q), host(kc0), host(vc0), host(inp.block_table), host(inp.cache_seqlens),
        host(inp.cu_seqlens_q), host(inp.k_new), host(inp.v_new), dtype=case.dtype,
        causal=case.causal)
    err = np.abs(out.float().cpu().numpy() - r_out).max()
    assert err <= 2e-3, f"{case.name}: out err {err}"
    l = lse.cpu().numpy().astype(np.float64)
    fin = ~np.isneginf(r_lse)
    assert np.array_equal(np.isneginf(l), ~fin)
    assert (np.abs(l[fin] - r_lse[fin]) <= 1e-4 * np.abs(r_lse[fin]) + 1e-6).all()
    say(f"  bit-identical, out err vs oracle {err:.3g}")


def test_noalloc_equals_workspace_entry_point_twice():
    assert torch.cuda.is_available()
    first = Case(name="noalloc_gqa_decode", q_lens=[1] * 6, cache_seqlens=[3000, 5000, 700, 4100, 64, 2222],
                 num_heads_q=32, num_heads_kv=4, head_dim=128, dtype="bf16", page_size=16,
                 append=True, causal=True, seed=8101)
    second = Case(name="noalloc_mixed_small", q_lens=[1, 37, 2], cache_seqlens=[900, 0, 333],
                  num_heads_q=8, num_heads_kv=8, head_dim=64, dtype="f16", page_size=32,
                  append=True, causal=True, seed=8102)
    both_entry_points(first, 8)
    both_entry_points(second, 3)


def test_noalloc_rejects_a_plan_past_its_scratch():
    # 4096 rows x 32 heads x 128 dims at a forced budget of 128 splits: far
    # more partials than the static array holds; nothing is launched
    c = wl.Case(name="noalloc_too_big", q_lens=[1] * 4096, cache_seqlens=[16] * 4096,
                num_heads_q=32, num_heads_kv=32, head_dim=128, dtype="f16", page_size=16,
                causal=True, seed=8103)
    inp = make_inputs(c, "cuda")
    out = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attn_fwd_noalloc(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                  inp.cache_seqlens, inp.cu_seqlens_q, out=out, softmax_lse=lse,
                                  max_seqlen_q=1, causal=True, num_splits=128)
    assert e.value.status == pa.PA_ERR_SCRATCH
