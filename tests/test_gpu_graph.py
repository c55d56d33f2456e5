"""Graph capture of one paged_attn_fwd call.

One call (append + attention with its split-KV merge) on fixed device buffers
is captured once into a HIP graph and replayed with different batches loaded
into the same buffers: prefill chunks and decode sequences of different
lengths, with the unused sequence slots padded as (0, 0) (no new tokens, empty
cache), the static-shape batch padding the unified-kernel discussion relies on
for graph capture.  Every replay - each batch twice, with eager work and
synchronisations between replays - must match an eager call on the same
buffers bit for bit (out, lse and the cache bytes after the append), and the
oracle within the usual bars.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_lds_amd as pa
import workloads as wl
from workloads import host

pytestmark = pytest.mark.gpu

SLOTS, T_STATIC, MAXQ, HQ, HKV, D, P = 6, 96, 64, 8, 2, 128, 16
WIDTH = 80                      # table entries per slot: keys per slot <= 1280
SPLITS = 3                      # forced budget: the split merge is in the graph too

# (q_lens, cache_seqlens) per batch; trailing slots are (0, 0) padding
BATCHES = [
    ([40, 1, 1, 0, 0, 0], [0, 300, 700, 0, 0, 0]),
    ([64, 1, 1, 1, 20, 0], [100, 50, 1000, 5, 30, 0]),
    ([1, 1, 1, 1, 1, 1], [17, 1200, 64, 640, 3, 999]),
]


def _cu(q_lens):
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


def _load(buf, q_lens, cache_lens, seed, kc0, vc0):
    """Write one batch's metadata and data into the static buffers (eager)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    buf["cu"].copy_(torch.from_numpy(_cu(q_lens)))
    buf["seqlens"].copy_(torch.tensor(cache_lens, dtype=torch.int32))
    for name in ("q", "k_new", "v_new"):
        t = buf[name]
        t.copy_(torch.rand(t.shape, generator=g, device="cuda", dtype=torch.float32).to(t.dtype))
    buf["k_cache"].copy_(kc0)
    buf["v_cache"].copy_(vc0)
    buf["out"].zero_()
    buf["lse"].zero_()


def _call(buf):
    pa.paged_attn_fwd(buf["q"], buf["k_cache"], buf["v_cache"], buf["table"], buf["seqlens"],
                      buf["cu"], max_seqlen_q=MAXQ, max_seqlen_k=WIDTH * P, k_new=buf["k_new"],
                      v_new=buf["v_new"], causal=True, num_splits=SPLITS, out=buf["out"],
                      softmax_lse=buf["lse"], workspace=buf["ws"], aux_stream=buf["aux"])


def _snapshot(buf):
    return {k: buf[k].clone() for k in ("out", "lse", "k_cache", "v_cache")}


# "auto": the binding's second stream, so the captured call forks the decode
# units off and joins them back; None: one launch on the captured stream
@pytest.mark.parametrize("aux", ["auto", None])
def test_graph_replays_match_eager_calls(aux):
    assert torch.cuda.is_available()
    rng = np.random.default_rng(5150)
    num_pages = SLOTS * WIDTH
    buf = {
        "q": torch.empty(T_STATIC, HQ, D, dtype=torch.float16, device="cuda"),
        "k_new": torch.empty(T_STATIC, HKV, D, dtype=torch.float16, device="cuda"),
        "v_new": torch.empty(T_STATIC, HKV, D, dtype=torch.float16, device="cuda"),
        "k_cache": torch.empty(num_pages, P, HKV, D, dtype=torch.float16, device="cuda"),
        "v_cache": torch.empty(num_pages, P, HKV, D, dtype=torch.float16, device="cuda"),
        "table": torch.from_numpy(rng.permutation(num_pages).astype(np.int32)
                                  .reshape(SLOTS, WIDTH)).cuda(),
        "seqlens": torch.zeros(SLOTS, dtype=torch.int32, device="cuda"),
        "cu": torch.zeros(SLOTS + 1, dtype=torch.int32, device="cuda"),
        "out": torch.empty(T_STATIC, HQ, D, dtype=torch.float16, device="cuda"),
        "lse": torch.empty(T_STATIC, HQ, dtype=torch.float32, device="cuda"),
    }
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(5151)
    kc0 = torch.rand(buf["k_cache"].shape, generator=g0, device="cuda").half()
    vc0 = torch.rand(buf["v_cache"].shape, generator=g0, device="cuda").half()
    args = pa.make_args(buf["q"], buf["k_cache"], buf["v_cache"], buf["table"], buf["seqlens"],
                        buf["cu"], max_seqlen_q=MAXQ, max_seqlen_k=WIDTH * P,
                        k_new=buf["k_new"], v_new=buf["v_new"], causal=True, num_splits=SPLITS,
                        softmax_scale=None, out=buf["out"], softmax_lse=buf["lse"], workspace=None)
    need = pa.paged_attn_workspace_size(args)
    assert need > 0, "a forced split budget needs a workspace"
    buf["ws"] = torch.empty(need, dtype=torch.uint8, device="cuda")
    buf["aux"] = aux

    # eager results of every batch on the static buffers
    eager = []
    for i, (ql, cl) in enumerate(BATCHES):
        _load(buf, ql, cl, 6000 + i, kc0, vc0)
        _call(buf)
        torch.cuda.synchronize()
        eager.append(_snapshot(buf))
        # the oracle on the same bytes: the covered rows only
        n = int(sum(ql))
        ref_out, ref_lse, ref_kc, ref_vc = oracle.paged_attention(
            host(buf["q"][:n]), host(kc0), host(vc0), host(buf["table"]), np.array(cl, np.int32),
            _cu(ql), host(buf["k_new"][:n]), host(buf["v_new"][:n]), dtype="f16", causal=True)
        o = eager[-1]["out"][:n].float().cpu().numpy().astype(np.float64)
        assert np.abs(o - ref_out).max(initial=0.0) <= 2e-3, f"batch {i}: out vs oracle"
        lse = eager[-1]["lse"][:n].cpu().numpy().astype(np.float64)
        fin = ~np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(lse), ~fin), f"batch {i}: -inf pattern"
        assert (np.abs(lse[fin] - ref_lse[fin]) <= 1e-4 * np.abs(ref_lse[fin]) + 1e-6).all()
        assert np.array_equal(host(eager[-1]["k_cache"]), ref_kc), f"batch {i}: k pool"
        assert np.array_equal(host(eager[-1]["v_cache"]), ref_vc), f"batch {i}: v pool"

    # capture once (after a warm-up call on a side stream), on batch 0's data
    _load(buf, *BATCHES[0], 6000, kc0, vc0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(buf)
    torch.cuda.synchronize()

    # replay each batch twice, with eager work and syncs in between
    for rep in range(2):
        for i, (ql, cl) in enumerate(BATCHES):
            _load(buf, ql, cl, 6000 + i, kc0, vc0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = _snapshot(buf)
            for k in ("out", "lse", "k_cache", "v_cache"):
                assert torch.equal(got[k], eager[i][k]), f"replay {rep} batch {i}: {k} differs"
            # unrelated eager work between replays
            x = torch.rand(1 << 20, device="cuda")
            assert float((x * 2).sum()) > 0


@pytest.mark.parametrize("make", [lambda: wl.mha_decode(1, 512), lambda: wl.mha_decode(8, 1024),
                                  lambda: wl.unified_varlen(100, heads=12, head_dim=64)],
                         ids=["decode_1x512", "decode_8x1024", "unified_nq100_h12x64"])
def test_graph_sweep_points_replay_bit_exact(make):
    # the graph sweep's three points with the library's own split budget: a
    # captured call replayed three times, with eager work and syncs between,
    # gives the eager call's outputs and pools bit for bit
    c = make()
    inp = wl.make_inputs(c, "cuda")
    out = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device="cuda")
    kn = inp.k_new if c.append else None
    vn = inp.v_new if c.append else None
    args = pa.make_args(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                        inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                        max_seqlen_k=inp.max_seqlen_k, k_new=kn, v_new=vn, causal=c.causal,
                        num_splits=0, out=out, softmax_lse=lse)
    ws = torch.empty(max(1, pa.paged_attn_workspace_size(args)), dtype=torch.uint8, device="cuda")
    kc0, vc0 = inp.k_cache.clone(), inp.v_cache.clone()

    def call():
        pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                          inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                          max_seqlen_k=inp.max_seqlen_k, k_new=kn, v_new=vn, causal=c.causal,
                          out=out, softmax_lse=lse, workspace=ws)

    def reset():
        inp.k_cache.copy_(kc0)
        inp.v_cache.copy_(vc0)
        out.zero_()
        lse.zero_()

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, inp.k_cache, inp.v_cache)]
    reset()
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
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((out, lse, inp.k_cache, inp.v_cache), ref,
                                   ("out", "lse", "k_cache", "v_cache")):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
