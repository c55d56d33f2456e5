"""Memory safety of the HIP path: the failure class of the flash-attention
thread "Add support for small page sizes" (an illegal memory access from a
paged append + causal attention call repeated in a loop, later traced with a
memory checker to reads past the block table).

  * Guard bands: every buffer of a call - inputs, outputs, the split
    workspace and both pools - sits inside a larger allocation whose bytes
    before and after it hold a sentinel.  After one call of each workload
    shape the sentinels are intact, the read-only inputs are unchanged byte
    for byte, every output row of a sequence was written, output rows past
    cu_seqlens_q[batch] were not, and the only pool rows that changed are the
    append targets, which hold the new rows bit for bit.
  * The reproduction loop: 100 calls in the reproduction script's shape (4
    sequences x 170 new tokens, 32 heads x 128, fp16, page 16, a 1000-page
    pool, append + causal, empty caches, a fresh table and fresh values each
    call - distinct page ids, the reading the workloads use), each checked
    against the oracle, stopping at the first mismatch.
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
GUARD = 1 << 16          # sentinel bytes on each side of every buffer
SENTINEL = 0x5A          # byte pattern of guards and unwritten outputs


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    assert pa._lib() is not None


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A tensor placed GUARD bytes into a sentinel-filled byte buffer."""

    def __init__(self, name, like=None, shape=None, dtype=None, fill=None):
        self.name = name
        shape = tuple(like.shape) if like is not None else tuple(shape)
        dtype = like.dtype if like is not None else dtype
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = n
        self.buf = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)
        if like is not None:
            self.t.copy_(like)
        elif fill is not None:
            self.t.view(torch.uint8).fill_(fill)

    def guards_intact(self):
        return bool((self.buf[:GUARD] == SENTINEL).all()) and \
            bool((self.buf[GUARD + self.nbytes:] == SENTINEL).all())


def target_rows(inp):
    """Pool rows (page * P + slot, or b * alloc + pos) the append writes, in
    token order, and the packed token each one takes."""
    c = inp.case
    cu = host(inp.cu_seqlens_q)
    table = host(inp.block_table)
    rows, toks = [], []
    if not c.append:
        return np.asarray(rows, np.int64), np.asarray(toks, np.int64)
    for b in range(c.batch):
        L = c.cache_seqlens[b]
        for i in range(int(cu[b + 1] - cu[b])):
            pos = L + i
            if table is None:
                rows.append(b * inp.k_cache.shape[1] + pos)
            else:
                rows.append(int(table[b, pos // c.page_size]) * c.page_size + pos % c.page_size)
            toks.append(int(cu[b]) + i)
    return np.asarray(rows, np.int64), np.asarray(toks, np.int64)


def run_guarded(case, num_splits=None, pad_rows=0, rotary=False):
    """One call with every buffer guarded; `pad_rows` extra rows of q / out /
    lse (and k_new / v_new) past cu_seqlens_q[batch], which the call must leave
    alone."""
    say(f"case {case.name} seed {case.seed} splits {num_splits} pad {pad_rows} rotary {rotary} "
        "(guard bands)")
    inp = make_inputs(case, "cuda")
    T = case.total_q + pad_rows

    def padded(t):
        if t is None or pad_rows == 0:
            return t
        extra = torch.full((pad_rows,) + tuple(t.shape[1:]), 0.25, dtype=t.dtype, device="cuda")
        return torch.cat([t, extra])

    g = {}
    g["q"] = Guarded("q", padded(inp.q))
    g["k_cache"] = Guarded("k_cache", inp.k_cache)
    g["v_cache"] = Guarded("v_cache", inp.v_cache)
    if inp.block_table is not None:
        g["block_table"] = Guarded("block_table", inp.block_table)
    g["cache_seqlens"] = Guarded("cache_seqlens", inp.cache_seqlens)
    g["cu_seqlens_q"] = Guarded("cu_seqlens_q", inp.cu_seqlens_q)
    if case.append:
        g["k_new"] = Guarded("k_new", padded(inp.k_new))
        g["v_new"] = Guarded("v_new", padded(inp.v_new))
    rot = {}
    if rotary:
        cos, sin = wl.rotary_tables(max(case.keys_visible()) + 1, case.head_dim, case.dtype)
        g["rotary_cos"] = Guarded("rotary_cos", cos)
        g["rotary_sin"] = Guarded("rotary_sin", sin)
        rot = dict(rotary_cos=g["rotary_cos"].t, rotary_sin=g["rotary_sin"].t)
    g["out"] = Guarded("out", shape=(T, case.num_heads_q, case.head_dim), dtype=inp.q.dtype,
                       fill=SENTINEL)
    g["softmax_lse"] = Guarded("softmax_lse", shape=(T, case.num_heads_q), dtype=torch.float32,
                               fill=SENTINEL)
    tens = {k: v.t for k, v in g.items()}
    splits = case.num_splits if num_splits is None else num_splits
    kw = dict(max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k,
              k_new=tens.get("k_new"), v_new=tens.get("v_new"), causal=case.causal,
              num_splits=splits)
    args = pa.make_args(tens["q"], tens["k_cache"], tens["v_cache"], tens.get("block_table"),
                        tens["cache_seqlens"], tens["cu_seqlens_q"], **kw)
    need = pa.paged_attn_workspace_size(args)
    if need > 0:
        g["workspace"] = Guarded("workspace", shape=(need,), dtype=torch.uint8, fill=0xC3)
    before = {k: v.buf.clone() for k, v in g.items() if k not in ("out", "softmax_lse", "workspace")}
    pa.paged_attn_fwd(tens["q"], tens["k_cache"], tens["v_cache"], tens.get("block_table"),
                      tens["cache_seqlens"], tens["cu_seqlens_q"], out=tens["out"],
                      softmax_lse=tens["softmax_lse"],
                      workspace=g["workspace"].t if "workspace" in g else None, **kw, **rot)
    torch.cuda.synchronize()
    for k, v in g.items():
        assert v.guards_intact(), f"{case.name}: bytes around {k} were written"
    # read-only inputs unchanged byte for byte
    for k in before:
        if k in ("k_cache", "v_cache"):
            continue
        assert torch.equal(g[k].buf, before[k]), f"{case.name}: input {k} was modified"
    # pools: only the append targets changed, and they hold the new rows
    rows, toks = target_rows(inp)
    for k, new in (("k_cache", "k_new"), ("v_cache", "v_new")):
        now = g[k].t.view(torch.int16).reshape(-1, case.num_heads_kv * case.head_dim)
        was = before[k][GUARD:GUARD + g[k].nbytes].view(torch.int16).reshape(now.shape)
        changed = (now != was).any(dim=1).nonzero().flatten().cpu().numpy()
        if not case.append:
            assert changed.size == 0, f"{case.name}: {k} changed without an append"
            continue
        assert np.isin(changed, rows).all(), \
            f"{case.name}: {k} rows outside the append targets changed: {changed[~np.isin(changed, rows)][:8]}"
        if not (rotary and k == "k_cache"):
            idx = torch.from_numpy(rows).cuda()
            src = g[new].t.view(torch.int16).reshape(T, -1)[torch.from_numpy(toks).cuda()]
            assert torch.equal(now.index_select(0, idx), src), f"{case.name}: {k} targets differ"
    # outputs: every row of a sequence written, rows past cu[batch] untouched
    R = case.total_q
    out_b = g["out"].t.view(torch.uint8).reshape(T, -1)
    lse_b = g["softmax_lse"].t.view(torch.uint8).reshape(T, -1)
    # (no output value can carry the sentinel bits: values are in [0, 1), and
    # the sentinel is 203.25 in fp16, 1.5e16 in bf16 and in fp32)
    assert not (g["out"].t[:R].view(torch.int16) == SENTINEL * 0x0101).any(), \
        f"{case.name}: out rows not written"
    assert not (g["softmax_lse"].t[:R].view(torch.int32) == SENTINEL * 0x01010101).any(), \
        f"{case.name}: lse rows not written"
    if pad_rows:
        assert (out_b[R:] == SENTINEL).all() and (lse_b[R:] == SENTINEL).all(), \
            f"{case.name}: rows past cu_seqlens_q[batch] were written"
    del g, before, inp
    torch.cuda.empty_cache()


def mixed_prefill_decode():
    return Case(name="mixed_gqa_prefill_decode", q_lens=[40, 1, 3, 1, 200], cache_seqlens=[0, 900, 17, 33, 64],
                num_heads_q=16, num_heads_kv=4, head_dim=128, dtype="bf16", page_size=32,
                append=True, causal=True, seed=7301)


GUARDED = [
    ("tiny_decode", lambda: wl.tiny_decode(), [0, 3], 0),
    ("tiny_decode_padded", lambda: wl.tiny_decode(), [2], 3),
    ("mha_decode_b16_ctx1024_append", lambda: wl.mha_decode(16, 1024, append=True), [0], 0),
    ("mha_decode_b4_ctx512_p256", lambda: wl.mha_decode(4, 512, page_size=256), [0, 4], 0),
    ("gqa_long_split_paged", lambda: wl.gqa_long_split(paged=True), [0, 128], 0),
    ("gqa_long_split_contig", lambda: wl.gqa_long_split(paged=False), [0], 0),
    ("causal_prefill_4x170", lambda: wl.causal_prefill_append(170, "uniform"), [0], 5),
    ("causal_prefill_4x2048", lambda: wl.causal_prefill_append(2048, "zero"), [0], 0),
    ("unified_nq100_32x128", lambda: wl.unified_varlen(100), [0, 2], 0),
    ("unified_nq1000_12x64", lambda: wl.unified_varlen(1000, heads=12, head_dim=64), [0], 2),
    ("multi_token_q16", lambda: wl.multi_token_decode(8, 700, 16), [0, 3], 0),
    ("mixed_gqa", mixed_prefill_decode, [0, 2], 4),
]


@pytest.mark.parametrize("name,make,splits,pad", GUARDED, ids=[x[0] for x in GUARDED])
def test_guard_bands(name, make, splits, pad):
    for s in splits:
        run_guarded(make(), num_splits=s, pad_rows=pad)


@pytest.mark.parametrize("make", [lambda: wl.unified_varlen(100, heads=8, head_dim=128),
                                  lambda: wl.mha_decode(8, 1000, append=True)])
def test_guard_bands_with_rotary(make):
    run_guarded(make(), rotary=True)


def test_reproduction_loop_100_calls():
    bs, seq_len, heads, hd, P, num_pages = 4, 170, 32, 128, 16, 1000
    width = -(-seq_len // P)
    say("reproduction-shaped loop: 100 calls of 4 x 170 tokens, 32 x 128 fp16, page 16, "
        "1000-page pool")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6000)
    k_cache = torch.rand((num_pages, P, heads, hd), generator=gen, device="cuda").half()
    v_cache = torch.rand((num_pages, P, heads, hd), generator=gen, device="cuda").half()
    cache_seqlens = torch.zeros(bs, dtype=torch.int32, device="cuda")
    cu = torch.arange(0, (bs + 1) * seq_len, seq_len, dtype=torch.int32, device="cuda")
    cu_h = host(cu)
    out = torch.empty((bs * seq_len, heads, hd), dtype=torch.float16, device="cuda")
    lse = torch.empty((bs * seq_len, heads), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(6000)
    for it in range(100):
        q = torch.rand((bs * seq_len, heads, hd), generator=gen, device="cuda").half()
        k = torch.rand((bs * seq_len, heads, hd), generator=gen, device="cuda").half()
        v = torch.rand((bs * seq_len, heads, hd), generator=gen, device="cuda").half()
        table_h = rng.permutation(num_pages)[:bs * width].astype(np.int32).reshape(bs, width)
        table = torch.from_numpy(table_h).cuda()
        kc0, vc0 = k_cache.clone(), v_cache.clone()
        pa.paged_attn_fwd(q, k_cache, v_cache, table, cache_seqlens, cu, max_seqlen_q=seq_len,
                          k_new=k, v_new=v, causal=True, out=out, softmax_lse=lse)
        torch.cuda.synchronize()
        # the oracle on a compact pool of the sequences' own pages (the caches
        # are empty, so every key it attends over is one it appended itself)
        flat = torch.from_numpy(table_h.reshape(-1).astype(np.int64)).cuda()
        compact = np.arange(bs * width, dtype=np.int32).reshape(bs, width)
        ref_o, ref_l, ref_kc, ref_vc = oracle.paged_attention(
            host(q), host(kc0.index_select(0, flat)), host(vc0.index_select(0, flat)), compact,
            np.zeros(bs, np.int32), cu_h, host(k), host(v), dtype="f16", causal=True)
        err = np.abs(out.float().cpu().numpy() - ref_o).max()
        assert err <= OUT_TOL, f"call {it}: out err {err}"
        l = lse.cpu().numpy().astype(np.float64)
        assert (np.abs(l - ref_l) <= LSE_REL * np.abs(ref_l) + LSE_ABS).all(), f"call {it}: lse"
        # the table's pages hold what the oracle wrote; every other page is as before
        assert np.array_equal(host(k_cache.index_select(0, flat)), ref_kc), f"call {it}: K pages"
        assert np.array_equal(host(v_cache.index_select(0, flat)), ref_vc), f"call {it}: V pages"
        others = torch.ones(num_pages, dtype=torch.bool, device="cuda")
        others[flat] = False
        assert torch.equal(k_cache[others].view(torch.int16), kc0[others].view(torch.int16)), \
            f"call {it}: a K page outside the table changed"
        assert torch.equal(v_cache[others].view(torch.int16), vc0[others].view(torch.int16)), \
            f"call {it}: a V page outside the table changed"
        if it % 25 == 24:
            say(f"  {it + 1} calls ok, last out err {err:.3g}")
