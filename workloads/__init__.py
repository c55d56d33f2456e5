"""Seeded synthetic inputs for the paged KV-cache attention forward pass.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no attention arithmetic: it only draws values, lays sequences out in
pages and builds the metadata tensors, so that the HIP path and the CPU oracle
can be fed the same bytes.

Layouts follow the reproduction script in the flash-attention thread "Add
support for small page sizes": K/V pools [num_pages, page_size, num_kv_heads,
head_dim], block_table [batch, width] int32, cache_seqlens [batch] int32; the
varlen form (packed [total_q, heads, head_dim] with cu_seqlens_q) follows the
vLLM thread "Unify the kernel used in flash attention backend".

Recipe (stated once, used everywhere):
  * page ids: ``numpy.random.default_rng(seed).permutation(num_pages)``; each
    sequence takes the next cdiv(K_b, page_size) ids, so no page is shared;
    table columns past a sequence's pages hold a poison value that a correct
    reader never touches.
  * values: ``torch.Generator(device).manual_seed(seed)`` drawn in the order
    q, k_cache, v_cache, k_new, v_new; "uniform01" draws uniform [0, 1) in
    fp32 and rounds to the storage dtype (round-to-nearest-even); "normal3"
    draws 3 * N(0, 1) for q and keys (sharper softmax) and uniform [0, 1) for
    values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

POISON = {"neg1": -1, "intmax": 2**31 - 1, "big": 1 << 30, "zero": 0}

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


@dataclasses.dataclass
class Case:
    """One attention call's shapes and data recipe."""
    name: str
    q_lens: List[int]
    cache_seqlens: List[int]
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    dtype: str = "f16"
    page_size: Optional[int] = 16          # None -> contiguous cache
    contig_alloc: int = 0                  # contiguous mode: tokens per sequence
    append: bool = False                   # k_new / v_new given
    causal: bool = False
    num_splits: int = 0
    pool_factor: float = 2.0               # pool = factor x needed pages
    num_pages: Optional[int] = None        # explicit pool size
    table_width: Optional[int] = None      # explicit block_table width
    values: str = "uniform01"
    poison: str = "neg1"
    seed: int = 0
    max_seqlen_k_hint: int = 0             # host bound passed to the library (0: derive)

    @property
    def batch(self) -> int:
        return len(self.q_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def group(self) -> int:
        return self.num_heads_q // self.num_heads_kv

    def keys_visible(self) -> List[int]:
        """K_b: keys sequence b attends over (cache plus appended tokens)."""
        return [L + (n if self.append else 0) for L, n in zip(self.cache_seqlens, self.q_lens)]


@dataclasses.dataclass
class Inputs:
    case: Case
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]
    cache_seqlens: torch.Tensor
    cu_seqlens_q: torch.Tensor
    k_new: Optional[torch.Tensor]
    v_new: Optional[torch.Tensor]
    max_seqlen_q: int
    max_seqlen_k: int
    pages_of: List[np.ndarray]             # physical page ids of each sequence (paged mode)


def _fill(shape, gen, device, dtype, dist, chunk_elems=1 << 28):
    """Seeded fill in fp32, rounded to ``dtype``; drawn in row chunks."""
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        if dist == "uniform01":
            t = torch.rand(e - s, generator=gen, device=device, dtype=torch.float32)
        elif dist == "normal3":
            t = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32) * 3.0
        else:
            raise ValueError(dist)
        flat[s:e] = t.to(out.dtype)
    return out


def build_table(case: Case, rng: np.random.Generator):
    """Page ids per sequence, the pool size and the (poisoned) block table."""
    P = case.page_size
    Kb = case.keys_visible()
    need = [cdiv(k, P) for k in Kb]
    total_need = sum(need)
    num_pages = case.num_pages if case.num_pages is not None else max(
        1, int(math.ceil(case.pool_factor * total_need)))
    if total_need > num_pages:
        raise ValueError("pool too small for the visible keys")
    width = case.table_width if case.table_width is not None else max(1, max(need) if need else 1)
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((case.batch, width), POISON[case.poison], dtype=np.int32)
    pages_of = []
    off = 0
    for b, n in enumerate(need):
        ids = perm[off:off + n]
        off += n
        table[b, :n] = ids
        pages_of.append(ids)
    return num_pages, table, pages_of


def make_inputs(case: Case, device="cuda") -> Inputs:
    rng = np.random.default_rng(case.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(case.seed)
    B, hq, hkv, d = case.batch, case.num_heads_q, case.num_heads_kv, case.head_dim
    T = case.total_q
    Kb = case.keys_visible()
    qdist = "normal3" if case.values == "normal3" else "uniform01"

    if case.page_size is None:
        alloc = case.contig_alloc or max(1, max(Kb) if Kb else 1)
        if max(Kb, default=0) > alloc:
            raise ValueError("contiguous allocation too small")
        table = None
        pages_of = []
        pool_shape = (B, alloc, hkv, d)
    else:
        num_pages, table_np, pages_of = build_table(case, rng)
        table = torch.from_numpy(table_np).to(device)
        pool_shape = (num_pages, case.page_size, hkv, d)

    q = _fill((T, hq, d), gen, device, case.dtype, qdist)
    k_cache = _fill(pool_shape, gen, device, case.dtype, qdist)
    v_cache = _fill(pool_shape, gen, device, case.dtype, "uniform01")
    k_new = v_new = None
    if case.append:
        k_new = _fill((T, hkv, d), gen, device, case.dtype, qdist)
        v_new = _fill((T, hkv, d), gen, device, case.dtype, "uniform01")

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(case.q_lens)
    return Inputs(
        case=case, q=q, k_cache=k_cache, v_cache=v_cache, block_table=table,
        cache_seqlens=torch.tensor(case.cache_seqlens, dtype=torch.int32, device=device),
        cu_seqlens_q=torch.from_numpy(cu).to(device),
        k_new=k_new, v_new=v_new,
        max_seqlen_q=max(case.q_lens, default=0),
        max_seqlen_k=case.max_seqlen_k_hint or max(Kb, default=0),
        pages_of=pages_of,
    )


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of an fp16/bf16 tensor as a host numpy uint16 array."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype in (torch.float16, torch.bfloat16):
        return bits(t)
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# The five workload families.  Seeds: 1000 * family index + point index.
# ---------------------------------------------------------------------------

def tiny_decode(num_splits=0, seed=0, poison="neg1") -> Case:
    """batch 2, 4 q = 4 kv heads, head_dim 64, fp16, cache {37, 100}, page 16,
    32-page pool, table = a seeded permutation of distinct ids, one token per
    sequence, no causal mask."""
    return Case(name="tiny_decode", q_lens=[1, 1], cache_seqlens=[37, 100],
                num_heads_q=4, num_heads_kv=4, head_dim=64, dtype="f16", page_size=16,
                num_pages=32, table_width=7, causal=False, num_splits=num_splits,
                seed=seed, poison=poison)


def mha_decode(batch, ctx, page_size=16, append=False, seed=None) -> Case:
    """32 heads x 128, fp16, every sequence at `ctx` cached tokens, 1 new token."""
    return Case(name=f"mha_decode_b{batch}_ctx{ctx}_p{page_size}", q_lens=[1] * batch,
                cache_seqlens=[ctx] * batch, num_heads_q=32, num_heads_kv=32, head_dim=128,
                dtype="f16", page_size=page_size, append=append, causal=True,
                seed=1000 + (seed if seed is not None else batch + ctx))


def gqa_long_split(paged=True, num_splits=0, hint_alloc=True, seed=2000) -> Case:
    """batch 8, 64 q / 8 kv heads x 128, bf16, cache lengths uniform in
    [2048, 32768] inside a 131072-token allocation per sequence."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(2048, 32768, size=8, endpoint=True)]
    alloc = 131072
    return Case(name="gqa_long_split" + ("_paged" if paged else "_contig"), q_lens=[1] * 8,
                cache_seqlens=lens, num_heads_q=64, num_heads_kv=8, head_dim=128, dtype="bf16",
                page_size=16 if paged else None, contig_alloc=0 if paged else alloc,
                table_width=alloc // 16 if paged else None, causal=True,
                num_splits=num_splits, seed=seed,
                max_seqlen_k_hint=alloc if hint_alloc else max(lens))


def causal_prefill_append(nq, prefix="zero", seed=3000) -> Case:
    """batch 4, nq new tokens per sequence, 32 heads x 128, fp16, page 16, cache
    0 or uniform [0, 512], new K/V written into the pages, causal."""
    rng = np.random.default_rng(seed)
    L = [0] * 4 if prefix == "zero" else [int(x) for x in rng.integers(0, 512, 4, endpoint=True)]
    return Case(name=f"causal_prefill_append_nq{nq}_{prefix}", q_lens=[nq] * 4, cache_seqlens=L,
                num_heads_q=32, num_heads_kv=32, head_dim=128, dtype="f16", page_size=16,
                append=True, causal=True, seed=seed + nq)


def multi_token_decode(batch, ctx, q_len, heads_q=32, heads_kv=32, dtype="f16", seed=5000) -> Case:
    """speculative-decoding scoring: every sequence at cache `ctx` with `q_len`
    new tokens (q_len * heads_q / heads_kv <= 16 packed rows, so one decode
    unit each); head_dim 128, page 16, new K/V appended, causal."""
    return Case(name=f"multi_token_decode_b{batch}_ctx{ctx}_q{q_len}_h{heads_q}x{heads_kv}",
                q_lens=[q_len] * batch, cache_seqlens=[ctx] * batch, num_heads_q=heads_q,
                num_heads_kv=heads_kv, head_dim=128, dtype=dtype, page_size=16, append=True,
                causal=True, seed=seed + batch + ctx + q_len + heads_q)


def unified_varlen(nq, heads=32, head_dim=128, prefix=0, seed=4000) -> Case:
    """one prefill chunk of nq tokens (cache `prefix`) plus 64 decode sequences of
    one token each with cache uniform in [512, 4096]; fp16, page 16, causal,
    new K/V for every token appended."""
    rng = np.random.default_rng(seed)
    dec = [int(x) for x in rng.integers(512, 4096, 64, endpoint=True)]
    return Case(name=f"unified_varlen_nq{nq}_h{heads}x{head_dim}", q_lens=[nq] + [1] * 64,
                cache_seqlens=[prefix] + dec, num_heads_q=heads, num_heads_kv=heads,
                head_dim=head_dim, dtype="f16", page_size=16, append=True, causal=True,
                seed=seed + nq + heads)


def rotary_tables(rows: int, rotary_dim: int, dtype="f16", device="cuda", base=10000.0,
                  kind="angles", seed=0):
    """cos / sin tables [rows, rotary_dim / 2] in the storage dtype, inputs of
    the fused rotary embedding.  kind "angles": cos / sin of m * base^(-2i /
    rotary_dim) for position m and pair i (evaluated in fp64, rounded once);
    kind "random": seeded uniform [-1, 1) values (the rotation formula does not
    need a true rotation, and random tables exercise every table element)."""
    half = rotary_dim // 2
    if kind == "angles":
        theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
        ang = np.arange(rows, dtype=np.float64)[:, None] * theta[None, :]
        c, s = np.cos(ang), np.sin(ang)
    elif kind == "random":
        rng = np.random.default_rng(seed)
        c = rng.uniform(-1.0, 1.0, (rows, half))
        s = rng.uniform(-1.0, 1.0, (rows, half))
    else:
        raise ValueError(kind)
    td = TORCH_DTYPE[dtype]
    return (torch.from_numpy(c).to(td).to(device).contiguous(),
            torch.from_numpy(s).to(td).to(device).contiguous())
