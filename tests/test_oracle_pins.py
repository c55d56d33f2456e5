"""Pins for the CPU oracle: tie it to things other than itself.

Every test here runs on the CPU.  Together they are chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign, an off-by-one in the causal
limit, a transposed operand, a wrong page index or kv-head mapping, a broken
split merge) fails at least one of them:

* brute-force dense attention (numpy/scipy, no pages) on random tiny shapes;
* closed forms: zero query, a single visible key, constant values, and
  hand-derived worked examples in tests/golden/closed_forms.json;
* invariants: physical page relabelling, page size (16...256 and contiguous),
  poisoned table tails, split-and-combine versus unsplit, causal decode versus
  non-causal, non-causal invariance under key order, GQA versus MHA with
  repeated kv heads, varlen versus one call per
  sequence, (0, 0) padding slots;
* append: bit-exact against a numpy fancy-index scatter, every other slot
  untouched;
* exact widening of every fp16 / bf16 bit pattern against numpy / torch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import dense

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# Test-local construction of paged inputs from logical sequences.  This is the
# test's own numpy scatter, independent of the oracle's gather.
# ---------------------------------------------------------------------------

def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    t = t.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def random_case(rng, *, batch, q_lens, cached, hq, hkv, d, P, append, dtype, contiguous=False,
                dist="uniform", pool_extra=3, width_extra=2, poison=-1):
    """Logical per-sequence K/V, packed q / new rows, and a paged pool holding them."""
    K_b = [c + (n if append else 0) for c, n in zip(cached, q_lens)]
    T = int(sum(q_lens))

    def draw(shape):
        if dist == "uniform":
            return rng.random(shape)
        return 3.0 * rng.standard_normal(shape)

    q = to_bits(draw((T, hq, d)), dtype)
    k_log = [to_bits(draw((k, hkv, d)), dtype) for k in K_b]
    v_log = [to_bits(rng.random((k, hkv, d)), dtype) for k in K_b]
    cu = np.zeros(batch + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    k_new = v_new = None
    if append:
        k_new = np.concatenate([k_log[b][cached[b]:] for b in range(batch)], 0).reshape(T, hkv, d)
        v_new = np.concatenate([v_log[b][cached[b]:] for b in range(batch)], 0).reshape(T, hkv, d)
    if contiguous:
        alloc = max(K_b + [1]) + 3
        kc = to_bits(rng.random((batch, alloc, hkv, d)), dtype)
        vc = to_bits(rng.random((batch, alloc, hkv, d)), dtype)
        for b in range(batch):
            kc[b, :cached[b]] = k_log[b][:cached[b]]
            vc[b, :cached[b]] = v_log[b][:cached[b]]
        table = None
    else:
        need = [-(-k // P) for k in K_b]
        num_pages = sum(need) + pool_extra
        perm = rng.permutation(num_pages).astype(np.int32)
        width = max(need + [1]) + width_extra
        table = np.full((batch, width), poison, np.int32)
        kc = to_bits(rng.random((num_pages, P, hkv, d)), dtype)
        vc = to_bits(rng.random((num_pages, P, hkv, d)), dtype)
        off = 0
        for b in range(batch):
            table[b, :need[b]] = perm[off:off + need[b]]
            off += need[b]
            for j in range(cached[b]):          # only the cached prefix is pre-filled
                kc[table[b, j // P], j % P] = k_log[b][j]
                vc[table[b, j // P], j % P] = v_log[b][j]
    return dict(q=q, k_log=k_log, v_log=v_log, kc=kc, vc=vc, table=table,
                seqlens=np.asarray(cached, np.int32), cu=cu, k_new=k_new, v_new=v_new)


def run_oracle(c, *, dtype, causal, scale=None):
    return oracle.paged_attention(c["q"], c["kc"], c["vc"], c["table"], c["seqlens"], c["cu"],
                                  c["k_new"], c["v_new"], dtype=dtype, causal=causal,
                                  scale=scale)


def run_dense(c, *, dtype, causal, scale=None):
    q = from_bits(c["q"], dtype)
    ks = [from_bits(k, dtype) for k in c["k_log"]]
    vs = [from_bits(v, dtype) for v in c["v_log"]]
    return dense.attention_varlen(q, ks, vs, c["cu"], causal=causal, scale=scale)


def assert_close_lse(a, b, tol):
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    if fin.any():
        assert np.max(np.abs(a[fin] - b[fin])) <= tol


# ---------------------------------------------------------------------------
# Exact widening of the storage formats.
# ---------------------------------------------------------------------------

def test_widening_all_fp16_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.bits_to_double("f16", int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_widening_all_bf16_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bits_to_double("bf16", int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------------------
# Brute force.
# ---------------------------------------------------------------------------

@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), batch=st.integers(1, 4),
       heads=st.sampled_from([(1, 1), (2, 1), (4, 2), (4, 4), (8, 2), (6, 3)]),
       d=st.sampled_from([8, 16, 64]), P=st.sampled_from([16, 32, 64, 128, 256]),
       append=st.booleans(), causal=st.booleans(), dtype=st.sampled_from(["f16", "bf16"]),
       contiguous=st.booleans(), dist=st.sampled_from(["uniform", "normal3"]))
def test_oracle_matches_dense_bruteforce(seed, batch, heads, d, P, append, causal, dtype,
                                         contiguous, dist):
    rng = np.random.default_rng(seed)
    q_lens = [int(x) for x in rng.integers(0, 7, batch)]
    cached = [int(x) for x in rng.integers(0, 60, batch)]
    c = random_case(rng, batch=batch, q_lens=q_lens, cached=cached, hq=heads[0], hkv=heads[1],
                    d=d, P=P, append=append, dtype=dtype, contiguous=contiguous, dist=dist)
    out, lse, _, _ = run_oracle(c, dtype=dtype, causal=causal)
    ref_out, ref_lse = run_dense(c, dtype=dtype, causal=causal)
    assert np.max(np.abs(out - ref_out), initial=0.0) <= 1e-12 * max(1.0, np.abs(ref_out).max(initial=0))
    assert_close_lse(lse, ref_lse, 1e-11)


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------

def test_golden_closed_forms():
    data = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))
    for case in data["cases"]:
        dtype = "f16"
        k = np.asarray(case["k"], np.float64)[:, None, :]
        v = np.asarray(case["v"], np.float64)[:, None, :]
        q = np.asarray(case["q"], np.float64)[:, None, :]
        n_q, n_k = q.shape[0], k.shape[0]
        cached = case.get("cached", n_k if not case["causal"] else n_k - n_q)
        appended = n_k - cached
        assert appended in (0, n_q)
        P = 16
        kc = np.zeros((2, P, 1, 2), np.uint16)
        vc = np.zeros((2, P, 1, 2), np.uint16)
        kc[1, :cached, 0] = to_bits(k[:cached, 0], dtype)
        vc[1, :cached, 0] = to_bits(v[:cached, 0], dtype)
        table = np.array([[1]], np.int32)
        kn = vn = None
        if appended:
            kn = to_bits(k[cached:], dtype)
            vn = to_bits(v[cached:], dtype)
        out, lse, _, _ = oracle.paged_attention(
            to_bits(q, dtype), kc, vc, table, np.array([cached], np.int32),
            np.array([0, n_q], np.int32), kn, vn, dtype=dtype, causal=case["causal"],
            scale=case["scale"])
        exp_out = np.asarray(case["out"], np.float64).reshape(n_q, 2)
        exp_lse = np.asarray(case["lse"], np.float64).reshape(n_q)
        assert np.max(np.abs(out[:, 0, :] - exp_out)) < 1e-14, case["name"]
        assert np.max(np.abs(lse[:, 0] - exp_lse)) < 1e-14, case["name"]


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(11)
    c = random_case(rng, batch=3, q_lens=[1, 4, 2], cached=[5, 0, 33], hq=4, hkv=2, d=16, P=16,
                    append=True, dtype="f16")
    c["q"][:] = 0
    out, lse, _, _ = run_oracle(c, dtype="f16", causal=causal)
    for b in range(3):
        n_q = c["cu"][b + 1] - c["cu"][b]
        K = len(c["v_log"][b])
        V = from_bits(c["v_log"][b], "f16")          # [K, Hkv, D]
        for i in range(n_q):
            n_vis = (K - n_q + i + 1) if causal else K
            row = c["cu"][b] + i
            for h in range(4):
                g = h // 2
                assert abs(lse[row, h] - math.log(n_vis)) < 1e-14
                assert np.max(np.abs(out[row, h] - V[:n_vis, g].mean(0))) < 1e-14


def test_single_visible_key_returns_that_value():
    rng = np.random.default_rng(12)
    # cache empty, 3 new tokens, causal: token 0 sees exactly key 0.
    c = random_case(rng, batch=2, q_lens=[3, 1], cached=[0, 0], hq=2, hkv=2, d=32, P=16,
                    append=True, dtype="bf16", dist="normal3")
    out, lse, _, _ = run_oracle(c, dtype="bf16", causal=True)
    for b, row in ((0, 0), (1, 3)):
        V = from_bits(c["v_log"][b], "bf16")
        K = from_bits(c["k_log"][b], "bf16")
        q = from_bits(c["q"], "bf16")[row]
        for h in range(2):
            assert np.array_equal(out[row, h], V[0, h])
            assert abs(lse[row, h] - (q[h] @ K[0, h]) / math.sqrt(32)) < 1e-12


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(13)
    c = random_case(rng, batch=2, q_lens=[2, 5], cached=[40, 17], hq=4, hkv=4, d=16, P=32,
                    append=True, dtype="f16", dist="normal3")
    const = to_bits(np.full((1,), 0.375), "f16")[0]
    c["vc"][:] = const
    c["v_new"][:] = const
    out, _, _, _ = run_oracle(c, dtype="f16", causal=True)
    assert np.max(np.abs(out - 0.375)) < 1e-15


def test_empty_key_set_gives_zero_and_neg_inf():
    rng = np.random.default_rng(14)
    c = random_case(rng, batch=2, q_lens=[1, 2], cached=[0, 9], hq=2, hkv=1, d=8, P=16,
                    append=False, dtype="f16")
    out, lse, _, _ = run_oracle(c, dtype="f16", causal=False)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1:]))
    # causal with more new tokens than keys: the first rows see nothing
    c2 = random_case(rng, batch=1, q_lens=[4], cached=[2], hq=1, hkv=1, d=8, P=16,
                     append=False, dtype="f16")
    out2, lse2, _, _ = run_oracle(c2, dtype="f16", causal=True)
    assert np.all(np.isneginf(lse2[:2])) and np.all(out2[:2] == 0.0)
    assert np.all(np.isfinite(lse2[2:]))


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------

def test_physical_page_relabelling_is_bit_invariant():
    rng = np.random.default_rng(21)
    c = random_case(rng, batch=3, q_lens=[1, 6, 2], cached=[50, 30, 77], hq=4, hkv=2, d=64,
                    P=16, append=True, dtype="f16", dist="normal3")
    out, lse, kc, vc = run_oracle(c, dtype="f16", causal=True)
    n = c["kc"].shape[0]
    pi = rng.permutation(n).astype(np.int32)
    c2 = dict(c)
    c2["kc"] = np.empty_like(c["kc"])
    c2["vc"] = np.empty_like(c["vc"])
    c2["kc"][pi] = c["kc"]
    c2["vc"][pi] = c["vc"]
    t = c["table"].copy()
    live = t >= 0
    t[live] = pi[t[live]]
    c2["table"] = t
    out2, lse2, kc2, vc2 = run_oracle(c2, dtype="f16", causal=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    assert np.array_equal(kc2[pi], kc) and np.array_equal(vc2[pi], vc)


def test_page_size_and_contiguous_give_identical_bits():
    results = []
    for P in (16, 32, 64, 128, 256, None):
        rng = np.random.default_rng(22)    # same logical data every time
        c = random_case(rng, batch=2, q_lens=[3, 1], cached=[100, 260], hq=2, hkv=2, d=16,
                        P=P or 16, append=True, dtype="bf16", contiguous=P is None)
        out, lse, _, _ = run_oracle(c, dtype="bf16", causal=True)
        results.append((out, lse))
    for out, lse in results[1:]:
        assert np.array_equal(out, results[0][0]) and np.array_equal(lse, results[0][1])


@pytest.mark.parametrize("poison", [-1, 2**31 - 1, 1 << 30, 0])
def test_poisoned_table_tail_is_never_read(poison):
    rng = np.random.default_rng(23)
    base = random_case(rng, batch=2, q_lens=[1, 3], cached=[31, 16], hq=2, hkv=2, d=16, P=16,
                       append=True, dtype="f16", poison=-1)
    ref = run_oracle(base, dtype="f16", causal=True)
    c = dict(base)
    t = base["table"].copy()
    t[t == -1] = poison
    c["table"] = t
    got = run_oracle(c, dtype="f16", causal=True)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)


def test_out_of_pool_page_inside_the_live_range_is_an_error():
    rng = np.random.default_rng(24)
    c = random_case(rng, batch=1, q_lens=[1], cached=[20], hq=1, hkv=1, d=8, P=16,
                    append=False, dtype="f16")
    c["table"][0, 1] = 10**6
    with pytest.raises(ValueError):
        run_oracle(c, dtype="f16", causal=False)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 128])
def test_split_and_combine_equals_unsplit(S):
    rng = np.random.default_rng(25 + S)
    c = random_case(rng, batch=3, q_lens=[1, 2, 5], cached=[90, 7, 200], hq=4, hkv=1, d=16,
                    P=16, append=True, dtype="f16", dist="normal3")
    out, lse, kc, vc = run_oracle(c, dtype="f16", causal=True)
    K_b = [len(k) for k in c["k_log"]]
    parts_o, parts_l = [], []
    for s in range(S):
        # tile-aligned windows of 32 keys, some of them empty when S is large
        tiles = [-(-k // 32) for k in K_b]
        chunk = [-(-t // S) for t in tiles]
        kb = np.array([s * ch * 32 for ch in chunk], np.int32)
        ke = np.array([min((s + 1) * ch * 32, k) for ch, k in zip(chunk, K_b)], np.int32)
        o, l = oracle.attention(c["q"], kc, vc, c["table"], c["seqlens"], c["cu"], dtype="f16",
                                appended=True, causal=True, key_begin=kb, key_end=ke)
        parts_o.append(o.reshape(-1, 16))
        parts_l.append(l.reshape(-1))
    mo, ml = oracle.combine(np.stack(parts_o), np.stack(parts_l))
    assert np.max(np.abs(mo - out.reshape(-1, 16))) <= 1e-12
    assert_close_lse(ml, lse.reshape(-1), 1e-12)


def test_combine_of_all_empty_splits():
    o = np.zeros((3, 2, 4))
    l = np.full((3, 2), -np.inf)
    mo, ml = oracle.combine(o, l)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))


def test_causal_decode_equals_noncausal():
    rng = np.random.default_rng(26)
    for append in (False, True):
        c = random_case(rng, batch=4, q_lens=[1, 1, 1, 1], cached=[1, 17, 64, 100], hq=8, hkv=2,
                        d=32, P=16, append=append, dtype="f16", dist="normal3")
        a = run_oracle(c, dtype="f16", causal=True)
        b = run_oracle(c, dtype="f16", causal=False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_noncausal_result_ignores_key_order():
    # without the causal mask attention is a function of the key set: shuffling
    # the (K, V) rows within each sequence changes the fp64 result only by
    # summation order
    rng = np.random.default_rng(29)
    c = random_case(rng, batch=3, q_lens=[2, 1, 3], cached=[50, 7, 130], hq=4, hkv=2, d=32, P=16,
                    append=False, dtype="bf16", contiguous=True, dist="normal3")
    a_out, a_lse, _, _ = run_oracle(c, dtype="bf16", causal=False)
    kc, vc = c["kc"].copy(), c["vc"].copy()
    for b, L in enumerate(c["seqlens"]):
        perm = rng.permutation(int(L))
        kc[b, :L] = c["kc"][b, perm]
        vc[b, :L] = c["vc"][b, perm]
    b_out, b_lse, _, _ = oracle.paged_attention(c["q"], kc, vc, None, c["seqlens"], c["cu"],
                                                dtype="bf16", causal=False)
    assert np.max(np.abs(a_out - b_out)) <= 1e-13 * max(1.0, np.abs(a_out).max())
    assert np.max(np.abs(a_lse - b_lse)) <= 1e-13 * max(1.0, np.abs(a_lse).max())
    # a causal call does depend on the order (a planted check that the shuffle bites)
    c_out = oracle.paged_attention(c["q"], kc, vc, None, c["seqlens"], c["cu"], dtype="bf16",
                                   causal=True)[0]
    d_out = run_oracle(c, dtype="bf16", causal=True)[0]
    assert np.max(np.abs(c_out - d_out)) > 1e-6


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(27)
    G = 4
    c = random_case(rng, batch=2, q_lens=[3, 1], cached=[20, 45], hq=8, hkv=2, d=16, P=16,
                    append=True, dtype="bf16", dist="normal3")
    gqa = run_oracle(c, dtype="bf16", causal=True)
    m = dict(c)
    for key in ("kc", "vc", "k_new", "v_new"):
        m[key] = np.repeat(c[key], G, axis=-2)
    mha = run_oracle(m, dtype="bf16", causal=True)
    assert np.array_equal(gqa[0], mha[0]) and np.array_equal(gqa[1], mha[1])


def test_varlen_equals_one_call_per_sequence():
    rng = np.random.default_rng(28)
    q_lens, cached = [4, 1, 0, 7], [10, 33, 5, 0]
    c = random_case(rng, batch=4, q_lens=q_lens, cached=cached, hq=2, hkv=2, d=16, P=16,
                    append=True, dtype="f16", dist="normal3")
    out, lse, kc, vc = run_oracle(c, dtype="f16", causal=True)
    for b in range(4):
        s, e = c["cu"][b], c["cu"][b + 1]
        one = dict(q=c["q"][s:e], kc=c["kc"], vc=c["vc"], table=c["table"][b:b + 1],
                   seqlens=c["seqlens"][b:b + 1], cu=np.array([0, e - s], np.int32),
                   k_new=c["k_new"][s:e], v_new=c["v_new"][s:e])
        o1, l1, _, _ = run_oracle(one, dtype="f16", causal=True)
        assert np.array_equal(o1, out[s:e]) and np.array_equal(l1, lse[s:e])


def test_zero_length_padding_slots_are_no_ops():
    rng = np.random.default_rng(29)
    c = random_case(rng, batch=2, q_lens=[5, 1], cached=[3, 40], hq=2, hkv=2, d=16, P=16,
                    append=True, dtype="f16")
    out, lse, kc, vc = run_oracle(c, dtype="f16", causal=True)
    p = dict(c)
    p["cu"] = np.concatenate([c["cu"], [c["cu"][-1]] * 3]).astype(np.int32)
    p["seqlens"] = np.concatenate([c["seqlens"], [0, 0, 0]]).astype(np.int32)
    p["table"] = np.concatenate([c["table"], np.full((3, c["table"].shape[1]), -1, np.int32)])
    out2, lse2, kc2, vc2 = run_oracle(p, dtype="f16", causal=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)


# ---------------------------------------------------------------------------
# Append.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P", [16, 64, 256])
def test_append_matches_numpy_scatter(P):
    rng = np.random.default_rng(30 + P)
    c = random_case(rng, batch=3, q_lens=[5, 0, 40], cached=[14, 3, 250], hq=2, hkv=2, d=16,
                    P=P, append=True, dtype="f16")
    kc, vc = oracle.kv_append(c["kc"], c["vc"], c["table"], c["seqlens"], c["cu"],
                              c["k_new"], c["v_new"])
    ek, ev = c["kc"].copy(), c["vc"].copy()
    written = np.zeros(ek.shape[:2], bool)
    for b in range(3):
        n = c["cu"][b + 1] - c["cu"][b]
        pos = c["seqlens"][b] + np.arange(n)
        pages = c["table"][b, pos // P]
        ek[pages, pos % P] = c["k_new"][c["cu"][b]:c["cu"][b + 1]]
        ev[pages, pos % P] = c["v_new"][c["cu"][b]:c["cu"][b + 1]]
        written[pages, pos % P] = True
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    assert np.array_equal(kc[~written], c["kc"][~written])
    # and the appended rows are exactly the logical sequence tail
    for b in range(3):
        for j in range(c["seqlens"][b], len(c["k_log"][b])):
            assert np.array_equal(kc[c["table"][b, j // P], j % P], c["k_log"][b][j])


def test_append_contiguous_mode():
    rng = np.random.default_rng(40)
    c = random_case(rng, batch=2, q_lens=[3, 2], cached=[4, 0], hq=2, hkv=2, d=8, P=16,
                    append=True, dtype="bf16", contiguous=True)
    kc, vc = oracle.kv_append(c["kc"], c["vc"], None, c["seqlens"], c["cu"], c["k_new"], c["v_new"])
    for b in range(2):
        L = c["seqlens"][b]
        n = c["cu"][b + 1] - c["cu"][b]
        assert np.array_equal(kc[b, L:L + n], c["k_new"][c["cu"][b]:c["cu"][b + 1]])
        assert np.array_equal(kc[b, L + n:], c["kc"][b, L + n:])
