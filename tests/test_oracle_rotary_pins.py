"""Pins for the oracle's rotary position embedding (``oracle/rotary.py``).

CPU only.  A plausible slip in the rotation - a dropped term, a wrong sign,
the wrong pairing, a wrong table index or position, a wrong rounding - fails
at least one of these:

* the hand-worked example in tests/golden/rotary_worked.json (both pairings,
  several table rows, a position past the table);
* norm preservation of every pair under true rotation tables;
* the relative-position property: rotated q_m . k_n depends only on m - n;
* composition: rotating by m and then by n equals rotating by m + n;
* the two pairings are one rotation seen through a fixed permutation;
* correct rounding of the 16-bit result against exact rational arithmetic;
* the positions the attention call gives each packed row, against a list
  written out here, and the call equals attention on pre-rotated inputs.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import rotary

HERE = os.path.dirname(os.path.abspath(__file__))


def to_bits(x, dtype):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    t = t.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(b, dtype):
    b = np.asarray(b, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def angle_tables(rows, rotary_dim, base=10000.0):
    """cos / sin of m * base^(-2i / rotary_dim) in fp64 (the usual RoPE angles)."""
    half = rotary_dim // 2
    theta = base ** (-2.0 * np.arange(half) / rotary_dim)
    ang = np.arange(rows)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_golden_worked_example(dtype):
    g = json.load(open(os.path.join(HERE, "golden", "rotary_worked.json")))
    x = np.asarray(g["x"], np.float64)
    cos_b = to_bits(g["cos"], dtype)
    sin_b = to_bits(g["sin"], dtype)
    # four copies of the row at positions 2, 0, 1 and 3 (3 is past the table)
    xb = np.tile(to_bits(x, dtype)[None, None, :], (4, 1, 1))
    pos = np.array([g["position"], 0, 1, 3])
    half = rotary.rotate_bits(xb, cos_b, sin_b, pos, dtype=dtype, interleaved=False)
    inter = rotary.rotate_bits(xb, cos_b, sin_b, pos, dtype=dtype, interleaved=True)
    assert np.array_equal(from_bits(half[0, 0], dtype), g["half_split"]["out"])
    assert np.array_equal(from_bits(inter[0, 0], dtype), g["interleaved"]["out"])
    for r in (half, inter):
        assert np.array_equal(from_bits(r[1, 0], dtype), g["position_0"]["out"])
        assert np.array_equal(r[3], xb[3])          # position outside the table: untouched
    assert np.array_equal(from_bits(half[2, 0], dtype), g["position_1_half_split"]["out"])


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("rotary_dim,d", [(16, 16), (32, 64), (64, 64), (128, 128)])
def test_pair_norms_are_preserved(interleaved, rotary_dim, d):
    rng = np.random.default_rng(11)
    cos, sin = angle_tables(300, rotary_dim)
    x = rng.standard_normal((20, 3, d))
    pos = rng.integers(0, 300, 20)
    y = rotary.rotate(x, cos, sin, pos, interleaved=interleaved)
    f, s = rotary.pair_index(rotary_dim, interleaved)
    n0 = x[:, :, f] ** 2 + x[:, :, s] ** 2
    n1 = y[:, :, f] ** 2 + y[:, :, s] ** 2
    assert np.max(np.abs(n1 - n0) / (n0 + 1e-300)) < 1e-13
    assert np.array_equal(y[:, :, rotary_dim:], x[:, :, rotary_dim:])
    # a genuine change happened wherever the angle is not a multiple of 2 pi
    assert not np.allclose(y[pos > 0][:, :, :rotary_dim], x[pos > 0][:, :, :rotary_dim])


@pytest.mark.parametrize("interleaved", [False, True])
def test_dot_products_depend_on_relative_position(interleaved):
    rng = np.random.default_rng(12)
    rd = 64
    cos, sin = angle_tables(600, rd)
    q = rng.standard_normal((1, 1, rd))
    k = rng.standard_normal((1, 1, rd))

    def score(m, n):
        qm = rotary.rotate(q, cos, sin, [m], interleaved=interleaved)
        kn = rotary.rotate(k, cos, sin, [n], interleaved=interleaved)
        return float(np.sum(qm * kn))

    for m, n in [(5, 3), (100, 0), (17, 40), (0, 0)]:
        base = score(m, n)
        for s in (1, 7, 250):
            assert abs(score(m + s, n + s) - base) <= 1e-11 * max(1.0, abs(base))
    # and it does depend on the offset
    assert abs(score(9, 0) - score(0, 0)) > 1e-3


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotations_compose_by_adding_positions(interleaved):
    rng = np.random.default_rng(13)
    rd = 32
    cos, sin = angle_tables(200, rd)
    x = rng.standard_normal((6, 2, 48))
    m = np.array([0, 1, 5, 30, 60, 99])
    n = np.array([3, 0, 8, 41, 60, 100])
    twice = rotary.rotate(rotary.rotate(x, cos, sin, m, interleaved=interleaved), cos, sin, n,
                          interleaved=interleaved)
    once = rotary.rotate(x, cos, sin, m + n, interleaved=interleaved)
    assert np.max(np.abs(twice - once)) < 1e-12


def test_pairings_are_one_rotation_under_a_permutation():
    rng = np.random.default_rng(14)
    rd, d = 32, 40
    cos, sin = angle_tables(50, rd)
    x = rng.standard_normal((5, 2, d))
    pos = rng.integers(0, 50, 5)
    half = rd // 2
    # element i of the half-split layout sits at 2i (i < half) or 2(i-half)+1
    order = np.concatenate([np.ravel(np.column_stack([np.arange(half), np.arange(half) + half])),
                            np.arange(rd, d)])
    y_half = rotary.rotate(x, cos, sin, pos, interleaved=False)
    y_inter = rotary.rotate(x[:, :, order], cos, sin, pos, interleaved=True)
    assert np.array_equal(y_inter, y_half[:, :, order])


def _neighbours16(v, dtype):
    """The 16-bit values on either side of the finite 16-bit value v (values
    here stay far below the largest finite one)."""
    b = int(to_bits(np.array([v]), dtype)[0])
    sign, mag = b & 0x8000, b & 0x7FFF
    pats = [0x0001, 0x8001] if mag == 0 else [sign | (mag + 1), sign | (mag - 1)]
    return from_bits(np.array(pats, np.uint16), dtype)


def _is_nearest(exact: Fraction, got: float, neighbours) -> bool:
    d0 = abs(exact - Fraction(got))
    return all(d0 <= abs(exact - Fraction(float(n))) for n in neighbours)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounding_against_exact_rationals(dtype):
    """Each rotated element is a nearest fp32 of the exact value, rounded to a
    nearest 16-bit value; checked with Fractions and neighbour comparisons, no
    library rounding involved."""
    rng = np.random.default_rng(15)
    rd = 16
    n = 40
    xb = to_bits(rng.standard_normal((n, 1, rd)) * 4, dtype)
    cb = to_bits(rng.uniform(-1, 1, (n, rd // 2)), dtype)
    sb = to_bits(rng.uniform(-1, 1, (n, rd // 2)), dtype)
    pos = np.arange(n)
    for inter in (False, True):
        got = from_bits(rotary.rotate_bits(xb, cb, sb, pos, dtype=dtype, interleaved=inter), dtype)
        x = from_bits(xb, dtype)
        c = from_bits(cb, dtype)
        s = from_bits(sb, dtype)
        f_idx, s_idx = rotary.pair_index(rd, inter)
        for r in range(n):
            for i in range(rd // 2):
                a, b = Fraction(x[r, 0, f_idx[i]]), Fraction(x[r, 0, s_idx[i]])
                ci, si = Fraction(c[r, i]), Fraction(s[r, i])
                for exact, idx in ((a * ci - b * si, f_idx[i]), (b * ci + a * si, s_idx[i])):
                    f32 = np.float32(float(exact))
                    nb32 = [np.nextafter(f32, np.float32(np.inf)),
                            np.nextafter(f32, np.float32(-np.inf))]
                    assert _is_nearest(exact, float(f32), nb32)
                    out = got[r, 0, idx]
                    assert _is_nearest(Fraction(float(f32)), out, _neighbours16(out, dtype))


def test_token_positions_against_a_written_out_list():
    seq = np.array([5, 0, 7, 2], np.int32)
    cu = np.array([0, 2, 5, 5, 6], np.int32)      # q_lens 2, 3, 0, 1
    assert rotary.token_positions(seq, cu, appended=True).tolist() == [5, 6, 0, 1, 2, 2]
    assert rotary.token_positions(seq, cu, appended=False).tolist() == [3, 4, -3, -2, -1, 1]
    assert rotary.token_positions(seq, cu, appended=True, total=8).tolist() == \
        [5, 6, 0, 1, 2, 2, -1, -1]


@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("interleaved", [False, True])
def test_attention_call_rotates_each_row_at_its_position(append, interleaved):
    """paged_attention(rotary=...) equals attention on inputs rotated here at
    positions written out by hand, and the appended keys are stored rotated."""
    dtype = "bf16"
    rng = np.random.default_rng(16 + append + 2 * interleaved)
    P, hq, hkv, d, rd = 16, 4, 2, 32, 16
    cached = [20, 3, 40]
    q_lens = [3, 1, 2]
    cu = np.array([0, 3, 4, 6], np.int32)
    # positions: appended -> cached + i; otherwise cached - q_len + i
    pos = ([20, 21, 22, 3, 40, 41] if append else [17, 18, 19, 2, 38, 39])
    num_pages = 12
    kc = to_bits(rng.standard_normal((num_pages, P, hkv, d)), dtype)
    vc = to_bits(rng.random((num_pages, P, hkv, d)), dtype)
    table = np.array([[0, 1, -1, -1], [2, -1, -1, -1], [3, 4, 5, -1]], np.int32)
    q = to_bits(rng.standard_normal((6, hq, d)), dtype)
    kn = to_bits(rng.standard_normal((6, hkv, d)), dtype) if append else None
    vn = to_bits(rng.random((6, hkv, d)), dtype) if append else None
    cos, sin = angle_tables(64, rd)
    tab = (to_bits(cos, dtype), to_bits(sin, dtype), interleaved)
    seq = np.array(cached, np.int32)
    out, lse, kc1, vc1 = oracle.paged_attention(q, kc, vc, table, seq, cu, kn, vn, dtype=dtype,
                                                causal=True, rotary=tab)
    q_r = rotary.rotate_bits(q, tab[0], tab[1], pos, dtype=dtype, interleaved=interleaved)
    kn_r = (rotary.rotate_bits(kn, tab[0], tab[1], pos, dtype=dtype, interleaved=interleaved)
            if append else None)
    ref_out, ref_lse, ref_kc, ref_vc = oracle.paged_attention(q_r, kc, vc, table, seq, cu, kn_r,
                                                              vn, dtype=dtype, causal=True)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
    assert np.array_equal(kc1, ref_kc) and np.array_equal(vc1, ref_vc)
    assert not np.array_equal(q_r, q)
    if append:
        # the stored row of sequence 0's token 1 (position 21: page 1, slot 5)
        assert np.array_equal(kc1[1, 5], kn_r[1]) and not np.array_equal(kc1[1, 5], kn[1])
        assert np.array_equal(vc1[1, 5], vn[1])
