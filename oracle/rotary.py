"""Rotary position embedding, CPU oracle (numpy fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library never
imports this module.

The flash-attention thread "Add support for small page sizes" reports that the
paged key/value-cache kernel also applies a fused rotary embedding (RoPE) to
the incoming queries and keys.  The pages give no formula for it, so this is
the standard rotary position embedding (Su et al., RoFormer): the leading
``rotary_dim`` elements of every head row form rotary_dim/2 pairs, and pair i
of a token at position m is turned by the angle whose cosine and sine are
``cos[m, i]`` and ``sin[m, i]`` (tables the caller supplies):

    a' = a * cos - b * sin
    b' = b * cos + a * sin

Two pairings are in use: the half-split form pairs elements (i, i + rotary_dim/2)
(GPT-NeoX layout); the interleaved form pairs (2i, 2i + 1) (GPT-J layout).
Elements at or past ``rotary_dim`` pass through unchanged.

Readings where the pages are silent:
  * position of a token: the position it has in its sequence, K_b - q_len_b + i
    for new token i of sequence b (K_b keys attended, bottom-right alignment) -
    cache_seqlens[b] + i when the call appends the new rows; queries and new
    keys of one token share it;
  * a token whose position falls outside the table (negative or >= rows) is
    left unrotated;
  * precision: the tables come in the element type; the rotation is evaluated
    exactly (both products of 16-bit values are exact in fp64, and so is their
    difference up to one final rounding that never changes the fp32 result),
    rounded to fp32 and then to the element type, round-to-nearest-even each
    time.  That is the value fp32 arithmetic gives on a device, where the two
    products are exact in fp32 as well.

Pins (``tests/test_oracle_pins.py``): a hand-worked example of both pairings
(``tests/golden/rotary_worked.json``), norm preservation per pair, the
relative-position property of rotated dot products, composition of rotations,
position 0 as the identity, the permutation that maps one pairing onto the
other, correct rounding against exact rational arithmetic, and the positions
the attention call assigns against a test-local list.
"""
from __future__ import annotations

import numpy as np
import torch


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit patterns (uint16) -> float64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype in ("f16", "fp16", "float16"):
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> fp32 -> 16-bit patterns, round-to-nearest-even at both steps."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype in ("f16", "fp16", "float16"):
        return f32.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(np.ascontiguousarray(f32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pair_index(rotary_dim: int, interleaved: bool):
    """Element indices (first, second) of the rotary_dim/2 pairs of a head row."""
    half = rotary_dim // 2
    i = np.arange(half)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + half


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, positions, *, interleaved: bool):
    """Exact (fp64) rotation of x [n, H, D] at positions [n].

    cos / sin: float64 [rows, rotary_dim / 2].  Rows whose position lies outside
    [0, rows) come back unchanged, as do elements at or past rotary_dim.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    rows, half = cos.shape
    rotary_dim = 2 * half
    if x.shape[-1] < rotary_dim:
        raise ValueError("rotary_dim exceeds the head size")
    pos = np.asarray(positions, dtype=np.int64)
    live = (pos >= 0) & (pos < rows)
    first, second = pair_index(rotary_dim, interleaved)
    c = cos[pos[live]][:, None, :]            # [n_live, 1, half]
    s = sin[pos[live]][:, None, :]
    a = x[live][:, :, first]
    b = x[live][:, :, second]
    sub = x[live]
    sub[:, :, first] = a * c - b * s
    sub[:, :, second] = b * c + a * s
    x[live] = sub
    return x


def rotate_bits(x_bits, cos_bits, sin_bits, positions, *, dtype: str, interleaved: bool):
    """The rotation on 16-bit patterns: widen, rotate exactly, round (fp32, then
    the element type).  Elements that are not rotated keep their bit patterns."""
    xb = np.array(x_bits, dtype=np.uint16, copy=True)
    half = np.asarray(cos_bits).shape[1]
    rot = rotate(widen(xb, dtype), widen(cos_bits, dtype), widen(sin_bits, dtype), positions,
                 interleaved=interleaved)
    pos = np.asarray(positions, dtype=np.int64)
    live = (pos >= 0) & (pos < np.asarray(cos_bits).shape[0])
    sub = xb[live]
    sub[:, :, :2 * half] = narrow(rot[live][:, :, :2 * half], dtype)
    xb[live] = sub
    return xb


def token_positions(cache_seqlens, cu_seqlens_q, *, appended: bool, total=None) -> np.ndarray:
    """Position of every packed new row: K_b - q_len_b + i for token i of
    sequence b; rows past cu_seqlens_q[batch] (static padding) get -1."""
    seq = np.asarray(cache_seqlens, dtype=np.int64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    total = int(cu[-1]) if total is None else int(total)
    pos = np.full(total, -1, dtype=np.int64)
    for b in range(seq.shape[0]):
        n = int(cu[b + 1] - cu[b])
        k_b = int(seq[b]) + (n if appended else 0)
        pos[cu[b]:cu[b + 1]] = k_b - n + np.arange(n)
    return pos
