"""CPU fp64 oracle for the paged KV-cache attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``paged_kv_cache_lds_amd``) never imports it, and the two share no
code: this side is plain C (``paged_attn_oracle.c``, built with gcc) plus the
numpy brute force in ``dense.py``.

Every function takes host numpy arrays.  fp16/bf16 tensors are passed as their
raw 16-bit patterns (``numpy.uint16``); the C code widens them exactly to
double.  Results are unrounded fp64.

Pins (in ``tests/test_oracle_pins.py``): brute-force dense attention on tiny
inputs, closed forms (zero query, one key, constant values, hand-computed
two-key cases under ``tests/golden/``), invariance under physical page
relabelling, page size and poisoned table tails, split-combine equals unsplit,
causal decode equals non-causal, GQA equals MHA with repeated kv heads,
varlen equals per-sequence calls, and bit-exact append against a numpy
scatter.  The rotary embedding (``rotary.py``) has pins of its own, listed in
that module.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

from . import rotary as _rotary

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "paged_attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
_DTYPES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_bits_to_double.restype = ctypes.c_double
        lib.oracle_bits_to_double.argtypes = [i, ctypes.c_uint16]
        lib.oracle_kv_append.restype = i
        lib.oracle_kv_append.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p, p, p]
        lib.oracle_attention.restype = i
        lib.oracle_attention.argtypes = [i, i, i, i, i, i, i, i, i, p, p, p, p, p, p,
                                         i, i, ctypes.c_double, p, p, p, p, i]
        lib.oracle_combine.restype = None
        lib.oracle_combine.argtypes = [i, ctypes.c_long, i, p, p, p, p]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dt)


def bits_to_double(dtype: str, bits: int) -> float:
    return _load().oracle_bits_to_double(_DTYPES[dtype], int(bits))


def kv_append(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, k_new, v_new,
              page_size=None, contig_alloc=0, rotary=None, dtype="f16"):
    """Return copies of the pools with the new rows written (bit copies).

    k_cache/v_cache: uint16 [num_pages, P, Hkv, D] (paged) or
    [batch, alloc, Hkv, D] (contiguous, block_table None).  With
    ``rotary=(cos_bits, sin_bits, interleaved)`` the new keys are first rotated
    at their positions cache_seqlens[b] + i (``oracle.rotary``); values never are.
    """
    kc = np.array(k_cache, dtype=np.uint16, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.uint16, copy=True, order="C")
    bt = _c(block_table, np.int32)
    seq = _c(cache_seqlens, np.int32)
    cu = _c(cu_seqlens_q, np.int32)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    if rotary is not None:
        cos_b, sin_b, inter = rotary
        pos = _rotary.token_positions(seq, cu, appended=True, total=kn.shape[0])
        kn = np.ascontiguousarray(_rotary.rotate_bits(kn, cos_b, sin_b, pos, dtype=dtype,
                                                      interleaved=bool(inter)))
    batch = seq.shape[0]
    if bt is None:
        num_pages, P, hkv, d = kc.shape[0], kc.shape[1], kc.shape[2], kc.shape[3]
        contig_alloc = P
        P, num_pages, mpp = 1, 0, 0
    else:
        num_pages, P, hkv, d = kc.shape
        mpp = bt.shape[1]
    rc = _load().oracle_kv_append(batch, hkv, d, P, num_pages, mpp, contig_alloc,
                                  _ptr(kc), _ptr(vc), _ptr(bt), _ptr(seq), _ptr(cu),
                                  _ptr(kn), _ptr(vn))
    if rc != 0:
        raise ValueError("oracle_kv_append: target row outside the pool")
    return kc, vc


def attention(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q, *,
              dtype="f16", appended=False, causal=False, scale=None,
              key_begin=None, key_end=None, threads=0):
    """Gather-then-softmax attention in fp64 (pool already holds any new rows).

    q: uint16 [total_q, Hq, D].  Returns (out float64 [total_q, Hq, D],
    lse float64 [total_q, Hq]).
    """
    qb = _c(q, np.uint16)
    kc = _c(k_cache, np.uint16)
    vc = _c(v_cache, np.uint16)
    bt = _c(block_table, np.int32)
    seq = _c(cache_seqlens, np.int32)
    cu = _c(cu_seqlens_q, np.int32)
    total_q, hq, d = qb.shape
    if d > 512:
        raise ValueError("oracle supports head_dim <= 512")
    if bt is None:
        batch_alloc, alloc, hkv, _ = kc.shape
        P, num_pages, mpp, contig = 1, 0, 0, alloc
    else:
        num_pages, P, hkv, _ = kc.shape
        mpp, contig = bt.shape[1], 0
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kb = _c(key_begin, np.int32)
    ke = _c(key_end, np.int32)
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    lse = np.zeros((total_q, hq), dtype=np.float64)
    rc = _load().oracle_attention(_DTYPES[dtype], seq.shape[0], hq, hkv, d, P, num_pages, mpp,
                                  contig, _ptr(qb), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(seq),
                                  _ptr(cu), int(bool(appended)), int(bool(causal)), float(scale),
                                  _ptr(kb), _ptr(ke), _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle_attention: key row outside the pool")
    return out, lse


def paged_attention(q, k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q,
                    k_new=None, v_new=None, *, dtype="f16", causal=False, scale=None,
                    threads=0, rotary=None):
    """The whole call: rotate (if ``rotary``), append (if k_new/v_new), then attend.

    ``rotary=(cos_bits, sin_bits, interleaved)`` applies the rotary embedding of
    ``oracle.rotary`` to the queries and the new keys, each token at its
    position K_b - q_len_b + i, before anything else.
    Returns (out, lse, k_cache_after, v_cache_after).
    """
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if rotary is not None:
        cos_b, sin_b, inter = rotary
        pos = _rotary.token_positions(cache_seqlens, cu_seqlens_q, appended=k_new is not None,
                                      total=np.asarray(q).shape[0])
        q = _rotary.rotate_bits(q, cos_b, sin_b, pos, dtype=dtype, interleaved=bool(inter))
    kc, vc = k_cache, v_cache
    if k_new is not None:
        kc, vc = kv_append(k_cache, v_cache, block_table, cache_seqlens, cu_seqlens_q,
                           k_new, v_new, rotary=rotary, dtype=dtype)
    out, lse = attention(q, kc, vc, block_table, cache_seqlens, cu_seqlens_q, dtype=dtype,
                         appended=k_new is not None, causal=causal, scale=scale,
                         threads=threads)
    return out, lse, kc, vc


def combine(o_parts, lse_parts):
    """Merge split partials: o_parts [S, rows, D], lse_parts [S, rows] (fp64)."""
    op = _c(o_parts, np.float64)
    lp = _c(lse_parts, np.float64)
    S, rows, d = op.shape
    out = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    _load().oracle_combine(S, rows, d, _ptr(op), _ptr(lp), _ptr(out), _ptr(lse))
    return out, lse
