"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes mirror matches the C struct layout, host-side
validation returns the documented status codes without launching anything,
and the split heuristic has its documented properties."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_cache_lds_amd as pa
from paged_kv_cache_lds_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:paged_attn|paged_kv)_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pa.library_path() if os.path.exists(pa.library_path()) else _build.build())
    names = declared_functions()
    assert set(names) == set(pa.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(r"\bT " + n + r"\b", out), n


def test_ctypes_struct_matches_c_layout():
    fields = [f[0] for f in pa._Args._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "paged_attn.h"', "int main(void){",
           'printf("%zu\\n", sizeof(pa_fwd_args));']
    for f in fields:
        src.append(f'printf("%zu\\n", offsetof(pa_fwd_args, {f}));')
    src.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write("\n".join(src))
        exe = os.path.join(d, "t")
        subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        vals = [int(x) for x in subprocess.check_output([exe]).split()]
    assert vals[0] == ctypes.sizeof(pa._Args)
    for f, off in zip(fields, vals[1:]):
        assert getattr(pa._Args, f).offset == off, f


def valid_args(**over):
    a = pa._Args()
    a.dtype, a.batch, a.total_q, a.max_seqlen_q = 0, 2, 2, 1
    a.num_heads_q, a.num_heads_kv, a.head_dim = 4, 4, 64
    a.page_size, a.num_pages, a.max_pages_per_seq = 16, 32, 7
    a.causal, a.num_splits, a.softmax_scale = 0, 0, 0.0
    fake = 0x1000
    for f in ("q", "k_cache", "v_cache", "block_table", "cache_seqlens", "cu_seqlens_q", "out",
              "softmax_lse"):
        setattr(a, f, fake)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def call_fwd(a):
    return pa._lib().paged_attn_fwd(ctypes.byref(a), None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(softmax_lse=None), 1), (dict(cu_seqlens_q=None), 1),
    (dict(k_new=0x1000), 1),                       # k_new without v_new
    (dict(dtype=7), 3),
    (dict(head_dim=96), 4), (dict(page_size=24), 4), (dict(page_size=8), 4), (dict(page_size=512), 4),
    (dict(num_heads_q=6), 2), (dict(num_splits=129), 2), (dict(num_splits=-1), 2),
    (dict(batch=0), 2), (dict(causal=2), 2), (dict(reserved0=1), 2),
    (dict(block_table=None, contig_alloc=0), 2),
    (dict(num_splits=4), 5),                       # splits need a workspace
    # rotary embedding fields
    (dict(rotary_cos=0x3000, rotary_dim=32, rotary_rows=8), 1),           # cos without sin
    (dict(rotary_dim=32), 2), (dict(rotary_rows=4), 2), (dict(rotary_interleaved=1), 2),
    (dict(rotary_cos=0x3000, rotary_sin=0x4000, rotary_dim=8, rotary_rows=8), 2),
    (dict(rotary_cos=0x3000, rotary_sin=0x4000, rotary_dim=24, rotary_rows=8), 2),
    (dict(rotary_cos=0x3000, rotary_sin=0x4000, rotary_dim=128, rotary_rows=8), 2),  # > head_dim
    (dict(rotary_cos=0x3000, rotary_sin=0x4000, rotary_dim=32, rotary_rows=0), 2),
    (dict(rotary_cos=0x3000, rotary_sin=0x4000, rotary_dim=32, rotary_rows=8,
          rotary_interleaved=2), 2),
    (dict(reserved1=1), 2),
    # 16-byte alignment of every buffer moved in 16-byte vectors
    (dict(q=0x1008), 7), (dict(out=0x1002), 7), (dict(k_cache=0x1004), 7),
    (dict(rotary_cos=0x3008, rotary_sin=0x4000, rotary_dim=32, rotary_rows=8), 7),
    # row strides of q / k_new / v_new
    (dict(q_row_stride=8), 2), (dict(q_row_stride=-256), 2), (dict(q_row_stride=4 * 64 + 4), 7),
    (dict(k_new=0x100000, v_new=0x200000, k_new_row_stride=64), 2),
    (dict(k_new=0x100000, v_new=0x200000, k_new_row_stride=4 * 64 + 8, v_new_row_stride=260), 7),
    # new rows overlapping a pool they are appended to
    (dict(k_new=0x1000, v_new=0x900000), 2), (dict(k_new=0x900000, v_new=0x1200), 2),
])
def test_host_validation_codes(over, code):
    assert call_fwd(valid_args(**over)) == code


def test_null_args_pointer():
    assert pa._lib().paged_attn_fwd(None, None) == 1
    assert pa._lib().paged_kv_append(None, None) == 1


def test_workspace_size_and_splits_for_are_host_only():
    a = valid_args(num_splits=4)
    need = pa.paged_attn_workspace_size(a)
    # S * total_q * Hq * (D + 1) fp32, each part padded to 256 bytes
    assert need >= 4 * 2 * 4 * 65 * 4
    assert pa.paged_attn_splits_for(a) == 4
    a.workspace, a.workspace_bytes = 0x2000, need - 1
    assert call_fwd(a) == 5
    assert pa.paged_attn_workspace_size(valid_args(num_splits=1)) == 0
    assert pa.paged_attn_splits_for(valid_args(head_dim=96)) == -1


def test_plan_keeps_pair_units_whole():
    # 50 sequences x 32 kv heads at 4096 keys: the plan runs 800 units over
    # pairs of kv heads and keeps them unsplit, though the heuristic alone
    # would give 800 units two splits
    kw = dict(total_q=50, max_seqlen_q=1, num_heads_q=32, num_heads_kv=32, head_dim=128,
              max_seqlen_k=4096, num_pages=50 * 256, max_pages_per_seq=256)
    assert pa.paged_attn_num_splits(50, 50, 16, 16, 128, 1, 4096, 256) == 2
    assert pa.paged_attn_splits_for(valid_args(batch=50, **kw)) == 1
    # 12 sequences: 384 one-head units, which take the heuristic's two splits
    kw.update(total_q=12, num_pages=12 * 256)
    assert pa.paged_attn_splits_for(valid_args(batch=12, **kw)) == 2


def test_status_strings():
    for code in range(10):
        assert pa.paged_attn_status_string(code) != "unknown status"
    assert pa.paged_attn_status_string(99) == "unknown status"


def test_split_heuristic_properties():
    ns = pa.paged_attn_num_splits
    # the machine is already full -> no split
    assert ns(256, 256, 32, 32, 128, 1, 4096, 256) == 1
    # long-context GQA decode with few sequences -> splits, up to two units
    # per compute unit while every split keeps >= 64 key tiles
    s = ns(8, 8, 64, 8, 128, 1, 131072, 256)
    assert 2 <= s <= 128
    assert s == 8
    assert ns(16, 16, 64, 8, 128, 1, 12288, 256) == 4
    assert ns(16, 16, 64, 8, 128, 1, 2048, 256) == 2        # 64-tile splits: one unit per CU
    assert ns(32, 32, 64, 8, 128, 1, 8192, 256) == 1        # the CUs are already full
    # MHA keeps one unit per compute unit
    assert ns(4, 4, 32, 32, 128, 1, 8192, 256) == 2
    # never more splits than 8-tile chunks of the key bound, never above 128
    assert ns(1, 1, 1, 1, 128, 1, 32 * 8 * 3, 256) <= 3
    # a range that allows only two 8-tile splits is halved only while the
    # units fill at most a quarter of the compute units; three may split
    assert ns(1, 1, 32, 32, 128, 1, 512, 256) == 2
    assert ns(2, 2, 32, 32, 128, 1, 512, 256) == 2
    assert ns(4, 4, 32, 32, 128, 1, 512, 256) == 1
    assert ns(4, 4, 32, 32, 128, 1, 32 * 8 * 2 + 32 * 7, 256) == 1
    assert ns(1, 1, 32, 32, 128, 1, 32 * 8 * 3, 256) == 3
    for b in (1, 2, 4, 8, 16, 64):
        for k in (1, 100, 4096, 131072, 2**31 - 1):
            v = ns(b, b, 8, 1, 128, 1, k, 256)
            assert 1 <= v <= 128
    # below one unit per compute unit, more work units never ask for more
    # splits; from one unit per compute unit on, at most two
    prev = 129
    for b in range(1, 8):
        v = ns(b, b, 32, 32, 128, 1, 65536, 256)
        assert v <= prev
        prev = v
    for b in range(8, 600, 7):
        assert ns(b, b, 32, 32, 128, 1, 65536, 256) in (1, 2)
    # one to four units per compute unit that leave some compute units a unit
    # more than others (1.5 or 2.5 per CU) split in two; whole units per CU,
    # short key ranges and four or more units per CU stay whole
    assert ns(12, 12, 32, 32, 128, 1, 4096, 256) == 2       # 384 units
    assert ns(20, 20, 32, 32, 128, 1, 8192, 256) == 2       # 640 units
    assert ns(48, 48, 64, 8, 128, 1, 8192, 256) == 2        # 384 units, grouped heads
    for b in (8, 16, 24, 40, 48, 80):
        assert ns(b, b, 32, 32, 128, 1, 4096, 256) == 1
    assert ns(12, 12, 32, 32, 128, 1, 1024, 256) == 1       # 32-tile splits would not fit
    assert ns(36, 36, 32, 32, 128, 1, 4096, 256) == 1       # 1152 units: 4.5 per CU
    # depends only on its arguments (pure, host-known sizes)
    assert ns(8, 8, 64, 8, 128, 1, 131072, 256) == ns(8, 8, 64, 8, 128, 1, 131072, 256)
    # degenerate inputs
    assert ns(0, 0, 1, 1, 64, 1, 10, 256) == 1
    assert ns(4, 4, 4, 4, 64, 1, 0, 256) == 1


def test_sizing_queries_ignore_data_pointers():
    a = valid_args(num_splits=3)
    for f in ("q", "k_cache", "v_cache", "block_table", "cache_seqlens", "cu_seqlens_q", "out",
              "softmax_lse"):
        setattr(a, f, None)
    a.contig_alloc = 256          # no table -> contiguous mode sizes
    assert pa.paged_attn_splits_for(a) == 3
    assert pa.paged_attn_workspace_size(a) > 0
    assert call_fwd(a) == 1       # the forward call itself still needs its pointers


def test_slabs_of_two_gib_or_more_are_rejected():
    # one page of 256 tokens x 64 kv heads x 128 dims x 2 B = 4 MiB is fine (the
    # call then stops at the missing workspace, before any launch)
    assert call_fwd(valid_args(page_size=256, num_heads_q=64, num_heads_kv=64,
                               head_dim=128, num_splits=4)) == 5
    # a contiguous allocation of 2^31 bytes per sequence is not
    a = valid_args(block_table=None, contig_alloc=1 << 20, num_heads_q=8, num_heads_kv=8,
                   head_dim=128)
    assert call_fwd(a) == 4


def test_noalloc_entry_point_host_checks():
    # the allocation-free entry point validates like paged_attn_fwd, ignores
    # the workspace fields, and rejects a plan whose split-KV scratch exceeds
    # its static 64 MiB array before anything is launched
    f = pa._lib().paged_attn_fwd_noalloc
    assert f(None, None) == 1
    assert f(ctypes.byref(valid_args(head_dim=96)), None) == 4
    assert f(ctypes.byref(valid_args(q=None)), None) == 1
    big = valid_args(total_q=4096, max_seqlen_q=2048, num_splits=128)
    need = pa.paged_attn_workspace_size(big)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), None) == pa.PA_ERR_SCRATCH
    # a forced split whose partials fit would need a workspace in paged_attn_fwd,
    # but is not refused for it here (it stops at no check: a decode batch of
    # 2 rows with 4 splits is well within the array) - only sizes are compared
    small = valid_args(num_splits=4)
    assert 0 < pa.paged_attn_workspace_size(small) <= pa.NOALLOC_SCRATCH_BYTES


@settings(max_examples=300, deadline=None)
@given(batch=st.integers(1, 300), hkv=st.sampled_from([1, 2, 4, 8, 12, 16, 32]),
       group=st.sampled_from([1, 2, 4, 8]), d=st.sampled_from([64, 128]),
       q_len=st.integers(1, 40), ctx=st.integers(1, 200000), forced=st.sampled_from([0, 1, 3, 128]))
def test_plan_queries_are_consistent(batch, hkv, group, d, q_len, ctx, forced):
    # the host-only sizing queries over random shapes: a split count in
    # [1, 128] (a forced one honoured), and a workspace exactly when a row
    # can have partials
    pages = -(-ctx // 16)
    a = valid_args(batch=batch, total_q=batch * q_len, max_seqlen_q=q_len, num_heads_q=hkv * group,
                   num_heads_kv=hkv, head_dim=d, max_seqlen_k=ctx, num_pages=batch * pages,
                   max_pages_per_seq=pages, num_splits=forced)
    s = pa.paged_attn_splits_for(a)
    assert 1 <= s <= 128
    if forced:
        assert s == forced
    ws = pa.paged_attn_workspace_size(a)
    assert (ws > 0) == (s > 1)
    if s > 1:
        # every row of every split: an fp32 output row and its lse
        assert ws >= s * batch * q_len * hkv * group * (d + 1) * 4
