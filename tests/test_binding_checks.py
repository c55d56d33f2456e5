"""The Python binding rejects every malformed call before anything reaches the
library: wrong shapes, mismatched dtypes, host tensors.  A host tensor or a
short metadata tensor would otherwise be read by the kernels through a wrong
address or past its end.  Runs without a GPU: shape checks come first, and a
well-shaped call on host tensors stops at the device check."""
import pytest
import torch

import paged_kv_cache_lds_amd as pa


def good(**over):
    """A well-shaped decode call on host tensors: batch 2, 8 q / 2 kv heads x 64,
    page 16, 8-page pool, table width 3, with k_new / v_new."""
    t = dict(
        q=torch.zeros(2, 8, 64, dtype=torch.float16),
        k_cache=torch.zeros(8, 16, 2, 64, dtype=torch.float16),
        v_cache=torch.zeros(8, 16, 2, 64, dtype=torch.float16),
        block_table=torch.zeros(2, 3, dtype=torch.int32),
        cache_seqlens=torch.zeros(2, dtype=torch.int32),
        cu_seqlens_q=torch.tensor([0, 1, 2], dtype=torch.int32),
        k_new=torch.zeros(2, 2, 64, dtype=torch.float16),
        v_new=torch.zeros(2, 2, 64, dtype=torch.float16),
        out=torch.zeros(2, 8, 64, dtype=torch.float16),
        softmax_lse=torch.zeros(2, 8, dtype=torch.float32),
    )
    t.update(over)
    return t


def fwd(t):
    return pa.paged_attn_fwd(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["cache_seqlens"], t["cu_seqlens_q"], max_seqlen_q=1,
                             k_new=t["k_new"], v_new=t["v_new"], out=t["out"],
                             softmax_lse=t["softmax_lse"])


def append(t):
    return pa.paged_kv_append(t["k_cache"], t["v_cache"], t["block_table"], t["cache_seqlens"],
                              t["cu_seqlens_q"], t["k_new"], t["v_new"], max_seqlen_q=1)


F16, I32 = torch.float16, torch.int32

BAD_SHAPES = [
    ("cu_seqlens_q short", dict(cu_seqlens_q=torch.tensor([0, 1], dtype=I32))),
    ("cu_seqlens_q long", dict(cu_seqlens_q=torch.tensor([0, 1, 2, 2], dtype=I32))),
    ("block_table rows", dict(block_table=torch.zeros(1, 3, dtype=I32))),
    ("block_table 1-d", dict(block_table=torch.zeros(6, dtype=I32))),
    ("v_cache shape", dict(v_cache=torch.zeros(4, 16, 2, 64, dtype=F16))),
    ("v_cache heads", dict(v_cache=torch.zeros(8, 16, 1, 64, dtype=F16))),
    ("k_cache head_dim", dict(k_cache=torch.zeros(8, 16, 2, 128, dtype=F16),
                              v_cache=torch.zeros(8, 16, 2, 128, dtype=F16))),
    ("k_cache 3-d", dict(k_cache=torch.zeros(8, 16, 128, dtype=F16),
                         v_cache=torch.zeros(8, 16, 128, dtype=F16))),
    ("k_new rows", dict(k_new=torch.zeros(1, 2, 64, dtype=F16))),
    ("k_new heads", dict(k_new=torch.zeros(2, 8, 64, dtype=F16))),
    ("v_new dim", dict(v_new=torch.zeros(2, 2, 32, dtype=F16))),
    ("k_new alone", dict(v_new=None)),
    ("out rows", dict(out=torch.zeros(1, 8, 64, dtype=F16))),
    ("out heads", dict(out=torch.zeros(2, 4, 64, dtype=F16))),
    ("lse shape", dict(softmax_lse=torch.zeros(2, 4, dtype=torch.float32))),
    ("lse 1-d", dict(softmax_lse=torch.zeros(16, dtype=torch.float32))),
    ("cache_seqlens 2-d", dict(cache_seqlens=torch.zeros(2, 1, dtype=I32))),
]


@pytest.mark.parametrize("name,over", BAD_SHAPES, ids=[n for n, _ in BAD_SHAPES])
def test_forward_rejects_bad_shapes(name, over):
    with pytest.raises(ValueError):
        fwd(good(**over))


@pytest.mark.parametrize("over", [
    dict(cache_seqlens=torch.zeros(2, dtype=torch.int64)),
    dict(block_table=torch.zeros(2, 3, dtype=torch.int64)),
    dict(out=torch.zeros(2, 8, 64, dtype=torch.bfloat16)),
    dict(softmax_lse=torch.zeros(2, 8, dtype=torch.float16)),
    dict(k_cache=torch.zeros(8, 16, 2, 64, dtype=torch.bfloat16)),
    dict(k_new=torch.zeros(2, 2, 64, dtype=torch.bfloat16)),
])
def test_forward_rejects_wrong_dtypes(over):
    with pytest.raises(TypeError):
        fwd(good(**over))


def test_contiguous_cache_needs_batch_rows():
    t = good(block_table=None, k_cache=torch.zeros(3, 32, 2, 64, dtype=F16),
             v_cache=torch.zeros(3, 32, 2, 64, dtype=F16))
    with pytest.raises(ValueError, match="batch"):
        fwd(t)


def test_host_tensors_are_rejected():
    # every shape is right; the tensors are on the host
    with pytest.raises(ValueError, match="GPU tensor"):
        fwd(good())
    with pytest.raises(ValueError, match="GPU tensor"):
        append(good())


@pytest.mark.parametrize("name,over", [b for b in BAD_SHAPES if not b[0].startswith(("out", "lse"))],
                         ids=[n for n, _ in BAD_SHAPES if not n.startswith(("out", "lse"))])
def test_append_rejects_bad_shapes(name, over):
    with pytest.raises(ValueError):
        append(good(**over))
