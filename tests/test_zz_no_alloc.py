"""msa_sparse_attn_decode_static (the decode attention whose split partials live in
the library's static scratch, for callers that cannot allocate) against
msa_sparse_attn_decode with a caller workspace, through the C ABI on MI355X:
bit-identical out and lse (same kernels, same split count), on two calls in a
row, the second with a smaller input, for bf16 and FP8 caches; and the scratch
limit is refused on the device path as on the host."""

import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
import test_gpu_parity as T

pytestmark = pytest.mark.gpu
say = T.say


def _ids(w, inp, geom, cache, dev):
    B = w.num_seqs
    scores = torch.empty((B, w.num_sel_groups, cache.max_blocks), dtype=torch.float32,
                         device=dev)
    ids = torch.empty((B, w.num_sel_groups, w.topk), dtype=torch.int32, device=dev)
    msa.msa_index_scores(geom, cache, None, inp["q_idx"], scores)
    msa.msa_select_topk_blocks(scores, w.topk, ids)
    return ids


def _compare(w, dev, splits):
    inp, geom, cache = T.setup(w, dev, permute=True)
    ids = _ids(w, inp, geom, cache, dev)
    ref_out, ref_lse = torch.empty_like(inp["q"]), torch.empty(inp["q"].shape[:2],
                                                               dtype=torch.float32, device=dev)
    ws = msa.workspace(msa.msa_decode_workspace_size(geom, w.num_seqs, w.topk, splits), dev)
    msa.msa_sparse_attn_decode(geom, cache, inp["q"], ids, w.topk, ref_out, ws, ref_lse, splits)
    out = torch.full_like(inp["q"], 3.0)
    lse = torch.full(inp["q"].shape[:2], 3.0, dtype=torch.float32, device=dev)
    msa.msa_sparse_attn_decode_static(geom, cache, inp["q"], ids, w.topk, out, lse, splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "out differs from the workspace call"
    assert torch.equal(lse, ref_lse), "lse differs from the workspace call"


@pytest.mark.parametrize("fmt", ["plain", "fp8"])
def test_static_decode_equals_workspace_decode(fmt, gpu_device):
    big = synth.small_workload(q_lens=None, seq_lens=(20000, 3000, 131, 9000, 70000, 640),
                               num_q_heads=64, num_kv_heads=4, num_idx_heads=8,
                               num_sel_groups=4, topk=9, cache_format=fmt)
    small = synth.small_workload(q_lens=None, seq_lens=(700, 1300), num_q_heads=64,
                                 num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=4,
                                 cache_format=fmt)
    for w, splits in ((big, 0), (small, 0), (big, 3), (small, 1)):
        say(f"static decode {fmt} B={w.num_seqs} splits={splits}")
        _compare(w, gpu_device, splits)


def test_static_decode_size_limit(gpu_device):
    """A shape whose partials exceed the static scratch is refused (nothing runs)."""
    w = synth.small_workload(q_lens=None, seq_lens=(300,) * 600, num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=4)
    geom = T.geometry(w)
    need = msa.msa_decode_workspace_size(geom, w.num_seqs, w.topk, 0)
    assert need > msa.STATIC_SCRATCH_BYTES
    inp, geom, cache = T.setup(w, gpu_device)
    ids = torch.zeros((w.num_seqs, 4, w.topk), dtype=torch.int32, device=gpu_device)
    out = torch.empty_like(inp["q"])
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_attn_decode_static(geom, cache, inp["q"], ids, w.topk, out)
    assert e.value.status == 3
