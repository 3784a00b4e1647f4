"""The path under HIP graph capture: the library allocates, frees and
synchronizes nothing, so a whole step (indexer, top-k, attention, combine) can
be captured and replayed. Every replay is checked bit for bit against the eager
step, with eager work and synchronizations between replays, and after the query
buffers are refilled in place (a replay reads the live buffers)."""

import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
import test_gpu_parity as T_

pytestmark = pytest.mark.gpu
say = T_.say


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                 # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def make_step(w, inp, geom, cache, dev, static=False, staged=False):
    """Pre-allocated outputs and a step that writes them (no allocation inside).
    static: decode attention through msa_sparse_attn_decode_static (no workspace);
    staged: prefill attention through msa_sparse_attn_prefill_staged."""
    T = w.tokens_per_seq
    if w.is_decode:
        rows, batch = w.total_q, None
    else:
        batch = msa.make_batch(w.seq_lens, w.q_lens, dev)
        rows = batch.total_q if w.per_token else batch.total_units
    bufs = dict(scores=torch.empty((rows, w.num_sel_groups, cache.max_blocks),
                                   dtype=torch.float32, device=dev),
                ids=torch.empty((rows, w.num_sel_groups, w.topk), dtype=torch.int32, device=dev),
                out=torch.empty_like(inp["q"]),
                lse=torch.empty(inp["q"].shape[:2], dtype=torch.float32, device=dev))
    if w.is_decode:
        ws = msa.workspace(msa.msa_decode_workspace_size(geom, w.total_q, w.topk, 0), dev)
    elif w.per_token:
        ws = msa.workspace(msa.msa_prefill_tokens_workspace_size(geom, batch.total_units,
                                                                 batch.total_q, w.topk), dev)
    elif staged:
        ws = msa.workspace(msa.msa_prefill_workspace_size(geom, cache, batch.total_units,
                                                          w.topk), dev)
    else:
        ws = None

    def step():
        if w.is_decode and T > 1:
            msa.msa_index_scores_per_token(geom, cache, T, inp["q_idx"], bufs["scores"])
        elif w.per_token:
            msa.msa_index_scores_prefill_tokens(geom, cache, batch, inp["q_idx"], bufs["scores"])
        else:
            msa.msa_index_scores(geom, cache, batch, inp["q_idx"], bufs["scores"])
        msa.msa_select_topk_blocks(bufs["scores"], w.topk, bufs["ids"])
        if w.is_decode and T > 1:
            msa.msa_sparse_attn_decode_per_token(geom, cache, T, inp["q"], bufs["ids"], w.topk,
                                                 bufs["out"], ws, bufs["lse"])
        elif w.is_decode and static:
            msa.msa_sparse_attn_decode_static(geom, cache, inp["q"], bufs["ids"], w.topk,
                                              bufs["out"], bufs["lse"])
        elif w.is_decode:
            msa.msa_sparse_attn_decode(geom, cache, inp["q"], bufs["ids"], w.topk, bufs["out"],
                                       ws, bufs["lse"])
        elif w.per_token:
            msa.msa_sparse_attn_prefill_tokens(geom, cache, batch, inp["q"], bufs["ids"], w.topk,
                                               bufs["out"], ws, bufs["lse"])
        elif staged:
            msa.msa_sparse_attn_prefill_staged(geom, cache, batch, inp["q"], bufs["ids"], w.topk,
                                               bufs["out"], ws, bufs["lse"])
        else:
            msa.msa_sparse_attn_prefill(geom, cache, batch, inp["q"], bufs["ids"], w.topk,
                                        bufs["out"], bufs["lse"])
    return step, bufs


CASES = {
    "decode": dict(seq_lens=(3000, 700, 129, 20000), q_lens=None, topk=5),
    "decode_per_token": dict(seq_lens=(3000, 700, 131), q_lens=None, tokens_per_seq=4, topk=5),
    "decode_fp8": dict(seq_lens=(3000, 700, 129), q_lens=None, topk=5, cache_format="fp8"),
    "prefill": dict(seq_lens=(1500, 700), q_lens=(600, 700), topk=4),
    "prefill_fp8": dict(seq_lens=(1500, 700), q_lens=(600, 700), topk=4, cache_format="fp8"),
    # one selection group over 8 heads of 64 channels: the wide prefill indexer
    "prefill_one_group_fp8": dict(seq_lens=(1500, 300), q_lens=(400, 300), num_q_heads=16,
                                  num_kv_heads=4, num_idx_heads=8, num_sel_groups=1, topk=5,
                                  cache_format="fp8"),
    "prefill_one_group": dict(seq_lens=(1500, 300), q_lens=(400, 300), num_q_heads=16,
                              num_kv_heads=4, num_idx_heads=8, num_sel_groups=1, topk=5),
    # per-token selection in prefill: the per-row indexer, the wave top-k, the union
    # kernel (zeroes its masks, then ORs them: every replay rebuilds them) and attention
    "prefill_tokens": dict(seq_lens=(1500, 700), q_lens=(600, 700), topk=4, per_token=True),
    "prefill_tokens_fp8_one_group": dict(seq_lens=(1500, 300), q_lens=(400, 300),
                                         num_q_heads=16, num_kv_heads=4, num_idx_heads=8,
                                         num_sel_groups=1, topk=5, cache_format="fp8",
                                         per_token=True),
    # FP8 prefill through the staged attention: the slot map is reset, kept blocks
    # claimed and converted, then attended, on every replay
    "prefill_fp8_staged": dict(seq_lens=(1500, 700), q_lens=(600, 700), topk=4,
                               cache_format="fp8", staged=True),
    "prefill_fp8_staged_one_group": dict(seq_lens=(1500, 300), q_lens=(400, 300),
                                         num_q_heads=16, num_kv_heads=4, num_idx_heads=8,
                                         num_sel_groups=1, topk=5, cache_format="fp8",
                                         staged=True),
    # more cache blocks than kept entries: slots claimed through the slot map
    "prefill_fp8_staged_claimed": dict(seq_lens=(20000, 700), q_lens=(200, 700), topk=4,
                                       cache_format="fp8", staged=True),
    # the decode attention that keeps its partials in the library's static scratch
    "decode_static": dict(seq_lens=(3000, 700, 129, 20000), q_lens=None, topk=5,
                          static=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name, gpu_device):
    kw = dict(CASES[name])
    static = kw.pop("static", False)
    staged = kw.pop("staged", False)
    w = synth.small_workload(**kw)
    say(f"graph {name}")
    inp, geom, cache = T_.setup(w, gpu_device, permute=True)
    step, bufs = make_step(w, inp, geom, cache, gpu_device, static, staged)
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in bufs.items()}
    g = capture(step)
    scratch = torch.randn(1 << 20, device=gpu_device)
    for rep in range(4):
        for v in bufs.values():
            v.fill_(0) if v.dtype != torch.int32 else v.fill_(-7)
        scratch.mul_(1.0001).add_(1.0)       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], eager[k]), f"replay {rep}: {k} differs"
    # new queries in the same buffers: a replay reads them
    inp["q"].copy_(torch.flip(inp["q"], dims=[0]))
    inp["q_idx"].copy_(torch.flip(inp["q_idx"], dims=[0]))
    step()
    torch.cuda.synchronize()
    eager2 = {k: v.clone() for k, v in bufs.items()}
    assert not torch.equal(eager2["out"], eager["out"])
    for k in bufs:
        bufs[k].zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for k in bufs:
        assert torch.equal(bufs[k], eager2[k]), f"replay after refill: {k} differs"
