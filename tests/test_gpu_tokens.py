"""Per-query-token selection for T new tokens per sequence (multi-token decode),
on MI355X through the C ABI, against the oracle's token_units path.

Each token row is its own unit (its own scores, diagonal block, top-k and causal
attention). Bars as for decode: scores within the dot-product bound, ids exact
outside near ties, out max-abs 2e-2 (bf16) / 1e-5 (fp32), lse 1e-3. With T = 1
the per-token calls equal the decode calls bit for bit."""

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import parity as P
import test_gpu_parity as T_
import test_gpu_fp8 as F

pytestmark = pytest.mark.gpu
say, host = T_.say, T_.host


def run_tokens(w, inp, geom, cache, num_splits=0):
    res = msa.decode_per_token(geom, cache, w.tokens_per_seq, inp["q"], inp["q_idx"], w.topk,
                               num_splits)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def tokens_parity(w, inp, cache, res, where):
    if w.cache_format == "fp8":
        kc, vc, ki = F.decoded(F.fp8_host(cache))
    else:
        kc, ki = host(inp["k_cache"]), host(inp["k_idx_cache"])
        vc = host(synth.v_token_major(inp["v_cache"]))
    q, qi = host(inp["q"]), host(inp["q_idx"])
    bt = inp["block_table"].cpu().numpy()
    units = O.token_units(w.seq_lens, w.tokens_per_seq)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    P.check_scores(res["scores"].numpy(), ref, P.score_tolerance(qi, ki, w.num_sel_groups),
                   where)
    ids = res["ids"].numpy()
    P.check_ids(ids, ref, units, w.topk, where)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    return P.check_attention(host(res["out"]), res["lse"].numpy(), out, lse, w.dtype, where)


CASES = {
    # tokens straddle block boundaries (e.g. 129 - 4 .. 128), and short sequences
    "t4_mixed": dict(seq_lens=(700, 129, 1000, 4, 131, 2048), tokens_per_seq=4, topk=4),
    "t2_m3_heads": dict(seq_lens=(20000, 3000, 130, 9000), tokens_per_seq=2, num_q_heads=64,
                        num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=9),
    "t8_one_group_g16_d64": dict(seq_lens=(5000, 777, 135), tokens_per_seq=8, num_q_heads=16,
                                 num_kv_heads=1, head_dim=64, num_idx_heads=4, idx_head_dim=32,
                                 num_sel_groups=1, topk=7),
    "t3_f32": dict(dtype="f32", seq_lens=(3000, 700, 258), tokens_per_seq=3, num_q_heads=4,
                   num_kv_heads=1, head_dim=64, num_idx_heads=1, idx_head_dim=32,
                   num_sel_groups=1, topk=4),
    "t4_fp8": dict(seq_lens=(6000, 300, 129), tokens_per_seq=4, cache_format="fp8", topk=5),
    "t5_topk_covers_all": dict(seq_lens=(900, 300), tokens_per_seq=5, topk=12),
}


@pytest.mark.parametrize("name", list(CASES))
def test_per_token_parity(name, gpu_device):
    w = synth.small_workload(q_lens=None, **CASES[name])
    say(f"per-token {name}")
    inp, geom, cache = T_.setup(w, gpu_device, permute=True)
    res = run_tokens(w, inp, geom, cache)
    tokens_parity(w, inp, cache, res, name)


def test_one_token_equals_decode(gpu_device):
    w = synth.small_workload(seq_lens=(700, 1000, 129, 5), q_lens=None, topk=4)
    say("per-token T=1 vs decode")
    inp, geom, cache = T_.setup(w, gpu_device)
    a = run_tokens(w, inp, geom, cache, num_splits=3)
    b = T_.run_gpu(w, inp, geom, cache, gpu_device, num_splits=3)
    for k in ("scores", "ids", "out", "lse"):
        assert torch.equal(a[k], b[k]), k


def test_per_token_split_counts_agree(gpu_device):
    w = synth.small_workload(seq_lens=(6000, 2500), q_lens=None, tokens_per_seq=4, topk=11)
    say("per-token split counts")
    inp, geom, cache = T_.setup(w, gpu_device)
    base = run_tokens(w, inp, geom, cache, num_splits=1)
    for s in (2, 5, 11, 0):
        r = run_tokens(w, inp, geom, cache, num_splits=s)
        assert torch.equal(r["ids"], base["ids"])
        assert (r["out"].float() - base["out"].float()).abs().max() <= 2e-2
        assert (r["lse"] - base["lse"]).abs().max() <= 1e-4


def test_per_token_full_size_1m_sampled(gpu_device):
    """The 1M decode with 4 tokens per sequence (the benchmark's launch): sampled
    token rows, every group's scores and ids, every KV head's attention."""
    w = synth.WORKLOADS["decode_1m_b8_t4"]
    say(f"{w.name} generate")
    inp, geom, cache = T_.setup(w, gpu_device)
    say(f"{w.name} run")
    res = run_tokens(w, inp, geom, cache)
    units = O.token_units(w.seq_lens, w.tokens_per_seq)
    T_.sampled_parity(w, inp, res, units, T_._sample_units(units, 3, 5), rows_per_unit=1)
    sc = res["scores"].numpy()
    # every token's diagonal is the last block: +inf there, finite before it
    assert np.isposinf(sc[:, :, -1]).all() and np.isfinite(sc[:, :, :-1]).all()
    del inp, cache
    torch.cuda.empty_cache()
