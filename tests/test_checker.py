"""The whole-path comparison the GPU parity tests use (scores, ids, out, lse against
the oracle) accepts the oracle's own results and rejects planted mistakes, on
random geometries built on the host. Runs without a GPU."""

import numpy as np
import pytest
import torch

from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import test_gpu_parity as T
import test_gpu_random as R


def oracle_result(w, inp):
    """The path's outputs computed by the oracle, in the layout the GPU calls return."""
    q, qi = T.host(inp["q"]), T.host(inp["q_idx"])
    kc, ki = T.host(inp["k_cache"]), T.host(inp["k_idx_cache"])
    vc = T.host(synth.v_token_major(inp["v_cache"]))
    bt = inp["block_table"].cpu().numpy()
    units = O.decode_units(w.seq_lens) if w.is_decode else O.prefill_units(w.seq_lens, w.q_lens)
    scores = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    ids = O.select(scores, units, w.topk)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    return dict(scores=torch.from_numpy(scores.astype(np.float32)),
                ids=torch.from_numpy(ids),
                out=torch.from_numpy(out.astype(np.float32)).to(torch.bfloat16),
                lse=torch.from_numpy(lse.astype(np.float32)))


def bf16_case(decode):
    for seed in range(40):
        w, fmt, permute = R.draw_case(seed, decode)
        if fmt == "bf16":
            return w, permute
    raise AssertionError("no bf16 case drawn")


@pytest.mark.parametrize("decode", [False, True])
def test_checker_accepts_oracle_and_rejects_mistakes(decode):
    w, permute = bf16_case(decode)
    inp = synth.make_inputs(w, torch.device("cpu"), permute=permute)
    res = oracle_result(w, inp)
    T.full_parity(w, inp, res, "oracle against itself")

    def planted(key, change):
        bad = {k: v.clone() for k, v in res.items()}
        change(bad[key])
        with pytest.raises(AssertionError):
            T.full_parity(w, inp, bad, f"planted mistake in {key}")

    def bump_out(t):
        t[0, 0, 0] = (t[0, 0, 0].float() + 0.1).to(t.dtype)

    def bump_lse(t):
        t[-1, -1] += 0.01

    def bump_score(t):
        u, g = t.shape[0] - 1, 0
        row = t[u, g]
        finite = torch.isfinite(row).nonzero().flatten()
        if len(finite) == 0:          # a unit with only its diagonal block: spoil the +inf
            row[0] = -1.0
        else:
            row[finite[0]] += 1.0

    def swap_id(t):
        u = t.shape[0] - 1
        row = t[u, 0]
        kept = int((row >= 0).sum())
        # point the last kept block of the row at a block that was not kept
        row[kept - 1] = int(row[: kept].max()) + 1 if kept > 0 else 0

    planted("out", bump_out)
    planted("lse", bump_lse)
    planted("scores", bump_score)
    planted("ids", swap_id)
