"""Attention calls on id lists that the selection never produces, on MI355X
through the C ABI, against the CPU oracle: every listed block is masked by
position, so order does not matter, a block after the unit's diagonal adds
nothing (and is not read), a list without the diagonal attends the other
blocks, entries after the first -1 are ignored, and a query row with no visible
key gets out 0 and lse -inf. Bars as everywhere: out max-abs 2e-2 (bf16) or
1e-5 (fp32), lse 1e-3, and exactly 0 / -inf for the rows that see nothing."""

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import parity as P
import test_gpu_parity as T
import test_gpu_fp8 as F

pytestmark = pytest.mark.gpu
say, host = T.say, T.host


def hand_ids(units, nsel, topk, max_blocks, seed):
    """Per (unit, group) an id list of one of several malformed kinds; returns the
    ids array and the kind of each row."""
    rng = np.random.default_rng(seed)
    ids = np.full((len(units), nsel, topk), -1, dtype=np.int32)
    kinds = []
    for u, un in enumerate(units):
        tau = un["tau"]
        for g in range(nsel):
            kind = (u * nsel + g) % 6
            before = rng.permutation(tau)[:max(0, min(topk - 2, tau))].tolist()
            future = [b for b in range(tau + 1, max_blocks)]
            if kind == 0:          # the selection's blocks, shuffled (diagonal not last)
                row = before + [tau]
                rng.shuffle(row)
            elif kind == 1:        # no diagonal block
                row = before
            elif kind == 2:        # a future block listed last, in the diagonal's place
                row = before + [tau] + future[:1]
            elif kind == 3:        # only future blocks (nothing visible)
                row = future[:2]
            elif kind == 4:        # nothing listed
                row = []
            else:                  # ids after a -1 are ignored
                row = before[:1] + [tau, -1] + before[1:2]
            row = row[:topk]
            ids[u, g, :len(row)] = row
            kinds.append(kind)
    return ids, kinds


def check_rows(go, gl, ref_out, ref_lse, dtype, where):
    seen = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), seen), f"{where}: rows with no visible key differ"
    assert np.all(go[~seen] == 0) and np.all(gl[~seen] == -np.inf), where
    if seen.any():
        P.check_attention(go[seen], gl[seen], ref_out[seen], ref_lse[seen], dtype, where)


CASES = {
    "bf16": dict(seq_lens=(1500, 700, 300), q_lens=(800, 700, 50), topk=6),
    "bf16_g16_d64": dict(seq_lens=(1300,), q_lens=(700,), num_q_heads=16, num_kv_heads=1,
                         head_dim=64, num_idx_heads=2, idx_head_dim=32, num_sel_groups=1,
                         topk=5),
    "fp8": dict(seq_lens=(1500, 700), q_lens=(800, 700), topk=6, cache_format="fp8"),
    "f32": dict(dtype="f32", seq_lens=(700, 300), q_lens=(300, 300), num_q_heads=4,
                num_kv_heads=1, head_dim=64, num_idx_heads=2, idx_head_dim=32,
                num_sel_groups=1, topk=5),
}


def host_caches(w, inp, cache):
    if w.cache_format == "fp8":
        kc, vc, _ = F.decoded(F.fp8_host(cache))
        return kc, vc
    return host(inp["k_cache"]), host(synth.v_token_major(inp["v_cache"]))


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_any_ids(name, gpu_device):
    w = synth.small_workload(**CASES[name])
    say(f"prefill any ids {name}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    units = O.prefill_units(w.seq_lens, w.q_lens)
    ids, kinds = hand_ids(units, w.num_sel_groups, w.topk, cache.max_blocks, 7)
    assert len(set(kinds)) == min(6, len(kinds))
    out = torch.full_like(inp["q"], 7.0)
    lse = torch.full(inp["q"].shape[:2], 7.0, dtype=torch.float32, device=gpu_device)
    msa.msa_sparse_attn_prefill(geom, cache, batch, inp["q"], torch.from_numpy(ids).to(gpu_device),
                                w.topk, out, lse)
    torch.cuda.synchronize()
    kc, vc = host_caches(w, inp, cache)
    ref_out, ref_lse = O.attention(units, ids, host(inp["q"]), kc, vc,
                                   inp["block_table"].cpu().numpy(), w.seq_lens,
                                   w.num_sel_groups)
    check_rows(host(out), lse.cpu().numpy(), ref_out, ref_lse, w.dtype, name)


@pytest.mark.parametrize("name", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_any_ids(name, splits, gpu_device):
    kw = dict(CASES[name])
    kw.pop("q_lens")
    kw["seq_lens"] = (3000, 700, 129, 5000)
    w = synth.small_workload(q_lens=None, **kw)
    say(f"decode any ids {name} splits={splits}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    units = O.decode_units(w.seq_lens)
    ids, kinds = hand_ids(units * 3, w.num_sel_groups, w.topk, cache.max_blocks, 11)
    out_all = []
    for rep in range(3):      # three id sets over the same sequences
        part = ids[rep * len(units):(rep + 1) * len(units)]
        res_out = torch.full_like(inp["q"], 7.0)
        res_lse = torch.full(inp["q"].shape[:2], 7.0, dtype=torch.float32, device=gpu_device)
        ws = msa.workspace(msa.msa_decode_workspace_size(geom, w.num_seqs, w.topk, splits),
                           gpu_device)
        msa.msa_sparse_attn_decode(geom, cache, inp["q"], torch.from_numpy(part).to(gpu_device),
                                   w.topk, res_out, ws, res_lse, splits)
        torch.cuda.synchronize()
        kc, vc = host_caches(w, inp, cache)
        ref_out, ref_lse = O.attention(units, part, host(inp["q"]), kc, vc,
                                       inp["block_table"].cpu().numpy(), w.seq_lens,
                                       w.num_sel_groups)
        check_rows(host(res_out), res_lse.cpu().numpy(), ref_out, ref_lse, w.dtype,
                   f"{name} rep {rep}")
        out_all.append(res_out)
