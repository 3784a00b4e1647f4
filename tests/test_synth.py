"""Seeded synthetic inputs: determinism, shapes, layout and planting (CPU)."""

import math

import numpy as np
import torch

from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O


def test_workload_shapes_match_their_names():
    W = synth.WORKLOADS
    assert W["prefill_32k"].max_blocks == 256 and W["prefill_32k"].topk == 16
    assert W["decode_128k_b64"].num_phys_blocks == 64 * 1024 and W["decode_128k_b64"].topk == 33
    assert W["decode_1m_b8"].num_phys_blocks == 8 * 8192 and W["decode_1m_b8"].topk == 64
    c5 = W["chunked_prefill"]
    assert [c5.blocks(r) for r in range(4)] == [8256, 4160, 1088, 320]
    t = W["tiny_prefill_fp32"]
    assert t.max_blocks == 16 and t.num_q_heads == 4 and t.num_kv_heads == 1
    for w in W.values():
        assert w.num_q_heads % w.num_kv_heads == 0
        assert w.num_sel_groups in (1, w.num_kv_heads)


def test_plant_amplitude_gives_two_sigma_lift():
    for w in synth.WORKLOADS.values():
        hs = w.num_idx_heads // w.num_sel_groups
        a = synth.plant_amplitude(w)
        assert math.isclose(hs * a * a, 2 * math.sqrt(hs * w.idx_head_dim), rel_tol=1e-12)
    assert abs(synth.plant_amplitude(synth.WORKLOADS["prefill_32k"]) - 3.3636) < 1e-3


def test_planted_blocks_per_span_and_range():
    w = synth.WORKLOADS["prefill_32k"]
    ids = synth.planted_blocks(w, 0, 2)
    assert len(ids) == 8 * 8 and len(set(ids.tolist())) == len(ids)
    for s0 in range(0, 256, 32):
        assert ((ids >= s0) & (ids < s0 + 32)).sum() == 8
    d = synth.WORKLOADS["decode_1m_b8"]
    ids = synth.planted_blocks(d, 3, 1)
    assert len(ids) == 63 and ids.max() < 8191          # never the query's own block
    assert not np.array_equal(ids, synth.planted_blocks(d, 3, 2))


def test_inputs_are_deterministic_and_layout_independent():
    w = synth.small_workload(seq_lens=(700, 300), q_lens=(300, 300))
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    c = synth.make_inputs(w, permute=True)
    bt_a, bt_c = a["block_table"].numpy(), c["block_table"].numpy()
    assert sorted(bt_c[0, :6].tolist() + bt_c[1, :3].tolist()) == list(range(9))
    for r in range(2):
        for blk in range(w.blocks(r)):
            for key in ("k_cache", "v_cache", "k_idx_cache"):
                assert torch.equal(a[key][bt_a[r, blk]], c[key][bt_c[r, blk]])
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (600, 8, 128)
    assert a["cu_q_lens"].tolist() == [0, 300, 600]


def test_chunked_generation_does_not_change_values():
    w = synth.small_workload(seq_lens=(1500,), q_lens=(10,))
    a = synth.make_inputs(w, chunk_blocks=2048)
    b = synth.make_inputs(w, chunk_blocks=2048)
    assert torch.equal(a["k_idx_cache"], b["k_idx_cache"])


def test_planted_blocks_win_the_selection():
    """The planting makes the planted blocks stand out: with k = planted + 1 the
    oracle keeps mostly planted blocks (margins exist, as the workloads intend)."""
    w = synth.small_workload(seq_lens=(4096,), q_lens=None, plant_count=6, plant_span=None,
                             topk=7, num_idx_heads=8, num_sel_groups=4, num_q_heads=8,
                             num_kv_heads=4)
    inp = synth.make_inputs(w)
    qi = synth.to_host_f32(inp["q_idx"])
    ki = synth.to_host_f32(inp["k_idx_cache"])
    bt = inp["block_table"].numpy()
    units = O.decode_units(w.seq_lens)
    S = O.index_scores(units, qi, ki, bt, 4, bt.shape[1])
    ids = O.select(S, units, w.topk)
    hit = 0
    for g in range(4):
        planted = set(synth.planted_blocks(w, 0, g).tolist())
        hit += len(planted & set(ids[0, g].tolist()))
    assert hit >= 0.75 * 4 * 6
