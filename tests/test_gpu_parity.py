"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

Small cases are compared in full; the full-size workloads are compared on a
seeded sample of units (units are independent, so the oracle computes each
sampled unit alone from the same inputs)."""

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import parity as P

pytestmark = pytest.mark.gpu
BLK = 128


def say(msg):
    print(f"[case] {msg}", flush=True)


def geometry(w):
    return msa.Geometry(w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_idx_heads,
                        w.idx_head_dim, w.num_sel_groups, w.dtype, w.cache_format)


def cache_of(inp):
    return msa.Cache(inp["k_cache"], inp["v_cache"], inp["k_idx_cache"], inp["block_table"],
                     inp["seq_lens"], inp.get("k_scale"), inp.get("v_scale"),
                     inp.get("k_idx_scale"))


def setup(w, dev, permute=False):
    inp = synth.make_inputs(w, dev, permute=permute)
    return inp, geometry(w), cache_of(inp)


def run_gpu(w, inp, geom, cache, dev, num_splits=0, staged=False):
    if w.is_decode:
        res = msa.decode(geom, cache, inp["q"], inp["q_idx"], w.topk, num_splits)
    else:
        batch = msa.make_batch(w.seq_lens, w.q_lens, dev)
        res = msa.prefill(geom, cache, batch, inp["q"], inp["q_idx"], w.topk, staged=staged)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def host(t):
    return synth.to_host_f32(t)


def full_parity(w, inp, res, where):
    q, qi = host(inp["q"]), host(inp["q_idx"])
    kc, ki = host(inp["k_cache"]), host(inp["k_idx_cache"])
    vc = host(synth.v_token_major(inp["v_cache"]))
    bt = inp["block_table"].cpu().numpy()
    units = O.decode_units(w.seq_lens) if w.is_decode else O.prefill_units(w.seq_lens, w.q_lens)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    tol = P.score_tolerance(qi, ki, w.num_sel_groups)
    P.check_scores(res["scores"].numpy(), ref, tol, where)
    ids = res["ids"].numpy()
    P.check_ids(ids, ref, units, w.topk, where)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    return P.check_attention(host(res["out"]), res["lse"].numpy(), out, lse, w.dtype, where)


SMALL_PREFILL = {
    "one_request": dict(seq_lens=(700,), q_lens=(300,)),
    "ragged_permuted": dict(seq_lens=(1000, 260, 129, 5), q_lens=(1000, 200, 1, 5), topk=4,
                            permute=True),
    "one_selection_group": dict(seq_lens=(900,), q_lens=(650,), num_sel_groups=1),
    "g16_d64_di32": dict(seq_lens=(1300,), q_lens=(700,), num_q_heads=16, num_kv_heads=1,
                         head_dim=64, num_idx_heads=2, idx_head_dim=32, num_sel_groups=1),
    "mha_g1": dict(seq_lens=(600,), q_lens=(600,), num_q_heads=4, num_kv_heads=4,
                   num_idx_heads=4, num_sel_groups=4),
    "topk_covers_all": dict(seq_lens=(1000,), q_lens=(1000,), topk=16),
    "topk_one": dict(seq_lens=(1000,), q_lens=(500,), topk=1),
    "m3_heads": dict(seq_lens=(1100,), q_lens=(600,), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=5),
    "m3_heads_one_group": dict(seq_lens=(1500, 300), q_lens=(400, 300), num_q_heads=64,
                               num_kv_heads=4, num_idx_heads=8, num_sel_groups=1, topk=6),
    "f32_ragged": dict(dtype="f32", seq_lens=(700, 300), q_lens=(300, 300), num_q_heads=4,
                       num_kv_heads=1, head_dim=64, num_idx_heads=2, idx_head_dim=32,
                       num_sel_groups=1),
    "f32_d128": dict(dtype="f32", seq_lens=(520,), q_lens=(400,)),
    # more than 64 kept blocks per unit: the kernel's block ids come in chunks of 64
    "kept_blocks_over_64": dict(seq_lens=(10245,), q_lens=(261,), topk=80),
    "topk_150_of_157": dict(seq_lens=(20000,), q_lens=(160,), topk=150),
    # one selection group 256 channels wide over 32-channel indexer heads (the 512-wide
    # groups are m3_heads_one_group: 8 heads of 64 channels)
    "one_group_di32_w256": dict(seq_lens=(1500, 200), q_lens=(700, 200), num_idx_heads=8,
                                idx_head_dim=32, num_sel_groups=1, topk=5),
}


@pytest.mark.parametrize("name", list(SMALL_PREFILL))
def test_small_prefill_parity(name, gpu_device):
    kw = dict(SMALL_PREFILL[name])
    permute = kw.pop("permute", False)
    w = synth.small_workload(**kw)
    say(f"prefill {name}")
    inp, geom, cache = setup(w, gpu_device, permute)
    res = run_gpu(w, inp, geom, cache, gpu_device)
    full_parity(w, inp, res, name)


SMALL_DECODE = {
    "mixed_lengths": dict(seq_lens=(700, 1000, 129, 5, 128, 1024, 4000), topk=4),
    "m3_heads": dict(seq_lens=(20000, 3000, 131, 9000), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=9),
    "one_selection_group_g16_d64": dict(seq_lens=(5000, 777), num_q_heads=16, num_kv_heads=1,
                                        head_dim=64, num_idx_heads=4, idx_head_dim=32,
                                        num_sel_groups=1, topk=7),
    "topk_covers_all": dict(seq_lens=(900, 300), topk=12),
    "f32": dict(dtype="f32", seq_lens=(3000, 700), num_q_heads=4, num_kv_heads=1,
                head_dim=64, num_idx_heads=1, idx_head_dim=32, num_sel_groups=1, topk=4),
    "kept_blocks_over_64": dict(seq_lens=(12000, 700), topk=80),
    "topk_1000": dict(seq_lens=(150000, 9000, 128), topk=1000),
}


@pytest.mark.parametrize("name", list(SMALL_DECODE))
def test_small_decode_parity(name, gpu_device):
    w = synth.small_workload(q_lens=None, **SMALL_DECODE[name])
    say(f"decode {name}")
    inp, geom, cache = setup(w, gpu_device, permute=True)
    res = run_gpu(w, inp, geom, cache, gpu_device)
    full_parity(w, inp, res, name)


def test_decode_split_counts_agree(gpu_device):
    w = synth.small_workload(q_lens=None, seq_lens=(20000, 3000, 131, 9000), num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=9)
    inp, geom, cache = setup(w, gpu_device)
    outs = {}
    for s in (1, 2, 7, 0, 9):
        say(f"decode splits={s}")
        outs[s] = run_gpu(w, inp, geom, cache, gpu_device, num_splits=s)
    for s in (2, 7, 0, 9):
        assert torch.equal(outs[s]["ids"], outs[1]["ids"])
        d = (outs[s]["out"].float() - outs[1]["out"].float()).abs().max().item()
        assert d <= 2 * 2.0 ** -8, f"splits={s}: {d}"       # two bf16 roundings apart at most
        assert (outs[s]["lse"] - outs[1]["lse"]).abs().max().item() < 1e-5


def test_tiny_prefill_fp32_workload(gpu_device):
    w = synth.WORKLOADS["tiny_prefill_fp32"]
    say("tiny_prefill_fp32")
    inp, geom, cache = setup(w, gpu_device)
    res = run_gpu(w, inp, geom, cache, gpu_device)
    full_parity(w, inp, res, w.name)


def test_determinism_and_layout_invariance(gpu_device):
    """Two runs are bit-identical; a permuted physical layout is bit-identical."""
    for kw in (dict(seq_lens=(1500, 700), q_lens=(800, 700), num_q_heads=64, num_kv_heads=4,
                    num_idx_heads=8, num_sel_groups=4, topk=5),
               dict(seq_lens=(9000, 2000), q_lens=None, num_q_heads=64, num_kv_heads=4,
                    num_idx_heads=8, num_sel_groups=4, topk=9)):
        w = synth.small_workload(**kw)
        say(f"determinism {'decode' if w.is_decode else 'prefill'}")
        inp, geom, cache = setup(w, gpu_device)
        a = run_gpu(w, inp, geom, cache, gpu_device)
        b = run_gpu(w, inp, geom, cache, gpu_device)
        inp2, geom2, cache2 = setup(w, gpu_device, permute=True)
        c = run_gpu(w, inp2, geom2, cache2, gpu_device)
        for k in ("scores", "ids", "out", "lse"):
            assert torch.equal(a[k], b[k]), k
            assert torch.equal(a[k], c[k]), k


def generic_row_rule(row, topk):
    valid = [b for b in range(len(row)) if row[b] != -np.inf]
    key = lambda b: (-(row[b] + 0.0), b)          # -0.0 and +0.0 tie
    kept = sorted(sorted(valid, key=key)[:topk])
    return kept + [-1] * (topk - len(kept))


def test_topk_rows_exact(gpu_device):
    rng = np.random.default_rng(5)
    rows = []
    rows.append(np.array([3, 1, 3, 2, np.inf, -np.inf, -np.inf], np.float32))
    rows.append(np.array([-0.0, 0.0, -1e-30, 1e-30, np.inf], np.float32))
    rows.append(np.full(9, -np.inf, np.float32))                    # nothing to keep
    # lengths on both sides of the register-resident kernel's sizes (512 * 1, 2, 4, 8, 16,
    # 32 entries) and of its limit, past which rows take the streaming kernel
    for n in (1, 2, 31, 128, 513, 1000, 2048, 4000, 8192, 8256, 16384, 16385, 20011):
        r = rng.integers(-4, 5, size=n).astype(np.float32)           # heavy ties
        r[rng.integers(0, n)] = np.inf
        r[rng.random(n) < 0.2] = -np.inf
        rows.append(r)
        rows.append(rng.standard_normal(n).astype(np.float32) * 1e3)
        rows.append((rng.standard_normal(n) * 1e-38).astype(np.float32))   # denormals
    for topk in (1, 4, 33, 64, 300):
        for r in rows:
            say(f"topk n={len(r)} k={topk}")
            s = torch.from_numpy(r).to(gpu_device)[None]
            ids = torch.empty((1, topk), dtype=torch.int32, device=gpu_device)
            msa.msa_select_topk_blocks(s, topk, ids)
            assert ids.cpu().numpy()[0].tolist() == generic_row_rule(r.astype(np.float64), topk)


def test_empty_prefill_batch_launches_nothing(gpu_device):
    w = synth.small_workload(seq_lens=(300, 200), q_lens=(1, 1))
    inp, geom, cache = setup(w, gpu_device)
    batch = msa.make_batch([300, 200], [0, 0], gpu_device)
    assert batch.total_units == 0
    scores = torch.empty((0, 2, cache.max_blocks), dtype=torch.float32, device=gpu_device)
    msa.msa_index_scores(geom, cache, batch, inp["q_idx"][:0], scores)
    ids = torch.empty((0, 2, w.topk), dtype=torch.int32, device=gpu_device)
    msa.msa_select_topk_blocks(scores, w.topk, ids)
    out = torch.empty_like(inp["q"][:0])
    msa.msa_sparse_attn_prefill(geom, cache, batch, inp["q"][:0], ids, w.topk, out)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# full-size workloads, sampled units
# ----------------------------------------------------------------------------

def _mini_cache(cache_t, bt_row, blocks, heads):
    """Host float32 copy of the given logical blocks and heads of one request, with
    a block table mapping those logical ids to rows of the copy."""
    idx = torch.as_tensor(np.asarray(bt_row)[blocks].astype(np.int64), device=cache_t.device)
    mini = host(cache_t[:, heads].index_select(0, idx))
    bt = np.zeros(max(blocks) + 1, dtype=np.int64)
    bt[blocks] = np.arange(len(blocks))
    return mini, bt


def sampled_parity(w, inp, res, units, picks, rows_per_unit=16, seed=0):
    rng = np.random.default_rng(seed)
    bt_all = inp["block_table"].cpu().numpy()
    nsel, Hs = w.num_sel_groups, w.num_idx_heads // w.num_sel_groups
    G = w.num_q_heads // w.num_kv_heads
    scores, ids = res["scores"].numpy(), res["ids"].numpy()
    q_all, qi_all = inp["q"], inp["q_idx"]
    worst = [0.0, 0.0]
    for u in picks:
        un = units[u]
        r, tau = un["r"], un["tau"]
        say(f"{w.name} unit {u} (r={r}, tau={tau})")
        rows = slice(un["row0"], un["row1"])
        for g in range(nsel):
            heads = slice(g * Hs, (g + 1) * Hs)
            cand = list(range(tau)) if tau > 0 else [0]
            ki, btm = _mini_cache(inp["k_idx_cache"], bt_all[r], cand, heads)
            qi = host(qi_all[rows, heads])
            ref = O.unit_block_scores(qi, ki, btm, tau, 1, scores.shape[2])
            tol = P.score_tolerance(qi, ki, 1)
            P.check_scores(scores[u, g][None, None], ref[None], tol, f"{w.name} u{u} g{g}")
            ok, _ = P.ids_acceptable(ids[u, g], ref[0], tau, w.topk)
            assert ok, f"{w.name} u{u} g{g}: ids {ids[u, g]}"
        # attention on a sample of the unit's rows, every query head
        n = un["row1"] - un["row0"]
        pick_rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, rows_per_unit)]))
        for j in range(w.num_kv_heads):
            g = j if nsel == w.num_kv_heads else 0
            kept = [int(b) for b in ids[u, g] if b >= 0]
            kc, btm = _mini_cache(inp["k_cache"], bt_all[r], kept, slice(j, j + 1))
            vc, _ = _mini_cache(synth.v_token_major(inp["v_cache"]), bt_all[r], kept,
                                slice(j, j + 1))
            qh = host(q_all[un["row0"]:un["row1"], j * G:(j + 1) * G])
            for t in pick_rows:
                o, l = O.unit_attention(qh[t:t + 1], un["pos0"] + t, ids[u, g][None], kc, vc,
                                        btm, int(w.seq_lens[r]), 1)
                go = host(res["out"][un["row0"] + t, j * G:(j + 1) * G])[None]
                gl = res["lse"][un["row0"] + t, j * G:(j + 1) * G].numpy()[None]
                d = P.check_attention(go, gl, o, l, w.dtype, f"{w.name} u{u} row{t} kv{j}")
                worst = [max(worst[0], d[0]), max(worst[1], d[1])]
    return worst


def _sample_units(units, n, seed):
    rng = np.random.default_rng(seed)
    U = len(units)
    picks = {0, U - 1} | set(rng.choice(U, size=min(n, U), replace=False).tolist())
    return sorted(picks)


def all_unit_indexing(w, inp, res, units):
    """Scores (dot-product bound) and ids (near-tie rule) of EVERY unit and group
    against the oracle, one sequence's blocks on the host at a time."""
    bt_all = inp["block_table"].cpu().numpy()
    scores, ids = res["scores"].numpy(), res["ids"].numpy()
    near = 0
    for r in range(w.num_seqs):
        us = [u for u, un in enumerate(units) if un["r"] == r]
        tau_max = max(units[u]["tau"] for u in us)
        blocks = list(range(max(tau_max, 1)))
        ki, btm = _mini_cache(inp["k_idx_cache"], bt_all[r], blocks, slice(None))
        for u in us:
            un = units[u]
            qi = host(inp["q_idx"][un["row0"]:un["row1"]])
            ref = O.unit_block_scores(qi, ki, btm, un["tau"], w.num_sel_groups, scores.shape[2])
            P.check_scores(scores[u][None], ref[None], P.score_tolerance(qi, ki, w.num_sel_groups),
                           f"{w.name} u{u}")
            for g in range(w.num_sel_groups):
                ok, exact = P.ids_acceptable(ids[u, g], ref[g], un["tau"], w.topk)
                assert ok, f"{w.name} u{u} g{g}: ids {ids[u, g]}"
                near += not exact
        del ki
    say(f"{w.name}: scores and ids of all {len(units)} units checked ({near} near-tie rows)")


@pytest.mark.parametrize("name", ["prefill_32k", "chunked_prefill", "prefill_32k_sel1"])
def test_full_size_prefill_sampled(name, gpu_device):
    w = synth.WORKLOADS[name]
    say(f"{name} generate")
    inp, geom, cache = setup(w, gpu_device)
    say(f"{name} run")
    res = run_gpu(w, inp, geom, cache, gpu_device)
    units = O.prefill_units(w.seq_lens, w.q_lens)
    if name != "chunked_prefill":       # 1.5e13 oracle flop: sampled below
        all_unit_indexing(w, inp, res, units)
    picks = _sample_units(units, 4, 1)
    # the first and last tile of every request
    for r in range(w.num_seqs):
        ur = [i for i, un in enumerate(units) if un["r"] == r]
        picks += [ur[0], ur[-1]]
    sampled_parity(w, inp, res, units, sorted(set(picks)), rows_per_unit=8)
    del inp, cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_128k_b64", "decode_1m_b8", "decode_ragged_b64",
                                  "decode_1m_b8_sel1"])
def test_full_size_decode_sampled(name, gpu_device):
    w = synth.WORKLOADS[name]
    say(f"{name} generate")
    inp, geom, cache = setup(w, gpu_device)
    say(f"{name} run")
    res = run_gpu(w, inp, geom, cache, gpu_device)
    units = O.decode_units(w.seq_lens)
    all_unit_indexing(w, inp, res, units)
    sampled_parity(w, inp, res, units, _sample_units(units, 2, 2), rows_per_unit=1)
    # every row is finite before its diagonal, +inf there and -inf after it
    sc = res["scores"].numpy()
    for u, un in enumerate(units):
        tau = un["tau"]
        assert np.isfinite(sc[u, :, :tau]).all() and np.isposinf(sc[u, :, tau]).all()
        assert np.isneginf(sc[u, :, tau + 1:]).all()
    del inp, cache
    torch.cuda.empty_cache()


def test_decode_many_sequences(gpu_device):
    """More sequences than the decode indexer's compacted schedule holds (16384):
    it falls back to visiting every (sequence, block) pair. Sampled sequences are
    checked against the oracle, every row's +inf / -inf pattern in full."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 390, size=16500).tolist()
    w = synth.small_workload(seq_lens=lens, q_lens=None, num_q_heads=4, num_kv_heads=1,
                             head_dim=64, num_idx_heads=1, idx_head_dim=32, num_sel_groups=1,
                             topk=2, plant_count=1, plant_span=None)
    say("decode 16500 sequences")
    inp, geom, cache = setup(w, gpu_device)
    res = run_gpu(w, inp, geom, cache, gpu_device)
    units = O.decode_units(w.seq_lens)
    sampled_parity(w, inp, res, units, _sample_units(units, 24, 9), rows_per_unit=1)
    sc = res["scores"].numpy()
    tau = np.array([un["tau"] for un in units])
    cols = np.arange(sc.shape[2])[None, :]
    s0 = sc[:, 0, :]
    assert np.isfinite(s0[cols < tau[:, None]]).all()
    assert np.isposinf(s0[cols == tau[:, None]]).all()
    assert np.isneginf(s0[cols > tau[:, None]]).all()


def test_msa_log_prints_launches(gpu_device, monkeypatch):
    """MSA_LOG=1: every launch of a prefill and a decode step prints its kernel and
    launch geometry to stderr (the library's debugging aid)."""
    import test_abi as A
    monkeypatch.setenv("MSA_LOG", "1")
    pre = synth.small_workload(seq_lens=(700, 300), q_lens=(300, 300))
    dec = synth.small_workload(seq_lens=(3000, 700), q_lens=None, topk=5)
    say("MSA_LOG launches")

    def run():
        for w in (pre, dec):
            inp, geom, cache = setup(w, gpu_device)
            run_gpu(w, inp, geom, cache, gpu_device)
        torch.cuda.synchronize()

    text = A._stderr_of(run)
    for kernel in ("index_prefill_bf16_kernel", "topk_rows_", "attn_prefill_bf16_kernel",
                   "index_decode_kernel", "attn_decode_bf16_kernel", "combine_kernel"):
        assert f"msa: launch {kernel}" in text, (kernel, text[:2000])
    assert "grid (" in text and "block (" in text
