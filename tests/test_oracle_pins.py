"""Pins of the CPU oracle against facts fixed outside it: hand-worked examples,
closed forms, library routines on special cases, brute force on tiny inputs and
invariants of the definition. CPU only."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLK = 128


def _f(x):
    return float(x) if not isinstance(x, str) else float(x.replace("inf", "Infinity")
                                                         .replace("Infinity", "inf"))


# ----------------------------------------------------------------------------
# test-side helpers (independent of the oracle's code)
# ----------------------------------------------------------------------------

def paged(rng, seq_lens, heads, dim, permute=True, fill=None):
    """A random paged cache [P][heads][128][dim] and its block table."""
    nbs = [(L + BLK - 1) // BLK for L in seq_lens]
    P = sum(nbs) + 2                    # two spare physical blocks never referenced
    cache = rng.standard_normal((P, heads, BLK, dim)) if fill is None else fill((P, heads, BLK, dim))
    perm = rng.permutation(P) if permute else np.arange(P)
    bt = np.zeros((len(seq_lens), max(nbs)), dtype=np.int32)
    base = 0
    for r, nb in enumerate(nbs):
        bt[r, :nb] = perm[base:base + nb]
        base += nb
    return cache, bt


def logical(cache, bt_row, L):
    """[L][heads][dim] by fancy indexing the block table."""
    nb = (L + BLK - 1) // BLK
    x = cache[bt_row[:nb]]                                  # [nb][H][128][dim]
    return np.transpose(x, (0, 2, 1, 3)).reshape(nb * BLK, x.shape[1], x.shape[3])[:L]


def dense_reference(q, k_log, v_log, positions, scale):
    """Dense causal GQA attention with torch SDPA in float64, and lse with scipy."""
    T, Hq, D = q.shape
    Hkv = k_log.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][T][D]
    kt = torch.from_numpy(k_log).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(v_log).permute(1, 0, 2).repeat_interleave(G, 0)
    keys = np.arange(k_log.shape[0])
    mask = torch.from_numpy(keys[None, :] <= np.asarray(positions)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
    logits = (torch.matmul(qt, kt.transpose(1, 2)) * scale).numpy()   # [Hq][T][L]
    logits = np.where(mask.numpy()[None], logits, -np.inf)
    lse = scipy.special.logsumexp(logits, axis=2).T                    # [T][Hq]
    return out, lse


CASES = [
    # seq_lens, q_lens, Hq, Hkv
    ([1], [1], 1, 1),
    ([5], [5], 4, 1),
    ([127], [127], 2, 1),
    ([128], [128], 4, 2),
    ([129], [129], 4, 2),
    ([300], [300], 8, 2),
    ([1000], [1000], 4, 4),
    ([700, 260, 129], [300, 260, 1], 8, 2),
    ([513, 384], [1, 200], 4, 1),
]


@pytest.mark.parametrize("seq_lens,q_lens,Hq,Hkv", CASES)
@pytest.mark.parametrize("sel", ["kv", "one"])
def test_dense_when_topk_covers_all_blocks(seq_lens, q_lens, Hq, Hkv, sel):
    """k >= number of blocks: MSA is exactly dense causal GQA attention."""
    rng = np.random.default_rng(11)
    D, Hi, Di = 16, 2 * Hkv, 8
    nsel = Hkv if sel == "kv" else 1
    kc, bt = paged(rng, seq_lens, Hkv, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], Hi, BLK, Di))
    T = sum(q_lens)
    q = rng.standard_normal((T, Hq, D))
    qi = rng.standard_normal((T, Hi, Di))
    topk = bt.shape[1] + 3
    res = O.run_prefill(q, qi, kc, vc, ki, bt, seq_lens, q_lens, nsel, topk)
    row = 0
    for r, (L, n) in enumerate(zip(seq_lens, q_lens)):
        pos = np.arange(L - n, L)
        out, lse = dense_reference(q[row:row + n], logical(kc, bt[r], L),
                                   logical(vc, bt[r], L), pos, 1 / math.sqrt(D))
        np.testing.assert_allclose(res["out"][row:row + n], out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][row:row + n], lse, rtol=1e-12, atol=1e-12)
        row += n


@pytest.mark.parametrize("L", [1, 77, 128])
def test_single_block_is_plain_softmax(L):
    """One block: plain causal softmax attention over that block (any k)."""
    rng = np.random.default_rng(3)
    D = 32
    kc, bt = paged(rng, [L], 2, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 2, BLK, 8))
    q = rng.standard_normal((L, 4, D))
    qi = rng.standard_normal((L, 2, 8))
    res = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [L], 2, 1)
    assert (res["ids"][:, :, 0] == 0).all()
    out, lse = dense_reference(q, logical(kc, bt[0], L), logical(vc, bt[0], L),
                               np.arange(L), 1 / math.sqrt(D))
    np.testing.assert_allclose(res["out"], out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse, rtol=1e-12, atol=1e-12)


def test_topk_one_attends_only_the_diagonal_block():
    """k = 1 keeps only the query's own block: plain softmax over its prefix."""
    rng = np.random.default_rng(4)
    L, n, D = 700, 300, 32
    kc, bt = paged(rng, [L], 1, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 1, BLK, 8))
    q = rng.standard_normal((n, 2, D))
    qi = rng.standard_normal((n, 1, 8))
    res = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [n], 1, 1)
    k_log, v_log = logical(kc, bt[0], L), logical(vc, bt[0], L)
    for t in range(0, n, 37):
        p = L - n + t
        b0 = (p // BLK) * BLK
        out, lse = dense_reference(q[t:t + 1], k_log[b0:p + 1], v_log[b0:p + 1],
                                   [p - b0], 1 / math.sqrt(D))
        np.testing.assert_allclose(res["out"][t], out[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][t], lse[0], rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    """q = 0: uniform weights, out = mean of V over the visible keys, lse = ln|V_t|."""
    rng = np.random.default_rng(5)
    L, n, D, topk = 900, 420, 16, 3
    kc, bt = paged(rng, [L], 2, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 4, BLK, 8))
    q = np.zeros((n, 4, D))
    qi = rng.standard_normal((n, 4, 8))
    res = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [n], 2, topk)
    v_log = logical(vc, bt[0], L)
    for u, un in enumerate(res["units"]):
        for t in range(un["row0"], un["row1"]):
            p = un["pos0"] + (t - un["row0"])
            for i in range(4):
                j = i // 2
                kept = [b for b in res["ids"][u, j] if b >= 0]
                vis = [s for b in kept for s in range(b * BLK, min(b * BLK + BLK, p + 1))]
                assert len(vis) == sum(BLK for b in kept if b < un["tau"]) + p - un["tau"] * BLK + 1
                np.testing.assert_allclose(res["out"][t, i], v_log[vis, j].mean(0), atol=1e-12)
                assert abs(res["lse"][t, i] - math.log(len(vis))) < 1e-12


def test_constant_values_pass_through():
    rng = np.random.default_rng(6)
    L, n, D = 600, 600, 16
    kc, bt = paged(rng, [L], 1, D)
    c = rng.standard_normal(D)
    vc = np.broadcast_to(c, kc.shape).copy()
    ki = rng.standard_normal((kc.shape[0], 1, BLK, 8))
    q = rng.standard_normal((n, 2, D)) * 3
    qi = rng.standard_normal((n, 1, 8))
    res = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [n], 1, 2)
    np.testing.assert_allclose(res["out"], np.broadcast_to(c, res["out"].shape), atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(7)
    L, n, D, G = 640, 250, 16, 4
    kc, bt = paged(rng, [L], 2, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 4, BLK, 8))
    q = rng.standard_normal((n, 2 * G, D))
    qi = rng.standard_normal((n, 4, 8))
    gqa = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [n], 1, 2)
    mha = O.run_prefill(q, qi, np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1), ki, bt,
                        [L], [n], 1, 2)
    assert (gqa["ids"] == mha["ids"]).all()
    np.testing.assert_allclose(gqa["out"], mha["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gqa["lse"], mha["lse"], rtol=1e-13, atol=1e-13)


def test_prefill_row_equals_decode_with_same_ids():
    rng = np.random.default_rng(8)
    L, n, D = 1000, 500, 16
    kc, bt = paged(rng, [L], 2, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 2, BLK, 8))
    q = rng.standard_normal((n, 4, D))
    qi = rng.standard_normal((n, 2, 8))
    res = O.run_prefill(q, qi, kc, vc, ki, bt, [L], [n], 2, 3)
    for u, un in enumerate(res["units"]):
        t = un["row0"] + (un["row1"] - un["row0"]) // 2
        p = un["pos0"] + t - un["row0"]
        o, l = O.unit_attention(q[t:t + 1], p, res["ids"][u], kc, vc, bt[0], p + 1, 2)
        np.testing.assert_allclose(o[0], res["out"][t], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l[0], res["lse"][t], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# indexer scores
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("nsel", [1, 2])
def test_scores_brute_force_loops(nsel):
    """Explicit loops over queries, keys, heads and dims on a tiny chunked case."""
    rng = np.random.default_rng(9)
    seq_lens, q_lens, Hi, Di = [300, 200], [50, 130], 4, 3
    ki, bt = paged(rng, seq_lens, Hi, Di)
    qi = rng.standard_normal((sum(q_lens), Hi, Di))
    units = O.prefill_units(seq_lens, q_lens)
    S = O.index_scores(units, qi, ki, bt, nsel, bt.shape[1])
    Hs = Hi // nsel
    for u, un in enumerate(units):
        for g in range(nsel):
            for b in range(bt.shape[1]):
                if b > un["tau"] or b >= (seq_lens[un["r"]] + BLK - 1) // BLK:
                    assert S[u, g, b] == -np.inf
                    continue
                if b == un["tau"]:
                    assert S[u, g, b] == np.inf
                    continue
                best = -np.inf
                for t in range(un["row0"], un["row1"]):
                    for s in range(b * BLK, b * BLK + BLK):
                        blk, row = bt[un["r"], s // BLK], s % BLK
                        acc = 0.0
                        for h in range(g * Hs, g * Hs + Hs):
                            for d in range(Di):
                                acc += qi[t, h, d] * ki[blk, h, row, d]
                        best = max(best, acc)
                assert abs(S[u, g, b] - best) <= 1e-12 * max(1.0, abs(best))


def test_scores_constant_block_closed_form():
    """k_idx constant within a block: S_g(b) = max_t sum_h q_idx[t,h] . c_h(b)."""
    rng = np.random.default_rng(10)
    L, n, Hi, Di = 900, 200, 4, 8
    nb = (L + BLK - 1) // BLK
    c = rng.standard_normal((nb, Hi, Di))
    bt = np.arange(nb, dtype=np.int32)[None][:, ::-1].copy()         # reversed layout
    ki = np.empty((nb, Hi, BLK, Di))
    for b in range(nb):
        ki[bt[0, b]] = c[b][:, None, :]
    qi = rng.standard_normal((n, Hi, Di))
    units = O.prefill_units([L], [n])
    S = O.index_scores(units, qi, ki, bt, 2, nb)
    for u, un in enumerate(units):
        rows = qi[un["row0"]:un["row1"]]
        for g in range(2):
            for b in range(un["tau"]):
                want = max(float(np.sum(rows[t, 2 * g:2 * g + 2] * c[b, 2 * g:2 * g + 2]))
                           for t in range(len(rows)))
                assert abs(S[u, g, b] - want) < 1e-12


def test_zero_keys_tie_to_lowest_ids():
    """All-zero indexer keys: every candidate scores exactly 0, so the kept blocks
    are the lowest ids 0..K-2 plus the diagonal."""
    rng = np.random.default_rng(12)
    L, n = 1500, 400
    ki, bt = paged(rng, [L], 2, 8, fill=np.zeros)
    qi = rng.standard_normal((n, 2, 8))
    units = O.prefill_units([L], [n])
    S = O.index_scores(units, qi, ki, bt, 1, bt.shape[1])
    ids = O.select(S, units, 4)
    for u, un in enumerate(units):
        tau = un["tau"]
        assert (S[u, 0, :tau] == 0).all()
        K = min(4, tau + 1)
        assert list(ids[u, 0]) == list(range(K - 1)) + [tau] + [-1] * (4 - K)


def test_group_isolation():
    """Only group 1's indexer heads carry signal: group 0 scores are exactly 0."""
    rng = np.random.default_rng(13)
    L, n = 700, 300
    ki, bt = paged(rng, [L], 4, 8)
    qi = rng.standard_normal((n, 4, 8))
    qi[:, :2] = 0.0
    units = O.prefill_units([L], [n])
    S = O.index_scores(units, qi, ki, bt, 2, bt.shape[1])
    for u, un in enumerate(units):
        assert (S[u, 0, :un["tau"]] == 0).all()
        assert (S[u, 1, :un["tau"]] != 0).all()


def test_planted_dominant_block_is_kept():
    rng = np.random.default_rng(14)
    L, n = 2000, 600
    ki, bt = paged(rng, [L], 2, 16)
    qi = rng.standard_normal((n, 2, 16))
    direction = qi.sum(axis=0)                       # shared direction of the queries
    planted = 3
    ki[bt[0, planted]] = 50.0 * direction[:, None, :] / np.linalg.norm(direction)
    qi += 2.0 * direction / np.linalg.norm(direction)
    units = O.prefill_units([L], [n])
    ids = O.select(O.index_scores(units, qi, ki, bt, 1, bt.shape[1]), units, 2)
    for u, un in enumerate(units):
        if un["tau"] > planted:
            assert planted in ids[u, 0]


def test_positive_scaling_keeps_selection():
    rng = np.random.default_rng(15)
    L, n = 1600, 500
    ki, bt = paged(rng, [L], 2, 8)
    qi = rng.standard_normal((n, 2, 8))
    units = O.prefill_units([L], [n])
    a = O.select(O.index_scores(units, qi, ki, bt, 2, bt.shape[1]), units, 3)
    b = O.select(O.index_scores(units, 2.5 * qi, ki, bt, 2, bt.shape[1]), units, 3)
    assert (a == b).all()


def test_block_table_permutation_is_exact():
    rng = np.random.default_rng(16)
    seq_lens, q_lens, D = [800, 300], [400, 300], 16
    ident = {}
    for permute in (False, True):
        r2 = np.random.default_rng(17)
        kc, bt = paged(r2, seq_lens, 2, D, permute=False)
        vc = r2.standard_normal(kc.shape)
        ki = r2.standard_normal((kc.shape[0], 2, BLK, 8))
        if permute:
            perm = rng.permutation(kc.shape[0])
            inv = np.argsort(perm)
            kc, vc, ki = kc[perm], vc[perm], ki[perm]
            bt = inv[bt].astype(np.int32)
        q = r2.standard_normal((sum(q_lens), 4, D))
        qi = r2.standard_normal((sum(q_lens), 2, 8))
        ident[permute] = O.run_prefill(q, qi, kc, vc, ki, bt, seq_lens, q_lens, 2, 3)
    for key in ("scores", "ids", "out", "lse"):
        assert np.array_equal(ident[False][key], ident[True][key]), key


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------

def generic_row_rule(row, topk):
    """Top-k of a row by (score desc, index asc) over entries above -inf, ascending."""
    valid = [b for b in range(len(row)) if row[b] != -np.inf]
    kept = sorted(sorted(valid, key=lambda b: (-row[b], b))[:topk])
    return kept + [-1] * (topk - len(kept))


def test_select_matches_generic_row_rule():
    rng = np.random.default_rng(18)
    for _ in range(400):
        n = int(rng.integers(1, 40))
        tau = int(rng.integers(0, n))
        row = np.full(n, -np.inf)
        row[:tau] = rng.integers(-3, 4, size=tau).astype(float)   # many ties
        row[tau] = np.inf
        topk = int(rng.integers(1, n + 3))
        want = generic_row_rule(row, topk)
        got = O.select_blocks(row, tau, topk)
        assert got == want
        kept = [b for b in got if b >= 0]
        assert tau in kept and kept == sorted(set(kept)) and len(kept) == min(topk, tau + 1)
        out = [b for b in range(tau) if b not in kept]
        for a in kept:
            for b in out:
                assert (row[a], -a) > (row[b], -b)


def test_select_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "select_cases.json")))["cases"]
    for c in cases:
        row = np.array([_f(x) for x in c["scores"]])
        tau = int(np.where(row == np.inf)[0][0])
        assert O.select_blocks(row, tau, c["topk"]) == c["expected"], c


# ----------------------------------------------------------------------------
# hand-worked example
# ----------------------------------------------------------------------------

def _hand_cache():
    ki = np.zeros((3, 2, BLK, 2))
    ki[0, 0, :, :] = [1.0, 0.0]
    ki[0, 1, :, :] = [0.0, 1.0]
    ki[0, 0, 5, :] = [2.0, 0.0]
    ki[1, 0, 2, :] = [0.0, 3.0]
    ki[2] = 1.0
    return ki


def test_hand_example_indexer():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))["indexer"]
    ki = _hand_cache()
    bt = np.array([[0, 1, 2]], dtype=np.int32)
    qi = np.array(g["q_idx"])[None]
    units = O.decode_units([g["seq_len"]])
    assert units[0]["pos0"] == g["query_pos"]
    for nsel in (1, 2):
        S = O.index_scores(units, qi, ki, bt, nsel, 3)
        want = np.array([[_f(x) for x in row] for row in g[f"expected_scores_nsel{nsel}"]])
        assert np.array_equal(S[0], want)
        for k, ids in g[f"expected_ids_nsel{nsel}"].items():
            assert O.select(S, units, int(k))[0].tolist() == ids


def test_hand_example_attention():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))["attention"]
    kc = np.zeros((1, 1, BLK, 1))
    vc = np.zeros((1, 1, BLK, 1))
    kc[0, 0, :3, 0] = g["keys"]
    vc[0, 0, :3, 0] = g["values"]
    q = np.full((3, 1, 1), g["q"])
    out, lse = O.unit_attention(q, 0, np.array([[0]]), kc, vc, np.array([0]), 3, 1,
                                scale=g["scale"])
    np.testing.assert_allclose(out[:, 0, 0], g["expected_out"], rtol=1e-14)
    np.testing.assert_allclose(lse[:, 0], g["expected_lse"], rtol=1e-14, atol=1e-15)


def test_hand_example_units():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))["units"]
    assert O.prefill_units(g["seq_lens"], g["q_lens"]) == g["expected"]


def test_planted_pins_would_catch_a_transposed_group():
    """Sanity of the pins themselves: a mistaken group slicing (heads taken
    interleaved instead of contiguous) changes the scores of the isolation case."""
    rng = np.random.default_rng(19)
    ki, bt = paged(rng, [400], 4, 8)
    qi = rng.standard_normal((100, 4, 8))
    qi[:, :2] = 0.0
    units = O.prefill_units([400], [100])
    un = units[0]
    wrong = max(float(np.max(qi[t, 0::2].reshape(-1) @ O.logical_block(ki, bt[0], 0, slice(0, 4, 2))
                             .reshape(BLK, -1).T)) for t in range(un["row0"], un["row1"]))
    assert wrong != 0.0


# ---------------------------------------------------------------------------
# QK-norm, partial RoPE and cache insert (the new-token step before the path)
# ---------------------------------------------------------------------------

def _golden_qk():
    with open(os.path.join(GOLDEN, "qk_norm_rope.json")) as f:
        return json.load(f)


def test_rms_norm_golden():
    for case in _golden_qk()["rms_norm"]:
        got = O.rms_norm(np.array(case["x"]), np.array(case["w"]), case["eps"])
        np.testing.assert_allclose(got, case["out"], rtol=1e-15, atol=1e-15)


def test_rope_golden():
    for case in _golden_qk()["rope"]:
        x = np.array(case["x"], dtype=np.float64)[None, None, :]
        got = O.rope(x, np.array([case["pos"]]), case["theta"], case["rotary_dim"])[0, 0]
        np.testing.assert_allclose(got, case["out"], rtol=1e-15, atol=1e-15)


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 3, 64))
    y = O.rms_norm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(64), 0.0), y, rtol=1e-13)
    # a large eps shrinks every output towards zero
    assert np.max(np.abs(O.rms_norm(x, np.ones(64), 1e12))) < 1e-4


def test_rope_matches_complex_rotation():
    """Independent formulation: channels (i, i + r/2) as the complex number
    x_i + 1j * x_{i + r/2}, multiplied by exp(1j * p * theta^(-2i/r))."""
    rng = np.random.default_rng(12)
    T, H, D, r, theta = 6, 3, 16, 8, 777.0
    x = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 10 ** 6, T)
    got = O.rope(x, pos, theta, r)
    for t in range(T):
        for i in range(r // 2):
            z = complex(x[t, 0, i], x[t, 0, i + r // 2]) * np.exp(
                1j * pos[t] * theta ** (-2.0 * i / r))
            assert abs(got[t, 0, i] - z.real) < 1e-9 * max(1.0, abs(z))
            assert abs(got[t, 0, i + r // 2] - z.imag) < 1e-9 * max(1.0, abs(z))
    np.testing.assert_array_equal(got[..., r:], x[..., r:])   # pass-through channels


def test_rope_rotation_invariants():
    rng = np.random.default_rng(13)
    T, D, r, theta = 5, 32, 16, 10000.0
    q = rng.standard_normal((T, 1, D))
    k = rng.standard_normal((T, 1, D))
    m = rng.integers(0, 5000, T).astype(np.float64)
    n = rng.integers(0, 5000, T).astype(np.float64)
    zero = np.zeros(T)
    np.testing.assert_allclose(O.rope(q, zero, theta, r), q, rtol=0, atol=0)
    back = O.rope(O.rope(q, m, theta, r), -m, theta, r)
    np.testing.assert_allclose(back, q, atol=1e-10)
    np.testing.assert_allclose(O.rope(O.rope(q, m, theta, r), n, theta, r),
                               O.rope(q, m + n, theta, r), atol=1e-9)
    # the rotary part makes dot products depend on the position difference only
    lhs = np.sum(O.rope(q, m, theta, r) * O.rope(k, n, theta, r), axis=-1)
    rhs = np.sum(O.rope(q, m - n, theta, r) * k, axis=-1)
    np.testing.assert_allclose(lhs, rhs, atol=1e-9)
    # each rotated pair keeps its length
    y = O.rope(q, m, theta, r)
    np.testing.assert_allclose(y[..., :r // 2] ** 2 + y[..., r // 2:r] ** 2,
                               q[..., :r // 2] ** 2 + q[..., r // 2:r] ** 2, rtol=1e-12)


def _insert_case(permute):
    rng = np.random.default_rng(14)
    seq_lens, q_lens = [300, 129], [300, 2]
    Hq, Hkv, D, Hi, Di = 4, 2, 16, 2, 8
    units = O.prefill_units(seq_lens, q_lens)
    T = sum(q_lens)
    nb = [(L + 127) // 128 for L in seq_lens]
    P = sum(nb)
    perm = rng.permutation(P)
    phys = perm if permute else np.arange(P)
    bt = np.zeros((2, max(nb)), dtype=np.int64)
    bt[0, :nb[0]] = phys[:nb[0]]
    bt[1, :nb[1]] = phys[nb[0]:]
    arrs = dict(q=rng.standard_normal((T, Hq, D)), k=rng.standard_normal((T, Hkv, D)),
                v=rng.standard_normal((T, Hkv, D)), ki=rng.standard_normal((T, Hi, Di)))
    caches = [np.full((P, Hkv, 128, D), 9.0), np.full((P, Hkv, 128, D), 8.0),
              np.full((P, Hi, 128, Di), 7.0)]
    wq, wk = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    res = O.qk_norm_rope_insert(units, arrs["q"], arrs["k"], arrs["v"], arrs["ki"], wq, wk,
                                1e-6, 5e5, 8, caches[0], caches[1], caches[2], bt)
    return units, arrs, caches, (wq, wk), bt, res


def test_insert_places_rows_and_leaves_the_rest():
    units, arrs, caches, (wq, wk), bt, (q_out, kc, vc, ic) = _insert_case(False)
    toks = O.token_positions(units)
    touched = set()
    for row, r, p in toks:
        phys, slot = int(bt[r][p // 128]), p % 128
        touched.add((phys, slot))
        np.testing.assert_array_equal(vc[phys, :, slot], arrs["v"][row])
        np.testing.assert_array_equal(ic[phys, :, slot], arrs["ki"][row])
        kn = O.rope(O.rms_norm(arrs["k"][row][None], wk, 1e-6), np.array([p]), 5e5, 8)[0]
        np.testing.assert_allclose(kc[phys, :, slot], kn, rtol=1e-14)
        qn = O.rope(O.rms_norm(arrs["q"][row][None], wq, 1e-6), np.array([p]), 5e5, 8)[0]
        np.testing.assert_allclose(q_out[row], qn, rtol=1e-14)
    for phys in range(kc.shape[0]):
        for slot in range(128):
            if (phys, slot) not in touched:
                assert np.all(kc[phys, :, slot] == 9.0) and np.all(vc[phys, :, slot] == 8.0)
                assert np.all(ic[phys, :, slot] == 7.0)


def test_insert_is_independent_of_physical_placement():
    u0, _, _, _, bt0, (q0, k0, v0, i0) = _insert_case(False)
    u1, _, _, _, bt1, (q1, k1, v1, i1) = _insert_case(True)
    np.testing.assert_array_equal(q0, q1)
    for r in range(bt0.shape[0]):
        for b in range(bt0.shape[1]):
            if r == 1 and b >= 2:
                continue
            np.testing.assert_array_equal(k0[bt0[r, b]], k1[bt1[r, b]])
            np.testing.assert_array_equal(v0[bt0[r, b]], v1[bt1[r, b]])
            np.testing.assert_array_equal(i0[bt0[r, b]], i1[bt1[r, b]])


# ----------------------------------------------------------------------------
# FP8 cache format: E4M3 codes, power-of-two scale per 32 channels
# ----------------------------------------------------------------------------

def _golden_fp8():
    with open(os.path.join(GOLDEN, "fp8_e4m3.json")) as f:
        return json.load(f)


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_golden():
    g = _golden_fp8()
    for e in g["decode"]:
        v = float(O.e4m3_decode(int(e["code"], 16)))
        assert v == e["value"] and math.copysign(1, v) == math.copysign(1, e["value"]), e
    for e in g["encode"]:
        assert int(O.e4m3_encode(e["value"])) == int(e["code"], 16), e
    for e in g["exponent"]:
        assert int(O.mx_exponent(e["amax"])) == e["e"], e


def test_e4m3_decode_matches_torch_float8():
    ref = _torch_e4m3_values()
    got = O.e4m3_decode(np.arange(256))
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), ~fin)            # exactly the two NaN codes
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e4m3_encode_matches_torch_cast_on_a_dense_sweep():
    vals = np.unique(_torch_e4m3_values()[np.isfinite(_torch_e4m3_values())])
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(3)
    x = np.concatenate([vals, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        rng.uniform(-448, 448, 20000), rng.normal(size=20000) * 3,
                        rng.normal(size=5000) * 1e-3])
    x = np.clip(x, -448, 448).astype(np.float32)          # exactly representable inputs
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_encode_is_nearest_and_monotone():
    rng = np.random.default_rng(4)
    x = np.sort(rng.uniform(-448, 448, 5000))
    c = O.e4m3_encode(x)
    v = O.e4m3_decode(c)
    assert np.all(np.diff(v) >= 0)
    grid = np.unique(O.e4m3_decode(np.arange(256))[np.isfinite(O.e4m3_decode(np.arange(256)))])
    best = np.abs(grid[None, :] - x[:, None]).min(axis=1)
    assert np.allclose(np.abs(v - x), best, rtol=0, atol=0)


def test_mx_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(5)
    a = np.concatenate([np.exp2(rng.uniform(-40, 40, 4000)), 448 * np.exp2(np.arange(-20, 20)),
                        1.75 * np.exp2(np.arange(-20, 20)),
                        np.nextafter(1.75 * np.exp2(np.arange(-20, 20)), np.inf)])
    e = O.mx_exponent(a).astype(np.float64)
    assert np.all(a / np.exp2(e) <= 448.0)
    assert np.all(a / np.exp2(e - 1) > 448.0)


def test_mx_quantize_error_bound_and_top_binade():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(50, 4, 128)) * np.exp2(rng.integers(-6, 6, size=(50, 4, 1)))
    codes, scales = O.mx_quantize(x)
    assert codes.dtype == np.uint8 and scales.shape == (50, 4, 4)
    y = O.mx_dequantize(codes, scales)
    e = (scales.astype(np.float64) - O.SCALE_BIAS).repeat(O.SCALE_BLOCK, axis=-1)
    half_ulp = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.exp2(e))
    assert np.all(np.abs(y - x) <= half_ulp)
    # the largest magnitude of each block lands in the top binade [224, 448]
    top = np.abs(O.e4m3_decode(codes)).reshape(50, 4, 4, 32).max(axis=-1)
    assert np.all((top >= 224) & (top <= 448))


def test_mx_round_trip_of_representable_blocks_and_scaling():
    rng = np.random.default_rng(7)
    x = rng.normal(size=(20, 64)) * 10
    c, s = O.mx_quantize(x)
    y = O.mx_dequantize(c, s)
    c2, s2 = O.mx_quantize(y)                  # values already on the grid come back
    assert np.array_equal(O.mx_dequantize(c2, s2), y)
    # codes too, unless a block's largest code is exactly 224 (then the smaller
    # exponent fits as well and is the one chosen)
    top = np.abs(O.e4m3_decode(c)).reshape(20, 2, 32).max(axis=-1)
    same = (top > 224).repeat(32, axis=-1).reshape(20, 64)
    assert np.array_equal(c[same], c2[same]) and np.array_equal(s[top > 224], s2[top > 224])
    for k in (-5, 1, 9):                       # a power-of-two factor moves only the scales
        c3, s3 = O.mx_quantize(x * 2.0 ** k)
        assert np.array_equal(c, c3) and np.array_equal(s3.astype(int), s.astype(int) + k)


def test_mx_blocks_are_independent():
    rng = np.random.default_rng(8)
    x = rng.normal(size=(3, 128))
    c, s = O.mx_quantize(x)
    x2 = x.copy()
    x2[:, 32:64] *= 1000.0
    c2, s2 = O.mx_quantize(x2)
    keep = np.r_[0:32, 64:128]
    assert np.array_equal(c[:, keep], c2[:, keep]) and np.array_equal(s[:, [0, 2, 3]],
                                                                      s2[:, [0, 2, 3]])
    assert np.all(s2[:, 1].astype(int) == s[:, 1].astype(int) + 10)   # 1000 ~ 2^10 lift


def test_insert_fp8_is_quantized_insert():
    rng = np.random.default_rng(9)
    Hq, Hkv, D, Hi, Di, P = 4, 2, 64, 2, 32, 3
    units = O.prefill_units([200], [150])
    T = 150
    q, k, v = (rng.normal(size=(T, h, D)) for h in (Hq, Hkv, Hkv))
    ki = rng.normal(size=(T, Hi, Di))
    wq, wk = 1 + 0.1 * rng.normal(size=D), 1 + 0.1 * rng.normal(size=D)
    bt = np.array([[2, 0]])
    caches = dict(k=rng.integers(0, 0x7E, (P, Hkv, 128, D)).astype(np.uint8),
                  v=rng.integers(0, 0x7E, (P, Hkv, 128, D)).astype(np.uint8),
                  i=rng.integers(0, 0x7E, (P, Hi, 128, Di)).astype(np.uint8),
                  k_s=rng.integers(100, 140, (P, Hkv, 128, D // 32)).astype(np.uint8),
                  v_s=rng.integers(100, 140, (P, Hkv, 128, D // 32)).astype(np.uint8),
                  i_s=rng.integers(100, 140, (P, Hi, 128, Di // 32)).astype(np.uint8))
    q8, out = O.qk_norm_rope_insert_fp8(units, q, k, v, ki, wq, wk, 1e-6, 1e4, 32, caches, bt)
    z = np.zeros((P, Hkv, 128, D))
    q64, kc, vc, ic = O.qk_norm_rope_insert(units, q, k, v, ki, wq, wk, 1e-6, 1e4, 32, z, z,
                                            np.zeros((P, Hi, 128, Di)), bt)
    assert np.array_equal(q8, q64)
    new = np.zeros((P, 128), dtype=bool)
    new[2, 50:128] = True                       # positions 50..199 of the request
    new[0, 0:72] = True
    for name in ("k", "v", "i", "k_s", "v_s", "i_s"):
        a, b = out[name].transpose(0, 2, 1, 3), caches[name].transpose(0, 2, 1, 3)
        assert np.array_equal(a[~new], b[~new]), name
    for codes, sc, ref in (("k", "k_s", kc), ("v", "v_s", vc), ("i", "i_s", ic)):
        c_ref, s_ref = O.mx_quantize(ref.transpose(0, 2, 1, 3)[new])
        assert np.array_equal(out[codes].transpose(0, 2, 1, 3)[new], c_ref), codes
        assert np.array_equal(out[sc].transpose(0, 2, 1, 3)[new], s_ref), sc


# ----------------------------------------------------------------------------
# per-query-token selection (multi-token decode)
# ----------------------------------------------------------------------------

def test_token_units_one_token_is_decode():
    seq = [1, 128, 129, 700, 4096]
    assert O.token_units(seq, 1) == O.decode_units(seq)


@pytest.mark.parametrize("seq_lens,T", [([300, 129, 1000], 4), ([130, 640], 3), ([8, 256], 8)])
def test_token_units_rows_positions_and_diagonals(seq_lens, T):
    units = O.token_units(seq_lens, T)
    assert len(units) == len(seq_lens) * T
    for r, L in enumerate(seq_lens):
        for i in range(T):
            un = units[r * T + i]
            p = L - T + i
            assert (un["r"], un["row0"], un["row1"], un["pos0"]) == (r, r * T + i, r * T + i + 1, p)
            assert un["tau"] * BLK <= p < (un["tau"] + 1) * BLK


def _tokens_case(rng, seq_lens, T, Hq=8, Hkv=2, D=16, Hi=4, Di=8):
    kc, bt = paged(rng, seq_lens, Hkv, D)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], Hi, BLK, Di))
    n = len(seq_lens) * T
    return kc, vc, ki, bt, rng.standard_normal((n, Hq, D)), rng.standard_normal((n, Hi, Di))


@pytest.mark.parametrize("nsel", [2, 1])
def test_token_scores_pool_to_the_tile_scores(nsel):
    """Max-pooling the per-token block scores over tokens that share a diagonal
    block gives the tile-level score of those tokens (the prefill unit)."""
    rng = np.random.default_rng(21)
    seq_lens, T = [700, 300, 1000], 5           # all three keep their T tokens in one block
    kc, vc, ki, bt, q, qi = _tokens_case(rng, seq_lens, T)
    tok = O.token_units(seq_lens, T)
    per_tok = O.index_scores(tok, qi, ki, bt, nsel, bt.shape[1])
    tile_units = O.prefill_units(seq_lens, [T] * len(seq_lens))
    assert len(tile_units) == len(seq_lens)
    tile = O.index_scores(tile_units, qi, ki, bt, nsel, bt.shape[1])
    for r in range(len(seq_lens)):
        pooled = per_tok[r * T:(r + 1) * T].max(axis=0)
        inf = ~np.isfinite(tile[r])
        np.testing.assert_array_equal(pooled[inf], tile[r][inf])
        # the library product sums in another order for another number of rows
        np.testing.assert_allclose(pooled[~inf], tile[r][~inf], rtol=1e-13, atol=1e-13)


def test_token_scores_brute_force():
    """Per-token scores by explicit loops over keys, heads and channels."""
    rng = np.random.default_rng(22)
    seq_lens, T, nsel = [260, 131], 3, 2         # the second sequence straddles blocks 0/1
    kc, vc, ki, bt, q, qi = _tokens_case(rng, seq_lens, T)
    res = O.index_scores(O.token_units(seq_lens, T), qi, ki, bt, nsel, bt.shape[1])
    Hs = ki.shape[1] // nsel
    for r, L in enumerate(seq_lens):
        for i in range(T):
            p = L - T + i
            tau = p // BLK
            for g in range(nsel):
                for b in range(bt.shape[1]):
                    got = res[r * T + i, g, b]
                    if b > tau:
                        assert got == -np.inf
                    elif b == tau:
                        assert got == np.inf
                    else:
                        best = -np.inf
                        for s in range(BLK):
                            acc = 0.0
                            for h in range(g * Hs, (g + 1) * Hs):
                                for d in range(ki.shape[3]):
                                    acc += qi[r * T + i, h, d] * ki[bt[r][b], h, s, d]
                            best = max(best, acc)
                        assert abs(got - best) <= 1e-12 * max(1.0, abs(best))


@pytest.mark.parametrize("seq_lens,T", [([700, 260, 129], 4), ([130, 1000], 2), ([8], 8)])
def test_tokens_dense_when_topk_covers_all_blocks(seq_lens, T):
    """k >= number of blocks: every token attends densely and causally."""
    rng = np.random.default_rng(23)
    kc, vc, ki, bt, q, qi = _tokens_case(rng, seq_lens, T)
    res = O.run_tokens(q, qi, kc, vc, ki, bt, seq_lens, T, 2, bt.shape[1] + 2)
    for r, L in enumerate(seq_lens):
        rows = slice(r * T, (r + 1) * T)
        out, lse = dense_reference(q[rows], logical(kc, bt[r], L), logical(vc, bt[r], L),
                                   np.arange(L - T, L), 1 / math.sqrt(q.shape[2]))
        np.testing.assert_allclose(res["out"][rows], out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][rows], lse, rtol=1e-12, atol=1e-12)


def test_tokens_last_token_is_the_decode_step():
    """The last of a sequence's T tokens sees what a one-token decode at the same
    position sees: same scores, ids and output."""
    rng = np.random.default_rng(24)
    seq_lens, T = [900, 333], 4
    kc, vc, ki, bt, q, qi = _tokens_case(rng, seq_lens, T)
    res = O.run_tokens(q, qi, kc, vc, ki, bt, seq_lens, T, 2, 3)
    last = [r * T + T - 1 for r in range(len(seq_lens))]
    dec = O.run_decode(q[last], qi[last], kc, vc, ki, bt, seq_lens, 2, 3)
    np.testing.assert_array_equal(res["scores"][last], dec["scores"])
    np.testing.assert_array_equal(res["ids"][last], dec["ids"])
    np.testing.assert_allclose(res["out"][last], dec["out"], rtol=0, atol=0)


# ----------------------------------------------------------------------------
# new-token placement: hand-worked rows, requests and positions
# ----------------------------------------------------------------------------

def test_token_positions_golden():
    """Which stored row is which (request, position), and where the insert writes
    it: a ragged batch worked by hand (tests/golden/token_positions.json)."""
    with open(os.path.join(GOLDEN, "token_positions.json")) as f:
        gold = json.load(f)
    units = O.prefill_units(gold["seq_lens"], gold["q_lens"])
    assert units == gold["expected_units"]
    toks = O.token_positions(units)
    assert [list(t) for t in toks] == gold["expected_tokens"]
    # the insert writes row `row` to logical block p // 128, row p % 128 of its request
    rng = np.random.default_rng(21)
    Hq, Hkv, D, Hi, Di = 2, 1, 8, 1, 4
    T = sum(gold["q_lens"])
    nb = [(L + 127) // 128 for L in gold["seq_lens"]]
    bt = np.zeros((3, max(nb)), dtype=np.int64)
    phys = rng.permutation(sum(nb))
    base = 0
    for r, n in enumerate(nb):
        bt[r, :n] = phys[base:base + n]
        base += n
    # each new token's V row is its row number in every channel: the slot it lands
    # in then names the row
    v = np.repeat(np.arange(T, dtype=np.float64)[:, None, None] + 1, D, axis=2)
    zeros = np.zeros((sum(nb), Hkv, 128, D))
    _, _, vc, _ = O.qk_norm_rope_insert(
        units, rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)), v,
        rng.standard_normal((T, Hi, Di)), np.ones(D), np.ones(D), 1e-6, 1e4, 0,
        zeros, zeros, np.zeros((sum(nb), Hi, 128, Di)), bt)
    req_of_row = [t[1] for t in gold["expected_tokens"]]
    for row, b, slot in gold["expected_cache_slots"]:
        r = req_of_row[row]
        assert np.all(vc[bt[r][b], 0, slot] == row + 1), (row, b, slot)
    assert np.count_nonzero(vc[:, 0, :, 0]) == T


# ----------------------------------------------------------------------------
# attention over an arbitrary id list (not the selection's own output)
# ----------------------------------------------------------------------------

def _block_masked_reference(q, k_log, v_log, positions, blocks, L, scale):
    """Softmax attention over the keys of `blocks` (a set of logical block ids)
    that are at or before each query's position: torch SDPA in float64 with that
    mask, lse with scipy. Rows without any such key are left out (NaN)."""
    keys = np.arange(k_log.shape[0])
    member = np.isin(keys // BLK, np.array(sorted(blocks), dtype=np.int64)) & (keys < L)
    mask = member[None, :] & (keys[None, :] <= np.asarray(positions)[:, None])
    T, Hq, D = q.shape
    G = Hq // k_log.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k_log).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(v_log).permute(1, 0, 2).repeat_interleave(G, 0)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale).permute(1, 0, 2).numpy()
    logits = (torch.matmul(qt, kt.transpose(1, 2)) * scale).numpy()
    lse = scipy.special.logsumexp(np.where(mask[None], logits, -np.inf), axis=2).T
    return out, lse, mask.any(axis=1)


@pytest.mark.parametrize("case", range(6))
def test_attention_over_any_id_list(case):
    """The kept list is a set of blocks masked by position: order does not matter,
    blocks after the unit's diagonal add nothing, a list without the diagonal
    attends the remaining blocks, and a row with no visible key gets out 0 and
    lse -inf (checked against SDPA over the same key set)."""
    rng = np.random.default_rng(100 + case)
    L, n, D, Hq, Hkv = 900, 200, 16, 4, 2       # blocks 0..7; units tau 5 and 6
    kc, bt = paged(rng, [L], Hkv, D)
    vc = rng.standard_normal(kc.shape)
    q = rng.standard_normal((n, Hq, D))
    units = O.prefill_units([L], [n])
    k_log, v_log = logical(kc, bt[0], L), logical(vc, bt[0], L)
    for un in units:
        tau = un["tau"]
        lists = {
            0: [tau, 2, 0],                          # unsorted
            1: [1, 3, -1, 4],                        # no diagonal; entries after -1 ignored
            2: [0, tau + 1, tau],                    # a future block
            3: [tau + 1],                            # only a future block: nothing visible
            4: [tau, 4, 1, 3, 0, 2],                 # every block up to tau, shuffled
            5: [-1, 0, 1],                           # empty list
        }[case]
        kept = []
        for b in lists:
            if b < 0:
                break
            kept.append(b)
        ids = np.array([lists, lists], dtype=np.int32)      # both selection groups
        rows = slice(un["row0"], un["row1"])
        out, lse = O.unit_attention(q[rows], un["pos0"], ids, kc, vc, bt[0], L, Hkv)
        pos = un["pos0"] + np.arange(un["row1"] - un["row0"])
        ref, ref_lse, seen = _block_masked_reference(q[rows], k_log, v_log, pos, kept, L,
                                                     1 / math.sqrt(D))
        np.testing.assert_allclose(out[seen], ref[seen], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[seen], ref_lse[seen], rtol=1e-12, atol=1e-12)
        assert np.all(out[~seen] == 0) and np.all(lse[~seen] == -np.inf)
        if case in (3, 5):
            assert not seen.any()
        else:
            assert seen.all()


# ----------------------------------------------------------------------------
# per-query-token selection in prefill
# ----------------------------------------------------------------------------

PT_CASES = [([700, 260, 129], [300, 260, 1]), ([1000], [1000]), ([513, 384], [200, 129]),
            ([5], [5])]


@pytest.mark.parametrize("seq_lens,q_lens", PT_CASES)
def test_prefill_token_units_rows_positions_and_diagonals(seq_lens, q_lens):
    """One unit per new token, in row order: request r's tokens follow those of
    requests 0..r-1, token i of request r sits at L_r - n_r + i, its diagonal
    block is position // 128."""
    units = O.prefill_token_units(seq_lens, q_lens)
    assert len(units) == sum(q_lens)
    row = 0
    for r, (L, n) in enumerate(zip(seq_lens, q_lens)):
        for i in range(n):
            un = units[row]
            p = L - n + i
            assert (un["r"], un["row0"], un["row1"], un["pos0"], un["tau"]) == \
                (r, row, row + 1, p, p // BLK)
            row += 1


def test_prefill_token_units_of_equal_chunks_are_the_multi_token_decode():
    seq = [300, 129, 1000, 8]
    for T in (1, 3, 8):
        assert O.prefill_token_units(seq, [T] * len(seq)) == O.token_units(seq, T)


@pytest.mark.parametrize("nsel", [2, 1])
def test_prefill_token_scores_pool_to_the_tile_scores(nsel):
    """Max-pooling the per-token block scores over the tokens of each prefill tile
    gives the tile-level scores of the tile path, entry by entry."""
    rng = np.random.default_rng(31)
    seq_lens, q_lens = [700, 260, 129], [300, 260, 1]
    kc, bt = paged(rng, seq_lens, 2, 16)
    ki = rng.standard_normal((kc.shape[0], 4, BLK, 8))
    qi = rng.standard_normal((sum(q_lens), 4, 8))
    tok = O.index_scores(O.prefill_token_units(seq_lens, q_lens), qi, ki, bt, nsel, bt.shape[1])
    tiles = O.prefill_units(seq_lens, q_lens)
    tile = O.index_scores(tiles, qi, ki, bt, nsel, bt.shape[1])
    for u, un in enumerate(tiles):
        pooled = tok[un["row0"]:un["row1"]].max(axis=0)
        inf = ~np.isfinite(tile[u])
        np.testing.assert_array_equal(pooled[inf], tile[u][inf])
        np.testing.assert_allclose(pooled[~inf], tile[u][~inf], rtol=1e-13, atol=1e-13)


def test_prefill_token_scores_brute_force():
    """Per-token scores of a chunked prefill by explicit loops over keys, heads and
    channels, through the block table."""
    rng = np.random.default_rng(32)
    seq_lens, q_lens, nsel = [300, 140], [45, 20], 2      # chunks straddling blocks
    kc, bt = paged(rng, seq_lens, 1, 8)
    ki = rng.standard_normal((kc.shape[0], 2, BLK, 4))
    qi = rng.standard_normal((sum(q_lens), 2, 4))
    res = O.index_scores(O.prefill_token_units(seq_lens, q_lens), qi, ki, bt, nsel,
                         bt.shape[1])
    row = 0
    for r, (L, n) in enumerate(zip(seq_lens, q_lens)):
        for i in range(n):
            p = L - n + i
            tau = p // BLK
            for g in range(nsel):
                for b in range(bt.shape[1]):
                    got = res[row, g, b]
                    if b > tau:
                        assert got == -np.inf
                    elif b == tau:
                        assert got == np.inf
                    else:
                        best = -np.inf
                        for s in range(BLK):
                            acc = 0.0
                            for d in range(4):
                                acc += qi[row, g, d] * ki[bt[r][b], g, s, d]
                            best = max(best, acc)
                        assert abs(got - best) <= 1e-12 * max(1.0, abs(best))
            row += 1


@pytest.mark.parametrize("seq_lens,q_lens", PT_CASES)
def test_prefill_tokens_dense_when_topk_covers_all_blocks(seq_lens, q_lens):
    """k >= number of blocks: every token attends densely and causally (SDPA)."""
    rng = np.random.default_rng(33)
    kc, bt = paged(rng, seq_lens, 2, 16)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 4, BLK, 8))
    T = sum(q_lens)
    q, qi = rng.standard_normal((T, 8, 16)), rng.standard_normal((T, 4, 8))
    res = O.run_prefill_tokens(q, qi, kc, vc, ki, bt, seq_lens, q_lens, 2, bt.shape[1] + 1)
    row = 0
    for r, (L, n) in enumerate(zip(seq_lens, q_lens)):
        out, lse = dense_reference(q[row:row + n], logical(kc, bt[r], L), logical(vc, bt[r], L),
                                   np.arange(L - n, L), 1 / math.sqrt(16))
        np.testing.assert_allclose(res["out"][row:row + n], out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][row:row + n], lse, rtol=1e-12, atol=1e-12)
        row += n


def test_prefill_tokens_select_per_token():
    """Each token keeps its own diagonal and min(k, tau + 1) blocks, chosen by its own
    scores; a dominant block planted for one token only is kept by that token and,
    where it loses to nothing, not by the others."""
    rng = np.random.default_rng(34)
    seq_lens, q_lens, topk = [1000], [300], 3
    kc, bt = paged(rng, seq_lens, 1, 8)
    vc = rng.standard_normal(kc.shape)
    ki = rng.standard_normal((kc.shape[0], 1, BLK, 8)) * 0.01
    qi = rng.standard_normal((300, 1, 8)) * 0.01
    # token 150 (position 850, block 6) gets a direction that block 2's keys share;
    # the other tokens have no component along it
    u = np.zeros(8)
    u[0] = 1.0
    qi[:, 0, 0] = 0.0
    base = O.run_prefill_tokens(rng.standard_normal((300, 2, 8)), qi, kc, vc, ki, bt,
                                seq_lens, q_lens, 1, topk)
    ki[bt[0][2], 0] += 10 * u
    qi[150, 0] += 10 * u
    q = rng.standard_normal((300, 2, 8))
    res = O.run_prefill_tokens(q, qi, kc, vc, ki, bt, seq_lens, q_lens, 1, topk)
    for row, un in enumerate(res["units"]):
        kept = [b for b in res["ids"][row, 0] if b >= 0]
        assert un["tau"] in kept and len(kept) == min(topk, un["tau"] + 1)
        assert kept == sorted(kept) and max(kept) == un["tau"]
        assert kept == O.select_blocks(res["scores"][row, 0], un["tau"], topk)[:len(kept)]
    assert 2 in res["ids"][150, 0] and 2 not in base["ids"][150, 0]
    # every other token's scores and selection are those of the unplanted keys
    others = [row for row in range(300) if row != 150]
    np.testing.assert_allclose(res["scores"][others], base["scores"][others], rtol=0,
                               atol=1e-15)
    np.testing.assert_array_equal(res["ids"][others], base["ids"][others])
