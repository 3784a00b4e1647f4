"""Per-query-token selection in prefill on MI355X through the C ABI, against the
oracle's prefill_token_units path: every new token scores the blocks with its own
indexer query, keeps its own top-k and attends over its own blocks (the unit's
rows are attended 32 at a time over the union of their lists). Bars of the tile
path: scores within the dot-product bound, ids exact outside near ties (then
attention is compared on the GPU's ids), out max-abs 2e-2 (bf16) or 1e-5
(fp32), lse 1e-3. Small cases are compared in full; the 32k prefill on a seeded
sample of rows."""

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


def run_tokens(w, inp, geom, cache, dev):
    batch = msa.make_batch(w.seq_lens, w.q_lens, dev)
    res = msa.prefill_tokens(geom, cache, batch, inp["q"], inp["q_idx"], w.topk)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in res.items()}


def host_caches(w, inp, cache):
    if w.cache_format == "fp8":
        return F.decoded(F.fp8_host(cache))
    return (host(inp["k_cache"]), host(synth.v_token_major(inp["v_cache"])),
            host(inp["k_idx_cache"]))


def tokens_parity(w, inp, cache, res, where):
    kc, vc, ki = host_caches(w, inp, cache)
    q, qi = host(inp["q"]), host(inp["q_idx"])
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_token_units(w.seq_lens, w.q_lens)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    P.check_scores(res["scores"].numpy(), ref, P.score_tolerance(qi, ki, w.num_sel_groups), where)
    ids = res["ids"].numpy()
    differ = P.check_ids(ids, ref, units, w.topk, where)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    d = P.check_attention(host(res["out"]), res["lse"].numpy(), out, lse, w.dtype, where)
    say(f"{where}: {len(units)} rows, {differ} near-tie rows, out {d[0]:.2e}, lse {d[1]:.2e}")


CASES = {
    "one_request": dict(seq_lens=(700,), q_lens=(300,), topk=4),
    "ragged_permuted": dict(seq_lens=(1000, 260, 129, 5), q_lens=(1000, 200, 1, 5), topk=4,
                            permute=True),
    "m3_heads": dict(seq_lens=(1100,), q_lens=(600,), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=5),
    "one_group_512_wide": dict(seq_lens=(1500, 300), q_lens=(400, 300), num_q_heads=64,
                               num_kv_heads=4, num_idx_heads=8, num_sel_groups=1, topk=6),
    "one_group_256_wide": dict(seq_lens=(1500, 200), q_lens=(700, 200), num_idx_heads=8,
                               idx_head_dim=32, num_sel_groups=1, topk=5),
    "g16_d64_di32": dict(seq_lens=(1300,), q_lens=(700,), num_q_heads=16, num_kv_heads=1,
                         head_dim=64, num_idx_heads=2, idx_head_dim=32, num_sel_groups=1),
    "topk_covers_all": dict(seq_lens=(1000,), q_lens=(1000,), topk=16),
    # 12 query heads per KV head: a work-group of one 32-row slab takes 8 heads, so the
    # second group of 8 has 4 waves without a head; tiles of 56 and 4 rows leave
    # slabs without rows
    "g12_partial_heads": dict(seq_lens=(900,), q_lens=(700,), num_q_heads=24, num_kv_heads=2,
                              topk=5),
    "fp8_g12_partial_heads": dict(seq_lens=(900,), q_lens=(700,), num_q_heads=24,
                                  num_kv_heads=2, topk=5, cache_format="fp8"),
    "topk_one": dict(seq_lens=(1000,), q_lens=(500,), topk=1),
    # unions of more than 64 blocks: the kernel's union ids come in chunks of 64
    "union_over_64": dict(seq_lens=(12000,), q_lens=(300,), topk=40),
    # a table of 2063 blocks and top-80: a slab's union may outgrow the 2048 row-mask
    # words the union kernel keeps in LDS, so it ORs the masks with global atomics
    "union_global_masks": dict(seq_lens=(264000,), q_lens=(140,), topk=80),
    "f32_ragged": dict(dtype="f32", seq_lens=(700, 300), q_lens=(300, 300), num_q_heads=4,
                       num_kv_heads=1, head_dim=64, num_idx_heads=2, idx_head_dim=32,
                       num_sel_groups=1),
    "fp8": dict(seq_lens=(1500, 700), q_lens=(800, 700), topk=6, cache_format="fp8",
                permute=True),
    "fp8_one_group_512": dict(seq_lens=(1500,), q_lens=(600,), num_q_heads=64, num_kv_heads=4,
                              num_idx_heads=8, num_sel_groups=1, topk=6, cache_format="fp8"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_tokens_parity(name, gpu_device):
    kw = dict(CASES[name])
    permute = kw.pop("permute", False)
    w = synth.small_workload(**kw)
    say(f"prefill tokens {name}")
    inp, geom, cache = T.setup(w, gpu_device, permute)
    res = run_tokens(w, inp, geom, cache, gpu_device)
    tokens_parity(w, inp, cache, res, name)


def test_prefill_tokens_equal_chunks_match_per_token_decode(gpu_device):
    """T new tokens per sequence through the prefill per-token calls and through the
    multi-token decode calls: the same rows, so the same scores and ids bit for bit,
    and outputs within two bf16 roundings."""
    T_ = 4
    w = synth.small_workload(q_lens=(T_, T_, T_), seq_lens=(9000, 3000, 700), num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=9)
    say("prefill tokens = per-token decode")
    inp, geom, cache = T.setup(w, gpu_device)
    a = run_tokens(w, inp, geom, cache, gpu_device)
    b = msa.decode_per_token(geom, cache, T_, inp["q"], inp["q_idx"], w.topk)
    torch.cuda.synchronize()
    b = {k: v.cpu() for k, v in b.items()}
    # each within the dot-product bound of the exact score, so within twice it of
    # each other (the MFMA and the dot2 paths sum in different orders)
    tol = P.score_tolerance(host(inp["q_idx"]), host(inp["k_idx_cache"]), w.num_sel_groups)
    sa, sb = a["scores"].numpy(), b["scores"].numpy()
    inf = ~np.isfinite(sb)
    assert np.array_equal(sa[inf], sb[inf])
    assert (np.abs(sa[~inf] - sb[~inf]) <= 2 * np.broadcast_to(tol[None, :, None], sb.shape)[~inf]).all()
    same = (a["ids"] == b["ids"]).all(dim=2).all(dim=1)      # rows selecting the same blocks
    assert same.float().mean().item() >= 0.5
    d = (a["out"][same].float() - b["out"][same].float()).abs().max().item()
    assert d <= 2 * 2.0 ** -7, d
    assert (a["lse"][same] - b["lse"][same]).abs().max().item() < 1e-4


def test_prefill_tokens_pool_to_the_tile_scores(gpu_device):
    """Max over a tile's per-token scores equals the tile path's score of that
    unit (both kernels, the same products: equal up to the fp32 summation order)."""
    w = synth.small_workload(seq_lens=(1500, 400), q_lens=(900, 400), num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4, topk=5)
    say("prefill tokens pool to tiles")
    inp, geom, cache = T.setup(w, gpu_device)
    a = run_tokens(w, inp, geom, cache, gpu_device)
    b = T.run_gpu(w, inp, geom, cache, gpu_device)
    units = O.prefill_units(w.seq_lens, w.q_lens)
    tol = P.score_tolerance(host(inp["q_idx"]), host(inp["k_idx_cache"]), w.num_sel_groups)
    for u, un in enumerate(units):
        pooled = a["scores"][un["row0"]:un["row1"]].numpy().max(axis=0)
        tile = b["scores"][u].numpy()
        inf = ~np.isfinite(tile)
        assert np.array_equal(pooled[inf], tile[inf])
        fin = ~inf
        assert (np.abs(pooled[fin] - tile[fin]) <=
                2 * np.broadcast_to(tol[:, None], tile.shape)[fin]).all()


@pytest.mark.parametrize("name", ["prefill_32k", "prefill_32k_sel1"])
def test_prefill_tokens_full_size_sampled(name, gpu_device):
    w = synth.WORKLOADS[name]
    say(f"{name} tokens generate")
    inp, geom, cache = T.setup(w, gpu_device)
    say(f"{name} tokens run")
    res = run_tokens(w, inp, geom, cache, gpu_device)
    units = O.prefill_token_units(w.seq_lens, w.q_lens)
    rng = np.random.default_rng(3)
    rows = sorted({0, 127, 128, len(units) - 1} | set(rng.choice(len(units), 12, False).tolist())
                  # the last and first rows of neighbouring 32-row slabs (each slab's rows
                  # are attended over their own union) in an early, a middle and a late tile
                  | {b + o for b in (1024, 16384, 30720) for o in (31, 32, 63, 64, 95, 96)})
    bt = inp["block_table"].cpu().numpy()
    nsel, Hs = w.num_sel_groups, w.num_idx_heads // w.num_sel_groups
    G = w.num_q_heads // w.num_kv_heads
    scores, ids = res["scores"].numpy(), res["ids"].numpy()
    for t in rows:
        un = units[t]
        tau = un["tau"]
        say(f"{name} row {t} (tau={tau})")
        for g in range(nsel):
            heads = slice(g * Hs, (g + 1) * Hs)
            cand = list(range(tau)) if tau > 0 else [0]
            ki, btm = T._mini_cache(inp["k_idx_cache"], bt[0], cand, heads)
            qi = host(inp["q_idx"][t:t + 1, heads])
            ref = O.unit_block_scores(qi, ki, btm, tau, 1, scores.shape[2])
            P.check_scores(scores[t, g][None, None], ref[None], P.score_tolerance(qi, ki, 1),
                           f"{name} row {t} g{g}")
            ok, _ = P.ids_acceptable(ids[t, g], ref[0], tau, w.topk)
            assert ok, f"{name} row {t} g{g}: ids {ids[t, g]}"
        for j in range(w.num_kv_heads):
            g = j if nsel == w.num_kv_heads else 0
            kept = [int(b) for b in ids[t, g] if b >= 0]
            kc, btm = T._mini_cache(inp["k_cache"], bt[0], kept, slice(j, j + 1))
            vc, _ = T._mini_cache(synth.v_token_major(inp["v_cache"]), bt[0], kept,
                                  slice(j, j + 1))
            qh = host(inp["q"][t:t + 1, j * G:(j + 1) * G])
            o, l = O.unit_attention(qh, un["pos0"], ids[t, g][None], kc, vc, btm,
                                    int(w.seq_lens[0]), 1)
            P.check_attention(host(res["out"][t:t + 1, j * G:(j + 1) * G]),
                              res["lse"][t:t + 1, j * G:(j + 1) * G].numpy(), o, l, w.dtype,
                              f"{name} row {t} kv{j}")
    # every row's entries at and after its diagonal
    tau = np.array([un["tau"] for un in units])
    cols = np.arange(scores.shape[2])[None, :]
    for g in range(nsel):
        sg = scores[:, g, :]
        assert np.isposinf(sg[cols == tau[:, None]]).all()
        assert np.isneginf(sg[cols > tau[:, None]]).all()
        assert np.isfinite(sg[cols < tau[:, None]]).all()
    del inp, cache
    torch.cuda.empty_cache()
