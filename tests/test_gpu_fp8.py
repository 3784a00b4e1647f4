"""FP8 caches on MI355X through the C ABI, against the CPU oracle.

Format: E4M3 codes with one power-of-two scale per 32 channels of a token's head
row (`oracle.msa_oracle.mx_quantize`). Readers (decode indexer, decode
attention) are compared with the oracle run on the decoded cache values, with
the bars of the plain path: scores within the dot-product bound, ids exact
outside near ties, out max-abs 2e-2, lse 1e-3. The writer (the new-token step)
is compared byte for byte where both sides quantize the same bf16 values (V and
indexer keys: codes and scale bytes); K is quantized from the fp32 normalized,
rotated key, so its decoded value must lie within one E4M3 rounding of the
oracle's exact key: |d| <= max(2^-4 |k|, 2^-9 2^e) + 1e-5 max(1, |k|) with e the
oracle's block exponent (the GPU's fp32 block maximum may pick e + 1), and its
exponent within 1 of the oracle's. Every byte that is not a new token's is
unchanged."""

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import parity as P
import test_gpu_parity as T
import test_gpu_insert as I

pytestmark = pytest.mark.gpu
BLK = 128
say, host = T.say, T.host


def fp8_host(cache):
    """Token-major host copies of the codes and scale bytes of FP8 caches."""
    n = lambda t: t.cpu().numpy()
    return dict(k=n(cache.k_cache), k_s=n(cache.k_scale),
                v=n(cache.v_cache).transpose(0, 1, 3, 2), v_s=n(cache.v_scale).transpose(0, 1, 3, 2),
                i=n(cache.k_idx_cache), i_s=n(cache.k_idx_scale))


def decoded(h):
    return (O.mx_dequantize(h["k"], h["k_s"]), O.mx_dequantize(h["v"], h["v_s"]),
            O.mx_dequantize(h["i"], h["i_s"]))


def decode_parity(w, inp, cache, res, where):
    kc, vc, ki = decoded(fp8_host(cache))
    q, qi = host(inp["q"]), host(inp["q_idx"])
    bt = inp["block_table"].cpu().numpy()
    units = O.decode_units(w.seq_lens)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    P.check_scores(res["scores"].numpy(), ref, P.score_tolerance(qi, ki, w.num_sel_groups),
                   where)
    ids = res["ids"].numpy()
    P.check_ids(ids, ref, units, w.topk, where)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    return P.check_attention(host(res["out"]), res["lse"].numpy(), out, lse, w.dtype, where)


DECODE_CASES = {
    "mixed_lengths": dict(seq_lens=(700, 1000, 129, 5, 128, 1024, 4000), topk=4),
    "m3_heads": dict(seq_lens=(20000, 3000, 131, 9000), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=9),
    "one_group_g16_d64_di32": dict(seq_lens=(5000, 777), num_q_heads=16, num_kv_heads=1,
                                   head_dim=64, num_idx_heads=4, idx_head_dim=32,
                                   num_sel_groups=1, topk=7),
    "topk_covers_all": dict(seq_lens=(900, 300), topk=12),
    "kept_blocks_over_64": dict(seq_lens=(12000, 700), topk=80),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_fp8_decode_parity(name, gpu_device):
    w = synth.small_workload(q_lens=None, cache_format="fp8", **DECODE_CASES[name])
    say(f"fp8 decode {name}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    decode_parity(w, inp, cache, res, name)


@pytest.mark.parametrize("num_seqs", [5000, 16500])
def test_fp8_decode_many_sequences(num_seqs, gpu_device):
    """Many short sequences: the decode indexer's dynamic LDS holds the schedule's
    prefix sums (up to 16384 sequences; beyond, every (sequence, block) pair is
    visited) followed by the block's staged scale bytes."""
    rng = np.random.default_rng(num_seqs)
    lens = rng.integers(1, 390, size=num_seqs).tolist()
    w = synth.small_workload(seq_lens=lens, q_lens=None, num_q_heads=4, num_kv_heads=1,
                             head_dim=64, num_idx_heads=2, idx_head_dim=64, num_sel_groups=1,
                             topk=2, plant_count=1, plant_span=None, cache_format="fp8")
    say(f"fp8 decode {num_seqs} sequences")
    inp, geom, cache = T.setup(w, gpu_device)
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    decode_parity(w, inp, cache, res, f"fp8 {num_seqs} sequences")


def test_fp8_decode_split_counts_agree(gpu_device):
    w = synth.small_workload(seq_lens=(6000, 2500), q_lens=None, cache_format="fp8", topk=11)
    say("fp8 split counts")
    inp, geom, cache = T.setup(w, gpu_device)
    base = T.run_gpu(w, inp, geom, cache, gpu_device, num_splits=1)
    for s in (2, 5, 11, 0):
        r = T.run_gpu(w, inp, geom, cache, gpu_device, num_splits=s)
        assert torch.equal(r["ids"], base["ids"])
        assert (r["out"].float() - base["out"].float()).abs().max() <= 2e-2
        assert (r["lse"] - base["lse"]).abs().max() <= 1e-4


def check_k_rows(after, ref, mask, where):
    """K codes of the new rows: decoded within one E4M3 rounding of the exact key."""
    k_gpu = O.mx_dequantize(after["k"], after["k_s"]).transpose(0, 2, 1, 3)[mask]
    k_ref = ref["k_exact"].transpose(0, 2, 1, 3)[mask]
    e_ref = ref["k_s"].transpose(0, 2, 1, 3)[mask].astype(np.int64) - O.SCALE_BIAS
    e_gpu = after["k_s"].transpose(0, 2, 1, 3)[mask].astype(np.int64) - O.SCALE_BIAS
    assert np.abs(e_gpu - e_ref).max() <= 1, f"{where}: K scale exponents differ by > 1"
    e = np.repeat(e_ref, O.SCALE_BLOCK, axis=-1).astype(np.float64)
    tol = (np.maximum(2.0 ** -4 * np.abs(k_ref), 2.0 ** -9 * np.exp2(e)) +
           1e-5 * np.maximum(1.0, np.abs(k_ref)))
    err = np.abs(k_gpu - k_ref)
    assert (err <= tol).all(), f"{where}: K codes off by {err.max():.3e}"
    return int((e_gpu != e_ref).sum())


def compare_fp8_insert(w, units, bt, before, after, q_out, new, rope, where):
    q_ref, ref = O.qk_norm_rope_insert_fp8(
        units, host(new["q"]), host(new["k"]), host(new["v"]), host(new["k_idx"]),
        host(new["q_norm_w"]), host(new["k_norm_w"]), rope["eps"], rope["theta"],
        rope["rotary_dim"], before, bt)
    # the exact keys the oracle quantized, for the K bound
    z = np.zeros(before["k"].shape)
    _, k_exact, _, _ = O.qk_norm_rope_insert(
        units, host(new["q"]), host(new["k"]), host(new["v"]), host(new["k_idx"]),
        host(new["q_norm_w"]), host(new["k_norm_w"]), rope["eps"], rope["theta"],
        rope["rotary_dim"], z, np.zeros(before["v"].shape), np.zeros(before["i"].shape), bt)
    rows = sorted({r for un in units for r in range(un["row0"], un["row1"])})
    I.check_rounded(q_out[rows], q_ref[rows], w.dtype, f"{where} q")
    for name in ("v", "v_s", "i", "i_s"):
        assert np.array_equal(after[name], ref[name]), f"{where}: {name} differs"
    m = I.new_token_mask(units, bt, after["k"].shape[0])
    for name in ("k", "k_s"):
        a, b = after[name].transpose(0, 2, 1, 3), before[name].transpose(0, 2, 1, 3)
        assert np.array_equal(a[~m], b[~m]), f"{where}: {name} outside the new rows moved"
    return check_k_rows(after, dict(ref, k_exact=k_exact), m, where)


INSERT_PREFILL = {
    "ragged": dict(kw=dict(seq_lens=(700, 300, 1000), q_lens=(300, 300, 333)), permute=True,
                   rope=dict(rotary_dim=64, eps=1e-6, theta=1e4)),
    "m3_heads": dict(kw=dict(seq_lens=(520, 1300), q_lens=(520, 389), num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4),
                     permute=False, rope=dict(rotary_dim=64, eps=1e-6, theta=1e6)),
    "d64_di32": dict(kw=dict(seq_lens=(600, 130), q_lens=(350, 130), head_dim=64,
                             idx_head_dim=32), permute=True,
                     rope=dict(rotary_dim=32, eps=1e-6, theta=1e4)),
}


@pytest.mark.parametrize("name", list(INSERT_PREFILL))
def test_fp8_insert_prefill(name, gpu_device):
    case = INSERT_PREFILL[name]
    w = synth.small_workload(cache_format="fp8", **case["kw"])
    say(f"fp8 insert prefill {name}")
    inp, geom, cache = T.setup(w, gpu_device, case["permute"])
    new = synth.make_new_tokens(w, gpu_device)
    before = fp8_host(cache)
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    q_out = torch.full_like(new["q"], float("nan"))
    I.run_insert(geom, cache, batch, new, case["rope"], q_out)
    compare_fp8_insert(w, units, bt, before, fp8_host(cache), host(q_out), new, case["rope"],
                       name)


def _fp8_decode_cache(w, dev, seed):
    """Small FP8 caches for decode sequences of any length (the last block of each
    sequence has its own physical block; other table entries are never written)."""
    rng = np.random.default_rng(seed)
    B = w.num_seqs
    P_ = B + 3
    mb = max(w.blocks(r) for r in range(B))
    bt = rng.integers(B, P_, size=(B, mb)).astype(np.int32)
    own = rng.permutation(B)
    for r in range(B):
        bt[r, w.blocks(r) - 1] = own[r]
    H, D, Hi, Di = w.num_kv_heads, w.head_dim, w.num_idx_heads, w.idx_head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def codes(*shape):       # finite E4M3 codes (0x7F / 0xFF are NaN)
        c = torch.randint(0, 0x7F, shape, generator=g, device=dev, dtype=torch.int32)
        sign = torch.randint(0, 2, shape, generator=g, device=dev, dtype=torch.int32) * 0x80
        return (c | sign).to(torch.uint8)

    def scales(*shape):
        return torch.randint(120, 134, shape, generator=g, device=dev,
                             dtype=torch.int32).to(torch.uint8)

    cache = msa.Cache(codes(P_, H, BLK, D), codes(P_, H, D, BLK), codes(P_, Hi, BLK, Di),
                      torch.from_numpy(bt).to(dev),
                      torch.tensor(w.seq_lens, dtype=torch.int32, device=dev),
                      scales(P_, H, BLK, D // 32), scales(P_, H, D // 32, BLK),
                      scales(P_, Hi, BLK, Di // 32))
    return cache, bt


@pytest.mark.parametrize("seq_lens", [(1, 128, 129, 1000, 1048576, 777777, 256)])
def test_fp8_insert_decode(seq_lens, gpu_device):
    w = synth.small_workload(seq_lens=seq_lens, q_lens=None, cache_format="fp8",
                             num_q_heads=64, num_kv_heads=4, num_idx_heads=8, num_sel_groups=4)
    rope = dict(rotary_dim=64, eps=1e-6, theta=1e7)
    say("fp8 insert decode")
    geom = T.geometry(w)
    cache, bt = _fp8_decode_cache(w, gpu_device, 5)
    new = synth.make_new_tokens(w, gpu_device)
    before = fp8_host(cache)
    q_out = torch.full_like(new["q"], float("nan"))
    I.run_insert(geom, cache, None, new, rope, q_out)
    compare_fp8_insert(w, O.decode_units(w.seq_lens), bt, before, fp8_host(cache), host(q_out),
                       new, rope, "decode")


def test_fp8_insert_then_decode_step(gpu_device):
    """A real FP8 decode step: the new tokens are quantized into the caches by the
    HIP path, then scored, selected and attended from them."""
    w = synth.small_workload(seq_lens=(20000, 3000, 131, 9000), q_lens=None, cache_format="fp8",
                             num_q_heads=64, num_kv_heads=4, num_idx_heads=8, num_sel_groups=4,
                             topk=9)
    say("fp8 insert + decode")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    new = synth.make_new_tokens(w, gpu_device)
    before = fp8_host(cache)
    bt = inp["block_table"].cpu().numpy()
    q = I.run_insert(geom, cache, None, new, synth.ROPE, torch.empty_like(new["q"]))
    compare_fp8_insert(w, O.decode_units(w.seq_lens), bt, before, fp8_host(cache), host(q), new,
                       synth.ROPE, "insert")
    inp = dict(inp, q=q)
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    decode_parity(w, inp, cache, res, "decode after insert")


def _mini_fp8(codes_t, scales_t, bt_row, blocks, heads, d_major=False):
    """Decoded float64 copy [n][heads][128][dim] of some logical blocks, and the
    block table mapping those logical ids to rows of the copy."""
    idx = torch.as_tensor(np.asarray(bt_row)[blocks].astype(np.int64), device=codes_t.device)
    c = codes_t[:, heads].index_select(0, idx).cpu().numpy()
    s = scales_t[:, heads].index_select(0, idx).cpu().numpy()
    if d_major:
        c, s = c.transpose(0, 1, 3, 2), s.transpose(0, 1, 3, 2)
    bt = np.zeros(max(blocks) + 1, dtype=np.int64)
    bt[blocks] = np.arange(len(blocks))
    return O.mx_dequantize(c, s), bt


def test_fp8_full_size_decode_1m_sampled(gpu_device):
    """The 1M-context decode on FP8 caches (the benchmark's launch): sampled
    sequences, every group's scores and ids, every KV head's attention."""
    w = synth.WORKLOADS["decode_1m_b8_fp8"]
    say(f"{w.name} generate")
    inp, geom, cache = T.setup(w, gpu_device)
    say(f"{w.name} run")
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    units = O.decode_units(w.seq_lens)
    bt_all = inp["block_table"].cpu().numpy()
    Hs, G = w.num_idx_heads // w.num_sel_groups, w.num_q_heads // w.num_kv_heads
    scores, ids = res["scores"].numpy(), res["ids"].numpy()
    for u in T._sample_units(units, 2, 2):
        un = units[u]
        r, tau = un["r"], un["tau"]
        say(f"{w.name} unit {u}")
        qi_all = host(inp["q_idx"][r:r + 1])
        for g in range(w.num_sel_groups):
            heads = slice(g * Hs, (g + 1) * Hs)
            ki, btm = _mini_fp8(inp["k_idx_cache"], inp["k_idx_scale"], bt_all[r],
                                list(range(tau)), heads)
            qi = qi_all[:, heads]
            ref = O.unit_block_scores(qi, ki, btm, tau, 1, scores.shape[2])
            P.check_scores(scores[u, g][None, None], ref[None], P.score_tolerance(qi, ki, 1),
                           f"u{u} g{g}")
            ok, _ = P.ids_acceptable(ids[u, g], ref[0], tau, w.topk)
            assert ok, f"u{u} g{g}: ids {ids[u, g]}"
        for j in range(w.num_kv_heads):
            g = j if w.num_sel_groups == w.num_kv_heads else 0
            kept = [int(b) for b in ids[u, g] if b >= 0]
            kc, btm = _mini_fp8(inp["k_cache"], inp["k_scale"], bt_all[r], kept, slice(j, j + 1))
            vc, _ = _mini_fp8(inp["v_cache"], inp["v_scale"], bt_all[r], kept, slice(j, j + 1),
                              d_major=True)
            qh = host(inp["q"][r:r + 1, j * G:(j + 1) * G])
            o, l = O.unit_attention(qh, un["pos0"], ids[u, j][None], kc, vc, btm,
                                    int(w.seq_lens[r]), 1)
            P.check_attention(host(res["out"][r:r + 1, j * G:(j + 1) * G]),
                              res["lse"][r:r + 1, j * G:(j + 1) * G].numpy(), o, l, w.dtype,
                              f"u{u} kv{j}")
    sc = res["scores"].numpy()
    assert np.isposinf(sc[:, :, -1]).all() and np.isfinite(sc[:, :, :-1]).all()
    del inp, cache
    torch.cuda.empty_cache()


def prefill_index_parity(w, inp, cache, scores, ids, where):
    _, _, ki = decoded(fp8_host(cache))
    qi = host(inp["q_idx"])
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    P.check_scores(scores, ref, P.score_tolerance(qi, ki, w.num_sel_groups), where)
    P.check_ids(ids, ref, units, w.topk, where)


PREFILL_INDEX = {
    "m3_heads": dict(seq_lens=(1100,), q_lens=(600,), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=5),
    "ragged_permuted": dict(seq_lens=(1000, 260, 129, 5), q_lens=(1000, 200, 1, 5), topk=4),
    "one_head_groups_di32": dict(seq_lens=(1300,), q_lens=(700,), num_q_heads=16,
                                 num_kv_heads=4, head_dim=64, num_idx_heads=4, idx_head_dim=32,
                                 num_sel_groups=4, topk=3),
    "four_heads_di32": dict(seq_lens=(900, 400), q_lens=(500, 400), num_idx_heads=4,
                            idx_head_dim=32, num_sel_groups=1, topk=4),
}


@pytest.mark.parametrize("name", list(PREFILL_INDEX))
def test_fp8_prefill_indexer_parity(name, gpu_device):
    w = synth.small_workload(cache_format="fp8", **PREFILL_INDEX[name])
    say(f"fp8 prefill indexer {name}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    scores = torch.empty((batch.total_units, w.num_sel_groups, cache.max_blocks),
                         dtype=torch.float32, device=gpu_device)
    ids = torch.empty((batch.total_units, w.num_sel_groups, w.topk), dtype=torch.int32,
                      device=gpu_device)
    msa.msa_index_scores(geom, cache, batch, inp["q_idx"], scores)
    msa.msa_select_topk_blocks(scores, w.topk, ids)
    torch.cuda.synchronize()
    prefill_index_parity(w, inp, cache, scores.cpu().numpy(), ids.cpu().numpy(), name)


def prefill_parity(w, inp, cache, res, where):
    kc, vc, ki = decoded(fp8_host(cache))
    q, qi = host(inp["q"]), host(inp["q_idx"])
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    ref = O.index_scores(units, qi, ki, bt, w.num_sel_groups, bt.shape[1])
    P.check_scores(res["scores"].numpy(), ref, P.score_tolerance(qi, ki, w.num_sel_groups),
                   where)
    ids = res["ids"].numpy()
    P.check_ids(ids, ref, units, w.topk, where)
    out, lse = O.attention(units, ids, q, kc, vc, bt, w.seq_lens, w.num_sel_groups)
    return P.check_attention(host(res["out"]), res["lse"].numpy(), out, lse, w.dtype, where)


PREFILL_FULL = {
    "one_request": dict(seq_lens=(700,), q_lens=(300,)),
    "ragged_permuted": dict(seq_lens=(1000, 260, 129, 5), q_lens=(1000, 200, 1, 5), topk=4),
    "m3_heads": dict(seq_lens=(1100,), q_lens=(600,), num_q_heads=64, num_kv_heads=4,
                     num_idx_heads=8, num_sel_groups=4, topk=5),
    "g16_d64_di32": dict(seq_lens=(1300,), q_lens=(700,), num_q_heads=16, num_kv_heads=1,
                         head_dim=64, num_idx_heads=2, idx_head_dim=32, num_sel_groups=1),
    "topk_covers_all": dict(seq_lens=(1000,), q_lens=(1000,), topk=16),
    "kept_blocks_over_64": dict(seq_lens=(10245,), q_lens=(261,), topk=80),
    "m3_heads_one_group": dict(seq_lens=(1500, 300), q_lens=(400, 300), num_q_heads=64,
                               num_kv_heads=4, num_idx_heads=8, num_sel_groups=1, topk=6),
    "one_group_di32_w256": dict(seq_lens=(1500, 200), q_lens=(700, 200), num_idx_heads=8,
                                idx_head_dim=32, num_sel_groups=1, topk=5),
    # more cache blocks than the units keep in all (staged: slots claimed per kept
    # pair instead of copies where the cache holds the blocks)
    "long_prefixes": dict(seq_lens=(20000, 3000), q_lens=(130, 200), topk=5),
    "long_prefix_one_group": dict(seq_lens=(12000,), q_lens=(300,), num_sel_groups=1, topk=3),
}


@pytest.mark.parametrize("staged", [False, True], ids=["direct", "staged"])
@pytest.mark.parametrize("name", list(PREFILL_FULL))
def test_fp8_prefill_parity(name, staged, gpu_device):
    """direct: the attention kernel converts the codes it reads; staged: every kept
    (block, KV head) is converted once into the workspace and the bf16 kernel reads
    the copies (msa_sparse_attn_prefill_staged)."""
    w = synth.small_workload(cache_format="fp8", **PREFILL_FULL[name])
    say(f"fp8 prefill {name} {'staged' if staged else 'direct'}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    res = T.run_gpu(w, inp, geom, cache, gpu_device, staged=staged)
    prefill_parity(w, inp, cache, res, name)


STAGED_EXACT = {
    # copies where the cache holds the blocks (blocks <= units * topk)
    "in_place": dict(seq_lens=(1500, 700, 129), q_lens=(600, 700, 129), topk=5),
    # claimed slots (blocks > units * topk), one selection group
    "claimed": dict(seq_lens=(20000, 900), q_lens=(260, 129), topk=4, num_sel_groups=1),
}


@pytest.mark.parametrize("name", list(STAGED_EXACT))
def test_fp8_prefill_staged_equals_bf16_path(name, gpu_device):
    """The staged copies are exact: attending them equals the bf16 prefill call on
    bf16 caches holding the decoded values, bit for bit (same kernel, same inputs)."""
    w = synth.small_workload(cache_format="fp8", num_q_heads=64, num_kv_heads=4,
                             num_idx_heads=8, **dict(dict(num_sel_groups=4), **STAGED_EXACT[name]))
    say(f"fp8 staged ({name}) against bf16 caches of the decoded values")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    res = msa.prefill(geom, cache, batch, inp["q"], inp["q_idx"], w.topk, staged=True)
    h = fp8_host(cache)
    kd = torch.from_numpy(O.mx_dequantize(h["k"], h["k_s"])).to(torch.bfloat16)
    vd = torch.from_numpy(O.mx_dequantize(h["v"], h["v_s"])).to(torch.bfloat16)
    id_ = torch.from_numpy(O.mx_dequantize(h["i"], h["i_s"])).to(torch.bfloat16)
    k16 = kd.to(gpu_device).contiguous()
    v16 = vd.transpose(2, 3).to(gpu_device).contiguous()          # back to d-major
    c16 = msa.Cache(k16, v16, id_.to(gpu_device), inp["block_table"], inp["seq_lens"])
    g16 = msa.Geometry(w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_idx_heads,
                       w.idx_head_dim, w.num_sel_groups, "bf16", "plain")
    out = torch.empty_like(inp["q"])
    lse = torch.empty(inp["q"].shape[:2], dtype=torch.float32, device=gpu_device)
    msa.msa_sparse_attn_prefill(g16, c16, batch, inp["q"], res["ids"], w.topk, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), res["out"].cpu())
    assert torch.equal(lse.cpu(), res["lse"].cpu())


def test_fp8_insert_then_prefill_step(gpu_device):
    """A chunked prefill on FP8 caches: the chunk's tokens are quantized into the
    caches by the HIP path (after a cached prefix), then scored, selected and
    attended from them."""
    w = synth.small_workload(seq_lens=(1500, 700), q_lens=(600, 700), topk=4, cache_format="fp8",
                             num_q_heads=64, num_kv_heads=4, num_idx_heads=8, num_sel_groups=4)
    say("fp8 insert + prefill")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    new = synth.make_new_tokens(w, gpu_device)
    before = fp8_host(cache)
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    q = I.run_insert(geom, cache, batch, new, synth.ROPE, torch.empty_like(new["q"]))
    compare_fp8_insert(w, units, bt, before, fp8_host(cache), host(q), new, synth.ROPE,
                       "insert")
    inp = dict(inp, q=q)
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    prefill_parity(w, inp, cache, res, "prefill after insert")


@pytest.mark.parametrize("name,staged", [("prefill_32k_fp8", False), ("prefill_32k_fp8", True),
                                         ("prefill_32k_fp8_sel1", True)])
def test_fp8_full_size_prefill_32k_sampled(name, staged, gpu_device):
    """The 32k prefill on FP8 caches (the benchmark's launches, four selection groups
    or one; the staged attention is the one the benchmark times): sampled units,
    every group's scores and ids, attention of sampled rows for every KV head."""
    w = synth.WORKLOADS[name]
    say(f"{w.name} generate")
    inp, geom, cache = T.setup(w, gpu_device)
    say(f"{w.name} run" + (" staged" if staged else ""))
    res = T.run_gpu(w, inp, geom, cache, gpu_device, staged=staged)
    units = O.prefill_units(w.seq_lens, w.q_lens)
    bt_all = inp["block_table"].cpu().numpy()
    Hs, G = w.num_idx_heads // w.num_sel_groups, w.num_q_heads // w.num_kv_heads
    scores, ids = res["scores"].numpy(), res["ids"].numpy()
    rng = np.random.default_rng(4)
    for u in T._sample_units(units, 4, 1):
        un = units[u]
        r, tau = un["r"], un["tau"]
        say(f"{w.name} unit {u} (tau={tau})")
        rows = slice(un["row0"], un["row1"])
        for g in range(w.num_sel_groups):
            heads = slice(g * Hs, (g + 1) * Hs)
            cand = list(range(tau)) if tau > 0 else [0]
            ki, btm = _mini_fp8(inp["k_idx_cache"], inp["k_idx_scale"], bt_all[r], cand, heads)
            qi = host(inp["q_idx"][rows, heads])
            ref = O.unit_block_scores(qi, ki, btm, tau, 1, scores.shape[2])
            P.check_scores(scores[u, g][None, None], ref[None], P.score_tolerance(qi, ki, 1),
                           f"u{u} g{g}")
            ok, _ = P.ids_acceptable(ids[u, g], ref[0], tau, w.topk)
            assert ok, f"u{u} g{g}: ids {ids[u, g]}"
        n = un["row1"] - un["row0"]
        pick = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 8)]))
        for j in range(w.num_kv_heads):
            g = j if w.num_sel_groups == w.num_kv_heads else 0
            kept = [int(b) for b in ids[u, g] if b >= 0]
            kc, btm = _mini_fp8(inp["k_cache"], inp["k_scale"], bt_all[r], kept, slice(j, j + 1))
            vc, _ = _mini_fp8(inp["v_cache"], inp["v_scale"], bt_all[r], kept, slice(j, j + 1),
                              d_major=True)
            qh = host(inp["q"][rows, j * G:(j + 1) * G])
            for t in pick:
                o, l = O.unit_attention(qh[t:t + 1], un["pos0"] + t, ids[u, g][None], kc, vc,
                                        btm, int(w.seq_lens[r]), 1)
                P.check_attention(host(res["out"][un["row0"] + t, j * G:(j + 1) * G])[None],
                                  res["lse"][un["row0"] + t, j * G:(j + 1) * G].numpy()[None],
                                  o, l, w.dtype, f"u{u} row{t} kv{j}")
    del inp, cache
    torch.cuda.empty_cache()
