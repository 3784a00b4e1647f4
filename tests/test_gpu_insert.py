"""Parity of the new-token step (QK-norm + partial RoPE + K/V/k_idx insert,
msa_qk_norm_rope_insert) with the CPU oracle, on MI355X, through the C ABI.

Bar: V and indexer keys are moved bit-exactly and every cache entry that is not a
new token's is left bit-identical. Normalized and rotated queries and keys
follow the oracle within the rounding of the storage dtype: for bf16 one
rounding (at most 2^-8 of the value) plus 1e-5 of fp32 arithmetic slack; for
fp32, 1e-5 relative to max(1, |value|)."""

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from block_sparse_long_11_amd import synth
from oracle import msa_oracle as O
import test_gpu_parity as T

pytestmark = pytest.mark.gpu
BLK = 128
say = T.say
host = T.host


def check_rounded(gpu, ref, dtype, where):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    slack = 1e-5 * np.maximum(1.0, np.abs(ref))
    tol = (2.0 ** -8 * np.abs(ref) + slack) if dtype == "bf16" else slack
    err = np.abs(gpu - ref)
    bad = err > tol
    assert not bad.any(), (f"{where}: {int(bad.sum())} entries off, worst "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max()) if err.size else 0.0


def oracle_insert(units, new, cache_h, bt, rope):
    """Oracle over host copies: returns (q_full, k_cache, v_cache token-major, k_idx)."""
    return O.qk_norm_rope_insert(units, host(new["q"]), host(new["k"]), host(new["v"]),
                                 host(new["k_idx"]), host(new["q_norm_w"]),
                                 host(new["k_norm_w"]), rope["eps"], rope["theta"],
                                 rope["rotary_dim"], cache_h["k"], cache_h["v"], cache_h["i"],
                                 bt)


def cache_host(cache):
    return dict(k=host(cache.k_cache), v=host(synth.v_token_major(cache.v_cache)),
                i=host(cache.k_idx_cache))


def new_token_mask(units, bt, P):
    """[P][128] True where a new token is written."""
    m = np.zeros((P, BLK), dtype=bool)
    for un in units:
        for t in range(un["row1"] - un["row0"]):
            p = un["pos0"] + t
            m[bt[un["r"]][p // BLK], p % BLK] = True
    return m


def compare_insert(w, units, bt, before, after, q_out, ref, where):
    """after/before: host caches; ref: the oracle's (q_full, kc, vc, ic)."""
    q_ref, kc_ref, vc_ref, ic_ref = ref
    P = after["k"].shape[0]
    m = new_token_mask(units, bt, P)
    rows = sorted({r for un in units for r in range(un["row0"], un["row1"])})
    eq = check_rounded(q_out[rows], q_ref[rows], w.dtype, f"{where} q")
    ek = check_rounded(after["k"].transpose(0, 2, 1, 3)[m], kc_ref.transpose(0, 2, 1, 3)[m],
                       w.dtype, f"{where} k")
    # untouched key rows: bit-identical to before
    keep = ~m
    assert np.array_equal(after["k"].transpose(0, 2, 1, 3)[keep],
                          before["k"].transpose(0, 2, 1, 3)[keep]), f"{where}: k rows moved"
    # V and indexer keys: every entry equals the oracle's exactly
    assert np.array_equal(after["v"], vc_ref.astype(np.float32)), f"{where}: v_cache differs"
    assert np.array_equal(after["i"], ic_ref.astype(np.float32)), f"{where}: k_idx differs"
    return eq, ek


def run_insert(geom, cache, batch, new, rope, q_out=None):
    out = msa.msa_qk_norm_rope_insert(geom, cache, batch, new["q"], new["k"], new["v"],
                                      new["k_idx"], new["q_norm_w"], new["k_norm_w"],
                                      rope["eps"], rope["theta"], rope["rotary_dim"], q_out)
    torch.cuda.synchronize()
    return out


PREFILL_CASES = {
    # ragged chunks: units start at 8-aligned and unaligned offsets and end short
    "bf16_rd64": dict(kw=dict(seq_lens=(700, 300, 1000), q_lens=(300, 300, 333)),
                      rope=dict(rotary_dim=64, eps=1e-6, theta=1e4), permute=True),
    "bf16_m3_heads": dict(kw=dict(seq_lens=(520, 1300), q_lens=(520, 389), num_q_heads=64,
                                  num_kv_heads=4, num_idx_heads=8, num_sel_groups=4),
                          rope=dict(rotary_dim=64, eps=1e-6, theta=1e4), permute=False),
    "bf16_full_rotation": dict(kw=dict(seq_lens=(900,), q_lens=(900,)),
                               rope=dict(rotary_dim=128, eps=1e-5, theta=1e6), permute=True),
    "bf16_rd16": dict(kw=dict(seq_lens=(400,), q_lens=(257,)),
                      rope=dict(rotary_dim=16, eps=1e-6, theta=5e5), permute=False),
    "bf16_no_rope": dict(kw=dict(seq_lens=(400,), q_lens=(199,)),
                         rope=dict(rotary_dim=0, eps=1e-6, theta=1e4), permute=False),
    "bf16_d64": dict(kw=dict(seq_lens=(600, 130), q_lens=(350, 130), head_dim=64,
                             idx_head_dim=32),
                     rope=dict(rotary_dim=32, eps=1e-6, theta=1e4), permute=True),
    "bf16_fewer_idx_heads": dict(kw=dict(seq_lens=(333,), q_lens=(333,), num_q_heads=8,
                                         num_kv_heads=4, num_idx_heads=2, num_sel_groups=1),
                                 rope=dict(rotary_dim=64, eps=1e-6, theta=1e4), permute=False),
    "f32_d128": dict(kw=dict(dtype="f32", seq_lens=(520, 77), q_lens=(400, 77)),
                     rope=dict(rotary_dim=64, eps=1e-6, theta=1e4), permute=True),
    "f32_d64_rd8": dict(kw=dict(dtype="f32", seq_lens=(300,), q_lens=(300,), head_dim=64,
                                idx_head_dim=32, num_q_heads=4, num_kv_heads=1,
                                num_idx_heads=1, num_sel_groups=1),
                        rope=dict(rotary_dim=8, eps=1e-6, theta=1e4), permute=False),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_insert_prefill_parity(name, gpu_device):
    case = PREFILL_CASES[name]
    w = synth.small_workload(**case["kw"])
    rope = case["rope"]
    say(f"insert prefill {name}")
    inp, geom, cache = T.setup(w, gpu_device, case["permute"])
    new = synth.make_new_tokens(w, gpu_device)
    before = cache_host(cache)
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    q_out = torch.full_like(new["q"], float("nan"))
    run_insert(geom, cache, batch, new, rope, q_out)
    ref = oracle_insert(units, new, before, bt, rope)
    compare_insert(w, units, bt, before, cache_host(cache), host(q_out), ref, name)


def test_insert_in_place_equals_out_of_place(gpu_device):
    w = synth.small_workload(seq_lens=(700, 300), q_lens=(300, 300))
    rope = synth.ROPE
    say("insert in place")
    inp, geom, cache = T.setup(w, gpu_device)
    new = synth.make_new_tokens(w, gpu_device)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    q_sep = torch.empty_like(new["q"])
    run_insert(geom, cache, batch, new, rope, q_sep)
    k_first = cache.k_cache.clone()
    q_in = new["q"].clone()
    run_insert(geom, cache, batch, dict(new, q=q_in), rope, None)
    assert torch.equal(q_in.view(torch.int16), q_sep.view(torch.int16))
    assert torch.equal(cache.k_cache.view(torch.int16), k_first.view(torch.int16))


def _decode_cache(w, dev, seed):
    """Small caches for decode sequences of any length: only each sequence's last
    block is backed by its own physical block; the other table entries point at
    shared blocks and are never written."""
    rng = np.random.default_rng(seed)
    B = w.num_seqs
    P = B + 3
    mb = max(w.blocks(r) for r in range(B))
    bt = rng.integers(B, P, size=(B, mb)).astype(np.int32)
    own = rng.permutation(B)
    for r in range(B):
        bt[r, w.blocks(r) - 1] = own[r]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def rnd(*shape):
        return torch.randn(shape, generator=g, device=dev).to(dt)

    H, D = w.num_kv_heads, w.head_dim
    return msa.Cache(rnd(P, H, BLK, D), rnd(P, H, D, BLK),
                     rnd(P, w.num_idx_heads, BLK, w.idx_head_dim),
                     torch.from_numpy(bt).to(dev),
                     torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)), bt


DECODE_CASES = {
    # positions at block starts and ends, mid-block, and near 2^20
    "bf16_edges": dict(seq_lens=(1, 128, 129, 1000, 1048576, 777777, 256),
                       rope=dict(rotary_dim=64, eps=1e-6, theta=1e4)),
    "bf16_m3_heads_1m": dict(seq_lens=(1048576, 1048575, 1040000, 5), num_q_heads=64,
                             num_kv_heads=4, num_idx_heads=8, num_sel_groups=4,
                             rope=dict(rotary_dim=64, eps=1e-6, theta=1e7)),
    "f32": dict(dtype="f32", seq_lens=(3000, 700, 1048576), num_q_heads=4, num_kv_heads=1,
                head_dim=64, num_idx_heads=1, idx_head_dim=32, num_sel_groups=1,
                rope=dict(rotary_dim=32, eps=1e-6, theta=1e4)),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_insert_decode_parity(name, gpu_device):
    kw = dict(DECODE_CASES[name])
    rope = kw.pop("rope")
    w = synth.small_workload(q_lens=None, **kw)
    say(f"insert decode {name}")
    geom = T.geometry(w)
    cache, bt = _decode_cache(w, gpu_device, 11)
    new = synth.make_new_tokens(w, gpu_device)
    before = cache_host(cache)
    q_out = torch.full_like(new["q"], float("nan"))
    run_insert(geom, cache, None, new, rope, q_out)
    units = O.decode_units(w.seq_lens)
    ref = oracle_insert(units, new, before, bt, rope)
    compare_insert(w, units, bt, before, cache_host(cache), host(q_out), ref, name)


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_insert_then_path_end_to_end(mode, gpu_device):
    """One real step: the new tokens are normalized, rotated and inserted by the
    HIP path, then scored, selected and attended; the step's outputs match the
    oracle run on the inserted caches and queries."""
    if mode == "prefill":
        w = synth.small_workload(seq_lens=(1500, 700), q_lens=(600, 700), topk=4)
    else:
        w = synth.small_workload(seq_lens=(20000, 3000, 131, 9000), q_lens=None,
                                 num_q_heads=64, num_kv_heads=4, num_idx_heads=8,
                                 num_sel_groups=4, topk=9)
    say(f"insert + {mode}")
    inp, geom, cache = T.setup(w, gpu_device, permute=True)
    new = synth.make_new_tokens(w, gpu_device)
    before = cache_host(cache)
    bt = inp["block_table"].cpu().numpy()
    batch = None if w.is_decode else msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    units = O.decode_units(w.seq_lens) if w.is_decode else O.prefill_units(w.seq_lens,
                                                                           w.q_lens)
    q = run_insert(geom, cache, batch, new, synth.ROPE, torch.empty_like(new["q"]))
    ref = oracle_insert(units, new, before, bt, synth.ROPE)
    compare_insert(w, units, bt, before, cache_host(cache), host(q), ref, f"{mode} insert")
    inp = dict(inp, q=q, k_cache=cache.k_cache, v_cache=cache.v_cache,
               k_idx_cache=cache.k_idx_cache)
    res = T.run_gpu(w, inp, geom, cache, gpu_device)
    T.full_parity(w, inp, res, f"{mode} after insert")


def _token_slots(units, bt):
    """Physical block and row of every new token, in row order."""
    toks = O.token_positions(units)
    phys = np.array([bt[r][p // BLK] for _, r, p in toks], dtype=np.int64)
    row = np.array([p % BLK for _, _, p in toks], dtype=np.int64)
    return phys, row


@pytest.mark.parametrize("name", ["prefill_32k", "decode_1m_b8"])
def test_full_size_insert_sampled(name, gpu_device):
    """The launch the benchmark times, on the full workload: sampled units against
    the oracle (each unit alone, on a copy of its one block), and at full size the
    property that every new token's V and indexer-key rows are its input's bits."""
    w = synth.WORKLOADS[name]
    say(f"{name} insert generate")
    inp, geom, cache = T.setup(w, gpu_device)
    new = synth.make_new_tokens(w, gpu_device)
    batch = None if w.is_decode else msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    units = O.decode_units(w.seq_lens) if w.is_decode else O.prefill_units(w.seq_lens,
                                                                           w.q_lens)
    bt = inp["block_table"].cpu().numpy()
    picks = T._sample_units(units, 6, 3)

    def block_copy(u):
        ph = int(bt[units[u]["r"]][units[u]["pos0"] // BLK])
        return dict(k=host(cache.k_cache[ph:ph + 1]),
                    v=host(synth.v_token_major(cache.v_cache[ph:ph + 1])),
                    i=host(cache.k_idx_cache[ph:ph + 1]))

    before = {u: block_copy(u) for u in picks}
    q_out = torch.empty_like(new["q"])
    say(f"{name} insert run")
    run_insert(geom, cache, batch, new, synth.ROPE, q_out)

    for u in picks:
        un = units[u]
        n = un["row1"] - un["row0"]
        say(f"{name} insert unit {u} (r={un['r']}, pos0={un['pos0']}, rows={n})")
        sub = [dict(r=0, tau=un["tau"], row0=0, row1=n, pos0=un["pos0"])]
        bt_u = np.zeros((1, un["pos0"] // BLK + 1), dtype=np.int64)    # block -> copy 0
        rows = slice(un["row0"], un["row1"])
        new_u = {k: (v if k.endswith("_norm_w") else v[rows]) for k, v in new.items()}
        ref = oracle_insert(sub, new_u, before[u], bt_u, synth.ROPE)
        compare_insert(w, sub, bt_u, before[u], block_copy(u), host(q_out[rows]), ref,
                       f"{name} unit {u}")

    phys, row = _token_slots(units, bt)
    pi = torch.from_numpy(phys).to(gpu_device)
    ri = torch.from_numpy(row).to(gpu_device)
    as16 = torch.int16 if w.dtype == "bf16" else torch.int32
    v_put = cache.v_cache[pi, :, :, ri]                      # [T][H_kv][D]
    assert torch.equal(v_put.view(as16), new["v"].view(as16)), f"{name}: V rows"
    i_put = cache.k_idx_cache[pi, :, ri, :]                  # [T][H_i][D_i]
    assert torch.equal(i_put.view(as16), new["k_idx"].view(as16)), f"{name}: k_idx rows"
    del inp, cache, new, q_out
    torch.cuda.empty_cache()
