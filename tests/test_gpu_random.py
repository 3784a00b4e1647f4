"""Seeded random geometries through the whole path (scores, ids, out, lse), against
the CPU oracle, on bf16, fp32 and FP8 caches.

Each case draws a valid geometry (KV heads, GQA group size, head dims, indexer
heads per selection group, one selection group or one per KV head), a ragged
batch (1-4 requests, lengths 1-2600, prefill chunks of any size up to the whole
request, or 2-8 new tokens per sequence each with its own selection), k, and an
identity or permuted block table, from its own seed; the oracle's work is kept
to a few seconds a case by redrawing the batch. Bars are those of the fixed
cases: scores within the dot-product bound, ids exact outside near ties, out
max-abs 2e-2 (bf16) or 1e-5 (fp32), lse 1e-3."""

import numpy as np
import pytest

from block_sparse_long_11_amd import synth
import test_gpu_parity as T
import test_gpu_fp8 as F
import test_gpu_tokens as K

pytestmark = pytest.mark.gpu
BLK = 128
ORACLE_BUDGET = 1.5e9   # multiply-adds of the oracle's attention per case


def draw_case(seed, decode, per_token=False):
    rng = np.random.default_rng(1000 + seed)
    fmt = ["bf16", "bf16", "fp8", "fp8", "f32"][seed % 5]
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    di = int(rng.choice([32, 64]))
    nsel = int(rng.choice([1, hkv]))
    hs = int(rng.choice([1, 2, 4, 8]))
    tokens = int(rng.integers(2, 9)) if per_token else 1   # new tokens per sequence
    while True:
        n = int(rng.integers(1, 5))
        lens = [max(int(x), tokens) for x in rng.integers(1, 2600, size=n)]
        q_lens = None if decode else [int(rng.integers(1, L + 1)) for L in lens]
        topk = int(rng.integers(1, 25))
        rows = n * tokens if decode else sum(q_lens)
        kept = min(topk, max(lens) // BLK + 1) * BLK
        if rows * hkv * g * kept * d <= ORACLE_BUDGET:
            break
    kw = dict(num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d, num_idx_heads=nsel * hs,
              idx_head_dim=di, num_sel_groups=nsel, topk=topk, seed=seed,
              tokens_per_seq=tokens)
    if fmt == "fp8":
        kw["cache_format"] = "fp8"
    w = synth.small_workload(dtype="f32" if fmt == "f32" else "bf16", seq_lens=lens,
                             q_lens=q_lens, **kw)
    return w, fmt, bool(rng.integers(0, 2))


def describe(w, fmt, permute):
    return (f"{fmt} T={w.tokens_per_seq} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
            f"Hi={w.num_idx_heads} Di={w.idx_head_dim} nsel={w.num_sel_groups} "
            f"k={w.topk} lens={w.seq_lens} q={w.q_lens} permute={permute}")


def run_case(seed, decode, dev):
    w, fmt, permute = draw_case(seed, decode)
    where = f"{'decode' if decode else 'prefill'} seed {seed}: {describe(w, fmt, permute)}"
    T.say(where)
    inp, geom, cache = T.setup(w, dev, permute=permute)
    res = T.run_gpu(w, inp, geom, cache, dev)
    if fmt == "fp8":
        check = F.decode_parity if decode else F.prefill_parity
        check(w, inp, cache, res, where)
    else:
        T.full_parity(w, inp, res, where)


@pytest.mark.parametrize("seed", range(20))
def test_random_prefill(seed, gpu_device):
    run_case(seed, False, gpu_device)


@pytest.mark.parametrize("seed", range(15))
def test_random_decode(seed, gpu_device):
    run_case(seed, True, gpu_device)


@pytest.mark.parametrize("seed", range(12))
def test_random_per_token(seed, gpu_device):
    """Several new tokens per sequence (2-8), each with its own selection."""
    w, fmt, permute = draw_case(100 + seed, True, per_token=True)
    where = f"per-token seed {seed}: {describe(w, fmt, permute)}"
    T.say(where)
    inp, geom, cache = T.setup(w, gpu_device, permute=permute)
    res = K.run_tokens(w, inp, geom, cache)
    K.tokens_parity(w, inp, cache, res, where)


def draw_rope(seed, w):
    rng = np.random.default_rng(5000 + seed)
    dims = [0] + [r for r in (8, 16, 32, 64, 128)
                  if r <= w.head_dim and (r >= 16 or w.dtype == "f32")]
    return dict(rotary_dim=int(rng.choice(dims)), eps=float(rng.choice([1e-6, 1e-5])),
                theta=float(rng.choice([1e4, 5e5, 1e6])))


@pytest.mark.parametrize("seed", range(12))
def test_random_insert_prefill(seed, gpu_device):
    """The new-token step (QK-norm, partial RoPE, K / V / indexer-key insert) on random
    geometries, chunks and rotary settings, on bf16, fp32 and FP8 caches."""
    import torch
    import block_sparse_long_11_amd as msa
    from oracle import msa_oracle as O
    import test_gpu_insert as I

    w, fmt, permute = draw_case(200 + seed, False)
    rope = draw_rope(seed, w)
    where = f"insert seed {seed}: {describe(w, fmt, permute)} rope={rope}"
    T.say(where)
    inp, geom, cache = T.setup(w, gpu_device, permute=permute)
    new = synth.make_new_tokens(w, gpu_device)
    fp8 = fmt == "fp8"
    before = F.fp8_host(cache) if fp8 else I.cache_host(cache)
    bt = inp["block_table"].cpu().numpy()
    units = O.prefill_units(w.seq_lens, w.q_lens)
    batch = msa.make_batch(w.seq_lens, w.q_lens, gpu_device)
    q_out = torch.full_like(new["q"], float("nan"))
    I.run_insert(geom, cache, batch, new, rope, q_out)
    if fp8:
        F.compare_fp8_insert(w, units, bt, before, F.fp8_host(cache), T.host(q_out), new, rope,
                             where)
    else:
        ref = I.oracle_insert(units, new, before, bt, rope)
        I.compare_insert(w, units, bt, before, I.cache_host(cache), T.host(q_out), ref, where)
