"""Seeded synthetic inputs for the MSA path: queries, indexer queries, the
block-major K/V/indexer-key caches, block tables and sequence lengths.

This module draws random numbers and lays them out. It holds none of the
method's arithmetic (no scoring, no selection, no attention), so both the HIP
path and the CPU oracle can be fed from it.

Workloads (shapes of the long-context prefill and decode settings the MSA pages
describe: 128-token KV blocks, 64 query heads over 4 KV heads, up to 1M tokens
of context):

  tiny_prefill_fp32   fp32, 1 x 2048 tokens, 4 q / 1 kv heads, D 64, indexer
                      1 x 32, top-k 4, 2 planted blocks per group
  prefill_32k         bf16, 1 x 32768 tokens, 64/4 heads, D 128, indexer 8 x 64,
                      top-k 16, 8 planted blocks per 32-block span
  decode_128k_b64     bf16, 64 sequences x 131072 cached tokens, 1 query each,
                      top-k 33 (32 + diagonal), 32 planted blocks per sequence
  decode_1m_b8        bf16, 8 sequences x 1048576 cached tokens, top-k 64,
                      63 planted blocks per sequence
  chunked_prefill     bf16, 4 requests, each an 8192-token chunk after cached
                      prefixes of 1M / 512k / 128k / 32k tokens, top-k 64,
                      8 planted blocks per 32-block span
  decode_1m_b8_fp8,   the 1M decode and the 32k prefill on FP8 caches (E4M3
  prefill_32k_fp8     codes, a power-of-two scale per 32 channels of a row)
  decode_ragged_b64   bf16, 64 sequences of mixed context (1 x 1M, 3 x 256k,
                      12 x 64k, 48 x 4k tokens), top-k 32: a ragged decode batch
  decode_1m_b8_t4     the 1M decode with 4 new tokens per sequence, each
                      selecting its own blocks (speculative verification)
  prefill_32k_tokens  the 32k prefill with per-query-token selection: every new
                      token selects its own 16 blocks

Planting ("relevant blocks"): for every (sequence, selection group g) a seeded
unit direction u_h is drawn per indexer head h of the group; a * u_h is added to
that head's indexer query of every query token of the sequence and to that head's
indexer key of every token of each planted block. The mean lift of a planted
pair's group score is then H_s * a^2; a is chosen so that this equals twice the
standard deviation sqrt(H_s * D_i) of an unplanted pair score. Values are drawn
N(0,1) in fp32, planted, then rounded once to the storage dtype.
"""

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

BLOCK = 128

# stream ids of the seeded draws
_T_Q, _T_K, _T_V, _T_QIDX, _T_KIDX, _T_PLANT_POS, _T_PLANT_DIR, _T_PERM = range(8)
_T_NEW_Q, _T_NEW_K, _T_NEW_V, _T_NEW_KIDX, _T_NORM_W, _T_ROW_SCALE = range(8, 14)
_T_SCALE_K, _T_SCALE_V, _T_SCALE_KIDX = range(14, 17)
SCALE_BLOCK = 32

# Rotary settings of the new-token step: rotary_dim 64 of head_dim 128 (partial
# rotary factor 0.5); eps and theta are not given by the pages, these are the
# usual RMSNorm epsilon and the original rotary base.
ROPE = dict(rotary_dim=64, eps=1e-6, theta=10000.0)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16"
    seq_lens: List[int]             # cached tokens per request, new ones included
    q_lens: Optional[List[int]]     # new query tokens per request; None = decode
    num_q_heads: int = 64
    num_kv_heads: int = 4
    head_dim: int = 128
    num_idx_heads: int = 8
    idx_head_dim: int = 64
    num_sel_groups: int = 4
    topk: int = 16
    plant_count: int = 8            # planted blocks per span per (seq, group)
    plant_span: Optional[int] = 32  # span in blocks; None = whole context
    seed: int = 0
    cache_format: str = "plain"     # "plain" or "fp8" (E4M3 codes + power-of-two scales)
    tokens_per_seq: int = 1         # decode: new tokens per sequence, each selecting its own
    per_token: bool = False         # prefill: every new token selects its own blocks

    @property
    def is_decode(self):
        return self.q_lens is None

    @property
    def num_seqs(self):
        return len(self.seq_lens)

    def blocks(self, r):
        return (self.seq_lens[r] + BLOCK - 1) // BLOCK

    @property
    def max_blocks(self):
        return max(self.blocks(r) for r in range(self.num_seqs))

    @property
    def num_phys_blocks(self):
        return sum(self.blocks(r) for r in range(self.num_seqs))

    @property
    def total_q(self):
        return self.num_seqs * self.tokens_per_seq if self.is_decode else sum(self.q_lens)

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_prefill_fp32": Workload(
        "tiny_prefill_fp32", "f32", [2048], [2048], num_q_heads=4, num_kv_heads=1,
        head_dim=64, num_idx_heads=1, idx_head_dim=32, num_sel_groups=1, topk=4,
        plant_count=2, plant_span=None, seed=1001),
    "prefill_32k": Workload(
        "prefill_32k", "bf16", [32768], [32768], topk=16, plant_count=8,
        plant_span=32, seed=1002),
    "decode_128k_b64": Workload(
        "decode_128k_b64", "bf16", [131072] * 64, None, topk=33, plant_count=32,
        plant_span=None, seed=1003),
    "decode_1m_b8": Workload(
        "decode_1m_b8", "bf16", [1048576] * 8, None, topk=64, plant_count=63,
        plant_span=None, seed=1004),
    "chunked_prefill": Workload(
        "chunked_prefill", "bf16",
        [1048576 + 8192, 524288 + 8192, 131072 + 8192, 32768 + 8192], [8192] * 4,
        topk=64, plant_count=8, plant_span=32, seed=1005),
    "decode_1m_b8_fp8": Workload(
        "decode_1m_b8_fp8", "bf16", [1048576] * 8, None, topk=64, plant_count=63,
        plant_span=None, seed=1004, cache_format="fp8"),
    "prefill_32k_fp8": Workload(
        "prefill_32k_fp8", "bf16", [32768], [32768], topk=16, plant_count=8,
        plant_span=32, seed=1002, cache_format="fp8"),
    "decode_ragged_b64": Workload(
        "decode_ragged_b64", "bf16",
        [1048576] + [262144] * 3 + [65536] * 12 + [4096] * 48, None, topk=32,
        plant_count=31, plant_span=None, seed=1006),
    "decode_1m_b8_t4": Workload(
        "decode_1m_b8_t4", "bf16", [1048576] * 8, None, topk=64, plant_count=63,
        plant_span=None, seed=1004, tokens_per_seq=4),
    # one selection group: the 8 indexer heads summed into one score that selects the
    # blocks of every KV head (the same bytes as the 4-group layout)
    "prefill_32k_sel1": Workload(
        "prefill_32k_sel1", "bf16", [32768], [32768], num_sel_groups=1, topk=16,
        plant_count=8, plant_span=32, seed=1002),
    "prefill_32k_fp8_sel1": Workload(
        "prefill_32k_fp8_sel1", "bf16", [32768], [32768], num_sel_groups=1, topk=16,
        plant_count=8, plant_span=32, seed=1002, cache_format="fp8"),
    # per-query-token selection in prefill: every one of the 32768 new tokens scores,
    # selects and attends its own 16 blocks
    "prefill_32k_tokens": Workload(
        "prefill_32k_tokens", "bf16", [32768], [32768], topk=16, plant_count=8,
        plant_span=32, seed=1002, per_token=True),
    "decode_1m_b8_sel1": Workload(
        "decode_1m_b8_sel1", "bf16", [1048576] * 8, None, num_sel_groups=1, topk=64,
        plant_count=63, plant_span=None, seed=1004),
}


def plant_amplitude(w: Workload) -> float:
    """a with H_s * a^2 = 2 * sqrt(H_s * D_i)."""
    hs = w.num_idx_heads // w.num_sel_groups
    return math.sqrt(2.0 * math.sqrt(w.idx_head_dim / hs))


def _np_rng(w, *stream):
    return np.random.default_rng([w.seed, *stream])


def planted_blocks(w: Workload, r: int, g: int) -> np.ndarray:
    """Logical ids of the planted blocks of (sequence r, group g), sorted.

    Blocks are drawn uniformly without replacement within each span of
    plant_span blocks (or over the whole context). In decode the last block,
    which holds the query, is never a candidate and is not planted."""
    nb = w.blocks(r)
    limit = nb - 1 if w.is_decode else nb
    if limit <= 0:                       # one block, the query's own: nothing to plant
        return np.zeros(0, dtype=np.int64)
    rng = _np_rng(w, _T_PLANT_POS, r, g)
    span = w.plant_span or limit
    out = []
    for s0 in range(0, limit, span):
        n = min(span, limit - s0)
        c = min(w.plant_count, n)
        out.extend((s0 + rng.choice(n, size=c, replace=False)).tolist())
    return np.array(sorted(out), dtype=np.int64)


def plant_directions(w: Workload, r: int, g: int) -> np.ndarray:
    """Unit directions [H_s][D_i] (float32) of (sequence r, group g)."""
    hs = w.num_idx_heads // w.num_sel_groups
    d = _np_rng(w, _T_PLANT_DIR, r, g).standard_normal((hs, w.idx_head_dim))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    return d.astype(np.float32)


def physical_permutation(w: Workload, permute=False) -> np.ndarray:
    """perm[i] = physical block holding the i-th block of the packed order
    (request 0's blocks, then request 1's, ...). Identity unless permute."""
    P = w.num_phys_blocks
    return _np_rng(w, _T_PERM).permutation(P) if permute else np.arange(P)


def block_table(w: Workload, permute=False) -> np.ndarray:
    """int32 [B][max_blocks]: request r's logical block b -> physical block.

    The packed order lays the requests' blocks one after another; permute=True
    scatters them with a seeded permutation of the physical blocks (the logical
    content is the same either way). Entries past a request's last block point at
    physical block 0 and are never read."""
    perm = physical_permutation(w, permute)
    bt = np.zeros((w.num_seqs, w.max_blocks), dtype=np.int32)
    base = 0
    for r in range(w.num_seqs):
        nb = w.blocks(r)
        bt[r, :nb] = perm[base:base + nb]
        base += nb
    return bt


def _torch_dtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _randn(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _gen(w, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed) * 1000 + stream)
    return g


def make_inputs(w: Workload, device="cpu", permute=False, chunk_blocks=2048):
    """All inputs of a workload as torch tensors on `device`.

    Returns a dict with q [T][H_q][D], q_idx [T][H_i][D_i], k_cache
    [P][H_kv][128][D], v_cache [P][H_kv][D][128] (each block's values stored
    d-major), k_idx_cache [P][H_i][128][D_i] (all in the workload dtype),
    block_table int32 [B][max_blocks], seq_lens int32 [B], q_lens int32 [B]
    (decode: tokens_per_seq each) and cu_q_lens int32 [B+1]. The caches are drawn chunk by chunk
    of physical blocks so that only one fp32 chunk is alive at a time.

    With w.cache_format == "fp8" the caches are uint8 E4M3 codes and the dict also
    holds k_scale [P][H_kv][128][D/32], v_scale [P][H_kv][D/32][128] and
    k_idx_scale [P][H_i][128][D_i/32] (bytes e + 127): each 32-channel block of a
    token row gets a seeded exponent e from {-7, -6, -5} (the range the writer's
    rule gives N(0,1) rows), and its codes are torch's float8_e4m3fn cast of the
    drawn values times 2^-e, clamped to +-448 (beyond 3.5 sigma at e = -7)."""
    dt = _torch_dtype(w)
    B, P = w.num_seqs, w.num_phys_blocks
    T = w.total_q
    H_q, H_kv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    H_i, D_i, n_sel = w.num_idx_heads, w.idx_head_dim, w.num_sel_groups
    hs = H_i // n_sel
    a = plant_amplitude(w)
    bt = block_table(w, permute)
    perm = physical_permutation(w, permute)
    q_lens = [w.tokens_per_seq] * B if w.is_decode else list(w.q_lens)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)

    # packed block index of (request, logical block): base[r] + b
    base = np.concatenate([[0], np.cumsum([w.blocks(r) for r in range(B)])]).astype(np.int64)
    plants = {}            # (r, g) -> (planted logical ids, directions)
    for r in range(B):
        for g in range(n_sel):
            plants[(r, g)] = (planted_blocks(w, r, g), plant_directions(w, r, g))

    out = {}
    out["q"] = _randn(_gen(w, _T_Q, device), (T, H_q, D), device).to(dt)

    qi = _randn(_gen(w, _T_QIDX, device), (T, H_i, D_i), device)
    for r in range(B):
        for g in range(n_sel):
            u = torch.from_numpy(plants[(r, g)][1]).to(device)
            qi[cu[r]:cu[r + 1], g * hs:(g + 1) * hs, :] += a * u
    out["q_idx"] = qi.to(dt)

    fp8 = w.cache_format == "fp8"

    def cache(stream, heads, dim, plant, d_major=False, scale_stream=None):
        # drawn in packed order, chunk by chunk, then scattered to physical blocks;
        # d_major stores each block's [128][dim] rows transposed as [dim][128]
        gen = _gen(w, stream, device)
        shape = (P, heads, dim, BLOCK) if d_major else (P, heads, BLOCK, dim)
        res = torch.empty(shape, dtype=torch.uint8 if fp8 else dt, device=device)
        if fp8:
            sgen = _gen(w, scale_stream, device)
            nb = dim // SCALE_BLOCK
            sshape = (P, heads, nb, BLOCK) if d_major else (P, heads, BLOCK, nb)
            scales = torch.empty(sshape, dtype=torch.uint8, device=device)
        for c0 in range(0, P, chunk_blocks):
            c1 = min(P, c0 + chunk_blocks)
            x = _randn(gen, (c1 - c0, heads, BLOCK, dim), device)
            if plant:
                for (r, g), (ids, u) in plants.items():
                    packed = base[r] + ids
                    sel = packed[(packed >= c0) & (packed < c1)] - c0
                    if len(sel):
                        idx = torch.from_numpy(sel).to(device)
                        ut = torch.from_numpy(u).to(device)[None, :, None, :]
                        x[idx, g * hs:(g + 1) * hs] += a * ut
            dst = torch.from_numpy(perm[c0:c1]).to(device)
            if fp8:
                # exponents of the range a writer picks for N(0,1) rows (the smallest
                # e with max|x| / 2^e <= 448 over 32 channels is about -7)
                e = torch.randint(-7, -4, (c1 - c0, heads, BLOCK, dim // SCALE_BLOCK),
                                  generator=sgen, device=device, dtype=torch.int32)
                y = x * torch.exp2(-e.float()).repeat_interleave(SCALE_BLOCK, dim=3)
                codes = y.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
                sc = (e + 127).to(torch.uint8)
                res[dst] = codes.transpose(2, 3).contiguous() if d_major else codes
                scales[dst] = sc.transpose(2, 3).contiguous() if d_major else sc
                del y, codes, e
            else:
                res[dst] = (x.transpose(2, 3) if d_major else x).to(dt)
            del x
        return (res, scales) if fp8 else res

    if fp8:
        out["k_cache"], out["k_scale"] = cache(_T_K, H_kv, D, False, scale_stream=_T_SCALE_K)
        out["v_cache"], out["v_scale"] = cache(_T_V, H_kv, D, False, d_major=True,
                                               scale_stream=_T_SCALE_V)
        out["k_idx_cache"], out["k_idx_scale"] = cache(_T_KIDX, H_i, D_i, True,
                                                       scale_stream=_T_SCALE_KIDX)
    else:
        out["k_cache"] = cache(_T_K, H_kv, D, False)
        out["v_cache"] = cache(_T_V, H_kv, D, False, d_major=True)
        out["k_idx_cache"] = cache(_T_KIDX, H_i, D_i, True)
    out["block_table"] = torch.from_numpy(bt).to(device)
    out["seq_lens"] = torch.tensor(w.seq_lens, dtype=torch.int32, device=device)
    out["q_lens"] = torch.tensor(q_lens, dtype=torch.int32, device=device)
    out["cu_q_lens"] = torch.from_numpy(cu).to(device)
    return out


def make_new_tokens(w: Workload, device="cpu", rows=None):
    """Raw inputs of the new tokens before QK-norm and RoPE, as torch tensors in
    the workload dtype: q [T][H_q][D], k and v [T][H_kv][D], k_idx [T][H_i][D_i]
    (T = rows, default the workload's new-token count) and the norm weights
    q_norm_w, k_norm_w [D].

    Entries are N(0,1); every (token, head) row of q and k is multiplied by
    exp(N(0, 1/2)) so that rows reach the norm with varied magnitudes. The
    weights are 1 + N(0, 1/5^2)."""
    dt = _torch_dtype(w)
    T = w.total_q if rows is None else rows
    H_q, H_kv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    sc = _gen(w, _T_ROW_SCALE, device)

    def scaled(stream, heads):
        x = _randn(_gen(w, stream, device), (T, heads, D), device)
        return (x * torch.exp(0.5 * _randn(sc, (T, heads, 1), device))).to(dt)

    wg = _gen(w, _T_NORM_W, device)
    return dict(
        q=scaled(_T_NEW_Q, H_q), k=scaled(_T_NEW_K, H_kv),
        v=_randn(_gen(w, _T_NEW_V, device), (T, H_kv, D), device).to(dt),
        k_idx=_randn(_gen(w, _T_NEW_KIDX, device), (T, w.num_idx_heads, w.idx_head_dim),
                     device).to(dt),
        q_norm_w=(1.0 + 0.2 * _randn(wg, (D,), device)).to(dt),
        k_norm_w=(1.0 + 0.2 * _randn(wg, (D,), device)).to(dt))


def v_token_major(v_cache: torch.Tensor) -> torch.Tensor:
    """View of a d-major V cache [P][H][D][128] as [P][H][128][D]."""
    return v_cache.transpose(2, 3)


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 NumPy copy of a float32/bf16 tensor (for the CPU side)."""
    return t.detach().to("cpu", torch.float32).numpy()


def small_workload(dtype="bf16", seq_lens=(700,), q_lens=(300,), **kw) -> Workload:
    """A small case for parity tests: defaults to a 4 q / 2 kv head layout."""
    base = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, num_idx_heads=4,
                idx_head_dim=64, num_sel_groups=2, topk=3, plant_count=2,
                plant_span=8, seed=7)
    base.update(kw)
    return Workload("small", dtype, list(seq_lens),
                    None if q_lens is None else list(q_lens), **base)
