"""Benchmark of the MSA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM: indexer scores -> block top-k -> sparse attention
(prefill), or indexer -> top-k -> split-KV decode attention -> combine (decode).
Default workload: the 32k-token prefill (64 q / 4 kv heads, D 128, indexer 8 x 64,
top-k 16); the 1M-context decode (8 x 1,048,576 tokens, top-k 64) is measured in
the same run as a second line item.

Prints ONE JSON line. `value` is selected-KV tokens per second: the sum over
(query token, KV head) of the selected keys that query can see, per second.
`roofline` is for the step's dominant kernel, with its average launch duration
measured by HIP events recorded on the launch stream around every launch in the
timed region. `cpu_baseline` times the CPU oracle on a bounded sample of units.
`qk_norm_rope_insert` times the step that precedes the path (QK-norm, partial
RoPE and the insert of the new tokens' K, V and indexer keys) on each workload's
new tokens, per launch, against the HBM peak; it is not part of the step.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_long_11_amd as msa            # noqa: E402
from block_sparse_long_11_amd import synth         # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CSRC = os.path.join(ROOT, "block_sparse_long_11_amd", "csrc")
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
BLK = 128


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# measured peaks: the probes of libmsa_probe.so (include/msa_probe.h)
# ----------------------------------------------------------------------------

def measured_peaks(dev):
    """Practical ceilings on this GPU: a streaming read of 4 GiB with 16-byte
    non-temporal loads and a device copy of 1 GiB (each the best of several grid
    sizes), dense bf16 MFMA loops on register operands and MFMA next to VALU work on
    one SIMD. Timed with HIP events on the launch stream."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_long_11_amd", "libmsa_probe.so"))
    lib.msa_probe_stream_read.restype = ctypes.c_int
    lib.msa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p]
    for name in ("msa_probe_mfma_bf16", "msa_probe_mfma_bf16_random"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.msa_probe_copy.restype = ctypes.c_int
    lib.msa_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.msa_probe_mfma_valu.restype = ctypes.c_int
    lib.msa_probe_mfma_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(65536 * 4, dtype=torch.float32, device=dev)

    def timed(launch, reps):
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = launch()
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            best = min(best, a.elapsed_time(b) * 1e-3)
        return best

    hbm = {}
    for groups in (2048, 4096, 8192, 16384):
        t = timed(lambda: lib.msa_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                     groups, ctypes.c_void_p(sink.data_ptr()),
                                                     stream), 4)
        hbm[groups] = nbytes / t / 1e9
    # a plain copy of 1 GiB between the buffer's first and third quarter
    cbytes = 1 << 30
    copy = {}
    for groups in (2048, 4096, 8192):
        t = timed(lambda: lib.msa_probe_copy(ctypes.c_void_p(buf.data_ptr()),
                                             ctypes.c_void_p(buf.data_ptr() + 2 * cbytes),
                                             cbytes, groups, stream), 3)
        copy[groups] = 2 * cbytes / t / 1e9
    del buf
    groups, iters = 1024, 20000
    flops = groups * 4 * iters * 8 * 32768
    timed(lambda: lib.msa_probe_mfma_bf16(groups, 2000, ctypes.c_void_p(sink.data_ptr()),
                                          stream), 1)      # clock ramp
    t = timed(lambda: lib.msa_probe_mfma_bf16(groups, iters, ctypes.c_void_p(sink.data_ptr()),
                                              stream), 3)
    t_rand = timed(lambda: lib.msa_probe_mfma_bf16_random(
        groups, iters, ctypes.c_void_p(sink.data_ptr()), stream), 3)
    # MFMA and softmax-like fp32 VALU work of two waves on one SIMD: alone and together
    co_groups, co_iters = 1024, 2000
    co = {mode: timed(lambda: lib.msa_probe_mfma_valu(co_groups, co_iters, mode,
                                                      ctypes.c_void_p(sink.data_ptr()), stream),
                      3) * 1e3 for mode in (1, 2, 3)}
    hidden = (co[1] + co[2] - co[3]) / min(co[1], co[2])
    best_g = max(hbm, key=hbm.get)
    best_c = max(copy, key=copy.get)
    return dict(hbm_gbs=hbm[best_g], copy_gbs=copy[best_c], mfma_bf16_tflops=flops / t / 1e12,
                mfma_bf16_random_tflops=flops / t_rand / 1e12,
                mfma_valu_coexec=dict(mfma_ms=co[1], valu_ms=co[2], both_ms=co[3],
                                      hidden_frac_of_smaller=hidden,
                                      probe="one work-group of 8 waves per CU; waves 0-3: "
                                            f"{co_iters} rounds of 16 random-operand MFMAs, "
                                            "waves 4-7: as many rounds of a softmax tile's "
                                            "fp32 work (max3 tree, 16 x fma+exp2+add, 8 packs)"),
                hbm_probe=f"streaming read of 4 GiB, 16-byte non-temporal loads, 8 in flight "
                          f"per thread, best of {sorted(hbm)} work-groups (best {best_g})",
                copy_probe=f"device copy of 1 GiB (read + write bytes counted), 16-byte loads and "
                           f"stores, 8 in flight per thread, best of {sorted(copy)} work-groups "
                           f"(best {best_c})",
                mfma_probe="v_mfma_f32_32x32x16_bf16, 8 independent chains per wave, "
                           f"{groups} work-groups of 4 waves, register operands (small "
                           "constants; the random-operand figure uses full-mantissa values "
                           "uniform in (-1.7, 1.7))")


def geometry(w):
    return msa.Geometry(w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_idx_heads,
                        w.idx_head_dim, w.num_sel_groups, w.dtype, w.cache_format)


def cache_row_bytes(w, dim):
    """Bytes of one token's head row in a cache: bf16, or FP8 codes plus one
    scale byte per 32 channels."""
    if w.cache_format == "fp8":
        return dim + dim // 32
    return dim * (2 if w.dtype == "bf16" else 4)


# ----------------------------------------------------------------------------
# work accounting
# ----------------------------------------------------------------------------

def selected_kv_tokens(w, ids, units):
    """Sum over (query token, KV head) of visible selected keys."""
    total = 0
    nsel = w.num_sel_groups
    for u, un in enumerate(units):
        tau, n = un["tau"], un["num_rows"]
        for j in range(w.num_kv_heads):
            g = j if nsel == w.num_kv_heads else 0
            kept = ids[u, g]
            full = int(np.sum((kept >= 0) & (kept < tau))) * BLK
            # diagonal: query at pos0 + t sees pos0 + t - 128 tau + 1 keys of it
            first = un["pos0"] - tau * BLK + 1
            diag = n * first + n * (n - 1) // 2
            total += n * full + diag
    return total


def selected_kv_tokens_rows(w, ids):
    """Per-token prefill: sum over (new token, KV head) of the visible keys of that
    token's own kept blocks (ids [total_q][n_sel][topk])."""
    pos = np.concatenate([np.arange(L - n, L) for L, n in zip(w.seq_lens, w.q_lens)])
    tau = pos // BLK
    total = 0
    for j in range(w.num_kv_heads):
        g = j if w.num_sel_groups == w.num_kv_heads else 0
        kept = ids[:, g, :]
        full = ((kept >= 0) & (kept < tau[:, None])).sum(axis=1) * BLK
        total += int(full.sum() + (pos - tau * BLK + 1).sum())
    return total


def plan_units(w):
    if w.is_decode:   # one unit per new token (T = tokens_per_seq per sequence)
        T = w.tokens_per_seq
        return [dict(r=r, tau=(L - T + i) // BLK, pos0=L - T + i, num_rows=1)
                for r, L in enumerate(w.seq_lens) for i in range(T)]
    plan = msa.msa_prefill_plan(w.seq_lens, w.q_lens)
    return [dict(r=int(p[0]), tau=int(p[1]), row0=int(p[2]), num_rows=int(p[3]),
                 pos0=int(p[4])) for p in plan]


def index_decode_bytes(w):
    """Indexer keys every non-diagonal block must stream, plus q_idx and scores."""
    per_block = w.num_idx_heads * BLK * cache_row_bytes(w, w.idx_head_dim)
    blocks = sum(w.blocks(r) - 1 for r in range(w.num_seqs))
    q = w.total_q * w.num_idx_heads * w.idx_head_dim * 2
    scores = w.total_q * w.num_sel_groups * w.max_blocks * 4
    return blocks * per_block + q + scores


# ----------------------------------------------------------------------------
# timed runs
# ----------------------------------------------------------------------------

class Runner:
    """Holds a workload's resident inputs and outputs and launches one step,
    recording HIP events around each launch on the current stream."""

    def __init__(self, w, dev, permute=False):
        self.w, self.dev = w, dev
        log(f"{w.name}: generating inputs on {dev}" + (" (permuted block table)" if permute else ""))
        self.inp = synth.make_inputs(w, dev, permute=permute)
        self.geom = geometry(w)
        self.cache = msa.Cache(self.inp["k_cache"], self.inp["v_cache"],
                               self.inp["k_idx_cache"], self.inp["block_table"],
                               self.inp["seq_lens"], self.inp.get("k_scale"),
                               self.inp.get("v_scale"), self.inp.get("k_idx_scale"))
        U = w.total_q if (w.is_decode or w.per_token) else \
            len(msa.msa_prefill_plan(w.seq_lens, w.q_lens))
        self.batch = None if w.is_decode else msa.make_batch(w.seq_lens, w.q_lens, dev)
        self.scores = torch.empty((U, w.num_sel_groups, self.cache.max_blocks),
                                  dtype=torch.float32, device=dev)
        self.ids = torch.empty((U, w.num_sel_groups, w.topk), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.inp["q"])
        self.lse = torch.empty(self.inp["q"].shape[:2], dtype=torch.float32, device=dev)
        if w.is_decode:
            self.ws = msa.workspace(msa.msa_decode_workspace_size(self.geom, w.total_q,
                                                                  w.topk, 0), dev)
        elif w.per_token:
            self.ws = msa.workspace(msa.msa_prefill_tokens_workspace_size(
                self.geom, self.batch.total_units, w.total_q, w.topk), dev)
        # FP8 prefill: the staged attention (kept blocks converted to bf16 once each)
        self.staged = w.cache_format == "fp8" and not w.is_decode and not w.per_token
        if self.staged:
            self.ws = msa.workspace(msa.msa_prefill_workspace_size(
                self.geom, self.cache, self.batch.total_units, w.topk), dev)
        self.names = ["index_scores", "select_topk_blocks",
                      "sparse_attn_decode" if w.is_decode else "sparse_attn_prefill"]

    def step(self, events=None):
        w, i = self.w, self.inp
        ev = events or [None] * 4
        T = w.tokens_per_seq
        if ev[0] is not None:
            ev[0].record()
        if w.is_decode and T > 1:
            msa.msa_index_scores_per_token(self.geom, self.cache, T, i["q_idx"], self.scores)
        elif w.per_token:
            msa.msa_index_scores_prefill_tokens(self.geom, self.cache, self.batch, i["q_idx"],
                                                self.scores)
        else:
            msa.msa_index_scores(self.geom, self.cache, self.batch, i["q_idx"], self.scores)
        if ev[1] is not None:
            ev[1].record()
        msa.msa_select_topk_blocks(self.scores, w.topk, self.ids)
        if ev[2] is not None:
            ev[2].record()
        if w.is_decode and T > 1:
            msa.msa_sparse_attn_decode_per_token(self.geom, self.cache, T, i["q"], self.ids,
                                                 w.topk, self.out, self.ws, self.lse)
        elif w.is_decode:
            msa.msa_sparse_attn_decode(self.geom, self.cache, i["q"], self.ids, w.topk,
                                       self.out, self.ws, self.lse)
        elif w.per_token:
            msa.msa_sparse_attn_prefill_tokens(self.geom, self.cache, self.batch, i["q"],
                                               self.ids, w.topk, self.out, self.ws, self.lse)
        elif self.staged:
            msa.msa_sparse_attn_prefill_staged(self.geom, self.cache, self.batch, i["q"],
                                               self.ids, w.topk, self.out, self.ws, self.lse)
        else:
            msa.msa_sparse_attn_prefill(self.geom, self.cache, self.batch, i["q"], self.ids,
                                        w.topk, self.out, self.lse)
        if ev[3] is not None:
            ev[3].record()

    def timed(self, steps, warmup):
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for e in evs:
            self.step(e)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start.elapsed_time(stop)
        per = {n: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs]))
               for k, n in enumerate(self.names)}
        return total_ms / steps, per, wall


TRAFFIC_SOURCE = ("committed rocprofv3 counter profile (profiles/pmc_traffic.json: FETCH_SIZE and "
                  "WRITE_SIZE per launch, scaled by a plain-copy calibration), used only while the "
                  "code of the kernel's source file (comments aside) is unchanged; not measured in "
                  "this run")


def source_code_hash(path):
    """sha256 of a source file's code: comments removed and whitespace runs
    collapsed, so that an edit of comments alone keeps the hash."""
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def measured_traffic(kernel_key, source_file):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a plain copy), or
    None when there is no entry or the kernel's source code changed since it was
    taken."""
    try:
        with open(PMC_SUMMARY) as f:
            summ = json.load(f)
        e = summ["kernels"][kernel_key]
        if source_code_hash(os.path.join(CSRC, source_file)) != e["source_code_sha256"]:
            return None
        return e["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def attn_prefill_traffic(workload, staged):
    """Prefill attention's HBM bytes per call; the staged call adds its slot marking
    and block conversion launches to the attention's."""
    keys = ["attn_prefill"] + (["stage_mark", "stage_convert"] if staged else [])
    parts = [measured_traffic(f"{workload}:{k}", "attn_prefill.hip") for k in keys]
    return None if any(v is None for v in parts) else sum(parts)


def graph_ms_per_step(runner, steps, warmup):
    """The same step captured once in a HIP graph and replayed: the time per
    replay, without the launch gaps between the step's kernels."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        runner.step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner.step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def cold_ms_per_step(runner, steps, flush_bytes=1 << 30):
    """The step timed with cold caches: before every step a 1 GiB buffer (four
    times the 256 MB Infinity Cache, far more than the L2s) is written and then
    read, so the step's inputs come from HBM and the caches hold clean lines (the
    read writes the flush's dirty lines back before the step starts; after a
    write alone the step would also pay for that write-back). Only the step is
    inside the events."""
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device=runner.dev)
    sink = torch.empty(1, dtype=torch.float32, device=runner.dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        scratch.fill_(float(i))
        torch.amax(scratch, dim=0, keepdim=True, out=sink)
        a.record()
        runner.step()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    del scratch
    return ms


def measure(w, dev, steps, warmup, permute=False):
    r = Runner(w, dev, permute)
    ms, per, wall = r.timed(steps, warmup)
    units = plan_units(w)
    ids = r.ids.cpu().numpy()
    tokens = selected_kv_tokens_rows(w, ids) if w.per_token else \
        selected_kv_tokens(w, ids, units)
    G = w.num_q_heads // w.num_kv_heads
    res = dict(workload=w.name, ms_per_step=ms, kernel_ms=per, wall_s=wall,
               selected_kv_tokens_per_step=tokens, value=tokens / (ms * 1e-3),
               graph_ms_per_step=graph_ms_per_step(r, steps, warmup),
               cold_ms_per_step=cold_ms_per_step(r, steps))
    if w.is_decode:
        nbytes = index_decode_bytes(w)
        t = per["index_scores"] * 1e-3
        res["roofline"] = dict(kernel="index_scores (decode)", bound="hbm",
                               achieved=nbytes / t / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                               frac=nbytes / t / 1e9 / HBM_PEAK_GBS,
                               traffic=measured_traffic(f"{w.name}:index_decode",
                                                        "index_scores.hip"),
                               traffic_source=TRAFFIC_SOURCE, algorithmic_bytes=nbytes)
        # whole decode step against HBM: the algorithmic bytes of all four launches
        kv = tokens * cache_row_bytes(w, w.head_dim) * 2   # K and V rows of the selected keys
        step_bytes = nbytes + kv + 2 * w.total_q * w.num_q_heads * w.head_dim * 2
        res["step_hbm_frac"] = step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
        res["step_algorithmic_bytes"] = step_bytes
    else:
        flops = 4.0 * w.head_dim * G * tokens       # QK^T and PV over the visible pairs
        t = per["sparse_attn_prefill"] * 1e-3
        kname = "sparse_attn_prefill"
        if r.staged:
            kname += "_staged (kept FP8 blocks converted to bf16 once each, then attended)"
        res["roofline"] = dict(kernel=kname, bound="mfma",
                               achieved=flops / t / 1e12, peak=MFMA_BF16_PEAK_TFLOPS,
                               unit="TFLOP/s", frac=flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                               traffic=attn_prefill_traffic(w.name, r.staged),
                               traffic_source=TRAFFIC_SOURCE, algorithmic_flops=flops)
    res["_runner"] = r
    return res


def insert_bytes(w):
    """Algorithmic HBM bytes of one msa_qk_norm_rope_insert launch over all new
    tokens: q, k, v and k_idx read once; q_out, the K and V cache rows and the
    indexer-key rows written once (the norm weights and the plan are negligible)."""
    sz = 2 if w.dtype == "bf16" else 4
    T = w.total_q
    read = T * (w.num_q_heads * w.head_dim + 2 * w.num_kv_heads * w.head_dim
                + w.num_idx_heads * w.idx_head_dim) * sz
    written = T * (w.num_q_heads * w.head_dim * sz + 2 * w.num_kv_heads *
                   cache_row_bytes(w, w.head_dim) +
                   w.num_idx_heads * cache_row_bytes(w, w.idx_head_dim))
    return read + written


def measure_insert(runner, launches=20, warmup=10):
    """Times msa_qk_norm_rope_insert on the workload's new tokens (partial RoPE over
    64 of 128 channels): HIP events on the launch stream around every launch."""
    w, dev = runner.w, runner.dev
    new = synth.make_new_tokens(w, dev)
    rope = synth.ROPE

    batch = runner.batch
    if w.is_decode and w.tokens_per_seq > 1:   # several tokens per sequence: a planned batch
        batch = msa.make_batch(w.seq_lens, [w.tokens_per_seq] * w.num_seqs, dev)

    def launch():
        msa.msa_qk_norm_rope_insert(runner.geom, runner.cache, batch, new["q"], new["k"],
                                    new["v"], new["k_idx"], new["q_norm_w"], new["k_norm_w"],
                                    rope["eps"], rope["theta"], rope["rotary_dim"], runner.out)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = insert_bytes(w)
    gbs = nbytes / (us * 1e-6) / 1e9
    del new
    return dict(workload=w.name, new_tokens=w.total_q, rotary_dim=rope["rotary_dim"],
                us_per_launch=us, bound="hbm", algorithmic_bytes=nbytes, achieved=gbs,
                unit="GB/s", peak=HBM_PEAK_GBS, frac=gbs / HBM_PEAK_GBS,
                traffic=measured_traffic(f"{w.name}:insert", "qk_insert.hip"))


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of units
# ----------------------------------------------------------------------------

def _mini(cache_t, bt_row, blocks):
    """Host float32 copy of some logical blocks of one request and the block
    table that maps those logical ids to rows of the copy."""
    idx = torch.as_tensor(np.asarray(bt_row)[blocks].astype(np.int64), device=cache_t.device)
    mini = synth.to_host_f32(cache_t.index_select(0, idx))
    bt = np.zeros(max(blocks) + 1, dtype=np.int64)
    bt[blocks] = np.arange(len(blocks))
    return mini, bt


def blas_info():
    """BLAS library and thread count numpy's products run on."""
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return dict(blas=f"{info[0].get('internal_api')} {info[0].get('version')}",
                        blas_threads=info[0].get("num_threads"))
    except Exception:   # threadpoolctl missing or failing: report what numpy says
        pass
    return dict(blas="unknown", blas_threads=None)


def cpu_baseline(w, runner, budget_s=15.0, max_units=None):
    """The oracle as it stands, timed on this host's cores over a seeded sample of
    units (the copies of each unit's inputs to the host are not timed)."""
    from oracle import msa_oracle as O
    units = plan_units(w)
    order = np.random.default_rng(0).permutation(len(units))
    inp = runner.inp
    bt = inp["block_table"].cpu().numpy()
    cores = len(os.sched_getaffinity(0))
    done, tokens, t_used = 0, 0, 0.0
    for u in order:
        if max_units is not None and done >= max_units:
            break
        un = units[u]
        r, tau = un["r"], un["tau"]
        rows = slice(r, r + 1) if w.is_decode else slice(un["row0"], un["row0"] + un["num_rows"])
        q, qi = synth.to_host_f32(inp["q"][rows]), synth.to_host_f32(inp["q_idx"][rows])
        ki, bti = _mini(inp["k_idx_cache"], bt[r], list(range(max(tau, 1))))
        t0 = time.perf_counter()
        S = O.unit_block_scores(qi, ki, bti, tau, w.num_sel_groups, bt.shape[1])
        ids = np.array([O.select_blocks(S[g], tau, w.topk)
                        for g in range(w.num_sel_groups)], dtype=np.int32)
        t_used += time.perf_counter() - t0
        kept = sorted({int(b) for b in ids.reshape(-1) if b >= 0})
        kc, btk = _mini(inp["k_cache"], bt[r], kept)
        vc, _ = _mini(synth.v_token_major(inp["v_cache"]), bt[r], kept)
        t0 = time.perf_counter()
        O.unit_attention(q, un["pos0"], ids, kc, vc, btk, int(w.seq_lens[r]), w.num_sel_groups)
        t_used += time.perf_counter() - t0
        tokens += selected_kv_tokens(w, ids[None], [un])
        done += 1
        if t_used > budget_s:
            break
    rate = tokens / t_used
    return dict(value=rate, unit="selected-KV tokens/s", cores=cores, kind="oracle",
                sample=f"{done} of {len(units)} units of {w.name} (seeded order), whole oracle "
                       f"path per unit (scores, top-k, attention) in float64, {t_used:.1f} s "
                       f"of oracle time",
                extrapolated_step_s=t_used * len(units) / done,
                extrapolation="sampled units' oracle time scaled by units per step "
                              "(units are independent)",
                **blas_info())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="prefill_32k", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--second", default="decode_1m_b8",
                    help="second workload measured in the same run ('none' to skip)")
    ap.add_argument("--extra", default="decode_1m_b8_fp8,prefill_32k_fp8,decode_1m_b8_t4,"
                                      "decode_ragged_b64,chunked_prefill,decode_128k_b64,"
                                      "prefill_32k_sel1,prefill_32k_fp8_sel1,decode_1m_b8_sel1,"
                                      "prefill_32k_tokens",
                    help="more workloads measured in the same run (FP8 caches, several "
                         "tokens per sequence, ragged batches, the chunked prefill, the "
                         "128k batched decode, one selection group), comma-separated "
                         "('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (streaming read, MFMA loop)")
    ap.add_argument("--permute", action="store_true",
                    help="scatter every workload's blocks over the physical cache by a seeded "
                         "permutation (the default block table is the identity)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(sequences and KV heads shard with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": src.numel() * 4,
                          "bytes_written": dst.numel() * 4}))
        return
    msa.lib()
    peaks = None
    if not args.no_probes:
        peaks = measured_peaks(dev)
        co = peaks["mfma_valu_coexec"]
        log(f"measured peaks: HBM read {peaks['hbm_gbs']:.0f} GB/s, copy "
            f"{peaks['copy_gbs']:.0f} GB/s, bf16 MFMA "
            f"{peaks['mfma_bf16_tflops']:.0f} TFLOP/s (random operands "
            f"{peaks['mfma_bf16_random_tflops']:.0f}); MFMA {co['mfma_ms']:.3f} ms, VALU "
            f"{co['valu_ms']:.3f} ms, both {co['both_ms']:.3f} ms on one SIMD")
        torch.cuda.empty_cache()

    w = synth.WORKLOADS[args.workload]
    main_res = measure(w, dev, args.steps, args.warmup, args.permute)
    log(f"{w.name}: {main_res['ms_per_step']:.3f} ms/step, kernels {main_res['kernel_ms']}")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(w, main_res["_runner"], args.cpu_budget)
    inserts = [measure_insert(main_res["_runner"])]
    log(f"{w.name}: insert {inserts[-1]['us_per_launch']:.1f} us")
    del main_res["_runner"]
    torch.cuda.empty_cache()

    second = None
    if args.second != "none" and args.second != args.workload:
        w2 = synth.WORKLOADS[args.second]
        second = measure(w2, dev, args.steps, args.warmup, args.permute)
        log(f"{w2.name}: {second['ms_per_step']:.3f} ms/step, kernels {second['kernel_ms']}")
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on a sample of the second workload")
            second["cpu_baseline"] = cpu_baseline(w2, second["_runner"], args.cpu_budget / 2,
                                                  max_units=2)
        inserts.append(measure_insert(second["_runner"]))
        log(f"{w2.name}: insert {inserts[-1]['us_per_launch']:.1f} us")
        del second["_runner"]
        torch.cuda.empty_cache()

    extra = []
    for name in ([] if args.extra == "none" else args.extra.split(",")):
        if name in (args.workload, args.second):
            continue
        w3 = synth.WORKLOADS[name]
        res = measure(w3, dev, args.steps, args.warmup, args.permute)
        log(f"{w3.name}: {res['ms_per_step']:.3f} ms/step, kernels {res['kernel_ms']}")
        inserts.append(measure_insert(res["_runner"]))
        log(f"{w3.name}: insert {inserts[-1]['us_per_launch']:.1f} us")
        del res["_runner"]
        torch.cuda.empty_cache()
        extra.append(res)

    def add_measured(res):
        rf = res["roofline"]
        if peaks is None:
            return
        mp = peaks["hbm_gbs"] if rf["bound"] == "hbm" else peaks["mfma_bf16_tflops"]
        rf["measured_peak"] = mp
        rf["frac_of_measured_peak"] = rf["achieved"] / mp
        if rf["bound"] == "mfma":
            rf["frac_of_random_operand_mfma_peak"] = \
                rf["achieved"] / peaks["mfma_bf16_random_tflops"]

    for r in [main_res] + ([second] if second else []) + extra:
        add_measured(r)
    if peaks is not None:
        # the insert writes as many bytes as it reads: a plain copy is its ceiling
        for ins in inserts:
            ins["copy_rate_gbs"] = peaks["copy_gbs"]
            ins["frac_of_copy_rate"] = ins["achieved"] / peaks["copy_gbs"]

    config = dict(workload=w.name, batch=w.num_seqs,
                  seq_lens=w.seq_lens if len(set(w.seq_lens)) > 1 else w.seq_lens[0],
                  q_per_seq=(w.q_lens[0] if w.q_lens else 1), q_heads=w.num_q_heads,
                  kv_heads=w.num_kv_heads, head_dim=w.head_dim, block=BLK, topk=w.topk,
                  indexer=f"{w.num_idx_heads}x{w.idx_head_dim}",
                  selection_groups=w.num_sel_groups)
    line = {
        "metric": "selected-KV tokens/sec",
        "value": main_res["value"],
        "unit": "selected-KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) with planted blocks), inputs resident in HBM"
                + (", block table permuted" if args.permute else ""),
        "config": config,
        "graph_ms_per_step": main_res["graph_ms_per_step"],
        "cold_ms_per_step": main_res["cold_ms_per_step"],
        "kernel_ms": main_res["kernel_ms"],
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
    }
    if second is not None:
        line["second_workload"] = {k: second[k] for k in (
            "workload", "value", "ms_per_step", "graph_ms_per_step", "cold_ms_per_step",
            "kernel_ms", "roofline", "step_hbm_frac", "cpu_baseline") if k in second}
    if extra:
        # the same workloads on FP8 caches (E4M3 codes, power-of-two scale per 32
        # channels), decode with several new tokens per sequence (each selecting its
        # own blocks), a ragged decode batch, the chunked prefill over long cached
        # prefixes, the 64-sequence 128k decode, and one selection group summing all
        # indexer heads
        line["extra_workloads"] = [{k: r[k] for k in (
            "workload", "value", "ms_per_step", "graph_ms_per_step", "cold_ms_per_step",
            "kernel_ms", "roofline", "step_hbm_frac") if k in r} for r in extra]
    # the new-token step before the path (QK-norm + partial RoPE + cache insert),
    # timed on its own: not part of the step above
    line["qk_norm_rope_insert"] = inserts
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
