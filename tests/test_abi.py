"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import block_sparse_long_11_amd as msa
from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not msa.lib_path().exists():
        pytest.fail("libmsa.so is not built (run __graft_entry__.build())")
    return msa.lib()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(msa_[a-z_]+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(msa.EXPORTS), (names, sorted(msa.EXPORTS))
    raw = ctypes.CDLL(str(msa.lib_path()))
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings_and_version(lib):
    assert lib.msa_version() >= 2
    assert lib.msa_status_string(0) == b"MSA_OK"
    assert lib.msa_status_string(3) == b"MSA_ERR_WORKSPACE_TOO_SMALL"


def _geom(**kw):
    base = dict(num_q_heads=64, num_kv_heads=4, head_dim=128, num_idx_heads=8,
                idx_head_dim=64, num_sel_groups=4, block_size=128, dtype=msa.MSA_BF16,
                cache_format=msa.MSA_CACHE_PLAIN)
    base.update(kw)
    return msa._Geom(*[base[f] for f, _ in msa._Geom._fields_])


FAKE = 0x1000    # never dereferenced: validation fails before any launch


def _cache(**kw):
    base = dict(k_cache=FAKE, v_cache=FAKE, k_idx_cache=FAKE, num_phys_blocks=10,
                block_table=FAKE, max_blocks_per_seq=4, seq_lens=FAKE, num_seqs=2,
                k_scale=FAKE, v_scale=FAKE, k_idx_scale=FAKE)
    base.update(kw)
    return msa._Cache(*[base[f] for f, _ in msa._Cache._fields_])


BAD_GEOMS = [
    (dict(num_q_heads=63), INVALID),
    (dict(num_kv_heads=0), INVALID),
    (dict(num_sel_groups=2), INVALID),
    (dict(num_idx_heads=6), INVALID),
    (dict(block_size=64), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(idx_head_dim=48), UNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=4), UNSUPPORTED),     # G = 32 on bf16
    (dict(num_idx_heads=12, num_sel_groups=4), UNSUPPORTED),  # 3 heads per group
    (dict(cache_format=2), UNSUPPORTED),
    (dict(cache_format=msa.MSA_CACHE_FP8_E4M3, dtype=msa.MSA_F32), UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_GEOMS)
def test_bad_geometry_rejected_by_every_call(lib, kw, status):
    g, c = _geom(**kw), _cache()
    st = lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), None, FAKE, FAKE, None)
    assert st == status
    assert lib.msa_last_error()
    b = msa._Batch(FAKE, 4, 100)
    st = lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                     FAKE, 16, 0.0, FAKE, None, None)
    assert st == status
    st = lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 16, 0.0, 0,
                                    FAKE, 1 << 30, FAKE, None, None)
    assert st == status
    assert lib.msa_decode_workspace_size(ctypes.byref(g), 8, 64, 0) == 0


def test_null_and_size_errors(lib):
    g = _geom()
    assert lib.msa_index_scores(None, None, None, FAKE, FAKE, None) == INVALID
    c = _cache(k_idx_cache=None)
    assert lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), None, FAKE, FAKE, None) == INVALID
    c = _cache(num_seqs=0)
    assert lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), None, FAKE, FAKE, None) == INVALID
    c = _cache()
    assert lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), None, None, FAKE, None) == INVALID
    b = msa._Batch(None, 3, 10)
    assert lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE, FAKE,
                                None) == INVALID
    assert lib.msa_select_topk_blocks(FAKE, 4, 10, 0, FAKE, None) == INVALID
    assert lib.msa_select_topk_blocks(FAKE, 4, 0, 3, FAKE, None) == INVALID
    assert lib.msa_select_topk_blocks(None, 4, 10, 3, FAKE, None) == INVALID
    assert lib.msa_select_topk_blocks(FAKE, -1, 10, 3, FAKE, None) == INVALID
    b = msa._Batch(FAKE, 3, 10)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                       FAKE, 0, 0.0, FAKE, None, None) == INVALID
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                       FAKE, 4, float("nan"), FAKE, None, None) == INVALID
    c = _cache(v_cache=None)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                       FAKE, 4, 0.0, FAKE, None, None) == INVALID


def test_decode_workspace_checks(lib):
    g, c = _geom(), _cache(num_seqs=8)
    need = lib.msa_decode_workspace_size(ctypes.byref(g), 8, 64, 0)
    auto = (512 + 31) // 32             # splits for 8 x 4 units (about 512 work-groups)
    parts = 8 * 64 * min(auto, 64)
    assert need == ((parts * 128 * 4 + 255) // 256) * 256 + ((parts * 4 + 255) // 256) * 256
    assert lib.msa_decode_workspace_size(ctypes.byref(g), 8, 64, 3) < need
    st = lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 64, 0.0, 0,
                                    FAKE, need - 1, FAKE, None, None)
    assert st == WS_SMALL
    st = lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 64, 0.0, 0,
                                    FAKE + 4, need, FAKE, None, None)
    assert st == INVALID                # misaligned workspace
    st = lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 64, 0.0, 0,
                                    None, need, FAKE, None, None)
    assert st == INVALID


@pytest.mark.parametrize("seed", range(20))
def test_prefill_plan_matches_oracle_units(lib, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    seq = rng.integers(1, 3000, size=B)
    ql = np.array([int(rng.integers(0, L + 1)) for L in seq])
    units = msa.msa_prefill_plan(seq, ql)
    ref = O.prefill_units(seq.tolist(), ql.tolist())
    assert len(units) == len(ref)
    for row, un in zip(units.tolist(), ref):
        assert row == [un["r"], un["tau"], un["row0"], un["row1"] - un["row0"], un["pos0"]]


def test_prefill_plan_rejects_bad_lengths(lib):
    with pytest.raises(msa.MsaError) as e:
        msa.msa_prefill_plan([100, 50], [101, 3])
    assert e.value.status == INVALID
    with pytest.raises(msa.MsaError):
        msa.msa_prefill_plan([0], [0])
    # query rows past an int32 row index: refused while counting, before any unit
    big = 2**31 - 1
    with pytest.raises(msa.MsaError) as e:
        msa.msa_prefill_plan([big, big], [big, 2])
    assert e.value.status == INVALID and "query rows" in str(e.value)
    with pytest.raises(ValueError, match="outside int32"):
        msa.msa_prefill_plan(np.array([2**32 + 300]), np.array([10]))


def test_binding_checks_tensors_before_calling(lib):
    geom = msa.Geometry(8, 2, 128, 4, 64, 2, "bf16")
    P = 4
    cache = msa.Cache(torch.zeros(P, 2, 128, 128, dtype=torch.bfloat16),
                      torch.zeros(P, 2, 128, 128, dtype=torch.bfloat16),
                      torch.zeros(P, 4, 128, 64, dtype=torch.float32),      # wrong dtype
                      torch.zeros(1, 4, dtype=torch.int32), torch.tensor([500], dtype=torch.int32))
    with pytest.raises(TypeError):
        msa.msa_index_scores(geom, cache, None, torch.zeros(1, 4, 64, dtype=torch.bfloat16),
                             torch.zeros(1, 2, 4))
    cache.k_idx_cache = torch.zeros(P, 4, 128, 32, dtype=torch.bfloat16)     # wrong D_i
    with pytest.raises(ValueError):
        msa.msa_index_scores(geom, cache, None, torch.zeros(1, 4, 64, dtype=torch.bfloat16),
                             torch.zeros(1, 2, 4))


def _insert(lib, g, c, b, eps=1e-6, theta=1e6, rd=64, q=FAKE, k=FAKE, v=FAKE, ki=FAKE,
            qw=FAKE, kw=FAKE, qo=FAKE):
    return lib.msa_qk_norm_rope_insert(ctypes.byref(g), ctypes.byref(c),
                                       None if b is None else ctypes.byref(b), q, k, v, ki, qw,
                                       kw, eps, theta, rd, qo, None)


def test_insert_argument_checks(lib):
    g, c, b = _geom(), _cache(), msa._Batch(FAKE, 3, 300)
    assert _insert(lib, g, c, msa._Batch(None, 0, 0)) == OK      # empty batch: nothing to do
    assert _insert(lib, g, c, b, eps=-1.0) == INVALID
    assert _insert(lib, g, c, b, eps=float("nan")) == INVALID
    assert _insert(lib, g, c, b, eps=float("inf")) == INVALID
    assert _insert(lib, g, c, b, theta=0.0) == INVALID
    assert _insert(lib, g, c, b, theta=float("nan")) == INVALID
    for rd in (8, 48, 256, -64):            # bf16 needs a power of two in [16, D]
        assert _insert(lib, g, c, b, rd=rd) == UNSUPPORTED, rd
    assert _insert(lib, _geom(dtype=msa.MSA_F32), c, b, rd=4) == UNSUPPORTED
    for kw in ("q", "k", "v", "ki", "qw", "kw", "qo"):
        assert _insert(lib, g, c, b, **{kw: None}) == INVALID, kw
    assert _insert(lib, g, _cache(k_idx_cache=None), b) == INVALID
    assert _insert(lib, g, _cache(v_cache=None), None) == INVALID
    assert _insert(lib, _geom(head_dim=96), c, b) == UNSUPPORTED
    assert lib.msa_last_error()


def test_insert_binding_checks_shapes(lib):
    geom = msa.Geometry(8, 2, 128, 4, 64, 2, "bf16")
    P, bf = 4, torch.bfloat16
    cache = msa.Cache(torch.zeros(P, 2, 128, 128, dtype=bf), torch.zeros(P, 2, 128, 128, dtype=bf),
                      torch.zeros(P, 4, 128, 64, dtype=bf), torch.zeros(1, 4, dtype=torch.int32),
                      torch.tensor([500], dtype=torch.int32))
    q = torch.zeros(1, 8, 128, dtype=bf)
    kv = torch.zeros(1, 2, 128, dtype=bf)
    ki = torch.zeros(1, 4, 64, dtype=bf)
    w = torch.ones(128, dtype=bf)
    with pytest.raises(ValueError):
        msa.msa_qk_norm_rope_insert(geom, cache, None, q, kv, kv, ki, w, torch.ones(64, dtype=bf),
                                    1e-6, 1e6, 64)
    with pytest.raises(ValueError):
        msa.msa_qk_norm_rope_insert(geom, cache, None, q, kv, torch.zeros(1, 2, 64, dtype=bf), ki,
                                    w, w, 1e-6, 1e6, 64)
    with pytest.raises(TypeError):
        msa.msa_qk_norm_rope_insert(geom, cache, None, q.float(), kv, kv, ki, w, w, 1e-6, 1e6, 64)


def test_fp8_cache_checks(lib):
    g = _geom(cache_format=msa.MSA_CACHE_FP8_E4M3)
    c = _cache()
    b = msa._Batch(FAKE, 3, 300)
    c = _cache(k_scale=None)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                       FAKE, 4, 0.0, FAKE, None, None) == INVALID
    # scale arrays are required where a call reads or writes that cache
    c = _cache(k_idx_scale=None)
    assert lib.msa_index_scores(ctypes.byref(g), ctypes.byref(c), None, FAKE, FAKE,
                                None) == INVALID
    c = _cache(v_scale=None)
    assert lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 16, 0.0, 0,
                                      FAKE, 1 << 30, FAKE, None, None) == INVALID
    for kw in ("k_scale", "v_scale", "k_idx_scale"):
        assert _insert(lib, g, _cache(**{kw: None}), b) == INVALID, kw
    # plain caches ignore the scale pointers
    g0, c0 = _geom(), _cache(k_scale=None, v_scale=None, k_idx_scale=None)
    assert _insert(lib, g0, c0, msa._Batch(None, 0, 0)) == OK


def test_per_token_checks(lib):
    g, c = _geom(), _cache()
    for T in (0, 9, -1):
        assert lib.msa_index_scores_per_token(ctypes.byref(g), ctypes.byref(c), T, FAKE, FAKE,
                                              None) == UNSUPPORTED, T
        assert lib.msa_sparse_attn_decode_per_token(ctypes.byref(g), ctypes.byref(c), T, FAKE,
                                                    FAKE, 16, 0.0, 0, FAKE, 1 << 30, FAKE, None,
                                                    None) == UNSUPPORTED, T
    assert lib.msa_index_scores_per_token(ctypes.byref(g), ctypes.byref(c), 4, None, FAKE,
                                          None) == INVALID
    need = lib.msa_decode_workspace_size(ctypes.byref(g), 2 * 4, 16, 0)
    assert lib.msa_sparse_attn_decode_per_token(ctypes.byref(g), ctypes.byref(c), 4, FAKE, FAKE,
                                                16, 0.0, 0, FAKE, need - 1, FAKE, None,
                                                None) == WS_SMALL


def test_missing_library_raises(tmp_path, monkeypatch):
    """Without the built library the binding refuses to run: there is no CPU path
    to fall back to."""
    monkeypatch.setattr(msa, "_LIB_PATH", tmp_path / "libmsa.so")
    monkeypatch.setattr(msa, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        msa.lib()
    scores = torch.zeros((1, 1, 4), dtype=torch.float32)
    ids = torch.zeros((1, 1, 2), dtype=torch.int32)
    with pytest.raises(RuntimeError, match="missing"):
        msa.msa_select_topk_blocks(scores, 2, ids)


@pytest.mark.parametrize("scale", [float("inf"), float("-inf"), float("nan")])
def test_softmax_scale_must_be_finite(lib, scale):
    """A non-finite scale is rejected by every attention call before any launch
    (<= 0 selects 1/sqrt(D); +inf would make the online softmax NaN)."""
    g, c, b = _geom(), _cache(), msa._Batch(FAKE, 3, 300)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), FAKE,
                                       FAKE, 4, scale, FAKE, None, None) == INVALID
    assert b"finite" in lib.msa_last_error()
    assert lib.msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 16, scale, 0,
                                      FAKE, 1 << 30, FAKE, None, None) == INVALID
    assert lib.msa_sparse_attn_decode_per_token(ctypes.byref(g), ctypes.byref(c), 2, FAKE, FAKE,
                                                16, scale, 0, FAKE, 1 << 30, FAKE, None,
                                                None) == INVALID
    assert lib.msa_sparse_attn_decode_static(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 16,
                                             scale, 0, FAKE, None, None) == INVALID


def test_static_decode_rejects_what_does_not_fit(lib):
    """The static-scratch decode refuses, before touching the GPU, a shape whose
    partials exceed MSA_STATIC_SCRATCH_BYTES, and checks arguments like the
    workspace form."""
    g = _geom()
    limit = msa.STATIC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert f"#define MSA_STATIC_SCRATCH_BYTES ({limit // (1 << 20)}u * 1024u * 1024u)" in text
    # 64 sequences of 64 query heads, one split each: 64 * 64 * 128 * 4 B = 2 MiB fits;
    # 8192 sequences need 256 MiB
    small = lib.msa_decode_workspace_size(ctypes.byref(g), 64, 16, 1)
    assert 0 < small <= limit
    big = lib.msa_decode_workspace_size(ctypes.byref(g), 8192, 16, 1)
    assert big > limit
    c = _cache(num_seqs=8192)
    assert lib.msa_sparse_attn_decode_static(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 16,
                                             0.0, 1, FAKE, None, None) == WS_SMALL
    assert b"static scratch" in lib.msa_last_error()
    c = _cache(num_seqs=8)
    assert lib.msa_sparse_attn_decode_static(ctypes.byref(g), ctypes.byref(c), None, FAKE, 16,
                                             0.0, 0, FAKE, None, None) == INVALID
    assert lib.msa_sparse_attn_decode_static(ctypes.byref(g), ctypes.byref(c), FAKE, FAKE, 0,
                                             0.0, 0, FAKE, None, None) == INVALID
    assert lib.msa_sparse_attn_decode_static(ctypes.byref(_geom(head_dim=96)), ctypes.byref(c),
                                             FAKE, FAKE, 16, 0.0, 0, FAKE, None,
                                             None) == UNSUPPORTED


def test_prefill_tokens_checks(lib):
    """Per-token prefill calls: argument checks before any launch, workspace size."""
    g, c, b = _geom(), _cache(), msa._Batch(FAKE, 3, 300)
    assert lib.msa_index_scores_prefill_tokens(ctypes.byref(g), ctypes.byref(c), None, FAKE,
                                               FAKE, None) == INVALID
    assert lib.msa_index_scores_prefill_tokens(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b),
                                               None, FAKE, None) == INVALID
    empty = msa._Batch(None, 0, 0)
    assert lib.msa_index_scores_prefill_tokens(ctypes.byref(g), ctypes.byref(c),
                                               ctypes.byref(empty), None, None, None) == OK
    need = lib.msa_prefill_tokens_workspace_size(ctypes.byref(g), 3, 300, 16)
    al = lambda x: (x + 255) // 256 * 256
    # union sizes per (unit, group, 32-row slab), union ids, one row-mask word per id
    assert need == al(3 * 4 * 4 * 4) + al(300 * 4 * 16 * 4) + al(300 * 4 * 16 * 4)
    assert lib.msa_prefill_tokens_workspace_size(ctypes.byref(_geom(dtype=msa.MSA_F32)), 3, 300,
                                                 16) == 0
    call = lambda ws, nbytes, **kw: lib.msa_sparse_attn_prefill_tokens(
        ctypes.byref(kw.get("g", g)), ctypes.byref(kw.get("c", c)), ctypes.byref(b), FAKE, FAKE,
        kw.get("topk", 16), kw.get("scale", 0.0), ws, nbytes, FAKE, None, None)
    assert call(FAKE * 256, need - 1) == WS_SMALL
    assert call(None, need) == INVALID
    assert call(FAKE + 4, need) == INVALID               # misaligned
    assert call(FAKE * 256, need, topk=0) == INVALID
    assert call(FAKE * 256, need, scale=float("inf")) == INVALID
    assert call(FAKE * 256, need, c=_cache(max_blocks_per_seq=131073)) == UNSUPPORTED
    assert call(FAKE * 256, need, g=_geom(head_dim=96)) == UNSUPPORTED


def test_prefill_staged_checks(lib):
    """Staged prefill attention: workspace size (0 off FP8; FP8: slot map, slot list and
    bf16 copies of K and V for H_kv * min(blocks, units * topk) slots) and the argument
    checks before any launch."""
    fp8 = _geom(cache_format=msa.MSA_CACHE_FP8_E4M3)
    c, b = _cache(), msa._Batch(FAKE, 3, 300)
    size = lambda g, cache, units, topk: lib.msa_prefill_workspace_size(
        ctypes.byref(g), None if cache is None else ctypes.byref(cache), units, topk)
    assert size(_geom(), c, 3, 16) == 0
    assert size(_geom(dtype=msa.MSA_F32), c, 3, 16) == 0
    assert size(fp8, None, 3, 16) == 0
    assert size(fp8, c, 3, 0) == 0
    al = lambda x: (x + 255) // 256 * 256
    for phys, units, topk in ((10, 3, 16), (1000, 3, 2), (4096, 256, 16)):
        S = 4 * min(phys, units * topk)
        expect = 256 + al(phys * 4 * 4) + al(S * 4) + 2 * S * 128 * 128 * 2
        assert size(fp8, _cache(num_phys_blocks=phys), units, topk) == expect
    need = size(fp8, c, 3, 16)
    call = lambda ws, nbytes, **kw: lib.msa_sparse_attn_prefill_staged(
        ctypes.byref(kw.get("g", fp8)), ctypes.byref(c), ctypes.byref(b), FAKE, FAKE,
        kw.get("topk", 16), kw.get("scale", 0.0), ws, nbytes, FAKE, None, None)
    assert call(FAKE * 256, need - 1) == WS_SMALL
    assert call(None, need) == INVALID
    assert call(FAKE + 4, need) == INVALID               # misaligned
    assert call(FAKE * 256, need, topk=0) == INVALID
    assert call(FAKE * 256, need, scale=float("nan")) == INVALID
    assert call(FAKE * 256, need, g=_geom(head_dim=96, cache_format=msa.MSA_CACHE_FP8_E4M3)) \
        == UNSUPPORTED
    empty = msa._Batch(None, 0, 0)
    assert lib.msa_sparse_attn_prefill_staged(ctypes.byref(fp8), ctypes.byref(c),
                                              ctypes.byref(empty), None, None, 16, 0.0, None, 0,
                                              None, None, None) == OK


def test_probe_library_exports_and_checks():
    """libmsa_probe.so (the bench's peak-rate probes) exports every function of
    include/msa_probe.h and rejects bad arguments before any launch (-1)."""
    path = os.path.join(ROOT, "block_sparse_long_11_amd", "libmsa_probe.so")
    if not os.path.exists(path):
        pytest.fail("libmsa_probe.so is not built (run __graft_entry__.build())")
    text = open(os.path.join(ROOT, "include", "msa_probe.h")).read()
    names = sorted(set(re.findall(r"^int\s+(msa_probe_[a-z0-9_]+)\s*\(", text, re.M)))
    assert names == ["msa_probe_copy", "msa_probe_mfma_bf16", "msa_probe_mfma_bf16_random",
                     "msa_probe_mfma_valu", "msa_probe_stream_read"]
    plib = ctypes.CDLL(path)
    for n in names:
        getattr(plib, n).restype = ctypes.c_int
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    plib.msa_probe_stream_read.argtypes = [vp, sz, ctypes.c_int, vp, vp]
    assert plib.msa_probe_stream_read(FAKE, 1000, 64, FAKE, None) == -1      # not 32 KiB units
    assert plib.msa_probe_stream_read(FAKE, 32768, 0, FAKE, None) == -1
    assert plib.msa_probe_stream_read(None, 32768, 64, FAKE, None) == -1
    plib.msa_probe_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    far = FAKE + (1 << 30)
    assert plib.msa_probe_copy(FAKE, far, 1000, 64, None) == -1           # not 16-byte units
    assert plib.msa_probe_copy(FAKE, FAKE + 4096, 8192, 64, None) == -1   # overlap
    assert plib.msa_probe_copy(FAKE + 8, far, 4096, 64, None) == -1       # unaligned
    assert plib.msa_probe_copy(FAKE, far, 4096, 0, None) == -1
    assert plib.msa_probe_copy(None, far, 4096, 64, None) == -1
    for n in ("msa_probe_mfma_bf16", "msa_probe_mfma_bf16_random"):
        fn = getattr(plib, n)
        fn.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
        assert fn(0, 10, FAKE, None) == -1
        assert fn(64, 0, FAKE, None) == -1
        assert fn(64, 10, None, None) == -1
    plib.msa_probe_mfma_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    assert plib.msa_probe_mfma_valu(64, 10, 0, FAKE, None) == -1
    assert plib.msa_probe_mfma_valu(64, 10, 4, FAKE, None) == -1
    assert plib.msa_probe_mfma_valu(32769, 10, 3, FAKE, None) == -1


def _stderr_of(fn):
    """Runs fn() with file descriptor 2 redirected to a temporary file; returns the
    text written there (the library prints with stdio, below Python's sys.stderr)."""
    import tempfile
    with tempfile.TemporaryFile(mode="w+b") as tmp:
        saved = os.dup(2)
        try:
            os.dup2(tmp.fileno(), 2)
            fn()
        finally:
            ctypes.CDLL(None).fflush(None)
            os.dup2(saved, 2)
            os.close(saved)
        tmp.seek(0)
        return tmp.read().decode()


def test_msa_log_reports_refused_calls(lib, monkeypatch):
    """MSA_LOG=1: a refused call prints its reason to stderr; unset, nothing."""
    c, b = _cache(), msa._Batch(FAKE, 3, 300)
    call = lambda: lib.msa_sparse_attn_prefill(None, ctypes.byref(c), ctypes.byref(b), FAKE, FAKE,
                                               16, 0.0, FAKE, None, None)
    monkeypatch.delenv("MSA_LOG", raising=False)
    assert _stderr_of(call) == ""
    monkeypatch.setenv("MSA_LOG", "1")
    text = _stderr_of(call)
    assert "msa: refused (status 1): geom is NULL" in text
    monkeypatch.setenv("MSA_LOG", "0")
    assert _stderr_of(call) == ""


def test_validate_block_table_and_ids(lib):
    """Host debugging aids: a block table whose sequences' blocks are physical blocks
    passes; the first entry outside [0, num_phys_blocks) is named; id lists pass with
    distinct in-range entries before their first -1 (entries after it are ignored) and
    fail on an out-of-range or repeated entry."""
    bt = torch.tensor([[3, 0, 7, -5], [1, 2, -1, -1]], dtype=torch.int32)
    sl = torch.tensor([300, 200], dtype=torch.int32)     # 3 and 2 blocks
    msa.msa_validate_block_table(bt, sl, 8)
    with pytest.raises(msa.MsaError, match=r"block_table\[0\]\[2\] = 7"):
        msa.msa_validate_block_table(bt, sl, 7)
    with pytest.raises(msa.MsaError, match="more than 4 blocks"):
        msa.msa_validate_block_table(bt, torch.tensor([600, 1], dtype=torch.int32), 8)
    bt2 = bt.clone()
    bt2[1, 1] = -1
    with pytest.raises(msa.MsaError, match=r"block_table\[1\]\[1\] = -1"):
        msa.msa_validate_block_table(bt2, sl, 8)
    ids = torch.tensor([[[0, 3, 2, -1]], [[5, -1, 5, 99]]], dtype=torch.int32)
    msa.msa_validate_ids(ids, 6)
    with pytest.raises(msa.MsaError, match="row 0 group 0 entry 1 is 3"):
        msa.msa_validate_ids(ids, 3)
    bad = ids.clone()
    bad[0, 0, 2] = 0
    with pytest.raises(msa.MsaError, match="row 0 group 0 lists a block twice"):
        msa.msa_validate_ids(bad, 6)
    # the oracle's selection (ascending, the diagonal last, -1 padded) passes
    rng = np.random.default_rng(3)
    rows = [[O.select_blocks(rng.standard_normal(8), tau, 5) for tau in (0, 2, 7)]]
    msa.msa_validate_ids(torch.tensor(np.asarray(rows, dtype=np.int32).transpose(1, 0, 2)), 8)
    assert lib.msa_validate_ids(None, 0, 1, 4, 8) == OK
    assert lib.msa_validate_ids(None, 1, 1, 4, 8) == INVALID
    # the binding refuses what the C call would misread: a short seq_lens, wrong
    # ranks, and values that a cast to int32 would wrap
    with pytest.raises(ValueError, match="entries for"):
        msa.msa_validate_block_table(bt, sl[:1], 8)
    with pytest.raises(ValueError, match="2-D"):
        msa.msa_validate_block_table(bt[0], sl, 8)
    with pytest.raises(ValueError, match="outside int32"):
        msa.msa_validate_ids(torch.tensor([[[2**32 + 1, -1]]], dtype=torch.int64), 8)
    msa.msa_validate_ids(torch.tensor([[[1, 0, -1]]], dtype=torch.int64), 8)
    msa.msa_validate_ids(torch.zeros(0, 1, 4, dtype=torch.int32), 8)
