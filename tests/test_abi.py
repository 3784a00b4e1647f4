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
