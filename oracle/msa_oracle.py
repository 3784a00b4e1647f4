"""CPU oracle for MiniMax Sparse Attention (MSA): block indexer scores, block top-k
selection and exact softmax attention over the selected 128-token KV blocks.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code, header, table or helper with the HIP library.

Plain NumPy in float64. Inputs may be float32 or float64 arrays (bf16 inputs are
passed as their exact float32 upcast); every product and sum here is float64.

Sources (the pages this follows):
  [dd]   daily.dev, "MiniMax M3: 1M-token multimodal reasoning model now available
         with NVIDIA and vLLM support": sections "Summary" and "What makes M3
         different" (128-token KV blocks, top blocks kept per query).
  [feat] models.inteligile.com, "MiniMax-M3" feature page, table "Checked in its
         code": rows "Indexer-selected sparse attention (DeepSeek Sparse
         Attention)" (indexer scores keys per head, pools into blocks,
         topk = min(topk_blocks, num_key_blocks), -inf selections become -1),
         "Grouped-query attention" (64 query heads share 4 KV heads through
         repeat_kv) and "Learnable attention sink" (plain fp32 softmax, no sink).
  [vllm] 24-ai.news, "MiniMax M3 in vLLM: Day-0-Unterstuetzung ...", section
         "Warum ist ein Million-Token-Kontext eine Serving-Herausforderung?"
         (each query or GQA query group scores all blocks; KV-block-major layout).

Where the pages leave a step open this module takes these readings:
  * score of a (query, key) pair for selection group g = sum over the group's
    indexer heads of the raw dot product q_idx . k_idx (no scale, no softmax);
  * block score = max over the block's keys and over the unit's queries;
  * a unit is (request, 128-aligned query tile, group) in prefill and
    (sequence, group) in decode; its "diagonal" block is the block that holds its
    queries and is always kept; blocks after it are masked (causal);
  * ties in block score go to the lower block id; ids are returned ascending and
    padded with -1;
  * query head i reads KV head i // (H_q / H_kv); with n_sel == H_kv selection
    group g drives KV head g, with n_sel == 1 one selection serves every KV head.

Cache layout (block-major, paged): cache[phys_block][head][token_in_block][dim],
block_table[r][logical_block] = phys_block, seq_lens[r] = tokens of request r
including its new ones.

New tokens before the steps above (qk_norm_rope_insert), from [feat] rows "QK
normalization" (queries and keys each go through a per-head RMSNorm before the
rotary embedding) and "Partial RoPE" (partial_rotary_factor 0.5, rotary_dim 64:
only the first rotary_dim channels of each head are rotated, the rest pass
through) and [dd] "Serving options" (fused QK-norm + RoPE + KV insert). Readings:
  * RMSNorm of a head vector x (its head_dim channels): x / sqrt(mean(x^2) + eps)
    times a weight vector of length head_dim shared by all heads; eps is given;
  * rotation of position p: channel i < rotary_dim/2 pairs with i + rotary_dim/2
    (the rotate-half form), angle p * theta**(-2 i / rotary_dim), theta given;
  * K is normalized and rotated before it is written to the cache, V and the
    indexer keys are written as given; q_idx is not touched.
"""

import math

import numpy as np

BLOCK = 128


# ----------------------------------------------------------------------------
# units
# ----------------------------------------------------------------------------

def prefill_units(seq_lens, q_lens):
    """Units of a (chunked) prefill batch.

    Request r has seq_lens[r] tokens in its cache, the last q_lens[r] of which are
    its new queries, at positions seq_lens[r]-q_lens[r] ... seq_lens[r]-1, stored
    contiguously in the query arrays after those of requests 0..r-1. Queries are
    grouped by the 128-token block holding their position; that block is the
    unit's diagonal block tau.

    Returns a list of dicts with r, tau, row0, row1 (query rows [row0, row1)) and
    pos0 (the position of row0).
    """
    units = []
    row = 0
    for r, (L, n) in enumerate(zip(seq_lens, q_lens)):
        L, n = int(L), int(n)
        assert 0 <= n <= L
        first = L - n
        p = first
        while p < L:
            tau = p // BLOCK
            end = min((tau + 1) * BLOCK, L)
            units.append(dict(r=r, tau=tau, row0=row + (p - first),
                              row1=row + (end - first), pos0=p))
            p = end
        row += n
    return units


def decode_units(seq_lens):
    """One unit per sequence: its single new query sits at position L-1."""
    return [dict(r=r, tau=(int(L) - 1) // BLOCK, row0=r, row1=r + 1, pos0=int(L) - 1)
            for r, L in enumerate(seq_lens)]


def token_units(seq_lens, tokens_per_seq):
    """Per-query-token units of a multi-token decode ([feat] row "Indexer-selected
    sparse attention": the model's selection is shaped [B, H_idx, S_q, topk], one
    block list per query token). Sequence r has T = tokens_per_seq new tokens,
    rows r*T + i at positions L-T+i (i < T), each a unit of its own: it scores the
    blocks with its own indexer query, keeps its own diagonal block and top-k,
    and attends causally. T = 1 is decode_units."""
    T = int(tokens_per_seq)
    units = []
    for r, L in enumerate(seq_lens):
        L = int(L)
        assert L >= T
        for i in range(T):
            p = L - T + i
            units.append(dict(r=r, tau=p // BLOCK, row0=r * T + i, row1=r * T + i + 1, pos0=p))
    return units


def prefill_token_units(seq_lens, q_lens):
    """Per-query-token units of a (chunked) prefill batch ([feat] row
    "Indexer-selected sparse attention": the selection is shaped [B, H_idx, S_q,
    topk], one block list per query token). Every new token is a unit of its own:
    its row (the same row layout as prefill_units), its position p, its diagonal
    block p // 128. A batch of T new tokens per sequence is token_units."""
    units = []
    for un in prefill_units(seq_lens, q_lens):
        for i in range(un["row1"] - un["row0"]):
            p = un["pos0"] + i
            units.append(dict(r=un["r"], tau=p // BLOCK, row0=un["row0"] + i,
                              row1=un["row0"] + i + 1, pos0=p))
    return units


# ----------------------------------------------------------------------------
# paged cache access
# ----------------------------------------------------------------------------

def logical_block(cache, bt_row, b, heads=None):
    """All 128 tokens of logical block b, float64 [128][heads][dim]."""
    blk = np.asarray(cache[int(bt_row[b])], dtype=np.float64)   # [heads][128][dim]
    if heads is not None:
        blk = blk[heads]
    return np.transpose(blk, (1, 0, 2))


# ----------------------------------------------------------------------------
# step 1: indexer block scores
# ----------------------------------------------------------------------------

def unit_block_scores(q_idx_rows, k_idx_cache, bt_row, tau, n_sel, row_len):
    """Block scores of one unit, float64 [n_sel][row_len].

    For candidate block b < tau:
        S_g(b) = max over the unit's queries t and the block's keys s of
                 sum over indexer heads h of group g of q_idx[t,h,:] . k_idx[s,h,:]
    ([feat] "scores keys per head and pools into blocks"; the group sum and the
    max pooling are the readings listed in the module docstring.)
    S_g(tau) = +inf marks the always-kept diagonal block; blocks after tau and
    entries past the request's last block are -inf (causal masking, the -inf
    convention of [feat]).
    """
    q_idx_rows = np.asarray(q_idx_rows, dtype=np.float64)
    T, H_i, D_i = q_idx_rows.shape
    assert H_i % n_sel == 0
    H_s = H_i // n_sel
    S = np.full((n_sel, row_len), -np.inf)
    for g in range(n_sel):
        heads = slice(g * H_s, (g + 1) * H_s)
        # the group's heads concatenated: one dot product of length H_s * D_i
        qg = q_idx_rows[:, heads, :].reshape(T, H_s * D_i)
        for b in range(tau):
            kg = logical_block(k_idx_cache, bt_row, b, heads).reshape(BLOCK, H_s * D_i)
            pair = qg @ kg.T                      # [T][128] pair scores
            S[g, b] = pair.max()
        S[g, tau] = np.inf
    return S


def index_scores(units, q_idx, k_idx_cache, block_table, n_sel, row_len):
    """Scores for every unit: float64 [U][n_sel][row_len]."""
    out = np.empty((len(units), n_sel, row_len))
    for u, un in enumerate(units):
        out[u] = unit_block_scores(q_idx[un["row0"]:un["row1"]], k_idx_cache,
                                   block_table[un["r"]], un["tau"], n_sel, row_len)
    return out


# ----------------------------------------------------------------------------
# step 2: block selection
# ----------------------------------------------------------------------------

def select_blocks(scores_g, tau, topk):
    """Kept blocks of one (unit, group) row, ascending, padded with -1.

    K = min(topk, tau + 1) blocks are kept ([feat]: topk = min(topk_blocks,
    num_key_blocks), with the tau + 1 causally visible blocks as the key
    blocks): the diagonal tau plus the K - 1 candidates b < tau of highest score,
    equal scores ordered by lower block id.
    """
    K = min(topk, tau + 1)
    candidates = sorted(range(tau), key=lambda b: (-float(scores_g[b]), b))
    kept = sorted([tau] + candidates[:K - 1])
    return kept + [-1] * (topk - len(kept))


def select(scores, units, topk):
    """ids int32 [U][n_sel][topk] for all units."""
    U, n_sel, _ = scores.shape
    ids = np.empty((U, n_sel, topk), dtype=np.int32)
    for u in range(U):
        for g in range(n_sel):
            ids[u, g] = select_blocks(scores[u, g], units[u]["tau"], topk)
    return ids


# ----------------------------------------------------------------------------
# step 3: exact softmax attention over the kept blocks
# ----------------------------------------------------------------------------

def unit_attention(q_rows, pos0, ids_unit, k_cache, v_cache, bt_row, seq_len, n_sel,
                   scale=None):
    """Exact attention of one unit's queries over its kept blocks.

    q_rows [T][H_q][D]; query row t sits at position pos0 + t.
    ids_unit [n_sel][topk]. Query head i reads KV head j = i // G with G = H_q/H_kv
    ([feat] "Grouped-query attention": repeat_kv); the selection row used is group
    j when n_sel == H_kv and group 0 when n_sel == 1.

    Visible keys of query t: every token s of a kept block with s <= pos0 + t and
    s < seq_len. Logits z_s = scale * q . k_s (scale 1/sqrt(D) by default);
    out = sum_s softmax(z)_s v_s and lse = log sum_s exp(z_s), natural log.
    The softmax is plain, with no sink logit and no output gate ([feat] row
    "Learnable attention sink").
    The kept list is read as a set of block ids: the entries before its first -1
    (the padding; anything after it is ignored), in any order; a block after the
    query (or past seq_len) adds no key. A query with no visible key at all (a list the selection never makes:
    no block up to its own position) has an empty softmax: out 0, lse -inf.
    Returns out [T][H_q][D] and lse [T][H_q], float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    T, H_q, D = q_rows.shape
    H_kv = k_cache.shape[1]
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((T, H_q, D))
    lse = np.zeros((T, H_q))
    positions = pos0 + np.arange(T)
    for j in range(H_kv):
        g = j if n_sel == H_kv else 0
        listed = []
        for b in ids_unit[g]:
            if b < 0:
                break
            listed.append(int(b))
        # blocks holding at least one key of the request
        blocks = [b for b in listed if b * BLOCK < seq_len]
        keys = np.concatenate([np.arange(b * BLOCK, min((b + 1) * BLOCK, seq_len))
                               for b in blocks] + [np.zeros(0, dtype=np.int64)])
        # K/V rows line up with `keys`: both walk the kept blocks in the same
        # order, each block cut at seq_len.
        K, V = _trim_blocks(k_cache, v_cache, bt_row, blocks, seq_len, j, D)
        visible = keys[None, :] <= positions[:, None]          # [T][nkeys]
        seen = visible.any(axis=1)                              # [T]
        for i in range(j * G, (j + 1) * G):
            z = scale * (q_rows[:, i, :] @ K.T)                 # [T][nkeys]
            z = np.where(visible, z, -np.inf)
            m = np.where(seen, z.max(axis=1, initial=-np.inf), 0.0)[:, None]
            e = np.where(visible, np.exp(z - m), 0.0)
            ssum = e.sum(axis=1, keepdims=True)
            out[:, i, :] = np.where(seen[:, None], e / np.where(ssum > 0, ssum, 1.0), 0.0) @ V
            lse[:, i] = np.where(seen, (m + np.log(np.where(ssum > 0, ssum, 1.0)))[:, 0],
                                 -np.inf)
    return out, lse


def _trim_blocks(k_cache, v_cache, bt_row, blocks, seq_len, j, D):
    """K and V rows (float64 [nkeys][D]) of KV head j over the kept blocks, in
    block order, each block cut at seq_len (every block holds at least one key)."""
    ks, vs = [np.zeros((0, D))], [np.zeros((0, D))]
    for b in blocks:
        n = min(BLOCK, seq_len - b * BLOCK)
        ks.append(logical_block(k_cache, bt_row, b, slice(j, j + 1))[:n, 0, :])
        vs.append(logical_block(v_cache, bt_row, b, slice(j, j + 1))[:n, 0, :])
    return np.concatenate(ks), np.concatenate(vs)


def attention(units, ids, q, k_cache, v_cache, block_table, seq_lens, n_sel, scale=None):
    """out [rows][H_q][D] and lse [rows][H_q] over all units."""
    q = np.asarray(q)
    rows = max(un["row1"] for un in units)
    out = np.zeros((rows,) + q.shape[1:])
    lse = np.zeros((rows, q.shape[1]))
    for u, un in enumerate(units):
        o, l = unit_attention(q[un["row0"]:un["row1"]], un["pos0"], ids[u], k_cache,
                              v_cache, block_table[un["r"]], int(seq_lens[un["r"]]),
                              n_sel, scale)
        out[un["row0"]:un["row1"]] = o
        lse[un["row0"]:un["row1"]] = l
    return out, lse


# ----------------------------------------------------------------------------
# whole path
# ----------------------------------------------------------------------------

def max_blocks(seq_lens):
    return max((int(L) + BLOCK - 1) // BLOCK for L in seq_lens)


def run_prefill(q, q_idx, k_cache, v_cache, k_idx_cache, block_table, seq_lens, q_lens,
                n_sel, topk, scale=None, row_len=None):
    """Index, select and attend for a chunked prefill batch."""
    units = prefill_units(seq_lens, q_lens)
    row_len = row_len or block_table.shape[1]
    scores = index_scores(units, q_idx, k_idx_cache, block_table, n_sel, row_len)
    ids = select(scores, units, topk)
    out, lse = attention(units, ids, q, k_cache, v_cache, block_table, seq_lens, n_sel,
                         scale)
    return dict(units=units, scores=scores, ids=ids, out=out, lse=lse)


def run_decode(q, q_idx, k_cache, v_cache, k_idx_cache, block_table, seq_lens, n_sel,
               topk, scale=None, row_len=None):
    """Index, select and attend for one decode step (one query per sequence)."""
    units = decode_units(seq_lens)
    row_len = row_len or block_table.shape[1]
    scores = index_scores(units, q_idx, k_idx_cache, block_table, n_sel, row_len)
    ids = select(scores, units, topk)
    out, lse = attention(units, ids, q, k_cache, v_cache, block_table, seq_lens, n_sel,
                         scale)
    return dict(units=units, scores=scores, ids=ids, out=out, lse=lse)


def run_tokens(q, q_idx, k_cache, v_cache, k_idx_cache, block_table, seq_lens,
               tokens_per_seq, n_sel, topk, scale=None, row_len=None):
    """Index, select and attend for a multi-token decode step with per-token
    selection (token_units): rows r*T + i of q and q_idx."""
    units = token_units(seq_lens, tokens_per_seq)
    row_len = row_len or block_table.shape[1]
    scores = index_scores(units, q_idx, k_idx_cache, block_table, n_sel, row_len)
    ids = select(scores, units, topk)
    out, lse = attention(units, ids, q, k_cache, v_cache, block_table, seq_lens, n_sel,
                         scale)
    return dict(units=units, scores=scores, ids=ids, out=out, lse=lse)


def run_prefill_tokens(q, q_idx, k_cache, v_cache, k_idx_cache, block_table, seq_lens,
                       q_lens, n_sel, topk, scale=None, row_len=None):
    """Index, select and attend for a prefill batch with per-query-token selection
    (prefill_token_units): each new token scores the blocks with its own indexer
    query, keeps its diagonal and its own top-k, and attends causally over them."""
    units = prefill_token_units(seq_lens, q_lens)
    row_len = row_len or block_table.shape[1]
    scores = index_scores(units, q_idx, k_idx_cache, block_table, n_sel, row_len)
    ids = select(scores, units, topk)
    out, lse = attention(units, ids, q, k_cache, v_cache, block_table, seq_lens, n_sel,
                         scale)
    return dict(units=units, scores=scores, ids=ids, out=out, lse=lse)


# ----------------------------------------------------------------------------
# new tokens: QK-norm, partial RoPE and cache insert
# ----------------------------------------------------------------------------

def rms_norm(x, w, eps):
    """RMSNorm over the last axis ([feat] "QK normalization": per head)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope(x, pos, theta, rotary_dim):
    """Rotary embedding of the first rotary_dim channels of x[..., T, H, D]-like
    arrays whose leading axis is the token axis; pos[T] are the token positions
    ([feat] "Partial RoPE": channel i pairs with i + rotary_dim/2)."""
    x = np.asarray(x, dtype=np.float64)
    half = rotary_dim // 2
    inv = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]        # [T][half]
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    out = x.copy()
    x1, x2 = x[..., :half], x[..., half:rotary_dim]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rotary_dim] = x2 * c + x1 * s
    return out


def token_positions(units):
    """(row, request, position) of every new token of the units, in row order."""
    rows = []
    for u in units:
        for i in range(u["row1"] - u["row0"]):
            rows.append((u["row0"] + i, u["r"], u["pos0"] + i))
    rows.sort()
    return rows


def qk_norm_rope_insert(units, q, k, v, k_idx, q_norm_w, k_norm_w, eps, theta, rotary_dim,
                        k_cache, v_cache, k_idx_cache, block_table):
    """Normalize and rotate the new queries and keys; write K, V and the indexer
    keys of every new token into copies of the caches (token-major layout
    cache[phys][head][row][dim]). Token at row t, request r, position p goes to
    physical block block_table[r][p // 128], row p % 128.

    Returns (q_out [T][H_q][D], k_cache, v_cache, k_idx_cache), all float64."""
    toks = token_positions(units)
    rows = np.array([t[0] for t in toks], dtype=np.int64)
    pos = np.array([t[2] for t in toks], dtype=np.float64)
    q_out = rope(rms_norm(np.asarray(q, np.float64)[rows], q_norm_w, eps), pos, theta,
                 rotary_dim)
    k_new = rope(rms_norm(np.asarray(k, np.float64)[rows], k_norm_w, eps), pos, theta,
                 rotary_dim)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    ic = np.array(k_idx_cache, dtype=np.float64)
    v64 = np.asarray(v, np.float64)
    i64 = np.asarray(k_idx, np.float64)
    for n, (row, r, p) in enumerate(toks):
        phys = int(block_table[r][p // BLOCK])
        kc[phys, :, p % BLOCK, :] = k_new[n]
        vc[phys, :, p % BLOCK, :] = v64[row]
        ic[phys, :, p % BLOCK, :] = i64[row]
    q_full = np.zeros(np.asarray(q).shape, dtype=np.float64)
    q_full[rows] = q_out
    return q_full, kc, vc, ic



# ----------------------------------------------------------------------------
# FP8 caches: E4M3 codes with one power-of-two scale per 32 channels of a row
# ----------------------------------------------------------------------------
# [dd] "What's coming" lists FP8 KV-cache paths; the pages give no format. Read
# here as the OCP 8-bit floating-point E4M3 encoding (1 sign bit, 4 exponent bits
# with bias 7, 3 mantissa bits; exponent field 15 with mantissa 7 is NaN, so the
# largest finite magnitude is 1.75 * 2^8 = 448; exponent field 0 holds the
# subnormals m/8 * 2^-6) with one scale per block of 32 consecutive channels of
# one token's head vector. The scale is a power of two 2^e, stored as the byte
# e + 127 (the OCP E8M0 scale encoding), e the smallest integer with
# max|x| / 2^e <= 448; each channel stores the E4M3 code nearest to x / 2^e
# (ties to the even code). The value a code stands for is decode(code) * 2^e.

E4M3_MAX = 448.0
SCALE_BLOCK = 32
SCALE_BIAS = 127


def e4m3_decode(codes):
    """Values (float64) of E4M3 codes; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m / 8.0 * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, v)


_E4M3_POS = e4m3_decode(np.arange(0x7F))          # codes 0x00..0x7E, increasing


def e4m3_encode(y):
    """E4M3 code (uint8) of the value nearest to each y, ties to the even code.
    Requires |y| <= 448. The sign is kept, also when the result is zero."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    assert np.all(mag <= E4M3_MAX), "value outside the E4M3 range"
    hi = np.clip(np.searchsorted(_E4M3_POS, mag, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi, d_lo = _E4M3_POS[hi] - mag, mag - _E4M3_POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def mx_exponent(amax):
    """Smallest integer e with amax / 2^e <= 448 (amax >= 0), within [-127, 127];
    amax == 0 gives -127."""
    a = np.asarray(amax, dtype=np.float64)
    frac, k = np.frexp(a)                    # a = frac * 2^k, frac in [0.5, 1)
    e = (k - 1) - 8 + (2.0 * frac > 1.75)   # a = (2 frac) * 2^(k-1)
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(x):
    """x [..., C] (C a multiple of 32) -> (codes uint8 [..., C], scale bytes uint8
    [..., C/32]): one scale per 32 consecutive channels of the last axis."""
    x = np.asarray(x, dtype=np.float64)
    blk = x.reshape(x.shape[:-1] + (x.shape[-1] // SCALE_BLOCK, SCALE_BLOCK))
    e = mx_exponent(np.abs(blk).max(axis=-1))
    codes = e4m3_encode(blk / np.exp2(e.astype(np.float64))[..., None])
    return codes.reshape(x.shape), (e + SCALE_BIAS).astype(np.uint8)


def mx_dequantize(codes, scales):
    """Values (float64 [..., C]) of codes [..., C] with scale bytes [..., C/32]."""
    codes = np.asarray(codes)
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (-1, SCALE_BLOCK))
    e = np.asarray(scales, dtype=np.float64) - SCALE_BIAS
    return (v * np.exp2(e)[..., None]).reshape(codes.shape)


def qk_norm_rope_insert_fp8(units, q, k, v, k_idx, q_norm_w, k_norm_w, eps, theta,
                            rotary_dim, caches, block_table):
    """The new-token step into FP8 caches. caches is a dict of token-major code and
    scale arrays: k, v [P][H_kv][128][D] with k_s, v_s [P][H_kv][128][D/32], and
    i [P][H_i][128][D_i] with i_s [P][H_i][128][D_i/32]. Each new token's K (after
    norm and rotation), V and indexer-key rows are quantized row by row and
    replace that token's codes and scales; nothing else changes.

    Returns (q_out float64, new caches dict)."""
    toks = token_positions(units)
    rows = np.array([t[0] for t in toks], dtype=np.int64)
    pos = np.array([t[2] for t in toks], dtype=np.float64)
    q_out = rope(rms_norm(np.asarray(q, np.float64)[rows], q_norm_w, eps), pos, theta,
                 rotary_dim)
    k_new = rope(rms_norm(np.asarray(k, np.float64)[rows], k_norm_w, eps), pos, theta,
                 rotary_dim)
    out = {name: np.array(a) for name, a in caches.items()}
    kq, ks = mx_quantize(k_new)
    vq, vs = mx_quantize(np.asarray(v, np.float64)[rows])
    iq, is_ = mx_quantize(np.asarray(k_idx, np.float64)[rows])
    for n, (row, r, p) in enumerate(toks):
        phys, slot = int(block_table[r][p // BLOCK]), p % BLOCK
        out["k"][phys, :, slot], out["k_s"][phys, :, slot] = kq[n], ks[n]
        out["v"][phys, :, slot], out["v_s"][phys, :, slot] = vq[n], vs[n]
        out["i"][phys, :, slot], out["i_s"][phys, :, slot] = iq[n], is_[n]
    q_full = np.zeros(np.asarray(q).shape, dtype=np.float64)
    q_full[rows] = q_out
    return q_full, out
