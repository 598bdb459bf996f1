"""Plain fp64 definition of the CSA / HCA attention step over a compressed KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and literal on
purpose: each function is the definition written out with numpy, no blocking,
fusion or reordering beyond it.

Page: "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence
Review" (dimensionstp.github.io), abbreviated PAGE below.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 storage <-> fp64 values


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: a bf16 is the upper 16 bits of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


_BF16_MAX = float.fromhex("0x1.fep127")  # (2 - 2^-7) * 2^127


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 (one rounding, to nearest, ties to even).

    bf16 keeps 8 significant bits; below its smallest normal 2^-126 the spacing
    is fixed at 2^-133.  The value is scaled by a power of two so that one bf16
    spacing becomes 1, rounded with numpy's rint (ties to even) and scaled back;
    values past the largest finite bf16 after rounding become infinities.
    NaN maps to the quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = f * 2^e with 0.5 <= |f| < 1
    shift = np.maximum(e.astype(np.int64) - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -shift)), shift)
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


def to_bf16_values(x) -> np.ndarray:
    """fp64 values after a round trip through bf16 storage."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


# --------------------------------------------------------------------------------------
# compression


def fp8_e4m3_values(codes) -> np.ndarray:
    """Values of FP8 E4M3 codes (the OCP 8-bit floating point E4M3 format): bit 7 the
    sign, bits 6..3 the exponent with bias 7, bits 2..0 the mantissa; exponent field
    0 is subnormal (m * 2^-9), otherwise (1 + m/8) * 2^(e - 7); S.1111.111 is NaN and
    there are no infinities (largest finite value 448)."""
    c = np.asarray(codes).astype(np.int64) & 255
    sign, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


KV8_ROW_BYTES = 192   # 64 FP8 bytes (dims 0..63), then 64 bf16 values (dims 64..127)


def kv8_values(rows) -> np.ndarray:
    """Values of mixed-storage KV rows [N, 192] (uint8) as fp64 [N, 128].

    PAGE section 3-2 item 2 (component table): the KV cache keeps the RoPE dims in
    BF16 and the rest in FP8.  Reading: of the 128 dims of a compressed entry the last
    64 are the RoPE dims; a row stores dims 0..63 as FP8 E4M3 codes (one scale per
    tensor, 1) in bytes 0..63 and dims 64..127 as bf16 (little-endian) in bytes
    64..191.  The same row format serves the K and the V cache."""
    r = np.asarray(rows, dtype=np.uint8).reshape(-1, KV8_ROW_BYTES)
    lo = fp8_e4m3_values(r[:, :64])
    hi = bf16_bits_to_f64(np.ascontiguousarray(r[:, 64:]).view("<u2"))
    return np.concatenate([lo, hi], axis=1)


def kv_compress(x, c: int) -> np.ndarray:
    """Sequence-direction compression: one entry per complete block of c tokens.

    PAGE section 2-1 and section 3-2 item 2 (component table): CSA turns every 4
    tokens into one compressed entry, HCA every 128 tokens; both models use the
    ratios 4 and 128.  The page does not give the pooling operator; the workload
    fixes the mean.  Entry j is the mean of tokens j*c .. j*c+c-1.  A tail of
    T mod c tokens forms no entry: the page keeps tokens that are not yet ready
    for compression in a separate state cache (section 3-2 item 4).

    x: [T, D] values; returns [T // c, D] fp64 means (not yet rounded to bf16)."""
    x = np.asarray(x, dtype=np.float64)
    t, d = x.shape
    n = t // c
    return x[: n * c].reshape(n, c, d).mean(axis=1)


def compress_to_cache(x, c: int) -> np.ndarray:
    """Compressed entries as stored in the bf16 cache (bit patterns)."""
    return f64_to_bf16_bits(kv_compress(x, c))


def fp8_e4m3_round(x) -> np.ndarray:
    """FP8 E4M3 codes of fp64 values: the nearest finite E4M3 value (ties to the code
    with an even mantissa), magnitudes beyond the largest finite value 448 clamped to
    it, the sign kept (a negative value that rounds to zero gives -0).

    Written as the definition: every non-negative finite magnitude is listed with its
    code, and each input picks the closest one by brute force."""
    x = np.asarray(x, dtype=np.float64)
    codes = np.arange(128)
    mags = fp8_e4m3_values(codes)
    finite = ~np.isnan(mags)
    codes, mags = codes[finite], mags[finite]          # 0x00 .. 0x7E, increasing
    a = np.minimum(np.abs(x), mags[-1]).reshape(-1, 1)
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best                                  # one or two candidates
    even = tied & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(tied, axis=1))
    out = codes[pick].reshape(x.shape) | np.where(np.signbit(x), 128, 0)
    return out.astype(np.uint8)


def compress_to_cache_kv8(x, c: int) -> np.ndarray:
    """Compressed entries as stored in a mixed KV cache: rows [T // c, 192] (uint8)
    holding the fp64 block means, dims 0..63 rounded once to FP8 E4M3 and dims
    64..127 once to bf16 (the row format of kv8_values)."""
    m = kv_compress(x, c)
    lo = fp8_e4m3_round(m[:, :64])
    hi = f64_to_bf16_bits(m[:, 64:]).astype("<u2").view(np.uint8).reshape(len(m), 128)
    return np.concatenate([lo, hi], axis=1)


# --------------------------------------------------------------------------------------
# CSA selection


def n_visible(pos: int, c: int, n_entries: int) -> int:
    """Number of compressed entries a query at absolute position `pos` may see.

    The workload states that a query sees only compressed blocks that end
    before its position.  Block j spans tokens j*c .. j*c+c-1, so it ends
    before `pos` iff j*c + c - 1 < pos, i.e. (j+1)*c <= pos; visible entries are
    therefore 0 .. floor(pos/c)-1, capped by the entries the cache holds.  A
    decoding query sits at position L after L context tokens and sees all
    floor(L/c) entries."""
    return int(min(pos // c, n_entries))


def index_scores(q_idx, k_idx) -> np.ndarray:
    """Indexer scores s_j = sum_d q[d] * k[j, d] in exact integer arithmetic.

    PAGE section 3-2 item 4: CSA has an indexer whose Q.K path picks the
    entries to attend (trained there with FP4 quantisation-aware training).
    The workload fixes the form: int8 query and keys of width d_idx, dot
    product accumulated exactly (int32 cannot overflow: |s| <= d * 127^2)."""
    q = np.asarray(q_idx, dtype=np.int64)
    k = np.asarray(k_idx, dtype=np.int64)
    return k @ q


def fp4_values(codes) -> np.ndarray:
    """Values of FP4 E2M1 codes (OCP Microscaling formats, E2M1 element type): bit 3
    is the sign, bits 2..1 the exponent with bias 1, bit 0 the mantissa; exponent
    field 0 is subnormal (m * 2^-1), otherwise (1 + m/2) * 2^(e - 1)."""
    c = np.asarray(codes).astype(np.int64) & 15
    sign, e, m = c >> 3, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(sign == 1, -mag, mag)


def fp4_unpack(packed) -> np.ndarray:
    """Packed FP4 [..., n/2] bytes -> codes [..., n]: element 2i sits in the low
    nibble of byte i, element 2i + 1 in the high nibble."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    return np.stack([b & 15, b >> 4], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])


def index_scores_fp4(q_fp4, k_fp4) -> np.ndarray:
    """FP4 indexer scores: J_j = 256 * sum_d q[d] * k[j, d] over E2M1 values, exactly.

    PAGE section 3-2 item 4: the CSA indexer's Q.K path is trained with FP4
    quantisation-aware training.  Reading: query and keys are E2M1 codes (d_idx = 64,
    32 packed bytes per vector) with one power-of-two scale per tensor; a positive
    common factor cannot change the ranking, so the score is the dot product of the
    code values in a fixed power-of-two unit: x256 (every product is a multiple of
    1/4, so J is an exact integer, a multiple of 64, |J| <= 64 * 6 * 6 * 256 =
    589,824 < 2^20: the same range as the int8 scores)."""
    q = fp4_values(fp4_unpack(q_fp4))
    k = fp4_values(fp4_unpack(k_fp4))
    return np.rint(256.0 * (k @ q)).astype(np.int64)   # exact: quarter-multiples far below 2^53


def csa_query_fp4(q, q_fp4, pos: int, Kc, Vc, k_fp4, c: int, topk: int, scale: float):
    """One CSA query token with the FP4 indexer: FP4 scores -> top-k -> sparse attention."""
    n_vis = n_visible(pos, c, Kc.shape[0])
    scores = index_scores_fp4(q_fp4, k_fp4)
    idx = topk_select(scores, n_vis, topk)
    o, lse, p = attention(q, np.asarray(Kc)[idx], np.asarray(Vc)[idx], scale)
    return {"o": o, "lse": lse, "p": p, "idx": idx, "scores": scores, "n_vis": n_vis}


def topk_select(scores, n_vis: int, k: int) -> np.ndarray:
    """Indices of the top-k visible entries, returned in ascending index order.

    PAGE section 3-2 item 2 (component table): CSA keeps a sparse top-k of the
    compressed entries.  Entries are ranked by score, high first; among equal
    scores the lower index ranks first (the workload's tie rule).  With k >=
    n_vis every visible entry is kept."""
    s = np.asarray(scores, dtype=np.int64)[:n_vis]
    order = np.lexsort((np.arange(n_vis), -s))   # last key is the primary key
    return np.sort(order[: min(k, n_vis)])


def index_scores_rows(q_idx, k_idx) -> np.ndarray:
    """index_scores of many query rows against one key set: [rows, entries].

    The same integers, from one fp64 matrix product: every product is an integer of
    magnitude at most 2^14 and every partial sum at most 2^20, far inside fp64's exact
    integer range (2^53), so the summation order cannot change the result."""
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)
    return np.rint(q @ k.T).astype(np.int64)


def index_scores_fp4_rows(q_fp4, k_fp4) -> np.ndarray:
    """index_scores_fp4 of many query rows: [rows, entries], exactly (products are
    quarter-multiples of magnitude at most 36, sums at most 2304)."""
    q = fp4_values(fp4_unpack(q_fp4))
    k = fp4_values(fp4_unpack(k_fp4))
    return np.rint(256.0 * (q @ k.T)).astype(np.int64)


def topk_select_rows(scores, n_vis, k: int) -> np.ndarray:
    """topk_select of every row of a score matrix: [rows, k] with row r's
    min(k, n_vis[r]) selected indices ascending, then -1.

    The ranking is topk_select's, written as one integer key per entry: rank by
    (score desc, index asc) is rank by (2^21 - score) * N + index ascending (scores
    lie in [-2^20, 2^20], indices below N), with entries at or past n_vis[r] given
    the largest key.  The k smallest keys of a row are that row's selection."""
    s = np.asarray(scores, dtype=np.int64)
    rows, n = s.shape
    if n == 0 or k <= 0:
        return np.full((rows, max(k, 0)), -1, dtype=np.int64)
    nv = np.minimum(np.asarray(n_vis, dtype=np.int64).reshape(rows), n)
    j = np.arange(n, dtype=np.int64)[None, :]
    key = ((1 << 21) - s) * n + j
    key = np.where(j < nv[:, None], key, np.iinfo(np.int64).max)
    kk = min(k, n)
    part = np.argpartition(key, kk - 1, axis=1)[:, :kk] if kk < n else np.tile(j, (rows, 1))
    out = np.full((rows, k), -1, dtype=np.int64)
    for r in range(rows):
        m = int(min(k, nv[r]))
        pick = part[r][np.argsort(key[r, part[r]], kind="stable")][:m]
        out[r, :m] = np.sort(pick)
    return out


# --------------------------------------------------------------------------------------
# attention


def attention(q, K, V, scale: float):
    """Softmax attention of H query heads over n entries (one shared KV head).

    PAGE sections 2-1 and 3-2 item 2: CSA runs sparse attention over the
    selected compressed entries, HCA dense attention over all of them; both are
    ordinary softmax attention over compressed K/V.  logits = scale * q K^T,
    p = softmax(logits) per head, o = p V, lse = log sum exp(logits).

    q: [H, D]; K, V: [n, D].  Returns (o [H, D], lse [H], p [H, n]).  With n = 0
    the output is 0 and lse is -inf."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    h, d = q.shape
    n = K.shape[0]
    if n == 0:
        return np.zeros((h, d)), np.full(h, -np.inf), np.zeros((h, 0))
    logits = scale * (q @ K.T)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    l = w.sum(axis=1, keepdims=True)
    p = w / l
    o = p @ V
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse, p


def csa_query(q, q_idx, pos: int, Kc, Vc, k_idx, c: int, topk: int, scale: float):
    """One CSA query token: indexer scores -> top-k -> sparse attention.

    Kc, Vc: compressed cache values [N, D]; k_idx: indexer keys [N, d_idx]."""
    n_vis = n_visible(pos, c, Kc.shape[0])
    scores = index_scores(q_idx, k_idx)
    idx = topk_select(scores, n_vis, topk)
    o, lse, p = attention(q, np.asarray(Kc)[idx], np.asarray(Vc)[idx], scale)
    return {"o": o, "lse": lse, "p": p, "idx": idx, "scores": scores, "n_vis": n_vis}


def hca_query(q, pos: int, Kc, Vc, m: int, scale: float):
    """One HCA query token: dense attention over every visible entry.

    PAGE section 3-2 item 2 (component table): HCA compresses 128 tokens per
    entry and attends densely, with no selection."""
    n_vis = n_visible(pos, m, Kc.shape[0])
    o, lse, p = attention(q, np.asarray(Kc)[:n_vis], np.asarray(Vc)[:n_vis], scale)
    return {"o": o, "lse": lse, "p": p, "n_vis": n_vis}


# --------------------------------------------------------------------------------------
# sliding-window branch over the state cache


def window_tokens(pos: int, w: int, pos0: int, n_buf: int):
    """Raw tokens the sliding-window branch of a query at position `pos` attends.

    PAGE section 3-2 item 2: CSA and HCA both add a branch that sees the most
    recent tokens uncompressed (window 128 in the config table); section 3-2
    item 4: those tokens, and the tail not yet ready for compression, live in a
    state cache apart from the compressed cache.  Reading: the window is the w
    raw tokens strictly before the query, absolute positions [pos - w, pos) (the
    compressed blocks a query sees also end before it).  The state buffer holds
    the tokens at positions pos0 .. pos0 + n_buf - 1; the window is what of it
    falls in that range.  Returns buffer indices [lo, hi), lo <= hi."""
    lo = max(pos - w, pos0) - pos0
    hi = min(pos, pos0 + n_buf) - pos0
    lo = min(max(lo, 0), n_buf)
    return lo, max(hi, lo)


def attention_union(q, K, V, Kw, Vw, scale: float):
    """Attention over the compressed branch's entries and the window's raw tokens.

    Reading: the window branch adds its keys to the same softmax (one
    distribution over both key sets); the page gives no weights that a separate
    combination of two branches would need.  Plain definition: concatenate the
    two key / value sets and attend."""
    D = np.asarray(q).shape[-1]
    K = np.asarray(K, np.float64).reshape(-1, D)
    V = np.asarray(V, np.float64).reshape(-1, D)
    Kw = np.asarray(Kw, np.float64).reshape(-1, D)
    Vw = np.asarray(Vw, np.float64).reshape(-1, D)
    return attention(q, np.concatenate([K, Kw]), np.concatenate([V, Vw]), scale)


def csa_query_swa(q, q_idx, pos: int, Kc, Vc, k_idx, c: int, topk: int, scale: float,
                  Kw, Vw, pos0: int, w: int):
    """CSA query with the sliding-window branch: the selected compressed entries and
    the window's raw tokens (Kw, Vw: the state buffer starting at position pos0)."""
    n_vis = n_visible(pos, c, Kc.shape[0])
    idx = topk_select(index_scores(q_idx, k_idx), n_vis, topk)
    lo, hi = window_tokens(pos, w, pos0, np.asarray(Kw).shape[0])
    o, lse, p = attention_union(q, np.asarray(Kc)[idx], np.asarray(Vc)[idx],
                                np.asarray(Kw)[lo:hi], np.asarray(Vw)[lo:hi], scale)
    return {"o": o, "lse": lse, "p": p, "idx": idx, "n_vis": n_vis, "window": (lo, hi)}


def hca_query_swa(q, pos: int, Kc, Vc, m: int, scale: float, Kw, Vw, pos0: int, w: int):
    """HCA query with the sliding-window branch: every visible compressed entry and
    the window's raw tokens."""
    n_vis = n_visible(pos, m, Kc.shape[0])
    lo, hi = window_tokens(pos, w, pos0, np.asarray(Kw).shape[0])
    o, lse, p = attention_union(q, np.asarray(Kc)[:n_vis], np.asarray(Vc)[:n_vis],
                                np.asarray(Kw)[lo:hi], np.asarray(Vw)[lo:hi], scale)
    return {"o": o, "lse": lse, "p": p, "n_vis": n_vis, "window": (lo, hi)}


# --------------------------------------------------------------------------------------
# attention sink


def attention_sink(q, K, V, scale: float, sink):
    """Softmax attention with a sink: one more logit per head that takes part in the
    normalisation and carries no value.

    PAGE section 3-2 item 2 lists an attention sink among the parts of the CSA /
    HCA attention without defining it.  Reading: head h has a scalar logit
    sink[h] (natural-log units, like the scaled q.K logits) that joins the
    softmax as an extra key with a zero value row:
        p_j = exp(l_j) / (exp(sink_h) + sum_i exp(l_i)),   o_h = sum_j p_j V_j,
        lse_h = log(exp(sink_h) + sum_i exp(l_i)).
    sink[h] = -inf is plain attention.  Returns (o [H, D], lse [H], p [H, n])."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64).reshape(-1, q.shape[-1])
    V = np.asarray(V, dtype=np.float64).reshape(-1, q.shape[-1])
    z = np.asarray(sink, dtype=np.float64).reshape(-1)
    h, n = q.shape[0], K.shape[0]
    logits = np.concatenate([scale * (q @ K.T), z[:, None]], axis=1)   # the sink is column n
    m = logits.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):   # a head whose every logit is -inf
        w = np.where(np.isneginf(logits), 0.0, np.exp(logits - m))
    l = w.sum(axis=1, keepdims=True)
    p = np.divide(w, l, out=np.zeros_like(w), where=l > 0)
    o = p[:, :n] @ V
    lse = np.where(l[:, 0] > 0, m[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return o, lse, p[:, :n]


def csa_query_sink(q, q_idx, pos: int, Kc, Vc, k_idx, c: int, topk: int, scale: float, sink,
                   Kw=None, Vw=None, pos0: int = 0, w: int = 0):
    """CSA query with a sink, and optionally the sliding-window branch: one softmax
    over the selected entries, the window's raw tokens and the sink."""
    n_vis = n_visible(pos, c, Kc.shape[0])
    idx = topk_select(index_scores(q_idx, k_idx), n_vis, topk)
    D = np.asarray(q).shape[-1]
    lo, hi = (0, 0) if Kw is None else window_tokens(pos, w, pos0, np.asarray(Kw).shape[0])
    Kw_ = np.zeros((0, D)) if Kw is None else np.asarray(Kw, np.float64)[lo:hi]
    Vw_ = np.zeros((0, D)) if Vw is None else np.asarray(Vw, np.float64)[lo:hi]
    o, lse, p = attention_sink(q, np.concatenate([np.asarray(Kc, np.float64)[idx], Kw_]),
                               np.concatenate([np.asarray(Vc, np.float64)[idx], Vw_]), scale, sink)
    return {"o": o, "lse": lse, "p": p, "idx": idx, "n_vis": n_vis, "window": (lo, hi)}


def hca_query_sink(q, pos: int, Kc, Vc, m: int, scale: float, sink, Kw=None, Vw=None,
                   pos0: int = 0, w: int = 0):
    """HCA query with a sink, and optionally the sliding-window branch."""
    n_vis = n_visible(pos, m, Kc.shape[0])
    D = np.asarray(q).shape[-1]
    lo, hi = (0, 0) if Kw is None else window_tokens(pos, w, pos0, np.asarray(Kw).shape[0])
    Kw_ = np.zeros((0, D)) if Kw is None else np.asarray(Kw, np.float64)[lo:hi]
    Vw_ = np.zeros((0, D)) if Vw is None else np.asarray(Vw, np.float64)[lo:hi]
    o, lse, p = attention_sink(q, np.concatenate([np.asarray(Kc, np.float64)[:n_vis], Kw_]),
                               np.concatenate([np.asarray(Vc, np.float64)[:n_vis], Vw_]), scale,
                               sink)
    return {"o": o, "lse": lse, "p": p, "n_vis": n_vis, "window": (lo, hi)}


# --------------------------------------------------------------------------------------
# composed steps


def csa_decode(q, q_idx, ctx_len: int, Kc, Vc, k_idx, c: int, topk: int, scale: float):
    """Decode: the new token sits at position ctx_len and sees all floor(L/c) entries."""
    return csa_query(q, q_idx, ctx_len, Kc, Vc, k_idx, c, topk, scale)


def hca_decode(q, ctx_len: int, Kc, Vc, m: int, scale: float):
    return hca_query(q, ctx_len, Kc, Vc, m, scale)


def hybrid_decode(layers, ctx_len: int, scale: float):
    """A stack of independent layers, CSA on even layers and HCA on odd ones.

    PAGE section 3-2 item 2: CSA and HCA layers are interleaved.  The page
    gives no projections, so layers do not feed one another here: each layer
    attends its own cache with its own query.  `layers` is a list of dicts with
    keys q, Kc, Vc and, for CSA layers, q_idx, k_idx, c, topk; HCA layers carry m."""
    out = []
    for li, L in enumerate(layers):
        if li % 2 == 0:
            out.append(csa_decode(L["q"], L["q_idx"], ctx_len, L["Kc"], L["Vc"], L["k_idx"],
                                  L["c"], L["topk"], scale))
        else:
            out.append(hca_decode(L["q"], ctx_len, L["Kc"], L["Vc"], L["m"], scale))
    return out


def csa_prefill(q, q_idx, ctx_len: int, Kc_ctx, Vc_ctx, new_k, new_v, k_idx, c: int,
                topk: int, scale: float, rows=None):
    """Chunked prefill: compress the new tokens, append them, then run every new query.

    New token i sits at position ctx_len + i.  The new raw tokens are mean-pooled
    into floor(T_new / c) entries appended after the context entries (ctx_len
    must be a multiple of c so that no block straddles the two).  Each query
    then runs `csa_query` under the block visibility rule.  `rows` restricts the
    queries evaluated (a sample); the appended entries are always returned.

    Returns (new_entries_k_bits, new_entries_v_bits, per-query results)."""
    assert ctx_len % c == 0
    nk = compress_to_cache(new_k, c)
    nv = compress_to_cache(new_v, c)
    Kc = np.concatenate([np.asarray(Kc_ctx, np.float64), bf16_bits_to_f64(nk)], axis=0)
    Vc = np.concatenate([np.asarray(Vc_ctx, np.float64), bf16_bits_to_f64(nv)], axis=0)
    t = np.asarray(q).shape[0]
    rows = range(t) if rows is None else rows
    res = {int(i): csa_query(q[i], q_idx[i], ctx_len + int(i), Kc, Vc, k_idx, c, topk, scale)
           for i in rows}
    return nk, nv, res
