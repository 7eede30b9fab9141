"""Plain fp64 CPU oracle for Multi-head Latent Attention (MLA) decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
never imports, links or calls it, and it imports nothing from the GPU library:
it depends on numpy alone.

What it computes is the *unabsorbed* definition: it rebuilds every head's key
and value from the cached latent with the up-projections and runs textbook
softmax attention.  The absorbed form used by the GPU path is algebraically the
same computation (the katajob interview page, section "Why it is not just extra
work at decode time", states the up-projections fold into the query and output
sides exactly), so the plain definition is the reference for it.

Notation (rows are vectors, weights stored [in, out], as in the numpy snippet on
the katajob page, section "code", and the torch pseudo-code on the bembew
article, section "Implementation Logic"):

* c_t = h_t W_down                     latent of token t, the only cached content
* k_R,t = RoPE(h_t W_KR, t)            decoupled positional key, one per token
* K^C[t, i] = c_t W_UK[:, i*d_h:(i+1)*d_h]   per-head content key (head-major columns)
* V[t, i]   = c_t W_UV[:, i*d_v:(i+1)*d_v]   per-head value
* key of head i = [K^C[t, i] ; k_R,t]  (concatenation)
* query of head i at position p = [q^C_i ; RoPE(q^R_i, p)]
* s[t, i] = (query_i . key_i,t) * softmax_scale, t <= p
* o_i = sum_t softmax_t(s[:, i]) V[t, i]

Readings of points the pages leave open (each also listed in the design notes):

1. The page allows either joining or summing the content and positional key (bembew, "Implementation
   Logic", step 5): read as concatenation, so the two dot products add.
2. k_R is one vector per token shared by all heads (bembew "Decoupling RoPE",
   talentme "Core Definition", and the podcast, which caches the latent next to one
   small positional part); q^R is per head (zenaique follow-up question
   "Why does MLA need a decoupled RoPE key").
3. RoPE is not defined on the pages (bembew calls ``apply_rope`` without a body):
   textbook rotary embedding with interleaved pairs (2j, 2j+1) rotated by
   pos * base^(-2j/d_R).  The pairing convention is parity unpinned.
4. Query j of an Sq-token step of a sequence with kv_len tokens sits at
   p = kv_len - Sq + j and attends to tokens t <= p.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------- RoPE

def rope(v: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``v`` by pos * base^(-2j/d).

    Position enters only through this rotation, and only the positional parts
    (k_R, q^R) are rotated: the bembew article, "Decoupling RoPE from
    Compression"; the katajob page, last sentences of "Why it is not just extra
    work at decode time".  ``pos`` broadcasts against ``v.shape[:-1]``.
    """
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    assert d % 2 == 0
    j = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


# ------------------------------------------------------------- projections (tiny case)

def project_from_hidden(x, W_down, W_KR, W_Q, W_QR, heads, d_h, d_r, query_rows):
    """Latent, raw positional key and the two query parts from hidden states x [L, d_model].

    c = x W_down is the down-projection (katajob "The mechanism", and the
    numpy snippet ``latent = x @ W_down``); k_R raw = x W_KR is the separate
    positional projection (bembew "Implementation Logic", step 3).  The query
    parts are reshaped head-major, as the snippet reshapes keys to
    (seq, n_heads, d_head).
    """
    x = np.asarray(x, dtype=np.float64)
    C = x @ np.asarray(W_down, dtype=np.float64)
    KR = x @ np.asarray(W_KR, dtype=np.float64)
    xq = x[np.asarray(query_rows)]
    qC = (xq @ np.asarray(W_Q, dtype=np.float64)).reshape(len(query_rows), heads, d_h)
    qR = (xq @ np.asarray(W_QR, dtype=np.float64)).reshape(len(query_rows), heads, d_r)
    return C, KR, qC, qR


# ------------------------------------------------------------ reconstruction

def up_project(C: np.ndarray, W: np.ndarray, heads: int, d_head: int) -> np.ndarray:
    """Per-head keys or values rebuilt from the latent: (C W).reshape(L, heads, d_head).

    katajob "code": ``keys = (latent @ W_up_k).reshape(seq, n_heads, d_head)``;
    bembew "Low-Rank Decomposition and Latent Vectors" (K = W c, V = W c).
    """
    C = np.asarray(C, dtype=np.float64)
    return (C @ np.asarray(W, dtype=np.float64)).reshape(C.shape[0], heads, d_head)


# ------------------------------------------------------------------ attention

def decode(C, KRraw, qC, qR, W_UK, W_UV, kv_len, softmax_scale, rope_base=10000.0,
           heads=None, chunk=2048, keys_rotated=False):
    """Textbook softmax attention for the Sq queries of one sequence, unabsorbed.

    Inputs (fp64 after upcast):
      C      [L, d_c]      cached latents (L >= kv_len rows; only the first kv_len are used)
      KRraw  [L, d_R]      positional keys before RoPE (token t is rotated at position t);
                           with keys_rotated=True they are taken as already rotated, as the
                           cache stores them (RoPE applied when the token is written): this
                           serves attention over rows read back from a cache, e.g. the
                           dequantised rows of an fp8 cache
      qC     [Sq, H, d_h]  content queries;   qR [Sq, H, d_R] positional queries before RoPE
      W_UK   [d_c, H*d_h]  W_UV [d_c, H*d_v]  head-major up-projections
      heads  optional list of head indices to evaluate (default: all)

    Returns dict with
      o      [Sq, h, d_v]  sum_t w[t] V[t, i]                       (the layer output per head)
      o_lat  [Sq, h, d_c]  sum_t w[t] c_t                           (latent-space output)
      lse    [Sq, h]       log sum_t exp(s[t])                      (natural log)

    Two passes over the tokens in chunks of ``chunk`` rows (memory only, no
    change to the arithmetic): pass 1 rebuilds K^C and forms every score, the
    softmax is taken over all of them at once, pass 2 rebuilds V and sums.
    """
    C = np.asarray(C, dtype=np.float64)
    KRraw = np.asarray(KRraw, dtype=np.float64)
    qC = np.asarray(qC, dtype=np.float64)
    qR = np.asarray(qR, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    Sq, H, d_h = qC.shape
    d_r = qR.shape[-1]
    d_c = C.shape[1]
    d_v = W_UV.shape[1] // H
    L = int(kv_len)
    assert 1 <= Sq <= L <= C.shape[0]
    hs = np.arange(H) if heads is None else np.asarray(heads)
    nh = len(hs)
    # Column blocks of the selected heads (head-major: head i owns columns i*d .. i*d+d-1).
    cols_k = (hs[:, None] * d_h + np.arange(d_h)[None, :]).reshape(-1)
    cols_v = (hs[:, None] * d_v + np.arange(d_v)[None, :]).reshape(-1)
    Wk = W_UK[:, cols_k]
    Wv = W_UV[:, cols_v]

    pos_q = L - Sq + np.arange(Sq)                       # reading 4
    kR = KRraw[:L] if keys_rotated else rope(KRraw[:L], np.arange(L), rope_base)   # [L, d_R]
    qRr = rope(qR[:, hs], pos_q[:, None], rope_base)     # [Sq, nh, d_R]
    qCs = qC[:, hs]                                      # [Sq, nh, d_h]

    # pass 1: scores s[j, t, i]
    s = np.empty((Sq, L, nh))
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        KC = up_project(C[t0:t1], Wk, nh, d_h)           # [n, nh, d_h]
        content = np.einsum("jid,tid->jti", qCs, KC)
        positional = np.einsum("jir,tr->jti", qRr, kR[t0:t1])
        s[:, t0:t1, :] = (content + positional) * softmax_scale
    # causal visibility: query j sees t <= pos_q[j]
    t_idx = np.arange(L)
    visible = t_idx[None, :] <= pos_q[:, None]           # [Sq, L]
    s = np.where(visible[:, :, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    w = e / den                                          # [Sq, L, nh]
    lse = (m + np.log(den))[:, 0, :]

    # pass 2: weighted sums of values and of latents
    o = np.zeros((Sq, nh, d_v))
    o_lat = np.zeros((Sq, nh, d_c))
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        V = up_project(C[t0:t1], Wv, nh, d_v)            # [n, nh, d_v]
        o += np.einsum("jti,tiv->jiv", w[:, t0:t1], V)
        o_lat += np.einsum("jti,tc->jic", w[:, t0:t1], C[t0:t1])
    return {"o": o, "o_lat": o_lat, "lse": lse}


def absorbed_query(qC, qR, W_UK, q_pos, rope_base=10000.0):
    """[q^C_i W_UK,i^T ; RoPE(q^R_i, p)] for each query row and head: shape [Sq, H, d_c + d_R].

    The key up-projection folded into the query side (katajob "solid answer"
    and "Why it is not just extra work at decode time"; zenaique "Concept
    explanation": reconstruction fused into the attention matmuls).  With
    k^C = c W_UK,i, the content score q^C . k^C equals (q^C W_UK,i^T) . c.
    """
    qC = np.asarray(qC, dtype=np.float64)
    qR = np.asarray(qR, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    Sq, H, d_h = qC.shape
    d_c = W_UK.shape[0]
    Wk = W_UK.reshape(d_c, H, d_h)                       # [d_c, H, d_h]
    q_lat = np.einsum("jid,cid->jic", qC, Wk)
    q_rot = rope(qR, np.asarray(q_pos)[:, None], rope_base)
    return np.concatenate([q_lat, q_rot], axis=-1)


def decode_absorbed(C, KRraw, qC, qR, W_UK, W_UV, kv_len, softmax_scale, rope_base=10000.0):
    """The absorbed form in fp64: attention against [c ; k_R] with the folded query,
    latent-space weighted sum, then W_UV applied once per query.

    Used only to pin the oracle (absorbed == unabsorbed, an algebraic identity,
    katajob "Why it is not just extra work at decode time").
    """
    C = np.asarray(C, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    Sq, H, _ = np.shape(qC)
    d_c = C.shape[1]
    d_v = W_UV.shape[1] // H
    L = int(kv_len)
    pos_q = L - Sq + np.arange(Sq)
    qa = absorbed_query(qC, qR, W_UK, pos_q, rope_base)                  # [Sq, H, d_c+d_R]
    rows = np.concatenate([C[:L], rope(KRraw[:L], np.arange(L), rope_base)], axis=1)
    s = np.einsum("jir,tr->jti", qa, rows) * softmax_scale
    visible = np.arange(L)[None, :] <= pos_q[:, None]
    s = np.where(visible[:, :, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    w = e / den
    o_lat = np.einsum("jti,tc->jic", w, C[:L])
    o = np.einsum("jic,civ->jiv", o_lat, W_UV.reshape(d_c, H, d_v))
    return {"o": o, "o_lat": o_lat, "lse": (m + np.log(den))[:, 0, :]}


def out_project(o_lat, W_UV):
    """o_i = o_lat_i W_UV,i for each query row and head: the value up-projection applied once
    per query on the output side (katajob "solid answer")."""
    o_lat = np.asarray(o_lat, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    Sq, H, d_c = o_lat.shape
    return np.einsum("jic,civ->jiv", o_lat, W_UV.reshape(d_c, H, -1))


def model_output(o, W_O):
    """The layer's output in the model width: the heads' values concatenated head-major and
    projected by W_O [H*d_v, d_model], out = concat_i(o_i) W_O = sum_i o_i W_O[i*d_v:(i+1)*d_v].
    The output projection the value up-projection folds into (katajob "solid answer")."""
    o = np.asarray(o, dtype=np.float64)
    Sq, H, d_v = o.shape
    return o.reshape(Sq, H * d_v) @ np.asarray(W_O, dtype=np.float64)


def fold_output_weights(W_UV, W_O, heads):
    """W_O'_i = W_UV,i W_O,i  [d_c, d_model] for every head i, stacked [H, d_c, d_model]: with it
    the output is sum_i o_lat_i W_O'_i, the value up-projection folded into the output projection
    (katajob "solid answer"), straight from the latent-space output."""
    W_UV = np.asarray(W_UV, dtype=np.float64)
    W_O = np.asarray(W_O, dtype=np.float64)
    d_c = W_UV.shape[0]
    d_v = W_UV.shape[1] // heads
    return np.stack([W_UV[:, i * d_v:(i + 1) * d_v] @ W_O[i * d_v:(i + 1) * d_v] for i in range(heads)])


def attention(q, K, V, softmax_scale):
    """Textbook softmax attention of one query row per head over a per-head key/value cache, the
    cache MLA replaces (zenaique "What MLA caches versus what MHA and GQA cache": every head keeps
    its own key and value per token; grouped-query attention shares one key/value head among a
    group of query heads).

      q [Hq, d]   K [L, Hkv, d]   V [L, Hkv, dv]   query head i reads key/value head i // (Hq/Hkv)
    Returns o [Hq, dv] and lse [Hq] (natural log); L = 0 gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq = q.shape[0]
    L, Hkv = K.shape[0], K.shape[1]
    group = Hq // Hkv
    kv = np.arange(Hq) // group
    if L == 0:
        return {"o": np.zeros((Hq, V.shape[-1])), "lse": np.full(Hq, -np.inf)}
    s = np.einsum("id,tid->it", q, K[:, kv]) * softmax_scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    o = np.einsum("it,tid->id", e / den, V[:, kv])
    return {"o": o, "lse": (m + np.log(den))[:, 0]}


# --------------------------------------------------------------- fp8 e4m3 storage

def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3fn value (ties to even, saturating at +-448), as float64.

    e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities;
    normals 2^-6 .. 448, subnormals multiples of 2^-9.  Storing the latent at
    lower precision composes with MLA (katajob, section "Compression as
    architecture versus compression as post-processing").
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # exponent of the binade (a = m * 2^ex with m in [0.5, 1) -> floor(log2 a) = ex - 1),
    # clamped to the subnormal range
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)
    step = np.exp2(e - 3.0)                          # spacing of representable values
    q = np.round(a / step) * step                     # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    return np.sign(x) * q


def quantize_rows_fp8(rows: np.ndarray):
    """Per-token fp8 storage: scale = amax(row)/448 (1.0 for an all-zero row), codes = e4m3(row/scale).

    Returns (codes as float64 values, scales float32) so that row ~= codes * scale.
    The stored scale is a float32 quantity, and the code of each value is decided in that
    precision: the row is taken in fp32 (a bf16 latent exactly, a rotated positional key
    rounded once), the scale is fp32(amax) / 448 in fp32 and the quotient value / scale is
    an fp32 division, which e4m3_round then rounds exactly to the nearest code.
    """
    rows = np.asarray(rows, dtype=np.float64).astype(np.float32)
    amax = np.abs(rows).max(axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (rows / scale[..., None]).astype(np.float32)
    codes = e4m3_round(quot.astype(np.float64))
    return codes, scale


# ------------------------------------------------- block-scaled fp8 e4m3 storage
#
# The katajob page (section "Compression as architecture versus compression as post-processing")
# counts per-block scales among what a quantised cache depends on, and has a low-precision latent
# compose with MLA.  The block-scaled format reads that as: the cache rows of
# a page are cut into tiles of 32 tokens x 32 columns, each tile has one power-of-two scale
# 2^e, and each value is stored as the e4m3 code of value / 2^e.  Tokens arrive one call at a
# time, so a tile's scale is decided by the rows it holds so far: a call takes, for each tile it
# writes, e = the largest exponent any of the tile's rows needs (its earlier rows' exponent
# included, unless the call writes the tile's first row), re-encodes the earlier rows' codes at
# the new scale when e grew, and encodes its own rows at e.

TILE_TOKENS = 32
TILE_COLS = 32
BLOCK_E_MIN, BLOCK_E_MAX = -126, 127


def block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (the tile's largest magnitude then encodes without
    saturating), clamped to [-126, 127]; -126 for amax == 0.  Exact: amax = m 2^x with m in
    [0.5, 1) lies in [2^(x-1), 2^x), and 448 2^(x-9) = 0.875 2^x, so e is x - 9 or x - 8."""
    a = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    e = x.astype(np.int64) - 9
    e = np.where(a > E4M3_MAX * np.exp2(e.astype(np.float64)), e + 1, e)
    e = np.where(a > 0, e, BLOCK_E_MIN)
    return np.clip(e, BLOCK_E_MIN, BLOCK_E_MAX).astype(np.int64)


def append_block_fp8(codes: np.ndarray, exps: np.ndarray, rows: np.ndarray, p0: int) -> None:
    """One append call of a sequence into its block-scaled cache, in place.

    codes [capacity, row] float64: the code values (e4m3 values) of every position; exps
    [capacity / 32, row / 32] int: the tile exponents.  rows [n, row]: the new rows at positions
    p0 .. p0 + n - 1 (the latent exactly and the rotated positional key, both as the fp32
    values the cache is written from).  Positions before p0 must already be in the cache."""
    rows = np.asarray(rows, dtype=np.float64).astype(np.float32).astype(np.float64)
    n, width = rows.shape
    nb = width // TILE_COLS
    p1 = p0 + n
    for k in range(p0 // TILE_TOKENS, (p1 - 1) // TILE_TOKENS + 1 if n > 0 else 0):
        t0, t1 = k * TILE_TOKENS, (k + 1) * TILE_TOKENS
        a, b = max(t0, p0), min(t1, p1)                     # new rows of this tile
        new = rows[a - p0:b - p0].reshape(b - a, nb, TILE_COLS)
        e_new = block_exponent(np.abs(new).max(axis=(0, 2)))   # [nb]
        fresh = a == t0
        if not fresh:                                       # rows t0 .. a-1 were written earlier
            e_old = exps[k].astype(np.int64)
            e_new = np.maximum(e_new, e_old)
            old = codes[t0:a].reshape(a - t0, nb, TILE_COLS)
            shift = np.exp2((e_old - e_new).astype(np.float64))[None, :, None]
            codes[t0:a] = e4m3_round(old * shift).reshape(a - t0, width)
        codes[a:b] = e4m3_round(new * np.exp2(-e_new.astype(np.float64))[None, :, None]).reshape(b - a, width)
        exps[k] = e_new


def dequantize_block_fp8(codes: np.ndarray, exps: np.ndarray, L: int) -> np.ndarray:
    """Row values of positions 0 .. L-1: code * 2^e of the tile (token / 32, column / 32)."""
    t = np.arange(L)
    e = exps[t // TILE_TOKENS]                                   # [L, nb]
    scale = np.repeat(np.exp2(e.astype(np.float64)), TILE_COLS, axis=1)
    return codes[:L] * scale


# -------------------------------------------------------------- closed forms

def mha_cache_elements_per_token(heads: int, d_head: int) -> int:
    """Keys and values for every head: 2 * H * d (zenaique "What MLA caches versus what MHA and
    GQA cache"; talentme "Key Problems Solved": 2 H d values per token)."""
    return 2 * heads * d_head


def mla_cache_elements_per_token(d_c: int, d_r: int) -> int:
    """The latent plus the decoupled positional key (the podcast: both, and nothing else, are
    cached per token)."""
    return d_c + d_r


def gqa_cache_bytes_per_token(layers: int, kv_heads: int, d_head: int, bytes_per_value: int) -> int:
    """layers * kv_heads * d_head * 2 (K and V) * bytes (the podcast's illustrative sizing)."""
    return layers * kv_heads * d_head * 2 * bytes_per_value
