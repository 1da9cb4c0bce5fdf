"""Plain float64 CPU oracle of Multi-head Latent Attention over a latent cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP library: it has its own bf16 decoding and rounding, its
own RoPE, its own page addressing and its own softmax.  It is deliberately
slow and obvious: per-head K and V are materialised from the latent exactly as
the non-absorbed description reads, and every step is a plain NumPy
expression.

Sources (the pages carry no code; each function names the passage it follows):
  [blog]  yapayzekasozluk.tr, "Multi-head Latent Attention (MLA) Nedir?"
          sections "MLA nasil calisir?" (compression, decompression,
          decoupled RoPE) and "MLA'nin avantajlari ve hesap maliyeti".
  [scale] LLMScale, "GQA, MQA ve MLA: attention KV cache'i nasil belirler",
          sections "Multi-head attention (MHA)", "Grouped-query attention
          (GQA)", "Multi-head latent attention (MLA)".
  [arch]  openarchlab, "MLA - latent KV, decoupled RoPE va matrix
          absorption", sections 1 (definition), 2 (flow), 3 (solution:
          cache formulas), 4 (profiling), 5 (examples), 6 (terms).

Readings where the pages leave a step open (all pinned by tests/test_oracle_*):
  * RoPE (named, not written out, in [blog] "Decoupled RoPE" and [arch] 1):
    the rotary embedding of RoFormer with adjacent pairs (2i, 2i+1),
    theta_i = base^(-2i/d), position p as a float64 angle p*theta_i.
  * One rotary key k_R per token, shared by all heads ([scale] MLA: the head
    count drops out of the per-token cache size); one rotary query part q_R
    per head.
  * V is up-projected from the content latent c only ([arch] 1: only the
    position branch is kept apart from the latent).
  * Score of head h against token t:  sigma * (q_C,h . K_C,h,t + q_R,h . k_R,t),
    softmax over t, natural-log LSE.  sigma is an input.
  * Decode: the query sits at position seq_len-1 and sees all seq_len rows,
    including its own row written in the same step ([arch] 2: project, then
    write, then read).
  * Prefill: query i of a fresh sequence sees rows t <= i.
  * 8-bit cache rows ([blog] "MLA ve diger optimizasyonlarla iliskisi"
    allows 8-bit storage of the cached vector; [arch] 3 mentions its scales):
    E4M3 codes of the bf16 row over one power-of-two scale per row, nearest
    code with ties to even; see the section "8-bit cache rows" below.
  * Query compression and output projection ([blog] "MLA nasil calisir?",
    [arch] 1): c_Q = W_DQ h, per head [q_C | q_R] = W_UQ,h c_Q, and
    y = W_O [o_1 | ... | o_H]; see the section at the end of this file.
  * Prefill onto a cached prefix (the pages ask for prefill to be measured
    under real serving shapes, [arch] 4; they do not spell out chunking): the
    new tokens of a sequence follow ``prefix`` tokens already in the cache;
    new query i sits at position prefix + i and sees rows t <= prefix + i.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------


def from_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored values to float64.  bf16 arrives as raw uint16 patterns:
    the value is the float32 whose upper 16 bits are the pattern."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 value (8 significant bits), ties to even.

    Single rounding straight from float64: scale each value by a power of two
    so its 8 significant bits sit left of the binary point, round half-even,
    scale back (both scalings are exact)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# cache-size formulas ([scale] MHA / GQA / MLA; [arch] 3 and 5)
# --------------------------------------------------------------------------


def mla_cache_bytes_per_token(layers: int, d_c: int, d_r: int, elem_bytes: int) -> int:
    """Per-token MLA cache: layers x (latent width + rotary key width) x bytes.
    The head count does not enter ([scale] MLA; [arch] 3)."""
    return layers * (d_c + d_r) * elem_bytes


def mla_cache_bytes(layers: int, tokens: int, d_c: int, d_r: int, elem_bytes: int) -> int:
    """Ideal MLA cache of one sequence: L x T x (d_c + d_R) x b ([arch] 3)."""
    return tokens * mla_cache_bytes_per_token(layers, d_c, d_r, elem_bytes)


def gqa_cache_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Uniform GQA: 2 x L x H_KV x d_h x b per token ([arch] 3).  With
    kv_heads equal to the query heads this is the MHA formula ([scale] MHA)."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def gqa_equivalent_groups(d_c: int, d_r: int, head_dim: int) -> float:
    """Number of K/V head pairs whose cache equals one MLA latent row."""
    return (d_c + d_r) / (2.0 * head_dim)


# --------------------------------------------------------------------------
# rotary embedding ([blog] "Decoupled RoPE"; [arch] 1 and 6)
# --------------------------------------------------------------------------


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate adjacent pairs (x_2i, x_2i+1) of the last axis by angle pos*theta_i,
    theta_i = base^(-2i/d).  ``pos`` broadcasts against x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    p = np.asarray(pos, dtype=np.float64)
    p = np.broadcast_to(p, x.shape[:-1])
    ang = p[..., None] * theta
    cs, sn = np.cos(ang), np.sin(ang)
    ev, od = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = ev * cs - od * sn
    out[..., 1::2] = ev * sn + od * cs
    return out


# --------------------------------------------------------------------------
# step 1: project the hidden state to the cached row ([arch] 2 step 1;
#         [blog] compression + decoupled RoPE)
# --------------------------------------------------------------------------


def latent_rows(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray, positions, base: float) -> np.ndarray:
    """row_n = [c_KV,n | k_R,n] with c_KV,n = W_DKV h_n and
    k_R,n = RoPE(W_KR h_n, p_n).  float64, unrounded.  Shapes: h [N, D],
    w_dkv [d_c, D], w_kr [d_R, D] -> [N, d_c + d_R]."""
    c = h @ w_dkv.T
    kr = rope(h @ w_kr.T, np.asarray(positions), base)
    return np.concatenate([c, kr], axis=-1)


# --------------------------------------------------------------------------
# step 2: write the cache in the engine's layout ([arch] 2 step 2;
#         paged cache: [blog] "MLA ve diger optimizasyonlarla iliskisi")
# --------------------------------------------------------------------------


def scatter_rows(pool: np.ndarray, rows: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Return a copy of ``pool`` [num_pages, P, R] with row n stored at slot
    slots[n] (page slots[n] // P, offset slots[n] % P); slot -1 is skipped."""
    out = np.array(pool, copy=True)
    P = out.shape[1]
    for n, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        out[s // P, s % P, :] = rows[n]
    return out


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Rows 0..length-1 of one sequence: token t lives in page
    block_table_row[t // P] at offset t % P."""
    P = pool.shape[1]
    out = np.empty((length, pool.shape[2]), dtype=pool.dtype)
    for t in range(length):
        out[t] = pool[int(block_table_row[t // P]), t % P]
    return out


# --------------------------------------------------------------------------
# 8-bit cache rows ([blog] "MLA ve diger optimizasyonlarla iliskisi": the
# cached vector may be stored with 8 bits per value, MLA and quantization
# combine; [arch] 3: the cache formula leaves out the quantization scales)
#
# Readings (the pages name neither format nor scale granularity):
#   * 8-bit values are E4M3 floats: sign, 4 exponent bits (bias 7), 3 mantissa
#     bits; exponent field 0 holds the subnormals m * 2^-9; code S.1111.111 is
#     NaN and the largest finite magnitude is 448 (S.1111.110).  There is no
#     infinity.
#   * One scale per cached row (token), a power of two 2^e: the smallest e
#     with amax <= 448 * 2^e, where amax is the largest magnitude of the
#     row, and e >= -126; an all-zero row takes e = 0.
#   * The row is first rounded to bf16 (the values a bf16 cache would hold),
#     then every value x becomes the E4M3 code nearest to x / 2^e, ties to
#     the even code; a result of -0 is stored as +0 (code 0).
#   * Stored value = E4M3 value of the code times 2^e.
#   * Page layout: the P rows of R codes, then P float32 scales (little
#     endian), so a page holds P * (R + 4) bytes.
# --------------------------------------------------------------------------


def e4m3_value(code) -> np.ndarray:
    """Float64 value of E4M3 codes (NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def quantize_e4m3(x) -> np.ndarray:
    """E4M3 code of each value of x (float64, |x| <= 448): the nearest finite
    code, ties to the code with an even mantissa; zero results get code 0.

    Written from the format: below 2^-6 the grid is the multiples of 2^-9;
    above, a binade [2^k, 2^(k+1)) holds 8 values spaced 2^(k-3).  The value
    is scaled so that the grid spacing becomes 1, rounded half-even to an
    integer, and re-encoded."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.abs(x) <= 448.0), "value outside the E4M3 range"
    a = np.abs(x)
    _, k = np.frexp(a)                       # a = f 2^k, 0.5 <= f < 1  (k = floor(log2 a) + 1)
    k = np.where(a > 0, k - 1, -10)          # floor(log2 a)
    k = np.maximum(k, -6)                    # subnormal range shares the 2^-6 binade spacing
    step = np.exp2(k - 3.0)                  # grid spacing in this binade
    n = np.round(a / step)                   # half-even integer count of steps (exact division)
    # n = 16 means the value rounded up into the next binade
    up = n >= 16
    k = np.where(up, k + 1, k)
    n = np.where(up, n / 2, n)
    sub = (k == -6) & (n < 8)                # subnormal: exponent field 0, mantissa n
    ef = np.where(sub, 0, k + 7)
    mf = np.where(sub, n, n - 8)
    code = (ef.astype(np.int64) << 3) | mf.astype(np.int64)
    code = np.where(np.signbit(x) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def row_scale_exponent(amax: float) -> int:
    """Smallest e >= -126 with amax <= 448 * 2^e (0 for amax = 0)."""
    if amax == 0.0:
        return 0
    e = -126
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return e


def quantize_row_fp8(row) -> Tuple[np.ndarray, float]:
    """One cached row -> (R codes, scale 2^e).  The row is rounded to bf16
    first; the scale comes from the bf16 row's largest magnitude."""
    r = round_bf16(np.asarray(row, dtype=np.float64))
    e = row_scale_exponent(float(np.max(np.abs(r))) if r.size else 0.0)
    return quantize_e4m3(r / 2.0 ** e), 2.0 ** e


def dequantize_rows_fp8(codes, scales) -> np.ndarray:
    """Stored values: E4M3 value of each code times its row's scale."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def pack_fp8_pages(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [num_pages, P, R] uint8 and scales [num_pages, P] -> page bytes
    [num_pages, P * (R + 4)]: the P rows, then the P float32 scales."""
    npg, P, R = codes.shape
    out = np.empty((npg, P * (R + 4)), dtype=np.uint8)
    out[:, :P * R] = codes.reshape(npg, P * R)
    out[:, P * R:] = np.asarray(scales, dtype="<f4").reshape(npg, P).view(np.uint8).reshape(npg, 4 * P)
    return out


def unpack_fp8_pages(pages: np.ndarray, P: int, R: int) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse of pack_fp8_pages: (codes [num_pages, P, R], scales [num_pages, P] float64)."""
    pages = np.asarray(pages, dtype=np.uint8)
    npg = pages.shape[0]
    codes = pages[:, :P * R].reshape(npg, P, R)
    scales = np.ascontiguousarray(pages[:, P * R:P * (R + 4)]).view("<f4").reshape(npg, P).astype(np.float64)
    return codes, scales


def write_rows_fp8(pages: np.ndarray, rows: np.ndarray, slots, P: int) -> np.ndarray:
    """Quantize each row and store codes and scale at its slot of the page
    bytes (a copy is returned; slot -1 is skipped)."""
    R = rows.shape[1]
    codes, scales = unpack_fp8_pages(pages, P, R)
    codes, scales = codes.copy(), scales.copy()
    for n, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        codes[s // P, s % P], scales[s // P, s % P] = quantize_row_fp8(rows[n])
    return pack_fp8_pages(codes, scales)


def fp8_pool_values(pages: np.ndarray, P: int, R: int) -> np.ndarray:
    """Float64 pool [num_pages, P, R] of the stored values of page bytes; the
    decode and prefill functions below read it like any other pool."""
    codes, scales = unpack_fp8_pages(pages, P, R)
    return dequantize_rows_fp8(codes, scales)


# --------------------------------------------------------------------------
# step 3: read -- the plain, non-absorbed form ([blog] decompression:
#         K and V are regenerated from c_KV per head)
# --------------------------------------------------------------------------


def _attend(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """Softmax over the last axis of ``scores`` [T], weighted sum of
    ``values`` [T, d]; returns (output [d], natural-log LSE)."""
    m = float(np.max(scores))
    w = np.exp(scores - m)
    l = float(np.sum(w))
    return (w @ values) / l, m + math.log(l)


def decode_one(q: np.ndarray, rows: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
               q_pos: int, d_c: int, sigma: float, base: float,
               heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One decode query of one sequence, every head, non-absorbed.

    q    [H, d_n + d_R]  pre-RoPE query per head ([q_C | q_R])
    rows [T, d_c + d_R]  the sequence's cached rows, float64
    w_uk [H, d_n, d_c], w_uv [H, d_v, d_c]
    Returns o [H, d_v], lse [H] (only ``heads`` filled if given, others NaN).
    """
    H, dq = q.shape
    d_n = w_uk.shape[1]
    d_v = w_uv.shape[1]
    C = rows[:, :d_c]
    KR = rows[:, d_c:]
    o = np.full((H, d_v), np.nan)
    lse = np.full(H, np.nan)
    if rows.shape[0] == 0:
        o[:] = 0.0
        lse[:] = -np.inf
        return o, lse
    for h in (range(H) if heads is None else heads):
        q_c = q[h, :d_n]
        q_r = rope(q[h, d_n:], q_pos, base)
        K_c = C @ w_uk[h].T            # [T, d_n]   K_C,h,t = W_UK,h c_t
        V = C @ w_uv[h].T              # [T, d_v]   V_h,t   = W_UV,h c_t
        s = sigma * (K_c @ q_c + KR @ q_r)
        o[h], lse[h] = _attend(s, V)
    return o, lse


def decode(q: np.ndarray, pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
           w_uk: np.ndarray, w_uv: np.ndarray, d_c: int, sigma: float, base: float,
           seqs: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None):
    """Batched decode: sequence b's query q[b] at position seq_lens[b]-1 over
    its seq_lens[b] cached rows.  Returns o [B, H, d_v], lse [B, H] (NaN for
    sequences not in ``seqs``)."""
    B, H, _ = q.shape
    d_v = w_uv.shape[1]
    o = np.full((B, H, d_v), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        rows = gather_rows(pool, block_table[b], L)
        o[b], lse[b] = decode_one(q[b], rows, w_uk, w_uv, L - 1, d_c, sigma, base, heads)
    return o, lse


def prefill_one(q: np.ndarray, rows: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                d_c: int, sigma: float, base: float,
                queries: Optional[Sequence[int]] = None,
                heads: Optional[Sequence[int]] = None,
                prefix: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Causal prefill of the T new tokens of one sequence that follow
    ``prefix`` cached tokens (0: a fresh sequence): new query i sits at
    position prefix + i and sees rows t <= prefix + i.  q [T, H, d_n + d_R],
    rows [prefix + T, R] (all of the sequence's rows).  Returns o [T, H, d_v]
    and lse [T, H]; entries outside ``queries`` x ``heads`` are NaN."""
    T, H, _ = q.shape
    d_n = w_uk.shape[1]
    d_v = w_uv.shape[1]
    assert rows.shape[0] >= prefix + T
    C = rows[:, :d_c]
    KR = rows[:, d_c:]
    qi = np.arange(T) if queries is None else np.asarray(queries)
    o = np.full((T, H, d_v), np.nan)
    lse = np.full((T, H), np.nan)
    for h in (range(H) if heads is None else heads):
        K_c = C @ w_uk[h].T
        V = C @ w_uv[h].T
        for i in qi.tolist():
            p = prefix + i
            q_c = q[i, h, :d_n]
            q_r = rope(q[i, h, d_n:], p, base)
            s = sigma * (K_c[: p + 1] @ q_c + KR[: p + 1] @ q_r)
            o[i, h], lse[i, h] = _attend(s, V[: p + 1])
    return o, lse


# --------------------------------------------------------------------------
# absorbed order ([arch] 1 and 6: fold W_UK into the query, apply W_UV
# after the weighted latent sum -- same function, different order)
# --------------------------------------------------------------------------


def absorb_query(q: np.ndarray, w_uk: np.ndarray, q_pos, d_n: int, base: float) -> np.ndarray:
    """q~[..., h, :d_c] = W_UK,h^T q_C,h ;  q~[..., h, d_c:] = RoPE(q_R,h, p).
    q [N, H, d_n + d_R], q_pos [N] -> [N, H, d_c + d_R]."""
    q_c = q[..., :d_n]
    q_r = rope(q[..., d_n:], np.asarray(q_pos)[..., None], base)
    q_lat = np.einsum("nhj,hjc->nhc", q_c, w_uk)
    return np.concatenate([q_lat, q_r], axis=-1)


def absorbed_logits(q_abs: np.ndarray, rows: np.ndarray, sigma: float) -> np.ndarray:
    """Scores of absorbed queries q_abs [H, R] against cached rows [T, R]:
    sigma * q~_h . row_t  -> [H, T]."""
    return sigma * (q_abs @ rows.T)


def nonabsorbed_logits(q: np.ndarray, rows: np.ndarray, w_uk: np.ndarray, q_pos: int,
                       d_c: int, sigma: float, base: float) -> np.ndarray:
    """The same scores computed with per-head K materialised -> [H, T]."""
    H = q.shape[0]
    d_n = w_uk.shape[1]
    C, KR = rows[:, :d_c], rows[:, d_c:]
    out = np.empty((H, rows.shape[0]))
    for h in range(H):
        out[h] = sigma * ((C @ w_uk[h].T) @ q[h, :d_n] + KR @ rope(q[h, d_n:], q_pos, base))
    return out


# --------------------------------------------------------------------------
# merging partial softmax results over disjoint token ranges
# --------------------------------------------------------------------------


def partial_softmax(scores: np.ndarray, latents: np.ndarray):
    """(m, l, acc) of one token range: m = max s, l = sum e^(s-m),
    acc = sum e^(s-m) latent.  An empty range gives (-inf, 0, 0)."""
    if scores.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(latents.shape[1])
    m = float(np.max(scores))
    w = np.exp(scores - m)
    return m, float(np.sum(w)), w @ latents


def merge_partials(parts) -> Tuple[np.ndarray, float]:
    """Combine (m_s, l_s, acc_s): m* = max m_s, weights e^(m_s - m*), normalised
    latent sum and natural-log LSE.  Empty parts carry weight 0."""
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    m_star = float(np.max(ms))
    if m_star == -np.inf:
        return np.zeros_like(parts[0][2]), -np.inf
    wts = np.array([0.0 if p[0] == -np.inf else math.exp(p[0] - m_star) for p in parts])
    l_star = float(sum(w * p[1] for w, p in zip(wts, parts)))
    acc = sum(w * p[2] for w, p in zip(wts, parts))
    return acc / l_star, m_star + math.log(l_star)


# --------------------------------------------------------------------------
# query low-rank compression and the output projection ([blog] "MLA nasil
# calisir?", last paragraph: the queries go through the same kind of
# compression; [arch] 1: the decompression matrices are folded into the
# query and the output matrices)
#
# Readings (the pages name the steps, not their shapes or a normalisation):
#   * c_Q,n = W_DQ h_n, a d_cq-wide query latent, not normalised;
#   * per head, [q_C | q_R] = W_UQ,h c_Q,n with W_UQ [H, d_n + d_R, d_cq];
#     q_R is rotated at the token's position exactly as before;
#   * y_n = W_O [o_n,1 | ... | o_n,H] with W_O [D, H d_v]: head h's output
#     meets columns h d_v .. h d_v + d_v - 1 of W_O.
# The folded ("absorbed") weights below are the same function in another
# order; the plain order above is the definition.
# --------------------------------------------------------------------------


def compress_query(h: np.ndarray, w_dq: np.ndarray) -> np.ndarray:
    """c_Q = W_DQ h: h [N, D], w_dq [d_cq, D] -> [N, d_cq]."""
    return h @ w_dq.T


def query_from_latent(c_q: np.ndarray, w_uq: np.ndarray) -> np.ndarray:
    """Per-head pre-RoPE query [q_C | q_R] = W_UQ,h c_Q: c_q [N, d_cq],
    w_uq [H, d_n + d_R, d_cq] -> [N, H, d_n + d_R]."""
    return np.einsum("nc,hjc->nhj", c_q, w_uq)


def output_projection(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y = W_O [o_1 | ... | o_H]: o [N, H, d_v] (heads in order), w_o
    [D, H d_v] -> [N, D]."""
    return o.reshape(o.shape[0], -1) @ w_o.T


def folded_query_weights(w_uq: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """W_UK folded into W_UQ: per head [W_UK,h^T W_UQ,h[:d_n] ; W_UQ,h[d_n:]],
    [H, d_c + d_R, d_cq], so that the absorbed query (before RoPE of its last
    d_R values) is this matrix times c_Q."""
    d_n = w_uk.shape[1]
    content = np.einsum("hjc,hjk->hck", w_uk, w_uq[:, :d_n])
    return np.concatenate([content, w_uq[:, d_n:]], axis=1)


def folded_output_weights(w_o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """W_UV folded into W_O: per head W_O,h W_UV,h, [H, D, d_c], so that
    y = sum_h W_OV,h lat_h for the softmax-weighted latent sums lat_h."""
    H, d_v, _ = w_uv.shape
    D = w_o.shape[0]
    return np.einsum("dhv,hvc->hdc", w_o.reshape(D, H, d_v), w_uv)
