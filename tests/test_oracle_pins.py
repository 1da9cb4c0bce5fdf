"""Pins of the CPU oracle against facts fixed outside itself.

Each test checks the oracle against something the pages print, a closed form,
an independent brute-force implementation, or a library routine -- never
against a retyped copy of its own formula.  A final block plants plausible
mistakes into a copy of the oracle and checks that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from mla_latent_kv_22_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# cache-size figures printed on the pages
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "cache_bytes.json")) as f:
        return json.load(f)


def test_cache_bytes_arch_example():
    g = _golden()
    e = g["arch_example_mla"]
    assert O.mla_cache_bytes_per_token(e["layers"], e["d_c"], e["d_r"], e["elem_bytes"]) == e["bytes_per_token"]
    e = g["arch_example_gqa"]
    assert O.gqa_cache_bytes_per_token(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"]) == e["bytes_per_token"]


def test_cache_bytes_v3():
    g = _golden()
    e = g["scale_v3_per_token"]
    per_tok = O.mla_cache_bytes_per_token(e["layers"], e["d_c"], e["d_r"], e["elem_bytes"])
    assert per_tok == 70272
    assert round(per_tok / 1024, 1) == e["printed_kib_per_token"]
    e8 = g["scale_v3_8k"]
    total = O.mla_cache_bytes(e["layers"], e8["tokens"], e["d_c"], e["d_r"], e["elem_bytes"])
    assert round(total / 2**20) == e8["printed_mla_mib"]
    r = e8["per_head_formula_reading"]
    per_head = O.gqa_cache_bytes_per_token(e["layers"], r["heads"], r["head_dim"], e["elem_bytes"])
    assert round(per_head * e8["tokens"] / 2**30, 2) == e8["printed_per_head_gib"]
    assert round(per_head / per_tok, 1) == e8["printed_ratio"]
    # the head count does not enter the MLA figure: per token it equals the
    # uniform-GQA formula with the 2.25 KV-head groups LLMScale prints
    # (at the 128-wide heads of that comparison), whatever the query heads
    groups = _golden()["scale_v2_groups"]["printed_groups"]
    assert O.gqa_cache_bytes_per_token(e["layers"], groups, 128, e["elem_bytes"]) == per_tok
    for heads in (16, 128):
        assert O.gqa_cache_bytes_per_token(e["layers"], heads, 128, e["elem_bytes"]) / per_tok == heads / groups


def test_gqa_equivalent_groups():
    e = _golden()["scale_v2_groups"]
    assert O.gqa_equivalent_groups(e["d_c"], e["d_r"], e["head_dim"]) == e["printed_groups"]


def test_gqa_mha_ratio():
    e = _golden()["scale_llama33_70b"]
    gqa = O.gqa_cache_bytes_per_token(80, e["kv_heads"], 128, 2)
    mha = O.gqa_cache_bytes_per_token(80, e["query_heads"], 128, 2)
    assert mha / gqa == e["printed_mha_kib"] / e["printed_gqa_kib"] == 8.0


# ---------------------------------------------------------------------------
# storage conversions
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3F81, 0x7F7F], dtype=np.uint16)
    v = O.from_storage(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0
    assert v[3] == 1.0 + 2.0 ** -7
    assert v[4] == (2 - 2.0 ** -7) * 2.0 ** 127


def test_round_bf16_ties_and_cross_implementation():
    ulp = 2.0 ** -7
    assert O.round_bf16(np.array([1.0 + ulp / 2]))[0] == 1.0            # tie -> even
    assert O.round_bf16(np.array([1.0 + 1.5 * ulp]))[0] == 1.0 + 2 * ulp  # tie -> even
    assert O.round_bf16(np.array([1.0 + 0.51 * ulp]))[0] == 1.0 + ulp
    assert O.round_bf16(np.array([-3.0]))[0] == -3.0
    # independent implementation (integer bit trick on float32) agrees on float32 inputs
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    a = O.round_bf16(x.astype(np.float64))
    b = O.from_storage(I.f32_to_bf16_bits(x), "bf16")
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# RoPE closed forms
# ---------------------------------------------------------------------------

def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(16)
    assert np.array_equal(O.rope(x, 0, 10000.0), x)                       # position 0 is identity
    for p in (1, 7, 4095, 32767):
        y = O.rope(x, p, 10000.0)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12         # rotation keeps the norm
    # d = 2: theta_0 = 1, so [1, 0] rotates to [cos p, sin p]
    for p in (1, 2, 3, 100):
        assert np.allclose(O.rope(np.array([1.0, 0.0]), p, 10000.0), [math.cos(p), math.sin(p)], atol=1e-15)
    # last pair of d=4 turns with theta_1 = base^(-1/2)
    y = O.rope(np.array([0.0, 0.0, 1.0, 0.0]), 3, 100.0)
    assert np.allclose(y, [0, 0, math.cos(0.3), math.sin(0.3)], atol=1e-15)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((5, 3), (100, 1), (8191, 17), (12, 12)):
        lhs = O.rope(q, m, 10000.0) @ O.rope(k, n, 10000.0)
        rhs = O.rope(q, m - n, 10000.0) @ k
        assert abs(lhs - rhs) < 1e-10


def test_rope_batched_positions():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 4, 8))
    pos = np.array([0, 5, 9])
    y = O.rope(x, pos[:, None], 10000.0)
    for i in range(3):
        for j in range(4):
            assert np.allclose(y[i, j], O.rope(x[i, j], pos[i], 10000.0), atol=0, rtol=0)


# ---------------------------------------------------------------------------
# brute force: plain Python loops over tiny inputs, written from the
# definition independently of the vectorised oracle
# ---------------------------------------------------------------------------

def _bf_rope(v, p, base):
    d = len(v)
    out = []
    for i in range(d // 2):
        a = p * base ** (-2.0 * i / d)
        out += [v[2 * i] * math.cos(a) - v[2 * i + 1] * math.sin(a),
                v[2 * i] * math.sin(a) + v[2 * i + 1] * math.cos(a)]
    return out


def _bf_rows(h, w_dkv, w_kr, pos, base):
    rows = []
    for n in range(len(h)):
        c = [sum(w_dkv[i][j] * h[n][j] for j in range(len(h[n]))) for i in range(len(w_dkv))]
        kr = [sum(w_kr[i][j] * h[n][j] for j in range(len(h[n]))) for i in range(len(w_kr))]
        rows.append(c + _bf_rope(kr, pos[n], base))
    return rows


def _bf_decode(q, rows, w_uk, w_uv, q_pos, d_c, sigma, base, causal_len=None):
    H, d_n, d_v = len(q), len(w_uk[0]), len(w_uv[0])
    T = len(rows) if causal_len is None else causal_len
    outs, lses = [], []
    for h in range(H):
        qr = _bf_rope(list(q[h][d_n:]), q_pos, base)
        sc = []
        for t in range(T):
            kc = [sum(w_uk[h][j][c] * rows[t][c] for c in range(d_c)) for j in range(d_n)]
            s = sum(q[h][j] * kc[j] for j in range(d_n))
            s += sum(qr[i] * rows[t][d_c + i] for i in range(len(qr)))
            sc.append(sigma * s)
        m = max(sc)
        e = [math.exp(s - m) for s in sc]
        l = sum(e)
        vs = [[sum(w_uv[h][j][c] * rows[t][c] for c in range(d_c)) for j in range(d_v)] for t in range(T)]
        outs.append([sum(e[t] * vs[t][j] for t in range(T)) / l for j in range(d_v)])
        lses.append(m + math.log(l))
    return np.array(outs), np.array(lses)


def _tiny(seed, H=2, T=5, D=6, d_c=4, d_r=2, d_n=3, d_v=3, wstd=0.7):
    rng = np.random.default_rng(seed)
    return dict(
        h=rng.standard_normal((T, D)), w_dkv=rng.standard_normal((d_c, D)) * wstd,
        w_kr=rng.standard_normal((d_r, D)) * wstd, w_uk=rng.standard_normal((H, d_n, d_c)) * wstd,
        w_uv=rng.standard_normal((H, d_v, d_c)) * wstd, q=rng.standard_normal((H, d_n + d_r)),
        d_c=d_c, sigma=1.0 / math.sqrt(d_n + d_r), base=10000.0, T=T)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_brute_force_decode(seed):
    t = _tiny(seed)
    pos = np.arange(t["T"])
    rows = O.latent_rows(t["h"], t["w_dkv"], t["w_kr"], pos, t["base"])
    rows_bf = _bf_rows(t["h"].tolist(), t["w_dkv"].tolist(), t["w_kr"].tolist(), pos.tolist(), t["base"])
    assert _rel(rows, rows_bf) < 1e-12
    o, lse = O.decode_one(t["q"], rows, t["w_uk"], t["w_uv"], t["T"] - 1, t["d_c"], t["sigma"], t["base"])
    o_bf, lse_bf = _bf_decode(t["q"].tolist(), rows_bf, t["w_uk"].tolist(), t["w_uv"].tolist(),
                              t["T"] - 1, t["d_c"], t["sigma"], t["base"])
    assert _rel(o, o_bf) < 1e-12
    assert np.max(np.abs(lse - lse_bf)) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_prefill(seed):
    t = _tiny(seed, T=6)
    rng = np.random.default_rng(100 + seed)
    H = t["q"].shape[0]
    qs = rng.standard_normal((t["T"], H, t["q"].shape[1]))
    rows = O.latent_rows(t["h"], t["w_dkv"], t["w_kr"], np.arange(t["T"]), t["base"])
    o, lse = O.prefill_one(qs, rows, t["w_uk"], t["w_uv"], t["d_c"], t["sigma"], t["base"])
    rows_l = rows.tolist()
    for i in range(t["T"]):
        o_bf, lse_bf = _bf_decode(qs[i].tolist(), rows_l, t["w_uk"].tolist(), t["w_uv"].tolist(), i,
                                  t["d_c"], t["sigma"], t["base"], causal_len=i + 1)
        assert _rel(o[i], o_bf) < 1e-12
        assert np.max(np.abs(lse[i] - lse_bf)) < 1e-12


# ---------------------------------------------------------------------------
# library-routine special cases
# ---------------------------------------------------------------------------

def test_absorbed_equals_sdpa_mqa():
    """Absorbed MLA is MQA with one shared key [c | k_R], value c and H
    query heads q~; torch's SDPA on that, then W_UV per head, must match."""
    rng = np.random.default_rng(11)
    H, T, D, d_c, d_r, d_n, d_v = 4, 37, 24, 16, 8, 8, 8
    h = rng.standard_normal((T, D))
    w_dkv, w_kr = rng.standard_normal((d_c, D)) * 0.3, rng.standard_normal((d_r, D)) * 0.3
    w_uk, w_uv = rng.standard_normal((H, d_n, d_c)) * 0.3, rng.standard_normal((H, d_v, d_c)) * 0.3
    q = rng.standard_normal((H, d_n + d_r))
    sigma, base, qpos = 0.29, 10000.0, T - 1
    rows = O.latent_rows(h, w_dkv, w_kr, np.arange(T), base)
    o, lse = O.decode_one(q, rows, w_uk, w_uv, qpos, d_c, sigma, base)
    # absorbed query built here with plain numpy + the relative-position-pinned rope
    q_lat = np.stack([w_uk[i].T @ q[i, :d_n] for i in range(H)])
    q_rot = np.stack([O.rope(q[i, d_n:], qpos, base) for i in range(H)])
    qa = torch.tensor(np.concatenate([q_lat, q_rot], 1), dtype=torch.float64)[None, :, None, :]
    k = torch.tensor(rows, dtype=torch.float64)[None, None].expand(1, H, T, d_c + d_r)
    v = torch.tensor(rows[:, :d_c], dtype=torch.float64)[None, None].expand(1, H, T, d_c)
    lat = torch.nn.functional.scaled_dot_product_attention(qa, k, v, scale=sigma)[0, :, 0, :].numpy()
    o_ref = np.stack([w_uv[i] @ lat[i] for i in range(H)])
    assert _rel(o, o_ref) < 1e-12
    s = sigma * (qa[0, :, 0, :].numpy() @ rows.T)
    lse_ref = np.log(np.sum(np.exp(s), axis=1))
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_identity_weights_textbook_attention():
    """H = 1, W_UK = W_UV = I (d_n = d_v = d_c): plain single-head attention
    with key [c | k_R], query [q_C | RoPE(q_R)], value c."""
    rng = np.random.default_rng(12)
    T, D, d_c, d_r = 19, 10, 6, 4
    h = rng.standard_normal((T, D))
    w_dkv, w_kr = rng.standard_normal((d_c, D)) * 0.4, rng.standard_normal((d_r, D)) * 0.4
    eye = np.eye(d_c)[None]
    q = rng.standard_normal((1, d_c + d_r))
    rows = O.latent_rows(h, w_dkv, w_kr, np.arange(T), 500.0)
    o, lse = O.decode_one(q, rows, eye, eye, T - 1, d_c, 0.5, 500.0)
    qq = np.concatenate([q[0, :d_c], O.rope(q[0, d_c:], T - 1, 500.0)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(qq)[None, None, None], torch.tensor(rows)[None, None],
        torch.tensor(rows[:, :d_c])[None, None], scale=0.5)[0, 0, 0].numpy()
    assert _rel(o[0], ref) < 1e-12


def test_causal_prefill_equals_sdpa_causal():
    rng = np.random.default_rng(13)
    H, T, D, d_c, d_r, d_n, d_v = 3, 23, 12, 8, 4, 6, 5
    h = rng.standard_normal((T, D))
    w_dkv, w_kr = rng.standard_normal((d_c, D)) * 0.3, rng.standard_normal((d_r, D)) * 0.3
    w_uk, w_uv = rng.standard_normal((H, d_n, d_c)) * 0.3, rng.standard_normal((H, d_v, d_c)) * 0.3
    q = rng.standard_normal((T, H, d_n + d_r))
    base, sigma = 10000.0, 0.35
    rows = O.latent_rows(h, w_dkv, w_kr, np.arange(T), base)
    o, lse = O.prefill_one(q, rows, w_uk, w_uv, d_c, sigma, base)
    for i in range(H):
        K = np.concatenate([rows[:, :d_c] @ w_uk[i].T, rows[:, d_c:]], 1)
        V = rows[:, :d_c] @ w_uv[i].T
        Q = np.concatenate([q[:, i, :d_n], np.stack([O.rope(q[t, i, d_n:], t, base) for t in range(T)])], 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
            is_causal=True, scale=sigma)[0, 0].numpy()
        assert _rel(o[:, i], ref) < 1e-12


def _prefix_case(seed, P, L):
    rng = np.random.default_rng(seed)
    H, D, d_c, d_r, d_n, d_v = 3, 12, 8, 4, 6, 5
    T = P + L
    h = rng.standard_normal((T, D))
    w_dkv, w_kr = rng.standard_normal((d_c, D)) * 0.3, rng.standard_normal((d_r, D)) * 0.3
    w_uk, w_uv = rng.standard_normal((H, d_n, d_c)) * 0.3, rng.standard_normal((H, d_v, d_c)) * 0.3
    q = rng.standard_normal((T, H, d_n + d_r))
    base, sigma = 10000.0, 0.35
    rows = O.latent_rows(h, w_dkv, w_kr, np.arange(T), base)
    return dict(H=H, d_c=d_c, d_n=d_n, w_uk=w_uk, w_uv=w_uv, q=q, base=base, sigma=sigma, rows=rows)


@pytest.mark.parametrize("P,L", [(7, 5), (0, 6), (13, 1)])
def test_prefix_prefill_equals_sdpa_bottom_right_mask(P, L):
    """Prefill onto a prefix of P cached tokens is attention of the L new
    queries (positions P..P+L-1) over all P+L keys with the causal mask aligned
    to the last key: torch's SDPA with that explicit boolean mask."""
    c = _prefix_case(40 + P, P, L)
    q, rows, d_c, d_n = c["q"][P:], c["rows"], c["d_c"], c["d_n"]
    o, lse = O.prefill_one(q, rows, c["w_uk"], c["w_uv"], d_c, c["sigma"], c["base"], prefix=P)
    mask = torch.tensor(np.arange(P + L)[None, :] <= (P + np.arange(L))[:, None])
    for i in range(c["H"]):
        K = np.concatenate([rows[:, :d_c] @ c["w_uk"][i].T, rows[:, d_c:]], 1)
        V = rows[:, :d_c] @ c["w_uv"][i].T
        Q = np.concatenate([q[:, i, :d_n], np.stack([O.rope(q[t, i, d_n:], P + t, c["base"]) for t in range(L)])], 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
            attn_mask=mask, scale=c["sigma"])[0, 0].numpy()
        assert _rel(o[:, i], ref) < 1e-12
        s = c["sigma"] * (Q @ K.T)
        s[~mask.numpy()] = -np.inf
        lse_ref = np.log(np.sum(np.exp(s), axis=1))
        assert np.max(np.abs(lse[:, i] - lse_ref)) < 1e-12


def test_prefix_prefill_is_the_tail_of_a_full_prefill():
    """Causal attention by position: the new rows of a prefill onto a prefix
    equal the last rows of a prefill of the whole sequence."""
    P, L = 9, 6
    c = _prefix_case(50, P, L)
    args = (c["w_uk"], c["w_uv"], c["d_c"], c["sigma"], c["base"])
    o_full, lse_full = O.prefill_one(c["q"], c["rows"], *args)
    o_tail, lse_tail = O.prefill_one(c["q"][P:], c["rows"], *args, prefix=P)
    assert np.max(np.abs(o_tail - o_full[P:])) < 1e-12
    assert np.max(np.abs(lse_tail - lse_full[P:])) < 1e-12


def test_prefix_prefill_of_one_token_is_decode():
    """One new token after P cached ones is the decode query at position P
    over P + 1 rows."""
    P = 11
    c = _prefix_case(51, P, 1)
    o_p, lse_p = O.prefill_one(c["q"][P:], c["rows"], c["w_uk"], c["w_uv"], c["d_c"], c["sigma"], c["base"],
                               prefix=P)
    o_d, lse_d = O.decode_one(c["q"][P], c["rows"], c["w_uk"], c["w_uv"], P, c["d_c"], c["sigma"], c["base"])
    assert np.max(np.abs(o_p[0] - o_d)) < 1e-12
    assert np.max(np.abs(lse_p[0] - lse_d)) < 1e-12


# ---------------------------------------------------------------------------
# invariants the pages state
# ---------------------------------------------------------------------------

def test_absorbed_and_nonabsorbed_logits_agree():
    """Switching the projection order keeps the logits (openarchlab 4 and 6)."""
    rng = np.random.default_rng(21)
    H, T, d_c, d_r, d_n = 8, 50, 64, 16, 32
    rows = rng.standard_normal((T, d_c + d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) * 0.02
    q = rng.standard_normal((1, H, d_n + d_r)) * 0.3
    qa = O.absorb_query(q, w_uk, np.array([T - 1]), d_n, 10000.0)[0]
    la = O.absorbed_logits(qa, rows, 0.2)
    ln = O.nonabsorbed_logits(q[0], rows, w_uk, T - 1, d_c, 0.2, 10000.0)
    assert _rel(la, ln) < 1e-12


def test_position_branch_changes_scores():
    """Same content latent, different rotary key -> different scores; with
    q_R = 0 they are equal (openarchlab 5)."""
    rng = np.random.default_rng(22)
    H, D, d_c, d_r, d_n = 4, 16, 8, 4, 6
    w_dkv, w_kr = rng.standard_normal((d_c, D)), rng.standard_normal((d_r, D))
    w_uk = rng.standard_normal((H, d_n, d_c))
    hvec = rng.standard_normal(D)
    h = np.stack([hvec, hvec])
    rows = O.latent_rows(h, w_dkv, w_kr, np.array([3, 900]), 10000.0)
    assert np.array_equal(rows[0, :d_c], rows[1, :d_c])
    assert not np.allclose(rows[0, d_c:], rows[1, d_c:])
    q = rng.standard_normal((H, d_n + d_r))
    s = O.nonabsorbed_logits(q, rows, w_uk, 1000, d_c, 1.0, 10000.0)
    assert np.all(np.abs(s[:, 0] - s[:, 1]) > 1e-6)
    q0 = q.copy()
    q0[:, d_n:] = 0
    s0 = O.nonabsorbed_logits(q0, rows, w_uk, 1000, d_c, 1.0, 10000.0)
    assert np.array_equal(s0[:, 0], s0[:, 1])


def test_single_token_context():
    rng = np.random.default_rng(23)
    H, d_c, d_r, d_n, d_v = 3, 8, 4, 5, 7
    rows = rng.standard_normal((1, d_c + d_r))
    w_uk, w_uv = rng.standard_normal((H, d_n, d_c)), rng.standard_normal((H, d_v, d_c))
    q = rng.standard_normal((H, d_n + d_r))
    o, lse = O.decode_one(q, rows, w_uk, w_uv, 0, d_c, 0.4, 10000.0)
    for i in range(H):
        assert _rel(o[i], w_uv[i] @ rows[0, :d_c]) < 1e-14
    s = O.nonabsorbed_logits(q, rows, w_uk, 0, d_c, 0.4, 10000.0)[:, 0]
    assert np.max(np.abs(lse - s)) < 1e-14


def test_empty_context():
    o, lse = O.decode_one(np.ones((2, 6)), np.zeros((0, 6)), np.ones((2, 3, 4)), np.ones((2, 5, 4)),
                          0, 4, 1.0, 10000.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("cuts", [(0, 64), (0, 1, 64), (0, 10, 11, 40, 64), (0, 32, 32, 64)])
def test_partition_merge_equals_whole(cuts):
    """Any split of the token axis into ranges merges to the unsplit softmax."""
    rng = np.random.default_rng(24)
    s = rng.standard_normal(64) * 3
    lat = rng.standard_normal((64, 9))
    whole, lse_whole = O.merge_partials([O.partial_softmax(s, lat)])
    parts = [O.partial_softmax(s[a:b], lat[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    merged, lse = O.merge_partials(parts)
    w = np.exp(s - s.max())
    assert _rel(whole, (w @ lat) / w.sum()) < 1e-14
    assert _rel(merged, whole) < 1e-13
    assert abs(lse - lse_whole) < 1e-13
    assert abs(lse - (s.max() + math.log(w.sum()))) < 1e-13


def test_softmax_shift_invariance():
    rng = np.random.default_rng(25)
    s = rng.standard_normal(40)
    lat = rng.standard_normal((40, 3))
    a, la = O.merge_partials([O.partial_softmax(s, lat)])
    b, lb = O.merge_partials([O.partial_softmax(s + 1000.0, lat)])
    assert _rel(a, b) < 1e-12 and abs((lb - la) - 1000.0) < 1e-9


def test_scatter_gather_roundtrip_and_skip():
    rng = np.random.default_rng(26)
    pool = np.full((5, 4, 3), -7.0)
    rows = rng.standard_normal((6, 3))
    slots = np.array([0, 5, 19, -1, 8, 13])
    out = O.scatter_rows(pool, rows, slots)
    for n, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(out[s // 4, s % 4], rows[n])
    touched = {int(s) for s in slots if s >= 0}
    for s in range(20):
        if s not in touched:
            assert np.all(out[s // 4, s % 4] == -7.0)
    bt = np.array([3, 1, 4])
    g = O.gather_rows(out, bt, 9)
    for t in range(9):
        assert np.array_equal(g[t], out[bt[t // 4], t % 4])


def test_one_hot_projection_selects_hidden_values():
    rng = np.random.default_rng(27)
    D, d_c, d_r = 12, 5, 4
    h = rng.standard_normal((3, D))
    sel = rng.permutation(D)[: d_c + d_r]
    w = np.zeros((d_c + d_r, D))
    w[np.arange(d_c + d_r), sel] = 1.0
    rows = O.latent_rows(h, w[:d_c], w[d_c:], np.zeros(3, dtype=int), 10000.0)
    assert np.array_equal(rows, h[:, sel])


def test_decode_batch_uses_block_table():
    rng = np.random.default_rng(28)
    H, d_c, d_r, d_n, d_v, P = 2, 4, 2, 3, 3, 4
    pool = rng.standard_normal((6, P, d_c + d_r))
    w_uk, w_uv = rng.standard_normal((H, d_n, d_c)), rng.standard_normal((H, d_v, d_c))
    q = rng.standard_normal((2, H, d_n + d_r))
    bt = np.array([[5, 0], [2, 3]])
    lens = np.array([7, 3])
    o, lse = O.decode(q, pool, bt, lens, w_uk, w_uv, d_c, 0.5, 10000.0)
    for b in range(2):
        rows = np.concatenate([pool[bt[b, 0]], pool[bt[b, 1]]])[: lens[b]]
        ob, lb = O.decode_one(q[b], rows, w_uk, w_uv, lens[b] - 1, d_c, 0.5, 10000.0)
        assert np.array_equal(o[b], ob) and np.array_equal(lse[b], lb)


# ---------------------------------------------------------------------------
# 8-bit cache rows: E4M3 codes with one power-of-two scale per row
# ---------------------------------------------------------------------------

def _torch_e4m3_codes(x):
    """torch's own float -> float8_e4m3fn conversion (round to nearest even),
    with -0 folded into +0 as the oracle stores it."""
    c = torch.as_tensor(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    return np.where(c == 0x80, 0, c)


def test_e4m3_values_match_torch_float8():
    codes = np.arange(256)
    ours = O.e4m3_value(codes)
    ref = torch.as_tensor(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref)) and int(np.isnan(ours).sum()) == 2
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # facts of the format: 448 is the largest finite value, 2^-9 the smallest
    # positive, 2^-6 the smallest normal, and codes 0x00..0x7E increase
    assert np.nanmax(ours) == 448.0 and ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6
    assert np.all(np.diff(ours[:0x7F]) > 0)


def test_e4m3_quantize_matches_torch_cast():
    rng = np.random.default_rng(5)
    # float32 inputs (torch converts through float32; the cache's inputs are
    # bf16 values over a power of two, so float32 holds them exactly)
    grid = O.e4m3_value(np.arange(0x7F)).astype(np.float32)
    mids = (grid[1:] + grid[:-1]) / 2                     # exact ties
    x = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
                        rng.uniform(-448, 448, 20000).astype(np.float32),
                        np.exp2(rng.uniform(-14, np.log2(448), 20000)).astype(np.float32),
                        np.array([0.0, 2.0 ** -11, 3 * 2.0 ** -11, 448.0], np.float32)]).astype(np.float64)
    x = np.concatenate([x, -x])
    assert np.array_equal(O.quantize_e4m3(x).astype(np.int64), _torch_e4m3_codes(x))


def test_e4m3_quantize_inverts_decode():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)])
    assert np.array_equal(O.quantize_e4m3(O.e4m3_value(codes)).astype(np.int64), codes)


@pytest.mark.parametrize("amax", [0.0, 2.0 ** -130, 1e-30, 0.37, 1.0, 224.0, 224.0001, 448.0, 448.5, 3.0e5, 1e30])
def test_row_scale_exponent_bounds(amax):
    e = O.row_scale_exponent(amax)
    if amax == 0.0:
        assert e == 0
        return
    assert amax <= 448.0 * 2.0 ** e
    assert e == -126 or amax > 448.0 * 2.0 ** (e - 1)


def test_quantize_row_error_bound_and_scale():
    rng = np.random.default_rng(6)
    for mag in (1e-3, 1.0, 37.0, 1e4):
        row = rng.standard_normal(576) * mag
        codes, scale = O.quantize_row_fp8(row)
        bf = O.round_bf16(row)
        assert math.log2(scale) == int(math.log2(scale))            # a power of two
        amax = float(np.max(np.abs(bf)))
        assert 224.0 < amax / scale <= 448.0
        deq = O.e4m3_value(codes) * scale
        # nearest grid point: at most half a step, 2^-4 of the value's binade
        # base for normals, 2^-10 scale for subnormals
        half = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(bf) / scale, 2.0 ** -6))) - 4), 2.0 ** -10) * scale
        assert np.all(np.abs(deq - bf) <= half)
        assert np.array_equal(codes.astype(np.int64), _torch_e4m3_codes(bf / scale))


def test_fp8_pages_layout_and_roundtrip():
    rng = np.random.default_rng(7)
    P, R, npg = 4, 6, 3
    codes = rng.integers(0, 0x7F, size=(npg, P, R)).astype(np.uint8)
    scales = np.exp2(rng.integers(-5, 5, size=(npg, P))).astype(np.float64)
    pages = O.pack_fp8_pages(codes, scales)
    assert pages.shape == (npg, P * (R + 4))
    # row t of page g starts at byte R t; its scale is the little-endian
    # float32 at byte P R + 4 t
    g, t = 2, 3
    assert bytes(pages[g, R * t:R * t + R]) == bytes(codes[g, t])
    assert np.frombuffer(bytes(pages[g, P * R + 4 * t:P * R + 4 * t + 4]), "<f4")[0] == scales[g, t]
    c2, s2 = O.unpack_fp8_pages(pages, P, R)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_fp8_write_one_hot_rows_and_skip():
    # selection weights and position 0: the row is the chosen hidden values
    # exactly, so its codes are torch's E4M3 casts of those values over the
    # row's scale; slot -1 leaves the pages unchanged
    rng = np.random.default_rng(8)
    D, d_c, d_r, P = 12, 6, 2, 4
    h = O.round_bf16(rng.standard_normal((3, D)) * 3.0)
    sel = rng.permutation(D)[:d_c + d_r]
    w = np.zeros((d_c + d_r, D))
    w[np.arange(d_c + d_r), sel] = 1.0
    rows = O.latent_rows(h, w[:d_c], w[d_c:], np.zeros(3), 10000.0)
    assert np.array_equal(rows, h[:, sel])
    pages0 = np.full((2, P * (d_c + d_r + 4)), 0x5A, dtype=np.uint8)
    pages = O.write_rows_fp8(pages0, rows, np.array([5, -1, 2]), P)
    codes, scales = O.unpack_fp8_pages(pages, P, d_c + d_r)
    for n, slot in ((0, 5), (2, 2)):
        sc = scales[slot // P, slot % P]
        assert sc == 2.0 ** O.row_scale_exponent(float(np.max(np.abs(rows[n]))))
        assert np.array_equal(codes[slot // P, slot % P].astype(np.int64), _torch_e4m3_codes(rows[n] / sc))
    c0, s0 = O.unpack_fp8_pages(pages0, P, d_c + d_r)
    untouched = [(g, t) for g in range(2) for t in range(P) if g * P + t not in (5, 2)]
    for g, t in untouched:
        assert np.array_equal(codes[g, t], c0[g, t])
        assert s0[g, t] == scales[g, t] or (np.isnan(s0[g, t]) and np.isnan(scales[g, t]))


def test_fp8_pool_decode_equals_decode_of_its_values():
    # a pool whose codes all have scale 1 holds E4M3 values, which bf16 holds
    # exactly: decoding the 8-bit pool equals decoding those values
    rng = np.random.default_rng(9)
    B, H, T, P, d_c, d_r, d_n, d_v = 2, 3, 9, 4, 8, 4, 5, 6
    R = d_c + d_r
    npg = B * ((T + P - 1) // P)
    codes = rng.integers(0, 0x7F, size=(npg, P, R)).astype(np.uint8)
    codes ^= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)  # random signs
    codes[codes == 0xFF] = 0x7E
    scales = np.exp2(rng.integers(-9, -4, size=(npg, P))).astype(np.float64)
    pages = O.pack_fp8_pages(codes, scales)
    vals = O.fp8_pool_values(pages, P, R)
    assert np.array_equal(O.round_bf16(vals), vals)
    bt = rng.permutation(npg).reshape(B, -1).astype(np.int32)
    q = rng.standard_normal((B, H, d_n + d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) * 0.3
    w_uv = rng.standard_normal((H, d_v, d_c)) * 0.3
    lens = np.array([T, T - 3])
    o8, l8 = O.decode(q, vals, bt, lens, w_uk, w_uv, d_c, 0.4, 10000.0)
    # the same values written out element by element from codes and scales
    manual = np.empty_like(vals)
    for g in range(npg):
        for t in range(P):
            manual[g, t] = [float(torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn).double())
                            * scales[g, t] for c in codes[g, t]]
    o_ref, l_ref = O.decode(q, manual, bt, lens, w_uk, w_uv, d_c, 0.4, 10000.0)
    assert np.array_equal(o8, o_ref) and np.array_equal(l8, l_ref)


# ---------------------------------------------------------------------------
# query compression and output projection ([blog] "MLA nasil calisir?";
# [arch] 1 and 6: folding the decompression matrices into the query and the
# output matrices changes the order, not the function)
# ---------------------------------------------------------------------------

def _qo_case(seed, H=3, T=17, D=14, d_c=8, d_r=4, d_n=5, d_v=6, d_cq=7):
    rng = np.random.default_rng(seed)
    return dict(
        rows=rng.standard_normal((T, d_c + d_r)), h=rng.standard_normal((1, D)),
        w_dq=rng.standard_normal((d_cq, D)) * 0.4, w_uq=rng.standard_normal((H, d_n + d_r, d_cq)) * 0.4,
        w_uk=rng.standard_normal((H, d_n, d_c)) * 0.4, w_uv=rng.standard_normal((H, d_v, d_c)) * 0.4,
        w_o=rng.standard_normal((D, H * d_v)) * 0.4, d_c=d_c, d_r=d_r, d_n=d_n, sigma=0.3, base=10000.0, pos=T - 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_folded_query_weights_give_the_same_logits(seed):
    c = _qo_case(seed)
    c_q = O.compress_query(c["h"], c["w_dq"])
    q = O.query_from_latent(c_q, c["w_uq"])[0]
    plain = O.nonabsorbed_logits(q, c["rows"], c["w_uk"], c["pos"], c["d_c"], c["sigma"], c["base"])
    w_qk = O.folded_query_weights(c["w_uq"], c["w_uk"])
    qa = np.einsum("hjc,c->hj", w_qk, c_q[0])
    qa[:, c["d_c"]:] = O.rope(qa[:, c["d_c"]:], c["pos"], c["base"])
    folded = c["sigma"] * (qa @ c["rows"].T)
    assert _rel(folded, plain) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_folded_output_weights_give_the_same_output(seed):
    c = _qo_case(seed)
    q = O.query_from_latent(O.compress_query(c["h"], c["w_dq"]), c["w_uq"])[0]
    o, _ = O.decode_one(q, c["rows"], c["w_uk"], c["w_uv"], c["pos"], c["d_c"], c["sigma"], c["base"])
    y = O.output_projection(o[None], c["w_o"])[0]
    # folded: the softmax-weighted latent sums of each head through W_O,h W_UV,h
    s = O.nonabsorbed_logits(q, c["rows"], c["w_uk"], c["pos"], c["d_c"], c["sigma"], c["base"])
    p = np.exp(s - s.max(axis=1, keepdims=True))
    lat = (p / p.sum(axis=1, keepdims=True)) @ c["rows"][:, : c["d_c"]]
    y_folded = np.einsum("hdc,hc->d", O.folded_output_weights(c["w_o"], c["w_uv"]), lat)
    assert _rel(y_folded, y) < 1e-12


def test_brute_force_query_and_output_projection():
    c = _qo_case(3, H=2, T=4, D=5, d_c=3, d_r=2, d_n=2, d_v=2, d_cq=3)
    h, w_dq, w_uq, w_o = c["h"][0].tolist(), c["w_dq"].tolist(), c["w_uq"].tolist(), c["w_o"].tolist()
    cq = [sum(w_dq[i][j] * h[j] for j in range(len(h))) for i in range(len(w_dq))]
    q_bf = [[sum(w_uq[hh][j][i] * cq[i] for i in range(len(cq))) for j in range(len(w_uq[0]))]
            for hh in range(len(w_uq))]
    q = O.query_from_latent(O.compress_query(c["h"], c["w_dq"]), c["w_uq"])[0]
    assert _rel(q, q_bf) < 1e-12
    rng = np.random.default_rng(4)
    o = rng.standard_normal((2, 2, 2))  # [N, H, d_v]
    y = O.output_projection(o, c["w_o"])
    for n in range(2):
        for d in range(len(w_o)):
            ref = sum(w_o[d][hh * 2 + v] * o[n, hh, v] for hh in range(2) for v in range(2))
            assert abs(y[n, d] - ref) < 1e-12


def test_projected_decode_equals_sdpa_then_output_matmul():
    """From h to y: the compressed query, MLA decode and the output projection
    equal torch's SDPA over one shared key [c | k_R] and value c (float64),
    followed by W_UV,h per head and W_O, written out with torch matmuls."""
    c = _qo_case(5, H=4, T=29, D=16, d_c=8, d_r=4, d_n=6, d_v=5, d_cq=9)
    q = O.query_from_latent(O.compress_query(c["h"], c["w_dq"]), c["w_uq"])[0]
    o, _ = O.decode_one(q, c["rows"], c["w_uk"], c["w_uv"], c["pos"], c["d_c"], c["sigma"], c["base"])
    y = O.output_projection(o[None], c["w_o"])[0]
    d_n, d_c, H = c["d_n"], c["d_c"], q.shape[0]
    cq_t = torch.nn.functional.linear(torch.tensor(c["h"]), torch.tensor(c["w_dq"]))[0]
    q_t = torch.stack([torch.tensor(c["w_uq"][i]) @ cq_t for i in range(H)])
    qa = torch.stack([torch.cat([torch.tensor(c["w_uk"][i]).T @ q_t[i, :d_n],
                                 torch.tensor(O.rope(q_t[i, d_n:].numpy(), c["pos"], c["base"]))]) for i in range(H)])
    K = torch.tensor(c["rows"])[None, None].expand(1, H, -1, -1)
    V = torch.tensor(c["rows"][:, :d_c])[None, None].expand(1, H, -1, -1)
    lat = torch.nn.functional.scaled_dot_product_attention(qa[None, :, None, :], K, V, scale=c["sigma"])[0, :, 0]
    heads = [torch.tensor(c["w_uv"][i]) @ lat[i] for i in range(H)]
    y_ref = torch.tensor(c["w_o"]) @ torch.cat(heads)
    assert _rel(y, y_ref.numpy()) < 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: a copy of the oracle with one plausible slip must fail a pin
# ---------------------------------------------------------------------------

_ORIG_ROPE = O.rope


def _mut_rope_sign(x, pos, base):
    x = np.asarray(x, np.float64)
    y = np.empty_like(x)
    d = x.shape[-1]
    i = np.arange(d // 2)
    ang = np.broadcast_to(np.asarray(pos, np.float64), x.shape[:-1])[..., None] * np.power(base, -2.0 * i / d)
    y[..., 0::2] = x[..., 0::2] * np.cos(ang) + x[..., 1::2] * np.sin(ang)
    y[..., 1::2] = -x[..., 0::2] * np.sin(ang) + x[..., 1::2] * np.cos(ang)
    return y


def _mut_rope_halfsplit_q_only(x, pos, base):
    # pairs (i, i + d/2) instead of (2i, 2i+1): only consistent if both q and k use it
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.arange(d).reshape(2, d // 2).T.reshape(-1)
    y = np.empty_like(x)
    y[..., perm] = _ORIG_ROPE(x[..., perm], pos, base)
    return y


def _mut_decode_one(slip):
    """decode_one with one slip: 'drop_kr' omits the rotary term,
    'sigma_content_only' scales only the content term."""
    def f(q, rows, w_uk, w_uv, q_pos, d_c, sigma, base, heads=None):
        H = q.shape[0]
        d_n = w_uk.shape[1]
        C, KR = rows[:, :d_c], rows[:, d_c:]
        o = np.full((H, w_uv.shape[1]), np.nan)
        lse = np.full(H, np.nan)
        for h in (range(H) if heads is None else heads):
            qr = O.rope(q[h, d_n:], q_pos, base)
            content = (C @ w_uk[h].T) @ q[h, :d_n]
            if slip == "drop_kr":
                s = sigma * content
            else:
                s = sigma * content + KR @ qr
            m = s.max()
            w = np.exp(s - m)
            o[h] = (w @ (C @ w_uv[h].T)) / w.sum()
            lse[h] = m + math.log(w.sum())
        return o, lse
    return f


def _mut_prefill_peek(q, rows, w_uk, w_uv, d_c, sigma, base, queries=None, heads=None, prefix=0):
    """prefill that lets query i also see row i+1 (causal mask off by one)."""
    T, H, _ = q.shape
    d_n = w_uk.shape[1]
    o = np.full((T, H, w_uv.shape[1]), np.nan)
    lse = np.full((T, H), np.nan)
    for h in (range(H) if heads is None else heads):
        K = rows[:, :d_c] @ w_uk[h].T
        V = rows[:, :d_c] @ w_uv[h].T
        for i in (range(T) if queries is None else queries):
            n = min(rows.shape[0], prefix + i + 2)
            s = sigma * (K[:n] @ q[i, h, :d_n] + rows[:n, d_c:] @ O.rope(q[i, h, d_n:], prefix + i, base))
            m = s.max()
            w = np.exp(s - m)
            o[i, h] = (w @ V[:n]) / w.sum()
            lse[i, h] = m + math.log(w.sum())
    return o, lse


def _mut_prefill_prefix_position(q, rows, w_uk, w_uv, d_c, sigma, base, queries=None, heads=None, prefix=0):
    """prefill onto a prefix that rotates the new queries as if they started at
    position 0 (the prefix left out of the query position)."""
    T, H, _ = q.shape
    d_n = w_uk.shape[1]
    o = np.full((T, H, w_uv.shape[1]), np.nan)
    lse = np.full((T, H), np.nan)
    for h in (range(H) if heads is None else heads):
        K = rows[:, :d_c] @ w_uk[h].T
        V = rows[:, :d_c] @ w_uv[h].T
        for i in (range(T) if queries is None else queries):
            n = prefix + i + 1
            s = sigma * (K[:n] @ q[i, h, :d_n] + rows[:n, d_c:] @ O.rope(q[i, h, d_n:], i, base))
            m = s.max()
            w = np.exp(s - m)
            o[i, h] = (w @ V[:n]) / w.sum()
            lse[i, h] = m + math.log(w.sum())
    return o, lse


def _wuk_as_transposed(w_uk):
    """W_UK [H, d_n, d_c] read with the layout [H, d_c, d_n] (a row-major
    buffer taken in the wrong order), given back as [H, d_n, d_c]."""
    H, d_n, d_c = w_uk.shape
    return np.ascontiguousarray(w_uk).reshape(H, d_c, d_n).transpose(0, 2, 1)


def _mut_wuk_transposed(orig, pos):
    """An oracle function that reads its W_UK argument (position pos) with
    the transposed layout.  Applied to decode, prefill, absorption and the
    logits alike, the oracle stays self-consistent, so only pins with their
    own indexing of W_UK can catch it."""
    def f(*args, **kw):
        args = list(args)
        args[pos] = _wuk_as_transposed(np.asarray(args[pos]))
        return orig(*args, **kw)
    return f


# position of the W_UK argument of each oracle function
_WUK_ARG = {"decode_one": 2, "prefill_one": 2, "absorb_query": 1, "nonabsorbed_logits": 2}


def _mut_prefill_no_mask(q, rows, w_uk, w_uv, d_c, sigma, base, queries=None, heads=None, prefix=0):
    """prefill with the causal mask dropped: every query sees every row."""
    T, H, _ = q.shape
    d_n = w_uk.shape[1]
    o = np.full((T, H, w_uv.shape[1]), np.nan)
    lse = np.full((T, H), np.nan)
    for h in (range(H) if heads is None else heads):
        K = rows[:, :d_c] @ w_uk[h].T
        V = rows[:, :d_c] @ w_uv[h].T
        for i in (range(T) if queries is None else queries):
            s = sigma * (K @ q[i, h, :d_n] + rows[:, d_c:] @ O.rope(q[i, h, d_n:], prefix + i, base))
            m = s.max()
            w = np.exp(s - m)
            o[i, h] = (w @ V) / w.sum()
            lse[i, h] = m + math.log(w.sum())
    return o, lse


def _mut_output_value_major(o, w_o):
    """output projection that flattens the head outputs value-major."""
    return np.transpose(o, (0, 2, 1)).reshape(o.shape[0], -1) @ w_o.T


def _mut_query_from_latent_transposed(c_q, w_uq):
    """W_UQ [H, d_n + d_R, d_cq] read with the layout [H, d_cq, d_n + d_R]."""
    H, J, C = w_uq.shape
    return np.einsum("nc,hcj->nhj", c_q, np.ascontiguousarray(w_uq).reshape(H, C, J))


def _mut_attend_log2(scores, values):
    m = float(np.max(scores))
    w = np.exp(scores - m)
    return (w @ values) / w.sum(), m + math.log2(w.sum())


def _mut_quantize_ties_away(x):
    # round half away from zero instead of half to even
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, k = np.frexp(a)
    k = np.maximum(np.where(a > 0, k - 1, -10), -6)
    step = np.exp2(k - 3.0)
    n = np.floor(a / step + 0.5)
    up = n >= 16
    k = np.where(up, k + 1, k)
    n = np.where(up, n / 2, n)
    sub = (k == -6) & (n < 8)
    code = (np.where(sub, 0, k + 7).astype(np.int64) << 3) | np.where(sub, n, n - 8).astype(np.int64)
    code = np.where(np.signbit(x) & (code != 0), code | 0x80, code)
    return code.astype(np.uint8)


def _mut_scale_exponent_plus_one(amax):
    import oracle.mla_oracle as M
    return M._orig_row_scale_exponent(amax) + (1 if amax > 0 else 0)


def _mut_unpack_scales_first(pages, P, R):
    pages = np.asarray(pages, dtype=np.uint8)
    npg = pages.shape[0]
    scales = np.ascontiguousarray(pages[:, :4 * P]).view("<f4").reshape(npg, P).astype(np.float64)
    codes = pages[:, 4 * P:4 * P + P * R].reshape(npg, P, R)
    return codes, scales


@pytest.mark.parametrize("mutation", ["rope_sign", "rope_pairing", "drop_kr", "sigma_content_only",
                                      "causal_off_by_one", "lse_log2", "prefix_position",
                                      "fp8_ties_away", "fp8_scale_exponent", "fp8_scales_first",
                                      "wuk_transposed", "causal_mask_dropped", "output_value_major",
                                      "wuq_transposed"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    import oracle.mla_oracle as M

    def patch(name, fn):
        monkeypatch.setattr(M, name, fn)
        monkeypatch.setattr(O, name, fn, raising=False)

    if mutation == "rope_sign":
        patch("rope", _mut_rope_sign)
    elif mutation == "rope_pairing":
        patch("rope", _mut_rope_halfsplit_q_only)
    elif mutation in ("drop_kr", "sigma_content_only"):
        patch("decode_one", _mut_decode_one(mutation))
    elif mutation == "causal_off_by_one":
        patch("prefill_one", _mut_prefill_peek)
    elif mutation == "lse_log2":
        patch("_attend", _mut_attend_log2)
    elif mutation == "prefix_position":
        patch("prefill_one", _mut_prefill_prefix_position)
    elif mutation == "fp8_ties_away":
        patch("quantize_e4m3", _mut_quantize_ties_away)
    elif mutation == "fp8_scale_exponent":
        monkeypatch.setattr(M, "_orig_row_scale_exponent", M.row_scale_exponent, raising=False)
        patch("row_scale_exponent", _mut_scale_exponent_plus_one)
    elif mutation == "fp8_scales_first":
        patch("unpack_fp8_pages", _mut_unpack_scales_first)
    elif mutation == "wuk_transposed":
        for name, pos in _WUK_ARG.items():
            patch(name, _mut_wuk_transposed(getattr(M, name), pos))
    elif mutation == "causal_mask_dropped":
        patch("prefill_one", _mut_prefill_no_mask)
    elif mutation == "output_value_major":
        patch("output_projection", _mut_output_value_major)
    elif mutation == "wuq_transposed":
        patch("query_from_latent", _mut_query_from_latent_transposed)
    pins = [test_rope_closed_forms, lambda: test_brute_force_decode(0), lambda: test_brute_force_prefill(0),
            test_absorbed_equals_sdpa_mqa, test_causal_prefill_equals_sdpa_causal,
            test_absorbed_and_nonabsorbed_logits_agree, test_single_token_context,
            test_identity_weights_textbook_attention, lambda: test_prefix_prefill_equals_sdpa_bottom_right_mask(7, 5),
            test_prefix_prefill_is_the_tail_of_a_full_prefill, test_prefix_prefill_of_one_token_is_decode,
            test_e4m3_quantize_matches_torch_cast, test_e4m3_quantize_inverts_decode,
            lambda: test_row_scale_exponent_bounds(0.37), test_quantize_row_error_bound_and_scale,
            test_fp8_pages_layout_and_roundtrip, test_fp8_write_one_hot_rows_and_skip,
            lambda: test_folded_query_weights_give_the_same_logits(0),
            lambda: test_folded_output_weights_give_the_same_output(0),
            test_brute_force_query_and_output_projection, test_projected_decode_equals_sdpa_then_output_matmul]
    caught = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught mutation {mutation}"
