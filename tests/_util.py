"""Shared helpers of the test suite: tolerances, oracle runs over the seeded
inputs (the oracle reads the same stored values the GPU reads)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O

# max relative error per output tensor: ||g - o||_inf / ||o||_inf
TOL = {"f32": 1e-4, "bf16": 2e-2}
# max absolute error of the natural-log LSE (values of order ln T + score)
LSE_TOL = {"f32": 1e-4, "bf16": 2e-2}


def spike_lse_tol(dtype, lse_ref) -> float:
    """LSE bound where one score dominates and is huge (the spike tests): the
    bf16 absorbed query carries a relative rounding of up to 2^-9 per element,
    which moves a score whose terms all share one sign by up to 2^-9 of its
    value, and the LSE follows that score."""
    big = float(np.max(np.abs(np.asarray(lse_ref)[np.isfinite(lse_ref)]), initial=0.0))
    return LSE_TOL[dtype] + (2.0 ** -9 * big if dtype == "bf16" else 0.0)


def rel_err(g, o) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if np.isnan(g).any():
        return float("inf")
    den = np.max(np.abs(o))
    return float(np.max(np.abs(g - o)) / (den if den > 0 else 1.0))


def lse_err(g, o) -> float:
    """Largest absolute LSE error; entries that are -inf on both sides (empty
    sequences) count as equal, a -inf on one side only as infinitely wrong."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if np.any(np.isneginf(g) != np.isneginf(o)) or np.isnan(g).any():
        return float("inf")
    fin = ~np.isneginf(o)
    if not np.any(fin):
        return 0.0
    return float(np.max(np.abs(g[fin] - o[fin])))


def full_path(cfg) -> bool:
    """Workloads whose every cached row is written from h in the step (the
    same rule the input builder uses)."""
    return cfg.prefill or cfg.dtype == "f32"


def _weights(cfg, inp):
    w = O.from_storage(inp["w_dkr"], cfg.dtype)
    return w[: cfg.d_c], w[cfg.d_c:]


def seq_rows(cfg, inp, b):
    """float64 rows [L, R] of sequence b as the oracle sees them after this
    step's cache write: rows computed by the oracle from h are rounded to the
    storage type; pre-written rows are the stored values, gathered through the
    block table by the oracle's own page addressing."""
    L = int(inp["seq_lens"][b])
    w_dkv, w_kr = _weights(cfg, inp)
    if full_path(cfg):
        c0, c1 = int(inp["cu_seqlens"][b]), int(inp["cu_seqlens"][b + 1])
        h = O.from_storage(inp["h"][c0:c1], cfg.dtype)
        return O.round_storage(O.latent_rows(h, w_dkv, w_kr, inp["positions"][c0:c1], cfg.rope_base), cfg.dtype)
    rows = O.from_storage(O.gather_rows(inp["rows"], inp["block_table"][b], L), cfg.dtype)
    if L > 0:
        h = O.from_storage(inp["h"][b: b + 1], cfg.dtype)
        new = O.latent_rows(h, w_dkv, w_kr, inp["positions"][b: b + 1], cfg.rope_base)
        rows[L - 1] = O.round_storage(new, cfg.dtype)[0]
    return rows


def oracle_decode(cfg, inp, seqs, heads=None):
    """o [len(seqs), H, d_v], lse [len(seqs), H] for the listed sequences."""
    q = O.from_storage(inp["q"], cfg.dtype)
    w_uk = O.from_storage(inp["w_uk"], cfg.dtype)
    w_uv = O.from_storage(inp["w_uv"], cfg.dtype)
    os_, ls_ = [], []
    for b in seqs:
        rows = seq_rows(cfg, inp, b)
        o, l = O.decode_one(q[b], rows, w_uk, w_uv, int(inp["seq_lens"][b]) - 1, cfg.d_c, cfg.softmax_scale,
                            cfg.rope_base, heads=heads)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
