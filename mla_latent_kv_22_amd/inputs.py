"""Seeded synthetic inputs for the MLA latent-cache path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no projection, no RoPE, no attention).  Both the CPU
oracle and the HIP path receive exactly the arrays built here: bf16 values are
carried as their raw 16-bit patterns (numpy ``uint16``), fp32 values as
``float32``.

Workloads follow the shapes of the pages' running example (DeepSeek-V2/V3 MLA:
latent width d_c = kv_lora_rank = 512, decoupled rotary key width d_R =
qk_rope_head_dim = 64; LLMScale page, section "Multi-head latent attention
(MLA)") and the five decode / prefill workloads this library is measured on.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` stream):
  1. sequence lengths (ragged workload only)
  2. page permutation (paged workloads only)
  3. W_DKV, W_KR, W_UK, W_UV           ~ N(0, 0.02^2)
  4. hidden states h                    ~ N(0, 1)
  5. pre-written latent rows            ~ N(0, 1)   (decode-only workloads)
  6. queries q = [q_C | q_R] per head   ~ N(0, 0.02^2 * hidden)
The query projection W_Q.h is the caller's GEMM and sits outside the library,
so q is drawn directly with the variance W_Q.h has under the stated init.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np

PAGE_SIZE = 64
WEIGHT_STD = 0.02
ROPE_BASE = 10000.0


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    hidden: int
    num_heads: int
    d_c: int
    d_r: int
    qk_nope: int
    v_head: int
    dtype: str            # "f32" or "bf16"
    batch: int
    seq_len: int          # context length T (max length for ragged)
    min_seq_len: int = 0  # >0 selects ragged lengths U{min_seq_len .. seq_len}
    paged: bool = False   # random page permutation instead of contiguous pages
    prefill: bool = False
    page_size: int = PAGE_SIZE
    rope_base: float = ROPE_BASE
    weight_std: float = WEIGHT_STD

    @property
    def row_width(self) -> int:
        return self.d_c + self.d_r

    @property
    def qk_head(self) -> int:
        return self.qk_nope + self.d_r

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt of the per-head score width of the non-absorbed form.
        return 1.0 / float(np.sqrt(self.qk_nope + self.d_r))


TINY = Config("tiny_f32", 256, 8, 64, 16, 32, 32, "f32", 2, 256)
V2LITE = Config("v2lite_decode", 2048, 16, 512, 64, 128, 128, "bf16", 16, 4096)
V3 = Config("v3_decode", 7168, 128, 512, 64, 128, 128, "bf16", 64, 8192)
RAGGED = Config("v3_paged_ragged", 7168, 128, 512, 64, 128, 128, "bf16", 128, 32768,
                min_seq_len=512, paged=True)
PREFILL = Config("v3_prefill", 7168, 128, 512, 64, 128, 128, "bf16", 4, 4096,
                 paged=True, prefill=True)
CONFIGS: Dict[str, Config] = {c.name: c for c in (TINY, V2LITE, V3, RAGGED, PREFILL)}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **kw)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit pattern (storage conversion)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _normal(rng: np.random.Generator, shape, std: float, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, std^2) drawn in float32 chunks (bounded host memory), stored as dtype."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:e] = _store(v, dtype)
    return out.reshape(shape)


def seq_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.min_seq_len > 0:
        return rng.integers(cfg.min_seq_len, cfg.seq_len, size=cfg.batch, endpoint=True).astype(np.int32)
    return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)


def make(cfg: Config, seed: int = 0, with_rows: bool = True,
         lengths=None) -> Dict[str, np.ndarray]:
    """Build every input of one step of ``cfg``.

    Returns a dict with:
      seq_lens   int32 [B]          context length per sequence (decode) / tokens per sequence (prefill)
      block_table int32 [B, max_pages]  page holding tokens i*P .. i*P+P-1 of sequence b
      num_pages  int                pool size in pages
      w_dkr      [R, D]             rows 0..d_c-1 = W_DKV, rows d_c..R-1 = W_KR
      w_uk       [H, d_n, d_c]      K_C,h = W_UK,h . c
      w_uv       [H, d_v, d_c]      V_h   = W_UV,h . c
      h          [N, D]             hidden states of the tokens written this step
      positions  int32 [N]          their positions
      slots      int64 [N]          their cache slots (page * P + offset)
      rows       [num_pages, P, R]  pre-written latent rows (decode workloads; zero rows elsewhere)
      q          [Nq, H, d_n+d_R]   pre-RoPE queries ([q_C | q_R] per head)
      q_positions int32 [Nq]
    """
    rng = np.random.default_rng(seed)
    P = cfg.page_size
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int32)
        assert lens.shape == (cfg.batch,)
    else:
        lens = seq_lengths(cfg, rng)
    pages_per_seq = (lens.astype(np.int64) + P - 1) // P
    num_pages = int(pages_per_seq.sum())
    max_pages = int(pages_per_seq.max())
    if cfg.paged:
        perm = rng.permutation(num_pages).astype(np.int32)
    else:
        perm = np.arange(num_pages, dtype=np.int32)
    block_table = np.zeros((cfg.batch, max_pages), dtype=np.int32)
    start = 0
    for b in range(cfg.batch):
        n = int(pages_per_seq[b])
        block_table[b, :n] = perm[start:start + n]
        start += n

    R, D, H = cfg.row_width, cfg.hidden, cfg.num_heads
    w_dkv = _normal(rng, (cfg.d_c, D), cfg.weight_std, cfg.dtype)
    w_kr = _normal(rng, (cfg.d_r, D), cfg.weight_std, cfg.dtype)
    w_uk = _normal(rng, (H, cfg.qk_nope, cfg.d_c), cfg.weight_std, cfg.dtype)
    w_uv = _normal(rng, (H, cfg.v_head, cfg.d_c), cfg.weight_std, cfg.dtype)
    w_dkr = np.concatenate([w_dkv, w_kr], axis=0)

    full_path = cfg.prefill or cfg.dtype == "f32"
    if full_path:
        # every context token is projected and written by the cache-write step
        positions = np.concatenate([np.arange(int(L), dtype=np.int32) for L in lens])
        seq_of_tok = np.repeat(np.arange(cfg.batch), lens)
    else:
        # decode: the newest token of each sequence is written this step
        # (an empty sequence writes nothing: slot -1)
        positions = np.maximum(lens - 1, 0).astype(np.int32)
        seq_of_tok = np.arange(cfg.batch)
    slots = (block_table[seq_of_tok, positions // P].astype(np.int64) * P + positions % P).astype(np.int64)
    if not full_path:
        slots[lens == 0] = -1
    h = _normal(rng, (positions.shape[0], D), 1.0, cfg.dtype)

    if with_rows and not full_path:
        rows = _normal(rng, (num_pages, P, R), 1.0, cfg.dtype)
    else:
        rows = np.zeros((num_pages, P, R), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)

    q_std = cfg.weight_std * float(np.sqrt(D))
    if cfg.prefill:
        q_positions = positions.copy()
    else:
        q_positions = np.maximum(lens - 1, 0).astype(np.int32)
    q = _normal(rng, (q_positions.shape[0], H, cfg.qk_head), q_std, cfg.dtype)
    cu = np.zeros(cfg.batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(seq_lens=lens, block_table=block_table, num_pages=num_pages, w_dkr=w_dkr,
                w_uk=w_uk, w_uv=w_uv, h=h, positions=positions, slots=slots, rows=rows,
                q=q, q_positions=q_positions, cu_seqlens=cu)


# query rank of the query compression; no workload names one, so the V3
# shapes take DeepSeek-V3's (1536) and the tiny fp32 shape a small one
Q_RANK = {"tiny_f32": 48}
Q_RANK_DEFAULT = 1536


def projection_inputs(cfg: Config, n_tokens: int, seed: int, d_cq: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of the query compression and the output projection, drawn from
    their own stream (fixed order): W_DQ [d_cq, D], W_UQ [H, d_n + d_R, d_cq],
    W_O [D, H d_v] ~ N(0, std^2) with the workload's weight std; hidden states
    h [n_tokens, D] ~ N(0, 1); positions U{0 .. seq_len - 1}; attention
    outputs o [n_tokens, H, d_v] ~ N(0, 1/64) (the order of a softmax average
    of W_UV-projected N(0, 1) rows)."""
    rng = np.random.default_rng(seed)
    d_cq = d_cq or Q_RANK.get(cfg.name, Q_RANK_DEFAULT)
    D, H = cfg.hidden, cfg.num_heads
    w_dq = _normal(rng, (d_cq, D), cfg.weight_std, cfg.dtype)
    w_uq = _normal(rng, (H, cfg.qk_head, d_cq), cfg.weight_std, cfg.dtype)
    w_o = _normal(rng, (D, H * cfg.v_head), cfg.weight_std, cfg.dtype)
    h = _normal(rng, (n_tokens, D), 1.0, cfg.dtype)
    positions = rng.integers(0, cfg.seq_len, size=n_tokens).astype(np.int32)
    o = _normal(rng, (n_tokens, H, cfg.v_head), 0.125, cfg.dtype)
    return dict(d_cq=d_cq, w_dq=w_dq, w_uq=w_uq, w_o=w_o, h=h, positions=positions, o=o)


def fp8_pages(num_pages: int, P: int, R: int, rng: np.random.Generator) -> np.ndarray:
    """Random 8-bit cache pages [num_pages, P * (R + 4)] for decode inputs:
    per page, P rows of R E4M3 codes (random sign, exponent field 4..7 so the
    values lie between 1/8 and 15/8, any mantissa; one code in 32 is zero and
    one in 32 a subnormal), then P float32 row scales 2^k with k drawn from
    -1..1 (stored values of the order of N(0, 1) rows).  A plain random draw
    of the stored format, not a quantization."""
    shape = (num_pages, P, R)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << np.uint8(7)
    ef = rng.integers(4, 8, size=shape, dtype=np.uint8)
    mf = rng.integers(0, 8, size=shape, dtype=np.uint8)
    kind = rng.integers(0, 32, size=shape)
    ef = np.where(kind == 0, 0, ef).astype(np.uint8)                 # subnormal (or zero when mf = 0)
    mf = np.where(kind == 1, 0, mf).astype(np.uint8)
    ef = np.where(kind == 1, 0, ef).astype(np.uint8)                 # zero
    codes = (sign | (ef << np.uint8(3)) | mf).astype(np.uint8)
    codes = np.where(codes == 0x80, 0, codes).astype(np.uint8)
    scales = np.exp2(rng.integers(-1, 2, size=(num_pages, P))).astype("<f4")
    out = np.empty((num_pages, P * (R + 4)), dtype=np.uint8)
    out[:, :P * R] = codes.reshape(num_pages, P * R)
    out[:, P * R:] = scales.view(np.uint8).reshape(num_pages, 4 * P)
    return out


def digest(arrays: Dict[str, np.ndarray]) -> str:
    """sha256 over the raw bytes of every array (determinism check)."""
    m = hashlib.sha256()
    for k in sorted(arrays):
        v = arrays[k]
        m.update(k.encode())
        m.update(np.ascontiguousarray(np.asarray(v)).tobytes())
    return m.hexdigest()
