"""Host-side plumbing shared by the tests and the benchmark: dims from a
workload description, uploads of the seeded inputs, and one decode step /
prefill through the C ABI.  No method arithmetic lives here."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import mla
from .inputs import Config


def dims_for(cfg: Config, flags: int = 0) -> mla.Dims:
    return mla.make_dims(cfg.hidden, cfg.num_heads, cfg.d_c, cfg.d_r, cfg.qk_nope, cfg.v_head, cfg.page_size,
                         cfg.dtype, cfg.rope_base, cfg.softmax_scale, flags)


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload a host array; bf16 arrays arrive as uint16 bit patterns."""
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 as uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DecodeStep:
    """Device buffers of one decode step: write the newest rows, absorb the
    queries, run split-T decode + combine."""

    def __init__(self, cfg: Config, inp: Dict[str, np.ndarray], flags: int = 0, device="cuda",
                 pool: Optional[torch.Tensor] = None):
        self.cfg, self.d = cfg, dims_for(cfg, flags)
        dt = cfg.dtype
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.pool = pool if pool is not None else to_device(inp["rows"], dt, device)
        self.w_dkr = to_device(inp["w_dkr"], dt, device)
        self.w_uk = to_device(inp["w_uk"], dt, device)
        self.w_uv = to_device(inp["w_uv"], dt, device)
        self.h = to_device(inp["h"], dt, device)
        self.positions = to_device(inp["positions"], "i32", device)
        self.slots = to_device(inp["slots"], "i64", device)
        self.q = to_device(inp["q"], dt, device)
        self.q_positions = to_device(inp["q_positions"], "i32", device)
        self.block_table = to_device(inp["block_table"], "i32", device)
        self.seq_lens = to_device(inp["seq_lens"], "i32", device)
        self.max_seq_len = int(inp["seq_lens"].max()) if len(inp["seq_lens"]) else 0
        B, H = cfg.batch, cfg.num_heads
        self.q_abs = torch.empty((B, H, cfg.row_width), dtype=tdt, device=device)
        self.out = torch.empty((B, H, cfg.v_head), dtype=tdt, device=device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=device)
        ws = mla.decode_workspace_size(self.d, B, self.max_seq_len)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        # the cache write's workspace: 8-bit row staging and the split-K partials
        wws = mla.write_cache_workspace_size(self.d, int(inp["h"].shape[0]))
        self.write_ws = torch.empty(max(wws, 1), dtype=torch.uint8, device=device)
        # mla_write_absorb's workspace: counters (zero before the first call) and partials
        waws = mla.write_absorb_workspace_size(self.d, int(inp["h"].shape[0]))
        self.wa_ws = torch.zeros(max(waws, 1), dtype=torch.uint8, device=device)

    def write(self, stream=None, pool=None):
        mla.write_cache(self.d, self.h, self.w_dkr, self.positions, self.slots, self.pool if pool is None else pool,
                        stream, workspace=self.write_ws)

    def write_absorb(self, stream=None, pool=None):
        """The cache write and the absorption in one call (mla_write_absorb)."""
        mla.write_absorb(self.d, self.h, self.w_dkr, self.positions, self.slots, self.pool if pool is None else pool,
                         self.q, self.w_uk, self.q_positions, self.q_abs, self.wa_ws, stream)

    def absorb(self, stream=None):
        mla.absorb_q(self.d, self.q, self.w_uk, self.q_positions, self.q_abs, stream)

    def attend(self, stream=None, pool=None):
        mla.decode(self.d, self.q_abs, self.pool if pool is None else pool, self.block_table, self.seq_lens,
                   self.max_seq_len, self.w_uv, self.out, self.lse, self.workspace, stream)

    def step(self, stream=None, pool=None, side_stream=None, fused=True):
        """Cache write, absorption, decode.  By default the first two are one
        mla_write_absorb call; fused=False makes them two calls.  With
        side_stream, the cache write (which only touches the new rows) runs
        there concurrently with the absorption, and decode waits for both."""
        pool = self.pool if pool is None else pool
        main = stream if stream is not None else torch.cuda.current_stream()
        if side_stream is not None:
            side_stream.wait_stream(main)
            self.write(side_stream, pool)
            self.absorb(main)
            main.wait_stream(side_stream)
        elif fused:
            self.write_absorb(main, pool)
        else:
            self.write(main, pool)
            self.absorb(main)
        self.attend(main, pool)


class Prefill:
    """Device buffers of one prefill: write every row, then causal attention."""

    def __init__(self, cfg: Config, inp: Dict[str, np.ndarray], flags: int = 0, device="cuda"):
        self.cfg, self.d = cfg, dims_for(cfg, flags)
        dt = cfg.dtype
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.pool = to_device(inp["rows"], dt, device)
        self.w_dkr = to_device(inp["w_dkr"], dt, device)
        self.w_uk = to_device(inp["w_uk"], dt, device)
        self.w_uv = to_device(inp["w_uv"], dt, device)
        self.h = to_device(inp["h"], dt, device)
        self.positions = to_device(inp["positions"], "i32", device)
        self.slots = to_device(inp["slots"], "i64", device)
        self.q = to_device(inp["q"], dt, device)
        self.block_table = to_device(inp["block_table"], "i32", device)
        self.cu = to_device(inp["cu_seqlens"], "i32", device)
        self.max_seq_len = int(inp["seq_lens"].max())
        N, H = self.q.shape[0], cfg.num_heads
        self.out = torch.empty((N, H, cfg.v_head), dtype=tdt, device=device)
        self.lse = torch.empty((N, H), dtype=torch.float32, device=device)
        ws = mla.prefill_workspace_size(self.d, N)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)

    def write(self, stream=None):
        mla.write_cache(self.d, self.h, self.w_dkr, self.positions, self.slots, self.pool, stream)

    def attend(self, stream=None):
        mla.prefill(self.d, self.q, self.pool, self.block_table, self.cu, self.max_seq_len, self.w_uk, self.w_uv,
                    self.out, self.lse, self.workspace, stream)
