"""mla_write_absorb (the decode step's cache write and query absorption in
one launch) against the two separate calls: the cache pool and the absorbed
queries must be bit-identical, on the fused path and on the sequential one."""
import numpy as np
import pytest
import torch

from mla_latent_kv_22_amd import harness, inputs as I, mla
from tests._util import need_gpu

pytestmark = pytest.mark.gpu


# fused: the case meets the one-launch conditions (bf16, 1..64 tokens, d_n = 128,
# d_c = 512); the others take the two calls in sequence
@pytest.mark.parametrize("cfg,fused", [
    (I.scaled(I.V3, seq_len=128, paged=True), True),                            # 64 tokens, D = 7168, H = 128
    (I.scaled(I.V3, hidden=512, batch=3, seq_len=150, paged=True), True),       # 3 tokens
    (I.scaled(I.V3, hidden=1024, batch=37, seq_len=100, paged=True), True),     # 37 tokens: ragged token tiles
    (I.scaled(I.V2LITE, batch=64, seq_len=96), True),                           # H = 16
    (I.scaled(I.V3, hidden=512, batch=70, seq_len=64, paged=True), False),      # 70 tokens: two calls
    (I.TINY, False),                                                            # fp32: two calls
], ids=["v3_64", "v3dims_3", "v3dims_37", "v2lite_64", "v3dims_70_sequential", "tiny_f32_sequential"])
def test_write_absorb_matches_separate_calls(cfg, fused):
    need_gpu()
    print(f"[case] write_absorb {cfg.name} B={cfg.batch} D={cfg.hidden} H={cfg.num_heads} fused={fused}", flush=True)
    inp = I.make(cfg, 3)
    slots = inp["slots"].copy()
    slots[::7] = -1  # skipped tokens
    inp = dict(inp, slots=slots)
    a = harness.DecodeStep(cfg, inp)
    b = harness.DecodeStep(cfg, inp)
    a.write()
    a.absorb()
    b.write_absorb()
    torch.cuda.synchronize()
    assert np.array_equal(harness.to_host_bits(a.pool), harness.to_host_bits(b.pool)), "cache pools differ"
    assert np.array_equal(harness.to_host_bits(a.q_abs), harness.to_host_bits(b.q_abs)), "absorbed queries differ"


def test_write_absorb_empty_parts():
    """No rows to write: only the absorption runs; no queries: only the write."""
    need_gpu()
    print("[case] write_absorb empty parts", flush=True)
    cfg = I.scaled(I.V3, hidden=512, batch=5, seq_len=64, paged=True)
    inp = I.make(cfg, 4)
    a = harness.DecodeStep(cfg, inp)
    b = harness.DecodeStep(cfg, inp)
    a.absorb()
    mla.write_absorb(b.d, None, b.w_dkr, b.positions, b.slots, b.pool, b.q, b.w_uk, b.q_positions, b.q_abs)
    torch.cuda.synchronize()
    assert np.array_equal(harness.to_host_bits(a.q_abs), harness.to_host_bits(b.q_abs))
    assert np.array_equal(harness.to_host_bits(a.pool), harness.to_host_bits(b.pool))  # pool untouched
    a.write()
    mla.write_absorb(b.d, b.h, b.w_dkr, b.positions, b.slots, b.pool, None, b.w_uk, b.q_positions, b.q_abs)
    torch.cuda.synchronize()
    assert np.array_equal(harness.to_host_bits(a.pool), harness.to_host_bits(b.pool))
