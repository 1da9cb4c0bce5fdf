"""GPU parity of the causal prefill (cache write of every token, then causal
attention with per-head K/V up-projected from the latent) against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from mla_latent_kv_22_amd import harness, inputs as I
from tests._util import TOL, lse_err, need_gpu, rel_err, seq_rows

pytestmark = pytest.mark.gpu


def _run(cfg, inp):
    pf = harness.Prefill(cfg, inp)
    pf.write()
    pf.attend()
    torch.cuda.synchronize()
    return pf


def _check(cfg, inp, pf, seq, queries=None, heads=None):
    c0 = int(inp["cu_seqlens"][seq])
    L = int(inp["seq_lens"][seq])
    rows = seq_rows(cfg, inp, seq)
    q = O.from_storage(inp["q"][c0:c0 + L], cfg.dtype)
    o_ref, l_ref = O.prefill_one(q, rows, O.from_storage(inp["w_uk"], cfg.dtype),
                                 O.from_storage(inp["w_uv"], cfg.dtype), cfg.d_c, cfg.softmax_scale,
                                 cfg.rope_base, queries=queries, heads=heads)
    out = O.from_storage(harness.to_host_bits(pf.out[c0:c0 + L]), cfg.dtype)
    lse = pf.lse[c0:c0 + L].cpu().numpy().astype(np.float64)
    qi = np.arange(L) if queries is None else np.asarray(queries)
    hi = np.arange(cfg.num_heads) if heads is None else np.asarray(heads)
    sel = np.ix_(qi, hi)
    e_o, e_l = rel_err(out[sel], o_ref[sel]), lse_err(lse[sel], l_ref[sel])
    print(f"  seq {seq}: out rel err {e_o:.3e}  lse err {e_l:.3e}", flush=True)
    assert e_o < TOL[cfg.dtype] and e_l < TOL[cfg.dtype]


@pytest.mark.parametrize("cfg", [
    I.scaled(I.PREFILL, hidden=256, num_heads=8, batch=3, seq_len=130, min_seq_len=1),
    I.scaled(I.PREFILL, hidden=128, num_heads=4, batch=2, seq_len=70, min_seq_len=1, d_c=64, d_r=16,
             qk_nope=32, v_head=48, dtype="f32"),
], ids=["v3dims_bf16", "small_f32"])
def test_prefill_small(cfg):
    need_gpu()
    print(f"[case] prefill small {cfg.name} {cfg.dtype}", flush=True)
    inp = I.make(cfg, 3)
    pf = _run(cfg, inp)
    for s in range(cfg.batch):
        _check(cfg, inp, pf, s)


@pytest.mark.slow
def test_prefill_full_size_sampled():
    """4 x 4096 tokens, H=128: sequence 0 at 12 query rows (first, last and
    spread) over all heads, sequence 3 at 4 rows over 16 heads."""
    need_gpu()
    print("[case] prefill full size", flush=True)
    cfg = I.PREFILL
    inp = I.make(cfg, 0)
    pf = _run(cfg, inp)
    _check(cfg, inp, pf, 0, queries=[0, 1, 2, 63, 64, 65, 1000, 2047, 2048, 3333, 4094, 4095])
    _check(cfg, inp, pf, 3, queries=[0, 777, 4000, 4095], heads=list(range(0, 128, 8)))
