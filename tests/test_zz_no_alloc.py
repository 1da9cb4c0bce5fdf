"""mla_decode_noalloc (the decode entry point that allocates nothing: its
partial results live in the library's per-device scratch array) against
mla_decode with a workspace, through the C ABI, on two calls in a row, the
second with a smaller input; plus its size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from mla_latent_kv_22_amd import harness, inputs as I, mla
from tests._util import LSE_TOL, TOL, lse_err, need_gpu, oracle_decode, rel_err

pytestmark = pytest.mark.gpu


def _case(label):
    print(f"[case] {label}", flush=True)


def _pair(cfg, seed, flags=0, lengths=None):
    """(workspace outputs, no-alloc outputs, step) on one input."""
    inp = I.make(cfg, seed, lengths=lengths)
    st = harness.DecodeStep(cfg, inp, flags=flags)
    st.step()
    torch.cuda.synchronize()
    ref_out, ref_lse = harness.to_host_bits(st.out).copy(), st.lse.cpu().numpy().copy()
    st.out.zero_()
    st.lse.fill_(123.0)
    mla.decode_noalloc(st.d, st.q_abs, st.pool, st.block_table, st.seq_lens, st.max_seq_len, st.w_uv, st.out, st.lse)
    torch.cuda.synchronize()
    return inp, (ref_out, ref_lse), (harness.to_host_bits(st.out).copy(), st.lse.cpu().numpy().copy())


@pytest.mark.parametrize("flags", [0, mla.FLAG_GENERIC], ids=["mfma", "generic"])
def test_noalloc_matches_workspace_decode_twice(flags):
    need_gpu()
    big = I.scaled(I.RAGGED, hidden=512, batch=6, seq_len=3000, min_seq_len=200)
    small = I.scaled(I.RAGGED, hidden=512, batch=3, seq_len=700, min_seq_len=1)
    for cfg, seed in ((big, 5), (small, 6)):
        _case(f"noalloc vs workspace {cfg.name} B={cfg.batch} T<={cfg.seq_len} flags={flags}")
        inp, (ro, rl), (go, gl) = _pair(cfg, seed, flags)
        # same kernels and, at these sizes, the same work split: identical bits
        assert np.array_equal(go, ro) and np.array_equal(gl, rl)
        o_ref, l_ref = oracle_decode(cfg, inp, list(range(cfg.batch)))
        e_o = rel_err(O.from_storage(go, cfg.dtype), o_ref)
        e_l = lse_err(gl.astype(np.float64), l_ref)
        print(f"  out rel err {e_o:.3e}  lse err {e_l:.3e}", flush=True)
        assert e_o < TOL[cfg.dtype] and e_l < LSE_TOL[cfg.dtype]


def test_noalloc_v3_shape_and_size_limit():
    need_gpu()
    _case("noalloc at the V3 decode shape, then a call beyond the scratch size")
    cfg = I.scaled(I.V3, batch=16, seq_len=4096)
    inp, (ro, rl), (go, gl) = _pair(cfg, 0)
    assert np.array_equal(go, ro) and np.array_equal(gl, rl)
    d = harness.dims_for(cfg)
    L = mla.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    # 4096 sequences of 8192 tokens need far more than the scratch holds
    st = L.mla_decode_noalloc(ctypes.byref(d), fake, fake, 4, fake, 1 << 16, fake, 4096, 8192, fake, fake, None,
                              None)
    assert st == -4  # MLA_ERR_WORKSPACE
