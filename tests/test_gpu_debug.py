"""The MLA_DEBUG library (libmla_debug.so, same ABI) on the GPU.  On valid
inputs it gives the release library's bits and a device error word of 0.
With a corrupted block table, slot mapping, sequence lengths or prefill
offsets, every kernel still exits normally: the error word names the fault,
a bad block-table entry acts as page 0 and a bad slot is skipped.  The
corrupted inputs are only ever given to the debug library, whose kernels
check each entry before forming an address from it (the predicates are the
ones tests/test_checks_host.py proves on the CPU)."""
import numpy as np
import pytest
import torch

from mla_latent_kv_22_amd import harness, inputs as I, mla
from tests._util import need_gpu

pytestmark = pytest.mark.gpu


def _case(label):
    print(f"[case] {label}", flush=True)


CFG = I.scaled(I.RAGGED, hidden=512, batch=6, seq_len=3000, min_seq_len=200)


def _decode(cfg, inp, flags=0):
    st = harness.DecodeStep(cfg, inp, flags=flags)
    st.step()
    torch.cuda.synchronize()
    return harness.to_host_bits(st.out).copy(), st.lse.cpu().numpy().copy()


@pytest.mark.parametrize("flags", [0, mla.FLAG_GENERIC], ids=["mfma", "generic"])
def test_debug_build_valid_inputs_same_bits(flags):
    need_gpu()
    _case(f"debug build, valid decode inputs, flags={flags}")
    inp = I.make(CFG, 5)
    out_r, lse_r = _decode(CFG, inp, flags)
    assert mla.get_device_error() == 0  # the release library never sets the word
    with mla.debug_library():
        assert mla.debug_build()
        assert mla.get_device_error() == 0
        out_d, lse_d = _decode(CFG, inp, flags)
        assert mla.get_device_error() == 0
    assert np.array_equal(out_d, out_r) and np.array_equal(lse_d, lse_r)


def test_debug_build_bad_block_table_entries():
    need_gpu()
    _case("debug build, block-table entries out of range")
    inp = I.make(CFG, 6)
    npg = int(inp["num_pages"])
    bad = inp["block_table"].copy()
    bad[1, 2] = npg + 7
    bad[3, 0] = -5
    bad[5, 10] = 2 ** 31 - 1
    # what the debug kernels must compute: the bad entries read as page 0
    ref_bt = bad.copy()
    ref_bt[1, 2] = ref_bt[3, 0] = ref_bt[5, 10] = 0
    out_r, lse_r = _decode(CFG, dict(inp, block_table=ref_bt))
    for flags in (0, mla.FLAG_GENERIC):
        with mla.debug_library():
            mla.get_device_error()
            out_d, lse_d = _decode(CFG, dict(inp, block_table=bad), flags)
            err = mla.get_device_error()
        print(f"  flags={flags} error word {err}", flush=True)
        assert err == mla.DEVERR_PAGE
        if flags == 0:
            assert np.array_equal(out_d, out_r) and np.array_equal(lse_d, lse_r)
        assert np.all(np.isfinite(lse_d))


def test_debug_build_bad_slots_are_skipped():
    need_gpu()
    _case("debug build, slots out of range")
    cfg = I.scaled(I.V3, hidden=512, batch=5, seq_len=150, paged=True)
    inp = I.make(cfg, 1)
    npg, P, R = int(inp["num_pages"]), cfg.page_size, cfg.row_width
    slots = inp["slots"].copy()
    slots[1] = npg * P + 100
    slots[3] = -9
    sentinel = np.full(inp["rows"].shape, 0xC0E8, dtype=np.uint16)
    ref_slots = slots.copy()
    ref_slots[1] = ref_slots[3] = -1
    st = harness.DecodeStep(cfg, dict(inp, slots=ref_slots), pool=harness.to_device(sentinel, "bf16"))
    st.write()
    torch.cuda.synchronize()
    ref = harness.to_host_bits(st.pool).copy()
    with mla.debug_library():
        mla.get_device_error()
        st = harness.DecodeStep(cfg, dict(inp, slots=slots), pool=harness.to_device(sentinel, "bf16"))
        st.write()
        err = mla.get_device_error()
    assert err == mla.DEVERR_SLOT
    assert np.array_equal(harness.to_host_bits(st.pool), ref)


def test_debug_build_lengths_beyond_bounds():
    need_gpu()
    _case("debug build, decode lengths and prefill offsets beyond their bounds")
    inp = I.make(CFG, 7)
    lens = inp["seq_lens"].copy()
    cap = int(lens.max())
    longest = int(np.argmax(lens))
    lens[longest] = cap + 50  # longer than max_seq_len: clamped to it (its pages cover cap tokens)
    short = (longest + 1) % len(lens)
    lens[short] = -3          # negative: an empty sequence
    with mla.debug_library():
        mla.get_device_error()
        st = harness.DecodeStep(CFG, inp)
        st.seq_lens = harness.to_device(lens.astype(np.int32), "i32")
        st.max_seq_len = cap
        st.absorb()
        st.attend()
        err = mla.get_device_error()
    assert err == mla.DEVERR_LENGTH
    assert np.all(np.isneginf(st.lse.cpu().numpy()[short]))
    # prefill: cu_seqlens whose second entry lies far past the tokens
    pcfg = I.scaled(I.PREFILL, hidden=512, batch=2, seq_len=100)
    pin = I.make(pcfg, 3)
    with mla.debug_library():
        pf = harness.Prefill(pcfg, pin)
        pf.write()
        assert mla.get_device_error() == 0
        cu = pin["cu_seqlens"].copy()
        cu[1] = 10 ** 6
        pf.cu = harness.to_device(cu.astype(np.int32), "i32")
        pf.attend()
        err = mla.get_device_error()
    assert err == mla.DEVERR_LENGTH
