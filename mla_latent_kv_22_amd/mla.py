"""ctypes binding of libmla.so (C ABI in include/mla.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, and a negative status becomes an exception.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  Importing this module does not load the library; the first call
does, and raises if it is missing.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")
# the same ABI built with MLA_DEBUG: device-side index checks and the error word
DEBUG_LIB_PATH = os.path.join(_HERE, "libmla_debug.so")

F32, BF16 = 0, 1
FLAG_GENERIC = 1
FLAG_FP8_CACHE = 2
OP_WRITE_CACHE, OP_ABSORB_Q, OP_DECODE, OP_PREFILL = 0, 1, 2, 3

_SYMBOLS = ("mla_write_cache", "mla_write_cache_ws", "mla_write_cache_workspace_size", "mla_absorb_q",
            "mla_decode_workspace_size", "mla_decode", "mla_prefill_workspace_size", "mla_prefill",
            "mla_prefill_kv", "mla_cache_bytes", "mla_page_bytes", "mla_status_string", "mla_uses_fast_path",
            "mla_get_device_error", "mla_debug_build", "mla_decode_noalloc", "mla_project_q_workspace_size",
            "mla_project_q", "mla_project_out_workspace_size", "mla_project_out", "mla_write_absorb",
            "mla_write_absorb_workspace_size")
DEVERR_PAGE, DEVERR_SLOT, DEVERR_LENGTH = 1, 2, 4


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_c", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("qk_nope", ctypes.c_int32), ("v_head", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_int32)]


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_libs = {}
_use_debug = False


@contextlib.contextmanager
def debug_library():
    """Route the calls of this module through libmla_debug.so inside the block."""
    global _use_debug
    old, _use_debug = _use_debug, True
    try:
        yield lib()
    finally:
        _use_debug = old


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built): libmla.so, or
    libmla_debug.so inside ``debug_library()``."""
    path = DEBUG_LIB_PATH if _use_debug else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m mla_latent_kv_22_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        L.mla_write_cache.argtypes = [dp, vp, vp, vp, vp, i32, vp, i32, vp]
        L.mla_write_cache_ws.argtypes = [dp, vp, vp, vp, vp, i32, vp, i32, vp, sz, vp]
        L.mla_write_cache_workspace_size.argtypes = [dp, i32]
        L.mla_write_cache_workspace_size.restype = sz
        L.mla_page_bytes.argtypes = [dp]
        L.mla_page_bytes.restype = sz
        L.mla_absorb_q.argtypes = [dp, vp, vp, vp, i32, vp, vp]
        L.mla_decode_workspace_size.argtypes = [dp, i32, i32]
        L.mla_decode_workspace_size.restype = sz
        L.mla_decode.argtypes = [dp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.mla_decode_noalloc.argtypes = [dp, vp, vp, i32, vp, i32, vp, i32, i32, vp, vp, vp, vp]
        L.mla_prefill_workspace_size.argtypes = [dp, i32]
        L.mla_prefill_workspace_size.restype = sz
        L.mla_prefill.argtypes = [dp, vp, vp, i32, vp, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.mla_prefill_kv.argtypes = [dp, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.mla_cache_bytes.argtypes = [dp, i64, i32]
        L.mla_cache_bytes.restype = sz
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_uses_fast_path.argtypes = [dp, i32]
        L.mla_get_device_error.argtypes = [ctypes.POINTER(ctypes.c_int32), vp]
        L.mla_project_q_workspace_size.argtypes = [dp, i32, i32]
        L.mla_project_q_workspace_size.restype = sz
        L.mla_project_q.argtypes = [dp, i32, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
        L.mla_project_out_workspace_size.argtypes = [dp, i32]
        L.mla_project_out_workspace_size.restype = sz
        L.mla_project_out.argtypes = [dp, vp, vp, i32, vp, vp, sz, vp]
        L.mla_debug_build.argtypes = []
        L.mla_write_absorb.argtypes = [dp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, i32, vp, vp, sz, vp]
        L.mla_write_absorb_workspace_size.argtypes = [dp, i32]
        L.mla_write_absorb_workspace_size.restype = sz
        for f in ("mla_write_cache", "mla_write_cache_ws", "mla_absorb_q", "mla_decode", "mla_decode_noalloc",
                  "mla_prefill",
                  "mla_prefill_kv", "mla_uses_fast_path", "mla_get_device_error", "mla_debug_build",
                  "mla_project_q", "mla_project_out", "mla_write_absorb"):
            getattr(L, f).restype = ctypes.c_int
        _libs[path] = L
    return _libs[path]


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def make_dims(hidden, num_heads, d_c, d_r, qk_nope, v_head, page_size, dtype, rope_base, softmax_scale,
              flags=0) -> Dims:
    return Dims(hidden, num_heads, d_c, d_r, qk_nope, v_head, page_size,
                BF16 if dtype in ("bf16", BF16, torch.bfloat16) else F32, rope_base, softmax_scale, flags)


# --------------------------------------------------------------------------- helpers

def _torch_dtype(d: Dims):
    return torch.bfloat16 if d.dtype == BF16 else torch.float32


def _pool_dtype(d: Dims):
    """8-bit pools are byte tensors [num_pages, page_bytes]."""
    return torch.uint8 if d.flags & FLAG_FP8_CACHE else _torch_dtype(d)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MLAError(status, what)


# --------------------------------------------------------------------------- calls

def write_cache(d: Dims, h, w_dkr, positions, slot_mapping, pool, stream=None, workspace=None) -> None:
    """mla_write_cache, or mla_write_cache_ws when a workspace is given (the
    8-bit cache needs one: write_cache_workspace_size bytes)."""
    dt = _torch_dtype(d)
    n = 0 if h is None else int(h.shape[0])
    num_pages = int(pool.shape[0])
    args = (ctypes.byref(d), _ptr(h, "h", dt), _ptr(w_dkr, "w_dkr", dt), _ptr(positions, "positions", torch.int32),
            _ptr(slot_mapping, "slot_mapping", torch.int64), n, _ptr(pool, "pool", _pool_dtype(d)), num_pages)
    if workspace is None:
        _check(lib().mla_write_cache(*args, _stream(stream)), "mla_write_cache")
    else:
        _check(lib().mla_write_cache_ws(*args, _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
                                        _stream(stream)), "mla_write_cache_ws")


def write_cache_workspace_size(d: Dims, n_tokens: int) -> int:
    return int(lib().mla_write_cache_workspace_size(ctypes.byref(d), int(n_tokens)))


def page_bytes(d: Dims) -> int:
    return int(lib().mla_page_bytes(ctypes.byref(d)))


def absorb_q(d: Dims, q, w_uk, positions, q_abs, stream=None) -> None:
    dt = _torch_dtype(d)
    _check(lib().mla_absorb_q(ctypes.byref(d), _ptr(q, "q", dt), _ptr(w_uk, "w_uk", dt),
                              _ptr(positions, "positions", torch.int32), int(q.shape[0]),
                              _ptr(q_abs, "q_abs", dt), _stream(stream)), "mla_absorb_q")


def write_absorb_workspace_size(d: Dims, n_write: int) -> int:
    return int(lib().mla_write_absorb_workspace_size(ctypes.byref(d), int(n_write)))


def write_absorb(d: Dims, h, w_dkr, positions, slot_mapping, pool, q, w_uk, q_positions, q_abs, workspace=None,
                 stream=None) -> None:
    """mla_write_absorb: write_cache then absorb_q, in one launch where it
    applies.  workspace: write_absorb_workspace_size bytes, zero-filled before
    its first use (each call leaves its counters at zero)."""
    dt = _torch_dtype(d)
    n_w = 0 if h is None else int(h.shape[0])
    n_q = 0 if q is None else int(q.shape[0])
    ws = None if workspace is None else _ptr(workspace, "workspace", torch.uint8)
    _check(lib().mla_write_absorb(ctypes.byref(d), _ptr(h, "h", dt), _ptr(w_dkr, "w_dkr", dt),
                                  _ptr(positions, "positions", torch.int32),
                                  _ptr(slot_mapping, "slot_mapping", torch.int64), n_w,
                                  _ptr(pool, "pool", _pool_dtype(d)), int(pool.shape[0]), _ptr(q, "q", dt),
                                  _ptr(w_uk, "w_uk", dt), _ptr(q_positions, "q_positions", torch.int32), n_q,
                                  _ptr(q_abs, "q_abs", dt), ws, 0 if workspace is None else workspace.numel(),
                                  _stream(stream)), "mla_write_absorb")


def decode_workspace_size(d: Dims, batch: int, max_seq_len: int) -> int:
    return int(lib().mla_decode_workspace_size(ctypes.byref(d), int(batch), int(max_seq_len)))


def decode(d: Dims, q_abs, pool, block_table, seq_lens, max_seq_len: int, w_uv, out, lse, workspace,
           stream=None) -> None:
    dt = _torch_dtype(d)
    _check(lib().mla_decode(ctypes.byref(d), _ptr(q_abs, "q_abs", dt), _ptr(pool, "pool", _pool_dtype(d)),
                            int(pool.shape[0]), _ptr(block_table, "block_table", torch.int32),
                            int(block_table.shape[1]), _ptr(seq_lens, "seq_lens", torch.int32),
                            int(seq_lens.shape[0]), int(max_seq_len), _ptr(w_uv, "w_uv", dt),
                            _ptr(out, "out", dt), _ptr(lse, "lse", torch.float32),
                            _ptr(workspace, "workspace", torch.uint8),
                            0 if workspace is None else workspace.numel(), _stream(stream)), "mla_decode")


def decode_noalloc(d: Dims, q_abs, pool, block_table, seq_lens, max_seq_len: int, w_uv, out, lse,
                   stream=None) -> None:
    """mla_decode_noalloc: mla_decode with the partial results in the
    library's own per-device scratch array (no workspace)."""
    dt = _torch_dtype(d)
    _check(lib().mla_decode_noalloc(ctypes.byref(d), _ptr(q_abs, "q_abs", dt), _ptr(pool, "pool", _pool_dtype(d)),
                                    int(pool.shape[0]), _ptr(block_table, "block_table", torch.int32),
                                    int(block_table.shape[1]), _ptr(seq_lens, "seq_lens", torch.int32),
                                    int(seq_lens.shape[0]), int(max_seq_len), _ptr(w_uv, "w_uv", dt),
                                    _ptr(out, "out", dt), _ptr(lse, "lse", torch.float32), _stream(stream)),
           "mla_decode_noalloc")


def prefill_workspace_size(d: Dims, total_tokens: int) -> int:
    return int(lib().mla_prefill_workspace_size(ctypes.byref(d), int(total_tokens)))


def prefill(d: Dims, q, pool, block_table, cu_seqlens, max_seq_len: int, w_uk, w_uv, out, lse, workspace,
            stream=None) -> None:
    dt = _torch_dtype(d)
    _check(lib().mla_prefill(ctypes.byref(d), _ptr(q, "q", dt), _ptr(pool, "pool", dt), int(pool.shape[0]),
                             _ptr(block_table, "block_table", torch.int32), int(block_table.shape[1]),
                             _ptr(cu_seqlens, "cu_seqlens", torch.int32), int(cu_seqlens.shape[0]) - 1,
                             int(q.shape[0]), int(max_seq_len), _ptr(w_uk, "w_uk", dt), _ptr(w_uv, "w_uv", dt),
                             _ptr(out, "out", dt), _ptr(lse, "lse", torch.float32),
                             _ptr(workspace, "workspace", torch.uint8),
                             0 if workspace is None else workspace.numel(), _stream(stream)), "mla_prefill")


def prefill_kv(d: Dims, q, pool, block_table, cu_seqlens_q, cu_seqlens_kv, total_kv: int, max_q_len: int,
               max_kv_len: int, w_uk, w_uv, out, lse, workspace, stream=None) -> None:
    """Prefill of the new tokens (q rows) onto sequences with a cached prefix:
    sequence i's keys are its cu_seqlens_kv[i+1] - cu_seqlens_kv[i] cached
    tokens, the last q_len of them new."""
    dt = _torch_dtype(d)
    _check(lib().mla_prefill_kv(ctypes.byref(d), _ptr(q, "q", dt), _ptr(pool, "pool", dt), int(pool.shape[0]),
                                _ptr(block_table, "block_table", torch.int32), int(block_table.shape[1]),
                                _ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                                _ptr(cu_seqlens_kv, "cu_seqlens_kv", torch.int32), int(cu_seqlens_q.shape[0]) - 1,
                                int(q.shape[0]), int(total_kv), int(max_q_len), int(max_kv_len),
                                _ptr(w_uk, "w_uk", dt), _ptr(w_uv, "w_uv", dt), _ptr(out, "out", dt),
                                _ptr(lse, "lse", torch.float32), _ptr(workspace, "workspace", torch.uint8),
                                0 if workspace is None else workspace.numel(), _stream(stream)), "mla_prefill_kv")


def cache_bytes(d: Dims, tokens: int, layers: int) -> int:
    return int(lib().mla_cache_bytes(ctypes.byref(d), int(tokens), int(layers)))


def uses_fast_path(d: Dims, op: int) -> int:
    return int(lib().mla_uses_fast_path(ctypes.byref(d), int(op)))


def get_device_error(stream=None) -> int:
    """mla_get_device_error: waits for the stream, returns and clears the
    device error word (MLA_DEVERR_* bits)."""
    v = ctypes.c_int32(0)
    _check(lib().mla_get_device_error(ctypes.byref(v), _stream(stream)), "mla_get_device_error")
    return int(v.value)


def debug_build() -> bool:
    return bool(lib().mla_debug_build())


def project_q_workspace_size(d: Dims, d_cq: int, n_tokens: int) -> int:
    return int(lib().mla_project_q_workspace_size(ctypes.byref(d), int(d_cq), int(n_tokens)))


def project_q(d: Dims, h, w_dq, w_uq, w_uk, positions, q_abs, workspace, stream=None) -> None:
    """mla_project_q: c_Q = W_DQ h, q = W_UQ c_Q, then the absorbed queries."""
    dt = _torch_dtype(d)
    _check(lib().mla_project_q(ctypes.byref(d), int(w_dq.shape[0]), _ptr(h, "h", dt), _ptr(w_dq, "w_dq", dt),
                               _ptr(w_uq, "w_uq", dt), _ptr(w_uk, "w_uk", dt),
                               _ptr(positions, "positions", torch.int32), int(h.shape[0]), _ptr(q_abs, "q_abs", dt),
                               _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
           "mla_project_q")


def project_out_workspace_size(d: Dims, n_tokens: int) -> int:
    return int(lib().mla_project_out_workspace_size(ctypes.byref(d), int(n_tokens)))


def project_out(d: Dims, o, w_o, y, workspace=None, stream=None) -> None:
    """mla_project_out: y = W_O [o_1 | ... | o_H]."""
    dt = _torch_dtype(d)
    _check(lib().mla_project_out(ctypes.byref(d), _ptr(o, "o", dt), _ptr(w_o, "w_o", dt), int(o.shape[0]),
                                 _ptr(y, "y", dt), _ptr(workspace, "workspace", torch.uint8),
                                 0 if workspace is None else workspace.numel(), _stream(stream)), "mla_project_out")
