"""ctypes binding of libmla_decode.so: same entry points as include/mla_decode.h.

Argument marshalling only.  Every step of the decode runs in the library's HIP kernels;
there is no Python or CPU fallback.  If the shared library is missing this module raises
on first use rather than degrading silently.

Tensor arguments may be torch tensors (their ``data_ptr()`` is passed) or raw integer
device addresses.  ``stream`` defaults to torch's current HIP stream.
"""

from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mla_decode.h")

MLA_F32, MLA_BF16 = 0, 1
PAGE_SIZE = 64
MLA_FLAG_DEVICE_CHECKS = 1
MLA_FLAG_QUERY_LATENT = 2
MLA_FLAG_OUTPUT_LATENT = 4
MLA_LATENT_FP8 = 1
MLA_DEVERR_SEQLEN, MLA_DEVERR_BLOCK = 1, 2
STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_UNSUPPORTED",
          4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_DTYPE", 6: "MLA_ERR_HIP", 7: "MLA_ERR_ALIGN"}


class MlaParams(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("num_heads", c_int32), ("num_branches", c_int32),
        ("d_nope", c_int32), ("d_v", c_int32), ("d_latent", c_int32), ("d_rope", c_int32),
        ("page_size", c_int32), ("max_pages_per_seq", c_int32), ("max_seqlen", c_int32),
        ("num_splits", c_int32), ("dtype", c_int32), ("flags", c_int32), ("num_pages", c_int32),
        ("num_queries", c_int32), ("latent_format", c_int32),
        ("latent_stride_tok", c_int64), ("latent_stride_seq", c_int64),
        ("rope_stride_tok", c_int64), ("rope_stride_seq", c_int64),
        ("block_table_stride", c_int64),
        ("softmax_scale", c_float), ("out_scale", c_float), ("rope_theta", c_float),
        ("latent_scale", c_float),
    ]

    def copy(self) -> "MlaParams":
        c = MlaParams()
        ctypes.pointer(c)[0] = self
        return c


class MlaAppendParams(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("d_model", c_int32), ("d_latent", c_int32), ("d_rope", c_int32),
        ("page_size", c_int32), ("max_pages_per_seq", c_int32), ("capacity", c_int32),
        ("dtype", c_int32),
        ("latent_stride_tok", c_int64), ("latent_stride_seq", c_int64),
        ("rope_stride_tok", c_int64), ("rope_stride_seq", c_int64),
        ("block_table_stride", c_int64), ("rope_theta", c_float),
        ("latent_format", c_int32), ("latent_scale", c_float),
    ]


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_str(status)}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mlra_latent_kv_amd.build`")
    # torch ships its own copy of the HIP runtime; load it first so that the library binds to
    # that copy (same soname) and shares torch's device memory and streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(MlaParams)
    lib.mla_workspace_size.argtypes = [P, ctypes.POINTER(c_size_t)]
    lib.mla_num_splits.argtypes = [P, ctypes.POINTER(c_int32)]
    dec = [P] + [c_void_p] * 10 + [c_size_t, c_void_p]
    lib.mla_decode.argtypes = dec
    lib.mlra_decode.argtypes = dec
    lib.mla_decode_timed.argtypes = dec + [c_void_p]
    lib.mlra_decode_timed.argtypes = dec + [c_void_p]
    lib.mla_decode_noalloc.argtypes = [P] + [c_void_p] * 10
    lib.mla_decode_gated.argtypes = [P] + [c_void_p] * 11 + [c_size_t, c_void_p]
    lib.mlra_decode_gated.argtypes = [P] + [c_void_p] * 11 + [c_size_t, c_void_p]
    PA = ctypes.POINTER(MlaAppendParams)
    lib.mla_append_workspace_size.argtypes = [PA, ctypes.POINTER(c_size_t)]
    lib.mla_cache_append.argtypes = [PA] + [c_void_p] * 8 + [c_int32, c_void_p, c_void_p,
                                                               c_size_t, c_void_p]
    lib.mla_rope_rotate.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_float,
                                    c_int32, c_void_p]
    lib.mla_prefill_workspace_size.argtypes = [P, ctypes.POINTER(c_size_t)]
    lib.mla_prefill.argtypes = dec
    lib.mla_prefill_timed.argtypes = dec + [c_void_p]
    lib.mla_status_str.argtypes = [c_int32]
    lib.mla_status_str.restype = ctypes.c_char_p
    for f in ("mla_workspace_size", "mla_num_splits", "mla_decode", "mlra_decode",
              "mla_decode_timed", "mlra_decode_timed", "mla_decode_noalloc", "mla_rope_rotate",
              "mla_decode_gated", "mlra_decode_gated",
              "mla_append_workspace_size", "mla_cache_append", "mla_prefill_workspace_size",
              "mla_prefill", "mla_prefill_timed"):
        getattr(lib, f).restype = c_int32
    _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list:
    """Names of the functions include/mla_decode.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ml\w+)\s*\(", text, flags=re.M)))


def status_str(status: int) -> str:
    try:
        return load().mla_status_str(status).decode()
    except Exception:  # library missing: still give a readable name
        return STATUS.get(status, f"status {status}")


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_size(params: MlaParams) -> int:
    n = c_size_t(0)
    st = load().mla_workspace_size(ctypes.byref(params), ctypes.byref(n))
    if st:
        raise MlaError(st, "mla_workspace_size")
    return n.value


def num_splits(params: MlaParams) -> int:
    n = c_int32(0)
    st = load().mla_num_splits(ctypes.byref(params), ctypes.byref(n))
    if st:
        raise MlaError(st, "mla_num_splits")
    return n.value


def _decode(fname, params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
            workspace, workspace_bytes=None, stream=None, check=True, events=None) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    args = [ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(latent), _ptr(rope),
            _ptr(seqlens), _ptr(block_table), _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace),
            workspace_bytes, _stream(stream)]
    if events is not None:
        fname += "_timed"
        args.append(ctypes.cast(events, c_void_p))
    st = getattr(load(), fname)(*args)
    if check and st:
        raise MlaError(st, fname)
    return st


def mla_decode(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
               workspace, workspace_bytes=None, stream=None, check=True, events=None) -> int:
    """``events``: optional ctypes array of 5 hipEvent_t -> calls mla_decode_timed."""
    return _decode("mla_decode", params, q_nope, q_rope, latent, rope, seqlens, block_table,
                   w_uk, w_uv, out, workspace, workspace_bytes, stream, check, events)


def mlra_decode(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                workspace, workspace_bytes=None, stream=None, check=True, events=None) -> int:
    return _decode("mlra_decode", params, q_nope, q_rope, latent, rope, seqlens, block_table,
                   w_uk, w_uv, out, workspace, workspace_bytes, stream, check, events)


def _decode_gated(fname, params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk,
                  w_uv, gate, out, workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = getattr(load(), fname)(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(latent),
                                _ptr(rope), _ptr(seqlens), _ptr(block_table), _ptr(w_uk),
                                _ptr(w_uv), _ptr(gate), _ptr(out), _ptr(workspace),
                                workspace_bytes, _stream(stream))
    if check and st:
        raise MlaError(st, fname)
    return st


def mla_decode_gated(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv,
                     gate, out, workspace, workspace_bytes=None, stream=None, check=True) -> int:
    return _decode_gated("mla_decode_gated", params, q_nope, q_rope, latent, rope, seqlens,
                         block_table, w_uk, w_uv, gate, out, workspace, workspace_bytes, stream,
                         check)


def mlra_decode_gated(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv,
                      gate, out, workspace, workspace_bytes=None, stream=None, check=True) -> int:
    return _decode_gated("mlra_decode_gated", params, q_nope, q_rope, latent, rope, seqlens,
                         block_table, w_uk, w_uv, gate, out, workspace, workspace_bytes, stream,
                         check)


def prefill_workspace_size(params: MlaParams) -> int:
    n = c_size_t(0)
    st = load().mla_prefill_workspace_size(ctypes.byref(params), ctypes.byref(n))
    if st:
        raise MlaError(st, "mla_prefill_workspace_size")
    return n.value


def mla_prefill(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                workspace, workspace_bytes=None, stream=None, check=True, events=None) -> int:
    """The un-absorbed many-query step (see include/mla_decode.h, mla_prefill); ``events``:
    optional ctypes array of 3 hipEvent_t -> calls mla_prefill_timed."""
    return _decode("mla_prefill", params, q_nope, q_rope, latent, rope, seqlens, block_table,
                   w_uk, w_uv, out, workspace, workspace_bytes, stream, check, events)


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # MLA_NOALLOC_SCRATCH_BYTES


def mla_decode_noalloc(params, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv,
                       out, stream=None, check=True) -> int:
    """mla_decode with the library's static scratch instead of a caller workspace."""
    st = load().mla_decode_noalloc(ctypes.byref(params), _ptr(q_nope), _ptr(q_rope), _ptr(latent),
                                   _ptr(rope), _ptr(seqlens), _ptr(block_table), _ptr(w_uk),
                                   _ptr(w_uv), _ptr(out), _stream(stream))
    if check and st:
        raise MlaError(st, "mla_decode_noalloc")
    return st


def mla_rope_rotate(x, row_stride: int, pos, n_rows: int, d_rope: int, theta: float, dtype: int,
                    stream=None, check=True) -> int:
    st = load().mla_rope_rotate(_ptr(x), row_stride, _ptr(pos), n_rows, d_rope, theta, dtype,
                                _stream(stream) if n_rows else None)
    if check and st:
        raise MlaError(st, "mla_rope_rotate")
    return st


def append_workspace_size(params: MlaAppendParams) -> int:
    n = c_size_t(0)
    st = load().mla_append_workspace_size(ctypes.byref(params), ctypes.byref(n))
    if st:
        raise MlaError(st, "mla_append_workspace_size")
    return n.value


def mla_cache_append(params, hidden, w_dkv, w_kr, latent, rope, seqlens, block_table, free_pages,
                     n_free: int, pages_used, workspace, workspace_bytes=None, stream=None,
                     check=True) -> int:
    """One decode step's cache write (see include/mla_decode.h, mla_cache_append)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load().mla_cache_append(ctypes.byref(params), _ptr(hidden), _ptr(w_dkv), _ptr(w_kr),
                                 _ptr(latent), _ptr(rope), _ptr(seqlens), _ptr(block_table),
                                 _ptr(free_pages), n_free, _ptr(pages_used), _ptr(workspace),
                                 workspace_bytes, _stream(stream))
    if check and st:
        raise MlaError(st, "mla_cache_append")
    return st
