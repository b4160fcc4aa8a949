"""ctypes binding of libkvmem.so (include/kvmem.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  torch tensors are used for device memory and streams; their
data pointers are passed straight through.  Loading fails loudly when the
library has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvmem.so")

KVMEM_OK, KVMEM_E_ARG, KVMEM_E_UNSUPPORTED, KVMEM_E_WORKSPACE, KVMEM_E_HIP = range(5)
KVMEM_F32, KVMEM_BF16 = 0, 1
KVMEM_DEVERR_PAGE, KVMEM_DEVERR_BLOCK = 1, 2

EXPORTED = [
    "kvmem_index_bytes",
    "kvmem_build_index",
    "kvmem_score_select_scratch_bytes",
    "kvmem_score_select",
    "kvmem_materialize",
    "kvmem_stage_view",
    "kvmem_attend_scratch_bytes",
    "kvmem_attend",
    "kvmem_attend_noalloc",
    "kvmem_update_index",
    "kvmem_append",
    "kvmem_attend_append",
    "kvmem_attend_paged_scratch_bytes",
    "kvmem_attend_paged",
    "kvmem_materialize_attend",
    "kvmem_attention_mass_scratch_bytes",
    "kvmem_attention_mass",
    "kvmem_view_tokens",
    "kvmem_status_string",
    "kvmem_version",
]


class Geom(ctypes.Structure):
    _fields_ = [("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("block_tokens", c_int32), ("kv_dtype", c_int32)]


class Workspace(ctypes.Structure):
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("block_table", c_void_p),
                ("n_tokens_host", c_void_p), ("n_sessions", c_int32), ("max_blocks", c_int32),
                ("n_pages", c_int32), ("dev_error", c_void_p)]


class KVMemError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libkvmem.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or os.environ.get("KVMEM_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m block_sparse_decode_amd.build`")
    # PyTorch wheels bring their own HIP runtime.  Loading it first makes the
    # library bind to that same runtime, so device memory allocated by torch
    # and the library's kernels live in one runtime (loading the library first
    # would pull in a second runtime and every launch on torch memory fails).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    lib.kvmem_index_bytes.argtypes = [POINTER(Geom), c_int32, c_int32]
    lib.kvmem_index_bytes.restype = c_size_t
    lib.kvmem_build_index.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_void_p]
    lib.kvmem_build_index.restype = c_int32
    lib.kvmem_score_select_scratch_bytes.argtypes = [POINTER(Geom), c_int32, c_int32, c_int32]
    lib.kvmem_score_select_scratch_bytes.restype = c_size_t
    lib.kvmem_score_select.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_void_p, c_int32,
                                       c_void_p, c_float, c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvmem_score_select.restype = c_int32
    lib.kvmem_materialize.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p,
                                      c_int32, c_float, c_void_p, c_void_p, c_void_p]
    lib.kvmem_materialize.restype = c_int32
    lib.kvmem_stage_view.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p]
    lib.kvmem_stage_view.restype = c_int32
    lib.kvmem_attend_scratch_bytes.argtypes = [POINTER(Geom), c_int32, c_int32, c_int32]
    lib.kvmem_attend_scratch_bytes.restype = c_size_t
    lib.kvmem_attend.argtypes = [POINTER(Geom), c_int32, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                 c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvmem_attend.restype = c_int32
    lib.kvmem_attend_noalloc.argtypes = [POINTER(Geom), c_int32, c_void_p, c_int32, c_void_p, c_float, c_void_p,
                                         c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p]
    lib.kvmem_attend_noalloc.restype = c_int32
    lib.kvmem_update_index.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_void_p, c_void_p]
    lib.kvmem_update_index.restype = c_int32
    lib.kvmem_append.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                 c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p]
    lib.kvmem_append.restype = c_int32
    lib.kvmem_attend_append.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p, c_float,
                                        c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]
    lib.kvmem_attend_append.restype = c_int32
    lib.kvmem_attend_paged_scratch_bytes.argtypes = [POINTER(Geom), c_int32, c_int32, c_int32]
    lib.kvmem_attend_paged_scratch_bytes.restype = c_size_t
    lib.kvmem_attend_paged.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p, c_float,
                                       c_void_p, c_int32, c_void_p, c_float, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvmem_attend_paged.restype = c_int32
    lib.kvmem_materialize_attend.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p, c_float,
                                             c_void_p, c_int32, c_void_p, c_int32, c_float, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvmem_materialize_attend.restype = c_int32
    lib.kvmem_attention_mass_scratch_bytes.argtypes = [POINTER(Geom), c_int32, c_int32, c_int32]
    lib.kvmem_attention_mass_scratch_bytes.restype = c_size_t
    lib.kvmem_attention_mass.argtypes = [POINTER(Geom), POINTER(Workspace), c_void_p, c_int32, c_void_p, c_float,
                                         c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvmem_attention_mass.restype = c_int32
    lib.kvmem_view_tokens.argtypes = [c_int32, c_void_p, c_int32, c_int32, c_void_p]
    lib.kvmem_view_tokens.restype = c_int32
    lib.kvmem_status_string.argtypes = [c_int32]
    lib.kvmem_status_string.restype = ctypes.c_char_p
    lib.kvmem_version.argtypes = []
    lib.kvmem_version.restype = c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kvmem_status_string(int(status)).decode()


def _p(x) -> int | None:
    """Device/host pointer of a torch tensor or numpy array (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    if isinstance(x, int):
        return x
    assert x.is_contiguous(), "tensors passed to the library must be contiguous"
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != KVMEM_OK:
        raise KVMemError(status, where)


def make_geom(n_q_heads: int, n_kv_heads: int, dtype: str, head_dim: int = 128, block_tokens: int = 32) -> Geom:
    return Geom(n_q_heads, n_kv_heads, head_dim, block_tokens, KVMEM_BF16 if dtype == "bf16" else KVMEM_F32)


def make_workspace(k_pool, v_pool, block_table, n_tokens_host: np.ndarray, dev_error=None) -> Workspace:
    """n_tokens_host must stay alive (and unchanged) while the struct is used."""
    assert n_tokens_host.dtype == np.int32 and n_tokens_host.flags["C_CONTIGUOUS"]
    S, max_blocks = block_table.shape
    return Workspace(_p(k_pool), _p(v_pool), _p(block_table), n_tokens_host.ctypes.data, S, max_blocks,
                     int(k_pool.shape[0]), _p(dev_error))


# --- the entry points (same names as the C ABI) ------------------------------

def kvmem_index_bytes(geom: Geom, n_sessions: int, max_blocks: int) -> int:
    return int(load().kvmem_index_bytes(ctypes.byref(geom), n_sessions, max_blocks))


def kvmem_build_index(geom: Geom, ws: Workspace, index, stream=None, check: bool = True) -> int:
    st = load().kvmem_build_index(ctypes.byref(geom), ctypes.byref(ws), _p(index), _stream(stream))
    if check:
        _check(st, "kvmem_build_index")
    return st


def kvmem_score_select_scratch_bytes(geom: Geom, n_sessions: int, max_blocks: int, T: int) -> int:
    return int(load().kvmem_score_select_scratch_bytes(ctypes.byref(geom), n_sessions, max_blocks, T))


def kvmem_score_select(geom: Geom, ws: Workspace, index, q, T: int, q_norm_w, eps: float, k_select: int,
                       n_recent: int, view_blocks, view_tokens_host: np.ndarray, scores=None, agg=None,
                       scratch=None, scratch_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_score_select(ctypes.byref(geom), ctypes.byref(ws), _p(index), _p(q), T, _p(q_norm_w),
                                   eps, k_select, n_recent, _p(view_blocks), _p(view_tokens_host), _p(scores),
                                   _p(agg), _p(scratch), scratch_bytes, _stream(stream))
    if check:
        _check(st, "kvmem_score_select")
    return st


def kvmem_materialize(geom: Geom, ws: Workspace, view_blocks, n_list: int, view_tokens_host: np.ndarray,
                      max_view: int, rope_theta: float, k_view, v_view, stream=None, check: bool = True) -> int:
    st = load().kvmem_materialize(ctypes.byref(geom), ctypes.byref(ws), _p(view_blocks), n_list,
                                  _p(view_tokens_host), max_view, rope_theta, _p(k_view), _p(v_view),
                                  _stream(stream))
    if check:
        _check(st, "kvmem_materialize")
    return st


def kvmem_stage_view(geom: Geom, ws: Workspace, view_blocks, n_list: int, view_tokens_host: np.ndarray, stage_k,
                     stage_v, stage_table, stage_list, stream=None, check: bool = True) -> int:
    st = load().kvmem_stage_view(ctypes.byref(geom), ctypes.byref(ws), _p(view_blocks), n_list,
                                 _p(view_tokens_host), _p(stage_k), _p(stage_v), _p(stage_table), _p(stage_list),
                                 _stream(stream))
    if check:
        _check(st, "kvmem_stage_view")
    return st


def kvmem_attend_scratch_bytes(geom: Geom, n_sessions: int, T: int, max_view: int) -> int:
    return int(load().kvmem_attend_scratch_bytes(ctypes.byref(geom), n_sessions, T, max_view))


def kvmem_attend(geom: Geom, n_sessions: int, q, T: int, q_norm_w, eps: float, k_view, v_view,
                 view_tokens_host: np.ndarray, max_view: int, rope_theta: float, out, scratch=None,
                 scratch_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_attend(ctypes.byref(geom), n_sessions, _p(q), T, _p(q_norm_w), eps, _p(k_view),
                             _p(v_view), _p(view_tokens_host), max_view, rope_theta, _p(out), _p(scratch),
                             scratch_bytes, _stream(stream))
    if check:
        _check(st, "kvmem_attend")
    return st


NOALLOC_SCRATCH_BYTES = 32 << 20      # KVMEM_NOALLOC_SCRATCH_BYTES


def kvmem_attend_noalloc(geom: Geom, n_sessions: int, q, T: int, q_norm_w, eps: float, k_view, v_view,
                         view_tokens_host: np.ndarray, max_view: int, rope_theta: float, out, stream=None,
                         check: bool = True) -> int:
    st = load().kvmem_attend_noalloc(ctypes.byref(geom), n_sessions, _p(q), T, _p(q_norm_w), eps, _p(k_view),
                                     _p(v_view), _p(view_tokens_host), max_view, rope_theta, _p(out),
                                     _stream(stream))
    if check:
        _check(st, "kvmem_attend_noalloc")
    return st


def kvmem_update_index(geom: Geom, ws: Workspace, first_block_host: np.ndarray | None, index, stream=None,
                       check: bool = True) -> int:
    if first_block_host is not None:
        assert first_block_host.dtype == np.int32
    st = load().kvmem_update_index(ctypes.byref(geom), ctypes.byref(ws), _p(first_block_host), _p(index),
                                   _stream(stream))
    if check:
        _check(st, "kvmem_update_index")
    return st


def kvmem_append(geom: Geom, ws: Workspace, k_pool, v_pool, k_new, v_new, T_new: int,
                 view_tokens_host: np.ndarray, max_view: int, rope_theta: float, k_view, v_view, stream=None,
                 check: bool = True) -> int:
    assert view_tokens_host.dtype == np.int32
    st = load().kvmem_append(ctypes.byref(geom), ctypes.byref(ws), _p(k_pool), _p(v_pool), _p(k_new), _p(v_new),
                             T_new, _p(view_tokens_host), max_view, rope_theta, _p(k_view), _p(v_view),
                             _stream(stream))
    if check:
        _check(st, "kvmem_append")
    return st


def kvmem_attend_append(geom: Geom, ws: Workspace, q, T: int, q_norm_w, eps: float, k_view, v_view,
                        view_tokens_host: np.ndarray, max_view: int, rope_theta: float, out, k_pool, v_pool, k_new,
                        v_new, T_new: int, scratch=None, scratch_bytes: int | None = None, stream=None,
                        check: bool = True) -> int:
    assert view_tokens_host.dtype == np.int32
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_attend_append(ctypes.byref(geom), ctypes.byref(ws), _p(q), T, _p(q_norm_w), eps, _p(k_view),
                                    _p(v_view), _p(view_tokens_host), max_view, rope_theta, _p(out), _p(k_pool),
                                    _p(v_pool), _p(k_new), _p(v_new), T_new, _p(scratch), scratch_bytes,
                                    _stream(stream))
    if check:
        _check(st, "kvmem_attend_append")
    return st


def kvmem_attend_paged_scratch_bytes(geom: Geom, n_sessions: int, T: int, n_list: int) -> int:
    return int(load().kvmem_attend_paged_scratch_bytes(ctypes.byref(geom), n_sessions, T, n_list))


def kvmem_attend_paged(geom: Geom, ws: Workspace, q, T: int, q_norm_w, eps: float, view_blocks, n_list: int,
                       view_tokens_host: np.ndarray, rope_theta: float, out, scratch=None,
                       scratch_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_attend_paged(ctypes.byref(geom), ctypes.byref(ws), _p(q), T, _p(q_norm_w), eps,
                                   _p(view_blocks), n_list, _p(view_tokens_host), rope_theta, _p(out), _p(scratch),
                                   scratch_bytes, _stream(stream))
    if check:
        _check(st, "kvmem_attend_paged")
    return st


def kvmem_materialize_attend(geom: Geom, ws: Workspace, q, T: int, q_norm_w, eps: float, view_blocks, n_list: int,
                             view_tokens_host: np.ndarray, max_view: int, rope_theta: float, k_view, v_view, out,
                             scratch=None, scratch_bytes: int | None = None, stream=None, check: bool = True) -> int:
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_materialize_attend(ctypes.byref(geom), ctypes.byref(ws), _p(q), T, _p(q_norm_w), eps,
                                         _p(view_blocks), n_list, _p(view_tokens_host), max_view, rope_theta,
                                         _p(k_view), _p(v_view), _p(out), _p(scratch), scratch_bytes, _stream(stream))
    if check:
        _check(st, "kvmem_materialize_attend")
    return st


def kvmem_attention_mass_scratch_bytes(geom: Geom, n_sessions: int, T: int, max_blocks: int) -> int:
    return int(load().kvmem_attention_mass_scratch_bytes(ctypes.byref(geom), n_sessions, T, max_blocks))


def kvmem_attention_mass(geom: Geom, ws: Workspace, q, T: int, q_norm_w, eps: float, view_blocks, n_list: int,
                         rope_theta: float, mass, lse=None, scratch=None, scratch_bytes: int | None = None,
                         stream=None, check: bool = True) -> int:
    if scratch_bytes is None:
        scratch_bytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = load().kvmem_attention_mass(ctypes.byref(geom), ctypes.byref(ws), _p(q), T, _p(q_norm_w), eps,
                                     _p(view_blocks), n_list, rope_theta, _p(mass), _p(lse), _p(scratch),
                                     scratch_bytes, _stream(stream))
    if check:
        _check(st, "kvmem_attention_mass")
    return st


def kvmem_view_tokens(n_tokens_host: np.ndarray, k_select: int, n_recent: int, check: bool = True) -> np.ndarray:
    """View lengths kvmem_score_select will report for these history lengths
    (host only); returns them as a new int32 array."""
    n = np.ascontiguousarray(n_tokens_host, dtype=np.int32)
    out = np.zeros(max(1, len(n)), np.int32)
    st = load().kvmem_view_tokens(len(n), _p(n), k_select, n_recent, _p(out))
    if check:
        _check(st, "kvmem_view_tokens")
    return out[:len(n)]


def kvmem_version() -> int:
    return int(load().kvmem_version())
