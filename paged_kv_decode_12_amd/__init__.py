"""Batched paged-KV decode attention for AMD MI355X (gfx950).

Thin ctypes binding over ``libpkvd.so`` (C ABI in ``include/pkvd.h``).  This
module only marshals arguments: it turns torch tensors into strided
descriptors, passes torch's current HIP stream and maps status codes to
exceptions.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  If the library has not been built, importing this
package raises ImportError.

Semantics follow flashinfer.cudnn.cudnn_batch_decode_with_kv_cache
(Parameters, Returns, Note): see ``decode``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["decode", "bind_decode", "merge_states", "plan", "workspace_bytes",
           "reserve_workspace", "library_path", "PkvdError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKVD_LIBRARY selects another build of the same library (A/B comparisons)
_LIB_PATH = os.environ.get("PKVD_LIBRARY") or os.path.join(_HERE, "libpkvd.so")

_BF16, _F16, _F32, _I32 = 0, 1, 2, 3
_DT = {torch.bfloat16: _BF16, torch.float16: _F16, torch.float32: _F32, torch.int32: _I32}


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class PkvdError(RuntimeError):
    """A HIP or workspace failure reported by the library."""


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it first (python paged_kv_decode_12_amd/build.py "
            "or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(_Tensor)
    lib.pkvd_decode.restype = ctypes.c_int
    lib.pkvd_decode.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                P, P, P, ctypes.c_void_p]
    lib.pkvd_decode_workspace_bytes.restype = ctypes.c_int
    lib.pkvd_decode_workspace_bytes.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.pkvd_reserve_workspace.restype = ctypes.c_int
    lib.pkvd_reserve_workspace.argtypes = [ctypes.c_size_t]
    lib.pkvd_decode_plan.restype = ctypes.c_int
    lib.pkvd_decode_plan.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int64 * 6)]
    lib.pkvd_last_error.restype = ctypes.c_char_p
    lib.pkvd_status_string.restype = ctypes.c_char_p
    lib.pkvd_status_string.argtypes = [ctypes.c_int]
    lib.pkvd_version.restype = ctypes.c_char_p
    lib.pkvd_merge_states.restype = ctypes.c_int
    lib.pkvd_merge_states.argtypes = [P, P, P, P, P, ctypes.c_void_p]
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def _desc(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dim() > 4:
        raise ValueError("tensors of more than 4 dimensions are not accepted")
    d = _Tensor()
    d.data = t.data_ptr()
    d.dtype = _DT.get(t.dtype, -1)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.strides[i] = t.stride(i)
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _check(status: int):
    if status == 0:
        return
    msg = _lib.pkvd_last_error().decode() or _lib.pkvd_status_string(status).decode()
    if status == 1:
        raise ValueError(msg)
    if status == 2:
        raise NotImplementedError(msg)
    raise PkvdError(msg)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens_kv: torch.Tensor, scale: Optional[float] = None,
           q_len_per_req: int = 1, window_left: int = -1, sinks: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           return_lse: bool = False, stream=None):
    """Batched decode attention over a paged KV cache.

    q            (B * q_len_per_req, Hq, D) bf16/fp16; head_dim innermost and dense
    k_cache      (num_pages, Hkv, page_size, D); v_cache the same
    block_tables (B, C) int32;  seq_lens_kv (B,) int32 on q's device
    scale        defaults to 1 / sqrt(D)
    sinks        optional (Hq,) float32 sink logits
    out / lse    optional caller-owned outputs; allocated here when None
    Returns out, or (out, lse) when return_lse or lse is given.  lse is the
    base-2 log-sum-exp over each row's visible keys.  Enqueued on torch's
    current stream of q's device (or ``stream``); never synchronises.
    """
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("seq_lens_kv", seq_lens_kv),
                    ("sinks", sinks), ("out", out), ("lse", lse)):
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{name} must be a GPU tensor on q's device ({dev})")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = return_lse or lse is not None
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    with torch.cuda.device(q.device):
        st = _lib.pkvd_decode(_ref(_desc(q)), _ref(_desc(k_cache)), _ref(_desc(v_cache)),
                              _ref(_desc(block_tables)), _ref(_desc(seq_lens_kv)),
                              float(scale), int(q_len_per_req), int(window_left),
                              _ref(_desc(sinks)), _ref(_desc(out)),
                              _ref(_desc(lse) if want_lse else None), ctypes.c_void_p(stream))
    _check(st)
    return (out, lse) if want_lse else out


class BoundDecode:
    """One decode call with its arguments marshalled once (see bind_decode).

    Calling it enqueues pkvd_decode on torch's current stream of q's device
    (or the given stream) and returns out, or (out, lse).  The tensors are
    held, not copied: write new inputs into them in place between calls.
    """

    def __init__(self, q, k_cache, v_cache, block_tables, seq_lens_kv, scale, q_len_per_req,
                 window_left, sinks, out, lse):
        self._tensors = (q, k_cache, v_cache, block_tables, seq_lens_kv, sinks, out, lse)
        self._descs = [_desc(t) for t in self._tensors]
        self._refs = [_ref(d) for d in self._descs]
        self._scale = ctypes.c_float(scale)
        self._lq = ctypes.c_int32(q_len_per_req)
        self._wl = ctypes.c_int32(window_left)
        self._device = q.device
        self._result = (out, lse) if lse is not None else out

    def __call__(self, stream=None):
        r = self._refs
        if stream is None:
            stream = torch.cuda.current_stream(self._device).cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        st = _lib.pkvd_decode(r[0], r[1], r[2], r[3], r[4], self._scale, self._lq, self._wl,
                              r[5], r[6], r[7], ctypes.c_void_p(stream))
        _check(st)
        return self._result


def bind_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_tables: torch.Tensor, seq_lens_kv: torch.Tensor,
                scale: Optional[float] = None, q_len_per_req: int = 1, window_left: int = -1,
                sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, return_lse: bool = False) -> BoundDecode:
    """The arguments of ``decode`` marshalled once, for calls repeated on the
    same buffers (a decode step of a serving loop, a benchmark): the returned
    object enqueues the same pkvd_decode call each time it is called, without
    rebuilding the descriptors.  Outputs are allocated here when None.  The
    library checks every argument on every call, as for ``decode``.  The
    current device must be q's device when it is called."""
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("seq_lens_kv", seq_lens_kv),
                    ("sinks", sinks), ("out", out), ("lse", lse)):
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{name} must be a GPU tensor on q's device ({dev})")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    if (return_lse or lse is not None) and lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    return BoundDecode(q, k_cache, v_cache, block_tables, seq_lens_kv, float(scale),
                       int(q_len_per_req), int(window_left), sinks, out, lse)


def merge_states(v: torch.Tensor, s: torch.Tensor, sinks: Optional[torch.Tensor] = None,
                 v_out: Optional[torch.Tensor] = None, s_out: Optional[torch.Tensor] = None,
                 return_lse: bool = True, stream=None):
    """Cascade merge of S partial states over disjoint key sets (pkvd_merge_states).

    v (S, rows, heads, D) bf16/fp16/fp32 and s (S, rows, heads) fp32 base-2
    LSEs, both contiguous; sinks optional (heads,) fp32 logits added to the
    denominator only.  Returns v_out (rows, heads, D), or (v_out, s_out) when
    return_lse.  Enqueued on torch's current stream of v's device.
    """
    dev = v.device
    for name, t in (("v", v), ("s", s), ("sinks", sinks), ("v_out", v_out), ("s_out", s_out)):
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{name} must be a GPU tensor on v's device ({dev})")
    if v_out is None:
        v_out = torch.empty(v.shape[1:], dtype=v.dtype, device=dev)
    if return_lse and s_out is None:
        s_out = torch.empty(v.shape[1:3], dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    with torch.cuda.device(dev):
        st = _lib.pkvd_merge_states(_ref(_desc(v)), _ref(_desc(s)), _ref(_desc(sinks)),
                                    _ref(_desc(v_out)), _ref(_desc(s_out)),
                                    ctypes.c_void_p(stream))
    _check(st)
    return (v_out, s_out) if s_out is not None else v_out


def plan(q, k_cache, block_tables, q_len_per_req: int = 1, window_left: int = -1) -> dict:
    """The launch plan the library picks for these shapes (host only)."""
    res = (ctypes.c_int64 * 6)()
    _check(_lib.pkvd_decode_plan(_ref(_desc(q)), _ref(_desc(k_cache)), _ref(_desc(block_tables)),
                                 int(q_len_per_req), int(window_left), ctypes.byref(res)))
    keys = ("path", "rows_per_tile", "row_tiles", "waves", "min_wave_blocks", "workgroups")
    d = dict(zip(keys, list(res)))
    d["path"] = {0: "valu", 1: "mfma"}[d["path"]]
    return d


def workspace_bytes(q, k_cache, block_tables, q_len_per_req: int = 1,
                    window_left: int = -1) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.pkvd_decode_workspace_bytes(_ref(_desc(q)), _ref(_desc(k_cache)),
                                            _ref(_desc(block_tables)), int(q_len_per_req),
                                            int(window_left), ctypes.byref(n)))
    return n.value


def reserve_workspace(nbytes: int, device=None) -> None:
    """Grow the library-owned split workspace of ``device`` before graph capture."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(_lib.pkvd_reserve_workspace(int(nbytes)))


def version() -> str:
    return _lib.pkvd_version().decode()
