"""Batched paged-KV decode attention for AMD MI355X (gfx950).

Thin ctypes binding over ``libpkvd.so`` (C ABI in ``include/pkvd.h``).  This
module only marshals arguments: it turns torch tensors into strided
descriptors, passes torch's current HIP stream and maps status codes to
exceptions.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  If the library has not been built, importing this
package raises ImportError.

Semantics follow flashinfer.cudnn.cudnn_batch_decode_with_kv_cache
(Parameters, Returns, Note): see ``decode``; packed query rows, the mask type
and the output scale and type follow
flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache (summary,
Parameters): see ``batch_decode_with_paged_kv_cache``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["decode", "batch_decode_with_paged_kv_cache", "batch_prefill", "bind_decode",
           "merge_states", "plan",
           "plan_ex", "schedule_stats", "workspace_bytes", "reserve_workspace", "set_workspace",
           "reload_tuning",
           "library_path", "PkvdError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKVD_LIBRARY selects another build of the same library (A/B comparisons)
_LIB_PATH = os.environ.get("PKVD_LIBRARY") or os.path.join(_HERE, "libpkvd.so")

_BF16, _F16, _F32, _I32 = 0, 1, 2, 3
_DT = {torch.bfloat16: _BF16, torch.float16: _F16, torch.float32: _F32, torch.int32: _I32}


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class _DecodeArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.POINTER(_Tensor)), ("k_cache", ctypes.POINTER(_Tensor)),
                ("v_cache", ctypes.POINTER(_Tensor)), ("block_tables", ctypes.POINTER(_Tensor)),
                ("seq_lens_kv", ctypes.POINTER(_Tensor)), ("qo_indptr", ctypes.POINTER(_Tensor)),
                ("q_len", ctypes.c_int32), ("mask", ctypes.c_int32),
                ("window_left", ctypes.c_int32), ("scale", ctypes.c_float),
                ("out_scale", ctypes.c_float), ("sinks", ctypes.POINTER(_Tensor)),
                ("out", ctypes.POINTER(_Tensor)), ("lse", ctypes.POINTER(_Tensor)),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


_MASKS = {"causal": 0, "dense": 1, "variable_window": 2}


class _PrefillArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.POINTER(_Tensor)), ("k", ctypes.POINTER(_Tensor)),
                ("v", ctypes.POINTER(_Tensor)), ("qo_indptr", ctypes.POINTER(_Tensor)),
                ("kv_indptr", ctypes.POINTER(_Tensor)), ("max_seq_len_q", ctypes.c_int32),
                ("mask", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_starts", ctypes.POINTER(_Tensor)),
                ("window_ends", ctypes.POINTER(_Tensor)), ("sm_scale", ctypes.c_float),
                ("output_scale", ctypes.c_float), ("out", ctypes.POINTER(_Tensor))]


class PkvdError(RuntimeError):
    """A HIP or workspace failure reported by the library."""


_ABI_VERSION = "0.2.0"   # pkvd_version() of the argument lists this binding passes


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it first (python paged_kv_decode_12_amd/build.py "
            "or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.pkvd_version.restype = ctypes.c_char_p
    if lib.pkvd_version().decode() != _ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} reports version {lib.pkvd_version().decode()}, this "
                          f"binding passes the arguments of {_ABI_VERSION}: rebuild the library")
    P = ctypes.POINTER(_Tensor)
    lib.pkvd_decode.restype = ctypes.c_int
    lib.pkvd_decode.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                P, P, P, ctypes.c_void_p]
    lib.pkvd_decode_workspace_bytes.restype = ctypes.c_int
    lib.pkvd_decode_workspace_bytes.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.pkvd_reserve_workspace.restype = ctypes.c_int
    lib.pkvd_reserve_workspace.argtypes = [ctypes.c_size_t]
    lib.pkvd_workspace_capacity.restype = ctypes.c_int
    lib.pkvd_workspace_capacity.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.pkvd_decode_plan.restype = ctypes.c_int
    lib.pkvd_decode_plan.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int64 * 6)]
    lib.pkvd_last_error.restype = ctypes.c_char_p
    lib.pkvd_status_string.restype = ctypes.c_char_p
    lib.pkvd_status_string.argtypes = [ctypes.c_int]
    lib.pkvd_version.restype = ctypes.c_char_p
    lib.pkvd_merge_states.restype = ctypes.c_int
    lib.pkvd_merge_states.argtypes = [P, P, P, P, P, ctypes.c_void_p]
    A = ctypes.POINTER(_DecodeArgs)
    lib.pkvd_decode_ex.restype = ctypes.c_int
    lib.pkvd_decode_ex.argtypes = [A, ctypes.c_void_p]
    lib.pkvd_decode_ex_plan.restype = ctypes.c_int
    lib.pkvd_decode_ex_plan.argtypes = [A, ctypes.POINTER(ctypes.c_int64 * 8),
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.pkvd_set_workspace.restype = ctypes.c_int
    lib.pkvd_set_workspace.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.pkvd_reload_tuning.restype = None
    lib.pkvd_reload_tuning.argtypes = []
    lib.pkvd_prefill.restype = ctypes.c_int
    lib.pkvd_prefill.argtypes = [ctypes.POINTER(_PrefillArgs), ctypes.c_void_p]
    lib.pkvd_schedule_stats.restype = ctypes.c_int
    lib.pkvd_schedule_stats.argtypes = [A, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_int64 * 8)]
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


def _stream_of(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _same_device(dev, named):
    for name, t in named:
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError(f"{name} must be a GPU tensor on q's device ({dev})")


def _ex_args(q, k_cache, v_cache, block_tables, seq_lens_kv, qo_indptr, q_len, mask, window_left,
             scale, out_scale, sinks, out, lse, workspace):
    """A pkvd_decode_args struct plus the descriptors it points to (kept alive
    by the returned tuple)."""
    descs = [_desc(t) for t in (q, k_cache, v_cache, block_tables, seq_lens_kv, qo_indptr, sinks,
                                out, lse)]
    P = ctypes.POINTER(_Tensor)
    ptr = lambda d: ctypes.pointer(d) if d is not None else P()
    x = _DecodeArgs()
    (x.q, x.k_cache, x.v_cache, x.block_tables, x.seq_lens_kv, x.qo_indptr, x.sinks, x.out,
     x.lse) = [ptr(d) for d in descs]
    x.q_len = int(q_len)
    x.mask = _MASKS[mask]
    x.window_left = int(window_left)
    x.scale = float(scale)
    x.out_scale = float(out_scale)
    if workspace is not None:
        x.workspace = workspace.data_ptr()
        x.workspace_bytes = workspace.numel() * workspace.element_size()
    return x, descs


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens_kv: torch.Tensor, scale: Optional[float] = None,
           q_len_per_req: int = 1, window_left: int = -1, sinks: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           return_lse: bool = False, stream=None, *, qo_indptr: Optional[torch.Tensor] = None,
           mask_type: str = "causal", out_scale: float = 1.0, out_dtype=None,
           workspace: Optional[torch.Tensor] = None):
    """Batched decode attention over a paged KV cache.

    q            (B * q_len_per_req, Hq, D) bf16/fp16; head_dim innermost and dense;
                 or token-major (B, SQ, Hq, D); or packed (total_q, Hq, D) with
                 qo_indptr ((B + 1,) int32 cumulative row offsets on q's device,
                 q_len_per_req then being the largest rows per request)
    k_cache      (num_pages, Hkv, page_size, D); v_cache the same
    block_tables (B, C) int32;  seq_lens_kv (B,) int32 on q's device
    scale        defaults to 1 / sqrt(D)
    sinks        optional (Hq,) float32 sink logits
    mask_type    "causal" (bottom-right) or "dense"
    out_scale    factor on the output;  out_dtype bf16 / fp16 / fp32 (default: q's)
    workspace    optional caller-owned device buffer (zero-filled before its
                 first use; see workspace_bytes / plan_ex)
    out / lse    optional caller-owned outputs; allocated here when None
    Returns out, or (out, lse) when return_lse or lse is given.  lse is the
    base-2 log-sum-exp over each row's visible keys.  Enqueued on torch's
    current stream of q's device (or ``stream``); never synchronises.  The
    plain form (fixed rows, causal, out_scale 1, out of q's dtype, no
    per-call workspace) calls pkvd_decode; any other pkvd_decode_ex.
    """
    dev = q.device
    _same_device(dev, (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                       ("block_tables", block_tables), ("seq_lens_kv", seq_lens_kv),
                       ("sinks", sinks), ("out", out), ("lse", lse), ("qo_indptr", qo_indptr),
                       ("workspace", workspace)))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    want_lse = return_lse or lse is not None
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    stream = _stream_of(stream, dev)
    plain = (qo_indptr is None and mask_type == "causal" and out_scale == 1.0 and q.dim() == 3
             and out.dtype == q.dtype and workspace is None)
    with torch.cuda.device(dev):
        if plain:
            st = _lib.pkvd_decode(_ref(_desc(q)), _ref(_desc(k_cache)), _ref(_desc(v_cache)),
                                  _ref(_desc(block_tables)), _ref(_desc(seq_lens_kv)),
                                  float(scale), int(q_len_per_req), int(window_left),
                                  _ref(_desc(sinks)), _ref(_desc(out)),
                                  _ref(_desc(lse) if want_lse else None), ctypes.c_void_p(stream))
        else:
            x, keep = _ex_args(q, k_cache, v_cache, block_tables, seq_lens_kv, qo_indptr,
                               q_len_per_req, mask_type, window_left, scale, out_scale, sinks,
                               out, lse if want_lse else None, workspace)
            st = _lib.pkvd_decode_ex(ctypes.byref(x), ctypes.c_void_p(stream))
    _check(st)
    return (out, lse) if want_lse else out


def batch_decode_with_paged_kv_cache(q: torch.Tensor, paged_kv_cache, block_tables: torch.Tensor,
                                     seq_lens_kv: torch.Tensor, *, seq_len_q: int = 1,
                                     qo_indptr: Optional[torch.Tensor] = None,
                                     max_seq_len_q: Optional[int] = None,
                                     mask_type: str = "dense", window_left: int = -1,
                                     kv_layout: str = "HND", bmm1_scale: Optional[float] = None,
                                     bmm2_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                                     out_dtype=None, sinks: Optional[torch.Tensor] = None,
                                     return_lse: bool = False, workspace=None, stream=None):
    """Fixed or packed-query paged decode (the argument set of
    flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache).

    q            [B, Hq, D] (one token), token-major [B, SQ, Hq, D] for a fixed
                 seq_len_q > 1, or packed [total_q, Hq, D] with qo_indptr
    paged_kv_cache  a (K, V) tuple of (pages, Hkv, page_size, D) tensors, or one
                 combined (pages, 2, Hkv, page_size, D) tensor (HND layout)
    max_seq_len_q  packed capacity; when omitted it is derived from qo_indptr
                 once (a device-to-host read, so that form is not
                 graph-capturable), unless a non-default seq_len_q supplies it
    mask_type    "dense" (default, as documented) or "causal" (bottom-right)
    bmm1_scale   softmax scale (default 1 / sqrt(D));  bmm2_scale  output factor
    out_dtype    output dtype (default: out's, else q's)
    Returns the output in q's layout, or (out, lse) with return_lse.
    """
    if kv_layout != "HND":
        raise NotImplementedError("only the HND paged layout is built")
    if isinstance(paged_kv_cache, (tuple, list)):
        k_cache, v_cache = paged_kv_cache
    else:
        if paged_kv_cache.dim() != 5 or paged_kv_cache.shape[1] != 2:
            raise ValueError("a combined paged_kv_cache must be (pages, 2, Hkv, page_size, D)")
        k_cache, v_cache = paged_kv_cache[:, 0], paged_kv_cache[:, 1]
    if qo_indptr is not None:
        if q.dim() != 3:
            raise ValueError("packed queries are [total_q, Hq, D]")
        if max_seq_len_q is None:
            if seq_len_q != 1:
                max_seq_len_q = seq_len_q
            else:
                qo = qo_indptr.cpu()
                max_seq_len_q = max(1, int((qo[1:] - qo[:-1]).max())) if qo.numel() > 1 else 1
        elif seq_len_q != 1 and seq_len_q != max_seq_len_q:
            raise ValueError("seq_len_q and max_seq_len_q disagree")
        q_len = int(max_seq_len_q)
    else:
        if max_seq_len_q is not None and max_seq_len_q != seq_len_q:
            raise ValueError("in fixed-query mode max_seq_len_q must equal seq_len_q")
        q_len = int(seq_len_q)
        if q.dim() == 4 and q.shape[1] != q_len:
            raise ValueError("a [B, SQ, Hq, D] query needs SQ == seq_len_q")
        if q.dim() == 3 and q_len != 1:
            raise ValueError("a fixed seq_len_q > 1 query is token-major [B, SQ, Hq, D]")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    return decode(q, k_cache, v_cache, block_tables, seq_lens_kv, scale=bmm1_scale,
                  q_len_per_req=q_len, window_left=window_left, sinks=sinks, out=out,
                  return_lse=return_lse, stream=stream, qo_indptr=qo_indptr,
                  mask_type=mask_type, out_scale=bmm2_scale, out_dtype=out_dtype,
                  workspace=workspace)


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


def batch_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                  qo_indptr: Optional[torch.Tensor] = None,
                  kv_indptr: Optional[torch.Tensor] = None, mask_type: str = "dense",
                  window_left: int = -1,
                  variable_window_token_starts: Optional[torch.Tensor] = None,
                  variable_window_token_ends: Optional[torch.Tensor] = None,
                  sm_scale: Optional[float] = None, output_scale: float = 1.0, out_dtype=None,
                  out: Optional[torch.Tensor] = None, max_seq_len_q: Optional[int] = None,
                  stream=None) -> torch.Tensor:
    """Context attention over fixed [B, S, H, D] or packed [total, H, D] q, k, v
    (the argument set of flashinfer.attention.prims_ts.batch_prefill; pkvd_prefill).

    mask_type "dense", "causal" (bottom-right) or "variable_window" (fixed
    shapes; inclusive int32 [B, Sq] bounds).  With packed rows the largest
    query count sizes the grid: pass max_seq_len_q, or it is derived from
    qo_indptr here (a device-to-host read).  Returns out (q's shape, out_dtype
    or out's dtype or q's).  Enqueued on torch's current stream as two
    kernels (the second recomputes, with a rescaling pass, the row groups
    whose probabilities overflowed their format in the first, which marks
    them in out); never synchronises otherwise.
    """
    dev = q.device
    _same_device(dev, (("q", q), ("k", k), ("v", v), ("qo_indptr", qo_indptr),
                       ("kv_indptr", kv_indptr), ("out", out),
                       ("variable_window_token_starts", variable_window_token_starts),
                       ("variable_window_token_ends", variable_window_token_ends)))
    if (qo_indptr is None) != (kv_indptr is None):
        raise ValueError("qo_indptr and kv_indptr are given together")
    if qo_indptr is not None and max_seq_len_q is None:
        qo = qo_indptr.cpu()
        max_seq_len_q = max(1, int((qo[1:] - qo[:-1]).max())) if qo.numel() > 1 else 1
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    descs = [_desc(t) for t in (q, k, v, qo_indptr, kv_indptr, variable_window_token_starts,
                                variable_window_token_ends, out)]
    P = ctypes.POINTER(_Tensor)
    ptr = lambda d: ctypes.pointer(d) if d is not None else P()
    x = _PrefillArgs()
    (x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, x.window_starts, x.window_ends, x.out) = \
        [ptr(d) for d in descs]
    x.max_seq_len_q = int(max_seq_len_q or 0)
    x.mask = _MASKS[mask_type]
    x.window_left = int(window_left)
    x.sm_scale = float(sm_scale)
    x.output_scale = float(output_scale)
    with torch.cuda.device(dev):
        st = _lib.pkvd_prefill(ctypes.byref(x), ctypes.c_void_p(_stream_of(stream, dev)))
    _check(st)
    return out


def plan(q, k_cache, block_tables, q_len_per_req: int = 1, window_left: int = -1) -> dict:
    """The launch plan the library picks for a pkvd_decode call (host only)."""
    res = (ctypes.c_int64 * 6)()
    _check(_lib.pkvd_decode_plan(_ref(_desc(q)), _ref(_desc(k_cache)), _ref(_desc(block_tables)),
                                 int(q_len_per_req), int(window_left), ctypes.byref(res)))
    keys = ("path", "rows_per_tile", "row_tiles", "waves", "min_wave_blocks", "workgroups")
    d = dict(zip(keys, list(res)))
    d["path"] = {0: "valu", 1: "mfma"}[d["path"]]
    return d


def plan_ex(q, k_cache, block_tables, q_len: int = 1, window_left: int = -1, *,
            qo_indptr=None, mask_type: str = "causal") -> dict:
    """The plan of a pkvd_decode_ex call (host only; shapes are read, data
    never): path, tiling, grid, merge mode, whole-unit mode and the
    workspace bytes it needs."""
    x, keep = _ex_args(q, k_cache, k_cache, block_tables, None, qo_indptr, q_len, mask_type,
                       window_left, 1.0, 1.0, None, None, None, None)
    res = (ctypes.c_int64 * 8)()
    nbytes = ctypes.c_size_t(0)
    _check(_lib.pkvd_decode_ex_plan(ctypes.byref(x), ctypes.byref(res), ctypes.byref(nbytes)))
    keys = ("path", "rows_per_tile", "row_tiles", "waves", "min_wave_blocks", "workgroups",
            "merge_kernel", "unit_mode")
    d = dict(zip(keys, list(res)))
    d["path"] = {0: "valu", 1: "mfma"}[d["path"]]
    d["workspace_bytes"] = nbytes.value
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


def workspace_capacity(device=None) -> int:
    """Bytes the workspace of ``device``'s next decode holds (pkvd_workspace_capacity)."""
    n = ctypes.c_size_t(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(_lib.pkvd_workspace_capacity(ctypes.byref(n)))
    return n.value


def set_workspace(buf: Optional[torch.Tensor], device=None) -> None:
    """Bind a caller-owned device buffer (any dtype, 256-byte aligned, kept
    alive by the caller) as the workspace of later calls on its device, or
    unbind with None (pkvd_set_workspace; zero-fills the buffer)."""
    dev = buf.device if buf is not None else (device if device is not None
                                              else torch.cuda.current_device())
    with torch.cuda.device(dev):
        if buf is None:
            _check(_lib.pkvd_set_workspace(None, 0))
        else:
            _check(_lib.pkvd_set_workspace(ctypes.c_void_p(buf.data_ptr()),
                                           buf.numel() * buf.element_size()))


def schedule_stats(q, k_cache, block_tables, seq_lens_kv, q_len: int = 1, window_left: int = -1,
                   *, qo_indptr=None, mask_type: str = "causal") -> dict:
    """Host replay of the schedule a pkvd_decode_ex call with these shapes
    would run over the given lengths (pkvd_schedule_stats): blocks, waves,
    units, units cut between waves and their pieces, and inconsistencies
    found (0 for a sound schedule).  Tensors may live on the CPU; only the
    lengths (and packed offsets) are read."""
    import numpy as np
    n = np.ascontiguousarray(seq_lens_kv.detach().cpu().numpy().astype(np.int32))
    qo = None if qo_indptr is None else np.ascontiguousarray(
        qo_indptr.detach().cpu().numpy().astype(np.int32))
    x, keep = _ex_args(q, k_cache, k_cache, block_tables, None, qo_indptr, q_len, mask_type,
                       window_left, 1.0, 1.0, None, None, None, None)
    res = (ctypes.c_int64 * 8)()
    _check(_lib.pkvd_schedule_stats(ctypes.byref(x), n.ctypes.data,
                                    None if qo is None else qo.ctypes.data, ctypes.byref(res)))
    keys = ("blocks", "waves", "units", "cut_units", "pieces", "max_pieces", "errors",
            "virtual_blocks")
    return dict(zip(keys, list(res)))


def reload_tuning() -> None:
    """Re-read the PKVD_* planner overrides from the environment."""
    _lib.pkvd_reload_tuning()


def version() -> str:
    return _lib.pkvd_version().decode()
