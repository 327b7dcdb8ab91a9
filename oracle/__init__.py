"""fp64 CPU oracle for batched paged-KV decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.  It shares
no code with the HIP path; the two meet only in the seeded inputs of
``workloads``.

The arithmetic lives in ``oracle.c`` (plain C, two-pass softmax in double
precision); this module marshals arrays into it.  See that file's header for
the passages of the documentation each step follows.

Parity status of each function:
  decode          pinned (tests/test_oracle.py: brute force, closed forms,
                  logsumexp, sink, window, causal prefix, GQA, page permutation,
                  page-size repack, merge of disjoint ranges, hand-worked
                  golden cases; packed rows, dense rows and the output scale
                  against the brute force and hand-worked cases)
  merge_states    pinned (merge of disjoint key ranges equals the union)
  prefill         pinned (tests/test_oracle.py: hand-worked cases, torch
                  brute force over masks / GQA / packed rows, equality with
                  the decode definition on one-page caches, closed forms,
                  window key counts, variable windows equal to the causal
                  window, packed rows equal to per-request fixed calls)
  decode, lse with sinks present: the keys-only reading of the LSE is a
                  reading, not fixed by the pages -> parity unpinned for that
                  combination.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "_build", "liboracle_san.so")
# another build of the same source (the sanitized one) for checking runs
_LIB_OVERRIDE = os.environ.get("PKVD_ORACLE_LIBRARY")

BF16, F16 = 0, 1
_ERRORS = {1: "bad argument", 2: "visible key maps outside the page pool", 3: "out of memory"}

_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no fast-math); with
    sanitize, into _build/liboracle_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer (load it with PKVD_ORACLE_LIBRARY and the gcc
    ASan runtime preloaded)."""
    out = _SAN_LIB if sanitize else _LIB
    if sanitize or force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-g"] if sanitize else []
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11"] + san +
                              ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            p, i64, i64,                 # q
            p, i64, i64, i64,            # k
            p, i64, i64, i64,            # v
            ctypes.c_int, i64, i64, i64, i64, i64, i64,
            p, i64, i64,                 # block tables
            p, ctypes.c_double, i64, i64,
            p, ctypes.c_int, ctypes.c_double,   # qo_indptr, causal, out_scale
            p, i64, i64,                 # sinks, key range
            p, i64,                      # sel
            p, p, p, ctypes.c_int]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill.argtypes = [
            p, i64, i64, p, i64, i64, p, i64, i64,      # q, k, v (row, head strides)
            ctypes.c_int, i64, i64, i64, i64, i64, i64,  # dtype, B, Hq, Hkv, D, Sq, Sk
            p, p, ctypes.c_int, i64, p, p,              # qo, kvo, mask, window_left, starts, ends
            ctypes.c_double, ctypes.c_double, p, i64, p, ctypes.c_int]
        lib.oracle_merge_states.restype = None
        lib.oracle_merge_states.argtypes = [p, p, i64, i64, p, p, p]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        _lib = lib
    return _lib


def _bits(t):
    """A torch bf16/fp16 tensor as a uint16 numpy view (no copy), plus its dtype code."""
    import torch
    code = {torch.bfloat16: BF16, torch.float16: F16}[t.dtype]
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16), code


def _i32(t):
    a = t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)
    assert a.dtype == np.int32
    return a


def decode_bits(bits: int, dtype: int) -> float:
    lib = _load()
    return lib.oracle_decode_bf16(bits) if dtype == BF16 else lib.oracle_decode_f16(bits)


def decode(inputs: dict, sel=None, key_range=None, nthreads: int = 0,
           sinks="inputs"):
    """Reference attention for an inputs dict (see ``workloads``).

    Optional keys: ``qo_indptr`` ((B + 1,) int32 cumulative row offsets of
    packed query rows), ``mask_type`` ("causal", the default, or "dense") and
    ``out_scale`` (factor on the output, default 1).  q may be (rows, Hq, D)
    or token-major (B, SQ, Hq, D).

    Returns (out [count, D], lse [count], lse_with_sink [count]) as float64
    numpy arrays; ``count`` is rows*Hq in row-major (row, head) order, or
    len(sel) for an explicit list of flat indices row*Hq + head.
    """
    lib = _load()
    q, k, v = inputs["q"], inputs["k_cache"], inputs["v_cache"]
    if q.dim() == 4:
        q = q.reshape(q.shape[0] * q.shape[1], q.shape[2], q.shape[3])
    qb, code = _bits(q)
    kb, kcode = _bits(k)
    vb, vcode = _bits(v)
    assert code == kcode == vcode
    assert qb.strides[-1] == 2 and kb.strides[-1] == 2 and vb.strides[-1] == 2
    e = 2  # bytes per element
    bt = _i32(inputs["block_tables"])
    n = np.ascontiguousarray(_i32(inputs["seq_lens_kv"]))
    assert bt.strides[1] == 4
    s = inputs["sinks"] if isinstance(sinks, str) else sinks
    s_arr = None if s is None else np.ascontiguousarray(
        s.detach().cpu().numpy() if hasattr(s, "detach") else np.asarray(s), dtype=np.float32)
    R, Hq, D = q.shape
    B = bt.shape[0]
    Lq = int(inputs["q_len_per_req"])
    qo = inputs.get("qo_indptr")
    qo_arr = None if qo is None else np.ascontiguousarray(_i32(qo))
    if qo_arr is None:
        assert R == B * Lq
    else:
        assert qo_arr.shape == (B + 1,) and int(qo_arr[-1]) == R
        Lq = max(1, Lq)
    causal = {"causal": 1, "dense": 0}[inputs.get("mask_type", "causal")]
    out_scale = float(inputs.get("out_scale", 1.0))
    P, Hkv, ps, Dk = k.shape
    assert Dk == D and tuple(v.shape) == tuple(k.shape)
    if sel is None:
        sel_arr, count = None, R * Hq
    else:
        sel_arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
        count = sel_arr.size
    out = np.empty((count, D), dtype=np.float64)
    lse = np.empty((count,), dtype=np.float64)
    lse_ws = np.empty((count,), dtype=np.float64)
    klo, khi = (0, np.iinfo(np.int64).max) if key_range is None else key_range
    ptr = lambda a: None if a is None else a.ctypes.data
    st = lib.oracle_decode(
        ptr(qb), qb.strides[0] // e, qb.strides[1] // e,
        ptr(kb), kb.strides[0] // e, kb.strides[1] // e, kb.strides[2] // e,
        ptr(vb), vb.strides[0] // e, vb.strides[1] // e, vb.strides[2] // e,
        code, B, Hq, Hkv, D, ps, P,
        ptr(bt), bt.strides[0] // 4, bt.shape[1],
        ptr(n), float(inputs["scale"]), Lq, int(inputs["window_left"]),
        ptr(qo_arr), causal, out_scale,
        ptr(s_arr), int(klo), int(khi),
        ptr(sel_arr), count,
        ptr(out), ptr(lse), ptr(lse_ws), int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_decode: {_ERRORS.get(st, st)}")
    return out, lse, lse_ws


_PREFILL_MASKS = {"causal": 0, "dense": 1, "variable_window": 2}


def prefill(inputs: dict, sel=None, nthreads: int = 0):
    """Reference context attention (flashinfer.attention.prims_ts.batch_prefill)
    for an inputs dict with keys q, k, v (fixed [B, S, H, D] or packed
    [total, H, D] with qo_indptr and kv_indptr), mask_type, window_left,
    window_starts / window_ends (variable_window), sm_scale, output_scale.
    Returns out [count, D] float64 (rows x Hq in row-major order, or the
    flat indices row * Hq + head listed in sel)."""
    lib = _load()
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    qo, kvo = inputs.get("qo_indptr"), inputs.get("kv_indptr")
    if qo is None:
        B, Sq, Hq, D = q.shape
        Sk, Hkv = k.shape[1], k.shape[2]
        q, k, v = (t.reshape(t.shape[0] * t.shape[1], t.shape[2], t.shape[3]) for t in (q, k, v))
    else:
        B = qo.numel() - 1
        Sq = Sk = 0
        _, Hq, D = q.shape
        Hkv = k.shape[1]
    qb, code = _bits(q)
    kb, kcode = _bits(k)
    vb, vcode = _bits(v)
    assert code == kcode == vcode
    e = 2
    qo_a = None if qo is None else np.ascontiguousarray(_i32(qo))
    kvo_a = None if kvo is None else np.ascontiguousarray(_i32(kvo))
    mask = _PREFILL_MASKS[inputs.get("mask_type", "dense")]
    st_a = en_a = None
    if mask == 2:
        st_a = np.ascontiguousarray(_i32(inputs["window_starts"]))
        en_a = np.ascontiguousarray(_i32(inputs["window_ends"]))
    rows = q.shape[0]
    sel_arr = None if sel is None else np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    count = rows * Hq if sel is None else sel_arr.size
    out = np.empty((count, D), dtype=np.float64)
    scale = inputs.get("sm_scale")
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    ptr = lambda a: None if a is None else a.ctypes.data
    st = lib.oracle_prefill(
        ptr(qb), qb.strides[0] // e, qb.strides[1] // e,
        ptr(kb), kb.strides[0] // e, kb.strides[1] // e,
        ptr(vb), vb.strides[0] // e, vb.strides[1] // e,
        code, B, Hq, Hkv, D, Sq, Sk, ptr(qo_a), ptr(kvo_a), mask,
        int(inputs.get("window_left", -1)), ptr(st_a), ptr(en_a), scale,
        float(inputs.get("output_scale", 1.0)), ptr(sel_arr), count, ptr(out), int(nthreads))
    if st != 0:
        raise ValueError(f"oracle_prefill: {_ERRORS.get(st, st)}")
    return out


def merge_states(o, lse, sink=None):
    """Merge S partial states (o [S, D], lse [S], base 2) of one row."""
    lib = _load()
    o = np.ascontiguousarray(o, dtype=np.float64)
    l = np.ascontiguousarray(lse, dtype=np.float64)
    S, D = o.shape
    out = np.empty((D,), dtype=np.float64)
    res = np.empty((1,), dtype=np.float64)
    sk = None if sink is None else np.array([sink], dtype=np.float64)
    lib.oracle_merge_states(o.ctypes.data, l.ctypes.data, S, D,
                            None if sk is None else sk.ctypes.data,
                            out.ctypes.data, res.ctypes.data)
    return out, float(res[0])
