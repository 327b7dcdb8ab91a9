"""pkvd_decode_static (the entry point that allocates nothing: its workspace is
a static device array) against pkvd_decode, called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _lib():
    import paged_kv_decode_12_amd as pk
    lib = pk._lib
    P = ctypes.POINTER(pk._Tensor)
    lib.pkvd_decode_static.restype = ctypes.c_int
    lib.pkvd_decode_static.argtypes = [P, P, P, P, P, ctypes.c_float, ctypes.c_int32,
                                       ctypes.c_int32, P, P, P, ctypes.c_void_p]
    return pk, lib


def _static_call(pk, lib, d, out, lse):
    descs = [pk._desc(t) for t in (d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["seq_lens_kv"], d.get("sinks"), out, lse)]
    r = [None if x is None else ctypes.byref(x) for x in descs]
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.pkvd_decode_static(r[0], r[1], r[2], r[3], r[4], float(d["scale"]),
                                int(d["q_len_per_req"]), int(d["window_left"]), r[5], r[6], r[7],
                                ctypes.c_void_p(stream))
    assert st == 0, lib.pkvd_last_error()


def _dev(inp):
    d = dict(inp)
    for k in ("q", "k_cache", "v_cache", "block_tables", "seq_lens_kv", "sinks"):
        if d.get(k) is not None:
            d[k] = d[k].cuda()
    return d


def test_static_entry_point_matches_decode_and_allocates_nothing():
    pk, lib = _lib()
    big = workloads.make_case(B=16, Hq=32, Hkv=8, D=128, page_size=16,
                              seq_lens=tuple(range(700, 700 + 16 * 150, 150)), seed=51,
                              sinks=True)
    small = workloads.make_case(B=3, Hq=8, Hkv=2, D=64, page_size=16, seq_lens=(40, 300, 5),
                                q_len_per_req=2, window_left=50, seed=52)
    cases = [big, small, big]
    devs = [_dev(c) for c in cases]
    # reference outputs of the existing entry point (pkvd_decode; it may allocate)
    refs = []
    for d in devs:
        o, l = pk.decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens_kv"],
                         scale=d["scale"], q_len_per_req=d["q_len_per_req"],
                         window_left=d["window_left"], sinks=d.get("sinks"), return_lse=True)
        refs.append((o, l))
    outs = [(torch.empty_like(o), torch.empty_like(l)) for o, l in refs]
    torch.cuda.synchronize()
    # two calls in a row, the second smaller, then the first again; the
    # device memory the static array occupies is claimed when the library's
    # code object is loaded (at the first call on the device, which also looks
    # up the array's address), and no call after that claims any
    _static_call(pk, lib, devs[0], *outs[0])
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for d, (o, l) in zip(devs[1:], outs[1:]):
        _static_call(pk, lib, d, o, l)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    for i, ((o, l), (ro, rl), c) in enumerate(zip(outs, refs, cases)):
        # the same plan and kernels as pkvd_decode: the same bits
        assert torch.equal(o, ro), i
        assert torch.equal(l, rl), i
        ref_out, ref_lse, _ = oracle.decode(c)
        err = float(np.abs(o.float().cpu().numpy().reshape(-1, o.shape[-1]) - ref_out).max())
        lerr = float(np.abs(l.cpu().numpy().reshape(-1) - ref_lse).max())
        print(f"static call {i}: max|out err|={err:.3e} max|lse err|={lerr:.3e}", flush=True)
        assert err <= 2e-2 and lerr <= 1e-3
