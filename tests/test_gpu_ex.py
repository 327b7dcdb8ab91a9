"""GPU parity of the extended call (pkvd_decode_ex) against the fp64 oracle:
packed query rows (qo_indptr), the dense mask, token-major queries, the
output scale and output types, the argument set of
flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache, and
caller-owned workspaces (per call, bound, concurrent streams, graph capture).

Tolerances as in test_gpu_parity: max |out - ref| <= 2e-2 (bf16 / fp16 / fp32
outputs: the kernel's arithmetic is the same whatever the output type) and
max |lse - ref| <= 1e-3, plus <= 1e-2 relative to the largest output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import (LSE_ATOL, OUT_ATOL, _pk, compare, config_inputs, log, schedule,
                             to_dev)

pytestmark = pytest.mark.gpu

ODT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def to_dev_ex(inp):
    d = to_dev(inp)
    if d.get("qo_indptr") is not None:
        d["qo_indptr"] = d["qo_indptr"].cuda()
    return d


def run_ex(d, out_dtype=None, lse=True, **kw):
    pk = _pk()
    res = pk.decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens_kv"],
                    scale=d["scale"], q_len_per_req=d["q_len_per_req"],
                    window_left=d["window_left"], sinks=d.get("sinks"), return_lse=lse,
                    qo_indptr=d.get("qo_indptr"), mask_type=d.get("mask_type", "causal"),
                    out_scale=d.get("out_scale", 1.0), out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    out, l = res if lse else (res, None)
    o = out.float().cpu().numpy().reshape(-1, out.shape[-1])
    return o, (None if l is None else l.cpu().numpy().reshape(-1)), out


# ----------------------------------------------------------------------------
# packed rows, masks, output scale and type on small cases
# ----------------------------------------------------------------------------
PACKED = []
for D in (64, 128):
    for g, qls in ((1, (1, 3, 0, 2)), (2, (2, 2, 1, 0)), (4, (1, 1, 1, 1)), (4, (4, 0, 2, 3)),
                   (8, (1, 2, 0, 4))):
        PACKED.append(dict(D=D, Hq=2 * g, Hkv=2, q_lens=qls, seq_lens=(17, 300, 9, 64)))
PACKED.append(dict(D=128, Hq=8, Hkv=2, q_lens=(3, 1, 4), seq_lens=(5, 2000, 40), window_left=30,
                   sinks=True))
PACKED.append(dict(D=64, Hq=16, Hkv=2, q_lens=(2, 4, 1), seq_lens=(33, 100, 3), window_left=0,
                   page_size=5))
PACKED.append(dict(D=128, Hq=4, Hkv=4, q_lens=(0, 0, 3), seq_lens=(3, 4, 700), page_size=48))


def _id(c):
    return ",".join(f"{k}={v}" for k, v in c.items())


@pytest.mark.parametrize("mask", ["causal", "dense"])
@pytest.mark.parametrize("case", PACKED, ids=[_id(c) for c in PACKED])
def test_packed_rows(case, mask):
    kw = dict(B=len(case["seq_lens"]), page_size=16, seed=13, mask_type=mask, out_scale=0.75)
    kw.update(case)
    inp = workloads.make_case(**kw)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev_ex(inp)
    for sched in ("auto", "cut7", "mk_cut7", "unit"):
        for odt in ("bf16", "fp32"):
            log(f"[packed] {_id(case)} mask={mask} schedule={sched} out={odt}")
            with schedule(sched):
                out, lse, _ = run_ex(d, out_dtype=ODT[odt])
            compare(f"packed/{_id(case)}/{mask}/{sched}/{odt}", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("odt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_output_types_and_scale(dtype, odt):
    """Any of bf16 / fp16 / fp32 out for either input type, times out_scale;
    an fp32 output is the same arithmetic without the final rounding."""
    inp = workloads.make_case(B=3, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(70, 1, 600),
                              dtype=dtype, sinks=True, out_scale=-1.5, window_left=200)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev_ex(inp)
    out, lse, t = run_ex(d, out_dtype=ODT[odt])
    assert t.dtype == ODT[odt]
    compare(f"types/{dtype}->{odt}", out, lse, ref_out, ref_lse)
    if odt == "fp32":
        # rounding the fp32 output gives the bf16 / fp16 call's output exactly
        o16, _, t16 = run_ex(d, out_dtype=ODT[dtype])
        assert torch.equal(t.to(ODT[dtype]), t16)


def test_token_major_query_and_dense_default():
    """batch_decode_with_paged_kv_cache: a fixed seq_len_q > 1 query is
    token-major [B, SQ, Hq, D] and the default mask is dense."""
    pk = _pk()
    inp = workloads.make_case(B=3, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(9, 400, 60),
                              q_len_per_req=3, mask_type="dense")
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev_ex(inp)
    q4 = d["q"].contiguous().reshape(3, 3, 8, 128)
    out, lse = pk.batch_decode_with_paged_kv_cache(q4, (d["k_cache"], d["v_cache"]),
                                                   d["block_tables"], d["seq_lens_kv"],
                                                   seq_len_q=3, return_lse=True)
    torch.cuda.synchronize()
    assert out.shape == q4.shape and lse.shape == (3, 3, 8)
    compare("token_major", out.float().cpu().numpy().reshape(-1, 128),
            lse.cpu().numpy().reshape(-1), ref_out, ref_lse)


def test_combined_paged_kv_cache_and_derived_max_len():
    """One combined (pages, 2, Hkv, ps, D) cache; packed queries whose
    max_seq_len_q the wrapper derives from qo_indptr; bmm2_scale and out_dtype."""
    pk = _pk()
    inp = workloads.make_case(B=4, Hq=16, Hkv=2, D=64, page_size=16, seq_lens=(20, 5, 900, 64),
                              q_lens=(1, 3, 2, 4), mask_type="causal", out_scale=2.0)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev_ex(inp)
    kv = torch.stack([d["k_cache"], d["v_cache"]], dim=1).contiguous()
    out = pk.batch_decode_with_paged_kv_cache(d["q"], kv, d["block_tables"], d["seq_lens_kv"],
                                              qo_indptr=d["qo_indptr"], mask_type="causal",
                                              bmm2_scale=2.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    compare("combined_kv_packed", out.cpu().numpy().reshape(-1, 64), None, ref_out, ref_lse)


def test_spec_verify_shape_ragged():
    """The speculative-verify batch shape (B 32, Hq 32, Hkv 8, D 128, page 16,
    up to 4 query tokens) with ragged per-request query lengths 1..4 as
    packed rows, causal, with LSE: sampled rows against the oracle."""
    w = workloads.CONFIGS["spec_verify"]
    g = torch.Generator().manual_seed(4242)
    qls = torch.randint(1, 5, (w.B,), generator=g).tolist()
    lens = torch.randint(w.kv_lo, w.kv_hi + 1, (w.B,), generator=g).tolist()
    inp = workloads.make_case(B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.page_size,
                              seq_lens=lens, q_lens=qls, seed=4243)
    rows = sum(qls)
    sel = sorted(set(torch.randint(0, rows * w.Hq, (600,), generator=g).tolist()))
    ref_out, ref_lse, _ = oracle.decode(inp, sel=sel)
    d = to_dev_ex(inp)
    for sched in ("auto", "mk_cut7"):
        log(f"[spec_ragged] schedule={sched} rows={rows}")
        with schedule(sched):
            out, lse, _ = run_ex(d)
        compare(f"spec_ragged/{sched}", out[sel], lse[sel], ref_out, ref_lse)


# ----------------------------------------------------------------------------
# full-size workloads through the extended call
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["llama3_8b", "sink_window"])
def test_config_fp32_output_scaled(name):
    """A full workload with an fp32 output and out_scale 0.5: the oracle's
    output times 0.5 (sampled rows), LSE unchanged."""
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev_ex(inp)
    d["out_scale"] = 0.5
    out, lse, _ = run_ex(d, out_dtype=torch.float32)
    compare(f"{name}/fp32x0.5", out, lse, 0.5 * ref_out, ref_lse)


# ----------------------------------------------------------------------------
# caller-owned workspaces
# ----------------------------------------------------------------------------
def _ws_case(seed, lens):
    return workloads.make_case(B=len(lens), Hq=8, Hkv=2, D=128, page_size=16, seq_lens=lens,
                               seed=seed, sinks=True)


def test_per_call_workspace_and_concurrent_streams():
    """Two decodes on two streams, each with its own workspace (cut units
    merged in place, so both use arrival counters), run at the same time;
    each matches the oracle.  A too-small workspace is refused."""
    pk = _pk()
    cases = [_ws_case(31, (3000, 17, 900, 2500)), _ws_case(32, (1200, 4000, 64))]
    refs = [oracle.decode(c) for c in cases]
    devs = [to_dev_ex(c) for c in cases]
    with schedule("cut64"):
        need = [pk.plan_ex(d["q"], d["k_cache"], d["block_tables"], 1)["workspace_bytes"]
                for d in devs]
        wss = [torch.zeros(n, dtype=torch.uint8, device="cuda") for n in need]
        with pytest.raises(_pk().PkvdError):
            pk.decode(devs[0]["q"], devs[0]["k_cache"], devs[0]["v_cache"],
                      devs[0]["block_tables"], devs[0]["seq_lens_kv"],
                      workspace=wss[0][:need[0] - 256])
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        torch.cuda.synchronize()
        outs = []
        for it in range(3):
            res = []
            for d, ws, st in zip(devs, wss, streams):
                with torch.cuda.stream(st):
                    res.append(pk.decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                         d["seq_lens_kv"], sinks=d["sinks"], return_lse=True,
                                         workspace=ws, mask_type="causal"))
            torch.cuda.synchronize()
            outs.append(res)
    for it, res in enumerate(outs):
        for (o, l), (ro, rl, _) in zip(res, refs):
            compare(f"streams/{it}", o.float().cpu().numpy().reshape(-1, 128),
                    l.cpu().numpy().reshape(-1), ro, rl)


def test_bound_workspace():
    """pkvd_set_workspace: calls use the bound buffer (and fail cleanly when it
    is too small) until it is unbound."""
    pk = _pk()
    c = _ws_case(33, (2000, 50, 700))
    ro, rl, _ = oracle.decode(c)
    d = to_dev_ex(c)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens_kv"])
    with schedule("cut64"):
        need = pk.workspace_bytes(d["q"], d["k_cache"], d["block_tables"])
        buf = torch.empty(need, dtype=torch.uint8, device="cuda")
        small = torch.empty(8192, dtype=torch.uint8, device="cuda")
        try:
            pk.set_workspace(small)
            with pytest.raises(pk.PkvdError):
                pk.decode(*args, sinks=d["sinks"])
            pk.set_workspace(buf)
            for it in range(2):
                o, l = pk.decode(*args, sinks=d["sinks"], return_lse=True)
                torch.cuda.synchronize()
                compare(f"bound/{it}", o.float().cpu().numpy().reshape(-1, 128),
                        l.cpu().numpy().reshape(-1), ro, rl)
        finally:
            pk.set_workspace(None)
        o, l = pk.decode(*args, sinks=d["sinks"], return_lse=True)
        torch.cuda.synchronize()
        compare("unbound", o.float().cpu().numpy().reshape(-1, 128), l.cpu().numpy().reshape(-1),
                ro, rl)


def test_graph_replay_after_larger_eager_call():
    """A graph captured on the library's workspace keeps working after an eager
    call grows that workspace (the old buffer is kept, not freed), and a call
    that would have to grow it during a capture fails instead of allocating."""
    pk = _pk()
    small = _ws_case(34, (300, 900))
    big = workloads.make_case(B=64, Hq=8, Hkv=2, D=128, page_size=16,
                              seq_lens=tuple([1500] * 64), seed=35)
    rs = oracle.decode(small)
    ds, db = to_dev_ex(small), to_dev_ex(big)
    with schedule("cut64"):
        pk.reserve_workspace(pk.workspace_bytes(ds["q"], ds["k_cache"], ds["block_tables"]))
        out = torch.empty_like(ds["q"])
        lse = torch.empty(ds["q"].shape[:2], dtype=torch.float32, device="cuda")
        args = (ds["q"], ds["k_cache"], ds["v_cache"], ds["block_tables"], ds["seq_lens_kv"])
        pk.decode(*args, sinks=ds["sinks"], out=out, lse=lse)
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(graph, stream=st):
                pk.decode(*args, sinks=ds["sinks"], out=out, lse=lse)
        torch.cuda.synchronize()
    # a larger plan (more waves and units) grows the library workspace
    with schedule("auto"):
        need_big = pk.workspace_bytes(db["q"], db["k_cache"], db["block_tables"])
        assert need_big > pk.workspace_bytes(ds["q"], ds["k_cache"], ds["block_tables"])
        pk.decode(db["q"], db["k_cache"], db["v_cache"], db["block_tables"], db["seq_lens_kv"])
        torch.cuda.synchronize()
    for it in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare(f"graph_after_growth/{it}", out.float().cpu().numpy().reshape(-1, 128),
                lse.cpu().numpy().reshape(-1), rs[0], rs[1])
    # a call that needs more than the workspace holds, inside a capture: an
    # error, no allocation (the capture itself ends cleanly, empty); one that
    # fits what the workspace already holds is captured
    huge = workloads.make_case(B=64, Hq=32, Hkv=2, D=128, page_size=16,
                               seq_lens=tuple([1500] * 64), seed=36)
    dh = to_dev_ex(huge)
    with schedule("auto"):
        with env_waves("4096"):
            need_h = pk.workspace_bytes(dh["q"], dh["k_cache"], dh["block_tables"])
            assert need_h > need_big
            # earlier tests of the session may have grown the workspace
            # beyond need_h already: then the capture needs no growth
            fits = pk.workspace_capacity() >= need_h
            st2 = torch.cuda.Stream()
            st2.wait_stream(torch.cuda.current_stream())
            g2 = torch.cuda.CUDAGraph()
            raised = False
            with torch.cuda.stream(st2):
                with torch.cuda.graph(g2, stream=st2):
                    try:
                        pk.decode(dh["q"], dh["k_cache"], dh["v_cache"], dh["block_tables"],
                                  dh["seq_lens_kv"])
                    except pk.PkvdError as e:
                        raised = "capturing" in str(e)
            torch.cuda.synchronize()
            assert raised != fits, (fits, raised)


class env_waves:
    def __init__(self, n):
        from test_gpu_parity import env
        self.e = env(PKVD_WAVES=n, PKVD_MIN_WAVE_BLOCKS="1")

    def __enter__(self):
        self.e.__enter__()

    def __exit__(self, *a):
        self.e.__exit__(*a)
