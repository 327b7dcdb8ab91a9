"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances: max |out - ref| <= 2e-2 on bf16/fp16 outputs and max |lse - ref|
<= 1e-3 on the fp32 base-2 LSE.  Because outputs shrink like 1/sqrt(n) at
long contexts, every comparison also bounds the error relative to the largest
reference output (<= 1e-2).
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

OUT_ATOL = 2e-2
LSE_ATOL = 1e-3
REL = 1e-2


def _pk():
    import paged_kv_decode_12_amd as pk
    return pk


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    d = dict(inp)
    for k in ("q", "k_cache", "v_cache", "block_tables", "seq_lens_kv", "sinks"):
        if d.get(k) is not None:
            d[k] = d[k].cuda()
    return d


def run_gpu(dinp, lse=True, **kw):
    pk = _pk()
    res = pk.decode(dinp["q"], dinp["k_cache"], dinp["v_cache"], dinp["block_tables"],
                    dinp["seq_lens_kv"], scale=dinp["scale"],
                    q_len_per_req=dinp["q_len_per_req"], window_left=dinp["window_left"],
                    sinks=dinp.get("sinks"), return_lse=lse, **kw)
    torch.cuda.synchronize()
    if lse:
        out, l = res
        return out.float().cpu().numpy().reshape(-1, out.shape[-1]), l.cpu().numpy().reshape(-1)
    return res.float().cpu().numpy().reshape(-1, res.shape[-1]), None


def compare(name, out, lse, ref_out, ref_lse, out_atol=OUT_ATOL, lse_atol=LSE_ATOL):
    assert np.isfinite(out).all(), f"{name}: non-finite output"
    err = np.abs(out - ref_out)
    scale = max(np.abs(ref_out).max(), 1e-30)
    rms_rel = float(np.sqrt((err ** 2).mean()) / max(np.sqrt((ref_out ** 2).mean()), 1e-30))
    msg = (f"{name}: max|err|={err.max():.3e} max|ref|={scale:.3e} "
           f"max|err|/max|ref|={err.max() / scale:.3e} rms_rel={rms_rel:.3e}")
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse)), f"{name}: -inf rows differ"
        lerr = np.abs(lse[fin] - ref_lse[fin]).max() if fin.any() else 0.0
        msg += f" max|lse err|={lerr:.3e}"
        assert lerr <= lse_atol, msg
    log(msg)
    assert err.max() <= out_atol, msg
    assert err.max() / scale <= REL, msg


_CACHE = {}


def config_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        inp = workloads.make_config(name)
        ref = oracle.decode(inp)
        _CACHE[name] = (inp, ref)
    return _CACHE[name]


CONFIGS = list(workloads.CONFIGS)


@pytest.mark.parametrize("name", CONFIGS)
def test_config_parity(name):
    log(f"[parity] config={name}")
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev(inp)
    log(f"[parity] plan={_pk().plan(d['q'], d['k_cache'], d['block_tables'], d['q_len_per_req'], d['window_left'])}")
    out, lse = run_gpu(d, lse=True)
    compare(name, out, lse, ref_out, ref_lse)
    out2, _ = run_gpu(d, lse=False)
    compare(name + "/no_lse", out2, None, ref_out, ref_lse)
    # with a fixed split of the work (the default), the call without LSE
    # output writes the same out bit for bit
    np.testing.assert_array_equal(out, out2)


@pytest.mark.parametrize("name", CONFIGS)
def test_config_poison(name):
    """NaN in unused pages, tail slots and a padding page: output unchanged."""
    log(f"[poison] config={name}")
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    bad = dict(inp)
    bad["k_cache"], bad["v_cache"], bad["block_tables"] = workloads._poison(
        inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["seq_lens_kv"],
        inp["workload"].page_size)
    out, lse = run_gpu(to_dev(bad), lse=True)
    compare(name + "/poison", out, lse, ref_out, ref_lse)


SCHEDULES = {
    "auto": {},
    "cut7": {"PKVD_WAVES": "7", "PKVD_MIN_WAVE_BLOCKS": "1"},
    "cut64": {"PKVD_WAVES": "64", "PKVD_MIN_WAVE_BLOCKS": "1"},
    # the other engine than the planner picks (MFMA for <= 4 rows, VALU for > 4)
    "mfma_cut7": {"PKVD_FORCE_PATH": "1", "PKVD_WAVES": "7", "PKVD_MIN_WAVE_BLOCKS": "1"},
    "valu": {"PKVD_FORCE_PATH": "0"},
    # cut units merged by the second kernel instead of by their last piece
    "mk_cut7": {"PKVD_MERGE_KERNEL": "1", "PKVD_WAVES": "7", "PKVD_MIN_WAVE_BLOCKS": "1"},
    "mk_mfma_cut64": {"PKVD_MERGE_KERNEL": "1", "PKVD_FORCE_PATH": "1", "PKVD_WAVES": "64",
                      "PKVD_MIN_WAVE_BLOCKS": "1"},
    # slices weighted by the wave's position on its SIMD (5 or 3 fuller
    # workgroups, so that groups hold second waves: the engines that run two
    # waves per SIMD, VALU 8-row tiles and MFMA at D = 64), merged in place
    # and by the merge kernel
    "weighted": {"PKVD_WAVES": "40", "PKVD_MIN_WAVE_BLOCKS": "1", "PKVD_GROUPS": "5",
                 "PKVD_SLOT_W": "140,100", "PKVD_FORCE_PATH": "0"},
    "mk_weighted": {"PKVD_WAVES": "24", "PKVD_MIN_WAVE_BLOCKS": "1", "PKVD_GROUPS": "3",
                    "PKVD_SLOT_W": "90,120", "PKVD_MERGE_KERNEL": "1", "PKVD_FORCE_PATH": "1"},
    # virtual blocks ahead of every unit in the sliced space (slices that
    # start units hold fewer real blocks; some slices hold none)
    "segcost": {"PKVD_SEG_COST": "5", "PKVD_WAVES": "64", "PKVD_MIN_WAVE_BLOCKS": "1"},
    "mk_segcost": {"PKVD_SEG_COST": "3", "PKVD_WAVES": "40", "PKVD_MIN_WAVE_BLOCKS": "1",
                   "PKVD_GROUPS": "5", "PKVD_SLOT_W": "130,100", "PKVD_MERGE_KERNEL": "1",
                   "PKVD_FORCE_PATH": "0"},
    # whole units: slice bounds snap to unit starts (few waves, and the default grid)
    "unit": {"PKVD_UNIT_MODE": "1"},
    "unit_w5": {"PKVD_UNIT_MODE": "1", "PKVD_WAVES": "5", "PKVD_MIN_WAVE_BLOCKS": "1"},
}


class schedule:
    """Temporarily force the persistent grid's wave count (env knobs)."""

    def __init__(self, name):
        self.env = SCHEDULES[name]

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.env}
        os.environ.update(self.env)
        _pk().reload_tuning()

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        _pk().reload_tuning()


class env:
    """Temporarily set environment knobs of the planner."""

    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update(self.kv)
        _pk().reload_tuning()

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        _pk().reload_tuning()


@pytest.mark.parametrize("name,path", [("llama3_8b", "1"), ("spec_verify", "0"),
                                       ("sink_window", "0"), ("long_ctx", "0")])
def test_config_other_engine(name, path):
    """Full-size configs on the engine the planner does not pick for them."""
    log(f"[engine] config={name} PKVD_FORCE_PATH={path}")
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev(inp)
    with env(PKVD_FORCE_PATH=path):
        p = _pk().plan(d["q"], d["k_cache"], d["block_tables"], d["q_len_per_req"],
                       d["window_left"])
        log(f"[engine] plan={p}")
        assert p["path"] == {"0": "valu", "1": "mfma"}[path]
        out, lse = run_gpu(d, lse=True)
    compare(f"{name}/path{path}", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("name,mode", [("llama3_8b", "1"), ("long_ctx", "0"), ("spec_verify", "0"),
                                       ("sink_window", "1"), ("sink_window", "0")])
def test_config_other_merge(name, mode):
    """Full-size configs with the merge mode the planner does not pick for them
    (the sink + window batch, streamed as whole units by default, is cut into
    block slices here and merged both ways)."""
    log(f"[merge] config={name} PKVD_MERGE_KERNEL={mode}")
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev(inp)
    with env(PKVD_MERGE_KERNEL=mode, PKVD_UNIT_MODE="0"):
        out, lse = run_gpu(d, lse=True)
        out2, lse2 = run_gpu(d, lse=True)
    compare(f"{name}/merge{mode}", out, lse, ref_out, ref_lse)
    compare(f"{name}/merge{mode}/again", out2, lse2, ref_out, ref_lse)


@pytest.mark.parametrize("knobs", [{}, {"PKVD_MERGE_KERNEL": "1"}, {"PKVD_FORCE_PATH": "1"}],
                         ids=["in_place", "merge_kernel", "mfma"])
def test_determinism(knobs):
    """The split of the work depends on shapes and lengths only, so repeat
    calls are bitwise identical."""
    name = "llama3_8b"
    log(f"[determinism] {knobs}")
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev(inp)
    with env(**knobs):
        a, la = run_gpu(d)
        b, lb = run_gpu(d)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    compare(f"{name}/{knobs}", a, la, ref_out, ref_lse)


@pytest.mark.parametrize("name", ["llama3_8b", "long_ctx"])
def test_schedule_invariance(name):
    """Other wave counts and slice weights (units cut at other places, merged
    from more pieces) agree with the oracle; the default split twice."""
    inp, (ref_out, ref_lse, _) = config_inputs(name)
    d = to_dev(inp)
    for knobs in ({}, {}, {"PKVD_WAVES": "1"}, {"PKVD_WAVES": "333", "PKVD_MIN_WAVE_BLOCKS": "1"},
                  {"PKVD_WAVES": "5000", "PKVD_MIN_WAVE_BLOCKS": "1"},
                  {"PKVD_SLOT_W": "124,100"}, {"PKVD_SLOT_W": "100,130"},
                  {"PKVD_SLOT_W": "100"},
                  {"PKVD_FORCE_PATH": "0", "PKVD_SLOT_W": "300,100"},
                  {"PKVD_FORCE_PATH": "0", "PKVD_SLOT_W": "100,250", "PKVD_MERGE_KERNEL": "1"},
                  {"PKVD_SEG_COST": "3"}, {"PKVD_SEG_COST": "0"},
                  {"PKVD_SEG_COST": "17", "PKVD_MERGE_KERNEL": "1"},
                  {"PKVD_SEG_COST": "40", "PKVD_MERGE_KERNEL": "0"}):
        log(f"[invariance] config={name} {knobs}")
        with env(**knobs):
            o, l = run_gpu(d)
        compare(f"{name}/{knobs}", o, l, ref_out, ref_lse)


# ----------------------------------------------------------------------------
# edge sweep on small cases
# ----------------------------------------------------------------------------
EDGE = []
for D in (64, 128):
    for ps in (1, 5, 16, 48, 64):
        EDGE.append(dict(D=D, page_size=ps, seq_lens=(1, ps - 1 if ps > 1 else 2, ps, ps + 1, 3 * ps + 7)))
for g, Lq in ((1, 1), (2, 1), (3, 1), (4, 1), (5, 1), (8, 1), (1, 4), (4, 2), (4, 4), (8, 4), (3, 3)):
    EDGE.append(dict(Hq=2 * g, Hkv=2, q_len_per_req=Lq, seq_lens=(Lq, Lq + 1, 17, 300), D=128))
for wl in (0, 1, 15, 16, 100, 400):
    EDGE.append(dict(window_left=wl, seq_lens=(1, 16, 33, 300), D=64, Hq=8, Hkv=1))
    EDGE.append(dict(window_left=wl, seq_lens=(4, 16, 33, 300), D=128, Hq=8, Hkv=2,
                     q_len_per_req=4, sinks=True))
EDGE.append(dict(sinks=True, sink_std=4.0, seq_lens=(3, 40, 200), Hq=16, Hkv=2, D=64,
                 dtype="fp16"))
EDGE.append(dict(dtype="fp16", value_std=0.5, seq_lens=(7, 500), Hq=8, Hkv=1, D=128))
EDGE.append(dict(q_pad_heads=8, bt_pad=3, seq_lens=(9, 70, 129), Hq=8, Hkv=2, D=128))
EDGE.append(dict(value_std=3.0, seq_lens=(64, 1000), Hq=4, Hkv=1, D=128))   # wide score range
EDGE.append(dict(C=40, seq_lens=(640, 17), Hq=4, Hkv=4, D=64, page_size=16))
# the largest pages built (256) and a large non-power-of-two page size
EDGE.append(dict(D=128, page_size=256, seq_lens=(1, 255, 256, 257, 1300), Hq=8, Hkv=2))
EDGE.append(dict(D=64, page_size=128, seq_lens=(3, 128, 129, 700), Hq=16, Hkv=2,
                 q_len_per_req=2, window_left=150))
EDGE.append(dict(D=128, page_size=200, seq_lens=(199, 200, 201, 999), Hq=4, Hkv=1,
                 sinks=True))


def _edge_id(c):
    return ",".join(f"{k}={v}" for k, v in c.items())


@pytest.mark.parametrize("case", EDGE, ids=[_edge_id(c) for c in EDGE])
@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_edge_sweep(case, sched):
    kw = dict(B=len(case["seq_lens"]), Hq=4, Hkv=2, D=64, page_size=16, seed=7)
    kw.update(case)
    inp = workloads.make_case(**kw)
    log(f"[edge] {_edge_id(case)} schedule={sched}")
    ref_out, ref_lse, _ = oracle.decode(inp)
    with schedule(sched):
        out, lse = run_gpu(to_dev(inp))
    # outputs far above 1 (value_std > 1) carry bf16 rounding of up to 2^-8 |out|
    atol = max(OUT_ATOL, 2.0 ** -7 * float(np.abs(ref_out).max()))
    compare(_edge_id(case), out, lse, ref_out, ref_lse, out_atol=atol)


# A long request over many waves: units cut into more pieces than one
# candidate batch of the merge holds (64), on the VALU engine, merged in
# place from equal slices (4-row tiles, one wave per SIMD: the reciprocal
# set-up), in place from weighted slices (8-row tiles, two waves per SIMD:
# the general set-up) and by the merge kernel.  Entries: knobs, query heads.
MANY_PIECES = {
    "inplace_equal": (dict(PKVD_WAVES="300", PKVD_MIN_WAVE_BLOCKS="1", PKVD_MERGE_KERNEL="0",
                           PKVD_FORCE_PATH="0"), 8),
    "inplace_weighted": (dict(PKVD_WAVES="300", PKVD_MIN_WAVE_BLOCKS="1", PKVD_GROUPS="38",
                              PKVD_SLOT_W="140,100", PKVD_MERGE_KERNEL="0", PKVD_FORCE_PATH="0"),
                         16),
    "kernel": (dict(PKVD_WAVES="300", PKVD_MIN_WAVE_BLOCKS="1", PKVD_MERGE_KERNEL="1",
                    PKVD_FORCE_PATH="0"), 8),
}


@pytest.mark.parametrize("sched", list(MANY_PIECES))
def test_units_of_many_pieces(sched):
    pk = _pk()
    knobs, hq = MANY_PIECES[sched]
    inp = workloads.make_case(B=3, Hq=hq, Hkv=2, D=128, page_size=16, seq_lens=(8192, 3000, 17),
                              seed=11)
    log(f"[many-pieces] schedule={sched}")
    with env(**knobs):
        st = pk.schedule_stats(inp["q"], inp["k_cache"], inp["block_tables"], inp["seq_lens_kv"])
        assert st["errors"] == 0 and st["max_pieces"] > 64, st
        out, lse = run_gpu(to_dev(inp))
    ref_out, ref_lse, _ = oracle.decode(inp)
    compare(f"many-pieces/{sched}", out, lse, ref_out, ref_lse)


def test_combined_kv_tensor():
    """K and V as views of one (pages, 2, Hkv, ps, D) tensor (strided pages)."""
    inp = workloads.make_case(B=3, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(5, 60, 131), seed=3)
    kv = torch.stack([inp["k_cache"], inp["v_cache"]], dim=1).contiguous()
    comb = dict(inp, k_cache=kv[:, 0], v_cache=kv[:, 1])
    ref_out, ref_lse, _ = oracle.decode(comb)
    out, lse = run_gpu(to_dev(comb))
    compare("combined_kv", out, lse, ref_out, ref_lse)


def test_short_rows_out_of_contract():
    """n < q_len_per_req: the rows with no visible key give out = 0, lse = -inf."""
    inp = workloads.make_case(B=2, Hq=4, Hkv=2, D=64, page_size=16, seq_lens=(2, 30),
                              q_len_per_req=4, seed=5)
    ref_out, ref_lse, _ = oracle.decode(inp)
    out, lse = run_gpu(to_dev(inp))
    compare("short_rows", out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("sched", ["cut7", "auto", "mk_cut7", "weighted", "mk_weighted", "segcost",
                                   "mk_segcost"])
def test_graph_replay(sched):
    """Capture one call in a HIP graph (workspace reserved first) and replay it
    several times with eager work in between; every replay matches the oracle,
    and equals the eager call bit for bit (the split of the work is fixed)."""
    pk = _pk()
    inp = workloads.make_case(B=4, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(100, 900, 33, 2000),
                              seed=9)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev(inp)
    log(f"[graph] schedule={sched}")
    with schedule(sched):
        pk.reserve_workspace(pk.workspace_bytes(d["q"], d["k_cache"], d["block_tables"]))
        out = torch.empty_like(d["q"])
        lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device="cuda")
        args = (d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens_kv"])
        pk.decode(*args, out=out, lse=lse)
        torch.cuda.synchronize()
        eager_o, eager_l = out.clone(), lse.clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                pk.decode(*args, out=out, lse=lse)
        torch.cuda.synchronize()
        for it in range(4):
            out.zero_()
            lse.zero_()
            _ = (d["q"].float() * 2).sum()          # unrelated eager work
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            o = out.float().cpu().numpy().reshape(-1, out.shape[-1])
            compare(f"graph/{sched}/{it}", o, lse.cpu().numpy().reshape(-1), ref_out, ref_lse)
            assert torch.equal(out, eager_o), it
            assert torch.equal(lse, eager_l), it


def test_bound_decode():
    """bind_decode marshals once; repeated calls equal decode() bit for bit
    and follow in-place updates of the inputs."""
    pk = _pk()
    inp = workloads.make_case(B=3, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(5, 300, 131),
                              sinks=True, seed=11)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev(inp)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens_kv"])
    kw = dict(scale=d["scale"], q_len_per_req=d["q_len_per_req"], window_left=d["window_left"],
              sinks=d.get("sinks"))
    e_out, e_lse = pk.decode(*args, return_lse=True, **kw)
    call = pk.bind_decode(*args, return_lse=True, **kw)
    for it in range(3):
        out, lse = call()
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(lse, e_lse), it
    compare("bound", out.float().cpu().numpy().reshape(-1, out.shape[-1]),
            lse.cpu().numpy().reshape(-1), ref_out, ref_lse)
    # new query values written in place are picked up by the next call
    d["q"].mul_(-1)
    out2, _ = call()
    e2 = pk.decode(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2, e2)


# ----------------------------------------------------------------------------
# cascade merge (pkvd_merge_states)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("S,D,sinks", [(1, 64, False), (2, 128, True), (5, 100, False),
                                       (70, 128, True)])
def test_merge_states_parity(dtype, S, D, sinks):
    """pkvd_merge_states against the oracle's merge of the same states (the
    states' rounded values), with empty states (lse = -inf, v = NaN)."""
    pk = _pk()
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    g = torch.Generator().manual_seed(100 + S + D)
    R, H = 3, 4
    v = torch.randn(S, R, H, D, generator=g).to(tdt)
    s = (torch.randn(S, R, H, generator=g) * 3 + 5).float()
    if S > 1:
        s[0, 1, :] = -float("inf")           # an empty state in some rows
        v[0, 1, :, :] = float("nan")         # ... whose values are never read
    s[:, 2, 1] = -float("inf")               # a row with no state at all
    sk = (torch.randn(H, generator=g) * 2).float() if sinks else None
    log(f"[merge] dtype={dtype} S={S} D={D} sinks={sinks}")
    out, lse = pk.merge_states(v.cuda(), s.cuda(), sinks=None if sk is None else sk.cuda())
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    # an empty state weighs 0: its (NaN) values take no part in the definition
    vv = np.nan_to_num(v.double().numpy(), nan=0.0)
    ss = s.double().numpy()
    tol = 1e-5 if dtype == "fp32" else OUT_ATOL
    for r in range(R):
        for h in range(H):
            ref_o, ref_l = oracle.merge_states(vv[:, r, h, :], ss[:, r, h],
                                               None if sk is None else float(sk[h]))
            if ref_l == -np.inf:
                assert lse[r, h] == -np.inf and np.all(out[r, h] == 0), (r, h)
                continue
            assert np.isfinite(out[r, h]).all(), (r, h)
            assert np.abs(out[r, h] - ref_o).max() <= tol, (r, h, np.abs(out[r, h] - ref_o).max())
            assert abs(lse[r, h] - ref_l) <= LSE_ATOL, (r, h, lse[r, h], ref_l)


@pytest.mark.parametrize("sinks", [False, True])
def test_cascade_merge_equals_full_decode(sinks):
    """Decoding a request's keys as two requests (the first k pages, the
    rest) and merging the two states with pkvd_merge_states (the sink only in
    the merge) equals decoding all keys at once."""
    pk = _pk()
    inp = workloads.make_case(B=1, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=(1000,),
                              sinks=sinks, seed=21)
    ref_out, ref_lse, _ = oracle.decode(inp)
    d = to_dev(inp)
    n, k = 1000, 20                            # split after 20 pages = 320 keys
    bt = d["block_tables"]
    ncol = -(-n // 16)
    two_bt = torch.zeros(2, ncol, dtype=torch.int32, device="cuda")
    two_bt[0, :k] = bt[0, :k]
    two_bt[1, :ncol - k] = bt[0, k:ncol]
    lens = torch.tensor([16 * k, n - 16 * k], dtype=torch.int32, device="cuda")
    q2 = d["q"].repeat(2, 1, 1).contiguous()
    part_out, part_lse = pk.decode(q2, d["k_cache"], d["v_cache"], two_bt, lens,
                                   scale=d["scale"], return_lse=True)
    v = part_out.view(2, 1, *part_out.shape[1:]).contiguous()
    s = part_lse.view(2, 1, part_lse.shape[1]).contiguous()
    out, lse = pk.merge_states(v, s, sinks=d.get("sinks"))
    full_out, full_lse = pk.decode(d["q"], d["k_cache"], d["v_cache"], bt, d["seq_lens_kv"],
                                   scale=d["scale"], sinks=d.get("sinks"), return_lse=True)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().reshape(-1, out.shape[-1])
    compare("cascade", o, lse.cpu().numpy().reshape(-1), ref_out, ref_lse)
    assert (out.float() - full_out.float()).abs().max().item() <= OUT_ATOL
    assert (lse - full_lse).abs().max().item() <= LSE_ATOL


@pytest.mark.parametrize("B,sched", [(3000, "auto"), (8192, "auto"), (3000, "mk_segcost"),
                                     (8192, "cut64")])
def test_large_batches_with_empty_requests(B, sched):
    """Thousands of short requests, some empty (n = 0: no visible key, out = 0,
    lse = -inf): the request search takes two or three 64-way levels and the
    empty requests hold no (virtual) blocks; 8192 is the largest batch built."""
    g = torch.Generator().manual_seed(B)
    lens = torch.randint(0, 41, (B,), generator=g)
    lens[::97] = 0
    inp = workloads.make_case(B=B, Hq=4, Hkv=2, D=64, page_size=16, seq_lens=tuple(lens.tolist()),
                              seed=B + 1)
    ref_out, ref_lse, _ = oracle.decode(inp)
    log(f"[large] B={B} schedule={sched} empty={(lens == 0).sum().item()}")
    with schedule(sched):
        out, lse = run_gpu(to_dev(inp))
    compare(f"large_B{B}_{sched}", out, lse, ref_out, ref_lse)
