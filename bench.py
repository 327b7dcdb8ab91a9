#!/usr/bin/env python3
"""Throughput of batched paged-KV decode on one MI355X.

One step = one pkvd_decode call over one seeded synthetic batch already
resident in HBM.  Default workload: the Llama-3-8B-shaped batch (B=64, Hq=32,
Hkv=8, D=128, page_size=16, seq_lens_kv uniform in [512, 4096], bf16).

Printed metric: effective KV-read GB/s = algorithmic K+V bytes per call / time
per call, where algorithmic bytes = 2 * D * elt * Hkv * sum_b |keys some row of
request b can see| (each K/V byte once per kv head).

Also reported:
  roofline      the average duration of one call (the decode kernel, plus the
                merge kernel when the plan uses it), from HIP events on the
                launch stream around the timed back-to-back calls, against the
                8 TB/s HBM3E peak;
  cpu_baseline  the fp64 CPU oracle (test infrastructure) timed on the host
                cores on the same workload, as a reported baseline only;
  cold          per-call time with the 256 MB Infinity Cache and L2 flushed by a
                1 GiB read before every call (outside the events).

roofline.traffic is the HBM bytes per launch that rocprofv3's FETCH_SIZE and
WRITE_SIZE counters gave for this workload, scaled by what the same counters
read for a plain device copy of known size (``--copy-calibration`` runs that
copy).  The figures live in profiles/decode_<workload>_hbm_traffic.txt together
with a SHA-256 of the kernel sources they were taken with; when the sources
have changed since, traffic is null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective KV-read GB/s (% of HBM peak) and µs/call, batched paged decode"
HBM_PEAK_GBS = 8000.0


def kv_bytes(inp) -> int:
    """Algorithmic K+V bytes of one call: every key some row of a request can
    see (the union of the rows' causal/window ranges), once per kv head."""
    Lq, wl = inp["q_len_per_req"], inp["window_left"]
    k = inp["k_cache"]
    elt, Hkv, D = k.element_size(), k.shape[1], k.shape[-1]
    keys = 0
    for n in inp["seq_lens_kv"].tolist():
        keys += n if wl < 0 else min(n, wl + Lq)
    return 2 * D * elt * Hkv * keys


# sources each kernel family is built from (its counters stay valid while these do not change)
PREFILL_ONLY = ("prefill_kernel.hip", "prefill_args.h", "prefill_api.cpp")
PREFILL_SHARED = ("engine_mfma.h", "decode_common.h", "decode_args.h", "schedule.h", "api_util.h",
                  "pkvd.h")


def kernel_source_hash(op: str = "decode") -> str:
    """SHA-256 over the sources and build flags one kernel family is built
    from (what its counters measured): op "decode" (decode and merge kernels)
    or "prefill"."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pkvd_build", os.path.join(ROOT, "paged_kv_decode_12_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = hashlib.sha256()
    for path in b.SOURCES + b.HEADERS:
        name = os.path.basename(path)
        if op == "prefill" and name not in PREFILL_ONLY + PREFILL_SHARED:
            continue
        if op == "decode" and name in PREFILL_ONLY:
            continue
        with open(path, "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    h.update(" ".join(b.FLAGS[:-2]).encode())      # flags minus the machine-specific -I paths
    return h.hexdigest()


def stored_traffic(workload: str, op: str = "decode"):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{op}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash(op):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE
    and WRITE_SIZE counters (each dispatch reads and writes exactly nbytes)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": nbytes, "dispatches": reps}),
          flush=True)


def bench_merge_states(args):
    """The cascade merge (pkvd_merge_states) on S = 16 bf16 states of the
    llama3_8b batch's 64 x 32 (row, head) pairs, D = 128, with sinks: HBM
    bytes per call = S (D elt + 4) read + (D elt + 4) written per pair."""
    import numpy as np
    import torch
    import oracle
    import paged_kv_decode_12_amd as pk

    S, R, H, D = 16, 64, 32, 128
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = torch.Generator().manual_seed(2024)
    v_cpu = torch.randn(S, R, H, D, generator=g).to(torch.bfloat16)
    s_cpu = (torch.randn(S, R, H, generator=g) * 3 + 5).float()
    sk_cpu = torch.randn(H, generator=g).float()
    v, s, sk = v_cpu.to(dev), s_cpu.to(dev), sk_cpu.to(dev)
    out = torch.empty(R, H, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(R, H, dtype=torch.float32, device=dev)
    nbytes = R * H * (S * (D * 2 + 4) + D * 2 + 4)
    step = lambda: pk.merge_states(v, s, sinks=sk, v_out=out, s_out=lse)
    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    # spot check of a few (row, head) pairs against the oracle's merge
    o = out.float().cpu().numpy()
    err = 0.0
    for r, h in ((0, 0), (17, 5), (63, 31)):
        ref, _ = oracle.merge_states(v_cpu[:, r, h].double().numpy(),
                                     s_cpu[:, r, h].double().numpy(), float(sk_cpu[h]))
        err = max(err, float(np.abs(o[r, h] - ref).max()))
    print(json.dumps({"op": "merge_states", "us_per_call": round(us, 3),
                      "GBps": round(nbytes / (us * 1e-6) / 1e9, 2), "bytes_per_call": nbytes,
                      "config": {"S": S, "rows": R, "heads": H, "D": D, "dtype": "bf16",
                                 "sinks": True},
                      "steps": args.steps, "max_abs_err_sampled": err}), flush=True)


def prefill_flops(inp) -> int:
    """Algorithmic flops of one context-attention call: 4 * D per visible
    (query row, query head, key) triple (2 D for q . k, 2 D for p . v)."""
    import numpy as np
    q, k = inp["q"], inp["k"]
    D, Hq = q.shape[-1], q.shape[-2]
    mask, wl = inp["mask_type"], inp["window_left"]
    if inp.get("qo_indptr") is not None:
        qo, kvo = inp["qo_indptr"].tolist(), inp["kv_indptr"].tolist()
        lens = [(qo[b + 1] - qo[b], kvo[b + 1] - kvo[b]) for b in range(len(qo) - 1)]
    else:
        lens = [(q.shape[1], k.shape[1])] * q.shape[0]
    pairs = 0
    for b, (sq, sk) in enumerate(lens):
        i = np.arange(sq, dtype=np.int64)
        if mask == "variable_window":
            lo = np.maximum(inp["window_starts"][b].numpy().astype(np.int64), 0)
            hi = np.minimum(inp["window_ends"][b].numpy().astype(np.int64), sk - 1)
        else:
            p = sk - sq + i
            hi = np.minimum(p if mask == "causal" else np.full_like(i, sk - 1), sk - 1)
            lo = np.zeros_like(i) if wl < 0 else np.maximum(p - wl, 0)
        pairs += int(np.maximum(hi - lo + 1, 0).sum())
    return 4 * D * Hq * pairs


def bench_prefill(args):
    """Context attention (pkvd_prefill) on one of the prefill workloads:
    TFLOP/s of algorithmic flops (4 D per visible query-key pair and head)
    against the dense bf16/fp16 MFMA peak, HIP events around `steps`
    back-to-back calls on the launch stream; sampled rows checked against the
    oracle, which is also timed on those rows as the CPU baseline."""
    import numpy as np
    import torch
    import workloads
    import paged_kv_decode_12_amd as pk
    name = args.config if args.config in workloads.PREFILL_CONFIGS else "prefill_causal_d128"
    inp = workloads.make_prefill_config(name)
    flops = prefill_flops(inp)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = torch.empty_like(d["q"])
    step = lambda: pk.batch_prefill(d["q"], d["k"], d["v"], qo_indptr=d.get("qo_indptr"),
                                    kv_indptr=d.get("kv_indptr"), mask_type=d["mask_type"],
                                    window_left=d["window_left"], sm_scale=d["sm_scale"],
                                    output_scale=d["output_scale"], out=out,
                                    max_seq_len_q=d.get("max_seq_len_q"))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    tflops = flops / (us * 1e-6) / 1e12
    peak = 2500.0
    res = {"op": "prefill", "metric": "context-attention TFLOP/s (4 D flops per visible "
                                      "query-key pair and head)",
           "value": round(tflops, 2), "unit": "TFLOP/s", "us_per_call": round(us, 3),
           "steps": args.steps, "warmup": args.warmup,
           "dtype": "bf16" if inp["q"].dtype == torch.bfloat16 else "fp16",
           "config": {"workload": name, **{k: v for k, v in workloads.PREFILL_CONFIGS[name].items()
                                          if k != "seed"}},
           "flops_per_call": flops,
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                        "traffic": stored_traffic(name, "prefill")}}
    if not args.no_check or args.cpu_seconds > 0:
        import oracle
        rows = out.shape[0] * (out.shape[1] if out.dim() == 4 else 1)
        Hq = out.shape[-2]
        g = torch.Generator().manual_seed(7)
        sel = sorted(set(torch.randint(0, rows * Hq, (64,), generator=g).tolist()) |
                     {rows * Hq - 1})
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t = time.perf_counter()
        ref = oracle.prefill(inp, sel=sel, nthreads=threads)
        t_cpu = time.perf_counter() - t
        got = out.float().cpu().numpy().reshape(-1, out.shape[-1])[sel]
        res["check"] = {"max_abs_err_out_sampled": float(np.abs(got - ref).max()),
                        "rows_sampled": len(sel)}
        sflops = flops / (rows * Hq) * len(sel)   # the sample's share (rows differ in length)
        res["cpu_baseline"] = {"value": round(sflops / t_cpu / 1e12, 6), "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{len(sel)} sampled (row, head) pairs of {name}, "
                                         f"{t_cpu:.2f} s, fp64 C + OpenMP (flops prorated by "
                                         "the mean visible keys per row)",
                               "cpu": cpu_model()}
    print(json.dumps(res), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _ceiling_lib():
    import ctypes
    path = os.path.join(ROOT, "paged_kv_decode_12_amd", "libpkvd_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "pkvd_ceiling_abi") or lib.pkvd_ceiling_abi() != 2:
        raise SystemExit(f"{path} is stale (argument lists differ): rebuild it")
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.pkvd_ceiling_stream_read.restype = ctypes.c_int
    c = ctypes.c_int
    lib.pkvd_ceiling_stream_read.argtypes = [p, i64, c, c, p, p]
    lib.pkvd_ceiling_paged_gather.restype = ctypes.c_int
    lib.pkvd_ceiling_paged_gather.argtypes = [p, p, p, p, i64, c, c, c, c, c, p, p]
    return lib


def decode_blocks(inp):
    """Byte offsets (K and V) of every 16-key block a decode call of these
    inputs streams: per (request, kv head), the blocks covering the keys some
    row of the request sees, in the decode's unit order."""
    import numpy as np
    k, v = inp["k_cache"], inp["v_cache"]
    elt = k.element_size()
    P, Hkv, ps, D = k.shape
    if ps < 16 or ps & (ps - 1):
        raise SystemExit("the paged-gather ceiling needs a power-of-two page_size >= 16")
    bt = inp["block_tables"].numpy()
    Lq, wl = inp["q_len_per_req"], inp["window_left"]
    ko, vo = [], []
    for b, n in enumerate(inp["seq_lens_kv"].tolist()):
        lo = 0 if wl < 0 else max(0, n - Lq - wl)
        if n <= lo:
            continue
        blocks = np.arange(lo // 16, (n - 1) // 16 + 1, dtype=np.int64)
        pages = bt[b, (blocks * 16) // ps].astype(np.int64)
        slot = (blocks * 16) % ps
        for h in range(Hkv):
            ko.append((pages * k.stride(0) + h * k.stride(1) + slot * D) * elt)
            vo.append((pages * v.stride(0) + h * v.stride(1) + slot * D) * elt)
    return np.concatenate(ko), np.concatenate(vo), 16 * D * elt


def bench_ceiling(args):
    """Memory-system references for a workload's bytes (ceiling.hip): a plain
    streaming read of the decode's algorithmic byte count, and the decode's own
    16-key block gather (every K/V block it streams, no arithmetic), with
    loads into registers or staged through LDS.  Same grid as the decode
    (its plan's waves); times from HIP events around `steps` back-to-back
    launches."""
    import numpy as np
    import torch
    import workloads
    import paged_kv_decode_12_amd as pk
    lib = _ceiling_lib()
    w = workloads.CONFIGS[args.config]
    inp = workloads.make_config(args.config)
    nbytes = kv_bytes(inp)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    plan = pk.plan(inp["q"], inp["k_cache"], inp["block_tables"], w.q_len_per_req, w.window_left)
    wpg = 4 * args.waves_per_simd
    nw = 256 * wpg if args.waves_per_simd != 1 else int(plan["waves"])
    sink = torch.empty(nw * 64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.op == "stream_read":
        total = (nbytes + 1023) // 1024 * 1024
        buf = torch.ones(total // 4, dtype=torch.int32, device=dev)
        call = lambda: lib.pkvd_ceiling_stream_read(buf.data_ptr(), total, nw, wpg,
                                                    sink.data_ptr(), stream.cuda_stream)
        read_bytes = total
    else:
        ko, vo, blk = decode_blocks(inp)
        k, v = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
        kot = torch.from_numpy(ko).to(dev)
        vot = torch.from_numpy(vo).to(dev)
        call = lambda: lib.pkvd_ceiling_paged_gather(k.data_ptr(), v.data_ptr(), kot.data_ptr(),
                                                     vot.data_ptr(), ko.size, blk, nw, wpg,
                                                     args.pf, 1 if args.lds else 0,
                                                     sink.data_ptr(), stream.cuda_stream)
        read_bytes = 2 * ko.size * blk
    for _ in range(args.warmup):
        if call() != 0:
            raise SystemExit("ceiling kernel launch failed")
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    kind = args.op + ("_lds" if args.op == "paged_gather" and args.lds else "")
    print(json.dumps({"op": kind, "config": args.config, "waves": nw,
                      "blocks_in_flight_per_wave": args.pf if args.op == "paged_gather" else None,
                      "us_per_launch": round(us, 3),
                      "bytes_read_per_launch": read_bytes,
                      "GBps_read": round(read_bytes / (us * 1e-6) / 1e9, 1),
                      "frac_of_peak": round(read_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "decode_kv_bytes": nbytes,
                      "decode_us_at_this_rate": round(nbytes / (read_bytes / us), 2),
                      "steps": args.steps}), flush=True)


# ----------------------------------------------------------------------------
# rocprofv3 csv -> profiles/ summaries
# ----------------------------------------------------------------------------
PROFILE_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL {t} rocprofv3 {what} -d "
               "$REPO/gpurun_out/prof/{tag} -o {tag} --output-format csv -- python3 $REPO/bench.py "
               "{bargs}")


def _csv_rows(pattern):
    import csv
    import glob
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise SystemExit(f"no rocprofv3 output matches {pattern}")
    out = []
    for f in files:
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def _per_dispatch(rows, counter, kfilter):
    """`counter` per dispatch of kernels whose name contains kfilter, summed
    over its instances (SEs, XCDs) -- or, for the GRBM_ cycle counters, their
    maximum (rocprofv3's own reduction for them) -> per-dispatch list."""
    per = {}
    agg = max if counter.startswith("GRBM_") else (lambda a, b: a + b)
    for r in rows:
        if kfilter in r["Kernel_Name"] and r["Counter_Name"] == counter:
            k = r["Dispatch_Id"]
            per[k] = agg(per[k], float(r["Counter_Value"])) if k in per else float(r["Counter_Value"])
    return [per[k] for k in sorted(per, key=int)]


DERIVED = ["MfmaUtil", "VALUBusy", "OccupancyPercent", "LDSBankConflict"]

SQ_SETS = {
    "sq_a": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
             "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY",
             "GRBM_GUI_ACTIVE"],
    "sq_b": ["SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU",
             "SQ_ACTIVE_INST_ANY", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
             "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"],
    # where issue time goes: waiting (any / for an instruction / for LDS) vs active by type
    "sq_c": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
             "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA",
             "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"],
}


def summarize(args):
    """Write a profiles/ summary from rocprofv3 csv output under --prof-dir
    (the directory a rocprofv3 -d run wrote).  Kinds: trace (kernel-trace
    statistics), fetch / write (FETCH_SIZE or WRITE_SIZE in KiB per dispatch,
    combined into one traffic file once both exist), sq_a / sq_b (SQ counter
    sets), calibration (a plain 1 GiB copy: the counter scale factors)."""
    import statistics
    kind, d, w = args.summarize, args.prof_dir, args.config
    pre = args.op == "prefill"
    fam = "prefill" if pre else "decode"          # file prefix and kernel family
    kfilter = "prefill_kernel" if pre else "decode_kernel"
    bargs = (f"--op prefill --config {w} --steps 5 --warmup 1 --cpu-seconds 0 --no-check" if pre
             else f"--config {w} --steps 10 --warmup 2 --cold-iters 0 --cpu-seconds 0 --no-check")
    sha = kernel_source_hash(fam)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if kind == "calibration":
        f = _per_dispatch(_csv_rows(d + "/fetch/**/*counter_collection.csv"), "FETCH_SIZE", "copyBuffer")
        wr = _per_dispatch(_csv_rows(d + "/write/**/*counter_collection.csv"), "WRITE_SIZE", "copyBuffer")
        nbytes = 1 << 30
        L = ["# FETCH_SIZE / WRITE_SIZE calibration: a plain 1 GiB device-to-device copy",
             "# (torch copy_ -> __amd_rocclr_copyBuffer), each dispatch reads and writes exactly 1 GiB",
             "command_fetch: " + PROFILE_CMD.format(t=60, what="--pmc FETCH_SIZE", tag="calib/fetch",
                                                    bargs="--copy-calibration"),
             "command_write: " + PROFILE_CMD.format(t=60, what="--pmc WRITE_SIZE", tag="calib/write",
                                                    bargs="--copy-calibration"),
             f"dispatches: {len(f)}",
             f"fetch_kib_per_dispatch: {statistics.mean(f):.2f}",
             f"write_kib_per_dispatch: {statistics.mean(wr):.2f}",
             f"bytes_per_dispatch: {nbytes}",
             f"fetch_factor: {nbytes / (statistics.mean(f) * 1024):.4f}   (bytes = FETCH_SIZE KiB * 1024 * factor)",
             f"write_factor: {nbytes / (statistics.mean(wr) * 1024):.4f}   (bytes = WRITE_SIZE KiB * 1024 * factor)"]
        path = os.path.join(ROOT, "profiles", "copy_1GiB_counter_calibration.txt")
    elif kind == "trace":
        import workloads
        kt = _csv_rows(d + "/**/*kernel_trace.csv")
        dec = [r for r in kt if kfilter in r["Kernel_Name"]]
        # the second kernel of a call: the merge (decode), the rescaling pass (prefill)
        second = "prefill_safe_kernel" if pre else "merge_kernel"
        mer = [r for r in kt if second in r["Kernel_Name"]]
        dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        dec.sort(key=lambda r: int(r["Start_Timestamp"]))
        mer.sort(key=lambda r: int(r["Start_Timestamp"]))
        dd = [dur(r) for r in dec]
        # the run's dispatches in order: warmup calls, the timed back-to-back
        # calls (what ms_per_step measures) and, for the decode, the calls
        # with events around each (a diagnostic loop whose recorded events
        # hold each kernel back and make it slower)
        nw_, ns_ = (1, 5) if pre else (2, 10)

        def block(xs, lo, hi):
            xs = xs[lo:hi]
            return (f"{len(xs)}  mean_us: {statistics.mean(xs):.2f}  median_us: "
                    f"{statistics.median(xs):.2f}  min_us: {min(xs):.2f}  max_us: {max(xs):.2f}"
                    if xs else "0")
        nbytes = (prefill_flops(workloads.make_prefill_config(w)) if pre
                  else kv_bytes(workloads.make_config(w)))
        r0 = dec[0]
        tag = os.path.basename(d.rstrip("/"))
        L = [f"# {fam} kernel, {w} workload: rocprofv3 kernel trace statistics",
             "command: " + PROFILE_CMD.format(t=180, what="--kernel-trace --stats", tag=tag, bargs=bargs),
             f"source_sha256: {sha}",
             f"kernel: {r0['Kernel_Name']}",
             f"grid: {r0.get('Grid_Size_X', r0.get('Grid_Size'))} work-items, workgroup "
             f"{r0.get('Workgroup_Size_X', r0.get('Workgroup_Size'))}, LDS {r0.get('LDS_Block_Size')} B, "
             f"VGPR {r0.get('VGPR_Count')}, AGPR {r0.get('Accum_VGPR_Count')}, SGPR {r0.get('SGPR_Count')}",
             f"dispatches: {len(dd)}  median_us: {statistics.median(dd):.2f}  mean_us: "
             f"{statistics.mean(dd):.2f}  min_us: {min(dd):.2f}  max_us: {max(dd):.2f}"]
        timed = dd[nw_:nw_ + ns_] or dd
        L += [f"timed_dispatches (calls {nw_ + 1}..{nw_ + ns_}, back to back): "
              + block(dd, nw_, nw_ + ns_)]
        if not pre:
            L += [f"event_bracketed_dispatches (calls {nw_ + ns_ + 1}..): "
                  + block(dd, nw_ + ns_, len(dd))]
        tot = statistics.mean(dd)
        tot_t = statistics.mean(timed)
        if mer:
            md = [dur(r) for r in mer]
            mt = md[nw_:nw_ + ns_] or md
            L += [f"{second}: {mer[0]['Kernel_Name'][:100]}",
                  f"{second.split('_kernel')[0]}_dispatches: {len(md)}  median_us: "
                  f"{statistics.median(md):.2f}  mean_us: {statistics.mean(md):.2f}",
                  f"{second.split('_kernel')[0]}_timed_dispatches: " + block(md, nw_, nw_ + ns_),
                  f"{fam}_plus_{second.split('_kernel')[0]}_mean_us: {tot + statistics.mean(md):.2f}",
                  f"timed_{fam}_plus_{second.split('_kernel')[0]}_mean_us: "
                  f"{tot_t + statistics.mean(mt):.2f}"]
            tot += statistics.mean(md)
            tot_t += statistics.mean(mt)
        if pre:
            L += [f"algorithmic_flops_per_launch: {nbytes}",
                  f"TFLOPs_at_mean: {nbytes / tot / 1e6:.1f}  ({nbytes / tot / 1e6 / 25:.1f}% of "
                  "2.5 PFLOP/s dense bf16/fp16 MFMA)",
                  f"TFLOPs_at_timed_mean: {nbytes / tot_t / 1e6:.1f}  "
                  f"({nbytes / tot_t / 1e6 / 25:.1f}% of 2.5 PFLOP/s)"]
        else:
            L += [f"algorithmic_kv_bytes_per_launch: {nbytes}",
                  f"effective_GBps_at_mean: {nbytes / tot / 1e3:.1f}  ({nbytes / tot / 1e3 / 80:.1f}% "
                  "of 8 TB/s)",
                  f"effective_GBps_at_timed_mean: {nbytes / tot_t / 1e3:.1f}  "
                  f"({nbytes / tot_t / 1e3 / 80:.1f}% of 8 TB/s)"]
        L += [
              "", "# kernel_stats.csv (all kernels of the run)",
              "name | calls | average_ns | min_ns | max_ns | percentage"]
        for r in _csv_rows(d + "/**/*kernel_stats.csv"):
            L.append(f"{r['Name'][:110]} | {r['Calls']} | {r['AverageNs']} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {r['Percentage']}")
        path = os.path.join(ROOT, "profiles", f"{fam}_{w}_kernel_trace.txt")
    elif kind in ("fetch", "write"):
        import workloads
        cal = {}
        for line in open(os.path.join(ROOT, "profiles", "copy_1GiB_counter_calibration.txt")):
            if line.startswith("fetch_factor:"):
                cal["fetch"] = float(line.split()[1])
            if line.startswith("write_factor:"):
                cal["write"] = float(line.split()[1])
        counter = kind.upper() + "_SIZE"
        v = _per_dispatch(_csv_rows(d + "/**/*counter_collection.csv"), counter, kfilter)
        part = os.path.join(ROOT, "profiles", f".{fam}_{w}_{kind}.part")
        tag = os.path.basename(d.rstrip("/"))
        with open(part, "w") as fh:
            fh.write(json.dumps({"kib": statistics.mean(v), "min": min(v), "max": max(v), "n": len(v),
                                 "factor": cal[kind], "sha": sha,
                                 "cmd": PROFILE_CMD.format(t=90, what=f"--pmc {counter}", tag=tag,
                                                           bargs=bargs)}))
        other = os.path.join(ROOT, "profiles",
                             f".{fam}_{w}_{'write' if kind == 'fetch' else 'fetch'}.part")
        if not os.path.exists(other):
            print(f"stored {kind}; summarise the other counter to write the traffic file")
            return
        fp = json.load(open(part if kind == "fetch" else other))
        wp = json.load(open(other if kind == "fetch" else part))
        os.remove(part)
        os.remove(other)
        if pre:   # q, k, v read once and out written once
            pin = workloads.make_prefill_config(w)
            nbytes = sum(pin[t].numel() * pin[t].element_size() for t in ("q", "k", "v", "q"))
        else:
            nbytes = kv_bytes(workloads.make_config(w))
        fb, wb = int(fp["kib"] * 1024 * fp["factor"]), int(wp["kib"] * 1024 * wp["factor"])
        L = [f"# {fam} kernel, {w} workload: HBM traffic per launch from rocprofv3 counters",
             "# (one counter per run; scaled by the 1 GiB copy calibration in copy_1GiB_counter_calibration.txt)",
             f"command_fetch: {fp['cmd']}", f"command_write: {wp['cmd']}",
             f"source_sha256: {sha}", f"dispatches: {fp['n']}",
             f"fetch_kib_per_dispatch: {fp['kib']:.2f} (min {fp['min']:.2f}, max {fp['max']:.2f})",
             f"write_kib_per_dispatch: {wp['kib']:.2f} (min {wp['min']:.2f}, max {wp['max']:.2f})",
             f"fetch_factor: {fp['factor']:.4f}", f"write_factor: {wp['factor']:.4f}",
             f"fetch_bytes_per_launch: {fb}", f"write_bytes_per_launch: {wb}",
             f"traffic_bytes_per_launch: {fb + wb}",
             (f"algorithmic_bytes_per_launch (q, k, v read once, out written once): {nbytes}" if pre
              else f"algorithmic_kv_bytes_per_launch: {nbytes}"),
             f"{'traffic' if pre else 'fetch'}_over_algorithmic: {(fb + wb if pre else fb) / nbytes:.4f}"]
        path = os.path.join(ROOT, "profiles", f"{fam}_{w}_hbm_traffic.txt")
    elif kind == "derived":
        rows = _csv_rows(d + "/**/*counter_collection.csv")
        vals = {n: statistics.mean(_per_dispatch(rows, n, kfilter)) for n in DERIVED}
        tag = os.path.basename(d.rstrip("/"))
        L = [f"# {fam} kernel, {w} workload: rocprofv3's derived metrics per dispatch (its own "
             "expressions, evaluated by rocprofv3; mean over the run's dispatches)",
             "command: " + PROFILE_CMD.format(t=90, what="--pmc " + " ".join(DERIVED), tag=tag,
                                              bargs=bargs),
             f"source_sha256: {sha}"]
        L += [f"{n}: {vals[n]:.3f}" for n in DERIVED]
        L += ["# MfmaUtil % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE max over XCDs * SIMDs)",
              "# VALUBusy % = SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE (max over XCDs)",
              "# OccupancyPercent = 400 SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CUs / 32 (waves of 32 slots)",
              "# LDSBankConflict % = SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / CUs"]
        path = os.path.join(ROOT, "profiles", f"{fam}_{w}_derived_counters.txt")
    elif kind in SQ_SETS:
        rows = _csv_rows(d + "/**/*counter_collection.csv")
        names = SQ_SETS[kind]
        vals = {n: statistics.mean(_per_dispatch(rows, n, kfilter)) for n in names}
        cus, simds, xcds = 256, 1024, 8
        # rocprofv3's csv gives GRBM_GUI_ACTIVE summed over the 8 XCDs (8x the
        # dispatch's cycles); its own derived metrics take the maximum over
        # XCDs, which the sum / 8 stands for here
        gui = vals["GRBM_GUI_ACTIVE"] / xcds
        tag = os.path.basename(d.rstrip("/"))
        L = [f"# {fam} kernel, {w} workload: SQ counters per dispatch (mean over the run's dispatches, "
             "summed over SEs and XCDs)",
             "command: " + PROFILE_CMD.format(t=90, what="--pmc " + " ".join(names), tag=tag, bargs=bargs),
             f"source_sha256: {sha}"]
        L += [f"{n}: {vals[n]:.0f}" for n in names]
        L.append("# derived (rocprofv3's own definitions; 256 CUs, 1024 SIMDs, GRBM_GUI_ACTIVE / 8 "
                 "per XCD; cycle counters named *_CYCLES / SQ_WAIT_* / SQ_ACTIVE_* as the csv gives "
                 "them):")
        if kind == "sq_a":
            L += [f"MfmaUtil_pct: {100 * vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * simds):.2f}   "
                  "(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs))",
                  f"VALUBusy_pct: {100 * vals['SQ_ACTIVE_INST_VALU'] / cus / gui:.2f}   "
                  "(100 * SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE)",
                  f"Occupancy_pct: {400 * vals['SQ_WAVE_CYCLES'] / gui / cus / 32:.2f}   "
                  "(400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CUs / 32)",
                  f"waves_per_CU: {vals['SQ_WAVES'] / cus:.2f}",
                  f"wait_inst_any_frac_of_wave_cycles: {vals['SQ_WAIT_INST_ANY'] / max(vals['SQ_WAVE_CYCLES'], 1):.3f}",
                  f"valu_insts_per_wave: {vals['SQ_INSTS_VALU'] / max(vals['SQ_WAVES'], 1):.0f}",
                  f"mfma_insts_per_wave: {vals['SQ_INSTS_MFMA'] / max(vals['SQ_WAVES'], 1):.0f}"]
        elif kind == "sq_c":
            wc = max(vals["SQ_WAVE_CYCLES"], 1)
            L += [f"wait_any_frac_of_wave_cycles: {vals['SQ_WAIT_ANY'] / wc:.3f}",
                  f"wait_inst_any_frac_of_wave_cycles: {vals['SQ_WAIT_INST_ANY'] / wc:.3f}",
                  f"wait_inst_lds_frac_of_wave_cycles: {vals['SQ_WAIT_INST_LDS'] / wc:.3f}",
                  f"active_lds_frac_of_wave_cycles: {vals['SQ_ACTIVE_INST_LDS'] / wc:.3f}",
                  f"active_misc_frac_of_wave_cycles: {vals['SQ_ACTIVE_INST_MISC'] / wc:.3f}",
                  f"active_scalar_frac_of_wave_cycles: {vals['SQ_ACTIVE_INST_SCA'] / wc:.3f}",
                  f"LDS_busy_pct: {100 * vals['SQ_LDS_IDX_ACTIVE'] / gui / cus:.2f}   "
                  "(SQ_LDS_IDX_ACTIVE / GRBM_GUI_ACTIVE / CUs)"]
        else:
            L += [f"LDSBankConflict_pct: {100 * vals['SQ_LDS_BANK_CONFLICT'] / gui / cus:.3f}   "
                  "(100 * SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / CUs)",
                  f"lds_insts: {vals['SQ_INSTS_LDS']:.0f}   vmem_rd_insts: {vals['SQ_INSTS_VMEM_RD']:.0f}",
                  f"mfma_mops_bf16_f16 (x512 = flops): {vals['SQ_INSTS_VALU_MFMA_MOPS_BF16'] + vals['SQ_INSTS_VALU_MFMA_MOPS_F16']:.0f}"]
        path = os.path.join(ROOT, "profiles", f"{fam}_{w}_{kind}_counters.txt")
    else:
        raise SystemExit(f"unknown summary kind {kind}")
    with open(path, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print("\n".join(L[:12]))
    print("wrote", path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--cold-iters", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU-baseline leg (0 disables it)")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--op", choices=("decode", "merge_states", "stream_read", "paged_gather",
                                     "prefill"),
                    default="decode",
                    help="merge_states: time the cascade merge on 16 states of the "
                         "llama3_8b batch's rows instead of the decode; stream_read / "
                         "paged_gather: memory-system references for the workload's bytes; "
                         "prefill: context attention on --config prefill_* (TFLOP/s)")
    ap.add_argument("--lds", action="store_true",
                    help="paged_gather: stage the blocks through LDS instead of registers")
    ap.add_argument("--pf", type=int, default=3,
                    help="paged_gather: 16-key blocks in flight per wave (2, 3, 4, 6, 8)")
    ap.add_argument("--waves-per-simd", type=int, default=1, choices=(1, 2),
                    help="stream_read / paged_gather: 1 (the decode's grid) or 2 waves per SIMD")
    ap.add_argument("--summarize", default=None,
                    help="write a profiles/ summary from rocprofv3 csv output: trace, fetch, "
                         "write, sq_a, sq_b, sq_c, derived or calibration (with --prof-dir; "
                         "--op prefill for the prefill kernel)")
    ap.add_argument("--prof-dir", default=None, help="the rocprofv3 -d directory to summarise")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this decode kernel is measured on a single "
              "MI355X; multi-GPU sharding is a design note, not a built path.", file=sys.stderr)
        sys.exit(2)

    if args.summarize:
        summarize(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.op in ("stream_read", "paged_gather"):
        bench_ceiling(args)
        return
    if args.op == "merge_states":
        bench_merge_states(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return

    import numpy as np
    import torch
    import workloads
    import paged_kv_decode_12_amd as pk

    w = workloads.CONFIGS[args.config]
    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    inp = workloads.make_config(args.config)
    nbytes = kv_bytes(inp)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=dev) if w.return_lse else None
    plan = pk.plan(d["q"], d["k_cache"], d["block_tables"], w.q_len_per_req, w.window_left)
    pk.reserve_workspace(pk.workspace_bytes(d["q"], d["k_cache"], d["block_tables"],
                                            w.q_len_per_req, w.window_left))

    # the call's arguments are marshalled once (as a serving loop would), so
    # the host enqueues each step in a few microseconds and the timed region
    # measures the GPU, not the Python binding
    step = pk.bind_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                          d["seq_lens_kv"], scale=w.scale, q_len_per_req=w.q_len_per_req,
                          window_left=w.window_left, sinks=d["sinks"], out=out, lse=lse)

    print(f"[bench] warmup {args.warmup}, plan {plan}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` back-to-back calls between two HIP events on
    # the launch stream (torch's current stream, which the binding passes to
    # the library).  An event recorded between two calls holds the second
    # kernel back by several microseconds, so none is recorded inside the
    # region: the average launch duration is the region's time / steps, as a
    # decode loop issuing calls back to back sees it.
    stream = torch.cuda.current_stream(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    launch_ms = ms_per_step
    print(f"[bench] timed {args.steps} steps: {total_ms:.3f} ms (wall {wall * 1e3:.1f} ms)",
          file=sys.stderr, flush=True)

    # diagnostic, outside the timed region: events around each of a few calls
    per_call_us = []
    for _ in range(min(args.steps, 50)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        per_call_us.append((a, b))
    torch.cuda.synchronize()
    per_call_us = [a.elapsed_time(b) * 1e3 for a, b in per_call_us]

    # cold calls: evict the MALL/L2 by reading 1 GiB between calls, outside the
    # events (a read leaves the caches clean; a write flush would leave dirty
    # lines whose write-back then overlaps the timed call)
    cold_us = []
    if args.cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_iters):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold_us.append(a.elapsed_time(b) * 1e3)
        del flush

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.config, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "page_size": w.page_size, "q_len_per_req": w.q_len_per_req,
                   "seq_lens_kv": [w.kv_lo, w.kv_hi], "window_left": w.window_left,
                   "sinks": w.sinks, "return_lse": w.return_lse, "seed": w.seed,
                   "kv_bytes_per_call": nbytes},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "plan": plan,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(args.config),
                     "kernel": "one pkvd_decode call (the decode kernel, plus the merge "
                               "kernel when the plan uses it)",
                     "launch_us": round(launch_ms * 1e3, 3),
                     "events_around_each_call_us": round(float(np.mean(per_call_us)), 3)
                     if per_call_us else None},
    }
    if cold_us:
        cold_med = float(np.median(cold_us))
        result["cold"] = {"us_median": round(cold_med, 3),
                          "us_p10": round(float(np.percentile(cold_us, 10)), 3),
                          "us_p90": round(float(np.percentile(cold_us, 90)), 3),
                          "GBs_median": round(nbytes / (cold_med * 1e-6) / 1e9, 2)}

    # CPU baseline and a spot check of this very output against the oracle
    if args.cpu_seconds > 0 or not args.no_check:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        ref = None
        runs, t_cpu = 0, 0.0
        while True:
            t = time.perf_counter()
            ref = oracle.decode(inp, nthreads=threads)
            t_cpu += time.perf_counter() - t
            runs += 1
            if args.cpu_seconds <= 0 or t_cpu >= args.cpu_seconds:
                break
        if args.cpu_seconds > 0:
            per = t_cpu / runs
            result["cpu_baseline"] = {
                "value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": f"the whole {args.config} batch (all {inp['q'].shape[0] * w.Hq} "
                          f"row-heads), {runs} run(s), {per:.3f} s each, fp64 C + OpenMP",
                "cpu": cpu_model()}
        if not args.no_check:
            got = out.float().cpu().numpy().reshape(-1, w.D)
            err = float(np.abs(got - ref[0]).max())
            chk = {"max_abs_err_out": err}
            if lse is not None:
                chk["max_abs_err_lse"] = float(np.abs(lse.cpu().numpy().reshape(-1) - ref[1]).max())
            result["check"] = chk

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
