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
  cold          per-call time with the 256 MB Infinity Cache and L2 flushed
                before every call (outside the events).

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


def kernel_source_hash() -> str:
    """SHA-256 over the library's sources and build flags (what the counters measured)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pkvd_build", os.path.join(ROOT, "paged_kv_decode_12_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = hashlib.sha256()
    for path in b.SOURCES + b.HEADERS:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    h.update(" ".join(b.FLAGS[:-2]).encode())      # flags minus the machine-specific -I paths
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
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
    ap.add_argument("--op", choices=("decode", "merge_states"), default="decode",
                    help="merge_states: time the cascade merge on 16 states of the "
                         "llama3_8b batch's rows instead of the decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this decode kernel is measured on a single "
              "MI355X; multi-GPU sharding is a design note, not a built path.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.op == "merge_states":
        bench_merge_states(args)
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

    # cold calls: flush the MALL/L2 with a 1 GiB write between calls, outside the events
    cold_us = []
    if args.cold_iters > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(args.cold_iters):
            flush.fill_(1.0)
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
                "cpu": platform.processor() or platform.machine()}
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
