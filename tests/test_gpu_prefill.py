"""GPU parity of context attention (pkvd_prefill) against the fp64 oracle:
fixed and packed rows, causal / dense / windowed / variable-window masks,
head_dim 128 and 256, GQA, bf16 / fp16 inputs, bf16 / fp16 / fp32 outputs and
the output scale (flashinfer.attention.prims_ts.batch_prefill, summary and
Parameters).

Tolerances as for the decode: max |out - ref| <= 2e-2 and <= 1e-2 relative
to the largest reference output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

OUT_ATOL = 2e-2
REL = 1e-2
ODT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def log(*a):
    print(*a, flush=True)


def run(inp, out_dtype=None):
    import paged_kv_decode_12_amd as pk
    dev = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = pk.batch_prefill(dev["q"], dev["k"], dev["v"], qo_indptr=dev.get("qo_indptr"),
                           kv_indptr=dev.get("kv_indptr"), mask_type=dev["mask_type"],
                           window_left=dev["window_left"],
                           variable_window_token_starts=dev.get("window_starts"),
                           variable_window_token_ends=dev.get("window_ends"),
                           sm_scale=dev["sm_scale"], output_scale=dev["output_scale"],
                           out_dtype=out_dtype, max_seq_len_q=dev.get("max_seq_len_q"))
    torch.cuda.synchronize()
    assert out.shape == inp["q"].shape
    return out.float().cpu().numpy().reshape(-1, out.shape[-1])


def compare(name, got, ref):
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    msg = f"{name}: max|err|={err.max():.3e} max|ref|={scale:.3e} rel={err.max() / scale:.3e}"
    log(msg)
    assert err.max() <= OUT_ATOL, msg
    assert err.max() / scale <= REL, msg


CASES = []
for D in (128, 256):
    for mask, wl in (("causal", -1), ("dense", -1), ("causal", 37), ("dense", 5)):
        CASES.append(dict(D=D, B=2, Sq=150, Sk=150, Hq=4, Hkv=2, mask_type=mask, window_left=wl))
    CASES.append(dict(D=D, B=2, Sq=70, Sk=333, Hq=4, Hkv=1, mask_type="causal", window_left=-1))
    CASES.append(dict(D=D, B=1, Sq=200, Sk=90, Hq=2, Hkv=2, mask_type="causal", window_left=-1))
    CASES.append(dict(D=D, B=3, Hq=6, Hkv=3, q_lens=(1, 0, 130), kv_lens=(40, 7, 260),
                      mask_type="causal", window_left=-1))
    CASES.append(dict(D=D, B=3, Hq=4, Hkv=4, q_lens=(65, 17, 3), kv_lens=(65, 0, 300),
                      mask_type="dense", window_left=20))
CASES.append(dict(D=128, B=1, Sq=1, Sk=1, Hq=1, Hkv=1, mask_type="causal", window_left=-1))
CASES.append(dict(D=128, B=2, Sq=64, Sk=64, Hq=8, Hkv=2, mask_type="causal", window_left=0,
                  dtype="fp16", value_std=0.5))
CASES.append(dict(D=256, B=2, Sq=33, Sk=129, Hq=2, Hkv=1, mask_type="dense", window_left=-1,
                  dtype="fp16", pad_heads=2))


def _id(c):
    return ",".join(f"{k}={v}" for k, v in c.items())


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_prefill_cases(case):
    inp = workloads.make_prefill_case(seed=31, output_scale=0.8, **case)
    ref = oracle.prefill(inp)
    for odt in (None, "fp32"):
        log(f"[prefill] {_id(case)} out={odt}")
        got = run(inp, None if odt is None else ODT[odt])
        compare(f"{_id(case)}/{odt}", got, ref)


@pytest.mark.parametrize("D", [128, 256])
def test_prefill_variable_window(D):
    """Per-query inclusive [start, end] bounds (fixed shapes), random bounds and
    bounds equal to the causal window."""
    g = torch.Generator().manual_seed(D)
    B, Sq, Sk = 2, 100, 180
    starts = torch.randint(0, Sk, (B, Sq), generator=g)
    ends = torch.minimum(starts + torch.randint(0, 90, (B, Sq), generator=g),
                         torch.tensor(Sk - 1))
    inp = workloads.make_prefill_case(B=B, Sq=Sq, Sk=Sk, Hq=4, Hkv=2, D=D,
                                      mask_type="variable_window",
                                      window=(starts.tolist(), ends.tolist()), seed=41)
    compare(f"varwin/D{D}", run(inp), oracle.prefill(inp))


@pytest.mark.parametrize("name", list(workloads.PREFILL_CONFIGS))
def test_prefill_configs_sampled(name):
    """The measured prefill workloads at full size: sampled (row, head) pairs
    (first and last rows of requests included) against the oracle."""
    inp = workloads.make_prefill_config(name)
    rows, Hq = inp["q"].shape[0] * (inp["q"].shape[1] if inp["q"].dim() == 4 else 1), \
        inp["q"].shape[-2]
    g = torch.Generator().manual_seed(7)
    sel = set(torch.randint(0, rows * Hq, (400,), generator=g).tolist())
    sel |= {0, Hq - 1, rows * Hq - 1, (rows - 1) * Hq}
    sel = sorted(sel)
    ref = oracle.prefill(inp, sel=sel)
    log(f"[prefill_cfg] {name} rows={rows}")
    got = run(inp)
    compare(name, got[sel], ref)


@pytest.mark.parametrize("out_dtype", [None, "fp32"])
@pytest.mark.parametrize("dtype,sm_scale", [("bf16", 30.0), ("fp16", 3.0)])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_large_logits(D, dtype, sm_scale, out_dtype):
    """Scores spread over hundreds of base-2 units: earlier keys exceed the
    score of a row's last visible key by far more than the fast pass allows
    (2^128 for bf16 probabilities, 2^24 for fp16), so every workgroup's fast
    pass overflows and the rescaling kernel recomputes it."""
    inp = workloads.make_prefill_case(B=2, Sq=140, Sk=300, Hq=4, Hkv=2, D=D, dtype=dtype,
                                      mask_type="causal", seed=77)
    inp["sm_scale"] = sm_scale
    compare(f"large_logits/D{D}/{dtype}/{out_dtype}", run(inp, ODT.get(out_dtype)),
            oracle.prefill(inp))


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (256, 16, 4)])
def test_prefill_large_logits_many_items(D, Hq, Hkv):
    """Every fast pass overflows and there are more workgroup items (512)
    than CUs: each workgroup of the rescaling kernel recomputes several.
    Sampled rows against the oracle."""
    inp = workloads.make_prefill_case(B=4, Sq=1024, Sk=1024, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                                      mask_type="causal", seed=79)
    inp["sm_scale"] = 30.0
    rows = 4 * 1024
    g = torch.Generator().manual_seed(9)
    sel = sorted(set(torch.randint(0, rows * Hq, (300,), generator=g).tolist())
                 | {0, rows * Hq - 1})
    got = run(inp)
    compare(f"large_logits_many/D{D}", got[sel], oracle.prefill(inp, sel=sel))


# bit patterns of signalling NaNs in each output format (what an output
# buffer may hold from an earlier call or from the allocator)
SNAN = {"bf16": (torch.int16, 0x7F85), "fp16": (torch.int16, 0x7D05),
        "fp32": (torch.int32, 0x7FA5A5A5)}


@pytest.mark.parametrize("out_name", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_some_overflow_snan_out(D, out_name):
    """One kv head of one request has keys scaled far up (its workgroups'
    fast passes overflow, the others' do not), written into an output
    buffer that starts out full of signalling NaNs: every row must hold the
    oracle's value afterwards."""
    import paged_kv_decode_12_amd as pk
    inp = workloads.make_prefill_case(B=3, Hq=8, Hkv=2, D=D, dtype="fp16", q_lens=(90, 1, 200),
                                      kv_lens=(90, 50, 260), mask_type="causal", seed=78)
    k = inp["k"].clone()
    r0, r1 = int(inp["kv_indptr"][2]), int(inp["kv_indptr"][3])
    k[r0:r1, 1] *= 12.0   # request 2, kv head 1
    inp["k"] = k
    dt, bits = SNAN[out_name]
    out = torch.full(inp["q"].shape, bits, dtype=dt, device="cuda").view(ODT[out_name])
    dev = {n: (v.cuda() if torch.is_tensor(v) else v) for n, v in inp.items()}
    pk.batch_prefill(dev["q"], dev["k"], dev["v"], qo_indptr=dev["qo_indptr"],
                     kv_indptr=dev["kv_indptr"], mask_type="causal", sm_scale=dev["sm_scale"],
                     out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(-1, D)
    compare(f"some_overflow/D{D}/{out_name}", got, oracle.prefill(inp))
