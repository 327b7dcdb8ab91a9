"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, validates arguments before any HIP call and plans launches
from shapes alone.  No call here reaches a kernel: every descriptor set is
either invalid or only passed to the planning entry points."""
import ctypes
import os
import re

import pytest
import torch

import paged_kv_decode_12_amd as pk
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkvd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkvd_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "pkvd_decode" in names and len(names) >= 7
    lib = ctypes.CDLL(pk.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert pk.version().count(".") == 2
    for code in range(5):
        assert pk._lib.pkvd_status_string(code)


class FakeDev:
    """Descriptors over fake, 256-byte aligned addresses.  Only used where the
    library must reject the call before touching memory."""

    def __init__(self, inp):
        self.inp = inp

    def desc(self, t, addr):
        d = pk._desc(t)
        d.data = addr
        return d

    def call(self, **over):
        inp = dict(self.inp)
        inp.update(over)
        base = 1 << 32
        ds = {}
        for i, name in enumerate(["q", "k_cache", "v_cache", "block_tables", "seq_lens_kv",
                                  "sinks", "out", "lse"]):
            t = inp.get(name)
            ds[name] = None if t is None else self.desc(t, base + (i << 24))
        r = lambda x: None if x is None else ctypes.byref(x)
        return pk._lib.pkvd_decode(r(ds["q"]), r(ds["k_cache"]), r(ds["v_cache"]),
                                   r(ds["block_tables"]), r(ds["seq_lens_kv"]),
                                   float(inp.get("scale", 0.1)), int(inp.get("q_len_per_req", 1)),
                                   int(inp.get("window_left", -1)), r(ds["sinks"]), r(ds["out"]),
                                   r(ds["lse"]), None)


def base_inputs(**kw):
    inp = workloads.make_case(B=2, Hq=4, Hkv=2, D=64, page_size=16, seq_lens=(5, 40), **kw)
    R, Hq, D = inp["q"].shape
    inp["q"] = inp["q"].contiguous()
    inp["out"] = torch.empty(R, Hq, D, dtype=inp["q"].dtype)
    inp["lse"] = torch.empty(R, Hq, dtype=torch.float32)
    return inp


BAD = [
    ("q_rank", lambda i: dict(q=i["q"][0])),
    ("q_dtype", lambda i: dict(q=i["q"].float())),
    ("kv_dtype_mismatch", lambda i: dict(k_cache=i["k_cache"].half())),
    ("kv_shape_mismatch", lambda i: dict(v_cache=i["v_cache"][:, :1].contiguous())),
    ("q_rows_not_B_times_Lq", lambda i: dict(q_len_per_req=2)),
    ("heads_not_multiple", lambda i: dict(q=torch.zeros(2, 3, 64, dtype=torch.bfloat16),
                                           out=torch.zeros(2, 3, 64, dtype=torch.bfloat16),
                                           lse=None)),
    ("window_below_minus_one", lambda i: dict(window_left=-2)),
    ("q_len_zero", lambda i: dict(q_len_per_req=0)),
    ("bt_dtype", lambda i: dict(block_tables=i["block_tables"].long())),
    ("bt_row_not_contiguous", lambda i: dict(block_tables=i["block_tables"].t())),
    ("seq_lens_dtype", lambda i: dict(seq_lens_kv=i["seq_lens_kv"].long())),
    ("seq_lens_len", lambda i: dict(seq_lens_kv=i["seq_lens_kv"][:1])),
    ("sinks_dtype", lambda i: dict(sinks=torch.zeros(4, dtype=torch.float16))),
    ("sinks_len", lambda i: dict(sinks=torch.zeros(3))),
    ("out_dtype", lambda i: dict(out=i["out"].float())),
    ("out_strided", lambda i: dict(out=torch.zeros(2, 64, 4, dtype=torch.bfloat16).transpose(1, 2))),
    ("lse_dtype", lambda i: dict(lse=i["lse"].double())),
    ("lse_shape", lambda i: dict(lse=i["lse"][:, :2].contiguous())),
    ("q_head_dim_strided", lambda i: dict(q=torch.zeros(2, 64, 4, dtype=torch.bfloat16).transpose(1, 2))),
    ("q_unaligned_rows", lambda i: dict(q=torch.zeros(2, 4, 68, dtype=torch.bfloat16)[:, :, :64])),
    ("kv_tile_not_contiguous", lambda i: dict(k_cache=i["k_cache"].transpose(2, 3).contiguous().transpose(2, 3))),
    ("scale_nan", lambda i: dict(scale=float("nan"))),
    ("missing_out", lambda i: dict(out=None)),
]


@pytest.mark.parametrize("name,mut", BAD, ids=[b[0] for b in BAD])
def test_invalid_arguments(name, mut):
    inp = base_inputs()
    st = FakeDev(inp).call(**mut(inp))
    assert st == 1, (name, st, pk._lib.pkvd_last_error())
    assert pk._lib.pkvd_last_error()


@pytest.mark.parametrize("D,ps", [(96, 16), (256, 16), (64, 512)])
def test_unsupported_shapes(D, ps):
    inp = workloads.make_case(B=1, Hq=2, Hkv=1, D=D, page_size=ps, seq_lens=(3,))
    inp["q"] = inp["q"].contiguous()
    inp["out"] = torch.empty_like(inp["q"])
    inp["lse"] = None
    assert FakeDev(inp).call() == 2


def test_plans_of_the_workloads():
    """Shape-only plans: the path follows rows = (Hq/Hkv) * q_len_per_req; the
    persistent grid and its workspace do not depend on the lengths."""
    for name, w in workloads.CONFIGS.items():
        q = torch.empty(w.B * w.q_len_per_req, w.Hq, w.D, dtype=torch.bfloat16)
        k = torch.empty(1, w.Hkv, w.page_size, w.D, dtype=torch.bfloat16)
        bt = torch.empty(w.B, w.C, dtype=torch.int32)
        p = pk.plan(q, k, bt, w.q_len_per_req, w.window_left)
        rows = (w.Hq // w.Hkv) * w.q_len_per_req
        assert p["rows_per_tile"] * p["row_tiles"] >= rows
        # MFMA (16-row tiles) for more than 4 rows; VALU tiles of 4 otherwise
        if rows > 4:
            assert (p["path"], p["rows_per_tile"]) == ("mfma", 16)
        else:
            assert p["path"] == "valu" and p["rows_per_tile"] == (4 if rows <= 4 else 8)
        assert p["row_tiles"] == -(-rows // p["rows_per_tile"])
        # one workgroup per CU holds 4 to 16 waves (4 SIMDs x waves per SIMD)
        assert p["workgroups"] * 16 >= p["waves"] >= 1
        ws = pk.workspace_bytes(q, k, bt, w.q_len_per_req, w.window_left)
        assert ws >= 2 * p["waves"] * p["rows_per_tile"] * (w.D + 1) * 4


def test_sinks_beyond_lds_staging_unsupported():
    """The decode kernel stages the sink logits in LDS (at most 4096 heads)."""
    Hq = 4104
    inp = base_inputs()
    q = torch.zeros(2, Hq, 64, dtype=torch.bfloat16)
    st = FakeDev(inp).call(q=q, out=torch.zeros_like(q), lse=None, sinks=torch.zeros(Hq))
    assert st == 2, pk._lib.pkvd_last_error()
    assert b"sinks" in pk._lib.pkvd_last_error()


MERGE_BAD = [
    ("v_rank", dict(v=(2, 3, 4))),
    ("v_dtype", dict(v_dtype=torch.float64)),
    ("s_shape", dict(s=(2, 3, 5))),
    ("s_dtype", dict(s_dtype=torch.float16)),
    ("out_shape", dict(v_out=(3, 4, 8))),
    ("out_dtype", dict(out_dtype=torch.float32)),
    ("s_out_shape", dict(s_out=(3, 5))),
    ("sinks_len", dict(sinks=(5,))),
    ("zero_states", dict(v=(0, 3, 4, 16), s=(0, 3, 4))),
]


@pytest.mark.parametrize("name,kw", MERGE_BAD, ids=[b[0] for b in MERGE_BAD])
def test_merge_states_invalid_arguments(name, kw):
    """pkvd_merge_states rejects bad descriptors before any HIP call."""
    def t(shape, dtype):
        return torch.zeros(shape, dtype=dtype)
    v = t(kw.get("v", (2, 3, 4, 16)), kw.get("v_dtype", torch.bfloat16))
    s = t(kw.get("s", (2, 3, 4)), kw.get("s_dtype", torch.float32))
    vo = t(kw.get("v_out", (3, 4, 16)), kw.get("out_dtype", torch.bfloat16))
    so = t(kw.get("s_out", (3, 4)), torch.float32)
    sk = t(kw["sinks"], torch.float32) if "sinks" in kw else None
    descs = [pk._desc(x) for x in (v, s, sk, vo, so)]
    for i, d in enumerate(descs):
        if d is not None:
            d.data = 0x100000 * (i + 1)   # never dereferenced
    r = lambda x: None if x is None else ctypes.byref(x)
    st = pk._lib.pkvd_merge_states(*[r(d) for d in descs], None)
    assert st == 1, (name, st, pk._lib.pkvd_last_error())
    assert pk._lib.pkvd_last_error()
