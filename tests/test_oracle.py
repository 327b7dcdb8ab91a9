"""Pins for the fp64 CPU oracle (runs without a GPU).

Each test checks the oracle against something other than itself: the
documentation's statements, closed forms, textbook identities, library routines
(torch.softmax / torch.logsumexp in fp64 on densely gathered K/V) and
brute force on tiny inputs.  The passages are those of
flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters, Note) and
flashinfer.attention.prims_ts.batch_prefill (summary: causal is bottom-right
aligned, a window keeps at most window_left + 1 keys per causal row) and
flashinfer.attention.prims_ts.batch_decode_with_paged_kv_cache (summary:
packed query rows through qo_indptr; Parameters: mask_type, bmm2_scale).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LOG2E = 1.0 / math.log(2.0)


# ----------------------------------------------------------------------------
# independent dense brute force built from torch library routines
# ----------------------------------------------------------------------------
def dense_reference(inp, with_sinks=True):
    """Gather each request's K/V densely with torch indexing, then fp64
    torch.softmax over an explicit boolean mask (plus an appended sink logit
    column whose value row is zero) and torch.logsumexp * log2(e).  Packed
    rows (``qo_indptr``), dense rows (``mask_type``) and the output factor
    (``out_scale``) are honoured when the inputs carry them."""
    q = inp["q"].double()
    if q.dim() == 4:
        q = q.reshape(-1, q.shape[2], q.shape[3])
    k = inp["k_cache"].double()
    v = inp["v_cache"].double()
    bt = inp["block_tables"].long()
    n_all = inp["seq_lens_kv"].long()
    Lq, wl, scale = inp["q_len_per_req"], inp["window_left"], inp["scale"]
    causal = inp.get("mask_type", "causal") == "causal"
    out_scale = float(inp.get("out_scale", 1.0))
    B = bt.shape[0]
    if inp.get("qo_indptr") is not None:
        qo = [int(x) for x in inp["qo_indptr"].tolist()]
    else:
        qo = [b * Lq for b in range(B + 1)]
    sinks = inp["sinks"] if with_sinks else None
    R, Hq, D = q.shape
    P, Hkv, ps, _ = k.shape
    g = Hq // Hkv
    outs = torch.zeros(R, Hq, D, dtype=torch.float64)
    lses = torch.full((R, Hq), -math.inf, dtype=torch.float64)
    for b in range(B):
        n = int(n_all[b])
        lq = qo[b + 1] - qo[b]
        j = torch.arange(n)
        pages = bt[b, j // ps]
        slots = j % ps
        for h in range(Hq):
            kvh = h // g
            Kd = k[pages, kvh, slots]            # [n, D]
            Vd = v[pages, kvh, slots]
            for i in range(lq):
                r = qo[b] + i
                diag = n - lq + i
                mask = (j <= diag) if causal else torch.ones(n, dtype=torch.bool)
                if wl >= 0:
                    mask &= j >= diag - wl
                s = scale * (Kd @ q[r, h])
                s = torch.where(mask, s, torch.tensor(-math.inf, dtype=torch.float64))
                if not bool(mask.any()):
                    continue
                lses[r, h] = torch.logsumexp(s, 0) * LOG2E
                if sinks is not None:
                    s = torch.cat([s, torch.tensor([float(sinks[h])], dtype=torch.float64)])
                    Vx = torch.cat([Vd, torch.zeros(1, D, dtype=torch.float64)])
                else:
                    Vx = Vd
                p = torch.softmax(s, 0)
                outs[r, h] = out_scale * (p @ Vx)
    return outs.reshape(R * Hq, D).numpy(), lses.reshape(-1).numpy()


def run(inp, **kw):
    out, lse, lse_ws = oracle.decode(inp, **kw)
    return out, lse, lse_ws


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------
def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"inf": math.inf, "nan": math.nan}))


def test_format_fixture():
    gold = json.load(open(os.path.join(GOLD, "float_formats.json")))
    for code, key in ((oracle.BF16, "bf16"), (oracle.F16, "fp16")):
        for bits, expr in gold[key]:
            got = oracle.decode_bits(int(bits, 16), code)
            want = _ev(expr)
            if math.isnan(want):
                assert math.isnan(got), (key, bits)
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want), (key, bits, got)


def test_formats_exhaustive_vs_library():
    """All 65536 codes against numpy's binary16 and torch's bfloat16."""
    codes = np.arange(65536, dtype=np.uint16)
    f16 = codes.view(np.float16).astype(np.float64)
    bf16 = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    for code, ref in ((oracle.F16, f16), (oracle.BF16, bf16)):
        got = np.array([oracle.decode_bits(int(c), code) for c in codes])
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ----------------------------------------------------------------------------
# hand-worked cases
# ----------------------------------------------------------------------------
def _golden_inputs(common, case):
    dt = torch.bfloat16
    q = torch.tensor(case["q"], dtype=torch.float32).to(dt)
    k = torch.tensor(common["k_cache"], dtype=torch.float32).to(dt)
    v = torch.tensor(common["v_cache"], dtype=torch.float32).to(dt)
    return dict(q=q, k_cache=k, v_cache=v,
                block_tables=torch.tensor(common["block_tables"], dtype=torch.int32),
                seq_lens_kv=torch.tensor(common["seq_lens_kv"], dtype=torch.int32),
                sinks=None if case["sinks"] is None else torch.tensor(case["sinks"], dtype=torch.float32),
                scale=case["scale"], q_len_per_req=case["q_len_per_req"],
                window_left=case["window_left"])


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "hand_worked.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked(case):
    gold = json.load(open(os.path.join(GOLD, "hand_worked.json")))
    inp = _golden_inputs(gold["common"], case)
    out, lse, lse_ws = run(inp)
    env = {"__builtins__": {}, "e": math.e, "log2": math.log2, "ln": math.log}
    want_out = np.array([[eval(x, env) for x in row] for row in case["out"]], dtype=np.float64)
    want_lse = np.array([eval(x, env) for x in case["lse"]], dtype=np.float64)
    want_ws = np.array([eval(x, env) for x in case["lse_with_sink"]], dtype=np.float64)
    np.testing.assert_allclose(out, want_out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_ws, want_ws, rtol=0, atol=1e-13)
    ref_out, ref_lse = dense_reference(inp)
    np.testing.assert_allclose(ref_out, want_out, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# brute force over random tiny shapes
# ----------------------------------------------------------------------------
@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(B=st.integers(1, 3), g=st.sampled_from([1, 2, 3]), Hkv=st.integers(1, 2),
       D=st.sampled_from([1, 3, 8]), ps=st.sampled_from([1, 2, 3, 5]),
       Lq=st.integers(1, 3), wl=st.sampled_from([-1, 0, 1, 4]),
       sinks=st.booleans(), dtype=st.sampled_from(["bf16", "fp16"]),
       seed=st.integers(0, 10_000), data=st.data())
def test_brute_force_tiny(B, g, Hkv, D, ps, Lq, wl, sinks, dtype, seed, data):
    lens = data.draw(st.lists(st.integers(Lq, 12), min_size=B, max_size=B))
    inp = workloads.make_case(B=B, Hq=g * Hkv, Hkv=Hkv, D=D, page_size=ps, seq_lens=lens,
                              q_len_per_req=Lq, window_left=wl, sinks=sinks, dtype=dtype,
                              seed=seed, extra_pages=2, bt_pad=1, q_pad_heads=1)
    out, lse, _ = run(inp)
    ref_out, ref_lse = dense_reference(inp)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_brute_force_small_configs():
    """The tiny workload and a cut-down copy of each other workload's structure."""
    for inp in [workloads.make_config("tiny"),
                workloads.make_case(B=3, Hq=8, Hkv=2, D=16, page_size=4, seq_lens=(4, 9, 17),
                                    q_len_per_req=4, seed=3),
                workloads.make_case(B=2, Hq=8, Hkv=1, D=8, page_size=16, seq_lens=(40, 33),
                                    window_left=7, sinks=True, dtype="fp16", value_std=0.5,
                                    seed=4)]:
        out, lse, _ = run(inp)
        ref_out, ref_lse = dense_reference(inp)
        np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------
def _case(**kw):
    base = dict(B=2, Hq=4, Hkv=2, D=8, page_size=4, seq_lens=(7, 13), seed=11)
    base.update(kw)
    return workloads.make_case(**base)


def test_lse_is_logsumexp_times_log2e():
    """Note / LSE convention: lse = torch.logsumexp(scaled scores) * log2(e)."""
    inp = _case(seq_lens=(30, 17), q_len_per_req=1)
    _, lse, _ = run(inp)
    q, bt = inp["q"].double(), inp["block_tables"].long()
    k = inp["k_cache"].double()
    for b, n in enumerate(inp["seq_lens_kv"].tolist()):
        j = torch.arange(n)
        for h in range(4):
            kd = k[bt[b, j // 4], h // 2, j % 4]
            s = inp["scale"] * (kd @ q[b, h])
            want = float(torch.logsumexp(s, 0)) / math.log(2.0)
            assert abs(lse[b * 4 + h] - want) < 1e-12


def test_zero_query_is_mean_of_visible_values():
    """q = 0: every visible key gets the same weight -> out = mean of visible V
    rows and lse = log2(#visible).  With a window the count is
    min(window_left + 1, diag + 1) (batch_prefill summary: at most
    window_left + 1 keys per causal row)."""
    for wl in (-1, 0, 2, 5, 100):
        inp = _case(seq_lens=(7, 13), q_len_per_req=3, window_left=wl)
        inp["q"] = torch.zeros_like(inp["q"])
        out, lse, _ = run(inp)
        bt = inp["block_tables"].long()
        v = inp["v_cache"].double()
        for b, n in enumerate((7, 13)):
            for i in range(3):
                diag = n - 3 + i
                cnt = diag + 1 if wl < 0 else min(wl + 1, diag + 1)
                lo = diag + 1 - cnt
                j = torch.arange(lo, diag + 1)
                for h in range(4):
                    vd = v[bt[b, j // 4], h // 2, j % 4]
                    r = (b * 3 + i) * 4 + h
                    np.testing.assert_allclose(out[r], vd.mean(0).numpy(), atol=1e-14, rtol=0)
                    assert abs(lse[r] - math.log2(cnt)) < 1e-13


def test_single_visible_key():
    """One visible key: out is that key's value row, lse = score * log2(e)."""
    inp = _case(seq_lens=(1, 5), q_len_per_req=1, window_left=0)
    out, lse, _ = run(inp)
    q, k, v, bt = (inp["q"].double(), inp["k_cache"].double(), inp["v_cache"].double(),
                   inp["block_tables"].long())
    for b, n in enumerate((1, 5)):
        j = n - 1
        for h in range(4):
            page, slot = bt[b, j // 4], j % 4
            r = b * 4 + h
            np.testing.assert_array_equal(out[r], v[page, h // 2, slot].numpy())
            s = inp["scale"] * float(q[b, h] @ k[page, h // 2, slot])
            assert abs(lse[r] - s / math.log(2)) < 1e-13


def test_window_at_least_n_is_no_window():
    a = _case(seq_lens=(7, 13), window_left=-1, q_len_per_req=2)
    b = _case(seq_lens=(7, 13), window_left=12, q_len_per_req=2)
    oa, la, _ = run(a)
    ob, lb, _ = run(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_causal_row_equals_prefix_decode():
    """Parameters / q_len_per_req: row i sees keys 0 .. n - Lq + i, i.e. it is
    a one-token decode on the prefix of n - Lq + 1 + i keys."""
    Lq = 4
    for wl in (-1, 3):
        multi = _case(B=1, seq_lens=(21,), q_len_per_req=Lq, window_left=wl, sinks=True)
        om, lm, _ = run(multi)
        for i in range(Lq):
            single = dict(multi)
            single["q"] = multi["q"][i:i + 1]
            single["q_len_per_req"] = 1
            single["seq_lens_kv"] = torch.tensor([21 - Lq + 1 + i], dtype=torch.int32)
            os_, ls, _ = run(single)
            np.testing.assert_array_equal(om[i * 4:(i + 1) * 4], os_)
            np.testing.assert_array_equal(lm[i * 4:(i + 1) * 4], ls)


def test_last_causal_row_is_unmasked():
    multi = _case(B=2, seq_lens=(9, 14), q_len_per_req=3)
    om, lm, _ = run(multi)
    for b, n in enumerate((9, 14)):
        single = dict(multi)
        single["q"] = multi["q"][b * 3 + 2:b * 3 + 3]
        single["q_len_per_req"] = 1
        single["block_tables"] = multi["block_tables"][b:b + 1]
        single["seq_lens_kv"] = torch.tensor([n], dtype=torch.int32)
        os_, ls, _ = run(single)
        r = (b * 3 + 2) * 4
        np.testing.assert_array_equal(om[r:r + 4], os_)


def test_gqa_equals_mha_on_repeated_heads():
    """Note: query head h reads kv head h // (Hq / Hkv).  Repeating every kv
    head g times gives an MHA cache with identical results."""
    g = 3
    inp = _case(Hq=6, Hkv=2, seq_lens=(9, 14), q_len_per_req=2, window_left=4, sinks=True)
    o1, l1, _ = run(inp)
    mha = dict(inp)
    mha["k_cache"] = inp["k_cache"].repeat_interleave(g, dim=1).contiguous()
    mha["v_cache"] = inp["v_cache"].repeat_interleave(g, dim=1).contiguous()
    o2, l2, _ = run(mha)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_mha_head_isolation():
    """Hq = Hkv: changing kv head 1 changes only query head 1."""
    inp = _case(Hq=2, Hkv=2, seq_lens=(9, 14))
    o1, _, _ = run(inp)
    mod = dict(inp)
    mod["k_cache"] = inp["k_cache"].clone()
    mod["k_cache"][:, 1] = -mod["k_cache"][:, 1]
    o2, _, _ = run(mod)
    o1, o2 = o1.reshape(-1, 2, 8), o2.reshape(-1, 2, 8)
    np.testing.assert_array_equal(o1[:, 0], o2[:, 0])
    assert np.abs(o1[:, 1] - o2[:, 1]).max() > 1e-3


def test_page_permutation_invariance():
    """Permuting physical pages and rewriting block_tables leaves every output
    unchanged (Parameters / block_tables: the table is the only page map)."""
    inp = _case(seq_lens=(7, 13), q_len_per_req=2, window_left=3, sinks=True, extra_pages=4)
    o1, l1, w1 = run(inp)
    P = inp["k_cache"].shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    moved = dict(inp)
    moved["k_cache"] = inp["k_cache"][perm].contiguous()     # new page x holds old page perm[x]
    moved["v_cache"] = inp["v_cache"][perm].contiguous()
    moved["block_tables"] = inv[inp["block_tables"].long()].to(torch.int32)
    o2, l2, w2 = run(moved)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(w1, w2)


def test_page_size_repack_invariance():
    """The same logical keys stored with page sizes 1, 4 and 16 give identical
    results (key j lives in page j // page_size, slot j % page_size)."""
    base = _case(page_size=16, seq_lens=(7, 13), q_len_per_req=2, window_left=5, sinks=True)
    o1, l1, _ = run(base)
    bt = base["block_tables"].long()
    for ps in (1, 4):
        ks, vs, rows = [], [], []
        for b, n in enumerate((7, 13)):
            j = torch.arange(n)
            kd = base["k_cache"][bt[b, j // 16], :, j % 16]     # [n, Hkv, D]
            vd = base["v_cache"][bt[b, j // 16], :, j % 16]
            npg = -(-n // ps)
            pad = npg * ps - n
            kd = torch.cat([kd, torch.zeros(pad, *kd.shape[1:], dtype=kd.dtype)])
            vd = torch.cat([vd, torch.zeros(pad, *vd.shape[1:], dtype=vd.dtype)])
            ks.append(kd.view(npg, ps, *kd.shape[1:]).transpose(1, 2))
            vs.append(vd.view(npg, ps, *vd.shape[1:]).transpose(1, 2))
            rows.append(npg)
        k = torch.cat(ks).contiguous()
        v = torch.cat(vs).contiguous()
        C = max(rows)
        table = torch.zeros((2, C), dtype=torch.int32)
        off = 0
        for b, npg in enumerate(rows):
            table[b, :npg] = torch.arange(off, off + npg, dtype=torch.int32)
            off += npg
        rep = dict(base, k_cache=k, v_cache=v, block_tables=table)
        o2, l2, _ = run(rep)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_sink_is_extra_logit_with_zero_value():
    """Parameters / sinks: out_sink = out_nosink * S / (S + e^sink) with
    S = 2^lse (keys only); lse is unchanged; lse_with_sink = log2(S + e^sink)."""
    inp = _case(seq_lens=(7, 13), q_len_per_req=2, window_left=4, sinks=True)
    o_s, l_s, w_s = run(inp)
    o_n, l_n, w_n = run(inp, sinks=None)
    np.testing.assert_array_equal(l_s, l_n)
    np.testing.assert_array_equal(l_n, w_n)
    Hq = 4
    sink = np.tile(inp["sinks"].double().numpy(), o_s.shape[0] // Hq)
    S = np.exp2(l_n)
    factor = S / (S + np.exp(sink))
    np.testing.assert_allclose(o_s, o_n * factor[:, None], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(w_s, np.log2(S + np.exp(sink)), rtol=1e-13, atol=1e-13)


def test_sink_limits():
    inp = _case(seq_lens=(7, 13), sinks=True)
    o_n, _, _ = run(inp, sinks=None)
    o_lo, _, _ = run(inp, sinks=torch.full((4,), -1e30))
    np.testing.assert_array_equal(o_lo, o_n)
    o_hi, _, _ = run(inp, sinks=torch.full((4,), 80.0))
    assert np.abs(o_hi).max() < 1e-25


def test_merge_of_disjoint_ranges_equals_union():
    """Note / LSE convention: base-2 LSE states of disjoint key ranges merge
    (cascade merge) to the state of their union, sinks applied once."""
    inp = _case(seq_lens=(29, 31), q_len_per_req=2, window_left=-1, sinks=True)
    o_full, l_full, _ = run(inp)
    cuts = [0, 5, 11, 12, 30, 1 << 40]
    parts = [run(inp, key_range=(a, b), sinks=None) for a, b in zip(cuts[:-1], cuts[1:])]
    sinks = inp["sinks"].double().numpy()
    for idx in range(o_full.shape[0]):
        o = np.stack([p[0][idx] for p in parts])
        l = np.array([p[1][idx] for p in parts])
        mo, ml = oracle.merge_states(o, l, sink=sinks[idx % 4])
        np.testing.assert_allclose(mo, o_full[idx], rtol=1e-12, atol=1e-14)
        assert abs(ml - l_full[idx]) < 1e-12


def test_empty_rows_are_zero_and_minus_inf():
    """Out of contract (n < q_len_per_req): rows with no visible key give
    out = 0 and lse = -inf, never NaN."""
    inp = _case(B=2, seq_lens=(1, 6), q_len_per_req=3)
    out, lse, _ = run(inp)
    rows = out.reshape(2, 3, 4, 8)
    l = lse.reshape(2, 3, 4)
    assert np.all(rows[0, :2] == 0) and np.all(np.isneginf(l[0, :2]))
    assert np.all(np.isfinite(l[0, 2])) and np.all(np.isfinite(l[1]))


def test_selected_rows_match_full():
    inp = _case(seq_lens=(7, 13), q_len_per_req=2, sinks=True)
    o, l, w = run(inp)
    sel = [15, 0, 3, 9]
    o2, l2, w2 = run(inp, sel=sel)
    np.testing.assert_array_equal(o[sel], o2)
    np.testing.assert_array_equal(l[sel], l2)


def test_poison_never_read():
    """NaN in every slot past a request's length, in unused pages and in a
    page that padding columns point to: the oracle never dereferences them."""
    clean = workloads.make_config("tiny")
    bad = workloads.make_config("tiny", poison=True)
    o1, l1, _ = run(clean)
    o2, l2, _ = run(bad)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------
# packed query rows, dense rows, output scale
# (batch_decode_with_paged_kv_cache: summary; Parameters qo_indptr,
#  max_seq_len_q, mask_type, bmm2_scale)
# ----------------------------------------------------------------------------
def _packed_golden():
    gold = json.load(open(os.path.join(GOLD, "hand_worked_packed.json")))
    c = gold["common"]
    dt = torch.bfloat16
    base = dict(q=torch.tensor(c["q"], dtype=torch.float32).to(dt),
                k_cache=torch.tensor(c["k_cache"], dtype=torch.float32).to(dt),
                v_cache=torch.tensor(c["v_cache"], dtype=torch.float32).to(dt),
                block_tables=torch.tensor(c["block_tables"], dtype=torch.int32),
                seq_lens_kv=torch.tensor(c["seq_lens_kv"], dtype=torch.int32),
                qo_indptr=torch.tensor(c["qo_indptr"], dtype=torch.int32),
                sinks=None, scale=1.0, q_len_per_req=2)
    return gold, base


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "hand_worked_packed.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked_packed(case):
    _, base = _packed_golden()
    inp = dict(base, mask_type=case["mask_type"], window_left=case["window_left"],
               out_scale=case["out_scale"])
    out, lse, _ = run(inp)
    env = {"__builtins__": {}, "e": math.e, "log2": math.log2, "ln": math.log}
    want_out = np.array([[eval(x, env) for x in row] for row in case["out"]], dtype=np.float64)
    want_lse = np.array([eval(x, env) for x in case["lse"]], dtype=np.float64)
    np.testing.assert_allclose(out, want_out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-13)
    ref_out, ref_lse = dense_reference(inp)
    np.testing.assert_allclose(ref_out, want_out, rtol=0, atol=1e-14)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(B=st.integers(1, 4), g=st.sampled_from([1, 2, 3]), Hkv=st.integers(1, 2),
       D=st.sampled_from([1, 3, 8]), ps=st.sampled_from([1, 2, 5]),
       wl=st.sampled_from([-1, 0, 1, 4]), mask=st.sampled_from(["causal", "dense"]),
       sinks=st.booleans(), out_scale=st.sampled_from([1.0, 0.5, -2.0]),
       seed=st.integers(0, 10_000), data=st.data())
def test_brute_force_packed(B, g, Hkv, D, ps, wl, mask, sinks, out_scale, seed, data):
    """Packed rows of varying length (zero included), both masks and an
    output factor against the dense torch brute force."""
    qls = data.draw(st.lists(st.integers(0, 4), min_size=B, max_size=B))
    lens = [data.draw(st.integers(max(q, 1), 12)) for q in qls]
    if sum(qls) == 0:
        qls[0] = 1
    inp = workloads.make_case(B=B, Hq=g * Hkv, Hkv=Hkv, D=D, page_size=ps, seq_lens=lens,
                              q_lens=qls, window_left=wl, sinks=sinks, mask_type=mask,
                              out_scale=out_scale, seed=seed, extra_pages=2, bt_pad=1,
                              q_pad_heads=1)
    out, lse, _ = run(inp)
    ref_out, ref_lse = dense_reference(inp)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_packed_equals_per_request_fixed_calls():
    """A packed batch equals, row for row, fixed-length calls on each request
    alone (its block-table row, its length, its rows of q)."""
    qls = (3, 0, 1, 4)
    lens = (9, 5, 14, 20)
    for mask in ("causal", "dense"):
        for wl in (-1, 2):
            inp = _case(B=4, seq_lens=lens, q_lens=qls, mask_type=mask, window_left=wl,
                        sinks=True, out_scale=1.5)
            o, l, _ = run(inp)
            qo = inp["qo_indptr"].tolist()
            for b, lq in enumerate(qls):
                if lq == 0:
                    continue
                one = dict(inp, q=inp["q"][qo[b]:qo[b + 1]], qo_indptr=None,
                           q_len_per_req=lq, block_tables=inp["block_tables"][b:b + 1],
                           seq_lens_kv=inp["seq_lens_kv"][b:b + 1])
                ob, lb, _ = run(one)
                np.testing.assert_array_equal(o[qo[b] * 4:qo[b + 1] * 4], ob)
                np.testing.assert_array_equal(l[qo[b] * 4:qo[b + 1] * 4], lb)


def test_fixed_lengths_through_qo_indptr_equal_fixed_rows():
    """qo_indptr = [0, Lq, 2 Lq, ...] is the fixed layout."""
    fixed = _case(B=3, seq_lens=(6, 9, 13), q_len_per_req=3, window_left=3, sinks=True)
    packed = dict(fixed, qo_indptr=torch.arange(0, 10, 3, dtype=torch.int32))
    o1, l1, _ = run(fixed)
    o2, l2, _ = run(packed)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_dense_row_equals_full_one_token_decode():
    """mask_type dense without a window: every row of a request sees all n
    keys, so each row equals a one-token decode of that row over n keys."""
    multi = _case(B=2, seq_lens=(9, 14), q_len_per_req=3, mask_type="dense", sinks=True)
    om, lm, _ = run(multi)
    for r in range(6):
        b = r // 3
        single = dict(multi, q=multi["q"][r:r + 1], q_len_per_req=1, mask_type="causal",
                      block_tables=multi["block_tables"][b:b + 1],
                      seq_lens_kv=multi["seq_lens_kv"][b:b + 1])
        os_, ls, _ = run(single)
        np.testing.assert_array_equal(om[r * 4:(r + 1) * 4], os_)
        np.testing.assert_array_equal(lm[r * 4:(r + 1) * 4], ls)


def test_one_token_rows_ignore_the_mask_type():
    """With one token per request the diagonal is the last key: both masks agree."""
    a = _case(seq_lens=(7, 13), window_left=4, sinks=True, mask_type="causal")
    b = dict(a, mask_type="dense")
    oa, la, _ = run(a)
    ob, lb, _ = run(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_output_scale_is_a_factor_on_the_output_only():
    """bmm2_scale: q = 0 gives out_scale x the mean of the visible V rows and
    an LSE of log2(#visible), whatever the scale."""
    for s in (0.25, -3.0):
        inp = _case(seq_lens=(7, 13), q_len_per_req=2, window_left=3, out_scale=s)
        inp["q"] = torch.zeros_like(inp["q"])
        out, lse, _ = run(inp)
        bt = inp["block_tables"].long()
        v = inp["v_cache"].double()
        for b, n in enumerate((7, 13)):
            for i in range(2):
                diag = n - 2 + i
                cnt = min(4, diag + 1)
                j = torch.arange(diag + 1 - cnt, diag + 1)
                for h in range(4):
                    vd = v[bt[b, j // 4], h // 2, j % 4]
                    r = (b * 2 + i) * 4 + h
                    np.testing.assert_allclose(out[r], s * vd.mean(0).numpy(), atol=1e-14, rtol=0)
                    assert abs(lse[r] - math.log2(cnt)) < 1e-13


def test_token_major_query_is_the_row_layout():
    """Fixed seq_len_q > 1: a [B, SQ, Hq, D] query is read as B * SQ rows."""
    inp = _case(B=2, seq_lens=(9, 14), q_len_per_req=3)
    o1, l1, _ = run(inp)
    tm = dict(inp, q=inp["q"].reshape(2, 3, 4, 8))
    o2, l2, _ = run(tm)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------
# context attention (batch_prefill: summary and Parameters)
# ----------------------------------------------------------------------------
def prefill_reference(inp):
    """Dense torch brute force: fp64 torch.softmax over explicit boolean masks
    per (request, query head), packed or fixed rows."""
    q, k, v = inp["q"].double(), inp["k"].double(), inp["v"].double()
    mask = inp.get("mask_type", "dense")
    wl = inp.get("window_left", -1)
    scale = inp.get("sm_scale") or 1.0 / math.sqrt(q.shape[-1])
    osc = inp.get("output_scale", 1.0)
    if inp.get("qo_indptr") is None:
        B, Sq, Hq, D = q.shape
        Sk = k.shape[1]
        qs = [q[b] for b in range(B)]
        ks = [k[b] for b in range(B)]
        vs = [v[b] for b in range(B)]
    else:
        qo = inp["qo_indptr"].tolist()
        kvo = inp["kv_indptr"].tolist()
        B = len(qo) - 1
        Hq, D = q.shape[1], q.shape[2]
        qs = [q[qo[b]:qo[b + 1]] for b in range(B)]
        ks = [k[kvo[b]:kvo[b + 1]] for b in range(B)]
        vs = [v[kvo[b]:kvo[b + 1]] for b in range(B)]
    g = Hq // k.shape[-2]
    outs = []
    for b in range(B):
        sq, sk = qs[b].shape[0], ks[b].shape[0]
        o = torch.zeros(sq, Hq, D, dtype=torch.float64)
        j = torch.arange(sk)
        for i in range(sq):
            diag = sk - sq + i
            if mask == "variable_window":
                m = (j >= int(inp["window_starts"][b, i])) & (j <= int(inp["window_ends"][b, i]))
            else:
                m = (j <= diag) if mask == "causal" else torch.ones(sk, dtype=torch.bool)
                if wl >= 0:
                    m &= j >= diag - wl
            if not bool(m.any()):
                continue
            for h in range(Hq):
                s = scale * (ks[b][:, h // g] @ qs[b][i, h])
                s = torch.where(m, s, torch.tensor(-math.inf, dtype=torch.float64))
                o[i, h] = osc * (torch.softmax(s, 0) @ vs[b][:, h // g])
        outs.append(o.reshape(-1, D))
    return torch.cat(outs).numpy()


def _prefill_golden(case):
    gold = json.load(open(os.path.join(GOLD, "hand_worked_prefill.json")))
    c = gold["common"]
    dt = torch.bfloat16
    q = torch.tensor([[[[1.0, 0.0]]] * case["Sq"]]).to(dt)
    inp = dict(q=q, k=torch.tensor(c["k"], dtype=torch.float32).to(dt),
               v=torch.tensor(c["v"], dtype=torch.float32).to(dt), mask_type=case["mask_type"],
               window_left=case["window_left"], output_scale=case["output_scale"], sm_scale=1.0)
    if "starts" in case:
        inp["window_starts"] = torch.tensor(case["starts"], dtype=torch.int32)
        inp["window_ends"] = torch.tensor(case["ends"], dtype=torch.int32)
    return inp


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "hand_worked_prefill.json")))["cases"],
                         ids=lambda c: c["name"])
def test_prefill_hand_worked(case):
    inp = _prefill_golden(case)
    out = oracle.prefill(inp)
    env = {"__builtins__": {}, "e": math.e}
    want = np.array([[eval(x, env) for x in row] for row in case["out"]], dtype=np.float64)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(prefill_reference(inp), want, rtol=0, atol=1e-14)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(B=st.integers(1, 3), g=st.sampled_from([1, 2, 3]), Hkv=st.integers(1, 2),
       D=st.sampled_from([1, 4, 8]), mask=st.sampled_from(["causal", "dense", "variable_window"]),
       wl=st.sampled_from([-1, 0, 2, 5]), packed=st.booleans(),
       osc=st.sampled_from([1.0, 0.5]), dtype=st.sampled_from(["bf16", "fp16"]),
       seed=st.integers(0, 10_000), data=st.data())
def test_prefill_brute_force(B, g, Hkv, D, mask, wl, packed, osc, dtype, seed, data):
    """Masks, windows, GQA, packed rows and the output scale against the torch
    brute force (variable windows only with fixed shapes, as documented)."""
    if mask == "variable_window":
        packed = False
        wl = -1
    if packed:
        ql = data.draw(st.lists(st.integers(0, 6), min_size=B, max_size=B))
        kl = data.draw(st.lists(st.integers(0, 9), min_size=B, max_size=B))
        if sum(ql) == 0:
            ql[0] = 1
        inp = workloads.make_prefill_case(B=B, Hq=g * Hkv, Hkv=Hkv, D=D, q_lens=ql, kv_lens=kl,
                                          mask_type=mask, window_left=wl, output_scale=osc,
                                          dtype=dtype, seed=seed, pad_heads=1)
    else:
        Sq = data.draw(st.integers(1, 6))
        Sk = data.draw(st.integers(1, 9))
        win = None
        if mask == "variable_window":
            st_ = [[data.draw(st.integers(0, Sk - 1)) for _ in range(Sq)] for _ in range(B)]
            en_ = [[data.draw(st.integers(s, Sk - 1)) for s in row] for row in st_]
            win = (st_, en_)
        inp = workloads.make_prefill_case(B=B, Sq=Sq, Sk=Sk, Hq=g * Hkv, Hkv=Hkv, D=D,
                                          mask_type=mask, window_left=wl, output_scale=osc,
                                          window=win, dtype=dtype, seed=seed, pad_heads=1)
    np.testing.assert_allclose(oracle.prefill(inp), prefill_reference(inp), rtol=1e-12, atol=1e-13)


def test_prefill_equals_decode_definition_on_one_page_caches():
    """Causal context attention of Sq queries over Sk keys is the decode's
    bottom-right causal multi-token definition (q_len_per_req = Sq) on a cache
    holding each request's keys in one page: two independent definitions."""
    B, Sq, Sk, Hq, Hkv, D = 3, 4, 11, 6, 2, 8
    for wl in (-1, 3):
        p = workloads.make_prefill_case(B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, mask_type="causal",
                                        window_left=wl, seed=8)
        dec = dict(q=p["q"].reshape(B * Sq, Hq, D), k_cache=p["k"].transpose(1, 2).contiguous(),
                   v_cache=p["v"].transpose(1, 2).contiguous(),
                   block_tables=torch.arange(B, dtype=torch.int32).view(B, 1),
                   seq_lens_kv=torch.full((B,), Sk, dtype=torch.int32), sinks=None,
                   scale=p["sm_scale"], q_len_per_req=Sq, window_left=wl)
        out_d, _, _ = oracle.decode(dec)
        np.testing.assert_allclose(oracle.prefill(p), out_d, rtol=1e-13, atol=1e-15)


def test_prefill_zero_query_window_counts():
    """q = 0: every visible key weighs the same, so the output is the mean of
    the visible values; with a window a causal row keeps min(window_left + 1,
    p_i + 1) keys (summary), also when Sq < Sk."""
    B, Sq, Sk, D = 2, 3, 8, 4
    for wl in (-1, 0, 2, 20):
        p = workloads.make_prefill_case(B=B, Sq=Sq, Sk=Sk, Hq=2, Hkv=1, D=D, mask_type="causal",
                                        window_left=wl, seed=9)
        p["q"] = torch.zeros_like(p["q"])
        out = oracle.prefill(p).reshape(B, Sq, 2, D)
        v = p["v"].double()
        for b in range(B):
            for i in range(Sq):
                diag = Sk - Sq + i
                cnt = diag + 1 if wl < 0 else min(wl + 1, diag + 1)
                np.testing.assert_allclose(out[b, i, 0], v[b, diag + 1 - cnt:diag + 1, 0].mean(0).numpy(),
                                           atol=1e-14, rtol=0)


def test_prefill_variable_window_equal_to_causal_window():
    """variable_window bounds set to [p_i - window_left, p_i] give the causal
    window's result."""
    B, Sq, Sk, wl = 2, 5, 9, 2
    p = workloads.make_prefill_case(B=B, Sq=Sq, Sk=Sk, Hq=4, Hkv=2, D=8, mask_type="causal",
                                    window_left=wl, seed=10)
    starts = [[max(0, Sk - Sq + i - wl) for i in range(Sq)] for _ in range(B)]
    ends = [[Sk - Sq + i for i in range(Sq)] for _ in range(B)]
    vw = dict(p, mask_type="variable_window", window_left=-1,
              window_starts=torch.tensor(starts, dtype=torch.int32),
              window_ends=torch.tensor(ends, dtype=torch.int32))
    np.testing.assert_array_equal(oracle.prefill(p), oracle.prefill(vw))


def test_prefill_packed_equals_per_request_fixed():
    """Packed rows equal fixed calls on each request alone."""
    ql, kl = (3, 1, 4), (5, 1, 9)
    for mask in ("causal", "dense"):
        p = workloads.make_prefill_case(B=3, Hq=4, Hkv=2, D=8, q_lens=ql, kv_lens=kl,
                                        mask_type=mask, window_left=2, seed=12)
        out = oracle.prefill(p)
        qo, kvo = p["qo_indptr"].tolist(), p["kv_indptr"].tolist()
        for b in range(3):
            one = dict(p, q=p["q"][qo[b]:qo[b + 1]].unsqueeze(0),
                       k=p["k"][kvo[b]:kvo[b + 1]].unsqueeze(0),
                       v=p["v"][kvo[b]:kvo[b + 1]].unsqueeze(0), qo_indptr=None, kv_indptr=None)
            np.testing.assert_array_equal(out[qo[b] * 4:qo[b + 1] * 4], oracle.prefill(one))


def test_prefill_gqa_equals_mha():
    p = workloads.make_prefill_case(B=2, Sq=4, Sk=7, Hq=6, Hkv=2, D=8, mask_type="causal", seed=13)
    mha = dict(p, k=p["k"].repeat_interleave(3, dim=2).contiguous(),
               v=p["v"].repeat_interleave(3, dim=2).contiguous())
    np.testing.assert_array_equal(oracle.prefill(p), oracle.prefill(mha))
