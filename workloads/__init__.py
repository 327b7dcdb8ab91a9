"""Seeded synthetic inputs for batched paged-KV decode.

This module only draws random numbers and lays them out as a paged KV cache
(pages, block tables, sequence lengths). It holds none of the attention
arithmetic: both the fp64 CPU oracle and the HIP path consume what it returns.

Layouts follow flashinfer.cudnn.cudnn_batch_decode_with_kv_cache (Parameters):
  q            (B * q_len_per_req, Hq, D), rows of one request consecutive
  k_cache      (num_pages, Hkv, page_size, D)   ("HND" page layout)
  v_cache      (num_pages, Hkv, page_size, D)
  block_tables (B, C) int32, row b lists the physical pages of request b
  seq_lens_kv  (B,) int32
  sinks        (Hq,) float32 or None

Every tensor is returned on the CPU; callers move it to a device themselves.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

__all__ = ["Workload", "CONFIGS", "make_config", "make_case", "seq_lens_of", "make_prefill_case",
           "PREFILL_CONFIGS", "make_prefill_config"]

_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """Shape and distribution parameters of one synthetic decode batch."""

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    q_len_per_req: int = 1
    kv_lo: int = 1          # sequence lengths drawn uniformly from [kv_lo, kv_hi]
    kv_hi: int = 256
    dtype: str = "bf16"
    value_std: float = 1.0  # q, K, V ~ N(0, value_std^2)
    window_left: int = -1
    sinks: bool = False
    return_lse: bool = False
    pool: str = "exact"     # "exact": pool = sum of pages needed, shuffled
                            # "fixed": pool = B * C pages, block_tables = randperm.view(B, C)
    seed: int = 0

    @property
    def C(self) -> int:
        """Block-table width: pages needed by the longest possible request."""
        return -(-self.kv_hi // self.page_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The five workloads of this decode kernel.  Seeds 1001..1005.
CONFIGS = {
    "tiny": Workload("tiny", B=4, Hq=8, Hkv=2, D=128, page_size=16, kv_lo=1, kv_hi=256,
                     return_lse=True, pool="fixed", seed=1001),
    "llama3_8b": Workload("llama3_8b", B=64, Hq=32, Hkv=8, D=128, page_size=16,
                          kv_lo=512, kv_hi=4096, return_lse=True, seed=1002),
    "long_ctx": Workload("long_ctx", B=4, Hq=64, Hkv=8, D=128, page_size=64,
                         kv_lo=32768, kv_hi=131072, seed=1003),
    "spec_verify": Workload("spec_verify", B=32, Hq=32, Hkv=8, D=128, page_size=16,
                            q_len_per_req=4, kv_lo=1024, kv_hi=8192, return_lse=True,
                            seed=1004),
    "sink_window": Workload("sink_window", B=128, Hq=64, Hkv=8, D=64, page_size=16,
                            kv_lo=2048, kv_hi=16384, dtype="fp16", value_std=0.5,
                            window_left=127, sinks=True, seed=1005),
}


def _randn_chunked(shape: Sequence[int], gen: torch.Generator, std: float,
                   dtype: torch.dtype, chunk_rows: int = 4096) -> torch.Tensor:
    """randn drawn page by page (dim 0) so large pools never hold an fp32 copy."""
    out = torch.empty(tuple(shape), dtype=dtype)
    n0 = shape[0]
    for s in range(0, n0, chunk_rows):
        e = min(n0, s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=gen)
        if std != 1.0:
            x.mul_(std)
        out[s:e] = x.to(dtype)
    return out


def seq_lens_of(w: Workload | str) -> torch.Tensor:
    """The sequence lengths make_config draws for ``w`` (its first draw),
    without drawing the rest of the batch."""
    if isinstance(w, str):
        w = CONFIGS[w]
    gen = torch.Generator().manual_seed(w.seed)
    return torch.randint(w.kv_lo, w.kv_hi + 1, (w.B,), generator=gen, dtype=torch.int32)


def make_config(w: Workload | str, poison: bool = False,
                seq_lens: Optional[Sequence[int]] = None) -> dict:
    """Draw one batch for workload ``w``.

    Draw order (fixed): seq_lens, page permutation, q, K, V, sinks.
    ``poison=True`` adds a NaN page that every unused block-table column points
    to, and fills every slot past a request's length with NaN, so any read of
    data outside the visible keys shows up in the result.
    ``seq_lens`` overrides the drawn lengths (the draw still happens, so the
    remaining streams are unchanged).
    """
    if isinstance(w, str):
        w = CONFIGS[w]
    gen = torch.Generator().manual_seed(w.seed)
    dt = _DTYPES[w.dtype]
    B, ps, C = w.B, w.page_size, w.C

    n = torch.randint(w.kv_lo, w.kv_hi + 1, (B,), generator=gen, dtype=torch.int32)
    if seq_lens is not None:
        n = torch.tensor(list(seq_lens), dtype=torch.int32)
        assert n.numel() == B
    pages_needed = [(-(-int(x) // ps)) for x in n.tolist()]

    if w.pool == "fixed":
        P = B * C
        perm = torch.randperm(P, generator=gen).to(torch.int32)
        block_tables = perm.view(B, C).clone()
    else:
        P = max(1, sum(pages_needed))
        perm = torch.randperm(P, generator=gen).to(torch.int32)
        block_tables = torch.zeros((B, C), dtype=torch.int32)
        off = 0
        for b, npg in enumerate(pages_needed):
            block_tables[b, :npg] = perm[off:off + npg]
            off += npg

    q = _randn_chunked((B * w.q_len_per_req, w.Hq, w.D), gen, w.value_std, dt)
    k = _randn_chunked((P, w.Hkv, ps, w.D), gen, w.value_std, dt)
    v = _randn_chunked((P, w.Hkv, ps, w.D), gen, w.value_std, dt)
    sinks = torch.randn((w.Hq,), generator=gen, dtype=torch.float32) if w.sinks else None

    if poison:
        k, v, block_tables = _poison(k, v, block_tables, n, ps)

    return dict(workload=w, q=q, k_cache=k, v_cache=v, block_tables=block_tables,
                seq_lens_kv=n, sinks=sinks, scale=w.scale,
                q_len_per_req=w.q_len_per_req, window_left=w.window_left,
                return_lse=w.return_lse)


def _poison(k, v, block_tables, n, ps):
    """NaN in every slot no request may read, plus a NaN page for padding columns."""
    nan = float("nan")
    P = k.shape[0]
    k = torch.cat([k, torch.full_like(k[:1], nan)], 0)
    v = torch.cat([v, torch.full_like(v[:1], nan)], 0)
    used = torch.zeros(P + 1, dtype=torch.bool)
    bt = block_tables.clone()
    for b in range(bt.shape[0]):
        nb = int(n[b])
        npg = -(-nb // ps)
        row = bt[b]
        used[row[:npg].long()] = True
        row[npg:] = P                       # padding columns -> NaN page
        if npg > 0 and nb % ps:
            last = int(row[npg - 1])
            k[last, :, nb % ps:, :] = nan    # tail slots past the length
            v[last, :, nb % ps:, :] = nan
    unused = (~used[:P]).nonzero().flatten()
    if unused.numel():
        k[unused] = nan
        v[unused] = nan
    return k, v, bt


def make_case(B: int = 2, Hq: int = 4, Hkv: int = 2, D: int = 64, page_size: int = 16,
              seq_lens: Sequence[int] = (5, 40), q_len_per_req: int = 1,
              window_left: int = -1, sinks: bool = False, dtype: str = "bf16",
              value_std: float = 1.0, extra_pages: int = 3, C: Optional[int] = None,
              bt_pad: int = 0, seed: int = 0, q_pad_heads: int = 0,
              sink_std: float = 1.0, q_lens: Optional[Sequence[int]] = None,
              mask_type: str = "causal", out_scale: float = 1.0) -> dict:
    """A small explicit case for edge sweeps.

    ``extra_pages`` unused pages are added to the pool; ``bt_pad`` extra int32
    columns separate block-table rows (row stride C + bt_pad); ``q_pad_heads``
    makes q a head-slice of a wider tensor (arbitrary head/batch strides).
    ``q_lens`` packs the query rows: request b gets q_lens[b] rows and the
    case carries ``qo_indptr`` (cumulative offsets, B + 1 entries) with
    ``q_len_per_req`` = max(q_lens) as the per-request capacity.
    ``mask_type`` ("causal" or "dense") and ``out_scale`` are passed through.
    """
    qo_indptr = None
    if q_lens is not None:
        assert len(q_lens) == B
        qo_indptr = torch.zeros(B + 1, dtype=torch.int32)
        qo_indptr[1:] = torch.cumsum(torch.tensor(list(q_lens), dtype=torch.int64), 0).to(torch.int32)
        q_len_per_req = max(1, max(q_lens))
    gen = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    ps = page_size
    n = torch.tensor(list(seq_lens), dtype=torch.int32)
    assert n.numel() == B
    need = [(-(-int(x) // ps)) for x in n.tolist()]
    if C is None:
        C = max(1, max(need))
    P = sum(need) + extra_pages
    P = max(P, 1)
    perm = torch.randperm(P, generator=gen).to(torch.int32)
    bt_full = torch.zeros((B, C + bt_pad), dtype=torch.int32)
    off = 0
    for b, npg in enumerate(need):
        bt_full[b, :npg] = perm[off:off + npg]
        off += npg
    block_tables = bt_full[:, :C]
    rows = B * q_len_per_req if qo_indptr is None else int(qo_indptr[-1])
    qw = torch.randn((rows, Hq + q_pad_heads, D), generator=gen) * value_std
    q = qw.to(dt)[:, q_pad_heads:, :]
    k = (torch.randn((P, Hkv, ps, D), generator=gen) * value_std).to(dt)
    v = (torch.randn((P, Hkv, ps, D), generator=gen) * value_std).to(dt)
    s = (torch.randn((Hq,), generator=gen) * sink_std).float() if sinks else None
    w = Workload("case", B=B, Hq=Hq, Hkv=Hkv, D=D, page_size=ps,
                 q_len_per_req=q_len_per_req, kv_lo=int(n.min()), kv_hi=int(n.max()),
                 dtype=dtype, value_std=value_std, window_left=window_left,
                 sinks=sinks, return_lse=True, seed=seed)
    return dict(workload=w, q=q, k_cache=k, v_cache=v, block_tables=block_tables,
                seq_lens_kv=n, sinks=s, scale=1.0 / math.sqrt(D),
                q_len_per_req=q_len_per_req, window_left=window_left, return_lse=True,
                qo_indptr=qo_indptr, mask_type=mask_type, out_scale=out_scale)



def make_prefill_case(B: int = 2, Sq: int = 5, Sk: int = 9, Hq: int = 4, Hkv: int = 2,
                      D: int = 128, dtype: str = "bf16", value_std: float = 1.0,
                      q_lens: Optional[Sequence[int]] = None,
                      kv_lens: Optional[Sequence[int]] = None, mask_type: str = "causal",
                      window_left: int = -1, output_scale: float = 1.0,
                      window: Optional[Sequence[Sequence[int]]] = None, seed: int = 0,
                      pad_heads: int = 0) -> dict:
    """Inputs of one context-attention (prefill) call (batch_prefill's layout).

    Fixed: q [B, Sq, Hq, D], k and v [B, Sk, Hkv, D].  Packed (q_lens and
    kv_lens given): q [sum q_lens, Hq, D], k and v [sum kv_lens, Hkv, D] with
    qo_indptr / kv_indptr (cumulative, B + 1 entries).  ``window`` =
    (starts, ends) as [B][Sq] nested lists gives the variable_window bounds.
    ``pad_heads`` makes q, k and v head slices of wider tensors (free strides).
    Draw order: q, k, v.
    """
    gen = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]

    def draw(shape):
        full = list(shape)
        full[-2] += pad_heads
        x = (torch.randn(tuple(full), generator=gen) * value_std).to(dt)
        return x[..., pad_heads:, :] if pad_heads else x

    d = dict(mask_type=mask_type, window_left=window_left, output_scale=output_scale,
             sm_scale=1.0 / math.sqrt(D))
    if q_lens is not None:
        assert kv_lens is not None and len(q_lens) == len(kv_lens) == B
        qo = torch.zeros(B + 1, dtype=torch.int32)
        kvo = torch.zeros(B + 1, dtype=torch.int32)
        qo[1:] = torch.cumsum(torch.tensor(list(q_lens)), 0).to(torch.int32)
        kvo[1:] = torch.cumsum(torch.tensor(list(kv_lens)), 0).to(torch.int32)
        d.update(q=draw((int(qo[-1]), Hq, D)), k=draw((int(kvo[-1]), Hkv, D)),
                 v=draw((int(kvo[-1]), Hkv, D)), qo_indptr=qo, kv_indptr=kvo,
                 max_seq_len_q=max(1, max(q_lens)))
    else:
        d.update(q=draw((B, Sq, Hq, D)), k=draw((B, Sk, Hkv, D)), v=draw((B, Sk, Hkv, D)))
    if window is not None:
        d["window_starts"] = torch.tensor(window[0], dtype=torch.int32).reshape(B, Sq)
        d["window_ends"] = torch.tensor(window[1], dtype=torch.int32).reshape(B, Sq)
    return d


# Context-attention (prefill) workloads measured and parity-tested beside the
# decode: a fixed causal batch at head_dim 128 and 256, a packed ragged batch
# and a windowed one.  Seeds 2001..2004.
PREFILL_CONFIGS = {
    "prefill_causal_d128": dict(B=4, Sq=4096, Sk=4096, Hq=32, Hkv=8, D=128, mask_type="causal",
                                seed=2001),
    "prefill_causal_d256": dict(B=4, Sq=4096, Sk=4096, Hq=16, Hkv=4, D=256, mask_type="causal",
                                seed=2002),
    "prefill_packed_d128": dict(B=8, Hq=32, Hkv=8, D=128, mask_type="causal", seed=2003,
                                lens=(512, 4096)),
    "prefill_window_d128": dict(B=4, Sq=4096, Sk=4096, Hq=32, Hkv=8, D=128, mask_type="causal",
                                window_left=1023, seed=2004),
}


def make_prefill_config(name: str) -> dict:
    """Draw one prefill workload of PREFILL_CONFIGS (packed lengths uniform in
    the stated range, equal query and key lengths per request)."""
    c = dict(PREFILL_CONFIGS[name])
    lens = c.pop("lens", None)
    if lens is not None:
        g = torch.Generator().manual_seed(c["seed"] + 100000)
        n = torch.randint(lens[0], lens[1] + 1, (c["B"],), generator=g).tolist()
        c.update(q_lens=n, kv_lens=n)
    return make_prefill_case(**c)
