"""Seeded synthetic workloads for the attention forward and backward passes.

This module only draws random tensors with the shapes, dtypes and value
distributions of the workloads the pages discuss; it contains none of the
attention arithmetic. Both the fp64 oracle (``oracle/``) and the HIP path
(``tiled_prefill_amd``) are fed from here, so they see identical bits.

Layouts (the pages fix none; this is the usual flash-attention convention):
  q, o : [B, Sq, Hq, d]
  k, v : [B, Sk, Hkv, d]
  lse  : [B, Hq, Sq] (fp32 on the GPU side)

Every tensor is drawn in fp32 from ``torch.Generator('cpu').manual_seed(seed)``
(standard normal, times ``std``) and then rounded on the CPU to the workload's
dtype, so the oracle can upcast exactly the values the GPU receives.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int               # key length (the padded maximum for varlen)
    d: int
    causal: bool
    window_left: int = -1  # -1: unlimited
    std: float = 1.0
    varlen: bool = False  # per-sequence key lengths drawn uniformly in [varlen_lo, Sk]
    varlen_lo: int = 0
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The six forward workloads. Shapes follow the pages' discussion of decode
# ("分块策略与调度" §5: long KV with few heads, split-KV), speculative verification
# (the occupancy blog's verify-attention shapes) and long-context prefill
# ("分块策略与调度" §3: causal and sliding-window block skipping).
WORKLOADS = {
    "decode_fp32": Workload(
        "decode_fp32", "fp32", B=1, Hq=4, Hkv=4, Sq=1, Sk=256, d=64, causal=False,
        note="tiny fp32 decode; num_splits swept 1..8"),
    "gqa_decode_bf16": Workload(
        "gqa_decode_bf16", "bf16", B=1, Hq=32, Hkv=4, Sq=1, Sk=32768, d=128, causal=False,
        note="long-context GQA decode, group 8, grid B*Hkv = 4 without splitting"),
    "spec_verify_fp32": Workload(
        "spec_verify_fp32", "fp32", B=2, Hq=16, Hkv=16, Sq=17, Sk=2065, d=128, causal=True,
        note="speculative verify: the 17 query rows are the last 17 key positions"),
    "causal_prefill_bf16": Workload(
        "causal_prefill_bf16", "bf16", B=1, Hq=32, Hkv=32, Sq=8192, Sk=8192, d=128, causal=True,
        std=0.5, note="causal prefill with block skipping"),
    "window_prefill_bf16": Workload(
        "window_prefill_bf16", "bf16", B=4, Hq=32, Hkv=8, Sq=4096, Sk=4096, d=128, causal=True,
        window_left=1024, note="sliding-window causal prefill"),
    "varlen_decode_bf16": Workload(
        "varlen_decode_bf16", "bf16", B=16, Hq=32, Hkv=8, Sq=1, Sk=16384, d=128, causal=False,
        varlen=True, varlen_lo=512, note="batched decode, key lengths uniform in [512, 16384]"),
}


def make_inputs(w: Workload, seed: int = 0, device: Optional[str] = None):
    """Draw (q, k, v, seqlens_k) for workload ``w`` from ``seed``.

    Returns CPU tensors (or tensors moved to ``device``). ``seqlens_k`` is an
    int32 tensor of shape [B] for varlen workloads and ``None`` otherwise.
    The k/v tensors of a varlen workload are padded to ``w.Sk`` rows; rows at
    or beyond a sequence's length hold random values that must never be read
    into the result.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((w.B, w.Sq, w.Hq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Sk, w.Hkv, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Sk, w.Hkv, w.d), generator=g, dtype=torch.float32)
    if w.std != 1.0:
        q.mul_(w.std)
        k.mul_(w.std)
        v.mul_(w.std)
    dt = w.torch_dtype
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    seqlens = None
    if w.varlen:
        seqlens = torch.randint(w.varlen_lo, w.Sk + 1, (w.B,), generator=g, dtype=torch.int32)
    if device is not None:
        q, k, v = q.to(device), k.to(device), v.to(device)
        if seqlens is not None:
            seqlens = seqlens.to(device)
    return q, k, v, seqlens


def small_case(seed: int, dtype: str, B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int,
               std: float = 1.0, seqlens=None):
    """Random (q, k, v) of an arbitrary small shape, same recipe as ``make_inputs``."""
    w = Workload("small", dtype, B, Hq, Hkv, Sq, Sk, d, causal=False, std=std)
    q, k, v, _ = make_inputs(w, seed)
    return q, k, v


# Latent-attention verify workloads (attn_fwd_dv; keys 576 wide, values 512, one
# KV head shared by Hq query heads, causal over the last Sq positions):
# name -> (B, Hq, Sq, Sk). The first is the verify parity shape printed on the
# occupancy blog page; the second its long-prefix case (the 65k prefix for which
# the page derives 32 KV splits).
LATENT_WORKLOADS = {
    "latent_verify_bf16": (2, 16, 17, 2065),
    "latent_verify_long_bf16": (1, 16, 17, 65536),
}


def latent_case(seed: int, B: int, Hq: int, Sq: int, Sk: int, d: int = 576, dv: int = 512,
                std: float = 1.0, dtype: str = "bf16"):
    """Random latent-attention verify inputs: one KV head shared by the Hq query
    heads, q/k rows d wide, v rows dv wide; N(0, 1) * std in fp32, rounded on the
    CPU to the dtype (the recipe of ``make_inputs``)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = (torch.randn((B, Sq, Hq, d), generator=g) * std).to(td)
    k = (torch.randn((B, Sk, 1, d), generator=g) * std).to(td)
    v = (torch.randn((B, Sk, 1, dv), generator=g) * std).to(td)
    return q, k, v


def random_partials(seed: int, S: int, rows: int, d: int, p_empty: float = 0.25):
    """Random split partials (O_s [S, rows, d] fp32, lse_s [S, rows] fp32).

    A fraction ``p_empty`` of the (split, row) entries are empty splits:
    lse = -inf and O = 0, as a split with no visible key would leave them.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    o = torch.randn((S, rows, d), generator=g, dtype=torch.float32)
    lse = torch.randn((S, rows), generator=g, dtype=torch.float32) * 4.0
    empty = torch.rand((S, rows), generator=g) < p_empty
    lse[empty] = float("-inf")
    o[empty] = 0.0
    return o, lse


# Backward workloads: the two bf16 prefill shapes above, run through the
# backward pass (the pages describe its loop order and scheduler but measure no
# backward workload, so the forward's prefill shapes stand in).
BWD_WORKLOADS = {
    "causal_prefill_bwd_bf16": WORKLOADS["causal_prefill_bf16"].replace(name="causal_prefill_bwd_bf16"),
    "window_prefill_bwd_bf16": WORKLOADS["window_prefill_bf16"].replace(name="window_prefill_bwd_bf16"),
}


def output_grad(seed: int, shape, dtype: str = "bf16", std: float = 1.0, device=None):
    """Random output gradient dO of the given shape ([B, Sq, Hq, d]) from its own
    seeded generator (seed + 7919, so it is independent of the q, k, v draw of the
    same seed); N(0, 1) * std in fp32, rounded on the CPU to the dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed) + 7919)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    t = t.to(torch.float32 if dtype == "fp32" else torch.bfloat16)
    return t.to(device) if device is not None else t
