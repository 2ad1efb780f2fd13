"""Seeded synthetic inputs for grouped-query attention decode.

This module holds no attention arithmetic: it only draws tensors.  It is the
one piece that both the HIP path's callers (tests, bench) and the float64
oracle consume, so that both see the exact same stored values.

Recipe (stated once, used everywhere):
  * one ``torch.Generator`` per problem, seeded with the workload's seed, on
    the device the tensors are made on;
  * draw order: q, then k, then v, then seq_lens;
  * q, k, v ~ N(0, 1) drawn in float32, then rounded to bf16 with
    round-to-nearest-even where the workload is bf16 (fp32 workloads keep the
    float32 draw); k and v are drawn one batch row at a time;
  * seq_lens: every sequence holds T rows for dense workloads; ragged
    workloads draw seq_lens[b] uniformly from the inclusive range [lo, hi];
  * cache rows beyond seq_lens[b] hold the same N(0,1) draw, or NaN when a
    caller asks for a poisoned tail (to prove those rows are never read).

The shapes follow the workloads the pages discuss: the Exaone4-1.2B decode
layer (32 query heads, 8 KV heads, head dim 64, context 4096) from "Same GQA,
Different Execution Cost Across Backends" (sections 1 and 8), a batched GQA-8
decode at head dim 128, a multi-query (single KV head) decode as in "빠른
Transformer 디코딩 — Multi-Query Attention", and a sweep of the KV-head count
from MHA to MQA as in "질의 헤드는 그대로, 키·값 헤드만 줄인다" (the table of
the three names on one axis).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    G: int
    D: int
    T: int
    sq: int
    dtype: str          # "f32", "bf16" or "f16": the type of q, k and v; out is fp32
    seed: int
    ragged: Optional[Tuple[int, int]] = None   # inclusive (lo, hi) for seq_lens

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 decode, oracle finishes well under a second
    "tiny_f32_b1_h32_g8_d64_t256": Workload(
        "tiny_f32_b1_h32_g8_d64_t256", B=1, H=32, G=8, D=64, T=256, sq=1,
        dtype="f32", seed=1001),
    # one Exaone4-1.2B-shaped decode layer
    "exaone_b1_h32_g8_d64_t4096": Workload(
        "exaone_b1_h32_g8_d64_t4096", B=1, H=32, G=8, D=64, T=4096, sq=1,
        dtype="bf16", seed=1002),
    # batched GQA-8 decode, ragged lengths in [1024, 4096]
    "batched_b32_h32_g8_d128_t4096_ragged": Workload(
        "batched_b32_h32_g8_d128_t4096_ragged", B=32, H=32, G=8, D=128,
        T=4096, sq=1, dtype="bf16", seed=1003, ragged=(1024, 4096)),
    # multi-query decode: one KV head for 32 query heads
    "mqa_b64_h32_g1_d128_t8192": Workload(
        "mqa_b64_h32_g1_d128_t8192", B=64, H=32, G=1, D=128, T=8192, sq=1,
        dtype="bf16", seed=1004),
    # group-size sweep with two new tokens per step (causal among them)
    "sweep_b16_h32_g32_d128_t16384_sq2": Workload(
        "sweep_b16_h32_g32_d128_t16384_sq2", B=16, H=32, G=32, D=128,
        T=16384, sq=2, dtype="bf16", seed=1005),
    "sweep_b16_h32_g8_d128_t16384_sq2": Workload(
        "sweep_b16_h32_g8_d128_t16384_sq2", B=16, H=32, G=8, D=128,
        T=16384, sq=2, dtype="bf16", seed=1006),
    "sweep_b16_h32_g4_d128_t16384_sq2": Workload(
        "sweep_b16_h32_g4_d128_t16384_sq2", B=16, H=32, G=4, D=128,
        T=16384, sq=2, dtype="bf16", seed=1007),
    "sweep_b16_h32_g1_d128_t16384_sq2": Workload(
        "sweep_b16_h32_g1_d128_t16384_sq2", B=16, H=32, G=1, D=128,
        T=16384, sq=2, dtype="bf16", seed=1008),
    # 64 new query tokens per sequence (causal among them) on a ragged cache:
    # 256 query rows share each KV head
    "multitoken_b8_h32_g8_d128_t4096_sq64": Workload(
        "multitoken_b8_h32_g8_d128_t4096_sq64", B=8, H=32, G=8, D=128, T=4096,
        sq=64, dtype="bf16", seed=1009, ragged=(1024, 4096)),
}

# The workload the benchmark times: batched GQA-8 decode at B=32, T=4096.
HEADLINE = "batched_b32_h32_g8_d128_t4096_ragged"


def _randn(shape, gen, device, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def make_inputs(w: Workload, device="cpu", poison_tail: bool = False):
    """Draw q [B,H,sq,D], k/v [B,G,T,D], seq_lens [B] int32 for workload w.

    Returns a dict with keys q, k, v, seq_lens (all on ``device``).
    ``poison_tail`` fills cache rows at or beyond seq_lens[b] with NaN.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = w.torch_dtype
    q = _randn((w.B, w.H, w.sq, w.D), gen, device, dt)
    k = torch.empty((w.B, w.G, w.T, w.D), dtype=dt, device=device)
    for b in range(w.B):
        k[b] = _randn((w.G, w.T, w.D), gen, device, dt)
    v = torch.empty_like(k)
    for b in range(w.B):
        v[b] = _randn((w.G, w.T, w.D), gen, device, dt)
    if w.ragged is not None:
        lo, hi = w.ragged
        seq_lens = torch.randint(lo, hi + 1, (w.B,), generator=gen,
                                 device=device, dtype=torch.int64).to(torch.int32)
    else:
        seq_lens = torch.full((w.B,), w.T, dtype=torch.int32, device=device)
    if poison_tail:
        lens = seq_lens.cpu().tolist()
        for b, L in enumerate(lens):
            if L < w.T:
                k[b, :, L:, :] = float("nan")
                v[b, :, L:, :] = float("nan")
    return {"q": q, "k": k, "v": v, "seq_lens": seq_lens}


def make_custom(B, H, G, D, T, sq, dtype="bf16", seed=0, seq_lens=None,
                device="cpu", poison_tail=False):
    """Same recipe for an arbitrary shape (used by edge-case tests).

    ``seq_lens``: None (all T), an int range tuple (lo, hi) drawn after v, or
    an explicit list of ints.
    """
    ragged = seq_lens if isinstance(seq_lens, tuple) else None
    w = Workload("custom", B=B, H=H, G=G, D=D, T=T, sq=sq, dtype=dtype,
                 seed=seed, ragged=ragged)
    x = make_inputs(w, device=device, poison_tail=False)
    if isinstance(seq_lens, (list,)):
        x["seq_lens"] = torch.tensor(seq_lens, dtype=torch.int32, device=device)
    if poison_tail:
        lens = x["seq_lens"].cpu().tolist()
        for b, L in enumerate(lens):
            L = max(0, min(L, T))
            if L < T:
                x["k"][b, :, L:, :] = float("nan")
                x["v"][b, :, L:, :] = float("nan")
    return x
