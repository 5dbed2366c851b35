"""Seeded synthetic q/k/v generators shared by the oracle side and the GPU side.

This module holds no arithmetic of the attention method: it only draws random
numbers and casts them to the storage dtype.  Both the CPU oracle tests and the
HIP path consume exactly the bytes produced here.

Recipe (one workload = one seed):
  * one ``torch.Generator`` seeded with the workload's seed;
  * draw q, k, v in that order as float32 ``randn`` in logical (B, H, N, D) shape;
  * video-DiT workload only: then draw a per-(head, channel) offset ~ N(0, sigma=2)
    and add it to every token of k (the K outlier pattern that mean smoothing is
    meant to remove);
  * large-magnitude variants only (``qk_scale``, ``outliers``): q and k are multiplied
    by qk_scale; with outliers = (f_chan, f_tok), 4 channels of every head (drawn with
    torch.randperm from the same generator) are multiplied by f_chan in q and k, and 1%
    of the tokens of every head (likewise drawn) by f_tok -- the outlier channels and
    tokens of real activations, which drive the block scales, and with them the
    dequantisation factor of the scores, up by one to two orders of magnitude;
  * cast to fp16 / bf16 with round-to-nearest-even (torch's ``.to``);
  * NHD layout = the same logical tensor stored as (B, N, H, D), contiguous.

The workload shapes mirror the benchmarks the SageAttention pages describe:
a tiny smoke case, an LLM prefill shape, a video-DiT self-attention shape
(CogVideoX-like, N = 17776), the kernel-throughput sweep over N = 1K..32K at
head dim 128, and a grouped-query case with an odd head dim.
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import List, Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "workload", "make_qkv", "sweep_workloads"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str          # "fp16" | "bf16"
    layout: str         # "HND" | "NHD"
    causal: bool
    pv: str             # "fp16" | "fp8"
    accum: str          # "fp32" | "fp16+fp32"
    seed: int
    k_offset_sigma: Optional[float] = None
    qk_scale: float = 1.0
    outliers: Optional[Tuple[float, float]] = None   # (channel factor, token factor)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    def ops(self) -> float:
        """Effective attention operations 4*B*H*Nq*Nkv*D, halved when causal."""
        o = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.D
        return o / 2 if self.causal else o


# The five workload families.  Seeds are fixed per family (0..4).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 256, 256, 64, "fp16", "HND", False, "fp16", "fp32", 0),
    "llm_prefill": Workload("llm_prefill", 1, 8, 8, 2048, 2048, 128, "fp16", "HND", False, "fp16", "fp32", 1),
    "video_dit": Workload("video_dit", 1, 24, 24, 17776, 17776, 64, "bf16", "NHD", False, "fp8", "fp32", 2,
                          k_offset_sigma=2.0),
    "seq_sweep": Workload("seq_sweep", 4, 32, 32, 8192, 8192, 128, "bf16", "HND", False, "fp8", "fp16+fp32", 3),
    "gqa": Workload("gqa", 2, 32, 8, 8192, 8192, 128, "bf16", "NHD", True, "fp16", "fp32", 4),
}

SWEEP_N = (1024, 2048, 4096, 8192, 16384, 32768)


def workload(name: str, **overrides) -> Workload:
    return WORKLOADS[name].with_(**overrides)


def sweep_workloads(causal: bool) -> List[Workload]:
    return [WORKLOADS["seq_sweep"].with_(Nq=n, Nkv=n, causal=causal) for n in SWEEP_N]


def _to_layout(x: torch.Tensor, layout: str) -> torch.Tensor:
    if layout == "HND":
        return x.contiguous()
    if layout == "NHD":
        return x.transpose(1, 2).contiguous()
    raise ValueError(f"unknown layout {layout!r}")


def make_qkv(w: Workload, seed: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Return CPU tensors (q, k, v) in ``w.layout`` and ``w.dtype``."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    q = torch.randn(w.B, w.Hq, w.Nq, w.D, generator=g, dtype=torch.float32)
    k = torch.randn(w.B, w.Hkv, w.Nkv, w.D, generator=g, dtype=torch.float32)
    v = torch.randn(w.B, w.Hkv, w.Nkv, w.D, generator=g, dtype=torch.float32)
    if w.k_offset_sigma is not None:
        off = torch.randn(w.Hkv, w.D, generator=g, dtype=torch.float32) * w.k_offset_sigma
        k += off[None, :, None, :]
    if w.qk_scale != 1.0:
        q *= w.qk_scale
        k *= w.qk_scale
    if w.outliers is not None:
        fc, ft = w.outliers
        for x in (q, k):
            for h in range(x.shape[1]):
                x[:, h, :, torch.randperm(w.D, generator=g)[:4]] *= fc
                n = x.shape[2]
                x[:, h, torch.randperm(n, generator=g)[:max(1, n // 100)], :] *= ft
    dt = w.torch_dtype
    return (_to_layout(q.to(dt), w.layout), _to_layout(k.to(dt), w.layout), _to_layout(v.to(dt), w.layout))


# ----------------------------------------------------------------------------- packed variable-length batches

@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """Sequences of different lengths packed along one token axis (sageattn_varlen)."""
    name: str
    lens_q: Tuple[int, ...]
    lens_k: Tuple[int, ...]
    Hq: int
    Hkv: int
    D: int
    dtype: str = "bf16"
    causal: bool = False
    pv: str = "fp16"
    accum: str = "fp32"
    seed: int = 0
    k_offset_sigma: Optional[float] = None

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16

    @property
    def B(self) -> int:
        return len(self.lens_q)

    def ops(self) -> float:
        """4 * H * sum_b(visible query-key pairs) * D."""
        total = 0.0
        for nq, nk in zip(self.lens_q, self.lens_k):
            if self.causal:
                off = nk - nq
                total += sum(max(0, min(nk, i + off + 1)) for i in range(nq))
            else:
                total += nq * nk
        return 4.0 * self.Hq * total * self.D


def make_varlen(w: VarlenWorkload):
    """CPU tensors q (total_q, Hq, D), k, v (total_k, Hkv, D) and int32 prefix sums
    cu_q, cu_k: randn in fp32 from one seeded generator (q, k, v, then the key offset,
    one per (head, channel), shared by every token), cast to the workload dtype."""
    g = torch.Generator().manual_seed(w.seed)
    tq, tk = sum(w.lens_q), sum(w.lens_k)
    q = torch.randn(tq, w.Hq, w.D, generator=g, dtype=torch.float32)
    k = torch.randn(tk, w.Hkv, w.D, generator=g, dtype=torch.float32)
    v = torch.randn(tk, w.Hkv, w.D, generator=g, dtype=torch.float32)
    if w.k_offset_sigma is not None:
        k += torch.randn(w.Hkv, w.D, generator=g, dtype=torch.float32)[None] * w.k_offset_sigma
    cu_q = torch.tensor([0] + list(itertools.accumulate(w.lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(itertools.accumulate(w.lens_k)), dtype=torch.int32)
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt), cu_q, cu_k
