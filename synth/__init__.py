"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random tensors and names the workloads; it holds none
of the attention arithmetic. Both sides of every parity check (the HIP path and
the CPU oracle) receive exactly the tensors produced here: the HIP path gets
them in their storage dtype on the GPU, the oracle gets the same values
widened to float64.

Recipe (one draw per call): a CPU ``torch.Generator`` seeded with the
workload's seed draws q, k, v and dO, in that order, as i.i.d. N(0, 1) float32
samples; each is then rounded to the workload's storage dtype on the CPU.

Workload shapes follow the pages' cases: the 4096-token, 32-head case
(page "FlashAttention：为什么少搬数据，反而算得更快", §06), the 8192-token,
32-head FP16 case (page "FlashAttention技术原理详解：通过内存优化加速注意力计算")
and the small-batch decode case whose score row is 1 x history (page
"FlashAttention：为什么少搬数据，反而算得更快", §09).
"""

from __future__ import annotations

import dataclasses
import math

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    d: int
    dtype: str  # "f32" | "bf16" | "f16"
    causal: bool
    seed: int
    backward: bool = True

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flop(self) -> float:
        """Two GEMMs of the forward, halved when causal (metric convention)."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nkv * self.d
        return f * 0.5 if self.causal else f

    def bwd_flop(self) -> float:
        """Five GEMMs of the backward: 2.5x the forward count."""
        return 2.5 * self.fwd_flop()

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads; several have causal / head-count variants.
WORKLOADS = {
    "c1": Workload("c1", 1, 1, 1, 256, 256, 64, "f32", False, 11, backward=False),
    "c1c": Workload("c1c", 1, 1, 1, 256, 256, 64, "f32", True, 11, backward=False),
    "c2": Workload("c2", 2, 16, 16, 1024, 1024, 64, "bf16", False, 21),
    "c2c": Workload("c2c", 2, 16, 16, 1024, 1024, 64, "bf16", True, 21),
    "c3": Workload("c3", 1, 32, 32, 4096, 4096, 128, "bf16", True, 31),
    "c4": Workload("c4", 1, 32, 32, 8192, 8192, 128, "f16", True, 41),
    "c5g": Workload("c5g", 4, 32, 8, 2048, 2048, 128, "bf16", True, 51),
    "c5m": Workload("c5m", 4, 32, 1, 2048, 2048, 128, "bf16", True, 52),
    "c5dg": Workload("c5dg", 16, 32, 8, 1, 8192, 128, "bf16", True, 53, backward=False),
    "c5dm": Workload("c5dm", 16, 32, 1, 1, 8192, 128, "bf16", True, 54, backward=False),
}


def make_inputs(w: Workload, with_grad: bool | None = None):
    """Draw (q, k, v, dO) on the CPU in the workload's storage dtype.

    dO is drawn only when the workload has a backward (or ``with_grad``).
    """
    if with_grad is None:
        with_grad = w.backward
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    dt = w.torch_dtype
    q = torch.randn((w.B, w.Hq, w.Nq, w.d), generator=g, dtype=torch.float32).to(dt)
    k = torch.randn((w.B, w.Hkv, w.Nkv, w.d), generator=g, dtype=torch.float32).to(dt)
    v = torch.randn((w.B, w.Hkv, w.Nkv, w.d), generator=g, dtype=torch.float32).to(dt)
    do = None
    if with_grad:
        do = torch.randn((w.B, w.Hq, w.Nq, w.d), generator=g, dtype=torch.float32).to(dt)
    return q, k, v, do


def random_tensors(shape_q, shape_kv, dtype: str, seed: int, with_grad: bool = False):
    """Same recipe as :func:`make_inputs` for ad-hoc shapes (edge cases)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = _DTYPES[dtype]
    q = torch.randn(shape_q, generator=g, dtype=torch.float32).to(dt)
    k = torch.randn(shape_kv, generator=g, dtype=torch.float32).to(dt)
    v = torch.randn(shape_kv, generator=g, dtype=torch.float32).to(dt)
    do = torch.randn(shape_q, generator=g, dtype=torch.float32).to(dt) if with_grad else None
    return q, k, v, do


def to_f64(t):
    """Widen a CPU tensor to a float64 numpy array (exact for f32/bf16/f16)."""
    return t.detach().to("cpu", torch.float64).numpy()


def ramp_tensors(shape_q, shape_kv, dtype: str, seed: int, ramp: str, peak: float = 32.0,
                 with_grad: bool = False):
    """Score-range stress inputs: q and k drawn as |N(0, 1)| (so every score
    q . k is positive and grows with the size of k), each key row j of k
    multiplied by a factor r_j that varies along the sequence, v and dO as
    N(0, 1). ``ramp`` picks r_j for N_kv keys:

    * "up":   r_j = 1 + (peak - 1) j / (N_kv - 1), each later key tile scores higher;
    * "down": the reverse, the first tile holds every row's maximum;
    * "wave": r_j = 1 + (peak - 1) (1 + sin(j / 40)) / 2, maxima come and go.

    Same generator recipe as :func:`random_tensors` (q, k, v, dO in that order),
    rounded to the storage dtype at the end.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = _DTYPES[dtype]
    q = torch.randn(shape_q, generator=g, dtype=torch.float32).abs()
    k = torch.randn(shape_kv, generator=g, dtype=torch.float32).abs()
    v = torch.randn(shape_kv, generator=g, dtype=torch.float32)
    do = torch.randn(shape_q, generator=g, dtype=torch.float32) if with_grad else None
    n = shape_kv[-2]
    j = torch.arange(n, dtype=torch.float32)
    t = j / max(n - 1, 1)
    if ramp == "up":
        r = 1.0 + (peak - 1.0) * t
    elif ramp == "down":
        r = 1.0 + (peak - 1.0) * (1.0 - t)
    elif ramp == "wave":
        r = 1.0 + (peak - 1.0) * 0.5 * (1.0 + torch.sin(j / 40.0))
    else:
        raise ValueError(ramp)
    k = k * r[:, None]
    return q.to(dt), k.to(dt), v.to(dt), (do.to(dt) if do is not None else None)


def random_device_tensor(shape, dtype: str, seed: int, device="cuda"):
    """One i.i.d. N(0, 1) tensor drawn directly on the device (for inputs of
    several GiB that are never drawn on the host): a device generator seeded
    with ``seed`` draws the values in the storage dtype. Tests copy back the
    rows the oracle needs, so both sides still see the same values."""
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=_DTYPES[dtype], device=device)
