"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic.  Both the HIP path (through its callers) and the oracle
receive the very same bit patterns produced here.

Recipe: values are sampled in float32 on the CPU with a seeded
``torch.Generator`` (uniform via ``rand``, normal via ``randn`` scaled by the
standard deviation) and rounded once to bf16/fp16 or to the 8-bit E4M3 / E5M2
codes with torch's round-to-nearest-even conversions (float32 inputs keep the
sampled values; the distributions stay far inside the 8-bit formats' range).
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
          "f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}
BYTE_KINDS = ("f8e4m3", "f8e5m2")


def torch_dtype(kind: str) -> torch.dtype:
    return _TORCH[kind]


@dataclass(frozen=True)
class Dist:
    kind: str          # "uniform" or "normal"
    a: float           # uniform: low;  normal: mean
    b: float           # uniform: high; normal: standard deviation

    def sample(self, shape, seed: int, dtype: torch.dtype) -> torch.Tensor:
        g = torch.Generator().manual_seed(int(seed))
        if self.kind == "uniform":
            x = torch.rand(shape, generator=g, dtype=torch.float32) * (self.b - self.a) + self.a
        elif self.kind == "normal":
            x = torch.randn(shape, generator=g, dtype=torch.float32) * self.b + self.a
        else:
            raise ValueError(self.kind)
        return x.to(dtype)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_kind: str                 # "bf16", "f16", "f32", "f8e4m3" or "f8e5m2"
    out_kind: str                # "f32" or "bf16"
    alpha: float
    beta: float
    dist_a: Dist
    dist_b: Dist
    seeds: tuple
    dist_c: Dist = None          # existing C when beta != 0
    gate_up: bool = False
    act: str = ""                # gate/up epilogue activation: "" (G and U) or "swiglu" (one output)
    b_kmajor: bool = False       # B stored [N, K] (K contiguous; one-byte inputs need it)
    split: bool = False          # run with K cut into the plan's ranges (gemm_run_split)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K * (2 if self.gate_up else 1)


WORKLOADS = {
    "square256": Workload(
        "square256", 256, 256, 256, "bf16", "f32", 1.0, 0.0,
        Dist("uniform", -1.0, 1.0), Dist("uniform", -1.0, 1.0), (1001, 1002),
        notes="single 256^3 GEMM, bf16 in, fp32 out"),
    "square4096": Workload(
        "square4096", 4096, 4096, 4096, "bf16", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0 / math.sqrt(4096)), Dist("normal", 0.0, 1.0 / math.sqrt(4096)),
        (2001, 2002), notes="4096^3 GEMM, bf16 in, bf16 out"),
    "ragged": Workload(
        "ragged", 1000, 1537, 999, "f16", "f32", 1.5, -0.5,
        Dist("uniform", -2.0, 2.0), Dist("uniform", -2.0, 2.0), (3001, 3002, 3003),
        dist_c=Dist("uniform", -1.0, 1.0), notes="ragged edges, in-place fp32 C"),
    "gate_up": Workload(
        "gate_up", 4096, 11008, 4096, "bf16", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.02), (4001, 4002, 4003),
        gate_up=True, notes="x[4096,4096] times W_gate and W_up [4096,11008]"),
    "gate_up_swiglu": Workload(
        "gate_up_swiglu", 4096, 11008, 4096, "bf16", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.02), (4001, 4002, 4003),
        gate_up=True, act="swiglu", notes="silu(x W_gate) * (x W_up), one bf16 output"),
    "square4096_f32": Workload(
        "square4096_f32", 4096, 4096, 4096, "f32", "f32", 1.0, 0.0,
        Dist("normal", 0.0, 1.0 / math.sqrt(4096)), Dist("normal", 0.0, 1.0 / math.sqrt(4096)),
        (2101, 2102), notes="4096^3 GEMM, binary32 in and out"),
    # one-byte inputs: A [M, K] and B stored [N, K], both K-contiguous
    "square4096_f8": Workload(
        "square4096_f8", 4096, 4096, 4096, "f8e4m3", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 1.0),
        (2201, 2202), b_kmajor=True, notes="4096^3 GEMM, E4M3 in (B stored [N, K]), bf16 out"),
    "gate_up_f8": Workload(
        "gate_up_f8", 4096, 11008, 4096, "f8e4m3", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.25), (4101, 4102, 4103),
        gate_up=True, b_kmajor=True, notes="x[4096,4096] E4M3 times W_gate and W_up stored [11008,4096] E4M3"),
    "skinny": Workload(
        "skinny", 16, 28672, 8192, "bf16", "f32", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.02), (5001, 5002, 5003),
        notes="M=16 bandwidth-bound GEMM"),
    # the same with the weights stored [N, K] (the usual storage of a linear layer's weight)
    "skinny_kmajor": Workload(
        "skinny_kmajor", 16, 28672, 8192, "bf16", "f32", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.02), (5101, 5102, 5103), b_kmajor=True,
        notes="M=16 bandwidth-bound GEMM, B stored [28672, 8192]"),
    "skinny_f8": Workload(
        "skinny_f8", 16, 28672, 8192, "f8e4m3", "f32", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.25), (5201, 5202, 5203), b_kmajor=True,
        notes="M=16 bandwidth-bound GEMM, E4M3 A and B, B stored [28672, 8192]"),
    # 384 tokens through a 4096 -> 11008 projection: 129 tiles of 128 x 256 (86 of 256 x 256)
    "prefill_384": Workload(
        "prefill_384", 384, 11008, 4096, "bf16", "bf16", 1.0, 0.0,
        Dist("normal", 0.0, 1.0 / 64), Dist("normal", 0.0, 1.0 / 64), (5401, 5402),
        notes="mid-size M: 384 x 11008 x 4096 GEMM on 128-row tiles"),
    # a decode batch of 32 through a 14336 -> 4096 projection: 64 strips of B, K cut into ranges
    "skinny_split": Workload(
        "skinny_split", 32, 4096, 14336, "bf16", "f32", 1.0, 0.0,
        Dist("normal", 0.0, 1.0), Dist("normal", 0.0, 0.02), (5301, 5302, 5303), b_kmajor=True, split=True,
        notes="M=32 bandwidth-bound GEMM on a small grid, B stored [4096, 14336], K split"),
}


@dataclass(frozen=True)
class NormWorkload:
    """Row normalisation Y = X * inv_rms(X) * G over [M, D] rows."""
    name: str
    M: int
    D: int
    in_kind: str                 # X and G: "f32", "bf16" or "f16"
    out_kind: str                # Y
    eps: float
    dist_x: Dist
    dist_g: Dist
    seeds: tuple
    notes: str = ""

    def bytes(self) -> int:
        isz = 4 if self.in_kind == "f32" else 2
        osz = 4 if self.out_kind == "f32" else 2
        return self.M * self.D * (isz + osz) + self.D * isz


NORM_WORKLOADS = {
    # the Phobos example's shape: f32 rows of D = 256, eps = 1e-6; a million rows (1 GiB each way)
    "rms_norm": NormWorkload(
        "rms_norm", 1 << 20, 256, "f32", "f32", 1e-6,
        Dist("normal", 0.0, 1.0), Dist("uniform", 0.5, 1.5), (6001, 6002),
        notes="f32 rows of 256, as in the page's rms_norm kernel"),
    # the step before a projection in a transformer block: bf16 activations, D = 4096
    "rms_norm_bf16": NormWorkload(
        "rms_norm_bf16", 65536, 4096, "bf16", "bf16", 1e-6,
        Dist("normal", 0.0, 1.0), Dist("uniform", 0.5, 1.5), (6101, 6102),
        notes="bf16 rows of 4096 (512 MiB each way)"),
}


def make_norm_inputs(w: NormWorkload, rows=None):
    """CPU tensors X [M, D] (or only the listed rows, drawn from the same stream) and G [D]."""
    dt = torch_dtype(w.in_kind)
    x = w.dist_x.sample((w.M, w.D), w.seeds[0], dt)
    if rows is not None:
        x = x[rows].contiguous()
    return {"X": x, "G": w.dist_g.sample((w.D,), w.seeds[1], dt)}


@dataclass(frozen=True)
class AttnWorkload:
    """Softmax attention over `batch` independent (query, key, value) sets."""
    name: str
    batch: int
    sq: int
    sk: int
    d: int
    in_kind: str                 # Q, K, V: "bf16" or "f16"
    out_kind: str                # O
    dist: Dist                   # entries of Q, K and V
    seeds: tuple                 # Q, K, V
    notes: str = ""

    def flops(self) -> float:
        return 4.0 * self.batch * self.sq * self.sk * self.d

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


ATTN_WORKLOADS = {
    # a transformer prefill: 4 sequences x 16 heads, 4096 tokens, head dimension 128
    "attention": AttnWorkload(
        "attention", 64, 4096, 4096, 128, "bf16", "bf16", Dist("normal", 0.0, 1.0), (7001, 7002, 7003),
        notes="64 (batch x head) entries, 4096 queries and keys, d = 128, scale 1/sqrt(d)"),
}


def make_attn_inputs(w: AttnWorkload):
    """CPU tensors Q [batch, sq, d], K and V [batch, sk, d]."""
    dt = torch_dtype(w.in_kind)
    return {"Q": w.dist.sample((w.batch, w.sq, w.d), w.seeds[0], dt),
            "K": w.dist.sample((w.batch, w.sk, w.d), w.seeds[1], dt),
            "V": w.dist.sample((w.batch, w.sk, w.d), w.seeds[2], dt)}


def make_inputs(w: Workload):
    """CPU tensors: dict with A [M,K], B [K,N] (N contiguous) or Wg/Wu, and C_in."""
    dt = torch_dtype(w.in_kind)
    out = {"A": w.dist_a.sample((w.M, w.K), w.seeds[0], dt)}
    if w.gate_up:
        out["Wg"] = w.dist_b.sample((w.K, w.N), w.seeds[1], dt)
        out["Wu"] = w.dist_b.sample((w.K, w.N), w.seeds[2], dt)
    else:
        out["B"] = w.dist_b.sample((w.K, w.N), w.seeds[1], dt)
    if w.dist_c is not None:
        out["C"] = w.dist_c.sample((w.M, w.N), w.seeds[2], torch.float32)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw patterns of a CPU tensor: bf16/fp16 as a uint16 numpy array, float32 as uint32,
    E4M3 / E5M2 as uint8."""
    if t.dtype == torch.float32:
        return t.contiguous().view(torch.int32).numpy().view(np.uint32)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.contiguous().view(torch.uint8).numpy()
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(t.dtype)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def uniform(shape, seed, kind, lo=-1.0, hi=1.0):
    return Dist("uniform", lo, hi).sample(shape, seed, torch_dtype(kind))


def normal(shape, seed, kind, std=1.0):
    return Dist("normal", 0.0, std).sample(shape, seed, torch_dtype(kind))
