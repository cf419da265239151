"""Seeded synthetic inputs for the owner-side Muon step.

This module draws numbers and encodes them in the stored dtypes; it holds none
of the optimizer's arithmetic.  The HIP path's tests, the bench and the CPU
oracle's tests all take their inputs from here, so both sides see the same
bytes.

Every matrix is drawn on its own from a PCG64 stream keyed by
``SeedSequence([workload_id, param_index, matrix_index, kind_id])``, so any
single matrix of a large workload can be regenerated without the rest.  Values
are drawn in float64, rounded to float32 (round-to-nearest-even) and, for
bfloat16 tensors, rounded once more to bfloat16 (round-to-nearest-even).

The workloads follow the shapes the pages discuss: the 74 skinny [24, 10240]
parameters fused into one batch (HyperParallel RFC, item 3), MoE expert tensors
[E, M, N] orthogonalised per expert (HyperParallel-FSDP §6.3; RFC item 2), all
Muon matrices of a 32-layer dense decoder, and a large 8192 x 28672 batch with
a low-rank-plus-noise gradient.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Newton-Schulz coefficients of the constant-coefficient quintic (used for
# every step), and the other hyperparameters of the workloads below.
DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)

KIND_IDS = {"grad": 0, "momentum": 1, "param": 2}


# ----------------------------------------------------------------------------
# storage encodings
# ----------------------------------------------------------------------------
def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 (numpy's cast is round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (round-to-nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(f64_to_f32(x))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values -> stored representation (uint16 bits for bf16, float32)."""
    if dtype == BF16:
        return f64_to_bf16_bits(x)
    if dtype == F32:
        return f64_to_f32(x)
    raise ValueError(dtype)


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """stored representation -> exact float64 values."""
    if dtype == BF16:
        return bf16_bits_to_f64(x)
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# workload definitions
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]          # [M,N], [M,1,N] or [E,M,N]
    dtype: str = BF16                # param and grad dtype

    @property
    def matrix_shape(self) -> Tuple[int, int]:
        if len(self.shape) == 2:
            return (self.shape[0], self.shape[1])
        if len(self.shape) == 3 and self.shape[1] == 1:
            return (self.shape[0], self.shape[2])
        if len(self.shape) == 3:
            return (self.shape[1], self.shape[2])
        raise ValueError(self.shape)

    @property
    def num_matrices(self) -> int:
        if len(self.shape) == 3 and self.shape[1] != 1:
            return self.shape[0]
        return 1


@dataclass(frozen=True)
class HParams:
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    eps: float = 1e-7
    nesterov: bool = True
    ns_steps: int = 5
    coeffs: Tuple[float, ...] = DEFAULT_COEFFS     # 3 (constant) or 3*ns_steps
    scale: str = "rms"                              # "rms" -> 0.2*sqrt(max(M,N)); "none" -> 1
    precision: str = "bf16"                         # "bf16" | "bf16_x32" | "bf16_x32c" | "f32"


@dataclass
class Workload:
    name: str
    wid: int
    params: List[ParamSpec]
    grad_recipe: str                 # "normal" | "row_scaled" | "low_rank_noise"
    momentum_recipe: str             # "zeros" | "normal"
    hp: HParams = field(default_factory=HParams)
    grad_scale: float = 1.0
    sequential_seed0: bool = False   # draw g, M, W in that order from default_rng(0)

    # -- drawing ------------------------------------------------------------
    def _rng(self, pi: int, mi: int, kind: str) -> np.random.Generator:
        ss = np.random.SeedSequence([self.wid, pi, mi, KIND_IDS[kind]])
        return np.random.Generator(np.random.PCG64(ss))

    def matrix_f64(self, pi: int, mi: int, kind: str) -> np.ndarray:
        """Float64 draw of one [M,N] matrix (before the storage rounding)."""
        spec = self.params[pi]
        M, N = spec.matrix_shape
        if self.sequential_seed0:
            assert pi == 0 and mi == 0
            rng = np.random.default_rng(0)
            g = rng.standard_normal((M, N))
            mom = rng.standard_normal((M, N))
            w = rng.normal(0.0, 0.02, (M, N))
            return {"grad": g, "momentum": mom, "param": w}[kind]
        rng = self._rng(pi, mi, kind)
        if kind == "param":
            return rng.normal(0.0, 0.02, (M, N))
        if kind == "momentum":
            if self.momentum_recipe == "zeros":
                return np.zeros((M, N))
            return rng.standard_normal((M, N))
        # gradient
        if self.grad_recipe == "normal":
            return rng.standard_normal((M, N)) * self.grad_scale
        if self.grad_recipe == "row_scaled":
            g = rng.standard_normal((M, N)) * self.grad_scale
            r = np.exp(rng.uniform(np.log(0.1), np.log(10.0), (M, 1)))
            return g * r
        if self.grad_recipe == "low_rank_noise":
            rank = 64
            U = rng.standard_normal((M, rank))
            V = rng.standard_normal((N, rank))
            E = rng.standard_normal((M, N))
            E *= 0.1                                    # N(0, 0.01): variance 0.01
            return U @ V.T + E
        raise ValueError(self.grad_recipe)

    def matrix(self, pi: int, mi: int, kind: str) -> np.ndarray:
        """Stored encoding of one matrix: uint16 bf16 bits or float32."""
        dtype = F32 if kind == "momentum" else self.params[pi].dtype
        return encode(self.matrix_f64(pi, mi, kind), dtype)

    def stored_dtype(self, pi: int, kind: str) -> str:
        return F32 if kind == "momentum" else self.params[pi].dtype

    def tensor(self, pi: int, kind: str) -> np.ndarray:
        """Stored encoding of a whole parameter tensor, in its own shape."""
        spec = self.params[pi]
        mats = [self.matrix(pi, mi, kind) for mi in range(spec.num_matrices)]
        return np.stack(mats).reshape(spec.shape)

    def nominal_ns_flops(self) -> float:
        """4 m^2 n + 2 m^3 per Newton-Schulz step per matrix, m = min(M, N)."""
        tot = 0.0
        for p in self.params:
            M, N = p.matrix_shape
            m, n = min(M, N), max(M, N)
            tot += p.num_matrices * self.hp.ns_steps * (4.0 * m * m * n + 2.0 * m ** 3)
        return tot

    def num_elements(self) -> int:
        return sum(int(np.prod(p.shape)) for p in self.params)


def _decoder32() -> List[ParamSpec]:
    out = []
    for layer in range(32):
        for nm in ("q", "k", "v", "o"):
            out.append(ParamSpec(f"l{layer}.{nm}", (4096, 4096)))
        out.append(ParamSpec(f"l{layer}.gate", (11008, 4096)))
        out.append(ParamSpec(f"l{layer}.up", (11008, 4096)))
        out.append(ParamSpec(f"l{layer}.down", (4096, 11008)))
    return out


WORKLOADS: Dict[str, Workload] = {
    # one fp32 128x256 matrix; g and M ~ N(0,1), W ~ N(0, 0.02^2), seed 0
    "single_128x256_f32": Workload(
        "single_128x256_f32", 0, [ParamSpec("w", (128, 256), F32)],
        "normal", "normal", HParams(precision="f32"), sequential_seed0=True),
    # 74 skinny [24, 10240] parameters fused into one batch
    "fused_74x24x10240": Workload(
        "fused_74x24x10240", 1,
        [ParamSpec(f"p{i}", (24, 10240)) for i in range(74)],
        "normal", "zeros", HParams(precision="bf16")),
    # MoE expert tensors, row norms scaled log-uniformly in [0.1, 10]
    "moe_experts": Workload(
        "moe_experts", 2,
        [ParamSpec("experts_a", (32, 24, 10240)), ParamSpec("experts_b", (64, 2048, 7168))],
        "row_scaled", "zeros", HParams(precision="bf16"), grad_scale=1e-3),
    # the skinny expert tensor of moe_experts alone (same seeds, so the same
    # matrices): a small HBM-bound batch of its own
    "moe_experts_24x10240": Workload(
        "moe_experts_24x10240", 2,
        [ParamSpec("experts_a", (32, 24, 10240))],
        "row_scaled", "zeros", HParams(precision="bf16"), grad_scale=1e-3),
    # every Muon matrix of a 32-layer dense decoder (hidden 4096, MLP 11008)
    "decoder32_h4096_f11008": Workload(
        "decoder32_h4096_f11008", 3, _decoder32(),
        "normal", "zeros", HParams(precision="bf16")),
    # 16 x [8192, 28672] + 16 x [28672, 8192], rank-64 + noise gradients
    "large_8192x28672": Workload(
        "large_8192x28672", 4,
        [ParamSpec(f"a{i}", (8192, 28672)) for i in range(16)]
        + [ParamSpec(f"b{i}", (28672, 8192)) for i in range(16)],
        "low_rank_noise", "zeros", HParams(precision="bf16_x32")),
}


def small_workload(name: str, shapes: List[Tuple[int, ...]], dtype: str = BF16,
                   grad_recipe: str = "normal", momentum_recipe: str = "normal",
                   wid: int = 100, hp: Optional[HParams] = None,
                   grad_scale: float = 1.0) -> Workload:
    """Ad-hoc workload for parity tests (ragged shapes, edge cases)."""
    return Workload(name, wid, [ParamSpec(f"t{i}", tuple(s), dtype) for i, s in enumerate(shapes)],
                    grad_recipe, momentum_recipe, hp or HParams(), grad_scale=grad_scale)
