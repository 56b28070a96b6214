"""Seeded synthetic inputs for the batched Muon step.

This module holds no arithmetic of the optimizer: it only defines the
workload shapes and draws gradients, momentum buffers and parameters from
seeded generators. Both the CPU oracle's tests and the GPU path's tests and
benchmark take their inputs from here, so that the two sides always see the
same stored values.

Workloads stand in for the model gradients of the HyperParallel-FSDP paper's
training runs (arXiv:2609.21594, section 7); no dataset or trained weight is
involved. The shapes are those of a dense transformer's attention and MLP
projections and of a mixture-of-experts expert bank; an expert weight
[E, M, N] is E independent M x N matrices (paper section 6.3).

Recipe (per matrix, independently regenerable):
  * RNG: numpy Generator(PCG64) seeded with SeedSequence([config_id, group,
    index, tensor]) where tensor is 0 = grad, 1 = momentum, 2 = params.
    The tiny fp32 configuration instead draws all grads, then all momentum,
    from default_rng(0) as one array each.
  * Normal draws are made in float32 and multiplied by the scale in float32;
    Student-t draws (nu = 3) are made in float64, scaled, cast to float32.
  * bf16 values are the float32 values rounded to nearest-even bf16; the
    stored bf16 bits are what both sides consume.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, List, Optional, Sequence, Tuple

import numpy as np

GRAD, MOMENTUM, PARAMS = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Group:
    """`count` matrices of shape rows x cols, stored row-major."""
    rows: int
    cols: int
    count: int
    name: str = ""
    # idle(index) -> True when this matrix's gradient is scaled by zero
    idle_every: int = 0          # 0 = never; k = matrix j is idle iff (j // per) % k == 0
    idle_group_size: int = 1     # matrices per expert sharing the idle flag


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    config_id: int
    description: str
    groups: Tuple[Group, ...]
    dtype: str                   # "f32" or "bf16": params and grads
    grad_dist: str               # "normal" or "student_t3"
    grad_scale: float
    momentum_init: str           # "zero" or "normal"
    params_init: str             # "zero" or "normal"
    lr: float = 0.02
    beta: float = 0.95
    ns_steps: int = 5
    seed0_bulk: bool = False     # tiny config: grads then momentum from default_rng(0)

    def matrices(self) -> List[Tuple[int, int, int, int]]:
        """(group index, index in group, rows, cols) for every matrix, in call order."""
        out = []
        for gi, g in enumerate(self.groups):
            for j in range(g.count):
                out.append((gi, j, g.rows, g.cols))
        return out

    def is_idle(self, gi: int, j: int) -> bool:
        g = self.groups[gi]
        if g.idle_every <= 0:
            return False
        return (j // g.idle_group_size) % g.idle_every == 0

    @property
    def num_matrices(self) -> int:
        return sum(g.count for g in self.groups)


def _moe_bank() -> Tuple[Group, ...]:
    # 256 experts, each owning one 2048x1408 and one 1408x2048 matrix; expert e
    # is idle (gradient x 0) iff e % 10 == 0, i.e. 26 of 256 experts.
    return (Group(2048, 1408, 256, "expert_w_in", idle_every=10),
            Group(1408, 2048, 256, "expert_w_out", idle_every=10))


WORKLOADS = {
    "tiny_fp32": Workload(
        key="tiny_fp32", config_id=1,
        description="tiny fp32 group: 4 matrices 64x128, grads and momentum N(0,1) from seed 0",
        groups=(Group(64, 128, 4, "tiny"),),
        dtype="f32", grad_dist="normal", grad_scale=1.0,
        momentum_init="normal", params_init="zero", seed0_bulk=True),
    "attn_2048": Workload(
        key="attn_2048", config_id=2,
        description="dense attention projections: 32 x 2048x2048 bf16, grads N(0,1e-3)",
        groups=(Group(2048, 2048, 32, "attn_proj"),),
        dtype="bf16", grad_dist="normal", grad_scale=1e-3,
        momentum_init="zero", params_init="zero"),
    "mlp_4096x14336": Workload(
        key="mlp_4096x14336", config_id=3,
        description="dense MLP: 32 x 4096x14336 up/gate + 32 x 14336x4096 down bf16",
        groups=(Group(4096, 14336, 32, "mlp_up_gate"), Group(14336, 4096, 32, "mlp_down")),
        dtype="bf16", grad_dist="normal", grad_scale=1e-3,
        momentum_init="zero", params_init="zero"),
    "moe_bank_2048x1408": Workload(
        key="moe_bank_2048x1408", config_id=4,
        description="MoE expert bank: 256 x 2048x1408 + 256 x 1408x2048 bf16, 10% idle experts",
        groups=_moe_bank(),
        dtype="bf16", grad_dist="normal", grad_scale=1e-3,
        momentum_init="zero", params_init="zero"),
    "moe_stack_7168": Workload(
        key="moe_stack_7168", config_id=5,
        description="mixed MoE layer stack: 4 x 7168x7168, 2 x 7168x18432, 128 x 7168x2048 bf16, t3 grads",
        groups=(Group(7168, 7168, 4, "attn"), Group(7168, 18432, 2, "dense_mlp"),
                Group(7168, 2048, 128, "experts")),
        dtype="bf16", grad_dist="student_t3", grad_scale=1e-3,
        momentum_init="zero", params_init="zero"),
}


# --------------------------------------------------------------------------
# bf16 storage helpers (value encoding only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Stored:
    """One stored tensor: `values` as float32 (exactly what is stored) and,
    for bf16, the raw `bits` (uint16) that go to the device."""
    values: np.ndarray
    bits: Optional[np.ndarray] = None

    def as_f64(self) -> np.ndarray:
        return self.values.astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> Stored:
    if dtype == "f32":
        return Stored(np.ascontiguousarray(x32, dtype=np.float32))
    bits = f32_to_bf16_bits(x32)
    return Stored(bf16_bits_to_f32(bits), bits)


def _rng(w: Workload, gi: int, j: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.config_id, gi, j, tensor])))


def _draw(rng: np.random.Generator, shape, dist: str, scale: float) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        return x
    if dist == "student_t3":
        return (rng.standard_t(3.0, size=shape) * scale).astype(np.float32)
    raise ValueError(dist)


def _bulk_seed0(w: Workload):
    g = w.groups[0]
    rng = np.random.default_rng(0)
    grads = rng.standard_normal((g.count, g.rows, g.cols)).astype(np.float32)
    mom = rng.standard_normal((g.count, g.rows, g.cols)).astype(np.float32)
    return grads, mom


def grad(w: Workload, gi: int, j: int) -> Stored:
    g = w.groups[gi]
    if w.seed0_bulk:
        return _store(_bulk_seed0(w)[0][j], w.dtype)
    x = _draw(_rng(w, gi, j, GRAD), (g.rows, g.cols), w.grad_dist, w.grad_scale)
    if w.is_idle(gi, j):
        x = np.zeros_like(x)
    return _store(x, w.dtype)


def momentum(w: Workload, gi: int, j: int) -> np.ndarray:
    """Momentum buffers are always float32."""
    g = w.groups[gi]
    if w.momentum_init == "zero":
        return np.zeros((g.rows, g.cols), np.float32)
    if w.seed0_bulk:
        return np.ascontiguousarray(_bulk_seed0(w)[1][j])
    return _rng(w, gi, j, MOMENTUM).standard_normal((g.rows, g.cols), dtype=np.float32)


def params(w: Workload, gi: int, j: int) -> Stored:
    g = w.groups[gi]
    if w.params_init == "zero":
        return _store(np.zeros((g.rows, g.cols), np.float32), w.dtype)
    return _store(_rng(w, gi, j, PARAMS).standard_normal((g.rows, g.cols), dtype=np.float32) * np.float32(0.02), w.dtype)


def parallel_map(fn, items: Sequence, threads: Optional[int] = None) -> list:
    """Map over items with a thread pool (numpy's generators release the GIL)."""
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


# --------------------------------------------------------------------------
# Ad-hoc cases (parity tests at small and ragged sizes)
# --------------------------------------------------------------------------

def random_case(seed: int, shapes: Sequence[Tuple[int, int]], dtype: str, *,
                grad_scale: float = 1e-3, momentum_init: str = "normal",
                params_init: str = "normal", zero: Sequence[int] = ()) -> List[dict]:
    """Seeded inputs for arbitrary shapes: a list of dicts with keys
    grad (Stored), momentum (float32 array), params (Stored)."""
    out = []
    for i, (r, c) in enumerate(shapes):
        base = [1000 + seed, i]
        rg = np.random.Generator(np.random.PCG64(np.random.SeedSequence(base + [GRAD])))
        g = rg.standard_normal((r, c), dtype=np.float32) * np.float32(grad_scale)
        if i in zero:
            g = np.zeros_like(g)
        if momentum_init == "zero":
            m = np.zeros((r, c), np.float32)
        else:
            rm = np.random.Generator(np.random.PCG64(np.random.SeedSequence(base + [MOMENTUM])))
            m = rm.standard_normal((r, c), dtype=np.float32) * np.float32(grad_scale)
        if params_init == "zero":
            p = np.zeros((r, c), np.float32)
        else:
            rp = np.random.Generator(np.random.PCG64(np.random.SeedSequence(base + [PARAMS])))
            p = rp.standard_normal((r, c), dtype=np.float32) * np.float32(0.02)
        out.append(dict(grad=_store(g, dtype), momentum=m, params=_store(p, dtype)))
    return out
