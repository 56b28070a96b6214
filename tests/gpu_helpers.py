"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its binding, run the oracle on the same stored values,
and compare."""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

import workloads

BF16_TOL = 2e-2   # relative Frobenius error of the update, bf16 path
F32_TOL = 1e-4    # relative Frobenius error of the update, float32 path
MOM_TOL = 1e-6    # relative Frobenius error of the momentum buffer


def torch_mod():
    import torch
    return torch


def to_device(st: workloads.Stored, dtype: str):
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(st.bits.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(st.values, np.float32))
    return t.to("cuda")


def from_device(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    d = float(np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64)))
    if nb == 0.0:
        return 0.0 if d == 0.0 else math.inf
    return d / nb


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def upload_case(case: List[dict], dtype: str):
    """Device tensors (params, grads, momentum) for a random_case list."""
    torch = torch_mod()
    P = [to_device(c["params"], dtype) for c in case]
    G = [to_device(c["grad"], dtype) for c in case]
    M = [torch.from_numpy(c["momentum"].copy()).to("cuda") for c in case]
    return P, G, M


def oracle_case(case: List[dict], lr: float, beta: float, ns_steps: int, **opts):
    import oracle
    out = []
    for c in case:
        out.append(oracle.muon_matrix_step(c["params"].as_f64(), c["grad"].as_f64(),
                                           c["momentum"].astype(np.float64), lr, beta, ns_steps, **opts))
    return out


def check_update(p0: np.ndarray, p1_gpu: np.ndarray, p1_ref: np.ndarray, dtype: str, tol: float) -> float:
    """Relative error of the applied update, allowing the final rounding of
    p to `dtype` (half an ulp per element) on top of `tol`."""
    upd_ref = p1_ref - p0
    nref = float(np.linalg.norm(upd_ref))
    err = float(np.linalg.norm(p1_gpu - p1_ref))
    if dtype == "bf16":
        err = max(0.0, err - 0.5 * float(np.linalg.norm(bf16_ulp(p1_ref))))
    else:
        err = max(0.0, err - 0.5 * float(np.linalg.norm(np.spacing(np.abs(p1_ref).astype(np.float32)))))
    if nref == 0.0:
        return 0.0 if err == 0.0 else math.inf
    return err / nref
