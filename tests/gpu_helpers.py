"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its binding, run the oracle on the same stored values,
compare, and keep a record of every comparison.

Error measures of an update (p0 -> p1) against the oracle's fp64 p1_ref:
  * err: ||p1_gpu - rnd(p1_ref)||_F / ||p1_ref - p0||_F, where rnd rounds to
    the stored type (bf16 round-to-nearest-even, or float32): the GPU's p1
    is stored in that type, so a bit-exact update scores 0. When p0 is not
    zero, the rounding of p1 = alpha*p0 - gamma*O to the stored type is
    quantisation of |p1|, not of the update, and half an ulp of p1_ref per
    element is allowed on top; with p0 = 0 (every workload) there is no
    allowance.
  * raw: ||p1_gpu - p1_ref||_F / ||p1_ref - p0||_F (for the record).
  * tile: the largest err taken over 256 x 256 tiles of the matrix (each
    tile's own reference norm), so that one wrong block cannot hide inside
    a whole-matrix norm. Bound: TILE_FACTOR times the matrix bound.
Every comparison is appended to RECORDS; tests/conftest.py prints a summary
of them at the end of the session.
"""
from __future__ import annotations

import math
import os
from typing import List, Sequence

import numpy as np

import workloads

BF16_TOL = 2e-2   # relative Frobenius error of the update, bf16 path
F32_TOL = 1e-4    # relative Frobenius error of the update, float32 path
MOM_TOL = 1e-6    # relative Frobenius error of the momentum buffer
TILE = 256        # edge of the tiles of the per-tile bound
TILE_FACTOR = 2.5  # per-tile bound = TILE_FACTOR x the matrix bound

RECORDS: List[dict] = []


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


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """x rounded to the stored type (bf16: nearest even, via float32)."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x32)).astype(np.float64)
    return x32.astype(np.float64)


def _ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_ulp(x)
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)


def _current_test() -> str:
    t = os.environ.get("PYTEST_CURRENT_TEST", "?")
    return t.rsplit(" (", 1)[0].split("::", 1)[-1]


def _record(kind: str, label: str, shape, err: float, raw: float, tile: float, tol: float, **extra) -> dict:
    r = dict(test=_current_test(), kind=kind, label=label, shape=tuple(int(s) for s in shape), err=err,
             raw=raw, tile=tile, tol=tol, **extra)
    RECORDS.append(r)
    return r


def compare(got: np.ndarray, ref: np.ndarray, base: np.ndarray, dtype: str) -> tuple:
    """(err, raw, tile) of got against ref, relative to ref - base (see the
    module docstring)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    base = np.asarray(base, np.float64)
    upd = ref - base
    d = got - round_to(ref, dtype)
    allow = np.any(base != 0)
    ulp2 = (0.5 * _ulp(ref, dtype)) ** 2 if allow else None

    def measure(sl):
        n = float(np.linalg.norm(upd[sl]))
        e = float(np.linalg.norm(d[sl]))
        if allow:
            e = max(0.0, e - math.sqrt(float(np.sum(ulp2[sl]))))
        if n == 0.0:
            return 0.0 if e == 0.0 else math.inf
        return e / n

    err = measure((slice(None), slice(None)))
    nraw = float(np.linalg.norm(upd))
    draw = float(np.linalg.norm(got - ref))
    raw = (0.0 if draw == 0.0 else math.inf) if nraw == 0.0 else draw / nraw
    tile = 0.0
    rows, cols = got.shape
    for i in range(0, rows, TILE):
        for j in range(0, cols, TILE):
            tile = max(tile, measure((slice(i, i + TILE), slice(j, j + TILE))))
    return err, raw, tile


def check_update(p0: np.ndarray, p1_gpu: np.ndarray, p1_ref: np.ndarray, dtype: str, tol: float,
                 label: str = "") -> float:
    """Error of the applied update (module docstring); records it, checks
    the per-tile bound, and returns the whole-matrix error for the caller's
    own bound."""
    err, raw, tile = compare(p1_gpu, p1_ref, p0, dtype)
    r = _record("update", label, np.shape(p1_gpu), err, raw, tile, tol)
    assert tile <= TILE_FACTOR * tol, r
    return err


def check_output(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, tol: float, label: str = "") -> float:
    """Error of an orthogonalized output O against the oracle's (no base)."""
    err, raw, tile = compare(o_gpu, o_ref, np.zeros_like(np.asarray(o_ref)), dtype)
    r = _record("output", label, np.shape(o_gpu), err, raw, tile, tol)
    assert tile <= TILE_FACTOR * tol, r
    return err


def check_momentum(m_gpu: np.ndarray, m_ref: np.ndarray, label: str = "") -> float:
    e = rel_fro(m_gpu, np.asarray(m_ref, np.float32))
    RECORDS.append(dict(test=_current_test(), kind="momentum", label=label, shape=tuple(np.shape(m_gpu)),
                        err=e, raw=e, tile=e, tol=MOM_TOL))
    return e


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


FORM_NAMES = ("square", "direct", "folded")


def summary_lines(records: Sequence[dict]) -> List[str]:
    """One line per test (per test and polynomial form, where a comparison's
    label names the form): comparisons, worst err / raw / tile (update and
    output comparisons) and the worst momentum error."""
    by_test = {}
    for r in records:
        form = r["label"].split(" ", 1)[0] if r["label"] else ""
        key = f"{r['test']} [{form}]" if form in FORM_NAMES and r["kind"] != "momentum" else r["test"]
        by_test.setdefault(key, []).append(r)
    lines = []
    for t, rs in by_test.items():
        cmp_ = [r for r in rs if r["kind"] != "momentum"]
        mom = [r["err"] for r in rs if r["kind"] == "momentum"]
        s = f"{t}: {len(cmp_)} compared"
        if cmp_:
            w = max(cmp_, key=lambda r: r["err"] / r["tol"])
            s += (f", worst err {w['err']:.3e} (raw {w['raw']:.3e}, tile {max(r['tile'] for r in cmp_):.3e}, "
                  f"bar {w['tol']:.0e}) at {w['shape'][0]}x{w['shape'][1]}{' ' + w['label'] if w['label'] else ''}")
        if mom:
            s += f"; momentum {max(mom):.1e}"
        lines.append(s)
    return lines
