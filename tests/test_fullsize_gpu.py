"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (one muon_step over the whole workload): every matrix runs on the
GPU, a sample of matrices is checked against the fp64 oracle, and every
matrix is checked for finite output and exact zero updates where the
gradient is zero.

Samples: attention 2048^2: 4 of 32; MoE bank: 8 of 512 (idle experts and
both orientations included); MLP: one up/gate and one (transposed) down
matrix; mixed stack: one 7168^2 attention matrix and two 7168x2048
experts. The two 7168x18432 MLP matrices are checked by a property that
holds at any size: for a wide G with update O = U phi(S) V^T, G O^T =
U S phi(S) U^T is symmetric positive semidefinite, and ||O||_2 <= max phi
< 1.21."""
import time

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import BF16_TOL, MOM_TOL, check_update, from_device, rel_fro, to_device

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def _upload_workload(w):
    import torch
    mats = w.matrices()

    def gen(item):
        gi, j, r, c = item
        return workloads.grad(w, gi, j).bits

    t0 = time.time()
    P, G, M = [], [], []
    chunk = 64
    for s in range(0, len(mats), chunk):
        bits = workloads.parallel_map(gen, mats[s:s + chunk])
        for (gi, j, r, c), b in zip(mats[s:s + chunk], bits):
            G.append(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda"))
            P.append(torch.zeros((r, c), dtype=torch.bfloat16, device="cuda"))
            M.append(torch.zeros((r, c), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    _log(f"{w.key}: uploaded {len(mats)} matrices in {time.time() - t0:.1f}s")
    return P, G, M


def _run_and_check(w, samples, prop_groups=()):
    import torch
    import newton_schulz_10_amd as nsa
    P, G, M = _upload_workload(w)
    t0 = time.time()
    nsa.muon_step(list(zip(P, G, M)), w.lr, w.beta, w.ns_steps)
    torch.cuda.synchronize()
    _log(f"{w.key}: GPU step {time.time() - t0:.2f}s")
    mats = w.matrices()
    # every matrix: finite; idle experts: exact no-op
    for k, (gi, j, r, c) in enumerate(mats):
        if w.is_idle(gi, j):
            assert torch.count_nonzero(P[k]) == 0 and torch.count_nonzero(M[k]) == 0, k
        else:
            assert torch.isfinite(P[k].float()).all(), k
    worst = 0.0
    for k in samples:
        gi, j, r, c = mats[k]
        t1 = time.time()
        g = workloads.grad(w, gi, j).as_f64()
        p0 = np.zeros((r, c))
        rp, rb, _ = oracle.muon_matrix_step(p0, g, np.zeros((r, c)), w.lr, w.beta, w.ns_steps)
        e = check_update(p0, from_device(P[k]), rp, "bf16", BF16_TOL)
        em = rel_fro(from_device(M[k]), rb.astype(np.float32))
        _log(f"{w.key}: matrix {k} ({r}x{c}) rel err {e:.3e} momentum {em:.1e} oracle {time.time() - t1:.1f}s")
        worst = max(worst, e)
        assert e <= BF16_TOL and em <= MOM_TOL, (k, e, em)
    for k in prop_groups:
        gi, j, r, c = mats[k]
        gt = G[k].float()
        o = -P[k].float() / (w.lr * 0.2 * max(r, c) ** 0.5)   # p0 = 0: p1 = -lr*scale*O
        if r > c:
            gt, o = gt.t(), o.t()
        s = gt @ o.t()
        asym = (torch.linalg.norm(s - s.t()) / torch.linalg.norm(s)).item()
        smax = torch.linalg.matrix_norm(o, ord=2).item()
        ev_min = torch.linalg.eigvalsh(0.5 * (s + s.t()).double()).min().item() / torch.linalg.matrix_norm(s.double(), ord=2).item()
        _log(f"{w.key}: matrix {k} ({r}x{c}) G O^T asymmetry {asym:.2e}, ||O||_2 {smax:.3f}, min eig/||.|| {ev_min:.2e}")
        assert asym <= BF16_TOL and smax <= 1.25 and ev_min >= -BF16_TOL
    return worst


def test_attention_2048_full():
    _run_and_check(workloads.WORKLOADS["attn_2048"], samples=[0, 9, 22, 31])


def test_moe_bank_full():
    # 0 and 256 are idle experts (both orientations); 1, 255, 257, 511 live.
    _run_and_check(workloads.WORKLOADS["moe_bank_2048x1408"], samples=[0, 1, 137, 255, 256, 257, 390, 511])


def test_mlp_4096x14336_full():
    _run_and_check(workloads.WORKLOADS["mlp_4096x14336"], samples=[5, 40])


def test_moe_stack_7168_full():
    w = workloads.WORKLOADS["moe_stack_7168"]
    # order: 4 attention, 2 dense MLP, 128 experts
    _run_and_check(w, samples=[1, 6, 133], prop_groups=[4, 5])
