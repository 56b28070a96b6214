"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (one muon_step over the whole workload): every matrix runs on the
GPU, a sample of matrices is checked against the fp64 oracle, and every
matrix is checked for finite output and exact zero updates where the
gradient is zero.

Oracle samples (indices in call order):
  * attention 2048^2: all 32;
  * MoE bank: 24 of 512 -- 4 idle experts (2 of each orientation) and 20
    live matrices spread over both orientations and all three batches;
  * MLP: 2 up/gate (4096 x 14336) and 2 transposed down (14336 x 4096);
  * mixed stack: 1 attention (7168^2), 1 dense MLP (7168 x 18432) and 8
    experts (7168 x 2048, transposed).
The other dense-MLP matrix of the stack is also checked by a property that
holds at any size: for a wide G with update O = U phi(S) V^T, G O^T =
U S phi(S) U^T is symmetric positive semidefinite, and ||O||_2 <= max phi
< 1.21."""
import time

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import BF16_TOL, MOM_TOL, check_momentum, check_update, from_device

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


FORMS = ("square", "direct", "folded")   # the default form of the NS step first


def _run_and_check(w, samples, prop_groups=()):
    """Runs the whole workload once per polynomial form (params and momentum
    reset to zero in between), keeps the sampled matrices' results, then
    compares each sample of each form with one oracle computation."""
    import torch
    import newton_schulz_10_amd as nsa
    P, G, M = _upload_workload(w)
    mats = w.matrices()
    kept = {}
    for form in FORMS:
        for t in P + M:
            t.zero_()
        t0 = time.time()
        nsa.muon_step(list(zip(P, G, M)), w.lr, w.beta, w.ns_steps, poly_form=form)
        torch.cuda.synchronize()
        _log(f"{w.key}: GPU step ({form} form) {time.time() - t0:.2f}s")
        # every matrix: finite; idle experts: exact no-op
        for k, (gi, j, r, c) in enumerate(mats):
            if w.is_idle(gi, j):
                assert torch.count_nonzero(P[k]) == 0 and torch.count_nonzero(M[k]) == 0, k
            else:
                assert torch.isfinite(P[k].float()).all(), k
        kept[form] = {k: (from_device(P[k]), from_device(M[k])) for k in samples}
    worst = 0.0
    for k in samples:
        gi, j, r, c = mats[k]
        t1 = time.time()
        g = workloads.grad(w, gi, j).as_f64()
        p0 = np.zeros((r, c))
        rp, rb, _ = oracle.muon_matrix_step(p0, g, np.zeros((r, c)), w.lr, w.beta, w.ns_steps)
        for form in FORMS:
            p1, m1 = kept[form][k]
            e = check_update(p0, p1, rp, "bf16", BF16_TOL, label=f"{form} #{k}")
            em = check_momentum(m1, rb, label=f"#{k}")
            _log(f"{w.key}: matrix {k} ({r}x{c}) {form} form rel err {e:.3e} momentum {em:.1e} "
                 f"oracle {time.time() - t1:.1f}s")
            worst = max(worst, e)
            assert e <= BF16_TOL and em <= MOM_TOL, (k, form, e, em)
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
    _run_and_check(workloads.WORKLOADS["attn_2048"], samples=list(range(32)))


MOE_IDLE = [0, 130, 326, 506]   # experts 0, 130 (2048 x 1408) and 70, 250 (1408 x 2048)
MOE_LIVE = [1, 37, 77, 101, 137, 169, 171, 203, 255, 257, 289, 311, 341, 342, 377, 401, 433, 469, 500, 511]


def test_moe_bank_full():
    w = workloads.WORKLOADS["moe_bank_2048x1408"]
    mats = w.matrices()
    assert all(w.is_idle(*mats[k][:2]) for k in MOE_IDLE)
    assert not any(w.is_idle(*mats[k][:2]) for k in MOE_LIVE)
    _run_and_check(w, samples=MOE_IDLE + MOE_LIVE)


def test_mlp_4096x14336_full():
    # 0, 17: up/gate 4096 x 14336; 32, 63: down 14336 x 4096 (transposed)
    _run_and_check(workloads.WORKLOADS["mlp_4096x14336"], samples=[0, 17, 32, 63])


def test_moe_stack_7168_full():
    w = workloads.WORKLOADS["moe_stack_7168"]
    # order: 4 attention, 2 dense MLP, 128 experts
    _run_and_check(w, samples=[1, 5, 6, 20, 45, 70, 95, 110, 120, 133], prop_groups=[4])
