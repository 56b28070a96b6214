"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded, stored inputs, plus bitwise invariants of the batched
design. Tolerances: relative Frobenius error of the update <= 1e-4 on the
float32 path and <= 2e-2 on the bf16 path; momentum <= 1e-6."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import (BF16_TOL, F32_TOL, MOM_TOL, check_momentum, check_output, check_update, from_device,
                         oracle_case, rel_fro, to_device, upload_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsa():
    import torch
    import newton_schulz_10_amd as m
    m.load()
    torch.cuda.init()
    return m


def _print(*a):
    print(*a, flush=True)


def run_case(nsa, case, dtype, lr=0.02, beta=0.95, ns_steps=5, **opts):
    import torch
    P, G, M = upload_case(case, dtype)
    nsa.muon_step(list(zip(P, G, M)), lr, beta, ns_steps, **opts)
    torch.cuda.synchronize()
    return [from_device(p) for p in P], [from_device(m) for m in M]


def assert_parity(case, dtype, p1, m1, ref, tol):
    worst = 0.0
    for i, (c, (rp, rb, ro)) in enumerate(zip(case, ref)):
        p0 = c["params"].as_f64()
        e = check_update(p0, p1[i], rp, dtype, tol, label=f"#{i}")
        em = check_momentum(m1[i], rb, label=f"#{i}")
        worst = max(worst, e)
        assert e <= tol, (i, p0.shape, e)
        assert em <= MOM_TOL, (i, p0.shape, em)
        if not np.any(rp - p0):
            assert np.array_equal(p1[i], p0), i  # zero update must be exact
    return worst


# ---- tiny float32 configuration --------------------------------------------

def test_tiny_fp32_config(nsa):
    w = workloads.WORKLOADS["tiny_fp32"]
    case = [dict(grad=workloads.grad(w, gi, j), momentum=workloads.momentum(w, gi, j),
                 params=workloads.params(w, gi, j)) for gi, j, _, _ in w.matrices()]
    p1, m1 = run_case(nsa, case, "f32", w.lr, w.beta, w.ns_steps)
    ref = oracle_case(case, w.lr, w.beta, w.ns_steps)
    worst = assert_parity(case, "f32", p1, m1, ref, F32_TOL)
    _print("tiny_fp32 worst rel err", worst)


def test_tiny_fp32_closed_form_3x5(nsa):
    import torch
    g = np.random.default_rng(0).standard_normal((3, 5)).astype(np.float32)
    x = torch.from_numpy(g).cuda()
    out = torch.empty_like(x)
    nsa.muon_orthogonalize([x], [out], 5)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(g.astype(np.float64))
    assert check_output(from_device(out), ref, "f32", F32_TOL, label="3x5") <= F32_TOL


# ---- small and ragged shapes, several tiles -------------------------------

RAGGED = [(200, 333), (333, 200), (128, 128), (256, 640), (1, 1), (1, 7), (7, 1), (64, 128),
          (130, 300), (129, 1000), (300, 130), (384, 256),
          # short side padded to an odd multiple of 128 (half tile row), and
          # an odd number of 256-column tiles
          (300, 520), (600, 700), (700, 600), (384, 896)]


@pytest.mark.parametrize("dtype,tol", [("bf16", BF16_TOL), ("f32", F32_TOL)])
def test_ragged_shapes(nsa, dtype, tol):
    case = workloads.random_case(1, RAGGED, dtype, params_init="zero")
    p1, m1 = run_case(nsa, case, dtype)
    ref = oracle_case(case, 0.02, 0.95, 5)
    worst = assert_parity(case, dtype, p1, m1, ref, tol)
    _print(dtype, "ragged worst rel err", worst)


@pytest.mark.parametrize("dtype,tol", [("bf16", BF16_TOL), ("f32", F32_TOL)])
def test_random_shapes(nsa, dtype, tol):
    # A seeded sweep of shapes in [1, 900]^2 (both orientations, every
    # padding remainder and tile geometry that small sizes reach), one call.
    rng = np.random.default_rng(2024)
    shapes = [(int(r), int(c)) for r, c in rng.integers(1, 901, size=(20, 2))]
    case = workloads.random_case(17, shapes, dtype, params_init="zero")
    _print("random shapes", dtype, shapes)
    p1, m1 = run_case(nsa, case, dtype)
    ref = oracle_case(case, 0.02, 0.95, 5)
    worst = assert_parity(case, dtype, p1, m1, ref, tol)
    _print(dtype, "random shapes worst rel err", worst)


def test_banded_tile_orders(nsa):
    # More than 8 tile rows and columns: Gram/Poly tiles go in bands of 4
    # tile rows and Update tiles in groups of 4 rows, column-major inside
    # (2304 = 9 tile rows; 2432 = 9.5, with the half row of wide tiles;
    # 2560 = 10 tile columns).
    shapes = [(2304, 2560), (2560, 2432)]
    case = workloads.random_case(16, shapes, "bf16", params_init="zero")
    _print("banded tile orders", shapes)
    p1, m1 = run_case(nsa, case, "bf16")
    ref = oracle_case(case, 0.02, 0.95, 5)
    worst = assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)
    _print("banded tile orders worst rel err", worst)


def test_fp32_nonzero_params_and_options(nsa):
    shapes = [(96, 160), (160, 96), (64, 64)]
    case = workloads.random_case(2, shapes, "f32")
    opts = dict(weight_decay=0.1, scale_rule="original", momentum_form="sgd")
    p1, m1 = run_case(nsa, case, "f32", 0.05, 0.9, 5, **opts)
    ref = oracle_case(case, 0.05, 0.9, 5, weight_decay=0.1, scale_rule="original", momentum_form="sgd")
    assert_parity(case, "f32", p1, m1, ref, F32_TOL)
    p1, m1 = run_case(nsa, case, "f32", 0.05, 0.9, 3, nesterov=False, scale_rule="none")
    ref = oracle_case(case, 0.05, 0.9, 3, nesterov=False, scale_rule="none")
    assert_parity(case, "f32", p1, m1, ref, F32_TOL)


def test_bf16_nonzero_params_weight_decay(nsa):
    case = workloads.random_case(3, [(256, 384), (384, 256)], "bf16")
    p1, m1 = run_case(nsa, case, "bf16", 0.02, 0.95, 5, weight_decay=0.1)
    ref = oracle_case(case, 0.02, 0.95, 5, weight_decay=0.1)
    assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)


def test_bf16_fused_apply_orientation_scale(nsa):
    # bf16 shapes with rows and columns multiples of 8 take the apply fused
    # into the last Update GEMM. scale_rule "original" (sqrt(max(1, rows/cols)))
    # differs between a matrix and its transpose, so wide and tall members
    # must each get their own factor; nonzero params and weight decay
    # exercise p' = alpha*p - gamma*O. The 300x520 member (rows not a
    # multiple of 8) takes the separate apply pass in the same call.
    case = workloads.random_case(15, [(256, 384), (384, 256), (128, 640), (640, 128), (300, 520)], "bf16")
    p1, m1 = run_case(nsa, case, "bf16", 0.02, 0.95, 5, weight_decay=0.05, scale_rule="original")
    ref = oracle_case(case, 0.02, 0.95, 5, weight_decay=0.05, scale_rule="original")
    assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)


def test_coefficient_table(nsa):
    table = [(3.0, -3.2, 1.2), (3.4445, -4.775, 2.0315), (2.9, -3.0, 1.1), (3.4, -4.7, 2.0), (1.875, -1.25, 0.375)]
    for dtype, tol in (("f32", F32_TOL), ("bf16", BF16_TOL)):
        case = workloads.random_case(4, [(192, 320), (320, 192)], dtype, params_init="zero")
        p1, m1 = run_case(nsa, case, dtype, coeffs=table)
        ref = oracle_case(case, 0.02, 0.95, 5, coeffs=table)
        assert_parity(case, dtype, p1, m1, ref, tol)


def test_coefficient_table_with_cubic_steps(nsa):
    # c = 0 in two steps: the cubic Newton-Schulz step X <- 1.5 X - 0.5 X X^T X.
    # The bf16 path completes a I + b A + c A^2 to a square only when c != 0;
    # these steps take the other form (b A + a I with the A tile).
    table = [(3.4445, -4.775, 2.0315), (1.5, -0.5, 0.0), (3.4445, -4.775, 2.0315), (1.5, -0.5, 0.0),
             (3.4445, -4.775, 2.0315)]
    for dtype, tol in (("f32", F32_TOL), ("bf16", BF16_TOL)):
        case = workloads.random_case(14, [(192, 320), (320, 192), (300, 520)], dtype, params_init="zero")
        p1, m1 = run_case(nsa, case, dtype, coeffs=table)
        ref = oracle_case(case, 0.02, 0.95, 5, coeffs=table)
        assert_parity(case, dtype, p1, m1, ref, tol)


@pytest.mark.parametrize("steps", [0, 1, 2])
def test_few_ns_steps(nsa, steps):
    for dtype, tol in (("f32", F32_TOL), ("bf16", BF16_TOL)):
        case = workloads.random_case(5, [(128, 256), (100, 60)], dtype, params_init="zero")
        p1, m1 = run_case(nsa, case, dtype, ns_steps=steps)
        ref = oracle_case(case, 0.02, 0.95, steps)
        assert_parity(case, dtype, p1, m1, ref, tol)


def test_orthogonalize_entry(nsa):
    import torch
    rng = np.random.default_rng(6)
    for dtype, tol in (("f32", F32_TOL), ("bf16", BF16_TOL)):
        st = [workloads._store(rng.standard_normal((144, 272)).astype(np.float32) * 1e-3, dtype) for _ in range(3)]
        ins = [to_device(s, dtype) for s in st]
        outs = [torch.empty_like(x) for x in ins]
        nsa.muon_orthogonalize(ins, outs, 5)
        # in place as well
        nsa.muon_orthogonalize([ins[2]], [ins[2]], 5)
        torch.cuda.synchronize()
        for k, s in enumerate(st):
            ref = oracle.newton_schulz(s.as_f64())
            assert check_output(from_device(outs[k]), ref, dtype, tol, label=f"#{k}") <= tol
        assert np.array_equal(from_device(ins[2]), from_device(outs[2]))


def test_orthogonalize_expert_shapes_and_zero(nsa):
    # muon_orthogonalize at the expert-bank shape in both orientations (the
    # output is written by the last Update's fused apply: along rows for the
    # wide member, through transposing gathers for the tall one) with an
    # all-zero member beside the tall one (skipped on the device, its output
    # must be exactly zero), and a tall shape that takes the separate apply
    # pass (300 x 130). Outputs start as NaN so every element is checked.
    import torch
    rng = np.random.default_rng(7)
    for shape, zero in (((2048, 1408), True), ((1408, 2048), False), ((300, 130), False)):
        st = [workloads._store(rng.standard_normal(shape).astype(np.float32) * 1e-3, "bf16")]
        if zero:
            st.append(workloads._store(np.zeros(shape, np.float32), "bf16"))
        ins = [to_device(s, "bf16") for s in st]
        outs = [torch.full_like(x, float("nan")) for x in ins]
        nsa.muon_orthogonalize(ins, outs, 5)
        torch.cuda.synchronize()
        ref = oracle.newton_schulz(st[0].as_f64())
        assert check_output(from_device(outs[0]), ref, "bf16", BF16_TOL, label=f"{shape}") <= BF16_TOL
        if zero:
            o = from_device(outs[1])
            assert not np.any(np.isnan(o)) and not np.any(o)


# ---- bitwise invariants of the batched design ------------------------------

def _bits(ts):
    return [t.detach().cpu().view(-1).view(__import__("torch").int16 if t.element_size() == 2 else __import__("torch").int32).numpy().copy()
            for t in ts]


def test_batch_partition_invariance_and_determinism(nsa):
    import torch
    shapes = [(256, 384)] * 6 + [(384, 256)] * 3
    case = workloads.random_case(7, shapes, "bf16")
    outs = []
    for cap in (0, 256 * 384, 3 * 256 * 384, 0):
        P, G, M = upload_case(case, "bf16")
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5, batch_cap_elems=cap)
        torch.cuda.synchronize()
        outs.append(_bits(P) + _bits(M))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_repeat_calls_bitwise_with_claimed_tiles(nsa):
    # 40 matrices of 1024 x 1536: 400 Gram tiles (4 diagonal per matrix) over
    # at most 256 workgroups, so tiles are claimed from the per-XCD counters;
    # repeated calls, and a split into other batches in between, must give
    # the same bits (every tile computed once, counters zeroed per launch).
    import torch
    shapes = [(1024, 1536)] * 24 + [(1536, 1024)] * 16
    case = workloads.random_case(17, shapes, "bf16")
    outs = []
    for cap in (0, 7 * 1024 * 1536, 0):
        P, G, M = upload_case(case, "bf16")
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5, batch_cap_elems=cap)
        torch.cuda.synchronize()
        outs.append(_bits(P))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    # and the result is the Muon update: spot-check two matrices against
    # the oracle
    sub = [case[0], case[30]]
    ref = oracle_case(sub, 0.02, 0.95, 5)
    P, G, M = upload_case(case, "bf16")
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for c, i, (rp, _, _) in zip(sub, (0, 30), ref):
        e = check_update(c["params"].as_f64(), from_device(P[i]), rp, "bf16", BF16_TOL, label=f"#{i}")
        assert e <= BF16_TOL, (i, e)


def test_mixed_call_equals_per_group_calls(nsa):
    import torch
    shapes = [(256, 640), (128, 128), (640, 256), (128, 128), (200, 100)]
    case = workloads.random_case(8, shapes, "bf16")
    P, G, M = upload_case(case, "bf16")
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    P2, G2, M2 = upload_case(case, "bf16")
    for idx in ([0, 2], [1, 3], [4]):
        nsa.muon_step([(P2[i], G2[i], M2[i]) for i in idx], 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for a, b in zip(_bits(P) + _bits(M), _bits(P2) + _bits(M2)):
        assert np.array_equal(a, b)


def test_tall_equals_transposed_wide_twin(nsa):
    import torch
    case = workloads.random_case(9, [(384, 256)], "bf16")
    P, G, M = upload_case(case, "bf16")
    Pt = [P[0].t().contiguous()]
    Gt = [G[0].t().contiguous()]
    Mt = [M[0].t().contiguous()]
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    nsa.muon_step(list(zip(Pt, Gt, Mt)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert torch.equal(P[0], Pt[0].t()) and torch.equal(M[0], Mt[0].t())


def test_group_step_entry_and_expert_bank(nsa):
    import torch
    # [E, M, N] bank: E independent matrices (never flattened).
    E, r, c = 6, 128, 192
    case = workloads.random_case(10, [(r, c)] * E, "bf16", params_init="zero")
    P, G, M = upload_case(case, "bf16")
    bankP, bankG, bankM = torch.stack(P), torch.stack(G), torch.stack(M)
    nsa.muon_group_step([bankP], [bankG], [bankM], 0.02, 0.95, 5)
    nsa.muon_group_step(P, G, M, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for e in range(E):
        assert torch.equal(bankP[e], P[e]) and torch.equal(bankM[e], M[e])
    ref = oracle_case(case, 0.02, 0.95, 5)
    assert_parity(case, "bf16", [from_device(p) for p in P], [from_device(m) for m in M], ref, BF16_TOL)


def test_a1b_tensor_is_one_matrix(nsa):
    # An [A, 1, B] tensor is one A x B matrix of the (A, B) group (section
    # 6.6, Figure 10(a)), not A matrices of 1 x B: its step is bitwise the
    # A x B tensor's, and matches the oracle. Wide and tall.
    import torch
    case = workloads.random_case(12, [(192, 320), (320, 192)], "bf16")
    P, G, M = upload_case(case, "bf16")
    P3, G3, M3 = ([t.clone().unsqueeze(1) for t in ts] for ts in (P, G, M))
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    nsa.muon_step(list(zip(P3, G3, M3)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for i in range(2):
        assert P3[i].shape == (P[i].shape[0], 1, P[i].shape[1])
        assert torch.equal(P3[i].squeeze(1), P[i]) and torch.equal(M3[i].squeeze(1), M[i]), i
    ref = oracle_case(case, 0.02, 0.95, 5)
    assert_parity(case, "bf16", [from_device(p) for p in P], [from_device(m) for m in M], ref, BF16_TOL)


def test_zero_and_nan_matrices(nsa):
    import torch
    case = workloads.random_case(11, [(128, 256)] * 3, "bf16", momentum_init="zero", zero=(1,))
    P, G, M = upload_case(case, "bf16")
    G[2].view(-1)[17] = float("nan")
    p_before = [p.clone() for p in P]
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert torch.equal(P[1], p_before[1])           # zero grad and momentum: exact no-op
    assert torch.count_nonzero(M[1]) == 0
    assert torch.isnan(P[2].float()).any()          # NaN propagates within its matrix
    assert torch.isfinite(P[0].float()).all()       # ... and nowhere else
    ref = oracle_case(case[:1], 0.02, 0.95, 5)
    assert check_update(case[0]["params"].as_f64(), from_device(P[0]), ref[0][0], "bf16", BF16_TOL) <= BF16_TOL


def test_zero_matrices_with_weight_decay(nsa):
    # Zero-gradient (idle) members skip the NS GEMMs on the bf16 path; their
    # update is still the decay p' = (1 - lr*wd) p, bitwise as the general
    # formula with O = 0 gives. Tall and wide members, a member whose shape
    # takes the separate apply pass (300 x 130), and live members alongside.
    shapes = [(256, 384), (384, 256), (256, 384), (384, 256), (300, 130), (130, 300)]
    case = workloads.random_case(16, shapes, "bf16", momentum_init="zero", zero=(0, 3, 4))
    p1, m1 = run_case(nsa, case, "bf16", 0.02, 0.95, 5, weight_decay=0.1)
    ref = oracle_case(case, 0.02, 0.95, 5, weight_decay=0.1)
    assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)
    alpha = np.float32(1.0 - float(np.float32(0.02)) * float(np.float32(0.1)))   # as the library forms it
    for i in (0, 3, 4):
        p0 = case[i]["params"].as_f64().astype(np.float32)
        want = workloads._store(p0 * alpha, "bf16").as_f64()
        assert np.array_equal(p1[i], want), i


def test_large_tall_members_stored_row_order(nsa):
    # Tall members with more 64x64 tiles than the workgroups resident on the
    # chip (2048) take the momentum and apply passes' tiles along the stored
    # rows. bf16: a live 4160 x 2048 member (2176 tiles) against the oracle,
    # and an idle 8192 x 4096 member whose decay runs in the separate apply
    # pass, checked exactly. float32: a live 4224 x 2112 member (2178 tiles),
    # whose update runs in the separate apply pass.
    case = workloads.random_case(31, [(4160, 2048), (8192, 4096)], "bf16", momentum_init="zero", zero=(1,))
    p1, m1 = run_case(nsa, case, "bf16", 0.02, 0.95, 5, weight_decay=0.1)
    ref = oracle_case(case[:1], 0.02, 0.95, 5, weight_decay=0.1)
    assert_parity(case[:1], "bf16", p1[:1], m1[:1], ref, BF16_TOL)
    alpha = np.float32(1.0 - float(np.float32(0.02)) * float(np.float32(0.1)))   # as the library forms it
    p0 = case[1]["params"].as_f64().astype(np.float32)
    assert np.array_equal(p1[1], workloads._store(p0 * alpha, "bf16").as_f64())
    assert not np.any(m1[1])
    case = workloads.random_case(32, [(4224, 2112)], "f32")
    p1, m1 = run_case(nsa, case, "f32", 0.02, 0.95, 5)
    ref = oracle_case(case, 0.02, 0.95, 5)
    assert_parity(case, "f32", p1, m1, ref, F32_TOL)


def test_maximum_dimension(nsa):
    # One side at the largest accepted dimension (2^20): an 8 x 2^20 member
    # (a Gram K loop of 32768 slabs, 2048 wide Update tiles) and its tall
    # twin (32768 momentum tiles, taken along the stored rows).
    case = workloads.random_case(33, [(8, 1 << 20), (1 << 20, 8)], "bf16", momentum_init="zero")
    p1, m1 = run_case(nsa, case, "bf16", 0.02, 0.95, 5)
    ref = oracle_case(case, 0.02, 0.95, 5)
    assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)


def test_non_default_stream(nsa):
    import torch
    case = workloads.random_case(12, [(256, 256)] * 2, "bf16")
    P, G, M = upload_case(case, "bf16")
    P2, G2, M2 = upload_case(case, "bf16")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    s.synchronize()
    nsa.muon_step(list(zip(P2, G2, M2)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(P, P2))


def test_call_does_not_synchronize_the_device(nsa):
    # A bounded spin kernel on one stream is still running when a call on
    # another stream has returned: the call only enqueues work (no device
    # or stream synchronisation), and its results are right once its own
    # stream is synchronised.
    import torch
    case = workloads.random_case(13, [(256, 384), (384, 256)], "bf16")
    P, G, M = upload_case(case, "bf16")
    Pw, Gw, Mw = upload_case(case, "bf16")
    nsa.muon_step(list(zip(Pw, Gw, Mw)), 0.02, 0.95, 5)   # loads the kernels once
    torch.cuda.synchronize()
    busy, s = torch.cuda.Stream(), torch.cuda.Stream()
    done = torch.cuda.Event()
    with torch.cuda.stream(busy):
        torch.cuda._sleep(1 << 30)   # about half a second of spinning, then it ends
        done.record()
    with torch.cuda.stream(s):
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    still_running = not done.query()
    s.synchronize()
    torch.cuda.synchronize()
    assert still_running
    p1 = [from_device(p) for p in P]
    m1 = [from_device(m) for m in M]
    assert_parity(case, "bf16", p1, m1, oracle_case(case, 0.02, 0.95, 5), BF16_TOL)


def test_alloc_failure_leaves_state_unchanged(nsa, monkeypatch):
    import torch
    case = workloads.random_case(13, [(128, 256)], "bf16")
    P, G, M = upload_case(case, "bf16")
    p0, m0 = P[0].clone(), M[0].clone()
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    with pytest.raises(nsa.MuonError) as ei:
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert torch.equal(P[0], p0) and torch.equal(M[0], m0)


def test_checkpoint_resume_bitwise(nsa):
    import torch
    case = workloads.random_case(14, [(256, 384), (384, 256)], "bf16")
    P, G, M = upload_case(case, "bf16")
    for _ in range(2):
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    saved = [t.cpu().clone() for t in P + M]
    for _ in range(2):
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    P2 = [t.cuda() for t in saved[:2]]
    M2 = [t.cuda() for t in saved[2:]]
    for _ in range(2):
        nsa.muon_step(list(zip(P2, G, M2)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(P + M, P2 + M2))


# ---- the two polynomial forms; per-parameter coefficient sets; eps, rms ----

@pytest.mark.parametrize("form", ["direct", "square", "folded"])
def test_poly_forms_ragged(nsa, form):
    # Both bf16 forms of the NS step against the oracle over the ragged
    # shapes (the square form, the default, completes the polynomial to a
    # square so that no epilogue reads an operand tile; the direct form is
    # the page's, with the operand tiles read in the epilogues).
    case = workloads.random_case(1, RAGGED, "bf16", params_init="zero")
    p1, m1 = run_case(nsa, case, "bf16", poly_form=form)
    ref = oracle_case(case, 0.02, 0.95, 5)
    worst = assert_parity(case, "bf16", p1, m1, ref, BF16_TOL)
    _print(form, "form ragged worst rel err", worst)


@pytest.mark.parametrize("form", ["square", "folded", "direct"])
def test_drain_epilogue_edges(nsa, form):
    # Shapes whose tiles reach the edges of the per-wave (drain) epilogues:
    # 1408 x 1280 has m_pad = 5 * 256 + 128 (wide 128 x 512 tiles in
    # every role) and an odd number of 256-column tiles, so the last wide
    # Update tile has two waves past the padded width; both orientations;
    # 24 + 8 matrices give more Update, Gram and Poly tiles than
    # workgroups, so workgroups go on from a drained tile to the next (full,
    # diagonal or wide). Sampled matrices against the oracle, all finite.
    import torch
    shapes = [(1408, 1280)] * 12 + [(1280, 1408)] * 12 + [(640, 896)] * 4 + [(896, 640)] * 4
    case = workloads.random_case(41, shapes, "bf16", params_init="zero")
    P, G, M = upload_case(case, "bf16")
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5, poly_form=form)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(p.float()).all()) for p in P)
    for i in (0, 11, 12, 23, 24, 31):
        c = case[i]
        rp, rb, _ = oracle.muon_matrix_step(c["params"].as_f64(), c["grad"].as_f64(),
                                            c["momentum"].astype(np.float64), 0.02, 0.95, 5)
        e = check_update(c["params"].as_f64(), from_device(P[i]), rp, "bf16", BF16_TOL,
                         label=f"{form} #{i} {shapes[i][0]}x{shapes[i][1]}")
        assert e <= BF16_TOL, (form, i, e)
        assert check_momentum(from_device(M[i]), rb, label=f"#{i}") <= MOM_TOL


def test_per_parameter_coefficient_sets(nsa):
    # HyperParallel-FSDP section 6.2: per-parameter coefficient sets. Three
    # sets over matrices of two shapes, with same-shaped matrices on
    # different sets; every matrix against the oracle with its own table,
    # and the mixed call bitwise equal to one call per set.
    import torch
    quintic = [(3.4445, -4.775, 2.0315)] * 5
    other = [(3.0, -3.2, 1.2), (3.4445, -4.775, 2.0315), (2.9, -3.0, 1.1), (3.4, -4.7, 2.0), (1.875, -1.25, 0.375)]
    cubic = [(1.5, -0.5, 0.0)] * 5
    sets = [quintic, other, cubic]
    shapes = [(256, 384), (384, 256), (256, 384), (200, 330), (256, 384), (330, 200)]
    set_of = [0, 1, 2, 1, 1, 2]
    for dtype, tol in (("bf16", BF16_TOL), ("f32", F32_TOL)):
        case = workloads.random_case(30, shapes, dtype, params_init="zero")
        P, G, M = upload_case(case, dtype)
        nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5, coeff_sets=sets, coeff_set_of=set_of)
        P2, G2, M2 = upload_case(case, dtype)
        for k in range(3):
            idx = [i for i, s in enumerate(set_of) if s == k]
            nsa.muon_step([(P2[i], G2[i], M2[i]) for i in idx], 0.02, 0.95, 5, coeffs=sets[k])
        torch.cuda.synchronize()
        for a, b in zip(_bits(P) + _bits(M), _bits(P2) + _bits(M2)):
            assert np.array_equal(a, b)
        for i, c in enumerate(case):
            rp, rb, _ = oracle.muon_matrix_step(c["params"].as_f64(), c["grad"].as_f64(),
                                                c["momentum"].astype(np.float64), 0.02, 0.95, 5,
                                                coeffs=sets[set_of[i]])
            e = check_update(c["params"].as_f64(), from_device(P[i]), rp, dtype, tol, label=f"set {set_of[i]} #{i}")
            assert e <= tol, (dtype, i, e)


def test_eps_and_rms_target_options(nsa):
    # A non-default epsilon large enough to change the normalisation (eps =
    # 0.1 against ||u||_F of about 0.3 here) and a non-default RMS target.
    for dtype, tol in (("f32", F32_TOL), ("bf16", BF16_TOL)):
        case = workloads.random_case(31, [(192, 320), (320, 192), (100, 60)], dtype, params_init="zero")
        p1, m1 = run_case(nsa, case, dtype, 0.02, 0.95, 5, eps=0.1, rms_target=0.35)
        ref = oracle_case(case, 0.02, 0.95, 5, eps=0.1, rms_target=0.35)
        assert_parity(case, dtype, p1, m1, ref, tol)
        # the options matter: the default eps gives a different update
        other = oracle_case(case, 0.02, 0.95, 5, rms_target=0.35)
        assert rel_fro(ref[0][0], other[0][0]) > 10 * tol
