"""GPU tests of two front-end forms of the step, through the C ABI:

* fp32 master tensors iterated on bf16 MFMA (`ns_dtype`), and bf16 tensors
  iterated in fp32, each against the fp64 oracle on the same stored values;
* logical matrices given as strided views into physical parameters (the
  model adapter of the HyperParallel-FSDP paper, section 6.6: heads of a
  fused QKV weight, interleaved gate/up rows, column blocks), which must
  give bitwise the result of the same matrices passed contiguously, and
  leave every element outside the views untouched.

Tolerances: relative Frobenius error of the update <= 2e-2 where the NS
iterate is bf16, <= 1e-4 where it is fp32; momentum <= 1e-6."""
import numpy as np
import pytest

import workloads
from gpu_helpers import BF16_TOL, F32_TOL, MOM_TOL, check_momentum, check_update, from_device, oracle_case

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


def _dev(st, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(st.bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(st.values, np.float32)).cuda()


# ---- NS element type different from the tensors' ---------------------------

SHAPES = [(256, 384), (384, 256), (300, 520), (64, 64), (128, 640)]


@pytest.mark.parametrize("tensors,ns,tol", [("f32", "bf16", BF16_TOL), ("bf16", "f32", F32_TOL)])
def test_ns_dtype_against_oracle(nsa, tensors, ns, tol):
    import torch
    case = workloads.random_case(40, SHAPES, tensors, zero=(3,))
    P = [_dev(c["params"], tensors) for c in case]
    G = [_dev(c["grad"], tensors) for c in case]
    M = [torch.from_numpy(c["momentum"].copy()).cuda() for c in case]
    nsd = torch.bfloat16 if ns == "bf16" else torch.float32
    _print("ns_dtype case", tensors, ns, SHAPES)
    nsa.muon_step(list(zip(P, G, M)), 0.02, 0.95, 5, weight_decay=0.0, ns_dtype=nsd)
    torch.cuda.synchronize()
    ref = oracle_case(case, 0.02, 0.95, 5)
    worst = 0.0
    for i, (c, (rp, rb, _)) in enumerate(zip(case, ref)):
        p0 = c["params"].as_f64()
        e = check_update(p0, from_device(P[i]), rp, tensors, tol, label=f"{ns} NS #{i}")
        em = check_momentum(from_device(M[i]), rb, label=f"#{i}")
        worst = max(worst, e)
        assert e <= tol, (i, SHAPES[i], e)
        assert em <= MOM_TOL, (i, SHAPES[i], em)
    _print(tensors, "tensors with", ns, "NS: worst rel err", worst)


def test_fp32_master_bf16_ns_update_is_the_bf16_iterate(nsa):
    # With momentum and params zero and grads exactly representable in
    # bf16, fp32 master tensors iterated in bf16 see the same NS input as
    # bf16 tensors, so their update is the same bf16 O: p1 = -gamma*O,
    # computed in fp32 instead of rounded to bf16.
    import torch
    shapes = [(256, 384), (384, 256), (300, 520), (128, 256)]
    case = workloads.random_case(41, shapes, "bf16", momentum_init="zero", params_init="zero", zero=(3,))
    P32 = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    G32 = [torch.from_numpy(c["grad"].values.copy()).cuda() for c in case]
    M32 = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    P16 = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    G16 = [_dev(c["grad"], "bf16") for c in case]
    M16 = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    nsa.muon_step(list(zip(P32, G32, M32)), 0.02, 0.95, 5, ns_dtype=torch.bfloat16)
    nsa.muon_step(list(zip(P16, G16, M16)), 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(M32[i], M16[i]), i
        # bf16 rounding of the fp32 update is the bf16 path's update.
        assert torch.equal(P32[i].to(torch.bfloat16), P16[i]), i
    assert not torch.any(P32[3]) and not torch.any(P16[3])   # zero grads: no update


# ---- strided logical-matrix views ------------------------------------------

def _physical(nsa, seed, shape, dtype):
    """A seeded physical parameter, its grad and its fp32 momentum."""
    import torch
    (c,) = workloads.random_case(seed, [shape], dtype)
    return _dev(c["params"], dtype), _dev(c["grad"], dtype), torch.from_numpy(c["momentum"].copy()).cuda()


def _layouts():
    """(physical shape, list of view index expressions) per parameter."""
    return [
        # fused QKV projection: three row blocks (contiguous, ld = cols)
        ((768, 512), [np.s_[0:256], np.s_[256:512], np.s_[512:768]]),
        # gate/up rows interleaved: even and odd rows (ld = 2 * cols), tall views
        ((768, 256), [np.s_[0::2], np.s_[1::2]]),
        # column blocks of a wide factor (ld = 640, views 256 and 384 wide)
        ((256, 640), [np.s_[:, 0:256], np.s_[:, 256:640]]),
        # column blocks with a gap left untouched (ld = 648 and 644: not a
        # multiple of 8, so the apply runs as its own pass)
        ((136, 648), [np.s_[:, 0:200], np.s_[:, 208:648]]),
        ((200, 644), [np.s_[:, 0:320], np.s_[:, 328:644]]),
        # ld = 642: rows not 4-element aligned (scalar edge accesses)
        ((96, 642), [np.s_[:, 0:128], np.s_[:, 136:642]]),
    ]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_views_equal_contiguous_matrices(nsa, dtype):
    import torch
    phys, views = [], []
    for k, (shape, idx) in enumerate(_layouts()):
        p, g, m = _physical(nsa, 50 + k, shape, dtype)
        phys.append((p, g, m, p.clone(), m.clone(), idx))
        for ix in idx:
            views.append((p[ix], g[ix], m[ix]))
    _print("views", dtype, [(tuple(v[0].shape), v[0].stride()) for v in views])
    # The same logical matrices, copied out contiguously, as plain matrices.
    copies = [(v[0].contiguous(), v[1].contiguous(), v[2].contiguous()) for v in views]
    nsa.muon_step_views(views, 0.02, 0.95, 5, weight_decay=0.01)
    nsa.muon_step(copies, 0.02, 0.95, 5, weight_decay=0.01)
    torch.cuda.synchronize()
    for j, (v, c) in enumerate(zip(views, copies)):
        assert torch.equal(v[0], c[0]), (j, tuple(v[0].shape))
        assert torch.equal(v[2], c[2]), (j, tuple(v[0].shape))
    # Elements outside every view are untouched.
    for p, g, m, p0, m0, idx in phys:
        mask = torch.ones(p.shape, dtype=torch.bool, device="cuda")
        for ix in idx:
            mask[ix] = False
        assert torch.equal(p[mask], p0[mask]) and torch.equal(m[mask], m0[mask])


def test_views_against_oracle(nsa):
    # One interleaved and one column-block view, checked against the fp64
    # oracle on the stored values of the view.
    import torch
    p, g, m = _physical(nsa, 60, (768, 256), "bf16")
    q, h, n = _physical(nsa, 61, (256, 640), "bf16")
    vs = [(p[1::2], g[1::2], m[1::2]), (q[:, 256:640], h[:, 256:640], n[:, 256:640])]
    before = [(from_device(a), from_device(b), from_device(c)) for a, b, c in vs]
    nsa.muon_step_views(vs, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    import oracle
    for (p0, g0, m0), (a, _, c) in zip(before, vs):
        rp, rb, _ = oracle.muon_matrix_step(p0, g0, m0, 0.02, 0.95, 5)
        e = check_update(p0, from_device(a), rp, "bf16", BF16_TOL, label="view")
        assert e <= BF16_TOL, (p0.shape, e)
        assert check_momentum(from_device(c), rb, label="view") <= MOM_TOL


def test_views_at_model_shapes(nsa):
    # Real shapes through the fused apply with a row stride other than the
    # view's width: a fused QKV projection (three 2048 x 2048 heads, ld =
    # 2048), an expert FC1 with gate/up rows interleaved (two 1408 x 2048
    # views, ld = 4096) and a tall weight split into column blocks (two
    # 2048 x 1408 views, ld = 2816). Bitwise equal to contiguous copies.
    import torch
    layouts = [((6144, 2048), [np.s_[0:2048], np.s_[2048:4096], np.s_[4096:6144]]),
               ((2816, 2048), [np.s_[0::2], np.s_[1::2]]),
               ((2048, 2816), [np.s_[:, 0:1408], np.s_[:, 1408:2816]])]
    views = []
    for k, (shape, idx) in enumerate(layouts):
        p, g, m = _physical(nsa, 70 + k, shape, "bf16")
        views += [(p[ix], g[ix], m[ix]) for ix in idx]
    _print("model-shape views", [(tuple(v[0].shape), v[0].stride()) for v in views])
    copies = [(v[0].contiguous(), v[1].contiguous(), v[2].contiguous()) for v in views]
    nsa.muon_step_views(views, 0.02, 0.95, 5)
    nsa.muon_step(copies, 0.02, 0.95, 5)
    torch.cuda.synchronize()
    for j, (v, c) in enumerate(zip(views, copies)):
        assert torch.equal(v[0], c[0]) and torch.equal(v[2], c[2]), (j, tuple(v[0].shape))


def test_views_of_fp32_masters_with_bf16_ns(nsa):
    # Strided views of fp32 master parameters iterated on bf16 MFMA: bitwise
    # the contiguous result, and within the bf16 bar of the oracle.
    import torch
    p, g, m = _physical(nsa, 80, (768, 512), "f32")
    vs = [(p[0::2], g[0::2], m[0::2]), (p[1::2, 0:256], g[1::2, 0:256], m[1::2, 0:256])]
    before = [(from_device(a), from_device(b), from_device(c)) for a, b, c in vs]
    copies = [(a.contiguous(), b.contiguous(), c.contiguous()) for a, b, c in vs]
    nsa.muon_step_views(vs, 0.02, 0.95, 5, ns_dtype=torch.bfloat16)
    nsa.muon_step(copies, 0.02, 0.95, 5, ns_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    import oracle
    for (p0, g0, m0), (a, _, c), (ca, _, cc) in zip(before, vs, copies):
        assert torch.equal(a, ca) and torch.equal(c, cc)
        rp, rb, _ = oracle.muon_matrix_step(p0, g0, m0, 0.02, 0.95, 5)
        e = check_update(p0, from_device(a), rp, "f32", BF16_TOL, label="fp32 master view")
        assert e <= BF16_TOL, (p0.shape, e)
        assert check_momentum(from_device(c), rb, label="view") <= MOM_TOL
