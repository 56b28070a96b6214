"""GPU test of muon_step_noalloc (the entry point that allocates no device
memory: its workspace is the library's static per-GPU array), through the
C ABI: two calls in a row, the second with a smaller input, each bitwise
equal to muon_step on the same inputs (batches never change a matrix's
result) and within the bf16 bar of the fp64 oracle; a matrix whose
workspace alone exceeds the array is rejected before anything changes."""
import numpy as np
import pytest

import workloads
from gpu_helpers import BF16_TOL, F32_TOL, check_update, from_device, oracle_case, upload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nsa():
    import torch
    import newton_schulz_10_amd as m
    m.load()
    torch.cuda.init()
    return m


def _bits(ts):
    import torch
    return [t.detach().cpu().view(-1).view(torch.int16 if t.element_size() == 2 else torch.int32).numpy().copy()
            for t in ts]


def _both(nsa, case, dtype, **opts):
    """Runs muon_step_noalloc and muon_step on separate copies of `case`;
    returns the noalloc tensors after checking they equal muon_step's."""
    import torch
    P, G, M = upload_case(case, dtype)
    P2, G2, M2 = upload_case(case, dtype)
    nsa.muon_step_noalloc(list(zip(P, G, M)), 0.02, 0.95, 5, **opts)
    nsa.muon_step(list(zip(P2, G2, M2)), 0.02, 0.95, 5, **opts)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(_bits(P) + _bits(M), _bits(P2) + _bits(M2))):
        assert np.array_equal(a, b), k
    return P, M


def test_noalloc_two_calls_match_muon_step(nsa):
    import torch
    # First call: 40 MoE-bank matrices (about 19.5 MB of bf16 workspace each,
    # so the 512 MiB array takes 26 at a time: two batches), in both
    # orientations, two of them idle, and ragged shapes.
    shapes = [(1408, 2048)] * 20 + [(2048, 1408)] * 20 + [(300, 520), (7, 1), (129, 1000)]
    case = workloads.random_case(50, shapes, "bf16", params_init="zero", momentum_init="zero", zero=(3, 27))
    plan = nsa.plan_query(shapes, torch.bfloat16)
    print("muon_step batches", [b["count"] for b in plan["batches"]], flush=True)
    P, M = _both(nsa, case, "bf16")
    sub = [0, 25, 40, 41, 42]
    ref = oracle_case([case[i] for i in sub], 0.02, 0.95, 5)
    for i, (rp, _, _) in zip(sub, ref):
        e = check_update(case[i]["params"].as_f64(), from_device(P[i]), rp, "bf16", BF16_TOL, label=f"noalloc #{i}")
        assert e <= BF16_TOL, (i, e)
    for i in (3, 27):   # idle: exact no-op
        assert torch.count_nonzero(P[i]) == 0
    # Second call, smaller: the array keeps the first call's contents, which
    # must not leak into this result.
    case2 = workloads.random_case(51, [(256, 384), (384, 256), (64, 128)], "bf16", params_init="zero")
    P, M = _both(nsa, case2, "bf16")
    ref = oracle_case(case2, 0.02, 0.95, 5)
    for i, (rp, _, _) in enumerate(ref):
        e = check_update(case2[i]["params"].as_f64(), from_device(P[i]), rp, "bf16", BF16_TOL, label=f"noalloc 2 #{i}")
        assert e <= BF16_TOL, (i, e)


def test_noalloc_fp32_and_options(nsa):
    case = workloads.random_case(52, [(192, 320), (320, 192), (100, 60)], "f32")
    P, M = _both(nsa, case, "f32", weight_decay=0.1, scale_rule="original")
    ref = oracle_case(case, 0.02, 0.95, 5, weight_decay=0.1, scale_rule="original")
    for i, (rp, _, _) in enumerate(ref):
        e = check_update(case[i]["params"].as_f64(), from_device(P[i]), rp, "f32", F32_TOL, label=f"noalloc f32 #{i}")
        assert e <= F32_TOL, (i, e)


def test_noalloc_rejects_a_matrix_larger_than_the_array(nsa):
    import torch
    # 7168 x 18432 bf16 needs about 733 MB of workspace (> 512 MiB).
    p = torch.zeros((7168, 18432), dtype=torch.bfloat16, device="cuda")
    g = torch.ones_like(p)
    m = torch.zeros((7168, 18432), dtype=torch.float32, device="cuda")
    small = upload_case(workloads.random_case(53, [(128, 256)], "bf16"), "bf16")
    before = [t.clone() for t in (small[0][0], small[2][0])]
    with pytest.raises(nsa.MuonError) as ei:
        nsa.muon_step_noalloc([(small[0][0], small[1][0], small[2][0]), (p, g, m)], 0.02, 0.95, 5)
    assert ei.value.status == 1
    assert "7168 x 18432" in str(ei.value) and "static workspace" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(p) == 0 and torch.count_nonzero(m) == 0
    assert torch.equal(small[0][0], before[0]) and torch.equal(small[2][0], before[1])
