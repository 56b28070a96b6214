"""CPU tests of the C ABI: the library loads and exports every symbol that
include/muon.h declares, the host-only planner, and argument validation
(every call here is rejected before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


@pytest.fixture(scope="module")
def lib():
    import newton_schulz_10_amd as nsa
    if not os.path.exists(nsa.library_path()):
        from newton_schulz_10_amd import build
        build.build_library()
    return nsa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("muon_group_step", "muon_step", "muon_orthogonalize", "muon_plan_query", "muon_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
        exported = set(re.findall(r"\bT (muon_\w+)", out))
        assert set(declared_functions()) <= exported


def test_python_binding_names_match_c(lib):
    import newton_schulz_10_amd as nsa
    for n in ("muon_group_step", "muon_step", "muon_orthogonalize"):
        assert callable(getattr(nsa, n))
    assert set(nsa.SYMBOLS) == set(declared_functions())


def test_status_strings_and_version(lib):
    assert lib.muon_status_string(0) == b"ok"
    assert lib.muon_status_string(3) == b"misaligned pointer"
    assert lib.muon_version() >= 100


def test_cpp_planner_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "test_plan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "newton_schulz_10_amd", "csrc"),
           os.path.join(ROOT, "tests", "cpp", "test_plan.cpp"),
           os.path.join(ROOT, "newton_schulz_10_amd", "csrc", "plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planner tests: ok" in r.stdout


# ---- plan through the library ---------------------------------------------

def test_plan_query_moe_bank(lib):
    import torch
    import newton_schulz_10_amd as nsa
    shapes = [(2048, 1408)] * 256 + [(1408, 2048)] * 256
    plan = nsa.plan_query(shapes, torch.bfloat16, compute_units=0)   # fewest batches
    assert [b["count"] for b in plan["batches"]] == [171, 171, 170]
    assert all(b["m"] == 1408 and b["n"] == 2048 for b in plan["batches"])
    assert plan["order"] == list(range(512))
    assert plan["workspace_bytes"] > 171 * 1408 * 2048 * 2 * 2
    # Fitted to 256 compute units: 128 matrices give 18*128 = 9*256 Gram/Poly
    # tiles and 44*128 = 22*256 Update tiles, whole rounds.
    fitted = nsa.plan_query(shapes, torch.bfloat16, compute_units=256)
    assert [b["count"] for b in fitted["batches"]] == [128] * 4
    assert fitted["order"] == list(range(512))
    with pytest.raises(nsa.MuonError):
        nsa.plan_query(shapes, torch.bfloat16, compute_units=-2)
    # The default does not fit (idle matrices are skipped on the device, so a
    # split fitted for all of them can leave a nearly empty last round).
    assert [b["count"] for b in nsa.plan_query(shapes, torch.bfloat16)["batches"]] == [171, 171, 170]
    nsa.plan_query(shapes, torch.bfloat16, compute_units=-1)   # current device, or none: accepted


def test_plan_query_mlp_and_stack(lib):
    import torch
    import newton_schulz_10_amd as nsa
    mlp = nsa.plan_query([(4096, 14336)] * 32 + [(14336, 4096)] * 32, torch.bfloat16, compute_units=0)
    assert [b["count"] for b in mlp["batches"]] == [8] * 8
    stack = nsa.plan_query([(7168, 7168)] * 4 + [(7168, 18432)] * 2 + [(7168, 2048)] * 128, torch.bfloat16,
                           compute_units=0)
    assert [(b["m"], b["n"], b["count"]) for b in stack["batches"]] == \
        [(7168, 18432, 2), (7168, 7168, 4)] + [(2048, 7168, 32)] * 4
    attn = nsa.plan_query([(2048, 2048)] * 32, torch.bfloat16, compute_units=0)
    assert [b["count"] for b in attn["batches"]] == [32]
    capped = nsa.plan_query([(2048, 2048)] * 32, torch.bfloat16, batch_cap_elems=5 * 2048 * 2048,
                            compute_units=0)
    assert [b["count"] for b in capped["batches"]] == [5, 5, 5, 5, 4, 4, 4]


# ---- validation: rejected before any device access -------------------------

def _fake(addr):
    return ctypes.c_void_p(addr)


def _call_step(lib, mats, lr=0.02, beta=0.95, steps=5, dtype=1, opts=None):
    import newton_schulz_10_amd as nsa
    arr = (nsa.Matrix * max(len(mats), 1))(*[nsa.Matrix(*m) for m in mats])
    o = None if opts is None else ctypes.byref(opts)
    rc = lib.muon_step(arr if mats else None, len(mats), lr, beta, steps, dtype, o, None)
    return rc, lib.muon_last_error().decode()


BASE = 0x7f0000000000


def test_validation_rejects_bad_arguments(lib):
    import newton_schulz_10_amd as nsa
    good = (BASE, BASE + 0x100000, BASE + 0x200000, 16, 32)
    assert _call_step(lib, [good], steps=65)[0] == 1
    assert _call_step(lib, [good], steps=-1)[0] == 1
    assert _call_step(lib, [good], lr=float("nan"))[0] == 1
    assert _call_step(lib, [good], beta=float("inf"))[0] == 1
    assert _call_step(lib, [good], dtype=9)[0] == 1
    rc, msg = _call_step(lib, [good, (BASE + 0x300000, 0, BASE + 0x400000, 16, 32)])
    assert rc == 1 and "grads[1]" in msg
    rc, msg = _call_step(lib, [good, (BASE + 0x300008, BASE + 0x310000, BASE + 0x400000, 16, 32)])
    assert rc == 3 and "params[1]" in msg
    rc, msg = _call_step(lib, [(BASE, BASE + 0x100000, BASE + 0x200000, 0, 32)])
    assert rc == 1 and "shape" in msg
    rc, msg = _call_step(lib, [(BASE, BASE + 0x100000, BASE + 0x200000, 16, (1 << 20) + 1)])
    assert rc == 1
    # params of matrix 0 overlap the grads of matrix 1
    rc, msg = _call_step(lib, [good, (BASE + 0x300000, BASE + 0x200, BASE + 0x400000, 16, 32)])
    assert rc == 1 and "overlaps" in msg
    # bad options
    o = nsa.Options()
    lib.muon_default_options(ctypes.byref(o))
    o.scale_rule = 5
    assert _call_step(lib, [good], opts=o)[0] == 1
    lib.muon_default_options(ctypes.byref(o))
    o.eps = -1.0
    assert _call_step(lib, [good], opts=o)[0] == 1
    lib.muon_default_options(ctypes.byref(o))
    bad = (ctypes.c_float * 15)(*([1.0] * 14 + [float("nan")]))
    o.coeffs = ctypes.cast(bad, ctypes.POINTER(ctypes.c_float))
    rc, msg = _call_step(lib, [good], opts=o)
    assert rc == 1 and "coeffs[14]" in msg
    # num < 0 and NULL table
    assert lib.muon_step(None, -1, 0.02, 0.95, 5, 1, None, None) == 1
    assert lib.muon_step(None, 2, 0.02, 0.95, 5, 1, None, None) == 1


def test_empty_calls_are_noops(lib):
    # count == 0 returns before any device work.
    assert lib.muon_step(None, 0, 0.02, 0.95, 5, 1, None, None) == 0
    assert lib.muon_group_step(None, None, None, 0, 4, 4, 0.02, 0.95, 5, 1, None) == 0
    assert lib.muon_orthogonalize(None, None, 0, 4, 4, 5, 1, None, None) == 0


def test_group_step_and_orthogonalize_validation(lib):
    arr = ctypes.c_void_p * 2
    p = arr(BASE, BASE + 0x10000)
    g = arr(BASE + 0x20000, BASE + 0x30000)
    m = arr(BASE + 0x40000, BASE + 0x50000)
    assert lib.muon_group_step(p, g, m, 2, 0, 4, 0.02, 0.95, 5, 1, None) == 1
    assert lib.muon_group_step(None, g, m, 2, 4, 4, 0.02, 0.95, 5, 1, None) == 1
    same = arr(BASE, BASE)  # two params at one address
    assert lib.muon_group_step(same, g, m, 2, 4, 4, 0.02, 0.95, 5, 1, None) == 1
    ins = arr(BASE, BASE + 0x10000)
    outs = arr(BASE + 8, BASE + 0x20000)
    assert lib.muon_orthogonalize(ins, outs, 2, 4, 4, 5, 1, None, None) == 3
    outs = arr(BASE + 0x10, BASE + 0x20000)  # partial overlap of in[0] and out[0]
    assert lib.muon_orthogonalize(ins, outs, 2, 4, 4, 5, 1, None, None) == 1


def test_alloc_failure_injection_is_host_side(lib, monkeypatch):
    # With MUON_TEST_FAIL_ALLOC=1 the call reports out-of-memory after
    # validation and before touching the device.
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    good = (BASE, BASE + 0x100000, BASE + 0x200000, 16, 32)
    rc, msg = _call_step(lib, [good])
    assert rc == 4 and "MUON_TEST_FAIL_ALLOC" in msg


# ---- strided logical-matrix views and the NS element type -----------------

def _call_views(lib, views, dtype=1, opts=None):
    """views: (param, grad, momentum, rows, cols, ld) with fake aligned addresses."""
    import newton_schulz_10_amd as nsa
    arr = (nsa.MatrixView * len(views))(*[nsa.MatrixView(*v) for v in views])
    rc = lib.muon_step_views(arr, len(views), 0.02, 0.95, 5, dtype,
                             ctypes.byref(opts) if opts is not None else None, None)
    return rc, lib.muon_last_error().decode()


def test_view_validation(lib, monkeypatch):
    # With MUON_TEST_FAIL_ALLOC=1 a call that passes validation reports
    # out-of-memory (4) before touching the device.
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    P, G, M = BASE, BASE + 0x1000000, BASE + 0x2000000
    # Two interleaved row views of a 64 x 256 bf16 parameter (even / odd
    # rows, stride 512 elements) with momentum laid out the same way.
    even = (P, G, M, 32, 256, 512)
    odd = (P + 512, G + 512, M + 1024, 32, 256, 512)
    assert _call_views(lib, [even, odd])[0] == 4
    # The same rows twice.
    rc, msg = _call_views(lib, [even, (P, G + 0x100000, M + 0x100000, 32, 256, 512)])
    assert rc == 1 and "overlaps" in msg
    # Column halves of a 64 x 256 parameter (ld 256, 128 columns each), and
    # a third view straddling them.
    left = (P, G, M, 64, 128, 256)
    right = (P + 256, G + 256, M + 512, 64, 128, 256)
    assert _call_views(lib, [left, right])[0] == 4
    mid = (P + 128, G + 0x100000, M + 0x100000, 64, 128, 256)
    rc, msg = _call_views(lib, [left, right, mid])
    assert rc == 1 and "params" in msg
    # ld 0 means contiguous; ld < cols and ld >= 2^31 are rejected.
    assert _call_views(lib, [(P, G, M, 64, 256, 0)])[0] == 4
    rc, msg = _call_views(lib, [(P, G, M, 64, 256, 255)])
    assert rc == 1 and "ld" in msg
    assert _call_views(lib, [(P, G, M, 64, 256, 1 << 31)])[0] == 1
    # A grad view that shares columns with its own param view, and one in
    # the other column half of the same rows (disjoint).
    assert _call_views(lib, [(P, P + 128, M, 64, 128, 256)])[0] == 1
    assert _call_views(lib, [(P, P + 256, M, 64, 128, 256)])[0] == 4
    assert lib.muon_step_views(None, 1, 0.02, 0.95, 5, 1, None, None) == 1
    assert lib.muon_step_views(None, 0, 0.02, 0.95, 5, 1, None, None) == 0


def test_ns_dtype_option(lib, monkeypatch):
    import newton_schulz_10_amd as nsa
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    good = (BASE, BASE + 0x100000, BASE + 0x200000, 16, 32)
    o = nsa.Options()
    lib.muon_default_options(ctypes.byref(o))
    assert o.ns_dtype == -1
    o.ns_dtype = 2
    rc, msg = _call_step(lib, [good], dtype=0, opts=o)
    assert rc == 1 and "ns_dtype" in msg
    o.ns_dtype = 1   # fp32 tensors, bf16 NS
    assert _call_step(lib, [good], dtype=0, opts=o)[0] == 4


def test_plan_query_follows_ns_dtype(lib):
    import torch
    import newton_schulz_10_amd as nsa
    f32 = nsa.plan_query([(300, 520)], dtype=torch.float32)
    mixed = nsa.plan_query([(300, 520)], dtype=torch.float32, ns_dtype=torch.bfloat16)
    bf = nsa.plan_query([(300, 520)], dtype=torch.bfloat16)
    # The NS element type sets the padding (fp32: 64; bf16: m to 128, n to 256)
    # and the workspace layout.
    assert (f32["batches"][0]["m_pad"], f32["batches"][0]["n_pad"]) == (320, 576)
    assert (mixed["batches"][0]["m_pad"], mixed["batches"][0]["n_pad"]) == (384, 768)
    assert mixed["batches"] == bf["batches"] and mixed["workspace_bytes"] == bf["workspace_bytes"]


def test_environment_switches(lib, monkeypatch):
    import newton_schulz_10_amd as nsa
    shapes = [(2048, 1408)] * 256 + [(1408, 2048)] * 256
    # MUON_BATCH_CAP replaces the default cap (options NULL or cap 0) ...
    assert len(nsa.plan_query(shapes)["batches"]) == 3
    monkeypatch.setenv("MUON_BATCH_CAP", str(64 * 1408 * 2048))
    assert [b["count"] for b in nsa.plan_query(shapes)["batches"]] == [64] * 8
    # ... but not an explicit cap, and malformed values are ignored.
    assert len(nsa.plan_query(shapes, batch_cap_elems=1 << 30)["batches"]) == 2
    monkeypatch.setenv("MUON_BATCH_CAP", "12abc")
    assert len(nsa.plan_query(shapes)["batches"]) == 3
    # MUON_PROFILE=1 turns the per-launch timing on when the library loads.
    code = ("import newton_schulz_10_amd as m; L = m.load(); "
            "print(L.muon_profile_enable(0), L.muon_profile_enable(0))")
    env = dict(os.environ, MUON_PROFILE="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.stdout.split() == ["1", "0"], r.stdout + r.stderr


def test_view_overlap_check_against_brute_force(lib, monkeypatch):
    # Random small strided views of one bf16 parameter, validated through
    # muon_step_views (MUON_TEST_FAIL_ALLOC=1: a call that passes validation
    # returns 4 before touching the device). Expected: rejection (1) iff two
    # views share a byte, or two views with different strides have
    # intersecting spans (the documented conservative rule).
    import numpy as np
    monkeypatch.setenv("MUON_TEST_FAIL_ALLOC", "1")
    rng = np.random.default_rng(7)
    P, G, M = BASE, BASE + 0x1000000, BASE + 0x2000000
    for trial in range(400):
        nv = int(rng.integers(2, 4))
        views, spans = [], []
        shared_ld = 8 * int(rng.integers(3, 6)) if rng.random() < 0.6 else None   # interleaving views
        for k in range(nv):
            rows = int(rng.integers(1, 5))
            cols = 8 * int(rng.integers(1, 4))
            ld = max(shared_ld, cols) if shared_ld else cols + 8 * int(rng.integers(0, 3))
            off = 8 * int(rng.integers(0, 24))           # elements; 16-byte aligned
            views.append((P + 2 * off, G + 0x10000 * (k + 1), M + 0x40000 * (k + 1), rows, cols, ld))
            b = set()
            for r in range(rows):
                start = 2 * (off + r * ld)
                b.update(range(start, start + 2 * cols))
            spans.append((2 * off, 2 * (off + (rows - 1) * ld + cols), ld, b))
        expect_bad = False
        for i in range(nv):
            for j in range(i + 1, nv):
                (lo1, hi1, ld1, b1), (lo2, hi2, ld2, b2) = spans[i], spans[j]
                if b1 & b2:
                    expect_bad = True
                elif ld1 != ld2 and lo1 < hi2 and lo2 < hi1:
                    expect_bad = True
        rc, msg = _call_views(lib, views)
        assert rc == (1 if expect_bad else 4), (trial, views, msg)


# ---- binding: tensor forms and the checks the C interface cannot make ------

def test_matrix_layout_tensor_forms():
    # HyperParallel-FSDP section 6.6 (Figure 10(a)): [A, B], [A, 1, B] and
    # [N, A, B] share the (A, B) group; section 6.3: [N, A, B] is N matrices.
    from newton_schulz_10_amd import matrix_layout
    assert matrix_layout((6, 10)) == [(0, 6, 10)]
    assert matrix_layout((6, 1, 10)) == [(0, 6, 10)]
    assert matrix_layout((3, 6, 10)) == [(0, 6, 10), (60, 6, 10), (120, 6, 10)]
    assert matrix_layout((1, 6, 10)) == [(0, 6, 10)]
    assert matrix_layout((1, 1, 10)) == [(0, 1, 10)]
    with pytest.raises(ValueError):
        matrix_layout((2, 3, 4, 5))
    with pytest.raises(ValueError):
        matrix_layout((7,))


def test_plan_groups_a1b_with_ab(lib):
    # A (6, 1, 10) tensor is one 6 x 10 matrix: it joins the (6, 10) group
    # with a [6, 10] matrix and the two matrices of a [2, 6, 10] bank, and a
    # [10, 6] matrix transposed.
    import torch
    import newton_schulz_10_amd as nsa
    shapes = [(r, c) for t in ((6, 10), (6, 1, 10), (2, 6, 10), (10, 6)) for _, r, c in nsa.matrix_layout(t)]
    assert shapes == [(6, 10), (6, 10), (6, 10), (6, 10), (10, 6)]
    plan = nsa.plan_query(shapes, torch.bfloat16)
    assert [(b["m"], b["n"], b["count"]) for b in plan["batches"]] == [(6, 10, 5)]


def test_binding_rejects_wrong_dtypes_and_host_tensors(lib):
    # The C interface sees only pointers; the binding must refuse tensors
    # whose element type or device the kernels would misread (a bf16
    # momentum would be written 4 bytes per element into 2-byte storage, a
    # host pointer would fault the GPU). Every rejection happens before any
    # call into the library, so no GPU is needed.
    import torch
    import newton_schulz_10_amd as nsa
    bf, f32 = torch.bfloat16, torch.float32
    p, g, m = torch.zeros(8, 16, dtype=bf), torch.zeros(8, 16, dtype=bf), torch.zeros(8, 16, dtype=f32)
    with pytest.raises(TypeError, match="momentum"):
        nsa.muon_step([(p, g, torch.zeros(8, 16, dtype=bf))], 0.02)
    with pytest.raises(TypeError, match="grad"):
        nsa.muon_step([(p, torch.zeros(8, 16, dtype=f32), m)], 0.02)
    with pytest.raises(TypeError):
        nsa.muon_step([(torch.zeros(8, 16, dtype=torch.float16), g, m)], 0.02)
    with pytest.raises(ValueError, match="expected the current GPU"):
        nsa.muon_step([(p, g, m)], 0.02)
    with pytest.raises(TypeError, match="momentum"):
        nsa.muon_group_step([p], [g], [torch.zeros(8, 16, dtype=bf)], 0.02)
    with pytest.raises(TypeError, match="grads"):
        nsa.muon_group_step([p], [torch.zeros(8, 16, dtype=f32)], [m], 0.02)
    with pytest.raises(ValueError, match="expected the current GPU"):
        nsa.muon_group_step([p], [g], [m], 0.02)
    with pytest.raises(TypeError, match="momentum"):
        nsa.muon_step_views([(p, g, torch.zeros(8, 16, dtype=bf))], 0.02)
    with pytest.raises(TypeError, match="grad"):
        nsa.muon_step_views([(p, torch.zeros(8, 16, dtype=f32), m)], 0.02)
    with pytest.raises(ValueError, match="expected the current GPU"):
        nsa.muon_step_views([(p, g, m)], 0.02)
    with pytest.raises(TypeError, match="outputs"):
        nsa.muon_orthogonalize([p], [torch.zeros(8, 16, dtype=f32)])
    with pytest.raises(ValueError, match="expected the current GPU"):
        nsa.muon_orthogonalize([p], [torch.zeros(8, 16, dtype=bf)])
