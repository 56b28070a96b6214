"""Python binding of libmuon, the MI355X batched Muon step (C ABI in
include/muon.h).

This module only marshals arguments: it turns torch tensors into device
pointers and shapes, passes the current HIP stream, and maps status codes
to exceptions. Every step of the computation runs in the library's HIP
kernels; there is no fallback. If libmuon.so is missing, importing the
library raises.

Tensor forms (the HyperParallel-FSDP paper, arXiv:2609.21594, section 6.6,
Figure 10(a): [A, B], [A, 1, B] and [N, A, B] parameters share the (A, B)
shape group):
  * [A, B]: one A x B matrix;
  * [A, 1, B]: one A x B matrix (the singleton middle axis is squeezed);
  * [N, A, B] with A > 1: N separate A x B matrices (section 6.3: an expert
    weight holds N independent matrices and is never flattened).

Every tensor must be a contiguous (or, for muon_step_views, unit column
stride) tensor on the current HIP device; params and grads share one dtype
(float32 or bfloat16) and momentum buffers are float32. The binding checks
this before calling the library, since the C interface only sees pointers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import torch  # loaded first: libmuon then binds to torch's HIP runtime

__all__ = ["MuonError", "matrix_layout", "muon_group_step", "muon_step", "muon_step_noalloc", "muon_step_views", "muon_orthogonalize", "plan_query",
           "profile_enable", "profile_read", "version", "library_path", "load"]

MUON_F32, MUON_BF16 = 0, 1
_DTYPES = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "misaligned pointer",
           4: "out of memory", 5: "HIP error"}


class MuonError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Options(ctypes.Structure):
    _fields_ = [("nesterov", ctypes.c_int), ("momentum_form", ctypes.c_int),
                ("weight_decay", ctypes.c_float), ("scale_rule", ctypes.c_int),
                ("rms_target", ctypes.c_float), ("eps", ctypes.c_float),
                ("coeffs", ctypes.POINTER(ctypes.c_float)), ("batch_cap_elems", ctypes.c_size_t),
                ("compute_units", ctypes.c_int), ("ns_dtype", ctypes.c_int), ("poly_form", ctypes.c_int),
                ("num_coeff_sets", ctypes.c_int), ("coeff_sets", ctypes.POINTER(ctypes.c_float)),
                ("coeff_set_of", ctypes.POINTER(ctypes.c_int))]


class Matrix(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int)]


class MatrixView(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("rows", ctypes.c_int), ("cols", ctypes.c_int), ("ld", ctypes.c_longlong)]


class PlanBatch(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int), ("m", ctypes.c_int), ("n", ctypes.c_int),
                ("m_pad", ctypes.c_int), ("n_pad", ctypes.c_int), ("first", ctypes.c_int),
                ("count", ctypes.c_int), ("coeff_set", ctypes.c_int)]


class ProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_LIB = None
SYMBOLS = ("muon_default_options", "muon_group_step", "muon_step", "muon_step_noalloc", "muon_step_views",
           "muon_orthogonalize",
           "muon_plan_query", "muon_status_string", "muon_last_error", "muon_version",
           "muon_profile_enable", "muon_profile_read")


def library_path() -> str:
    return os.environ.get("MUON_LIBRARY", os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon.so"))


def load() -> ctypes.CDLL:
    """Loads libmuon.so (raises ImportError if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m newton_schulz_10_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.muon_default_options.argtypes = [ctypes.POINTER(Options)]
    L.muon_default_options.restype = None
    L.muon_group_step.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), i, i, i,
                                  f, f, i, i, vp]
    L.muon_group_step.restype = i
    L.muon_step.argtypes = [ctypes.POINTER(Matrix), i, f, f, i, i, ctypes.POINTER(Options), vp]
    L.muon_step.restype = i
    L.muon_step_noalloc.argtypes = [ctypes.POINTER(Matrix), i, f, f, i, i, ctypes.POINTER(Options), vp]
    L.muon_step_noalloc.restype = i
    L.muon_step_views.argtypes = [ctypes.POINTER(MatrixView), i, f, f, i, i, ctypes.POINTER(Options), vp]
    L.muon_step_views.restype = i
    L.muon_orthogonalize.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i, i, i, i, i,
                                     ctypes.POINTER(Options), vp]
    L.muon_orthogonalize.restype = i
    L.muon_plan_query.argtypes = [ctypes.POINTER(i), ctypes.POINTER(i), i, i, ctypes.POINTER(Options),
                                  ctypes.POINTER(PlanBatch), i, ctypes.POINTER(i), ctypes.POINTER(i),
                                  ctypes.POINTER(ctypes.c_size_t)]
    L.muon_plan_query.restype = i
    L.muon_status_string.argtypes = [i]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_last_error.argtypes = []
    L.muon_last_error.restype = ctypes.c_char_p
    L.muon_version.argtypes = []
    L.muon_version.restype = i
    L.muon_profile_enable.argtypes = [i]
    L.muon_profile_enable.restype = i
    L.muon_profile_read.argtypes = [ctypes.POINTER(ProfileEntry), i, i]
    L.muon_profile_read.restype = i
    _LIB = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise MuonError(status, load().muon_last_error().decode(errors="replace"))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def matrix_layout(shape: Sequence[int]) -> List[Tuple[int, int, int]]:
    """(element offset, rows, cols) of each matrix a contiguous tensor of
    this shape holds: [A, B] and [A, 1, B] are one A x B matrix, [N, A, B]
    (A > 1) is N matrices of A x B (section 6.6, Figure 10(a); section 6.3)."""
    shape = tuple(int(d) for d in shape)
    if len(shape) == 2:
        return [(0, shape[0], shape[1])]
    if len(shape) == 3:
        e, r, c = shape
        if r == 1:
            return [(0, e, c)]
        return [(k * r * c, r, c) for k in range(e)]
    raise ValueError(f"expected a 2-D matrix, an [A, 1, B] matrix or an [N, A, B] bank, got {shape}")


def _on_current_device(t: torch.Tensor, what: str) -> None:
    """The library works on the current HIP device with device pointers."""
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor is on {t.device}, expected the current GPU")
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{what}: tensor is on {t.device}, but the current device is cuda:{cur}")


def _require_dtype(ts, what: str, dtype: torch.dtype) -> None:
    """Element type checks, made for every tensor of a call before any
    device check."""
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}: expected a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")


def _matrices(t: torch.Tensor, what: str, dtype: Optional[torch.dtype] = None) -> List[Tuple[int, int, int]]:
    """(device pointer, rows, cols) of each matrix held by a 2-D or 3-D
    tensor (see matrix_layout). `dtype`, if given, is required."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    layout = matrix_layout(t.shape)
    _on_current_device(t, what)
    es = t.element_size()
    return [(t.data_ptr() + off * es, r, c) for off, r, c in layout]


_NS_DTYPES = {None: -1, torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}


_POLY_FORMS = {"direct": 0, "square": 1, "folded": 2}


def _options(nesterov=True, momentum_form="ema", weight_decay=0.0, scale_rule="rms", rms_target=0.2,
             eps=1e-7, coeffs=None, batch_cap_elems=0, compute_units=0, ns_steps=5, ns_dtype=None,
             poly_form="square", coeff_sets=None, set_of_matrix=None):
    """muon_options from keyword arguments, and the ctypes buffers it points
    to (keep them alive for the call). coeff_sets: a list of per-step tables
    ([(a, b, c)] * ns_steps each); set_of_matrix: one set index per matrix
    of the call."""
    o = Options()
    load().muon_default_options(ctypes.byref(o))
    o.nesterov = 1 if nesterov else 0
    o.momentum_form = {"ema": 0, "sgd": 1}[momentum_form]
    o.weight_decay = weight_decay
    o.scale_rule = {"rms": 0, "original": 1, "none": 2}[scale_rule]
    o.rms_target = rms_target
    o.eps = eps
    keep = None
    if coeffs is not None:
        flat = [float(x) for triple in coeffs for x in triple]
        if len(flat) != 3 * ns_steps:
            raise ValueError(f"coeffs must hold ns_steps={ns_steps} triples")
        keep = (ctypes.c_float * len(flat))(*flat)
        o.coeffs = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    o.batch_cap_elems = batch_cap_elems
    o.compute_units = compute_units
    if ns_dtype not in _NS_DTYPES:
        raise TypeError(f"ns_dtype must be None, torch.float32 or torch.bfloat16, got {ns_dtype}")
    o.ns_dtype = _NS_DTYPES[ns_dtype]
    if poly_form not in _POLY_FORMS:
        raise ValueError(f"poly_form must be one of {sorted(_POLY_FORMS)}, got {poly_form!r}")
    o.poly_form = _POLY_FORMS[poly_form]
    keep = [keep]
    if coeff_sets is not None:
        if coeffs is not None:
            raise ValueError("give either coeffs (one table) or coeff_sets, not both")
        if set_of_matrix is None:
            raise ValueError("coeff_sets needs coeff_set_of")
        flat = []
        for t in coeff_sets:
            row = [float(x) for triple in t for x in triple]
            if len(row) != 3 * ns_steps:
                raise ValueError(f"each coefficient set must hold ns_steps={ns_steps} triples")
            flat += row
        sets = (ctypes.c_float * max(1, len(flat)))(*flat)
        idx = (ctypes.c_int * max(1, len(set_of_matrix)))(*[int(v) for v in set_of_matrix])
        o.num_coeff_sets = len(coeff_sets)
        o.coeff_sets = ctypes.cast(sets, ctypes.POINTER(ctypes.c_float))
        o.coeff_set_of = ctypes.cast(idx, ctypes.POINTER(ctypes.c_int))
        keep += [sets, idx]
    return o, keep


def _dtype(t: torch.Tensor) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")
    return _DTYPES[t.dtype]


def muon_group_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                    momentum: Sequence[torch.Tensor], lr: float, beta: float = 0.95, ns_steps: int = 5,
                    stream=None) -> None:
    """C `muon_group_step`: one Muon step over same-shaped matrices with
    default options. Each list entry is an m x n tensor or an [E, m, n] bank."""
    params, grads, momentum = list(params), list(grads), list(momentum)
    if not params:
        return
    dt = _dtype(params[0])
    pdt = params[0].dtype
    _require_dtype(params, "params", pdt)
    _require_dtype(grads, "grads", pdt)
    _require_dtype(momentum, "momentum", torch.float32)
    P = [x for t in params for x in _matrices(t, "params", pdt)]
    G = [x for t in grads for x in _matrices(t, "grads", pdt)]
    M = [x for t in momentum for x in _matrices(t, "momentum", torch.float32)]
    if not (len(P) == len(G) == len(M)):
        raise ValueError("params, grads and momentum hold different numbers of matrices")
    count = len(P)
    if count == 0:
        return
    m, n = P[0][1], P[0][2]
    for lst, what in ((P, "params"), (G, "grads"), (M, "momentum")):
        if any((r, c) != (m, n) for _, r, c in lst):
            raise ValueError(f"{what}: all matrices of a group must be {m} x {n}")
    arr = ctypes.c_void_p * count
    _check(load().muon_group_step(arr(*[p for p, _, _ in P]), arr(*[p for p, _, _ in G]),
                                  arr(*[p for p, _, _ in M]), count, m, n, lr, beta, ns_steps, dt,
                                  _stream(stream)))


def muon_step(mats: Iterable[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], lr: float,
              beta: float = 0.95, ns_steps: int = 5, stream=None, **options) -> None:
    """C `muon_step`: one Muon step over (param, grad, momentum) triples of
    any shapes; options as in muon_options (nesterov, momentum_form,
    weight_decay, scale_rule, rms_target, eps, coeffs, batch_cap_elems,
    compute_units, ns_dtype: None for the tensors' dtype, or
    torch.bfloat16 to iterate float32 master tensors on bf16 MFMA;
    poly_form: "square" (default), "direct" or "folded"; coeff_sets: a list of per-step
    coefficient tables with coeff_set_of: one set index per triple, which
    applies to every matrix the triple holds)."""
    _step("muon_step", mats, lr, beta, ns_steps, stream, options)


def muon_step_noalloc(mats: Iterable[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], lr: float,
                      beta: float = 0.95, ns_steps: int = 5, stream=None, **options) -> None:
    """C `muon_step_noalloc`: muon_step with the workspace in the library's
    static device array (no device allocation; calls that overlap on one
    GPU race on it). Arguments as muon_step."""
    _step("muon_step_noalloc", mats, lr, beta, ns_steps, stream, options)


def _step(entry: str, mats, lr: float, beta: float, ns_steps: int, stream, options: dict) -> None:
    """muon_step / muon_step_noalloc: marshals the triples and calls `entry`."""
    rows = []
    dt = None
    per_entry = options.pop("coeff_set_of", None)
    set_of = [] if per_entry is not None else None
    for t, (p, g, m) in enumerate(mats):
        d = _dtype(p)
        if dt is None:
            dt = d
        elif d != dt:
            raise TypeError("all params of one call must share a dtype")
        _require_dtype([g], "grad", p.dtype)
        _require_dtype([m], "momentum", torch.float32)
        P = _matrices(p, "param", p.dtype)
        G = _matrices(g, "grad", p.dtype)
        M = _matrices(m, "momentum", torch.float32)
        if not (len(P) == len(G) == len(M)):
            raise ValueError("param, grad and momentum hold different numbers of matrices")
        for (pp, r, c), (gp, r2, c2), (mp, r3, c3) in zip(P, G, M):
            if not ((r, c) == (r2, c2) == (r3, c3)):
                raise ValueError(f"shape mismatch {r}x{c} / {r2}x{c2} / {r3}x{c3}")
            rows.append(Matrix(pp, gp, mp, r, c))
            if set_of is not None:
                set_of.append(per_entry[t])
    if not rows:
        return
    o, keep = _options(ns_steps=ns_steps, set_of_matrix=set_of, **options)
    arr = (Matrix * len(rows))(*rows)
    _check(getattr(load(), entry)(arr, len(rows), lr, beta, ns_steps, dt, ctypes.byref(o), _stream(stream)))
    del keep


def muon_step_views(views: Iterable[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], lr: float,
                    beta: float = 0.95, ns_steps: int = 5, stream=None, **options) -> None:
    """C `muon_step_views`: one Muon step over logical matrices given as
    strided 2-D views (param, grad, momentum) into physical parameters, e.g.
    `W[h*d:(h+1)*d]` (a head of a fused QKV weight), `W[:, :k]` (a column
    block) or `W[0::2]` (interleaved rows). Each view needs unit column
    stride, and the three views of a matrix share one row stride. Updates
    land in place in the viewed tensors. Options as in muon_step."""
    rows = []
    dt = None
    views = list(views)
    for (p, g, m) in views:
        _dtype(p)
        _require_dtype([g], "grad", p.dtype)
        _require_dtype([m], "momentum", torch.float32)
    for (p, g, m) in views:
        for t, what, want in ((p, "param", None), (g, "grad", None), (m, "momentum", torch.float32)):
            if not isinstance(t, torch.Tensor) or t.dim() != 2:
                raise ValueError(f"{what}: expected a 2-D tensor view")
            want = p.dtype if want is None else want
            if t.dtype != want:
                raise TypeError(f"{what}: dtype {t.dtype}, expected {want}")
            if t.stride(1) != 1 and t.shape[1] > 1:
                raise ValueError(f"{what}: column stride must be 1, got {t.stride()}")
            _on_current_device(t, what)
        ld = p.stride(0) if p.shape[0] > 1 else p.shape[1]
        for t, what in ((g, "grad"), (m, "momentum")):
            if tuple(t.shape) != tuple(p.shape):
                raise ValueError(f"{what}: shape {tuple(t.shape)} differs from param {tuple(p.shape)}")
            if t.shape[0] > 1 and t.stride(0) != ld:
                raise ValueError(f"{what}: row stride {t.stride(0)} differs from param's {ld}")
        d = _dtype(p)
        if dt is None:
            dt = d
        elif d != dt:
            raise TypeError("all params of one call must share a dtype")
        rows.append(MatrixView(p.data_ptr(), g.data_ptr(), m.data_ptr(), p.shape[0], p.shape[1], ld))
    if not rows:
        return
    o, keep = _options(ns_steps=ns_steps, set_of_matrix=options.pop("coeff_set_of", None), **options)
    arr = (MatrixView * len(rows))(*rows)
    _check(load().muon_step_views(arr, len(rows), lr, beta, ns_steps, dt, ctypes.byref(o), _stream(stream)))
    del keep


def muon_orthogonalize(inputs: Sequence[torch.Tensor], outputs: Sequence[torch.Tensor], ns_steps: int = 5,
                       stream=None, eps: float = 1e-7, coeffs=None, batch_cap_elems: int = 0,
                       compute_units: int = 0, ns_dtype=None, poly_form: str = "square") -> None:
    """C `muon_orthogonalize`: outputs[i] = NS(inputs[i]) (same shapes)."""
    inputs, outputs = list(inputs), list(outputs)
    if not inputs and not outputs:
        return
    if not inputs:
        raise ValueError("inputs and outputs hold different numbers of matrices")
    dt = _dtype(inputs[0])
    idt = inputs[0].dtype
    _require_dtype(inputs, "inputs", idt)
    _require_dtype(outputs, "outputs", idt)
    I = [x for t in inputs for x in _matrices(t, "inputs", idt)]
    O = [x for t in outputs for x in _matrices(t, "outputs", idt)]
    if len(I) != len(O):
        raise ValueError("inputs and outputs hold different numbers of matrices")
    if not I:
        return
    m, n = I[0][1], I[0][2]
    if any((r, c) != (m, n) for _, r, c in I + O):
        raise ValueError("all matrices must share one shape")
    o, keep = _options(eps=eps, coeffs=coeffs, batch_cap_elems=batch_cap_elems, compute_units=compute_units,
                       ns_steps=ns_steps, ns_dtype=ns_dtype, poly_form=poly_form)
    arr = ctypes.c_void_p * len(I)
    _check(load().muon_orthogonalize(arr(*[p for p, _, _ in I]), arr(*[p for p, _, _ in O]), len(I), m, n,
                                     ns_steps, dt, ctypes.byref(o), _stream(stream)))
    del keep


def plan_query(shapes: Sequence[Tuple[int, int]], dtype: torch.dtype = torch.bfloat16,
               batch_cap_elems: int = 0, compute_units: int = 0, ns_dtype=None, coeff_set_of=None,
               num_coeff_sets: int = 0) -> dict:
    """C `muon_plan_query` (host only): the batches and order muon_step would
    use; coeff_set_of (one set index per matrix) with num_coeff_sets splits
    the shape groups by coefficient set."""
    L = load()
    n = len(shapes)
    rows = (ctypes.c_int * max(n, 1))(*[r for r, _ in shapes])
    cols = (ctypes.c_int * max(n, 1))(*[c for _, c in shapes])
    o, _keep = _options(batch_cap_elems=batch_cap_elems, compute_units=compute_units, ns_dtype=ns_dtype)
    if coeff_set_of is not None:
        idx = (ctypes.c_int * max(1, n))(*[int(v) for v in coeff_set_of])
        _keep.append(idx)
        o.num_coeff_sets = num_coeff_sets
        o.coeff_set_of = ctypes.cast(idx, ctypes.POINTER(ctypes.c_int))
    nb = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    _check(L.muon_plan_query(rows, cols, n, _DTYPES[dtype], ctypes.byref(o), None, 0, ctypes.byref(nb), None,
                             ctypes.byref(ws)))
    batches = (PlanBatch * max(nb.value, 1))()
    order = (ctypes.c_int * max(n, 1))()
    _check(L.muon_plan_query(rows, cols, n, _DTYPES[dtype], ctypes.byref(o), batches, nb.value, ctypes.byref(nb),
                             order, ctypes.byref(ws)))
    return {"batches": [dict(group=b.group, m=b.m, n=b.n, m_pad=b.m_pad, n_pad=b.n_pad, first=b.first,
                             count=b.count, coeff_set=b.coeff_set) for b in batches[:nb.value]],
            "order": list(order[:n]), "workspace_bytes": ws.value}


def profile_enable(on: bool = True) -> bool:
    return bool(load().muon_profile_enable(1 if on else 0))


def profile_read(reset: bool = True) -> dict:
    """Per kernel kind: launches, total_ms, flops, bytes (waits for the events)."""
    L = load()
    buf = (ProfileEntry * 32)()
    n = L.muon_profile_read(buf, 32, 1 if reset else 0)
    if n < 0:
        raise MuonError(-n, L.muon_last_error().decode(errors="replace"))
    return {e.name.decode(): dict(launches=e.launches, total_ms=e.total_ms, flops=e.flops, bytes=e.bytes)
            for e in buf[:n]}


def version() -> int:
    return load().muon_version()
