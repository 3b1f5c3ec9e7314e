"""MI355X (gfx950) Fast LapSum exact soft top-k: Python binding of liblapsum.so.

This module only marshals arguments: every step of the operator runs in the
HIP kernels of ``liblapsum.so`` (see ``include/lapsum.h``).  PyTorch provides
device memory and the current HIP stream.  There is no CPU fallback: if the
library is missing or the tensors are not on a GPU, the calls raise.

    p, b = lapsum_forward(r, k, t)          # r: [rows, n] fp32 on cuda
    dr, dk = lapsum_backward(g, p, b, t)

Source of the operator: "Fast LapSum: Exact Differentiable Top-k at Million
Scale", section 2.1 (eqs. (1)-(2), analytic VJP) and section 2.2 (full-sort
solver and probabilistic bracketing).
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LAPSUM_LIBRARY selects another build of the library (the LDS-poisoning
# debug copy); by default the in-tree liblapsum.so
LIB_PATH = os.environ.get("LAPSUM_LIBRARY") or os.path.join(_HERE, "liblapsum.so")

PATH_AUTO, PATH_ONCHIP, PATH_BUCKET, PATH_BRACKET, PATH_SORT, PATH_BISECT = 0, 1, 2, 3, 4, 5
PATHS = {"auto": PATH_AUTO, "onchip": PATH_ONCHIP, "bucket": PATH_BUCKET, "bracket": PATH_BRACKET,
         "sort": PATH_SORT, "bisect": PATH_BISECT}
FLAG_BRACKET, FLAG_HIT, FLAG_FALLBACK, FLAG_OVERFLOW, FLAG_DEGENERATE, FLAG_WIDENED, FLAG_INVALID = (
    0x1, 0x2, 0x4, 0x8, 0x10, 0x20, 0x40)
ONCHIP_MAX_N = 8192
(STAGE_ONCHIP_FWD, STAGE_INIT, STAGE_SAMPLE, STAGE_SELECT, STAGE_FILTER, STAGE_BAND, STAGE_BUCKET,
 STAGE_APPLY, STAGE_ONCHIP_BWD, STAGE_BWD_REDUCE, STAGE_BWD_APPLY, STAGE_SORT, STAGE_SOLVE, STAGE_BISECT,
 STAGE_COUNT) = range(15)
STAGE_NAMES = ["onchip_fwd", "init", "sample", "select", "filter", "band", "bucket", "apply",
               "onchip_bwd", "bwd_reduce", "bwd_apply", "sort", "solve", "bisect"]

EXPORTED = ["lapsum_options_init", "lapsum_status_string", "lapsum_plan", "lapsum_bracket_indices",
            "lapsum_workspace_bytes", "lapsum_forward", "lapsum_backward", "lapsum_backward_noalloc",
            "lapsum_midpoint_workspace_bytes", "lapsum_midpoint_mass"]
NOALLOC_SCRATCH_BYTES = 1 << 20  # LAPSUM_NOALLOC_SCRATCH_BYTES


class LapsumError(RuntimeError):
    pass


class RowStats(ctypes.Structure):
    _fields_ = [("a_lo", ctypes.c_double), ("a_hi", ctypes.c_double),
                ("tail_lo", ctypes.c_double), ("tail_hi", ctypes.c_double),
                ("count_lo", ctypes.c_int64), ("count_hi", ctypes.c_int64), ("band", ctypes.c_int64),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("sample_log2", ctypes.c_int32), ("delta", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("band_capacity", ctypes.c_int64),
                ("bracket_override", ctypes.POINTER(ctypes.c_double)),
                ("stats", ctypes.c_void_p), ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("widen_steps", ctypes.c_int32), ("spread_fallback", ctypes.c_int32),
                ("k_rows", ctypes.c_void_p), ("t_rows", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("sample_log2", ctypes.c_int32), ("m", ctypes.c_int64),
                ("lo", ctypes.c_int64), ("hi", ctypes.c_int64), ("band_capacity", ctypes.c_int64),
                ("band_onchip", ctypes.c_int32), ("filter_groups", ctypes.c_int32),
                ("forward_bytes", ctypes.c_uint64), ("backward_bytes", ctypes.c_uint64)]


STATS_DTYPE_FIELDS = [f for f, _ in RowStats._fields_]
_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load liblapsum.so (built in-tree by ``python -m sparse_selection_primitive_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LapsumError(f"{LIB_PATH} is missing: build it with `python -m sparse_selection_primitive_amd.build`")
    # torch first: the library must bind to the HIP runtime torch already
    # loaded (its own copy of libamdhip64), or streams and device pointers
    # would belong to a second runtime in the same process
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.lapsum_options_init.argtypes = [ctypes.POINTER(Options)]
    lib.lapsum_options_init.restype = None
    lib.lapsum_status_string.argtypes = [ctypes.c_int]
    lib.lapsum_status_string.restype = ctypes.c_char_p
    lib.lapsum_plan.argtypes = [i64, i64, dbl, dbl, ctypes.POINTER(Options), ctypes.POINTER(PlanInfo)]
    lib.lapsum_plan.restype = ctypes.c_int
    lib.lapsum_bracket_indices.argtypes = [i64, dbl, i64, dbl, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.lapsum_bracket_indices.restype = ctypes.c_int
    lib.lapsum_workspace_bytes.argtypes = [i64, i64, dbl, dbl, ctypes.POINTER(Options)]
    lib.lapsum_workspace_bytes.restype = ctypes.c_size_t
    lib.lapsum_forward.argtypes = [vp, i64, i64, dbl, dbl, vp, vp, vp, ctypes.c_size_t, ctypes.POINTER(Options), vp]
    lib.lapsum_forward.restype = ctypes.c_int
    lib.lapsum_backward.argtypes = [vp, vp, vp, i64, i64, dbl, vp, vp, vp, ctypes.c_size_t,
                                    ctypes.POINTER(Options), vp]
    lib.lapsum_backward.restype = ctypes.c_int
    lib.lapsum_backward_noalloc.argtypes = [vp, vp, vp, i64, i64, dbl, vp, vp, ctypes.POINTER(Options), vp]
    lib.lapsum_backward_noalloc.restype = ctypes.c_int
    lib.lapsum_midpoint_workspace_bytes.argtypes = [i64, i64]
    lib.lapsum_midpoint_workspace_bytes.restype = ctypes.c_size_t
    lib.lapsum_midpoint_mass.argtypes = [vp, i64, i64, i64, dbl, vp, vp, vp, ctypes.c_size_t, vp]
    lib.lapsum_midpoint_mass.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().lapsum_status_string(rc).decode()
        raise LapsumError(f"{what}: {msg} (status {rc})")


def make_options(path="auto", sample_log2=0, delta=0.0, seed=0, band_capacity=0, bracket_override=None,
                 stats_ptr=None, stage_events=None, widen_steps=0, k_rows_ptr=None, t_rows_ptr=None,
                 spread_fallback=0):
    opt = Options()
    load_library().lapsum_options_init(ctypes.byref(opt))
    opt.path = PATHS[path] if isinstance(path, str) else int(path)
    opt.sample_log2 = int(sample_log2)
    opt.delta = float(delta)
    opt.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    opt.band_capacity = int(band_capacity)
    opt.widen_steps = int(widen_steps)
    opt.spread_fallback = int(spread_fallback)
    opt.k_rows = k_rows_ptr
    opt.t_rows = t_rows_ptr
    keep = []
    if bracket_override is not None:
        arr = (ctypes.c_double * 2)(float(bracket_override[0]), float(bracket_override[1]))
        keep.append(arr)
        opt.bracket_override = ctypes.cast(arr, ctypes.POINTER(ctypes.c_double))
    if stats_ptr is not None:
        opt.stats = ctypes.c_void_p(stats_ptr)
    if stage_events is not None:
        arr = (ctypes.c_void_p * (2 * STAGE_COUNT))(*stage_events)
        keep.append(arr)
        opt.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    opt._keep = keep  # keep ctypes buffers alive with the struct
    return opt


def plan(rows: int, n: int, k: float, t: float, **opts) -> dict:
    """Host-only: path, sample size, bracket indices, capacity and workspace sizes."""
    info = PlanInfo()
    opt = make_options(**opts)
    _check(load_library().lapsum_plan(rows, n, float(k), float(t), ctypes.byref(opt), ctypes.byref(info)),
           "lapsum_plan")
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_ if f != "reserved"}


def bracket_indices(n: int, k: float, m: int, delta: float):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().lapsum_bracket_indices(n, float(k), m, float(delta), ctypes.byref(lo), ctypes.byref(hi)),
           "lapsum_bracket_indices")
    return lo.value, hi.value


def workspace_bytes(rows: int, n: int, k: float, t: float, **opts) -> int:
    opt = make_options(**opts)
    return int(load_library().lapsum_workspace_bytes(rows, n, float(k), float(t), ctypes.byref(opt)))


# --------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _workspace(nbytes: int, device):
    """A 256-byte-aligned device buffer of at least nbytes for one call:
    (buffer, aligned pointer, usable bytes).

    It comes from torch's caching allocator on the current stream, which is
    stream-ordered: once the call has been enqueued and the buffer dropped,
    its memory goes back to the pool and is handed out again only to work
    ordered after this call on the same stream (or to another stream after
    the allocator has seen this stream's work end).  So calls on different
    streams never share scratch memory, and a buffer is never reused while
    a kernel that reads it is still queued."""
    torch = _torch()
    if nbytes == 0:
        return None, None, 0
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    ptr = buf.data_ptr()
    return buf, ptr + ((-ptr) % 256), buf.numel() - ((-ptr) % 256)


def _as_rows(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise LapsumError(f"{name} must be a GPU tensor (no CPU path exists)")
    if x.dtype != torch.float32:
        raise LapsumError(f"{name} must be float32")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2:
        raise LapsumError(f"{name} must be [rows, n] or [n]")
    return x.contiguous()


def _per_row(x, rows: int, dev, name: str):
    """A per-row parameter tensor as a contiguous float64 [rows] tensor on
    dev (None for a scalar)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        return None
    if x.numel() != rows:
        raise LapsumError(f"{name} must be a scalar or hold one value per row ({rows})")
    return x.detach().reshape(rows).to(device=dev, dtype=torch.float64).contiguous()


def lapsum_forward(r, k, t, *, path="auto", sample_log2=0, delta=0.0, seed=0, band_capacity=0,
                   bracket_override=None, stats=False, stage_events=None, out=None, widen_steps=0,
                   spread_fallback=False):
    """p, b (and per-row stats if stats=True) for scores r [rows, n] fp32 on GPU.

    k and t are floats, or tensors with one value per row (on-chip and
    full-sort paths).  p is fp32 [rows, n]; b is fp64 [rows].  Stats is an
    int/float dict of per-row tensors (bracket ends, tail sums, counts, band
    size, flags).  spread_fallback: on the bracketing path, rows whose
    bracket misses are solved by the whole-row bucket launches on every
    workgroup instead of widening and one workgroup's fallback."""
    torch = _torch()
    lib = load_library()
    r2 = _as_rows(r, "r")
    rows, n = r2.shape
    dev = r2.device
    with torch.cuda.device(dev):
        kr, tr = _per_row(k, rows, dev, "k"), _per_row(t, rows, dev, "t")
        ks = 0.0 if kr is not None else float(k)
        ts = 0.0 if tr is not None else float(t)
        p = torch.empty_like(r2) if out is None else out[0]
        b = torch.empty(rows, dtype=torch.float64, device=dev) if out is None else out[1]
        st = torch.empty(rows * ctypes.sizeof(RowStats), dtype=torch.uint8, device=dev) if stats else None
        opt = make_options(path, sample_log2, delta, seed, band_capacity, bracket_override,
                           st.data_ptr() if st is not None else None, stage_events, widen_steps,
                           spread_fallback=int(bool(spread_fallback)))
        opt.k_rows = kr.data_ptr() if kr is not None else None
        opt.t_rows = tr.data_ptr() if tr is not None else None
        nbytes = int(lib.lapsum_workspace_bytes(rows, n, ks, ts, ctypes.byref(opt)))
        ws, wptr, wlen = _workspace(nbytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.lapsum_forward(r2.data_ptr(), rows, n, ks, ts, p.data_ptr(), b.data_ptr(),
                                wptr, wlen, ctypes.byref(opt), stream)
        del ws  # back to the pool, ordered after this call on its stream
        _check(rc, "lapsum_forward")
    if r.dim() == 1:
        p, b = p[0], b
    if stats:
        return p, b, decode_stats(st, rows)
    return p, b


def decode_stats(buf, rows: int) -> dict:
    """Per-row lapsum_row_stats (device bytes) -> dict of CPU tensors."""
    torch = _torch()
    raw = buf.cpu().numpy().tobytes()
    arr = (RowStats * rows).from_buffer_copy(raw)
    out = {f: [getattr(arr[i], f) for i in range(rows)] for f in STATS_DTYPE_FIELDS if f != "reserved"}
    return {f: torch.tensor(v) for f, v in out.items()}


def lapsum_backward(g, p, b, t, *, stats_buf=None, stage_events=None, out=None):
    """dr [rows, n] fp32 and dk [rows] fp32: the analytic VJP of the forward
    (t a float or one value per row, as in the forward)."""
    torch = _torch()
    lib = load_library()
    g2 = _as_rows(g, "g")
    p2 = _as_rows(p, "p")
    if g2.shape != p2.shape:
        raise LapsumError("g and p must have the same shape")
    rows, n = g2.shape
    dev = g2.device
    if not (isinstance(b, torch.Tensor) and b.is_cuda and b.dtype == torch.float64 and b.numel() == rows):
        raise LapsumError("b must be a float64 GPU tensor with one entry per row")
    with torch.cuda.device(dev):
        dr = torch.empty_like(g2) if out is None else out[0]
        dk = torch.empty(rows, dtype=torch.float32, device=dev) if out is None else out[1]
        tr = _per_row(t, rows, dev, "t")
        ts = 1.0 if tr is not None else float(t)
        opt = make_options(stats_ptr=stats_buf.data_ptr() if stats_buf is not None else None,
                           stage_events=stage_events)
        opt.t_rows = tr.data_ptr() if tr is not None else None
        nbytes = int(lib.lapsum_workspace_bytes(rows, n, 0.5 * n, ts, None))
        ws, wptr, wlen = _workspace(nbytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.lapsum_backward(g2.data_ptr(), p2.data_ptr(), b.contiguous().data_ptr(), rows, n, ts,
                                 dr.data_ptr(), dk.data_ptr(), wptr, wlen, ctypes.byref(opt), stream)
        del ws
        _check(rc, "lapsum_backward")
    if g.dim() == 1:
        dr = dr[0]
    return dr, dk


def lapsum_backward_noalloc(g, p, b, t, *, out=None):
    """The backward through the entry point that allocates nothing: the
    library keeps the streaming pass's partials in its own fixed device
    buffer (one per device), so no workspace is passed.  Calls that overlap
    on one device race on that buffer.  With ``out`` = (dr, dk) no tensor is
    allocated here either."""
    torch = _torch()
    lib = load_library()
    g2 = _as_rows(g, "g")
    p2 = _as_rows(p, "p")
    if g2.shape != p2.shape:
        raise LapsumError("g and p must have the same shape")
    rows, n = g2.shape
    dev = g2.device
    if not (isinstance(b, torch.Tensor) and b.is_cuda and b.dtype == torch.float64 and b.numel() == rows):
        raise LapsumError("b must be a float64 GPU tensor with one entry per row")
    with torch.cuda.device(dev):
        dr = torch.empty_like(g2) if out is None else out[0]
        dk = torch.empty(rows, dtype=torch.float32, device=dev) if out is None else out[1]
        tr = _per_row(t, rows, dev, "t")
        ts = 1.0 if tr is not None else float(t)
        opt = make_options()
        opt.t_rows = tr.data_ptr() if tr is not None else None
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.lapsum_backward_noalloc(g2.data_ptr(), p2.data_ptr(), b.contiguous().data_ptr(), rows, n, ts,
                                         dr.data_ptr(), dk.data_ptr(), ctypes.byref(opt), stream)
        _check(rc, "lapsum_backward_noalloc")
    if g.dim() == 1:
        dr = dr[0]
    return dr, dk


def midpoint_mass(r, k: int, t: float):
    """DFTopK diagnostic (section 2.3): per row, the fixed threshold
    b_mid = (s_(k) + s_(k+1))/2 of the k-th and (k+1)-th largest scores and
    the Laplace mass sum_i F((r_i - b_mid)/t) at it (fp64 tensors [rows]);
    mass / k - 1 is the fixed midpoint's budget drift.  k: integer in
    [1, n - 1]."""
    torch = _torch()
    lib = load_library()
    r2 = _as_rows(r, "r")
    rows, n = r2.shape
    if int(k) != k:
        raise LapsumError("midpoint_mass: k must be an integer")
    dev = r2.device
    with torch.cuda.device(dev):
        b_mid = torch.empty(rows, dtype=torch.float64, device=dev)
        mass = torch.empty(rows, dtype=torch.float64, device=dev)
        nbytes = int(lib.lapsum_midpoint_workspace_bytes(rows, n))
        ws, wptr, wlen = _workspace(max(nbytes, 1), dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.lapsum_midpoint_mass(r2.data_ptr(), rows, n, int(k), float(t), b_mid.data_ptr(), mass.data_ptr(),
                                      wptr, wlen, stream)
        del ws
        _check(rc, "lapsum_midpoint_mass")
    return b_mid, mass


def soft_topk(r, k, t, **kw):
    """Differentiable soft top-k: autograd wrapper over the two entry points.

    k may be a float or a tensor with one budget per row; a tensor k that
    requires grad receives dk, the derivative of the loss with respect to each
    row's budget.  t (float or one per row) gets no gradient."""
    torch = _torch()

    class _LapSum(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, kk):
            p, b = lapsum_forward(x, kk if kk is not None else k, t, **kw)
            ctx.save_for_backward(p, b)
            ctx.k_meta = None if kk is None else (kk.shape, kk.dtype, kk.device)
            return p

        @staticmethod
        def backward(ctx, gp):
            p, b = ctx.saved_tensors
            dr, dk = lapsum_backward(gp.contiguous(), p, b, t)
            gk = None
            if ctx.k_meta is not None and ctx.needs_input_grad[1]:
                shape, dtype, device = ctx.k_meta
                gk = dk.to(device=device, dtype=dtype).reshape(shape)
            return dr, gk

    return _LapSum.apply(r, k if isinstance(k, torch.Tensor) else None)


class Operator:
    """Prepared calls for a fixed (rows, n, k, t) and options: the options
    struct, workspace and stream are resolved once, so each call is a single
    C-ABI call with raw device pointers (for tight loops and benchmarks).
    Outputs are written into caller-provided tensors."""

    def __init__(self, rows: int, n: int, k: float, t: float, device=None, stream=None, path="auto", seed=0,
                 sample_log2=0, delta=0.0, band_capacity=0, bracket_override=None, stats_buf=None, widen_steps=0,
                 k_rows=None, t_rows=None, spread_fallback=False):
        """k_rows / t_rows: optional per-row values (tensors of one value per
        row; they replace k / t, which are then not used)."""
        torch = _torch()
        self.lib = load_library()
        self.rows, self.n, self.k, self.t = int(rows), int(n), float(k), float(t)
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.opt = make_options(path, sample_log2, delta, seed, band_capacity, bracket_override,
                                stats_buf.data_ptr() if stats_buf is not None else None, widen_steps=widen_steps,
                                spread_fallback=int(bool(spread_fallback)))
        self._k_rows = _per_row(k_rows, self.rows, self.device, "k_rows")
        self._t_rows = _per_row(t_rows, self.rows, self.device, "t_rows")
        self.opt.k_rows = self._k_rows.data_ptr() if self._k_rows is not None else None
        self.opt.t_rows = self._t_rows.data_ptr() if self._t_rows is not None else None
        nbytes = int(self.lib.lapsum_workspace_bytes(self.rows, self.n, self.k, self.t, ctypes.byref(self.opt)))
        self._ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device) if nbytes else None
        if self._ws is not None:
            ptr = self._ws.data_ptr()
            self.wptr, self.wlen = ptr + ((-ptr) % 256), self._ws.numel() - ((-ptr) % 256)
        else:
            self.wptr, self.wlen = None, 0
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.stream = s.cuda_stream
        self._opt_ref = ctypes.byref(self.opt)
        self._ev_arrays = {}

    def _opt_with_events(self, events):
        if events is None:
            self.opt.stage_events = None
            return self._opt_ref
        arr = (ctypes.c_void_p * (2 * STAGE_COUNT))(*events)
        self._ev_keep = arr
        self.opt.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        return self._opt_ref

    def forward(self, r, p, b, stage_events=None, stream=None):
        """stream: a raw hipStream_t (int) overriding the prepared one, e.g.
        the capturing stream inside ``torch.cuda.graph``."""
        rc = self.lib.lapsum_forward(r.data_ptr(), self.rows, self.n, self.k, self.t, p.data_ptr(), b.data_ptr(),
                                     self.wptr, self.wlen, self._opt_with_events(stage_events),
                                     self.stream if stream is None else stream)
        if rc:
            _check(rc, "lapsum_forward")

    def backward(self, g, p, b, dr, dk, stage_events=None, stream=None):
        rc = self.lib.lapsum_backward(g.data_ptr(), p.data_ptr(), b.data_ptr(), self.rows, self.n, self.t,
                                      dr.data_ptr(), dk.data_ptr(), self.wptr, self.wlen,
                                      self._opt_with_events(stage_events),
                                      self.stream if stream is None else stream)
        if rc:
            _check(rc, "lapsum_backward")
