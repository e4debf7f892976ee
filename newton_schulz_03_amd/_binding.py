"""ctypes binding of libmuon_mi355x.so: argument marshalling only.

Every step of the computation runs in the HIP library.  torch is used for
device memory (tensors, the workspace) and for the current HIP stream.  If the
library is missing the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmuon_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "muon_mi355x.h")

MUON_BF16, MUON_FP32 = 0, 1
MUON_OK, MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_ERR_HIP = range(5)
MAX_DIM = 65536
NOALLOC_MAX_WORKSPACE = 256 << 20  # MUON_NOALLOC_MAX_WORKSPACE
SIZE_MAX = ctypes.c_size_t(-1).value

QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)

EXPORTED = ("muon_workspace_bytes", "muon_workspace_bytes_ex", "muon_ns_batched",
            "muon_ns_batched_noalloc",
            "muon_step_batched",
            "muon_adamw_workspace_bytes", "muon_adamw_batched",
            "muon_status_string", "muon_last_error_detail", "muon_timing_enable",
            "muon_timing_read", "muon_timing_reset", "muon_hbm_stream")
KERNELS = ("prepare", "norm", "gram", "poly", "prod", "finish", "adamw", "prod_finish", "prod_first",
           "quant8", "gram8", "poly8", "prod8", "mom_in", "mom_out")


class MuonError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


class NsParams(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int32), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("c", ctypes.c_float), ("eps", ctypes.c_float), ("cu_budget", ctypes.c_int32),
                ("fp8_steps", ctypes.c_int32)]


class StepParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float), ("nesterov", ctypes.c_int32),
                ("ns", NsParams), ("momentum_host", ctypes.c_int32)]


class AdamWParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int32)]


_lib_handle: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m newton_schulz_03_amd.build, or __graft_entry__.build())")
    # torch brings its own copy of the HIP runtime.  Loaded first, it serves
    # this library too (one runtime per process); loaded after this library,
    # the library's runtime reported no device (hipErrorNoDevice) on MI355X.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i32, i64p, vpp, vp, sz = (ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_size_t)
    lib.muon_workspace_bytes.argtypes = [i32, i64p, i64p, i32]
    lib.muon_workspace_bytes.restype = sz
    lib.muon_workspace_bytes_ex.argtypes = [i32, i64p, i64p, i32, ctypes.c_uint32]
    lib.muon_workspace_bytes_ex.restype = sz
    lib.muon_ns_batched.argtypes = [i32, i64p, i64p, vpp, vpp, i32, ctypes.POINTER(NsParams), vp,
                                    sz, vp]
    lib.muon_ns_batched.restype = i32
    lib.muon_ns_batched_noalloc.argtypes = [i32, i64p, i64p, vpp, vpp, i32,
                                            ctypes.POINTER(NsParams), vp]
    lib.muon_ns_batched_noalloc.restype = i32
    lib.muon_step_batched.argtypes = [i32, i64p, i64p, vpp, vpp, vpp, i32,
                                      ctypes.POINTER(StepParams), vp, sz, vp]
    lib.muon_step_batched.restype = i32
    lib.muon_adamw_workspace_bytes.argtypes = [i32, i64p]
    lib.muon_adamw_workspace_bytes.restype = sz
    lib.muon_adamw_batched.argtypes = [i32, i64p, vpp, vpp, vpp, vpp, i32,
                                       ctypes.POINTER(AdamWParams), vp, sz, vp]
    lib.muon_adamw_batched.restype = i32
    lib.muon_status_string.argtypes = [i32]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_last_error_detail.argtypes = []
    lib.muon_last_error_detail.restype = ctypes.c_char_p
    lib.muon_timing_enable.argtypes = [i32]
    lib.muon_timing_enable.restype = i32
    lib.muon_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.muon_timing_read.restype = i32
    lib.muon_timing_reset.argtypes = []
    lib.muon_timing_reset.restype = i32
    lib.muon_hbm_stream.argtypes = [i32, vpp, i32, vpp, sz, i32, vp]
    lib.muon_hbm_stream.restype = i32
    _lib_handle = lib
    return lib


def status_string(status: int) -> str:
    return load_library().muon_status_string(status).decode()


def last_error_detail() -> str:
    return load_library().muon_last_error_detail().decode()


def _check(status: int, where: str) -> None:
    if status != MUON_OK:
        raise MuonError(status, where, last_error_detail())


def _i64_array(vals: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def _ptr_array(vals: Sequence[int]):
    return (ctypes.c_void_p * max(1, len(vals)))(*vals)


def _dtype_code(dtype) -> int:
    import torch

    if dtype == torch.bfloat16:
        return MUON_BF16
    if dtype == torch.float32:
        return MUON_FP32
    raise TypeError(f"unsupported dtype {dtype}: use torch.bfloat16 or torch.float32")


MUON_WS_FP8, MUON_WS_MOMENTUM_HOST = 1, 2


def workspace_bytes(shapes: Sequence[Tuple[int, int]], dtype, fp8: bool = False,
                    momentum_host: bool = False) -> int:
    """Device workspace bytes for a batch of (rows, cols) shapes (fp8: for a bf16
    call with e4m3 steps; momentum_host: for a step with the momentum in host memory)."""
    lib = load_library()
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    rows = _i64_array([int(r) for r, _ in shapes])
    cols = _i64_array([int(c) for _, c in shapes])
    flags = (MUON_WS_FP8 if fp8 else 0) | (MUON_WS_MOMENTUM_HOST if momentum_host else 0)
    if flags:
        n = lib.muon_workspace_bytes_ex(len(shapes), rows, cols, code, flags)
    else:
        n = lib.muon_workspace_bytes(len(shapes), rows, cols, code)
    if n == SIZE_MAX:
        raise MuonError(MUON_ERR_INVALID_ARG, "muon_workspace_bytes", last_error_detail())
    return int(n)


def allocate_workspace(shapes, dtype, device, fp8: bool = False, momentum_host: bool = False):
    """A uint8 device tensor usable as the workspace of a call over `shapes`
    (fp8: with e4m3 steps; momentum_host: a step with the momentum in host memory)."""
    import torch

    n = workspace_bytes(shapes, dtype, fp8, momentum_host)
    ws = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + max(n, 1)]


def _stream_handle(device) -> int:
    import torch

    return int(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(ts, name):
    import torch

    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError(f"{name}: tensors must live on a HIP device, got {dev}")
    for t in ts:
        if t.device != dev or t.dtype != ts[0].dtype:
            raise ValueError(f"{name}: every tensor must share one device and dtype")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous 2-D matrices")
    return dev


def ns_batched(xs: Sequence, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
               out: Optional[Sequence] = None, workspace=None, cu_budget: int = 0,
               fp8_steps: int = 0) -> List:
    """Newton-Schulz orthogonalization of a ragged batch of matrices on the GPU.

    Returns the outputs (new tensors, or `out` when given; out[i] may be xs[i]).
    Runs on the current HIP stream of the tensors' device.  cu_budget > 0 keeps
    the matrix-core launches to that many CUs (the rest stay free for other
    streams).  fp8_steps > 0 (bf16, fewer than steps): the first fp8_steps
    iterations take block-scaled e4m3 operands.
    """
    import torch

    lib = load_library()
    xs = list(xs)
    if not xs:
        return []
    dev = _check_tensors(xs, "xs")
    if out is None:
        out = [torch.empty_like(x) for x in xs]
    out = list(out)
    if len(out) != len(xs):
        raise ValueError("out must have one tensor per input")
    _check_tensors(out + xs, "out")
    shapes = [tuple(x.shape) for x in xs]
    if any(tuple(o.shape) != s for o, s in zip(out, shapes)):
        raise ValueError("out shapes must match the inputs")
    code = _dtype_code(xs[0].dtype)
    if workspace is None:
        workspace = allocate_workspace(shapes, xs[0].dtype, dev, fp8=fp8_steps > 0)
    a, b, c = (float(v) for v in coeffs)
    p = NsParams(int(steps), a, b, c, float(eps), int(cu_budget), int(fp8_steps))
    with torch.cuda.device(dev):
        st = lib.muon_ns_batched(len(xs), _i64_array([s[0] for s in shapes]),
                                 _i64_array([s[1] for s in shapes]),
                                 _ptr_array([x.data_ptr() for x in xs]),
                                 _ptr_array([o.data_ptr() for o in out]), code, ctypes.byref(p),
                                 ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                 ctypes.c_void_p(_stream_handle(dev)))
    _check(st, "muon_ns_batched")
    return out


def ns_batched_noalloc(xs: Sequence, out: Sequence, steps: int = 5, coeffs=QUINTIC,
                       eps: float = 1e-7, cu_budget: int = 0, fp8_steps: int = 0) -> List:
    """ns_batched through the allocation-free entry point: no workspace (the
    library's own array of NOALLOC_MAX_WORKSPACE bytes per GPU serves), and the
    caller passes the outputs.  Calls that overlap on one GPU race."""
    import torch

    lib = load_library()
    xs, out = list(xs), list(out)
    if not xs:
        return out
    if len(out) != len(xs):
        raise ValueError("out must have one tensor per input")
    dev = _check_tensors(out + xs, "xs/out")
    shapes = [tuple(x.shape) for x in xs]
    if any(tuple(o.shape) != s for o, s in zip(out, shapes)):
        raise ValueError("out shapes must match the inputs")
    a, b, c = (float(v) for v in coeffs)
    p = NsParams(int(steps), a, b, c, float(eps), int(cu_budget), int(fp8_steps))
    with torch.cuda.device(dev):
        st = lib.muon_ns_batched_noalloc(len(xs), _i64_array([s[0] for s in shapes]),
                                         _i64_array([s[1] for s in shapes]),
                                         _ptr_array([x.data_ptr() for x in xs]),
                                         _ptr_array([o.data_ptr() for o in out]),
                                         _dtype_code(xs[0].dtype), ctypes.byref(p),
                                         ctypes.c_void_p(_stream_handle(dev)))
    _check(st, "muon_ns_batched_noalloc")
    return out


def step_batched(ws: Sequence, gs: Sequence, ms: Sequence, lr: float = 0.02, beta: float = 0.95,
                 nesterov: bool = False, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7,
                 workspace=None, momentum_host: bool = False, cu_budget: int = 0,
                 fp8_steps: int = 0) -> None:
    """One Muon step over a ragged batch, in place on ws (weights) and ms (momentum).

    momentum_host: the momenta are pinned host tensors (pin_memory), updated in
    place: the step copies them to the device and back in chunks, overlapped
    with the Newton-Schulz work.
    """
    import torch

    lib = load_library()
    ws, gs, ms = list(ws), list(gs), list(ms)
    if not (len(ws) == len(gs) == len(ms)):
        raise ValueError("ws, gs and ms must have the same length")
    if not ws:
        return
    if momentum_host:
        dev = _check_tensors(ws + gs, "ws/gs")
        for m in ms:
            if m.device.type != "cpu" or not m.is_pinned() or m.dtype != ws[0].dtype or \
                    m.dim() != 2 or not m.is_contiguous():
                raise ValueError("ms: with momentum_host, every momentum must be a pinned, "
                                 "contiguous 2-D host tensor of the weights' dtype")
    else:
        dev = _check_tensors(ws + gs + ms, "ws/gs/ms")
    shapes = [tuple(w.shape) for w in ws]
    if any(tuple(g.shape) != s or tuple(m.shape) != s for g, m, s in zip(gs, ms, shapes)):
        raise ValueError("w, g and m of one matrix must share a shape")
    code = _dtype_code(ws[0].dtype)
    if workspace is None:
        workspace = allocate_workspace(shapes, ws[0].dtype, dev, fp8=fp8_steps > 0,
                                       momentum_host=momentum_host)
    a, b, c = (float(v) for v in coeffs)
    p = StepParams(float(lr), float(beta), 1 if nesterov else 0,
                   NsParams(int(steps), a, b, c, float(eps), int(cu_budget), int(fp8_steps)),
                   1 if momentum_host else 0)
    with torch.cuda.device(dev):
        st = lib.muon_step_batched(len(ws), _i64_array([s[0] for s in shapes]),
                                   _i64_array([s[1] for s in shapes]),
                                   _ptr_array([w.data_ptr() for w in ws]),
                                   _ptr_array([g.data_ptr() for g in gs]),
                                   _ptr_array([m.data_ptr() for m in ms]), code, ctypes.byref(p),
                                   ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                   ctypes.c_void_p(_stream_handle(dev)))
    _check(st, "muon_step_batched")


def adamw_workspace_bytes(numels: Sequence[int]) -> int:
    lib = load_library()
    numels = list(numels)
    n = lib.muon_adamw_workspace_bytes(len(numels), _i64_array(numels) if numels else None)
    if n == SIZE_MAX:
        raise MuonError(MUON_ERR_INVALID_ARG, "muon_adamw_workspace_bytes", last_error_detail())
    return n


def adamw_batched(params: Sequence, grads: Sequence, exp_avgs: Sequence, exp_avg_sqs: Sequence,
                  lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                  weight_decay: float = 1e-2, step: int = 1, workspace=None) -> None:
    """One AdamW step over a ragged batch of tensors, in place on params and the moments.

    params/grads: bf16 or fp32 (one dtype for all), contiguous; exp_avgs and
    exp_avg_sqs: fp32, same shapes.  `step` is the number of the step being
    taken (1 for the first).  Runs on the current HIP stream.
    """
    import torch

    lib = load_library()
    ps, gs, ms, vs = list(params), list(grads), list(exp_avgs), list(exp_avg_sqs)
    if not ps:
        return
    if not (len(ps) == len(gs) == len(ms) == len(vs)):
        raise ValueError("params, grads and moments must have one tensor each per entry")
    dev = ps[0].device
    if dev.type != "cuda":
        raise ValueError(f"params must live on a HIP device, got {dev}")
    for group, want in ((ps, ps[0].dtype), (gs, ps[0].dtype), (ms, torch.float32),
                        (vs, torch.float32)):
        for t in group:
            if t.device != dev or t.dtype != want or not t.is_contiguous():
                raise ValueError("tensors must be contiguous on one device; p and g share a "
                                 "dtype, the moments are float32")
    for p, g, m, v in zip(ps, gs, ms, vs):
        if not (p.shape == g.shape == m.shape == v.shape):
            raise ValueError("p, g, m and v of one entry must have the same shape")
    code = _dtype_code(ps[0].dtype)
    numels = [p.numel() for p in ps]
    if workspace is None:
        n = adamw_workspace_bytes(numels)
        ws = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device=dev)
        off = (-ws.data_ptr()) % 256
        workspace = ws[off:off + max(n, 1)]
    b1, b2 = (float(b) for b in betas)
    prm = AdamWParams(float(lr), b1, b2, float(eps), float(weight_decay), int(step))
    with torch.cuda.device(dev):
        st = lib.muon_adamw_batched(len(ps), _i64_array(numels),
                                    _ptr_array([t.data_ptr() for t in ps]),
                                    _ptr_array([t.data_ptr() for t in gs]),
                                    _ptr_array([t.data_ptr() for t in ms]),
                                    _ptr_array([t.data_ptr() for t in vs]), code,
                                    ctypes.byref(prm), ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel(), ctypes.c_void_p(_stream_handle(dev)))
    _check(st, "muon_adamw_batched")


def hbm_stream(ins: Sequence, outs: Sequence, nontemporal: bool = False) -> None:
    """Plain HBM stream (measurement aid): outs[k] <- ins[k % len(ins)] (two inputs
    into one output: their bitwise XOR), on the current stream.  1 or 2 inputs
    and outputs, uint8 device tensors of one size, a multiple of 16384 bytes."""
    import torch

    ins, outs = list(ins), list(outs)
    n = ins[0].numel() * ins[0].element_size()
    for t in ins + outs:
        if t.device.type != "cuda" or not t.is_contiguous() or t.numel() * t.element_size() != n:
            raise ValueError("hbm_stream: contiguous device tensors of one size")
    dev = ins[0].device
    with torch.cuda.device(dev):
        st = load_library().muon_hbm_stream(len(ins), _ptr_array([t.data_ptr() for t in ins]),
                                            len(outs), _ptr_array([t.data_ptr() for t in outs]),
                                            n, 1 if nontemporal else 0,
                                            ctypes.c_void_p(_stream_handle(dev)))
    _check(st, "muon_hbm_stream")


def timing_enable(on: bool = True) -> None:
    """Record HIP events around every kernel launch (process-wide) while on."""
    _check(load_library().muon_timing_enable(1 if on else 0), "muon_timing_enable")


def timing_reset() -> None:
    _check(load_library().muon_timing_reset(), "muon_timing_reset")


def timing_read() -> dict:
    """{kernel name: (total milliseconds, launches)} since the last reset."""
    lib = load_library()
    out = {}
    for k, name in enumerate(KERNELS):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib.muon_timing_read(k, ctypes.byref(ms), ctypes.byref(n)), "muon_timing_read")
        out[name] = (ms.value, n.value)
    return out
