"""ctypes binding of libmuon (include/libmuon.h).  Argument marshalling only:
every step of the optimizer runs in the library's HIP kernels.  Torch
tensors are accepted for device memory (their data_ptr()) and the current
HIP stream; nothing here computes on them.

There is no fallback: if libmuon.so is missing or fails to load, every call
raises."""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuon.so")

MUON_OK = 0
STATUS = {0: "MUON_OK", -1: "MUON_E_ARG", -2: "MUON_E_SHAPE", -3: "MUON_E_DTYPE",
          -4: "MUON_E_METHOD", -5: "MUON_E_WORKSPACE", -6: "MUON_E_HIP", -7: "MUON_E_PLAN",
          -8: "MUON_E_CAPACITY"}
MUON_NS_STANDARD, MUON_NS_GRAM, MUON_NS_AUTO, MUON_NS_GRAM_RESTART = 0, 1, 2, 3
MUON_F32, MUON_BF16 = 0, 1
MUON_KIND_MUON, MUON_KIND_ADAMW = 0, 1
MUON_SCALE_MOONLIGHT, MUON_SCALE_SPECTRAL, MUON_SCALE_UNIT_RMS = 0, 1, 2
MUON_COEFF_QUINTIC, MUON_COEFF_HYBRID = 0, 1

EXPORTED = ["muon_plan_create", "muon_plan_destroy", "muon_plan_workspace_bytes",
            "muon_plan_buckets", "muon_plan_units", "muon_step", "ns_orthogonalize",
            "ns_orthogonalize_workspace_bytes", "muon_timing_enable", "muon_timing_collect",
            "muon_ns_coefficients", "muon_status_string", "muon_version", "muon_probe_mfma",
            "muon_probe_copy", "ns_orthogonalize_noalloc", "muon_probe_copy_lds"]
NOALLOC_SCRATCH_BYTES = 64 << 20


class MuonError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")


class MuonParamShape(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("split_rows", ctypes.c_int64), ("scale_dim", ctypes.c_int64)]


class MuonParamPtrs(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("update_out", ctypes.c_void_p)]


class MuonHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
                ("coeffs", ctypes.POINTER(ctypes.c_float)), ("rms_scale", ctypes.c_float),
                ("adam_lr", ctypes.c_float), ("adam_beta1", ctypes.c_float),
                ("adam_beta2", ctypes.c_float), ("adam_eps", ctypes.c_float),
                ("adam_weight_decay", ctypes.c_float), ("adam_step", ctypes.c_int64),
                ("scale_mode", ctypes.c_int32), ("extra_scale", ctypes.c_float)]


class MuonPlanOptions(ctypes.Structure):
    _fields_ = [("ns_method", ctypes.c_int32), ("ns_dtype", ctypes.c_int32)]


class MuonKernelTiming(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


_lib = None


def lib():
    """Load libmuon.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmuon.so not built at {LIB_PATH}; run "
                           "python -m matrix_orthogonalizing_optimizer_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.muon_plan_create.argtypes = [ctypes.POINTER(MuonParamShape), i32, ctypes.POINTER(MuonPlanOptions),
                                   ctypes.POINTER(vp)]
    L.muon_plan_create.restype = i32
    L.muon_plan_destroy.argtypes = [vp]
    L.muon_plan_destroy.restype = None
    L.muon_plan_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    L.muon_plan_workspace_bytes.restype = i32
    L.muon_plan_buckets.argtypes = [vp, ctypes.POINTER(i32), sz, ctypes.POINTER(sz)]
    L.muon_plan_buckets.restype = i32
    L.muon_plan_units.argtypes = [vp, ctypes.POINTER(i64), sz, ctypes.POINTER(sz)]
    L.muon_plan_units.restype = i32
    L.muon_step.argtypes = [vp, ctypes.POINTER(MuonParamPtrs), i32, ctypes.POINTER(MuonHparams), vp, sz, vp]
    L.muon_step.restype = i32
    L.ns_orthogonalize.argtypes = [vp, i64, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float), i32, vp,
                                   sz, vp]
    L.ns_orthogonalize.restype = i32
    L.ns_orthogonalize_noalloc.argtypes = [vp, i64, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float), i32,
                                           vp]
    L.ns_orthogonalize_noalloc.restype = i32
    L.ns_orthogonalize_workspace_bytes.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz)]
    L.ns_orthogonalize_workspace_bytes.restype = i32
    L.muon_timing_enable.argtypes = [i32]
    L.muon_timing_enable.restype = i32
    L.muon_timing_collect.argtypes = [ctypes.POINTER(MuonKernelTiming), i32, ctypes.POINTER(i32)]
    L.muon_timing_collect.restype = i32
    L.muon_probe_mfma.argtypes = [i32, i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.muon_probe_mfma.restype = i32
    L.muon_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.muon_probe_copy.restype = i32
    L.muon_probe_copy_lds.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.muon_probe_copy_lds.restype = i32
    L.muon_ns_coefficients.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_float), sz]
    L.muon_ns_coefficients.restype = i32
    L.muon_status_string.argtypes = [i32]
    L.muon_status_string.restype = ctypes.c_char_p
    L.muon_version.argtypes = []
    L.muon_version.restype = i32
    _lib = L
    return L


def _check(fn, st):
    if st != MUON_OK:
        raise MuonError(fn, st)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _coeff_array(coeffs, steps):
    """Host array of steps x 3 floats for the library, or None (the quintic).
    ``coeffs``: one (a, b, c) triple (used at every step) or exactly ``steps``
    triples of finite numbers; anything else raises ValueError before the
    library reads 3 * steps floats from it."""
    if coeffs is None:
        return None
    import math
    if len(coeffs) == 3 and not hasattr(coeffs[0], "__len__"):
        coeffs = [coeffs] * int(steps)
    if len(coeffs) != steps:
        raise ValueError(f"coeffs: {len(coeffs)} rows for {steps} Newton-Schulz steps")
    flat = []
    for row in coeffs:
        if not hasattr(row, "__len__") or len(row) != 3:
            raise ValueError("coeffs: every row must be an (a, b, c) triple")
        vals = [float(x) for x in row]
        if not all(math.isfinite(v) for v in vals):
            raise ValueError("coeffs: non-finite coefficient")
        flat.extend(vals)
    return (ctypes.c_float * max(len(flat), 3))(*flat)


def _device_index(stream):
    """Index of the GPU the call's kernels run on: the stream's device, or
    the current device when the current stream is used."""
    import torch
    if stream is None or isinstance(stream, int):
        return torch.cuda.current_device()
    return stream.device.index


def _check_device(name, t, device_index):
    """A torch tensor handed to the library must live on the GPU the kernels
    run on: its data_ptr() is used as a device address there."""
    if t is None or isinstance(t, int) or not hasattr(t, "data_ptr"):
        return
    if not t.is_cuda:
        raise ValueError(f"{name}: a {t.device} tensor; the library needs device memory")
    if device_index is not None and t.device.index != device_index:
        raise ValueError(f"{name}: on {t.device}, the kernels run on cuda:{device_index}")


def _check_call_device(name, t, stream):
    """_check_device against the call's GPU, looked up only for device tensors."""
    if t is None or isinstance(t, int) or not hasattr(t, "data_ptr"):
        return
    _check_device(name, t, _device_index(stream) if t.is_cuda else None)


class Plan:
    """Owns a muon_plan handle (released on close / garbage collection)."""

    def __init__(self, handle: int, table):
        self.handle = handle
        self.table = list(table)

    def close(self):
        if self.handle:
            lib().muon_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def muon_plan_create(table: Sequence[Sequence[int]], ns_method: int = MUON_NS_STANDARD,
                     ns_dtype: int = -1) -> Plan:
    """table rows: (kind, dtype, rows, cols, split_rows, scale_dim)."""
    n = len(table)
    arr = (MuonParamShape * max(n, 1))()
    for i, r in enumerate(table):
        arr[i] = MuonParamShape(*[int(x) for x in r])
    opts = MuonPlanOptions(int(ns_method), int(ns_dtype))
    h = ctypes.c_void_p()
    _check("muon_plan_create", lib().muon_plan_create(arr, n, ctypes.byref(opts), ctypes.byref(h)))
    return Plan(h.value, table)


def muon_plan_workspace_bytes(plan: Plan) -> int:
    b = ctypes.c_size_t()
    _check("muon_plan_workspace_bytes", lib().muon_plan_workspace_bytes(plan.handle, ctypes.byref(b)))
    return b.value


def muon_plan_buckets(plan: Plan) -> List[tuple]:
    """[(m, n, tall, param_dtype, compute_dtype, method, first_unit, count), ...]"""
    ln = ctypes.c_size_t()
    _check("muon_plan_buckets", lib().muon_plan_buckets(plan.handle, None, 0, ctypes.byref(ln)))
    buf = (ctypes.c_int32 * max(ln.value, 1))()
    _check("muon_plan_buckets", lib().muon_plan_buckets(plan.handle, buf, ln.value, ctypes.byref(ln)))
    return [tuple(buf[i:i + 8]) for i in range(0, ln.value, 8)]


def muon_plan_units(plan: Plan) -> List[tuple]:
    """[(param, row0, rows, cols, tall, scale_dim), ...] in bucket order."""
    ln = ctypes.c_size_t()
    _check("muon_plan_units", lib().muon_plan_units(plan.handle, None, 0, ctypes.byref(ln)))
    buf = (ctypes.c_int64 * max(ln.value, 1))()
    _check("muon_plan_units", lib().muon_plan_units(plan.handle, buf, ln.value, ctypes.byref(ln)))
    return [tuple(buf[i:i + 6]) for i in range(0, ln.value, 6)]


def make_hparams(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True, ns_steps=5, coeffs=None,
                 rms_scale=0.2, adam_lr=3e-4, adam_beta1=0.9, adam_beta2=0.95, adam_eps=1e-8,
                 adam_weight_decay=0.1, adam_step=1, scale_mode=MUON_SCALE_MOONLIGHT, extra_scale=1.0):
    ca = _coeff_array(coeffs, ns_steps)
    hp = MuonHparams(lr, momentum, weight_decay, 1 if nesterov else 0, ns_steps,
                     ctypes.cast(ca, ctypes.POINTER(ctypes.c_float)) if ca is not None else None,
                     rms_scale, adam_lr, adam_beta1, adam_beta2, adam_eps, adam_weight_decay, adam_step,
                     scale_mode, extra_scale)
    hp._keep = ca  # keep the coefficient array alive with the struct
    return hp


def _check_buffer(name, t, rows, cols, dtype, device_index=None):
    """A torch tensor handed to muon_step must be the contiguous rows x cols
    device buffer of the table's dtype, on the GPU the kernels run on: the
    library addresses it from its pointer and the table alone.  Raw integer
    pointers and None pass unchecked (the library rejects a null pointer
    where one is required)."""
    if t is None or isinstance(t, int) or not hasattr(t, "data_ptr"):
        return
    import torch
    want = torch.float32 if dtype == MUON_F32 else torch.bfloat16
    if t.dtype != want:
        raise ValueError(f"{name}: dtype {t.dtype}, the table says {want}")
    if t.numel() != rows * cols or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {rows} x {cols} tensor, got {tuple(t.shape)}")
    _check_device(name, t, device_index)


def muon_step(plan: Plan, params, grads, moms, exp_avgs, exp_avg_sqs, hp: MuonHparams, workspace,
              stream=None, update_outs=None) -> None:
    """One optimizer step; lists follow the plan's table order (None where a
    buffer does not apply).  workspace: a device tensor (or pointer) of at
    least muon_plan_workspace_bytes(plan) bytes."""
    n = len(plan.table)
    for name, lst in (("params", params), ("grads", grads), ("moms", moms), ("exp_avgs", exp_avgs),
                      ("exp_avg_sqs", exp_avg_sqs), ("update_outs", update_outs)):
        if lst is not None and len(lst) != n:
            raise ValueError(f"{name}: {len(lst)} entries for a table of {n}")
    tensors = [t for lst in (params, grads, moms, exp_avgs, exp_avg_sqs, update_outs or [], [workspace])
               for t in lst if t is not None and hasattr(t, "data_ptr")]
    di = None
    if tensors:
        if not all(t.is_cuda for t in tensors):
            bad = next(t for t in tensors if not t.is_cuda)
            raise ValueError(f"muon_step: a {bad.device} tensor; the library needs device memory")
        di = _device_index(stream)
    _check_device("workspace", workspace, di)
    for i, (kind, dt, rows, cols, _split, _sd) in enumerate(plan.table):
        _check_buffer(f"params[{i}]", params[i], rows, cols, dt, di)
        _check_buffer(f"grads[{i}]", grads[i], rows, cols, dt, di)
        if kind == MUON_KIND_MUON:
            _check_buffer(f"moms[{i}]", moms[i], rows, cols, MUON_F32, di)
            if update_outs is not None:
                _check_buffer(f"update_outs[{i}]", update_outs[i], rows, cols, MUON_F32, di)
        else:
            _check_buffer(f"exp_avgs[{i}]", exp_avgs[i], rows, cols, MUON_F32, di)
            _check_buffer(f"exp_avg_sqs[{i}]", exp_avg_sqs[i], rows, cols, MUON_F32, di)
    arr = (MuonParamPtrs * max(n, 1))()
    for i in range(n):
        arr[i] = MuonParamPtrs(_ptr(params[i]), _ptr(grads[i]), _ptr(moms[i]), _ptr(exp_avgs[i]),
                               _ptr(exp_avg_sqs[i]),
                               _ptr(update_outs[i]) if update_outs is not None else None)
    wsz = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    if isinstance(workspace, tuple):
        workspace, wsz = workspace
    _check("muon_step", lib().muon_step(plan.handle, arr, n, ctypes.byref(hp), _ptr(workspace), wsz,
                                        _stream(stream)))


def ns_orthogonalize_workspace_bytes(rows: int, cols: int, dtype: int, method: int = MUON_NS_STANDARD) -> int:
    b = ctypes.c_size_t()
    _check("ns_orthogonalize_workspace_bytes",
           lib().ns_orthogonalize_workspace_bytes(rows, cols, dtype, method, ctypes.byref(b)))
    return b.value


def ns_orthogonalize(X, steps: int = 5, coeffs=None, method: int = MUON_NS_STANDARD, workspace=None,
                     stream=None, rows=None, cols=None, ld=None, dtype=None) -> None:
    """In place: X <- NewtonSchulz(X / ||X||_F).  X: a 2-D device tensor
    (fp32 or bf16, rows may be strided) or a raw pointer with rows/cols/ld/dtype."""
    ca = _coeff_array(coeffs, steps)
    if hasattr(X, "data_ptr"):
        import torch
        di = _device_index(stream) if X.is_cuda else None
        _check_device("X", X, di)
        if workspace is not None:
            _check_device("workspace", workspace, di)
        if X.dim() != 2 or X.stride(1) != 1:
            raise ValueError("X must be 2-D with unit column stride")
        rows, cols = X.shape
        ld = X.stride(0) if rows > 1 else cols
        dtype = MUON_F32 if X.dtype == torch.float32 else MUON_BF16
        if X.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("X must be float32 or bfloat16")
        if workspace is None:
            nb = ns_orthogonalize_workspace_bytes(rows, cols, dtype, method)
            workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=X.device)
    wsz = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    if isinstance(workspace, tuple):
        workspace, wsz = workspace
    _check("ns_orthogonalize",
           lib().ns_orthogonalize(_ptr(X), rows, cols, ld, dtype, steps,
                                  ca, method, _ptr(workspace), wsz, _stream(stream)))


def ns_orthogonalize_noalloc(X, steps: int = 5, coeffs=None, method: int = MUON_NS_STANDARD,
                             stream=None) -> None:
    """ns_orthogonalize with the library's own device scratch array (no
    workspace; nothing is allocated).  X: a 2-D fp32 or bf16 device tensor
    with unit column stride."""
    import torch
    ca = _coeff_array(coeffs, steps)
    di = _device_index(stream) if X.is_cuda else None
    _check_device("X", X, di)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    if X.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("X must be float32 or bfloat16")
    rows, cols = X.shape
    ld = X.stride(0) if rows > 1 else cols
    dtype = MUON_F32 if X.dtype == torch.float32 else MUON_BF16
    _check("ns_orthogonalize_noalloc",
           lib().ns_orthogonalize_noalloc(_ptr(X), rows, cols, ld, dtype, steps, ca, method,
                                          _stream(stream)))


def muon_timing_enable(enable: bool = True) -> None:
    _check("muon_timing_enable", lib().muon_timing_enable(1 if enable else 0))


def muon_timing_collect() -> dict:
    """{family: {"launches", "total_ms", "flops", "bytes"}} since the last collect."""
    cap = 32
    arr = (MuonKernelTiming * cap)()
    n = ctypes.c_int32()
    _check("muon_timing_collect", lib().muon_timing_collect(arr, cap, ctypes.byref(n)))
    return {arr[i].name.decode(): {"launches": arr[i].launches, "total_ms": arr[i].total_ms,
                                   "flops": arr[i].flops, "bytes": arr[i].bytes}
            for i in range(min(n.value, cap))}


def muon_probe_mfma(workgroups: int, iters: int, sink, stream=None) -> float:
    """Enqueue the register-only bf16 MFMA loop; returns its FLOPs.  sink:
    device tensor of at least `workgroups` float32."""
    _check_call_device("sink", sink, stream)
    if hasattr(sink, "numel") and sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink holds fewer than `workgroups` floats")
    flops = ctypes.c_double()
    _check("muon_probe_mfma", lib().muon_probe_mfma(workgroups, iters, _ptr(sink), ctypes.byref(flops),
                                                     _stream(stream)))
    return flops.value


def _check_copy_buffers(src, dst, nbytes, stream):
    for name, t in (("src", src), ("dst", dst)):
        _check_call_device(name, t, stream)
        if hasattr(t, "numel") and t.numel() * t.element_size() < nbytes:
            raise ValueError("buffer smaller than nbytes")


def muon_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    """Enqueue the streaming copy of nbytes from src to dst (device tensors)."""
    _check_copy_buffers(src, dst, nbytes, stream)
    _check("muon_probe_copy", lib().muon_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def muon_probe_copy_lds(src, dst, nbytes: int, stream=None) -> None:
    """Enqueue the streaming copy through the GEMMs' global -> LDS load path."""
    _check_copy_buffers(src, dst, nbytes, stream)
    _check("muon_probe_copy_lds", lib().muon_probe_copy_lds(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def muon_status_string(status: int) -> str:
    return lib().muon_status_string(status).decode()


def muon_ns_coefficients(kind: int, steps: int):
    """steps x 3 Newton-Schulz coefficients of a schedule kind, as a list of
    (a, b, c) tuples."""
    buf = (ctypes.c_float * (3 * steps))() if steps > 0 else (ctypes.c_float * 3)()
    _check("muon_ns_coefficients", lib().muon_ns_coefficients(kind, steps, buf, 3 * max(steps, 0)))
    return [tuple(buf[3 * k:3 * k + 3]) for k in range(steps)]


def muon_version() -> int:
    return lib().muon_version()
