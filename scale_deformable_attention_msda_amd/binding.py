"""ctypes binding of libmsda.so: argument marshalling only.

Every step of the sampling core runs in the HIP kernels behind the C ABI
(include/msda.h). torch is used for device memory and the current stream; if the
library is missing or was not built, every call raises instead of computing
anything elsewhere.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsda.so")

MSDA_F32 = 0
MSDA_BF16 = 1

MSDA_SUCCESS = 0
MSDA_ERROR_INVALID_VALUE = 1
MSDA_ERROR_NOT_SUPPORTED = 2
MSDA_ERROR_MISALIGNED = 3
MSDA_ERROR_LAUNCH = 4
MSDA_ERROR_WORKSPACE = 5
MSDA_ERROR_SCRATCH = 6

_lib = None


class MSDAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def load_library():
    """Load libmsda.so once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build(), "
                           "hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.msda_validate.argtypes = [vp, vp] + [i64] * 7 + [ci]
    lib.msda_validate.restype = ci
    lib.msda_forward.argtypes = [vp] * 6 + [i64] * 7 + [ci, vp]
    lib.msda_forward.restype = ci
    lib.msda_backward.argtypes = [vp] * 9 + [i64] * 7 + [ci, vp, ctypes.c_size_t, vp]
    lib.msda_backward.restype = ci
    lib.msda_backward_static.argtypes = [vp] * 9 + [i64] * 7 + [ci, vp]
    lib.msda_backward_static.restype = ci
    lib.msda_backward_workspace_size.argtypes = [vp, vp] + [i64] * 7 + [ci, ctypes.POINTER(ctypes.c_size_t)]
    lib.msda_backward_workspace_size.restype = ci
    lib.msda_fused_forward.argtypes = [vp] * 4 + [ci] + [vp] * 3 + [i64] * 7 + [ci, vp]
    lib.msda_fused_forward.restype = ci
    lib.msda_fused_backward.argtypes = [vp] * 4 + [ci] + [vp] * 7 + [i64] * 7 + [ci, vp, ctypes.c_size_t, vp]
    lib.msda_fused_backward.restype = ci
    lib.msda_fused_backward_workspace_size.argtypes = [vp, vp] + [i64] * 7 + [ci, ctypes.POINTER(ctypes.c_size_t)]
    lib.msda_fused_backward_workspace_size.restype = ci
    lib.msda_grouped_forward.argtypes = [vp] * 6 + [i64] * 8 + [ci, vp]
    lib.msda_grouped_forward.restype = ci
    lib.msda_grouped_backward.argtypes = [vp] * 9 + [i64] * 8 + [ci, vp, ctypes.c_size_t, vp]
    lib.msda_grouped_backward.restype = ci
    lib.msda_grouped_backward_workspace_size.argtypes = [vp, vp] + [i64] * 8 + [ci, ctypes.POINTER(ctypes.c_size_t)]
    lib.msda_grouped_backward_workspace_size.restype = ci
    lib.msda_status_string.argtypes = [ci]
    lib.msda_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def msda_status_string(status):
    return load_library().msda_status_string(int(status)).decode()


def _raise(status):
    if status != MSDA_SUCCESS:
        raise MSDAError(status, msda_status_string(status))


_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _call(device, stream, fn, *args, writes=()):
    """Calls entry point ``fn`` with ``args`` followed by a stream handle: ``stream``
    when given (a torch.cuda.Stream or a raw HIP stream handle), else torch's
    current stream on ``device``. ``device`` is made
    current for the call (the common case, already current, costs one query).

    With an explicit ``stream`` the tensors in ``writes`` (outputs and workspace,
    which torch allocated on its current stream) are recorded as used on that
    stream, so that the caching allocator does not hand their memory out again
    before the work queued there has finished."""
    idx = device.index
    if torch.cuda.current_device() != idx:
        with torch.cuda.device(idx):
            return _call(device, stream, fn, *args, writes=writes)
    if stream is None:
        if _current_raw_stream is not None:
            return fn(*args, _current_raw_stream(idx))
        return fn(*args, torch.cuda.current_stream(idx).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        s, used = stream.cuda_stream, stream
    else:
        s, used = int(stream), None
    status = fn(*args, s)
    if used is None:
        used = torch.cuda.ExternalStream(s, device=device)
    for t in writes:
        if t is not None:
            t.record_stream(used)
    return status


def _host_i64(a, shape, what):
    if type(a) is np.ndarray and a.dtype == np.int64 and a.shape == shape and a.flags.c_contiguous:
        return a
    if isinstance(a, torch.Tensor):
        if a.device.type != "cpu":
            raise ValueError(f"{what} must be a host array: the library reads it during the call")
        a = a.numpy()
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    if arr.size != math.prod(shape):
        raise ValueError(f"{what} has {arr.size} entries, expected shape {shape}")
    return arr.reshape(shape)


def _dtype_code(t):
    if t == torch.float32:
        return MSDA_F32
    if t == torch.bfloat16:
        return MSDA_BF16
    raise ValueError(f"unsupported dtype {t}: float32 or bfloat16")


def _dims(value, loc, attn, grouped=False):
    if value.dim() != 4 or loc.dim() != 6 or attn.dim() != 5:
        raise ValueError("expected value [N,S,M,D], loc [N,Lq,M,L,K,2], attn [N,Lq,M,L,K]")
    N, S, M, D = value.shape
    N2, Lq, M2, L, K, two = loc.shape
    if grouped:
        ok = M2 >= 1 and M % M2 == 0
    else:
        ok = M2 == M
    if (N2, two) != (N, 2) or not ok or tuple(attn.shape) != (N, Lq, M2, L, K):
        raise ValueError(f"shape mismatch: value {tuple(value.shape)}, loc {tuple(loc.shape)}, "
                         f"attn {tuple(attn.shape)}")
    return (N, S, M, D, L, Lq, K, M2) if grouped else (N, S, M, D, L, Lq, K)


def _device_tensor(t, what, dtype=None, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{what} is on {t.device}, value on {device}: all tensors of a call share one GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def msda_validate(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype=MSDA_F32):
    """Host-only argument check (no HIP call); returns the status code."""
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes") if L > 0 else np.zeros((0, 2), np.int64)
    ls = _host_i64(level_start, (L,), "level_start") if L > 0 else np.zeros((0,), np.int64)
    return load_library().msda_validate(ss.ctypes.data if L > 0 else None,
                                        ls.ctypes.data if L > 0 else None,
                                        N, S, M, D, L, Lq, K, dtype)


def msda_forward(value, spatial_shapes, level_start, loc, attn, out=None, stream=None):
    """out[N,Lq,M,D] (value's dtype) = attention-weighted bilinear samples, per head."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    dev = value.device
    _device_tensor(loc, "loc", torch.float32, device=dev)
    _device_tensor(attn, "attn", torch.float32, device=dev)
    N, S, M, D, L, Lq, K = _dims(value, loc, attn)
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    if out is None:
        out = torch.empty((N, Lq, M, D), dtype=value.dtype, device=dev)
    else:
        _device_tensor(out, "out", value.dtype, device=dev)
        if tuple(out.shape) != (N, Lq, M, D):
            raise ValueError(f"out must be {(N, Lq, M, D)}")
    _raise(_call(dev, stream, lib.msda_forward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, loc.data_ptr(), attn.data_ptr(),
            out.data_ptr(), N, S, M, D, L, Lq, K, dt, writes=(out,)))
    return out


def msda_backward_workspace_size(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype=MSDA_F32):
    """Bytes of device workspace msda_backward needs for these sizes."""
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    out = ctypes.c_size_t(0)
    _raise(load_library().msda_backward_workspace_size(ss.ctypes.data, ls.ctypes.data, N, S, M, D, L, Lq,
                                                       K, dtype, ctypes.byref(out)))
    return out.value


def msda_fused_backward_workspace_size(spatial_shapes, level_start, N, S, M, D, L, Lq, K, dtype=MSDA_F32):
    """Bytes of device workspace msda_fused_backward needs for these sizes."""
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    out = ctypes.c_size_t(0)
    _raise(load_library().msda_fused_backward_workspace_size(ss.ctypes.data, ls.ctypes.data, N, S, M, D, L, Lq,
                                                             K, dtype, ctypes.byref(out)))
    return out.value


def msda_backward(value, spatial_shapes, level_start, loc, attn, grad_out, grad_value=None,
                  grad_loc=None, grad_attn=None, workspace=None, stream=None):
    """(grad_value [N,S,M,D], grad_loc [N,Lq,M,L,K,2], grad_attn [N,Lq,M,L,K]), all float32.

    ``workspace``: optional uint8 device tensor of at least
    msda_backward_workspace_size bytes; allocated from torch's caching
    allocator when omitted."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    _device_tensor(loc, "loc", torch.float32, device=value.device)
    _device_tensor(attn, "attn", torch.float32, device=value.device)
    _device_tensor(grad_out, "grad_out", value.dtype, device=value.device)
    N, S, M, D, L, Lq, K = _dims(value, loc, attn)
    if tuple(grad_out.shape) != (N, Lq, M, D):
        raise ValueError(f"grad_out must be {(N, Lq, M, D)}")
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((N, S, M, D), dtype=torch.float32, device=dev)
    if grad_loc is None:
        grad_loc = torch.empty((N, Lq, M, L, K, 2), dtype=torch.float32, device=dev)
    if grad_attn is None:
        grad_attn = torch.empty((N, Lq, M, L, K), dtype=torch.float32, device=dev)
    for t, name, shape in ((grad_value, "grad_value", (N, S, M, D)),
                           (grad_loc, "grad_loc", (N, Lq, M, L, K, 2)),
                           (grad_attn, "grad_attn", (N, Lq, M, L, K))):
        _device_tensor(t, name, torch.float32, device=value.device)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    need = msda_backward_workspace_size(ss, ls, N, S, M, D, L, Lq, K, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _device_tensor(workspace, "workspace", torch.uint8, device=value.device)
    _raise(_call(dev, stream, lib.msda_backward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, loc.data_ptr(), attn.data_ptr(),
            grad_out.data_ptr(), grad_value.data_ptr(), grad_loc.data_ptr(), grad_attn.data_ptr(), N, S, M,
            D, L, Lq, K, dt, workspace.data_ptr(), workspace.numel(),
            writes=(grad_value, grad_loc, grad_attn, workspace)))
    return grad_value, grad_loc, grad_attn


def msda_backward_static(value, spatial_shapes, level_start, loc, attn, grad_out, grad_value, grad_loc,
                         grad_attn, stream=None):
    """msda_backward without a workspace: the library's static per-GPU scratch
    serves as one, so the call allocates nothing (the caller passes every
    output). Raises MSDAError (status MSDA_ERROR_SCRATCH) when the problem
    needs more than that scratch holds."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    dev = value.device
    _device_tensor(loc, "loc", torch.float32, device=dev)
    _device_tensor(attn, "attn", torch.float32, device=dev)
    _device_tensor(grad_out, "grad_out", value.dtype, device=dev)
    N, S, M, D, L, Lq, K = _dims(value, loc, attn)
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    for t, name, shape in ((grad_out, "grad_out", (N, Lq, M, D)), (grad_value, "grad_value", (N, S, M, D)),
                           (grad_loc, "grad_loc", (N, Lq, M, L, K, 2)),
                           (grad_attn, "grad_attn", (N, Lq, M, L, K))):
        if name != "grad_out":
            _device_tensor(t, name, torch.float32, device=dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    _raise(_call(dev, stream, lib.msda_backward_static,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, loc.data_ptr(), attn.data_ptr(),
            grad_out.data_ptr(), grad_value.data_ptr(), grad_loc.data_ptr(), grad_attn.data_ptr(), N, S, M,
            D, L, Lq, K, dt, writes=(grad_value, grad_loc, grad_attn)))
    return grad_value, grad_loc, grad_attn


def _fused_dims(value, ref, offsets, logits):
    """Sizes for the fused entry points. offsets / logits may carry G < M
    deformable groups (G dividing M); the call then runs with G heads of
    (M/G)*D channels, which is the same memory layout of value and out."""
    if value.dim() != 4 or ref.dim() != 3 or offsets.dim() != 6 or logits.dim() != 5:
        raise ValueError("expected value [N,S,M,D], ref [N,Lq,2|4], offsets [N,Lq,G,L,K,2], "
                         "logits [N,Lq,G,L,K]")
    N, S, M, D = value.shape
    N2, Lq, G, L, K, two = offsets.shape
    if (N2, two) != (N, 2) or G < 1 or M % G != 0 or tuple(logits.shape) != (N, Lq, G, L, K) or \
            tuple(ref.shape[:2]) != (N, Lq) or ref.shape[2] not in (2, 4):
        raise ValueError(f"shape mismatch: value {tuple(value.shape)}, ref {tuple(ref.shape)}, "
                         f"offsets {tuple(offsets.shape)}, logits {tuple(logits.shape)}")
    return N, S, M, D, L, Lq, K, int(ref.shape[2]), G


def msda_fused_forward(value, spatial_shapes, level_start, ref, offsets, logits, out=None, stream=None):
    """out[N,Lq,M,D] from raw predictions: attn = softmax of logits over (L, K),
    loc = reference point + offsets / (W_l, H_l) (ref [N,Lq,2]) or box centre +
    offsets * (w, h) (ref [N,Lq,4] = cx, cy, w, h), then the sampling core."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    for t, name in ((ref, "ref"), (offsets, "offsets"), (logits, "logits")):
        _device_tensor(t, name, torch.float32, device=value.device)
    N, S, M, D, L, Lq, K, rd, G = _fused_dims(value, ref, offsets, logits)
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    if out is None:
        out = torch.empty((N, Lq, M, D), dtype=value.dtype, device=value.device)
    else:
        _device_tensor(out, "out", value.dtype, device=value.device)
        if tuple(out.shape) != (N, Lq, M, D):
            raise ValueError(f"out must be {(N, Lq, M, D)}")
    _raise(_call(value.device, stream, lib.msda_fused_forward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, ref.data_ptr(), rd, offsets.data_ptr(),
            logits.data_ptr(), out.data_ptr(), N, S, G, M // G * D, L, Lq, K, dt, writes=(out,)))
    return out


def msda_fused_backward(value, spatial_shapes, level_start, ref, offsets, logits, grad_out, grad_value=None,
                        grad_offsets=None, grad_logits=None, grad_ref=None, need_grad_ref=True,
                        workspace=None, stream=None):
    """(grad_value, grad_offsets, grad_logits, grad_ref or None), float32, of
    msda_fused_forward. ``need_grad_ref=False`` skips the reference gradient."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    for t, name in ((ref, "ref"), (offsets, "offsets"), (logits, "logits")):
        _device_tensor(t, name, torch.float32, device=value.device)
    _device_tensor(grad_out, "grad_out", value.dtype, device=value.device)
    N, S, M, D, L, Lq, K, rd, G = _fused_dims(value, ref, offsets, logits)
    if tuple(grad_out.shape) != (N, Lq, M, D):
        raise ValueError(f"grad_out must be {(N, Lq, M, D)}")
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((N, S, M, D), dtype=torch.float32, device=dev)
    if grad_offsets is None:
        grad_offsets = torch.empty((N, Lq, G, L, K, 2), dtype=torch.float32, device=dev)
    if grad_logits is None:
        grad_logits = torch.empty((N, Lq, G, L, K), dtype=torch.float32, device=dev)
    if grad_ref is None and need_grad_ref:
        grad_ref = torch.empty((N, Lq, rd), dtype=torch.float32, device=dev)
    outs = [(grad_value, "grad_value", (N, S, M, D)), (grad_offsets, "grad_offsets", (N, Lq, G, L, K, 2)),
            (grad_logits, "grad_logits", (N, Lq, G, L, K))]
    if grad_ref is not None:
        outs.append((grad_ref, "grad_ref", (N, Lq, rd)))
    for t, name, shape in outs:
        _device_tensor(t, name, torch.float32, device=value.device)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    need = msda_fused_backward_workspace_size(ss, ls, N, S, G, M // G * D, L, Lq, K, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _device_tensor(workspace, "workspace", torch.uint8, device=value.device)
    _raise(_call(dev, stream, lib.msda_fused_backward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, ref.data_ptr(), rd, offsets.data_ptr(),
            logits.data_ptr(), grad_out.data_ptr(), grad_value.data_ptr(), grad_offsets.data_ptr(),
            grad_logits.data_ptr(), grad_ref.data_ptr() if grad_ref is not None else None, N, S, G,
            M // G * D, L, Lq, K, dt, workspace.data_ptr(), workspace.numel(),
            writes=(grad_value, grad_offsets, grad_logits, grad_ref, workspace)))
    return grad_value, grad_offsets, grad_logits, grad_ref


def msda_grouped_forward(value, spatial_shapes, level_start, loc, attn, out=None, stream=None):
    """out[N,Lq,M,D] with deformable groups: loc [N,Lq,G,L,K,2] and attn
    [N,Lq,G,L,K] shared by the M/G consecutive heads of each group."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    _device_tensor(loc, "loc", torch.float32, device=value.device)
    _device_tensor(attn, "attn", torch.float32, device=value.device)
    N, S, M, D, L, Lq, K, G = _dims(value, loc, attn, grouped=True)
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    if out is None:
        out = torch.empty((N, Lq, M, D), dtype=value.dtype, device=value.device)
    else:
        _device_tensor(out, "out", value.dtype, device=value.device)
        if tuple(out.shape) != (N, Lq, M, D):
            raise ValueError(f"out must be {(N, Lq, M, D)}")
    _raise(_call(value.device, stream, lib.msda_grouped_forward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, loc.data_ptr(), attn.data_ptr(),
            out.data_ptr(), N, S, M, D, L, Lq, K, G, dt, writes=(out,)))
    return out


def msda_grouped_backward(value, spatial_shapes, level_start, loc, attn, grad_out, grad_value=None,
                          grad_loc=None, grad_attn=None, workspace=None, stream=None):
    """(grad_value [N,S,M,D], grad_loc [N,Lq,G,L,K,2], grad_attn [N,Lq,G,L,K]) of
    msda_grouped_forward, float32."""
    lib = load_library()
    _device_tensor(value, "value")
    dt = _dtype_code(value.dtype)
    _device_tensor(loc, "loc", torch.float32, device=value.device)
    _device_tensor(attn, "attn", torch.float32, device=value.device)
    _device_tensor(grad_out, "grad_out", value.dtype, device=value.device)
    N, S, M, D, L, Lq, K, G = _dims(value, loc, attn, grouped=True)
    if tuple(grad_out.shape) != (N, Lq, M, D):
        raise ValueError(f"grad_out must be {(N, Lq, M, D)}")
    ss = _host_i64(spatial_shapes, (L, 2), "spatial_shapes")
    ls = _host_i64(level_start, (L,), "level_start")
    dev = value.device
    if grad_value is None:
        grad_value = torch.empty((N, S, M, D), dtype=torch.float32, device=dev)
    if grad_loc is None:
        grad_loc = torch.empty((N, Lq, G, L, K, 2), dtype=torch.float32, device=dev)
    if grad_attn is None:
        grad_attn = torch.empty((N, Lq, G, L, K), dtype=torch.float32, device=dev)
    for t, name, shape in ((grad_value, "grad_value", (N, S, M, D)),
                           (grad_loc, "grad_loc", (N, Lq, G, L, K, 2)),
                           (grad_attn, "grad_attn", (N, Lq, G, L, K))):
        _device_tensor(t, name, torch.float32, device=value.device)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    need = ctypes.c_size_t(0)
    _raise(lib.msda_grouped_backward_workspace_size(ss.ctypes.data, ls.ctypes.data, N, S, M, D, L, Lq, K, G, dt,
                                                    ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    else:
        _device_tensor(workspace, "workspace", torch.uint8, device=value.device)
    _raise(_call(dev, stream, lib.msda_grouped_backward,
            value.data_ptr(), ss.ctypes.data, ls.ctypes.data, loc.data_ptr(), attn.data_ptr(),
            grad_out.data_ptr(), grad_value.data_ptr(), grad_loc.data_ptr(), grad_attn.data_ptr(), N, S, M,
            D, L, Lq, K, G, dt, workspace.data_ptr(), workspace.numel(),
            writes=(grad_value, grad_loc, grad_attn, workspace)))
    return grad_value, grad_loc, grad_attn


class MSDeformAttnSampling(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libmsda.so."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start, loc, attn):
        ss = _host_i64(spatial_shapes, (loc.shape[3], 2), "spatial_shapes")
        ls = _host_i64(level_start, (loc.shape[3],), "level_start")
        ctx.save_for_backward(value, loc, attn)
        ctx.levels = (ss, ls)
        return msda_forward(value, ss, ls, loc, attn)

    @staticmethod
    def backward(ctx, grad_out):
        value, loc, attn = ctx.saved_tensors
        ss, ls = ctx.levels
        gv, gl, ga = msda_backward(value, ss, ls, loc, attn, grad_out.contiguous())
        return gv.to(value.dtype), None, None, gl, ga


def msda_sample(value, spatial_shapes, level_start, loc, attn):
    """Differentiable sampling core (value, loc and attn receive gradients)."""
    return MSDeformAttnSampling.apply(value, spatial_shapes, level_start, loc, attn)


class MSDeformAttnFused(torch.autograd.Function):
    """Autograd wrapper of the fused entry points (value, ref, offsets and
    logits receive gradients)."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start, ref, offsets, logits):
        ss = _host_i64(spatial_shapes, (offsets.shape[3], 2), "spatial_shapes")
        ls = _host_i64(level_start, (offsets.shape[3],), "level_start")
        ctx.save_for_backward(value, ref, offsets, logits)
        ctx.levels = (ss, ls)
        return msda_fused_forward(value, ss, ls, ref, offsets, logits)

    @staticmethod
    def backward(ctx, grad_out):
        value, ref, offsets, logits = ctx.saved_tensors
        ss, ls = ctx.levels
        gv, go, gz, gr = msda_fused_backward(value, ss, ls, ref, offsets, logits, grad_out.contiguous(),
                                             need_grad_ref=ctx.needs_input_grad[3])
        return gv.to(value.dtype), None, None, gr, go, gz


def msda_fused_sample(value, spatial_shapes, level_start, ref, offsets, logits):
    """Differentiable sampling core fed by raw offsets and logits."""
    return MSDeformAttnFused.apply(value, spatial_shapes, level_start, ref, offsets, logits)


class MSDeformAttnGrouped(torch.autograd.Function):
    """Autograd wrapper of the deformable-group entry points (loc and attn per
    group; value, loc and attn receive gradients)."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start, loc, attn):
        ss = _host_i64(spatial_shapes, (loc.shape[3], 2), "spatial_shapes")
        ls = _host_i64(level_start, (loc.shape[3],), "level_start")
        ctx.save_for_backward(value, loc, attn)
        ctx.levels = (ss, ls)
        return msda_grouped_forward(value, ss, ls, loc, attn)

    @staticmethod
    def backward(ctx, grad_out):
        value, loc, attn = ctx.saved_tensors
        ss, ls = ctx.levels
        gv, gl, ga = msda_grouped_backward(value, ss, ls, loc, attn, grad_out.contiguous())
        return gv.to(value.dtype), None, None, gl, ga


def msda_grouped_sample(value, spatial_shapes, level_start, loc, attn):
    """Differentiable sampling core with deformable groups."""
    return MSDeformAttnGrouped.apply(value, spatial_shapes, level_start, loc, attn)
