"""Python binding of libparo (the MI355X rotated W4A16 linear library).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and the current stream. The names
mirror the C ABI in include/paro.h.

Importing this package loads ``libparo.so`` from the package directory; if it
is missing the import fails loudly (build it with ``python -m
rotated_linear_amd._build``). There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libparo.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rotated_linear_amd._build`")

# PyTorch-ROCm ships its own HIP runtime (soname libamdhip64.so.7). Importing torch first makes
# libparo's libamdhip64.so.7 dependency bind to that already-loaded runtime, so device pointers
# and streams handed over from torch belong to the runtime that launches the kernels.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped() -> set:
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln}
    except OSError:
        return set()


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError(f"two HIP runtimes are loaded in this process: {sorted(_hip_runtimes_mapped())}")

GROUP = 128
MAX_D = 16384
MAX_K = 64
F16, F32 = 0, 1

STATUS = {0: "PARO_OK", 1: "PARO_EINVAL", 2: "PARO_ESHAPE", 3: "PARO_EPAIRS", 4: "PARO_ESCALE",
          5: "PARO_EWORKSPACE", 6: "PARO_EHIP"}


class paro_rotation(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("D", ctypes.c_int32), ("dev", ctypes.c_void_p)]


_vp, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_lib.paro_status_str.restype = ctypes.c_char_p
_lib.paro_status_str.argtypes = [_i]
_lib.paro_version.restype = _i
_lib.paro_rotation_bytes.restype = _sz
_lib.paro_rotation_bytes.argtypes = [_i, _i]
_lib.paro_rotation_encode.restype = _i
_lib.paro_rotation_encode.argtypes = [_i, _i, _vp, _vp, _vp, _vp, _sz]
_lib.paro_rotation_prepare.restype = _i
_lib.paro_rotation_prepare.argtypes = [_i, _i, _vp, _vp, _vp, _vp, _sz, ctypes.POINTER(paro_rotation), _vp]
_lib.paro_pack_weights.restype = _i
_lib.paro_pack_weights.argtypes = [ctypes.POINTER(paro_rotation), _i, _vp, _vp, _vp, _vp, _vp]
_lib.paro_rotate.restype = _i
_lib.paro_rotate.argtypes = [ctypes.POINTER(paro_rotation), _i, _vp, _vp, _vp]
_lib.paro_workspace_bytes.restype = _sz
_lib.paro_workspace_bytes.argtypes = [_i, _i, _i]
_lib.paro_w4a16_linear.restype = _i
_lib.paro_w4a16_linear.argtypes = [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]


class paro_linear_args(ctypes.Structure):
    """One call of paro_linear_batch (include/paro.h)."""
    _fields_ = [("rot", ctypes.POINTER(paro_rotation)), ("M", ctypes.c_int32), ("D", ctypes.c_int32),
                ("N", ctypes.c_int32), ("x", _vp), ("qweight", _vp), ("scales", _vp), ("zeros", _vp), ("y", _vp)]


_lib.paro_linear_batch_workspace_bytes.restype = _sz
_lib.paro_linear_batch_workspace_bytes.argtypes = [_i, ctypes.POINTER(paro_linear_args)]
_lib.paro_linear_batch.restype = _i
_lib.paro_linear_batch.argtypes = [_i, ctypes.POINTER(paro_linear_args), _i, _vp, _sz, _vp]
_lib.paro_rotated_linear.restype = _i
_lib.paro_rotated_linear.argtypes = [ctypes.POINTER(paro_rotation), _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                                     _sz, _vp]

_lib.paro_rotated_linear_noalloc.restype = _i
_lib.paro_rotated_linear_noalloc.argtypes = [ctypes.POINTER(paro_rotation), _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp]
_lib.paro_noalloc_max_bytes.restype = _sz
_lib.paro_noalloc_max_bytes.argtypes = []

EXPORTS = ("paro_status_str", "paro_version", "paro_rotation_bytes", "paro_rotation_encode", "paro_rotation_prepare",
           "paro_pack_weights", "paro_rotate", "paro_workspace_bytes", "paro_w4a16_linear",
           "paro_rotated_linear", "paro_linear_batch_workspace_bytes",
           "paro_linear_batch", "paro_rotated_linear_noalloc", "paro_noalloc_max_bytes")


class ParoError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_lib.paro_status_str(status).decode()}")


def _check(status: int, call: str) -> None:
    if status != 0:
        raise ParoError(status, call)


def lib() -> ctypes.CDLL:
    return _lib


def paro_status_str(status: int) -> str:
    return _lib.paro_status_str(status).decode()


def paro_version() -> int:
    return _lib.paro_version()


def paro_rotation_bytes(K: int, D: int) -> int:
    return _lib.paro_rotation_bytes(K, D)


def paro_workspace_bytes(M: int, D: int, N: int) -> int:
    return _lib.paro_workspace_bytes(M, D, N)


# --------------------------------------------------------------------------- #
# torch plumbing
# --------------------------------------------------------------------------- #

def _torch():
    import torch
    return torch


def _stream_ptr(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _want(t, dtype, shape, name):
    """Type, dtype, shape and contiguity of one tensor argument (inputs, outputs and workspaces
    alike); where it lives is checked by _on_gpu once every argument has passed this."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(named):
    """Every tensor of ``named`` (name -> tensor or None) lives on one and the same GPU."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")
    return dev


def _want_ws(ws):
    """A workspace: a contiguous one-dimensional uint8 tensor (its numel is its byte count)."""
    if ws is None:
        return
    _want(ws, _torch().uint8, (ws.numel(),), "ws")


def _host_transform(pairs, theta, scale):
    pairs = np.ascontiguousarray(np.asarray(pairs, np.int32))
    theta = np.ascontiguousarray(np.asarray(theta, np.float32))
    scale = np.ascontiguousarray(np.asarray(scale, np.float32))
    D = int(scale.shape[0])
    K = int(pairs.shape[0]) if pairs.ndim == 3 else 0
    if pairs.ndim != 3 or pairs.shape[1:] != (D // 2, 2) or theta.shape != (K, D // 2):
        raise ValueError("pairs must be [K][D/2][2] and theta [K][D/2] with D = len(scale)")
    return pairs, theta, scale, K, D


def paro_rotation_encode(pairs, theta, scale) -> np.ndarray:
    """Host-only: validate the transform and return its descriptor bytes (uint8 array)."""
    pairs, theta, scale, K, D = _host_transform(pairs, theta, scale)
    nbytes = _lib.paro_rotation_bytes(K, D)
    if nbytes == 0:
        raise ParoError(2, "paro_rotation_bytes")
    buf = np.zeros(nbytes, np.uint8)
    _check(_lib.paro_rotation_encode(K, D, pairs.ctypes.data_as(_vp), theta.ctypes.data_as(_vp),
                                     scale.ctypes.data_as(_vp), buf.ctypes.data_as(_vp), nbytes),
           "paro_rotation_encode")
    return buf


def descriptor_sections(buf: np.ndarray, K: int, D: int):
    """Views of an encoded descriptor: pairs (i, j) int [K][D/2][2], cs float32 [K][D/2][2],
    inv_s float32 [D], s float32 [D]."""
    def up(v):
        return (v + 255) // 256 * 256
    P = K * (D // 2)
    o_inv = up(P * 12)
    o_s = o_inv + up(D * 4)
    rec = buf[:P * 12].view(np.uint32).reshape(K, D // 2, 3)
    raw = rec[:, :, 0]
    pairs = np.stack([(raw & 0xFFFF) >> 2, raw >> 18], axis=-1).astype(np.int64)  # fields 4 i, 4 j
    cs = rec[:, :, 1:3].copy().view(np.float32)
    return pairs, cs, buf[o_inv:o_inv + D * 4].view(np.float32), buf[o_s:o_s + D * 4].view(np.float32)


class Rotation:
    """A prepared transform: the device descriptor (a uint8 tensor) and its C handle."""

    def __init__(self, K: int, D: int, desc, handle: paro_rotation):
        self.K, self.D, self.desc, self.handle = K, D, desc, handle

    @property
    def ptr(self):
        return ctypes.byref(self.handle)


def paro_rotation_prepare(pairs, theta, scale, device="cuda") -> Rotation:
    """pairs int32 [K][D/2][2], theta float32 [K][D/2], scale float32 [D] (host arrays)."""
    torch = _torch()
    pairs, theta, scale, K, D = _host_transform(pairs, theta, scale)
    nbytes = _lib.paro_rotation_bytes(K, D)
    if nbytes == 0:
        raise ParoError(2, "paro_rotation_bytes")
    desc = torch.empty(nbytes, dtype=torch.uint8, device=device)
    handle = paro_rotation()
    with torch.cuda.device(desc.device):
        st = _lib.paro_rotation_prepare(K, D, pairs.ctypes.data_as(_vp), theta.ctypes.data_as(_vp),
                                        scale.ctypes.data_as(_vp), _ptr(desc), nbytes, ctypes.byref(handle),
                                        _stream_ptr(desc.device))
    _check(st, "paro_rotation_prepare")
    return Rotation(K, D, desc, handle)


def paro_pack_weights(rot: Rotation, W, out=None):
    """W float16 [N][D] on the GPU -> (qweight uint8 [N][D/2], scales f16 [N][D/128], zeros f16 [N][D/128]).
    qweight's shape fixes its size only: its N*D/2 bytes hold the rows in blocks of 16, each
    block group by group (include/paro.h, "Packed weights"), so ``qweight[n]`` is not row n.
    ``out``: an optional (qweight, scales, zeros) tuple of tensors of those shapes to write."""
    torch = _torch()
    N, D = int(W.shape[0]), rot.D
    _want(W, torch.float16, (N, D), "W")
    if out is not None:
        qw, sc, z = out
        _want(qw, torch.uint8, (N, D // 2), "qweight")
        _want(sc, torch.float16, (N, D // GROUP), "scales")
        _want(z, torch.float16, (N, D // GROUP), "zeros")
    dev = _on_gpu({"W": W, **({"qweight": qw, "scales": sc, "zeros": z} if out is not None else {})})
    if out is None:
        qw = torch.empty((N, D // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((N, D // GROUP), dtype=torch.float16, device=dev)
        z = torch.empty((N, D // GROUP), dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        _check(_lib.paro_pack_weights(rot.ptr, N, _ptr(W), _ptr(qw), _ptr(sc), _ptr(z), _stream_ptr(dev)),
               "paro_pack_weights")
    return qw, sc, z


def paro_rotate(rot: Rotation, x, out=None):
    """x float16 [M][D] -> transformed activations float16 [M][D] (``out``: a tensor of that shape)."""
    torch = _torch()
    M = int(x.shape[0])
    _want(x, torch.float16, (M, rot.D), "x")
    if out is not None:
        _want(out, torch.float16, (M, rot.D), "out")
    dev = _on_gpu({"x": x, "out": out})
    xo = torch.empty_like(x) if out is None else out
    with torch.cuda.device(dev):
        _check(_lib.paro_rotate(rot.ptr, M, _ptr(x), _ptr(xo), _stream_ptr(dev)), "paro_rotate")
    return xo


def _ydt(t):
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("y must be float16 or float32")


def _linear_operands(x, qweight, scales, zeros, D, out, out_dtype, ws, what="x"):
    """Check one linear's operands (and a given output / workspace); returns (M, N, y dtype)."""
    torch = _torch()
    M, N = int(x.shape[0]), int(qweight.shape[0])
    _want(x, torch.float16, (M, D), what)
    _want(qweight, torch.uint8, (N, D // 2), "qweight")
    _want(scales, torch.float16, (N, D // GROUP), "scales")
    _want(zeros, torch.float16, (N, D // GROUP), "zeros")
    dtype = out_dtype or (out.dtype if out is not None else torch.float16)
    if dtype not in (torch.float16, torch.float32):
        raise TypeError("y must be float16 or float32")
    if out is not None:
        _want(out, dtype, (M, N), "out")
    _want_ws(ws)
    return M, N, dtype


def paro_w4a16_linear(x, qweight, scales, zeros, out_dtype=None, out=None, ws=None):
    """Plain group-wise INT4 linear: y = x . dequant(qweight, scales, zeros)^T."""
    torch = _torch()
    D = int(x.shape[1]) if x.dim() == 2 else -1
    M, N, dtype = _linear_operands(x, qweight, scales, zeros, D, out, out_dtype, ws)
    dev = _on_gpu({"x": x, "qweight": qweight, "scales": scales, "zeros": zeros, "out": out, "ws": ws})
    y = torch.empty((M, N), dtype=dtype, device=dev) if out is None else out
    need = _lib.paro_workspace_bytes(M, D, N)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(_lib.paro_w4a16_linear(M, D, N, _ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), _ydt(y),
                                      _ptr(ws), ws.numel() if ws is not None else 0, _stream_ptr(dev)),
               "paro_w4a16_linear")
    return y


def paro_rotated_linear(rot: Rotation, x, qweight, scales, zeros, out_dtype=None, out=None, ws=None):
    """Fused runtime path: y = transform(x) . dequant(qweight, scales, zeros)^T."""
    torch = _torch()
    D = rot.D
    M, N, dtype = _linear_operands(x, qweight, scales, zeros, D, out, out_dtype, ws)
    dev = _on_gpu({"x": x, "qweight": qweight, "scales": scales, "zeros": zeros, "out": out, "ws": ws})
    y = torch.empty((M, N), dtype=dtype, device=dev) if out is None else out
    need = _lib.paro_workspace_bytes(M, D, N)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(_lib.paro_rotated_linear(rot.ptr, M, N, _ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y),
                                        _ydt(y), _ptr(ws), ws.numel() if ws is not None else 0, _stream_ptr(dev)),
               "paro_rotated_linear")
    return y


def paro_noalloc_max_bytes() -> int:
    return _lib.paro_noalloc_max_bytes()


def paro_rotated_linear_noalloc(rot: Rotation, x, qweight, scales, zeros, out):
    """paro_rotated_linear without a workspace: the library's fixed scratch array serves as the
    workspace (for callers that cannot allocate). ``out`` (float16 or float32 [M][N]) is required,
    so nothing is allocated here either."""
    torch = _torch()
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    D = rot.D
    M, N, _ = _linear_operands(x, qweight, scales, zeros, D, out, None, None)
    dev = _on_gpu({"x": x, "qweight": qweight, "scales": scales, "zeros": zeros, "out": out})
    with torch.cuda.device(dev):
        _check(_lib.paro_rotated_linear_noalloc(rot.ptr, M, N, _ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros),
                                                _ptr(out), _ydt(out), _stream_ptr(dev)),
               "paro_rotated_linear_noalloc")
    return out


def paro_linear_batch(calls, out_dtype=None, outs=None, ws=None):
    """Independent linears in as few launches as possible (paro_linear_batch in include/paro.h).

    calls: sequence of (rot, x, qweight, scales, zeros) with rot a Rotation or None (plain INT4
    linear). Returns the list of outputs (new tensors of out_dtype, float16 by default, unless
    `outs` gives them)."""
    torch = _torch()
    n = len(calls)
    if outs is not None and len(outs) != n:
        raise ValueError(f"outs has {len(outs)} tensors for {n} calls")
    dtype = out_dtype or (outs[0].dtype if outs else torch.float16)
    shapes, named = [], {}
    for i, (rot, x, qweight, scales, zeros) in enumerate(calls):
        D = int(x.shape[1]) if x.dim() == 2 else -1
        if rot is not None and rot.D != D:
            raise ValueError(f"call {i}: x has {D} channels, the transform {rot.D}")
        M, N, _ = _linear_operands(x, qweight, scales, zeros, D, outs[i] if outs else None, dtype, None,
                                   what=f"calls[{i}].x")
        shapes.append((M, D, N))
        named.update({f"calls[{i}].x": x, f"calls[{i}].qweight": qweight, f"calls[{i}].scales": scales,
                      f"calls[{i}].zeros": zeros, f"outs[{i}]": outs[i] if outs else None})
    _want_ws(ws)
    named["ws"] = ws
    if n == 0:
        return []
    device = _on_gpu(named)
    arr = (paro_linear_args * n)()
    ys = []
    for i, ((rot, x, qweight, scales, zeros), (M, D, N)) in enumerate(zip(calls, shapes)):
        y = outs[i] if outs else torch.empty((M, N), dtype=dtype, device=device)
        ys.append(y)
        arr[i] = paro_linear_args(ctypes.pointer(rot.handle) if rot is not None else None, M, D, N, x.data_ptr(),
                                  qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), y.data_ptr())
    need = _lib.paro_linear_batch_workspace_bytes(n, arr)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    with torch.cuda.device(device):
        _check(_lib.paro_linear_batch(n, arr, _ydt(ys[0]), _ptr(ws), ws.numel() if ws is not None else 0,
                                      _stream_ptr(device)), "paro_linear_batch")
    return ys
