"""Python binding of librhtq.so (randomized Hadamard rotation + 4-bit quantisation).

The functions carry the names of the C entry points in include/rhtq.h and only
marshal arguments: torch provides device memory and the current HIP stream, every
step of the computation runs in the library's HIP kernels.  There is no CPU
fallback: calls on CPU tensors raise, and importing the package raises when the
library has not been built (python randomized_hadamard_rotation_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librhtq.so")

RHTQ_OK, RHTQ_EINVAL, RHTQ_EUNSUPPORTED, RHTQ_EHIP = 0, 1, 2, 3
RHTQ_IN_BF16, RHTQ_IN_F32, RHTQ_IN_F16 = 0, 1, 2
RHTQ_FMT_INT4, RHTQ_FMT_NVFP4, RHTQ_FMT_MXFP4 = 0, 1, 2
RHTQ_SCALE_F32, RHTQ_SCALE_F16, RHTQ_SCALE_E4M3, RHTQ_SCALE_E8M0 = 0, 1, 2, 3
RHTQ_TENSOR_SCALE_DYNAMIC, RHTQ_TENSOR_SCALE_GIVEN = 0, 1

_FMT = {"int4": RHTQ_FMT_INT4, "nvfp4": RHTQ_FMT_NVFP4, "mxfp4": RHTQ_FMT_MXFP4}
_SCALE = {"f32": RHTQ_SCALE_F32, "f16": RHTQ_SCALE_F16, "e4m3": RHTQ_SCALE_E4M3, "e8m0": RHTQ_SCALE_E8M0}
_DEFAULT_SCALE = {"int4": "f32", "nvfp4": "e4m3", "mxfp4": "e8m0"}
_DEFAULT_GROUP = {"nvfp4": 16, "mxfp4": 32}

EXPORTED = ["rhtq_abi_version", "rhtq_status_str", "rhtq_supported", "rhtq_rotate",
            "rhtq_forward", "rhtq_inverse", "rhtq_signs_from_seed", "rhtq_rotate_blocked",
            "rhtq_forward_blocked", "rhtq_inverse_blocked", "rhtq_stream_floor"]


class RhtqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python randomized_hadamard_rotation_amd/build.py`")
    # torch ships its own HIP runtime: load it first, so that the library binds to that runtime
    # rather than starting a second one from /opt/rocm (kernels enqueued on torch's streams from
    # another runtime fail to launch)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    ci = ctypes.c_int
    lib.rhtq_abi_version.restype = ci
    lib.rhtq_abi_version.argtypes = []
    lib.rhtq_status_str.restype = ctypes.c_char_p
    lib.rhtq_status_str.argtypes = [ci]
    lib.rhtq_supported.restype = ci
    lib.rhtq_supported.argtypes = [i32, ci, i32]
    lib.rhtq_rotate.restype = ci
    lib.rhtq_rotate.argtypes = [vp, ci, i64, i32, vp, vp, vp]
    lib.rhtq_forward.restype = ci
    lib.rhtq_forward.argtypes = [vp, ci, i64, i32, vp, ci, i32, ci, vp, vp, vp, ci, vp]
    lib.rhtq_inverse.restype = ci
    lib.rhtq_inverse.argtypes = [vp, vp, vp, i64, i32, vp, ci, i32, ci, vp, vp]
    lib.rhtq_signs_from_seed.restype = ci
    lib.rhtq_signs_from_seed.argtypes = [u64, i32, vp]
    lib.rhtq_rotate_blocked.restype = ci
    lib.rhtq_rotate_blocked.argtypes = [vp, ci, i64, i32, i32, vp, vp, vp]
    lib.rhtq_forward_blocked.restype = ci
    lib.rhtq_forward_blocked.argtypes = [vp, ci, i64, i32, i32, vp, ci, i32, ci, vp, vp, vp, ci, vp]
    lib.rhtq_inverse_blocked.restype = ci
    lib.rhtq_inverse_blocked.argtypes = [vp, vp, vp, i64, i32, i32, vp, ci, i32, ci, vp, vp]
    lib.rhtq_stream_floor.restype = ci
    lib.rhtq_stream_floor.argtypes = [vp, i64, i32, vp, vp, i32, vp]
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.rhtq_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != RHTQ_OK:
        raise RhtqError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _resolve_stream(stream):
    """(stream object, whether it differs from torch's current stream).  Copies and fills
    this wrapper makes are enqueued on the current stream, so another stream first waits for
    the current one."""
    torch = _torch()
    cur = torch.cuda.current_stream()
    if stream is None or stream.cuda_stream == cur.cuda_stream:
        return cur, False
    stream.wait_stream(cur)
    return stream, True


def _keep_for(stream, other, *ts):
    """Tensors this wrapper allocated (copies, signs, outputs) are used by work enqueued on
    `stream`; when that is not torch's current stream, tell the caching allocator so their
    memory is not handed out again before that work has run."""
    if other:
        for t in ts:
            if t is not None:
                t.record_stream(stream)


def _need_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("rhtq runs on the GPU only: pass device tensors")


def _expect(t, name, dtype, shape, device=None):
    """A caller-supplied buffer must match what the kernels will write or read: the C ABI
    takes bare pointers and cannot check sizes.  The device is checked last."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _signs_tensor(signs, n, device):
    """Device int8 [n] from a tensor / numpy array / None (marshalling only)."""
    torch = _torch()
    if signs is None:
        return None
    if isinstance(signs, np.ndarray):
        signs = torch.from_numpy(np.ascontiguousarray(signs.astype(np.int8)))
    if signs.dtype != torch.int8 or signs.numel() != n:
        raise ValueError("signs must be int8 with n entries")
    return signs.reshape(n).to(device).contiguous()


def _in_dtype(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        return RHTQ_IN_BF16
    if x.dtype == torch.float16:
        return RHTQ_IN_F16
    if x.dtype == torch.float32:
        return RHTQ_IN_F32
    raise ValueError("x must be bfloat16, float16 or float32")


def _rows(x):
    if x.dim() != 2:
        raise ValueError("x must be 2-D [tokens][n]")
    return x.shape


def _scale_torch_dtype(scale_dtype):
    torch = _torch()
    if scale_dtype not in _SCALE:
        raise ValueError(f"unknown scale_dtype {scale_dtype!r}")
    return {"f32": torch.float32, "f16": torch.float16, "e4m3": torch.uint8, "e8m0": torch.uint8}[scale_dtype]


def rhtq_abi_version() -> int:
    return lib.rhtq_abi_version()


def rhtq_status_str(status: int) -> str:
    return status_str(status)


def rhtq_supported(n: int, fmt: str = "int4", group: int = 0) -> bool:
    return bool(lib.rhtq_supported(n, _FMT[fmt], group))


def rhtq_signs_from_seed(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int8)
    _check(lib.rhtq_signs_from_seed(ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), n,
                                    out.ctypes.data_as(ctypes.c_void_p)), "rhtq_signs_from_seed")
    return out


def _same_device(dev, **ts):
    _need_device(*ts.values())
    for name, t in ts.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def rhtq_rotate(x, signs=None, out=None, stream=None, block=None):
    """y = H_n diag(signs) x / sqrt(n) per row, fp32 [tokens][n]; x is a bfloat16, float16 or
    float32 device tensor [tokens][n].  With block = b < n the
    rotation is block-diagonal: (I (x) H_b) diag(signs) x / sqrt(b).  An `out` passed in must
    be contiguous fp32 [tokens][n] on x's device."""
    torch = _torch()
    tokens, n = _rows(x)
    in_dtype = _in_dtype(x)
    if out is not None:
        _expect(out, "out", torch.float32, (tokens, n))
    _same_device(x.device, x=x, out=out)
    xc = x.contiguous()                  # bound to a local: it must outlive the call
    s = _signs_tensor(signs, n, xc.device)
    st, other = _resolve_stream(stream)
    own = out is None
    if own:
        out = torch.empty((tokens, n), dtype=torch.float32, device=xc.device)
    sp = ctypes.c_void_p(st.cuda_stream)
    if block is None or block == n:
        status = lib.rhtq_rotate(_ptr(xc), in_dtype, tokens, n, _ptr(s), _ptr(out), sp)
        where = "rhtq_rotate"
    else:
        status = lib.rhtq_rotate_blocked(_ptr(xc), in_dtype, tokens, n, block, _ptr(s), _ptr(out), sp)
        where = "rhtq_rotate_blocked"
    _check(status, where)
    _keep_for(st, other, xc if xc is not x else None, s, out if own else None)
    return out


def scale_shape(tokens: int, n: int, fmt: str, group: int):
    g = n if group == 0 else group
    if g <= 0 or n % g:
        raise ValueError(f"group {group} does not divide n = {n}")
    return (tokens, n // g)


def rhtq_forward(x, signs=None, fmt: str = "int4", group: int = 0, scale_dtype: str | None = None,
                 tensor_scale=None, tensor_scale_mode: str = "dynamic", packed=None, scales=None,
                 stream=None, block=None):
    """Rotate, quantise, pack x (bfloat16, float16 or float32 [tokens][n] on the device).
    Returns (packed uint8 [tokens][n/2], scales, tensor_scale).

    INT4: scales fp32/fp16 [tokens][n/group] (group 0 = one per row).
    NVFP4: scales uint8 E4M3 [tokens][n/16]; tensor_scale a device float32 [1]
    (written in 'dynamic' mode, read in 'given' mode).
    MXFP4: scales uint8 E8M0 [tokens][n/32].
    block = b < n: block-diagonal rotation (groups inside a block).
    Buffers passed in (packed, scales, tensor_scale) must have exactly these dtypes and
    shapes, be contiguous and live on x's device; anything else raises ValueError before
    any work is enqueued."""
    torch = _torch()
    if fmt not in _FMT:
        raise ValueError(f"unknown fmt {fmt!r}")
    if tensor_scale_mode not in ("dynamic", "given"):
        raise ValueError("tensor_scale_mode must be 'dynamic' or 'given'")
    tokens, n = _rows(x)
    in_dtype = _in_dtype(x)
    if scale_dtype is None:
        scale_dtype = _DEFAULT_SCALE[fmt]
    if group == 0:
        group = _DEFAULT_GROUP.get(fmt, 0)
    sdt = _scale_torch_dtype(scale_dtype)
    sshape = scale_shape(tokens, n, fmt, group)
    if packed is not None:
        _expect(packed, "packed", torch.uint8, (tokens, n // 2))
    if scales is not None:
        _expect(scales, "scales", sdt, sshape)
    if fmt == "nvfp4":
        if tensor_scale is not None:
            _expect(tensor_scale, "tensor_scale", torch.float32, (1,))
        elif tensor_scale_mode == "given":
            raise ValueError("tensor_scale_mode 'given' needs a tensor_scale")
    _same_device(x.device, x=x, packed=packed, scales=scales, tensor_scale=tensor_scale)
    xc = x.contiguous()                  # bound to a local: it must outlive the call
    s = _signs_tensor(signs, n, xc.device)
    st, other = _resolve_stream(stream)
    own_p, own_s = packed is None, scales is None
    own_t = fmt == "nvfp4" and tensor_scale is None
    if own_p:
        packed = torch.empty((tokens, n // 2), dtype=torch.uint8, device=xc.device)
    if own_s:
        scales = torch.empty(sshape, dtype=sdt, device=xc.device)
    if own_t:
        tensor_scale = torch.zeros(1, dtype=torch.float32, device=xc.device)
    mode = RHTQ_TENSOR_SCALE_DYNAMIC if tensor_scale_mode == "dynamic" else RHTQ_TENSOR_SCALE_GIVEN
    ts_ptr = _ptr(tensor_scale) if fmt == "nvfp4" else None
    sp = ctypes.c_void_p(st.cuda_stream)
    if block is None or block == n:
        status = lib.rhtq_forward(_ptr(xc), in_dtype, tokens, n, _ptr(s), _FMT[fmt], group,
                                  _SCALE[scale_dtype], _ptr(packed), _ptr(scales), ts_ptr, mode, sp)
        where = "rhtq_forward"
    else:
        status = lib.rhtq_forward_blocked(_ptr(xc), in_dtype, tokens, n, block, _ptr(s), _FMT[fmt], group,
                                          _SCALE[scale_dtype], _ptr(packed), _ptr(scales), ts_ptr, mode, sp)
        where = "rhtq_forward_blocked"
    _check(status, where)
    _keep_for(st, other, xc if xc is not x else None, s, packed if own_p else None,
              scales if own_s else None, tensor_scale if own_t else None)
    return packed, scales, tensor_scale


def rhtq_inverse(packed, scales, n: int, signs=None, fmt: str = "int4", group: int = 0,
                 scale_dtype: str | None = None, tensor_scale=None, out=None, stream=None, block=None):
    """Dequantise and undo the rotation: x_hat fp32 [tokens][n].  packed, scales and
    tensor_scale (NVFP4) must have the dtypes and shapes rhtq_forward returns for the same
    (tokens, n, fmt, group, scale_dtype); non-contiguous ones are read through contiguous
    copies.  An `out` passed in must be contiguous fp32 [tokens][n]."""
    torch = _torch()
    if fmt not in _FMT:
        raise ValueError(f"unknown fmt {fmt!r}")
    if packed.dim() != 2:
        raise ValueError("packed must be 2-D [tokens][n/2]")
    tokens = packed.shape[0]
    if scale_dtype is None:
        scale_dtype = _DEFAULT_SCALE[fmt]
    if group == 0:
        group = _DEFAULT_GROUP.get(fmt, 0)
    sdt = _scale_torch_dtype(scale_dtype)
    if packed.dtype != torch.uint8 or tuple(packed.shape) != (tokens, n // 2):
        raise ValueError(f"packed: {packed.dtype} {tuple(packed.shape)}, expected uint8 {(tokens, n // 2)}")
    sshape = scale_shape(tokens, n, fmt, group)
    if scales.dtype != sdt or tuple(scales.shape) != tuple(sshape):
        raise ValueError(f"scales: {scales.dtype} {tuple(scales.shape)}, expected {sdt} {sshape}")
    if fmt == "nvfp4":
        if tensor_scale is None:
            raise ValueError("NVFP4 needs its tensor_scale")
        if tensor_scale.dtype != torch.float32 or tensor_scale.numel() != 1:
            raise ValueError("tensor_scale must be one float32")
    if out is not None:
        _expect(out, "out", torch.float32, (tokens, n))
    dev = packed.device
    _same_device(dev, packed=packed, scales=scales, tensor_scale=tensor_scale if fmt == "nvfp4" else None,
                 out=out)
    # contiguous copies are bound to locals so that they outlive the call
    pc = packed.contiguous()
    sc = scales.contiguous()
    tc = tensor_scale.reshape(1).contiguous() if fmt == "nvfp4" else None
    s = _signs_tensor(signs, n, dev)
    st, other = _resolve_stream(stream)
    own = out is None
    if own:
        out = torch.empty((tokens, n), dtype=torch.float32, device=dev)
    sp = ctypes.c_void_p(st.cuda_stream)
    if block is None or block == n:
        status = lib.rhtq_inverse(_ptr(pc), _ptr(sc), _ptr(tc), tokens, n, _ptr(s), _FMT[fmt], group,
                                  _SCALE[scale_dtype], _ptr(out), sp)
        where = "rhtq_inverse"
    else:
        status = lib.rhtq_inverse_blocked(_ptr(pc), _ptr(sc), _ptr(tc), tokens, n, block, _ptr(s), _FMT[fmt],
                                          group, _SCALE[scale_dtype], _ptr(out), sp)
        where = "rhtq_inverse_blocked"
    _check(status, where)
    _keep_for(st, other, pc if pc is not packed else None, sc if sc is not scales else None,
              tc if (tc is not None and tc is not tensor_scale) else None, s, out if own else None)
    return out


def rhtq_stream_floor(x, packed, scales, stream=None):
    """The streaming floor of the forward call's launch shape (a measurement aid, not part of
    the method): reads x bf16 [tokens][n] (n = 4096 or 12288) and writes packed uint8
    [tokens][n/2] and the scale bytes of `scales` ([tokens][k], any dtype, 4 k * itemsize
    bytes per row a multiple of 4) with the forward kernel's grid and access pattern and no
    arithmetic beyond XOR folds of the loaded words.  Returns (packed, scales)."""
    torch = _torch()
    tokens, n = _rows(x)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    _expect(packed, "packed", torch.uint8, (tokens, n // 2))
    if scales.dim() != 2 or scales.shape[0] != tokens or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous [tokens][k] tensor")
    _same_device(x.device, x=x, packed=packed, scales=scales)
    xc = x.contiguous()
    st, other = _resolve_stream(stream)
    row_bytes = scales.shape[1] * scales.element_size()
    _check(lib.rhtq_stream_floor(_ptr(xc), tokens, n, _ptr(packed), _ptr(scales), row_bytes,
                                 ctypes.c_void_p(st.cuda_stream)), "rhtq_stream_floor")
    _keep_for(st, other, xc if xc is not x else None)
    return packed, scales
