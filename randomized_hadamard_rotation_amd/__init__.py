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
RHTQ_IN_BF16, RHTQ_IN_F32 = 0, 1
RHTQ_FMT_INT4, RHTQ_FMT_NVFP4, RHTQ_FMT_MXFP4 = 0, 1, 2
RHTQ_SCALE_F32, RHTQ_SCALE_F16, RHTQ_SCALE_E4M3, RHTQ_SCALE_E8M0 = 0, 1, 2, 3
RHTQ_TENSOR_SCALE_DYNAMIC, RHTQ_TENSOR_SCALE_GIVEN = 0, 1

_FMT = {"int4": RHTQ_FMT_INT4, "nvfp4": RHTQ_FMT_NVFP4, "mxfp4": RHTQ_FMT_MXFP4}
_SCALE = {"f32": RHTQ_SCALE_F32, "f16": RHTQ_SCALE_F16, "e4m3": RHTQ_SCALE_E4M3, "e8m0": RHTQ_SCALE_E8M0}
_DEFAULT_SCALE = {"int4": "f32", "nvfp4": "e4m3", "mxfp4": "e8m0"}
_DEFAULT_GROUP = {"nvfp4": 16, "mxfp4": 32}

EXPORTED = ["rhtq_abi_version", "rhtq_status_str", "rhtq_supported", "rhtq_rotate",
            "rhtq_forward", "rhtq_inverse", "rhtq_signs_from_seed", "rhtq_rotate_blocked",
            "rhtq_forward_blocked", "rhtq_inverse_blocked"]


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


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("rhtq runs on the GPU only: pass device tensors")


def _signs_tensor(signs, n, device):
    """Device int8 [n] from a tensor / numpy array / None (marshalling only)."""
    torch = _torch()
    if signs is None:
        return None
    if isinstance(signs, np.ndarray):
        signs = torch.from_numpy(np.ascontiguousarray(signs.astype(np.int8)))
    if signs.dtype != torch.int8 or signs.numel() != n:
        raise ValueError("signs must be int8 with n entries")
    return signs.to(device).contiguous()


def _in_dtype(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        return RHTQ_IN_BF16
    if x.dtype == torch.float32:
        return RHTQ_IN_F32
    raise ValueError("x must be bfloat16 or float32")


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


def rhtq_rotate(x, signs=None, out=None, stream=None, block=None):
    """y = H_n diag(signs) x / sqrt(n) per row, fp32 [tokens][n].  With block = b < n the
    rotation is block-diagonal: (I (x) H_b) diag(signs) x / sqrt(b)."""
    torch = _torch()
    _need_device(x)
    x = x.contiguous()
    tokens, n = x.shape
    s = _signs_tensor(signs, n, x.device)
    if out is None:
        out = torch.empty((tokens, n), dtype=torch.float32, device=x.device)
    if block is None or block == n:
        _check(lib.rhtq_rotate(_ptr(x), _in_dtype(x), tokens, n, _ptr(s), _ptr(out), _stream(stream)),
               "rhtq_rotate")
    else:
        _check(lib.rhtq_rotate_blocked(_ptr(x), _in_dtype(x), tokens, n, block, _ptr(s), _ptr(out),
                                       _stream(stream)), "rhtq_rotate_blocked")
    return out


def scale_shape(tokens: int, n: int, fmt: str, group: int):
    g = n if group == 0 else group
    return (tokens, n // g)


def rhtq_forward(x, signs=None, fmt: str = "int4", group: int = 0, scale_dtype: str | None = None,
                 tensor_scale=None, tensor_scale_mode: str = "dynamic", packed=None, scales=None,
                 stream=None, block=None):
    """Rotate, quantise, pack.  Returns (packed uint8 [tokens][n/2], scales, tensor_scale).

    INT4: scales fp32/fp16 [tokens][n/group] (group 0 = one per row).
    NVFP4: scales uint8 E4M3 [tokens][n/16]; tensor_scale a device float32 [1]
    (written in 'dynamic' mode, read in 'given' mode).
    MXFP4: scales uint8 E8M0 [tokens][n/32].
    block = b < n: block-diagonal rotation (groups inside a block)."""
    torch = _torch()
    _need_device(x)
    x = x.contiguous()
    tokens, n = x.shape
    if scale_dtype is None:
        scale_dtype = _DEFAULT_SCALE[fmt]
    if group == 0:
        group = _DEFAULT_GROUP.get(fmt, 0)
    s = _signs_tensor(signs, n, x.device)
    if packed is None:
        packed = torch.empty((tokens, n // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        sdt = {"f32": torch.float32, "f16": torch.float16, "e4m3": torch.uint8, "e8m0": torch.uint8}[scale_dtype]
        scales = torch.empty(scale_shape(tokens, n, fmt, group), dtype=sdt, device=x.device)
    if fmt == "nvfp4" and tensor_scale is None:
        tensor_scale = torch.zeros(1, dtype=torch.float32, device=x.device)
    mode = RHTQ_TENSOR_SCALE_DYNAMIC if tensor_scale_mode == "dynamic" else RHTQ_TENSOR_SCALE_GIVEN
    if block is None or block == n:
        _check(lib.rhtq_forward(_ptr(x), _in_dtype(x), tokens, n, _ptr(s), _FMT[fmt], group,
                                _SCALE[scale_dtype], _ptr(packed), _ptr(scales), _ptr(tensor_scale),
                                mode, _stream(stream)), "rhtq_forward")
    else:
        _check(lib.rhtq_forward_blocked(_ptr(x), _in_dtype(x), tokens, n, block, _ptr(s), _FMT[fmt], group,
                                        _SCALE[scale_dtype], _ptr(packed), _ptr(scales), _ptr(tensor_scale),
                                        mode, _stream(stream)), "rhtq_forward_blocked")
    return packed, scales, tensor_scale


def rhtq_inverse(packed, scales, n: int, signs=None, fmt: str = "int4", group: int = 0,
                 scale_dtype: str | None = None, tensor_scale=None, out=None, stream=None, block=None):
    """Dequantise and undo the rotation: x_hat fp32 [tokens][n]."""
    torch = _torch()
    _need_device(packed, scales, tensor_scale)
    tokens = packed.shape[0]
    if scale_dtype is None:
        scale_dtype = _DEFAULT_SCALE[fmt]
    if group == 0:
        group = _DEFAULT_GROUP.get(fmt, 0)
    s = _signs_tensor(signs, n, packed.device)
    if out is None:
        out = torch.empty((tokens, n), dtype=torch.float32, device=packed.device)
    if block is None or block == n:
        _check(lib.rhtq_inverse(_ptr(packed.contiguous()), _ptr(scales.contiguous()), _ptr(tensor_scale),
                                tokens, n, _ptr(s), _FMT[fmt], group, _SCALE[scale_dtype], _ptr(out),
                                _stream(stream)), "rhtq_inverse")
    else:
        _check(lib.rhtq_inverse_blocked(_ptr(packed.contiguous()), _ptr(scales.contiguous()), _ptr(tensor_scale),
                                        tokens, n, block, _ptr(s), _FMT[fmt], group, _SCALE[scale_dtype],
                                        _ptr(out), _stream(stream)), "rhtq_inverse_blocked")
    return out
