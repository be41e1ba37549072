"""CPU: the C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def R():
    import randomized_hadamard_rotation_amd as R
    return R


def declared_functions():
    inc = os.path.join(ROOT, "include")
    names = set()
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = open(os.path.join(inc, h)).read()
            names |= set(re.findall(r"^\s*(?:int|const char\*)\s+(rhtq_\w+)\s*\(", src, re.M))
    return sorted(names)


def test_exports_every_declared_symbol(R):
    decl = declared_functions()
    assert len(decl) == 11
    lib = ctypes.CDLL(R.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(R.EXPORTED) == decl


def test_abi_version_and_status_strings(R):
    assert R.rhtq_abi_version() == 4
    assert R.rhtq_status_str(0) == "ok"
    assert "invalid" in R.rhtq_status_str(1)
    assert "unsupported" in R.rhtq_status_str(2)
    assert "HIP" in R.rhtq_status_str(3)


def test_supported_matrix(R):
    for k in range(4, 15):
        assert R.rhtq_supported(1 << k, "int4", 0)
        assert R.rhtq_supported(1 << k, "nvfp4", 16)
        assert R.rhtq_supported(1 << k, "mxfp4", 32) == (k >= 5)
    for m in (256, 512, 1024, 2048):
        assert R.rhtq_supported(12 * m, "int4", 128)
    for m in (16, 32, 64, 128):
        assert R.rhtq_supported(172 * m, "int4", 0)
        assert R.rhtq_supported(172 * m, "int4", 16)
        assert R.rhtq_supported(172 * m, "nvfp4", 16)
        assert R.rhtq_supported(172 * m, "mxfp4", 32)
    assert R.rhtq_supported(11008, "int4", 128) and R.rhtq_supported(11008, "int4", 256)
    assert not R.rhtq_supported(11008, "int4", 512)    # 11008 = 21.5 x 512
    for bad in (0, 8, 32768, 100, 12 * 128, 12 * 4096, 172, 172 * 8, 172 * 256, 11000, 10752):
        assert not R.rhtq_supported(bad, "int4", 0)
    assert not R.rhtq_supported(4096, "int4", 96)      # not a power of two
    assert not R.rhtq_supported(4096, "int4", 8)       # below 16
    assert not R.rhtq_supported(4096, "nvfp4", 32)
    assert not R.rhtq_supported(4096, "mxfp4", 16)
    assert R.rhtq_supported(12288, "mxfp4", 32)


def test_signs_from_seed_matches_generator(R):
    from workloads import splitmix64_signs
    for seed in (0, 1, 12345, 2**63 + 7):
        for n in (1, 128, 4096, 12288):
            assert np.array_equal(R.rhtq_signs_from_seed(seed, n), splitmix64_signs(seed, n))


def test_host_validation(R):
    lib = R.lib
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: every call below fails validation
    mis = ctypes.c_void_p(0x100004)           # not 16-byte aligned
    s = ctypes.c_void_p(0)
    # rotate
    assert lib.rhtq_rotate(fake, 0, -1, 4096, None, fake, s) == R.RHTQ_EINVAL
    assert lib.rhtq_rotate(fake, 7, 4, 4096, None, fake, s) == R.RHTQ_EINVAL
    assert lib.rhtq_rotate(fake, 3, 4, 4096, None, fake, s) == R.RHTQ_EINVAL     # no input type 3
    assert lib.rhtq_rotate(mis, R.RHTQ_IN_F16, 4, 4096, None, fake, s) == R.RHTQ_EINVAL
    assert lib.rhtq_rotate(None, R.RHTQ_IN_F16, 0, 4096, None, None, s) == R.RHTQ_OK
    assert lib.rhtq_rotate(fake, 0, 4, 100, None, fake, s) == R.RHTQ_EUNSUPPORTED
    assert lib.rhtq_rotate(None, 0, 4, 4096, None, fake, s) == R.RHTQ_EINVAL
    assert lib.rhtq_rotate(mis, 0, 4, 4096, None, fake, s) == R.RHTQ_EINVAL
    assert lib.rhtq_rotate(fake, 0, 4, 4096, mis, fake, s) == R.RHTQ_EINVAL     # signs misaligned
    assert lib.rhtq_rotate(None, 0, 0, 4096, None, None, s) == R.RHTQ_OK   # empty: no-op
    # forward
    F = lambda *a: lib.rhtq_forward(*a)
    assert F(fake, 0, -2, 4096, None, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 0, 96, 0, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 0, 0, 2, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 1, 16, 1, fake, fake, fake, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 1, 16, 2, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    # MXFP4: group 32 with E8M0 scales only; no tensor scale needed
    assert F(fake, 0, 4, 4096, None, 2, 32, 2, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 2, 16, 3, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 0, 0, 3, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED
    assert F(fake, 0, 4, 4096, None, 2, 32, 4, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 3, 32, 3, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 1, 16, 2, fake, fake, fake, 9, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 9, 16, 2, fake, fake, fake, 0, s) == R.RHTQ_EINVAL
    assert F(None, 0, 4, 4096, None, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 0, 0, 0, mis, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, None, 0, 0, 0, fake, ctypes.c_void_p(0x100002), None, 0, s) == R.RHTQ_EINVAL
    assert F(fake, 0, 4, 4096, mis, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(None, 0, 0, 4096, None, 0, 0, 0, None, None, None, 0, s) == R.RHTQ_OK
    assert F(fake, 3, 4, 4096, None, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(mis, R.RHTQ_IN_F16, 4, 4096, None, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EINVAL
    assert F(None, R.RHTQ_IN_F16, 0, 4096, None, 0, 0, 0, None, None, None, 0, s) == R.RHTQ_OK
    # inverse
    I = lambda *a: lib.rhtq_inverse(*a)
    assert I(fake, fake, None, -1, 4096, None, 0, 0, 0, fake, s) == R.RHTQ_EINVAL
    assert I(fake, fake, None, 4, 4097, None, 0, 0, 0, fake, s) == R.RHTQ_EUNSUPPORTED
    assert I(fake, fake, None, 4, 4096, None, 1, 16, 2, fake, s) == R.RHTQ_EINVAL   # no tensor scale
    assert I(None, fake, None, 4, 4096, None, 0, 0, 0, fake, s) == R.RHTQ_EINVAL
    assert I(None, None, None, 0, 4096, None, 0, 0, 0, None, s) == R.RHTQ_OK
    assert lib.rhtq_signs_from_seed(1, -1, None) == R.RHTQ_EINVAL


def test_stream_floor_host_validation(R):
    lib = R.lib
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: every call below fails validation
    mis = ctypes.c_void_p(0x100002)
    s = ctypes.c_void_p(0)
    SF = lambda *a: lib.rhtq_stream_floor(*a)
    assert SF(fake, 4, 2048, fake, fake, 4, s) == R.RHTQ_EUNSUPPORTED
    assert SF(fake, 4, 11008, fake, fake, 4, s) == R.RHTQ_EUNSUPPORTED
    assert SF(fake, -1, 4096, fake, fake, 4, s) == R.RHTQ_EINVAL
    assert SF(fake, 4, 4096, fake, fake, 6, s) == R.RHTQ_EINVAL      # not a multiple of 4
    assert SF(fake, 4, 4096, fake, fake, 0, s) == R.RHTQ_EINVAL
    assert SF(fake, 4, 4096, fake, fake, 516, s) == R.RHTQ_EINVAL
    assert SF(None, 4, 4096, fake, fake, 4, s) == R.RHTQ_EINVAL
    assert SF(mis, 4, 4096, fake, fake, 4, s) == R.RHTQ_EINVAL       # x not 16-byte aligned
    assert SF(fake, 4, 4096, mis, fake, 4, s) == R.RHTQ_EINVAL
    assert SF(None, 0, 12288, None, None, 192, s) == R.RHTQ_OK       # empty: no-op


def test_python_binding_refuses_cpu_tensors(R):
    import torch
    with pytest.raises(ValueError):
        R.rhtq_rotate(torch.zeros(2, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        R.rhtq_forward(torch.zeros(2, 128, dtype=torch.bfloat16))


def test_blocked_host_validation(R):
    lib = R.lib
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: every call below fails validation
    s = ctypes.c_void_p(0)
    RB = lambda *a: lib.rhtq_rotate_blocked(*a)
    assert RB(fake, 0, 4, 4096, 100, None, fake, s) == R.RHTQ_EUNSUPPORTED     # block not a power of two
    assert RB(fake, 0, 4, 4096, 8, None, fake, s) == R.RHTQ_EUNSUPPORTED       # below 16
    assert RB(fake, 0, 4, 4096, 8192, None, fake, s) == R.RHTQ_EUNSUPPORTED    # above n
    assert RB(fake, 0, 4, 3072, 2048, None, fake, s) == R.RHTQ_EUNSUPPORTED    # does not divide n
    assert RB(fake, 0, 4, 11008, 512, None, fake, s) == R.RHTQ_EUNSUPPORTED    # 11008 = 21.5 x 512
    assert RB(fake, 0, 4, 11000, 11000, None, fake, s) == R.RHTQ_EUNSUPPORTED  # plain call: no H_11000
    assert RB(fake, 0, 4, (1 << 20) + 128, 128, None, fake, s) == R.RHTQ_EUNSUPPORTED
    assert RB(fake, 0, -1, 4096, 128, None, fake, s) == R.RHTQ_EINVAL
    assert RB(None, 0, 0, 4096, 128, None, None, s) == R.RHTQ_OK               # empty: no-op
    assert RB(fake, 0, 2**62, 4096, 16, None, fake, s) == R.RHTQ_EINVAL        # rows overflow
    FB = lambda *a: lib.rhtq_forward_blocked(*a)
    assert FB(fake, 0, 4, 4096, 128, None, 0, 0, 0, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED  # per-row
    assert FB(fake, 0, 4, 4096, 128, None, 0, 256, 0, fake, fake, None, 0, s) == R.RHTQ_EUNSUPPORTED  # group > block
    assert FB(None, 0, 4, 4096, 128, None, 0, 128, 1, fake, fake, None, 0, s) == R.RHTQ_EINVAL     # null x
    assert FB(None, 0, 0, 4096, 4096, None, 0, 0, 0, None, None, None, 0, s) == R.RHTQ_OK
    IB = lambda *a: lib.rhtq_inverse_blocked(*a)
    assert IB(fake, fake, None, 4, 4096, 128, None, 2, 16, 3, fake, s) == R.RHTQ_EUNSUPPORTED      # mxfp4 group 16
    assert IB(None, fake, None, 4, 4096, 128, None, 2, 32, 3, fake, s) == R.RHTQ_EINVAL


def test_python_binding_checks_caller_buffers(R):
    """Caller-supplied outputs and inverse inputs are checked for dtype, shape and contiguity
    before anything touches a device (the C ABI takes bare pointers and cannot)."""
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    bad = [
        dict(fmt="int4", scale_dtype="f32", scales=torch.empty(4, 1, dtype=torch.float16)),    # fp16 for f32
        dict(fmt="int4", group=128, scale_dtype="f16", scales=torch.empty(4, 1, dtype=torch.float16)),  # too few
        dict(fmt="int4", packed=torch.empty(4, 256, dtype=torch.uint8)),                       # n, not n/2
        dict(fmt="int4", packed=torch.empty(128, 4, dtype=torch.uint8).t()),                   # not contiguous
        dict(fmt="nvfp4", tensor_scale=torch.empty(2, dtype=torch.float32)),
        dict(fmt="nvfp4", tensor_scale_mode="given"),                                         # no g given
        dict(fmt="mxfp4", scales=torch.empty(4, 16, dtype=torch.uint8)),                       # blocks of 16
        dict(fmt="int4", group=96),                                                           # does not divide
        dict(fmt="fp4"),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            R.rhtq_forward(x, **kw)
    with pytest.raises(ValueError):
        R.rhtq_rotate(x, out=torch.empty(4, 256, dtype=torch.float16))
    with pytest.raises(ValueError):
        R.rhtq_rotate(torch.zeros(4, 2, 128, dtype=torch.bfloat16))
    p = torch.empty(4, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):   # fp16 scales where the default is fp32
        R.rhtq_inverse(p, torch.empty(4, 1, dtype=torch.float16), 256)
    with pytest.raises(ValueError):   # scales for a different group
        R.rhtq_inverse(p, torch.empty(4, 1, dtype=torch.float16), 256, group=128, scale_dtype="f16")
    with pytest.raises(ValueError):   # NVFP4 without its tensor scale
        R.rhtq_inverse(p, torch.empty(4, 16, dtype=torch.uint8), 256, fmt="nvfp4")
    with pytest.raises(ValueError):   # packed for another width
        R.rhtq_inverse(p, torch.empty(4, 1, dtype=torch.float32), 512)
    # well-formed CPU buffers get through the checks and stop at the device check
    with pytest.raises(ValueError, match="GPU only"):
        R.rhtq_inverse(p, torch.empty(4, 1, dtype=torch.float32), 256)
