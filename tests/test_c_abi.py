"""The C ABI used from C99 programs (tests/c/): the header compiles as C, the library links
with gcc, and a C program can drive the device.

CPU: rhtq_host_check.c calls the host-only entry points (version, status strings, support
matrix, sign generation, argument checks that fail before any device call); its sign vector
must equal the Python splitmix64 generator's.
GPU: rhtq_device_check.c allocates with the HIP runtime API, runs rhtq_forward (per-token
INT4) and rhtq_rotate on its own stream, and writes the results; they are checked against the
oracle on the same input."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
from oracle import check as C
from workloads import splitmix64_signs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "randomized_hadamard_rotation_amd")
SRC = os.path.join(ROOT, "tests", "c")


def _gcc(src, out, hip=False):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(PKG, "librhtq.so")):
        pytest.fail("librhtq.so is not built")
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include")]
    if hip:
        cmd += ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]
    cmd += [os.path.join(SRC, src), "-o", out, "-L", PKG, "-lrhtq", f"-Wl,-rpath,{PKG}"]
    if hip:
        cmd += ["-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=120)


def test_c_program_uses_the_host_entry_points(tmp_path):
    exe = str(tmp_path / "rhtq_host_check")
    _gcc("rhtq_host_check.c", exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("signs ")][0]
    signs = np.array([int(v) for v in line.split()[1:]], dtype=np.int8)
    assert np.array_equal(signs, splitmix64_signs(12345, 64))


@pytest.mark.gpu
def test_c_program_drives_the_device(tmp_path):
    T, N = 8, 4096
    exe, out = str(tmp_path / "rhtq_device_check"), str(tmp_path / "out.bin")
    _gcc("rhtq_device_check.c", exe, hip=True)
    print(f"[case] C program: rhtq_forward INT4 per-token + rhtq_rotate, {T} x {N} bf16", flush=True)
    r = subprocess.run([exe, out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(out, dtype=np.uint8)
    npk, nsc = T * N // 2, T * 4
    packed = raw[:npk].reshape(T, N // 2)
    scales = raw[npk:npk + nsc].view(np.float32).reshape(T, 1)
    y = raw[npk + nsc:].view(np.float32).reshape(T, N)
    # the program's input, x[t][j] = ((7 j + 13 t) mod 31 - 15) / 8 (exact in bf16)
    t, j = np.meshgrid(np.arange(T), np.arange(N), indexing="ij")
    x = ((7 * j + 13 * t) % 31 - 15) / 8.0
    y_ref = O.rotate(x, splitmix64_signs(7, N))
    C.check_rotation(y, y_ref)
    C.check_int4(packed, scales, y_ref, 0, "f32")
