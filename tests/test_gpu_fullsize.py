"""GPU parity over every row of each benchmark workload at its full size.

The device runs the workload exactly as the benchmark launches it (same shape, same
call); the oracle then checks every row, in row chunks over a pool of host processes
(tests/fullsize.py).  R3's limit -- at most 1e-4 of codes may differ, each by one step at
a rounding boundary -- is applied to the summed counts of the whole tensor.  Each case
prints its rows, codes, scale boundary cases, code mismatches (and their fraction) and the
worst R1 error of the device's rotation of the same input.
"""
import multiprocessing as mp
import os
import sys

import numpy as np
import pytest

from oracle import check as C
from tests import fullsize as F
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

# rows per oracle chunk, per workload (about 2-16 M elements each)
CASES = {
    "llama_4096_int4": 512,
    "downproj_12288_int4g128": 512,
    "kv_128_int4g128": 131072,
    "nvfp4_4096": 1024,
    "mxfp4_4096": 1024,
    "blockh128_4096_int4g128": 1024,
    "downproj7b_11008_int4g128": 512,
    "wide172_22016_int4g128": 256,
    "llama_4096_int4_f16": 512,
}


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def R():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import randomized_hadamard_rotation_amd as R
    return R


@pytest.fixture(scope="module")
def pool():
    try:
        procs = len(os.sched_getaffinity(0))
    except AttributeError:
        procs = os.cpu_count() or 1
    procs = max(1, min(16, procs))
    with mp.get_context("spawn").Pool(procs) as p:
        yield p


def _host(t):
    return t.detach().cpu().numpy()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(CASES))
def test_workload_every_row(R, pool, name, request):
    import torch
    w = WORKLOADS[name]
    say(f"{name} every row: {w.tokens} x {w.n} {w.fmt} group={w.group} scale={w.scale_dtype}"
        + (f" block={w.block}" if w.block else ""))
    x, s = generate(w, "cuda")
    block = w.block or None
    outs = {}
    packed, scales, g = R.rhtq_forward(x, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype, block=block)
    torch.cuda.synchronize()
    g_dyn = None if g is None else float(g.item())
    outs["dynamic" if w.fmt == "nvfp4" else "forward"] = (_host(packed), _host(scales), g_dyn)
    del packed, scales
    if w.fmt == "nvfp4":
        # one pass with the tensor scale given (the device's dynamic g, checked below)
        gt = torch.tensor([g_dyn], dtype=torch.float32, device="cuda")
        packed, scales, _ = R.rhtq_forward(x, s, fmt="nvfp4", group=16, scale_dtype="e4m3",
                                           tensor_scale=gt, tensor_scale_mode="given")
        torch.cuda.synchronize()
        outs["given"] = (_host(packed), _host(scales), g_dyn)
        del packed, scales
    y = R.rhtq_rotate(x, s, block=block)
    torch.cuda.synchronize()
    y_h = _host(y)
    del y
    bits = _host(x.view(torch.int16))
    del x
    torch.cuda.empty_cache()

    step = CASES[name]
    jobs = []
    for r0 in range(0, w.tokens, step):
        r1 = min(w.tokens, r0 + step)
        jobs.append({"bits": bits[r0:r1], "in_dtype": w.in_dtype, "signs": s, "block": w.block, "fmt": w.fmt,
                     "group": w.group,
                     "scale_dtype": w.scale_dtype, "y": y_h[r0:r1],
                     "outs": {k: (p[r0:r1], sc[r0:r1], gg) for k, (p, sc, gg) in outs.items()}})
    say(f"{name}: {len(jobs)} chunks of {step} rows")
    tot = F.merge(list(pool.imap_unordered(F.check_chunk, jobs)))
    assert tot["rows"] == w.tokens and tot["codes"] == w.tokens * w.n
    if w.fmt == "nvfp4":
        g_ref = np.float32(tot["amax"] / 2688.0)
        assert abs(g_dyn - float(g_ref)) <= C.SCALE_REL * float(g_ref), (g_dyn, g_ref)
        tot["tensor_scale"] = {"device": g_dyn, "oracle": float(g_ref)}
    for k in outs:
        C.check_fraction(tot[k]["code_mismatches"], tot["codes"])
        tot[k]["mismatch_fraction"] = tot[k]["code_mismatches"] / tot["codes"]
    assert tot["rot_max_rel_err"] <= C.ROT_REL
    print(f"[fullsize] {name}: {tot}", flush=True)
    parts = [f"{name} {w.tokens}x{w.n}: {tot['codes']} codes"]
    for k in outs:
        parts.append(f"{k} mismatches {tot[k]['code_mismatches']} ({tot[k]['mismatch_fraction']:.1e}), "
                     f"scale boundary cases {tot[k]['scale_boundary_cases']}")
    parts.append(f"worst R1 {tot['rot_max_rel_err']:.2e}")
    if "tensor_scale" in tot:
        ts = tot["tensor_scale"]
        parts.append(f"g rel diff {abs(ts['device'] - ts['oracle']) / ts['oracle']:.1e}")
    request.config.fullsize_lines.append("; ".join(parts))
