"""Whole-tensor parity at the benchmark's full sizes, run by tests/test_gpu_fullsize.py.

The device's outputs for every row of a full-size workload are compared with the oracle.
The oracle runs over row chunks in a pool of host processes (spawned, so that no worker
inherits the parent's GPU context).  Each chunk returns counts; the parent sums them and
applies R3's fraction limit to the whole tensor, so "at most 1e-4 of codes" is evaluated
over the entire configuration rather than per chunk.

Workers receive the bf16 or fp16 input as its 16-bit patterns and the device's outputs as
numpy arrays; none of them touches a GPU.
"""
from __future__ import annotations

import numpy as np

import oracle as O
from oracle import check as C


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16 or int16) -> fp64 values, exactly (a bf16 is the top half
    of an fp32)."""
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_chunk(job: dict) -> dict:
    """One row chunk: the oracle's rotation of x, then every rule against the device's
    rotation (R1), scales and codes (R2-R4).  Returns counts for the parent to sum."""
    if job.get("in_dtype") == "f16":
        x = np.asarray(job["bits"]).astype(np.int16).view(np.float16).astype(np.float64)   # exact
    else:
        x = bf16_bits_to_f64(job["bits"])
    s, block = job["signs"], job["block"]
    y_ref = O.rotate(x, s) if not block else O.rotate_blocked(x, s, block)
    rep = {"rows": int(x.shape[0]), "codes": int(x.size), "amax": float(np.max(np.abs(y_ref)))}
    if job.get("y") is not None:
        rep["rot_max_rel_err"] = C.check_rotation(job["y"], y_ref)["rot_max_rel_err"]
    fmt = job["fmt"]
    outs = job["outs"]   # {label: (packed, scales, g)}
    for label, (packed, scales, g) in outs.items():
        if fmt == "int4":
            r = C.check_int4(packed, scales, y_ref, job["group"], job["scale_dtype"], enforce_fraction=False)
        elif fmt == "mxfp4":
            r = C.check_mxfp4(packed, scales, y_ref, enforce_fraction=False)
        else:
            # the tensor scale is checked by the parent against the amax over all chunks; here
            # the block scales and codes follow the device's g (R2, R3)
            r = C.check_nvfp4(packed, scales, g, y_ref, g_ref=np.float32(g), enforce_fraction=False)
        rep[label] = r
    return rep


def merge(reports: list) -> dict:
    """Sum the per-chunk counts: rows, codes, per-output boundary cases and mismatches; the
    worst R1 error; the largest |y| of the oracle."""
    tot = {"rows": 0, "codes": 0, "amax": 0.0}
    for r in reports:
        tot["rows"] += r["rows"]
        tot["codes"] += r["codes"]
        tot["amax"] = max(tot["amax"], r["amax"])
        if "rot_max_rel_err" in r:
            tot["rot_max_rel_err"] = max(tot.get("rot_max_rel_err", 0.0), r["rot_max_rel_err"])
        for k, v in r.items():
            if isinstance(v, dict):
                t = tot.setdefault(k, {"scale_boundary_cases": 0, "code_mismatches": 0})
                t["scale_boundary_cases"] += v["scale_boundary_cases"]
                t["code_mismatches"] += v["code_mismatches"]
    return tot
