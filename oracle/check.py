"""Tolerance rules for comparing a device result with the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

R1  rotated fp32 values: per row, max|y_dev - y_ref| <= 1e-5 * max|y_ref|; a row
    whose reference is all zero must be exactly zero.
R2  scales: fp32 within 1e-6 relative of the oracle; fp16 / E4M3 bit-equal, except
    that adjacent storage values are accepted when the oracle's unrounded scale lies
    within 1e-6 relative of the midpoint between them (a rounding-boundary case);
    the NVFP4 tensor scale within 1e-6 relative.
R3  codes: compared with the oracle's codes recomputed from the device's stored
    scales.  A code may differ only when the oracle's pre-rounding value v lies within
    1e-4 (in scale units) of a rounding boundary and the codes are one step apart;
    such codes may make up at most 1e-4 of all codes.  Where v lies exactly on a
    boundary, both neighbours are nearest and the pages give no tie rule (QuaRot
    reviews page, reviewer 2 follow-up: nearest rounding), so the oracle's choice
    (ties to even) is one of two correct codes: such a mismatch is accepted and not
    counted against the 1e-4.
R4  invariants of the device output, in groups whose stored scale is a normal number of
    its storage type: INT4 codes in [-7, 7]; dequantisation error within half a step.
MXFP4 scales (E8M0 bytes) are exponents: equal, except adjacent where the oracle's block
maximum lies within 1e-6 relative of a power of two (the floor of log2 is a boundary case
there); codes then follow R3 under the device's stored scales.
"""
from __future__ import annotations

import numpy as np

from . import rht_oracle as O

INT4_BOUNDARY_BAND = 1e-4
CODE_MISMATCH_FRACTION = 1e-4
ROT_REL = 1e-5
SCALE_REL = 1e-6


class ParityError(AssertionError):
    pass


def check_rotation(y_dev: np.ndarray, y_ref: np.ndarray) -> dict:
    y_dev = np.asarray(y_dev, dtype=np.float64)
    err = np.max(np.abs(y_dev - y_ref), axis=-1)
    amax = np.max(np.abs(y_ref), axis=-1)
    zero = amax == 0
    if np.any(zero & (err != 0)):
        raise ParityError("R1: a zero row did not rotate to exact zeros")
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, amax))
    worst = float(np.max(rel)) if rel.size else 0.0
    if worst > ROT_REL:
        r = int(np.argmax(rel))
        raise ParityError(f"R1: row {r} relative error {worst:.3e} > {ROT_REL}")
    return {"rot_max_rel_err": worst}


def _adjacent_midpoint_ok(dev_vals, ref_vals, unrounded):
    mid = 0.5 * (dev_vals + ref_vals)
    return np.abs(unrounded - mid) <= SCALE_REL * np.abs(unrounded)


def check_int4_scales(s_dev, y_ref, group, scale_dtype) -> dict:
    yg = y_ref.reshape(y_ref.shape[0], -1, y_ref.shape[1] if group == 0 else group)
    amax = np.max(np.abs(yg), axis=-1)
    unrounded = amax / 7.0
    s_ref = O.int4_scale_store(amax, scale_dtype)
    s_dev = np.asarray(s_dev).reshape(s_ref.shape)
    if scale_dtype == "f32":
        d = np.abs(s_dev.astype(np.float64) - s_ref.astype(np.float64))
        bad = d > SCALE_REL * np.abs(s_ref.astype(np.float64))
        if np.any(bad):
            i = np.argwhere(bad)[0]
            raise ParityError(f"R2: fp32 scale at {tuple(i)}: {s_dev[tuple(i)]} vs {s_ref[tuple(i)]}")
        return {"scale_boundary_cases": 0}
    bits_dev = s_dev.view(np.uint16).astype(np.int64)
    bits_ref = s_ref.view(np.uint16).astype(np.int64)
    diff = bits_dev != bits_ref
    adjacent = np.abs(bits_dev - bits_ref) == 1
    ok = _adjacent_midpoint_ok(s_dev.astype(np.float64), s_ref.astype(np.float64), unrounded)
    bad = diff & ~(adjacent & ok)
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise ParityError(f"R2: fp16 scale at {i}: {s_dev[i]} vs {s_ref[i]} "
                          f"(unrounded {unrounded[i]!r})")
    return {"scale_boundary_cases": int(np.sum(diff))}


def _code_mismatch_check(dev, ref, v, boundary_dist, step_ok, what, enforce_fraction=True, tie=None):
    """Every mismatch must be a one-step boundary case (R3).  Returns the number of mismatches
    that count against the fraction limit (those where v is not exactly on a boundary, `tie`).
    The limit applies to a whole tensor: a caller that checks a tensor in row chunks passes
    enforce_fraction=False and applies check_fraction() to the summed counts."""
    mism = dev != ref
    if not np.any(mism):
        return 0
    allowed = mism & (boundary_dist <= INT4_BOUNDARY_BAND) & step_ok
    if np.any(mism & ~allowed):
        i = tuple(np.argwhere(mism & ~allowed)[0])
        raise ParityError(f"R3: {what} code at {i}: device {dev[i]} oracle {ref[i]} (v = {v[i]!r})")
    n_mism = int(np.sum(mism if tie is None else mism & ~tie))
    if enforce_fraction:
        check_fraction(n_mism, dev.size)
    return n_mism


def check_fraction(n_mism: int, n_codes: int) -> None:
    """R3's limit: boundary mismatches make up at most 1e-4 of all codes of the tensor."""
    if n_mism > CODE_MISMATCH_FRACTION * n_codes:
        raise ParityError(f"R3: {n_mism} boundary mismatches exceed {CODE_MISMATCH_FRACTION} "
                          f"of {n_codes} codes")


def check_int4(packed_dev, s_dev, y_ref, group, scale_dtype, enforce_fraction=True) -> dict:
    rep = check_int4_scales(s_dev, y_ref, group, scale_dtype)
    q_dev = O.unpack_nibbles(packed_dev, signed=True)
    T, n = y_ref.shape
    ng = np.asarray(s_dev).reshape(T, -1).shape[1]
    # R4 holds where the stored scale is a normal number of its storage type.  A scale
    # that saturated (fp16 65504), underflowed to 0 or became subnormal is too coarse
    # for the half-step bound and may legitimately clamp to -8; R3 still applies there.
    sd = np.asarray(s_dev, dtype=np.float64).reshape(T, ng)
    tiny = 2.0 ** -14 if scale_dtype == "f16" else 2.0 ** -126
    sat = np.repeat((sd >= 65504.0) | (sd < tiny), n // ng, axis=1)
    if np.any(((q_dev < -7) | (q_dev > 7)) & ~sat):
        raise ParityError("R4: INT4 code outside [-7, 7]")
    q_ref, v = O.int4_codes(y_ref, np.asarray(s_dev, dtype=np.float64), group)
    frac = np.abs(v - np.floor(v) - 0.5)
    rep["code_mismatches"] = _code_mismatch_check(
        q_dev, q_ref, v, frac, np.abs(q_dev.astype(int) - q_ref.astype(int)) == 1, "INT4", enforce_fraction,
        tie=frac == 0)
    # R4 dequantisation bound with the device's own scales
    yhat = O.dequantize(packed_dev, s_dev, "int4", group)
    sg = np.repeat(np.asarray(s_dev, dtype=np.float64).reshape(y_ref.shape[0], -1),
                   y_ref.shape[1] // np.asarray(s_dev).reshape(y_ref.shape[0], -1).shape[1], axis=1)
    if np.any((np.abs(yhat - y_ref) > 0.5 * sg * (1 + 1e-4) + 1e-30) & ~sat):
        raise ParityError("R4: INT4 dequantisation error above half a step")
    return rep


_E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def check_nvfp4(packed_dev, sc_dev, g_dev, y_ref, g_ref=None, enforce_fraction=True) -> dict:
    rep = {}
    if g_ref is None:
        g_ref = O.nvfp4_tensor_scale(y_ref)
    g_dev = np.float32(g_dev)
    if abs(float(g_dev) - float(g_ref)) > SCALE_REL * abs(float(g_ref)):
        raise ParityError(f"R2: tensor scale {g_dev!r} vs {g_ref!r}")
    # block scales against the oracle (given the device's g)
    T, n = y_ref.shape
    bmax = np.max(np.abs(y_ref.reshape(T, n // 16, 16)), axis=-1)
    if float(g_dev) == 0.0:
        sc_ref = np.zeros_like(bmax, dtype=np.uint8)
        sigma = np.zeros_like(bmax)
    else:
        sigma = bmax / (6.0 * np.float64(g_dev))
        sc_ref = O.e4m3_encode(sigma)
    sc_dev = np.asarray(sc_dev, dtype=np.uint8).reshape(sc_ref.shape)
    diff = sc_dev != sc_ref
    adjacent = np.abs(sc_dev.astype(int) - sc_ref.astype(int)) == 1
    ok = _adjacent_midpoint_ok(O.e4m3_decode(sc_dev), O.e4m3_decode(sc_ref), sigma)
    bad = diff & ~(adjacent & ok)
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise ParityError(f"R2: E4M3 scale at {i}: {sc_dev[i]:#x} vs {sc_ref[i]:#x} (sigma {sigma[i]!r})")
    rep["scale_boundary_cases"] = int(np.sum(diff))
    # codes given the device's stored scales
    c_dev = O.unpack_nibbles(packed_dev, signed=False).astype(np.uint8)
    c_ref, v = O.nvfp4_codes_from_scales(y_ref, sc_dev, g_dev)
    av = np.abs(v)
    dist = np.min(np.abs(av[..., None] - _E2M1_BOUNDS), axis=-1)
    tie = dist == 0
    mag_dev, mag_ref = (c_dev & 7).astype(int), (c_ref & 7).astype(int)
    same_sign = (c_dev & 8) == (c_ref & 8)
    one_step = same_sign & (np.abs(mag_dev - mag_ref) == 1)
    # +-0: both magnitudes zero, only the sign differs, |v| tiny
    signed_zero = (mag_dev == 0) & (mag_ref == 0) & (av < INT4_BOUNDARY_BAND)
    dist = np.where(signed_zero, 0.0, dist)
    rep["code_mismatches"] = _code_mismatch_check(c_dev, c_ref, v, dist, one_step | signed_zero,
                                                  "E2M1", enforce_fraction, tie=tie)
    return rep


def check_mxfp4(packed_dev, sb_dev, y_ref, enforce_fraction=True) -> dict:
    rep = {}
    T, n = y_ref.shape
    bmax = np.max(np.abs(y_ref.reshape(T, n // 32, 32)), axis=-1)
    sb_ref = (O.mxfp4_scale_exponent(bmax) + 127).astype(np.uint8)
    sb_dev = np.asarray(sb_dev, dtype=np.uint8).reshape(sb_ref.shape)
    diff = sb_dev != sb_ref
    adjacent = np.abs(sb_dev.astype(int) - sb_ref.astype(int)) == 1
    # distance of bmax to the power of two between the two candidate exponents
    p2 = np.ldexp(1.0, np.maximum(sb_dev, sb_ref).astype(np.int64) - 127 + 2)
    near = np.abs(bmax - p2) <= SCALE_REL * p2
    bad = diff & ~(adjacent & near)
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise ParityError(f"R2: E8M0 scale at {i}: {sb_dev[i]} vs {sb_ref[i]} (block max {bmax[i]!r})")
    rep["scale_boundary_cases"] = int(np.sum(diff))
    c_dev = O.unpack_nibbles(packed_dev, signed=False).astype(np.uint8)
    c_ref, v = O.mxfp4_codes_from_scales(y_ref, sb_dev)
    av = np.abs(v)
    dist = np.min(np.abs(av[..., None] - _E2M1_BOUNDS), axis=-1)
    tie = dist == 0
    mag_dev, mag_ref = (c_dev & 7).astype(int), (c_ref & 7).astype(int)
    same_sign = (c_dev & 8) == (c_ref & 8)
    one_step = same_sign & (np.abs(mag_dev - mag_ref) == 1)
    signed_zero = (mag_dev == 0) & (mag_ref == 0) & (av < INT4_BOUNDARY_BAND)
    dist = np.where(signed_zero, 0.0, dist)
    rep["code_mismatches"] = _code_mismatch_check(c_dev, c_ref, v, dist, one_step | signed_zero,
                                                  "E2M1", enforce_fraction, tie=tie)
    return rep
