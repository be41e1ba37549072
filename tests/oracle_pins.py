"""Pins of the CPU oracle to facts outside itself.

Each pin takes the oracle module as an argument so that the same checks can be
run against deliberately broken copies (tests/test_oracle_mutations.py): every
plausible mistake in the oracle must make at least one pin fail.

What fixes each pin:
  * scipy.linalg.hadamard -- an independent library construction of Sylvester H
  * integer identities    -- H H^T = n I, the involution H (H v) = n v
  * brute force           -- the fast transform equals the dense product on integers
  * closed forms          -- a signed Hadamard row rotates to sqrt(n) e_k (E3);
                             hand-derived worked examples E1 (n = 4) and E2 (n = 4096)
  * textbook rounding     -- round-half-even on INT4 and E2M1 ties
  * library casts         -- torch.float8_e4m3fn on in-range values, numpy float16
  * invariants            -- Parseval, round trip (QuaRot reviews, review 2 Summary:
                             the RHT is invertible up to machine precision)
"""
from __future__ import annotations

import math

import numpy as np
import scipy.linalg


def _check(cond, msg):
    if not cond:
        raise AssertionError(msg)


def pin_sylvester_matches_scipy(O):
    for k in range(0, 11):
        n = 1 << k
        _check(np.array_equal(O.sylvester(n), scipy.linalg.hadamard(n)), f"Sylvester H_{n} != scipy")


def pin_orthogonality(O):
    H12 = O.h12()
    _check(H12.shape == (12, 12) and set(np.unique(H12)) == {-1, 1}, "H12 entries must be +-1")
    _check(np.array_equal(H12 @ H12.T, 12 * np.eye(12, dtype=np.int64)), "H12 H12^T != 12 I")
    for n in [1, 2, 4, 64, 512, 12, 24, 48, 12 * 64, 12 * 128]:
        H = O.hadamard(n)
        _check(np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64)), f"H_{n} H^T != n I")


def pin_h172_williamson(O):
    """The order-172 factor: four symmetric, pairwise commuting +-1 circulants of order 43 whose
    squares sum to 172 I, and the array built from them is Hadamard (H H^T = 172 I)."""
    rows = O.williamson43_rows()
    mats = []
    for r in rows:
        r = np.asarray(r, dtype=np.int64)
        _check(r.shape == (43,) and set(np.unique(r)) <= {-1, 1} and r[0] == 1, "circulant first row")
        _check(np.array_equal(r[1:], r[1:][::-1]), "circulant must be symmetric (r[k] = r[43 - k])")
        mats.append(scipy.linalg.circulant(r).T)   # scipy's circulant has r as its first column
    S = sum(m @ m for m in mats)
    _check(np.array_equal(S, 172 * np.eye(43, dtype=np.int64)), "A^2 + B^2 + C^2 + D^2 != 172 I")
    for i in range(4):
        for j in range(4):
            _check(np.array_equal(mats[i] @ mats[j], mats[j] @ mats[i]), "circulants must commute")
    H = O.h172()
    _check(H.shape == (172, 172) and set(np.unique(H)) == {-1, 1}, "H172 entries must be +-1")
    _check(np.array_equal(H @ H.T, 172 * np.eye(172, dtype=np.int64)), "H172 H172^T != 172 I")
    # the first block row is [A B C D]
    _check(np.array_equal(H[:43, :43], mats[0]) and np.array_equal(H[:43, 129:], mats[3]), "block row 0")
    for n in [172, 344, 688]:
        Hn = O.hadamard(n)
        _check(np.array_equal(Hn @ Hn.T, n * np.eye(n, dtype=np.int64)), f"H_{n} H^T != n I")


def pin_fwht_equals_dense(O):
    rng = np.random.default_rng(11)
    for n in [1, 2, 4, 8, 16, 32, 64, 128, 256, 1024, 4096]:
        v = rng.integers(-1000, 1000, size=(3, n)).astype(np.float64)
        ref = v @ scipy.linalg.hadamard(n).T.astype(np.float64)
        _check(np.array_equal(O.fwht(v), ref), f"fwht != dense at n={n}")
        _check(np.array_equal(O.fwht(O.fwht(v)), n * v), f"fwht involution fails at n={n}")
    for m in [1, 2, 4, 16, 64, 256]:
        n = 12 * m
        v = rng.integers(-1000, 1000, size=(2, n)).astype(np.float64)
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        fast = O.rotate(v, s) * math.sqrt(n)
        dense = (v * s) @ O.hadamard(n).T.astype(np.float64)
        _check(np.allclose(fast, dense, rtol=0, atol=1e-9 * np.abs(dense).max()),
               f"fast 12x rotation != dense at n={n}")
    for m in [1, 2, 16]:
        n = 172 * m
        v = rng.integers(-1000, 1000, size=(2, n)).astype(np.float64)
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        fast = O.rotate(v, s) * math.sqrt(n)
        dense = (v * s) @ O.hadamard(n).T.astype(np.float64)
        _check(np.allclose(fast, dense, rtol=0, atol=1e-9 * np.abs(dense).max()),
               f"fast 172x rotation != dense at n={n}")


def pin_rotate_matches_scipy_definition(O):
    rng = np.random.default_rng(12)
    for n in [16, 128, 1024]:
        x = rng.standard_normal((4, n))
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        ref = scipy.linalg.hadamard(n).astype(np.float64) @ (x * s).T / math.sqrt(n)
        _check(np.allclose(O.rotate(x, s), ref.T, rtol=0, atol=1e-12), f"rotate != H D x / sqrt(n), n={n}")


def pin_parseval_and_roundtrip(O):
    rng = np.random.default_rng(13)
    for n in [16, 128, 4096, 12288, 3072, 11008, 2752]:
        x = rng.standard_normal((3, n)) * np.exp(rng.standard_normal(n))
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        y = O.rotate(x, s)
        _check(np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12),
               f"Parseval fails at n={n}")
        back = O.inverse_rotate(y, s)
        _check(np.max(np.abs(back - x)) <= 1e-12 * np.max(np.abs(x)), f"round trip fails at n={n}")


def _signed_row(O, n, k, s):
    """x_j = s_j * H_n[k][j] built from one row of the oracle's dense H."""
    f, m = O.split_width(n)
    if f == 1:
        i = np.arange(n)
        a = k & i
        pc = np.array([bin(int(t)).count("1") for t in a])
        row = np.where(pc & 1, -1.0, 1.0)
    else:
        row = np.kron(O.factor_matrix(f)[k // m].astype(np.float64), _signed_row(O, m, k % m, np.ones(m)))
    return row * s


def pin_e3_closed_form(O):
    """x = s * H_n[k] rotates to sqrt(n) e_k; its quantisation is fully determined."""
    rng = np.random.default_rng(14)
    for n, k in [(16, 5), (128, 77), (4096, 1234), (12288, 7000), (3072, 2049), (11008, 9000)]:
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        x = _signed_row(O, n, k, s)[None, :]
        y = O.rotate(x, s)
        e = np.zeros((1, n)); e[0, k] = math.sqrt(n)
        _check(np.max(np.abs(y - e)) <= 1e-9, f"E3 rotation at n={n}")
        # per-token INT4, fp32 scale: scale sqrt(n)/7, code 7 at k
        q, sc, _ = O.quantize_int4(y, 0, "f32")
        _check(sc[0, 0] == np.float32(math.sqrt(n) / 7.0), f"E3 per-token scale at n={n}")
        _check(q[0, k] == 7 and np.count_nonzero(q) == 1, f"E3 per-token codes at n={n}")
        # INT4 g128 fp16: only k's group has a (fp16-rounded) scale
        if n % 128 == 0:
            q, sc, _ = O.quantize_int4(y, 128, "f16")
            gk = k // 128
            _check(sc[0, gk] == np.float16(math.sqrt(n) / 7.0), f"E3 g128 scale at n={n}")
            _check(np.count_nonzero(sc) == 1 and q[0, k] == 7 and np.count_nonzero(q) == 1,
                   f"E3 g128 codes at n={n}")
        # NVFP4: the block of k has E4M3 448 (0x7E) and E2M1 6 (0b0111)
        c, bs, g, _ = O.quantize_nvfp4(y)
        _check(g == np.float32(math.sqrt(n) / 2688.0), f"E3 tensor scale at n={n}")
        _check(bs[0, k // 16] == 0x7E and np.count_nonzero(bs) == 1, f"E3 block scale at n={n}")
        _check(c[0, k] == 0b0111 and np.count_nonzero(c) == 1, f"E3 E2M1 code at n={n}")
    # n = 12288 group scale printed as a number: fp16(sqrt(12288)/7) = 15.8359375
    _check(float(np.float16(math.sqrt(12288) / 7.0)) == 15.8359375, "fp16 rounding of 110.85/7")


def pin_e1_worked_example(O):
    """n = 4, s = (+,-,+,+), x = (4.25, -1.25, 5.25, 3.25):
    s*x = (4.25, 1.25, 5.25, 3.25); H4 (s*x) = (14, 5, -3, 1); / 2 -> y = (7, 2.5, -1.5, 0.5).
    Per-token scale 7/7 = 1; RNE codes (7, 2, -2, 0); bytes 0x27, 0x0E."""
    x = np.array([[4.25, -1.25, 5.25, 3.25]])
    s = np.array([1, -1, 1, 1], dtype=np.int8)
    out = O.forward(x, s, "int4", 0, "f32")
    _check(np.array_equal(out["y"], [[7.0, 2.5, -1.5, 0.5]]), "E1 rotation")
    _check(out["scales"][0, 0] == 1.0, "E1 scale")
    _check(np.array_equal(out["codes"], [[7, 2, -2, 0]]), "E1 codes")
    _check(np.array_equal(out["packed"], [[0x27, 0x0E]]), "E1 packed bytes")


def e2_input(n: int = 4096, seed: int = 0):
    """E2: y* = (7, 2.5, -1.5, 0.5, 0, ...), x = s * (H y*) / sqrt(n).  For the
    Sylvester H, (H y*)_i = 7 + 2.5 (-1)^{i0} - 1.5 (-1)^{i1} + 0.5 (-1)^{i0+i1}
    takes the values 8.5, 2.5, 10.5, 6.5 for (i1 i0) = 00, 01, 10, 11; divided by
    sqrt(4096) = 64 they are exact in bf16."""
    i = np.arange(n)
    b0 = np.where(i & 1, -1.0, 1.0)
    b1 = np.where(i & 2, -1.0, 1.0)
    hy = 7.0 + 2.5 * b0 - 1.5 * b1 + 0.5 * b0 * b1
    rng = np.random.default_rng(seed)
    s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
    return (s * hy / math.sqrt(n))[None, :], s


def pin_e2_worked_example(O):
    x, s = e2_input()
    out = O.forward(x, s, "int4", 0, "f32")
    want = np.zeros((1, 4096)); want[0, :4] = [7.0, 2.5, -1.5, 0.5]
    _check(np.array_equal(out["y"], want), "E2 rotation")
    _check(out["scales"][0, 0] == 1.0, "E2 scale")
    _check(np.array_equal(out["codes"][0, :4], [7, 2, -2, 0]) and
           np.count_nonzero(out["codes"]) == 3, "E2 codes")
    _check(out["packed"][0, 0] == 0x27 and out["packed"][0, 1] == 0x0E and
           not np.any(out["packed"][0, 2:]), "E2 packed row")


def pin_int4_rounding(O):
    y = np.array([[0.5, 1.5, 2.5, -1.5, -2.5, -0.5, 3.49, 7.0]])
    # scale fixed to 1 through amax 7
    q, s, _ = O.quantize_int4(y, 0, "f32")
    _check(s[0, 0] == 1.0, "scale 7/7")
    _check(np.array_equal(q, [[0, 2, 2, -2, -2, 0, 3, 7]]), f"RNE ties: {q}")
    rng = np.random.default_rng(15)
    y = rng.standard_normal((50, 256)) * np.exp(rng.standard_normal((50, 1)))
    for group, sd in [(0, "f32"), (16, "f16"), (128, "f16"), (64, "f32")]:
        q, s, _ = O.quantize_int4(y, group, sd)
        _check(np.all(np.abs(q) <= 7), "-8 or beyond produced")
        g = y.shape[1] if group == 0 else group
        yhat = O.dequantize(O.pack_nibbles(q), s, "int4", group)
        step = np.repeat(s.astype(np.float64), g, axis=1)
        _check(np.all(np.abs(yhat - y) <= 0.5 * step * (1 + 1e-12)), "dequant error > s/2")
        amax_pos = np.argmax(np.abs(y.reshape(50, -1, g)), axis=-1)
        qa = np.take_along_axis(q.reshape(50, -1, g), amax_pos[..., None], axis=-1)
        if sd == "f32":
            _check(np.all(np.abs(qa) == 7), "group amax element must map to +-7")


def pin_fp16_storage(O):
    rng = np.random.default_rng(16)
    a = rng.random(1000) * 1e4
    _check(np.array_equal(O.int4_scale_store(a, "f16"), (a / 7.0).astype(np.float16)),
           "fp16 storage != numpy float16 RNE")
    _check(O.int4_scale_store(np.array([1e7]), "f16")[0] == np.float16(65504), "fp16 saturation")


def pin_e2m1(O):
    ties = {0.25: 0b0000, 0.75: 0b0010, 1.25: 0b0010, 1.75: 0b0100, 2.5: 0b0100,
            3.5: 0b0110, 5.0: 0b0110, 7.0: 0b0111, 100.0: 0b0111, -0.1: 0b1000,
            0.0: 0b0000, -6.0: 0b1111, 0.5: 0b0001, 2.9: 0b0101, -3.1: 0b1101}
    for v, c in ties.items():
        got = int(O.e2m1_encode(np.array([v]))[0])
        _check(got == c, f"E2M1({v}) = {got:#06b}, want {c:#06b}")
    for c in range(16):
        if c == 8:
            continue  # -0 decodes to 0 and re-encodes as +0
        _check(int(O.e2m1_encode(O.e2m1_decode(np.array([c])))[0]) == c, f"E2M1 enc(dec({c}))")
    # brute force: nearest grid point, ties to even code
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for v in np.linspace(0, 7, 2801):
        d = np.abs(grid - v)
        cands = np.flatnonzero(d == d.min())
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        _check(int(O.e2m1_encode(np.array([v]))[0]) == want, f"E2M1 brute force at {v}")


def pin_e4m3(O):
    import torch
    codes = np.arange(127, dtype=np.uint8)
    _check(np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes), "E4M3 enc(dec(c)) != c")
    _check(O.e4m3_decode(np.array([0x7E]))[0] == 448.0, "E4M3 max is 448")
    _check(O.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9, "E4M3 min subnormal")
    rng = np.random.default_rng(17)
    vals = np.concatenate([rng.random(4000) * 448.0, np.exp(rng.uniform(-14, 6, 4000)),
                           O.e4m3_values(),
                           0.5 * (O.e4m3_values()[1:] + O.e4m3_values()[:-1])])
    vals = vals[vals <= 448.0]
    ref = torch.tensor(vals, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    _check(np.array_equal(O.e4m3_encode(vals), ref), "E4M3 encode != torch float8_e4m3fn")
    _check(O.e4m3_encode(np.array([1e6]))[0] == 0x7E, "E4M3 saturates at 448")
    _check(O.e4m3_encode(np.array([1.01 * 2.0 ** -10]))[0] == 0x01, "E4M3 subnormal rounding")


def pin_nvfp4_invariants(O):
    rng = np.random.default_rng(18)
    x = rng.standard_normal((8, 256)) * np.exp(rng.standard_normal((8, 1)))
    s = np.where(rng.random(256) < 0.5, -1, 1).astype(np.int8)
    out = O.forward(x, s, "nvfp4", 16)
    y = out["y"]
    g = out["tensor_scale"]
    _check(g == np.float32(np.max(np.abs(y)) / 2688.0), "g = fl32(amax / (6 * 448))")
    t, j = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    _check(out["scales"][t, j // 16] == 0x7E, "amax block must take E4M3 448")
    _check(out["codes"][t, j] & 7 == 7, "amax element must take E2M1 6")
    yhat = O.dequantize(out["packed"], out["scales"], "nvfp4", 16, g)
    seff = np.repeat(O.e4m3_decode(out["scales"]) * np.float64(g), 16, axis=1)
    av = np.abs(y) / np.where(seff > 0, seff, 1)
    half_step = np.where(av < 2, 0.25, np.where(av < 4, 0.5, 1.0))
    half_step = np.where(av > 6, av - 6 + 0.0, half_step)
    _check(np.all(np.abs(yhat - y) <= half_step * seff * (1 + 1e-9) + 1e-300), "E2M1 dequant bound")
    # every block whose scale is a normal E4M3 value below 448 carries its maximum b to
    # b / (dec(s_b) g) within E4M3's half step of 6: the scale is b / (6 g) to 2^-4 relative
    bmax = np.max(np.abs(y.reshape(8, 16, 16)), axis=-1)
    dec = O.e4m3_decode(out["scales"])
    normal = (dec >= 2.0 ** -6) & (dec < 448.0) & (bmax > 0)
    r = bmax[normal] / (dec[normal] * np.float64(g))
    _check(normal.sum() > 64 and np.all((r >= 6 / (1 + 2.0 ** -4)) & (r <= 6 / (1 - 2.0 ** -4))),
           "block maxima must land near E2M1 6")


def pin_mxfp4_closed_form(O):
    """E3 for MXFP4: y = sqrt(n) e_k, so only k's 32-block is non-zero.  Its shared
    exponent is floor(log2(sqrt(n))) - 2 (OCP MX v1.0: the largest E2M1 normal is
    1.5 * 2^2); every other block stores exponent -127 (byte 0) and codes 0."""
    rng = np.random.default_rng(19)
    # (n, k, expected scale byte, expected E2M1 code at k)
    cases = [(128, 77, 127 + 1, 0b0111),      # 11.31 / 2 = 5.66 -> 6
             (4096, 1234, 127 + 4, 0b0110),   # 64 / 16 = 4
             (12288, 7000, 127 + 4, 0b0111),  # 110.85 / 16 = 6.93 -> saturates at 6
             (3072, 2049, 127 + 3, 0b0111)]   # 55.43 / 8 = 6.93 -> 6
    for n, k, sbyte, code in cases:
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        x = _signed_row(O, n, k, s)[None, :]
        out = O.forward(x, s, "mxfp4", 32)
        sb = out["scales"]
        _check(sb[0, k // 32] == sbyte, f"MXFP4 E3 scale byte at n={n}")
        _check(np.count_nonzero(sb) == 1, f"MXFP4 E3 other blocks at n={n}")
        _check(out["codes"][0, k] == code and np.count_nonzero(out["codes"]) == 1, f"MXFP4 E3 codes at n={n}")


def pin_mxfp4_worked_block(O):
    """A hand-made 32-block: maximum 7 * 2^3 = 56, so X = 2^(5 - 2) = 8, byte 130.
    Elements / 8: 5 -> 4 (tie, even mantissa), -2.5 -> -2, 0.75 -> 1, 0.25 -> 0,
    -0.2 -> -0 (sign kept), 7 -> 6 (saturation), 1.75 -> 2."""
    y = np.zeros((1, 64))
    y[0, :7] = np.array([5.0, -2.5, 0.75, 0.25, -0.2, 7.0, 1.75]) * 8.0
    c, sb, _ = O.quantize_mxfp4(y)
    _check(sb[0, 0] == 130 and sb[0, 1] == 0, "MXFP4 block scale bytes")
    _check(list(c[0, :7]) == [0b0110, 0b1100, 0b0010, 0b0000, 0b1000, 0b0111, 0b0100], "MXFP4 block codes")
    _check(not np.any(c[0, 7:]), "MXFP4 zero codes")
    # the E8M0 byte is an exponent with bias 127 (torch's float8_e8m0fnu decodes it the same way)
    import torch
    b = torch.tensor([0, 1, 127, 130, 254], dtype=torch.uint8)
    _check(torch.equal(b.view(torch.float8_e8m0fnu).float(),
                       torch.tensor([2.0 ** -127, 2.0 ** -126, 1.0, 8.0, 2.0 ** 127])), "E8M0 bias")
    yhat = O.dequantize(O.pack_nibbles(c), sb, "mxfp4", 32)
    _check(np.array_equal(yhat[0, :7], np.array([4.0, -2.0, 1.0, 0.0, -0.0, 6.0, 2.0]) * 8.0),
           "MXFP4 dequantisation")


def pin_mxfp4_invariants(O):
    """Every non-zero block's maximum lands in [4, 8) scale units (brute force over the
    candidate exponents), and dequantisation stays within half an E2M1 step, or below the
    saturation overshoot for maxima in [6, 8)."""
    rng = np.random.default_rng(20)
    x = rng.standard_normal((6, 512)) * np.exp(3 * rng.standard_normal((6, 1)))
    x[0, :64] = 0.0
    s = np.where(rng.random(512) < 0.5, -1, 1).astype(np.int8)
    out = O.forward(x, s, "mxfp4", 32)
    y = out["y"]
    bmax = np.max(np.abs(y.reshape(6, 16, 32)), axis=-1)
    for t in range(6):
        for b in range(16):
            if bmax[t, b] == 0:
                continue
            e = [k for k in range(-127, 128) if 2.0 ** (k + 2) <= bmax[t, b] < 2.0 ** (k + 3)]
            _check(len(e) == 1 and out["scales"][t, b] == e[0] + 127, "MXFP4 shared exponent")
    X = np.repeat(np.ldexp(1.0, out["scales"].astype(np.int64) - 127), 32, axis=1)
    yhat = O.dequantize(out["packed"], out["scales"], "mxfp4", 32)
    av = np.abs(y) / X
    bound = np.where(av < 2, 0.25, np.where(av < 4, 0.5, 1.0))
    bound = np.where(av > 6, av - 6, bound)
    _check(np.all(np.abs(yhat - y) <= bound * X * (1 + 1e-9)), "MXFP4 dequant bound")


def pin_blocked_rotation(O):
    """Block-diagonal rotation against its dense definition kron(I, H_b) D / sqrt(b) (scipy's
    Hadamard), block = n reducing to the full rotation, orthogonality and the exact inverse."""
    rng = np.random.default_rng(21)
    for n, b in [(64, 16), (256, 128), (512, 32), (3072, 1024), (96, 32)]:
        x = rng.standard_normal((3, n))
        s = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
        dense = np.kron(np.eye(n // b), scipy.linalg.hadamard(b)) * s[None, :] / math.sqrt(b)
        y = O.rotate_blocked(x, s, b)
        _check(np.max(np.abs(y - x @ dense.T)) <= 1e-12 * np.abs(y).max(), f"blocked rotation n={n} b={b}")
        _check(np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12), "blocked Parseval")
        _check(np.max(np.abs(O.inverse_rotate_blocked(y, s, b) - x)) <= 1e-12 * np.abs(x).max(), "blocked inverse")
    x = rng.standard_normal((2, 1024))
    s = np.where(rng.random(1024) < 0.5, -1, 1).astype(np.int8)
    _check(np.array_equal(O.rotate_blocked(x, s, 1024), O.rotate(x, s)), "block = n is the full rotation")


def pin_nvfp4_block_scale_closed_form(O):
    """NVFP4 block scales from a given tensor scale g ("Methodology checks for NVFP4 W4A4 on
    Qwen3-8B", NVFP4 results: E2M1 codes under E4M3 block scales).  A block's maximum b must
    map to the largest E2M1 magnitude 6, so its scale is b / (6 g), rounded to E4M3.  With
    g = 0.5 and block maxima b = 3 sigma, sigma exactly representable, the scale codes follow
    from the E4M3 layout alone (code = e << 3 | m, value (1 + m/8) 2^(e - 7), subnormal
    m 2^-9): 1.0 -> 0x38, 0.125 -> 0x20, 2.5 -> 0x42, 416 -> 0x7D, 3 * 2^-9 -> 0x03;
    the midpoints 1.0625 and 1.1875 round to the even mantissa (0x38, 0x3A).  Inside a
    block the values y / (dec(s_b) g) are chosen on the E2M1 grid and on its ties."""
    g = 0.5
    sigmas = [1.0, 0.125, 2.5, 416.0, 3 * 2.0 ** -9, 1.0625, 1.1875]
    want_sc = [0x38, 0x20, 0x42, 0x7D, 0x03, 0x38, 0x3A]
    # in units of dec(s_b) * g; the first entry (6 sigma / dec(s_b)) is the block maximum
    body = [-4.0, 3.0, 1.5, 0.5, 0.25, -0.75, 5.0, 2.5, -1.25, 0.0, 1.0, -2.0, 0.1, 3.5, 4.0]
    body_codes = [0b1110, 0b0101, 0b0011, 0b0001, 0b0000, 0b1010, 0b0110, 0b0100, 0b1010,
                  0b0000, 0b0010, 0b1100, 0b0000, 0b0110, 0b0110]
    dec = {0x38: 1.0, 0x20: 0.125, 0x42: 2.5, 0x7D: 416.0, 0x03: 3 * 2.0 ** -9, 0x3A: 1.25}
    y = np.zeros((1, 16 * len(sigmas)))
    want_codes = np.zeros(y.shape, dtype=np.int64)
    for b, (sig, sc) in enumerate(zip(sigmas, want_sc)):
        unit = dec[sc] * g
        y[0, 16 * b] = 6.0 * g * sig                 # block maximum b = 6 g sigma
        y[0, 16 * b + 1:16 * b + 16] = np.array(body) * unit
        v0 = 6.0 * sig / dec[sc]                     # the maximum in scale units
        want_codes[0, 16 * b] = int(O.e2m1_encode(np.array([v0]))[0])
        want_codes[0, 16 * b + 1:16 * b + 16] = body_codes
    # the maximum itself: 6 on exact blocks; 6.375 -> 6 and 5.7 -> 6 on the tie blocks
    _check(list(want_codes[0, ::16]) == [7] * 7, "block maxima land on E2M1 6")
    codes, sc, gg, _ = O.quantize_nvfp4(y, tensor_scale=g)
    _check(gg == np.float32(g), "given tensor scale is used as is")
    _check(list(sc[0]) == want_sc, f"NVFP4 block scales b/(6g): {[hex(int(c)) for c in sc[0]]}")
    _check(np.array_equal(codes, want_codes), "NVFP4 block codes")
    # dynamic g of the same tensor: g = fl32(A / 2688) with A = 6 * 0.5 * 416 = 1248
    codes_d, sc_d, g_d, _ = O.quantize_nvfp4(y)
    _check(g_d == np.float32(1248.0 / 2688.0), "dynamic g")
    _check(sc_d[0, 3] == 0x7E, "the tensor-maximum block takes E4M3 448")


def pin_int4_clamp_saturated_scale(O):
    """INT4 codes clamp to [-8, 7] (the tiny workload's definition: round half to even, clamp
    [-8, 7]).  Under absmax the clamp only acts when the stored scale is smaller than amax / 7:
    an fp16 scale saturates at 65504, so a group with amax 9 * 65504 is quantised in units of
    65504 and its values -9, -7.5, 9, 7.5, 3.5 (units) give -8, -8, 7, 7, 4."""
    u = 65504.0
    y = np.zeros((2, 32))
    y[0, :6] = np.array([-9.0, -7.5, 9.0, 7.5, 3.5, -6.5]) * u
    y[1, :4] = np.array([1.0, -7.0, 2.5, -0.5])    # an ordinary group next to it
    q, s, _ = O.quantize_int4(y, 16, "f16")
    _check(s[0, 0] == np.float16(65504) and s[0, 1] == 0, "saturated fp16 scale")
    _check(list(q[0, :6]) == [-8, -8, 7, 7, 4, -6] and not np.any(q[0, 6:]), f"clamped codes {q[0, :6]}")
    _check(float(s[1, 0]) == float(np.float16(1.0)), "scale 7/7 in the ordinary group")
    _check(list(q[1, :4]) == [1, -7, 2, 0], "ordinary group codes")
    # fp32 storage never saturates here: the same row gives +-7 at the maximum
    q32, s32, _ = O.quantize_int4(y[:1], 16, "f32")
    _check(list(q32[0, :3]) == [-7, -6, 7], "fp32 scale: the maximum maps to +-7")


ALL_PINS = [
    pin_sylvester_matches_scipy, pin_orthogonality, pin_h172_williamson, pin_fwht_equals_dense,
    pin_rotate_matches_scipy_definition, pin_parseval_and_roundtrip, pin_e3_closed_form,
    pin_e1_worked_example, pin_e2_worked_example, pin_int4_rounding, pin_fp16_storage,
    pin_e2m1, pin_e4m3, pin_nvfp4_invariants, pin_mxfp4_closed_form, pin_mxfp4_worked_block,
    pin_mxfp4_invariants, pin_blocked_rotation, pin_nvfp4_block_scale_closed_form,
    pin_int4_clamp_saturated_scale,
]
