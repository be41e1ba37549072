"""fp64 CPU oracle: randomized Hadamard transform, INT4 / NVFP4-style 4-bit
quantisation, nibble packing and the inverse.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg; never by the library's product path.

Sources (web pages on the subject; cited by title and section):

* "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (reviews page):
  - review 1, Summary: rotations that cannot be folded into weights are
    Hadamard matrices applied online with the Walsh-Hadamard fast algorithm;
    grouped quantisation is combined with the rotation.
  - review 2, Summary: the random Hadamard transform (RHT) is invertible up
    to machine precision and is followed by INT4 activation quantisation.
  - review 2, Questions: non-power-of-two widths need an extra factor;
    per-slice versus full rotation under tensor parallelism.
  - review 3, Strengths: the online Hadamard is applied to all activations
    and to the KV cache.
  - review 3, Questions: the Hadamard block computes Y = X H^T (row vectors).
  - reviewer 2 follow-up comment: activations are quantised with nearest
    rounding; post-RHT values are close to Gaussian; applying the RHT per
    batch of data is data parallelism.
* "incoh_rotate=true degrades W4 PPL on Qwen3-8B" (KronQ issue #2), Model
  Details table: hidden 4096 is a power of two, intermediate 12288 = 12 x 1024
  is Hadamard-compatible.
* "Methodology checks for NVFP4 W4A4 on Qwen3-8B" (rstation thread), the
  NVFP4 results and the block-Hadamard comment: NVFP4 = E2M1 codes with FP8
  E4M3 block scales (16-wide blocks) plus a tensor scale; INT4-g128; MXFP4 is
  compared against both after block-Hadamard rotation.
* The pages name MXFP4 but do not define it; its definition is the public OCP
  Microscaling Formats (MX) v1.0 specification: blocks of 32 elements share
  one power-of-two scale stored as E8M0, elements are E2M1.

Where the pages are silent the oracle takes these readings:
  R-norm   the transform is orthonormal: y = H_n D x / sqrt(n)
  R-order  Sylvester (natural) ordering, H[i][j] = (-1)^popcount(i & j)
  R-side   signs first, then H; for row vectors Y = X D H^T
  R-h12    the order-12 factor is the Williamson array built from A = J3 and
           B = J3 - 2 I3; for n = 12 m, H_n = H12 (x) H_m with j = j1*m + j2
  R-h172   the order-172 factor (QuaRot reviews, review 2 Questions: 172 is the
           non-power-of-two part of the Llama 2 7B width, 11008 = 172 x 64) is the Williamson array of four symmetric circulants of
           order 43 whose first rows are +1 at 0 and constant on each coset of the
           order-6 subgroup {1, 6, 7, 36, 37, 42} of the units mod 43 (cosets
           3^c * K, c = 0..6, signs in WILLIAMSON43); for n = 172 m, H_n = H172 (x) H_m
           with j = j1*m + j2, as for 12
  R-int4   symmetric absmax INT4: scale = amax / 7, stored (fp32 or fp16, RNE),
           codes = clamp(round_half_even(y / stored_scale), -8, 7); a zero
           group has scale 0 and codes 0
  R-pack   two codes per byte, even index in the low nibble, two's complement
  R-nvfp4  tensor scale g = fl32(amax(y) / (6 * 448)); per 16-block
           s_b = E4M3_RNE_sat(blockmax / (6 g)); codes = sign bit | E2M1 of
           |y| / (dec(s_b) g), ties to even; sign kept on values that round to 0
  R-e4m3   OCP FP8 E4M3FN: bias 7, max 448, subnormals, NaN never produced
  R-e2m1   OCP MX E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} <-> codes 0..7
  R-block  block-diagonal rotation ("block-Hadamard-128" in the NVFP4 methodology
           thread): one random sign vector over the whole row, then H_b on every
           contiguous b-block, normalised by 1/sqrt(b): y = (I (x) H_b) D x / sqrt(b)
  R-mxfp4  per 32-block X = 2^(floor(log2(blockmax)) - 2) (2 = exponent of the
           largest E2M1 normal, 6 = 1.5 * 2^2), exponent clamped to [-127, 127]
           and stored as the E8M0 byte exponent + 127; codes = sign bit | E2M1 of
           |y| / X (ties to even, saturating at 6); an all-zero block stores
           exponent -127 and codes 0

Parity of the H12 choice, the sign generator, the nibble order, the +-0 rule
and the NVFP4 amax source is by convention: the pages fix none of them
("parity unpinned" for those conventions; every other part is pinned by the
tests in tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sylvester", "h12", "h172", "WILLIAMSON43", "williamson43_rows", "factor_matrix", "hadamard", "split_width", "fwht", "rotate", "rotate_dense",
    "inverse_rotate", "int4_scale_store", "int4_codes", "quantize_int4", "pack_nibbles",
    "unpack_nibbles", "e4m3_values", "e4m3_encode", "e4m3_decode", "e2m1_values",
    "e2m1_encode", "e2m1_decode", "nvfp4_tensor_scale", "quantize_nvfp4",
    "nvfp4_codes_from_scales", "mxfp4_scale_exponent", "mxfp4_codes_from_scales",
    "quantize_mxfp4", "rotate_blocked", "inverse_rotate_blocked", "forward", "dequantize", "inverse",
]


# ---------------------------------------------------------------------------
# Hadamard matrices (QuaRot reviews, review 1 Summary; KronQ issue Model Details)
# ---------------------------------------------------------------------------

def sylvester(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n = 2^k: H[i][j] = (-1)^popcount(i & j)."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    i = np.arange(n, dtype=np.int64)
    a = i[:, None] & i[None, :]
    pc = np.zeros_like(a)
    while np.any(a):
        pc += a & 1
        a >>= 1
    return np.where(pc & 1, -1, 1).astype(np.int64)


def h12() -> np.ndarray:
    """Order-12 Hadamard matrix as the Williamson array

        [[ A,  B,  B,  B],
         [-B,  A, -B,  B],
         [-B,  B,  A, -B],
         [-B, -B,  B,  A]]      with A = J3 (all ones), B = J3 - 2 I3.

    A and B are symmetric circulants with A^2 + 3 B^2 = 12 I3, so the array
    satisfies H H^T = 12 I.  It is not symmetric: the inverse uses H^T.
    """
    A = np.ones((3, 3), dtype=np.int64)
    B = np.ones((3, 3), dtype=np.int64) - 2 * np.eye(3, dtype=np.int64)
    return np.block([[A, B, B, B],
                     [-B, A, -B, B],
                     [-B, B, A, -B],
                     [-B, -B, B, A]])


# Coset signs of the four order-43 circulants (A, B, C, D) of the order-172 factor:
# entry c is the sign of every k = 3^c * t mod 43, t in {1, 6, 7, 36, 37, 42}.
WILLIAMSON43 = (
    (+1, +1, +1, +1, -1, -1, -1),
    (-1, +1, +1, -1, -1, +1, -1),
    (-1, +1, -1, +1, +1, +1, -1),
    (-1, -1, +1, +1, -1, +1, +1),
)


def _circulant(first_row) -> np.ndarray:
    r = np.asarray(first_row, dtype=np.int64)
    p = r.size
    idx = (np.arange(p)[None, :] - np.arange(p)[:, None]) % p   # C[i][j] = r[(j - i) mod p]
    return r[idx]


def williamson43_rows() -> list:
    """First rows of the circulants A, B, C, D of order 43: +1 at index 0, and at every
    k = 3^c * t (mod 43), t in the order-6 subgroup, the sign WILLIAMSON43[.][c]."""
    p = 43
    sub = [1, 6, 7, 36, 37, 42]
    rows = []
    for signs in WILLIAMSON43:
        r = np.zeros(p, dtype=np.int64)
        r[0] = 1
        for c, sg in enumerate(signs):
            for t in sub:
                r[(pow(3, c, p) * t) % p] = sg
        rows.append(r)
    return rows


def h172() -> np.ndarray:
    """Order-172 Hadamard matrix as the Williamson array

        [[ A,  B,  C,  D],
         [-B,  A, -D,  C],
         [-C,  D,  A, -B],
         [-D, -C,  B,  A]]

    of the symmetric circulants of williamson43_rows(), which commute and satisfy
    A^2 + B^2 + C^2 + D^2 = 172 I43, so H H^T = 172 I.  Not symmetric: the inverse uses H^T."""
    A, B, C, D = (_circulant(r) for r in williamson43_rows())
    return np.block([[A, B, C, D],
                     [-B, A, -D, C],
                     [-C, D, A, -B],
                     [-D, -C, B, A]])


def factor_matrix(f: int) -> np.ndarray:
    """The non-power-of-two Kronecker factor of order f (12 or 172)."""
    if f == 12:
        return h12()
    if f == 172:
        return h172()
    raise ValueError(f"no factor of order {f}")


def split_width(n: int):
    """Return (f, m) with n = f * m, f in {1, 12, 172}, m a power of two."""
    if n >= 1 and n & (n - 1) == 0:
        return 1, n
    for f in (12, 172):
        if n % f == 0:
            m = n // f
            if m & (m - 1) == 0:
                return f, m
    raise ValueError(f"width {n} is none of 2^k, 12 * 2^k, 172 * 2^k")


def hadamard(n: int) -> np.ndarray:
    """Dense H_n: Sylvester for 2^k, H_f (x) H_m (Kronecker, the order-f factor outer) for
    f * 2^k, f = 12 or 172."""
    f, m = split_width(n)
    return sylvester(m) if f == 1 else np.kron(factor_matrix(f), sylvester(m))


# ---------------------------------------------------------------------------
# Rotation (QuaRot reviews: review 1 Summary, review 2 Summary, review 3 Questions)
# ---------------------------------------------------------------------------

def fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis
    (Sylvester order): for every index bit h, (a, b) -> (a + b, a - b)."""
    v = np.array(v, dtype=np.float64, copy=True)
    n = v.shape[-1]
    if n & (n - 1):
        raise ValueError("fwht needs a power-of-two length")
    lead = v.shape[:-1]
    h = 1
    while h < n:
        w = v.reshape(*lead, n // (2 * h), 2, h)
        a = w[..., 0, :].copy()
        b = w[..., 1, :]
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        h *= 2
    return v


def _as_f64(x) -> np.ndarray:
    """Read bf16 / fp16 / fp32 / fp64 input exactly into fp64 (bf16 and fp16 arrive as
    torch tensors; bf16 also as uint16 bit patterns)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _signs(signs, n):
    if signs is None:
        return np.ones(n, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (n,) or not np.all(np.abs(s) == 1):
        raise ValueError("signs must be a +-1 vector of length n")
    return s


def rotate(x, signs=None) -> np.ndarray:
    """y = H_n (s * x) / sqrt(n) for every row of x [T][n] (row form Y = X D H^T / sqrt(n)).

    Power-of-two widths use the fast Walsh-Hadamard transform; n = f m (f = 12, 172)
    applies H_m along the contiguous index j2 and H_f across j1 (j = j1 * m + j2).
    """
    x = _as_f64(x)
    n = x.shape[-1]
    u = x * _signs(signs, n)
    f, m = split_width(n)
    if f == 1:
        y = fwht(u)
    else:
        u = u.reshape(*u.shape[:-1], f, m)
        u = fwht(u)
        y = np.einsum("ab,...bj->...aj", factor_matrix(f).astype(np.float64), u).reshape(x.shape)
    return y / np.sqrt(n)


def rotate_blocked(x, signs, block: int) -> np.ndarray:
    """Block-diagonal rotation: y = (I_{n/b} (x) H_b) D x / sqrt(b) per row, with the signs s of
    length n applied before the blocks are transformed (NVFP4 methodology thread, the
    block-Hadamard-128 comment).  block = n is rotate()."""
    x = _as_f64(x)
    n = x.shape[-1]
    if block < 1 or block & (block - 1) or n % block:
        raise ValueError("block must be a power of two dividing n")
    u = (x * _signs(signs, n)).reshape(*x.shape[:-1], n // block, block)
    return (fwht(u) / np.sqrt(block)).reshape(x.shape)


def inverse_rotate_blocked(y, signs, block: int) -> np.ndarray:
    """x = D (I (x) H_b^T) y / sqrt(b): the exact inverse of rotate_blocked()."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    u = fwht(y.reshape(*y.shape[:-1], n // block, block)).reshape(y.shape)
    return u * _signs(signs, n) / np.sqrt(block)


def rotate_dense(x, signs=None) -> np.ndarray:
    """Same as rotate() by the definition Y = X D H^T / sqrt(n) with a dense matrix
    (small n only)."""
    x = _as_f64(x)
    n = x.shape[-1]
    H = hadamard(n).astype(np.float64)
    return (x * _signs(signs, n)) @ H.T / np.sqrt(n)


def inverse_rotate(y, signs=None) -> np.ndarray:
    """x = D H_n^T y / sqrt(n) per row: the exact inverse of rotate()."""
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    f, m = split_width(n)
    if f == 1:
        u = fwht(y)            # Sylvester H is symmetric
    else:
        v = y.reshape(*y.shape[:-1], f, m)
        v = np.einsum("ba,...bj->...aj", factor_matrix(f).astype(np.float64), v)   # H_f^T
        u = fwht(v).reshape(y.shape)
    return u * _signs(signs, n) / np.sqrt(n)


# ---------------------------------------------------------------------------
# INT4 (QuaRot reviews, review 2 Summary and reviewer 2 follow-up: INT4, nearest
# rounding; review 1 Summary and the NVFP4 thread: grouped INT4-g128)
# ---------------------------------------------------------------------------

def _group_view(y: np.ndarray, group: int) -> np.ndarray:
    T, n = y.shape
    g = n if group == 0 else group
    if n % g:
        raise ValueError("group must divide n")
    return y.reshape(T, n // g, g)


def int4_scale_store(amax: np.ndarray, scale_dtype: str) -> np.ndarray:
    """Stored INT4 scale: amax / 7 computed in fp64, then rounded to the storage
    type with round-to-nearest-even (fp16 saturates at its largest finite value)."""
    s = np.asarray(amax, dtype=np.float64) / 7.0
    if scale_dtype == "f32":
        return s.astype(np.float32)
    if scale_dtype == "f16":
        return np.minimum(s, 65504.0).astype(np.float16)
    raise ValueError(scale_dtype)


def int4_codes(y, stored_scale, group: int):
    """Codes for given stored scales: q = clamp(RNE(y / s), -8, 7); s == 0 -> 0.
    Returns (q int8 [T][n], v fp64 [T][n] = the pre-rounding value y / s)."""
    y = np.asarray(y, dtype=np.float64)
    yg = _group_view(y, group)
    s = np.asarray(stored_scale, dtype=np.float64).reshape(yg.shape[0], yg.shape[1], 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, yg / np.where(s > 0, s, 1.0), 0.0)
    q = np.clip(np.rint(v), -8, 7).astype(np.int8)
    return q.reshape(y.shape), v.reshape(y.shape)


def quantize_int4(y, group: int, scale_dtype: str):
    """Symmetric absmax INT4 per token (group 0) or per contiguous group.
    Returns (codes int8 [T][n], stored scales [T][groups], pre-rounding v)."""
    y = np.asarray(y, dtype=np.float64)
    amax = np.max(np.abs(_group_view(y, group)), axis=-1)
    s = int4_scale_store(amax, scale_dtype)
    q, v = int4_codes(y, s, group)
    return q, s, v


def pack_nibbles(q) -> np.ndarray:
    """Two 4-bit codes per byte, element 2k in the low nibble, 2k+1 in the high."""
    q = np.asarray(q).astype(np.int64)
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, signed: bool = True) -> np.ndarray:
    p = np.asarray(packed).astype(np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


# ---------------------------------------------------------------------------
# E4M3 and E2M1 (NVFP4 thread: NVFP4 with E4M3 block scales, 16-wide blocks).
# Grids from the OCP FP8 and OCP Microscaling format definitions.
# ---------------------------------------------------------------------------

def e4m3_values() -> np.ndarray:
    """Decoded value of every non-negative finite E4M3FN code 0x00..0x7E."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def _nearest_even(grid: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each a >= 0 (grid ascending, index parity =
    mantissa parity); exact ties go to the even index; beyond the top -> top."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= grid[-1], len(grid) - 1, idx)
    idx = np.where(a <= 0, 0, idx)
    return idx


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN code of non-negative x: nearest value, ties to even mantissa, saturate
    at 448 (code 0x7E); NaN is never produced."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0):
        raise ValueError("block scales are non-negative")
    return _nearest_even(e4m3_values(), x).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    mag = e4m3_values()[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e2m1_values() -> np.ndarray:
    return np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_encode(v) -> np.ndarray:
    """4-bit E2M1 code: bit 3 = sign of v (kept when the magnitude rounds to 0),
    bits 0-2 = nearest magnitude with ties to even, saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even(e2m1_values(), np.abs(v)).astype(np.uint8)
    return (np.where(np.signbit(v), 8, 0).astype(np.uint8) | mag).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64)
    mag = e2m1_values()[c & 7]
    return np.where(c & 8, -mag, mag)


# ---------------------------------------------------------------------------
# NVFP4-style quantisation
# ---------------------------------------------------------------------------

def nvfp4_tensor_scale(y) -> np.float32:
    """g = fl32(amax(|y|) / (6 * 448)) over the whole (rotated) tensor."""
    return np.float32(np.max(np.abs(np.asarray(y, dtype=np.float64))) / (6.0 * 448.0))


def nvfp4_codes_from_scales(y, scale_codes, g):
    """E2M1 codes for given E4M3 block-scale codes and tensor scale g.
    Returns (codes uint8 [T][n], v fp64 = y / (dec(s_b) g))."""
    y = np.asarray(y, dtype=np.float64)
    T, n = y.shape
    yb = y.reshape(T, n // 16, 16)
    seff = (e4m3_decode(scale_codes) * np.float64(np.float32(g))).reshape(T, n // 16, 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(seff > 0, yb / np.where(seff > 0, seff, 1.0), 0.0)
    codes = e2m1_encode(v)
    codes = np.where(seff > 0, codes, 0).astype(np.uint8)   # zero block -> 0b0000
    return codes.reshape(T, n), v.reshape(T, n)


def quantize_nvfp4(y, tensor_scale=None):
    """Returns (codes uint8 [T][n], scale codes uint8 [T][n/16], g float32, v).
    tensor_scale None -> computed from y (dynamic); otherwise the given g is used."""
    y = np.asarray(y, dtype=np.float64)
    T, n = y.shape
    g = nvfp4_tensor_scale(y) if tensor_scale is None else np.float32(tensor_scale)
    if g == 0:
        return (np.zeros((T, n), np.uint8), np.zeros((T, n // 16), np.uint8), g,
                np.zeros((T, n)))
    bmax = np.max(np.abs(y.reshape(T, n // 16, 16)), axis=-1)
    sigma = bmax / (6.0 * np.float64(g))
    sc = e4m3_encode(sigma)
    codes, v = nvfp4_codes_from_scales(y, sc, g)
    return codes, sc, g, v


def mxfp4_scale_exponent(bmax) -> np.ndarray:
    """Shared exponent of MX blocks with maxima bmax (OCP MX v1.0, shared scale):
    floor(log2(bmax)) - 2, clamped to [-127, 127]; -127 for an all-zero block.
    floor(log2) is read off frexp, which is exact for every positive double."""
    bmax = np.asarray(bmax, dtype=np.float64)
    _, ex = np.frexp(np.where(bmax > 0, bmax, 1.0))   # bmax = m * 2^ex, 0.5 <= m < 1
    e = np.where(bmax > 0, ex - 1 - 2, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp4_codes_from_scales(y, scale_bytes):
    """E2M1 codes of 32-blocks for given E8M0 scale bytes (exponent + 127).
    Returns (codes uint8 [T][n], v fp64 = y / X).  Blocks whose maximum is zero store
    code 0 (their values are all zero)."""
    y = np.asarray(y, dtype=np.float64)
    T, n = y.shape
    yb = y.reshape(T, n // 32, 32)
    X = np.ldexp(1.0, np.asarray(scale_bytes, dtype=np.int64) - 127).reshape(T, n // 32, 1)
    v = yb / X
    codes = e2m1_encode(v)
    zero = np.max(np.abs(yb), axis=-1, keepdims=True) == 0
    codes = np.where(zero, 0, codes).astype(np.uint8)
    return codes.reshape(T, n), v.reshape(T, n)


def quantize_mxfp4(y):
    """Returns (codes uint8 [T][n], scale bytes uint8 [T][n/32], v)."""
    y = np.asarray(y, dtype=np.float64)
    T, n = y.shape
    bmax = np.max(np.abs(y.reshape(T, n // 32, 32)), axis=-1)
    sb = (mxfp4_scale_exponent(bmax) + 127).astype(np.uint8)
    codes, v = mxfp4_codes_from_scales(y, sb)
    return codes, sb, v


# ---------------------------------------------------------------------------
# Whole forward / inverse
# ---------------------------------------------------------------------------

def forward(x, signs, fmt: str, group: int = 0, scale_dtype: str = "f32", tensor_scale=None,
            block: int | None = None):
    """Rotate (block-diagonally when block < n) then quantise then pack.  Returns a dict with
    y (fp64), codes, packed bytes, scales, tensor_scale (NVFP4) and the pre-rounding values v."""
    n = np.shape(x)[-1]
    y = rotate(x, signs) if block is None or block == n else rotate_blocked(x, signs, block)
    if fmt == "int4":
        q, s, v = quantize_int4(y, group, scale_dtype)
        return {"y": y, "codes": q, "packed": pack_nibbles(q), "scales": s,
                "tensor_scale": None, "v": v}
    if fmt == "nvfp4":
        if group != 16:
            raise ValueError("NVFP4 uses 16-wide blocks")
        c, sc, g, v = quantize_nvfp4(y, tensor_scale)
        return {"y": y, "codes": c, "packed": pack_nibbles(c), "scales": sc,
                "tensor_scale": g, "v": v}
    if fmt == "mxfp4":
        if group != 32:
            raise ValueError("MXFP4 uses 32-wide blocks")
        c, sb, v = quantize_mxfp4(y)
        return {"y": y, "codes": c, "packed": pack_nibbles(c), "scales": sb,
                "tensor_scale": None, "v": v}
    raise ValueError(fmt)


def dequantize(packed, scales, fmt: str, group: int = 0, tensor_scale=None) -> np.ndarray:
    """y_hat from packed codes: INT4 q * s; NVFP4 e2m1(code) * dec(s_b) * g;
    MXFP4 e2m1(code) * 2^(scale byte - 127)."""
    if fmt == "int4":
        q = unpack_nibbles(packed, signed=True).astype(np.float64)
        T, n = q.shape
        s = np.asarray(scales, dtype=np.float64).reshape(T, -1, 1)
        return (_group_view(q, group) * s).reshape(T, n)
    c = unpack_nibbles(packed, signed=False)
    if fmt == "mxfp4":
        T, n = c.shape
        X = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127).reshape(T, n // 32, 1)
        return (e2m1_decode(c).reshape(T, n // 32, 32) * X).reshape(T, n)
    T, n = c.shape
    seff = (e4m3_decode(scales) * np.float64(np.float32(tensor_scale))).reshape(T, n // 16, 1)
    return (e2m1_decode(c).reshape(T, n // 16, 16) * seff).reshape(T, n)


def inverse(packed, scales, signs, fmt: str, group: int = 0, tensor_scale=None,
            block: int | None = None) -> np.ndarray:
    """x_hat = D H^T y_hat / sqrt(n) (blockwise when block < n): dequantise, undo the rotation."""
    yh = dequantize(packed, scales, fmt, group, tensor_scale)
    if block is None or block == yh.shape[-1]:
        return inverse_rotate(yh, signs)
    return inverse_rotate_blocked(yh, signs, block)
