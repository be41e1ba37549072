"""CPU: plant plausible mistakes in copies of the oracle and require that a pin fails.

This guards the pins themselves: an oracle that dropped the normalisation, applied
the signs after H, transposed H12, used round-half-away, swapped nibbles, or got a
format constant wrong must not pass tests/oracle_pins.py.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

from tests import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "rht_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("rht_oracle_mut", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _no_norm(O):
    orig = O.rotate
    O.rotate = lambda x, signs=None: orig(x, signs) * math.sqrt(np.shape(x)[-1])


def _signs_after(O):
    orig_rot = O.rotate

    def rot(x, signs=None):
        y = orig_rot(x, None)
        return y if signs is None else y * np.asarray(signs, dtype=np.float64)
    O.rotate = rot


def _h12_transposed_in_rotate(O):
    """rotate() applies H12^T while the dense definition keeps H12.  (Transposing the
    table everywhere is a different but equally valid convention, not a mistake.)"""
    def rot(x, signs=None):
        x = O._as_f64(x)
        n = x.shape[-1]
        u = x * O._signs(signs, n)
        f, m = O.split_width(n)
        if f == 1:
            return O.fwht(u) / np.sqrt(n)
        u = O.fwht(u.reshape(*u.shape[:-1], f, m))
        return np.einsum("ba,...bj->...aj", O.factor_matrix(f).astype(np.float64), u).reshape(x.shape) / np.sqrt(n)
    O.rotate = rot


def _h172_transposed_in_rotate(O):
    """rotate() applies H172^T for 172 * 2^k widths only; H12 stays right."""
    orig = O.rotate

    def rot(x, signs=None):
        x = O._as_f64(x)
        n = x.shape[-1]
        f, m = O.split_width(n)
        if f != 172:
            return orig(x, signs)
        u = O.fwht((x * O._signs(signs, n)).reshape(*x.shape[:-1], f, m))
        return np.einsum("ba,...bj->...aj", O.h172().astype(np.float64), u).reshape(x.shape) / np.sqrt(n)
    O.rotate = rot


def _h172_coset_sign(O):
    """one coset sign of one order-43 circulant flipped"""
    w = [list(r) for r in O.WILLIAMSON43]
    w[2][3] *= -1
    O.WILLIAMSON43 = tuple(tuple(r) for r in w)


def _h172_array_sign(O):
    """the Williamson array with one block sign wrong (-D and D swapped in block row 1)"""
    def bad():
        A, B, C, D = (O._circulant(r) for r in O.williamson43_rows())
        return np.block([[A, B, C, D], [-B, A, D, -C], [-C, D, A, -B], [-D, -C, B, A]])
    O.h172 = bad


def _h12_typo(O):
    orig = O.h12

    def bad():
        h = orig().copy()
        h[4, 7] *= -1
        return h
    O.h12 = bad


def _round_half_away(O):
    class NP:
        def __getattr__(self, k):
            return getattr(np, k)
    fake = NP()
    fake.rint = lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)
    O.np = fake


def _swap_nibbles(O):
    orig = O.pack_nibbles
    O.pack_nibbles = lambda q: ((orig(q) >> 4) | (orig(q) << 4)).astype(np.uint8)


def _scale_over_8(O):
    orig = O.int4_scale_store
    O.int4_scale_store = lambda a, sd: orig(np.asarray(a) * 7.0 / 8.0, sd)


def _fp16_truncation(O):
    orig = O.int4_scale_store

    def trunc(a, sd):
        if sd != "f16":
            return orig(a, sd)
        s = np.asarray(a, dtype=np.float64) / 7.0
        r = s.astype(np.float16)
        return np.where(r.astype(np.float64) > s, np.nextafter(r, np.float16(0)), r).astype(np.float16)
    O.int4_scale_store = trunc


def _nvfp4_wrong_constant(O):
    O.nvfp4_tensor_scale = lambda y: np.float32(np.max(np.abs(np.asarray(y))) / (6.0 * 256.0))


def _e2m1_ties_up(O):
    orig = O.e2m1_encode
    O.e2m1_encode = lambda v: orig(np.asarray(v, dtype=np.float64) * (1 + 1e-12))


def _e4m3_truncate(O):
    vals = O.e4m3_values()

    def enc(x):
        x = np.asarray(x, dtype=np.float64)
        return np.clip(np.searchsorted(vals, x, side="right") - 1, 0, 126).astype(np.uint8)
    O.e4m3_encode = enc


def _fwht_skip_stage(O):
    orig = O.fwht

    def bad(v):
        v = np.asarray(v, dtype=np.float64)
        n = v.shape[-1]
        if n < 4:
            return orig(v)
        w = v.reshape(*v.shape[:-1], n // 2, 2).copy()
        # drop the first butterfly stage: run H over the other bits only
        out = orig(w.swapaxes(-1, -2)).swapaxes(-1, -2)
        return out.reshape(v.shape) if False else np.concatenate([out[..., 0], out[..., 1]], -1)
    O.fwht = bad


def _inverse_without_transpose(O):
    def inv(y, signs=None):
        y = np.asarray(y, dtype=np.float64)
        n = y.shape[-1]
        f, m = O.split_width(n)
        v = y.reshape(*y.shape[:-1], f, m)
        v = np.einsum("ab,...bj->...aj", O.h12().astype(np.float64), v) if f == 12 else v
        u = O.fwht(v).reshape(y.shape)
        return u * O._signs(signs, n) / np.sqrt(n)
    O.inverse_rotate = inv


def _mxfp4_emax_one(O):
    orig = O.mxfp4_scale_exponent
    O.mxfp4_scale_exponent = lambda b: np.clip(orig(b) + 1, -127, 127)


def _mxfp4_ceil(O):
    def exp_ceil(bmax):
        bmax = np.asarray(bmax, dtype=np.float64)
        e = np.where(bmax > 0, np.ceil(np.log2(np.where(bmax > 0, bmax, 1.0))) - 2, -127)
        return np.clip(e, -127, 127).astype(np.int64)
    O.mxfp4_scale_exponent = exp_ceil


def _mxfp4_bias_128(O):
    orig_q, orig_d = O.quantize_mxfp4, O.dequantize

    def q(y):
        c, sb, v = orig_q(y)
        return c, (sb.astype(np.int64) + 1).astype(np.uint8), v
    O.quantize_mxfp4 = q


def _blocked_norm_sqrt_n(O):
    orig = O.rotate_blocked
    O.rotate_blocked = lambda x, s, b: orig(x, s, b) * math.sqrt(b) / math.sqrt(np.shape(x)[-1])


def _blocked_signs_tiled(O):
    """signs of the first block reused for every block instead of the full-length vector"""
    orig = O.rotate_blocked

    def bad(x, s, b):
        n = np.shape(x)[-1]
        st = None if s is None else np.tile(np.asarray(s)[:b], n // b)
        return orig(x, st, b)
    O.rotate_blocked = bad


def _nvfp4_block_scale_over_4(O):
    """block scale b / (4 g) instead of b / (6 g): block maxima land on E2M1 4"""
    def q(y, tensor_scale=None):
        y = np.asarray(y, dtype=np.float64)
        T, n = y.shape
        g = O.nvfp4_tensor_scale(y) if tensor_scale is None else np.float32(tensor_scale)
        if g == 0:
            return (np.zeros((T, n), np.uint8), np.zeros((T, n // 16), np.uint8), g, np.zeros((T, n)))
        bmax = np.max(np.abs(y.reshape(T, n // 16, 16)), axis=-1)
        sc = O.e4m3_encode(bmax / (4.0 * np.float64(g)))
        codes, v = O.nvfp4_codes_from_scales(y, sc, g)
        return codes, sc, g, v
    O.quantize_nvfp4 = q


def _int4_symmetric_clamp(O):
    """INT4 codes clamped to [-7, 7] instead of [-8, 7]"""
    orig = O.int4_codes

    def codes(y, stored_scale, group):
        q, v = orig(y, stored_scale, group)
        return np.maximum(q, -7).astype(np.int8), v
    O.int4_codes = codes


MUTATIONS = [_no_norm, _signs_after, _h12_transposed_in_rotate, _h12_typo, _round_half_away,
             _swap_nibbles, _scale_over_8, _fp16_truncation, _nvfp4_wrong_constant,
             _e2m1_ties_up, _e4m3_truncate, _fwht_skip_stage, _inverse_without_transpose,
             _mxfp4_emax_one, _mxfp4_ceil, _mxfp4_bias_128, _blocked_norm_sqrt_n, _blocked_signs_tiled,
             _h172_transposed_in_rotate, _h172_coset_sign, _h172_array_sign, _nvfp4_block_scale_over_4,
             _int4_symmetric_clamp]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_some_pin_catches(mutate):
    O = fresh_oracle()
    mutate(O)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(O)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            failed.append((pin.__name__, str(e)[:80]))
    assert failed, f"no pin caught mutation {mutate.__name__}"
