"""CPU: the comparison rules of oracle/check.py on planted device results.

R3 accepts a one-step code difference only within 1e-4 of a rounding boundary, and counts such
differences against a 1e-4 share of the tensor's codes, except where the pre-rounding value lies
exactly on the boundary: both neighbours are then nearest (the QuaRot reviews page, reviewer 2's
follow-up, names nearest rounding and no tie rule), so either code is correct and none is counted.
"""
import numpy as np
import pytest

import oracle as O
from oracle import check as C


def _int4_row():
    # per-token scale: amax 7 -> s = 1 exactly, so v = y
    y = np.zeros((1, 16))
    y[0, :5] = [7.0, 1.5, 2.5000001, -3.0, -0.5]
    q, s, v = O.quantize_int4(y, 0, "f32")
    assert s[0, 0] == 1.0 and v[0, 1] == 1.5 and q[0, 1] == 2 and q[0, 4] == 0   # ties to even
    return y, q, s


def test_int4_exact_tie_either_neighbour():
    y, q, s = _int4_row()
    for plant in ((1, 1), (4, -1)):                     # 1.5 -> 1, -0.5 -> -1: the other nearest code
        qd = q.copy()
        qd[0, plant[0]] = plant[1]
        rep = C.check_int4(O.pack_nibbles(qd), s, y, 0, "f32")
        assert rep["code_mismatches"] == 0


def test_int4_near_boundary_counts_and_far_fails():
    y, q, s = _int4_row()
    qd = q.copy()
    qd[0, 2] = 2                                        # v = 2.5000001: within the band, not a tie
    with pytest.raises(C.ParityError, match="boundary mismatches exceed"):
        C.check_int4(O.pack_nibbles(qd), s, y, 0, "f32")
    assert C.check_int4(O.pack_nibbles(qd), s, y, 0, "f32", enforce_fraction=False)["code_mismatches"] == 1
    qd = q.copy()
    qd[0, 3] = -2                                       # v = -3: far from any boundary
    with pytest.raises(C.ParityError, match="R3: INT4 code"):
        C.check_int4(O.pack_nibbles(qd), s, y, 0, "f32")
    qd = q.copy()
    qd[0, 1] = 0                                        # tie, but two steps from the oracle's code
    with pytest.raises(C.ParityError):
        C.check_int4(O.pack_nibbles(qd), s, y, 0, "f32")


def test_mxfp4_exact_tie_either_neighbour():
    # block maximum 6 -> shared exponent 0 (scale 1), so v = y; 2.5 lies between E2M1 2 and 3
    y = np.zeros((1, 32))
    y[0, :3] = [6.0, 2.5, 2.50005]
    c, sb, v = O.quantize_mxfp4(y)
    assert sb[0, 0] == 127 and O.e2m1_decode(c[0, 1]) == 2.0       # ties to the even code
    cd = c.copy()
    cd[0, 1] = c[0, 1] + 1                              # 3.0: the other nearest value
    assert C.check_mxfp4(O.pack_nibbles(cd), sb, y)["code_mismatches"] == 0
    cd = c.copy()
    cd[0, 2] = c[0, 2] - 1                              # 2.50005: near the boundary, counted
    with pytest.raises(C.ParityError, match="boundary mismatches exceed"):
        C.check_mxfp4(O.pack_nibbles(cd), sb, y)
