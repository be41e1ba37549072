"""CPU: the oracle against what the pages and the mathematics fix (see tests/oracle_pins.py)."""
import numpy as np
import pytest

import oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_statistical_sanity_gaussianises_outliers():
    """Post-RHT values of heavy-tailed rows are close to Gaussian (QuaRot reviews,
    reviewer 2 follow-up): on KV-shaped rows with 1% spikes the excess kurtosis drops
    from ~20 to ~0; on llama-shaped rows the crest factor max|y| / rms(y) falls from
    the outlier-channel level to a few units."""
    from workloads import WORKLOADS, generate

    def kurt(a):
        a = a - a.mean(axis=1, keepdims=True)
        return np.mean(a ** 4, axis=1) / np.mean(a ** 2, axis=1) ** 2 - 3.0

    w = WORKLOADS["kv_128_int4g128"].with_tokens(4096)
    x, s = generate(w)
    xr = x.float().numpy().astype(np.float64)
    y = O.rotate(xr, s)
    rms = lambda a: np.sqrt(np.mean(a ** 2, axis=1, keepdims=True))
    # each 128-wide row normalised by its own rms, then 32 rows pooled per estimate
    kx = kurt((xr / rms(xr)).reshape(-1, 4096))
    ky = kurt((y / rms(y)).reshape(-1, 4096))
    assert np.median(kx) > 10.0
    assert abs(np.median(ky)) < 0.5

    w = WORKLOADS["llama_4096_int4"].with_tokens(64)
    x, s = generate(w)
    xr = x.float().numpy().astype(np.float64)
    y = O.rotate(xr, s)
    crest = lambda a: np.max(np.abs(a), axis=1) / np.sqrt(np.mean(a ** 2, axis=1))
    assert np.median(crest(xr)) > 15.0
    assert np.max(crest(y)) < 6.0


def test_rotation_lowers_int4_g128_error_on_outlier_data():
    """Grouped INT4-g128 error drops with the rotation on outlier data (the NVFP4
    methodology thread reports 144 of 145 linears improving under INT4-g128)."""
    from workloads import WORKLOADS, generate
    w = WORKLOADS["downproj_12288_int4g128"].with_tokens(16)
    x, s = generate(w)
    xr = x.float().numpy().astype(np.float64)
    q0, s0, _ = O.quantize_int4(xr, 128, "f16")
    err_plain = np.mean((O.dequantize(O.pack_nibbles(q0), s0, "int4", 128) - xr) ** 2)
    out = O.forward(xr, s, "int4", 128, "f16")
    xhat = O.inverse(out["packed"], out["scales"], s, "int4", 128)
    err_rot = np.mean((xhat - xr) ** 2)
    assert err_rot < 0.75 * err_plain


def test_golden_tiny_fixture_is_current():
    """tests/golden/tiny_128_int4.txt (written by make_golden.py from the oracle) still
    matches the oracle: any change to the oracle's arithmetic shows up here."""
    import os
    from workloads import WORKLOADS, generate
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_128_int4.txt")
    rows = [ln.split() for ln in open(path) if not ln.startswith("#")]
    w = WORKLOADS["tiny_128_int4"]
    x, s = generate(w)
    out = O.forward(x.numpy().astype(np.float64), s, "int4", 0, "f32")
    for t, (sb, pk) in enumerate(rows):
        assert np.float32(out["scales"][t, 0]).view(np.uint32) == int(sb, 16)
        assert out["packed"][t].tobytes().hex() == pk
