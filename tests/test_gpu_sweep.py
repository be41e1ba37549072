"""GPU: a seeded sweep over the call space.  Each case draws a supported width (powers of two
16 .. 16384, 12 x 2^k, 172 x 2^k), an input type, a format with a valid group and scale type, a
row count, signs or none, and sometimes a block-diagonal block (a further set of cases takes fp16
input); the device's rotation and
quantisation of every row are checked against the oracle by the same rules as the other parity
tests.  The draws are fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest

import oracle as O
from oracle import check as C
from workloads import splitmix64_signs

pytestmark = pytest.mark.gpu

POW2 = [1 << k for k in range(4, 15)]
TWELVE = [12 * (1 << k) for k in range(8, 12)]
W172 = [172 * (1 << k) for k in range(4, 8)]
WIDTHS = POW2 + TWELVE + W172
N_CASES = 160
N_F16_CASES = 48


def draw_case(rng, f16=False):
    n = int(rng.choice(WIDTHS))
    dtype = "fp32" if rng.random() < 0.35 else "bf16"
    if f16:
        dtype = "fp16"
    # block-diagonal on a quarter of the power-of-two-divisible widths
    block = None
    pow2_part = n & -n
    if rng.random() < 0.25 and pow2_part >= 32:
        block = int(rng.choice([b for b in POW2 if b < n and n % b == 0 and b <= pow2_part]))
    width = block or n
    fmts = ["int4", "nvfp4"] + (["mxfp4"] if width % 32 == 0 else [])
    fmt = str(rng.choice(fmts))
    if fmt == "int4":
        groups = [0] + [g for g in POW2 if g <= width and width % g == 0]
        if block:
            groups = [g for g in groups if g != 0]   # groups must lie inside a block
        group = int(rng.choice(groups))
        scale_dtype = str(rng.choice(["f32", "f16"]))
    elif fmt == "nvfp4":
        group, scale_dtype = 16, "e4m3"
    else:
        group, scale_dtype = 32, "e8m0"
    tokens = int(max(1, min(300, (1 << 21) // n) * rng.random()) + 1)
    signed = rng.random() < 0.8
    seed = int(rng.integers(1 << 30))
    return dict(n=n, dtype=dtype, block=block, fmt=fmt, group=group, scale_dtype=scale_dtype,
                tokens=tokens, signed=signed, seed=seed)


CASES = [draw_case(np.random.default_rng(1000 + i)) for i in range(N_CASES)] + \
        [draw_case(np.random.default_rng(5000 + i), f16=True) for i in range(N_F16_CASES)]


@pytest.fixture(scope="module")
def R():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import randomized_hadamard_rotation_amd as R
    return R


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{n}-{dtype}-{fmt}-g{group}-{scale_dtype}-t{tokens}-b{block}".format(**c))
def test_sweep_case(R, case):
    import torch
    c = case
    print(f"[case] {c}", flush=True)
    g = torch.Generator().manual_seed(c["seed"])
    xc = torch.randn(c["tokens"], c["n"], generator=g) * torch.exp(torch.randn(c["n"], generator=g))
    x = xc.to({"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[c["dtype"]])
    s = splitmix64_signs(c["seed"] & 0xFFFF, c["n"]) if c["signed"] else None
    blk = c["block"]
    y_ref = O.rotate(x, s) if not blk else O.rotate_blocked(x, s, blk)
    xd = x.to("cuda")
    y = R.rhtq_rotate(xd, s, block=blk)
    torch.cuda.synchronize()
    C.check_rotation(y.cpu().numpy(), y_ref)
    packed, scales, ts = R.rhtq_forward(xd, s, fmt=c["fmt"], group=c["group"], scale_dtype=c["scale_dtype"],
                                        block=blk)
    torch.cuda.synchronize()
    p, sc = packed.cpu().numpy(), scales.cpu().numpy()
    if c["fmt"] == "int4":
        C.check_int4(p, sc, y_ref, c["group"], c["scale_dtype"])
    elif c["fmt"] == "mxfp4":
        C.check_mxfp4(p, sc, y_ref)
    else:
        C.check_nvfp4(p, sc, float(ts.item()), y_ref)
