"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Each case prints what it runs before touching the GPU, so a failing run names it.
"""
import math
import os
import sys

import numpy as np
import pytest

import oracle as O
from oracle import check as C
from tests import oracle_pins as P
from workloads import WORKLOADS, generate, special_rows, splitmix64_signs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_128_int4.txt")


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


def dev():
    import torch
    return torch.device("cuda:0")


def to_np(t):
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy()
    return t.numpy()


def run_forward(R, x, s, fmt, group, scale_dtype, **kw):
    import torch
    if kw.get("block") in (0, None):
        kw.pop("block", None)
    packed, scales, ts = R.rhtq_forward(x, s, fmt=fmt, group=group, scale_dtype=scale_dtype, **kw)
    torch.cuda.synchronize()
    return to_np(packed), to_np(scales), (None if ts is None else float(ts.item()))


def ref_rotate(x, s, block=0):
    return O.rotate(x, s) if not block else O.rotate_blocked(x, s, block)


def check_forward(R, x, s, fmt, group, scale_dtype, rows=None, y_ref=None, g_ref=None, block=0):
    """Device forward of all rows of x; oracle on `rows` (all by default)."""
    packed, scales, g = run_forward(R, x, s, fmt, group, scale_dtype, block=block)
    if rows is None:
        rows = np.arange(x.shape[0])
    if y_ref is None:
        y_ref = ref_rotate(x[rows].cpu(), s, block)
    if fmt == "int4":
        return C.check_int4(packed[rows], scales[rows], y_ref, group, scale_dtype)
    if fmt == "mxfp4":
        return C.check_mxfp4(packed[rows], scales[rows], y_ref)
    return C.check_nvfp4(packed[rows], scales[rows], g, y_ref, g_ref)


def x_to(w, tokens=None):
    w = w if tokens is None else w.with_tokens(tokens)
    x, s = generate(w, "cpu")
    return x.to(dev()), s


# ----------------------------------------------------------------------------
# worked examples and closed forms
# ----------------------------------------------------------------------------

def test_tiny_fp32_matches_golden_fixture(R):
    say("tiny_128_int4 vs tests/golden/tiny_128_int4.txt")
    w = WORKLOADS["tiny_128_int4"]
    x, s = x_to(w)
    packed, scales, _ = run_forward(R, x, s, "int4", 0, "f32")
    rows = [ln.split() for ln in open(GOLDEN) if not ln.startswith("#")]
    gold_s = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(np.float32)
    gold_p = np.array([list(bytes.fromhex(r[1])) for r in rows], dtype=np.uint8)
    y_ref = O.rotate(x.cpu(), s)
    rep = C.check_int4(packed, scales, y_ref, 0, "f32")
    assert np.abs(scales[:, 0] - gold_s).max() <= 1e-6 * np.abs(gold_s).max()
    mism = int(np.sum(packed != gold_p))
    assert mism <= rep["code_mismatches"], (mism, rep)


def test_e2_exact_example(R):
    say("E2 n=4096 exact")
    import torch
    xe, s = P.e2_input(4096)
    x = torch.tensor(xe, dtype=torch.bfloat16, device=dev())
    assert np.array_equal(to_np(x), xe)          # bf16-exact input
    y = to_np(R.rhtq_rotate(x, s))
    want = np.zeros((1, 4096), np.float32)
    want[0, :4] = [7.0, 2.5, -1.5, 0.5]
    assert np.array_equal(y, want)
    packed, scales, _ = run_forward(R, x, s, "int4", 0, "f32")
    assert scales[0, 0] == 1.0
    assert packed[0, 0] == 0x27 and packed[0, 1] == 0x0E and not packed[0, 2:].any()


@pytest.mark.parametrize("n,k", [(16, 3), (128, 77), (4096, 1234), (12288, 7000), (3072, 2049),
                                 (16384, 9999), (24576, 123), (11008, 9000), (5504, 4321), (2752, 43),
                                 (22016, 21999)])
def test_e3_closed_form(R, n, k):
    say(f"E3 n={n} k={k}")
    import torch
    s = splitmix64_signs(5, n)
    xe = P._signed_row(O, n, k, s)[None, :]
    x = torch.tensor(np.repeat(xe, 3, axis=0), dtype=torch.bfloat16, device=dev())
    y = to_np(R.rhtq_rotate(x, s))
    e = np.zeros(n); e[k] = math.sqrt(n)
    assert np.max(np.abs(y - e)) <= 1e-5 * math.sqrt(n)
    packed, scales, _ = run_forward(R, x, s, "int4", 0, "f32")
    q = O.unpack_nibbles(packed)
    assert np.all(q[:, k] == 7) and np.count_nonzero(q) == 3
    assert np.all(scales[:, 0] == np.float32(math.sqrt(n) / 7.0)) or \
        np.allclose(scales[:, 0], math.sqrt(n) / 7.0, rtol=1e-6)
    if n % 128 == 0:
        packed, scales, _ = run_forward(R, x, s, "int4", 128, "f16")
        assert np.count_nonzero(scales) == 3
        assert np.all(scales[:, k // 128] == np.float16(math.sqrt(n) / 7.0))
    packed, scales, g = run_forward(R, x, s, "nvfp4", 16, "e4m3")
    c = O.unpack_nibbles(packed, signed=False)
    assert np.all(scales[:, k // 16] == 0x7E) and np.count_nonzero(scales) == 3
    assert np.all(c[:, k] == 0b0111)
    assert np.count_nonzero(c & 7) == 3
    if n % 32 == 0:
        # MXFP4: the block of k has exponent floor(log2(sqrt(n))) - 2, the rest exponent -127
        packed, scales, _ = run_forward(R, x, s, "mxfp4", 32, "e8m0")
        c = O.unpack_nibbles(packed, signed=False)
        ref = O.forward(xe, s, "mxfp4", 32)
        assert np.all(scales == ref["scales"]) and np.all(c == ref["codes"])


# ----------------------------------------------------------------------------
# the five workloads: reduced row counts (whole oracle) and full size (sampled rows)
# ----------------------------------------------------------------------------

REDUCED = [("tiny_128_int4", 64), ("llama_4096_int4", 203), ("downproj_12288_int4g128", 37),
           ("kv_128_int4g128", 4099), ("nvfp4_4096", 131), ("mxfp4_4096", 131),
           ("blockh128_4096_int4g128", 131), ("downproj7b_11008_int4g128", 37), ("wide172_22016_int4g128", 37)]


@pytest.mark.parametrize("name,tokens", REDUCED)
def test_workload_reduced(R, name, tokens):
    w = WORKLOADS[name]
    say(f"{name} reduced to {tokens} rows")
    x, s = x_to(w, tokens)
    rep = check_forward(R, x, s, w.fmt, w.group, w.scale_dtype, block=w.block)
    print(rep)


@pytest.mark.parametrize("name", ["llama_4096_int4", "downproj_12288_int4g128", "kv_128_int4g128",
                                  "nvfp4_4096", "mxfp4_4096", "blockh128_4096_int4g128",
                                  "downproj7b_11008_int4g128", "wide172_22016_int4g128"])
def test_workload_full_size_sampled(R, name):
    """Full-size input on the device in the same launch shape as the benchmark;
    the oracle checks sampled rows (first, last, every sink row it can find, random)."""
    import torch
    w = WORKLOADS[name]
    say(f"{name} full size {w.tokens} x {w.n}")
    x, s = generate(w, dev())
    T = w.tokens
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, T - 2, T - 1], rng.choice(T, 60, replace=False)]))
    xr = x.float().abs().amax(dim=1)
    big = torch.topk(xr, 4).indices.cpu().numpy()
    rows = np.unique(np.concatenate([rows, big]))
    g_ref = None
    if w.fmt == "nvfp4":
        # the tensor scale needs the amax over every row: oracle in chunks
        amax = 0.0
        for r0 in range(0, T, 2048):
            amax = max(amax, float(np.max(np.abs(O.rotate(x[r0:r0 + 2048].cpu(), s)))))
        g_ref = np.float32(amax / 2688.0)
    rep = check_forward(R, x, s, w.fmt, w.group, w.scale_dtype, rows=rows, g_ref=g_ref, block=w.block)
    print(rep)
    # properties over the whole output: INT4 codes never -8
    if w.fmt == "int4":
        packed, _, _ = R.rhtq_forward(x, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype,
                                      block=w.block or None)
        lo = (packed & 0xF)
        hi = (packed >> 4)
        assert not bool(((lo == 8) | (hi == 8)).any())


# Inputs of more than 2^31 elements: every element, code and scale index is 64-bit.  Row counts
# put element 2^31 inside the tensor; the oracle checks the rows around it, the first and the last
# (only those rows are copied to the host).
BEYOND_INT32 = [("llama_4096_int4", 2 ** 19 + 5), ("mxfp4_4096", 2 ** 19 + 3), ("kv_128_int4g128", 2 ** 24 + 3),
                ("downproj_12288_int4g128", 174763), ("downproj7b_11008_int4g128", 195085),
                ("downproj_12288_int4g128:n=24576", 87385), ("downproj7b_11008_int4g128:n=5504", 390170),
                ("wide172_22016_int4g128", 97548)]


@pytest.mark.parametrize("name,tokens", BEYOND_INT32)
def test_beyond_int32_elements(R, name, tokens):
    import dataclasses
    import torch
    base, _, n = name.partition(":n=")
    w = WORKLOADS[base].with_tokens(tokens)
    if n:
        w = dataclasses.replace(w, n=int(n))
    assert tokens * w.n > 2 ** 31
    say(f"{name} at {tokens} x {w.n} = {tokens * w.n} elements")
    x, s = generate(w, dev())
    rb = 2 ** 31 // w.n   # the row holding element 2^31
    rows = np.unique(np.array([0, rb - 1, rb, rb + 1, tokens - 1]))
    rows = rows[rows < tokens]
    rows_t = torch.from_numpy(rows).to(dev())
    packed, scales, _ = R.rhtq_forward(x, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
    torch.cuda.synchronize()
    y_ref = O.rotate(x[rows_t].cpu(), s)
    p_rows, s_rows = to_np(packed[rows_t]), to_np(scales[rows_t])
    if w.fmt == "int4":
        print(C.check_int4(p_rows, s_rows, y_ref, w.group, w.scale_dtype))
    else:
        print(C.check_mxfp4(p_rows, s_rows, y_ref))
    del x
    if name.startswith("kv_"):
        # the KV read path over the same > 2^31-element tensor
        xh = R.rhtq_inverse(packed, scales, w.n, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
        torch.cuda.synchronize()
        ref = O.inverse(p_rows, s_rows, s, w.fmt, w.group, None)
        err = np.max(np.abs(to_np(xh[rows_t]) - ref), axis=1)
        assert np.all(err <= 1e-5 * np.max(np.abs(ref), axis=1) + 1e-30)
        del xh
    del packed, scales
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# sweeps: every width, several token counts, signs on / off, fp32 input
# ----------------------------------------------------------------------------

WIDTHS = [16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 3072, 6144, 12288, 24576,
          2752, 5504, 11008, 22016]


@pytest.mark.parametrize("n", WIDTHS)
def test_rotate_every_width(R, n):
    import torch
    for tokens in (1, 3, 33):
        for seed in (None, 1):
            say(f"rotate n={n} tokens={tokens} signs={seed}")
            g = torch.Generator().manual_seed(n + tokens)
            xc = torch.randn(tokens, n, generator=g) * torch.exp(torch.randn(n, generator=g))
            s = None if seed is None else splitmix64_signs(seed, n)
            for dt in (torch.bfloat16, torch.float16, torch.float32):
                x = xc.to(dt).to(dev())
                y = to_np(R.rhtq_rotate(x, s))
                C.check_rotation(y, O.rotate(x.cpu(), s))


@pytest.mark.parametrize("n", WIDTHS)
def test_quantise_every_width(R, n):
    import torch
    g = torch.Generator().manual_seed(3 * n)
    xc = torch.randn(35, n, generator=g) * torch.exp(torch.randn(n, generator=g))
    s = splitmix64_signs(2, n)
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        x = xc.to(dt).to(dev())
        y_ref = O.rotate(x.cpu(), s)
        groups = [0, 16, 128] if n % 128 == 0 else [0, 16]
        for group in groups:
            for sd in ("f32", "f16"):
                say(f"int4 n={n} group={group} scale={sd} dtype={dt}")
                check_forward(R, x, s, "int4", group, sd, y_ref=y_ref)
        say(f"nvfp4 n={n} dtype={dt}")
        check_forward(R, x, s, "nvfp4", 16, "e4m3", y_ref=y_ref)
        if n >= 32:
            say(f"mxfp4 n={n} dtype={dt}")
            check_forward(R, x, s, "mxfp4", 32, "e8m0", y_ref=y_ref)


@pytest.mark.parametrize("n,tokens", [(4096, 3000), (128, 40000), (3072, 2500), (8192, 1100), (12288, 1100),
                                      (16384, 600), (24576, 600)])
def test_fp32_input_many_rows_per_wave(R, n, tokens):
    """fp32 input on the single-stage, 12288, 16384 and 24576 kernels (three exact bf16 terms per value
    for stage 1, no prefetch): more rows than the persistent grid, so waves take several units; INT4 g128 and
    per-token, dynamic NVFP4 (its tensor scale over all rows) and MXFP4 on sampled rows, the
    rotation of the same rows."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=n, tokens=tokens)
    xb, s = generate(w, dev())
    x = xb.float() * (1.0 + 1e-3 * torch.randn(xb.shape, device=dev()))   # values off the bf16 grid
    rows = np.unique(np.array([0, 1, 2, tokens // 3, tokens // 2, tokens - 3, tokens - 2, tokens - 1]))
    y_ref = O.rotate(x[rows].cpu(), s)
    C.check_rotation(to_np(R.rhtq_rotate(x, s))[rows], y_ref)
    for group, sd in ((128, "f16"), (0, "f32")):
        say(f"fp32 int4 n={n} tokens={tokens} group={group}")
        check_forward(R, x, s, "int4", group, sd, rows=rows, y_ref=y_ref)
    say(f"fp32 nvfp4 n={n} tokens={tokens}")
    packed, scales, g = run_forward(R, x, s, "nvfp4", 16, "e4m3")
    g_ref = np.float32(np.max(np.abs(O.rotate(x.cpu(), s))) / 2688.0)
    C.check_nvfp4(packed[rows], scales[rows], g, y_ref, g_ref)
    say(f"fp32 mxfp4 n={n} tokens={tokens}")
    check_forward(R, x, s, "mxfp4", 32, "e8m0", rows=rows, y_ref=y_ref)


@pytest.mark.parametrize("n", [8192, 16384, 22016, 11008, 5504, 2752, 12288, 24576])
def test_wide_rows_many_per_workgroup(R, n):
    """The multi-wave kernels (8192, 16384, 11008 = 172 x 64, 5504 and 2752 = 172 x 32 and 16 two
    and four rows at a time, 12288 = 12 x 1024, 24576 = 12 x 2048): 2503 rows (the last set of
    5504 or 2752 rows is partial),
    more than the resident workgroups, so every workgroup of the persistent kernel loops over
    several rows (per-token INT4 takes a barrier per row), and a count no grid divides.
    The oracle checks sampled rows (the dynamic NVFP4 tensor scale over all of them)."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=n, tokens=2503)
    say(f"wide rows n={n} tokens={w.tokens}")
    x, s = generate(w, dev())
    rows = np.unique(np.concatenate([np.arange(0, w.tokens, 37), [1, w.tokens - 2, w.tokens - 1]]))
    rows_t = torch.from_numpy(rows).to(dev())
    y_ref = O.rotate(x[rows_t].cpu(), s)
    y = R.rhtq_rotate(x, s)
    torch.cuda.synchronize()
    C.check_rotation(to_np(y[rows_t]), y_ref)
    del y
    g128 = 128 if n % 128 == 0 else 64   # 2752 = 64 x 43
    for fmt, group, sd in [("int4", 0, "f32"), ("int4", g128, "f16"), ("mxfp4", 32, "e8m0"), ("nvfp4", 16, "e4m3")]:
        say(f"wide rows n={n} {fmt} group={group}")
        packed, scales, ts = R.rhtq_forward(x, s, fmt=fmt, group=group, scale_dtype=sd)
        torch.cuda.synchronize()
        p_rows, s_rows = to_np(packed[rows_t]), to_np(scales[rows_t])
        if fmt == "int4":
            print(C.check_int4(p_rows, s_rows, y_ref, group, sd))
        elif fmt == "mxfp4":
            print(C.check_mxfp4(p_rows, s_rows, y_ref))
        else:
            amax = 0.0
            for r0 in range(0, w.tokens, 256):
                amax = max(amax, float(np.max(np.abs(O.rotate(x[r0:r0 + 256].cpu(), s)))))
            print(C.check_nvfp4(p_rows, s_rows, float(ts.item()), y_ref, np.float32(amax / 2688.0)))


INT4_GROUPS = ([(n, g) for n in (12288, 24576) for g in (0, 16, 32, 64, 128, 256, 512)]
               + [(12288, g) for g in (1024, 2048, 4096)]
               + [(11008, g) for g in (0, 16, 32, 64, 128, 256)] + [(5504, g) for g in (0, 16, 32, 64, 128)]
               + [(2752, g) for g in (0, 16, 32, 64)] + [(22016, g) for g in (0, 16, 32, 64, 128, 256, 512)])


@pytest.mark.parametrize("n,group", INT4_GROUPS)
def test_wide_every_int4_group(R, n, group):
    """Every INT4 group the wide kernels take, and per-token scales (a row maximum across the
    waves): 12288 = 12 x 1024 (two waves per row) and 24576 = 12 x 2048 (four), groups 16 .. 512
    from 8 values per lane, lane swaps and 0-4 DPP steps, and at 12288 groups of 1, 2 and 4 whole
    sub-rows (1024 .. 4096, maxima across both waves); 11008 = 172 x 64, 5504 = 172 x 32 and
    2752 = 172 x 16 (two and four rows per work row), groups of runs, a'-rows and a'-row pairs or
    quads.  Every row against the oracle, both scale types."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["downproj_12288_int4g128"], n=n, tokens=67)
    x, s = generate(w, dev())
    y_ref = O.rotate(x.cpu(), s)
    for sd in ("f32", "f16"):
        say(f"{n} int4 group={group} scale={sd}")
        print(check_forward(R, x, s, "int4", group, sd, y_ref=y_ref))


WHOLE_CHUNK_GROUPS = [(4096, 2048), (8192, 2048), (8192, 4096), (3072, 1024), (6144, 1024), (6144, 2048)]


@pytest.mark.parametrize("n,group", WHOLE_CHUNK_GROUPS)
def test_int4_groups_of_whole_chunks(R, n, group):
    """INT4 groups wider than the single-stage kernel's epilogue chunk (512 or 1024 elements) and
    narrower than the row: each chunk's maximum over the wave, then over the chunks of its group.
    Every row of 67 against the oracle, with one row of magnitude 1e30 (saturating fp16 scales),
    both scale types."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["downproj_12288_int4g128"], n=n, tokens=67)
    x, s = generate(w, dev())
    x[30] = special_rows("huge", n, 1, device=dev())[0]
    torch.cuda.synchronize()
    y_ref = O.rotate(x.cpu(), s)
    for sd in ("f32", "f16"):
        say(f"{n} int4 group={group} scale={sd}")
        print(check_forward(R, x, s, "int4", group, sd, y_ref=y_ref))


def test_12288_whole_subrow_groups_many_rows(R):
    """INT4 groups of 1024, 2048 and 4096 at width 12288 on more rows than the persistent grid has
    workgroups (so workgroups take several rows and reuse the LDS group maxima), with rows of
    magnitude 1e30 among them, whose fp16 scales saturate and whose codes clamp."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["downproj_12288_int4g128"], tokens=1100)
    x, s = generate(w, dev())
    x[7] = special_rows("huge", 12288, 1, device=dev())[0]
    x[1093] = special_rows("huge", 12288, 1, seed=8, device=dev())[0]
    torch.cuda.synchronize()
    y_ref = O.rotate(x.cpu(), s)
    for group in (1024, 2048, 4096):
        say(f"12288 int4 group={group} rows=1100 with saturating rows")
        print(check_forward(R, x, s, "int4", group, "f16", y_ref=y_ref))


def test_16384_large_groups_many_rows(R):
    """INT4 groups of 1024 .. 8192 at width 16384 (one wave's own 1024-groups, and groups spanning
    two or four waves, met in LDS) on more rows than the persistent grid has workgroups, with two
    rows of magnitude 1e30 whose fp16 scales saturate; bf16, fp16 and fp32 input; fp32 and fp16
    scales."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=16384, tokens=700)
    xb, s = generate(w, dev())
    xb[5] = special_rows("huge", 16384, 1, device=dev())[0]
    xb[690] = special_rows("huge", 16384, 1, seed=8, device=dev())[0]
    torch.cuda.synchronize()
    for dt in ("bf16", "f16", "f32"):
        if dt == "bf16":
            x = xb
        elif dt == "f16":
            x = (xb.float() * 0.25).clamp(-6e4, 6e4).to(torch.float16)   # the 1e30 rows saturate fp16
        else:
            x = xb.float() * (1.0 + 2.0 ** -12)
        y_ref = O.rotate(x.cpu(), s)
        for group, sd in ((1024, "f16"), (2048, "f32"), (4096, "f16"), (8192, "f32")):
            say(f"16384 int4 group={group} scale={sd} rows=700 input={dt}")
            print(check_forward(R, x, s, "int4", group, sd, y_ref=y_ref))


def test_24576_large_groups_many_rows(R):
    """INT4 groups of 1024 .. 8192 at width 24576 (each spans two or four waves, met in LDS) on more
    rows than the persistent grid has workgroups, with a row of magnitude 1e30 whose fp16 scales
    saturate; bf16, fp16 and fp32 input; fp32 and fp16 scales."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=24576, tokens=600)
    xb, s = generate(w, dev())
    xb[591] = special_rows("huge", 24576, 1, device=dev())[0]
    torch.cuda.synchronize()
    for dt in ("bf16", "f16", "f32"):
        if dt == "bf16":
            x = xb
        elif dt == "f16":
            x = (xb.float() * 0.25).clamp(-6e4, 6e4).to(torch.float16)
        else:
            x = xb.float() * (1.0 + 2.0 ** -12)
        y_ref = O.rotate(x.cpu(), s)
        for group, sd in ((1024, "f32"), (2048, "f16"), (4096, "f32"), (8192, "f16")):
            say(f"24576 int4 group={group} scale={sd} rows=600 input={dt}")
            print(check_forward(R, x, s, "int4", group, sd, y_ref=y_ref))


@pytest.mark.parametrize("n", [16, 32, 64])
def test_narrow_rows_ragged_units(R, n):
    """16-, 32- and 64-wide rows share a 512-element wave unit (32, 16 or 8 rows); 4099 rows
    leave a partial last unit.  Every row against the oracle, every format."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["kv_128_int4g128"], n=n, tokens=4099)
    say(f"narrow rows n={n} tokens={w.tokens}")
    x, s = generate(w, dev())
    y_ref = O.rotate(x.cpu(), s)
    C.check_rotation(to_np(R.rhtq_rotate(x, s)), y_ref)
    for fmt, group, sd in [("int4", 0, "f16"), ("int4", 16, "f32"), ("nvfp4", 16, "e4m3"), ("mxfp4", 32, "e8m0")]:
        if fmt == "mxfp4" and n < 32:
            continue
        say(f"narrow rows n={n} {fmt} group={group}")
        print(check_forward(R, x, s, fmt, group, sd, y_ref=y_ref))


def test_package_imported_before_torch():
    """A fresh process that imports the package before torch still launches on torch's
    runtime and stream, and gets the same bytes as this process."""
    import subprocess
    import torch
    import randomized_hadamard_rotation_amd as R
    say("package imported before torch, in a subprocess")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import randomized_hadamard_rotation_amd as R\n"
            "import torch\n"
            "from workloads import WORKLOADS, generate\n"
            "x, s = generate(WORKLOADS['llama_4096_int4'].with_tokens(33), 'cuda')\n"
            "p, sc, _ = R.rhtq_forward(x, s, fmt='int4')\n"
            "torch.cuda.synchronize()\n"
            "print(int(p.to(torch.int64).sum()), float(sc.double().sum()))\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    x, s = generate(WORKLOADS["llama_4096_int4"].with_tokens(33), dev())
    p, sc, _ = R.rhtq_forward(x, s, fmt="int4")
    torch.cuda.synchronize()
    assert r.stdout.split()[-2:] == [str(int(p.to(torch.int64).sum())), str(float(sc.double().sum()))]


def test_forced_launch_failure_reports_and_writes_nothing():
    """RHTQ_TEST_FAIL_LAUNCH=1 (fresh process): every entry point passes its argument checks,
    reports RHTQ_EHIP where it would launch, and leaves the outputs as they were; a bad argument
    still reports RHTQ_EINVAL first."""
    import subprocess
    say("forced launch failure, in a subprocess")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import torch\n"
            "import randomized_hadamard_rotation_amd as R\n"
            "x = torch.ones(8, 4096, dtype=torch.bfloat16, device='cuda')\n"
            "p = torch.full((8, 2048), 0xA5, dtype=torch.uint8, device='cuda')\n"
            "sc = torch.full((8, 1), 3.0, dtype=torch.float32, device='cuda')\n"
            "y = torch.full((8, 4096), 7.0, dtype=torch.float32, device='cuda')\n"
            "st = []\n"
            "for f in (lambda: R.rhtq_forward(x, None, fmt='int4', packed=p, scales=sc),\n"
            "          lambda: R.rhtq_rotate(x, None, out=y),\n"
            "          lambda: R.rhtq_inverse(p, sc, 4096, None, fmt='int4', out=y)):\n"
            "    try:\n"
            "        f(); st.append(0)\n"
            "    except R.RhtqError as e:\n"
            "        st.append(e.status)\n"
            "try:\n"
            "    R.rhtq_forward(x[:, :4000], None, fmt='int4'); st.append(0)\n"
            "except R.RhtqError as e:\n"
            "    st.append(e.status)\n"
            "except ValueError:\n"
            "    st.append(-1)\n"
            "torch.cuda.synchronize()\n"
            "ok = bool((p == 0xA5).all()) and bool((sc == 3.0).all()) and bool((y == 7.0).all())\n"
            "print(st, ok)\n") % ROOT
    env = dict(os.environ, RHTQ_TEST_FAIL_LAUNCH="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    statuses, ok = r.stdout.strip().splitlines()[-1].rsplit(" ", 1)
    st = [int(v) for v in statuses.strip("[]").split(",")]
    assert st[:3] == [3, 3, 3], r.stdout
    assert st[3] != 3, r.stdout   # rejected before the hook (unsupported width or bad argument)
    assert ok == "True", r.stdout


GENERIC_WIDTHS = [16, 128, 1024, 4096, 8192, 3072, 12288, 24576, 2752, 5504, 11008]


def test_generic_kernel_on_fast_widths(tmp_path):
    """RHTQ_FORCE_GENERIC=1 (fresh process) sends bf16 rows of widths that normally take a fast
    kernel through the generic LDS-staged kernel, the fallback for every other case: rotation,
    INT4 g16, NVFP4 (dynamic g) and MXFP4 against the oracle, 9 rows each."""
    import subprocess
    import torch
    say("generic kernel on the fast widths, in a subprocess")
    out = str(tmp_path / "generic.npz")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import numpy as np, torch\n"
            "import randomized_hadamard_rotation_amd as R\n"
            "from workloads import splitmix64_signs\n"
            "res = {}\n"
            "for n in %r:\n"
            "    g = torch.Generator().manual_seed(n)\n"
            "    x = (torch.randn(9, n, generator=g) * torch.exp(torch.randn(n, generator=g))).to(torch.bfloat16).cuda()\n"
            "    s = splitmix64_signs(4, n)\n"
            "    res[f'x{n}'] = x.float().cpu().numpy()\n"
            "    res[f'y{n}'] = R.rhtq_rotate(x, s).cpu().numpy()\n"
            "    for fmt, grp, sd in (('int4', 16, 'f16'), ('nvfp4', 16, 'e4m3'), ('mxfp4', 32, 'e8m0')):\n"
            "        if fmt == 'mxfp4' and n < 32: continue\n"
            "        p, sc, ts = R.rhtq_forward(x, s, fmt=fmt, group=grp, scale_dtype=sd)\n"
            "        res[f'p{fmt}{n}'] = p.cpu().numpy(); res[f's{fmt}{n}'] = sc.cpu().numpy()\n"
            "        if ts is not None: res[f't{fmt}{n}'] = ts.cpu().numpy()\n"
            "torch.cuda.synchronize()\n"
            "np.savez(%r, **res)\n"
            "print('done')\n") % (ROOT, GENERIC_WIDTHS, out)
    env = dict(os.environ, RHTQ_FORCE_GENERIC="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip().endswith("done"), r.stderr[-2000:]
    d = np.load(out)
    for n in GENERIC_WIDTHS:
        say(f"generic kernel n={n}")
        s = splitmix64_signs(4, n)
        y_ref = O.rotate(torch.from_numpy(d[f"x{n}"]).to(torch.bfloat16), s)
        C.check_rotation(d[f"y{n}"], y_ref)
        C.check_int4(d[f"pint4{n}"], d[f"sint4{n}"], y_ref, 16, "f16")
        amax = float(np.max(np.abs(y_ref)))
        C.check_nvfp4(d[f"pnvfp4{n}"], d[f"snvfp4{n}"], float(d[f"tnvfp4{n}"].reshape(-1)[0]), y_ref,
                      np.float32(amax / 2688.0))
        if n >= 32:
            C.check_mxfp4(d[f"pmxfp4{n}"], d[f"smxfp4{n}"], y_ref)


def test_nvfp4_given_tensor_scale(R):
    import torch
    w = WORKLOADS["nvfp4_4096"].with_tokens(77)
    x, s = x_to(w)
    say("nvfp4 given tensor scale")
    y_ref = O.rotate(x.cpu(), s)
    g = torch.tensor([0.37], dtype=torch.float32, device=dev())
    packed, scales, ts = R.rhtq_forward(x, s, fmt="nvfp4", tensor_scale=g, tensor_scale_mode="given")
    torch.cuda.synchronize()
    assert float(ts.item()) == np.float32(0.37)       # read, not overwritten
    C.check_nvfp4(to_np(packed), to_np(scales), np.float32(0.37), y_ref, g_ref=np.float32(0.37))


# ----------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["zeros", "constant", "tiny", "huge"])
def test_special_inputs(R, kind):
    for n in (128, 4096, 12288):
        say(f"special {kind} n={n}")
        x = special_rows(kind, n, 5, device=dev())
        s = splitmix64_signs(3, n)
        y_ref = O.rotate(x.cpu(), s)
        C.check_rotation(to_np(R.rhtq_rotate(x, s)), y_ref)
        check_forward(R, x, s, "int4", 0, "f32", y_ref=y_ref)
        check_forward(R, x, s, "int4", 128, "f16", y_ref=y_ref)
        check_forward(R, x, s, "nvfp4", 16, "e4m3", y_ref=y_ref)
        check_forward(R, x, s, "mxfp4", 32, "e8m0", y_ref=y_ref)


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_12288_halves_far_apart(R, in_dtype):
    """12288-wide rows whose halves (sub-rows 0-5 and 6-11, the shares of the kernel's two waves)
    differ in magnitude by about 2^116 or 2^60, in both orders, plus an ordinary row: taking the
    larger half into the smaller half's units must not leave fp32's range, and the rotation and
    codes must match the oracle (which keeps the tiny half's negligible contribution exactly)."""
    import torch
    n = 12288
    s = splitmix64_signs(12, n)
    g = torch.Generator().manual_seed(121)
    x = torch.randn(5, n, generator=g, dtype=torch.float64)
    for r, (lo, hi) in enumerate([(1e-20, 1e15), (1e15, 1e-20), (1e-9, 1e9), (1e9, 1e-9)]):
        x[r, : n // 2] *= lo
        x[r, n // 2:] *= hi
    x = x.to(torch.bfloat16 if in_dtype == "bf16" else torch.float32)
    say(f"12288 halves far apart, {in_dtype}")
    y_ref = O.rotate(x, s)
    xd = x.to(dev())
    C.check_rotation(to_np(R.rhtq_rotate(xd, s)), y_ref)
    check_forward(R, xd, s, "int4", 128, "f32", y_ref=y_ref)
    check_forward(R, xd, s, "int4", 0, "f32", y_ref=y_ref)
    check_forward(R, xd, s, "mxfp4", 32, "e8m0", y_ref=y_ref)
    check_forward(R, xd, s, "nvfp4", 16, "e4m3", y_ref=y_ref)


@pytest.mark.parametrize("n", [128, 4096, 12288, 16384, 24576])
def test_fp32_rows_near_the_normal_floor(R, n):
    """fp32 rows of magnitude 1e-35 .. 3e-38 (just above the fp32 denormal range) through the fp32
    fast paths: the three bf16 terms of each value must stay normal numbers (the matrix cores flush
    denormal operands), so the rotation meets R1 at every magnitude; INT4 g128 at 1e-35."""
    import torch
    s = splitmix64_signs(3, n)
    for scale in (1e-35, 1e-37, 3e-38):
        say(f"fp32 n={n} rows of magnitude {scale:g}")
        g = torch.Generator().manual_seed(n)
        x = (torch.randn(5, n, generator=g, dtype=torch.float64) * scale).to(torch.float32)
        y_ref = O.rotate(x, s)
        C.check_rotation(to_np(R.rhtq_rotate(x.to(dev()), s)), y_ref)
        if scale == 1e-35:
            check_forward(R, x.to(dev()), s, "int4", 128, "f32", y_ref=y_ref)


@pytest.mark.parametrize("n", [128, 4096, 12288, 24576, 16384])
def test_fp16_rows_near_and_below_the_normal_floor(R, n):
    """fp16 rows whose values sit around the fp16 normal floor (6.1e-5) and in its subnormal range:
    an fp16 input value is an exact operand of the f16 matrix-core instruction, so the rotation
    must meet R1 on rows made mostly or only of fp16 subnormals, and INT4 g128 / MXFP4 on them."""
    import torch
    s = splitmix64_signs(5, n)
    for scale in (1e-3, 6e-5, 1e-6):
        say(f"fp16 n={n} rows of magnitude {scale:g}")
        g = torch.Generator().manual_seed(n + 1)
        x = (torch.randn(5, n, generator=g, dtype=torch.float64) * scale).to(torch.float16)
        if scale == 1e-6:
            assert float(x.abs().max()) < 6.1e-5          # every value an fp16 subnormal
        y_ref = O.rotate(x, s)
        C.check_rotation(to_np(R.rhtq_rotate(x.to(dev()), s)), y_ref)
        check_forward(R, x.to(dev()), s, "int4", 128, "f32", y_ref=y_ref)
        check_forward(R, x.to(dev()), s, "mxfp4", 32, "e8m0", y_ref=y_ref)


@pytest.mark.parametrize("n,tokens", [(4096, 3000), (4096, 64), (1024, 5000), (128, 40000), (8192, 1100),
                                      (16384, 600), (12288, 1100), (24576, 300), (11008, 700), (22016, 300),
                                      (2752, 3000), (3072, 2500)])
def test_fp16_input_many_rows(R, n, tokens):
    """fp16 input on every kernel family (the paired and one-wave 4096 kernels, the two-stage,
    wide, 12288, 24576, 172 x 2^k and single-stage kernels): more rows than the persistent grids,
    INT4 per-token and g128, dynamic NVFP4 (tensor scale over all rows) and MXFP4 on sampled rows,
    and the rotation of the same rows."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=n, tokens=tokens)
    xb, s = x_to(w)
    # a quarter of the recipe: its sink-row outlier columns reach ~5e4, near fp16's largest value
    x = (xb.to(torch.float32) * 0.25).to(torch.float16)
    assert bool(torch.isfinite(x).all())
    rows = np.unique(np.array([0, 1, tokens // 3, tokens // 2, tokens - 2, tokens - 1]))
    amax = None
    g2 = 128 if n % 128 == 0 else 64
    for fmt, grp, sd in [("int4", 0, "f32"), ("int4", g2, "f16"), ("nvfp4", 16, "e4m3"), ("mxfp4", 32, "e8m0")]:
        say(f"fp16 n={n} rows={tokens} {fmt} g{grp}")
        g_ref = None
        if fmt == "nvfp4":
            if amax is None:
                step = max(1, (1 << 22) // n)
                amax = max(float(np.max(np.abs(O.rotate(x[r0:r0 + step].cpu(), s)))) for r0 in range(0, tokens, step))
            g_ref = np.float32(amax / 2688.0)
        check_forward(R, x, s, fmt, grp, sd, rows=rows, g_ref=g_ref)
    y = to_np(R.rhtq_rotate(x, s))
    C.check_rotation(y[rows], O.rotate(x[rows].cpu(), s))


@pytest.mark.parametrize("n,tokens", [(11008, 700), (22016, 300), (5504, 1101), (2752, 2101)])
def test_fp32_input_172_widths_many_rows(R, n, tokens):
    """fp32 input on the 172 x 2^k kernels (three passes of exact bf16 terms through the LDS
    tile): more rows than the persistent grid, odd row counts for the two- and four-row work
    rows, INT4 per-token and g64, dynamic NVFP4 and MXFP4 on sampled rows, and the rotation."""
    import dataclasses
    import torch
    w = dataclasses.replace(WORKLOADS["llama_4096_int4"], n=n, tokens=tokens)
    xb, s = x_to(w)
    x = xb.to(torch.float32) * (1.0 + 2.0 ** -12)   # values with more than 8 significant bits
    rows = np.unique(np.array([0, 1, tokens // 3, tokens // 2, tokens - 2, tokens - 1]))
    amax = None
    for fmt, grp, sd in [("int4", 0, "f32"), ("int4", 64, "f16"), ("nvfp4", 16, "e4m3"), ("mxfp4", 32, "e8m0")]:
        say(f"fp32 n={n} rows={tokens} {fmt} g{grp}")
        g_ref = None
        if fmt == "nvfp4":
            if amax is None:
                step = max(1, (1 << 22) // n)
                amax = max(float(np.max(np.abs(O.rotate(x[r0:r0 + step].cpu(), s)))) for r0 in range(0, tokens, step))
            g_ref = np.float32(amax / 2688.0)
        check_forward(R, x, s, fmt, grp, sd, rows=rows, g_ref=g_ref)
    y = to_np(R.rhtq_rotate(x, s))
    C.check_rotation(y[rows], O.rotate(x[rows].cpu(), s))
    # rows of magnitude 1e-30, above the 2^-110 floor of the unscaled lower terms
    xt = (torch.randn(3, n, generator=torch.Generator().manual_seed(n), dtype=torch.float64) * 1e-30).to(torch.float32)
    C.check_rotation(to_np(R.rhtq_rotate(xt.to(dev()), s)), O.rotate(xt, s))


def test_zero_tokens_is_noop(R):
    import torch
    say("tokens = 0")
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device=dev())
    R.rhtq_rotate(x)
    R.rhtq_forward(x)
    torch.cuda.synchronize()


@pytest.mark.parametrize("tokens", [4095, 4096, 4097, 4099])
def test_4096_row_count_paths(R, tokens):
    """Width 4096 runs two waves per row up to 4096 rows and one wave per row beyond: both sides of
    the switch, a row count that leaves workgroup slots past the last row, every format (sampled
    rows; the NVFP4 tensor scale over all rows)."""
    import torch
    w = WORKLOADS["llama_4096_int4"]
    x, s = x_to(w, tokens)
    rows = np.unique(np.array([0, 1, 2, 3, tokens // 2, tokens - 4, tokens - 3, tokens - 2, tokens - 1]))
    for fmt, grp, sd in [("int4", 0, "f32"), ("int4", 128, "f16"), ("nvfp4", 16, "e4m3"), ("mxfp4", 32, "e8m0")]:
        say(f"rows={tokens} {fmt} g{grp}")
        g_ref = None
        if fmt == "nvfp4":
            amax = max(float(np.max(np.abs(O.rotate(x[r0:r0 + 2048].cpu(), s)))) for r0 in range(0, tokens, 2048))
            g_ref = np.float32(amax / 2688.0)
        check_forward(R, x, s, fmt, grp, sd, rows=rows, g_ref=g_ref)
    y = to_np(R.rhtq_rotate(x, s))
    C.check_rotation(y[rows], O.rotate(x[rows].cpu(), s))


def test_deterministic(R):
    import torch
    for name in ("llama_4096_int4", "downproj_12288_int4g128", "kv_128_int4g128", "nvfp4_4096",
                 "mxfp4_4096"):
        w = WORKLOADS[name]
        say(f"determinism {name}")
        x, s = x_to(w, min(w.tokens, 512))
        a = run_forward(R, x, s, w.fmt, w.group, w.scale_dtype)
        b = run_forward(R, x, s, w.fmt, w.group, w.scale_dtype)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


# ----------------------------------------------------------------------------
# inverse
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["llama_4096_int4", "downproj_12288_int4g128", "kv_128_int4g128",
                                  "nvfp4_4096", "mxfp4_4096", "downproj7b_11008_int4g128",
                                  "wide172_22016_int4g128"])
def test_inverse_round_trip(R, name):
    import torch
    w = WORKLOADS[name]
    say(f"inverse {name}")
    x, s = x_to(w, 41)
    packed, scales, ts = R.rhtq_forward(x, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
    xh = R.rhtq_inverse(packed, scales, w.n, s, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype,
                        tensor_scale=ts)
    torch.cuda.synchronize()
    g = None if ts is None else float(ts.item())
    ref = O.inverse(to_np(packed), to_np(scales), s, w.fmt, w.group, g)
    err = np.max(np.abs(to_np(xh) - ref), axis=1)
    assert np.all(err <= 1e-5 * np.max(np.abs(ref), axis=1) + 1e-30)
    # round trip bound: ||x - x_hat|| <= sqrt(sum over groups |G| (s_G/2)^2) for INT4
    xr = to_np(x)
    if w.fmt == "int4":
        sc = to_np(scales).astype(np.float64)
        gsz = w.n if w.group == 0 else w.group
        bound = np.sqrt(np.sum(gsz * (sc / 2) ** 2, axis=1))
        assert np.all(np.linalg.norm(to_np(xh) - xr, axis=1) <= bound * (1 + 1e-4))
    # the rotation alone inverts to fp32 precision
    y = R.rhtq_rotate(x, s)
    torch.cuda.synchronize()
    assert np.allclose(O.inverse_rotate(to_np(y), s), xr, rtol=0, atol=1e-5 * np.abs(xr).max())


@pytest.mark.parametrize("n", [24576, 5504, 2752, 3072, 22016])
def test_inverse_round_trip_widths(R, n):
    """Inverse of the device's own codes at the 12 x 2^k and 172 x 2^k widths outside the bench
    workloads (INT4 g16 and MXFP4), against the oracle's inverse of the same codes; the rotation
    alone inverts to fp32 precision."""
    import torch
    g = torch.Generator().manual_seed(7 * n)
    x = (torch.randn(13, n, generator=g) * torch.exp(torch.randn(n, generator=g))).to(torch.bfloat16).to(dev())
    s = splitmix64_signs(6, n)
    for fmt, grp, sd in (("int4", 16, "f16"), ("mxfp4", 32, "e8m0")):
        say(f"inverse n={n} {fmt}")
        packed, scales, _ = R.rhtq_forward(x, s, fmt=fmt, group=grp, scale_dtype=sd)
        xh = R.rhtq_inverse(packed, scales, n, s, fmt=fmt, group=grp, scale_dtype=sd)
        torch.cuda.synchronize()
        ref = O.inverse(to_np(packed), to_np(scales), s, fmt, grp, None)
        err = np.max(np.abs(to_np(xh) - ref), axis=1)
        assert np.all(err <= 1e-5 * np.max(np.abs(ref), axis=1) + 1e-30)
    y = R.rhtq_rotate(x, s)
    torch.cuda.synchronize()
    xr = to_np(x)
    assert np.allclose(O.inverse_rotate(to_np(y), s), xr, rtol=0, atol=1e-5 * np.abs(xr).max())


@pytest.mark.parametrize("n", [64, 128, 256])
def test_inverse_kv_rows(R, n):
    """KV-cache read path (one INT4 scale per row, head dims 64 / 128 / 256): the device inverse of
    device codes against the oracle's inverse of the same codes, ragged row counts included."""
    import torch
    for tokens in (1, 7, 1000, 1031):
        for sd in ("f16", "f32"):
            for seed in (None, 4):
                say(f"inverse kv n={n} tokens={tokens} scale={sd} signs={seed}")
                g = torch.Generator().manual_seed(n + tokens)
                x = (torch.randn(tokens, n, generator=g) * torch.exp(torch.randn(tokens, 1, generator=g)))
                x = x.to(torch.bfloat16).to(dev())
                s = None if seed is None else splitmix64_signs(seed, n)
                packed, scales, _ = R.rhtq_forward(x, s, fmt="int4", group=n, scale_dtype=sd)
                xh = R.rhtq_inverse(packed, scales, n, s, fmt="int4", group=n, scale_dtype=sd)
                torch.cuda.synchronize()
                ref = O.inverse(to_np(packed), to_np(scales), s, "int4", n)
                err = np.max(np.abs(to_np(xh) - ref), axis=1)
                assert np.all(err <= 1e-6 * np.max(np.abs(ref), axis=1) + 1e-30), (n, tokens, sd, seed)


BLOCKED = [(4096, 128), (4096, 1024), (12288, 1024), (12288, 4096), (256, 128), (2048, 16), (8192, 2048),
           (1024, 512), (11008, 128), (11008, 256), (5120, 1024), (384, 128), (4096, 64), (384, 32),
           (8192, 32), (16384, 8192)]


@pytest.mark.parametrize("n,block", BLOCKED)
def test_blocked_rotation_and_quantisation(R, n, block):
    """Block-diagonal rotation (NVFP4 methodology thread, block-Hadamard-128): full-length signs, then
    H_b per block; every format whose groups fit a block; the inverse of the device's codes."""
    import torch
    g = torch.Generator().manual_seed(n + block)
    xc = torch.randn(21, n, generator=g) * torch.exp(torch.randn(n, generator=g))
    s = splitmix64_signs(8, n)
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        x = xc.to(dt).to(dev())
        y_ref = O.rotate_blocked(x.cpu(), s, block)
        say(f"blocked rotate n={n} b={block} dtype={dt}")
        C.check_rotation(to_np(R.rhtq_rotate(x, s, block=block)), y_ref)
        cases = [("int4", 16, "f16"), ("nvfp4", 16, "e4m3")]
        if block >= 32:
            cases.append(("mxfp4", 32, "e8m0"))
        if block >= 128:
            cases.append(("int4", 128, "f32"))
        for fmt, grp, sd in cases:
            say(f"blocked {fmt} g{grp} n={n} b={block} dtype={dt}")
            packed, scales, ts = R.rhtq_forward(x, s, fmt=fmt, group=grp, scale_dtype=sd, block=block)
            torch.cuda.synchronize()
            p, sc = to_np(packed), to_np(scales)
            if fmt == "int4":
                C.check_int4(p, sc, y_ref, grp, sd)
            elif fmt == "mxfp4":
                C.check_mxfp4(p, sc, y_ref)
            else:
                C.check_nvfp4(p, sc, float(ts.item()), y_ref)
            xh = R.rhtq_inverse(packed, scales, n, s, fmt=fmt, group=grp, scale_dtype=sd, tensor_scale=ts,
                                block=block)
            torch.cuda.synchronize()
            ref = O.inverse(p, sc, s, fmt, grp, None if ts is None else float(ts.item()), block=block)
            err = np.max(np.abs(to_np(xh) - ref), axis=1)
            assert np.all(err <= 1e-5 * np.max(np.abs(ref), axis=1) + 1e-30)


def test_binding_noncontiguous_and_side_stream(R):
    """The binding reads non-contiguous inputs through contiguous copies that live past the
    call, and work on a non-current stream gives the same bytes as on the current one."""
    import torch
    say("binding: non-contiguous x / packed / scales, side stream")
    w = WORKLOADS["llama_4096_int4"].with_tokens(64)
    x, s = x_to(w)
    xt = x.t().contiguous().t()
    assert not xt.is_contiguous() and torch.equal(xt, x)
    p0, s0, _ = R.rhtq_forward(x, s, fmt="int4", group=128, scale_dtype="f16")
    p1, s1, _ = R.rhtq_forward(xt, s, fmt="int4", group=128, scale_dtype="f16")
    side = torch.cuda.Stream()
    p2, s2, _ = R.rhtq_forward(xt, s, fmt="int4", group=128, scale_dtype="f16", stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(p0, p1) and torch.equal(s0, s1)
    assert torch.equal(p0, p2) and torch.equal(s0, s2)
    pn, sn = p0.t().contiguous().t(), s0.t().contiguous().t()
    assert not pn.is_contiguous()
    xh0 = R.rhtq_inverse(p0, s0, 4096, s, group=128, scale_dtype="f16")
    xh1 = R.rhtq_inverse(pn, sn, 4096, s, group=128, scale_dtype="f16", stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(xh0, xh1)
    # a caller's output buffers of the wrong size are refused before any launch
    with pytest.raises(ValueError):
        R.rhtq_forward(x, s, fmt="int4", group=128, scale_dtype="f16",
                       scales=torch.empty(64, 16, dtype=torch.float16, device=dev()))
