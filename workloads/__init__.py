"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and lays them out.  It holds none of
the rotation or quantisation arithmetic: both the HIP library and the CPU
oracle receive the same tensors and sign vectors from here and compute
independently.

Shapes and value structure stand in for the activations the pages discuss
(Qwen3-8B / Llama-2-7B widths 4096 and 12288 = 12 x 1024, KV-cache rows of
head_dim 128, 2048-token windows, 16,384 calibration tokens, attention-sink
tokens whose RMS is 30-50x that of ordinary tokens).  No model weights or
dataset items are involved.

Random sign vector: splitmix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  Output i of seed s is
``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` with the published mixing
function; the sign is -1 when the top bit of that output is set.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, count: int) -> np.ndarray:
    """First ``count`` outputs of splitmix64 started at ``seed`` (uint64 array)."""
    with np.errstate(over="ignore"):
        i = np.arange(1, count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def splitmix64_signs(seed: int, n: int) -> np.ndarray:
    """Random +-1 vector of length n as int8 (top bit of each output set -> -1)."""
    z = splitmix64(seed, n)
    return np.where((z >> np.uint64(63)) != 0, -1, 1).astype(np.int8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, value recipe and quantisation format."""

    name: str
    tokens: int            # rows handed to the library
    n: int                 # row width
    in_dtype: str          # "f32", "bf16" or "f16"
    recipe: str            # "gauss_outlier_cols", "llama_like", "kv_spikes"
    seed: int              # value seed
    sign_seed: int         # splitmix64 seed of the sign vector
    fmt: str               # "int4", "nvfp4" or "mxfp4"
    group: int             # 0 = per token
    scale_dtype: str       # "f32", "f16", "e4m3" or "e8m0"
    tokens_per_row: float = 1.0   # KV rows: 1/32 token per row (32 heads)
    description: str = ""
    block: int = 0                # block-diagonal rotation with blocks of this size (0: whole row)

    def with_tokens(self, tokens: int) -> "Workload":
        return dataclasses.replace(self, tokens=tokens)


# The five configurations.  `tokens` is the number of rows of width n.
WORKLOADS = {
    "tiny_128_int4": Workload(
        "tiny_128_int4", 64, 128, "f32", "gauss_outlier_cols", 1, 0, "int4", 0, "f32",
        description="64 x 128 fp32, N(0,1), 2 outlier columns x20; per-token INT4, fp32 scale"),
    "llama_4096_int4": Workload(
        "llama_4096_int4", 2048, 4096, "bf16", "llama_like", 2, 0, "int4", 0, "f32",
        description="2048 x 4096 bf16, log-normal channel scales, 8 outlier channels x50, "
                    "0.5% sink rows x40; per-token INT4, fp32 scale"),
    # the headline shape with fp16 input (QuaRot's baselines are FP16 models: reviews page, review 4
    # Weaknesses); the recipe is scaled by 1/4 so its largest values (~5e4) stay inside fp16's range
    "llama_4096_int4_f16": Workload(
        "llama_4096_int4_f16", 2048, 4096, "f16", "llama_like", 2, 0, "int4", 0, "f32",
        description="2048 x 4096 fp16, the llama-like recipe x 1/4; per-token INT4, fp32 scale"),
    # the headline shape with fp32 input: each value split into three exact bf16 terms for stage 1
    "llama_4096_int4_f32": Workload(
        "llama_4096_int4_f32", 2048, 4096, "f32", "llama_like", 2, 0, "int4", 0, "f32",
        description="2048 x 4096 fp32, the llama-like recipe; per-token INT4, fp32 scale"),
    "downproj_12288_int4g128": Workload(
        "downproj_12288_int4g128", 8192, 12288, "bf16", "llama_like", 3, 0, "int4", 128, "f16",
        description="8192 x 12288 bf16 (H12 x H1024), same value recipe; INT4 group 128, fp16 scales"),
    "kv_128_int4g128": Workload(
        "kv_128_int4g128", 32 * 32 * 4096, 128, "bf16", "kv_spikes", 4, 0, "int4", 128, "f16",
        tokens_per_row=1.0 / 32.0,
        description="KV cache [32 batch][32 heads][4096 tokens][128] bf16, N(0,1) with 1% x10; "
                    "one INT4 group of 128 per head-row, fp16 scales"),
    "nvfp4_4096": Workload(
        "nvfp4_4096", 16384, 4096, "bf16", "llama_like", 5, 0, "nvfp4", 16, "e4m3",
        description="16384 x 4096 bf16, llama-like recipe with sinks; E2M1 codes, E4M3 block-16 "
                    "scales, fp32 tensor scale = amax/(6*448)"),
    # block-Hadamard-128 before INT4-g128 on the hidden width (the NVFP4 methodology thread's ablation)
    "blockh128_4096_int4g128": Workload(
        "blockh128_4096_int4g128", 16384, 4096, "bf16", "llama_like", 7, 0, "int4", 128, "f16",
        description="16384 x 4096 bf16, llama-like recipe; block-diagonal H128 with full-length signs, "
                    "INT4 group 128, fp16 scales", block=128),
    # the Llama 2 7B down_proj input: intermediate width 11008 = 172 x 64 (QuaRot reviews, review 2
    # Questions name its non-power-of-two factor 172)
    "downproj7b_11008_int4g128": Workload(
        "downproj7b_11008_int4g128", 8192, 11008, "bf16", "llama_like", 8, 0, "int4", 128, "f16",
        description="8192 x 11008 bf16 (H172 x H64), llama-like recipe; INT4 group 128, fp16 scales"),
    "wide172_22016_int4g128": Workload(
        "wide172_22016_int4g128", 8192, 22016, "bf16", "llama_like", 9, 0, "int4", 128, "f16",
        description="8192 x 22016 bf16 (H172 x H128, the next 172 x 2^k width above 11008), llama-like "
                    "recipe; INT4 group 128, fp16 scales"),
    # MXFP4 on the NVFP4 shape: the thread compares the two FP4 formats on the same model
    "mxfp4_4096": Workload(
        "mxfp4_4096", 16384, 4096, "bf16", "llama_like", 6, 0, "mxfp4", 32, "e8m0",
        description="16384 x 4096 bf16, llama-like recipe with sinks; E2M1 codes with E8M0 "
                    "power-of-two scales per 32-block (OCP MX)"),
}


def _torch():
    import torch  # local import: the oracle tests can run with numpy only
    return torch


def generate(w: Workload, device="cpu"):
    """Return (x, signs) for workload w.

    x is a torch tensor [tokens, n] in w.in_dtype on `device`, drawn with
    torch.Generator(device).manual_seed(w.seed); values are produced in fp32
    and cast to bf16 with round-to-nearest-even when the dtype is bf16, or scaled
    by 1/4 (exact) and cast to fp16 the same way when it is f16.
    signs is an int8 numpy vector of length n.
    """
    torch = _torch()
    T, n = w.tokens, w.n
    g = torch.Generator(device=device).manual_seed(w.seed)
    if w.recipe == "gauss_outlier_cols":
        z = torch.randn(T, n, generator=g, device=device, dtype=torch.float32)
        cols = torch.randperm(n, generator=g, device=device)[:2]
        z[:, cols] *= 20.0
    elif w.recipe == "llama_like":
        sigma = torch.exp(0.5 * torch.randn(n, generator=g, device=device, dtype=torch.float32))
        cols = torch.randperm(n, generator=g, device=device)[:8]
        sinks = torch.randperm(T, generator=g, device=device)[: int(round(0.005 * T))]
        z = torch.randn(T, n, generator=g, device=device, dtype=torch.float32)
        z *= sigma
        z[:, cols] *= 50.0
        if sinks.numel():
            z[sinks, :] *= 40.0
    elif w.recipe == "kv_spikes":
        z = torch.randn(T, n, generator=g, device=device, dtype=torch.float32)
        spikes = torch.rand(T, n, generator=g, device=device, dtype=torch.float32) < 0.01
        z = torch.where(spikes, z * 10.0, z)
    else:
        raise ValueError(f"unknown recipe {w.recipe}")
    if w.in_dtype == "f32":
        x = z
    elif w.in_dtype == "f16":
        x = (z * 0.25).to(torch.float16)
    else:
        x = z.to(torch.bfloat16)
    return x.contiguous(), splitmix64_signs(w.sign_seed, n)


def special_rows(kind: str, n: int, tokens: int, seed: int = 7, device="cpu", dtype="bf16"):
    """Edge-case inputs: 'zeros', 'constant', 'tiny' (values near bf16 min normal) or
    'huge' (values near 1e30).  Pure data; no method arithmetic."""
    torch = _torch()
    g = torch.Generator(device=device).manual_seed(seed)
    if kind == "zeros":
        z = torch.zeros(tokens, n, device=device)
    elif kind == "constant":
        z = torch.full((tokens, n), 3.0, device=device)
    elif kind == "tiny":
        z = torch.randn(tokens, n, generator=g, device=device) * 1e-30
    elif kind == "huge":
        z = torch.randn(tokens, n, generator=g, device=device) * 1e30
    else:
        raise ValueError(kind)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return z.to(tdt).contiguous()


def sha256_of(t) -> str:
    """SHA-256 of a tensor's bytes (on host)."""
    torch = _torch()
    a = t.detach().to("cpu").contiguous()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.sha256(a.numpy().tobytes()).hexdigest()


def bytes_per_call(w: Workload, tensor_scale_dynamic: bool = True) -> int:
    """Algorithmic HBM bytes one forward call must move: read x once (twice for the
    dynamic NVFP4 tensor scale), write packed codes and scales, read the signs."""
    in_b = 4 if w.in_dtype == "f32" else 2
    rows = w.tokens
    x_bytes = rows * w.n * in_b
    codes = rows * w.n // 2
    if w.fmt == "int4":
        groups = 1 if w.group == 0 else w.n // w.group
        sbytes = rows * groups * (4 if w.scale_dtype == "f32" else 2)
        extra = 0
    elif w.fmt == "mxfp4":
        sbytes = rows * (w.n // 32)
        extra = 0
    else:
        sbytes = rows * (w.n // 16)
        extra = 4
        if tensor_scale_dynamic:
            x_bytes *= 2
    return x_bytes + codes + sbytes + extra + w.n

