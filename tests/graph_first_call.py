"""Run by tests/test_zz_graph.py in a fresh process: the first call of each persistent kernel
is made inside a HIP-graph capture (no eager call before it), and the replay must equal an
eager call made afterwards.  Prints one line per case; exits non-zero on a mismatch."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    import torch
    import randomized_hadamard_rotation_amd as R
    from workloads import WORKLOADS, generate
    ok = True
    # persistent kernels: 4096 (> 4096 rows), 12288, 11008, 22016; NVFP4 with its pre-pass
    for name, tokens in [("nvfp4_4096", 8192), ("downproj_12288_int4g128", 600), ("mxfp4_4096", 9000),
                         ("downproj7b_11008_int4g128", 700), ("wide172_22016_int4g128", 300)]:
        w = WORKLOADS[name].with_tokens(tokens)
        x, s = generate(w, "cuda")
        s_dev = torch.from_numpy(s).to("cuda")
        packed = torch.empty((tokens, w.n // 2), dtype=torch.uint8, device="cuda")
        sdt = {"f32": torch.float32, "f16": torch.float16, "e4m3": torch.uint8, "e8m0": torch.uint8}[w.scale_dtype]
        scales = torch.empty((tokens, w.n // w.group), dtype=sdt, device="cuda")
        ts = torch.zeros(1, dtype=torch.float32, device="cuda") if w.fmt == "nvfp4" else None
        print(f"[case] capture-first {name} x{tokens}", flush=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype, tensor_scale=ts,
                           packed=packed, scales=scales)
        g.replay()
        torch.cuda.synchronize()
        p1, s1 = packed.cpu().numpy().copy(), scales.cpu().numpy().copy()
        pe, se, _ = R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
        torch.cuda.synchronize()
        same = np.array_equal(p1, pe.cpu().numpy()) and np.array_equal(s1, se.cpu().numpy())
        print(f"capture-first {name}: {'ok' if same else 'MISMATCH'}", flush=True)
        ok &= same
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
