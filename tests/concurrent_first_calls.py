"""Run by tests/test_gpu_concurrency.py in a fresh process: eight host threads, each with a HIP
stream of its own, make the first calls of several kernel variants at the same time (two threads
share a variant, so its one-time launch-shape query is raced), five calls each.  The results of
every thread's last call must equal a sequential call made afterwards on the default stream.
Prints one line per case; exits non-zero on a mismatch or an error in a thread."""
import os
import sys
import threading

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CASES = [("llama_4096_int4", 512, "bf16"), ("downproj_12288_int4g128", 256, "bf16"),
         ("downproj7b_11008_int4g128", 256, "bf16"), ("nvfp4_4096", 1024, "bf16"),
         ("mxfp4_4096", 5000, "bf16"), ("llama_4096_int4", 512, "bf16"),
         ("kv_128_int4g128", 100000, "bf16"), ("llama_4096_int4", 512, "f16")]


def main():
    import torch
    import randomized_hadamard_rotation_amd as R
    from workloads import WORKLOADS, generate

    inputs = []
    for name, tokens, dt in CASES:
        w = WORKLOADS[name].with_tokens(tokens)
        x, s = generate(w, "cuda")
        if dt == "f16":
            x = (x.float() * 0.25).to(torch.float16)
        inputs.append((w, x, torch.from_numpy(s).to("cuda")))
    torch.cuda.synchronize()

    def call(w, x, s_dev):
        p, sc, ts = R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
        y = R.rhtq_rotate(x, s_dev)
        return p, sc, ts, y

    results, errors = [None] * len(CASES), [None] * len(CASES)
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            st = torch.cuda.Stream()
            w, x, s_dev = inputs[i]
            start.wait(timeout=120)
            with torch.cuda.stream(st):
                for _ in range(5):
                    out = call(w, x, s_dev)
            st.synchronize()
            results[i] = [None if t is None else t.cpu().numpy() for t in out]
        except Exception as e:   # reported by the main thread
            errors[i] = repr(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    print(f"[case] {len(CASES)} threads, first calls concurrent", flush=True)
    for t in threads:
        t.start()
    for t in threads:
        t.join()

    ok = True
    for i, (name, tokens, dt) in enumerate(CASES):
        if errors[i] is not None:
            print(f"{name} x{tokens} {dt}: ERROR {errors[i]}", flush=True)
            ok = False
            continue
        w, x, s_dev = inputs[i]
        ref = [None if t is None else t.cpu().numpy() for t in call(w, x, s_dev)]
        torch.cuda.synchronize()
        same = all((a is None and b is None) or np.array_equal(a, b) for a, b in zip(results[i], ref))
        print(f"{name} x{tokens} {dt}: {'ok' if same else 'MISMATCH'}", flush=True)
        ok &= same
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
