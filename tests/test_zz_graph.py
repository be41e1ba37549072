"""HIP graph capture of the library's calls (the benchmark times graph replays): a captured
rhtq_forward, replayed several times with eager work and synchronisation between the replays,
must reproduce the eager result bit for bit (INT4 one launch; dynamic NVFP4 three launches,
including the kernel that clears the tensor-scale word)."""
import numpy as np
import pytest

from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,tokens", [("llama_4096_int4", 2048), ("nvfp4_4096", 515),
                                         ("downproj_12288_int4g128", 37)])
def test_graph_replay_matches_eager(name, tokens):
    import torch
    import randomized_hadamard_rotation_amd as R
    w = WORKLOADS[name].with_tokens(tokens)
    x, s = generate(w, "cuda")
    s_dev = torch.from_numpy(s).to("cuda")
    p_e, sc_e, ts_e = R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype)
    torch.cuda.synchronize()
    ref = [p_e.cpu().numpy(), sc_e.cpu().numpy(), None if ts_e is None else ts_e.cpu().numpy()]

    packed = torch.empty_like(p_e)
    scales = torch.empty_like(sc_e)
    ts = None if ts_e is None else torch.empty_like(ts_e)
    # an eager call with the graph's buffers first (the capture-first case has its own test)
    R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype, tensor_scale=ts,
                   packed=packed, scales=scales)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.rhtq_forward(x, s_dev, fmt=w.fmt, group=w.group, scale_dtype=w.scale_dtype, tensor_scale=ts,
                       packed=packed, scales=scales)
    for k in range(4):
        packed.fill_(0xAB)
        scales.zero_()
        if ts is not None:
            ts.fill_(123.0)
        x.add_(0)   # eager work on the same stream between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(packed.cpu().numpy(), ref[0]), f"replay {k}: codes"
        assert np.array_equal(scales.cpu().numpy(), ref[1]), f"replay {k}: scales"
        if ts is not None:
            assert np.array_equal(ts.cpu().numpy(), ref[2]), f"replay {k}: tensor scale"


def test_first_call_inside_capture_fresh_process():
    """The first call of each persistent kernel (whose grid comes from an occupancy query made on
    that call) may be captured directly: no eager warm-up call is needed.  Runs in a fresh process
    so that no earlier test has made those calls."""
    import os
    import subprocess
    import sys
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "graph_first_call.py")
    r = subprocess.run([sys.executable, script], capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
