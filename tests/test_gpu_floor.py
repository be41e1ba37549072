"""GPU: the streaming-floor measurement kernel (include/rhtq_floor.h) reads every input word and
writes every output word of its launch shape: its XOR folds are recomputed on the host from the
input's bit patterns and compared word for word, at widths 4096 (one workgroup per row) and
12288 (persistent grid, more rows than workgroups so the grid-stride loop runs)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def expected_folds(x_bits_u32: np.ndarray, n: int, scale_words: int):
    rows = x_bits_u32.shape[0]
    F = n // 1024
    v = x_bits_u32.reshape(rows, 2, F, 64, 4)          # [row][wave][fragment][lane][word]
    packed = np.bitwise_xor.reduce(v, axis=4)          # [row][wave][fragment][lane]
    sw = (v[:, :, 0, :, 0] ^ v[:, :, F - 1, :, 3]).reshape(rows, 128)[:, :scale_words]
    return packed.reshape(rows, n // 8), sw


@pytest.mark.parametrize("n,rows,scale_bytes", [(4096, 37, 4), (4096, 2048, 4), (12288, 5, 192),
                                                (12288, 2500, 192), (12288, 3, 4)])
def test_stream_floor_folds(n, rows, scale_bytes):
    import torch
    import randomized_hadamard_rotation_amd as R
    print(f"[case] stream floor n={n} rows={rows} scale_bytes={scale_bytes}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n + rows)
    x = torch.randn((rows, n), device="cuda", generator=g).to(torch.bfloat16)
    packed = torch.full((rows, n // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, scale_bytes // 4), -1, dtype=torch.int32, device="cuda")
    R.rhtq_stream_floor(x, packed, scales)
    torch.cuda.synchronize()
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    x32 = np.ascontiguousarray(xb).view(np.uint32).reshape(rows, n // 2)
    want_p, want_s = expected_folds(x32, n, scale_bytes // 4)
    got_p = packed.cpu().numpy().view(np.uint32).reshape(rows, n // 8)
    got_s = scales.cpu().numpy().view(np.uint32)
    assert np.array_equal(got_p, want_p)
    assert np.array_equal(got_s, want_s)
