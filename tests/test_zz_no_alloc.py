"""The GEMM entry point that allocates nothing (``loop_op_gemm_static``: the
split-K partials in the library's static device array) against the entry
point with a caller workspace (``loop_op_gemm``), through the C ABI: two calls
in a row, the second smaller, each bit-identical to the workspace entry point
(same kernels, same split plan) and within 2^-8 of a float64 product; rows
beyond the array's limit are rejected."""
import numpy as np
import pytest

import synth
from gpu_util import torch_cuda, dev, host, say

pytestmark = pytest.mark.gpu

CASES = [
    # (M, N, K, epilogue): the decode gate/up with SwiGLU (24 MiB of partials),
    # then a smaller down projection with the residual epilogue
    (64, 12288, 4096, 3),
    (17, 4096, 12288, 2),
]


def _operands(torch, M, N, K, epi, tag):
    rows_b = 2 * N if epi == 3 else N
    A = synth.normal(synth.SEED_X, f"noalloc.A.{tag}", (M, K), 1.0, dtype="bf16")
    B = synth.normal(synth.SEED_W, f"noalloc.B.{tag}", (rows_b, K), 0.02, dtype="bf16")
    R = synth.normal(synth.SEED_X, f"noalloc.R.{tag}", (M, N), 1.0) if epi == 2 else None
    return A, B, R


def _reference(A, B, R, N, epi):
    a = synth.bf16_bits_to_f32(A).astype(np.float64)
    b = synth.bf16_bits_to_f32(B).astype(np.float64)
    y = a @ b.T
    if epi == 3:
        g, u = y[:, :N], y[:, N:]
        return g / (1 + np.exp(-g)) * u
    return y + R if epi == 2 else y


def test_static_scratch_gemm_matches_workspace_gemm():
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    s = torch.cuda.current_stream().cuda_stream
    ws = torch.empty((64 << 20) // 4, dtype=torch.float32, device="cuda")
    for i, (M, N, K, epi) in enumerate(CASES):
        A, B, R = _operands(torch, M, N, K, epi, i)
        dA, dB = dev(A, torch), dev(B, torch)
        out_dt = torch.bfloat16 if epi in (0, 3) else torch.float32
        outs = []
        for which in ("static", "workspace"):
            C = torch.zeros((M, N), dtype=out_dt, device="cuda")
            dR = dev(R, torch) if R is not None else None
            say("gemm", which, M, N, K, epi)
            if which == "static":
                L.loop_op_gemm_static(dA.data_ptr(), K, dB.data_ptr(), K, C.data_ptr(), N,
                                      dR.data_ptr() if dR is not None else 0, M, N, K, epi, stream=s)
            else:
                L.loop_op_gemm(dA.data_ptr(), K, dB.data_ptr(), K, C.data_ptr(), N,
                               dR.data_ptr() if dR is not None else 0, M, N, K, epi, stream=s,
                               ws=ws.data_ptr(), ws_bytes=ws.numel() * 4)
            torch.cuda.synchronize()
            outs.append(host(C))
        assert np.array_equal(outs[0], outs[1]), (M, N, K, epi)
        ref = _reference(A, B, R, N, epi)
        err = np.abs(outs[0] - ref).max() / np.abs(ref).max()
        print("static-scratch gemm %dx%dx%d epi %d: bit-identical to the workspace entry, %.2e vs float64"
              % (M, N, K, epi, err))
        assert err <= 2.0 ** -8


def test_static_scratch_gemm_rejects_rows_beyond_limit():
    torch = torch_cuda()
    import looped_hybrid_attention_amd as L
    M, N, K = L.LOOP_GEMM_STATIC_MAX_ROWS + 1, 256, 256
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(L.LoopError) as ei:
        L.loop_op_gemm_static(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, 0, M, N, K, 1)
    assert ei.value.code == -3 and "rows" in str(ei.value)
    with pytest.raises(L.LoopError):
        L.loop_op_gemm_static(0, K, B.data_ptr(), K, C.data_ptr(), N, 0, 4, N, K, 1)
