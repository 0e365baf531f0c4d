"""GEMM kernel parity: C = A . B^T on bf16 inputs against the float64 matrix
product of the same bf16 values, for every epilogue, at ragged small shapes
(several tiles plus tails, both tile configurations) and at the real
projection shapes of the model (sampled rows)."""
import numpy as np
import pytest

import synth
from gpu_util import torch_cuda, dev, host, stream, say, rel_err

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, tag, nB=None):
    a = synth.normal(synth.SEED_X, f"gemmA{tag}", (M, K), 1.0, dtype="bf16")
    b = synth.normal(synth.SEED_W, f"gemmB{tag}", (nB or N, K), 0.02, dtype="bf16")
    return a, b


def _ref(a, b, rows=None):
    A = synth.bf16_bits_to_f32(a).astype(np.float64)
    B = synth.bf16_bits_to_f32(b).astype(np.float64)
    if rows is not None:
        A = A[rows]
    return A @ B.T


SMALL = [(1, 64, 64), (37, 100, 128), (300, 520, 256), (64, 256, 64), (513, 300, 192),
         (1000, 1032, 256), (700, 768, 768), (600, 280, 64), (530, 300, 128)]


@pytest.mark.parametrize("M,N,K", SMALL)
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_gemm_small(M, N, K, epi):
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm", M, N, K, epi)
    a, b = _inputs(M, N, K, f"{M}.{N}.{K}")
    ref = _ref(a, b)
    A, B = dev(a, torch), dev(b, torch)
    if epi == 0:
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        R = None
    else:
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        R = None
        if epi == 2:
            r = synth.normal(synth.SEED_X, f"gemmR{M}", (M, N), 1.0)
            C.copy_(dev(r, torch))
            R = C
            ref = ref + r
    L.loop_op_gemm(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, R.data_ptr() if R is not None else 0,
                   M, N, K, epi, stream(torch))
    torch.cuda.synchronize()
    got = host(C)
    tol = 2 ** -8 if epi == 0 else 1e-5
    assert rel_err(got, ref) < tol


@pytest.mark.parametrize("M,F,K", [(5, 64, 64), (300, 96, 256), (1000, 768, 256), (513, 200, 128)])
def test_gemm_swiglu(M, F, K):
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm swiglu", M, F, K)
    a, b = _inputs(M, F, K, f"sw{M}.{F}", nB=2 * F)
    gu = _ref(a, b)
    g, u = gu[:, :F], gu[:, F:]
    ref = g / (1 + np.exp(-g)) * u
    C = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    A, B = dev(a, torch), dev(b, torch)   # keep the device buffers alive across the call
    L.loop_op_gemm(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), F, 0, M, F, K, 3, stream(torch))
    torch.cuda.synchronize()
    assert rel_err(host(C), ref) < 2 ** -7


# The projection shapes of one layer execution at full width, prefill of 8192
# tokens: full-attention in-proj, GDN in-proj, attention O, GDN O, gate/up,
# down.  Rows are sampled (the host product of all 8192 rows is not needed).
REAL = [(8192, 10240, 4096, 0), (8192, 8224, 4096, 0), (8192, 4096, 4096, 1),
        (8192, 4096, 2048, 2), (8192, 12288, 4096, 3), (8192, 4096, 12288, 2), (64, 4096, 12288, 1)]


@pytest.mark.parametrize("M,N,K,epi", REAL)
def test_gemm_real_shapes_sampled(M, N, K, epi):
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm real", M, N, K, epi)
    nB = 2 * N if epi == 3 else N
    a, b = _inputs(M, N, K, f"real{N}.{K}", nB=nB)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, M - 1],
                                     np.random.default_rng(0).integers(0, M, 24)]))
    rows = rows[rows < M]
    gu = _ref(a, b, rows)
    C = torch.empty((M, N), dtype=torch.bfloat16 if epi in (0, 3) else torch.float32, device="cuda")
    R = None
    if epi == 2:
        r = synth.normal(synth.SEED_X, f"gemmRreal{N}", (M, N), 1.0)
        C.copy_(dev(r, torch))
        R = C
        gu = gu + r[rows]
    A, B = dev(a, torch), dev(b, torch)
    ws = torch.empty(16 * M * 128, dtype=torch.float32, device="cuda")   # as the model passes one
    L.loop_op_gemm(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N,
                   R.data_ptr() if R is not None else 0, M, N, K, epi, stream(torch), ws.data_ptr(), ws.numel() * 4)
    torch.cuda.synchronize()
    got = host(C)[rows]
    if epi == 3:
        g, u = gu[:, :N], gu[:, N:]
        ref = g / (1 + np.exp(-g)) * u
        assert rel_err(got, ref) < 2 ** -7
    else:
        assert rel_err(got, gu) < (2 ** -8 if epi == 0 else 1e-5)


# The decode projections (up to 64 sequences: weight-streaming tiles, split K
# with fp32 partials summed in split order where the row tiles alone do not
# fill the chip, and the persistent stream over (tile, K step) units with its
# in-order partial fixup for gate/up at 1, 37 and 64 rows and a wider SwiGLU
# and a plain product with enough units), against the float64 product; also
# bit-identical reruns.  The large-M shapes with a narrow column remainder run
# that strip split-K.
DECODE = [(64, 10240, 4096, 0), (64, 8224, 4096, 0), (64, 4096, 4096, 2), (64, 4096, 2048, 1),
          (64, 12288, 4096, 3), (1, 12288, 4096, 3), (37, 12288, 4096, 3), (64, 8192, 4160, 3),
          (5, 24576, 3072, 0), (64, 4096, 12288, 2), (1, 4096, 12288, 2), (37, 520, 768, 3),
          (1024, 288, 1024, 0), (1024, 288, 1024, 2), (600, 1032, 512, 1),
          (17, 1000, 256, 1), (64, 300, 1280, 0), (50, 4100, 1024, 2), (3, 40, 512, 3),
          (50, 4000, 1024, 2), (17, 1000, 2048, 3)]


@pytest.mark.parametrize("M,N,K,epi", DECODE)
def test_gemm_split_k(M, N, K, epi):
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm split-k", M, N, K, epi)
    nB = 2 * N if epi == 3 else N
    a, b = _inputs(M, N, K, f"sk{N}.{K}", nB=nB)
    ref = _ref(a, b)
    A, B = dev(a, torch), dev(b, torch)
    ws = torch.empty(16 * M * 2 * N, dtype=torch.float32, device="cuda")
    outs = []
    for rep in range(2):
        C = torch.zeros((M, N), dtype=torch.bfloat16 if epi in (0, 3) else torch.float32, device="cuda")
        R = None
        if epi == 2:
            r = synth.normal(synth.SEED_X, f"gemmRsk{N}", (M, N), 1.0)
            C.copy_(dev(r, torch))
            R = C
        L.loop_op_gemm(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, R.data_ptr() if R is not None else 0,
                       M, N, K, epi, stream(torch), ws.data_ptr(), ws.numel() * 4)
        torch.cuda.synchronize()
        outs.append(host(C))
    assert np.array_equal(outs[0], outs[1])
    got = outs[0]
    if epi == 3:
        g, u = ref[:, :N], ref[:, N:]
        assert rel_err(got, g / (1 + np.exp(-g)) * u) < 2 ** -7
    elif epi == 2:
        assert rel_err(got, ref + r) < 1e-5
    else:
        assert rel_err(got, ref) < (2 ** -8 if epi == 0 else 1e-5)


@pytest.mark.parametrize("M,N,K,epi", [(1, 66000, 512, 1), (13, 65600, 1024, 1), (3, 70000, 512, 0)])
def test_gemm_wide_few_rows(M, N, K, epi):
    """Very wide products at few rows (the LM head at small batch, a ragged
    last column tile) on the weight-streaming tiles, against float64."""
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm wide", M, N, K, epi)
    a, b = _inputs(M, N, K, f"wide{M}.{N}.{K}")
    ref = _ref(a, b)
    A, B = dev(a, torch), dev(b, torch)
    C = torch.empty((M, N), dtype=torch.bfloat16 if epi == 0 else torch.float32, device="cuda")
    L.loop_op_gemm(A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, 0, M, N, K, epi, stream(torch))
    torch.cuda.synchronize()
    assert rel_err(host(C), ref) < (2 ** -8 if epi == 0 else 1e-5)
