"""Weight-only int8 / int4 GEMM (the decode projections' kernels, through
loop_op_gemm_quant) against the float64 product of the oracle's dequantized
weights: the codes come from the device quantizer (checked equal to the
oracle's here too), the reference from oracle.quant's codes of the same bf16
matrix.  M in {1, 17, 37, 64} reaches the 1, 2 and 4 activation-tile
variants with ragged rows; every epilogue; K up to 1024 with split K.
Bars: fp32 outputs 1e-5 (exact products, fp32 sums), bf16 outputs 2^-8,
SwiGLU 2^-7 (max |gpu - ref| / max |ref|)."""
import numpy as np
import pytest

import synth
from oracle import quant as oq
from gpu_util import torch_cuda, dev, host, stream, say, rel_err

pytestmark = pytest.mark.gpu

SHAPES = [(300, 512, 1), (520, 1024, 2), (200, 256, 0), (96, 384, 3)]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [1, 17, 37, 64])
@pytest.mark.parametrize("N,K,epi", SHAPES)
def test_quantized_gemm_matches_dequantized_product(bits, M, N, K, epi):
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    say("gemm quant", bits, M, N, K, epi)
    NB = 2 * N if epi == 3 else N
    tag = f"q{bits}.{N}.{K}"
    a = synth.normal(synth.SEED_X, f"gemmqA{M}.{K}", (M, K), 1.0, dtype="bf16")
    w = synth.normal(synth.SEED_W, f"gemmqB{tag}", (NB, K), 0.02, dtype="bf16")
    wf = synth.bf16_bits_to_f32(w)
    s = stream(torch)
    W = dev(w, torch)
    if bits == 8:
        q_ref, s_ref = oq.quantize_rows_int8(wf)
        Wd = oq.dequantize_rows(q_ref, s_ref, np.float64)
        Q = torch.empty((NB, K), dtype=torch.int8, device="cuda")
        S = torch.empty(NB, dtype=torch.float32, device="cuda")
        L.loop_quantize_int8(W.data_ptr(), NB, K, K, Q.data_ptr(), S.data_ptr(), s)
        ldq = K
    else:
        q_ref, s_ref = oq.quantize_groups_int4(wf)
        Wd = oq.dequantize_groups_int4(q_ref, s_ref).astype(np.float64)
        Q = torch.empty((NB, K // 2), dtype=torch.uint8, device="cuda")
        S = torch.empty((NB, K // 128), dtype=torch.float32, device="cuda")
        L.loop_quantize_int4(W.data_ptr(), NB, K, K, Q.data_ptr(), S.data_ptr(), s)
        ldq = K // 2
    torch.cuda.synchronize()
    q_gpu = host(Q)
    assert np.array_equal(q_gpu if bits == 8 else oq.unpack_int4(q_gpu), q_ref)
    assert np.array_equal(host(S), s_ref)
    ref = synth.bf16_bits_to_f32(a).astype(np.float64) @ Wd.T
    A = dev(a, torch)
    if epi in (0, 3):
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    else:
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    R = 0
    if epi == 2:
        r = synth.normal(synth.SEED_X, f"gemmqR{M}.{N}", (M, N), 1.0)
        C.copy_(dev(r, torch))
        R = C.data_ptr()
        ref = ref + r
    if epi == 3:
        g, u = ref[:, :N], ref[:, N:]
        ref = g / (1 + np.exp(-g)) * u
    ws = torch.empty(64 * M * NB, dtype=torch.float32, device="cuda")
    L.loop_op_gemm_quant(bits, A.data_ptr(), K, Q.data_ptr(), ldq, S.data_ptr(), C.data_ptr(), N, R, M, N, K, epi,
                         s, ws.data_ptr(), ws.numel() * 4)
    torch.cuda.synchronize()
    err = rel_err(host(C), ref)
    tol = {0: 2 ** -8, 1: 1e-5, 2: 1e-5, 3: 2 ** -7}[epi]
    say(f"int{bits} M {M} N {N} K {K} epi {epi}: {err:.2e} (bar {tol:.1e})")
    assert err < tol


def test_quantized_gemm_rejects_bad_arguments():
    import looped_hybrid_attention_amd as L
    torch = torch_cuda()
    A = torch.zeros((65, 256), dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros((64, 256), dtype=torch.int8, device="cuda")
    S = torch.zeros(64, dtype=torch.float32, device="cuda")
    C = torch.zeros((65, 64), dtype=torch.float32, device="cuda")
    for bits, M, K, ldq, code in ((8, 65, 256, 256, -2), (8, 4, 200, 256, -2), (3, 4, 256, 256, -1),
                                  (8, 4, 256, 200, -2), (4, 4, 256, 64, -2)):
        with pytest.raises(L.LoopError) as e:
            L.loop_op_gemm_quant(bits, A.data_ptr(), 256, Q.data_ptr(), ldq, S.data_ptr(), C.data_ptr(), 64, 0,
                                 M, 64, K, 1)
        assert e.value.code == code, (bits, M, K, ldq)
