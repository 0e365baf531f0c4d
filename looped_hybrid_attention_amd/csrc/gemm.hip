// bf16 MFMA GEMM for the projections of the layer:
//   C[M,N] = A[M,K] . B[N,K]^T, fp32 accumulation, fused epilogues
//   (bf16 store, fp32 store, fp32 residual add, SwiGLU of paired gate/up).
// The projections are the SwiGLU FFN and the attention / Gated-DeltaNet
// input and output projections of every layer execution ([P1 section 2]:
// three FFN matrices plus the attention projections per layer).
//
// Tiling: a BM x BN output tile per workgroup, K in steps of 64 staged
// through LDS (double-buffered, one barrier per step), the next step's global
// loads in flight during the MFMAs of the current one.  WM x WN waves, each
// computing (BM/WM) x (BN/WN) with v_mfma_f32_32x32x16_bf16.  LDS rows are
// padded by 16 bytes so the 16-byte operand reads of 32 consecutive rows hit
// distinct banks.
#include "common.h"
#include "launch.h"

namespace {

constexpr int BK = 64;
constexpr int LDSK = BK + 8;  // padded row length in bf16

struct GemmArgs {
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  void* C; int64_t ldc;
  const float* R;
  int M, N, K;   // N = output columns
  int swiglu_F;  // SwiGLU: offset of the up rows in B (= N)
};

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 32;  // 32x32 tiles per wave along M
  constexpr int TN = BN / WN / 32;  // along N (B-tile rows)
  constexpr int A_CHUNKS = BM * BK / 8 / NT;  // 16-byte chunks per thread
  constexpr int B_CHUNKS = BN * BK / 8 / NT;
  static_assert(A_CHUNKS * NT * 8 == BM * BK && B_CHUNKS * NT * 8 == BN * BK, "tile/thread split");
  static_assert(EPI != LOOP_EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs gate/up tiles");

  extern __shared__ __align__(16) uint16_t gemm_smem[];
  // Buffer b: A tile at b*STAGE, B tile right after it.
  constexpr int STAGE = (BM + BN) * LDSK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;

  // Output-tile coordinates.  Consecutive workgroups walk down M first inside
  // a band of N tiles so that concurrently running workgroups share B tiles
  // in L2.
  const int tiles_m = (g.M + BM - 1) / BM;
  const int m0 = (blockIdx.x % tiles_m) * BM;
  const int tn = blockIdx.x / tiles_m;
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? BN / 2 : BN;
  const int n0 = tn * OUT_BN;  // first output column

  // Global source rows of this thread's chunks.
  const uint16_t* a_src[A_CHUNKS];
  bool a_ok[A_CHUNKS];
  int a_lds[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    int c = tid + i * NT, r = c / (BK / 8), kc = c % (BK / 8);
    int gm = m0 + r;
    a_ok[i] = gm < g.M;
    a_src[i] = g.A + (int64_t)(a_ok[i] ? gm : 0) * g.lda + kc * 8;
    a_lds[i] = r * LDSK + kc * 8;
  }
  const uint16_t* b_src[B_CHUNKS];
  bool b_ok[B_CHUNKS];
  int b_lds[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    int c = tid + i * NT, r = c / (BK / 8), kc = c % (BK / 8);
    int gn;
    bool ok;
    if (EPI == LOOP_EPI_SWIGLU) {
      // B-tile rows come in 32-row blocks alternating gate / up of the same
      // output columns.
      int blk = r / 32, part = blk & 1, col = n0 + (blk >> 1) * 32 + (r & 31);
      ok = col < g.N;
      gn = part * g.swiglu_F + col;
    } else {
      gn = n0 + r;
      ok = gn < g.N;
    }
    b_ok[i] = ok;
    b_src[i] = g.B + (int64_t)(ok ? gn : 0) * g.ldb + kc * 8;
    b_lds[i] = r * LDSK + kc * 8;
  }

  uint4 ra[A_CHUNKS], rb[B_CHUNKS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
      if (!a_ok[i]) ra[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
      if (!b_ok[i]) rb[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<uint4*>(gemm_smem + buf * STAGE + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<uint4*>(gemm_smem + buf * STAGE + BM * LDSK + b_lds[i]) = rb[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  const int nk = g.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t* a_base = gemm_smem + cur * STAGE + (wm * (BM / WM) + lr) * LDSK + lk;
    const uint16_t* b_base = gemm_smem + cur * STAGE + BM * LDSK + (wn * (BN / WN) + lr) * LDSK + lk;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_base + i * 32 * LDSK + ks * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(b_base + j * 32 * LDSK + ks * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Lane holds column lr of each 32x32 tile and rows
  // 8*(r/4) + 4*(lane/32) + r%4.
  const int row_base = m0 + wm * (BM / WM) + 4 * (lane >> 5);
  if (EPI == LOOP_EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int col = n0 + (wn * (BN / WN)) / 2 + (j / 2) * 32 + lr;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
          if (row < g.M) {
            float gt = acc[i][j][r], up = acc[i][j + 1][r];
            reinterpret_cast<uint16_t*>(g.C)[(int64_t)row * g.ldc + col] = f2bf_bits(siluf_(gt) * up);
          }
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * (BN / WN) + j * 32 + lr;
    if (col >= g.N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= g.M) continue;
        const int64_t o = (int64_t)row * g.ldc + col;
        float v = acc[i][j][r];
        if (EPI == LOOP_EPI_BF16) {
          reinterpret_cast<uint16_t*>(g.C)[o] = f2bf_bits(v);
        } else if (EPI == LOOP_EPI_F32) {
          reinterpret_cast<float*>(g.C)[o] = v;
        } else {
          reinterpret_cast<float*>(g.C)[o] = g.R[o] + v;
        }
      }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + OUT_BN - 1) / OUT_BN);
  const size_t lds = 2 * (size_t)(BM + BN) * LDSK * sizeof(uint16_t);
  auto k = gemm_kernel<BM, BN, WM, WN, EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k, dim3(tiles), dim3(WM * WN * 64), lds, s, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& g, hipStream_t s) {
  if (g.M >= 512) return launch_cfg<256, 256, 2, 2, EPI>(g, s);
  return launch_cfg<64, 128, 2, 2, EPI>(g, s);
}

}  // namespace

hipError_t launch_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int M, int N, int K, int epi, hipStream_t s) {
  GemmArgs g{(const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc, R, M, N, K, N};
  switch (epi) {
    case LOOP_EPI_BF16: return launch_epi<LOOP_EPI_BF16>(g, s);
    case LOOP_EPI_F32: return launch_epi<LOOP_EPI_F32>(g, s);
    case LOOP_EPI_F32_RES: return launch_epi<LOOP_EPI_F32_RES>(g, s);
    case LOOP_EPI_SWIGLU: return launch_epi<LOOP_EPI_SWIGLU>(g, s);
  }
  return hipErrorInvalidValue;
}
