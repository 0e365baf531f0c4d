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

#include <algorithm>
#include <type_traits>

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
  float* part;   // split-K: fp32 partials [splits][M][N] ([splits][M][2][N] for SwiGLU)
  int kslice;    // split-K: K per split (blockIdx.y)
  const float* scale = nullptr;  // int8 weights: per-row scale (B is int8 [rows][ldb]);
                                 // int4: [rows][K / 128] group scales (B packed, ldb bytes)
  uint32_t scale_bytes = 0;      // int4: bytes of the scale array
};

template <int BM, int BN, int WM, int WN, int EPI, bool SPLIT>
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

  // Global source offsets (elements, 32-bit) of this thread's chunks from
  // the tile's row base.  Rows past M (or N) are clamped to a valid row: they
  // only feed output rows (columns) that are never stored.
  int a_off[A_CHUNKS], a_lds[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * NT, r = c / (BK / 8), kc = c % (BK / 8);
    a_off[i] = min(m0 + r, g.M - 1) * (int)g.lda + kc * 8;
    a_lds[i] = r * LDSK + kc * 8;
  }
  int b_off[B_CHUNKS], b_lds[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * NT, r = c / (BK / 8), kc = c % (BK / 8);
    int gn;
    if (EPI == LOOP_EPI_SWIGLU) {
      // B-tile rows come in 32-row blocks alternating gate / up of the same
      // output columns.
      const int blk = r / 32, part = blk & 1, col = min(n0 + (blk >> 1) * 32 + (r & 31), g.N - 1);
      gn = part * g.swiglu_F + col;
    } else {
      gn = min(n0 + r, g.N - 1);
    }
    b_off[i] = gn * (int)g.ldb + kc * 8;
    b_lds[i] = (BM + r) * LDSK + kc * 8;
  }
  // split-K: this workgroup's K range starts at blockIdx.y * kslice
  const uint16_t* Ak = g.A + (SPLIT ? blockIdx.y * g.kslice : 0);
  const uint16_t* Bk = g.B + (SPLIT ? blockIdx.y * g.kslice : 0);

  u32x4 ra[A_CHUNKS], rb[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(Ak + a_off[i]);
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(Bk + b_off[i]);
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(gemm_smem + a_lds[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(gemm_smem + b_lds[i]) = rb[i];

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  const int nk = (SPLIT ? g.kslice : g.K) / BK;
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int a_frag = (wm * (BM / WM) + lr) * LDSK + lk;
  const int b_frag = (BM + wn * (BN / WN) + lr) * LDSK + lk;
  __syncthreads();
  // One basic block per k-step: the next tile's global loads (the last step
  // re-reads its own tile, harmlessly), the MFMAs of the four 16-deep steps
  // with the next step's LDS fragments interleaved, then the next tile into
  // the other LDS buffer.
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* S = gemm_smem + (kt & 1) * STAGE;
    const int kn = min(kt + 1, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(Ak + kn + a_off[i]);
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(Bk + kn + b_off[i]);
    bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(S + a_frag + i * 32 * LDSK);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8*>(S + b_frag + j * 32 * LDSK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[nxt][i] = *reinterpret_cast<const bf16x8*>(S + a_frag + i * 32 * LDSK + (ks + 1) * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[nxt][j] = *reinterpret_cast<const bf16x8*>(S + b_frag + j * 32 * LDSK + (ks + 1) * 16);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32x32x16(af[cur][i], bfr[cur][j], acc[i][j]);
    }
    uint16_t* D = gemm_smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(D + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(D + b_lds[i]) = rb[i];
    // schedule: global loads first, first fragments, then for each of the
    // first three 16-deep steps its MFMAs interleaved with the next step's
    // fragment reads, the last step's MFMAs, the LDS stores.
    __builtin_amdgcn_sched_group_barrier(0x020, A_CHUNKS + B_CHUNKS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16 - 1; ++ks) {
#pragma unroll
      for (int f = 0; f < TM + TN; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN / (TM + TN) > 0 ? TM * TN / (TM + TN) : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, A_CHUNKS + B_CHUNKS, 0);
    __syncthreads();
  }

  // Epilogue.  Lane holds column lr of each 32x32 tile and rows
  // 8*(r/4) + 4*(lane/32) + r%4.
  const int row_base = m0 + wm * (BM / WM) + 4 * (lane >> 5);
  if (SPLIT) {
    // raw fp32 partials; SwiGLU keeps gate and up apart
    float* P = g.part + (int64_t)blockIdx.y * g.M * (EPI == LOOP_EPI_SWIGLU ? 2 * g.N : g.N);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int col, part = 0;
      if (EPI == LOOP_EPI_SWIGLU) {
        col = n0 + (wn * (BN / WN)) / 2 + (j / 2) * 32 + lr;
        part = j & 1;
      } else {
        col = n0 + wn * (BN / WN) + j * 32 + lr;
      }
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
          if (row >= g.M) continue;
          if (EPI == LOOP_EPI_SWIGLU) P[((int64_t)row * 2 + part) * g.N + col] = acc[i][j][r];
          else P[(int64_t)row * g.N + col] = acc[i][j][r];
        }
    }
    return;
  }
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

// Sum of the split-K partials in split order, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int splits) {
  const int64_t n_out = (int64_t)g.M * g.N;
  const int64_t stride = (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * n_out;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n_out; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / g.N, col = i % g.N;
    if (EPI == LOOP_EPI_SWIGLU) {
      float gt = 0.f, up = 0.f;
      for (int sp = 0; sp < splits; ++sp) {
        gt += g.part[sp * stride + (row * 2) * g.N + col];
        up += g.part[sp * stride + (row * 2 + 1) * g.N + col];
      }
      reinterpret_cast<uint16_t*>(g.C)[row * g.ldc + col] = f2bf_bits(siluf_(gt) * up);
    } else {
      float v = 0.f;
      for (int sp = 0; sp < splits; ++sp) v += g.part[sp * stride + i];
      const int64_t o = row * g.ldc + col;
      if (EPI == LOOP_EPI_BF16) reinterpret_cast<uint16_t*>(g.C)[o] = f2bf_bits(v);
      else if (EPI == LOOP_EPI_F32) reinterpret_cast<float*>(g.C)[o] = v;
      else reinterpret_cast<float*>(g.C)[o] = g.R[o] + v;
    }
  }
}

// Split-K sum fused with the next pre-norm (rows of a decode call): per row
// m, C = sum of the partials in split order (+ R), then
// hn = bf16(RMSNorm(C + X2; gain)) with X2 the loop input x, or none.
// One row per workgroup of 1024 threads, PER columns (4 apart by 1024) per
// thread; the split partials are summed in split order (SPL splits).
template <int EPI, int PER, int SPL>
__global__ __launch_bounds__(1024) void splitk_reduce_norm_kernel(GemmArgs g, const float* X2, const uint16_t* gain,
                                                                  uint16_t* hn, float eps) {
  static_assert(EPI == LOOP_EPI_F32 || EPI == LOOP_EPI_F32_RES, "fp32 output");
  __shared__ float red[16];
  const int64_t m = blockIdx.x;
  float pv[PER][SPL], rx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = min((int)threadIdx.x + 1024 * i, g.N - 1);
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) pv[i][sp] = g.part[((int64_t)sp * g.M + m) * g.N + c];
    const int64_t o = m * g.ldc + c;
    rx[i] = (EPI == LOOP_EPI_F32_RES ? g.R[o] : 0.f) + (X2 ? X2[o] : 0.f);
  }
  float y[PER];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + 1024 * i;
    float v = 0.f;
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) v += pv[i][sp];
    const int64_t o = m * g.ldc + c;
    float yv = 0.f;
    if (c < g.N) {
      // plain: C = R + v (and the norm input is C); loop: C = v, input C + X2
      const float cv = EPI == LOOP_EPI_F32_RES ? g.R[o] + v : v;
      reinterpret_cast<float*>(g.C)[o] = cv;
      yv = EPI == LOOP_EPI_F32_RES ? cv : v + rx[i];
    }
    y[i] = yv;
    ss += yv * yv;
  }
  ss = block_sum<1024>(ss, red);
  const float inv = rsqrtf(ss / g.N + eps);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + 1024 * i;
    if (c < g.N) hn[m * g.N + c] = f2bf_bits(y[i] * inv * bf2f(gain[c]));
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool SPLIT>
hipError_t launch_cfg(const GemmArgs& g, int splits, hipStream_t s) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? BN / 2 : BN;
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + OUT_BN - 1) / OUT_BN);
  const size_t lds = 2 * (size_t)(BM + BN) * LDSK * sizeof(uint16_t);
  auto k = gemm_kernel<BM, BN, WM, WN, EPI, SPLIT>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k, dim3(tiles, SPLIT ? splits : 1), dim3(WM * WN * 64), lds, s, g);
  if (SPLIT) {
    const int64_t n_out = (int64_t)g.M * g.N;
    const int blocks = (int)std::min<int64_t>((n_out + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(blocks), dim3(256), 0, s, g, splits);
  }
  return hipGetLastError();
}


// ------------------------------------------------- small M, stream over K
// Rows M <= 64 (decode): the output's 64 x 128 tiles (SwiGLU: 64 output
// columns, gate and up rows in alternating 32-row blocks) times the 64-deep
// K steps make U = tiles * nk units of equal work.  A persistent grid of P
// workgroups (two per CU) takes contiguous ranges [w U / P, (w + 1) U / P),
// so every workgroup streams the same number of weight bytes, and the
// register-staged loads run ST_PF units ahead straight across tile
// boundaries (no refill between tiles).  At the end of a tile (or of its
// range) a workgroup writes its fp32 partial sum into slot
// w - (first workgroup of the tile); stream_fixup_kernel adds a tile's slots
// in slot order (= K order) and applies the epilogue.  The partition depends
// on N, K and P only, so a row's result does not depend on M.
constexpr int ST_PF = 3;
DEV int stream_wg_of(int64_t u, int64_t U, int P) { return (int)(((u + 1) * P - 1) / U); }

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(GemmArgs g, int P) {
  constexpr int BM = 64, BN = 128, WN = 2, NT = 256, TM = 1, TN = 2, PF = ST_PF;
  constexpr int A_CHUNKS = BM * BK / 8 / NT;
  constexpr int B_CHUNKS = BN * BK / 8 / NT;
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? BN / 2 : BN;
  constexpr int STAGE = (BM + BN) * LDSK;
  extern __shared__ __align__(16) uint16_t gemm_smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int nk = g.K / BK;
  const int tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int64_t U = (int64_t)tiles * nk;
  const int w = blockIdx.x;
  // U >= P (the launcher's condition): every workgroup owns at least one
  // unit, so a tile's slots run without gaps from its first workgroup to its
  // last
  const int64_t u0 = (int64_t)w * U / P, u1 = (int64_t)(w + 1) * U / P;

  // this thread's 16-byte chunks: A rows (all of M, clamped), B rows of the
  // tile (row r, K chunk kc); the tile and the K step set the base
  int a_off[A_CHUNKS], a_lds[A_CHUNKS], b_r[B_CHUNKS], b_kc[B_CHUNKS], b_lds[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * NT, r = c / (BK / 8), kc = c % (BK / 8);
    a_off[i] = min(r, g.M - 1) * (int)g.lda + kc * 8;
    a_lds[i] = r * LDSK + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * NT;
    b_r[i] = c / (BK / 8);
    b_kc[i] = c % (BK / 8);
    b_lds[i] = (BM + b_r[i]) * LDSK + b_kc[i] * 8;
  }
  auto b_offset = [&](int i, int t, int ks) {
    const int r = b_r[i];
    int gn;
    if (EPI == LOOP_EPI_SWIGLU) {
      const int blk = r / 32;
      gn = (blk & 1) * g.swiglu_F + min(t * OUT_BN + (blk >> 1) * 32 + (r & 31), g.N - 1);
    } else {
      gn = min(t * OUT_BN + r, g.N - 1);
    }
    return gn * (int)g.ldb + ks * BK + b_kc[i] * 8;
  };
  u32x4 ra[PF][A_CHUNKS], rb[PF][B_CHUNKS];
  auto load = [&](int64_t u, u32x4 (&a)[A_CHUNKS], u32x4 (&b)[B_CHUNKS]) __attribute__((always_inline)) {
    const int t = (int)(u / nk), ks = (int)(u % nk);
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) a[i] = *reinterpret_cast<const u32x4*>(g.A + ks * BK + a_off[i]);
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) b[i] = *reinterpret_cast<const u32x4*>(g.B + b_offset(i, t, ks));
  };
  // unit u0 straight into LDS buffer 0; units u0 + 1 .. u0 + PF - 1 into the
  // register sets 0 .. PF - 2 (set of local unit j: (j - 1) % PF)
  {
    u32x4 a0[A_CHUNKS], b0[B_CHUNKS];
    load(u0, a0, b0);
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p) load(min(u0 + 1 + p, u1 - 1), ra[p], rb[p]);
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(gemm_smem + a_lds[i]) = a0[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(gemm_smem + b_lds[i]) = b0[i];
  }
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int a_frag = (wm * (BM / 2) + lr) * LDSK + lk;
  const int b_frag = (BM + wn * (BN / WN) + lr) * LDSK + lk;
  const int64_t pstride = (int64_t)(EPI == LOOP_EPI_SWIGLU ? 2 : 1) * g.M * g.N;
  __syncthreads();
  for (int64_t ub = u0; ub < u1; ub += PF) {
#pragma unroll
    for (int jp = 0; jp < PF; ++jp) {
      const int64_t u = ub + jp;
      if (u >= u1) break;
      const int j = (int)(u - u0);
      const int ld_set = (jp + PF - 1) % PF;
      load(min(u + PF, u1 - 1), ra[ld_set], rb[ld_set]);
      const uint16_t* S = gemm_smem + (j & 1) * STAGE;
      bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(S + a_frag + i * 32 * LDSK);
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) bfr[0][jj] = *reinterpret_cast<const bf16x8*>(S + b_frag + jj * 32 * LDSK);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        if (ks + 1 < BK / 16) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
            af[nxt][i] = *reinterpret_cast<const bf16x8*>(S + a_frag + i * 32 * LDSK + (ks + 1) * 16);
#pragma unroll
          for (int jj = 0; jj < TN; ++jj)
            bfr[nxt][jj] = *reinterpret_cast<const bf16x8*>(S + b_frag + jj * 32 * LDSK + (ks + 1) * 16);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int jj = 0; jj < TN; ++jj) acc[i][jj] = mfma32x32x16(af[cur][i], bfr[cur][jj], acc[i][jj]);
      }
      uint16_t* D = gemm_smem + ((j + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(D + a_lds[i]) = ra[jp][i];
#pragma unroll
      for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<u32x4*>(D + b_lds[i]) = rb[jp][i];
      if ((u + 1) % nk == 0 || u + 1 == u1) {
        // the workgroup's part of this tile: fp32 partials into its slot
        const int t = (int)(u / nk);
        const int slot = w - stream_wg_of((int64_t)t * nk, U, P);
        float* Pp = g.part + slot * pstride;
        const int row_base = wm * (BM / 2) + 4 * (lane >> 5);
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
          int col, part = 0;
          if (EPI == LOOP_EPI_SWIGLU) {
            col = t * OUT_BN + (wn * (BN / WN)) / 2 + (jj / 2) * 32 + lr;
            part = jj & 1;
          } else {
            col = t * OUT_BN + wn * (BN / WN) + jj * 32 + lr;
          }
          if (col < g.N) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
                if (row >= g.M) continue;
                if (EPI == LOOP_EPI_SWIGLU) Pp[((int64_t)row * 2 + part) * g.N + col] = acc[i][jj][r];
                else Pp[(int64_t)row * g.N + col] = acc[i][jj][r];
              }
          }
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[i][jj] = (f32x16){};
        }
      }
      __syncthreads();
    }
  }
}

// Sum of each tile's stream partials in slot order, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void stream_fixup_kernel(GemmArgs g, int P) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? 64 : 128;
  const int nk = g.K / BK;
  const int64_t U = (int64_t)((g.N + OUT_BN - 1) / OUT_BN) * nk;
  const int64_t n_out = (int64_t)g.M * g.N;
  const int64_t stride = (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * n_out;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n_out; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / g.N, col = i % g.N;
    const int t = (int)(col / OUT_BN);
    const int segs = stream_wg_of((int64_t)(t + 1) * nk - 1, U, P) - stream_wg_of((int64_t)t * nk, U, P) + 1;
    if (EPI == LOOP_EPI_SWIGLU) {
      float gt = 0.f, up = 0.f;
      for (int sp = 0; sp < segs; ++sp) {
        gt += g.part[sp * stride + (row * 2) * g.N + col];
        up += g.part[sp * stride + (row * 2 + 1) * g.N + col];
      }
      reinterpret_cast<uint16_t*>(g.C)[row * g.ldc + col] = f2bf_bits(siluf_(gt) * up);
    } else {
      float v = 0.f;
      for (int sp = 0; sp < segs; ++sp) v += g.part[sp * stride + i];
      const int64_t o = row * g.ldc + col;
      if (EPI == LOOP_EPI_BF16) reinterpret_cast<uint16_t*>(g.C)[o] = f2bf_bits(v);
      else if (EPI == LOOP_EPI_F32) reinterpret_cast<float*>(g.C)[o] = v;
      else reinterpret_cast<float*>(g.C)[o] = g.R[o] + v;
    }
  }
}

// Workgroups of the stream grid: two per CU of the 256-CU part (a fixed
// count, so that the partition, and with it every result, is the same on
// any device, and the workspace size can be computed without one).  Used
// where every workgroup gets at least ST_MIN_UNITS units: measured on the
// decode projections, the stream pays off on gate/up (24 units per
// workgroup: 51.9 against 55.8 us at 64 rows, 41.7 against 48.0 at one row)
// and loses on the input projections (8-10 units: the per-workgroup start and
// the extra partial slots cost more than the balance gains).
constexpr int ST_P = 512;
constexpr int ST_MIN_UNITS = 16;

// Partial bytes of the stream path for this call (0: the call cannot use it).
template <int EPI>
size_t stream_partial_bytes(const GemmArgs& g) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? 64 : 128;
  constexpr int P = ST_P;
  if (g.M < 1 || g.M > 64 || g.K % BK != 0 || g.N < 1 || g.N > 65536) return 0;
  const int nk = g.K / BK, tiles = (g.N + OUT_BN - 1) / OUT_BN;
  const int64_t U = (int64_t)tiles * nk;
  if (U < (int64_t)ST_MIN_UNITS * P || U > (1ll << 30)) return 0;
  const int64_t rows_b = (EPI == LOOP_EPI_SWIGLU) ? 2 * (int64_t)g.N : g.N;
  if (rows_b * g.ldb >= (1ll << 31) || (int64_t)g.M * g.lda >= (1ll << 31)) return 0;
  int max_segs = 1;
  for (int t = 0; t < tiles; ++t) {
    const int64_t a = (int64_t)t * nk, b = (int64_t)(t + 1) * nk - 1;
    const int segs = (int)(((b + 1) * P - 1) / U) - (int)(((a + 1) * P - 1) / U) + 1;
    max_segs = std::max(max_segs, segs);
  }
  return (size_t)max_segs * g.M * g.N * (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * sizeof(float);
}

template <int EPI>
hipError_t launch_stream(const GemmArgs& g, hipStream_t s) {
  constexpr int P = ST_P;
  constexpr size_t lds = 2 * (size_t)(64 + 128) * LDSK * sizeof(uint16_t);
  auto k = gemm_stream_kernel<EPI>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k, dim3(P), dim3(256), lds, s, g, P);
  const int64_t n_out = (int64_t)g.M * g.N;
  const int blocks = (int)std::min<int64_t>((n_out + 255) / 256, 4096);
  hipLaunchKernelGGL(stream_fixup_kernel<EPI>, dim3(blocks), dim3(256), 0, s, g, P);
  return hipGetLastError();
}

// ------------------------------------------------- large-M tiles, LDS copy
// 256 x 256 output tiles, K in steps of KB, four waves (one per SIMD), each
// computing 128 x 128 as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 with the
// accumulators in AGPRs.  The grid is persistent (one workgroup per CU, tiles
// blockIdx.x, + gridDim.x, ...) and the copy pipeline runs on across tiles:
// A and B go global -> LDS with buffer_load ... lds through two stages, the
// copies of step t + 1 issued at the top of step t, and the last step of a
// tile copies the first step of the workgroup's next tile, so that copy is in
// flight while the epilogue stores.  The barrier that publishes step t + 1
// sits before the MFMAs of step t's last 16-deep slice, so the next step's
// first operand reads overlap them.  Operand reads run one 16-deep slice
// ahead of the MFMAs.  Rows are unpadded (KB * 2 bytes); 16-byte chunk c of
// row r sits at c ^ swz(r), which puts the 128-bit operand reads of 16
// consecutive rows on distinct banks.
//
// The MFMA takes the B rows (output columns) as its first operand, so lane
// (lr, h) of a 32 x 32 tile holds output row lr and, for each q = 0..3, the
// four consecutive columns 8 q + 4 h .. + 3: the epilogue stores (and, for
// the residual, loads) 8 or 16 bytes per lane.
template <int KB, int NW>
struct DbShape {
  static constexpr int ROW = KB * 2;               // bytes of one operand row
  static constexpr int CPR = ROW / 16;             // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROW;           // rows per 1 KB copy instruction
  static constexpr int CPW = 256 / RPI / NW;       // copy instructions per wave per operand
  static constexpr int TILE = 256 * ROW;           // bytes of one operand tile
  static constexpr int STAGE = 2 * TILE;           // A then B
  static DEV int swz(int row) { return (row / (16 / CPR)) % CPR; }
};
constexpr int DB_BM = 256, DB_BN = 256;
constexpr int db_lds(int kb) { return 2 * 2 * 256 * kb * 2; }

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// four fp32 -> four bf16 (round to nearest even) as 8 bytes
DEV u32x2 pack_bf16x4(float a, float b, float c, float d) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Epilogue of a wave's 128 x (32 TN) block, one 32-row block at a time
// through the wave's own LDS region `ws` (the stage the last K step read):
// lane (lr, half) holds row lr and, for r = 4 q + e, column 32 j + 8 q + 4
// half + e (SwiGLU pairs tiles j (gate) and j + 1 (up) into output column
// 32 (j / 2) + 8 q + e); it writes its values there (16-byte chunks of a row
// XOR-swizzled by the row), then reads the block back row-major, so every
// global access of the wave covers whole rows: 16 bytes per lane, 512 B to
// 1 KB contiguous per row.  The residual is loaded the same way first.
template <int EPI, int TM, int TN>
DEV void db_epilogue(const GemmArgs& g, f32x16 (&acc)[TM][TN], uint8_t* ws, int row0, int col0, int lane) {
  constexpr bool F32 = EPI == LOOP_EPI_F32 || EPI == LOOP_EPI_F32_RES;
  constexpr int OCOLS = EPI == LOOP_EPI_SWIGLU ? 16 * TN : 32 * TN;  // output columns of the wave
  constexpr int RB = OCOLS * (F32 ? 4 : 2);                          // bytes of a block row in LDS
  constexpr int NCH = RB / 16;                                         // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;                                       // rows per wave access
  constexpr int NI = 32 / RPI;                                         // accesses per 32-row block
  static_assert(NCH <= 32 && RPI * RB == 1024, "epilogue block");
  const int lr = lane & 31, half = lane >> 5;
  const int rr = lane / NCH, cc = lane % NCH;  // row-major read back: row rr + RPI k, chunk cc
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t rb = row0 + 32 * i;
    if constexpr (F32) {
      f32x4 rv[NI];
      if constexpr (EPI == LOOP_EPI_F32_RES) {
#pragma unroll
        for (int k = 0; k < NI; ++k)
          rv[k] = *reinterpret_cast<const f32x4*>(g.R + (rb + rr + RPI * k) * g.ldc + col0 + 4 * cc);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * j + 2 * q + half;
          const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(ws + lr * RB + ((c ^ lr) % NCH) * 16) = v;
        }
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int r = rr + RPI * k;
        f32x4 v = *reinterpret_cast<const f32x4*>(ws + r * RB + ((cc ^ r) % NCH) * 16);
        if constexpr (EPI == LOOP_EPI_F32_RES) v += rv[k];
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(g.C) + (rb + r) * g.ldc + col0 + 4 * cc) = v;
      }
    } else {
      // 8-byte pieces c8 (four bf16) of a row: chunk c8 / 2, half c8 % 2
#pragma unroll
      for (int j = 0; j < TN; j += (EPI == LOOP_EPI_SWIGLU ? 2 : 1))
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = EPI == LOOP_EPI_SWIGLU ? siluf_(acc[i][j][4 * q + e]) * acc[i][j + 1][4 * q + e]
                                          : acc[i][j][4 * q + e];
          const int c8 = 8 * (EPI == LOOP_EPI_SWIGLU ? j / 2 : j) + 2 * q + half;
          *reinterpret_cast<u32x2*>(ws + lr * RB + (((c8 >> 1) ^ lr) % NCH) * 16 + (c8 & 1) * 8) =
              pack_bf16x4(o[0], o[1], o[2], o[3]);
        }
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int r = rr + RPI * k;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ws + r * RB + ((cc ^ r) % NCH) * 16);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(g.C) + (rb + r) * g.ldc + col0 + 8 * cc) = v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int EPI, int KB, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_db_kernel(GemmArgs g, uint32_t a_bytes, uint32_t b_bytes, int n_tiles) {
  using S = DbShape<KB, NW>;
  static_assert(KB % 32 == 0 && (NW == 4 || NW == 8), "ring shape");
  // waves: 2 along M (128 rows each) x NW / 2 along N (256 / (NW / 2) B rows)
  constexpr int WN = NW / 2, TM = 4, TN = 8 / WN, KS = KB / 16;
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? DB_BN / 2 : DB_BN;
  extern __shared__ __align__(16) uint8_t db_smem[];
  // the wave index is uniform: kept in an SGPR, LDS copy targets are scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_m = (g.M + DB_BM - 1) / DB_BM;

  // Only whole tiles (M and N multiples of 256 and OUT_BN, ldc a multiple
  // of 4, C and R 16-byte aligned): the launcher sends ragged edges to the
  // small tiles.  A tile's origin is then a scalar byte offset and the
  // per-lane offsets below do not depend on the tile.
  //
  // Per-lane byte offsets of this lane's 16-byte piece in each of the wave's
  // copy instructions per operand tile: instruction n fills rows RPI n ..
  // RPI n + RPI - 1, lane l row RPI n + l / CPR at chunk l % CPR (holding
  // logical chunk (l % CPR) ^ swz).  SwiGLU tiles alternate 32 gate rows and
  // the 32 matching up rows (F rows further on).
  int a_off[S::CPW], b_off[S::CPW];
#pragma unroll
  for (int i = 0; i < S::CPW; ++i) {
    const int row = (wave * S::CPW + i) * S::RPI + lane / S::CPR;
    const int c = (lane % S::CPR) ^ S::swz(row);
    a_off[i] = (row * (int)g.lda + c * 8) * 2;
    int gn = row;
    if (EPI == LOOP_EPI_SWIGLU) {
      const int blk = row / 32;
      gn = (blk & 1) * g.swiglu_F + (blk >> 1) * 32 + (row & 31);
    }
    b_off[i] = (gn * (int)g.ldb + c * 8) * 2;
  }
  auto tile_m0 = [&](int tile) { return (tile % tiles_m) * DB_BM; };
  auto tile_n0 = [&](int tile) { return (tile / tiles_m) * OUT_BN; };
  auto a_base = [&](int tile) { return tile_m0(tile) * (int)g.lda * 2; };
  auto b_base = [&](int tile) { return tile_n0(tile) * (int)g.ldb * 2; };
  const auto a_rsrc = buffer_rsrc(g.A, a_bytes);
  const auto b_rsrc = buffer_rsrc(g.B, b_bytes);
#define DB_COPY(sa_, sb_, stage_)                                                                  \
  {                                                                                                \
    uint8_t* S_ = db_smem + (stage_) * S::STAGE;                                                   \
    _Pragma("unroll") for (int i = 0; i < S::CPW; ++i)                                             \
        copy16_to_lds(a_rsrc, a_off[i], (sa_), (lds_void*)(S_ + (wave * S::CPW + i) * 1024));      \
    _Pragma("unroll") for (int i = 0; i < S::CPW; ++i)                                             \
        copy16_to_lds(b_rsrc, b_off[i], (sb_), (lds_void*)(S_ + S::TILE + (wave * S::CPW + i) * 1024)); \
  }
  // operand reads: lane (lr, half) row lr of each 32-row tile, chunk 2 ks + half
  const int lr = lane & 31, half = lane >> 5, sw = S::swz(lr);
  const int a_row = (wm * 128 + lr) * S::ROW, b_row = S::TILE + (wn * 32 * TN + lr) * S::ROW;
  bf16x8 fa[2][TM], fb[2][TN];
#define DB_READ(stage_, ks_, buf_)                                                                 \
  {                                                                                                \
    const uint8_t* S_ = db_smem + (stage_) * S::STAGE + (((2 * (ks_) + half) ^ sw) << 4);          \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                                 \
        fa[buf_][i] = *reinterpret_cast<const bf16x8*>(S_ + a_row + i * 32 * S::ROW);              \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                 \
        fb[buf_][j] = *reinterpret_cast<const bf16x8*>(S_ + b_row + j * 32 * S::ROW);              \
  }
#define DB_MFMA(buf_)                                                                              \
  _Pragma("unroll") for (int i = 0; i < TM; ++i)                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                               \
          acc[i][j] = mfma32x32x16(fb[buf_][j], fa[buf_][i], acc[i][j]);
// interleave: the TM + TN reads of the next slice spread over its TM x TN MFMAs
  constexpr int MPR = TM * TN / (TM + TN);
#define DB_SCHED()                                                                                 \
  _Pragma("unroll") for (int q = 0; q < TM + TN; ++q) {                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);                                           \
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
  }                                                                                                \
  if (TM * TN > MPR * (TM + TN)) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - MPR * (TM + TN), 0);

  const int nk = g.K / KB;
  int tile = blockIdx.x;
  DB_COPY(a_base(tile), b_base(tile), 0);
  wait_vmcnt<0>();
  lds_barrier();
  int s = 0;
  for (; tile < n_tiles; tile += gridDim.x) {
    const int m0 = tile_m0(tile), n0 = tile_n0(tile);
    const int ab = a_base(tile), bb = b_base(tile);
    // the last step copies the next tile's first (the last tile its own
    // first again, into a stage nothing reads)
    const int nxt = tile + (int)gridDim.x < n_tiles ? tile + (int)gridDim.x : tile;
    const int ab_next = a_base(nxt), bb_next = b_base(nxt);
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};
    // The MFMAs of a step's last slice run after the barrier that ends the
    // step, under the next step's first operand reads; at a tile's first
    // step they multiply zero operands.
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[1][i] = (bf16x8){};
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[1][j] = (bf16x8){};
    // One K step on stage s, copying the next step into the other stage.
    // Copies complete in issue order; the wait before the barrier leaves
    // nothing outstanding, so past it the other stage has landed for every
    // wave and every wave is done reading stage s.
    for (int t = 0; t < nk; ++t) {
      int left = nk - 1 - t;
      asm volatile("" : "+s"(left));  // keeps the loop whole (no peeled last step)
      const int sa = left == 0 ? ab_next : ab + (t + 1) * KB * 2;
      const int sb = left == 0 ? bb_next : bb + (t + 1) * KB * 2;
      DB_READ(s, 0, 0);
      DB_MFMA((KS - 1) & 1);
      DB_SCHED();
      DB_READ(s, 1, 1);
      DB_COPY(sa, sb, s ^ 1);
      DB_MFMA(0);
      __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * S::CPW / (TM * TN), 0);
      }
#pragma unroll
      for (int ks = 2; ks < KS; ++ks) {
        DB_READ(s, ks, ks & 1);
        DB_MFMA((ks - 1) & 1);
        DB_SCHED();
      }
      wait_vmcnt<0>();
      lds_barrier();
      s ^= 1;
    }
    DB_MFMA((KS - 1) & 1);

    // the stage the last step read is free: each wave's share of it holds
    // the wave's output blocks; the barrier keeps the next tile's first
    // copies into that stage behind every wave's epilogue
    db_epilogue<EPI, TM, TN>(g, acc, db_smem + (s ^ 1) * S::STAGE + wave * (S::STAGE / NW), m0 + wm * 128,
                             n0 + wn * (OUT_BN / WN), lane);
    lds_barrier();
  }
  // nothing may still be writing LDS when the workgroup ends
  wait_vmem();
#undef DB_COPY
#undef DB_READ
#undef DB_MFMA
#undef DB_SCHED
}

// ------------------------------------------------------- decode (M <= 64)
// Weight streaming for a batch of at most 64 rows: C^T[n][m] = B[n][k] .
// A[m][k]^T on v_mfma_f32_16x16x32_bf16.  Workgroup = 64 weight rows, wave w
// the 16 rows 16w.. (its A operand), walking K in 128-deep chunks: each wave
// streams its own rows front to back (16 rows x 64 bytes per load), loaded
// straight into registers three chunks ahead of the MFMAs.  The activations
// (B operand, all 64 rows of a chunk, hot in L2) are shared through LDS, also
// three chunks ahead: copied global -> LDS by buffer_load ... lds into a
// four-stage ring, 16-byte piece c of row r at c ^ (r % 16) so that the
// operand reads of 16 consecutive rows hit distinct banks.  SwiGLU takes 32 output columns per
// workgroup, each wave 8 gate rows then the 8 matching up rows, so a lane's
// partner in the pair sits 32 lanes away.  Calls with too few row tiles to
// fill the chip split K across workgroups (fp32 partials, summed in split
// order by splitk_reduce_kernel).
constexpr int SK_KC = 128;                    // K per chunk
constexpr int SK_ROWB = SK_KC * 2;            // bytes of one activation row in LDS
constexpr int SK_STAGE = 64 * SK_ROWB;        // 16 KB
constexpr int SK_NSET = 4;                    // ring stages / weight register sets (3 chunks ahead)
constexpr int SK_WAVES = 4;                   // waves (16 weight rows each) per workgroup

// int8 weight rows -> bf16 MFMA operand: bytes 8 h .. 8 h + 7 of a 16-byte
// load (the codes are integers in [-127, 127]: exact in bf16)
template <int H>
DEV bf16x8 i8x8_to_bf16(const u32x4& v) {
  const uint32_t lo = v[2 * H], hi = v[2 * H + 1];
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)(float)(int8_t)(lo >> (8 * e));
    r[4 + e] = (bf16)(float)(int8_t)(hi >> (8 * e));
  }
  return r;
}

// int4 codes of one group (offset by 8, in nibbles: byte i of each 4-byte
// word holds k = i low and k = i + 4 high) -> bf16 operand of the bf16 value
// nearest the float32 product code * s: fma(n, s, -8 s) is that product
// rounded once (8 s is exact), the conversion rounds it to bf16 (nearest
// even), as the oracle dequantizes
DEV bf16x8 i4x8_to_bf16(uint32_t word, float s, float m8s) {
  uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
  // hide the masks' known zero bits so that each byte converts with one
  // v_cvt_f32_ubyteN (otherwise the shift and mask are kept per element)
  asm("" : "+v"(lo), "+v"(hi));
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)__builtin_fmaf((float)((lo >> (8 * e)) & 0xFFu), s, m8s);
    r[4 + e] = (bf16)__builtin_fmaf((float)((hi >> (8 * e)) & 0xFFu), s, m8s);
  }
  return r;
}

// QB = 8: int8 weight rows with a per-row scale ([P1 section 7]'s
// weight-only INT8; codes and scales as the oracle defines them).  Lane group
// lg then loads bytes 32 lg .. 32 lg + 31 of its row's 128-deep chunk (two
// 16-byte loads, half the bytes of bf16) and MFMA step q takes the 8 of them
// at 32 lg + 8 q; the activation operand reads the same k (the reduction
// order within a chunk is permuted, identically on both operands).  The
// scale multiplies the row's dot products before the epilogue.
// QB = 4: int4 codes with one scale per row and 128-deep group (a chunk is
// one group): lane group lg loads the 16 bytes of k = 32 lg .. 32 lg + 31
// and the group's scale, and dequantizes to bf16 in registers (same k order
// as QB = 8).  In both, the chunk count needs not be a multiple of the ring
// depth (chunks past the end are loaded, not multiplied).
// MT: 16-row tiles of activations multiplied (M <= 16 MT); the copies still
// fill all 64 rows (clamped), so every wave's load count stays the same.
template <int EPI, bool SPLIT, int NW, int QB = 16, int MT = 4>
__global__ __launch_bounds__(64 * NW, 8 / NW) void gemm_skinny_kernel(GemmArgs g, uint32_t a_bytes, uint32_t b_bytes) {
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  static_assert(QB == 16 || QB == 8 || QB == 4, "weight bits");
  static_assert(MT >= 1 && MT <= 4, "activation row tiles");
  constexpr bool Q8 = QB == 8, Q4 = QB == 4;
  constexpr int CPW = 16 / NW;  // activation copies per wave per chunk
  constexpr int WL = QB == 16 ? 4 : QB == 8 ? 2 : 1;  // 16-byte weight loads per lane per chunk
  constexpr int WS = Q4 ? 1 : 0;                       // scale loads per lane per chunk
  __shared__ __align__(16) uint8_t sk_smem[SK_NSET * SK_STAGE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tile = blockIdx.x;
  // weight row of this lane's A-operand row (rows past N clamped: never stored)
  int wrow;
  if (EPI == LOOP_EPI_SWIGLU) {
    const int col = min(8 * NW * tile + 8 * wave + (l16 & 7), g.N - 1);
    wrow = (l16 < 8 ? 0 : g.swiglu_F) + col;
  } else {
    wrow = min(16 * NW * tile + 16 * wave + l16, g.N - 1);
  }
  const int k0 = SPLIT ? blockIdx.y * g.kslice : 0;
  const int nch = (SPLIT ? g.kslice : g.K) / SK_KC;
  const auto a_rsrc = buffer_rsrc(g.A, a_bytes);
  const auto b_rsrc = buffer_rsrc(g.B, b_bytes);
  // activation copies: instruction i of this wave fills rows 4 (4 wave + i) ..
  // + 3; lane l row + l / 16, piece l % 16 holding logical piece
  // (l % 16) ^ (row % 16)
  int a_off[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int row = 4 * (CPW * wave + i) + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    a_off[i] = (min(row, g.M - 1) * (int)g.lda + k0 + c * 8) * 2;
  }
  const int b_off = Q4   ? wrow * (int)g.ldb + k0 / 2 + lg * 16
                    : Q8 ? wrow * (int)g.ldb + k0 + lg * 32
                         : (wrow * (int)g.ldb + k0 + lg * 8) * 2;
  const auto s_rsrc = buffer_rsrc(g.scale, g.scale_bytes);
  const int s_off = Q4 ? (wrow * (g.K / SK_KC) + k0 / SK_KC) * 4 : 0;
#define SK_COPY(ch_, stage_)                                                                       \
  _Pragma("unroll") for (int i = 0; i < CPW; ++i)                                                  \
      copy16_to_lds(a_rsrc, a_off[i], (ch_) * SK_ROWB,                                             \
                    (lds_void*)(sk_smem + (stage_) * SK_STAGE + (CPW * wave + i) * 1024));
#define SK_WLOAD(ch_, set_)                                                                        \
  _Pragma("unroll") for (int q = 0; q < WL; ++q) w[set_][q] =                                      \
      Q4   ? buffer_load16(b_rsrc, b_off, (ch_) * (SK_KC / 2))                                      \
      : Q8 ? buffer_load16(b_rsrc, b_off + q * 16, (ch_) * SK_KC)                                   \
           : buffer_load16(b_rsrc, b_off + q * 64, (ch_) * SK_ROWB);                                \
  if (Q4) wsc[set_] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, s_off, (ch_) * 4, 0));

  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = (f32x4){0, 0, 0, 0};
  u32x4 w[SK_NSET][WL];
  float wsc[SK_NSET];  // int4: the chunk's group scale
#pragma unroll
  for (int p = 0; p < SK_NSET - 1; ++p) {
    SK_COPY(min(p, nch - 1), p);
    SK_WLOAD(min(p, nch - 1), p);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Every load is unconditional (past the end the last chunk is loaded again,
  // into the idle stage / registers), so every path has the same loads in
  // flight and the waits stay exact.  Chunk p's CPW copies are followed by
  // its WL weight loads (and WS scale loads); when chunk c starts, chunks
  // c + 1 and c + 2 were issued after chunk c's, so a count of twice a
  // chunk's loads still in flight means chunk c has landed.
  for (int c0 = 0; c0 < nch; c0 += SK_NSET) {
#pragma unroll
    for (int j = 0; j < SK_NSET; ++j) {
      const int c = c0 + j;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(CPW + WL + WS) * (SK_NSET - 2)>();
      lds_barrier();  // chunk c visible; every wave is done with chunk c - 1
      __builtin_amdgcn_sched_barrier(0);
      SK_COPY(min(c + SK_NSET - 1, nch - 1), (j + SK_NSET - 1) % SK_NSET);
      SK_WLOAD(min(c + SK_NSET - 1, nch - 1), (j + SK_NSET - 1) % SK_NSET);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* st = sk_smem + j * SK_STAGE;
      if (QB == 16 || c < nch) {
        const float m8s = Q4 ? -8.f * wsc[j] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x8 bfr[MT];
          const int piece = QB != 16 ? 4 * lg + q : 4 * q + lg;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            bfr[mt] = *reinterpret_cast<const bf16x8*>(st + (16 * mt + l16) * SK_ROWB + ((piece ^ l16) << 4));
          bf16x8 wa;
          if (Q4) wa = i4x8_to_bf16(w[j][0][q], wsc[j], m8s);
          else if (Q8) wa = (q & 1) ? i8x8_to_bf16<1>(w[j][q >> 1]) : i8x8_to_bf16<0>(w[j][q >> 1]);
          else wa = __builtin_bit_cast(bf16x8, w[j][q]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16x16x32(wa, bfr[mt], acc[mt]);
        }
      }
    }
  }
#undef SK_COPY
#undef SK_WLOAD
  wait_vmem();
  if (Q8) {  // row scales (A-operand row 4 lg + r of the wave)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * lg + r;
      int row;
      if (EPI == LOOP_EPI_SWIGLU) {
        const int col = min(8 * NW * tile + 8 * wave + (i & 7), g.N - 1);
        row = (i < 8 ? 0 : g.swiglu_F) + col;
      } else {
        row = min(16 * NW * tile + 16 * wave + i, g.N - 1);
      }
      const float sc = g.scale[row];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][r] *= sc;
    }
  }

  // lane holds C^T[row 4 lg + r of the wave][m = 16 mt + l16]
  if (EPI == LOOP_EPI_SWIGLU) {
    float up[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) up[mt][r] = __shfl_xor(acc[mt][r], 32, 64);
    if (lg >= 2) return;
    uint16_t* C = reinterpret_cast<uint16_t*>(g.C);
    const int col = 8 * NW * tile + 8 * wave + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + l16;
      if (m >= g.M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (col + r >= g.N) continue;
        if (SPLIT) {  // gate and up apart: [split][m][2][N]
          float* P = g.part + (((int64_t)blockIdx.y * g.M + m) * 2) * g.N + col + r;
          P[0] = acc[mt][r];
          P[g.N] = up[mt][r];
        } else {
          C[(int64_t)m * g.ldc + col + r] = f2bf_bits(siluf_(acc[mt][r]) * up[mt][r]);
        }
      }
    }
    return;
  }
  const int col = 16 * NW * tile + 16 * wave + 4 * lg;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + l16;
    if (m >= g.M) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (col + r >= g.N) continue;
      const float v = acc[mt][r];
      if (SPLIT) {
        g.part[((int64_t)blockIdx.y * g.M + m) * g.N + col + r] = v;
      } else {
        const int64_t o = (int64_t)m * g.ldc + col + r;
        if (EPI == LOOP_EPI_BF16) reinterpret_cast<uint16_t*>(g.C)[o] = f2bf_bits(v);
        else if (EPI == LOOP_EPI_F32) reinterpret_cast<float*>(g.C)[o] = v;
        else reinterpret_cast<float*>(g.C)[o] = g.R[o] + v;
      }
    }
  }
}

// launch with the fewest 16-row activation tiles that cover M
template <int EPI, bool SPLIT, int NW, int QB>
void launch_skinny_mt(dim3 grid, hipStream_t s, const GemmArgs& g, uint32_t a_bytes, uint32_t b_bytes) {
  if (g.M <= 16)
    hipLaunchKernelGGL((gemm_skinny_kernel<EPI, SPLIT, NW, QB, 1>), grid, dim3(64 * NW), 0, s, g, a_bytes, b_bytes);
  else if (g.M <= 32)
    hipLaunchKernelGGL((gemm_skinny_kernel<EPI, SPLIT, NW, QB, 2>), grid, dim3(64 * NW), 0, s, g, a_bytes, b_bytes);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<EPI, SPLIT, NW, QB, 4>), grid, dim3(64 * NW), 0, s, g, a_bytes, b_bytes);
}

// Split-K plans of the small-M paths: the split count a call takes when its
// partial buffer is large enough (shared by the launchers and
// gemm_small_m_partial_bytes).
template <int EPI, int NW>
int skinny_splits(const GemmArgs& g) {
  const int per = (EPI == LOOP_EPI_SWIGLU) ? 8 * NW : 16 * NW;  // output columns per workgroup
  const int tiles = (g.N + per - 1) / per;
  int splits = 1;
  while (tiles * splits < 256 && g.K % (SK_KC * SK_NSET * splits * 2) == 0) splits *= 2;
  return splits;
}

// M <= 64, K range of every workgroup a multiple of SK_NSET chunks, operands
// within 32-bit buffer offsets.
template <int EPI, int NW>
hipError_t launch_skinny_w(GemmArgs g, size_t ws_bytes, uint32_t a_bytes, uint32_t b_bytes, hipStream_t s) {
  const int per = (EPI == LOOP_EPI_SWIGLU) ? 8 * NW : 16 * NW;  // output columns per workgroup
  const int tiles = (g.N + per - 1) / per;
  const int splits = skinny_splits<EPI, NW>(g);
  const size_t need = (size_t)splits * g.M * g.N * (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * sizeof(float);
  if (splits > 1 && g.part && need <= ws_bytes) {
    g.kslice = g.K / splits;
    launch_skinny_mt<EPI, true, NW, 16>(dim3(tiles, splits), s, g, a_bytes, b_bytes);
    const int64_t n_out = (int64_t)g.M * g.N;
    const int blocks = (int)std::min<int64_t>((n_out + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(blocks), dim3(256), 0, s, g, splits);
  } else {
    launch_skinny_mt<EPI, false, NW, 16>(dim3(tiles), s, g, a_bytes, b_bytes);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_skinny(GemmArgs g, size_t ws_bytes, uint32_t a_bytes, uint32_t b_bytes, hipStream_t s) {
  return launch_skinny_w<EPI, SK_WAVES>(g, ws_bytes, a_bytes, b_bytes, s);
}

// Two stages of K = 64 (128 KB of LDS).  Measured slower on every shape:
// deeper rings of K = 32 steps (up to 5 stages, the whole 160 KB; 64-byte
// row pieces double the L2 requests), a five-slot ring of 64-deep operand
// pieces (the 160 KB; each B piece one step ahead, each A piece two), eight
// waves (two per SIMD, 128 x 64 each), an L2 warm-up of the step after next,
// K start staggered by column tile, and other tile orders.
constexpr int DB_KB = 64, DB_NW = 4;
template <int EPI>
hipError_t launch_db(const GemmArgs& g, uint32_t a_bytes, uint32_t b_bytes, hipStream_t s) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? DB_BN / 2 : DB_BN;
  constexpr int lds = db_lds(DB_KB);
  const int tiles = ((g.M + DB_BM - 1) / DB_BM) * ((g.N + OUT_BN - 1) / OUT_BN);
  auto k = gemm_db_kernel<EPI, DB_KB, DB_NW>;
  static int n_cu = 0;
  if (!n_cu) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  // one workgroup per CU (the LDS ring admits no second one)
  hipLaunchKernelGGL(k, dim3(std::min(tiles, n_cu)), dim3(64 * DB_NW), lds, s, g, a_bytes, b_bytes, tiles);
  return hipGetLastError();
}

// 64 x 128 tiles; calls with too few tiles to fill the chip split K so that
// tiles * splits reaches ~256-512 workgroups, if a large enough partial buffer
// is given.
template <int EPI>
int small_splits(const GemmArgs& g) {
  constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? 64 : 128;
  const int tiles = ((g.M + 63) / 64) * ((g.N + OUT_BN - 1) / OUT_BN);
  // fewer splits mean fewer fp32 partials to write and sum; measured on the
  // decode shapes (64 rows), ~256 workgroups suffice for K <= 4096 without
  // SwiGLU
  const int target = (EPI != LOOP_EPI_SWIGLU && g.K <= 4096 && g.M <= 64) ? 256 : 512;
  int splits = 1;
  if (g.M >= 512) {
    // many rows (the narrow column strip of a prefill projection): a split
    // count that does not depend on M, so that a row's result does not
    // depend on how many rows share the call (chunked prefill = whole)
    if (g.K % 256 == 0 && g.K >= 1024) splits = 4;
  } else {
    while (tiles * splits < target && g.K % (64 * splits * 2) == 0 && g.K / (splits * 2) >= 256) splits *= 2;
  }
  return splits;
}

template <int EPI>
hipError_t launch_small(GemmArgs g, size_t ws_bytes, hipStream_t s) {
  if (g.M <= 64 && g.part) {
    const size_t need = stream_partial_bytes<EPI>(g);
    if (need > 0 && need <= ws_bytes) return launch_stream<EPI>(g, s);
  }
  const int splits = small_splits<EPI>(g);
  const size_t need = (size_t)splits * g.M * g.N * (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * sizeof(float);
  if (splits > 1 && g.part && need <= ws_bytes) {
    g.kslice = g.K / splits;
    return launch_cfg<64, 128, 2, 2, EPI, true>(g, splits, s);
  }
  return launch_cfg<64, 128, 2, 2, EPI, false>(g, 1, s);
}

// Measured on the decode shapes (64 rows): the skinny tiles win where the
// output has at most 4096 columns and K at most 4096; the register-staged
// 64 x 128 tiles stream the wider and deeper weight matrices faster.
// Where the weight-streaming tiles beat the 64 x 128 split-K tiles (measured
// at M = 1 and 64 on the decode projections): up to 4096 columns with K up
// to 12288 (O and down projections), and very wide products at 16 rows or
// fewer (the LM head at small batch).
template <int EPI>
bool skinny_fits(const GemmArgs& g) {
  const int64_t rows_b = (EPI == LOOP_EPI_SWIGLU) ? 2 * (int64_t)g.N : g.N;
  const int64_t a_bytes = (int64_t)g.M * g.lda * 2, b_bytes = rows_b * g.ldb * 2;
  const bool shape = (g.N <= 4096 && g.K <= 12288) || (g.M <= 16 && g.N >= 65536);
  return g.M <= 64 && shape && g.K % (SK_KC * SK_NSET) == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         a_bytes < (1ll << 31) && b_bytes < (1ll << 31);
}

// Large M: 256 x 256 tiles; small M (decode): 64 x 128 tiles, split K.
template <int EPI>
hipError_t launch_epi(GemmArgs g, size_t ws_bytes, hipStream_t s) {
  // Large M: whole 256 x 256 tiles fed by LDS copies on the persistent
  // kernel; the ragged edges (fewer than 256 rows, or fewer than one tile
  // of columns) on 64 x 128 tiles, split K (e.g. 8224 columns: 1024 whole
  // tiles, and the last 32 columns in a fraction of another round of big
  // tiles).  Operands whose byte range does not fit the 32-bit buffer
  // offsets, or unaligned outputs, use the register-staged kernel (eight
  // waves, two per SIMD).
  if (g.M >= 512) {
    constexpr int OUT_BN = (EPI == LOOP_EPI_SWIGLU) ? DB_BN / 2 : DB_BN;
    const int64_t rows_b = (EPI == LOOP_EPI_SWIGLU) ? (int64_t)g.swiglu_F + g.N : g.N;
    const int64_t a_bytes = (int64_t)g.M * g.lda * 2, b_bytes = rows_b * g.ldb * 2;
    const int mm = g.M / DB_BM * DB_BM, nm = g.N / OUT_BN * OUT_BN;
    const int64_t c_align = (EPI == LOOP_EPI_BF16 || EPI == LOOP_EPI_SWIGLU) ? 8 : 4;  // 16-byte rows
    const bool aligned = g.ldc % c_align == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(g.R) & 15) == 0 && (g.lda & 7) == 0 && (g.ldb & 7) == 0;
    if (g.K % DB_KB == 0 && a_bytes < (1ll << 31) && b_bytes < (1ll << 31) && aligned && nm > 0) {
      const size_t esz = (EPI == LOOP_EPI_BF16 || EPI == LOOP_EPI_SWIGLU) ? 2 : 4;
      GemmArgs main = g;
      main.M = mm;
      main.N = nm;
      hipError_t e = launch_db<EPI>(main, (uint32_t)a_bytes, (uint32_t)b_bytes, s);
      if (e != hipSuccess) return e;
      if (nm < g.N) {  // all rows, columns nm .. N - 1 (SwiGLU: up rows stay swiglu_F further on)
        GemmArgs tail = g;
        tail.B = g.B + (int64_t)nm * g.ldb;
        tail.C = (uint8_t*)g.C + (int64_t)nm * esz;
        tail.R = g.R ? g.R + nm : nullptr;
        tail.N = g.N - nm;
        e = launch_small<EPI>(tail, ws_bytes, s);
        if (e != hipSuccess) return e;
      }
      if (mm < g.M) {  // rows mm .. M - 1, columns 0 .. nm - 1
        GemmArgs tail = g;
        tail.A = g.A + (int64_t)mm * g.lda;
        tail.C = (uint8_t*)g.C + (int64_t)mm * g.ldc * esz;
        tail.R = g.R ? g.R + (int64_t)mm * g.ldc : nullptr;
        tail.M = g.M - mm;
        tail.N = nm;
        e = launch_small<EPI>(tail, ws_bytes, s);
      }
      return e;
    }
    return launch_cfg<256, 256, 2, 4, EPI, false>(g, 1, s);
  }
  if (skinny_fits<EPI>(g)) {
    const int64_t rows_b = (EPI == LOOP_EPI_SWIGLU) ? 2 * (int64_t)g.N : g.N;
    return launch_skinny<EPI>(g, ws_bytes, (uint32_t)((int64_t)g.M * g.lda * 2), (uint32_t)(rows_b * g.ldb * 2), s);
  }
  return launch_small<EPI>(g, ws_bytes, s);
}

// Split-K partial bytes of a call with M < 512 rows when its buffer is large
// enough (0: the call does not split).
template <int EPI>
size_t small_m_partial_bytes(const GemmArgs& g) {
  if (!skinny_fits<EPI>(g) && g.M <= 64) {
    const size_t st = stream_partial_bytes<EPI>(g);
    if (st > 0) return st;
  }
  const int splits = skinny_fits<EPI>(g) ? skinny_splits<EPI, SK_WAVES>(g) : small_splits<EPI>(g);
  return splits > 1 ? (size_t)splits * g.M * g.N * (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * sizeof(float) : 0;
}

// Weight-only int8 / int4 (decode, M <= 64): the skinny tiles over the
// codes.  Splits as for bf16 (K in 128-deep chunks, any count per split).
// Measured: twice the workgroups (two per CU) is no faster; with the
// weights 2-4x smaller, each chunk's activation reads from LDS (16 KB per
// wave) and its M = 64 MFMAs, not the weight stream, set the time.
template <int EPI, int QB>
hipError_t launch_wq(GemmArgs g, size_t ws_bytes, uint32_t a_bytes, uint32_t b_bytes, hipStream_t s) {
  constexpr int NW = SK_WAVES;
  const int per = (EPI == LOOP_EPI_SWIGLU) ? 8 * NW : 16 * NW;
  const int tiles = (g.N + per - 1) / per;
  int splits = 1;
  while (tiles * splits < 256 && g.K % (SK_KC * splits * 2) == 0 && g.K / (splits * 2) >= 512) splits *= 2;
  const size_t need = (size_t)splits * g.M * g.N * (EPI == LOOP_EPI_SWIGLU ? 2 : 1) * sizeof(float);
  if (splits > 1 && g.part && need <= ws_bytes) {
    g.kslice = g.K / splits;
    launch_skinny_mt<EPI, true, NW, QB>(dim3(tiles, splits), s, g, a_bytes, b_bytes);
    const int64_t n_out = (int64_t)g.M * g.N;
    const int blocks = (int)std::min<int64_t>((n_out + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(blocks), dim3(256), 0, s, g, splits);
  } else {
    launch_skinny_mt<EPI, false, NW, QB>(dim3(tiles), s, g, a_bytes, b_bytes);
  }
  return hipGetLastError();
}

// per row of an int8 code matrix: scale = max |w| / 127, code = nearest
// integer to w / scale (ties to even), both in fp32 with correctly rounded
// division (the oracle takes the same decisions)
__global__ __launch_bounds__(256) void quantize_int8_kernel(const uint16_t* w, int64_t ldw, int K, int8_t* q,
                                                            int64_t ldq, float* scale) {
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  const uint16_t* wr = w + n * ldw;
  float mx = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) mx = fmaxf(mx, fabsf(bf2f(wr[k])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = __fdiv_rn(mx, 127.0f);
  if (threadIdx.x == 0) scale[n] = sc;
  for (int k = threadIdx.x; k < K; k += 256) {
    const float v = sc > 0.f ? rintf(__fdiv_rn(bf2f(wr[k]), sc)) : 0.f;
    q[n * ldq + k] = (int8_t)fminf(fmaxf(v, -127.f), 127.f);
  }
}

// per row n and 128-deep group: scale = max |w| / 7, codes = nearest integer
// to w / scale (ties to even) in [-7, 7], in fp32 with correctly rounded
// division as the oracle decides them; stored offset by 8 in nibbles, byte
// i of each 8-k run holding k = i (low) and k = i + 4 (high).  One wave per
// (row, group): lane l makes byte l of the group's 64.
__global__ __launch_bounds__(256) void quantize_int4_kernel(const uint16_t* w, int64_t ldw, int64_t N, int G,
                                                            uint8_t* q, int64_t ldq, float* scale) {
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= N * G) return;  // whole waves
  const int lane = threadIdx.x & 63;
  const int64_t n = unit / G;
  const int grp = (int)(unit % G);
  const int klo = SK_KC * grp + 8 * (lane >> 2) + (lane & 3);
  const float vlo = bf2f(w[n * ldw + klo]), vhi = bf2f(w[n * ldw + klo + 4]);
  float mx = fmaxf(fabsf(vlo), fabsf(vhi));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float sc = __fdiv_rn(mx, 7.0f);
  const float clo = sc > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(vlo, sc)), -7.f), 7.f) : 0.f;
  const float chi = sc > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(vhi, sc)), -7.f), 7.f) : 0.f;
  q[n * ldq + (int64_t)grp * (SK_KC / 2) + lane] = (uint8_t)(((int)clo + 8) | (((int)chi + 8) << 4));
  if (lane == 0) scale[n * G + grp] = sc;
}

}  // namespace

hipError_t launch_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int M, int N, int K, int epi, hipStream_t s, float* ws,
                       size_t ws_bytes) {
  GemmArgs g{(const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc, R, M, N, K, N, ws, K};
  switch (epi) {
    case LOOP_EPI_BF16: return launch_epi<LOOP_EPI_BF16>(g, ws_bytes, s);
    case LOOP_EPI_F32: return launch_epi<LOOP_EPI_F32>(g, ws_bytes, s);
    case LOOP_EPI_F32_RES: return launch_epi<LOOP_EPI_F32_RES>(g, ws_bytes, s);
    case LOOP_EPI_SWIGLU: return launch_epi<LOOP_EPI_SWIGLU>(g, ws_bytes, s);
  }
  return hipErrorInvalidValue;
}

size_t gemm_small_m_partial_bytes(int M, int N, int K, int epi, int64_t lda, int64_t ldb) {
  if (M <= 0 || M >= 512) return 0;
  GemmArgs g{nullptr, lda, nullptr, ldb, nullptr, N, nullptr, M, N, K, N, nullptr, K};
  switch (epi) {
    case LOOP_EPI_BF16: return small_m_partial_bytes<LOOP_EPI_BF16>(g);
    case LOOP_EPI_F32: return small_m_partial_bytes<LOOP_EPI_F32>(g);
    case LOOP_EPI_F32_RES: return small_m_partial_bytes<LOOP_EPI_F32_RES>(g);
    case LOOP_EPI_SWIGLU: return small_m_partial_bytes<LOOP_EPI_SWIGLU>(g);
  }
  return 0;
}

hipError_t launch_gemm_norm(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                            const float* R, const float* X2, const void* gain, void* hn, float eps, int M, int N,
                            int K, hipStream_t s, float* ws, size_t ws_bytes) {
  GemmArgs g{(const uint16_t*)A, lda, (const uint16_t*)B, ldb, C, ldc, R, M, N, K, N, ws, K};
  const int64_t a_bytes = (int64_t)M * lda * 2, b_bytes = (int64_t)N * ldb * 2;
  // the decode shape of the projection feeding the FFN norm: weight-streaming
  // tiles with split K, the split sum and the norm in one row pass
  if (M <= 64 && N <= 4096 && K <= 4096 && K % (SK_KC * SK_NSET) == 0 && lda % 8 == 0 &&
      ldb % 8 == 0 && a_bytes < (1ll << 31) && b_bytes < (1ll << 31)) {
    const int tiles = (N + 16 * SK_WAVES - 1) / (16 * SK_WAVES);
    int splits = 1;
    while (tiles * splits < 256 && splits < 8 && K % (SK_KC * SK_NSET * splits * 2) == 0) splits *= 2;
    if (splits > 1 && ws && (size_t)splits * M * N * sizeof(float) <= ws_bytes) {
      g.kslice = K / splits;
      auto launch = [&](auto epi_tag) {
        constexpr int EPI = decltype(epi_tag)::value;
        launch_skinny_mt<EPI, true, SK_WAVES, 16>(dim3(tiles, splits), s, g, (uint32_t)a_bytes, (uint32_t)b_bytes);
        if (splits == 4)
          hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 4>), dim3(M), dim3(1024), 0, s, g, X2,
                             (const uint16_t*)gain, (uint16_t*)hn, eps);
        else if (splits == 2)
          hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 2>), dim3(M), dim3(1024), 0, s, g, X2,
                             (const uint16_t*)gain, (uint16_t*)hn, eps);
        else
          hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 8>), dim3(M), dim3(1024), 0, s, g, X2,
                             (const uint16_t*)gain, (uint16_t*)hn, eps);
      };
      if (R) launch(std::integral_constant<int, LOOP_EPI_F32_RES>());
      else launch(std::integral_constant<int, LOOP_EPI_F32>());
      return hipGetLastError();
    }
  }
  hipError_t e = launch_gemm(A, lda, B, ldb, C, ldc, R, M, N, K, R ? LOOP_EPI_F32_RES : LOOP_EPI_F32, s, ws, ws_bytes);
  if (e != hipSuccess) return e;
  return launch_rmsnorm(C, X2, nullptr, ldc, gain, hn, M, N, eps, s);
}

static bool wq_args_ok(int bits, int M, int K, int64_t lda, int64_t ldb, const float* scale) {
  return (bits == 8 || bits == 4) && M >= 1 && M <= 64 && K % SK_KC == 0 && lda % 8 == 0 && ldb % 16 == 0 && scale;
}

hipError_t launch_gemm_wq(int bits, const void* A, int64_t lda, const void* Bq, int64_t ldb, const float* scale,
                          void* C, int64_t ldc, const float* R, int M, int N, int K, int epi, hipStream_t s, float* ws,
                          size_t ws_bytes) {
  if (!wq_args_ok(bits, M, K, lda, ldb, scale)) return hipErrorInvalidValue;
  GemmArgs g{(const uint16_t*)A, lda, (const uint16_t*)Bq, ldb, C, ldc, R, M, N, K, N, ws, K, scale};
  const int64_t rows_b = (epi == LOOP_EPI_SWIGLU) ? 2 * (int64_t)N : N;
  const int64_t a_bytes = (int64_t)M * lda * 2, b_bytes = rows_b * ldb;
  const int64_t s_bytes = rows_b * (K / SK_KC) * 4;
  if (a_bytes >= (1ll << 31) || b_bytes >= (1ll << 31) || s_bytes >= (1ll << 31)) return hipErrorInvalidValue;
  g.scale_bytes = (uint32_t)s_bytes;
  auto go = [&](auto qb) -> hipError_t {
    constexpr int QB = decltype(qb)::value;
    switch (epi) {
      case LOOP_EPI_BF16: return launch_wq<LOOP_EPI_BF16, QB>(g, ws_bytes, (uint32_t)a_bytes, (uint32_t)b_bytes, s);
      case LOOP_EPI_F32: return launch_wq<LOOP_EPI_F32, QB>(g, ws_bytes, (uint32_t)a_bytes, (uint32_t)b_bytes, s);
      case LOOP_EPI_F32_RES:
        return launch_wq<LOOP_EPI_F32_RES, QB>(g, ws_bytes, (uint32_t)a_bytes, (uint32_t)b_bytes, s);
      case LOOP_EPI_SWIGLU: return launch_wq<LOOP_EPI_SWIGLU, QB>(g, ws_bytes, (uint32_t)a_bytes, (uint32_t)b_bytes, s);
    }
    return hipErrorInvalidValue;
  };
  return bits == 8 ? go(std::integral_constant<int, 8>()) : go(std::integral_constant<int, 4>());
}

hipError_t launch_gemm_norm_wq(int bits, const void* A, int64_t lda, const void* Bq, int64_t ldb, const float* scale,
                               float* C, int64_t ldc, const float* R, const float* X2, const void* gain, void* hn,
                               float eps, int M, int N, int K, hipStream_t s, float* ws, size_t ws_bytes) {
  if (!wq_args_ok(bits, M, K, lda, ldb, scale)) return hipErrorInvalidValue;
  GemmArgs g{(const uint16_t*)A, lda, (const uint16_t*)Bq, ldb, C, ldc, R, M, N, K, N, ws, K, scale};
  const int64_t a_bytes = (int64_t)M * lda * 2, b_bytes = (int64_t)N * ldb, s_bytes = (int64_t)N * (K / SK_KC) * 4;
  if (a_bytes >= (1ll << 31) || b_bytes >= (1ll << 31) || s_bytes >= (1ll << 31)) return hipErrorInvalidValue;
  g.scale_bytes = (uint32_t)s_bytes;
  const int tiles = (N + 16 * SK_WAVES - 1) / (16 * SK_WAVES);
  int splits = 1;
  while (tiles * splits < 256 && splits < 8 && K % (SK_KC * splits * 2) == 0 && K / (splits * 2) >= 512) splits *= 2;
  if (N <= 4096 && splits > 1 && ws && (size_t)splits * M * N * sizeof(float) <= ws_bytes) {
    g.kslice = K / splits;
    auto launch = [&](auto epi_tag, auto qb) {
      constexpr int EPI = decltype(epi_tag)::value;
      constexpr int QB = decltype(qb)::value;
      launch_skinny_mt<EPI, true, SK_WAVES, QB>(dim3(tiles, splits), s, g, (uint32_t)a_bytes, (uint32_t)b_bytes);
      if (splits == 4)
        hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 4>), dim3(M), dim3(1024), 0, s, g, X2,
                           (const uint16_t*)gain, (uint16_t*)hn, eps);
      else if (splits == 2)
        hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 2>), dim3(M), dim3(1024), 0, s, g, X2,
                           (const uint16_t*)gain, (uint16_t*)hn, eps);
      else
        hipLaunchKernelGGL((splitk_reduce_norm_kernel<EPI, 4, 8>), dim3(M), dim3(1024), 0, s, g, X2,
                           (const uint16_t*)gain, (uint16_t*)hn, eps);
    };
    const auto res = std::integral_constant<int, LOOP_EPI_F32_RES>();
    const auto plain = std::integral_constant<int, LOOP_EPI_F32>();
    if (bits == 8) {
      if (R) launch(res, std::integral_constant<int, 8>());
      else launch(plain, std::integral_constant<int, 8>());
    } else {
      if (R) launch(res, std::integral_constant<int, 4>());
      else launch(plain, std::integral_constant<int, 4>());
    }
    return hipGetLastError();
  }
  hipError_t e = launch_gemm_wq(bits, A, lda, Bq, ldb, scale, C, ldc, R, M, N, K, R ? LOOP_EPI_F32_RES : LOOP_EPI_F32,
                                s, ws, ws_bytes);
  if (e != hipSuccess) return e;
  return launch_rmsnorm(C, X2, nullptr, ldc, gain, hn, M, N, eps, s);
}

hipError_t launch_quantize_int8(const void* w, int64_t ldw, int64_t N, int K, int8_t* q, int64_t ldq, float* scale,
                                hipStream_t s) {
  if (N <= 0 || K <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_int8_kernel, dim3((unsigned)N), dim3(256), 0, s, (const uint16_t*)w, ldw, K, q, ldq,
                     scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int4(const void* w, int64_t ldw, int64_t N, int K, uint8_t* q, int64_t ldq, float* scale,
                                hipStream_t s) {
  if (N <= 0 || K <= 0) return hipSuccess;
  if (K % SK_KC) return hipErrorInvalidValue;
  const int64_t units = N * (K / SK_KC);
  hipLaunchKernelGGL(quantize_int4_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, (const uint16_t*)w,
                     ldw, N, K / SK_KC, q, ldq, scale);
  return hipGetLastError();
}
