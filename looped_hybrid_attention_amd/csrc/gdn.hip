// Gated-DeltaNet (GDN) kernels: chunked prefill and single-token decode.
//
// [P1 section 3]: a linear-attention layer with a gate and the delta rule and
// a state whose size does not depend on the sequence length.  Reading: the
// gated delta rule of Yang, Kautz, Hatamizadeh (ICLR 2025),
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
// S in R^{Dv x Dk} (fp32), with alpha_t = exp(-softplus(a_t)),
// beta_t = sigmoid(b_t), q and k L2-normalised per head (eps), q scaled by
// 1/sqrt(Dk); output RMSNorm over Dv (one gain) times SiLU(z).
//
// Prefill uses the chunkwise form of the same recurrence (C = 64 tokens):
// with G_r = sum_{j<=r} log alpha_j, gamma = exp(G) and
// A[r,i] = beta_r exp(G_r - G_i) k_r.k_i (i < r):
//   T = (I + A)^-1, W = T diag(beta gamma) K, U~ = T diag(beta) V    (chunk-local)
//   U = U~ - W S0^T
//   O = diag(gamma) Q S0^T + (tril(exp(G_r - G_i)) * Q K^T) U
//   S_C = gamma_C S0 + U^T diag(exp(G_C - G)) K.
// The chunk-local part runs for all chunks in parallel; the carry of S is
// sequential over chunks but independent per row of S, so it is split over
// workgroups along Dv.
#include "common.h"
#include "launch.h"

namespace {

constexpr int CH = 64;   // chunk length

DEV float softplusf_(float x) { return x > 20.f ? x : log1pf(expf(x)); }

// fp32 MFMA 16x16x4 tile products from LDS (row-major operands).  Lane l
// supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16]; the result D
// holds rows 4*(l/16) + r (r = 0..3) of column l%16.
DEV f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// acc += A[0:16, 0:K] . B[0:16, 0:K]^T
DEV void mm_nt(f32x4& acc, const float* A, int lda, const float* B, int ldb, int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + i * lda + kk;
  const float* b = B + i * ldb + kk;
#pragma unroll
  for (int k = 0; k < K; k += 4) acc = mfma16x16x4f32(a[k], b[k], acc);
}
// The same MFMA with its result kept apart from its C operand: C stays live
// until the result exists, so the registers cannot partially overlap (the
// compiler otherwise may place a chain's result one register pair off its C
// operand, which the hardware does not compute correctly).
DEV f32x4 mfma16x16x4f32_apart(float a, float b, f32x4 c) {
  const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  asm volatile("" ::"v"(c), "v"(d));
  return d;
}
// acc += A[0:16, 0:16] . B[0:16, 0:16] with every result apart from its C
DEV void mm_nn16_apart(f32x4& acc, const float* A, int lda, const float* B, int ldb) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + i * lda + kk;
  const float* b = B + kk * ldb + i;
#pragma unroll
  for (int k = 0; k < 16; k += 4) acc = mfma16x16x4f32_apart(a[k], b[k * ldb], acc);
}
// acc += A[0:16, 0:K] . B[0:K, 0:16]
DEV void mm_nn(f32x4& acc, const float* A, int lda, const float* B, int ldb, int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + i * lda + kk;
  const float* b = B + kk * ldb + i;
#pragma unroll
  for (int k = 0; k < K; k += 4) acc = mfma16x16x4f32(a[k], b[k * ldb], acc);
}
// acc += A[0:K, 0:16]^T . B[0:K, 0:16]
DEV void mm_tn(f32x4& acc, const float* A, int lda, const float* B, int ldb, int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + kk * lda + i;
  const float* b = B + kk * ldb + i;
#pragma unroll
  for (int k = 0; k < K; k += 4) acc = mfma16x16x4f32(a[k * lda], b[k * ldb], acc);
}

// Two products in one pass (independent MFMA chains, so the second issues
// while the first is in flight).
// acc0 += A0[0:16, 0:K] . B[0:16, 0:K]^T, acc1 += A1[0:16, 0:K] . B[0:16, 0:K]^T
DEV void mm_nt2(f32x4& acc0, f32x4& acc1, const float* A0, const float* A1, int lda, const float* B, int ldb,
                int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a0 = A0 + i * lda + kk;
  const float* a1 = A1 + i * lda + kk;
  const float* b = B + i * ldb + kk;
#pragma unroll
  for (int k = 0; k < K; k += 4) {
    const float bk = b[k];
    acc0 = mfma16x16x4f32(a0[k], bk, acc0);
    acc1 = mfma16x16x4f32(a1[k], bk, acc1);
  }
}
// acc0 += A0[0:16, 0:K] . B0[0:K, 0:16], acc1 += A1[0:16, 0:K] . B1[0:K, 0:16]
DEV void mm_nn2(f32x4& acc0, f32x4& acc1, const float* A0, const float* A1, int lda, const float* B0,
                const float* B1, int ldb, int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a0 = A0 + i * lda + kk;
  const float* a1 = A1 + i * lda + kk;
  const float* b0 = B0 + kk * ldb + i;
  const float* b1 = B1 + kk * ldb + i;
#pragma unroll
  for (int k = 0; k < K; k += 4) {
    acc0 = mfma16x16x4f32(a0[k], b0[k * ldb], acc0);
    acc1 = mfma16x16x4f32(a1[k], b1[k * ldb], acc1);
  }
}

// acc0 += A . B0^T, acc1 += A . B1^T (shared A, [16][K] row-major operands)
DEV void mm_nt2s(f32x4& acc0, f32x4& acc1, const float* A, int lda, const float* B0, const float* B1, int ldb,
                 int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + i * lda + kk;
  const float* b0 = B0 + i * ldb + kk;
  const float* b1 = B1 + i * ldb + kk;
#pragma unroll
  for (int k = 0; k < K; k += 4) {
    const float ak = a[k];
    acc0 = mfma16x16x4f32(ak, b0[k], acc0);
    acc1 = mfma16x16x4f32(ak, b1[k], acc1);
  }
}
// acc += A[0:16, 0:K] . B[0:16, 0:K]^T as two interleaved chains (K % 8 == 0)
DEV void mm_nt_ilp(f32x4& acc, const float* A, int lda, const float* B, int ldb, int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + i * lda + kk;
  const float* b = B + i * ldb + kk;
  f32x4 acc1 = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < K; k += 8) {
    acc = mfma16x16x4f32(a[k], b[k], acc);
    acc1 = mfma16x16x4f32(a[k + 4], b[k + 4], acc1);
  }
  acc += acc1;
}
// acc0 += A[0:K, 0:16]^T . B0[0:K, 0:16], acc1 += A[0:K, 0:16]^T . B1[0:K, 0:16]
DEV void mm_tn2(f32x4& acc0, f32x4& acc1, const float* A, int lda, const float* B0, const float* B1, int ldb,
                int K) {
  const int l = threadIdx.x & 63, i = l & 15, kk = l >> 4;
  const float* a = A + kk * lda + i;
  const float* b0 = B0 + kk * ldb + i;
  const float* b1 = B1 + kk * ldb + i;
#pragma unroll
  for (int k = 0; k < K; k += 4) {
    const float ak = a[k * lda];
    acc0 = mfma16x16x4f32(ak, b0[k * ldb], acc0);
    acc1 = mfma16x16x4f32(ak, b1[k * ldb], acc1);
  }
}

// Operand staging for the fp32 MFMA with K read ahead: lane group kk takes
// the contiguous quarter k = kk K/4 .. of K (a permutation of K, applied to
// both operands of a product), so row operands are 128-bit LDS reads and all
// reads are issued before the MFMAs.
// this lane's quarter of row l%16 of a [16][K] row-major operand
template <int K>
DEV void row_quarter(float (&v)[K / 4], const float* A, int lda) {
  const int l = threadIdx.x & 63;
  const float* r = A + (l & 15) * lda + (l >> 4) * (K / 4);
#pragma unroll
  for (int q = 0; q < K / 16; ++q) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(r + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
  }
}
// this lane's quarter of column l%16 of a [K][16] row-major operand
template <int K>
DEV void col_quarter(float (&v)[K / 4], const float* B, int ldb) {
  const int l = threadIdx.x & 63;
  const float* c = B + (l >> 4) * (K / 4) * ldb + (l & 15);
#pragma unroll
  for (int q = 0; q < K / 4; ++q) v[q] = c[q * ldb];
}
// acc0 += a0 . b0, acc1 += a1 . b1 over staged quarters (two chains)
template <int K>
DEV void mma2(f32x4& acc0, f32x4& acc1, const float (&a0)[K / 4], const float (&b0)[K / 4],
              const float (&a1)[K / 4], const float (&b1)[K / 4]) {
#pragma unroll
  for (int q = 0; q < K / 4; ++q) {
    acc0 = mfma16x16x4f32(a0[q], b0[q], acc0);
    acc1 = mfma16x16x4f32(a1[q], b1[q], acc1);
  }
}

// Chunk workspace layout, per (seq b, head h, chunk c), fp32:
//   W, Qp, Up: [CH][DK]; UtT = Ut^T [DV][CH] and KdT = Kd^T [DK][CH]
//   (transposed: the scan reads them along the chunk's tokens); gC;
//   S_c (entry state) [DV][DK].
struct ChunkPtr {
  float *W, *UtT, *KdT, *Qp, *Up, *S;
  float* gC;
};
DEV ChunkPtr chunk_ptr(const GdnArgs& a, int b, int h, int c, int DK) {
  const int64_t cb = ((int64_t)b * a.H + h) * a.n_chunks + c;
  const int64_t mat = (int64_t)CH * DK;
  ChunkPtr p;
  p.W = a.W + cb * mat;
  p.UtT = a.Ut + cb * mat;
  p.KdT = a.Kd + cb * mat;
  p.Qp = a.Qg + cb * mat;
  p.Up = a.Mqk + cb * mat;
  p.S = a.Sc + cb * (int64_t)DK * DK;
  p.gC = a.gC + cb;
  return p;
}

// ------------------------------------------------------- chunk prep
// grid (chunk, head, seq), eight waves (two per SIMD, so that one's LDS reads
// overlap the other's MFMAs).  Writes W = T diag(beta gamma) K, Ut = T diag(beta) V,
// Kd = exp(G_C - G) K, Qp = gamma Q - Mqk W and Up = Mqk Ut, and gC, where
// Mqk = tril(exp(G_r - G_i)) * Q K^T and T = (I + A)^-1.  In the products
// wave w takes the 16-row tile w % 4 and half (w / 4) of the column tiles.
constexpr int PNT = 512;
template <int DK>
__global__ __launch_bounds__(PNT, 1) void gdn_chunk_prep_kernel(GdnArgs a) {
  constexpr int DV = DK;
  constexpr int LD = DK + 4;   // [CH][DK] rows
  constexpr int LC = CH + 4;   // [CH][CH] rows
  constexpr int XS = 20;       // rows of the 16x16 inverse scratch
  extern __shared__ __align__(16) float gsm[];
  float* sQ = gsm;                 // q^ ; later unchanged
  float* sK = sQ + CH * LD;        // k^ ; later W
  float* sV = sK + CH * LD;        // v  ; later Ut
  float* sA = sV + CH * LD;        // A ; later T diag(beta gamma)
  float* sT2 = sA + CH * LC;       // T diag(beta)
  float* sM = sT2 + CH * LC;       // Mqk
  float* sG = sM + CH * LC;        // cumulative log alpha
  float* sB = sG + CH;             // beta
  float* sEG = sB + CH;            // exp(G_r)
  float* sEK = sEG + CH;           // exp(G_C - G_r)
  float* sX = sEK + CH;            // [4][16][XS] products of the blocked inverse
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = c * CH;
  const int C = min(CH, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)b * a.T + t0;
  const ChunkPtr P = chunk_ptr(a, b, h, c, DK);

  // q, k, v of the chunk's rows: 8 threads per row, DK/8 dims each, every
  // load issued before any is used; q and k L2-normalised per row.
  {
    static_assert(CH * 8 == PNT, "8 threads per row");
    constexpr int PER = DK / 8;      // dims per thread
    constexpr int NV = PER / 8;      // 16-byte loads per tensor
    const int r = tid >> 3, part = tid & 7;
    const bool ok = r < C;
    const uint16_t* pr = a.proj + (row0 + min(r, C - 1)) * a.proj_stride;
    const int d0 = part * PER;
    u32x4 vq[NV], vk[NV], vv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      vq[i] = *reinterpret_cast<const u32x4*>(pr + a.off_q + h * DK + d0 + 8 * i);
      vk[i] = *reinterpret_cast<const u32x4*>(pr + a.off_k + h * DK + d0 + 8 * i);
      vv[i] = *reinterpret_cast<const u32x4*>(pr + a.off_v + h * DV + d0 + 8 * i);
    }
    float av = 0.f, bv = 0.f;
    if (part == 0) {
      av = bf2f(pr[a.off_a + h]);
      bv = bf2f(pr[a.off_b + h]);
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = bf2f((uint16_t)(vq[i][e >> 1] >> ((e & 1) * 16)));
        const float k = bf2f((uint16_t)(vk[i][e >> 1] >> ((e & 1) * 16)));
        sq += q * q;
        sk += k * k;
      }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      sq += __shfl_xor(sq, o, 64);
      sk += __shfl_xor(sk, o, 64);
    }
    const float iq = ok ? rsqrtf(sq + a.eps) * a.q_scale : 0.f;
    const float ik = ok ? rsqrtf(sk + a.eps) : 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + 8 * i + e;
        sQ[r * LD + d] = bf2f((uint16_t)(vq[i][e >> 1] >> ((e & 1) * 16))) * iq;
        sK[r * LD + d] = bf2f((uint16_t)(vk[i][e >> 1] >> ((e & 1) * 16))) * ik;
        sV[r * LD + d] = ok ? bf2f((uint16_t)(vv[i][e >> 1] >> ((e & 1) * 16))) : 0.f;
      }
    if (part == 0) {
      sG[r] = ok ? -softplusf_(av) : 0.f;
      sB[r] = ok ? sigmoidf_(bv) : 0.f;
    }
  }
  __syncthreads();
  if (wave == 0) {  // inclusive prefix sum of log alpha over the 64 rows
    float g = sG[lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(g, o, 64);
      if (lane >= o) g += u;
    }
    sG[lane] = g;
  }
  __syncthreads();
  const float GC = sG[C - 1];
  if (tid < CH) {
    sEG[tid] = __expf(sG[tid]);
    sEK[tid] = __expf(GC - sG[tid]);
  }
  if (tid == 0) *P.gC = __expf(GC);
  // A = beta_r exp(G_r - G_i) k_r.k_i (i < r), Mqk = exp(G_r - G_i) q_r.k_i (i <= r)
  const int rt = wave & 3, ch = wave >> 2;  // row tile, column half of the products
  {
    const int i16 = lane & 15, kk = lane >> 4;
    float aK[DK / 4], aQ[DK / 4];
    row_quarter<DK>(aK, sK + rt * 16 * LD, LD);
    row_quarter<DK>(aQ, sQ + rt * 16 * LD, LD);
#pragma unroll
    for (int n2 = 0; n2 < CH / 32; ++n2) {
      const int nt = ch * (CH / 32) + n2;
      f32x4 kk_acc = {0, 0, 0, 0}, qk_acc = {0, 0, 0, 0};
      float bK[DK / 4];
      row_quarter<DK>(bK, sK + nt * 16 * LD, LD);
      mma2<DK>(kk_acc, qk_acc, aK, bK, aQ, bK);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * kk + r, col = nt * 16 + i16;
        const float dec = col <= row ? __expf(sG[row] - sG[col]) : 0.f;
        sA[row * LC + col] = col < row ? sB[row] * dec * kk_acc[r] : 0.f;
        sM[row * LC + col] = col <= row ? dec * qk_acc[r] : 0.f;
      }
    }
  }
  __syncthreads();
  // Kd^T = (exp(G_C - G) k^)^T (rows >= C are zero because k^ is)
  for (int idx = tid; idx < CH * DK; idx += PNT) {
    const int d = idx / CH, r = idx % CH;
    P.KdT[idx] = sEK[r] * sK[r * LD + d];
  }
  // T = (I + A)^-1 (unit lower triangular) into sT2, in 16 x 16 blocks.
  // Diagonal blocks by forward substitution (wave w < 4: block w, lane j <
  // 16 owns column j); then, by block diagonal d = I - J = 1, 2, 3 (one block
  // per wave), T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ on the MFMA.
  if (wave < CH / 16) {
    const int I = wave, j = lane & 15;
    const float* Ab = sA + (16 * I) * LC + 16 * I;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc += Ab[r * LC + i] * t[i];
      t[r] = (r > j) ? -acc : t[r];
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sT2[(16 * I + i) * LC + 16 * I + j] = t[i];
    }
  }
  {
    for (int idx = tid; idx < CH * CH; idx += PNT) {  // blocks above the diagonal
      const int r = idx / CH, cc = idx % CH;
      if ((cc >> 4) > (r >> 4)) sT2[r * LC + cc] = 0.f;
    }
  }
  __syncthreads();
  {
    const int i16 = lane & 15, kk = lane >> 4;
    float* X = sX + wave * 16 * XS;
    for (int d = 1; d < CH / 16; ++d) {
      if (wave < CH / 16 - d) {
        const int J = wave, I = wave + d;
        f32x4 x = {0, 0, 0, 0};
        for (int K = J; K < I; ++K) mm_nn16_apart(x, sA + 16 * I * LC + 16 * K, LC, sT2 + 16 * K * LC + 16 * J, LC);
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(4 * kk + r) * XS + i16] = x[r];
        f32x4 y = {0, 0, 0, 0};
        mm_nn16_apart(y, sT2 + 16 * I * LC + 16 * I, LC, X, XS);
#pragma unroll
        for (int r = 0; r < 4; ++r) sT2[(16 * I + 4 * kk + r) * LC + 16 * J + i16] = -y[r];
      }
      __syncthreads();
    }
  }
  // T diag(beta gamma) -> sA (A is no longer needed), T diag(beta) -> sT2
  for (int idx = tid; idx < CH * CH; idx += PNT) {
    const int r = idx / CH, cc = idx % CH;
    const float tv = sT2[r * LC + cc];
    sA[r * LC + cc] = tv * sB[cc] * sEG[cc];
    sT2[r * LC + cc] = tv * sB[cc];
  }
  __syncthreads();
  // W = (T diag(beta gamma)) K^, Ut = (T diag(beta)) V; wave w: rows of tile
  // w % 4, column tiles of half w / 4
  constexpr int NTILE = DK / 16 / 2;
  f32x4 wacc[NTILE], uacc[NTILE];
  {
    float a0[CH / 4], a1[CH / 4];
    row_quarter<CH>(a0, sA + rt * 16 * LC, LC);
    row_quarter<CH>(a1, sT2 + rt * 16 * LC, LC);
#pragma unroll
    for (int n = 0; n < NTILE; ++n) {
      const int nt = ch * NTILE + n;
      wacc[n] = (f32x4){0, 0, 0, 0};
      uacc[n] = (f32x4){0, 0, 0, 0};
      float b0[CH / 4], b1[CH / 4];
      col_quarter<CH>(b0, sK + nt * 16, LD);
      col_quarter<CH>(b1, sV + nt * 16, LD);
      mma2<CH>(wacc[n], uacc[n], a0, b0, a1, b1);
    }
  }
  __syncthreads();  // sK, sV fully read: reuse them for W and Ut
  {
    const int i16 = lane & 15, kk = lane >> 4;
#pragma unroll
    for (int n = 0; n < NTILE; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * kk + r, col = (ch * NTILE + n) * 16 + i16;
        const bool ok = row < C;
        const float w = ok ? wacc[n][r] : 0.f, u = ok ? uacc[n][r] : 0.f;
        sK[row * LD + col] = w;
        sV[row * LD + col] = u;
        P.W[row * DK + col] = w;
      }
  }
  __syncthreads();
  for (int idx = tid; idx < CH * DV; idx += PNT) {  // Ut^T
    const int d = idx / CH, r = idx % CH;
    P.UtT[idx] = sV[r * LD + d];
  }
  // Qp = gamma Q - Mqk W, Up = Mqk Ut
  {
    const int i16 = lane & 15, kk = lane >> 4;
    float am[CH / 4];
    row_quarter<CH>(am, sM + rt * 16 * LC, LC);
#pragma unroll
    for (int n = 0; n < NTILE; ++n) {
      const int nt = ch * NTILE + n;
      f32x4 mw = {0, 0, 0, 0}, mu = {0, 0, 0, 0};
      float b0[CH / 4], b1[CH / 4];
      col_quarter<CH>(b0, sK + nt * 16, LD);
      col_quarter<CH>(b1, sV + nt * 16, LD);
      mma2<CH>(mw, mu, am, b0, am, b1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rt * 16 + 4 * kk + r, col = nt * 16 + i16;
        const bool ok = row < C;
        P.Qp[row * DK + col] = ok ? sEG[row] * sQ[row * LD + col] - mw[r] : 0.f;
        P.Up[row * DK + col] = ok ? mu[r] : 0.f;
      }
    }
  }
}

// ------------------------------------------------------- chunk scan
// One workgroup (eight waves) per (16 rows of S, head, seq): rows j0 .. j0+15
// of S carried over the chunks in order,
//   U = Ut - W S^T,   S <- gC S + U^T Kd.
// Chunk c + 1's W [CH][DK], Kd^T [DK][CH] and the 16 rows of Ut^T go global ->
// LDS by buffer_load ... lds while chunk c computes (two-stage ring; 16-byte
// piece p of row r stored at p ^ (r % 16), so that the 128-bit operand reads
// of 16 consecutive rows hit distinct banks), and chunk c + 2 is pulled into
// L2 (one 4-byte copy per 128-byte line, into a scratch corner of LDS) so
// that the copies of the next step hit L2.  Per chunk, two barriers:
//   U phase: waves 0..3 compute U for token tile w (32 fp32 MFMAs over all
//   of K), stored transposed [j][t] (the next phase reads it along t);
//   update: wave w updates S columns 16w .. 16w+15 from U^T and Kd^T
//   (16 MFMAs).
// The entry state of every chunk is written for the output kernel; the final
// state to the slot.  All Dv/16 row blocks of a (seq, head) read the same W
// and Kd, so they are placed on one XCD (workgroups go to XCDs round-robin
// by linear index): index = x + 8 ((g / 8) Dv/16 + jb) for group g = seq*H + head.
constexpr int N_XCD = 8;
constexpr int SCAN_NT = 512;
constexpr int SCAN_MAX_CHUNKS = 1024;  // chunks per sequence and call (65,536 tokens)
template <int DK, int SCAN_NT_ = SCAN_NT>
struct ScanLds {
  static constexpr int W_B = CH * DK * 4;     // W tile
  static constexpr int K_B = DK * CH * 4;     // Kd^T tile
  static constexpr int U_B = 16 * CH * 4;     // 16 rows of Ut^T
  static constexpr int STAGE = W_B + K_B + U_B;
  static constexpr int LS = DK + 4;           // S rows (floats)
  static constexpr int LP = CH + 4;           // U^T rows (floats)
  static constexpr int S_OFF = 2 * STAGE;
  static constexpr int P_OFF = S_OFF + 16 * LS * 4;
  static constexpr int X_OFF = P_OFF + 16 * LP * 4;  // L2 warm-up landing (4 bytes per lane)
  static constexpr int G_OFF = X_OFF + SCAN_NT_ * 4;      // gC of every chunk
  static constexpr int bytes = G_OFF + SCAN_MAX_CHUNKS * 4;
};
template <int DK>
__global__ __launch_bounds__(SCAN_NT, 1) void gdn_chunk_scan_kernel(GdnArgs a, int n_groups) {
  static_assert(DK == 64 || DK == 128, "scan tiling");
  using L = ScanLds<DK>;
  constexpr int LS = L::LS, LP = L::LP;
  constexpr int WI = L::W_B / 1024 / 8;       // W copy instructions per wave
  constexpr int KI = L::K_B / 1024 / 8;       // Kd^T copy instructions per wave
  constexpr int WPR = DK / 4;                 // 16-byte pieces per W row
  extern __shared__ __align__(16) uint8_t scan_smem[];
  float* sS = reinterpret_cast<float*>(scan_smem + L::S_OFF);
  float* sP = reinterpret_cast<float*>(scan_smem + L::P_OFF);   // U^T [16][LP]
  constexpr int NJB = DK / 16;
  const int xcd = blockIdx.x % N_XCD, q = blockIdx.x / N_XCD;
  const int g = (q / NJB) * N_XCD + xcd;
  if (g >= n_groups) return;
  const int j0 = (q % NJB) * 16, h = g % a.H, b = g / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, kk = lane >> 4;
  float* Sg = a.state + ((int64_t)a.seq_slot[b] * a.H + h) * (int64_t)DK * DK;  // [Dv][Dk]
  const bool fresh = a.pos[b] == 0;
  for (int idx = tid; idx < 16 * DK; idx += SCAN_NT) {
    const int j = idx / DK, k = idx % DK;
    sS[j * LS + k] = fresh ? 0.f : Sg[(int64_t)(j0 + j) * DK + k];
  }
  // copy sources (byte offsets within a chunk's tile): W instruction n =
  // WI wave + i fills rows (64 / WPR) n .., lane l row + l / WPR, piece
  // l % WPR holding logical piece (l % WPR) ^ (row % 16); Kd^T and Ut^T rows
  // hold 16 pieces: 4 rows per instruction
  int w_src[WI], k_src[KI], u_src;
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = (64 / WPR) * (wave * WI + i) + lane / WPR, p = lane % WPR;
    w_src[i] = (row * DK + ((p ^ (row & 15)) * 4)) * 4;
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int row = 4 * (wave * KI + i) + (lane >> 4), p = lane & 15;
    k_src[i] = (row * CH + ((p ^ (row & 15)) * 4)) * 4;
  }
  {
    const int row = 4 * (wave & 3) + (lane >> 4), p = lane & 15;  // waves 0..3: Ut^T rows
    u_src = ((j0 + row) * CH + ((p ^ (row & 15)) * 4)) * 4;
  }
  const int64_t cb0 = ((int64_t)b * a.H + h) * a.n_chunks;
  const int64_t mat = (int64_t)CH * DK;
  const auto w_rsrc = buffer_rsrc(a.W + cb0 * mat, (uint32_t)(a.n_chunks * mat * 4));
  const auto k_rsrc = buffer_rsrc(a.Kd + cb0 * mat, (uint32_t)(a.n_chunks * mat * 4));
  const auto u_rsrc = buffer_rsrc(a.Ut + cb0 * mat, (uint32_t)(a.n_chunks * mat * 4));
  // L2 warm-up source: the workgroup's share of the chunk (1/8 of the head's
  // W and Kd^T lines, its own 32 lines of Ut^T), one source tensor per wave
  // (wave-uniform, w % 3; lanes 32..63 repeat 0..31), so that every wave
  // issues exactly one copy
  const int xw = __builtin_amdgcn_readfirstlane(wave) % 3, jb = j0 / 16;
  const __amdgpu_buffer_rsrc_t x_rsrc = xw == 0 ? w_rsrc : (xw == 1 ? k_rsrc : u_rsrc);
  const int x_src = xw < 2 ? (jb * 32 + (lane & 31)) * 128 : j0 * CH * 4 + (lane & 31) * 128;
#define SCAN_WARM(c_)                                                                             \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lds_void*)(scan_smem + L::X_OFF + wave * 256), 4, \
                                           x_src, (c_) * (int)mat * 4, 0, 0);
#define SCAN_COPY(c_, st_)                                                                        \
  {                                                                                               \
    uint8_t* S_ = scan_smem + (st_) * L::STAGE;                                                   \
    const int so_ = (c_) * (int)mat * 4;                                                          \
    _Pragma("unroll") for (int i = 0; i < WI; ++i)                                                \
        copy16_to_lds(w_rsrc, w_src[i], so_, (lds_void*)(S_ + (wave * WI + i) * 1024));          \
    _Pragma("unroll") for (int i = 0; i < KI; ++i)                                                \
        copy16_to_lds(k_rsrc, k_src[i], so_, (lds_void*)(S_ + L::W_B + (wave * KI + i) * 1024)); \
    if (wave < 4) copy16_to_lds(u_rsrc, u_src, so_, (lds_void*)(S_ + L::W_B + L::K_B + wave * 1024)); \
  }
  float* sG = reinterpret_cast<float*>(scan_smem + L::G_OFF);
  for (int i = tid; i < a.n_chunks; i += SCAN_NT) sG[i] = a.gC[cb0 + i];
  // Issue order per chunk c: the copies of chunk c + 1, the warm-up of chunk
  // c + 2, the entry-state store of chunk c (all unconditional, clamped to
  // the last chunk, so every wave has the same operations in flight): at the
  // top of chunk c + 1, vmcnt(2) means its copies have landed.
  SCAN_COPY(0, 0);
  SCAN_WARM(min(1, a.n_chunks - 1));
  for (int c = 0; c < a.n_chunks; ++c) {
    // chunk c has landed (this wave's copies) and every wave has finished
    // chunk c - 1
    wait_vmcnt<2>();
    lds_barrier();  // (a fence here would drain the warm-up and the store)
    const uint8_t* st = scan_smem + (c & 1) * L::STAGE;
    {
      const int cn = min(c + 1, a.n_chunks - 1);  // past the end: the idle stage, harmlessly
      SCAN_COPY(cn, (c + 1) & 1);
      SCAN_WARM(min(c + 2, a.n_chunks - 1));
    }
    const float gC = sG[c];
    // entry state of chunk c (every lane stores; for Dk = 64 the second half
    // of the workgroup repeats the first)
    {
      const ChunkPtr P = chunk_ptr(a, b, h, c, DK);
      const int e = tid % (4 * DK);
      const int j = e / (DK / 4), k4 = (e % (DK / 4)) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(sS + j * LS + k4);
      *reinterpret_cast<f32x4*>(P.S + (int64_t)(j0 + j) * DK + k4) = v;
    }
    // U phase (waves 0..3): U^T[j][t] = Ut^T[j][t] - sum_k W[t][k] S[j][k]
    // for tokens t of tile wave.  Lane group kk takes k = DK/4 kk .. (a
    // permutation of K applied to both operands): 128-bit reads.
    if (wave < 4) {
      constexpr int KQ4 = DK / 4;
      const int row = 16 * wave + i16;
      const float* wr = reinterpret_cast<const float*>(st) + row * DK;
      const float* sr = sS + i16 * LS + KQ4 * kk;
      float av[KQ4], bv[KQ4];
#pragma unroll
      for (int qq = 0; qq < KQ4 / 4; ++qq) {
        const int pc = (KQ4 * kk) / 4 + qq;
        const f32x4 x = *reinterpret_cast<const f32x4*>(wr + 4 * (pc ^ (row & 15)));
        const f32x4 y = *reinterpret_cast<const f32x4*>(sr + 4 * qq);
#pragma unroll
        for (int e = 0; e < 4; ++e) { av[4 * qq + e] = x[e]; bv[4 * qq + e] = y[e]; }
      }
      f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < KQ4; i += 2) {
        acc0 = mfma16x16x4f32(av[i], bv[i], acc0);
        acc1 = mfma16x16x4f32(av[i + 1], bv[i + 1], acc1);
      }
      acc0 += acc1;
      // lane holds W S^T [t = 16 wave + 4 kk + r][j = i16]
      const float* ut = reinterpret_cast<const float*>(st + L::W_B + L::K_B) + i16 * CH;
      const int pc = 4 * wave + kk;  // Ut^T piece of t = 16 wave + 4 kk ..
      const f32x4 u = *reinterpret_cast<const f32x4*>(ut + 4 * (pc ^ i16));
      *reinterpret_cast<f32x4*>(sP + i16 * LP + 16 * wave + 4 * kk) = u - acc0;
    }
    lds_barrier();  // the next chunk's copies stay in flight
    // update: S[j][k] = gC S[j][k] + sum_t U[t][j] Kd[t][k] for the columns
    // k = 16 wave + i16.  Lane group kk takes t = 16 kk .. + 15.
    if (wave < DK / 16) {
      const float* kd = reinterpret_cast<const float*>(st + L::W_B) + (16 * wave + i16) * CH;
      const float* uu = sP + i16 * LP + 16 * kk;
      float av[16], bv[16];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int pc = 4 * kk + qq;
        const f32x4 u = *reinterpret_cast<const f32x4*>(uu + 4 * qq);
        const f32x4 y = *reinterpret_cast<const f32x4*>(kd + 4 * (pc ^ i16));
#pragma unroll
        for (int e = 0; e < 4; ++e) { av[4 * qq + e] = u[e]; bv[4 * qq + e] = y[e]; }
      }
      f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        acc0 = mfma16x16x4f32(av[i], bv[i], acc0);
        acc1 = mfma16x16x4f32(av[i + 1], bv[i + 1], acc1);
      }
      acc0 += acc1;
      // lane holds dS[j = 4 kk + r][k = 16 wave + i16]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* sp = sS + (4 * kk + r) * LS + 16 * wave + i16;
        *sp = gC * *sp + acc0[r];
      }
    }
  }
#undef SCAN_COPY
#undef SCAN_WARM
  wait_vmem();
  __syncthreads();
  for (int idx = tid; idx < 16 * DK; idx += SCAN_NT) {
    const int j = idx / DK, k = idx % DK;
    Sg[(int64_t)(j0 + j) * DK + k] = sS[j * LS + k];
  }
}

// ------------------------------------------------------- chunk output
// grid (chunk, head, seq), eight waves: O = Qp S_c^T + Up, then per token
// and head y = RMSNorm(o; g_o) * SiLU(z) -> bf16.
constexpr int ONT = 512;
template <int DK>
__global__ __launch_bounds__(ONT, 1) void gdn_chunk_out_kernel(GdnArgs a) {
  constexpr int DV = DK;
  constexpr int LD = DK + 4;
  constexpr int NQ = CH * DK / 4 / ONT;  // 16-byte pieces of Qp per thread
  constexpr int NS = DV * DK / 4 / ONT;  // of S_c
  constexpr int PER = DV / 8;            // output dims per thread (8 threads per row)
  static_assert(NQ * 4 * ONT == CH * DK && NS * 4 * ONT == DV * DK && CH * 8 == ONT, "thread split");
  extern __shared__ __align__(16) float gsm[];
  float* sQ = gsm;             // Qp [CH][LD], later O
  float* sS = sQ + CH * LD;    // S_c [DV][LD]
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int C = min(CH, a.T - c * CH);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ChunkPtr P = chunk_ptr(a, b, h, c, DK);
  // every global read first: Qp and S_c (for LDS), this thread's row piece
  // of Up and of the gate z
  const int r = tid >> 3, d0 = (tid & 7) * PER;
  const int64_t m = (int64_t)b * a.T + c * CH + min(r, C - 1);
  u32x4 rq[NQ], rs[NS], ru[PER / 4], rz[PER / 8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) rq[i] = *reinterpret_cast<const u32x4*>(P.Qp + (tid + i * ONT) * 4);
#pragma unroll
  for (int i = 0; i < NS; ++i) rs[i] = *reinterpret_cast<const u32x4*>(P.S + (tid + i * ONT) * 4);
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) ru[i] = *reinterpret_cast<const u32x4*>(P.Up + r * DK + d0 + 4 * i);
  const uint16_t* z = a.proj + m * a.proj_stride + a.off_z + h * DV + d0;
#pragma unroll
  for (int i = 0; i < PER / 8; ++i) rz[i] = *reinterpret_cast<const u32x4*>(z + 8 * i);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = (tid + i * ONT) * 4;
    *reinterpret_cast<u32x4*>(sQ + (e / DK) * LD + e % DK) = rq[i];
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = (tid + i * ONT) * 4;
    *reinterpret_cast<u32x4*>(sS + (e / DK) * LD + e % DK) = rs[i];
  }
  __syncthreads();
  // O = Qp S_c^T (+ Up below); wave w: rows of tile w % 4, the column
  // tiles of half w / 4, in pairs
  constexpr int NTILE = DV / 16 / 2;
  static_assert(NTILE % 2 == 0, "tile pairs");
  const int rt = wave & 3, ch = wave >> 2;
  f32x4 acc[NTILE];
  const int i16 = lane & 15, kk = lane >> 4;
#pragma unroll
  for (int n = 0; n < NTILE; n += 2) {
    const int nt = ch * NTILE + n;
    acc[n] = (f32x4){0, 0, 0, 0};
    acc[n + 1] = (f32x4){0, 0, 0, 0};
    mm_nt2s(acc[n], acc[n + 1], sQ + rt * 16 * LD, LD, sS + nt * 16 * LD, sS + (nt + 1) * 16 * LD, LD, DK);
  }
  __syncthreads();  // sQ fully read: reuse it for O
#pragma unroll
  for (int n = 0; n < NTILE; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) sQ[(rt * 16 + 4 * kk + q) * LD + (ch * NTILE + n) * 16 + i16] = acc[n][q];
  __syncthreads();
  // per token and head: y = RMSNorm(O + Up; g_o) * SiLU(z) -> bf16
  float v[PER];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[4 * i + e] = sQ[r * LD + d0 + 4 * i + e] + __uint_as_float(ru[i][e]);
      ss += v[4 * i + e] * v[4 * i + e];
    }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) ss += __shfl_xor(ss, o, 64);
  const float inv = rsqrtf(ss / DV + a.eps);
  if (r < C) {
    uint16_t* y = a.out + m * a.out_stride + h * DV + d0;
#pragma unroll
    for (int i = 0; i < PER / 8; ++i) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float f[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k = 8 * i + 2 * w + e;
          const float zf = bf2f((uint16_t)(rz[i][w] >> (16 * e)));
          f[e] = v[k] * inv * bf2f(a.o_norm[d0 + k]) * siluf_(zf);
        }
        o[w] = (uint32_t)f2bf_bits(f[0]) | ((uint32_t)f2bf_bits(f[1]) << 16);
      }
      *reinterpret_cast<u32x4*>(y + 8 * i) = o;
    }
  }
}

// ------------------------------------------------------------- decode
// Token-by-token recurrence (decode: one token per sequence; the tokens of a
// call in order).  One workgroup per (sequence, head) keeps the whole state
// S [Dv][Dk] in registers (eight waves): load j of wave w covers RPI whole
// rows, lane l holding the 4 entries k = 4 (l % CPR) .. of row
// w Dv/8 + j RPI + l / CPR,
// so every load and store is a contiguous 1 KB per wave.  Per row the two
// dot products S k and S q are reduced over the row's CPR lanes; then
//   u = beta (v - alpha S k),  S <- alpha S + u k^T,  o = S q,
// and wave 0 applies the output RMSNorm over Dv (gain g_o) times SiLU(z).
constexpr int DEC_W = 8;             // waves per workgroup of the decode recurrence

template <int DK>
__global__ __launch_bounds__(64 * DEC_W) void gdn_decode_kernel(GdnArgs a) {
  constexpr int CPR = DK / 4;           // 16-byte pieces per row of S
  constexpr int RPI = 64 / CPR;         // rows per wave load
  constexpr int NI = DK / DEC_W / RPI;  // loads per lane (each wave holds DK / DEC_W rows)
  static_assert(NI >= 1, "rows per wave");
  __shared__ float sq[DK], sk[DK], sv[DK], so[DK];
  __shared__ float sab[2];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kq = (lane % CPR) * 4;
  const int row0 = wave * (DK / DEC_W) + lane / CPR;  // row of load j: row0 + j * RPI
  float* Sg = a.state + ((int64_t)a.seq_slot[b] * a.H + h) * (int64_t)DK * DK + (int64_t)row0 * DK + kq;
  const bool fresh = a.pos[b] == 0;
  f32x4 S[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j)
    S[j] = fresh ? (f32x4){0, 0, 0, 0} : *reinterpret_cast<const f32x4*>(Sg + (int64_t)j * RPI * DK);
  for (int t = 0; t < a.T; ++t) {
    const int64_t m = (int64_t)b * a.T + t;
    const uint16_t* pr = a.proj + m * a.proj_stride;
    __syncthreads();  // the previous token's vectors are consumed
    if (wave == 0) {
      float qv[DK / 64], kv[DK / 64], s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        qv[e] = bf2f(pr[a.off_q + h * DK + lane + 64 * e]);
        kv[e] = bf2f(pr[a.off_k + h * DK + lane + 64 * e]);
        sv[lane + 64 * e] = bf2f(pr[a.off_v + h * DK + lane + 64 * e]);
        s1 += qv[e] * qv[e];
        s2 += kv[e] * kv[e];
      }
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      const float iq = rsqrtf(s1 + a.eps) * a.q_scale, ik = rsqrtf(s2 + a.eps);
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        sq[lane + 64 * e] = qv[e] * iq;
        sk[lane + 64 * e] = kv[e] * ik;
      }
      if (lane == 0) {
        sab[0] = expf(-softplusf_(bf2f(pr[a.off_a + h])));
        sab[1] = sigmoidf_(bf2f(pr[a.off_b + h]));
      }
    }
    __syncthreads();
    const float alpha = sab[0], beta = sab[1];
    const f32x4 kk = *reinterpret_cast<const f32x4*>(sk + kq);
    const f32x4 qq = *reinterpret_cast<const f32x4*>(sq + kq);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      float p = S[j][0] * kk[0] + S[j][1] * kk[1] + S[j][2] * kk[2] + S[j][3] * kk[3];
#pragma unroll
      for (int off = 1; off < CPR; off <<= 1) p += __shfl_xor(p, off, 64);
      const int row = row0 + j * RPI;
      const float u = beta * (sv[row] - alpha * p);
      S[j] = alpha * S[j] + u * kk;
      float o = S[j][0] * qq[0] + S[j][1] * qq[1] + S[j][2] * qq[2] + S[j][3] * qq[3];
#pragma unroll
      for (int off = 1; off < CPR; off <<= 1) o += __shfl_xor(o, off, 64);
      if (lane % CPR == 0) so[row] = o;
    }
    __syncthreads();
    if (wave == 0) {
      float v[DK / 64], ss = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        v[e] = so[lane + 64 * e];
        ss += v[e] * v[e];
      }
      ss = wave_sum(ss);
      const float inv = rsqrtf(ss / DK + a.eps);
      const uint16_t* z = pr + a.off_z + h * DK;
      uint16_t* y = a.out + m * a.out_stride + h * DK;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        const int d = lane + 64 * e;
        y[d] = f2bf_bits(v[e] * inv * bf2f(a.o_norm[d]) * siluf_(bf2f(z[d])));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NI; ++j) *reinterpret_cast<f32x4*>(Sg + (int64_t)j * RPI * DK) = S[j];
}

template <typename K>
hipError_t set_lds(K k, size_t bytes) {
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int DK>
hipError_t prefill_dk(const GdnArgs& a, int B, hipStream_t s) {
  if (a.n_chunks > SCAN_MAX_CHUNKS) return hipErrorInvalidValue;
  const size_t lds_prep = (3 * CH * (DK + 4) + 3 * CH * (CH + 4) + 4 * CH + 4 * 16 * 20) * sizeof(float);
  const size_t lds_out = (CH * (DK + 4) + DK * (DK + 4)) * sizeof(float);
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds(gdn_chunk_prep_kernel<DK>, lds_prep);
    if (e == hipSuccess) e = set_lds(gdn_chunk_out_kernel<DK>, lds_out);
    if (e == hipSuccess) e = set_lds(gdn_chunk_scan_kernel<DK>, ScanLds<DK>::bytes);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(gdn_chunk_prep_kernel<DK>, dim3(a.n_chunks, a.H, B), dim3(PNT), lds_prep, s, a);
  const int groups = (a.H * B + N_XCD - 1) / N_XCD * N_XCD;
  hipLaunchKernelGGL(gdn_chunk_scan_kernel<DK>, dim3(groups * (DK / 16)), dim3(SCAN_NT), ScanLds<DK>::bytes, s, a,
                     a.H * B);
  hipLaunchKernelGGL(gdn_chunk_out_kernel<DK>, dim3(a.n_chunks, a.H, B), dim3(ONT), lds_out, s, a);
  return hipGetLastError();
}

template <int DK>
hipError_t recurrent_dk(const GdnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(gdn_decode_kernel<DK>, dim3(a.H, B), dim3(64 * DEC_W), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gdn_chunks(int T) { return (T + CH - 1) / CH; }

hipError_t launch_gdn_prefill(const GdnArgs& a, int B, hipStream_t s) {
  if (B == 0 || a.T == 0) return hipSuccess;
  if (a.Dk == 128) return prefill_dk<128>(a, B, s);
  if (a.Dk == 64) return prefill_dk<64>(a, B, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gdn_recurrent(const GdnArgs& a, int B, hipStream_t s) {
  if (B == 0 || a.T == 0) return hipSuccess;
  if (a.Dk == 128) return recurrent_dk<128>(a, B, s);
  if (a.Dk == 64) return recurrent_dk<64>(a, B, s);
  return hipErrorInvalidValue;
}
