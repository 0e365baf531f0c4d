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
// With q^ = q qs / |q| and k^ = k / |k|, the normalisations become row scales
// of the raw bf16 projections, which are then exact MFMA operands:
//   W = (T diag(beta gamma / |k|)) K,  U~ = (T diag(beta)) V,
//   Mqk[t][i] = exp(G_t - G_i) qs / (|q_t| |k_i|) (q_t . k_i)   (i <= t),
//   O = diag(gamma qs / |q|) Q S0^T + Mqk U,
//   S_C = gamma_C S0 + (diag(exp(G_C - G) / |k|) U)^T K.
// Three kernels: the chunk-local part for all chunks in parallel (prep: W,
// U~, Mqk and the row scales), the carry of S over the chunks (scan: the rows
// of S are independent, so a head's rows are split over workgroups; it keeps
// each chunk's U and the raw-query product Q S0^T with the entering state),
// and the chunk outputs for all chunks in parallel (out: O from Q S0^T and U,
// then RMSNorm over Dv times SiLU(z)).  Every product runs on the bf16 MFMA with fp32
// accumulation: a raw projection is an exact bf16 operand, and an fp32
// operand x enters as three bf16 parts hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid) (24 significant bits, the fp32 value up to its last
// bit): against an exact operand three products, against another split
// operand the six whose parts' weights reach 2^-24, so the state and the
// recurrence keep fp32 accuracy.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace {

constexpr int CH = 64;   // chunk length
constexpr int SCS = 2 * CH + 4;  // row scales per chunk: sq[CH], dk[CH], gC (padded)

DEV float softplusf_(float x) { return x > 20.f ? x : log1pf(expf(x)); }

// The 16x16 blocks of the chunk inverse use the fp32 MFMA 16x16x4.  Lane l
// supplies A[m = l%16][k = l/16] and B[k = l/16][n = l%16]; the result D holds
// rows 4*(l/16) + r (r = 0..3) of column l%16.  The result is kept apart from
// its C operand: C stays live until the result exists, so the registers cannot
// partially overlap (the compiler otherwise may place a chain's result one
// register pair off its C operand, which the hardware does not compute
// correctly).
DEV f32x4 mfma16x16x4f32_apart(float a, float b, f32x4 c) {
  const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  asm volatile("" ::"v"(c), "v"(d));
  return d;
}
// The bf16 16x16x32 MFMA with its result kept apart from its C operand (as
// above).
DEV f32x4 mfma16x16x32_apart(const bf16x8& a, const bf16x8& b, f32x4 c) {
  const f32x4 d = mfma16x16x32(a, b, c);
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

// fp32 -> (hi, lo) bf16 pair: hi = bf16(x), lo = bf16(x - hi) (x - hi is exact)
DEV void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = f2bf(x);
  lo = f2bf(x - (float)hi);
}
// fp32 -> three bf16 parts, x = hi + mid + lo to fp32's last bit (each
// difference is exact)
DEV void split3(float x, bf16& hi, bf16& mid, bf16& lo) {
  hi = f2bf(x);
  const float r = x - (float)hi;
  mid = f2bf(r);
  lo = f2bf(r - (float)mid);
}
DEV uint16_t bits(bf16 x) { return __builtin_bit_cast(uint16_t, x); }
struct Split8 {
  bf16x8 h, m, l;
};
DEV Split8 split8(const float (&x)[8]) {
  Split8 s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 a, b, c;
    split3(x[e], a, b, c);
    s.h[e] = a;
    s.m[e] = b;
    s.l[e] = c;
  }
  return s;
}
DEV Split8 split8(const f32x4& x0, const f32x4& x1) {
  const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  return split8(x);
}
// acc += a . b for a split operand and an exact one (three products)
DEV f32x4 mma_se(const Split8& a, const bf16x8& b, f32x4 acc) {
  acc = mfma16x16x32(a.h, b, acc);
  acc = mfma16x16x32(a.m, b, acc);
  return mfma16x16x32(a.l, b, acc);
}
DEV f32x4 mma_es(const bf16x8& a, const Split8& b, f32x4 acc) {
  acc = mfma16x16x32(a, b.h, acc);
  acc = mfma16x16x32(a, b.m, acc);
  return mfma16x16x32(a, b.l, acc);
}
// acc += a . b for two split operands: the six products of weight >= 2^-24
// (smallest first)
DEV f32x4 mma_ss(const Split8& a, const Split8& b, f32x4 acc) {
  acc = mfma16x16x32(a.h, b.l, acc);
  acc = mfma16x16x32(a.l, b.h, acc);
  acc = mfma16x16x32(a.m, b.m, acc);
  acc = mfma16x16x32(a.h, b.m, acc);
  acc = mfma16x16x32(a.m, b.h, acc);
  return mfma16x16x32(a.h, b.h, acc);
}
// mma_ss with every result kept apart from its C operand (the chain's
// registers cannot then partially overlap)
DEV f32x4 mma_ss_apart(const Split8& a, const Split8& b, f32x4 acc) {
  acc = mfma16x16x32_apart(a.h, b.l, acc);
  acc = mfma16x16x32_apart(a.l, b.h, acc);
  acc = mfma16x16x32_apart(a.m, b.m, acc);
  acc = mfma16x16x32_apart(a.h, b.m, acc);
  acc = mfma16x16x32_apart(a.m, b.h, acc);
  return mfma16x16x32_apart(a.h, b.h, acc);
}
DEV bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
DEV bf16x8 glb8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// A transposed [DK][CH] bf16 tile (row k holds the chunk's 64 tokens) keeps
// its 16-byte groups of 8 tokens in the order g ^ kt_swz(k): the transposing
// 2-byte writes (8 consecutive k of one token per thread) and the 16-byte
// operand reads (16 consecutive k, one group each) then spread over the LDS
// banks.
DEV int kt_swz(int k) { return (k & 7) ^ ((k >> 3) & 7); }
DEV int kt_at(int k, int t) { return k * CH + 8 * ((t >> 3) ^ kt_swz(k)) + (t & 7); }

// The fp32 chunk workspaces are stored in the order the lanes read them, so
// that a wave's 16-byte-per-lane access is one contiguous kilobyte:
//   W [CH][Dk]: element (t, k) at the fragment of (t / 16, k / 32, (k / 4) % 2):
//     lane t % 16 + 16 ((k % 32) / 8), floats k % 4;
//   U~^T / U^T [Dv][CH]: element (j, x) at the fragment of (j / 16, x / 16):
//     lane j % 16 + 16 ((x % 16) / 4), floats x % 4;
//   Q S0^T [CH][Dv]: element (t, j) at the fragment of (j / 16, t / 16):
//     lane j % 16 + 16 ((t % 16) / 4), floats t % 4 (the same form, indexed
//     jx_frag<CH>(j, t)).
// Offsets in floats within a chunk's block.
template <int DK>
DEV int w_frag(int t, int k) {
  return ((((t >> 4) * (DK / 32) + (k >> 5)) * 2 + ((k >> 2) & 1)) * 64 + (t & 15) + 16 * ((k & 31) >> 3)) * 4 +
         (k & 3);
}
template <int NX>
DEV int jx_frag(int j, int x) {  // NX: columns of the matrix (CH or Dk)
  return (((j >> 4) * (NX / 16) + (x >> 4)) * 64 + (j & 15) + 16 * ((x & 15) >> 2)) * 4 + (x & 3);
}

// Chunk workspace of (sequence b, head h, chunk c): cb = (b H + h) n_chunks + c.
DEV int64_t chunk_index(const GdnArgs& a, int b, int h, int c) {
  return ((int64_t)b * a.H + h) * a.n_chunks + c;
}

// ------------------------------------------------------- chunk prep
// grid (chunk, head, seq), four waves.  From the chunk's raw q, k, v (bf16),
// a and b: the row norms, the cumulative log-gates G and beta; K K^T and
// Q K^T on the MFMA (raw operands); A and Mqk with their row / column scales;
// T = (I + A)^-1 in fp32 (diagonal 16x16 blocks by forward substitution,
// then the blocks below by block diagonals); W and U~ (T's scaled rows as
// split operands against the raw K^T, V^T).  Writes W [CH][Dk], U~^T
// [Dv][CH], Mqk (fp32), the raw K^T tile (bf16, kt_at order) and the row
// scales sq = gamma qs / |q|,
// dk = exp(G_C - G) / |k| and gC = exp(G_C).  Rows past the sequence's end
// are zero (q = k = v = 0, beta = 0, no decay).  The barriers order LDS
// accesses only: the global stores stay in flight.
constexpr int PNT = 256;
// LDS: q and k rows, K^T, V^T, A and T, the small arrays.  Where A and T fit
// in the q and k rows (Dk = 128) they take those bytes (they are formed only
// after every wave has read q and k): 74 KB, two workgroups per CU.
template <int DK>
constexpr bool prep_alias() {
  return CH * (DK + 8) * 2 >= CH * (CH + 4) * 4;
}
template <int DK>
constexpr int prep_lds_bytes() {
  return (2 * CH * (DK + 8) + 2 * DK * CH) * 2 + ((prep_alias<DK>() ? 0 : 2 * CH * (CH + 4)) + 4 * 16 * 20 + 6 * CH) * 4;
}
template <int DK>
__global__ __launch_bounds__(PNT, 2) void gdn_prep_kernel(GdnArgs a) {
  constexpr int DV = DK;
  constexpr int LR = DK + 8;   // bf16 stride of the [CH][DK] rows
  constexpr int LA = CH + 4;   // fp32 stride of the [CH][CH] rows
  constexpr int XS = 20;       // rows of the 16x16 inverse scratch
  constexpr int PPR = DK / 8;  // 16-byte pieces per row
  constexpr int NP = CH * PPR / PNT;
  static_assert(NP * PNT == CH * PPR && PPR <= 64, "row pieces");
  extern __shared__ __align__(16) uint8_t prep_smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(prep_smem);  // [CH][LR] raw q
  uint16_t* sK = sQ + CH * LR;                            // [CH][LR] raw k
  uint16_t* sKt = sK + CH * LR;                           // [DK][CH] raw k transposed (kt_at)
  uint16_t* sVt = sKt + DK * CH;                          // [DV][CH] raw v transposed (kt_at)
  constexpr bool ALIAS = prep_alias<DK>();
  float* sA = ALIAS ? reinterpret_cast<float*>(sQ) : reinterpret_cast<float*>(sVt + DV * CH);  // [CH][LA] A
  float* sT = ALIAS ? reinterpret_cast<float*>(sK) : sA + CH * LA;                            // [CH][LA] T
  float* sX = ALIAS ? reinterpret_cast<float*>(sVt + DV * CH) : sT + CH * LA;                 // [4][16][XS]
  float* sG = sX + 4 * 16 * XS;                           // cumulative log alpha
  float* sB = sG + CH;                                    // beta
  float* sNq = sB + CH;                                   // qs / |q|
  float* sNk = sNq + CH;                                  // 1 / |k|
  float* sSw = sNk + CH;                                  // beta gamma / |k|
  float* sSu = sSw + CH;                                  // beta
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = c * CH;
  const int C = min(CH, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int64_t row0 = (int64_t)b * a.T + t0;
  const int64_t cb = chunk_index(a, b, h, c);

  // q, k, v: all loads issued first; PPR consecutive threads hold a row
  {
    u32x4 vq[NP], vk[NP], vv[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * PNT, r = p / PPR, cp = p % PPR;
      const uint16_t* pr = a.proj + (row0 + min(r, C - 1)) * a.proj_stride;
      vq[i] = *reinterpret_cast<const u32x4*>(pr + a.off_q + h * DK + cp * 8);
      vk[i] = *reinterpret_cast<const u32x4*>(pr + a.off_k + h * DK + cp * 8);
      vv[i] = *reinterpret_cast<const u32x4*>(pr + a.off_v + h * DV + cp * 8);
    }
    float av = 0.f, bv = 0.f;
    if (tid < CH) {
      const uint16_t* pr = a.proj + (row0 + min(tid, C - 1)) * a.proj_stride;
      av = bf2f(pr[a.off_a + h]);
      bv = bf2f(pr[a.off_b + h]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * PNT, r = p / PPR, cp = p % PPR;
      if (r >= C) vq[i] = vk[i] = vv[i] = (u32x4){0, 0, 0, 0};
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = bf2f((uint16_t)(vq[i][e >> 1] >> ((e & 1) * 16)));
        const float k = bf2f((uint16_t)(vk[i][e >> 1] >> ((e & 1) * 16)));
        sq += q * q;
        sk += k * k;
      }
#pragma unroll
      for (int o = 1; o < PPR; o <<= 1) {
        sq += __shfl_xor(sq, o, 64);
        sk += __shfl_xor(sk, o, 64);
      }
      if (cp == 0) {
        sNq[r] = r < C ? rsqrtf(sq + a.eps) * a.q_scale : 0.f;
        sNk[r] = r < C ? rsqrtf(sk + a.eps) : 0.f;
      }
      *reinterpret_cast<u32x4*>(sQ + r * LR + cp * 8) = vq[i];
      *reinterpret_cast<u32x4*>(sK + r * LR + cp * 8) = vk[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKt[kt_at(cp * 8 + e, r)] = (uint16_t)(vk[i][e >> 1] >> ((e & 1) * 16));
        sVt[kt_at(cp * 8 + e, r)] = (uint16_t)(vv[i][e >> 1] >> ((e & 1) * 16));
      }
    }
    if (tid < CH) {
      sG[tid] = tid < C ? -softplusf_(av) : 0.f;
      sB[tid] = tid < C ? sigmoidf_(bv) : 0.f;
    }
  }
  lds_barrier();
  if (wave == 0) {  // inclusive prefix sum of log alpha over the 64 rows
    float g = sG[lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(g, o, 64);
      if (lane >= o) g += u;
    }
    sG[lane] = g;
  }
  lds_barrier();
  {  // the raw K^T tile (its swizzled LDS layout) for the scan's stage
    uint16_t* kt = a.Kt + cb * DK * CH;
#pragma unroll
    for (int i = 0; i < DK * CH / 8 / PNT; ++i) {
      const int p = tid + i * PNT;
      *reinterpret_cast<u32x4*>(kt + 8 * p) = *reinterpret_cast<const u32x4*>(sKt + 8 * p);
    }
  }
  const float GC = sG[C - 1];
  if (tid < CH) {
    const float g = sG[tid];
    sSw[tid] = sB[tid] * __expf(g) * sNk[tid];
    sSu[tid] = sB[tid];
    float* sc = a.sc + cb * SCS;
    sc[tid] = tid < C ? __expf(g) * sNq[tid] : 0.f;             // sq
    sc[CH + tid] = tid < C ? __expf(GC - g) * sNk[tid] : 0.f;   // dk
    if (tid == 0) sc[2 * CH] = __expf(GC);                      // gC
  }
  // K K^T -> A (strictly lower), Q K^T -> Mqk (lower incl. diagonal): the 10
  // lower 16x16 tiles of each; wave w takes jobs w, w + 4, ... (five each).
  // All products first, then a barrier: A overwrites the q and k rows.
  {
    float* Mq = a.Mq + cb * CH * CH;
    f32x4 accs[5];
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      const int job = wave + 4 * n;
      const bool qk = job >= 10;
      int q = qk ? job - 10 : job, I = 0;
      while (q > I) { q -= I + 1; ++I; }
      const int J = q;  // tile (I, J), J <= I
      const uint16_t* src = qk ? sQ : sK;
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        acc = mfma16x16x32_apart(lds8(src + (16 * I + l16) * LR + 32 * ks + 8 * lq),
                                 lds8(sK + (16 * J + l16) * LR + 32 * ks + 8 * lq), acc);
      accs[n] = acc;
    }
    lds_barrier();
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      const int job = wave + 4 * n;
      const bool qk = job >= 10;
      int q = qk ? job - 10 : job, I = 0;
      while (q > I) { q -= I + 1; ++I; }
      const int J = q;
      const f32x4 acc = accs[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * I + 4 * lq + r, col = 16 * J + l16;
        const float dec = col <= row ? __expf(sG[row] - sG[col]) : 0.f;
        if (!qk) {
          sA[row * LA + col] = col < row ? sB[row] * dec * sNk[row] * sNk[col] * acc[r] : 0.f;
        } else {
          Mq[row * CH + col] = dec * sNq[row] * sNk[col] * acc[r];
        }
      }
    }
    // the upper tiles: zero
    for (int idx = tid; idx < CH * CH; idx += PNT) {
      const int r = idx / CH, cc = idx % CH;
      if ((cc >> 4) > (r >> 4)) {
        sA[r * LA + cc] = 0.f;
        sT[r * LA + cc] = 0.f;
        Mq[idx] = 0.f;
      }
    }
  }
  lds_barrier();
  // T = (I + A)^-1, unit lower triangular.  Diagonal blocks by forward
  // substitution (wave w: block w, lane j < 16 owns column j); then, by block
  // diagonal d = I - J = 1, 2, 3 (one block per wave),
  // T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ on the fp32 MFMA.
  {
    const int I = wave, j = l16;
    const float* Ab = sA + (16 * I) * LA + 16 * I;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc += Ab[r * LA + i] * t[i];
      t[r] = (r > j) ? -acc : t[r];
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sT[(16 * I + i) * LA + 16 * I + j] = t[i];
    }
  }
  lds_barrier();
  {
    float* X = sX + wave * 16 * XS;
    for (int d = 1; d < CH / 16; ++d) {
      if (wave < CH / 16 - d) {
        const int J = wave, I = wave + d;
        f32x4 x = {0, 0, 0, 0};
        for (int K = J; K < I; ++K) mm_nn16_apart(x, sA + 16 * I * LA + 16 * K, LA, sT + 16 * K * LA + 16 * J, LA);
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(4 * lq + r) * XS + l16] = x[r];
        f32x4 y = {0, 0, 0, 0};
        mm_nn16_apart(y, sT + 16 * I * LA + 16 * I, LA, X, XS);
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * lq + r) * LA + 16 * J + l16] = -y[r];
      }
      lds_barrier();
    }
  }
  // W = (T diag(beta gamma / |k|)) K and U~ = (T diag(beta)) V: wave w takes
  // the rows of tile w; its A operands (the scaled rows of T, split in three
  // bf16 parts) once, then every column tile of W and of U~
  {
    Split8 tw_[CH / 32], tu_[CH / 32];
#pragma unroll
    for (int is = 0; is < CH / 32; ++is) {
      const float* tr = sT + (16 * wave + l16) * LA + 32 * is + 8 * lq;
      float xw[8], xu[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * is + 8 * lq + e;
        xw[e] = tr[e] * sSw[i];
        xu[e] = tr[e] * sSu[i];
      }
      tw_[is] = split8(xw);
      tu_[is] = split8(xu);
    }
    float* W = a.W + cb * CH * DK;
    float* Ut = a.Ut + cb * CH * DV;
    // W^T = K^T (T diag(beta gamma / |k|))^T: the lane then holds four
    // consecutive k of one token row, one 16-byte fragment piece
#pragma unroll 2
    for (int nt = 0; nt < DK / 16; ++nt) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int is = 0; is < CH / 32; ++is) acc = mma_es(lds8(sKt + kt_at(16 * nt + l16, 32 * is + 8 * lq)), tw_[is], acc);
      // lane: W[t = 16 wave + l16][k = 16 nt + 4 lq + r]
      *reinterpret_cast<f32x4*>(W + w_frag<DK>(16 * wave + l16, 16 * nt + 4 * lq)) = acc;
    }
#pragma unroll 2
    for (int nt = 0; nt < DV / 16; ++nt) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int is = 0; is < CH / 32; ++is) acc = mma_se(tu_[is], lds8(sVt + kt_at(16 * nt + l16, 32 * is + 8 * lq)), acc);
      // U~^T [DV][CH]: lane (t = 16 wave + 4 lq + r, dv = 16 nt + l16)
      *reinterpret_cast<f32x4*>(Ut + jx_frag<CH>(16 * nt + l16, 16 * wave + 4 * lq)) = acc;
    }
  }
}

// ------------------------------------------------------- chunk scan
// One workgroup (eight waves) per (16 rows j0 .. j0+15 of S, head, seq),
// carrying those rows of S over the chunks in order.  Per chunk (S = the
// entering state, its three bf16 parts in LDS; the fp32 state in registers,
// wave w < Dk/16 holding S[j][16w .. 16w+15]):
//   waves 0-3, token tile w:   U = U~ - W S^T (both operands split), stored
//                              over U~^T for the output kernel, the parts of
//                              (dk U)^T into LDS;
//   waves 4-7, token tile w-4: Q S^T (raw q rows exact, S split: the output
//                              kernel's product with the entering state, in
//                              the same order), stored for it;
//   barrier;
//   waves w < Dk/16:           S^T <- gC S^T + K^T (dk U)   (raw K^T stage);
//   the next copies and loads are issued; barrier.
// The chain over the chunks is bound by memory latency, so operands run
// ahead: the U waves' register operands (W rows, U~^T, dk) and the other
// waves' q rows three chunks ahead in three register sets, the raw K^T tile two chunks ahead in three LDS
// stages (buffer_load ... lds), and a later chunk is warmed into L2.  All
// Dv/16 row blocks of a (seq, head) read the same W and K, so they are placed
// on one XCD (workgroups go to XCDs round-robin by linear index): index =
// x + 8 ((g / 8) Dv/16 + jb) for group g = seq*H + head.
constexpr int N_XCD = 8;
constexpr int SCAN_NT = 512;
constexpr int SCAN_PF = 3;  // chunks of register operands in flight (and K^T stages)
constexpr int SCAN_MAX_CHUNKS = 1024;  // chunks per sequence and call (65,536 tokens)
// Register operands of one chunk for a U wave: W rows of its token tile, U~^T
// of row j for four tokens, dk of those tokens.
template <int DK>
struct ScanRegs {
  static constexpr int LOADS = 2 * (DK / 32) + 2;  // vector loads per chunk
  f32x4 w[DK / 32][2];
  f32x4 ut, dk;
};
// Register operands of one chunk for a Q wave: the raw q rows of its token
// tile (exact bf16 MFMA operands).
template <int DK>
struct ScanQRegs {
  static constexpr int LOADS = DK / 32;
  bf16x8 q[DK / 32];
};
template <int DK>
struct ScanLds {
  static constexpr int LS = DK + 8;   // bf16 stride of the S rows
  static constexpr int LU = CH + 8;   // bf16 stride of the (dk U)^T rows
  static constexpr int S_PART = 16 * LS;
  static constexpr int U_PART = 16 * LU;
  static constexpr int K_STAGE = DK * CH;
  // Dynamic LDS: the SCAN_PF K^T stages (bf16), then the landing area of the
  // L2 warm-up (4 bytes per thread).  Every LDS target of the asynchronous
  // copies lies here; the operands the waves write themselves (S, dk U
  // parts, gC) are separate static arrays, so the compiler sees that those
  // writes cannot touch a copy in flight and does not wait for the copies.
  static constexpr int warm_off = SCAN_PF * K_STAGE * 2;
  static constexpr int bytes = warm_off + SCAN_NT * 4;
};

DEV uint2 pack4(bf16 a, bf16 b, bf16 c, bf16 d) {
  return make_uint2((uint32_t)bits(a) | ((uint32_t)bits(b) << 16), (uint32_t)bits(c) | ((uint32_t)bits(d) << 16));
}
// the three parts of four consecutive values, stored 8 bytes each at p, p +
// part, p + 2 part (bf16 elements)
DEV void put_parts4(uint16_t* p, int part, const f32x4& x) {
  bf16 h[4], m[4], l[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) split3(x[r], h[r], m[r], l[r]);
  *reinterpret_cast<uint2*>(p) = pack4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint2*>(p + part) = pack4(m[0], m[1], m[2], m[3]);
  *reinterpret_cast<uint2*>(p + 2 * part) = pack4(l[0], l[1], l[2], l[3]);
}
DEV Split8 get_parts8(const uint16_t* p, int part) {
  Split8 v;
  v.h = lds8(p);
  v.m = lds8(p + part);
  v.l = lds8(p + 2 * part);
  return v;
}

template <int DK>
__global__ __launch_bounds__(SCAN_NT, 1) void gdn_scan_kernel(GdnArgs a, int n_groups) {
  static_assert(DK == 64 || DK == 128, "scan tiling");
  using L = ScanLds<DK>;
  using R = ScanRegs<DK>;
  constexpr int DV = DK;
  constexpr int LS = L::LS, LU = L::LU;
  constexpr int NKS = DK / 32;      // 32-deep steps over Dk
  constexpr int NKB = DK / 16;      // column blocks of S (update waves)
  constexpr int NJB = DV / 16;      // row blocks of S per head (workgroups)
  constexpr int KCP = DK * CH * 2 / 1024 / 8;  // 1 KB K^T copies per wave
  static_assert(KCP * 8 * 1024 == DK * CH * 2, "K^T copies");
  extern __shared__ __align__(16) uint16_t scan_lds[];
  __shared__ __align__(16) uint16_t sS[3 * L::S_PART];   // parts of S [16][LS]
  __shared__ __align__(16) uint16_t sD[3 * L::U_PART];   // parts of (dk U)^T [16][LU]
  __shared__ float sGc[SCAN_MAX_CHUNKS];                 // gC of every chunk
  uint16_t* sKt = scan_lds;                 // SCAN_PF stages of raw K^T [DK][CH] (kt_at)
  const int xcd = blockIdx.x % N_XCD, qb = blockIdx.x / N_XCD;
  const int g = (qb / NJB) * N_XCD + xcd;
  if (g >= n_groups) return;
  const int jb = qb % NJB, j0 = jb * 16, h = g % a.H, b = g / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int tw = wave & 3;  // token tile of the U phase
  float* Sg = a.state + ((int64_t)a.seq_slot[b] * a.H + h) * (int64_t)DV * DK;
  const bool fresh = a.pos[b] == 0;
  const int64_t cb0 = chunk_index(a, b, h, 0);
  const int n = a.n_chunks;

  // the state: wave w < NKB holds S[j0 + l16][16 w + 4 lq + r]
  f32x4 S = {0, 0, 0, 0};
  if (wave < NKB && !fresh) S = *reinterpret_cast<const f32x4*>(Sg + (int64_t)(j0 + l16) * DK + 16 * wave + 4 * lq);
  auto put_state = [&]() __attribute__((always_inline)) { put_parts4(sS + l16 * LS + 16 * wave + 4 * lq, L::S_PART, S); };

  const __amdgpu_buffer_rsrc_t r_k = buffer_rsrc(a.Kt + cb0 * DK * CH, (uint32_t)(n * DK * CH * 2));
  auto copy_k = [&](int c, int st) __attribute__((always_inline)) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(sKt + st * L::K_STAGE);
#pragma unroll
    for (int i = 0; i < KCP; ++i)
      copy16_to_lds(r_k, ((wave * KCP + i) * 64 + lane) * 16, c * DK * CH * 2,
                    (lds_void*)(dst + (wave * KCP + i) * 1024));
  };
  auto load = [&](int c, R& r) __attribute__((always_inline)) {
    const int64_t cb = cb0 + c;
    const float* sc = a.sc + cb * SCS;
    r.dk = *reinterpret_cast<const f32x4*>(sc + CH + 16 * tw + 4 * lq);
    r.ut = *reinterpret_cast<const f32x4*>(a.Ut + cb * DV * CH + jx_frag<CH>(j0 + l16, 16 * tw + 4 * lq));
    const float* w = a.W + cb * CH * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      r.w[ks][0] = *reinterpret_cast<const f32x4*>(w + w_frag<DK>(16 * tw + l16, 32 * ks + 8 * lq));
      r.w[ks][1] = *reinterpret_cast<const f32x4*>(w + w_frag<DK>(16 * tw + l16, 32 * ks + 8 * lq + 4));
    }
  };
  // q rows of chunk c for a Q wave (token tile tw; rows past the sequence
  // repeat its last one)
  using QR = ScanQRegs<DK>;
  auto load_q = [&](int c, QR& r) __attribute__((always_inline)) {
    const int t = min(c * CH + 16 * tw + l16, a.T - 1);
    const uint16_t* qr = a.proj + ((int64_t)b * a.T + t) * a.proj_stride + a.off_q + h * DK + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) r.q[ks] = glb8(qr + 32 * ks);
  };
  // L2 warm-up of a later chunk: the head's W, U~^T and K^T lines (128 bytes);
  // waves 0-2 take one source each, and the Dv/16 workgroups of the head
  // share its lines.  One 4-byte copy per line into a scratch corner of LDS
  // (never read).
  const __amdgpu_buffer_rsrc_t r_w = buffer_rsrc(a.W + cb0 * CH * DK, (uint32_t)(n * CH * DK * 4));
  const __amdgpu_buffer_rsrc_t r_u = buffer_rsrc(a.Ut + cb0 * CH * DV, (uint32_t)(n * CH * DV * 4));
  auto warm = [&](int c) __attribute__((always_inline)) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if (wv >= 3) return;
    lds_void* dst = (lds_void*)(reinterpret_cast<uint8_t*>(scan_lds) + L::warm_off + wv * 256);
    const int nl = wv == 0 ? CH * DK * 4 / 128 : wv == 1 ? CH * DV * 4 / 128 : DK * CH * 2 / 128;
    const int per = (nl + NJB - 1) / NJB;
    const int li = min(jb * per + lane, nl - 1);  // lanes past the share repeat a line
    // one resource per (wave-uniform) branch: a selected resource would be a
    // per-lane value
    if (wv == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, dst, 4, c * CH * DK * 4 + li * 128, 0, 0, 0);
    else if (wv == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(r_u, dst, 4, c * CH * DV * 4 + li * 128, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r_k, dst, 4, c * DK * CH * 2 + li * 128, 0, 0, 0);
  };

  // One chunk with register set `cur` (chunk c, c % SCAN_PF == I).  Before
  // the barrier that publishes the stage, this wave's K^T copies of chunk c
  // must have landed.  The vector memory counter counts stores as well as
  // loads, so at least YOUNGER operations were issued after those copies: the
  // copies of chunk c + 1, the loads of chunks c + 1 and c + 2 of the wave's
  // register sets and its stores (U of a U wave, Q S^T of a Q wave) of chunks
  // c - 1 and c (the L2 warm-ups, issued by three of the four U waves only,
  // are not counted).
  struct NoSplit {};
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool UW = decltype(role)::value;
    using RS = std::conditional_t<UW, R, QR>;
    // a U wave's W rows of the next chunk as split operands: split during the
    // previous chunk's update, off the path from the state to U
    struct WSplit {
      Split8 w[NKS];
    };
    std::conditional_t<UW, WSplit, NoSplit> ws;
    auto split_w = [&](const RS& set) __attribute__((always_inline)) {
      if constexpr (UW) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ws.w[ks] = split8(set.w[ks][0], set.w[ks][1]);
      }
    };
    constexpr int YOUNGER = 2 * RS::LOADS + KCP + 2;
    auto step = [&](auto Ic, RS& cur, const RS& next, int c) __attribute__((always_inline)) {
      constexpr int I = decltype(Ic)::value;
      if constexpr (!UW) {
        // (Q S^T)[t][j] for the tile's tokens with the entering state, in
        // the output kernel's order (three products per 32-deep step)
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          acc = mma_es(cur.q[ks], get_parts8(sS + l16 * LS + 32 * ks + 8 * lq, L::S_PART), acc);
        // lane: t = 16 tw + 4 lq + r, j = j0 + l16
        *reinterpret_cast<f32x4*>(a.Oq + (cb0 + c) * CH * DV + jx_frag<CH>(j0 + l16, 16 * tw + 4 * lq)) = acc;
      }
      if constexpr (UW) {
        // (W S^T)[t][j] for the tile's tokens (two accumulation chains)
        f32x4 acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < NKS; ks += 2) {
          acc = mma_ss(ws.w[ks], get_parts8(sS + l16 * LS + 32 * ks + 8 * lq, L::S_PART), acc);
          acc2 = mma_ss(ws.w[ks + 1], get_parts8(sS + l16 * LS + 32 * (ks + 1) + 8 * lq, L::S_PART), acc2);
        }
        // lane: t = 16 tw + 4 lq + r, j = l16: U^T[j][t] over U~^T (read
        // into registers chunks ago), (dk U)^T[j][t] into LDS
        f32x4 u, du;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u[r] = cur.ut[r] - (acc[r] + acc2[r]);
          du[r] = u[r] * cur.dk[r];
        }
        *reinterpret_cast<f32x4*>(a.Ut + (cb0 + c) * DV * CH + jx_frag<CH>(j0 + l16, 16 * tw + 4 * lq)) = u;
        put_parts4(sD + l16 * LU + 16 * tw + 4 * lq, L::U_PART, du);
      }
      wait_vmcnt<YOUNGER>();  // this wave's K^T copies of chunk c have landed
      lds_barrier();          // the younger loads and stores stay in flight
      if (wave < NKB) {
        // S^T <- gC S^T + K^T (dk U) for the rows k = 16 wave ..
        f32x4 acc = {0, 0, 0, 0};
        const uint16_t* kt = sKt + I * L::K_STAGE;
#pragma unroll
        for (int ts = 0; ts < CH / 32; ++ts)
          acc = mma_es(lds8(kt + kt_at(16 * wave + l16, 32 * ts + 8 * lq)),
                       get_parts8(sD + l16 * LU + 32 * ts + 8 * lq, L::U_PART), acc);
        const float gC = sGc[c];
        // lane: k = 16 wave + 4 lq + r, j = l16
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = gC * S[r] + acc[r];
        put_state();
      }
      split_w(next);  // chunk c + 1's W
      // the operands ahead: K^T of chunk c + 2 into the stage chunk c - 1
      // used, the U set's chunk c + 3, the L2 warm-up of chunk c + 4 (indices
      // past the end repeat the last chunk, harmlessly, so every wave of a
      // role issues the same operations)
      copy_k(min(c + 2, n - 1), (I + 2) % SCAN_PF);
      if constexpr (UW) load(min(c + SCAN_PF, n - 1), cur);
      else load_q(min(c + SCAN_PF, n - 1), cur);
      warm(min(c + SCAN_PF + 1, n - 1));
      lds_barrier();
    };
    static_assert(SCAN_PF == 3, "three register sets");
    RS r0, r1, r2;  // the wave's register sets (W rows and U~^T, or q rows)
    copy_k(0, 0);
    if constexpr (UW) load(0, r0);
    else load_q(0, r0);
    copy_k(min(1, n - 1), 1);
    if constexpr (UW) {
      load(min(1, n - 1), r1);
      load(min(2, n - 1), r2);
    } else {
      load_q(min(1, n - 1), r1);
      load_q(min(2, n - 1), r2);
    }
    warm(min(3, n - 1));
    if (wave < NKB) put_state();
    for (int i = tid; i < n; i += SCAN_NT) sGc[i] = a.sc[(cb0 + i) * SCS + 2 * CH];
    split_w(r0);
    // everything issued so far has landed (the first chunk's wait counts
    // fewer younger operations than the later ones)
    wait_vmem();
    __syncthreads();
    // whole rounds of three chunks, then the last one or two (the loop's only
    // back edge comes from the third step, so the compiler's waits for each
    // register set stay exact)
    int c = 0;
    for (; c + SCAN_PF <= n; c += SCAN_PF) {
      step(std::integral_constant<int, 0>(), r0, r1, c);
      step(std::integral_constant<int, 1>(), r1, r2, c + 1);
      step(std::integral_constant<int, 2>(), r2, r0, c + 2);
    }
    if (c < n) step(std::integral_constant<int, 0>(), r0, r1, c);
    if (c + 1 < n) step(std::integral_constant<int, 1>(), r1, r2, c + 1);
  };
  if (wave < 4) run(std::true_type());
  else run(std::false_type());
  wait_vmem();
  if (wave < NKB) *reinterpret_cast<f32x4*>(Sg + (int64_t)(j0 + l16) * DK + 16 * wave + 4 * lq) = S;
}

// ------------------------------------------------------- chunk output
// grid (chunk, head, seq), eight waves: from Q S_c^T and U (both stored by the
// scan), O = sq * (Q S_c^T) + Mqk U, then per token y = RMSNorm(O; g_o) *
// SiLU(z) over Dv -> bf16.  A 48 KB LDS region holds the three-part bf16 B
// operand U^T (rows j, 64 columns; 16-byte groups swizzled by (j / 2) % 8 so
// that the operand reads of 16 consecutive rows and the part writes spread
// over the banks).  Several workgroups share a CU.  Wave w: token tile w % 4
// and half w / 4 of the Dv columns.
constexpr int ONT = 512;
template <int DK>
struct OutLds {
  static constexpr int PART = DK * CH;     // one part of a [Dv][64] region (bf16)
  static constexpr int bytes = 3 * PART * 2 + 2 * CH * 4;
};
DEV int u_at(int j, int t) {  // element (j, t) of a [rows][64] part
  return j * CH + 8 * ((t >> 3) ^ ((j >> 1) & 7)) + (t & 7);
}

template <int DK>
__global__ __launch_bounds__(ONT, 4) void gdn_out_kernel(GdnArgs a) {
  constexpr int DV = DK;
  using L = OutLds<DK>;
  constexpr int NJT = DV / 32;              // 16-column tiles per wave (half of Dv)
  extern __shared__ __align__(16) uint16_t out_lds[];
  uint16_t* sR = out_lds;                   // the parts region
  float* sN = reinterpret_cast<float*>(sR + 3 * L::PART);  // [2][CH] sums of squares
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int C = min(CH, a.T - c * CH);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int tw = wave & 3, jh = wave >> 2;
  const int64_t cb = chunk_index(a, b, h, c);
  const int64_t tok = (int64_t)b * a.T + c * CH;
  const float* sc = a.sc + cb * SCS;
  auto parts = [&](int j, int col) {
    Split8 v;
    const int o = u_at(j, col);
    v.h = lds8(sR + o);
    v.m = lds8(sR + L::PART + o);
    v.l = lds8(sR + 2 * L::PART + o);
    return v;
  };
  // Lane: t = 16 tw + 4 lq + r, j = Dv/2 jh + 16 jt + l16: Q S_c^T and U^T of
  // the wave's tiles, its Mqk rows and row scales
  f32x4 o1[NJT], ut[NJT], mq[CH / 32][2], sq;
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) {
    const int j = DV / 2 * jh + 16 * jt + l16;
    o1[jt] = *reinterpret_cast<const f32x4*>(a.Oq + cb * CH * DV + jx_frag<CH>(j, 16 * tw + 4 * lq));
    ut[jt] = *reinterpret_cast<const f32x4*>(a.Ut + cb * DV * CH + jx_frag<CH>(j, 16 * tw + 4 * lq));
  }
  const int t = 16 * tw + l16;
  {
    const float* mr = a.Mq + cb * CH * CH + t * CH + 8 * lq;
#pragma unroll
    for (int is = 0; is < CH / 32; ++is) {
      mq[is][0] = *reinterpret_cast<const f32x4*>(mr + 32 * is);
      mq[is][1] = *reinterpret_cast<const f32x4*>(mr + 32 * is + 4);
    }
  }
  sq = *reinterpret_cast<const f32x4*>(sc + 16 * tw + 4 * lq);
  // the U^T parts of the wave's columns and tokens into the region
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
    put_parts4(sR + u_at(DV / 2 * jh + 16 * jt + l16, 16 * tw + 4 * lq), L::PART, ut[jt]);
  lds_barrier();
  uint16_t zv[NJT][4];
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = 16 * tw + 4 * lq + r;
      zv[jt][r] = a.proj[(tok + min(tr, C - 1)) * a.proj_stride + a.off_z + h * DV + DV / 2 * jh + 16 * jt + l16];
    }
  // O = sq * O1 + Mqk U
  Split8 ms[CH / 32];
#pragma unroll
  for (int is = 0; is < CH / 32; ++is) ms[is] = split8(mq[is][0], mq[is][1]);
  f32x4 o[NJT];
  f32x4 ss = {0, 0, 0, 0};
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) {
    const int j = DV / 2 * jh + 16 * jt + l16;
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int is = 0; is < CH / 32; ++is) acc = mma_ss_apart(ms[is], parts(j, 32 * is + 8 * lq), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o[jt][r] = sq[r] * o1[jt][r] + acc[r];
      ss[r] += o[jt][r] * o[jt][r];
    }
  }
  // per token: sum of squares over Dv (16 lanes x NJT tiles here, then the
  // other half of Dv through LDS)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) ss[r] += __shfl_xor(ss[r], m, 64);
  }
  if (l16 == 0) *reinterpret_cast<f32x4*>(sN + jh * CH + 16 * tw + 4 * lq) = ss;
  lds_barrier();
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(sN + 16 * tw + 4 * lq);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(sN + CH + 16 * tw + 4 * lq);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tr = 16 * tw + 4 * lq + r;
    const float inv = rsqrtf((s0[r] + s1[r]) / DV + a.eps);
    if (tr < C) {
      uint16_t* y = a.out + (tok + tr) * a.out_stride + h * DV + DV / 2 * jh + l16;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int j = DV / 2 * jh + 16 * jt + l16;
        y[16 * jt] = f2bf_bits(o[jt][r] * inv * bf2f(a.o_norm[j]) * siluf_(bf2f(zv[jt][r])));
      }
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
      // the last token's state goes out row by row, while later rows' loads
      // are still arriving
      if (t + 1 == a.T) *reinterpret_cast<f32x4*>(Sg + (int64_t)j * RPI * DK) = S[j];
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
}

template <typename K>
hipError_t set_lds(K k, size_t bytes) {
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int DK>
hipError_t prefill_dk(const GdnArgs& a, int B, hipStream_t s) {
  if (a.n_chunks > SCAN_MAX_CHUNKS) return hipErrorInvalidValue;
  constexpr size_t lds_prep = prep_lds_bytes<DK>();
  constexpr size_t lds_scan = ScanLds<DK>::bytes;
  constexpr size_t lds_out = OutLds<DK>::bytes;
  static bool attr = false;
  if (!attr) {
    hipError_t e = set_lds(gdn_prep_kernel<DK>, lds_prep);
    if (e == hipSuccess) e = set_lds(gdn_scan_kernel<DK>, lds_scan);
    if (e == hipSuccess) e = set_lds(gdn_out_kernel<DK>, lds_out);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(gdn_prep_kernel<DK>, dim3(a.n_chunks, a.H, B), dim3(PNT), lds_prep, s, a);
  const int groups = (a.H * B + N_XCD - 1) / N_XCD * N_XCD;
  hipLaunchKernelGGL(gdn_scan_kernel<DK>, dim3(groups * (DK / 16)), dim3(SCAN_NT), lds_scan, s, a, a.H * B);
  hipLaunchKernelGGL(gdn_out_kernel<DK>, dim3(a.n_chunks, a.H, B), dim3(ONT), lds_out, s, a);
  return hipGetLastError();
}

template <int DK>
hipError_t recurrent_dk(const GdnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(gdn_decode_kernel<DK>, dim3(a.H, B), dim3(64 * DEC_W), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gdn_chunks(int T) { return (T + CH - 1) / CH; }
int gdn_chunk_scales() { return SCS; }

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
