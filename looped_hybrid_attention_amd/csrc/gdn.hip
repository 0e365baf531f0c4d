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
constexpr int NT = 256;

DEV float softplusf_(float x) { return x > 20.f ? x : log1pf(expf(x)); }

// ------------------------------------------------------- chunk prep
// grid (chunk, head, seq).  Per chunk writes (fp32):
//   W [CH][Dk], Ut [CH][Dv], Qg = gamma*q^ [CH][Dk], Kd = exp(G_C - G)*k^ [CH][Dk],
//   Mqk [CH][CH] (lower incl. diagonal), gC.
template <int DK>
__global__ __launch_bounds__(NT, 1) void gdn_chunk_prep_kernel(GdnArgs a) {
  constexpr int DV = DK;
  constexpr int PK = DK + 1;  // padded LDS rows
  __shared__ float sQ[CH][PK], sK[CH][PK], sV[CH][PK];
  __shared__ float sA[CH][CH + 1], sT[CH][CH + 1];
  __shared__ float sG[CH], sB[CH];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = c * CH;
  const int C = min(CH, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)b * a.T + t0;

  // load + L2-normalise q, k; load v.  Wave w handles rows w, w+4, ...
  for (int r = wave; r < CH; r += NT / 64) {
    float qv[DK / 64], kv[DK / 64];
    float sq = 0.f, sk = 0.f;
    const bool ok = r < C;
    const uint16_t* pr = a.proj + (row0 + r) * a.proj_stride;
#pragma unroll
    for (int e = 0; e < DK / 64; ++e) {
      const int d = lane + 64 * e;
      qv[e] = ok ? bf2f(pr[a.off_q + h * DK + d]) : 0.f;
      kv[e] = ok ? bf2f(pr[a.off_k + h * DK + d]) : 0.f;
      sq += qv[e] * qv[e];
      sk += kv[e] * kv[e];
      sV[r][d] = ok ? bf2f(pr[a.off_v + h * DV + d]) : 0.f;
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    const float iq = rsqrtf(sq + a.eps) * a.q_scale, ik = rsqrtf(sk + a.eps);
#pragma unroll
    for (int e = 0; e < DK / 64; ++e) {
      sQ[r][lane + 64 * e] = qv[e] * iq;
      sK[r][lane + 64 * e] = kv[e] * ik;
    }
    if (lane == 0) {
      const float av = ok ? bf2f(pr[a.off_a + h]) : 0.f;
      const float bv = ok ? bf2f(pr[a.off_b + h]) : 0.f;
      sG[r] = ok ? -softplusf_(av) : 0.f;  // log alpha, cumulated below
      sB[r] = ok ? sigmoidf_(bv) : 0.f;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float g = 0.f;
    for (int r = 0; r < CH; ++r) {
      g += sG[r];
      sG[r] = g;
    }
  }
  __syncthreads();
  // A (strictly lower) and Mqk (lower incl. diagonal); 16 entries per thread
  for (int idx = tid; idx < CH * CH; idx += NT) {
    const int r = idx / CH, i = idx % CH;
    float kk = 0.f, qk = 0.f;
    if (i <= r) {
#pragma unroll 8
      for (int d = 0; d < DK; ++d) {
        kk += sK[r][d] * sK[i][d];
        qk += sQ[r][d] * sK[i][d];
      }
    }
    const float dec = i <= r ? expf(sG[r] - sG[i]) : 0.f;
    sA[r][i] = i < r ? sB[r] * dec * kk : 0.f;
    a.Mqk[(((int64_t)b * a.H + h) * a.n_chunks + c) * CH * CH + idx] = i <= r ? dec * qk : 0.f;
  }
  __syncthreads();
  // T = (I + A)^-1 by forward substitution, one row at a time
  for (int idx = tid; idx < CH * CH; idx += NT) sT[idx / CH][idx % CH] = (idx / CH == idx % CH) ? 1.f : 0.f;
  __syncthreads();
  for (int r = 1; r < CH; ++r) {
    if (tid < r) {
      const int j = tid;
      float s = 0.f;
      for (int i = j; i < r; ++i) s += sA[r][i] * sT[i][j];
      sT[r][j] = -s;
    }
    __syncthreads();
  }
  // W = T diag(beta gamma) K, Ut = T diag(beta) V; Qg, Kd
  const float GC = sG[C - 1];
  const int64_t base = (((int64_t)b * a.H + h) * a.n_chunks + c) * CH * DK;
  for (int idx = tid; idx < CH * DK; idx += NT) {
    const int r = idx / DK, d = idx % DK;
    float w = 0.f, u = 0.f;
    for (int i = 0; i <= r; ++i) {
      const float t = sT[r][i] * sB[i];
      w += t * expf(sG[i]) * sK[i][d];
      u += t * sV[i][d];
    }
    const bool ok = r < C;
    a.W[base + idx] = ok ? w : 0.f;
    a.Ut[base + idx] = ok ? u : 0.f;
    a.Qg[base + idx] = ok ? expf(sG[r]) * sQ[r][d] : 0.f;
    a.Kd[base + idx] = ok ? expf(GC - sG[r]) * sK[r][d] : 0.f;
  }
  if (tid == 0) a.gC[((int64_t)b * a.H + h) * a.n_chunks + c] = expf(GC);
}

// ------------------------------------------------------- chunk scan
// grid (Dv / DS, head, seq).  S rows [j0, j0 + DS) of one head, carried over
// the chunks in order.  O (fp32, before the output norm) -> a.o.
template <int DK, int DS>
__global__ __launch_bounds__(NT, 1) void gdn_chunk_scan_kernel(GdnArgs a) {
  constexpr int PK = DK + 1;
  __shared__ float sS[DS][PK];
  __shared__ float sW[CH][PK], sQ[CH][PK], sK[CH][PK];
  __shared__ float sM[CH][CH + 1];
  __shared__ float sU[CH][DS + 1];
  const int j0 = blockIdx.x * DS, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  float* Sg = a.state + ((int64_t)a.seq_slot[b] * a.H + h) * (int64_t)DK * DK;  // [Dv][Dk]
  const bool fresh = a.pos[b] == 0;
  for (int idx = tid; idx < DS * DK; idx += NT) {
    const int j = idx / DK, k = idx % DK;
    sS[j][k] = fresh ? 0.f : Sg[(int64_t)(j0 + j) * DK + k];
  }
  for (int c = 0; c < a.n_chunks; ++c) {
    const int64_t cb = ((int64_t)b * a.H + h) * a.n_chunks + c;
    const int C = min(CH, a.T - c * CH);
    __syncthreads();
    for (int idx = tid; idx < CH * DK; idx += NT) {
      const int r = idx / DK, k = idx % DK;
      sW[r][k] = a.W[cb * CH * DK + idx];
      sQ[r][k] = a.Qg[cb * CH * DK + idx];
      sK[r][k] = a.Kd[cb * CH * DK + idx];
    }
    for (int idx = tid; idx < CH * CH; idx += NT) sM[idx / CH][idx % CH] = a.Mqk[cb * CH * CH + idx];
    __syncthreads();
    // U = Ut - W S^T  (rows r, columns j of the slice)
    for (int idx = tid; idx < CH * DS; idx += NT) {
      const int r = idx / DS, j = idx % DS;
      float s = 0.f;
#pragma unroll 8
      for (int k = 0; k < DK; ++k) s += sW[r][k] * sS[j][k];
      sU[r][j] = a.Ut[cb * CH * DK + r * DK + j0 + j] - s;
    }
    __syncthreads();
    // O = Qg S^T + Mqk U
    for (int idx = tid; idx < CH * DS; idx += NT) {
      const int r = idx / DS, j = idx % DS;
      if (r >= C) continue;
      float s = 0.f;
#pragma unroll 8
      for (int k = 0; k < DK; ++k) s += sQ[r][k] * sS[j][k];
      for (int i = 0; i <= r; ++i) s += sM[r][i] * sU[i][j];
      const int64_t m = (int64_t)b * a.T + c * CH + r;
      a.o[(m * a.H + h) * DK + j0 + j] = s;
    }
    __syncthreads();
    // S = gC S + U^T Kd
    const float gC = a.gC[cb];
    for (int idx = tid; idx < DS * DK; idx += NT) {
      const int j = idx / DK, k = idx % DK;
      float s = gC * sS[j][k];
      for (int r = 0; r < CH; ++r) s += sU[r][j] * sK[r][k];
      sS[j][k] = s;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < DS * DK; idx += NT) {
    const int j = idx / DK, k = idx % DK;
    Sg[(int64_t)(j0 + j) * DK + k] = sS[j][k];
  }
}

// ------------------------------------------------ token recurrence (decode)
// grid (Dv / 16, head, seq); 16 rows of S per workgroup, 16 threads per row.
// Tokens of the call in order (T = 1 for decode).
template <int DK>
__global__ __launch_bounds__(NT) void gdn_recurrent_kernel(GdnArgs a) {
  constexpr int RPW = 16;             // rows per workgroup
  constexpr int KPT = DK / 16;        // k per thread
  __shared__ float sq[DK], sk[DK];
  __shared__ float sred[2];
  __shared__ float sab[2];
  const int j0 = blockIdx.x * RPW, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, j = tid / 16, kq = (tid % 16) * KPT;
  float* Sg = a.state + ((int64_t)a.seq_slot[b] * a.H + h) * (int64_t)DK * DK + (int64_t)(j0 + j) * DK + kq;
  const bool fresh = a.pos[b] == 0;
  float S[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) S[e] = fresh ? 0.f : Sg[e];
  for (int t = 0; t < a.T; ++t) {
    const int64_t m = (int64_t)b * a.T + t;
    const uint16_t* pr = a.proj + m * a.proj_stride;
    __syncthreads();
    if (tid < 64) {
      float qv[DK / 64], kv[DK / 64], s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        qv[e] = bf2f(pr[a.off_q + h * DK + tid + 64 * e]);
        kv[e] = bf2f(pr[a.off_k + h * DK + tid + 64 * e]);
        s1 += qv[e] * qv[e];
        s2 += kv[e] * kv[e];
      }
      s1 = wave_sum(s1);
      s2 = wave_sum(s2);
      const float iq = rsqrtf(s1 + a.eps) * a.q_scale, ik = rsqrtf(s2 + a.eps);
#pragma unroll
      for (int e = 0; e < DK / 64; ++e) {
        sq[tid + 64 * e] = qv[e] * iq;
        sk[tid + 64 * e] = kv[e] * ik;
      }
      if (tid == 0) {
        sab[0] = expf(-softplusf_(bf2f(pr[a.off_a + h])));
        sab[1] = sigmoidf_(bf2f(pr[a.off_b + h]));
      }
    }
    __syncthreads();
    const float alpha = sab[0], beta = sab[1];
    float sk_part = 0.f;
#pragma unroll
    for (int e = 0; e < KPT; ++e) sk_part += S[e] * sk[kq + e];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) sk_part += __shfl_xor(sk_part, off, 64);
    const float v = bf2f(pr[a.off_v + h * DK + j0 + j]);
    const float u = beta * (v - alpha * sk_part);
    float oq = 0.f;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      S[e] = alpha * S[e] + u * sk[kq + e];
      oq += S[e] * sq[kq + e];
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) oq += __shfl_xor(oq, off, 64);
    if ((tid & 15) == 0) a.o[(m * a.H + h) * DK + j0 + j] = oq;
  }
#pragma unroll
  for (int e = 0; e < KPT; ++e) Sg[e] = S[e];
  (void)sred;
}

// ------------------------------------------------------- output norm
// One wave per (token, head): y = RMSNorm(o; g_o) * SiLU(z) -> bf16.
template <int DV>
__global__ __launch_bounds__(256) void gdn_out_kernel(GdnArgs a, int M) {
  const int m = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (h >= a.H) return;
  const float* o = a.o + ((int64_t)m * a.H + h) * DV;
  const uint16_t* z = a.proj + (int64_t)m * a.proj_stride + a.off_z + h * DV;
  float v[DV / 64], ss = 0.f;
#pragma unroll
  for (int e = 0; e < DV / 64; ++e) {
    v[e] = o[lane + 64 * e];
    ss += v[e] * v[e];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / DV + a.eps);
  uint16_t* y = a.out + (int64_t)m * a.out_stride + h * DV;
#pragma unroll
  for (int e = 0; e < DV / 64; ++e) {
    const int d = lane + 64 * e;
    y[d] = f2bf_bits(v[e] * inv * bf2f(a.o_norm[d]) * siluf_(bf2f(z[d])));
  }
  (void)M;
}

template <int DK>
hipError_t prefill_dk(const GdnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(gdn_chunk_prep_kernel<DK>, dim3(a.n_chunks, a.H, B), dim3(NT), 0, s, a);
  constexpr int DS = 16;
  hipLaunchKernelGGL((gdn_chunk_scan_kernel<DK, DS>), dim3(DK / DS, a.H, B), dim3(NT), 0, s, a);
  hipLaunchKernelGGL(gdn_out_kernel<DK>, dim3(B * a.T, (a.H + 3) / 4), dim3(256), 0, s, a, B * a.T);
  return hipGetLastError();
}

template <int DK>
hipError_t recurrent_dk(const GdnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(gdn_recurrent_kernel<DK>, dim3(DK / 16, a.H, B), dim3(NT), 0, s, a);
  hipLaunchKernelGGL(gdn_out_kernel<DK>, dim3(B * a.T, (a.H + 3) / 4), dim3(256), 0, s, a, B * a.T);
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
