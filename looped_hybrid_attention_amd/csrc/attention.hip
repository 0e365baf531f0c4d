// Full-attention kernels: QK-norm + partial rotary + KV append, flash-style
// causal GQA prefill, split-L decode with a deterministic combine.
//
// [P1 section 3], [P2 section 3]: 16 query heads share 4 KV heads (GQA), head
// dim 256, QK normalisation, an attention output gate, rotary on a quarter of
// the dims (64 of 256).  [P1 section 4]: K and V of every KV head are cached
// in bf16, one cache per full-attention execution.  Readings: QK-norm is an
// RMSNorm over the head dim with one gain per q / k (shared by heads), before
// rotary; rotary rotates adjacent pairs (2i, 2i+1), i < R/2, by
// pos * theta^(-2i/R) (angle in double, cos/sin rounded to fp32); scale
// 1/sqrt(D); causal on absolute positions; output gate = elementwise sigmoid
// of the gate projection, applied before W_o.
//
// Cache layout per (execution slot, sequence slot): K [Hkv][max_seq][D] and
// V transposed [Hkv][D][max_seq], so that both the K.Q^T and the V^T.P^T
// products of the prefill read 16-byte runs from LDS.
#include "common.h"
#include "launch.h"

namespace {

// ---------------------------------------------------------------- prep
// One wave per (token, item); items: Hq query heads, Hkv key heads, Hkv
// value heads.  Lane holds D/64 consecutive dims.
template <int D>
__global__ __launch_bounds__(256) void qk_prep_kernel(AttnPrepArgs a) {
  constexpr int EPL = D / 64;
  const int m = blockIdx.x;  // token row
  const int item = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_items = a.Hq + 2 * a.Hkv;
  if (item >= n_items) return;
  const int b = m / a.T, t = m % a.T;
  const int pos = a.pos[b] + t;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* row = a.proj + (int64_t)m * a.proj_stride;
  const int d0 = lane * EPL;
  float x[EPL];
  if (item >= a.Hq + a.Hkv) {
    // value head: raw copy into the transposed cache
    const int kvh = item - a.Hq - a.Hkv;
    const uint16_t* src = row + 2 * a.Hq * D + a.Hkv * D + kvh * D + d0;
    uint16_t* vt = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq;
#pragma unroll
    for (int e = 0; e < EPL; ++e) vt[(int64_t)(d0 + e) * a.max_seq + pos] = src[e];
    return;
  }
  const bool is_q = item < a.Hq;
  const int head = is_q ? item : item - a.Hq;
  const uint16_t* src = is_q ? row + head * D : row + 2 * a.Hq * D + head * D;
  const uint16_t* gain = is_q ? a.q_norm : a.k_norm;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    x[e] = bf2f(src[d0 + e]);
    ss += x[e] * x[e];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / D + a.eps);
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = x[e] * inv * bf2f(gain[d0 + e]);
  // rotary on dims < R, adjacent pairs
  if (EPL >= 2) {
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      const int d = d0 + e;
      if (d < a.R) {
        const int i = d >> 1;
        const double th = pow((double)a.theta, -2.0 * i / a.R);
        const double ang = (double)pos * th;
        const float c = (float)cos(ang), s = (float)sin(ang);
        const float x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * c - x1 * s;
        x[e + 1] = x0 * s + x1 * c;
      }
    }
  } else {
    const float partner = __shfl_xor(x[0], 1, 64);
    if (d0 < a.R) {
      const int i = d0 >> 1;
      const double th = pow((double)a.theta, -2.0 * i / a.R);
      const double ang = (double)pos * th;
      const float c = (float)cos(ang), s = (float)sin(ang);
      x[0] = (d0 & 1) ? partner * s + x[0] * c : x[0] * c - partner * s;
    }
  }
  uint16_t* dst;
  if (is_q) {
    dst = a.q_out + ((int64_t)m * a.Hq + head) * D + d0;
  } else {
    dst = a.k_cache + ((slot_b * a.Hkv + head) * (int64_t)a.max_seq + pos) * D + d0;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = f2bf_bits(x[e]);
}

// ------------------------------------------------------- flash prefill
// Workgroup = (32-query tile, KV head, sequence); G waves, wave w = query head
// kvh*G + w.  Lane (h = lane/32, q = lane%32) owns query q of the tile.
// S^T = K . Q^T (32 keys x 32 queries per MFMA tile) leaves each lane with
// the scores of its own query, so the online softmax is lane-local (plus one
// exchange with lane ^ 32) and the probabilities feed O^T += V^T . P^T as the
// B operand without leaving registers; the key order inside a 16-key MFMA
// step is permuted identically on both operands.
constexpr int KT = 64;          // keys per LDS tile
template <int D>
struct FlashLds {
  static constexpr int KS = D + 8;   // padded K row (bf16)
  static constexpr int VS = KT + 8;  // padded V^T row (bf16)
  static constexpr int bytes = (KT * KS + D * VS) * 2;
};

template <int D, int G>
__global__ __launch_bounds__(64 * G, 1) void flash_prefill_kernel(FlashArgs a) {
  constexpr int NT = 64 * G;
  constexpr int NKS = D / 16;  // 16-dim MFMA steps of Q.K
  constexpr int NDT = D / 32;  // 32-dim output tiles
  using L = FlashLds<D>;
  extern __shared__ __align__(16) uint16_t flash_smem[];
  uint16_t* sK = flash_smem;
  uint16_t* sV = flash_smem + KT * L::KS;

  const int tile = (gridDim.x - 1) - blockIdx.x;  // heaviest (latest) tiles first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, ql = lane & 31;
  const int head = kvh * G + wave;
  const int t = tile * 32 + ql;
  const bool qvalid = t < a.T;
  const int p0 = a.pos[b];
  const int qpos = p0 + t;
  const int64_t m = (int64_t)b * a.T + t;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* Kc = a.k_cache + (slot_b * a.Hkv + kvh) * (int64_t)a.max_seq * D;
  const uint16_t* Vc = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq;
  const int L_valid = p0 + a.T;

  bf16x8 qf[NKS];
  {
    const uint16_t* qs = a.q + (m * a.Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qs + ks * 16 + h * 8) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = (f32x16){};
  float m_i = -1e30f, l_i = 0.f;
  const float scale = a.scale_log2;

  const int last_t = min(a.T, tile * 32 + 32) - 1;
  const int kv_end = min(p0 + last_t + 1, L_valid);
  for (int k0 = 0; k0 < kv_end; k0 += KT) {
    __syncthreads();
    // K tile: 64 keys x D
    for (int c = threadIdx.x; c < KT * D / 8; c += NT) {
      const int key = c / (D / 8), dc = c % (D / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k0 + key < L_valid) v = *reinterpret_cast<const uint4*>(Kc + (int64_t)(k0 + key) * D + dc * 8);
      *reinterpret_cast<uint4*>(sK + key * L::KS + dc * 8) = v;
    }
    // V^T tile: D rows x 64 keys
    for (int c = threadIdx.x; c < D * KT / 8; c += NT) {
      const int d = c / (KT / 8), kc = c % (KT / 8);
      const int kk = k0 + kc * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < L_valid) {
        v = *reinterpret_cast<const uint4*>(Vc + (int64_t)d * a.max_seq + kk);
        if (kk + 8 > L_valid) {
          uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (kk + j >= L_valid) e[j] = 0;
        }
      }
      *reinterpret_cast<uint4*>(sV + d * L::VS + kc * 8) = v;
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = (f32x16){};
      const uint16_t* kr = sK + (kt * 32 + ql) * L::KS + h * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + ks * 16);
        s[kt] = mfma32x32x16(kf, qf[ks], s[kt]);
      }
    }
    // mask + online softmax (lane-local for query ql)
    float mloc = -1e30f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        float v = s[kt][r] * scale;
        v = (key <= qpos) ? v : -1e30f;
        s[kt][r] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_i, mloc);
    const float alpha = exp2f(m_i - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = s[kt][r] > -1e29f ? exp2f(s[kt][r] - m_new) : 0.f;
        s[kt][r] = p;
        lsum += p;
      }
    lsum += __shfl_xor(lsum, 32, 64);
    l_i = l_i * alpha + lsum;
    m_i = m_new;
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] *= alpha;
    // O^T += V^T . P^T over the 64 keys in 4 steps of 16
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int kt = ks2 >> 1, sh = (ks2 & 1) * 8;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = f2bf(s[kt][sh + e]);
      const uint16_t* vr = sV + ql * L::VS + ks2 * 16 + 4 * h;
#pragma unroll
      for (int i = 0; i < NDT; ++i) {
        const uint16_t* vp = vr + i * 32 * L::VS;
        uint2 lo = *reinterpret_cast<const uint2*>(vp);
        uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
        uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[i] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pf, o[i]);
      }
    }
  }
  if (!qvalid) return;
  const float inv_l = 1.f / l_i;
  const uint16_t* g = a.gate + m * a.gate_stride + head * D;
  uint16_t* out = a.out + m * a.out_stride + head * D;
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = i * 32 + 8 * j + 4 * h;
      uint2 gv = *reinterpret_cast<const uint2*>(g + d);
      const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv);
      uint16_t r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = f2bf_bits(o[i][4 * j + e] * inv_l * sigmoidf_(bf2f(ge[e])));
      *reinterpret_cast<uint2*>(out + d) = *reinterpret_cast<uint2*>(r);
    }
}

// --------------------------------------------------------------- decode
// Workgroup = (split of DEC_SPLIT keys, KV head, sequence): the G query heads
// of the KV head against keys [split*DEC_SPLIT, min(pos+1, ...)).  HBM-bound:
// every K and V^T byte of the split is read once, straight into MFMA
// operands.  Scores S^T[key][g] = K . q^T with v_mfma_f32_16x16x32_bf16 (16
// keys x 16 head columns, G of them used); probabilities go through LDS as
// bf16 [g][key]; O^T[d][g] += V^T[d][key] . P[key][g] with the same MFMA.
// Writes per (head, split) the unnormalised o[D], the split max m and sum l;
// the combine kernel merges the splits in split order.
constexpr int DEC_NT = 256;
constexpr int DEC_SPLIT = 512;
constexpr int DEC_PS = DEC_SPLIT + 8;  // bf16 row of P in LDS

DEV f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(DEC_NT, 2) void decode_attn_kernel(DecodeAttnArgs a) {
  static_assert(G <= 16, "query heads per KV head");
  constexpr int NKS = D / 32;   // 32-dim steps of the score MFMA
  constexpr int NDT = D / 16;   // 16-dim output tiles
  __shared__ float sc[G][DEC_SPLIT];
  __shared__ __align__(16) uint16_t sp[16 * DEC_PS];
  __shared__ float sm[G], sl[G];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int pos = a.pos[b];
  const int k_begin = split * DEC_SPLIT;
  const int k_end = min(pos + 1, k_begin + DEC_SPLIT);
  float* part = a.partial + (((int64_t)b * a.Hq + kvh * G) * a.n_split + split) * (D + 2);
  const int64_t part_head_stride = (int64_t)a.n_split * (D + 2);
  if (k_begin >= k_end) {  // empty split: neutral element
    for (int i = threadIdx.x; i < G * (D + 2); i += DEC_NT) {
      const int g = i / (D + 2), c = i % (D + 2);
      part[g * part_head_stride + c] = c == D ? -1e30f : 0.f;
    }
    return;
  }
  const int nk = k_end - k_begin;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* Kc = a.k_cache + ((slot_b * a.Hkv + kvh) * (int64_t)a.max_seq + k_begin) * D;
  const uint16_t* Vc = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq + k_begin;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  // q^T operand: lane supplies q[g = l16][32 ks + 8 lg .. +8] (zero for g >= G)
  bf16x8 qf[NKS];
  {
    const uint16_t* qs = a.q + ((int64_t)b * a.Hq + kvh * G + min(l16, G - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 v = l16 < G ? *reinterpret_cast<const uint4*>(qs + ks * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // scores: each wave takes two 16-key groups at a time (32 loads per lane in
  // flight for D = 256), groups round-robin over the waves
  for (int g0 = wave * 32; g0 < nk; g0 += 4 * 32) {
    u32x4 kv[2][NKS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = g0 + 16 * u + l16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kv[u][ks] = key < nk ? *reinterpret_cast<const u32x4*>(Kc + (int64_t)key * D + ks * 32 + lg * 8)
                             : (u32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = mfma16x16x32(__builtin_bit_cast(bf16x8, kv[u][ks]), qf[ks], acc);
      // lane holds keys g0 + 16u + 4 lg + r of head l16
      if (l16 < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = g0 + 16 * u + 4 * lg + r;
          if (kk < DEC_SPLIT) sc[l16][kk] = kk < nk ? acc[r] * a.scale_log2 : -1e30f;
        }
      }
    }
  }
  __syncthreads();
  // per-head max and sum over the split (wave w: heads w, w+4, ...)
  for (int g = wave; g < G; g += 4) {
    float mx = -1e30f;
    for (int k = lane; k < nk; k += 64) mx = fmaxf(mx, sc[g][k]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < DEC_SPLIT; k += 64) {
      const float p = k < nk ? exp2f(sc[g][k] - mx) : 0.f;
      sum += p;
      sp[g * DEC_PS + k] = f2bf_bits(p);
    }
    sum = wave_sum(sum);
    if (lane == 0) { sm[g] = mx; sl[g] = sum; }
  }
  for (int i = threadIdx.x; i < (16 - G) * DEC_SPLIT; i += DEC_NT)
    sp[(G + i / DEC_SPLIT) * DEC_PS + i % DEC_SPLIT] = 0;
  __syncthreads();
  // O^T[d][g] += V^T[d][key] P[key][g]; wave w: d-tiles w, w+4, ...
  constexpr int TPW = (NDT + 3) / 4;
  f32x4 o[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) o[i] = (f32x4){0, 0, 0, 0};
  const int nsteps = (nk + 31) / 32;
  // four 32-key steps per iteration: their V^T loads are all in flight
  // before the MFMAs
  for (int st0 = 0; st0 < nsteps; st0 += 4) {
    u32x4 vv[4][TPW];
    bf16x8 pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kk = (st0 + u) * 32 + lg * 8;  // first of this lane's 8 keys
      pf[u] = kk < DEC_SPLIT ? *reinterpret_cast<const bf16x8*>(sp + l16 * DEC_PS + kk) : (bf16x8){};
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int dt = wave + 4 * i;
        u32x4 v = {0, 0, 0, 0};
        if (dt < NDT && kk < nk) {
          const int d = dt * 16 + l16;
          v = *reinterpret_cast<const u32x4*>(Vc + (int64_t)d * a.max_seq + kk);
          if (kk + 8 > nk) {
            uint16_t* e = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (kk + j >= nk) e[j] = 0;
          }
        }
        vv[u][i] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < TPW; ++i) o[i] = mfma16x16x32(__builtin_bit_cast(bf16x8, vv[u][i]), pf[u], o[i]);
  }
  // lane holds O^T[d = 16 dt + 4 lg + r][g = l16]
  if (l16 < G) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int dt = wave + 4 * i;
      if (dt >= NDT) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) part[l16 * part_head_stride + dt * 16 + 4 * lg + r] = o[i][r];
    }
  }
  if (threadIdx.x < G) {
    part[threadIdx.x * part_head_stride + D] = sm[threadIdx.x];
    part[threadIdx.x * part_head_stride + D + 1] = sl[threadIdx.x];
  }
}

// Merge the splits of one (sequence, query head) in split order; apply the
// output gate; store bf16.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeAttnArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const float* part = a.partial + ((int64_t)b * a.Hq + hq) * a.n_split * (D + 2);
  float M = -1e30f;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float Lsum = 0.f;
  for (int s = 0; s < a.n_split; ++s) Lsum += part[s * (D + 2) + D + 1] * exp2f(part[s * (D + 2) + D] - M);
  const uint16_t* g = a.gate + (int64_t)b * a.gate_stride + hq * D;
  uint16_t* out = a.out + (int64_t)b * a.out_stride + hq * D;
  for (int d = threadIdx.x; d < D; d += 256) {
    float o = 0.f;
    for (int s = 0; s < a.n_split; ++s) o += part[s * (D + 2) + d] * exp2f(part[s * (D + 2) + D] - M);
    out[d] = f2bf_bits(o / Lsum * sigmoidf_(bf2f(g[d])));
  }
}

template <int D>
hipError_t prep_d(const AttnPrepArgs& a, int M, hipStream_t s) {
  const int items = a.Hq + 2 * a.Hkv;
  hipLaunchKernelGGL(qk_prep_kernel<D>, dim3(M, (items + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t flash_dg(const FlashArgs& a, int B, hipStream_t s) {
  const size_t lds = FlashLds<D>::bytes;
  auto k = flash_prefill_kernel<D, G>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(k, dim3((a.T + 31) / 32, a.Hkv, B), dim3(64 * G), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t flash_d(const FlashArgs& a, int B, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return flash_dg<D, 1>(a, B, s);
    case 2: return flash_dg<D, 2>(a, B, s);
    case 4: return flash_dg<D, 4>(a, B, s);
    case 8: return flash_dg<D, 8>(a, B, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int G>
hipError_t decode_dg(const DecodeAttnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((decode_attn_kernel<D, G>), dim3(a.n_split, a.Hkv, B), dim3(DEC_NT), 0, s, a);
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.Hq, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t decode_d(const DecodeAttnArgs& a, int B, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return decode_dg<D, 1>(a, B, s);
    case 2: return decode_dg<D, 2>(a, B, s);
    case 4: return decode_dg<D, 4>(a, B, s);
    case 8: return decode_dg<D, 8>(a, B, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_prep(const AttnPrepArgs& a, int M, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (a.D == 256) return prep_d<256>(a, M, s);
  if (a.D == 64) return prep_d<64>(a, M, s);
  return hipErrorInvalidValue;
}

hipError_t launch_flash_prefill(const FlashArgs& a, int B, hipStream_t s) {
  if (B == 0 || a.T == 0) return hipSuccess;
  if (a.D == 256) return flash_d<256>(a, B, s);
  if (a.D == 64) return flash_d<64>(a, B, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, int B, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (a.D == 256) return decode_d<256>(a, B, s);
  if (a.D == 64) return decode_d<64>(a, B, s);
  return hipErrorInvalidValue;
}
