// Row kernels of the layer executions: embedding gather, RMSNorm, the fused
// dual-stream mHC transition between executions, hidden-state taps and the
// greedy argmax.  All HBM-bound; one workgroup of 256 threads per token row,
// the row held in registers, reductions in a fixed order (deterministic).
//
// mHC ([P1 section 5], [P1 section 6] reproduction's MHC.forward, [P4
// section 02]): inside the looped block two fp32 residual streams s0, s1.
// Per layer: read r = softmax(W_r [s0; s1] + b_r), x = r0 s0 + r1 s1; write
// w = softmax(W_w out + b_w), P = Sinkhorn_20(L), s_s' = P[s,0] s0 + P[s,1] s1
// + w_s out, where out = a + f is the layer's residual branch.  Fork at loop
// entry (s0 = s1 = h), merge at loop exit (h = (s0 + s1) / 2).  Sinkhorn:
// in the log domain subtract row log-sum-exp then column log-sum-exp, 20
// times, then a row softmax -- a 2x2 problem held in registers.
#include "common.h"
#include "launch.h"

namespace {

constexpr int NT = 256;

// Sinkhorn normalisation of a 2x2 logit matrix, fp32, in registers.
DEV void sinkhorn2(const float* L, int iters, float P[4]) {
  float m[4] = {L[0], L[1], L[2], L[3]};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {  // rows
      float a = m[2 * r], b = m[2 * r + 1];
      float mx = fmaxf(a, b);
      float lse = mx + logf(expf(a - mx) + expf(b - mx));
      m[2 * r] = a - lse;
      m[2 * r + 1] = b - lse;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // columns
      float a = m[c], b = m[2 + c];
      float mx = fmaxf(a, b);
      float lse = mx + logf(expf(a - mx) + expf(b - mx));
      m[c] = a - lse;
      m[2 + c] = b - lse;
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float a = m[2 * r], b = m[2 * r + 1];
    float mx = fmaxf(a, b);
    float ea = expf(a - mx), eb = expf(b - mx);
    P[2 * r] = ea / (ea + eb);
    P[2 * r + 1] = eb / (ea + eb);
  }
}

DEV void softmax2(float z0, float z1, float& p0, float& p1) {
  float mx = fmaxf(z0, z1);
  float e0 = expf(z0 - mx), e1 = expf(z1 - mx);
  p0 = e0 / (e0 + e1);
  p1 = e1 / (e0 + e1);
}

// Two block sums at once (one reduction pass).
DEV void block_sum2(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) { red[2 * w] = a; red[2 * w + 1] = b; }
  __syncthreads();
  a = b = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) { a += red[2 * i]; b += red[2 * i + 1]; }
}

__global__ __launch_bounds__(NT) void embed_kernel(const int32_t* ids, const uint16_t* E, float* h, int d,
                                                   int vocab) {
  const int64_t m = blockIdx.x;
  const int id = min(max(ids[m], 0), vocab - 1);  // out-of-range ids are clamped
  const uint16_t* src = E + (int64_t)id * d;
  float* dst = h + m * d;
  for (int i = threadIdx.x * 8; i < d; i += NT * 8) {
    uint4 v = *reinterpret_cast<const uint4*>(src + i);
    const uint16_t* p = reinterpret_cast<const uint16_t*>(&v);
    float4 lo = make_float4(bf2f(p[0]), bf2f(p[1]), bf2f(p[2]), bf2f(p[3]));
    float4 hi = make_float4(bf2f(p[4]), bf2f(p[5]), bf2f(p[6]), bf2f(p[7]));
    *reinterpret_cast<float4*>(dst + i) = lo;
    *reinterpret_cast<float4*>(dst + i + 4) = hi;
  }
}

// y = bf16(rmsnorm(x [+ x2]) * g) for row blockIdx.x (or rows[blockIdx.x]);
// F32: the same bf16 values stored as fp32.  With PER a multiple of 4 each
// thread takes groups of four contiguous columns, 4 (tid + q NT) .. (16-byte
// loads, all issued before the sums).
template <int PER, bool F32 = false>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(const float* x, const float* x2, const int32_t* rows,
                                                     int64_t x_stride, const uint16_t* g, void* y_out,
                                                     int d, float eps) {
  constexpr bool VEC = PER % 4 == 0;
  __shared__ float red[2 * NT / 64];
  const int64_t m = rows ? rows[blockIdx.x] : blockIdx.x;
  const float* xr = x + m * x_stride;
  const float* x2r = x2 ? x2 + m * x_stride : nullptr;
  auto col = [](int i) { return VEC ? 4 * ((int)threadIdx.x + (i / 4) * NT) + (i & 3) : (int)threadIdx.x + i * NT; };
  float v[PER];
  if (VEC) {
    f32x4 a[VEC ? PER / 4 : 1], b[VEC ? PER / 4 : 1];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int c = col(4 * q);
      a[q] = c < d ? *reinterpret_cast<const f32x4*>(xr + c) : (f32x4){0, 0, 0, 0};
      b[q] = (x2r && c < d) ? *reinterpret_cast<const f32x4*>(x2r + c) : (f32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < PER / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = a[q][e] + b[q][e];
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = col(i);
      v[i] = c < d ? xr[c] + (x2r ? x2r[c] : 0.f) : 0.f;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) ss += v[i] * v[i];
  float dummy = 0.f;
  block_sum2(ss, dummy, red);
  const float inv = rsqrtf(ss / d + eps);
  uint16_t* yr = reinterpret_cast<uint16_t*>(y_out) + (int64_t)blockIdx.x * d;
  float* yf = reinterpret_cast<float*>(y_out) + (int64_t)blockIdx.x * d;
  if (VEC) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int c = col(4 * q);
      if (c >= d) continue;
      const uint2 gv = *reinterpret_cast<const uint2*>(g + c);
      const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv);
      uint16_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f2bf_bits(v[4 * q + e] * inv * bf2f(ge[e]));
      if constexpr (F32)
        *reinterpret_cast<f32x4*>(yf + c) = (f32x4){bf2f(o[0]), bf2f(o[1]), bf2f(o[2]), bf2f(o[3])};
      else
        *reinterpret_cast<uint2*>(yr + c) = *reinterpret_cast<const uint2*>(o);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = col(i);
      if (c >= d) continue;
      const uint16_t o = f2bf_bits(v[i] * inv * bf2f(g[c]));
      if constexpr (F32) yf[c] = bf2f(o);
      else yr[c] = o;
    }
  }
}

// The transition from one execution to the next.
//   in  = TR_IN_H:     the state is h (plain residual, or just embedded)
//   in  = TR_IN_WRITE: mHC write of `out` into streams s0, s1 (this exec's
//                      write params and mix logits)
//   out = TR_OUT_NORM: h (merged if in = WRITE) -> xn = RMSNorm(h; g)
//   out = TR_OUT_READ: (fork if in = H) then the next exec's mHC read:
//                      x = r0 s0 + r1 s1, xn = RMSNorm(x; g)
//   out = TR_OUT_NONE: merge only (h written), no norm
// One row per workgroup of TNT threads, PER values per thread.
template <int TNT, int PER>
DEV void block_sum2_t(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) { red[2 * w] = a; red[2 * w + 1] = b; }
  __syncthreads();
  a = b = 0.f;
#pragma unroll
  for (int i = 0; i < TNT / 64; ++i) { a += red[2 * i]; b += red[2 * i + 1]; }
}

template <int TNT, int PER>
__global__ __launch_bounds__(TNT) void transition_kernel(TransitionArgs t) {
  // Element i of this thread: with PER >= 4, contiguous groups of four
  // (16-byte accesses), columns 4 (tid + (i/4) TNT) + i%4; else tid + i TNT.
  constexpr bool VEC = PER % 4 == 0;
  __shared__ float red[2 * TNT / 64];
  const int d = t.d;
  const int64_t o = (int64_t)blockIdx.x * d;
  auto col = [](int i) { return VEC ? 4 * ((int)threadIdx.x + (i / 4) * TNT) + (i & 3) : (int)threadIdx.x + i * TNT; };
#define TR_LOAD(dst_, src_, off_)                                                                  \
  {                                                                                                \
    if (VEC) {                                                                                     \
      _Pragma("unroll") for (int q = 0; q < PER / 4; ++q) {                                        \
        const int c_ = col(4 * q);                                                                 \
        const float4 v_ = c_ < d ? *reinterpret_cast<const float4*>((src_) + (off_) + c_) : make_float4(0, 0, 0, 0); \
        dst_[4 * q] = v_.x; dst_[4 * q + 1] = v_.y; dst_[4 * q + 2] = v_.z; dst_[4 * q + 3] = v_.w; \
      }                                                                                            \
    } else {                                                                                       \
      _Pragma("unroll") for (int i = 0; i < PER; ++i) dst_[i] = col(i) < d ? (src_)[(off_) + col(i)] : 0.f; \
    }                                                                                              \
  }
#define TR_STORE(dst_, off_, val_)                                                                 \
  {                                                                                                \
    if (VEC) {                                                                                     \
      _Pragma("unroll") for (int q = 0; q < PER / 4; ++q) {                                        \
        const int c_ = col(4 * q);                                                                 \
        if (c_ < d) *reinterpret_cast<float4*>((dst_) + (off_) + c_) =                             \
            make_float4(val_[4 * q], val_[4 * q + 1], val_[4 * q + 2], val_[4 * q + 3]);           \
      }                                                                                            \
    } else {                                                                                       \
      _Pragma("unroll") for (int i = 0; i < PER; ++i) if (col(i) < d) (dst_)[(off_) + col(i)] = val_[i]; \
    }                                                                                              \
  }
  float s0[PER], s1[PER];
  if (t.in_mode == TR_IN_WRITE) {
    float ov[PER], w0v[PER], w1v[PER];
    TR_LOAD(ov, t.out, o);
    TR_LOAD(s0, t.s0, o);
    TR_LOAD(s1, t.s1, o);
    TR_LOAD(w0v, t.write_w, 0);
    TR_LOAD(w1v, t.write_w, d);
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      z0 += w0v[i] * ov[i];
      z1 += w1v[i] * ov[i];
    }
    block_sum2_t<TNT, PER>(z0, z1, red);
    float w0, w1;
    softmax2(z0 + t.write_b[0], z1 + t.write_b[1], w0, w1);
    // the layer's 2x2 mix matrix (Sinkhorn of its logits, computed once per call)
    const float P0 = t.P[0], P1 = t.P[1], P2 = t.P[2], P3 = t.P[3];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float a = s0[i], b = s1[i];
      s0[i] = P0 * a + P1 * b + w0 * ov[i];
      s1[i] = P2 * a + P3 * b + w1 * ov[i];
    }
  } else {
    TR_LOAD(s0, t.h, o);
#pragma unroll
    for (int i = 0; i < PER; ++i) s1[i] = s0[i];
  }

  float xv[PER];
  if (t.out_mode == TR_OUT_READ) {
    float r00[PER], r01[PER], r10[PER], r11[PER];
    TR_LOAD(r00, t.read_w, 0);
    TR_LOAD(r01, t.read_w, d);
    TR_LOAD(r10, t.read_w, 2 * d);
    TR_LOAD(r11, t.read_w, 3 * d);
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      z0 += r00[i] * s0[i] + r01[i] * s1[i];
      z1 += r10[i] * s0[i] + r11[i] * s1[i];
    }
    block_sum2_t<TNT, PER>(z0, z1, red);
    float r0, r1;
    softmax2(z0 + t.read_b[0], z1 + t.read_b[1], r0, r1);
#pragma unroll
    for (int i = 0; i < PER; ++i) xv[i] = r0 * s0[i] + r1 * s1[i];
    TR_STORE(t.s0_out, o, s0);
    TR_STORE(t.s1_out, o, s1);
    TR_STORE(t.x_out, o, xv);
  } else {
    // plain state h: either unchanged (in = H) or the merge of the streams
#pragma unroll
    for (int i = 0; i < PER; ++i) xv[i] = t.in_mode == TR_IN_WRITE ? (s0[i] + s1[i]) * 0.5f : s0[i];
    if (t.in_mode == TR_IN_WRITE) TR_STORE(t.h_out, o, xv);
    if (t.out_mode == TR_OUT_NONE) return;
  }
  float ss = 0.f, dummy = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) ss += xv[i] * xv[i];
  block_sum2_t<TNT, PER>(ss, dummy, red);
  const float inv = rsqrtf(ss / d + t.eps);
  if (VEC) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int c = col(4 * q);
      if (c >= d) continue;
      const uint2 gv = *reinterpret_cast<const uint2*>(t.norm_g + c);
      const float g4[4] = {bf2f((uint16_t)gv.x), bf2f((uint16_t)(gv.x >> 16)), bf2f((uint16_t)gv.y),
                           bf2f((uint16_t)(gv.y >> 16))};
      uint2 y;
      y.x = (uint32_t)f2bf_bits(xv[4 * q] * inv * g4[0]) | ((uint32_t)f2bf_bits(xv[4 * q + 1] * inv * g4[1]) << 16);
      y.y = (uint32_t)f2bf_bits(xv[4 * q + 2] * inv * g4[2]) | ((uint32_t)f2bf_bits(xv[4 * q + 3] * inv * g4[3]) << 16);
      *reinterpret_cast<uint2*>(t.xn + o + c) = y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (col(i) < d) t.xn[o + col(i)] = f2bf_bits(xv[i] * inv * bf2f(t.norm_g[col(i)]));
  }
#undef TR_LOAD
#undef TR_STORE
}

// The 2x2 mix matrices of the loop layers (Sinkhorn of each layer's mix
// logits): one thread per layer.
__global__ void sinkhorn_layers_kernel(SinkhornBatch sb) {
  const int l = threadIdx.x;
  if (l < sb.n) sinkhorn2(sb.mix[l], sb.iters, sb.out + 4 * l);
}

// Hidden state at the last position of each sequence: h, or the mean of the
// streams inside the loop.  dst [B, d].
__global__ __launch_bounds__(NT) void tap_kernel(const float* h, const float* s0, const float* s1,
                                                 float* dst, int T, int d) {
  const int b = blockIdx.x;
  const int64_t o = ((int64_t)b * T + T - 1) * d;
  for (int c = threadIdx.x; c < d; c += NT)
    dst[(int64_t)b * d + c] = s0 ? (s0[o + c] + s1[o + c]) * 0.5f : h[o + c];
}

__global__ void sinkhorn_kernel(const float* mix, int iters, float* out) {
  if (threadIdx.x == 0) sinkhorn2(mix, iters, out);
}

// Argmax over the last axis, lowest index on ties.  Stage 1: per (row,
// chunk) partial; stage 2: per row over the partials.
DEV void better(float v, int i, float& bv, int& bi) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

DEV void block_argmax(float& bv, int& bi, float* sv, int* si) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(bv, off, 64);
    int oi = __shfl_xor(bi, off, 64);
    better(ov, oi, bv, bi);
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  bv = sv[0]; bi = si[0];
  for (int i = 1; i < NT / 64; ++i) better(sv[i], si[i], bv, bi);
}

__global__ __launch_bounds__(NT) void argmax_stage1(const float* x, int64_t n, int chunk, float* pv, int* pi) {
  __shared__ float sv[NT / 64];
  __shared__ int si[NT / 64];
  const int row = blockIdx.y, c = blockIdx.x;
  const float* xr = x + (int64_t)row * n;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  const int64_t lo = (int64_t)c * chunk, hi = min(n, lo + chunk);
  for (int64_t i = lo + threadIdx.x; i < hi; i += NT) better(xr[i], (int)i, bv, bi);
  block_argmax(bv, bi, sv, si);
  if (threadIdx.x == 0) { pv[row * gridDim.x + c] = bv; pi[row * gridDim.x + c] = bi; }
}

__global__ __launch_bounds__(NT) void argmax_stage2(const float* pv, const int* pi, int nchunks, int32_t* out) {
  __shared__ float sv[NT / 64];
  __shared__ int si[NT / 64];
  const int row = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < nchunks; i += NT) better(pv[row * nchunks + i], pi[row * nchunks + i], bv, bi);
  block_argmax(bv, bi, sv, si);
  if (threadIdx.x == 0) out[row] = bi;
}

// Positions of the next decode step of a replayed graph: pos[b] += 1.
__global__ void advance_pos_kernel(int32_t* pos, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) pos[b] += 1;
}

template <typename F>
hipError_t by_width(int d, F f) {
  if (d <= 256) return f(std::integral_constant<int, 1>());
  if (d <= 1024) return f(std::integral_constant<int, 4>());
  if (d <= 4096) return f(std::integral_constant<int, 16>());
  if (d <= 8192) return f(std::integral_constant<int, 32>());
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_embed(const int32_t* ids, const void* E, float* h, int M, int d, int vocab, hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(NT), 0, s, ids, (const uint16_t*)E, h, d, vocab);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, const float* x2, const int32_t* rows, int64_t x_stride,
                          const void* g, void* y, int M, int d, float eps, hipStream_t s) {
  if (M == 0) return hipSuccess;
  return by_width(d, [&](auto per) {
    hipLaunchKernelGGL(rmsnorm_kernel<decltype(per)::value>, dim3(M), dim3(NT), 0, s, x, x2, rows,
                       x_stride, (const uint16_t*)g, y, d, eps);
    return hipGetLastError();
  });
}

hipError_t launch_rmsnorm_f32(const float* x, const void* g, float* y, int M, int d, float eps, hipStream_t s) {
  if (M == 0) return hipSuccess;
  return by_width(d, [&](auto per) {
    hipLaunchKernelGGL((rmsnorm_kernel<decltype(per)::value, true>), dim3(M), dim3(NT), 0, s, x, nullptr, nullptr,
                       (int64_t)d, (const uint16_t*)g, (void*)y, d, eps);
    return hipGetLastError();
  });
}

hipError_t launch_transition(TransitionArgs t, hipStream_t s) {
  if (t.M == 0) return hipSuccess;
  t.rows_per_block = 1;
  if (t.d <= 256) hipLaunchKernelGGL((transition_kernel<256, 1>), dim3(t.M), dim3(256), 0, s, t);
  else if (t.d <= 1024) hipLaunchKernelGGL((transition_kernel<256, 4>), dim3(t.M), dim3(256), 0, s, t);
  // few rows (decode): more threads per row, so that more loads are in flight
  else if (t.d <= 4096 && t.M <= 256) hipLaunchKernelGGL((transition_kernel<1024, 4>), dim3(t.M), dim3(1024), 0, s, t);
  else if (t.d <= 4096) hipLaunchKernelGGL((transition_kernel<512, 8>), dim3(t.M), dim3(512), 0, s, t);
  else if (t.d <= 8192) hipLaunchKernelGGL((transition_kernel<1024, 8>), dim3(t.M), dim3(1024), 0, s, t);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_tap(const float* h, const float* s0, const float* s1, float* dst, int B, int T, int d,
                      hipStream_t s) {
  hipLaunchKernelGGL(tap_kernel, dim3(B), dim3(NT), 0, s, h, s0, s1, dst, T, d);
  return hipGetLastError();
}

hipError_t launch_sinkhorn_layers(const SinkhornBatch& sb, hipStream_t s) {
  if (sb.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sinkhorn_layers_kernel, dim3(1), dim3(64), 0, s, sb);
  return hipGetLastError();
}

hipError_t launch_sinkhorn(const float* mix, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(sinkhorn_kernel, dim3(1), dim3(64), 0, s, mix, iters, out);
  return hipGetLastError();
}

int argmax_chunks(int64_t n) { return (int)((n + 8191) / 8192); }

hipError_t launch_advance_pos(int32_t* pos, int B, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_pos_kernel, dim3((B + 255) / 256), dim3(256), 0, s, pos, B);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int rows, int64_t n, float* pv, int* pi, int32_t* out, hipStream_t s) {
  const int nc = argmax_chunks(n);
  hipLaunchKernelGGL(argmax_stage1, dim3(nc, rows), dim3(NT), 0, s, x, n, 8192, pv, pi);
  hipLaunchKernelGGL(argmax_stage2, dim3(rows), dim3(NT), 0, s, pv, pi, nc, out);
  return hipGetLastError();
}
