// Shared device helpers for the gfx950 kernels: bf16 conversion, vector
// types, MFMA wrappers, wave reductions.  CDNA4 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector (HIP's uint4 is a struct of unions that
// the compiler does not keep in registers when indexed from arrays).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define DEV __device__ __forceinline__

// bf16 <-> fp32.  bf16 -> fp32 is exact (shift); fp32 -> bf16 rounds to
// nearest even (gfx950's v_cvt_pk_bf16_f32).
DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
DEV float bf2f(bf16 b) { return (float)b; }
DEV bf16 f2bf(float f) { return (bf16)f; }
DEV uint16_t f2bf_bits(float f) { return __builtin_bit_cast(uint16_t, f2bf(f)); }

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%32][(l/32)*8 .. +8]
// and B^T[l%32][(l/32)*8 .. +8] (k-contiguous); the 16 results of lane l are
// D[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15.
DEV f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[l%16][(l/16)*8 .. +8]
// and B^T[l%16][(l/16)*8 .. +8]; its 4 results are D[4*(l/16) + r][l%16].
DEV f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum of one float per thread; `red` = __shared__ float[nwaves].
// All threads get the result.  Deterministic (fixed order).
template <int NT>
DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

// Hardware exp2 and reciprocal (about 1 ulp each): far below the bf16
// rounding that every consumer applies, and a fraction of the cost of an
// IEEE division.  Large |x| saturates correctly (rcp(inf) = 0).
DEV float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
DEV float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Global -> LDS copies that bypass registers (buffer_load ... lds, gfx950
// 16-byte form).  MUBUF rather than the FLAT form: with a FLAT LDS copy in
// flight the compiler waits for every outstanding LDS read at each use.
typedef __attribute__((address_space(3))) void lds_void;
// Raw buffer resource over `bytes` bytes at `base` (word 3: 32-bit data
// format, no swizzle, as CDNA expects for raw buffer loads).
DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Lane i's 16 bytes at `src` + voffset + soffset land at LDS byte `dst` + 16 i
// (dst and soffset wave-uniform).  Completion is counted by vmcnt.
DEV void copy16_to_lds(__amdgpu_buffer_rsrc_t src, int voffset, int soffset, lds_void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, voffset, soffset, 0, 0);
}
// 16 bytes at byte voffset + soffset of a raw buffer (zero past its size).
DEV u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0);
}
// Workgroup barrier after this wave's LDS accesses have completed.  Copies
// still in flight to other ring stages stay in flight: a fence would make the
// compiler drain them (it counts them as pending LDS writes).  The memory
// clobber keeps LDS accesses on their side of the barrier.
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// s_waitcnt with vmcnt(N), other counters untouched: at most the N newest
// vector memory operations of this wave are still outstanding (they complete
// in issue order).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt vmcnt(0): this wave's vector memory operations (LDS copies
// included) have completed.
DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
