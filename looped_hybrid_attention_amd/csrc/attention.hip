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
// V transposed in blocks of VB = 32 positions, [Hkv][max_seq/32][D][32], so
// that a block of keys is one contiguous run for both matrices and both the
// K.Q^T and the V^T.P^T
// products of the prefill read 16-byte runs from LDS.
#include "common.h"
#include "launch.h"

namespace {

constexpr int VB = 32;  // positions per block of the transposed V cache

// ---------------------------------------------------------------- prep
// QK-norm and partial rotary of one head vector, by one wave.
// rope_angles: cos / sin of the R/2 rotary frequencies at a position (angle
// pos * theta^(-2i/R) in double, rounded to fp32), entry i by the caller's
// thread i.  qk_norm_rope: RMSNorm over the D dims (sum of squares over the
// wave's lanes)
// times the gain, then the adjacent pairs (2i, 2i+1), i < R/2, rotated; the
// bf16 result is stored at dst, the 8-dim group c of the vector at group
// c ^ sw (sw = 0: in order).  Lane l holds the EPL = D/64 consecutive dims
// EPL l .. (D = 64: one dim, its rotary partner in the neighbouring lane).
DEV void rope_angles(int pos, int i, int R, float theta, float* rc, float* rs) {
  const double th = pow((double)theta, -2.0 * i / R);
  const double ang = (double)pos * th;
  rc[i] = (float)cos(ang);
  rs[i] = (float)sin(ang);
}
template <int D>
struct QkRaw {
  uint16_t x[D / 64];  // bf16 bits of the lane's dims
};
template <int D>
DEV QkRaw<D> qk_load(const uint16_t* src, int lane) {
  constexpr int EPL = D / 64;
  QkRaw<D> r;
  if constexpr (EPL == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(src + lane * EPL);
    r.x[0] = (uint16_t)v.x; r.x[1] = (uint16_t)(v.x >> 16);
    r.x[2] = (uint16_t)v.y; r.x[3] = (uint16_t)(v.y >> 16);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) r.x[e] = src[lane * EPL + e];
  }
  return r;
}
template <int D>
DEV void qk_gain(const uint16_t* gain, int lane, float (&g)[D / 64]) {
#pragma unroll
  for (int e = 0; e < D / 64; ++e) g[e] = bf2f(gain[lane * (D / 64) + e]);
}
template <int D>
DEV void qk_finish(const QkRaw<D>& r, const float (&g)[D / 64], const float* rc, const float* rs, int R, float eps,
                   uint16_t* dst, int sw, int lane) {
  constexpr int EPL = D / 64;
  const int d0 = lane * EPL;
  float x[EPL];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = bf2f(r.x[e]);
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += x[e] * x[e];
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / D + eps);
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = x[e] * inv * g[e];
  // rotary on dims < R, adjacent pairs (2i, 2i+1)
  if (EPL >= 2) {
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      const int d = d0 + e;
      if (d < R) {
        const float c = rc[d >> 1], sn = rs[d >> 1];
        const float x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * c - x1 * sn;
        x[e + 1] = x0 * sn + x1 * c;
      }
    }
  } else {
    const float partner = __shfl_xor(x[0], 1, 64);
    if (d0 < R) {
      const float c = rc[d0 >> 1], sn = rs[d0 >> 1];
      x[0] = (d0 & 1) ? partner * sn + x[0] * c : x[0] * c - partner * sn;
    }
  }
  uint16_t* o = dst + (((d0 >> 3) ^ sw) << 3) + (d0 & 7);
  if constexpr (EPL == 4) {
    uint2 v;
    v.x = (uint32_t)f2bf_bits(x[0]) | ((uint32_t)f2bf_bits(x[1]) << 16);
    v.y = (uint32_t)f2bf_bits(x[2]) | ((uint32_t)f2bf_bits(x[3]) << 16);
    *reinterpret_cast<uint2*>(o) = v;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = f2bf_bits(x[e]);
  }
}
template <int D>
DEV void qk_norm_rope(const uint16_t* src, const uint16_t* gain, const float* rc, const float* rs, int R,
                      float eps, uint16_t* dst, int sw, int lane) {
  float g[D / 64];
  qk_gain<D>(gain, lane, g);
  qk_finish<D>(qk_load<D>(src, lane), g, rc, rs, R, eps, dst, sw, lane);
}

// One workgroup per token: K of every KV head normalised, rotated and
// appended to the cache (the queries get the same treatment inside the
// attention kernels).  The rotary cos / sin of the token's position are
// computed once into LDS, and stored for the attention kernels ([M][R/2]
// pairs); the four waves take the heads in turn.
template <int D>
__global__ __launch_bounds__(256) void qk_prep_kernel(AttnPrepArgs a) {
  __shared__ float rc[D / 2], rs[D / 2];
  const int m = blockIdx.x;  // token row
  const int b = m / a.T, t = m % a.T;
  const int pos = a.pos[b] + t;
  const int64_t slot_b = a.seq_slot[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < a.R / 2) {
    rope_angles(pos, tid, a.R, a.theta, rc, rs);
    reinterpret_cast<float2*>(a.rope)[(int64_t)m * (a.R / 2) + tid] = make_float2(rc[tid], rs[tid]);
  }
  __syncthreads();
  const uint16_t* row = a.proj + (int64_t)m * a.proj_stride + 2 * a.Hq * D;
  for (int head = wave; head < a.Hkv; head += 4)
    qk_norm_rope<D>(row + head * D, a.k_norm, rc, rs, a.R, a.eps,
                    a.k_cache + ((slot_b * a.Hkv + head) * (int64_t)a.max_seq + pos) * D, 0, lane);
}

// V of a block of 64 tokens of one sequence and KV head into the transposed
// cache: rows of the projection in, staged in LDS, written out as 128-byte
// runs of each V^T row (the cache keeps V transposed for the PV products).
constexpr int VT_TOK = 64;
template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(AttnPrepArgs a) {
  constexpr int LS = D + 2;  // bf16 row in LDS (odd word stride: the column reads hit distinct banks)
  __shared__ __align__(4) uint16_t tile[VT_TOK * LS];
  const int t0 = blockIdx.x * VT_TOK, kvh = blockIdx.y, b = blockIdx.z;
  const int nt = min(VT_TOK, a.T - t0);
  const int tid = threadIdx.x;
  for (int i = tid; i < VT_TOK * (D / 8); i += 256) {
    const int t = i / (D / 8), c = i % (D / 8);
    if (t < nt) {
      const uint16_t* src = a.proj + ((int64_t)b * a.T + t0 + t) * a.proj_stride + 2 * a.Hq * D + a.Hkv * D +
                            kvh * D + c * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int w = 0; w < 4; ++w) *reinterpret_cast<uint32_t*>(tile + t * LS + c * 8 + 2 * w) = v[w];
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t slot_b = a.seq_slot[b];
  const int p = a.pos[b] + t0 + lane;  // position of this lane's token
  uint16_t* vt = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq + (int64_t)(p / VB) * D * VB + p % VB;
  if (lane < nt)
    for (int d = wave; d < D; d += 4) vt[d * VB] = tile[lane * LS + d];
}

// ------------------------------------------------------- flash prefill
// Workgroup = (query tile, KV head, sequence) with W = max(G, 4) waves; wave
// w takes query head kvh*G + w%G and 32 queries (w/G)*32 .. of the tile of
// QT = 32*W/G queries.  Lane (h = lane/32, q = lane%32) owns query q.
// S^T = K . Q^T (32 keys x 32 queries per MFMA tile) leaves each lane with
// the scores of its own query, so the online softmax is lane-local (plus one
// exchange with lane ^ 32), and the probabilities feed O^T += V^T . P^T as
// the B operand straight from registers.  That operand wants keys
// 16j + 8h .. +8 of 16-key step j in lane (q, h), while the score MFMA leaves
// the lane rows 8(r/4) + 4h + r%4; storing the K rows in LDS with bits 2 and
// 3 of their in-tile index swapped makes the two coincide.
//
// K [64 keys][D] and V^T [D][64 keys] tiles go global -> LDS directly
// (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, lane i
// at byte 16 i), double-buffered: the next tile's copies are issued before
// the current tile's MFMAs, waited for and fenced by one barrier after them.
// Rows are unpadded and their 16-byte chunks swizzled so that the operand
// reads of 16 consecutive rows (one LDS cycle of a 128-bit read: 64 banks)
// hit distinct banks: chunk c of K row r sits at c ^ (r % 16) (512-byte rows),
// chunk c of V^T row d at c ^ ((d / 2) % 8) (128-byte rows, two per bank
// sweep).  The loads pick their global source to realise both the swizzle and
// the K row order.
constexpr int KT = 64;  // keys per LDS tile
#ifndef FLASH_FD
#define FLASH_FD 4
#endif
template <int D>
struct FlashLds {
  static constexpr int KROW = D * 2;                   // bytes per K row
  static constexpr int VROW = KT * 2;                  // bytes per V^T row
  static constexpr int STAGE = KT * KROW + D * VROW;   // bytes per buffer
  static constexpr int bytes = 2 * STAGE;
};
DEV int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
template <int CR>
DEV int k_swz(int r) { return CR >= 16 ? (r & 15) : (r & 7); }
DEV int v_swz(int d) { return (d >> 1) & 7; }

template <int NDT, int FD, int VROW>
DEV void flash_pv(f32x16 (&o)[NDT], f32x16 (&s)[2], float& l, float m, float scale, const uint8_t* vr,
                  const int (&voff)[4]) {
  float lsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], scale, -m));
      s[kt][r] = p;
      lsum += p;
    }
  l += __shfl_xor(lsum, 32, 64) + lsum;
  bf16x8 pf[4];
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[ks2][e] = f2bf(s[ks2 >> 1][(ks2 & 1) * 8 + e]);
  bf16x8 vf[4 * NDT];
#define FLASH_VREAD(g_) vf[g_] = *reinterpret_cast<const bf16x8*>(vr + ((g_) % NDT) * 32 * VROW + voff[(g_) / NDT])
#pragma unroll
  for (int g = 0; g < FD; ++g) FLASH_VREAD(g);
#pragma unroll
  for (int g = 0; g < 4 * NDT; ++g) {
    if (g + FD < 4 * NDT) FLASH_VREAD(g + FD);
    o[g % NDT] = mfma32x32x16(vf[g], pf[g / NDT], o[g % NDT]);
  }
#undef FLASH_VREAD
  __builtin_amdgcn_sched_group_barrier(0x100, FD, 0);
#pragma unroll
  for (int g = 0; g < 4 * NDT; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (g + FD < 4 * NDT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <int D, int G>
__global__ __launch_bounds__(64 * (G < 4 ? 4 : G), 1) void flash_prefill_kernel(FlashArgs a) {
  constexpr int W = G < 4 ? 4 : G;
  constexpr int QT = 32 * W / G;
  constexpr int NKS = D / 16;  // 16-dim MFMA steps of Q.K
  constexpr int NDT = D / 32;  // 32-dim output tiles
  constexpr int CR = D / 8;    // 16-byte chunks per K row
  constexpr int KI = KT * CR / 64 / W;  // K copy instructions per wave and tile
  constexpr int VI = D * 8 / 64 / W;    // V^T copy instructions per wave and tile
  static_assert(KI * 64 * W == KT * CR && VI * 64 * W == D * 8, "tile / wave split");
  static_assert(CR >= 8, "swizzle needs 8 chunks per row");
  constexpr int FD = FLASH_FD;  // LDS operand reads in flight ahead of the MFMAs
  using L = FlashLds<D>;
  extern __shared__ __align__(16) uint8_t flash_smem[];

  const int tile = (gridDim.x - 1) - blockIdx.x;  // heaviest (latest) tiles first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, ql = lane & 31;
  const int head = kvh * G + wave % G;
  const int t = tile * QT + (wave / G) * 32 + ql;
  const bool qvalid = t < a.T;
  const int p0 = a.pos[b];
  const int qpos = p0 + t;
  const int64_t m = (int64_t)b * a.T + t;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* Kc = a.k_cache + (slot_b * a.Hkv + kvh) * (int64_t)a.max_seq * D;
  const uint16_t* Vc = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq;
  const int L_valid = p0 + a.T;
  const int kv_end = p0 + min(a.T, (tile + 1) * QT);
  const int nkt = (kv_end + KT - 1) / KT;

  // Global element offsets (from the tile's first key) of this lane's chunk
  // in each copy instruction of the wave.
  int k_src[KI], v_src[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int n = wave * KI + i;  // instruction index within the tile
    const int r = (n * 64 + lane) / CR, p = (n * 64 + lane) % CR;
    const int key = (r & ~31) | swap_bits23(r & 31);
    k_src[i] = key * D + (p ^ k_swz<CR>(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int n = wave * VI + i;
    const int d = (n * 64 + lane) / 8, p = (n * 64 + lane) % 8;
    const int lp = p ^ v_swz(d);  // keys 8 lp .. of the tile: block lp / 4 of its two
    v_src[i] = (lp / 4) * D * VB + d * VB + (lp % 4) * 8;
  }
  // Buffer resources over this (sequence, KV head)'s K and V^T blocks.  The
  // MUBUF form of the LDS copy keeps the compiler's LDS-read waits counted
  // (the FLAT form makes it wait for every outstanding LDS read).
  const auto k_rsrc = buffer_rsrc(Kc, a.max_seq * D * 2);
  const auto v_rsrc = buffer_rsrc(Vc, a.max_seq * D * 2);
#define FLASH_COPY(k0_, stage_)                                                               \
  {                                                                                           \
    uint8_t* S_ = flash_smem + (stage_) * L::STAGE;                                           \
    _Pragma("unroll") for (int i = 0; i < KI; ++i)                                            \
        copy16_to_lds(k_rsrc, ((k0_) * D + k_src[i]) * 2, 0, (lds_void*)(S_ + (wave * KI + i) * 1024)); \
    _Pragma("unroll") for (int i = 0; i < VI; ++i)                                            \
        copy16_to_lds(v_rsrc, ((k0_) / VB * D * VB + v_src[i]) * 2, 0,                       \
                      (lds_void*)(S_ + KT * L::KROW + (wave * VI + i) * 1024));               \
  }
  // V^T keys at or past L_valid may hold anything; P is 0 there but 0 * NaN
  // is not, so they are zeroed once the tile holding them has landed.
#define FLASH_ZERO_TAIL(k0_, stage_)                                                         \
  {                                                                                          \
    uint8_t* V_ = flash_smem + (stage_) * L::STAGE + KT * L::KROW;                           \
    const int first = max(L_valid - (k0_), 0);                                               \
    for (int d = tid; d < D; d += 64 * W)                                                    \
      for (int kk = first; kk < KT; ++kk)                                                    \
        *reinterpret_cast<uint16_t*>(V_ + d * L::VROW + (((kk >> 3) ^ v_swz(d)) << 4) + (kk & 7) * 2) = 0; \
  }
  // vmcnt(0): this wave's LDS copies have landed
#define FLASH_WAIT_COPIES() wait_vmem()

  // The queries: QK-norm and partial rotary here, from the projection, one
  // query vector per wave step into a scratch area (stage 1, which the first
  // tile leaves free; with eight waves both stages, before the first copy),
  // rows of D bf16 with 8-dim group c of row r at c ^ (r % 16), so that the
  // fragment reads of 16 rows hit distinct banks; the rotary cos / sin of the
  // tile's QT positions (from the prep kernel's table) after the stages.
  constexpr bool QS1 = W * 32 * D * 2 <= L::STAGE;
  const int RH = a.R / 2;
  float* rct = reinterpret_cast<float*>(flash_smem + L::bytes);
  float* rst = rct + QT * RH;
  uint16_t* qscr = reinterpret_cast<uint16_t*>(flash_smem + (QS1 ? L::STAGE : 0));
  if (QS1) FLASH_COPY(0, 0);
  for (int e = tid; e < QT * RH; e += 64 * W) {
    const int qi = e / RH, i = e % RH;
    const int tq = min(tile * QT + qi, a.T - 1);  // rows past T: any valid row
    const float2 cs = reinterpret_cast<const float2*>(a.rope)[((int64_t)b * a.T + tq) * RH + i];
    rct[qi * RH + i] = cs.x;
    rst[qi * RH + i] = cs.y;
  }
  __syncthreads();
  {
    // all 32 rows' loads in flight first (rows past T read as zero, which
    // the routine turns into zeros)
    const int q0 = (wave / G) * 32;  // the wave's first query within the tile
    QkRaw<D> raw[32];
#pragma unroll
    for (int qi = 0; qi < 32; ++qi) {
      const int tq = tile * QT + q0 + qi;
      if (tq < a.T) {
        raw[qi] = qk_load<D>(a.q + ((int64_t)b * a.T + tq) * a.q_stride + head * D, lane);
      } else {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) raw[qi].x[e] = 0;
      }
    }
    float gq[D / 64];
    qk_gain<D>(a.q_norm, lane, gq);
#pragma unroll
    for (int qi = 0; qi < 32; ++qi)
      qk_finish<D>(raw[qi], gq, rct + (q0 + qi) * RH, rst + (q0 + qi) * RH, a.R, a.eps, qscr + (wave * 32 + qi) * D,
                   qi & 15 & (CR - 1), lane);
  }
  __syncthreads();
  bf16x8 qf[NKS];
  {
    const uint16_t* qr = qscr + (wave * 32 + ql) * D;
    const int qsw = ql & 15 & (CR - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qr + (((2 * ks + h) ^ qsw) << 3));
  }
  if (!QS1) {
    __syncthreads();  // the scratch is read before the first tile lands there
    FLASH_COPY(0, 0);
  }
  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = (f32x16){};
  float m_i = -1e30f, l_i = 0.f;
  const float scale = a.scale_log2;
  const int ksw = k_swz<CR>(ql), vsw = v_swz(ql);  // swizzles of the rows this lane reads
  // Byte offsets of this lane's 16-byte chunk in its K row for the 16-dim
  // steps G = 0..7; the swizzle (< 16) leaves bit 4 of the chunk index alone,
  // so step G + 8 sits 256 bytes further (an immediate).  V^T: chunk of key
  // group q = 0..3.  Few per-lane registers, the rest immediates.
  int koff[8], voff[4];
#pragma unroll
  for (int st = 0; st < 8; ++st) koff[st] = ((2 * st + h) ^ ksw) << 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = ((2 * q + h) ^ vsw) << 4;
  const int qpos_lo = p0 + tile * QT + (wave / G) * 32;  // first query of the wave
  FLASH_WAIT_COPIES();
  __syncthreads();
  if (KT > L_valid) {
    FLASH_ZERO_TAIL(0, 0);
    __syncthreads();
  }

  // Tile loop.  The reference max moves rarely; when a tile needs it moved
  // the inner loop is left, O and l are rescaled outside it and the tile is
  // finished there, so that inside the loop O is only ever an MFMA
  // accumulator (no copies out of the accumulation registers).
  f32x16 s[2];
  float mloc;
  bool bump;
#define FLASH_SYNC(j_)                                                 \
  {                                                                    \
    FLASH_WAIT_COPIES();                                               \
    __syncthreads();                                                   \
    if ((j_) + 1 < nkt && ((j_) + 2) * KT > L_valid) {                 \
      FLASH_ZERO_TAIL(((j_) + 1) * KT, ((j_) + 1) & 1);                \
      __syncthreads();                                                 \
    }                                                                  \
  }
  int j = 0;
  for (;;) {
    for (; j < nkt; ++j) {
      const uint8_t* sK = flash_smem + (j & 1) * L::STAGE;
      const int k0 = j * KT;
      if (j + 1 < nkt) FLASH_COPY(k0 + KT, (j + 1) & 1);

      // S^T for the two 32-key halves: 2 NKS MFMAs alternating between the
      // halves (two independent accumulation chains keep the MFMA pipe full;
      // one chain issues at ~60 % of the rate), the K fragment reads kept FD
      // steps ahead of them
      s[0] = (f32x16){};
      s[1] = (f32x16){};
      {
        const uint8_t* kr = sK + ql * L::KROW;
        bf16x8 kf[2 * NKS];
#define FLASH_KREAD(g_)                                                                  \
  kf[g_] = *reinterpret_cast<const bf16x8*>(kr + ((g_) & 1) * 32 * L::KROW + koff[((g_) >> 1) & 7] + \
                                            (((g_) >> 4) << 8))
#pragma unroll
        for (int g = 0; g < FD; ++g) FLASH_KREAD(g);
#pragma unroll
        for (int g = 0; g < 2 * NKS; ++g) {
          if (g + FD < 2 * NKS) FLASH_KREAD(g + FD);
          s[g & 1] = mfma32x32x16(kf[g], qf[g >> 1], s[g & 1]);
        }
#undef FLASH_KREAD
        __builtin_amdgcn_sched_group_barrier(0x100, FD, 0);
#pragma unroll
        for (int g = 0; g < 2 * NKS; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (g + FD < 2 * NKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      // causal mask, only on tiles that reach past the wave's first query;
      // register r of half kt holds key k0 + 32 kt + swap_bits23(8 (r/4) + 4 h + r%4)
      if (k0 + KT - 1 > qpos_lo) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kt * 32 + swap_bits23(8 * (r >> 2) + 4 * h + (r & 3));
            s[kt][r] = (key <= qpos) ? s[kt][r] : -1e30f;
          }
      }
      // online softmax, lane-local for query ql (plus lane ^ 32), in log2
      // units.  The reference max m_i moves only when a tile's max exceeds
      // it by more than 8, so probabilities stay below 2^8 (O and l share
      // the reference: their ratio is exact).  Key 0 is in every query's
      // range, so the first tile sets m_i.
      mloc = -1e30f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * scale;
      bump = mloc > m_i + 8.f;
      if (__builtin_amdgcn_read_exec() & __ballot(bump)) break;
      flash_pv<NDT, FD, L::VROW>(o, s, l_i, m_i, scale, sK + KT * L::KROW + ql * L::VROW, voff);
      FLASH_SYNC(j);
    }
    if (j >= nkt) break;
    {
      const float m_new = bump ? mloc : m_i;
      const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[i] *= alpha;
      m_i = m_new;
    }
    flash_pv<NDT, FD, L::VROW>(o, s, l_i, m_i, scale, flash_smem + (j & 1) * L::STAGE + KT * L::KROW + ql * L::VROW,
                               voff);
    FLASH_SYNC(j);
    ++j;
  }
#undef FLASH_SYNC
#undef FLASH_COPY
#undef FLASH_ZERO_TAIL
#undef FLASH_WAIT_COPIES
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

// ------------------------------------------- flash prefill, two waves per SIMD
// The G = 4 case (four query heads per KV head) with eight waves, two per
// SIMD, so that one wave's softmax and LDS waits overlap the other's MFMAs.
// Workgroup = (32-query tile, KV head, sequence); wave w takes query head
// kvh*4 + w%4 and the 16 queries 16 (w/4) .. of the tile, on
// v_mfma_f32_16x16x32_bf16: lane (c = lane%16, rg = lane/16) owns query c.
// S^T = K . Q^T per 16-key block kb of the 64-key tile leaves the lane rows
// 4 rg + r (r = 0..3) of each block; the PV product O^T += V^T . P^T takes,
// per 32-key step ks, the keys 8 rg .. 8 rg + 7 of the step in lane group rg.
// K row i of the LDS tile (block i/16, group (i/4)%4, r = i%4) therefore
// holds key 32 (kb/2) + 8 rg + 4 (kb%2) + r: blocks 2ks and 2ks + 1 give lane
// group rg exactly the eight keys its PV operand needs, as they stand.  The
// running max and sum of a query are shared by its four lanes (reduced over
// lane ^ 16 and lane ^ 32).  K and V^T tiles as in the kernel above (direct
// copies, two stages, 16-byte chunks swizzled so that the 16 rows of one
// operand read hit distinct banks); the queries' QK-norm and rotary in the
// prologue, through stage 1.
DEV int f16_key_of_row(int i) { return 32 * (i >> 5) + 8 * ((i >> 2) & 3) + 4 * ((i >> 4) & 1) + (i & 3); }
template <int CR>
DEV int f16_kswz(int r) { return CR >= 16 ? (r & 15) : ((r >> 1) & 7); }

template <int NDB, int FD, int VROW>
DEV void flash16_pv(f32x4 (&o)[NDB], f32x4 (&s)[4], float& l, float m, float scale, const uint8_t* vr, int vsw,
                    int rg) {
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale, -m));
      s[kb][r] = p;
      lsum += p;
    }
  l += lsum;
  bf16x8 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[ks][e] = f2bf(s[2 * ks + (e >> 2)][e & 3]);
  bf16x8 vf[2 * NDB];
  // step g: output block g % NDB, key step g / NDB
#define F16_VREAD(g_) \
  vf[g_] = *reinterpret_cast<const bf16x8*>(vr + ((g_) % NDB) * 16 * VROW + (((4 * ((g_) / NDB) + rg) ^ vsw) << 4))
#pragma unroll
  for (int g = 0; g < FD; ++g) F16_VREAD(g);
#pragma unroll
  for (int g = 0; g < 2 * NDB; ++g) {
    if (g + FD < 2 * NDB) F16_VREAD(g + FD);
    o[g % NDB] = mfma16x16x32(vf[g], pf[g / NDB], o[g % NDB]);
  }
#undef F16_VREAD
  __builtin_amdgcn_sched_group_barrier(0x100, FD, 0);
#pragma unroll
  for (int g = 0; g < 2 * NDB; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (g + FD < 2 * NDB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <int D>
__global__ __launch_bounds__(512, 1) void flash16_prefill_kernel(FlashArgs a) {
  constexpr int G = 4, W = 8, QT = 32;
  constexpr int CR = D / 8;    // 16-byte chunks per K row
  constexpr int NDS = D / 32;  // 32-dim steps of K . Q^T
  constexpr int NDB = D / 16;  // 16-dim output blocks
  constexpr int KI = KT * CR / 64 / W;  // K copy instructions per wave and tile
  constexpr int VI = D * 8 / 64 / W;    // V^T copy instructions per wave and tile
  static_assert(KI >= 1 && VI >= 1 && KI * 64 * W == KT * CR && VI * 64 * W == D * 8, "tile / wave split");
  static_assert(CR >= 8, "swizzle needs 8 chunks per row");
  constexpr int FD = 4;  // LDS operand reads in flight ahead of the MFMAs
  using L = FlashLds<D>;
  static_assert(W * 16 * D * 2 <= L::STAGE, "query scratch in stage 1");
  extern __shared__ __align__(16) uint8_t flash_smem[];

  const int tile = (gridDim.x - 1) - blockIdx.x;  // heaviest (latest) tiles first
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, rg = lane >> 4;
  const int head = kvh * G + wave % G, qh = wave / G;
  const int t = tile * QT + qh * 16 + c;
  const bool qvalid = t < a.T;
  const int p0 = a.pos[b];
  const int qpos = p0 + t;
  const int64_t m = (int64_t)b * a.T + t;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* Kc = a.k_cache + (slot_b * a.Hkv + kvh) * (int64_t)a.max_seq * D;
  const uint16_t* Vc = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq;
  const int L_valid = p0 + a.T;
  const int kv_end = p0 + min(a.T, (tile + 1) * QT);
  const int nkt = (kv_end + KT - 1) / KT;

  int k_src[KI], v_src[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int n = wave * KI + i;
    const int r = (n * 64 + lane) / CR, p = (n * 64 + lane) % CR;
    k_src[i] = f16_key_of_row(r) * D + (p ^ f16_kswz<CR>(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int n = wave * VI + i;
    const int d = (n * 64 + lane) / 8, p = (n * 64 + lane) % 8;
    const int lp = p ^ v_swz(d);
    v_src[i] = (lp / 4) * D * VB + d * VB + (lp % 4) * 8;
  }
  const auto k_rsrc = buffer_rsrc(Kc, a.max_seq * D * 2);
  const auto v_rsrc = buffer_rsrc(Vc, a.max_seq * D * 2);
#define F16_COPY(k0_, stage_)                                                                 \
  {                                                                                           \
    uint8_t* S_ = flash_smem + (stage_) * L::STAGE;                                           \
    _Pragma("unroll") for (int i = 0; i < KI; ++i)                                            \
        copy16_to_lds(k_rsrc, ((k0_) * D + k_src[i]) * 2, 0, (lds_void*)(S_ + (wave * KI + i) * 1024)); \
    _Pragma("unroll") for (int i = 0; i < VI; ++i)                                            \
        copy16_to_lds(v_rsrc, ((k0_) / VB * D * VB + v_src[i]) * 2, 0,                       \
                      (lds_void*)(S_ + KT * L::KROW + (wave * VI + i) * 1024));               \
  }
#define F16_ZERO_TAIL(k0_, stage_)                                                           \
  {                                                                                          \
    uint8_t* V_ = flash_smem + (stage_) * L::STAGE + KT * L::KROW;                           \
    const int first = max(L_valid - (k0_), 0);                                               \
    for (int d = tid; d < D; d += 64 * W)                                                    \
      for (int kk = first; kk < KT; ++kk)                                                    \
        *reinterpret_cast<uint16_t*>(V_ + d * L::VROW + (((kk >> 3) ^ v_swz(d)) << 4) + (kk & 7) * 2) = 0; \
  }

  // queries: QK-norm and rotary into stage 1 (rows of D bf16, 8-dim group
  // g of wave row i at g ^ f16_kswz(i)), the rotary table after the stages
  const int RH = a.R / 2;
  float* rct = reinterpret_cast<float*>(flash_smem + L::bytes);
  float* rst = rct + QT * RH;
  uint16_t* qscr = reinterpret_cast<uint16_t*>(flash_smem + L::STAGE);
  F16_COPY(0, 0);
  for (int e = tid; e < QT * RH; e += 64 * W) {
    const int qi = e / RH, i = e % RH;
    const int tq = min(tile * QT + qi, a.T - 1);
    const float2 cs = reinterpret_cast<const float2*>(a.rope)[((int64_t)b * a.T + tq) * RH + i];
    rct[qi * RH + i] = cs.x;
    rst[qi * RH + i] = cs.y;
  }
  __syncthreads();
  {
    QkRaw<D> raw[16];
#pragma unroll
    for (int qi = 0; qi < 16; ++qi) {
      const int tq = tile * QT + qh * 16 + qi;
      if (tq < a.T) {
        raw[qi] = qk_load<D>(a.q + ((int64_t)b * a.T + tq) * a.q_stride + head * D, lane);
      } else {
#pragma unroll
        for (int e = 0; e < D / 64; ++e) raw[qi].x[e] = 0;
      }
    }
    float gq[D / 64];
    qk_gain<D>(a.q_norm, lane, gq);
#pragma unroll
    for (int qi = 0; qi < 16; ++qi)
      qk_finish<D>(raw[qi], gq, rct + (qh * 16 + qi) * RH, rst + (qh * 16 + qi) * RH, a.R, a.eps,
                   qscr + (wave * 16 + qi) * D, f16_kswz<CR>(qi), lane);
  }
  __syncthreads();
  const int ksw = f16_kswz<CR>(c), vsw = v_swz(c);
  bf16x8 qf[NDS];
  {
    const uint16_t* qr = qscr + (wave * 16 + c) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = *reinterpret_cast<const bf16x8*>(qr + (((4 * ds + rg) ^ ksw) << 3));
  }
  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_i = -1e30f, l_i = 0.f;
  const float scale = a.scale_log2;
  const int qpos_lo = p0 + tile * QT + qh * 16;  // first query of the wave
  wait_vmem();
  __syncthreads();
  if (KT > L_valid) {
    F16_ZERO_TAIL(0, 0);
    __syncthreads();
  }

  f32x4 s[4];
  float mloc;
  bool bump;
#define F16_SYNC(j_)                                                   \
  {                                                                    \
    wait_vmem();                                                       \
    __syncthreads();                                                   \
    if ((j_) + 1 < nkt && ((j_) + 2) * KT > L_valid) {                 \
      F16_ZERO_TAIL(((j_) + 1) * KT, ((j_) + 1) & 1);                  \
      __syncthreads();                                                 \
    }                                                                  \
  }
  int j = 0;
  for (;;) {
    for (; j < nkt; ++j) {
      const uint8_t* sK = flash_smem + (j & 1) * L::STAGE;
      const int k0 = j * KT;
      if (j + 1 < nkt) F16_COPY(k0 + KT, (j + 1) & 1);
      // S^T: step g multiplies key block g % 4 by dims 32 (g / 4) ..: four
      // independent accumulation chains
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      {
        const uint8_t* kr = sK + c * L::KROW;
        bf16x8 kf[4 * NDS];
#define F16_KREAD(g_) \
  kf[g_] = *reinterpret_cast<const bf16x8*>(kr + ((g_) & 3) * 16 * L::KROW + (((4 * ((g_) >> 2) + rg) ^ ksw) << 4))
#pragma unroll
        for (int g = 0; g < FD; ++g) F16_KREAD(g);
#pragma unroll
        for (int g = 0; g < 4 * NDS; ++g) {
          if (g + FD < 4 * NDS) F16_KREAD(g + FD);
          s[g & 3] = mfma16x16x32(kf[g], qf[g >> 2], s[g & 3]);
        }
#undef F16_KREAD
        __builtin_amdgcn_sched_group_barrier(0x100, FD, 0);
#pragma unroll
        for (int g = 0; g < 4 * NDS; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (g + FD < 4 * NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      // causal mask on tiles that reach past the wave's first query:
      // register r of block kb holds key k0 + f16_key_of_row(16 kb + 4 rg + r)
      if (k0 + KT - 1 > qpos_lo) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + f16_key_of_row(16 * kb + 4 * rg + r);
            s[kb][r] = (key <= qpos) ? s[kb][r] : -1e30f;
          }
      }
      // online softmax in log2 units; the reference max m_i moves only when
      // a tile's max exceeds it by more than 8
      mloc = -1e30f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, s[kb][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * scale;
      bump = mloc > m_i + 8.f;
      if (__builtin_amdgcn_read_exec() & __ballot(bump)) break;
      flash16_pv<NDB, FD, L::VROW>(o, s, l_i, m_i, scale, sK + KT * L::KROW + c * L::VROW, vsw, rg);
      F16_SYNC(j);
    }
    if (j >= nkt) break;
    {
      const float m_new = bump ? mloc : m_i;
      const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
      m_i = m_new;
    }
    flash16_pv<NDB, FD, L::VROW>(o, s, l_i, m_i, scale, flash_smem + (j & 1) * L::STAGE + KT * L::KROW + c * L::VROW,
                                 vsw, rg);
    F16_SYNC(j);
    ++j;
  }
#undef F16_SYNC
#undef F16_COPY
#undef F16_ZERO_TAIL
  // the query's sum over its four lanes (each holds the keys of its rows)
  l_i += __shfl_xor(l_i, 16, 64);
  l_i += __shfl_xor(l_i, 32, 64);
  if (!qvalid) return;
  const float inv_l = 1.f / l_i;
  const uint16_t* g = a.gate + m * a.gate_stride + head * D;
  uint16_t* out = a.out + m * a.out_stride + head * D;
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    const int d = 16 * i + 4 * rg;
    uint2 gv = *reinterpret_cast<const uint2*>(g + d);
    const uint16_t* ge = reinterpret_cast<const uint16_t*>(&gv);
    uint16_t r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = f2bf_bits(o[i][e] * inv_l * sigmoidf_(bf2f(ge[e])));
    *reinterpret_cast<uint2*>(out + d) = *reinterpret_cast<uint2*>(r);
  }
}

// --------------------------------------------------------------- decode
// Workgroup = (split of DEC_SPLIT keys, KV head, sequence): the G query heads
// of the KV head against keys [split*DEC_SPLIT, min(pos+1, ...)).  HBM-bound:
// every K and V^T byte of the split is read once, straight from HBM into MFMA
// operands, and nothing else touches memory inside the loop.
//
// Each wave takes 32-key steps (waves interleaved over the split) and keeps
// its own online softmax in registers.  Scores S^T[key][g] = K . q^T on
// v_mfma_f32_16x16x32_bf16 (16 keys x 16 head columns, G used), two passes
// per step.  The A-operand lane of row i loads key 8*(i/4) + 4u + i%4 in pass
// u, so the lane holding head g (= lane % 16) and row group lg (= lane / 16)
// ends up with exactly keys 8 lg .. 8 lg + 7: the bf16 probabilities of those
// keys are the B operand of O^T[d][g] += V^T[d][key] P[key][g] as they stand,
// with no exchange between lanes.  O^T accumulates in the same lanes (head g
// = lane % 16), so the softmax rescale is lane-local.  At the end the four
// waves merge through LDS and the workgroup writes, per head, the
// unnormalised o[D], its max m (log2 units) and its sum l; the combine kernel
// merges the splits in split order.
constexpr int DEC_NT = 256;
constexpr int DEC_SPLIT = DEC_SPLIT_KEYS;

template <int D, int G>
__global__ __launch_bounds__(DEC_NT, 2) void decode_attn_kernel(DecodeAttnArgs a) {
  static_assert(G <= 16, "query heads per KV head");
  constexpr int NKS = D / 32;   // 32-dim steps of the score MFMA
  constexpr int NDT = D / 16;   // 16-dim output tiles
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wo[4][G][D];
  __shared__ u32x4 sq[16 * D / 8];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int pos = a.pos[b];
  const int k_begin = split * DEC_SPLIT;
  const int k_end = min(pos + 1, k_begin + DEC_SPLIT);
  if (k_begin >= k_end) return;  // past the sequence: the combine never reads it
  const int nk = k_end - k_begin;
  const int64_t slot_b = a.seq_slot[b];
  const uint16_t* Kc = a.k_cache + ((slot_b * a.Hkv + kvh) * (int64_t)a.max_seq + k_begin) * D;
  const uint16_t* Vc = a.v_cache + (slot_b * a.Hkv + kvh) * (int64_t)D * a.max_seq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  // q^T operand, kept in LDS (registers go to the loads in flight): lane
  // supplies q[g = l16][32 ks + 8 lg .. +8], zero for g >= G.  QK-norm and
  // partial rotary of the G query heads here, from the projection.
  {
    __shared__ float rc[D / 2], rs[D / 2];
    const int lane0 = threadIdx.x & 63, wave0 = threadIdx.x >> 6;
    if (threadIdx.x < a.R / 2) {
      const float2 cs = reinterpret_cast<const float2*>(a.rope)[(int64_t)b * (a.R / 2) + threadIdx.x];
      rc[threadIdx.x] = cs.x;
      rs[threadIdx.x] = cs.y;
    }
    for (int i = G * D / 8 + threadIdx.x; i < 16 * D / 8; i += DEC_NT) sq[i] = (u32x4){0, 0, 0, 0};
    __syncthreads();
    for (int g = wave0; g < G; g += DEC_NT / 64)
      qk_norm_rope<D>(a.q + (int64_t)b * a.q_stride + (kvh * G + g) * D, a.q_norm, rc, rs, a.R, a.eps,
                      reinterpret_cast<uint16_t*>(sq) + g * D, 0, lane0);
    __syncthreads();
  }
  // Buffer loads: one 32-bit lane offset per step, the per-load displacements
  // in the instruction's immediate (K) or a scalar offset (V^T tiles).  The K
  // range ends at key nk, so K rows past it read as zero (and are masked).
  const int krow = 8 * (l16 >> 2) + (l16 & 3);  // key of this A-operand row in pass 0 (pass 1: + 4)
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(Kc, (uint32_t)nk * D * 2);
  // V^T range: this (sequence, head)'s blocks
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(Vc, (uint32_t)((int64_t)D * a.max_seq * 2));
  const int kvo = (krow * D + lg * 8) * 2;
  // V^T of the step's 32 keys is one block [D][32]: lane (l16, lg) reads dim
  // row 16 dt + l16, keys 8 lg ..
  const int vvo = (l16 * VB + lg * 8) * 2;

  float m = -1e30f, l = 0.f;  // running max (log2 units) and this lane's partial sum
  f32x4 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = (f32x4){0, 0, 0, 0};

  for (int kb = wave * 32; kb < nk; kb += 4 * 32) {
    u32x4 kv[2][NKS], vv[NDT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kv[u][ks] = buffer_load16(krs, kvo + (kb * D + u * 4 * D + ks * 32) * 2, 0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vv[dt] = buffer_load16(vrs, vvo + (k_begin + kb) / VB * (D * VB * 2), dt * 16 * VB * 2);
    if (kb + 32 > nk) {
      // ragged last step: V^T entries of keys at or past nk are zeroed (their
      // probabilities are zero, but the cache there may hold anything)
      const int kk = kb + lg * 8;  // first of this lane's 8 keys
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w = vv[dt][j];
          if (kk + 2 * j >= nk) w &= 0xFFFF0000u;
          if (kk + 2 * j + 1 >= nk) w &= 0x0000FFFFu;
          vv[dt][j] = w;
        }
    }
    // the two key groups' accumulations interleaved: two independent chains
    f32x4 sacc[2] = {(f32x4){0, 0, 0, 0}, (f32x4){0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        sacc[u] = mfma16x16x32(__builtin_bit_cast(bf16x8, kv[u][ks]),
                               __builtin_bit_cast(bf16x8, sq[l16 * (D / 8) + ks * 4 + lg]), sacc[u]);
    // lane holds keys kb + 8 lg + 4 u + r of head l16
    float sv[8];
    float mx = -1e30f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb + 8 * lg + 4 * u + r;
        sv[4 * u + r] = key < nk ? sacc[u][r] * a.scale_log2 : -1e30f;
        mx = fmaxf(mx, sv[4 * u + r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    m = m_new;
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = l16 < G ? exp2f(sv[j] - m_new) : 0.f;
      ps += p;
      pf[j] = f2bf(p);
    }
    l = l * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      o[dt] *= alpha;
      o[dt] = mfma16x16x32(__builtin_bit_cast(bf16x8, vv[dt]), pf, o[dt]);
    }
  }
  // this wave's sum over its keys: the four row groups of head l16
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (l16 < G) {
    if (lg == 0) { wm[wave][l16] = m; wl[wave][l16] = l; }
    // lane holds O^T[d = 16 dt + 4 lg + r][g = l16]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wo[wave][l16][dt * 16 + 4 * lg + r] = o[dt][r];
  }
  __syncthreads();
  float* part = a.partial + (((int64_t)b * a.Hq + kvh * G) * a.n_split + split) * (D + 2);
  const int64_t part_head_stride = (int64_t)a.n_split * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += DEC_NT) {
    const int g = i / D, dd = i % D;
    const float M = fmaxf(fmaxf(wm[0][g], wm[1][g]), fmaxf(wm[2][g], wm[3][g]));
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += wo[w][g][dd] * exp2f(wm[w][g] - M);
    part[g * part_head_stride + dd] = acc;
    if (dd == 0) {
      float Ls = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) Ls += wl[w][g] * exp2f(wm[w][g] - M);
      part[g * part_head_stride + D] = M;
      part[g * part_head_stride + D + 1] = Ls;
    }
  }
}

// Merge the splits of one (sequence, query head) in split order (only the
// splits that hold keys of the sequence); apply the output gate; store bf16.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeAttnArgs a) {
  __shared__ float wsplit[DEC_MAX_SPLITS];
  __shared__ float red[4];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int ns = (a.pos[b] + DEC_SPLIT) / DEC_SPLIT;  // splits holding keys 0..pos
  const float* part = a.partial + ((int64_t)b * a.Hq + hq) * a.n_split * (D + 2);
  float mloc = -1e30f;
  for (int s = threadIdx.x; s < ns; s += 256) mloc = fmaxf(mloc, part[s * (D + 2) + D]);
  mloc = wave_max(mloc);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int s = threadIdx.x; s < ns; s += 256) wsplit[s] = exp2f(part[s * (D + 2) + D] - M);
  __syncthreads();
  float Lsum = 0.f;
  for (int s = 0; s < ns; ++s) Lsum += part[s * (D + 2) + D + 1] * wsplit[s];
  const uint16_t* g = a.gate + (int64_t)b * a.gate_stride + hq * D;
  uint16_t* out = a.out + (int64_t)b * a.out_stride + hq * D;
  for (int d = threadIdx.x; d < D; d += 256) {
    float o = 0.f;
    int s = 0;
    for (; s + 8 <= ns; s += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[(s + j) * (D + 2) + d];
#pragma unroll
      for (int j = 0; j < 8; ++j) o += v[j] * wsplit[s + j];
    }
    for (; s < ns; ++s) o += part[s * (D + 2) + d] * wsplit[s];
    out[d] = f2bf_bits(o / Lsum * sigmoidf_(bf2f(g[d])));
  }
}

template <int D>
hipError_t prep_d(const AttnPrepArgs& a, int M, hipStream_t s) {
  hipLaunchKernelGGL(qk_prep_kernel<D>, dim3(M), dim3(256), 0, s, a);
  const int B = M / a.T;
  hipLaunchKernelGGL(v_transpose_kernel<D>, dim3((a.T + VT_TOK - 1) / VT_TOK, a.Hkv, B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t flash16_d(const FlashArgs& a, int B, hipStream_t s) {
  constexpr int QT = 32;
  constexpr size_t LDS_MAX = 160 * 1024;
  const size_t lds = FlashLds<D>::bytes + 2 * (size_t)QT * (a.R / 2) * sizeof(float);
  if (a.R < 0 || a.R > D || a.R % 2 || lds > LDS_MAX) return hipErrorInvalidValue;
  auto k = flash16_prefill_kernel<D>;
  // the kernel's static LDS counts against the same 160 KB: the dynamic
  // limit is raised to what the call asks for
  static size_t attr = 0;
  if (lds > attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = lds;
  }
  hipLaunchKernelGGL(k, dim3((a.T + QT - 1) / QT, a.Hkv, B), dim3(512), lds, s, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t flash_dg(const FlashArgs& a, int B, hipStream_t s) {
  if constexpr (G == 4) return flash16_d<D>(a, B, s);
  constexpr int W = G < 4 ? 4 : G;
  constexpr int QT = 32 * W / G;
  constexpr size_t LDS_MAX = 160 * 1024;
  // the two stages, then the rotary table of the tile's query positions
  const size_t lds = FlashLds<D>::bytes + 2 * (size_t)QT * (a.R / 2) * sizeof(float);
  if (a.R < 0 || a.R > D || a.R % 2 || lds > LDS_MAX) return hipErrorInvalidValue;
  auto k = flash_prefill_kernel<D, G>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_MAX);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(k, dim3((a.T + QT - 1) / QT, a.Hkv, B), dim3(64 * W), lds, s, a);
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
  if (a.R < 0 || a.R > D || a.R % 2) return hipErrorInvalidValue;
  if (a.split_len != DEC_SPLIT || a.n_split > DEC_MAX_SPLITS || (int64_t)a.n_split * DEC_SPLIT < a.max_seq)
    return hipErrorInvalidValue;
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
  if (a.R < 0 || a.R > a.D || a.R % 2) return hipErrorInvalidValue;
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
