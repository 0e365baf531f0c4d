// The model entry points: create / destroy, prefill, decode step, and the
// executor that replays the execution schedule over the shared weights.
//
// [P1 section 2], [P2 section 2]: the schedule runs the head layers, the
// shared block loop_passes times with the same weights, the tail layers,
// then the head.  [P1 section 4]: every execution owns its KV cache (full
// attention) or state (Gated-DeltaNet) slot in the arena.  [P1 section 5],
// [P1 section 6]: inside the loop the residual is the pair of mHC streams:
// fork on entry, read / mix / write per execution, merge on exit.
//
// Per execution (M = batch * tokens rows):
//   in-proj GEMM (xn -> proj, bf16)
//   mixer: full attention (prep + flash or split decode) or GDN (chunked or
//          recurrent) -> o (bf16, gated / normed)
//   O-proj GEMM: plain hmid = h + o W_o^T; loop a = o W_o^T
//   RMSNorm of hmid (plain) or x + a (loop) -> hn
//   gate/up GEMM with SwiGLU epilogue -> act
//   down GEMM: plain h = hmid + act W_down^T; loop out = a + act W_down^T
//   transition to the next execution (mHC write / fork / read / merge + the
//   next pre-norm) -> xn
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <set>

#include "host.h"

namespace {

constexpr size_t ALIGN = 256;
constexpr int DEC_SPLIT = DEC_SPLIT_KEYS;  // keys per decode-attention split (decode_attn_kernel)

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  size_t meta, h, hmid, x, a, s0, s1, xn, hn, proj, obuf, act, rope;
  size_t gW, gUt, gM, gKt, gSc, gS;
  size_t xf, logits, am_v, am_i, dec_part, mhc, splitk;
  size_t splitk_bytes;
  size_t total;
  int n_in_max, chunk_slots, n_split_max;
};

int n_in_full(const loop_config& c) { return 2 * c.n_q_heads * c.head_dim + 2 * c.n_kv_heads * c.head_dim; }
int n_in_gdn(const loop_config& c) { return 2 * c.gdn_heads * c.gdn_dk + 2 * c.gdn_heads * c.gdn_dv + 2 * c.gdn_heads; }

int64_t head_rows(const loop_config& c, int64_t M) {
  return std::max<int64_t>(c.max_batch, std::min<int64_t>(M, (int64_t)LOOP_VERIFY_MAX * c.max_batch));
}

Layout layout(const loop_config& c, int64_t M) {
  Layout L{};
  const int64_t d = c.d_model, B = c.max_batch;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
  // rows of the input projection padded to 8 elements: 16-byte vector reads
  L.n_in_max = (std::max(n_in_full(c), n_in_gdn(c)) + 7) / 8 * 8;
  L.meta = take(4 * B * sizeof(int32_t));
  L.h = take(M * d * 4);
  L.hmid = take(M * d * 4);
  L.x = take(M * d * 4);
  L.a = take(M * d * 4);
  L.s0 = take(M * d * 4);
  L.s1 = take(M * d * 4);
  L.xn = take(M * d * 2);
  L.hn = take(M * d * 2);
  L.proj = take(M * (int64_t)L.n_in_max * 2);
  L.obuf = take(M * (int64_t)std::max(c.n_q_heads * c.head_dim, c.gdn_heads * c.gdn_dv) * 2);
  L.act = take(M * (int64_t)c.d_ff * 2);
  L.rope = take(M * (int64_t)(c.rotary_dim / 2) * 2 * 4);
  // chunk workspace: (sum over sequences of their chunks) * heads
  L.chunk_slots = (int)((M + 63) / 64 + B);
  const int64_t cs = (int64_t)L.chunk_slots * c.gdn_heads;
  L.gW = take(cs * 64 * c.gdn_dk * 4);
  L.gUt = take(cs * 64 * c.gdn_dv * 4);
  L.gM = take(cs * 64 * 64 * 4);
  L.gKt = take(cs * 64 * c.gdn_dk * 2);
  L.gS = take(cs * 64 * c.gdn_dv * 4);
  L.gSc = take(cs * (int64_t)gdn_chunk_scales() * 4);
  // final-norm rows and argmax partials: one per sequence, or up to
  // LOOP_VERIFY_MAX per sequence for a verify step
  const int64_t HR = head_rows(c, M);
  L.xf = take(HR * d * 2);
  L.logits = take(B * (int64_t)std::max(c.vocab, 1) * 4);
  L.am_v = take(HR * (int64_t)argmax_chunks(std::max(c.vocab, 1)) * 4);
  L.am_i = take(HR * (int64_t)argmax_chunks(std::max(c.vocab, 1)) * 4);
  L.n_split_max = (c.max_seq + DEC_SPLIT - 1) / DEC_SPLIT;
  L.dec_part = take(B * (int64_t)c.n_q_heads * L.n_split_max * (c.head_dim + 2) * 4);
  L.mhc = take(std::max(c.loop_end - c.loop_start, 1) * 4 * 4);
  // split-K partials of the small-M (decode) projections: up to 16 splits of
  // [64 rows][widest output] (SwiGLU keeps gate and up: 2 x d_ff)
  {
    const int64_t rows = std::min<int64_t>(M, 512);
    const int64_t widest = std::max<int64_t>({2LL * c.d_ff, (int64_t)L.n_in_max, (int64_t)c.d_model});
    L.splitk_bytes = (size_t)(16 * rows * widest * 4);
    L.splitk = take(L.splitk_bytes);
  }
  L.total = off;
  return L;
}

}  // namespace

struct loop_model {
  loop_config cfg;
  std::vector<loop_layer_weights> lw;
  const void *embed, *final_norm, *head;
  char* arena;
  size_t arena_bytes;
  char* ws;
  size_t ws_bytes;
  Layout L;
  std::vector<ExecDesc> sched;
  // sched_p[p - 1]: the executions of a call that runs the block p times
  // (p = 1 .. loop_passes); each keeps its slot of the full schedule
  std::vector<std::vector<ExecDesc>> sched_p;
  // pass count each sequence slot was started with (0: not started by a
  // prefill from position 0 here)
  std::vector<int32_t> slot_passes;
  // int8 or int4 codes of the layer projections for decode steps (both
  // empty: bf16; at most one of them is set)
  std::vector<loop_q8_layer> q8;
  std::vector<loop_q4_layer> q4;
  std::vector<int32_t> meta_host;
  // kernel-class timing
  int prof_class = -1;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_events;
  size_t prof_used = 0;
};

extern "C" int64_t loop_workspace_bytes(const loop_config* c, int32_t max_tokens) {
  if (validate_config(c) || max_tokens <= 0) return -1;
  return (int64_t)layout(*c, max_tokens).total;
}

static int check_weights(const loop_config& c, const loop_weights* w, const std::vector<ExecDesc>& s) {
  if (!w) return loop_fail(LOOP_EINVAL, "weights are NULL");
  if (w->n_layers != c.n_layers || !w->layers) return loop_fail(LOOP_EINVAL, "weights: n_layers mismatch or no layer array");
  if (!w->final_norm) return loop_fail(LOOP_EINVAL, "weights: final_norm is NULL");
  if (c.vocab > 0 && (!w->embed || !w->head)) return loop_fail(LOOP_EINVAL, "weights: embed / head NULL with vocab > 0");
  for (int l = 0; l < c.n_layers; ++l) {
    const loop_layer_weights& x = w->layers[l];
    if (!x.attn_norm || !x.ffn_norm || !x.w_in || !x.w_o || !x.w_gateup || !x.w_down)
      return loop_fail(LOOP_EINVAL, "weights: layer %d misses a matrix or norm gain", l);
    const bool full = l % 4 == 3;
    if (full && (!x.q_norm || !x.k_norm)) return loop_fail(LOOP_EINVAL, "weights: layer %d needs q_norm, k_norm", l);
    if (!full && !x.o_norm) return loop_fail(LOOP_EINVAL, "weights: layer %d needs o_norm", l);
    const bool loop = l >= c.loop_start && l < c.loop_end;
    if (loop && (!x.mhc_read_w || !x.mhc_read_b || !x.mhc_write_w || !x.mhc_write_b || !x.mhc_mix))
      return loop_fail(LOOP_EINVAL, "weights: loop layer %d needs its mHC parameters", l);
  }
  (void)s;
  return 0;
}

extern "C" int loop_model_create(const loop_config* cfg, const loop_weights* w, void* d_arena,
                                 size_t arena_bytes, void* d_workspace, size_t ws_bytes,
                                 loop_model** out) {
  if (!out) return loop_fail(LOOP_EINVAL, "out is NULL");
  *out = nullptr;
  if (int e = validate_config(cfg)) return e;
  std::vector<ExecDesc> sched;
  build_schedule(*cfg, sched);
  if (int e = check_weights(*cfg, w, sched)) return e;
  const int64_t need_arena = loop_arena_bytes(cfg);
  const Layout L = layout(*cfg, cfg->max_tokens);
  if (!d_arena || arena_bytes < (size_t)need_arena)
    return loop_fail(LOOP_ECAPACITY, "arena: %zu bytes given, %lld needed", arena_bytes, (long long)need_arena);
  if (!d_workspace || ws_bytes < L.total)
    return loop_fail(LOOP_ECAPACITY, "workspace: %zu bytes given, %zu needed", ws_bytes, L.total);
  if (((uintptr_t)d_arena | (uintptr_t)d_workspace) % ALIGN)
    return loop_fail(LOOP_EINVAL, "arena and workspace must be %zu-byte aligned", ALIGN);
  int dev = 0;
  hipDeviceProp_t prop;
  hipError_t he = hipGetDevice(&dev);
  if (he == hipSuccess) he = hipGetDeviceProperties(&prop, dev);
  if (he != hipSuccess) return loop_hip_fail(he, "device query");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return loop_fail(LOOP_EDEVICE, "device is %s, gfx950 required", prop.gcnArchName);
  loop_model* m = new loop_model();
  m->cfg = *cfg;
  m->lw.assign(w->layers, w->layers + cfg->n_layers);
  m->embed = w->embed;
  m->final_norm = w->final_norm;
  m->head = w->head;
  m->arena = (char*)d_arena;
  m->arena_bytes = arena_bytes;
  m->ws = (char*)d_workspace;
  m->ws_bytes = ws_bytes;
  m->L = L;
  m->sched = sched;
  // Executions of a p-pass call: the head, the block's first p passes, the
  // tail, in schedule order, with the merge moved to the end of pass p.
  const int blk = cfg->loop_end - cfg->loop_start;
  for (int p = 1; p <= cfg->loop_passes; ++p) {
    std::vector<ExecDesc> sp;
    for (int e = 0; e < (int)sched.size(); ++e) {
      const bool in_block = e >= cfg->loop_start && e < cfg->loop_start + blk * cfg->loop_passes;
      if (in_block && (e - cfg->loop_start) / blk >= p) continue;
      ExecDesc d = sched[e];
      if (blk > 0 && in_block) d.merge = e == cfg->loop_start + blk * p - 1;
      sp.push_back(d);
    }
    m->sched_p.push_back(sp);
  }
  m->slot_passes.assign(cfg->max_batch, 0);
  *out = m;
  return 0;
}

extern "C" void loop_model_destroy(loop_model* m) {
  if (!m) return;
  for (auto& p : m->prof_events) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  delete m;
}

namespace {
// Scoped timing of one launch group of the selected class.
struct Prof {
  loop_model* m;
  hipStream_t s;
  int idx = -1;
  Prof(loop_model* m_, int cls, hipStream_t s_) : m(m_), s(s_) {
    if (m->prof_class != cls) return;
    if (m->prof_used == m->prof_events.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      m->prof_events.push_back({a, b});
    }
    idx = (int)m->prof_used++;
    (void)hipEventRecord(m->prof_events[idx].first, s);
  }
  ~Prof() {
    if (idx >= 0) (void)hipEventRecord(m->prof_events[idx].second, s);
  }
};
}  // namespace

extern "C" int loop_profile(loop_model* m, int32_t kernel_class) {
  if (!m) return loop_fail(LOOP_EINVAL, "model is NULL");
  if (kernel_class < -1 || kernel_class >= LOOP_K_NCLASS) return loop_fail(LOOP_EINVAL, "bad kernel class %d", kernel_class);
  m->prof_class = kernel_class;
  m->prof_used = 0;
  return 0;
}

extern "C" int loop_profile_read(loop_model* m, double* total_ms, int64_t* launches) {
  if (!m || !total_ms || !launches) return loop_fail(LOOP_EINVAL, "NULL argument");
  double t = 0;
  for (size_t i = 0; i < m->prof_used; ++i) {
    hipError_t e = hipEventSynchronize(m->prof_events[i].second);
    if (e != hipSuccess) return loop_hip_fail(e, "profile event");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, m->prof_events[i].first, m->prof_events[i].second);
    if (e != hipSuccess) return loop_hip_fail(e, "profile elapsed");
    t += ms;
  }
  *total_ms = t;
  *launches = (int64_t)m->prof_used;
  m->prof_used = 0;
  return 0;
}

namespace {

struct Call {
  int B, T, M;
  bool decode;
  const int32_t* d_pos;
  const int32_t* d_slot;
  const int32_t* d_last;
  const std::vector<ExecDesc>* sched;  // this call's executions
  bool taps_all = false;               // taps at every position (verify), not the last
};

#define HIP_TRY(x)                                              \
  do {                                                          \
    hipError_t e_ = (x);                                        \
    if (e_ != hipSuccess) return loop_hip_fail(e_, #x);         \
  } while (0)

template <typename T>
T* at(loop_model* m, size_t off) { return reinterpret_cast<T*>(m->ws + off); }

// The sequence mixer of one execution: from the in-projection output in the
// workspace (proj, rows of n_in_max) to the gated / normed mixer output
// (obuf, rows of *mix_width), with the execution's cache slot.
int run_mixer(loop_model* m, const Call& k, const ExecDesc& d, hipStream_t s, int* mix_width_out) {
  const loop_config& c = m->cfg;
  const Layout& L = m->L;
  const loop_layer_weights& w = m->lw[d.layer];
  const int M = k.M;
  uint16_t* proj = at<uint16_t>(m, L.proj);
  uint16_t* obuf = at<uint16_t>(m, L.obuf);
  int mix_width;
  if (d.full) {
    const int Hq = c.n_q_heads, Hkv = c.n_kv_heads, D = c.head_dim;
    mix_width = Hq * D;
    const int64_t kv_off = loop_cache_offset(&c, 0, d.slot, 0);
    const int64_t v_off = loop_cache_offset(&c, 1, d.slot, 0);
    AttnPrepArgs p{};
    p.proj = proj; p.proj_stride = L.n_in_max;
    p.T = k.T; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.R = c.rotary_dim; p.max_seq = c.max_seq;
    p.theta = c.rope_theta; p.eps = c.eps;
    p.pos = k.d_pos; p.seq_slot = k.d_slot;
    p.k_norm = (const uint16_t*)w.k_norm;
    p.rope = at<float>(m, L.rope);
    p.k_cache = (uint16_t*)(m->arena + kv_off);
    p.v_cache = (uint16_t*)(m->arena + v_off);
    {
      Prof pr(m, LOOP_K_ATTN_PREP, s);
      HIP_TRY(launch_attn_prep(p, M, s));
    }
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    if (!k.decode) {
      FlashArgs f{};
      f.q = proj; f.q_stride = L.n_in_max; f.q_norm = (const uint16_t*)w.q_norm;
      f.R = c.rotary_dim; f.eps = c.eps; f.rope = p.rope;
      f.T = k.T; f.Hq = Hq; f.Hkv = Hkv; f.D = D; f.max_seq = c.max_seq;
      f.pos = k.d_pos; f.seq_slot = k.d_slot; f.k_cache = p.k_cache; f.v_cache = p.v_cache;
      f.scale_log2 = scale_log2;
      f.gate = proj + Hq * D; f.gate_stride = L.n_in_max;
      f.out = obuf; f.out_stride = mix_width;
      Prof pr(m, LOOP_K_FLASH, s);
      HIP_TRY(launch_flash_prefill(f, k.B, s));
    } else {
      DecodeAttnArgs g{};
      g.q = proj; g.q_stride = L.n_in_max; g.q_norm = (const uint16_t*)w.q_norm;
      g.R = c.rotary_dim; g.eps = c.eps; g.rope = p.rope;
      g.Hq = Hq; g.Hkv = Hkv; g.D = D; g.max_seq = c.max_seq;
      g.pos = k.d_pos; g.seq_slot = k.d_slot; g.k_cache = p.k_cache; g.v_cache = p.v_cache;
      g.scale_log2 = scale_log2;
      g.split_len = DEC_SPLIT; g.n_split = L.n_split_max;
      g.partial = at<float>(m, L.dec_part);
      g.gate = proj + Hq * D; g.gate_stride = L.n_in_max;
      g.out = obuf; g.out_stride = mix_width;
      Prof pr(m, LOOP_K_DECODE_ATTN, s);
      HIP_TRY(launch_decode_attn(g, k.B, s));
    }
  } else {
    const int H = c.gdn_heads, Dk = c.gdn_dk, Dv = c.gdn_dv;
    mix_width = H * Dv;
    GdnArgs g{};
    g.proj = proj; g.proj_stride = L.n_in_max;
    g.off_q = 0; g.off_k = H * Dk; g.off_v = 2 * H * Dk; g.off_z = 2 * H * Dk + H * Dv;
    g.off_a = 2 * H * Dk + 2 * H * Dv; g.off_b = g.off_a + H;
    g.H = H; g.Dk = Dk; g.T = k.T; g.n_chunks = gdn_chunks(k.T);
    g.eps = c.eps; g.q_scale = (float)(1.0 / sqrt((double)Dk));
    g.pos = k.d_pos; g.seq_slot = k.d_slot;
    g.state = (float*)(m->arena + loop_cache_offset(&c, 2, d.slot, 0));
    g.W = at<float>(m, L.gW); g.Ut = at<float>(m, L.gUt); g.Mq = at<float>(m, L.gM);
    g.Kt = at<uint16_t>(m, L.gKt);
    g.sc = at<float>(m, L.gSc);
    g.Oq = at<float>(m, L.gS);
    g.o_norm = (const uint16_t*)w.o_norm;
    g.out = obuf; g.out_stride = mix_width;
    Prof pr(m, LOOP_K_GDN, s);
    if (k.decode) HIP_TRY(launch_gdn_recurrent(g, k.B, s));
    else HIP_TRY(launch_gdn_prefill(g, k.B, s));
  }
  *mix_width_out = mix_width;
  return 0;
}

int run_exec(loop_model* m, const Call& k, int e, hipStream_t s) {
  const loop_config& c = m->cfg;
  const Layout& L = m->L;
  const std::vector<ExecDesc>& sched = *k.sched;
  const ExecDesc& d = sched[e];
  const loop_layer_weights& w = m->lw[d.layer];
  const int M = k.M, dm = c.d_model;
  uint16_t* xn = at<uint16_t>(m, L.xn);
  uint16_t* proj = at<uint16_t>(m, L.proj);
  uint16_t* obuf = at<uint16_t>(m, L.obuf);
  float* h = at<float>(m, L.h);
  float* hmid = at<float>(m, L.hmid);
  float* x = at<float>(m, L.x);
  float* a = at<float>(m, L.a);
  const int n_in = d.full ? n_in_full(c) : n_in_gdn(c);
#define SK at<float>(m, L.splitk), L.splitk_bytes

  // decode steps with int8 or int4 codes registered use them for the four
  // projections (ldq: bytes per code row of a K-deep matrix)
  struct QW {
    int bits;
    const void *w_in, *w_o, *w_gateup, *w_down;
    const float *s_in, *s_o, *s_gateup, *s_down;
  } qw{};
  const QW* wq = nullptr;
  if (k.decode && !m->q8.empty()) {
    const loop_q8_layer& q = m->q8[d.layer];
    qw = {8, q.w_in, q.w_o, q.w_gateup, q.w_down, q.s_in, q.s_o, q.s_gateup, q.s_down};
    wq = &qw;
  } else if (k.decode && !m->q4.empty()) {
    const loop_q4_layer& q = m->q4[d.layer];
    qw = {4, q.w_in, q.w_o, q.w_gateup, q.w_down, q.s_in, q.s_o, q.s_gateup, q.s_down};
    wq = &qw;
  }
  auto ldq = [&](int K) -> int64_t { return qw.bits == 8 ? K : K / 2; };
  {
    Prof p(m, LOOP_K_GEMM_IN, s);
    if (wq)
      HIP_TRY(launch_gemm_wq(wq->bits, xn, dm, wq->w_in, ldq(dm), wq->s_in, proj, L.n_in_max, nullptr, M, n_in, dm,
                             LOOP_EPI_BF16, s, SK));
    else
      HIP_TRY(launch_gemm(xn, dm, w.w_in, dm, proj, L.n_in_max, nullptr, M, n_in, dm, LOOP_EPI_BF16, s, SK));
  }
  int mix_width = 0;
  if (int r = run_mixer(m, k, d, s, &mix_width)) return r;
  // O-proj, mid norm, FFN
  uint16_t* hn = at<uint16_t>(m, L.hn);
  uint16_t* act = at<uint16_t>(m, L.act);
  {
    // O-projection and the FFN pre-norm: plain hmid = h + o W_o^T, hn =
    // RMSNorm(hmid); loop a = o W_o^T, hn = RMSNorm(x + a)
    Prof p(m, LOOP_K_GEMM_O, s);
    if (wq && !d.loop)
      HIP_TRY(launch_gemm_norm_wq(wq->bits, obuf, mix_width, wq->w_o, ldq(mix_width), wq->s_o, hmid, dm, h, nullptr,
                                  w.ffn_norm, hn, c.eps, M, dm, mix_width, s, SK));
    else if (wq)
      HIP_TRY(launch_gemm_norm_wq(wq->bits, obuf, mix_width, wq->w_o, ldq(mix_width), wq->s_o, a, dm, nullptr, x,
                                  w.ffn_norm, hn, c.eps, M, dm, mix_width, s, SK));
    else if (!d.loop)
      HIP_TRY(launch_gemm_norm(obuf, mix_width, w.w_o, mix_width, hmid, dm, h, nullptr, w.ffn_norm, hn, c.eps, M, dm,
                               mix_width, s, SK));
    else
      HIP_TRY(launch_gemm_norm(obuf, mix_width, w.w_o, mix_width, a, dm, nullptr, x, w.ffn_norm, hn, c.eps, M, dm,
                               mix_width, s, SK));
  }
  {
    Prof p(m, LOOP_K_GEMM_GATEUP, s);
    if (wq)
      HIP_TRY(launch_gemm_wq(wq->bits, hn, dm, wq->w_gateup, ldq(dm), wq->s_gateup, act, c.d_ff, nullptr, M, c.d_ff,
                             dm, LOOP_EPI_SWIGLU, s, SK));
    else
      HIP_TRY(launch_gemm(hn, dm, w.w_gateup, dm, act, c.d_ff, nullptr, M, c.d_ff, dm, LOOP_EPI_SWIGLU, s, SK));
  }
  {
    Prof p(m, LOOP_K_GEMM_DOWN, s);
    float* dst = d.loop ? a : h;
    const float* res = d.loop ? a : hmid;
    if (wq)
      HIP_TRY(launch_gemm_wq(wq->bits, act, c.d_ff, wq->w_down, ldq(c.d_ff), wq->s_down, dst, dm, res, M, dm,
                             c.d_ff, LOOP_EPI_F32_RES, s, SK));
    else
      HIP_TRY(launch_gemm(act, c.d_ff, w.w_down, c.d_ff, dst, dm, res, M, dm, c.d_ff, LOOP_EPI_F32_RES, s, SK));
  }
  Prof prow(m, LOOP_K_ROWS, s);

  // transition to the next execution
  TransitionArgs t{};
  t.M = M; t.d = dm; t.iters = c.sinkhorn_iters; t.eps = c.eps;
  float* s0 = at<float>(m, L.s0);
  float* s1 = at<float>(m, L.s1);
  t.h = h; t.out = a; t.s0 = s0; t.s1 = s1;
  t.s0_out = s0; t.s1_out = s1; t.x_out = x; t.h_out = h; t.xn = xn;
  if (d.loop) {
    t.in_mode = TR_IN_WRITE;
    t.write_w = w.mhc_write_w; t.write_b = w.mhc_write_b;
    t.P = at<float>(m, L.mhc) + 4 * (d.layer - c.loop_start);
  } else {
    t.in_mode = TR_IN_H;
  }
  const bool last = e + 1 == (int)sched.size();
  if (last) {
    if (d.loop) {
      t.out_mode = TR_OUT_NONE;
      HIP_TRY(launch_transition(t, s));
    }
    return 0;
  }
  const ExecDesc& nd = sched[e + 1];
  const loop_layer_weights& nw = m->lw[nd.layer];
  t.norm_g = (const uint16_t*)nw.attn_norm;
  if (nd.loop && !nd.fork) {  // stay inside the loop
    t.out_mode = TR_OUT_READ;
    t.read_w = nw.mhc_read_w; t.read_b = nw.mhc_read_b;
    HIP_TRY(launch_transition(t, s));
  } else if (nd.fork) {       // enter the loop
    t.out_mode = TR_OUT_READ;
    t.read_w = nw.mhc_read_w; t.read_b = nw.mhc_read_b;
    HIP_TRY(launch_transition(t, s));
  } else if (d.loop) {        // leave the loop: merge + norm
    t.out_mode = TR_OUT_NORM;
    HIP_TRY(launch_transition(t, s));
  } else {                    // plain -> plain
    HIP_TRY(launch_rmsnorm(h, nullptr, nullptr, dm, nw.attn_norm, xn, M, dm, c.eps, s));
  }
  return 0;
}

// First transition: embedded (or given) h -> the first execution's input.
int run_entry(loop_model* m, const Call& k, hipStream_t s) {
  const loop_config& c = m->cfg;
  const Layout& L = m->L;
  const ExecDesc& d = (*k.sched)[0];
  const loop_layer_weights& w = m->lw[d.layer];
  float* h = at<float>(m, L.h);
  if (!d.loop) {
    HIP_TRY(launch_rmsnorm(h, nullptr, nullptr, c.d_model, w.attn_norm, at<uint16_t>(m, L.xn), k.M, c.d_model, c.eps, s));
    return 0;
  }
  TransitionArgs t{};
  t.M = k.M; t.d = c.d_model; t.iters = c.sinkhorn_iters; t.eps = c.eps;
  t.in_mode = TR_IN_H; t.out_mode = TR_OUT_READ;
  t.h = h; t.s0_out = at<float>(m, L.s0); t.s1_out = at<float>(m, L.s1); t.x_out = at<float>(m, L.x);
  t.read_w = w.mhc_read_w; t.read_b = w.mhc_read_b; t.norm_g = (const uint16_t*)w.attn_norm;
  t.xn = at<uint16_t>(m, L.xn);
  HIP_TRY(launch_transition(t, s));
  return 0;
}

int run_forward(loop_model* m, const Call& k, const int32_t* taps, int n_taps, float* d_taps, hipStream_t s) {
  const loop_config& c = m->cfg;
  const Layout& L = m->L;
  // the loop layers' mix matrices, once per call (they depend on weights only)
  if (c.loop_end > c.loop_start) {
    SinkhornBatch sb{};
    sb.n = c.loop_end - c.loop_start;
    sb.iters = c.sinkhorn_iters;
    sb.out = at<float>(m, L.mhc);
    for (int l = 0; l < sb.n; ++l) sb.mix[l] = m->lw[c.loop_start + l].mhc_mix;
    HIP_TRY(launch_sinkhorn_layers(sb, s));
  }
  if (int r = run_entry(m, k, s)) return r;
  for (int e = 0; e < (int)k.sched->size(); ++e) {
    if (int r = run_exec(m, k, e, s)) return r;
    for (int i = 0; i < n_taps; ++i) {
      if (taps[i] != e) continue;
      const ExecDesc& d = (*k.sched)[e];
      const bool streams = d.loop && !d.merge;
      // every position: M "sequences" of length 1
      const int tb = k.taps_all ? k.M : k.B, tt = k.taps_all ? 1 : k.T;
      HIP_TRY(launch_tap(at<float>(m, L.h), streams ? at<float>(m, L.s0) : nullptr,
                         streams ? at<float>(m, L.s1) : nullptr, d_taps + (int64_t)i * tb * c.d_model,
                         tb, tt, c.d_model, s));
    }
  }
  return 0;
}

int upload_meta(loop_model* m, int B, int T, const int32_t* pos, const int32_t* slots, hipStream_t s) {
  m->meta_host.assign(4 * m->cfg.max_batch, 0);
  for (int b = 0; b < B; ++b) {
    m->meta_host[b] = pos[b];
    m->meta_host[m->cfg.max_batch + b] = slots[b];
    m->meta_host[2 * m->cfg.max_batch + b] = b * T + T - 1;
  }
  HIP_TRY(hipMemcpyAsync(m->ws + m->L.meta, m->meta_host.data(), m->meta_host.size() * 4,
                         hipMemcpyHostToDevice, s));
  return 0;
}

int head_logits(loop_model* m, const Call& k, float* logits, hipStream_t s) {
  const loop_config& c = m->cfg;
  const Layout& L = m->L;
  uint16_t* xf = at<uint16_t>(m, L.xf);
  Prof p(m, LOOP_K_HEAD, s);
  HIP_TRY(launch_rmsnorm(at<float>(m, L.h), nullptr, k.d_last, c.d_model, m->final_norm, xf, k.B, c.d_model, c.eps, s));
  HIP_TRY(launch_gemm(xf, c.d_model, m->head, c.d_model, logits, c.vocab, nullptr, k.B, c.vocab, c.d_model,
                      LOOP_EPI_F32, s, at<float>(m, L.splitk), L.splitk_bytes));
  return 0;
}

// The call's block pass count (0 = the configuration's), checked against the
// count each sequence was started with.
int call_passes(loop_model* m, int32_t req, int B, const int32_t* slots, const int32_t* start, int* out) {
  const int p = req == 0 ? m->cfg.loop_passes : req;
  if (p < 1 || p > m->cfg.loop_passes)
    return loop_fail(LOOP_EINVAL, "loop_passes %d out of [1, %d]", req, m->cfg.loop_passes);
  for (int b = 0; b < B; ++b) {
    const int rec = m->slot_passes[slots[b]];
    const bool fresh = start && start[b] == 0;
    if (!fresh && rec != 0 && rec != p)
      return loop_fail(LOOP_EINVAL, "slot %d was started with %d loop passes, this call asks for %d", slots[b], rec, p);
  }
  *out = p;
  return 0;
}

int check_slots(const loop_config& c, int B, const int32_t* slots) {
  if (!slots) return loop_fail(LOOP_EINVAL, "slots is NULL");
  std::set<int> seen;
  for (int b = 0; b < B; ++b) {
    if (slots[b] < 0 || slots[b] >= c.max_batch) return loop_fail(LOOP_ECAPACITY, "slot %d out of [0, %d)", slots[b], c.max_batch);
    if (!seen.insert(slots[b]).second) return loop_fail(LOOP_EINVAL, "slot %d used twice", slots[b]);
  }
  return 0;
}

}  // namespace

extern "C" int loop_prefill(loop_model* m, const loop_prefill_args* a, void* stream) {
  if (!m || !a) return loop_fail(LOOP_EINVAL, "model or args NULL");
  const loop_config& c = m->cfg;
  const int B = a->batch, T = a->seq_len;
  if (B < 1 || B > c.max_batch) return loop_fail(LOOP_ECAPACITY, "batch %d out of [1, %d]", B, c.max_batch);
  if (T < 1) return loop_fail(LOOP_EINVAL, "seq_len must be >= 1");
  if (T > 65536) return loop_fail(LOOP_ECAPACITY, "seq_len %d above 65536 tokens per call (chunked prefill: several calls)", T);
  if ((int64_t)B * T > c.max_tokens) return loop_fail(LOOP_ECAPACITY, "batch*seq_len %lld > max_tokens %d", (long long)B * T, c.max_tokens);
  if (int r = check_slots(c, B, a->slots)) return r;
  if (!a->start_pos) return loop_fail(LOOP_EINVAL, "start_pos is NULL");
  for (int b = 0; b < B; ++b)
    if (a->start_pos[b] < 0 || (int64_t)a->start_pos[b] + T > c.max_seq)
      return loop_fail(LOOP_ECAPACITY, "start_pos %d + seq_len %d exceeds max_seq %d", a->start_pos[b], T, c.max_seq);
  if ((a->d_tokens != nullptr) == (a->d_hidden_in != nullptr))
    return loop_fail(LOOP_EINVAL, "exactly one of d_tokens / d_hidden_in must be given");
  if (a->d_tokens && c.vocab == 0) return loop_fail(LOOP_EINVAL, "token input needs vocab > 0");
  if (a->d_logits && c.vocab == 0) return loop_fail(LOOP_EINVAL, "logits need vocab > 0");
  if (a->n_taps < 0 || (a->n_taps > 0 && (!a->tap_exec || !a->d_taps))) return loop_fail(LOOP_EINVAL, "bad taps");
  int passes = 0;
  if (int r = call_passes(m, a->loop_passes, B, a->slots, a->start_pos, &passes)) return r;
  const std::vector<ExecDesc>& sched = m->sched_p[passes - 1];
  for (int i = 0; i < a->n_taps; ++i)
    if (a->tap_exec[i] < 0 || a->tap_exec[i] >= (int)sched.size()) return loop_fail(LOOP_EINVAL, "tap %d out of range", a->tap_exec[i]);
  hipStream_t s = (hipStream_t)stream;
  Call k{B, T, B * T, false, nullptr, nullptr, nullptr, &sched};
  k.taps_all = a->taps_all_positions != 0;
  const int32_t* meta = at<int32_t>(m, m->L.meta);
  k.d_pos = meta;
  k.d_slot = meta + c.max_batch;
  k.d_last = meta + 2 * c.max_batch;
  if (int r = upload_meta(m, B, T, a->start_pos, a->slots, s)) return r;
  float* h = at<float>(m, m->L.h);
  if (a->d_tokens) HIP_TRY(launch_embed(a->d_tokens, m->embed, h, k.M, c.d_model, c.vocab, s));
  else HIP_TRY(hipMemcpyAsync(h, a->d_hidden_in, (size_t)k.M * c.d_model * 4, hipMemcpyDeviceToDevice, s));
  if (int r = run_forward(m, k, a->tap_exec, a->n_taps, a->d_taps, s)) return r;
  for (int b = 0; b < B; ++b)
    if (a->start_pos[b] == 0) m->slot_passes[a->slots[b]] = passes;
  if (a->d_hidden_out)
    HIP_TRY(hipMemcpyAsync(a->d_hidden_out, h, (size_t)k.M * c.d_model * 4, hipMemcpyDeviceToDevice, s));
  if (a->d_final_out) HIP_TRY(launch_rmsnorm_f32(h, m->final_norm, a->d_final_out, k.M, c.d_model, c.eps, s));
  if (a->d_logits)
    if (int r = head_logits(m, k, a->d_logits, s)) return r;
  return 0;
}

namespace {

// Host checks of a decode step; the call's pass count on success.
int check_decode(loop_model* m, const loop_decode_args* a, int* passes) {
  if (!m || !a) return loop_fail(LOOP_EINVAL, "model or args NULL");
  const loop_config& c = m->cfg;
  const int B = a->batch;
  if (B < 1 || B > c.max_batch || B > c.max_tokens) return loop_fail(LOOP_ECAPACITY, "batch %d out of range", B);
  if ((!m->q8.empty() || !m->q4.empty()) && B > 64)
    return loop_fail(LOOP_ECAPACITY, "int8 / int4 decode takes at most 64 sequences per call");
  if (c.vocab == 0) return loop_fail(LOOP_EINVAL, "decode needs vocab > 0");
  if (!a->d_tokens || !a->pos) return loop_fail(LOOP_EINVAL, "d_tokens and pos are required");
  if (int r = check_slots(c, B, a->slots)) return r;
  for (int b = 0; b < B; ++b)
    if (a->pos[b] < 0 || a->pos[b] >= c.max_seq) return loop_fail(LOOP_ECAPACITY, "pos %d out of [0, %d)", a->pos[b], c.max_seq);
  return call_passes(m, a->loop_passes, B, a->slots, nullptr, passes);
}

// The device work of one decode step, with positions / slots / last rows at
// meta (pos [max_batch], slot [max_batch], last [max_batch]).
int enqueue_decode(loop_model* m, const loop_decode_args* a, int passes, const int32_t* meta, hipStream_t s) {
  const loop_config& c = m->cfg;
  const int B = a->batch;
  Call k{B, 1, B, true, nullptr, nullptr, nullptr, &m->sched_p[passes - 1]};
  k.d_pos = meta;
  k.d_slot = meta + c.max_batch;
  k.d_last = meta + 2 * c.max_batch;
  float* h = at<float>(m, m->L.h);
  HIP_TRY(launch_embed(a->d_tokens, m->embed, h, B, c.d_model, c.vocab, s));
  if (int r = run_forward(m, k, nullptr, 0, nullptr, s)) return r;
  if (a->d_hidden_out) HIP_TRY(hipMemcpyAsync(a->d_hidden_out, h, (size_t)B * c.d_model * 4, hipMemcpyDeviceToDevice, s));
  if (a->d_logits || a->d_next) {
    float* logits = a->d_logits ? a->d_logits : at<float>(m, m->L.logits);
    if (int r = head_logits(m, k, logits, s)) return r;
    if (a->d_next)
      HIP_TRY(launch_argmax(logits, B, c.vocab, at<float>(m, m->L.am_v), at<int>(m, m->L.am_i), a->d_next, s));
  }
  return 0;
}

}  // namespace

extern "C" int loop_decode_step(loop_model* m, const loop_decode_args* a, void* stream) {
  int passes = 0;
  if (int r = check_decode(m, a, &passes)) return r;
  hipStream_t s = (hipStream_t)stream;
  if (int r = upload_meta(m, a->batch, 1, a->pos, a->slots, s)) return r;
  return enqueue_decode(m, a, passes, at<int32_t>(m, m->L.meta), s);
}

struct loop_decode_graph {
  loop_model* m = nullptr;
  int B = 0;
  int steps_left = 0;
  std::vector<int32_t> pos;       // positions of the next launch (host mirror)
  int32_t* meta = nullptr;        // device: pos, slot, last rows [3][max_batch]
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" void loop_decode_graph_destroy(loop_decode_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->meta) (void)hipFree(g->meta);
  delete g;
}

extern "C" int loop_decode_graph_create(loop_model* m, const loop_decode_args* a, int32_t max_steps,
                                        loop_decode_graph** out) {
  if (!out) return loop_fail(LOOP_EINVAL, "out is NULL");
  *out = nullptr;
  int passes = 0;
  if (int r = check_decode(m, a, &passes)) return r;
  const loop_config& c = m->cfg;
  if (max_steps < 1) return loop_fail(LOOP_EINVAL, "max_steps must be >= 1");
  for (int b = 0; b < a->batch; ++b)
    if ((int64_t)a->pos[b] + max_steps > c.max_seq)
      return loop_fail(LOOP_ECAPACITY, "pos %d + %d steps exceeds max_seq %d", a->pos[b], max_steps, c.max_seq);
  loop_decode_graph* g = new loop_decode_graph;
  g->m = m;
  g->B = a->batch;
  g->steps_left = max_steps;
  g->pos.assign(a->pos, a->pos + a->batch);
  std::vector<int32_t> meta(3 * c.max_batch, 0);
  for (int b = 0; b < a->batch; ++b) {
    meta[b] = a->pos[b];
    meta[c.max_batch + b] = a->slots[b];
    meta[2 * c.max_batch + b] = b;
  }
  hipError_t e = hipMalloc(&g->meta, meta.size() * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemcpy(g->meta, meta.data(), meta.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    loop_decode_graph_destroy(g);
    return loop_hip_fail(e, "decode graph positions");
  }
  // capture on a stream of our own (default priority); relaxed mode lets the
  // launchers' one-time kernel attribute calls happen during the capture
  hipStream_t cs = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) {
    loop_decode_graph_destroy(g);
    return loop_hip_fail(e, "capture stream");
  }
  const int prof = m->prof_class;  // no timing events inside the graph
  m->prof_class = -1;
  int r = 0;
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e == hipSuccess) {
    r = enqueue_decode(m, a, passes, g->meta, cs);
    if (r == 0) {
      hipError_t e2 = launch_advance_pos(g->meta, a->batch, cs);
      if (e2 != hipSuccess) r = loop_hip_fail(e2, "advance positions");
    }
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    g->graph = graph;
  }
  m->prof_class = prof;
  (void)hipStreamDestroy(cs);
  if (r == 0 && e != hipSuccess) r = loop_hip_fail(e, "decode graph capture");
  if (r == 0) {
    e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) r = loop_hip_fail(e, "hipGraphInstantiate");
  }
  if (r) {
    loop_decode_graph_destroy(g);
    return r;
  }
  *out = g;
  return 0;
}

extern "C" int loop_decode_graph_launch(loop_decode_graph* g, void* stream) {
  if (!g) return loop_fail(LOOP_EINVAL, "graph is NULL");
  if (g->steps_left <= 0) return loop_fail(LOOP_ECAPACITY, "decode graph: all of its steps were launched");
  hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
  if (e != hipSuccess) return loop_hip_fail(e, "hipGraphLaunch");
  --g->steps_left;
  for (int32_t& p : g->pos) ++p;
  return 0;
}

extern "C" int loop_decode_graph_positions(const loop_decode_graph* g, int32_t* pos_out) {
  if (!g || !pos_out) return loop_fail(LOOP_EINVAL, "NULL argument");
  for (int b = 0; b < g->B; ++b) pos_out[b] = g->pos[b];
  return 0;
}

extern "C" int loop_verify_step(loop_model* m, const loop_verify_args* a, void* stream) {
  if (!m || !a) return loop_fail(LOOP_EINVAL, "model or args NULL");
  const loop_config& c = m->cfg;
  const int B = a->batch, K = a->k;
  if (B < 1 || B > c.max_batch) return loop_fail(LOOP_ECAPACITY, "batch %d out of [1, %d]", B, c.max_batch);
  if (K < 1 || K > LOOP_VERIFY_MAX) return loop_fail(LOOP_EINVAL, "k %d out of [1, %d]", K, LOOP_VERIFY_MAX);
  if ((int64_t)B * K > c.max_tokens) return loop_fail(LOOP_ECAPACITY, "batch*k %d > max_tokens %d", B * K, c.max_tokens);
  if (c.vocab == 0) return loop_fail(LOOP_EINVAL, "verify needs vocab > 0");
  if (!a->d_tokens || !a->pos) return loop_fail(LOOP_EINVAL, "d_tokens and pos are required");
  if (int r = check_slots(c, B, a->slots)) return r;
  for (int b = 0; b < B; ++b)
    if (a->pos[b] < 0 || (int64_t)a->pos[b] + K > c.max_seq)
      return loop_fail(LOOP_ECAPACITY, "pos %d + k %d exceeds max_seq %d", a->pos[b], K, c.max_seq);
  if (a->n_taps < 0 || (a->n_taps > 0 && (!a->tap_exec || !a->d_taps))) return loop_fail(LOOP_EINVAL, "bad taps");
  int passes = 0;
  if (int r = call_passes(m, a->loop_passes, B, a->slots, a->pos, &passes)) return r;
  const std::vector<ExecDesc>& sched = m->sched_p[passes - 1];
  for (int i = 0; i < a->n_taps; ++i)
    if (a->tap_exec[i] < 0 || a->tap_exec[i] >= (int)sched.size()) return loop_fail(LOOP_EINVAL, "tap %d out of range", a->tap_exec[i]);
  hipStream_t s = (hipStream_t)stream;
  Call k{B, K, B * K, false, nullptr, nullptr, nullptr, &sched};
  k.taps_all = true;
  const int32_t* meta = at<int32_t>(m, m->L.meta);
  k.d_pos = meta;
  k.d_slot = meta + c.max_batch;
  k.d_last = meta + 2 * c.max_batch;
  if (int r = upload_meta(m, B, K, a->pos, a->slots, s)) return r;
  float* h = at<float>(m, m->L.h);
  HIP_TRY(launch_embed(a->d_tokens, m->embed, h, k.M, c.d_model, c.vocab, s));
  if (int r = run_forward(m, k, a->tap_exec, a->n_taps, a->d_taps, s)) return r;
  for (int b = 0; b < B; ++b)
    if (a->pos[b] == 0) m->slot_passes[a->slots[b]] = passes;
  if (a->d_hidden_out) HIP_TRY(hipMemcpyAsync(a->d_hidden_out, h, (size_t)k.M * c.d_model * 4, hipMemcpyDeviceToDevice, s));
  if (a->d_logits || a->d_next) {
    if (!a->d_logits) return loop_fail(LOOP_EINVAL, "d_next needs d_logits (logits of every position)");
    // final norm and head over every position
    uint16_t* xf = at<uint16_t>(m, m->L.xf);
    HIP_TRY(launch_rmsnorm(h, nullptr, nullptr, c.d_model, m->final_norm, xf, k.M, c.d_model, c.eps, s));
    HIP_TRY(launch_gemm(xf, c.d_model, m->head, c.d_model, a->d_logits, c.vocab, nullptr, k.M, c.vocab, c.d_model,
                        LOOP_EPI_F32, s, at<float>(m, m->L.splitk), m->L.splitk_bytes));
    if (a->d_next)
      HIP_TRY(launch_argmax(a->d_logits, k.M, c.vocab, at<float>(m, m->L.am_v), at<int>(m, m->L.am_i), a->d_next, s));
  }
  return 0;
}

extern "C" int loop_exec_mixer(loop_model* m, const loop_mixer_args* a, void* stream) {
  if (!m || !a) return loop_fail(LOOP_EINVAL, "model or args NULL");
  const loop_config& c = m->cfg;
  const int B = a->batch, T = a->seq_len;
  if (a->exec < 0 || a->exec >= (int)m->sched.size())
    return loop_fail(LOOP_EINVAL, "exec %d out of [0, %d)", a->exec, (int)m->sched.size());
  if (B < 1 || B > c.max_batch) return loop_fail(LOOP_ECAPACITY, "batch %d out of [1, %d]", B, c.max_batch);
  if (T < 1) return loop_fail(LOOP_EINVAL, "seq_len must be >= 1");
  if (a->decode && T != 1) return loop_fail(LOOP_EINVAL, "the decode path takes one token per sequence");
  if (T > 65536) return loop_fail(LOOP_ECAPACITY, "seq_len %d above 65536 tokens per call", T);
  if ((int64_t)B * T > c.max_tokens) return loop_fail(LOOP_ECAPACITY, "batch*seq_len %lld > max_tokens %d", (long long)B * T, c.max_tokens);
  if (int r = check_slots(c, B, a->slots)) return r;
  if (!a->start_pos) return loop_fail(LOOP_EINVAL, "start_pos is NULL");
  for (int b = 0; b < B; ++b)
    if (a->start_pos[b] < 0 || (int64_t)a->start_pos[b] + T > c.max_seq)
      return loop_fail(LOOP_ECAPACITY, "start_pos %d + seq_len %d exceeds max_seq %d", a->start_pos[b], T, c.max_seq);
  const ExecDesc& d = m->sched[a->exec];
  const int n_in = d.full ? n_in_full(c) : n_in_gdn(c);
  const int width = d.full ? c.n_q_heads * c.head_dim : c.gdn_heads * c.gdn_dv;
  if (!a->d_proj || !a->d_out) return loop_fail(LOOP_EINVAL, "d_proj and d_out are required");
  if (a->ld_proj < n_in || a->ld_out < width)
    return loop_fail(LOOP_EINVAL, "ld_proj %lld < %d or ld_out %lld < %d", (long long)a->ld_proj, n_in,
                     (long long)a->ld_out, width);
  hipStream_t s = (hipStream_t)stream;
  Call k{B, T, B * T, a->decode != 0, nullptr, nullptr, nullptr, &m->sched};
  const int32_t* meta = at<int32_t>(m, m->L.meta);
  k.d_pos = meta;
  k.d_slot = meta + c.max_batch;
  k.d_last = meta + 2 * c.max_batch;
  if (int r = upload_meta(m, B, T, a->start_pos, a->slots, s)) return r;
  uint16_t* proj = at<uint16_t>(m, m->L.proj);
  HIP_TRY(hipMemcpy2DAsync(proj, (size_t)m->L.n_in_max * 2, a->d_proj, (size_t)a->ld_proj * 2, (size_t)n_in * 2,
                           (size_t)k.M, hipMemcpyDeviceToDevice, s));
  int mix_width = 0;
  if (int r = run_mixer(m, k, d, s, &mix_width)) return r;
  HIP_TRY(hipMemcpy2DAsync(a->d_out, (size_t)a->ld_out * 2, at<uint16_t>(m, m->L.obuf), (size_t)mix_width * 2,
                           (size_t)mix_width * 2, (size_t)k.M, hipMemcpyDeviceToDevice, s));
  return 0;
}

extern "C" int loop_model_set_int8(loop_model* m, const loop_q8_layer* layers) {
  if (!m) return loop_fail(LOOP_EINVAL, "model NULL");
  const loop_config& c = m->cfg;
  if (!layers) {
    m->q8.clear();
    return 0;
  }
  const int mix_full = c.n_q_heads * c.head_dim, mix_gdn = c.gdn_heads * c.gdn_dv;
  if (c.d_model % 128 || mix_full % 128 || mix_gdn % 128 || c.d_ff % 128)
    return loop_fail(LOOP_ESHAPE, "int8 decode needs d_model, the mixer widths and d_ff multiples of 128");
  for (int l = 0; l < c.n_layers; ++l) {
    const loop_q8_layer& q = layers[l];
    if (!q.w_in || !q.s_in || !q.w_o || !q.s_o || !q.w_gateup || !q.s_gateup || !q.w_down || !q.s_down)
      return loop_fail(LOOP_EINVAL, "int8 layer %d misses codes or scales", l);
    if (((uintptr_t)q.w_in | (uintptr_t)q.w_o | (uintptr_t)q.w_gateup | (uintptr_t)q.w_down) % 16)
      return loop_fail(LOOP_EINVAL, "int8 codes of layer %d must be 16-byte aligned", l);
  }
  m->q8.assign(layers, layers + c.n_layers);
  m->q4.clear();
  return 0;
}

extern "C" int loop_model_set_int4(loop_model* m, const loop_q4_layer* layers) {
  if (!m) return loop_fail(LOOP_EINVAL, "model NULL");
  const loop_config& c = m->cfg;
  if (!layers) {
    m->q4.clear();
    return 0;
  }
  const int mix_full = c.n_q_heads * c.head_dim, mix_gdn = c.gdn_heads * c.gdn_dv;
  if (c.d_model % 128 || mix_full % 128 || mix_gdn % 128 || c.d_ff % 128)
    return loop_fail(LOOP_ESHAPE, "int4 decode needs d_model, the mixer widths and d_ff multiples of 128");
  for (int l = 0; l < c.n_layers; ++l) {
    const loop_q4_layer& q = layers[l];
    if (!q.w_in || !q.s_in || !q.w_o || !q.s_o || !q.w_gateup || !q.s_gateup || !q.w_down || !q.s_down)
      return loop_fail(LOOP_EINVAL, "int4 layer %d misses codes or scales", l);
    if (((uintptr_t)q.w_in | (uintptr_t)q.w_o | (uintptr_t)q.w_gateup | (uintptr_t)q.w_down) % 16)
      return loop_fail(LOOP_EINVAL, "int4 codes of layer %d must be 16-byte aligned", l);
    if (((uintptr_t)q.s_in | (uintptr_t)q.s_o | (uintptr_t)q.s_gateup | (uintptr_t)q.s_down) % 4)
      return loop_fail(LOOP_EINVAL, "int4 scales of layer %d must be 4-byte aligned", l);
  }
  m->q4.assign(layers, layers + c.n_layers);
  m->q8.clear();
  return 0;
}

extern "C" int loop_debug_mhc(loop_model* m, float* d_out, void* stream) {
  if (!m || !d_out) return loop_fail(LOOP_EINVAL, "model or output NULL");
  const loop_config& c = m->cfg;
  for (int l = c.loop_start; l < c.loop_end; ++l)
    HIP_TRY(launch_sinkhorn(m->lw[l].mhc_mix, c.sinkhorn_iters, d_out + 4 * (l - c.loop_start), (hipStream_t)stream));
  return 0;
}
