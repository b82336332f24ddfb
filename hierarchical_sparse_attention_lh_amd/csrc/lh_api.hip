// Host side of the C ABI declared in include/lh_api.h: validation, the closed-form plan and
// launch sequencing.  Nothing here allocates device memory or synchronises the host (unless
// the environment sets LH_DEBUG_SYNC=1, which synchronises and checks after every launch).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "lh_internal.h"

// Forward workspace of lh_forward_noalloc: one array per GPU, held until the process ends.
// Host code must never pass this name to a kernel (on the host it is only a stand-in); it
// uses the device address hipGetSymbolAddress reports for the current device instead.
static __device__ __align__(256) unsigned char scratch[LH_NOALLOC_SCRATCH_BYTES];

namespace {

using lh::Levels;

constexpr int64_t kMaxTokens = int64_t(1) << 30;
// attention length bound: the staging loads address a tile with a 32-bit byte offset
constexpr int64_t kMaxAttnLen = int64_t(1) << 24;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = getenv("LH_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

lh_status launched(hipError_t err, hipStream_t st) {
  if (err != hipSuccess) return LH_ERR_LAUNCH;
  if (debug_sync()) {
    if (hipStreamSynchronize(st) != hipSuccess) return LH_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return LH_ERR_LAUNCH;
  }
  return LH_OK;
}

#define LH_TRY(expr)                  \
  do {                                \
    const lh_status s_ = (expr);      \
    if (s_ != LH_OK) return s_;       \
  } while (0)

// Checks every field of a config and fills the level table.  Pure host arithmetic.
lh_status check_config(const lh_config* c, Levels* lv) {
  if (c == nullptr) return LH_ERR_NULL;
  if (c->batch < 1 || c->n_tokens < 1 || c->heads < 1 || c->n_tokens > kMaxTokens ||
      c->batch * c->heads > 65535)
    return LH_ERR_SHAPE;
  if ((c->head_dim != 64 && c->head_dim != 128) || (c->dtype != LH_BF16 && c->dtype != LH_F32))
    return LH_ERR_DTYPE;
  if (c->levels < 1 || c->levels > LH_MAX_LEVELS) return LH_ERR_LEVELS;
  if (c->pool < 2 || c->pool > 16) return LH_ERR_POOL;
  if (c->select_mode != LH_SEL_REFINE && c->select_mode != LH_SEL_DIRECT)
    return LH_ERR_UNSUPPORTED;
  if (c->chunk < 16 || c->chunk > 2048 || (c->chunk & (c->chunk - 1)) != 0) return LH_ERR_CHUNK;
  if (c->scorer != LH_SCORE_K && c->scorer != LH_SCORE_QK && c->scorer != LH_SCORE_QKV)
    return LH_ERR_UNSUPPORTED;

  Levels L;
  memset(&L, 0, sizeof(L));
  L.L = c->levels;
  L.p = c->pool;
  L.B = c->batch;
  L.N = c->n_tokens;
  L.H = c->heads;
  L.D = c->head_dim;
  L.scorer = c->scorer;
  int64_t pw = 1;
  for (int l = 0; l < L.L; ++l) {
    L.pw[l] = pw;
    if (l + 1 < L.L) pw *= L.p;
    if (pw > kMaxTokens) return LH_ERR_SHAPE;
  }
  if (L.N % L.pw[L.L - 1] != 0) return LH_ERR_SHAPE;
  const bool pow2 = (L.p & (L.p - 1)) == 0;
  int lgp = 0;
  while ((1 << lgp) < L.p) ++lgp;
  for (int l = 0; l < LH_MAX_LEVELS; ++l) L.lg[l] = pow2 ? l * lgp : -1;
  int64_t off = 0, poff = 0;
  for (int l = 0; l < L.L; ++l) {
    L.n[l] = L.N / L.pw[l];
    L.off[l] = off;
    off += L.n[l];
    if (l >= 1) {
      L.poff[l] = poff;
      poff += L.n[l];
    }
  }
  L.P = off;
  L.P1 = poff;
  // REFINE selects at levels 1..L-1 and a kept entry enters as its p children; DIRECT selects
  // at levels 0..L-2 and a kept entry enters itself.  The coarsest level always enters whole.
  L.direct = c->select_mode == LH_SEL_DIRECT;
  L.sel_first = L.direct ? 0 : 1;
  L.sel_last = L.direct ? L.L - 2 : L.L - 1;
  int64_t soff = 0, S = L.n[L.L - 1];
  for (int l = L.sel_first; l <= L.sel_last; ++l) {
    if (c->k[l] < 0) return LH_ERR_K;
    const int64_t n = L.n[l];
    if (n > c->chunk && n % c->chunk != 0) return LH_ERR_CHUNK;
    L.keff[l] = c->k[l] < n ? c->k[l] : n;
    L.nchunk[l] = n > c->chunk ? n / c->chunk : 1;
    L.width[l] = n > c->chunk ? c->chunk : n;
    L.soff[l] = soff;
    soff += L.keff[l];
    S += (L.direct ? 1 : L.p) * L.keff[l];
  }
  L.K = soff;
  L.S = S;
  if (L.B * L.H * L.P > (int64_t(1) << 40) || L.P >= (int64_t(1) << 31)) return LH_ERR_SHAPE;
  if (L.S > kMaxAttnLen) return LH_ERR_SHAPE;
  if (lv) *lv = L;
  return LH_OK;
}

float resolved_scale(float s, int d) {
  return (s > 0.f && isfinite(s)) ? s : 1.0f / sqrtf(static_cast<float>(d));
}

void fill_plan(const lh_config* c, const Levels& L, lh_plan_info* info) {
  memset(info, 0, sizeof(*info));
  for (int l = 0; l < L.L; ++l) {
    info->level_size[l] = L.n[l];
    info->level_offset[l] = L.off[l];
    info->pooled_offset[l] = l >= 1 ? L.poff[l] : 0;
    info->k_eff[l] = L.keff[l];
    info->n_chunks[l] = L.nchunk[l];
    info->chunk_width[l] = L.width[l];
    if (L.nchunk[l] > 0) {
      info->quota_base[l] = L.keff[l] / L.nchunk[l];
      info->quota_rem[l] = L.keff[l] % L.nchunk[l];
    }
    info->sel_offset[l] = L.soff[l];
  }
  info->pyramid_total = L.P;
  info->pooled_rows = L.P1;
  info->sel_total = L.K;
  info->gathered_len = L.S;
  const int64_t Sp = lh::padded_len(L.S);
  info->gathered_pad = Sp;
  const size_t BH = static_cast<size_t>(L.B * L.H);
  const size_t D = static_cast<size_t>(L.D);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t pooled = static_cast<size_t>(L.B * L.P1) * L.H * D * 2;
  info->saved_gmap = take(BH * Sp * 4);
  info->saved_inv = take(BH * L.P * 4);
  info->saved_pq = take(pooled);
  info->saved_pk = take(pooled);
  info->saved_pv = take(pooled);
  info->saved_o = take(BH * Sp * D * 4);
  info->saved_lse = take(BH * Sp * 4);
  info->saved_bytes = o;
  if (c->dtype == LH_F32) {
    // float32 layers keep the bf16 rounding of their token rows (the attention's level-0 rows)
    info->saved_bytes += 3 * align256(static_cast<size_t>(L.B * L.N) * L.H * D * 2);
  }
  info->ws_forward_bytes = align256(BH * L.P * 4) + align256(BH * L.K * 4 + 4);
  info->ws_backward_bytes = align256(BH * Sp * D * 2) + align256(BH * Sp * 4) +
                            3 * align256(BH * Sp * D * 4);
  info->softmax_scale = resolved_scale(c->softmax_scale, L.D);
}

// Offset of the bf16 token copies (which = 0, 1, 2 for Q, K, V) a float32 layer keeps at the
// end of `saved`.
size_t raw_copy_offset(const lh_plan_info& P, const Levels& L, int which) {
  const size_t one = align256(static_cast<size_t>(L.B * L.N) * L.H * L.D * 2);
  return align256(P.saved_lse + static_cast<size_t>(L.B * L.H) * P.gathered_pad * 4) +
         which * one;
}

// Offsets of the backward workspace pieces.
struct BwdWs {
  size_t dog, delta, dq, dk, dv;
};
BwdWs bwd_layout(const Levels& L) {
  const size_t BH = static_cast<size_t>(L.B * L.H), D = L.D;
  const size_t Sp = static_cast<size_t>(lh::padded_len(L.S));
  BwdWs w;
  size_t o = 0;
  w.dog = o; o += align256(BH * Sp * D * 2);
  w.delta = o; o += align256(BH * Sp * 4);
  w.dq = o; o += align256(BH * Sp * D * 4);
  w.dk = o; o += align256(BH * Sp * D * 4);
  w.dv = o;
  return w;
}

lh_status need(const void* p) {
  if (p == nullptr) return LH_ERR_NULL;
  return aligned16(p) ? LH_OK : LH_ERR_ALIGN;
}

lh_status maybe(const void* p) { return (p == nullptr || aligned16(p)) ? LH_OK : LH_ERR_ALIGN; }

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
inline const char* at(const void* base, size_t off) {
  return static_cast<const char*>(base) + off;
}

// Device address of `scratch` on the current device, looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lh_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LH_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return LH_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LH_OK;
}

bool stride_ok(const int64_t st[3]) {
  return st[0] >= 0 && st[1] >= 0 && st[2] >= 0 && st[0] % 8 == 0 && st[1] % 8 == 0 &&
         st[2] % 8 == 0;
}

lh_status check_desc(const lh_attn_desc* d) {
  if (d == nullptr) return LH_ERR_NULL;
  if (d->batch < 1 || d->heads < 1 || d->seq < 1 || d->seq > kMaxAttnLen) return LH_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return LH_ERR_DTYPE;
  if (d->batch * d->heads * (lh::padded_len(d->seq) / 128) > 0x7fffffffLL) return LH_ERR_SHAPE;
  if (!stride_ok(d->q_stride) || !stride_ok(d->k_stride) || !stride_ok(d->v_stride) ||
      !stride_ok(d->o_stride))
    return LH_ERR_ALIGN;
  return LH_OK;
}

// An attention call over strided rows.
lh::AttnCall strided_call(const lh_attn_desc* d) {
  lh::AttnCall c;
  memset(&c, 0, sizeof(c));
  c.B = d->batch;
  c.H = d->heads;
  c.S = d->seq;
  c.D = static_cast<int32_t>(d->head_dim);
  c.scale = resolved_scale(d->scale, c.D);
  c.causal = d->causal != 0;
  c.o_rows = static_cast<int32_t>(d->seq);
  for (int i = 0; i < 3; ++i) {
    c.q_stride[i] = d->q_stride[i];
    c.k_stride[i] = d->k_stride[i];
    c.v_stride[i] = d->v_stride[i];
    c.o_stride[i] = d->o_stride[i];
    c.do_stride[i] = d->o_stride[i];
    c.g_stride[i] = d->o_stride[i];
  }
  return c;
}

// The layer's attention: causal, rows through gmap (L >= 2) or the token tensors themselves
// (L = 1, the identity map), outputs in the padded gathered layout [B, H, Sp, D].
lh::AttnCall layer_call(const Levels& L, float scale, const int32_t* gmap, const void* pq,
                        const void* pk, const void* pv) {
  lh::AttnCall c;
  memset(&c, 0, sizeof(c));
  c.B = L.B;
  c.H = L.H;
  c.S = L.S;
  c.D = L.D;
  c.scale = scale;
  c.causal = 1;
  const int64_t Sp = lh::padded_len(L.S);
  c.o_rows = static_cast<int32_t>(Sp);
  const int64_t tok[3] = {L.N * L.H * L.D, L.D, static_cast<int64_t>(L.H) * L.D};
  const int64_t gat[3] = {L.H * Sp * L.D, Sp * L.D, L.D};
  for (int i = 0; i < 3; ++i) {
    c.q_stride[i] = c.k_stride[i] = c.v_stride[i] = tok[i];
    c.o_stride[i] = c.do_stride[i] = c.g_stride[i] = gat[i];
  }
  c.mapped = L.L > 1;
  c.lv = &L;
  c.gmap = gmap;
  c.pq = pq;
  c.pk = pk;
  c.pv = pv;
  return c;
}

}  // namespace

extern "C" {

const char* lh_status_string(lh_status s) {
  // a C caller may pass any int: read it as one (an enum-typed load of a value outside the
  // enumerators is undefined in C++)
  int code;
  memcpy(&code, &s, sizeof(code));
  switch (code) {
    case LH_OK: return "ok";
    case LH_ERR_NULL: return "a required pointer is NULL";
    case LH_ERR_SHAPE: return "shape out of range or p^(L-1) does not divide N";
    case LH_ERR_LEVELS: return "levels outside [1, 8]";
    case LH_ERR_POOL: return "pool factor outside [2, 16]";
    case LH_ERR_K: return "negative per-level budget k";
    case LH_ERR_CHUNK: return "chunk not a power of two in [16, 2048] or does not divide a level";
    case LH_ERR_DTYPE: return "unsupported dtype or head_dim";
    case LH_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case LH_ERR_WORKSPACE: return "workspace too small";
    case LH_ERR_LAUNCH: return "kernel launch failed";
    case LH_ERR_UNSUPPORTED: return "option not implemented";
    case LH_ERR_SCRATCH: return "forward workspace exceeds the static scratch of lh_forward_noalloc";
  }
  return "unknown status";
}

lh_status lh_plan(const lh_config* cfg, lh_plan_info* info) {
  if (info == nullptr) return LH_ERR_NULL;
  Levels L;
  LH_TRY(check_config(cfg, &L));
  fill_plan(cfg, L, info);
  return LH_OK;
}

lh_status lh_pool_score(const lh_config* cfg, const void* q, const void* k, const void* v,
                        void* pq, void* pk, void* pv, int32_t pooled_dtype, float* scores,
                        lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(scores));
  LH_TRY(maybe(pq)); LH_TRY(maybe(pk)); LH_TRY(maybe(pv));
  if (pooled_dtype != LH_BF16 && pooled_dtype != LH_F32) return LH_ERR_DTYPE;
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_pool_score(L, cfg->dtype == LH_F32, q, k, v, pq, pk, pv,
                                        pooled_dtype == LH_F32, scores, st), st);
}

lh_status lh_topk(const lh_config* cfg, const float* scores, int32_t* sel, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(scores));
  if (L.K > 0) LH_TRY(need(sel));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_topk(L, scores, sel, st), st);
}

lh_status lh_pool_score_topk(const lh_config* cfg, const void* q, const void* k, const void* v,
                             void* pq, void* pk, void* pv, int32_t pooled_dtype, float* scores,
                             int32_t* sel, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(scores));
  LH_TRY(maybe(pq)); LH_TRY(maybe(pk)); LH_TRY(maybe(pv));
  if (L.K > 0) LH_TRY(need(sel));
  if (pooled_dtype != LH_BF16 && pooled_dtype != LH_F32) return LH_ERR_DTYPE;
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_pool_score_topk(L, cfg->dtype == LH_F32, q, k, v, pq, pk, pv,
                                             pooled_dtype == LH_F32, scores, sel, st), st);
}

lh_status lh_build_map(const lh_config* cfg, const int32_t* sel, int32_t* gmap, int32_t* inv,
                       lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  if (L.K > 0) LH_TRY(need(sel));
  LH_TRY(need(gmap)); LH_TRY(need(inv));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_build_map(L, sel, gmap, inv, st), st);
}

lh_status lh_gather(const lh_config* cfg, const void* q, const void* k, const void* v,
                    const void* pq, const void* pk, const void* pv, int32_t pooled_dtype,
                    const int32_t* sel, int32_t* gmap, int32_t* inv, void* qg, void* kg,
                    void* vg, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v));
  if (L.K > 0) LH_TRY(need(sel));
  LH_TRY(need(gmap)); LH_TRY(need(inv));
  if (L.L > 1) { LH_TRY(need(pq)); LH_TRY(need(pk)); LH_TRY(need(pv)); }
  LH_TRY(need(qg)); LH_TRY(need(kg)); LH_TRY(need(vg));
  if (pooled_dtype != LH_BF16 && pooled_dtype != LH_F32) return LH_ERR_DTYPE;
  auto st = static_cast<hipStream_t>(stream);
  LH_TRY(launched(lh::launch_build_map(L, sel, gmap, inv, st), st));
  const void* x[3] = {q, k, v};
  const void* px[3] = {pq, pk, pv};
  void* const rows[3] = {qg, kg, vg};
  return launched(lh::launch_gather(L, cfg->dtype == LH_F32, x, px, pooled_dtype == LH_F32, gmap,
                                    rows, st), st);
}

lh_status lh_attn_fwd(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                      float* o, float* lse, lh_stream_t stream) {
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(o)); LH_TRY(need(lse));
  auto st = static_cast<hipStream_t>(stream);
  const lh::AttnCall c = strided_call(desc);
  return launched(lh::launch_attn_fwd2(c, q, k, v, o, lse, st), st);
}

lh_status lh_attn_ws_bytes(const lh_attn_desc* desc, size_t* bytes) {
  LH_TRY(check_desc(desc));
  if (bytes == nullptr) return LH_ERR_NULL;
  *bytes = align256(static_cast<size_t>(desc->batch * desc->heads) *
                    static_cast<size_t>(lh::padded_len(desc->seq)) * 4);
  return LH_OK;
}

lh_status lh_attn_bwd(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                      const float* o, const float* lse, const void* dout, float* dq, float* dk,
                      float* dv, void* ws, size_t ws_bytes, lh_stream_t stream) {
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(o)); LH_TRY(need(lse));
  LH_TRY(need(dout)); LH_TRY(need(dq)); LH_TRY(need(dk)); LH_TRY(need(dv)); LH_TRY(need(ws));
  size_t want = 0;
  LH_TRY(lh_attn_ws_bytes(desc, &want));
  if (ws_bytes < want) return LH_ERR_WORKSPACE;
  auto st = static_cast<hipStream_t>(stream);
  const lh::AttnCall c = strided_call(desc);
  float* delta = static_cast<float*>(ws);
  LH_TRY(launched(lh::launch_attn_delta(c, dout, o, delta, st), st));
  return launched(lh::launch_attn_bwd2(3, c, q, k, v, dout, lse, delta, dq, dk, dv, st), st);
}

lh_status lh_attn_fwd_mapped(const lh_config* cfg, const void* q, const void* k, const void* v,
                             const void* pq, const void* pk, const void* pv,
                             const int32_t* gmap, float* og, float* lse, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(gmap)); LH_TRY(need(og));
  LH_TRY(need(lse));
  if (L.L > 1) { LH_TRY(need(pq)); LH_TRY(need(pk)); LH_TRY(need(pv)); }
  auto st = static_cast<hipStream_t>(stream);
  const lh::AttnCall c =
      layer_call(L, resolved_scale(cfg->softmax_scale, L.D), gmap, pq, pk, pv);
  return launched(lh::launch_attn_fwd2(c, q, k, v, og, lse, st), st);
}

lh_status lh_attn_bwd_mapped(const lh_config* cfg, const void* q, const void* k, const void* v,
                             const void* pq, const void* pk, const void* pv,
                             const int32_t* gmap, const float* lse, const float* delta,
                             const void* dog, float* dqg, float* dkg, float* dvg, int32_t passes,
                             lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  if (passes < 1 || passes > 3) return LH_ERR_UNSUPPORTED;
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(gmap)); LH_TRY(need(lse));
  LH_TRY(need(delta)); LH_TRY(need(dog));
  if (L.L > 1) { LH_TRY(need(pq)); LH_TRY(need(pk)); LH_TRY(need(pv)); }
  if (passes & 1) { LH_TRY(need(dkg)); LH_TRY(need(dvg)); }
  if (passes & 2) LH_TRY(need(dqg));
  auto st = static_cast<hipStream_t>(stream);
  const lh::AttnCall c =
      layer_call(L, resolved_scale(cfg->softmax_scale, L.D), gmap, pq, pk, pv);
  return launched(lh::launch_attn_bwd2(passes, c, q, k, v, dog, lse, delta, dqg, dkg, dvg, st),
                  st);
}

lh_status lh_scatter(const lh_config* cfg, const int32_t* inv, const float* og, void* y,
                     lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(inv)); LH_TRY(need(og)); LH_TRY(need(y));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_scatter(L, cfg->dtype == LH_F32, inv, og, y, st), st);
}

lh_status lh_scatter_bwd(const lh_config* cfg, const int32_t* gmap, const float* og,
                         const void* dy, void* dog, float* delta, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(gmap)); LH_TRY(need(og)); LH_TRY(need(dy)); LH_TRY(need(dog)); LH_TRY(need(delta));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_scatter_bwd(L, cfg->dtype == LH_F32, gmap, og, dy, dog, delta, st),
                  st);
}

lh_status lh_gather_pool_bwd(const lh_config* cfg, const int32_t* inv, const float* dqg,
                             const float* dkg, const float* dvg, void* dq, void* dk, void* dv,
                             lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(inv)); LH_TRY(need(dqg)); LH_TRY(need(dkg)); LH_TRY(need(dvg));
  LH_TRY(need(dq)); LH_TRY(need(dk)); LH_TRY(need(dv));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_gather_pool_bwd(L, cfg->dtype == LH_F32, inv, dqg, dkg, dvg, dq, dk,
                                             dv, st), st);
}

}  // extern "C"

namespace {

// Stages 1-5 on a validated config; `ws` holds at least P.ws_forward_bytes.
lh_status forward_body(const lh_config* cfg, const Levels& L, const lh_plan_info& P,
                       const void* q, const void* k, const void* v, void* y, void* saved,
                       void* ws, lh_stream_t stream) {
  auto st = static_cast<hipStream_t>(stream);
  const int32_t f32 = cfg->dtype == LH_F32;
  void* pq = at(saved, P.saved_pq);
  void* pk = at(saved, P.saved_pk);
  void* pv = at(saved, P.saved_pv);
  float* scores = reinterpret_cast<float*>(ws);
  int32_t* sel = reinterpret_cast<int32_t*>(at(ws, align256(L.B * L.H * L.P * 4)));
  int32_t* gmap = reinterpret_cast<int32_t*>(at(saved, P.saved_gmap));
  int32_t* inv = reinterpret_cast<int32_t*>(at(saved, P.saved_inv));
  float* og = reinterpret_cast<float*>(at(saved, P.saved_o));
  float* lse = reinterpret_cast<float*>(at(saved, P.saved_lse));

  // separate pooling and top-K launches: on MI355X they beat the fused pass of
  // lh_pool_score_topk (the pooling is HBM-bound either way; inside the fused workgroups the
  // top-K phase leaves the memory pipe idle)
  LH_TRY(launched(lh::launch_pool_score(L, f32, q, k, v, pq, pk, pv, 0, scores, st), st));
  LH_TRY(launched(lh::launch_topk(L, scores, sel, st), st));
  LH_TRY(launched(lh::launch_build_map(L, sel, gmap, inv, st), st));
  const void* rows[3] = {q, k, v};
  if (f32) {  // the attention reads bf16 token rows: round the float32 inputs once
    for (int i = 0; i < 3; ++i) {
      void* copy = at(saved, raw_copy_offset(P, L, i));
      LH_TRY(launched(lh::launch_to_bf16(static_cast<const float*>(rows[i]), copy,
                                         L.B * L.N * L.H * L.D, st), st));
      rows[i] = copy;
    }
  }
  const lh::AttnCall c = layer_call(L, P.softmax_scale, gmap, pq, pk, pv);
  LH_TRY(launched(lh::launch_attn_fwd2(c, rows[0], rows[1], rows[2], og, lse, st), st));
  return launched(lh::launch_scatter(L, f32, inv, og, y, st), st);
}

}  // namespace

extern "C" {

lh_status lh_forward(const lh_config* cfg, const void* q, const void* k, const void* v,
                     void* y, void* saved, void* ws, size_t ws_bytes, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(y)); LH_TRY(need(saved));
  lh_plan_info P;
  fill_plan(cfg, L, &P);
  if (P.ws_forward_bytes > 0) LH_TRY(need(ws));
  if (ws_bytes < P.ws_forward_bytes) return LH_ERR_WORKSPACE;
  return forward_body(cfg, L, P, q, k, v, y, saved, ws, stream);
}

lh_status lh_forward_noalloc(const lh_config* cfg, const void* q, const void* k, const void* v,
                             void* y, void* saved, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(y)); LH_TRY(need(saved));
  lh_plan_info P;
  fill_plan(cfg, L, &P);
  if (P.ws_forward_bytes > LH_NOALLOC_SCRATCH_BYTES) return LH_ERR_SCRATCH;
  void* ws = nullptr;
  LH_TRY(scratch_address(&ws));
  return forward_body(cfg, L, P, q, k, v, y, saved, ws, stream);
}

lh_status lh_backward(const lh_config* cfg, const void* q, const void* k, const void* v,
                      const void* saved, const void* dy, void* dq, void* dk, void* dv, void* ws,
                      size_t ws_bytes, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v));
  LH_TRY(need(saved)); LH_TRY(need(dy)); LH_TRY(need(dq)); LH_TRY(need(dk)); LH_TRY(need(dv));
  LH_TRY(need(ws));
  lh_plan_info P;
  fill_plan(cfg, L, &P);
  if (ws_bytes < P.ws_backward_bytes) return LH_ERR_WORKSPACE;
  auto st = static_cast<hipStream_t>(stream);
  const int32_t f32 = cfg->dtype == LH_F32;
  const BwdWs w = bwd_layout(L);
  const int32_t* gmap = reinterpret_cast<const int32_t*>(at(saved, P.saved_gmap));
  const int32_t* inv = reinterpret_cast<const int32_t*>(at(saved, P.saved_inv));
  const float* og = reinterpret_cast<const float*>(at(saved, P.saved_o));
  const float* lse = reinterpret_cast<const float*>(at(saved, P.saved_lse));
  void* dog = at(ws, w.dog);
  float* delta = reinterpret_cast<float*>(at(ws, w.delta));
  float* dqg = reinterpret_cast<float*>(at(ws, w.dq));
  float* dkg = reinterpret_cast<float*>(at(ws, w.dk));
  float* dvg = reinterpret_cast<float*>(at(ws, w.dv));
  const void* rows[3] = {q, k, v};
  if (f32)  // the bf16 token rows lh_forward kept
    for (int i = 0; i < 3; ++i) rows[i] = at(saved, raw_copy_offset(P, L, i));

  LH_TRY(launched(lh::launch_scatter_bwd(L, f32, gmap, og, dy, dog, delta, st), st));
  const lh::AttnCall c = layer_call(L, P.softmax_scale, gmap, at(saved, P.saved_pq),
                                    at(saved, P.saved_pk), at(saved, P.saved_pv));
  LH_TRY(launched(lh::launch_attn_bwd2(3, c, rows[0], rows[1], rows[2], dog, lse, delta, dqg,
                                       dkg, dvg, st), st));
  return launched(lh::launch_gather_pool_bwd(L, f32, inv, dqg, dkg, dvg, dq, dk, dv, st), st);
}

}  // extern "C"
