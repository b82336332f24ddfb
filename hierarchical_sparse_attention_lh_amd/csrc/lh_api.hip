// Host side of the C ABI declared in include/lh_api.h: validation, the closed-form plan and
// launch sequencing.  Nothing here allocates device memory or synchronises the host (unless
// the environment sets LH_DEBUG_SYNC=1, which synchronises and checks after every launch).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "lh_internal.h"

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

  Levels L;
  memset(&L, 0, sizeof(L));
  L.L = c->levels;
  L.p = c->pool;
  L.B = c->batch;
  L.N = c->n_tokens;
  L.H = c->heads;
  L.D = c->head_dim;
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
  info->saved_gmap = take(BH * Sp * 4);
  info->saved_inv = take(BH * L.P * 4);
  info->saved_q = take(BH * Sp * D * 2);
  info->saved_k = take(BH * Sp * D * 2);
  info->saved_v = take(BH * Sp * D * 2);
  info->saved_qt = take(BH * Sp * D * 2);
  info->saved_kt = take(BH * Sp * D * 2);
  info->saved_vt = take(BH * Sp * D * 2);
  info->saved_o = take(BH * Sp * D * 4);
  info->saved_lse = take(BH * Sp * 4);
  info->saved_bytes = o;
  const size_t pooled = align256(static_cast<size_t>(L.B * L.P1) * L.H * D * 2);
  info->ws_forward_bytes = 3 * pooled + align256(BH * L.P * 4) + align256(BH * L.K * 4 + 4);
  info->ws_backward_bytes = 2 * align256(BH * Sp * D * 2) + align256(BH * Sp * 4) +
                            3 * align256(BH * Sp * D * 4);
  info->softmax_scale = resolved_scale(c->softmax_scale, L.D);
}

// Offsets of the backward workspace pieces.
struct BwdWs {
  size_t dog, dogt, delta, dq, dk, dv;
};
BwdWs bwd_layout(const Levels& L) {
  const size_t BH = static_cast<size_t>(L.B * L.H), D = L.D;
  const size_t Sp = static_cast<size_t>(lh::padded_len(L.S));
  BwdWs w;
  size_t o = 0;
  w.dog = o; o += align256(BH * Sp * D * 2);
  w.dogt = o; o += align256(BH * Sp * D * 2);
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

lh_status check_desc(const lh_attn_desc* d) {
  if (d == nullptr) return LH_ERR_NULL;
  if (d->batch < 1 || d->heads < 1 || d->seq < 1 || d->seq > kMaxAttnLen) return LH_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return LH_ERR_DTYPE;
  if (d->batch * d->heads * (lh::padded_len(d->seq) / 128) > 0x7fffffffLL) return LH_ERR_SHAPE;
  return LH_OK;
}

}  // namespace

extern "C" {

const char* lh_status_string(lh_status s) {
  switch (s) {
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
                    const int32_t* gmap, const lh_gathered* out, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  if (out == nullptr) return LH_ERR_NULL;
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(gmap));
  if (L.L > 1) { LH_TRY(need(pq)); LH_TRY(need(pk)); LH_TRY(need(pv)); }
  LH_TRY(need(out->q)); LH_TRY(need(out->k)); LH_TRY(need(out->vt));
  LH_TRY(maybe(out->v)); LH_TRY(maybe(out->qt)); LH_TRY(maybe(out->kt));
  if (pooled_dtype != LH_BF16 && pooled_dtype != LH_F32) return LH_ERR_DTYPE;
  const void* x[3] = {q, k, v};
  const void* px[3] = {pq, pk, pv};
  void* const rows[3] = {out->q, out->k, out->v};
  void* const trans[3] = {out->qt, out->kt, out->vt};
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_gather(L, cfg->dtype == LH_F32, x, px, pooled_dtype == LH_F32, gmap,
                                    rows, trans, st), st);
}

lh_status lh_attn_fwd(const lh_attn_desc* desc, const void* q, const void* k, const void* vt,
                      float* o, float* lse, lh_stream_t stream) {
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(vt)); LH_TRY(need(o)); LH_TRY(need(lse));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_attn_fwd(desc->batch, desc->heads, desc->seq, desc->head_dim,
                                      resolved_scale(desc->scale, desc->head_dim), q, k, vt, o,
                                      lse, st), st);
}

lh_status lh_attn_bwd(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                      const void* qt, const void* kt, const float* lse, const float* delta,
                      const void* dout, const void* doutt, float* dq, float* dk, float* dv,
                      lh_stream_t stream) {
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(qt)); LH_TRY(need(kt));
  LH_TRY(need(lse)); LH_TRY(need(delta)); LH_TRY(need(dout)); LH_TRY(need(doutt));
  LH_TRY(need(dq)); LH_TRY(need(dk)); LH_TRY(need(dv));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_attn_bwd(desc->batch, desc->heads, desc->seq, desc->head_dim,
                                      resolved_scale(desc->scale, desc->head_dim), q, k, v, qt,
                                      kt, lse, delta, dout, doutt, dq, dk, dv, st), st);
}

lh_status lh_attn_bwd_dkdv(const lh_attn_desc* desc, const void* q, const void* k,
                           const void* v, const void* qt, const void* kt, const float* lse,
                           const float* delta, const void* dout, const void* doutt, float* dq,
                           float* dk, float* dv, lh_stream_t stream) {
  (void)kt;
  (void)dq;
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(qt)); LH_TRY(need(lse));
  LH_TRY(need(delta)); LH_TRY(need(dout)); LH_TRY(need(doutt)); LH_TRY(need(dk));
  LH_TRY(need(dv));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_attn_bwd_pass(1, desc->batch, desc->heads, desc->seq,
                                           desc->head_dim,
                                           resolved_scale(desc->scale, desc->head_dim), q, k, v,
                                           qt, nullptr, lse, delta, dout, doutt, nullptr, dk, dv,
                                           st), st);
}

lh_status lh_attn_bwd_dq(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                         const void* qt, const void* kt, const float* lse, const float* delta,
                         const void* dout, const void* doutt, float* dq, float* dk, float* dv,
                         lh_stream_t stream) {
  (void)qt;
  (void)doutt;
  (void)dk;
  (void)dv;
  LH_TRY(check_desc(desc));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(kt)); LH_TRY(need(lse));
  LH_TRY(need(delta)); LH_TRY(need(dout)); LH_TRY(need(dq));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_attn_bwd_pass(2, desc->batch, desc->heads, desc->seq,
                                           desc->head_dim,
                                           resolved_scale(desc->scale, desc->head_dim), q, k, v,
                                           nullptr, kt, lse, delta, dout, nullptr, dq, nullptr,
                                           nullptr, st), st);
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
                         const void* dy, void* dog, void* dogt, float* delta,
                         lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(gmap)); LH_TRY(need(og)); LH_TRY(need(dy)); LH_TRY(need(dog));
  LH_TRY(need(dogt)); LH_TRY(need(delta));
  auto st = static_cast<hipStream_t>(stream);
  return launched(lh::launch_scatter_bwd(L, cfg->dtype == LH_F32, gmap, og, dy, dog, dogt, delta,
                                         st), st);
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

lh_status lh_forward(const lh_config* cfg, const void* q, const void* k, const void* v,
                     void* y, void* saved, void* ws, size_t ws_bytes, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
  LH_TRY(need(q)); LH_TRY(need(k)); LH_TRY(need(v)); LH_TRY(need(y)); LH_TRY(need(saved));
  lh_plan_info P;
  fill_plan(cfg, L, &P);
  if (P.ws_forward_bytes > 0) LH_TRY(need(ws));
  if (ws_bytes < P.ws_forward_bytes) return LH_ERR_WORKSPACE;
  auto st = static_cast<hipStream_t>(stream);
  const int32_t f32 = cfg->dtype == LH_F32;

  const size_t pooled = align256(static_cast<size_t>(L.B * L.P1) * L.H * L.D * 2);
  void* pq = at(ws, 0);
  void* pk = at(ws, pooled);
  void* pv = at(ws, 2 * pooled);
  float* scores = reinterpret_cast<float*>(at(ws, 3 * pooled));
  int32_t* sel = reinterpret_cast<int32_t*>(at(ws, 3 * pooled + align256(L.B * L.H * L.P * 4)));
  int32_t* gmap = reinterpret_cast<int32_t*>(at(saved, P.saved_gmap));
  int32_t* inv = reinterpret_cast<int32_t*>(at(saved, P.saved_inv));
  float* og = reinterpret_cast<float*>(at(saved, P.saved_o));
  float* lse = reinterpret_cast<float*>(at(saved, P.saved_lse));

  LH_TRY(launched(lh::launch_pool_score(L, f32, q, k, v, pq, pk, pv, 0, scores, st), st));
  LH_TRY(launched(lh::launch_topk(L, scores, sel, st), st));
  LH_TRY(launched(lh::launch_build_map(L, sel, gmap, inv, st), st));
  const void* x[3] = {q, k, v};
  const void* px[3] = {pq, pk, pv};
  void* const rows[3] = {at(saved, P.saved_q), at(saved, P.saved_k), at(saved, P.saved_v)};
  void* const trans[3] = {at(saved, P.saved_qt), at(saved, P.saved_kt), at(saved, P.saved_vt)};
  LH_TRY(launched(lh::launch_gather(L, f32, x, px, 0, gmap, rows, trans, st), st));
  LH_TRY(launched(lh::launch_attn_fwd(L.B, L.H, L.S, L.D, P.softmax_scale, rows[0], rows[1],
                                      trans[2], og, lse, st), st));
  return launched(lh::launch_scatter(L, f32, inv, og, y, st), st);
}

lh_status lh_backward(const lh_config* cfg, const void* saved, const void* dy, void* dq,
                      void* dk, void* dv, void* ws, size_t ws_bytes, lh_stream_t stream) {
  Levels L;
  LH_TRY(check_config(cfg, &L));
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
  void* dogt = at(ws, w.dogt);
  float* delta = reinterpret_cast<float*>(at(ws, w.delta));
  float* dqg = reinterpret_cast<float*>(at(ws, w.dq));
  float* dkg = reinterpret_cast<float*>(at(ws, w.dk));
  float* dvg = reinterpret_cast<float*>(at(ws, w.dv));

  LH_TRY(launched(lh::launch_scatter_bwd(L, f32, gmap, og, dy, dog, dogt, delta, st), st));
  LH_TRY(launched(lh::launch_attn_bwd(L.B, L.H, L.S, L.D, P.softmax_scale, at(saved, P.saved_q),
                                      at(saved, P.saved_k), at(saved, P.saved_v),
                                      at(saved, P.saved_qt), at(saved, P.saved_kt), lse, delta, dog,
                                      dogt, dqg, dkg, dvg, st), st));
  return launched(lh::launch_gather_pool_bwd(L, f32, inv, dqg, dkg, dvg, dq, dk, dv, st), st);
}

}  // extern "C"
