// Stage 1+2: symmetric pyramid pool of Q, K, V and the per-head l2 score of pooled keys.
//
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "核心方法：金字塔池化与“外部选择”", item 1: Q, K and V are average-pooled together
// into a multi-level pyramid.  [EN] encorp.ai, "Услуги по внедряване на AI задават правилния
// въпрос за Lighthouse Attention", section "Как four-stage pipeline остава бърз, без да чупи
// градиентите?": entries are scored with per-head l2 norms (reading: of the pooled key row;
// [CB] "The Bottom Line" names the same projection-norm scorer, and two further readings are
// options: ||q_bar|| * ||k_bar|| and the norm of the concatenated [q_bar; k_bar; v_bar]).
//
// Design (HBM-bound scan): one thread owns 8 consecutive columns of a token row (one 16-byte
// bf16 load per token) and walks one coarsest block of p^(L-1) tokens, keeping a float32
// running mean per level in registers.  Every time a level-l block closes, the thread writes
// its 8 pooled columns; for the key stream the 8 squares are summed in float64 and reduced
// over the D/8 lanes of the head with cross-lane shuffles, and one lane writes the score.
// A wave reads 64 x 16 B = 1 KB of one token row per step: fully coalesced.  Q, K and V are
// separate grid rows (blockIdx.y) so the three streams run concurrently.  Under the DIRECT
// selection reading the raw key rows (level 0) are scored as well.
#include <type_traits>

#include "lh_chunk_topk.h"
#include "lh_internal.h"

namespace lh {
namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename Tin, typename Tout>
struct Ctx {
  const Tin* x;    // this thread's column in token row 0 of its batch
  Tout* px;        // this thread's column in pooled row 0 of its batch (or null)
  float* sc;       // scores of this (batch, head) (or null)
  int64_t row;     // elements per token row (H * D)
  int p;
  float inv_p;
  int hd8;         // D / 8 lanes per head
  bool writer;     // first lane of the head
  bool score0;     // also score the raw tokens (level 0; DIRECT selection reads them)
  int lds_level;   // scores of this level go to `lds` (entry j at lds[j - lds_base]); -1: none
  int64_t lds_base;
  float* lds;
};

// l2 norm of entry (level, j) of this head: the thread's 8 squares in float64, reduced over
// the head's D/8 lanes, written by the head's first lane.
template <typename Tin, typename Tout>
__device__ __forceinline__ void score(const Ctx<Tin, Tout>& c, const Levels& lv, int level,
                                      int64_t j, const float (&v)[8]) {
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += static_cast<double>(v[i]) * static_cast<double>(v[i]);
  for (int m = 1; m < c.hd8; m <<= 1) ss += __shfl_xor(ss, m);
  if (c.writer) {
    if (level == c.lds_level)
      c.lds[j - c.lds_base] = static_cast<float>(sqrt(ss));
    else
      c.sc[lv.off[level] + j] = static_cast<float>(sqrt(ss));
  }
}

template <typename Tin, typename Tout>
__device__ __forceinline__ void emit(const Ctx<Tin, Tout>& c, const Levels& lv, int level,
                                     int64_t j, const float (&v)[8]) {
  if (c.px) store8(c.px + (lv.poff[level] + j) * c.row, v);
  if (c.sc) score(c, lv, level, j, v);
}

// Mean over the p tokens starting at token t0 (level 1); loads are issued four at a time so
// that several 16-byte requests per thread are in flight.
template <typename Tin, typename Tout>
__device__ __forceinline__ void level1(const Ctx<Tin, Tout>& c, const Levels& lv, int64_t t0,
                                       float (&out)[8]) {
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < c.p; i0 += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < c.p) load8(c.x + (t0 + i0 + u) * c.row, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < c.p) {
        if (c.score0) score(c, lv, 0, t0 + i0 + u, v[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = acc[e] * c.inv_p;
}

// Level-2 block for p = 4: all 16 token loads are issued before any arithmetic or store, so
// the stores of one block's pooled rows do not hold back the next block's loads.
template <typename Tin, typename Tout>
__device__ __forceinline__ void level2_p4(const Ctx<Tin, Tout>& c, const Levels& lv, int64_t t0,
                                          float (&out)[8]) {
  float v[16][8];
#pragma unroll
  for (int u = 0; u < 16; ++u) load8(c.x + (t0 + u) * c.row, v[u]);
  if (c.score0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) score(c, lv, 0, t0 + u, v[u]);
  }
  float acc2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc2[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      m[e] = (((v[4 * i][e] + v[4 * i + 1][e]) + v[4 * i + 2][e]) + v[4 * i + 3][e]) * c.inv_p;
    emit(c, lv, 1, (t0 + 4 * i) / lv.pw[1], m);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc2[e] += m[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = acc2[e] * c.inv_p;
}

template <int LVL, typename Tin, typename Tout>
__device__ __forceinline__ void pool_block(const Ctx<Tin, Tout>& c, const Levels& lv, int64_t t0,
                                           float (&out)[8]) {
  if constexpr (LVL == 1) {
    level1(c, lv, t0, out);
  } else if (LVL == 2 && c.p == 4) {
    level2_p4(c, lv, t0, out);
    emit(c, lv, LVL, t0 / lv.pw[LVL], out);
    return;
  } else {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int64_t span = lv.pw[LVL - 1];
    for (int i = 0; i < c.p; ++i) {
      float ch[8];
      pool_block<LVL - 1>(c, lv, t0 + i * span, ch);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ch[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = acc[e] * c.inv_p;
  }
  emit(c, lv, LVL, t0 / lv.pw[LVL], out);
}

template <int L, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void pool_score_kernel(Levels lv, const Tin* __restrict__ q,
                                                         const Tin* __restrict__ k,
                                                         const Tin* __restrict__ v,
                                                         Tout* pq, Tout* pk, Tout* pv,
                                                         float* scores) {
  const int stream = blockIdx.y;  // 0 = Q, 1 = K, 2 = V
  const Tin* x = stream == 0 ? q : (stream == 1 ? k : v);
  Tout* px = stream == 0 ? pq : (stream == 1 ? pk : pv);
  if (px == nullptr && stream != 1) return;

  const int64_t G = static_cast<int64_t>(lv.H) * lv.D / 8;  // column groups per row
  const int64_t T = lv.pw[L - 1];                              // tokens per coarsest block
  const int64_t tiles = lv.N / T;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= lv.B * tiles * G) return;
  const int64_t g = gid % G;
  const int64_t tt = gid / G;
  const int64_t tile = tt % tiles;
  const int64_t b = tt / tiles;
  const int hd8 = lv.D / 8;
  const int64_t h = g / hd8;

  Ctx<Tin, Tout> c;
  c.row = G * 8;
  c.x = x + b * lv.N * c.row + g * 8;
  c.px = px ? px + b * lv.P1 * c.row + g * 8 : nullptr;
  c.sc = stream == 1 ? scores + (b * lv.H + h) * lv.P : nullptr;
  c.p = lv.p;
  c.inv_p = 1.0f / static_cast<float>(lv.p);
  c.hd8 = hd8;
  c.writer = (g % hd8) == 0;
  c.score0 = stream == 1 && lv.direct;
  c.lds_level = -1;
  c.lds_base = 0;
  c.lds = nullptr;

  float out[8];
  pool_block<L - 1>(c, lv, tile * T, out);
}

// ------------------------------------------------------------------ scorer variants
// The "qk" (||q_bar|| * ||k_bar||) and "qkv" (||[q_bar; k_bar; v_bar]||) scorers need the
// norms of the three pooled rows of one entry together, so here one thread pools Q, K and V
// of its 8 columns side by side (three loads per token instead of one thread per stream).
// The per-stream sums of squares are float64, reduced over the head's D/8 lanes before they
// are combined; the head's first lane writes the float32 score.
template <typename Tin, typename Tout>
struct Ctx3 {
  const Tin* x[3];  // this thread's column in token row 0 of its batch, per stream
  Tout* px[3];      // this thread's column in pooled row 0 of its batch, per stream (or null)
  float* sc;        // scores of this (batch, head)
  int64_t row;
  int p;
  float inv_p;
  int hd8;
  bool writer;
  bool score0;
  int scorer;       // 0 = k, 1 = qk, 2 = qkv
  int lds_level;    // scores of this level go to `lds` (entry j at lds[j - lds_base]); -1: none
  int64_t lds_base;
  float* lds;
};

__device__ __forceinline__ double lane_ssq(const float (&v)[8], int hd8) {
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += static_cast<double>(v[i]) * static_cast<double>(v[i]);
  for (int m = 1; m < hd8; m <<= 1) ss += __shfl_xor(ss, m);
  return ss;
}

template <typename Tin, typename Tout>
__device__ __forceinline__ void score3(const Ctx3<Tin, Tout>& c, const Levels& lv, int level,
                                       int64_t j, const float (&vq)[8], const float (&vk)[8],
                                       const float (&vv)[8]) {
  const double sk = lane_ssq(vk, c.hd8);
  double s;
  if (c.scorer == 0) {
    s = sqrt(sk);
  } else if (c.scorer == 1) {
    s = sqrt(lane_ssq(vq, c.hd8)) * sqrt(sk);
  } else {
    s = sqrt(lane_ssq(vq, c.hd8) + sk + lane_ssq(vv, c.hd8));
  }
  if (c.writer) {
    if (level == c.lds_level)
      c.lds[j - c.lds_base] = static_cast<float>(s);
    else
      c.sc[lv.off[level] + j] = static_cast<float>(s);
  }
}

template <typename Tin, typename Tout>
__device__ __forceinline__ void emit3(const Ctx3<Tin, Tout>& c, const Levels& lv, int level,
                                      int64_t j, const float (&v)[3][8]) {
#pragma unroll
  for (int s = 0; s < 3; ++s)
    if (c.px[s]) store8(c.px[s] + (lv.poff[level] + j) * c.row, v[s]);
  score3(c, lv, level, j, v[0], v[1], v[2]);
}

// Mean of the p tokens from t0 for all three streams; four tokens' loads are in flight at a
// time per stream.
template <typename Tin, typename Tout>
__device__ __forceinline__ void level1_3(const Ctx3<Tin, Tout>& c, const Levels& lv, int64_t t0,
                                         float (&out)[3][8]) {
  float acc[3][8];
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[s][e] = 0.f;
  for (int i0 = 0; i0 < c.p; i0 += 4) {
    float v[3][4][8];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u < c.p) load8(c.x[s] + (t0 + i0 + u) * c.row, v[s][u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < c.p) {
        if (c.score0) score3(c, lv, 0, t0 + i0 + u, v[0][u], v[1][u], v[2][u]);
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[s][e] += v[s][u][e];
      }
  }
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) out[s][e] = acc[s][e] * c.inv_p;
}

template <int LVL, typename Tin, typename Tout>
__device__ __forceinline__ void pool_block3(const Ctx3<Tin, Tout>& c, const Levels& lv,
                                            int64_t t0, float (&out)[3][8]) {
  if constexpr (LVL == 1) {
    level1_3(c, lv, t0, out);
  } else {
    float acc[3][8];
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[s][e] = 0.f;
    const int64_t span = lv.pw[LVL - 1];
    for (int i = 0; i < c.p; ++i) {
      float ch[3][8];
      pool_block3<LVL - 1>(c, lv, t0 + i * span, ch);
#pragma unroll
      for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[s][e] += ch[s][e];
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) out[s][e] = acc[s][e] * c.inv_p;
  }
  emit3(c, lv, LVL, t0 / lv.pw[LVL], out);
}

template <int L, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void pool_score3_kernel(Levels lv, int scorer,
                                                          const Tin* __restrict__ q,
                                                          const Tin* __restrict__ k,
                                                          const Tin* __restrict__ v,
                                                          Tout* pq, Tout* pk, Tout* pv,
                                                          float* scores) {
  const int64_t G = static_cast<int64_t>(lv.H) * lv.D / 8;
  const int64_t T = lv.pw[L - 1];
  const int64_t tiles = lv.N / T;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= lv.B * tiles * G) return;
  const int64_t g = gid % G;
  const int64_t tt = gid / G;
  const int64_t tile = tt % tiles;
  const int64_t b = tt / tiles;
  const int hd8 = lv.D / 8;
  const int64_t h = g / hd8;

  Ctx3<Tin, Tout> c;
  c.row = G * 8;
  const Tin* xs[3] = {q, k, v};
  Tout* ps[3] = {pq, pk, pv};
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    c.x[s] = xs[s] + b * lv.N * c.row + g * 8;
    c.px[s] = ps[s] ? ps[s] + b * lv.P1 * c.row + g * 8 : nullptr;
  }
  c.sc = scores + (b * lv.H + h) * lv.P;
  c.p = lv.p;
  c.inv_p = 1.0f / static_cast<float>(lv.p);
  c.hd8 = hd8;
  c.writer = (g % hd8) == 0;
  c.score0 = lv.direct;
  c.scorer = scorer;
  c.lds_level = -1;
  c.lds_base = 0;
  c.lds = nullptr;

  float out[3][8];
  pool_block3<L - 1>(c, lv, tile * T, out);
}

// ------------------------------------------------------ fused pool + score + top-K
// One workgroup per (batch, head, chunk c of the finest selected level f): it pools Q, K and
// V of the chunk's token span (W p^f tokens, a whole number of coarsest blocks), writes the
// pooled rows and the scores of the other levels, keeps level f's W scores in LDS and runs
// the chunk's bitonic top-K in place -- the scores of that level never leave the workgroup.
// The chunks of coarser levels span several workgroups; lh_topk's kernel selects those
// afterwards.  Threads: D/8 lanes per 16-byte column group of the head, 256 / (D/8)
// "walkers" taking the span's coarsest blocks in turn.
template <int L, bool SPLIT, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void pool_score_topk_kernel(Levels lv, int scorer,
                                                              const Tin* __restrict__ q,
                                                              const Tin* __restrict__ k,
                                                              const Tin* __restrict__ v,
                                                              Tout* pq, Tout* pk, Tout* pv,
                                                              float* scores, int32_t* sel) {
  __shared__ float fsc[kTopkMaxWidth];
  __shared__ uint64_t key[kTopkMaxWidth];
  __shared__ int32_t flag[kTopkMaxWidth];
  __shared__ int32_t part[kTopkThreads];
  const int f = lv.sel_first;
  const int64_t ch = blockIdx.x;
  const int64_t bh = blockIdx.y, b = bh / lv.H, h = bh % lv.H;
  const int W = static_cast<int>(lv.width[f]);
  const int64_t T = lv.pw[L - 1];
  const int64_t span = W * lv.pw[f];
  const int64_t t0 = ch * span, nblk = span / T;
  const int hd8 = lv.D / 8;
  const int g = threadIdx.x % hd8, walker = threadIdx.x / hd8, walkers = 256 / hd8;
  const int64_t row = static_cast<int64_t>(lv.H) * lv.D;
  const int64_t col = h * lv.D + g * 8;

  if constexpr (SPLIT) {
    // key scorer: (stream, block) items, one stream per item as in pool_score_kernel
    Ctx<Tin, Tout> c;
    c.row = row;
    c.p = lv.p;
    c.inv_p = 1.0f / static_cast<float>(lv.p);
    c.hd8 = hd8;
    c.writer = g == 0;
    c.lds_level = f;
    c.lds_base = ch * W;
    c.lds = fsc;
    for (int64_t it = walker; it < 3 * nblk; it += walkers) {
      const int stream = static_cast<int>(it / nblk);
      const int64_t blk = it % nblk;
      const Tin* x = stream == 0 ? q : (stream == 1 ? k : v);
      Tout* px = stream == 0 ? pq : (stream == 1 ? pk : pv);
      if (px == nullptr && stream != 1) continue;
      c.x = x + b * lv.N * row + col;
      c.px = px ? px + b * lv.P1 * row + col : nullptr;
      c.sc = stream == 1 ? scores + bh * lv.P : nullptr;
      c.score0 = stream == 1 && lv.direct;
      float out[8];
      pool_block<L - 1>(c, lv, t0 + blk * T, out);
    }
  } else {
    Ctx3<Tin, Tout> c;
    c.row = row;
    const Tin* xs[3] = {q, k, v};
    Tout* ps[3] = {pq, pk, pv};
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      c.x[s] = xs[s] + b * lv.N * row + col;
      c.px[s] = ps[s] ? ps[s] + b * lv.P1 * row + col : nullptr;
    }
    c.sc = scores + bh * lv.P;
    c.p = lv.p;
    c.inv_p = 1.0f / static_cast<float>(lv.p);
    c.hd8 = hd8;
    c.writer = g == 0;
    c.score0 = lv.direct;
    c.scorer = scorer;
    c.lds_level = f;
    c.lds_base = ch * W;
    c.lds = fsc;
    for (int64_t blk = walker; blk < nblk; blk += walkers) {
      float out[3][8];
      pool_block3<L - 1>(c, lv, t0 + blk * T, out);
    }
  }
  __syncthreads();
  const int64_t nch = lv.nchunk[f];
  const int64_t base = lv.keff[f] / nch, rem = lv.keff[f] % nch;
  const int quota = static_cast<int>(base + (ch < rem ? 1 : 0));
  const int64_t first_out = ch * base + (ch < rem ? ch : rem);
  chunk_topk(fsc, W, quota, ch * W, sel + bh * lv.K + lv.soff[f] + first_out, key, flag, part);
}

template <typename Tin, typename Tout>
hipError_t dispatch(const Levels& lv, const void* q, const void* k, const void* v, void* pq,
                    void* pk, void* pv, float* scores, hipStream_t st) {
  if (lv.scorer != LH_SCORE_K) {
    const int64_t G = static_cast<int64_t>(lv.H) * lv.D / 8;
    const int64_t total = lv.B * (lv.N / lv.pw[lv.L - 1]) * G;
    dim3 grid(static_cast<unsigned>((total + 255) / 256));
    const int sc = lv.scorer == LH_SCORE_QK ? 1 : 2;
    auto args3 = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, lv, sc, static_cast<const Tin*>(q),
                         static_cast<const Tin*>(k), static_cast<const Tin*>(v),
                         static_cast<Tout*>(pq), static_cast<Tout*>(pk), static_cast<Tout*>(pv),
                         scores);
    };
    switch (lv.L) {
      case 2: args3(pool_score3_kernel<2, Tin, Tout>); break;
      case 3: args3(pool_score3_kernel<3, Tin, Tout>); break;
      case 4: args3(pool_score3_kernel<4, Tin, Tout>); break;
      case 5: args3(pool_score3_kernel<5, Tin, Tout>); break;
      case 6: args3(pool_score3_kernel<6, Tin, Tout>); break;
      case 7: args3(pool_score3_kernel<7, Tin, Tout>); break;
      case 8: args3(pool_score3_kernel<8, Tin, Tout>); break;
      default: return hipSuccess;
    }
    return hipGetLastError();
  }
  const int64_t G = static_cast<int64_t>(lv.H) * lv.D / 8;
  const int64_t total = lv.B * (lv.N / lv.pw[lv.L - 1]) * G;
  dim3 grid(static_cast<unsigned>((total + 255) / 256), 3);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, lv, static_cast<const Tin*>(q),
                       static_cast<const Tin*>(k), static_cast<const Tin*>(v),
                       static_cast<Tout*>(pq), static_cast<Tout*>(pk), static_cast<Tout*>(pv),
                       scores);
  };
  switch (lv.L) {
    case 2: args(pool_score_kernel<2, Tin, Tout>); break;
    case 3: args(pool_score_kernel<3, Tin, Tout>); break;
    case 4: args(pool_score_kernel<4, Tin, Tout>); break;
    case 5: args(pool_score_kernel<5, Tin, Tout>); break;
    case 6: args(pool_score_kernel<6, Tin, Tout>); break;
    case 7: args(pool_score_kernel<7, Tin, Tout>); break;
    case 8: args(pool_score_kernel<8, Tin, Tout>); break;
    default: return hipSuccess;
  }
  return hipGetLastError();
}

bool pool_topk_fusable(const Levels& lv) {
  if (lv.L < 2 || lv.K == 0 || lv.sel_first > lv.sel_last) return false;
  const int f = lv.sel_first;
  const int64_t span = lv.width[f] * lv.pw[f];
  return span % lv.pw[lv.L - 1] == 0 && lv.width[f] <= kTopkMaxWidth;
}

template <typename Tin, typename Tout>
hipError_t dispatch_fused(const Levels& lv, const void* q, const void* k, const void* v,
                          void* pq, void* pk, void* pv, float* scores, int32_t* sel,
                          hipStream_t st) {
  dim3 grid(static_cast<unsigned>(lv.nchunk[lv.sel_first]), static_cast<unsigned>(lv.B * lv.H));
  const int sc = lv.scorer == LH_SCORE_K ? 0 : (lv.scorer == LH_SCORE_QK ? 1 : 2);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, lv, sc, static_cast<const Tin*>(q),
                       static_cast<const Tin*>(k), static_cast<const Tin*>(v),
                       static_cast<Tout*>(pq), static_cast<Tout*>(pk), static_cast<Tout*>(pv),
                       scores, sel);
  };
  auto by_levels = [&](auto split) {
    constexpr bool S = decltype(split)::value;
    switch (lv.L) {
      case 2: go(pool_score_topk_kernel<2, S, Tin, Tout>); break;
      case 3: go(pool_score_topk_kernel<3, S, Tin, Tout>); break;
      case 4: go(pool_score_topk_kernel<4, S, Tin, Tout>); break;
      case 5: go(pool_score_topk_kernel<5, S, Tin, Tout>); break;
      case 6: go(pool_score_topk_kernel<6, S, Tin, Tout>); break;
      case 7: go(pool_score_topk_kernel<7, S, Tin, Tout>); break;
      default: go(pool_score_topk_kernel<8, S, Tin, Tout>); break;
    }
  };
  if (sc == 0)
    by_levels(std::true_type{});
  else
    by_levels(std::false_type{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool_score_topk(const Levels& lv, int32_t in_f32, const void* q, const void* k,
                                  const void* v, void* pq, void* pk, void* pv, int32_t out_f32,
                                  float* scores, int32_t* sel, hipStream_t st) {
  if (!pool_topk_fusable(lv)) {  // separate passes
    hipError_t e = launch_pool_score(lv, in_f32, q, k, v, pq, pk, pv, out_f32, scores, st);
    if (e != hipSuccess) return e;
    return launch_topk(lv, scores, sel, st);
  }
  hipError_t e;
  if (in_f32)
    e = out_f32 ? dispatch_fused<float, float>(lv, q, k, v, pq, pk, pv, scores, sel, st)
                : dispatch_fused<float, uint16_t>(lv, q, k, v, pq, pk, pv, scores, sel, st);
  else
    e = out_f32 ? dispatch_fused<uint16_t, float>(lv, q, k, v, pq, pk, pv, scores, sel, st)
                : dispatch_fused<uint16_t, uint16_t>(lv, q, k, v, pq, pk, pv, scores, sel, st);
  if (e != hipSuccess) return e;
  return launch_topk_levels(lv, lv.sel_first + 1, lv.sel_last, scores, sel, st);
}

hipError_t launch_pool_score(const Levels& lv, int32_t in_f32, const void* q, const void* k,
                             const void* v, void* pq, void* pk, void* pv, int32_t out_f32,
                             float* scores, hipStream_t st) {
  if (lv.L < 2) return hipSuccess;
  if (in_f32) {
    return out_f32 ? dispatch<float, float>(lv, q, k, v, pq, pk, pv, scores, st)
                   : dispatch<float, uint16_t>(lv, q, k, v, pq, pk, pv, scores, st);
  }
  return out_f32 ? dispatch<uint16_t, float>(lv, q, k, v, pq, pk, pv, scores, st)
                 : dispatch<uint16_t, uint16_t>(lv, q, k, v, pq, pk, pv, scores, st);
}

}  // namespace lh
