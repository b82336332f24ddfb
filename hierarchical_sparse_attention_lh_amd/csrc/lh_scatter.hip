// Stage 5 and the token-side adjoints: scatter, scatter backward, gather+pool backward.
//
// [EN] encorp.ai, "Услуги по внедряване на AI задават правилния въпрос за Lighthouse
// Attention", section "Как four-stage pipeline остава бърз, без да чупи градиентите?": the
// attention outputs are spread back over the original positions with an offset that keeps
// causality, and gradients return to Q, K, V only through the gathered values.  [WS]
// wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// architecture figure caption under "核心方法：金字塔池化与“外部选择”": scatter-back closes
// the pipeline.
//
// Readings: entry (l, j) (causal position e = (j+1) p^l - 1) is added to tokens
// [e, e + p^l - 1]; tokens reached by nothing are 0.  Pool backward hands each source token
// of a gathered pooled entry 1/p^l of its gradient.
//
// Design: all three kernels are pull-based (each output element is written by exactly one
// thread, no atomics) and HBM-bound.  Scatter and gather+pool backward walk tokens: a
// thread owns 8 columns of the full token row and a run of 64 tokens, keeping every coarse
// level's current contribution in registers (reloaded only when that level's entry
// changes), so token rows are written whole and coarse rows are read once per run.
// Scatter backward owns 64 slots of one head, sums each slot's token span in float32,
// rounds once to bf16, writes the rows, and fuses Delta = rowsum(dO * O) for the attention
// backward.
#include "lh_internal.h"

namespace lh {
namespace {

__device__ __forceinline__ void ld8(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

__device__ __forceinline__ void ld8(const uint16_t* p, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void st8(uint16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// Non-temporal forms for the token-row outputs, which nothing in the layer reads back: the
// stores do not linger in the caches, and the kernels after them (pool of the next step,
// scatter backward) ran 4-7 % faster.
__device__ __forceinline__ void st8_nt(float* p, const float (&v)[8]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f4*>(p + 4));
}
__device__ __forceinline__ void st8_nt(uint16_t* p, const float (&v)[8]) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  __builtin_nontemporal_store(u, reinterpret_cast<u4*>(p));
}

// ----------------------------------------------------------------------------- scatter
// Token-walking layout shared by scatter and gather+pool backward: a thread owns 8 columns
// of the full token row (all heads side by side, so a wave writes 1 KB contiguous) and walks
// a run of kRun tokens in batches of 8.  Per batch it first loads every `inv` slot the batch
// needs -- level 0 for each token, and for each coarser level the few entries the batch
// touches -- as independent loads; then the rows of gathered entries, each coarse row once
// per entry (it stays in registers while the entry lasts).  Level-0 rows are loaded only for
// the few tokens that are gathered themselves.
constexpr int kRun = 64;
// KPRE prefetch slots per level: a batch of 8 consecutive tokens (aligned to 8) touches at
// most floor(7/p) + 2 entries of one level, so 3 slots serve p >= 4 and 5 serve p = 2, 3.
// Fewer slots keep the kernel at a higher occupancy (the p >= 4 form of gather+pool
// backward runs 14 % faster than with a 6-slot bound).

// OFFSET = 1: token t takes entry floor((t+1)/p^l) - 1 of level l (scatter); OFFSET = 0:
// entry floor(t/p^l) at weight 1/p^l (gather+pool backward).
// The lanes of one head (D/8 >= 8 consecutive lanes, q = 0.. within the group, first lane
// hbase of the wave) walk the same tokens: each batch's slot ids are loaded once per group,
// one id per lane, and spread to the group's lanes by shuffles.
template <int L, int OFFSET, int KPRE, typename Tout>
__device__ __forceinline__ void walk_tokens(const Levels& lv, const int32_t* __restrict__ iv,
                                            const float* __restrict__ rows, Tout* __restrict__ out,
                                            int64_t row, int t0, int t1, int q, int hbase) {
  float c[L][8];
  int cj[L];
  float w[L];
  w[0] = 1.0f;
#pragma unroll
  for (int l = 1; l < L; ++l) {
    cj[l] = -2;  // no entry cached
    w[l] = OFFSET ? 1.0f : w[l - 1] / static_cast<float>(lv.p);
  }
  for (int tb = t0; tb < t1; tb += 8) {
    const int tl = (tb + 8 < t1 ? tb + 8 : t1) - 1;  // last token of the batch
    const int32_t mine = (q < 8 && tb + q <= tl) ? iv[tb + q] : -1;
    int32_t mp[L];
    int jf[L];
#pragma unroll
    for (int l = 1; l < L; ++l) {
      jf[l] = level_div(lv, l, tb + OFFSET) - OFFSET;
      const int jl = level_div(lv, l, tl + OFFSET) - OFFSET;
      const int j = jf[l] + q;
      mp[l] = (q < KPRE && j >= 0 && j <= jl && j != cj[l]) ? iv[lv.off[l] + j] : -1;
    }
    int32_t s0[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) s0[u] = __shfl(mine, hbase + u);
    int32_t pre[L][KPRE];
#pragma unroll
    for (int l = 1; l < L; ++l)
#pragma unroll
      for (int i = 0; i < KPRE; ++i) pre[l][i] = __shfl(mp[l], hbase + i);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = tb + u;
      if (t > tl) break;
      float acc[8];
      if (s0[u] >= 0 && s0[u] < lv.S) {  // level 0: only a few percent of tokens are gathered
        ld8(rows + static_cast<int64_t>(s0[u]) * lv.D, acc);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      }
#pragma unroll
      for (int l = 1; l < L; ++l) {
        const int j = level_div(lv, l, t + OFFSET) - OFFSET;
        if (j != cj[l]) {
          cj[l] = j;
          const int32_t sl = pre[l][j - jf[l]];
          if (sl >= 0 && sl < lv.S) {
            ld8(rows + static_cast<int64_t>(sl) * lv.D, c[l]);
#pragma unroll
            for (int e = 0; e < 8; ++e) c[l][e] *= w[l];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) c[l][e] = 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += c[l][e];
      }
      st8_nt(out + static_cast<int64_t>(t) * row, acc);
    }
  }
}

template <int L, int KPRE, typename Tout>
__global__ __launch_bounds__(256) void scatter_kernel(Levels lv, int64_t Sp,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ og,
                                                      Tout* __restrict__ y) {
  const int hd8 = lv.D / 8;
  const int64_t G = static_cast<int64_t>(lv.H) * hd8;  // column groups per token row
  const int64_t runs = (lv.N + kRun - 1) / kRun;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= lv.B * runs * G) return;
  const int64_t g = gid % G;
  const int64_t rr = gid / G;
  const int64_t b = rr / runs;
  const int64_t t0 = (rr % runs) * kRun;
  const int64_t t1 = t0 + kRun < lv.N ? t0 + kRun : lv.N;
  const int64_t bh = b * lv.H + g / hd8;
  const int q = static_cast<int>(g % hd8);
  walk_tokens<L, 1, KPRE>(lv, inv + bh * lv.P, og + bh * Sp * lv.D + q * 8,
                          y + b * lv.N * G * 8 + g * 8, G * 8, static_cast<int>(t0),
                          static_cast<int>(t1), q, static_cast<int>(threadIdx.x & 63) - q);
}

// -------------------------------------------------------------------- scatter backward
template <int D, typename Tin>
__global__ __launch_bounds__(256) void scatter_bwd_kernel(
    Levels lv, int64_t Sp, const int32_t* __restrict__ gmap, const float* __restrict__ og,
    const Tin* __restrict__ dy, uint16_t* __restrict__ dog, float* __restrict__ delta) {
  constexpr int G = D / 8, SPP = 256 / G;
  constexpr int TS = 64;  // slots per workgroup
  const int64_t BH = lv.B * lv.H;
  const int64_t bh = blockIdx.x % BH;  // heads fastest: neighbouring slot ranges of all heads
  const int64_t b = bh / lv.H, h = bh % lv.H;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x / BH) * TS;
  const int g = threadIdx.x % G;
  const int64_t row = static_cast<int64_t>(lv.H) * D;
  const Tin* yb = dy + b * lv.N * row + h * D + g * 8;
#pragma unroll
  for (int pass = 0; pass < TS / SPP; ++pass) {
    const int sl = pass * SPP + threadIdx.x / G;
    const int64_t s = s0 + sl;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int32_t id = s < lv.S ? gmap[bh * Sp + s] : -1;
    if (id >= 0 && id < lv.P) {
      int l = 0;
      while (l < lv.L - 1 && id >= lv.off[l + 1]) ++l;
      const int64_t j = id - lv.off[l];
      const int64_t lo = (j + 1) * lv.pw[l] - 1;
      const int64_t hi = lo + lv.pw[l] < lv.N ? lo + lv.pw[l] : lv.N;
      // loads four rows ahead of the (sequential, order-preserving) accumulation
      int64_t t = lo;
      for (; t + 4 <= hi; t += 4) {
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) ld8(yb + (t + u) * row, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
      }
      for (; t < hi; ++t) {
        float v[8];
        ld8(yb + t * row, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[e];
      }
    }
    // round once to bf16; Delta uses the rounded values, as the attention backward does
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = bf16_to_f32(f32_to_bf16(acc[e]));
    st8(dog + (bh * Sp + s) * D + g * 8, r);
    float part = 0.f;
    if (s < lv.S) {  // padding rows of og are never read
      float o[8];
      ld8(og + (bh * Sp + s) * D + g * 8, o);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(r[e], o[e], part);
    }
    for (int m = 1; m < G; m <<= 1) part += __shfl_xor(part, m);
    if (g == 0) delta[bh * Sp + s] = part;
  }
}

// ------------------------------------------------------------- gather + pool backward
// Token-walking layout of scatter_kernel; blockIdx.y selects Q, K or V.
template <int L, int KPRE, typename Tout>
__global__ __launch_bounds__(256) void gather_pool_bwd_kernel(
    Levels lv, int64_t Sp, const int32_t* __restrict__ inv, const float* __restrict__ g0,
    const float* __restrict__ g1, const float* __restrict__ g2, Tout* __restrict__ d0,
    Tout* __restrict__ d1, Tout* __restrict__ d2) {
  const int which = blockIdx.y;
  const float* gx = which == 0 ? g0 : (which == 1 ? g1 : g2);
  Tout* dx = which == 0 ? d0 : (which == 1 ? d1 : d2);
  const int hd8 = lv.D / 8;
  const int64_t G = static_cast<int64_t>(lv.H) * hd8;
  const int64_t runs = (lv.N + kRun - 1) / kRun;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= lv.B * runs * G) return;
  const int64_t g = gid % G;
  const int64_t rr = gid / G;
  const int64_t b = rr / runs;
  const int64_t t0 = (rr % runs) * kRun;
  const int64_t t1 = t0 + kRun < lv.N ? t0 + kRun : lv.N;
  const int64_t bh = b * lv.H + g / hd8;
  const int q = static_cast<int>(g % hd8);
  walk_tokens<L, 0, KPRE>(lv, inv + bh * lv.P, gx + bh * Sp * lv.D + q * 8,
                          dx + b * lv.N * G * 8 + g * 8, G * 8, static_cast<int>(t0),
                          static_cast<int>(t1), q, static_cast<int>(threadIdx.x & 63) - q);
}

template <typename Tout>
hipError_t scatter_t(const Levels& lv, const int32_t* inv, const float* og, void* y,
                     hipStream_t st) {
  const int64_t Sp = padded_len(lv.S);
  const int64_t threads = lv.B * ((lv.N + kRun - 1) / kRun) * lv.H * (lv.D / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, lv, Sp, inv, og, static_cast<Tout*>(y));
  };
  const bool wide = lv.p < 4;  // 5 prefetch slots for p = 2, 3; 3 for p >= 4
  switch (lv.L) {
    case 1: wide ? go(scatter_kernel<1, 5, Tout>) : go(scatter_kernel<1, 3, Tout>); break;
    case 2: wide ? go(scatter_kernel<2, 5, Tout>) : go(scatter_kernel<2, 3, Tout>); break;
    case 3: wide ? go(scatter_kernel<3, 5, Tout>) : go(scatter_kernel<3, 3, Tout>); break;
    case 4: wide ? go(scatter_kernel<4, 5, Tout>) : go(scatter_kernel<4, 3, Tout>); break;
    case 5: wide ? go(scatter_kernel<5, 5, Tout>) : go(scatter_kernel<5, 3, Tout>); break;
    case 6: wide ? go(scatter_kernel<6, 5, Tout>) : go(scatter_kernel<6, 3, Tout>); break;
    case 7: wide ? go(scatter_kernel<7, 5, Tout>) : go(scatter_kernel<7, 3, Tout>); break;
    default: wide ? go(scatter_kernel<8, 5, Tout>) : go(scatter_kernel<8, 3, Tout>); break;
  }
  return hipGetLastError();
}

template <typename Tin>
hipError_t scatter_bwd_t(const Levels& lv, const int32_t* gmap, const float* og, const void* dy,
                         void* dog, float* delta, hipStream_t st) {
  const int64_t Sp = padded_len(lv.S);
  dim3 grid(static_cast<unsigned>(Sp / 64 * lv.B * lv.H));
  auto* a = static_cast<uint16_t*>(dog);
  if (lv.D == 64)
    hipLaunchKernelGGL((scatter_bwd_kernel<64, Tin>), grid, dim3(256), 0, st, lv, Sp, gmap, og,
                       static_cast<const Tin*>(dy), a, delta);
  else
    hipLaunchKernelGGL((scatter_bwd_kernel<128, Tin>), grid, dim3(256), 0, st, lv, Sp, gmap, og,
                       static_cast<const Tin*>(dy), a, delta);
  return hipGetLastError();
}

template <typename Tout>
hipError_t gpb_t(const Levels& lv, const int32_t* inv, const float* a, const float* b,
                 const float* c, void* x, void* y, void* z, hipStream_t st) {
  const int64_t Sp = padded_len(lv.S);
  const int64_t threads = lv.B * ((lv.N + kRun - 1) / kRun) * lv.H * (lv.D / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256), 3);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, lv, Sp, inv, a, b, c,
                       static_cast<Tout*>(x), static_cast<Tout*>(y), static_cast<Tout*>(z));
  };
  const bool wide = lv.p < 4;
  switch (lv.L) {
    case 1: wide ? go(gather_pool_bwd_kernel<1, 5, Tout>) : go(gather_pool_bwd_kernel<1, 3, Tout>); break;
    case 2: wide ? go(gather_pool_bwd_kernel<2, 5, Tout>) : go(gather_pool_bwd_kernel<2, 3, Tout>); break;
    case 3: wide ? go(gather_pool_bwd_kernel<3, 5, Tout>) : go(gather_pool_bwd_kernel<3, 3, Tout>); break;
    case 4: wide ? go(gather_pool_bwd_kernel<4, 5, Tout>) : go(gather_pool_bwd_kernel<4, 3, Tout>); break;
    case 5: wide ? go(gather_pool_bwd_kernel<5, 5, Tout>) : go(gather_pool_bwd_kernel<5, 3, Tout>); break;
    case 6: wide ? go(gather_pool_bwd_kernel<6, 5, Tout>) : go(gather_pool_bwd_kernel<6, 3, Tout>); break;
    case 7: wide ? go(gather_pool_bwd_kernel<7, 5, Tout>) : go(gather_pool_bwd_kernel<7, 3, Tout>); break;
    default: wide ? go(gather_pool_bwd_kernel<8, 5, Tout>) : go(gather_pool_bwd_kernel<8, 3, Tout>); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scatter(const Levels& lv, int32_t out_f32, const int32_t* inv,
                          const float* og, void* y, hipStream_t st) {
  return out_f32 ? scatter_t<float>(lv, inv, og, y, st) : scatter_t<uint16_t>(lv, inv, og, y, st);
}

hipError_t launch_scatter_bwd(const Levels& lv, int32_t in_f32, const int32_t* gmap,
                              const float* og, const void* dy, void* dog, float* delta,
                              hipStream_t st) {
  return in_f32 ? scatter_bwd_t<float>(lv, gmap, og, dy, dog, delta, st)
                : scatter_bwd_t<uint16_t>(lv, gmap, og, dy, dog, delta, st);
}

hipError_t launch_gather_pool_bwd(const Levels& lv, int32_t out_f32, const int32_t* inv,
                                  const float* dqg, const float* dkg, const float* dvg,
                                  void* dq, void* dk, void* dv, hipStream_t st) {
  return out_f32 ? gpb_t<float>(lv, inv, dqg, dkg, dvg, dq, dk, dv, st)
                 : gpb_t<uint16_t>(lv, inv, dqg, dkg, dvg, dq, dk, dv, st);
}

}  // namespace lh
