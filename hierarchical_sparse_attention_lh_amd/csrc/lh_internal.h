// Internal declarations shared by the host side (lh_api.cpp) and the HIP kernels.
// Not part of the public ABI; the public interface is include/lh_api.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lh_api.h"

namespace lh {

// Level table derived on the host from an lh_config (closed forms only), passed by value
// to kernels.  Level l has n[l] = N / p^l entries; pyramid id of (l, j) = off[l] + j.
struct Levels {
  int32_t L, p;
  int64_t B, N;
  int32_t H, D;
  int64_t n[LH_MAX_LEVELS];     // entries per level
  int64_t pw[LH_MAX_LEVELS];    // p^l (tokens per entry)
  int64_t off[LH_MAX_LEVELS];   // pyramid offsets
  int64_t poff[LH_MAX_LEVELS];  // rows of level l (>= 1) inside the pooled tensors
  int64_t keff[LH_MAX_LEVELS];  // kept entries at selected levels (0 elsewhere)
  int64_t nchunk[LH_MAX_LEVELS];
  int64_t width[LH_MAX_LEVELS]; // chunk width
  int64_t soff[LH_MAX_LEVELS];  // offset of the level's kept indices in sel
  int64_t P;                    // pyramid total
  int64_t P1;                   // pooled rows (levels >= 1)
  int64_t K;                    // sel_total
  int64_t S;                    // gathered length
  int32_t lg[LH_MAX_LEVELS];    // log2(p^l) when p is a power of two, else -1
  int32_t direct;               // selection reading: 0 = REFINE (levels 1..L-1, kept entries
                                // enter as their p children), 1 = DIRECT (levels 0..L-2, kept
                                // entries enter themselves)
  int32_t sel_first, sel_last;  // selected levels (sel_first > sel_last when none)
  int32_t scorer;               // lh_scorer
};

// floor(x / p^l) for non-negative x < 2^31, by a shift when p is a power of two.
__host__ __device__ __forceinline__ int level_div(const Levels& lv, int l, int x) {
  return lv.lg[l] >= 0 ? (x >> lv.lg[l]) : x / static_cast<int>(lv.pw[l]);
}

// ---------------------------------------------------------------- bf16 helpers
// bfloat16 values are carried as raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> packed bf16 pair (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Gathered-domain tensors are stored with their sequence length padded to a multiple of
// 128 (one forward query tile); padding rows are written as finite values (zeros).
inline int64_t padded_len(int64_t S) { return (S + 127) / 128 * 128; }

// One attention call: shapes, where the rows of Q, K, V live, and where results go.
// Strides are in elements for (batch, head, sequence position).  Mapped calls read row s of
// head (b, h) as pyramid entry gmap[b, h, s] of the token tensors q/k/v ([B, N, H, D]) or of
// the pooled levels pq/pk/pv ([B, P1, H, D]); the q/k/v strides are then unused.
struct AttnCall {
  int64_t B, H, S;
  int32_t D;
  float scale;
  int32_t causal;
  int32_t o_rows;  // rows per head written to O and to the gradients (S, or Sp when padded)
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3], g_stride[3];
  int32_t mapped;
  const Levels* lv;
  const int32_t* gmap;  // [B*H, Sp]
  const void* pq;
  const void* pk;
  const void* pv;
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.
hipError_t launch_pool_score(const Levels& lv, int32_t in_f32, const void* q, const void* k,
                             const void* v, void* pq, void* pk, void* pv, int32_t out_f32,
                             float* scores, hipStream_t st);
hipError_t launch_topk(const Levels& lv, const float* scores, int32_t* sel, hipStream_t st);
// Top-K of the chunks of levels first..last only.
hipError_t launch_topk_levels(const Levels& lv, int first, int last, const float* scores,
                              int32_t* sel, hipStream_t st);
// Pooling, scoring and top-K in one pass where the finest selected level's chunks cover whole
// coarsest blocks (its scores then stay in LDS and are not written to `scores`); otherwise
// launch_pool_score followed by launch_topk.
hipError_t launch_pool_score_topk(const Levels& lv, int32_t in_f32, const void* q,
                                  const void* k, const void* v, void* pq, void* pk, void* pv,
                                  int32_t out_f32, float* scores, int32_t* sel, hipStream_t st);
hipError_t launch_build_map(const Levels& lv, const int32_t* sel, int32_t* gmap, int32_t* inv,
                            hipStream_t st);
// Gathered rows [B, H, Sp, D] bf16 of q/k/v (level 0) or the pooled levels (gmap ids).
hipError_t launch_gather(const Levels& lv, int32_t in_f32, const void* x[3], const void* px[3],
                         int32_t pooled_f32, const int32_t* gmap, void* const rows[3],
                         hipStream_t st);
// float32 -> bf16 (round to nearest even), n elements (n a multiple of 8).
hipError_t launch_to_bf16(const float* x, void* y, int64_t n, hipStream_t st);
// Attention over strided or mapped rows (lh_attn.hip).  lse / delta are [B*H, Sp].
hipError_t launch_attn_fwd2(const AttnCall& c, const void* q, const void* k, const void* v,
                            float* o, float* lse, hipStream_t st);
// pass: 1 = key pass (dk, dv), 2 = query pass (dq), 3 = both; dout rows at c.do_stride,
// gradients at c.g_stride.
hipError_t launch_attn_bwd2(int pass, const AttnCall& c, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv, hipStream_t st);
// delta[b, h, s] = sum_d dout * o for s < S (rows at c.do_stride / c.o_stride), 0 up to Sp.
hipError_t launch_attn_delta(const AttnCall& c, const void* dout, const float* o, float* delta,
                             hipStream_t st);
hipError_t launch_scatter(const Levels& lv, int32_t out_f32, const int32_t* inv,
                          const float* og, void* y, hipStream_t st);
hipError_t launch_scatter_bwd(const Levels& lv, int32_t in_f32, const int32_t* gmap,
                              const float* og, const void* dy, void* dog, float* delta,
                              hipStream_t st);
hipError_t launch_gather_pool_bwd(const Levels& lv, int32_t out_f32, const int32_t* inv,
                                  const float* dqg, const float* dkg, const float* dvg,
                                  void* dq, void* dk, void* dv, hipStream_t st);

}  // namespace lh
