// Chunked bitonic top-K of one chunk, shared by the top-K kernel and the fused pool + score +
// top-K kernel.
//
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "核心方法：金字塔池化与“外部选择”", item 2: a chunked bitonic top-K kernel picks each
// level's top entries.  [CB] clawdbytes.com, "Lighthouse Attention: the training-time hierarchy
// that makes quadratic attention ...", section "Four-Stage Pipeline Wraps Standard
// FlashAttention": chunking makes the selection stratified rather than a global top-K.
//
// Reading: inside a chunk entries rank by (score descending, index ascending), NaN last; the
// chunk keeps the first `quota` of that order, written in ascending index order.
//
// Design: the chunk's W scores become 64-bit keys (an order-preserving transform of the
// float32 score in the high word, the index in the low word; padding up to the power of two
// W2 is ~0), so an ascending bitonic network over unique keys yields exactly the reading's
// order.  256 threads hold R = max(1, W2 / 256) consecutive keys each in registers.  A
// compare-exchange of elements i and i ^ j runs
//   * inside a thread when j < R (register swap),
//   * across lanes of one wave when j / R < 64: DPP quad_perm for lane distance 1 and 2,
//     ds_swizzle (bit-mask mode) for 4, 8 and 16, v_permlane32_swap for 32 -- no LDS memory,
//     no barrier,
//   * through LDS with a workgroup barrier only when the partner lives in another wave
//     (j >= 64 R: 3 of the 55 stages for W2 = 1024).
// The first `quota` keys of the sorted order then flag their indices in LDS and a workgroup
// prefix sum compacts the flagged indices, which leaves them ascending.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

constexpr int kTopkThreads = 256;
constexpr int kTopkMaxWidth = 2048;

// Ascending order of the returned key = score descending, NaN last; -0 counts as +0.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t idx) {
  uint32_t u = __float_as_uint(s);
  uint32_t hi;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    hi = 0xffffffffu;  // NaN ranks after every number
  } else {
    if (u == 0x80000000u) u = 0u;
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending by value
    hi = ~asc;                                                           // descending
  }
  return (static_cast<uint64_t>(hi) << 32) | idx;
}

// The value of lane (lane ^ m) of the wave, for m in {1, 2, 4, 8, 16, 32} (uniform).
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int m) {
  switch (m) {
    case 1:  // quad_perm [1, 0, 3, 2]
      return static_cast<uint32_t>(
          __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    case 2:  // quad_perm [2, 3, 0, 1]
      return static_cast<uint32_t>(
          __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    case 4:  // ds_swizzle bit-mask mode: and 0x1f, or 0, xor m
      return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), (4 << 10) | 0x1F));
    case 8:
      return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), (8 << 10) | 0x1F));
    case 16:
      return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), (16 << 10) | 0x1F));
    default: {  // 32: the swap leaves {own, partner} in the two results
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return r[0] + r[1] - v;
    }
  }
}

__device__ __forceinline__ uint64_t lane_xor64(uint64_t x, int m) {
  const uint32_t lo = lane_xor(static_cast<uint32_t>(x), m);
  const uint32_t hi = lane_xor(static_cast<uint32_t>(x >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Top-`quota` of the W (<= kTopkMaxWidth) scores s[0..W) of one chunk whose first entry has
// level-local index `start`; writes the kept indices (start + i), ascending, to out[0..quota).
// Every thread of the 256-thread workgroup calls it.  LDS scratch: key (W2 64-bit keys, used
// by the cross-wave stages), flag (W ints), part (256 ints).
template <int R, int LOGW2>
__device__ __forceinline__ void chunk_topk_r(const float* s, int W, int quota, int64_t start,
                                             int32_t* out, uint64_t* key, int32_t* flag,
                                             int32_t* part) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint64_t kv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = tid * R + r;
    kv[r] = i < W ? rank_key(s[i], static_cast<uint32_t>(i)) : ~0ull;
  }
  for (int i = tid; i < W; i += kTopkThreads) flag[i] = 0;

  // every stage's distances are compile-time constants once the two loops unroll
#pragma unroll
  for (int lk = 1; lk <= LOGW2; ++lk) {
#pragma unroll
    for (int lj = lk - 1; lj >= 0; --lj) {
      const int k = 1 << lk, j = 1 << lj;
      if (j < R) {  // partner in the same thread
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((r & j) == 0) {
            const int i = tid * R + r;
            const bool up = (i & k) == 0;
            const uint64_t a = kv[r], b = kv[r | j];
            const bool swap = (a > b) == up;
            kv[r] = swap ? b : a;
            kv[r | j] = swap ? a : b;
          }
        }
      } else if (j < 64 * R) {  // partner lane lane ^ (j / R) of the same wave
        const int m = j / R;
        const bool lower = (lane & m) == 0;
        const bool up = (tid & (k / R)) == 0;
        const bool take_min = lower == up;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint64_t y = lane_xor64(kv[r], m);
          kv[r] = take_min ? (y < kv[r] ? y : kv[r]) : (y > kv[r] ? y : kv[r]);
        }
      } else {  // partner in another wave: through LDS
#pragma unroll
        for (int r = 0; r < R; ++r) key[tid * R + r] = kv[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = tid * R + r;
          const uint64_t y = key[i ^ j];
          const bool lower = (i & j) == 0, up = (i & k) == 0;
          kv[r] = (lower == up) ? (y < kv[r] ? y : kv[r]) : (y > kv[r] ? y : kv[r]);
        }
        __syncthreads();
      }
    }
  }

  // flag the first `quota` ranks in index order (after every thread cleared its flags)
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (tid * R + r < quota) flag[static_cast<uint32_t>(kv[r])] = 1;
  __syncthreads();

  // compact: each thread owns a contiguous run of indices
  const int per = (W + kTopkThreads - 1) / kTopkThreads;
  const int lo = tid * per;
  const int hi = min(W, lo + per);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += flag[i];
  part[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - cnt;
  for (int i = lo; i < hi; ++i)
    if (flag[i]) out[pos++] = static_cast<int32_t>(start + i);
}

// Dispatch on R = W2 / 256 (at least 1).  A chunk whose quota is 0 writes nothing; one whose
// quota covers it keeps every entry.  Uniform across the workgroup.
__device__ __forceinline__ void chunk_topk(const float* s, int W, int quota, int64_t start,
                                           int32_t* out, uint64_t* key, int32_t* flag,
                                           int32_t* part) {
  if (quota <= 0) return;
  if (quota >= W) {
    for (int i = threadIdx.x; i < W; i += kTopkThreads) out[i] = static_cast<int32_t>(start + i);
    return;
  }
  int W2 = 16;
  while (W2 < W) W2 <<= 1;
  switch (W2) {
    case 16: chunk_topk_r<1, 4>(s, W, quota, start, out, key, flag, part); break;
    case 32: chunk_topk_r<1, 5>(s, W, quota, start, out, key, flag, part); break;
    case 64: chunk_topk_r<1, 6>(s, W, quota, start, out, key, flag, part); break;
    case 128: chunk_topk_r<1, 7>(s, W, quota, start, out, key, flag, part); break;
    case 256: chunk_topk_r<1, 8>(s, W, quota, start, out, key, flag, part); break;
    case 512: chunk_topk_r<2, 9>(s, W, quota, start, out, key, flag, part); break;
    case 1024: chunk_topk_r<4, 10>(s, W, quota, start, out, key, flag, part); break;
    default: chunk_topk_r<8, 11>(s, W, quota, start, out, key, flag, part); break;
  }
}

}  // namespace lh
