// Stage 3: chunked bitonic top-K, stratified per chunk.
//
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "核心方法：金字塔池化与“外部选择”", item 2: the top entries of every pyramid level are
// picked by a chunked bitonic top-K kernel.  [CB] clawdbytes.com, "Lighthouse Attention: the
// training-time hierarchy that makes quadratic attention ...", section "Four-Stage Pipeline
// Wraps Standard FlashAttention": the chunking makes the selection stratified rather than a
// global top-K.
//
// Reading: a chunk is C consecutive entries of the level being selected (the whole level when
// it is shorter); chunk c keeps floor(k/n_chunks) entries plus one if c < k mod n_chunks;
// inside a chunk entries rank by (score descending, index ascending), NaN last.
//
// Design: one workgroup per (batch*head, chunk) of the levels [first, last]; the chunk itself
// is selected by chunk_topk (register bitonic network, cross-lane exchanges inside a wave,
// LDS only between waves).
#include "lh_chunk_topk.h"
#include "lh_internal.h"

namespace lh {
namespace {

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Levels lv, int first, int last,
                                                            const float* __restrict__ scores,
                                                            int32_t* __restrict__ sel) {
  __shared__ uint64_t key[kTopkMaxWidth];
  __shared__ int32_t flag[kTopkMaxWidth];
  __shared__ int32_t part[kTopkThreads];

  // which level and chunk
  int64_t c = blockIdx.x;
  int level = first;
  while (level < last && c >= lv.nchunk[level]) {
    c -= lv.nchunk[level];
    ++level;
  }
  const int64_t bh = blockIdx.y;
  const int64_t nch = lv.nchunk[level];
  const int64_t base = lv.keff[level] / nch;
  const int64_t rem = lv.keff[level] % nch;
  const int quota = static_cast<int>(base + (c < rem ? 1 : 0));
  const int64_t first_out = c * base + (c < rem ? c : rem);
  const int W = static_cast<int>(lv.width[level]);
  const int64_t start = c * W;  // level-local index of the chunk's first entry
  chunk_topk(scores + bh * lv.P + lv.off[level] + start, W, quota, start,
             sel + bh * lv.K + lv.soff[level] + first_out, key, flag, part);
}

}  // namespace

hipError_t launch_topk_levels(const Levels& lv, int first, int last, const float* scores,
                              int32_t* sel, hipStream_t st) {
  if (lv.L < 2 || first > last) return hipSuccess;
  int64_t chunks = 0;
  for (int l = first; l <= last; ++l) chunks += lv.nchunk[l];
  if (chunks == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(lv.B * lv.H));
  hipLaunchKernelGGL(topk_kernel, grid, dim3(kTopkThreads), 0, st, lv, first, last, scores, sel);
  return hipGetLastError();
}

hipError_t launch_topk(const Levels& lv, const float* scores, int32_t* sel, hipStream_t st) {
  // REFINE: levels 1..L-1; DIRECT: 0..L-2
  return launch_topk_levels(lv, lv.sel_first, lv.sel_last, scores, sel, st);
}

}  // namespace lh
