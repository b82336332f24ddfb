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
// Design: one workgroup per (batch*head, chunk).  The chunk's scores become 64-bit keys
// (order-preserving transform of the float32 score in the high word, the index in the low
// word) so an ascending bitonic network over unique keys yields exactly the reading's
// order.  The network runs in LDS (<= 2048 keys, 16 KB); the kept entries are then marked
// in index order and compacted with a workgroup prefix sum, which leaves them ascending.
#include "lh_internal.h"

namespace lh {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxWidth = 2048;

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

__global__ __launch_bounds__(kThreads) void topk_kernel(Levels lv, int first, int last,
                                                        const float* __restrict__ scores,
                                                        int32_t* __restrict__ sel) {
  __shared__ uint64_t key[kMaxWidth];
  __shared__ int32_t flag[kMaxWidth];
  __shared__ int32_t part[kThreads];

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
  const float* s = scores + bh * lv.P + lv.off[level] + start;
  int32_t* out = sel + bh * lv.K + lv.soff[level] + first_out;
  const int tid = threadIdx.x;

  if (quota == 0) return;
  if (quota >= W) {  // the whole chunk is kept
    for (int i = tid; i < W; i += kThreads) out[i] = static_cast<int32_t>(start + i);
    return;
  }

  int W2 = 1;
  while (W2 < W) W2 <<= 1;
  for (int i = tid; i < W2; i += kThreads)
    key[i] = i < W ? rank_key(s[i], static_cast<uint32_t>(i)) : ~0ull;
  for (int i = tid; i < W; i += kThreads) flag[i] = 0;
  __syncthreads();

  // bitonic network, ascending
  for (int kk = 2; kk <= W2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (W2 >> 1); i += kThreads) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int b = a | j;
        const bool up = (a & kk) == 0;
        const uint64_t x = key[a], y = key[b];
        if ((x > y) == up) {
          key[a] = y;
          key[b] = x;
        }
      }
      __syncthreads();
    }
  }

  // mark the first `quota` ranks in index order
  for (int r = tid; r < quota; r += kThreads) flag[static_cast<uint32_t>(key[r])] = 1;
  __syncthreads();

  // compact: each thread owns a contiguous run of indices
  const int per = (W + kThreads - 1) / kThreads;
  const int lo = tid * per;
  const int hi = min(W, lo + per);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += flag[i];
  part[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - cnt;
  for (int i = lo; i < hi; ++i)
    if (flag[i]) out[pos++] = static_cast<int32_t>(start + i);
}

}  // namespace

hipError_t launch_topk(const Levels& lv, const float* scores, int32_t* sel, hipStream_t st) {
  if (lv.L < 2) return hipSuccess;
  const int first = lv.sel_first, last = lv.sel_last;  // REFINE: 1..L-1; DIRECT: 0..L-2
  int64_t chunks = 0;
  for (int l = first; l <= last; ++l) chunks += lv.nchunk[l];
  if (chunks == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(lv.B * lv.H));
  hipLaunchKernelGGL(topk_kernel, grid, dim3(kThreads), 0, st, lv, first, last, scores, sel);
  return hipGetLastError();
}

}  // namespace lh
