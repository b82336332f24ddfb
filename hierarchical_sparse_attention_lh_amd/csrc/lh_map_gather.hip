// Stage 4a/4b: the gathered order (gmap/inv) and the gathered rows.
//
// [EN] encorp.ai, "Услуги по внедряване на AI задават правилния въпрос за Lighthouse
// Attention", section "Как four-stage pipeline остава бърз, без да чупи градиентите?": the
// kept entries are collected into one contiguous dense subsequence; [WS] wispaper.ai,
// "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复", section
// "核心方法：金字塔池化与“外部选择”", item 3: that subsequence preserves causality, so plain
// causal attention runs on it.
//
// Reading: entry (l, j) sits at causal position e = (j+1) p^l - 1; the gathered set is the
// whole coarsest level plus the p children of every kept entry of levels 1..L-1, ordered by
// (e ascending, l ascending).
//
// Map design: the gathered set is the merge of L sorted lists (the coarsest level and, per
// selected level, the children of its kept entries).  The slot of an entry is its rank in its
// own list plus, for every other list, the number of that list's entries that precede it.
// For the coarsest list that count is a closed form; for a children list it is
// p * (kept parents below u/p) + (u mod p if parent u/p is kept), where u is the number of
// that level's entries complete before the position -- one binary search in the kept list.
// One thread per gathered entry; no atomics, no sort, and the result is the unique order.
//
// Gather design (lh_gather only: the layer's own attention reads the rows through gmap and
// never needs the copy): one workgroup per 64 slots of one head, rows copied with 16-byte
// vectors, rounded to bf16; padding slots S..Sp-1 are zeros.
#include "lh_internal.h"

namespace lh {
namespace {

__global__ __launch_bounds__(256) void fill_kernel(int32_t* __restrict__ p, int64_t n,
                                                   int32_t value) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<int4*>(p + i) = make_int4(value, value, value, value);
  } else {
    for (int64_t t = i; t < n; ++t) p[t] = value;
  }
}

// number of elements of the ascending list a[0..n) that are < x
__device__ __forceinline__ int64_t lower_bound(const int32_t* a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Number of gathered entries of level m whose causal position is <= T (T >= -1).
__device__ __forceinline__ int64_t count_upto(const Levels& lv, const int32_t* sel, int m,
                                              int64_t T) {
  const int64_t u = (T + 1) / lv.pw[m];  // level-m entries complete by token T
  if (m == lv.L - 1) return u < lv.n[m] ? u : lv.n[m];
  if (lv.direct) {  // level m entries are the kept entries of level m: count those below u
    return m <= lv.sel_last ? lower_bound(sel + lv.soff[m], lv.keff[m], u) : 0;
  }
  // level m entries are the children of kept entries of level m + 1
  const int32_t* kept = sel + lv.soff[m + 1];
  const int64_t nk = lv.keff[m + 1];
  const int64_t par = u / lv.p;
  const int64_t below = lower_bound(kept, nk, par);
  const int64_t partial = (below < nk && kept[below] == par) ? (u % lv.p) : 0;
  return lv.p * below + partial;
}

__global__ __launch_bounds__(256) void map_kernel(Levels lv, const int32_t* __restrict__ sel,
                                                  int32_t* __restrict__ gmap,
                                                  int32_t* __restrict__ inv, int64_t Sp) {
  const int64_t bh = blockIdx.y;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int32_t* s = sel + bh * lv.K;
  int32_t* g = gmap + bh * Sp;
  if (r >= Sp) return;
  if (r >= lv.S) {  // padding slots of the map
    g[r] = -1;
    return;
  }
  // list position -> (level m, index i, rank in own list)
  const int top = lv.L - 1;
  int m;
  int64_t i, own;
  if (r < lv.n[top]) {
    m = top;
    i = r;
    own = r;
  } else if (lv.direct) {  // the kept entries of levels 0..L-2, level by level
    int64_t rr = r - lv.n[top];
    int l = 0;
    while (l < lv.sel_last && rr >= lv.keff[l]) {
      rr -= lv.keff[l];
      ++l;
    }
    m = l;
    i = s[lv.soff[l] + rr];
    own = rr;
  } else {  // the p children of the kept entries of levels 1..L-1
    int64_t rr = r - lv.n[top];
    int l = 1;
    while (l < top && rr >= lv.p * lv.keff[l]) {
      rr -= lv.p * lv.keff[l];
      ++l;
    }
    m = l - 1;
    const int64_t parent = s[lv.soff[l] + rr / lv.p];
    i = parent * lv.p + rr % lv.p;
    own = rr;
  }
  const int64_t e = (i + 1) * lv.pw[m] - 1;
  int64_t slot = own;
  for (int mm = 0; mm < lv.L; ++mm) {
    if (mm == m) continue;
    // entries of a coarser-or-equal level precede only with a strictly smaller e; entries of
    // a finer level also precede on a tie in e.
    slot += count_upto(lv, s, mm, mm > m ? e - 1 : e);
  }
  const int64_t id = lv.off[m] + i;
  if (slot < 0 || slot >= lv.S || id < 0 || id >= lv.P) return;  // unreachable for valid sel
  g[slot] = static_cast<int32_t>(id);
  inv[bh * lv.P + id] = static_cast<int32_t>(slot);
}

__device__ __forceinline__ void load8_bf16(const uint16_t* p, uint4& out) {
  out = *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void load8_bf16(const float* p, uint4& out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out.x = pack_bf16x2(a.x, a.y);
  out.y = pack_bf16x2(a.z, a.w);
  out.z = pack_bf16x2(b.x, b.y);
  out.w = pack_bf16x2(b.z, b.w);
}

template <int D, typename Tin, typename Tpool>
__global__ __launch_bounds__(256) void gather_kernel(
    Levels lv, int64_t Sp, const Tin* __restrict__ x0, const Tin* __restrict__ x1,
    const Tin* __restrict__ x2, const Tpool* __restrict__ p0, const Tpool* __restrict__ p1,
    const Tpool* __restrict__ p2, const int32_t* __restrict__ gmap, uint16_t* r0, uint16_t* r1,
    uint16_t* r2) {
  constexpr int TS = 64;         // slots per workgroup
  constexpr int G = D / 8;       // 16-byte groups per row
  constexpr int SPP = 256 / G;   // slots per pass
  __shared__ int32_t ids[TS];

  const int64_t BH = lv.B * lv.H;
  const int64_t bh = blockIdx.x % BH;  // heads fastest: the heads' slices of a row together
  const int64_t b = bh / lv.H;
  const int64_t h = bh % lv.H;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x / BH) * TS;
  const int tid = threadIdx.x;
  if (tid < TS) {
    const int64_t s = s0 + tid;
    const int32_t id = s < lv.S ? gmap[bh * Sp + s] : -1;
    ids[tid] = (id >= 0 && id < lv.P) ? id : -1;  // out-of-range ids read as padding
  }
  __syncthreads();

  const int64_t row = static_cast<int64_t>(lv.H) * D;  // elements per token row
  const int g = tid % G;
  const int sl0 = tid / G;
  const int lvl_top = lv.L - 1;

  for (int which = 0; which < 3; ++which) {
    const Tin* x = which == 0 ? x0 : (which == 1 ? x1 : x2);
    const Tpool* px = which == 0 ? p0 : (which == 1 ? p1 : p2);
    uint16_t* ro = which == 0 ? r0 : (which == 1 ? r1 : r2);
#pragma unroll
    for (int pass = 0; pass < TS / SPP; ++pass) {
      const int sl = sl0 + pass * SPP;
      const int32_t id = ids[sl];
      uint4 val = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        int l = 0;
        while (l < lvl_top && id >= lv.off[l + 1]) ++l;
        const int64_t j = id - lv.off[l];
        if (l == 0) {
          load8_bf16(x + (b * lv.N + j) * row + h * D + g * 8, val);
        } else {
          load8_bf16(px + (b * lv.P1 + lv.poff[l] + j) * row + h * D + g * 8, val);
        }
      }
      *reinterpret_cast<uint4*>(ro + (bh * Sp + s0 + sl) * D + g * 8) = val;
    }
  }
}

template <int D, typename Tin, typename Tpool>
hipError_t gather_dispatch(const Levels& lv, int64_t Sp, const void* const x[3],
                           const void* const px[3], const int32_t* gmap, void* const rows[3],
                           hipStream_t st) {
  dim3 grid(static_cast<unsigned>(Sp / 64 * lv.B * lv.H));
  hipLaunchKernelGGL((gather_kernel<D, Tin, Tpool>), grid, dim3(256), 0, st, lv, Sp,
                     static_cast<const Tin*>(x[0]), static_cast<const Tin*>(x[1]),
                     static_cast<const Tin*>(x[2]), static_cast<const Tpool*>(px[0]),
                     static_cast<const Tpool*>(px[1]), static_cast<const Tpool*>(px[2]), gmap,
                     static_cast<uint16_t*>(rows[0]), static_cast<uint16_t*>(rows[1]),
                     static_cast<uint16_t*>(rows[2]));
  return hipGetLastError();
}

template <int D>
hipError_t gather_d(const Levels& lv, int64_t Sp, int32_t in_f32, const void* const x[3],
                    const void* const px[3], int32_t pooled_f32, const int32_t* gmap,
                    void* const rows[3], hipStream_t st) {
  if (in_f32)
    return pooled_f32 ? gather_dispatch<D, float, float>(lv, Sp, x, px, gmap, rows, st)
                      : gather_dispatch<D, float, uint16_t>(lv, Sp, x, px, gmap, rows, st);
  return pooled_f32 ? gather_dispatch<D, uint16_t, float>(lv, Sp, x, px, gmap, rows, st)
                    : gather_dispatch<D, uint16_t, uint16_t>(lv, Sp, x, px, gmap, rows, st);
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ x,
                                                      uint16_t* __restrict__ y, int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  uint4 u;
  load8_bf16(x + i * 8, u);
  *reinterpret_cast<uint4*>(y + i * 8) = u;
}

}  // namespace

hipError_t launch_build_map(const Levels& lv, const int32_t* sel, int32_t* gmap, int32_t* inv,
                            hipStream_t st) {
  const int64_t Sp = padded_len(lv.S);
  const int64_t ninv = lv.B * lv.H * lv.P;
  const int64_t nthreads = (ninv + 3) / 4;
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256),
                     0, st, inv, ninv, -1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>((Sp + 255) / 256), static_cast<unsigned>(lv.B * lv.H));
  hipLaunchKernelGGL(map_kernel, grid, dim3(256), 0, st, lv, sel, gmap, inv, Sp);
  return hipGetLastError();
}

hipError_t launch_gather(const Levels& lv, int32_t in_f32, const void* x[3], const void* px[3],
                         int32_t pooled_f32, const int32_t* gmap, void* const rows[3],
                         hipStream_t st) {
  const int64_t Sp = padded_len(lv.S);
  if (lv.D == 64) return gather_d<64>(lv, Sp, in_f32, x, px, pooled_f32, gmap, rows, st);
  return gather_d<128>(lv, Sp, in_f32, x, px, pooled_f32, gmap, rows, st);
}

hipError_t launch_to_bf16(const float* x, void* y, int64_t n, hipStream_t st) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0,
                     st, x, static_cast<uint16_t*>(y), n8);
  return hipGetLastError();
}

}  // namespace lh
