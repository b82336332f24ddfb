// Causal softmax attention over the gathered sequence: the layer's one dense contraction.
//
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "核心方法：金字塔池化与“外部选择”", item 3, and [HE] news.hamidun.com, "Nous Research
// introduced Lighthouse Attention to accelerate LLM training", section "How Lighthouse
// Attention Works": the gathered subsequence goes through ordinary causal scaled dot-product
// attention.  The pages call a stock FlashAttention kernel on another vendor's GPU; this is
// this library's own kernel for gfx950.
//
// Design (bf16 MFMA, float32 accumulate, online softmax in base 2):
//   * workgroup = 4 waves = 128 queries; wave = 32 queries; key tiles of 64.
//   * The score tile is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so a
//     lane owns one query (C column) and 32 of the tile's 64 keys: the running max and sum
//     are per-lane scalars, combined with the partner lane (l ^ 32) by one cross-lane swap.
//   * O^T = V^T P^T: P leaves the C registers as a bf16 hi/lo pair (two MFMAs, ~16-bit
//     probabilities) and is the B operand directly; V^T is stored with the k order of that
//     operand (swap23 layout), so each A operand is one 16-byte LDS read and P never
//     touches LDS.
//   * K and V^T tiles are staged with direct global->LDS loads into XOR-swizzled LDS rows,
//     double-buffered: the next tile is in flight while the current one is multiplied.  The
//     two buffers are separate LDS objects and the loop is unrolled by two so each use names
//     its buffer statically; the compiler then does not make the current tile's LDS reads
//     wait for the next tile's loads (it only waits at the barrier).
//   * Only diagonal and ragged-tail tiles evaluate the causal mask.  The running max moves
//     only when a row's maximum grows by more than 8 (base 2), so most tiles skip the
//     rescale of the accumulators; the final division by the row sum is exact either way.
//   * The row sum is a per-tile tree sum added to a Kahan-compensated total: thousands of
//     small terms otherwise drift by ~1e-4 relative, which the backward's Delta amplifies.
//   * Software pipeline (D = 64): the score product of key tile t+1 is issued inside the
//     softmax of tile t, one MFMA per short group of vector instructions, so each wave offers
//     the SIMD an even mix (one wave's vector work runs beside the other wave's MFMAs;
//     bunched vector work leaves the matrix core idle).  At D = 128 the pipeline's registers
//     would force one wave per SIMD, and the plain loop at two waves is faster.
//   * Workgroups are mapped XCD-aware (one contiguous range of heads per XCD), heavy
//     (diagonal-far) query tiles first.
#include <type_traits>

#include "lh_internal.h"
#include "lh_mfma.h"

namespace lh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;  // base-2 growth of the row max tolerated before a rescale

template <int D, bool PIPE>
__device__ __forceinline__ void attn_fwd_body(const uint16_t* __restrict__ q,
                                              const uint16_t* __restrict__ k,
                                              const uint16_t* __restrict__ vt,
                                              float* __restrict__ o, float* __restrict__ lse,
                                              int S, int Sp, int64_t BH, float sl2) {
  constexpr int BM = 128, BN = 64;
  __shared__ __attribute__((aligned(16))) uint16_t ks0[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t ks1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[D * BN];
  __shared__ __attribute__((aligned(16))) uint16_t vs1[D * BN];

  const int nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, BH * nqt);
  const int64_t bh = item / nqt;
  const int qt = nqt - 1 - static_cast<int>(item % nqt);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int myq = qw + lq;

  const uint16_t* kb = k + bh * Sp * D;
  const uint16_t* vb = vt + bh * D * Sp;

  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qreg[kk] = ld_op16(q + (bh * Sp + myq) * D + 16 * kk + hl * 8);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f, l_cmp = 0.f;

  const int kend = S < q0 + BM ? S : q0 + BM;
  const int nkt = (kend + BN - 1) / BN;

  auto stage_k = [&](int t, auto bufc) {
    stage_tile<BN, D, 256>(kb + static_cast<int64_t>(t) * BN * D, D,
                           decltype(bufc)::value ? ks1 : ks0, tid);
  };
  auto stage_v = [&](int t, auto bufc) {
    stage_tile<D, BN, 256>(vb + t * BN, Sp, decltype(bufc)::value ? vs1 : vs0, tid);
  };

  // S^T of one key tile: 32 keys x 32 queries per C block, two blocks.
  auto scores = [&](f32x16 (&sacc)[2], auto bufc) {
    const uint16_t* ksb = decltype(bufc)::value ? ks1 : ks0;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      sacc[b2] = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        sacc[b2] = mfma32(lds_op<D>(ksb, b2 * 32 + lq, 2 * kk + hl), qreg[kk], sacc[b2]);
    }
  };

  // Online softmax of score tile t and its P V^T product, with the score product of tile t+1
  // (into nxt, from K buffer !odd) woven into the same instruction stream.  The SIMD overlaps
  // one wave's vector instructions with the other wave's MFMAs best when neither stream
  // bunches, so the code is laid out as short chunks of one MFMA plus some vector work, and
  // sched_barrier keeps the compiler from regrouping them.
  auto soft_pv = [&](auto masked, int t, f32x16 (&sacc)[2], f32x16 (&nxt)[2], auto par) {
    constexpr bool odd = decltype(par)::value;
    const uint16_t* vsb = odd ? vs1 : vs0;
    const uint16_t* ksn = odd ? ks0 : ks1;
    // operands of both products; the LDS latency hides behind the row max
    bf16x8 ka[2][D / 16], va[4][D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) ka[b2][kk] = lds_op<D>(ksn, b2 * 32 + lq, 2 * kk + hl);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        va[t4][db] = lds_op<BN>(vsb, db * 32 + lq, 2 * t4 + hl);
    if constexpr (decltype(masked)::value) {
      const int k0 = t * BN;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key > myq || key >= S) sacc[b2][r] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b2][r]);
    mx = pair_max(mx) * sl2;
    const bool grow = mx > m_run + kSlack;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      l_run *= alpha;
      l_cmp *= alpha;
      m_run = m_new;
    }
    // score MFMAs of tile t+1, each with a quarter of the exponentials of tile t behind it
    constexpr int NS = 2 * (D / 16);  // score MFMAs per tile
    constexpr int EPC = 32 / NS;       // exponentials per chunk
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) nxt[b2] = zero16();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int kk = i >> 1, b2 = i & 1;
      nxt[b2] = mfma32(ka[b2][kk], qreg[kk], nxt[b2]);
#pragma unroll
      for (int u = 0; u < EPC; ++u) {
        const int e = i * EPC + u, eb = e >> 4, er = e & 15;
        sacc[eb][er] = __builtin_amdgcn_exp2f(fmaf(sacc[eb][er], sl2, -m_run));
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2 * EPC, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P V^T: the split of chunk t4 + 1 and the row sum run behind the MFMAs of chunk t4
    bf16x8 ph[4], pl[4];
    c_to_op2(sacc[0], 0, ph[0], pl[0]);
    float part[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = sacc[0][r] + sacc[1][r];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32(va[t4][db], pl[t4], oacc[db]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32(va[t4][db], ph[t4], oacc[db]);
      if (t4 < 3) c_to_op2(sacc[(t4 + 1) >> 1], (t4 + 1) & 1, ph[t4 + 1], pl[t4 + 1]);
      if (t4 == 0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) part[r] += part[r + 8];
      } else if (t4 == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) part[r] += part[r + 4];
      } else if (t4 == 2) {
        part[0] += part[2];
        part[1] += part[3];
        part[0] += part[1];
      } else {
        const float yk = part[0] - l_cmp;
        const float tk = l_run + yk;
        l_cmp = (tk - l_run) - yk;
        l_run = tk;
      }
#pragma unroll
      for (int i = 0; i < 2 * (D / 32); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline: while the softmax of tile t runs on the vector ALUs, the score
  // product of tile t+1 runs on the matrix cores.  LDS holds K(t+1) and V(t) during step t;
  // K(t+2) and V(t+1) are loaded into the buffers freed by step t-1.  At the last step the
  // score product reads a stale K buffer and its result is never used.
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto par) {
    constexpr bool odd = decltype(par)::value;
    if (t + 2 < nkt) stage_k(t + 2, std::integral_constant<bool, odd>{});
    if (t + 1 < nkt) stage_v(t + 1, std::integral_constant<bool, !odd>{});
    const int k0 = t * BN;
    if (k0 + BN - 1 > qw || k0 + BN > S)
      soft_pv(std::true_type{}, t, cur, nxt, par);
    else
      soft_pv(std::false_type{}, t, cur, nxt, par);
    wait_vmem();
    __syncthreads();
  };

  // Without the pipeline (D = 128): one key tile is S^T = K Q^T (two 32-key C blocks), the
  // online softmax, O^T += V^T P^T; two waves share each SIMD and one wave's softmax runs
  // beside the other's MFMAs.
  auto plain_tile = [&](auto masked, int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const uint16_t* ksb = B1 ? ks1 : ks0;
    const uint16_t* vsb = B1 ? vs1 : vs0;
    f32x16 sacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) sacc[b2] = zero16();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
        sacc[b2] = mfma32(lds_op<D>(ksb, b2 * 32 + lq, 2 * kk + hl), qreg[kk], sacc[b2]);
    if constexpr (decltype(masked)::value) {
      const int k0 = t * BN;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key > myq || key >= S) sacc[b2][r] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b2][r]);
    mx = pair_max(mx) * sl2;
    const bool grow = mx > m_run + kSlack;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      l_run *= alpha;
      l_cmp *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[b2][r] = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -m_run));
    float part[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = sacc[0][r] + sacc[1][r];
#pragma unroll
    for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
      for (int r = 0; r < w2; ++r) part[r] += part[r + w2];
    const float yk = part[0] - l_cmp;
    const float tk = l_run + yk;
    l_cmp = (tk - l_run) - yk;
    l_run = tk;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x8 ph, pl;
      c_to_op2(sacc[t4 >> 1], t4 & 1, ph, pl);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a = lds_op<BN>(vsb, db * 32 + lq, 2 * t4 + hl);
        oacc[db] = mfma32(a, pl, oacc[db]);
        oacc[db] = mfma32(a, ph, oacc[db]);
      }
    }
  };

  auto plain_step = [&](int t, auto bufc) {
    if (t + 1 < nkt) {
      stage_k(t + 1, std::integral_constant<bool, !decltype(bufc)::value>{});
      stage_v(t + 1, std::integral_constant<bool, !decltype(bufc)::value>{});
    }
    const int k0 = t * BN;
    if (k0 + BN - 1 > qw || k0 + BN > S)
      plain_tile(std::true_type{}, t, bufc);
    else
      plain_tile(std::false_type{}, t, bufc);
    wait_vmem();
    __syncthreads();
  };
  if constexpr (PIPE) {
    f32x16 sa[2], sb[2];
    stage_k(0, std::false_type{});
    stage_v(0, std::false_type{});
    if (nkt > 1) stage_k(1, std::true_type{});
    wait_vmem();
    __syncthreads();
    scores(sa, std::false_type{});
    __syncthreads();  // K(0)'s buffer is refilled by the first step
    for (int t = 0; t < nkt; t += 2) {
      step(t, sa, sb, std::false_type{});
      if (t + 1 < nkt) step(t + 1, sb, sa, std::true_type{});
    }
  } else {
    stage_k(0, std::false_type{});
    stage_v(0, std::false_type{});
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < nkt; t += 2) {
      plain_step(t, std::false_type{});
      if (t + 1 < nkt) plain_step(t + 1, std::true_type{});
    }
  }

  const float l_own = l_run - l_cmp;
  const float l_tot = pair_sum(l_own);
  const float inv_l = 1.0f / l_tot;
  float* orow = o + (bh * Sp + myq) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 val = make_float4(oacc[db][4 * g] * inv_l, oacc[db][4 * g + 1] * inv_l,
                                     oacc[db][4 * g + 2] * inv_l, oacc[db][4 * g + 3] * inv_l);
      *reinterpret_cast<float4*>(orow + db * 32 + g * 8 + hl * 4) = val;
    }
  if (hl == 0) lse[bh * Sp + myq] = m_run + log2f(l_tot);  // base-2 log-sum-exp
}

// Both run two waves per SIMD.  D = 64 uses the pipelined loop (~210 VGPRs); at D = 128 the
// pipelined loop would spill at two waves and runs 18 % slower at one, so D = 128 uses the
// plain loop (253 VGPRs).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_d64(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
             const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
             int S, int Sp, int64_t BH, float sl2) {
  attn_fwd_body<64, true>(q, k, vt, o, lse, S, Sp, BH, sl2);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_fwd_d128(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ vt, float* __restrict__ o, float* __restrict__ lse,
              int S, int Sp, int64_t BH, float sl2) {
  attn_fwd_body<128, false>(q, k, vt, o, lse, S, Sp, BH, sl2);
}

}  // namespace

hipError_t launch_attn_fwd(int64_t B, int64_t H, int64_t S, int32_t D, float scale,
                           const void* q, const void* k, const void* vt, float* o, float* lse,
                           hipStream_t st) {
  const int64_t Sp = padded_len(S);
  const int64_t BH = B * H;
  const unsigned blocks = static_cast<unsigned>(BH * (Sp / 128));
  const float sl2 = scale * kLog2e;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(vt);
  const int s32 = static_cast<int>(S), sp32 = static_cast<int>(Sp);
  if (D == 64)
    hipLaunchKernelGGL(attn_fwd_d64, dim3(blocks), dim3(256), 0, st, qq, kk, vv, o, lse,
                       s32, sp32, BH, sl2);
  else
    hipLaunchKernelGGL(attn_fwd_d128, dim3(blocks), dim3(256), 0, st, qq, kk, vv, o,
                       lse, s32, sp32, BH, sl2);
  return hipGetLastError();
}

}  // namespace lh
