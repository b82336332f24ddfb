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
//     probabilities) and is the B operand directly (the k order inside an instruction is
//     permuted identically on the V^T side, so P never touches LDS).  V^T comes
//     pre-transposed from the gather stage, so both A operands are plain 16-byte /
//     2 x 8-byte LDS reads.
//   * K and V^T tiles are double-buffered in LDS; the next tile's global loads are in flight
//     while the current tile is multiplied.
//   * Workgroups are mapped XCD-aware (one contiguous range of heads per XCD) and heavy
//     (diagonal-far) query tiles first.
#include "lh_internal.h"
#include "lh_mfma.h"

namespace lh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ vt,
                                                       float* __restrict__ o,
                                                       float* __restrict__ lse, int64_t S,
                                                       int64_t Sp, int64_t BH, float sl2) {
  constexpr int BM = 128, BN = 64;
  constexpr int KR = D + 8;   // K tile row stride in LDS (elements)
  constexpr int VR = BN + 8;  // V^T tile row stride in LDS
  constexpr int KG = D / 8, KPER = BN * KG / 256;
  constexpr int VG = BN / 8, VPER = D * VG / 256;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * KR];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][D * VR];

  const int64_t nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, BH * nqt);
  const int64_t bh = item / nqt;
  const int64_t qt = nqt - 1 - item % nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int64_t qw = qt * BM + wave * 32;
  const int64_t myq = qw + lq;

  const uint16_t* qb = q + bh * Sp * D;
  const uint16_t* kb = k + bh * Sp * D;
  const uint16_t* vb = vt + bh * D * Sp;

  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = ld_op16(qb + myq * D + 16 * kk + hl * 8);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  // running max (base-2 units) and the row sum; the sum is Kahan-compensated because
  // thousands of small probabilities are added to it (plain float32 summation drifts by
  // ~1e-4 relative at S ~ 1e4, which the backward's Delta = rowsum(dO * O) amplifies)
  float m_run = -INFINITY, l_run = 0.f, l_cmp = 0.f;

  const int64_t kend = S < (qt + 1) * BM ? S : (qt + 1) * BM;
  const int nkt = static_cast<int>((kend + BN - 1) / BN);

  u32x4 kreg[KPER], vreg[VPER];
  auto gload = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * BN;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int idx = tid + 256 * i, r = idx / KG, c = idx % KG;
      kreg[i] = *reinterpret_cast<const u32x4*>(kb + (k0 + r) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int idx = tid + 256 * i, r = idx / VG, c = idx % VG;
      vreg[i] = *reinterpret_cast<const u32x4*>(vb + r * Sp + k0 + c * 8);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int idx = tid + 256 * i, r = idx / KG, c = idx % KG;
      *reinterpret_cast<u32x4*>(&ks[buf][r * KR + c * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int idx = tid + 256 * i, r = idx / VG, c = idx % VG;
      *reinterpret_cast<u32x4*>(&vs[buf][r * VR + c * 8]) = vreg[i];
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);

    f32x16 sacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      sacc[b2] = zero16();
      const uint16_t* ka = &ks[buf][(b2 * 32 + lq) * KR + hl * 8];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc[b2] = mfma32(ld_op16(ka + 16 * kk), qreg[kk], sacc[b2]);
    }

    const int64_t k0 = static_cast<int64_t>(kt) * BN;
    if (k0 + BN - 1 > qw || k0 + BN > S) {
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key > myq || key >= S) sacc[b2][r] = -INFINITY;
        }
    }

    float mx = sacc[0][0];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[b2][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[b2][r] = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -m_new));
    float part[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = sacc[0][r] + sacc[1][r];
#pragma unroll
    for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
      for (int r = 0; r < w2; ++r) part[r] += part[r + w2];
    {
      l_run *= alpha;
      l_cmp *= alpha;
      const float yk = part[0] - l_cmp;
      const float tk = l_run + yk;
      l_cmp = (tk - l_run) - yk;
      l_run = tk;
    }

#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 ph, pl;
      c_to_op2(sacc[t >> 1], t & 1, ph, pl);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* va = &vs[buf][(db * 32 + lq) * VR + 16 * t + hl * 4];
        const bf16x8 a = ld_op8x2(va, va + 8);
        oacc[db] = mfma32(a, pl, oacc[db]);
        oacc[db] = mfma32(a, ph, oacc[db]);
      }
    }

    if (kt + 1 < nkt) swrite(buf ^ 1);
    __syncthreads();
  }

  const float l_own = l_run - l_cmp;
  const float l_tot = l_own + __shfl_xor(l_own, 32);
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
  if (hl == 0) lse[bh * Sp + myq] = m_run * kLn2 + __logf(l_tot);
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
  if (D == 64)
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(blocks), dim3(256), 0, st, qq, kk, vv, o, lse,
                       S, Sp, BH, sl2);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(blocks), dim3(256), 0, st, qq, kk, vv, o,
                       lse, S, Sp, BH, sl2);
  return hipGetLastError();
}

}  // namespace lh
