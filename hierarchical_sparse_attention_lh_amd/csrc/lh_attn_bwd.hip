// Backward of the causal attention over the gathered sequence.
//
// [EN] encorp.ai, "Услуги по внедряване на AI задават правилния въпрос за Lighthouse
// Attention", section "Как four-stage pipeline остава бърз, без да чупи градиентите?", and
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "深度洞察": gradients reach Q, K and V through the attention on the gathered values
// (the selection itself has none).
//
// With P = softmax rows (recomputed from the saved log-sum-exp) and Delta = rowsum(dO * O):
//   dV = P^T dO;  dP = dO V^T;  dS = P * (dP - Delta);  dQ = scale dS K;  dK = scale dS^T Q.
//
// Design: two deterministic passes, no atomics.
//   * key pass (dK, dV): workgroup = 128 keys (4 waves x 32); loops over 64-query tiles from
//     the diagonal down.  S = Q K^T and dP = dO V^T are computed with keys as the C column,
//     so P and dS leave the C registers as B operands of dV^T = dO^T P and dK^T = Q^T dS;
//     Q^T and dO^T tiles come pre-transposed from global memory.
//   * query pass (dQ): workgroup = 128 queries (4 waves x 32), the forward's layout:
//     S^T = K Q^T, dP^T = V dO^T, dS^T feeds dQ^T = K^T dS^T as the B operand.
// The query pass recomputes S and dP (two extra products) instead of accumulating dQ with
// atomics across key workgroups; the result is bitwise reproducible.  P and dS enter every
// product as a bf16 hi/lo pair (two MFMAs each): with single bf16 operands the gradients'
// error under cancellation exceeds their own output rounding several times over.
#include "lh_internal.h"
#include "lh_mfma.h"

namespace lh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------- key pass
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ qt,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ doutt,
    float* __restrict__ dk, float* __restrict__ dv, int64_t S, int64_t Sp, int64_t BH,
    float scale, float sl2) {
  constexpr int BK = 128, BQ = 64;
  constexpr int RR = D + 8;   // row-tile stride (elements)
  constexpr int TR = BQ + 8;  // transposed-tile stride
  constexpr int RG = D / 8, RPER = BQ * RG / 256;   // 16-byte loads per thread, row tiles
  constexpr int TG = BQ / 8, TPER = D * TG / 256;   // 16-byte loads per thread, transposed
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][BQ * RR];
  __shared__ __attribute__((aligned(16))) uint16_t ds_[2][BQ * RR];
  __shared__ __attribute__((aligned(16))) uint16_t qts[2][D * TR];
  __shared__ __attribute__((aligned(16))) uint16_t dts[2][D * TR];
  __shared__ __attribute__((aligned(16))) float ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float dl[2][BQ];

  const int64_t nkt = Sp / BK;
  const int64_t item = xcd_item(blockIdx.x, BH * nkt);
  const int64_t bh = item / nkt;
  const int64_t ktile = item % nkt;  // small key tiles have the most work: run them first
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int64_t K0 = ktile * BK;
  const int64_t kw = K0 + wave * 32;  // wave's first key
  const int64_t mykey = kw + lq;

  const uint16_t* qb = q + bh * Sp * D;
  const uint16_t* db_ = dout + bh * Sp * D;
  const uint16_t* qtb = qt + bh * D * Sp;
  const uint16_t* dtb = doutt + bh * D * Sp;
  const float* lb = lse + bh * Sp;
  const float* dlb = delta + bh * Sp;

  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kreg[kk] = ld_op16(k + (bh * Sp + mykey) * D + 16 * kk + hl * 8);
    vreg[kk] = ld_op16(v + (bh * Sp + mykey) * D + 16 * kk + hl * 8);
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) {
    dkacc[d2] = zero16();
    dvacc[d2] = zero16();
  }

  const int64_t qt0 = K0 / BQ;
  const int64_t nqt = (S + BQ - 1) / BQ;

  u32x4 rq[RPER], rd[RPER], tq[TPER], td[TPER];
  float rl = 0.f, rdl = 0.f;
  auto gload = [&](int64_t t) {
    const int64_t q0 = t * BQ;
#pragma unroll
    for (int i = 0; i < RPER; ++i) {
      const int idx = tid + 256 * i, r = idx / RG, c = idx % RG;
      rq[i] = *reinterpret_cast<const u32x4*>(qb + (q0 + r) * D + c * 8);
      rd[i] = *reinterpret_cast<const u32x4*>(db_ + (q0 + r) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < TPER; ++i) {
      const int idx = tid + 256 * i, r = idx / TG, c = idx % TG;
      tq[i] = *reinterpret_cast<const u32x4*>(qtb + r * Sp + q0 + c * 8);
      td[i] = *reinterpret_cast<const u32x4*>(dtb + r * Sp + q0 + c * 8);
    }
    if (tid < BQ) {
      rl = lb[q0 + tid] * kLog2e;
      rdl = dlb[q0 + tid];
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RPER; ++i) {
      const int idx = tid + 256 * i, r = idx / RG, c = idx % RG;
      *reinterpret_cast<u32x4*>(&qs[buf][r * RR + c * 8]) = rq[i];
      *reinterpret_cast<u32x4*>(&ds_[buf][r * RR + c * 8]) = rd[i];
    }
#pragma unroll
    for (int i = 0; i < TPER; ++i) {
      const int idx = tid + 256 * i, r = idx / TG, c = idx % TG;
      *reinterpret_cast<u32x4*>(&qts[buf][r * TR + c * 8]) = tq[i];
      *reinterpret_cast<u32x4*>(&dts[buf][r * TR + c * 8]) = td[i];
    }
    if (tid < BQ) {
      ls[buf][tid] = rl;
      dl[buf][tid] = rdl;
    }
  };

  if (qt0 < nqt) {
    gload(qt0);
    swrite(0);
  }
  __syncthreads();
  for (int64_t t = qt0; t < nqt; ++t) {
    const int buf = static_cast<int>((t - qt0) & 1);
    if (t + 1 < nqt) gload(t + 1);
    const int64_t q0 = t * BQ;

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      sacc[b2] = zero16();
      pacc[b2] = zero16();
      const uint16_t* qa = &qs[buf][(b2 * 32 + lq) * RR + hl * 8];
      const uint16_t* da = &ds_[buf][(b2 * 32 + lq) * RR + hl * 8];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(ld_op16(qa + 16 * kk), kreg[kk], sacc[b2]);
        pacc[b2] = mfma32(ld_op16(da + 16 * kk), vreg[kk], pacc[b2]);
      }
    }

    const bool edge = q0 < kw + 31 || q0 + BQ > S;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = b2 * 32 + g * 8 + hl * 4;  // 4 consecutive local queries
        const float4 l4 = *reinterpret_cast<const float4*>(&ls[buf][qi]);
        const float4 d4 = *reinterpret_cast<const float4*>(&dl[buf][qi]);
        const float lv4[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -lv4[u]));
          if (edge) {
            const int64_t qa = q0 + qi + u;
            if (qa < mykey || qa >= S) p = 0.f;
          }
          sacc[b2][r] = p;
          pacc[b2][r] = p * (pacc[b2][r] - dv4[u]);
        }
      }

#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x8 ph, pl, sh, sl;
      c_to_op2(sacc[t4 >> 1], t4 & 1, ph, pl);
      c_to_op2(pacc[t4 >> 1], t4 & 1, sh, sl);
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) {
        const uint16_t* da = &dts[buf][(d2 * 32 + lq) * TR + 16 * t4 + hl * 4];
        const uint16_t* qa = &qts[buf][(d2 * 32 + lq) * TR + 16 * t4 + hl * 4];
        const bf16x8 ao = ld_op8x2(da, da + 8), aq = ld_op8x2(qa, qa + 8);
        dvacc[d2] = mfma32(ao, pl, dvacc[d2]);
        dvacc[d2] = mfma32(ao, ph, dvacc[d2]);
        dkacc[d2] = mfma32(aq, sl, dkacc[d2]);
        dkacc[d2] = mfma32(aq, sh, dkacc[d2]);
      }
    }

    if (t + 1 < nqt) swrite(buf ^ 1);
    __syncthreads();
  }

  float* dkr = dk + (bh * Sp + mykey) * D;
  float* dvr = dv + (bh * Sp + mykey) * D;
  const bool live = mykey < S;
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 a = make_float4(dkacc[d2][4 * g] * scale, dkacc[d2][4 * g + 1] * scale,
                             dkacc[d2][4 * g + 2] * scale, dkacc[d2][4 * g + 3] * scale);
      float4 b = make_float4(dvacc[d2][4 * g], dvacc[d2][4 * g + 1], dvacc[d2][4 * g + 2],
                             dvacc[d2][4 * g + 3]);
      if (!live) a = b = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(dkr + d2 * 32 + g * 8 + hl * 4) = a;
      *reinterpret_cast<float4*>(dvr + d2 * 32 + g * 8 + hl * 4) = b;
    }
}

// -------------------------------------------------------------------------- query pass
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, float* __restrict__ dq, int64_t S, int64_t Sp,
    int64_t BH, float scale, float sl2) {
  constexpr int BM = 128, BN = 64;
  constexpr int RR = D + 8;
  constexpr int TR = BN + 8;
  constexpr int RG = D / 8, RPER = BN * RG / 256;
  constexpr int TG = BN / 8, TPER = D * TG / 256;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * RR];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BN * RR];
  __shared__ __attribute__((aligned(16))) uint16_t kts[2][D * TR];

  const int64_t nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, BH * nqt);
  const int64_t bh = item / nqt;
  const int64_t qtile = nqt - 1 - item % nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int64_t qw = qtile * BM + wave * 32;
  const int64_t myq = qw + lq;

  const uint16_t* kb = k + bh * Sp * D;
  const uint16_t* vb = v + bh * Sp * D;
  const uint16_t* ktb = kt + bh * D * Sp;

  bf16x8 qreg[D / 16], oreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qreg[kk] = ld_op16(q + (bh * Sp + myq) * D + 16 * kk + hl * 8);
    oreg[kk] = ld_op16(dout + (bh * Sp + myq) * D + 16 * kk + hl * 8);
  }
  const float l2 = lse[bh * Sp + myq] * kLog2e;
  const float dlt = delta[bh * Sp + myq];

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) dqacc[d2] = zero16();

  const int64_t kend = S < (qtile + 1) * BM ? S : (qtile + 1) * BM;
  const int nkt = static_cast<int>((kend + BN - 1) / BN);

  u32x4 rk[RPER], rv[RPER], tk[TPER];
  auto gload = [&](int t) {
    const int64_t k0 = static_cast<int64_t>(t) * BN;
#pragma unroll
    for (int i = 0; i < RPER; ++i) {
      const int idx = tid + 256 * i, r = idx / RG, c = idx % RG;
      rk[i] = *reinterpret_cast<const u32x4*>(kb + (k0 + r) * D + c * 8);
      rv[i] = *reinterpret_cast<const u32x4*>(vb + (k0 + r) * D + c * 8);
    }
#pragma unroll
    for (int i = 0; i < TPER; ++i) {
      const int idx = tid + 256 * i, r = idx / TG, c = idx % TG;
      tk[i] = *reinterpret_cast<const u32x4*>(ktb + r * Sp + k0 + c * 8);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RPER; ++i) {
      const int idx = tid + 256 * i, r = idx / RG, c = idx % RG;
      *reinterpret_cast<u32x4*>(&ks[buf][r * RR + c * 8]) = rk[i];
      *reinterpret_cast<u32x4*>(&vs[buf][r * RR + c * 8]) = rv[i];
    }
#pragma unroll
    for (int i = 0; i < TPER; ++i) {
      const int idx = tid + 256 * i, r = idx / TG, c = idx % TG;
      *reinterpret_cast<u32x4*>(&kts[buf][r * TR + c * 8]) = tk[i];
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();
  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nkt) gload(t + 1);
    const int64_t k0 = static_cast<int64_t>(t) * BN;

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      sacc[b2] = zero16();
      pacc[b2] = zero16();
      const uint16_t* ka = &ks[buf][(b2 * 32 + lq) * RR + hl * 8];
      const uint16_t* va = &vs[buf][(b2 * 32 + lq) * RR + hl * 8];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(ld_op16(ka + 16 * kk), qreg[kk], sacc[b2]);
        pacc[b2] = mfma32(ld_op16(va + 16 * kk), oreg[kk], pacc[b2]);
      }
    }
    const bool edge = k0 + BN - 1 > qw || k0 + BN > S;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -l2));
        if (edge) {
          const int64_t key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key > myq || key >= S) p = 0.f;
        }
        pacc[b2][r] = p * (pacc[b2][r] - dlt);
      }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x8 sh, sl;
      c_to_op2(pacc[t4 >> 1], t4 & 1, sh, sl);
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) {
        const uint16_t* ka = &kts[buf][(d2 * 32 + lq) * TR + 16 * t4 + hl * 4];
        const bf16x8 a = ld_op8x2(ka, ka + 8);
        dqacc[d2] = mfma32(a, sl, dqacc[d2]);
        dqacc[d2] = mfma32(a, sh, dqacc[d2]);
      }
    }
    if (t + 1 < nkt) swrite(buf ^ 1);
    __syncthreads();
  }

  float* dqr = dq + (bh * Sp + myq) * D;
  const bool live = myq < S;
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 a = make_float4(dqacc[d2][4 * g] * scale, dqacc[d2][4 * g + 1] * scale,
                             dqacc[d2][4 * g + 2] * scale, dqacc[d2][4 * g + 3] * scale);
      if (!live) a = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(dqr + d2 * 32 + g * 8 + hl * 4) = a;
    }
}

}  // namespace

hipError_t launch_attn_bwd_pass(int pass, int64_t B, int64_t H, int64_t S, int32_t D,
                                float scale, const void* q, const void* k, const void* v,
                                const void* qt, const void* kt, const float* lse,
                                const float* delta, const void* dout, const void* doutt,
                                float* dq, float* dk, float* dv, hipStream_t st) {
  const int64_t Sp = padded_len(S);
  const int64_t BH = B * H;
  const float sl2 = scale * kLog2e;
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* K = static_cast<const uint16_t*>(k);
  const auto* V = static_cast<const uint16_t*>(v);
  const auto* QT = static_cast<const uint16_t*>(qt);
  const auto* KT = static_cast<const uint16_t*>(kt);
  const auto* DO = static_cast<const uint16_t*>(dout);
  const auto* DOT = static_cast<const uint16_t*>(doutt);
  const unsigned blocks = static_cast<unsigned>(BH * (Sp / 128));
  if (pass & 1) {
    if (D == 64)
      hipLaunchKernelGGL(attn_bwd_kv_kernel<64>, dim3(blocks), dim3(256), 0, st, Q, K, V, QT,
                         lse, delta, DO, DOT, dk, dv, S, Sp, BH, scale, sl2);
    else
      hipLaunchKernelGGL(attn_bwd_kv_kernel<128>, dim3(blocks), dim3(256), 0, st, Q, K, V, QT,
                         lse, delta, DO, DOT, dk, dv, S, Sp, BH, scale, sl2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pass & 2) {
    if (D == 64)
      hipLaunchKernelGGL(attn_bwd_q_kernel<64>, dim3(blocks), dim3(256), 0, st, Q, K, V, KT,
                         lse, delta, DO, dq, S, Sp, BH, scale, sl2);
    else
      hipLaunchKernelGGL(attn_bwd_q_kernel<128>, dim3(blocks), dim3(256), 0, st, Q, K, V, KT,
                         lse, delta, DO, dq, S, Sp, BH, scale, sl2);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int64_t B, int64_t H, int64_t S, int32_t D, float scale,
                           const void* q, const void* k, const void* v, const void* qt,
                           const void* kt, const float* lse, const float* delta,
                           const void* dout, const void* doutt, float* dq, float* dk,
                           float* dv, hipStream_t st) {
  return launch_attn_bwd_pass(3, B, H, S, D, scale, q, k, v, qt, kt, lse, delta, dout, doutt, dq,
                              dk, dv, st);
}

}  // namespace lh
