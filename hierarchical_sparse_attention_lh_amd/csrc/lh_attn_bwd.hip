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
//     Q^T and dO^T come pre-transposed in the swap23 order those operands need.
//   * query pass (dQ): workgroup = 128 queries (4 waves x 32), the forward's layout:
//     S^T = K Q^T, dP^T = V dO^T, dS^T feeds dQ^T = K^T dS^T as the B operand.
// The query pass recomputes S and dP (two extra products) instead of accumulating dQ with
// atomics across key workgroups; the result is bitwise reproducible.  Tiles are staged with
// direct global->LDS loads into XOR-swizzled rows (double-buffered); only diagonal and
// ragged-tail tiles evaluate the causal mask.  P and dS enter every
// product as a bf16 hi/lo pair (two MFMAs each): with single bf16 operands the gradients'
// error under cancellation exceeds their own output rounding several times over.
#include <type_traits>

#include "lh_internal.h"
#include "lh_mfma.h"

namespace lh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------- key pass
template <int D, int BQ>
__device__ __forceinline__ void attn_bwd_kv_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ qt,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ doutt,
    float* __restrict__ dk, float* __restrict__ dv, int S, int Sp, int64_t BH, float scale,
    float sl2) {
  constexpr int BK = 128, NB = BQ / 32;  // NB blocks of 32 queries per tile
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t ds_[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t qts[2][D * BQ];
  __shared__ __attribute__((aligned(16))) uint16_t dts[2][D * BQ];
  __shared__ __attribute__((aligned(16))) float ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float dl[2][BQ];

  const int nkt = Sp / BK;
  const int64_t item = xcd_item(blockIdx.x, BH * nkt);
  const int64_t bh = item / nkt;
  const int ktile = static_cast<int>(item % nkt);  // small key tiles have the most work: first
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int K0 = ktile * BK;
  const int kw = K0 + wave * 32;  // wave's first key
  const int mykey = kw + lq;

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
    // -V: the dP product then accumulates Delta - dP on top of Delta (see tile)
    vreg[kk] = as_bf16x8(__builtin_bit_cast(u32x4, ld_op16(v + (bh * Sp + mykey) * D +
                                                           16 * kk + hl * 8)) ^
                         0x80008000u);
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) {
    dkacc[d2] = zero16();
    dvacc[d2] = zero16();
  }

  const int qt0 = K0 / BQ;
  const int nqt = (S + BQ - 1) / BQ;

  auto stage = [&](int t, int buf) {
    const int q0 = t * BQ;
    stage_tile<BQ, D, 256>(qb + static_cast<int64_t>(q0) * D, D, qs[buf], tid);
    stage_tile<BQ, D, 256>(db_ + static_cast<int64_t>(q0) * D, D, ds_[buf], tid);
    stage_tile<D, BQ, 256>(qtb + q0, Sp, qts[buf], tid);
    stage_tile<D, BQ, 256>(dtb + q0, Sp, dts[buf], tid);
    if (wave == 0 && lane < BQ) stage_f32x64(lb + q0, ls[buf], lane);
    if (wave == 1 && lane < BQ) stage_f32x64(dlb + q0, dl[buf], lane);
  };

  auto tile = [&](auto masked, int t, int buf) {
    const int q0 = t * BQ;
    // The C rows of a lane are queries b2*32 + g*8 + (l/32)*4 + [0..3] (g = r/4): four float4
    // reads give a lane its 16 per-row values of lse or Delta in register order.
    f32x16 sacc[NB], pacc[NB];
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) {
      sacc[b2] = zero16();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(&dl[buf][b2 * 32 + g * 8 + hl * 4]);
        pacc[b2][4 * g] = d4.x;
        pacc[b2][4 * g + 1] = d4.y;
        pacc[b2][4 * g + 2] = d4.z;
        pacc[b2][4 * g + 3] = d4.w;
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(lds_op<D>(qs[buf], b2 * 32 + lq, 2 * kk + hl), kreg[kk], sacc[b2]);
        pacc[b2] = mfma32(lds_op<D>(ds_[buf], b2 * 32 + lq, 2 * kk + hl), vreg[kk], pacc[b2]);
      }
    }
    // pacc now holds Delta - dP, so p * pacc = -dS (the sign is folded into the final scale)
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = b2 * 32 + g * 8 + hl * 4;  // 4 consecutive local queries
        const float4 l4 = *reinterpret_cast<const float4*>(&ls[buf][qi]);
        const float lv4[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -lv4[u]));
          if constexpr (decltype(masked)::value) {
            const int qa = q0 + qi + u;
            if (qa < mykey || qa >= S) p = 0.f;
          }
          sacc[b2][r] = p;
          pacc[b2][r] = p * pacc[b2][r];
        }
      }
#pragma unroll
    for (int t4 = 0; t4 < 2 * NB; ++t4) {
      bf16x8 ph, pl, sh, sl;
      c_to_op2(sacc[t4 >> 1], t4 & 1, ph, pl);
      c_to_op2(pacc[t4 >> 1], t4 & 1, sh, sl);
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) {
        const bf16x8 ao = lds_op<BQ>(dts[buf], d2 * 32 + lq, 2 * t4 + hl);
        const bf16x8 aq = lds_op<BQ>(qts[buf], d2 * 32 + lq, 2 * t4 + hl);
        dvacc[d2] = mfma32(ao, pl, dvacc[d2]);
        dvacc[d2] = mfma32(ao, ph, dvacc[d2]);
        dkacc[d2] = mfma32(aq, sl, dkacc[d2]);
        dkacc[d2] = mfma32(aq, sh, dkacc[d2]);
      }
    }
  };

  if (qt0 < nqt) stage(qt0, 0);
  wait_vmem();
  __syncthreads();
  for (int t = qt0; t < nqt; ++t) {
    const int buf = (t - qt0) & 1;
    if (t + 1 < nqt) stage(t + 1, buf ^ 1);
    const int q0 = t * BQ;
    if (q0 < kw + 31 || q0 + BQ > S)
      tile(std::true_type{}, t, buf);
    else
      tile(std::false_type{}, t, buf);
    wait_vmem();
    __syncthreads();
  }

  float* dkr = dk + (bh * Sp + mykey) * D;
  float* dvr = dv + (bh * Sp + mykey) * D;
  const bool live = mykey < S;
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float ns = -scale;  // dkacc holds -dS^T Q
      float4 a = make_float4(dkacc[d2][4 * g] * ns, dkacc[d2][4 * g + 1] * ns,
                             dkacc[d2][4 * g + 2] * ns, dkacc[d2][4 * g + 3] * ns);
      float4 b = make_float4(dvacc[d2][4 * g], dvacc[d2][4 * g + 1], dvacc[d2][4 * g + 2],
                             dvacc[d2][4 * g + 3]);
      if (!live) a = b = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(dkr + d2 * 32 + g * 8 + hl * 4) = a;
      *reinterpret_cast<float4*>(dvr + d2 * 32 + g * 8 + hl * 4) = b;
    }
}

// -------------------------------------------------------------------------- query pass
template <int D>
__device__ __forceinline__ void attn_bwd_q_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, float* __restrict__ dq, int S, int Sp, int64_t BH,
    float scale, float sl2) {
  constexpr int BM = 128, BN = 64;
  __shared__ __attribute__((aligned(16))) uint16_t ks0[BN * D], ks1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[BN * D], vs1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t kts0[D * BN], kts1[D * BN];

  const int nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, BH * nqt);
  const int64_t bh = item / nqt;
  const int qtile = nqt - 1 - static_cast<int>(item % nqt);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int Q0 = qtile * BM;
  const int qw = Q0 + wave * 32;
  const int myq = qw + lq;

  const uint16_t* kb = k + bh * Sp * D;
  const uint16_t* vb = v + bh * Sp * D;
  const uint16_t* ktb = kt + bh * D * Sp;

  bf16x8 qreg[D / 16], oreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qreg[kk] = ld_op16(q + (bh * Sp + myq) * D + 16 * kk + hl * 8);
    oreg[kk] = ld_op16(dout + (bh * Sp + myq) * D + 16 * kk + hl * 8);
  }
  const float l2 = lse[bh * Sp + myq];  // base-2 log-sum-exp
  const float dlt = delta[bh * Sp + myq];

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) dqacc[d2] = zero16();

  const int kend = S < Q0 + BM ? S : Q0 + BM;
  const int nkt = (kend + BN - 1) / BN;

  auto stage = [&](int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const int k0 = t * BN;
    stage_tile<BN, D, 256>(kb + static_cast<int64_t>(k0) * D, D, B1 ? ks1 : ks0, tid);
    stage_tile<BN, D, 256>(vb + static_cast<int64_t>(k0) * D, D, B1 ? vs1 : vs0, tid);
    stage_tile<D, BN, 256>(ktb + k0, Sp, B1 ? kts1 : kts0, tid);
  };

  auto tile = [&](auto masked, int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const uint16_t* ksb = B1 ? ks1 : ks0;
    const uint16_t* vsb = B1 ? vs1 : vs0;
    const uint16_t* ktsb = B1 ? kts1 : kts0;
    const int k0 = t * BN;
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      sacc[b2] = zero16();
      pacc[b2] = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(lds_op<D>(ksb, b2 * 32 + lq, 2 * kk + hl), qreg[kk], sacc[b2]);
        pacc[b2] = mfma32(lds_op<D>(vsb, b2 * 32 + lq, 2 * kk + hl), oreg[kk], pacc[b2]);
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -l2));
        if constexpr (decltype(masked)::value) {
          const int key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
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
        const bf16x8 a = lds_op<BN>(ktsb, d2 * 32 + lq, 2 * t4 + hl);
        dqacc[d2] = mfma32(a, sl, dqacc[d2]);
        dqacc[d2] = mfma32(a, sh, dqacc[d2]);
      }
    }
  };

  auto step = [&](int t, auto bufc) {
    if (t + 1 < nkt) stage(t + 1, std::integral_constant<bool, !decltype(bufc)::value>{});
    const int k0 = t * BN;
    if (k0 + BN - 1 > qw || k0 + BN > S)
      tile(std::true_type{}, t, bufc);
    else
      tile(std::false_type{}, t, bufc);
    wait_vmem();
    __syncthreads();
  };
  stage(0, std::false_type{});
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    step(t, std::false_type{});
    if (t + 1 < nkt) step(t + 1, std::true_type{});
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


// D = 64 fits two waves per SIMD in both passes (no AGPR shuffling, no spills); D = 128
// keeps the compiler's default.
#define LH_KV_ARGS                                                                          \
  const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,                          \
      const uint16_t *__restrict__ v, const uint16_t *__restrict__ qt,                     \
      const float *__restrict__ lse, const float *__restrict__ delta,                      \
      const uint16_t *__restrict__ dout, const uint16_t *__restrict__ doutt,               \
      float *__restrict__ dk, float *__restrict__ dv, int S, int Sp, int64_t BH,           \
      float scale, float sl2
#define LH_Q_ARGS                                                                           \
  const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,                          \
      const uint16_t *__restrict__ v, const uint16_t *__restrict__ kt,                     \
      const float *__restrict__ lse, const float *__restrict__ delta,                      \
      const uint16_t *__restrict__ dout, float *__restrict__ dq, int S, int Sp, int64_t BH, \
      float scale, float sl2

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_bwd_kv_d64(LH_KV_ARGS) {
  attn_bwd_kv_body<64, 64>(q, k, v, qt, lse, delta, dout, doutt, dk, dv, S, Sp, BH, scale,
                           sl2);
}
__global__ __launch_bounds__(256) void attn_bwd_kv_d128(LH_KV_ARGS) {
  attn_bwd_kv_body<128, 32>(q, k, v, qt, lse, delta, dout, doutt, dk, dv, S, Sp, BH, scale,
                            sl2);
}
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_bwd_q_d64(LH_Q_ARGS) {
  attn_bwd_q_body<64>(q, k, v, kt, lse, delta, dout, dq, S, Sp, BH, scale, sl2);
}
__global__ __launch_bounds__(256) void attn_bwd_q_d128(LH_Q_ARGS) {
  attn_bwd_q_body<128>(q, k, v, kt, lse, delta, dout, dq, S, Sp, BH, scale, sl2);
}
#undef LH_KV_ARGS
#undef LH_Q_ARGS

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
  const int s32 = static_cast<int>(S), sp32 = static_cast<int>(Sp);
  if (pass & 1) {
    if (D == 64)
      hipLaunchKernelGGL(attn_bwd_kv_d64, dim3(blocks), dim3(256), 0, st, Q, K, V, QT,
                         lse, delta, DO, DOT, dk, dv, s32, sp32, BH, scale, sl2);
    else
      hipLaunchKernelGGL(attn_bwd_kv_d128, dim3(blocks), dim3(256), 0, st, Q, K, V, QT,
                         lse, delta, DO, DOT, dk, dv, s32, sp32, BH, scale, sl2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pass & 2) {
    if (D == 64)
      hipLaunchKernelGGL(attn_bwd_q_d64, dim3(blocks), dim3(256), 0, st, Q, K, V, KT,
                         lse, delta, DO, dq, s32, sp32, BH, scale, sl2);
    else
      hipLaunchKernelGGL(attn_bwd_q_d128, dim3(blocks), dim3(256), 0, st, Q, K, V, KT,
                         lse, delta, DO, dq, s32, sp32, BH, scale, sl2);
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
