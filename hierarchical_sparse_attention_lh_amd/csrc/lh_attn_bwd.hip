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
//   * query pass (dQ): workgroup = 128 queries (4 waves x 32), the forward's layout, over
//     64-key tiles (32 at D = 128): S^T = K Q^T, dP^T = V dO^T, dS^T feeds dQ^T = K^T dS^T
//     as the B operand.
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
  // Each buffer is its own LDS object and every use names it statically (the loop below is
  // unrolled by two): the compiler can then tell that the direct loads filling one buffer do
  // not alias the reads of the other, and does not make a tile's first LDS read wait for the
  // next tile's loads.
  __shared__ __attribute__((aligned(16))) uint16_t qs0[BQ * D], qs1[BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t ds0[BQ * D], ds1[BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t qts0[D * BQ], qts1[D * BQ];
  __shared__ __attribute__((aligned(16))) uint16_t dts0[D * BQ], dts1[D * BQ];
  __shared__ __attribute__((aligned(16))) float ls0[BQ], ls1[BQ];
  __shared__ __attribute__((aligned(16))) float dl0[BQ], dl1[BQ];

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
  // per-lane operand offsets of the D = 64 tile (every operand row there holds 64 bf16)
  uint32_t loff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) loff[j] = lane_chunk_off<64>(lq, hl, j);

  auto stage = [&](int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const int q0 = t * BQ;
    stage_tile<BQ, D, 256>(qb + static_cast<int64_t>(q0) * D, D, B1 ? qs1 : qs0, tid);
    stage_tile<BQ, D, 256>(db_ + static_cast<int64_t>(q0) * D, D, B1 ? ds1 : ds0, tid);
    stage_tile<D, BQ, 256>(qtb + q0, Sp, B1 ? qts1 : qts0, tid);
    stage_tile<D, BQ, 256>(dtb + q0, Sp, B1 ? dts1 : dts0, tid);
    if (wave == 0 && lane < BQ) stage_f32x64(lb + q0, B1 ? ls1 : ls0, lane);
    if (wave == 1 && lane < BQ) stage_f32x64(dlb + q0, B1 ? dl1 : dl0, lane);
  };

  auto tile = [&](auto masked, int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const uint16_t* qsb = B1 ? qs1 : qs0;
    const uint16_t* dsb = B1 ? ds1 : ds0;
    const uint16_t* qtsb = B1 ? qts1 : qts0;
    const uint16_t* dtsb = B1 ? dts1 : dts0;
    const float* lsb = B1 ? ls1 : ls0;
    const float* dlb_ = B1 ? dl1 : dl0;
    const int q0 = t * BQ;
    // The C rows of a lane are queries b2*32 + g*8 + (l/32)*4 + [0..3] (g = r/4): four float4
    // reads give a lane its 16 per-row values of lse or Delta in register order.
    f32x16 sacc[NB], pacc[NB];
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) {
      sacc[b2] = zero16();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(&dlb_[b2 * 32 + g * 8 + hl * 4]);
        pacc[b2][4 * g] = d4.x;
        pacc[b2][4 * g + 1] = d4.y;
        pacc[b2][4 * g + 2] = d4.z;
        pacc[b2][4 * g + 3] = d4.w;
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(lds_op<D>(qsb, b2 * 32 + lq, 2 * kk + hl), kreg[kk], sacc[b2]);
        pacc[b2] = mfma32(lds_op<D>(dsb, b2 * 32 + lq, 2 * kk + hl), vreg[kk], pacc[b2]);
      }
    }
    // pacc now holds Delta - dP, so p * pacc = -dS (the sign is folded into the final scale)
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = b2 * 32 + g * 8 + hl * 4;  // 4 consecutive local queries
        const float4 l4 = *reinterpret_cast<const float4*>(&lsb[qi]);
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
        const bf16x8 ao = lds_op<BQ>(dtsb, d2 * 32 + lq, 2 * t4 + hl);
        const bf16x8 aq = lds_op<BQ>(qtsb, d2 * 32 + lq, 2 * t4 + hl);
        dvacc[d2] = mfma32(ao, pl, dvacc[d2]);
        dvacc[d2] = mfma32(ao, ph, dvacc[d2]);
        dkacc[d2] = mfma32(aq, sl, dkacc[d2]);
        dkacc[d2] = mfma32(aq, sh, dkacc[d2]);
      }
    }
  };

  // The same tile for D = 64 and 64 queries, laid out for the matrix cores: twelve groups of
  // four MFMAs (A: S and dP of one 32-query block, two k steps; V / K: the dV or dK update
  // of one 16-query chunk t4), each group carrying vector work whose inputs are complete:
  //   A00 -          A01 -            A10 b0 b1     A11 p0 d0     V0 p1   K0 d1
  //   V1 b2 b3       K1 p2 d2         V2 p3         K2 d3         V3 -    K3 -
  // (b = exp and dS of chunk t4, p / d = hi-lo split of P / dS of chunk t4).  A SIMD runs
  // one wave's vector instructions beside the other wave's MFMAs when both carry an even mix,
  // while vector work bunched between MFMA runs leaves the matrix core idle, so the layout is
  // fixed with scheduling barriers; the LDS operands of each group are read one group ahead.
  auto tile64 = [&](auto masked, int t, auto bufc) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool B1 = decltype(bufc)::value;
    const int q0 = t * BQ;
    const uint16_t* qsb = B1 ? qs1 : qs0;
    const uint16_t* dsb = B1 ? ds1 : ds0;
    const uint16_t* qtsb = B1 ? qts1 : qts0;
    const uint16_t* dtsb = B1 ? dts1 : dts0;
    const float* lsb = B1 ? ls1 : ls0;
    const float* dlb_ = B1 ? dl1 : dl0;
    f32x16 sacc[2], pacc[2];
    bf16x8 op[12][4];
    float4 lsv[2][4];
    bf16x8 ph[4], pl[4], sh[4], sl[4];
    // Every operand row here holds 64 bf16, so logical chunk 2j + l/32 of row 32m + lq sits at
    // byte 4096m + loff[j] of its tile.  The copies are opaque to the compiler, so the address
    // sums stay inside the loop and fold into instruction offsets instead of being hoisted
    // into dozens of live registers.
    uint32_t lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = loff[j];
      asm volatile("" : "+v"(lo[j]));
    }
    auto rd = [&](const uint16_t* tile_base, int m, int j) {
      return lds_at(tile_base, 4096 * m + lo[j]);
    };
    auto load_ops = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < 4) {
        constexpr int b2 = u >> 1, kh = u & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = 2 * kh + j;
          op[u][2 * j] = rd(qsb, b2, kk);
          op[u][2 * j + 1] = rd(dsb, b2, kk);
        }
      } else {
        constexpr int c = u - 4, t4 = c >> 1;
        const uint16_t* src = (c & 1) ? qtsb : dtsb;
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) op[u][d2] = rd(src, d2, t4);
      }
    };
    auto mfma_unit = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u < 4) {
        constexpr int b2 = u >> 1, kh = u & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = 2 * kh + j;
          sacc[b2] = mfma32(op[u][2 * j], kreg[kk], sacc[b2]);
          pacc[b2] = mfma32(op[u][2 * j + 1], vreg[kk], pacc[b2]);
        }
      } else if constexpr (((u - 4) & 1) == 0) {
        constexpr int t4 = (u - 4) >> 1;
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dvacc[d2] = mfma32(op[u][d2], pl[t4], dvacc[d2]);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dvacc[d2] = mfma32(op[u][d2], ph[t4], dvacc[d2]);
      } else {
        constexpr int t4 = (u - 4) >> 1;
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dkacc[d2] = mfma32(op[u][d2], sl[t4], dkacc[d2]);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dkacc[d2] = mfma32(op[u][d2], sh[t4], dkacc[d2]);
      }
    };
    auto load_ls = [&](int b2) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        lsv[b2][g] = *reinterpret_cast<const float4*>(&lsb[b2 * 32 + g * 8 + hl * 4]);
    };
    // P = exp2(S sl2 - lse) and p * (Delta - dP) for the 8 C registers of chunk t4
    auto b_unit = [&](int t4) {
      const int b2 = t4 >> 1, half = t4 & 1;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * half + gg;
        const float lv4[4] = {lsv[b2][g].x, lsv[b2][g].y, lsv[b2][g].z, lsv[b2][g].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -lv4[u]));
          if constexpr (MASK) {
            const int qa = q0 + b2 * 32 + g * 8 + hl * 4 + u;
            if (qa < mykey || qa >= S) p = 0.f;
          }
          sacc[b2][r] = p;
          pacc[b2][r] = p * pacc[b2][r];
        }
      }
    };
    auto sp_unit = [&](int t4) { c_to_op2(sacc[t4 >> 1], t4 & 1, ph[t4], pl[t4]); };
    auto sd_unit = [&](int t4) { c_to_op2(pacc[t4 >> 1], t4 & 1, sh[t4], sl[t4]); };
    // four {one MFMA, nv vector instructions} groups, then a fence
    auto layout = [&](auto nvc) {
      constexpr int nv = decltype(nvc)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using N0 = std::integral_constant<int, 0>;
    using N6 = std::integral_constant<int, 6>;
    using N12 = std::integral_constant<int, 12>;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    using I6 = std::integral_constant<int, 6>;
    using I7 = std::integral_constant<int, 7>;
    using I8 = std::integral_constant<int, 8>;
    using I9 = std::integral_constant<int, 9>;
    using I10 = std::integral_constant<int, 10>;
    using I11 = std::integral_constant<int, 11>;

    // dP accumulators start at Delta (rows in C-register order), score accumulators at 0;
    // block 1's seed is read just before its first MFMA group
    auto seed = [&](int b2) {
      sacc[b2] = zero16();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(&dlb_[b2 * 32 + g * 8 + hl * 4]);
        pacc[b2][4 * g] = d4.x;
        pacc[b2][4 * g + 1] = d4.y;
        pacc[b2][4 * g + 2] = d4.z;
        pacc[b2][4 * g + 3] = d4.w;
      }
    };
    seed(0);
    load_ops(I0{});
    __builtin_amdgcn_sched_barrier(0);
    load_ops(I1{});
    mfma_unit(I0{});
    layout(N0{});
    load_ops(I2{});
    seed(1);
    load_ls(0);
    mfma_unit(I1{});
    layout(N0{});
    load_ops(I3{});
    mfma_unit(I2{});
    b_unit(0);
    b_unit(1);
    layout(N12{});
    load_ops(I4{});
    mfma_unit(I3{});
    sp_unit(0);
    sd_unit(0);
    layout(N12{});
    load_ops(I5{});
    load_ls(1);
    mfma_unit(I4{});
    sp_unit(1);
    layout(N6{});
    load_ops(I6{});
    mfma_unit(I5{});
    sd_unit(1);
    layout(N6{});
    load_ops(I7{});
    mfma_unit(I6{});
    b_unit(2);
    b_unit(3);
    layout(N12{});
    load_ops(I8{});
    mfma_unit(I7{});
    sp_unit(2);
    sd_unit(2);
    layout(N12{});
    load_ops(I9{});
    mfma_unit(I8{});
    sp_unit(3);
    layout(N6{});
    load_ops(I10{});
    mfma_unit(I9{});
    sd_unit(3);
    layout(N6{});
    load_ops(I11{});
    mfma_unit(I10{});
    layout(N0{});
    mfma_unit(I11{});
    layout(N0{});
  };

  auto step = [&](int t, auto bufc) {
    if (t + 1 < nqt) stage(t + 1, std::integral_constant<bool, !decltype(bufc)::value>{});
    const int q0 = t * BQ;
    if constexpr (D == 64 && BQ == 64) {
      if (q0 < kw + 31 || q0 + BQ > S)
        tile64(std::true_type{}, t, bufc);
      else
        tile64(std::false_type{}, t, bufc);
    } else {
      if (q0 < kw + 31 || q0 + BQ > S)
        tile(std::true_type{}, t, bufc);
      else
        tile(std::false_type{}, t, bufc);
    }
    wait_vmem();
    __syncthreads();
  };
  if (qt0 < nqt) stage(qt0, std::false_type{});
  wait_vmem();
  __syncthreads();
  for (int t = qt0; t < nqt; t += 2) {
    step(t, std::false_type{});
    if (t + 1 < nqt) step(t + 1, std::true_type{});
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
template <int D, int BN>
__device__ __forceinline__ void attn_bwd_q_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const uint16_t* __restrict__ dout, float* __restrict__ dq, int S, int Sp, int64_t BH,
    float scale, float sl2) {
  constexpr int BM = 128, NBK = BN / 32;  // NBK blocks of 32 keys per tile
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
  // per-lane operand offsets: K / V rows (D elements) for k step kk, K^T rows (BN elements)
  // for 16-key chunk t4; row block m adds 64 * row length * m bytes
  uint32_t koff[D / 16], toff[BN / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) koff[j] = lane_chunk_off<D>(lq, hl, j);
#pragma unroll
  for (int j = 0; j < BN / 16; ++j) toff[j] = lane_chunk_off<BN>(lq, hl, j);

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
    // opaque copies: the address sums stay in the loop and fold into instruction offsets
    // instead of being hoisted into one live register per read
    uint32_t ko[D / 16], to[BN / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      ko[j] = koff[j];
      asm volatile("" : "+v"(ko[j]));
    }
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) {
      to[j] = toff[j];
      asm volatile("" : "+v"(to[j]));
    }
    f32x16 sacc[NBK], pacc[NBK];
#pragma unroll
    for (int b2 = 0; b2 < NBK; ++b2) {
      sacc[b2] = zero16();
      pacc[b2] = zero16();
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc[b2] = mfma32(lds_at(ksb, b2 * 64 * D + ko[kk]), qreg[kk], sacc[b2]);
        pacc[b2] = mfma32(lds_at(vsb, b2 * 64 * D + ko[kk]), oreg[kk], pacc[b2]);
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < NBK; ++b2)
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
    for (int t4 = 0; t4 < 2 * NBK; ++t4) {
      bf16x8 sh, sl;
      c_to_op2(pacc[t4 >> 1], t4 & 1, sh, sl);
#pragma unroll
      for (int d2 = 0; d2 < D / 32; ++d2) {
        const bf16x8 a = lds_at(ktsb, d2 * 64 * BN + to[t4]);
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

// Occupancy: at D = 64 both passes run two waves per SIMD (no AGPR traffic, no spills).  At
// D = 128 the query pass fits two waves with 32-key tiles (236 VGPRs; 8 % faster than 64-key
// tiles at one wave), while the key pass (128 accumulator and 64 K/V registers per lane)
// keeps one wave with AGPR accumulators.
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
  attn_bwd_q_body<64, 64>(q, k, v, kt, lse, delta, dout, dq, S, Sp, BH, scale, sl2);
}
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attn_bwd_q_d128(LH_Q_ARGS) {
  attn_bwd_q_body<128, 32>(q, k, v, kt, lse, delta, dout, dq, S, Sp, BH, scale, sl2);
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
