// gfx950 MFMA building blocks shared by the attention kernels.
//
// v_mfma_f32_32x32x16_bf16 (one wave, 64 lanes): C[32x32] += A[32x16] * B[16x32].
//   A operand: lane l holds row (l % 32), k = (l / 32) * 8 + [0..7]   (8 bf16)
//   B operand: lane l holds col (l % 32), k = (l / 32) * 8 + [0..7]   (8 bf16)
//   C/D:       lane l, register r holds row (r / 4) * 8 + (l / 32) * 4 + (r % 4), col (l % 32)
// The k order inside one instruction is free as long as A and B agree, which is how the
// probability / gradient tiles are fed straight from C registers into the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// 16 bytes from LDS / global as an MFMA operand
__device__ __forceinline__ bf16x8 ld_op16(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded (to nearest even) to bf16 and packed, a in the low half.  Written as one
// vector conversion so it becomes a single two-source v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// C registers 8*half .. 8*half+7 of one 32x32 tile as a B (or A) operand: for lane l these
// are rows (half*16) + {0..3, 8..11} + (l/32)*4 of the tile, i.e. the k index (l/32)*8 + ii
// of the next product maps to tile row 16*half + (ii/4)*8 + (l/32)*4 + (ii%4).
// They are split into two bf16 operands with hi + lo = value to about 16 significant bits:
// hi is the value truncated to bf16 (exact), lo the remainder (exact in float32) rounded to
// bf16.  Probabilities and score gradients enter every product
// as this pair (two MFMAs), so their rounding stays far below the gradients' bf16 output
// rounding; a single bf16 operand (8 bits) is not accurate enough under cancellation.
__device__ __forceinline__ void c_to_op2(const f32x16& c, int half, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = c[8 * half + 2 * i], x1 = c[8 * half + 2 * i + 1];
    const uint32_t t0 = __float_as_uint(x0) & 0xffff0000u;
    const uint32_t t1 = __float_as_uint(x1) & 0xffff0000u;
    h[i] = (t0 >> 16) | t1;
    l[i] = pk_bf16(x0 - __uint_as_float(t0), x1 - __uint_as_float(t1));
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 16-byte MFMA operand at a byte offset into an LDS tile.
__device__ __forceinline__ bf16x8 lds_at(const uint16_t* tile, uint32_t byte_off) {
  return ld_op16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(tile) +
                                                   byte_off));
}

// Lanes l and l ^ 32 exchange a value with one v_permlane32_swap (no LDS round trip); the
// swap leaves {x[l], x[l ^ 32]} in every lane, so symmetric reductions need no select.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Map a linear block id to a work item so that each of the 8 XCDs (workgroups are handed
// to XCDs round-robin) receives one contiguous range of items; items of one head then run
// on one XCD and share its L2.
__device__ __forceinline__ int64_t xcd_item(int64_t bid, int64_t total) {
  const int64_t x = bid % 8, k = bid / 8;
  const int64_t per = total / 8, rem = total % 8;
  return x * per + (x < rem ? x : rem) + k;
}

}  // namespace lh
