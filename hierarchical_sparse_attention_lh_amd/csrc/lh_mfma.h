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

// ------------------------------------------------------------------------------------------
// Operand-friendly layouts.
//
// Transposed tensors ([.., D, Sp]) store sequence position s at column swap23(s): bits 2 and 3
// of s exchanged (an involution).  Within each group of 16 the stored order is
// 0-3, 8-11, 4-7, 12-15, which is exactly the k order in which a C tile leaves an MFMA as the
// next product's B operand (see c_to_op2): the matching A operand of lane l is then the single
// 16-byte chunk 2*t + (l/32) of the row instead of two 8-byte pieces.
__host__ __device__ __forceinline__ int64_t swap23(int64_t s) {
  return (s & ~int64_t(12)) | ((s & 4) << 1) | ((s & 8) >> 1);
}

// LDS tiles are unpadded rows whose 16-byte chunks are XOR-swizzled.  The LDS serves a
// 16-byte-per-lane read 16 lanes at a time from 64 four-byte banks, i.e. sixteen 16-byte bank
// groups; the operand reads have 16 consecutive lanes on 16 consecutive rows at one logical
// chunk, so the swizzle makes those 16 (row, chunk) pairs land in 16 different groups.  A
// 128-byte row (64 bf16) fills half a bank line, so rows 2j and 2j+1 share the XOR key j;
// a 256-byte row (128 bf16) fills a whole line and each of 16 rows gets its own key.
template <int ROW_ELEMS>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int CPR = ROW_ELEMS / 8;                // 16-byte chunks per row
  constexpr int RPL = CPR >= 16 ? 1 : 16 / CPR;     // rows per 256-byte bank line
  return chunk ^ ((row / RPL) % CPR);
}

// 16-byte MFMA operand: logical chunk `chunk` of `row` in a swizzled LDS tile.
template <int ROW_ELEMS>
__device__ __forceinline__ bf16x8 lds_op(const uint16_t* tile, int row, int chunk) {
  return ld_op16(tile + row * ROW_ELEMS + (swz<ROW_ELEMS>(row, chunk) << 3));
}

// Byte offset of logical chunk 2j + l/32 in row lq of a swizzled tile of ROW_ELEMS bf16 per
// row.  Row 32m + lq has row lq's XOR key (checked below), so its chunk sits
// 64 * ROW_ELEMS * m bytes further: one per-lane offset per k step serves every 32-row block
// of every tile of that shape, and the rest of the address is an instruction immediate.
template <int ROW_ELEMS>
__device__ __forceinline__ uint32_t lane_chunk_off(int lq, int hl, int j) {
  constexpr int CPR = ROW_ELEMS / 8, RPL = CPR >= 16 ? 1 : 16 / CPR;  // as in swz
  static_assert((32 / RPL) % CPR == 0, "rows lq and 32m + lq must share the XOR key");
  return static_cast<uint32_t>(lq * ROW_ELEMS * 2 + (swz<ROW_ELEMS>(lq, 2 * j + hl) << 4));
}

// 16-byte MFMA operand at a byte offset into an LDS tile.
__device__ __forceinline__ bf16x8 lds_at(const uint16_t* tile, uint32_t byte_off) {
  return ld_op16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(tile) +
                                                   byte_off));
}

// Stage ROWS x ROW_ELEMS bf16 (row stride `gstride` elements in global memory) into a swizzled
// LDS tile with gfx950 direct global->LDS loads: each wave instruction moves 64 x 16 bytes into
// 1 KB of contiguous LDS, so lane l fetches the global chunk that belongs at LDS chunk
// (instruction base + l).  No VGPRs hold the data; completion is tracked by vmcnt.  The lane's
// byte offset from the (uniform) tile start is 32-bit, so the loads take the scalar-base +
// 32-bit-offset form and keep no 64-bit address per lane; callers bound
// (ROWS - 1) * gstride + ROW_ELEMS below 2^31 elements.
template <int ROWS, int ROW_ELEMS, int NT>
__device__ __forceinline__ void stage_tile(const uint16_t* g, int gstride, uint16_t* lds,
                                           int tid) {
  constexpr int CPR = ROW_ELEMS / 8;        // 16-byte chunks per row
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % NT == 0, "tile must be a whole number of 16-byte loads per thread");
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < CHUNKS / NT; ++i) {
    const int base = (i * (NT / 64) + wave) * 64;  // first LDS chunk of this wave instruction
    const int lin = base + lane;
    const int row = lin / CPR, pc = lin % CPR;
    const int c = swz<ROW_ELEMS>(row, pc);
    uint32_t boff = static_cast<uint32_t>(row * gstride + c * 8) * 2u;
    asm volatile("" : "+v"(boff));  // opaque: not re-associated with the tile base and hoisted
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(g) + boff, lds + base * 8, 16,
                                     0, 0);
  }
}

// 64 floats into LDS with one wave instruction (4 bytes per lane).
__device__ __forceinline__ void stage_f32x64(const float* g, float* lds, int lane) {
  uint32_t boff = 4u * lane;
  asm volatile("" : "+v"(boff));
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(g) + boff, lds, 4, 0, 0);
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
