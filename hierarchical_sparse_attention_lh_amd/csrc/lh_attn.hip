// Causal softmax attention over the gathered sequence and its backward: the layer's one
// dense contraction.
//
// [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
// section "核心方法：金字塔池化与“外部选择”", item 3, and [HE] news.hamidun.com, "Nous Research
// introduced Lighthouse Attention to accelerate LLM training", section "How Lighthouse
// Attention Works": the selected entries form a dense causal subsequence that goes through
// ordinary scaled dot-product attention.  [EN] encorp.ai, "Услуги по внедряване на AI задават
// правилния въпрос за Lighthouse Attention", section "Как four-stage pipeline остава бърз, без
// да чупи градиентите?": gradients reach Q, K and V through that attention (the selection has
// none).  The pages call a stock FlashAttention kernel on another vendor's GPU; these are this
// library's own kernels for gfx950.
//
// Forward: O = softmax(scale Q K^T + causal mask) V, with the base-2 log-sum-exp per row.
// Backward, with P recomputed from the saved log-sum-exp and Delta = rowsum(dO * O):
//   dV = P^T dO;  dP = dO V^T;  dS = P * (dP - Delta);  dQ = scale dS K;  dK = scale dS^T Q.
//
// Where rows come from.  A row of Q, K or V is read where it lives:
//   * strided: row s of head (b, h) at base + b*sb + h*sh + s*ss (dense attention straight
//     on a [B, N, H, D] tensor, or on a gathered [B, H, S, D] copy);
//   * mapped: row s of head (b, h) is pyramid entry id = gmap[b, h, s], a raw token row of the
//     input (id < N) or a pooled row (id - N) of the pooled levels -- the gathered sequence is
//     never materialised.  The ids of the tile after next are brought into LDS by a direct
//     load, so each staging load knows its address without waiting on memory.
// Tiles are staged with gfx950 direct global->LDS loads (no VGPR round trip) into row-major,
// XOR-swizzled LDS tiles, double-buffered.  Every MFMA operand that needs a tile transposed
// (V^T in the forward, dO^T and Q^T in the key pass, K^T in the query pass) is read from the
// row tile with two ds_read_b64_tr_b16 transposing LDS reads, so no transposed copy of any
// tensor exists.  The swizzle keeps both read kinds free of bank conflicts: sixteen rows at
// one logical 16-byte chunk, and four rows x 64 bytes for a transposing read, each land in
// distinct bank groups.
//
// Matrix products: v_mfma_f32_32x32x16_bf16 (lane layouts in lh_mfma.h).  Scores are
// computed with the key index as the C row (forward, query pass: S^T = K Q^T) or column (key
// pass: S = Q K^T) so that P and dS leave the C registers as the next product's B operand.
// P and dS enter every product as a bf16 hi/lo pair (about 16 significant bits): with single
// bf16 operands the gradients' error under cancellation exceeds their own bf16 output
// rounding several times over.  The forward row sum is Kahan-compensated per tile (Delta
// amplifies any error in O).  The backward is deterministic: a key pass writes dK and dV, a
// query pass recomputes S and dP and writes dQ; no atomics.
#include <type_traits>

#include "lh_internal.h"
#include "lh_mfma.h"

namespace lh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;  // base-2 growth of the row max tolerated before a rescale

// ------------------------------------------------------------------------ LDS layout
__device__ __forceinline__ constexpr int bitrev3(int x) {
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}

// XOR key of LDS tile row r (rows of D bf16).  D = 64: a 128-byte row fills half a 256-byte
// bank line, rows 2j and 2j + 1 share key bitrev3(j mod 8); D = 128: a row fills a line and
// gets ((r mod 4) << 2) | ((r / 4) mod 4).  Rows 16 t + r and r share a key (so does 32 m + r).
template <int D>
__device__ __forceinline__ int rkey(int r) {
  if constexpr (D == 64)
    return bitrev3((r >> 1) & 7);
  else
    return ((r & 3) << 2) | ((r >> 2) & 3);
}

// Byte offset of logical 16-byte chunk 2j + hl of row lq: one per-lane value per k step;
// row 32 m + lq of any tile of this row length is 64 D m bytes further.
template <int D>
__device__ __forceinline__ uint32_t op_off(int lq, int hl, int j) {
  return static_cast<uint32_t>(lq * D * 2 + (((2 * j + hl) ^ rkey<D>(lq)) << 4));
}

// Byte offset (within a 16-row chunk) of one of the two transposing reads (sec 0: rows 0-7,
// sec 1: rows 8-15) that give lane l the elements X[16 t + k][32 db + l % 32] for its 8 k
// values, in the k order in which c_to_op2 hands out the C registers of the other operand.
// ds_read_b64_tr_b16 hands output lane i of each group of 16 lanes element (i mod 4) of the
// 8-byte pieces addressed by lanes 4j + i / 4 (j = 0..3); so source lane s of group g
// addresses row 4 (g / 2) + s / 4 (+ 8 for sec 1), columns 32 db + 16 (g mod 2) + 4 (s mod 4).
template <int D>
__device__ __forceinline__ uint32_t tr_off(int lane, int db, int sec) {
  const int g = lane >> 4, s = lane & 15;
  const int r = (g >> 1) * 4 + (s >> 2) + 8 * sec;
  const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
  return static_cast<uint32_t>(r * D * 2 + (((col >> 3) ^ rkey<D>(r)) << 4) + ((col & 7) << 1));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ v4i16 ds_tr16(const uint16_t* tile, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((lds_char*)(const_cast<uint16_t*>(tile)) + off));
}

// The transposed operand X^T (d rows, 16 k values of chunk t) from a row tile X.
__device__ __forceinline__ bf16x8 tr_op(const uint16_t* tile, uint32_t off0, uint32_t off1) {
  const v4i16 a = ds_tr16(tile, off0), b = ds_tr16(tile, off1);
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// ------------------------------------------------------------------------ row sources
// Element (b, h, s, d) of a strided operand is x[b sb + h sh + s ss + d].  Mapped operands
// (n0 = N) read row id of head (b, h) from x when id < n0, else row id - n0 of px (batch
// stride psb, same head and row strides).  Strided operands have n0 beyond every id.
struct RowSrc {
  const uint16_t* x;
  const uint16_t* px;
  int64_t sb, sh, ss, psb, n0;
};

// One head's rows: row id at byte address x + id * rsb, plus `dp` when id >= n0 (dp moves the
// address into the pooled levels: ph - n0 * rsb - xh, a uniform byte difference).
struct HeadRows {
  const char* x;
  const char* pn;  // mapped: the pooled rows' base moved back by n0 rows, so that row id >= n0
                   // sits at pn + id * rsb, like a raw row at x + id * rsb
  int64_t dp;      // pn - x
  int64_t n0;
  uint32_t rsb;
  uint32_t n0b;    // n0 * rsb when the pyramid's rows span less than 4 GiB (32-bit offsets)
};

__device__ __forceinline__ HeadRows head_rows(const RowSrc& r, int64_t b, int64_t h) {
  HeadRows o;
  o.x = reinterpret_cast<const char*>(r.x + b * r.sb + h * r.sh);
  o.rsb = static_cast<uint32_t>(r.ss * 2);
  o.n0 = r.n0;
  o.dp = 0;
  o.pn = o.x;
  o.n0b = 0;
  if (r.px != nullptr) {
    const char* ph = reinterpret_cast<const char*>(r.px + b * r.psb + h * r.sh);
    o.dp = (ph - o.x) - r.n0 * static_cast<int64_t>(o.rsb);
    o.pn = o.x + o.dp;
    o.n0b = static_cast<uint32_t>(r.n0 * o.rsb);
  }
  return o;
}

__device__ __forceinline__ const uint16_t* row_ptr(const HeadRows& hr, int64_t id) {
  const int64_t off = id * static_cast<int64_t>(hr.rsb) + (id >= hr.n0 ? hr.dp : 0);
  return reinterpret_cast<const uint16_t*>(hr.x + off);
}

// Staging of a ROWS x D tile by 256 threads, 16 bytes per lane per load: load i of wave w
// fills LDS chunks (4i + w) * 64 .. + 63, i.e. rows (4i + w) * RPL .. + RPL - 1 (RPL = 64 / CPR
// rows per load), lane l taking row (4i + w) * RPL + l / CPR, logical chunk l % CPR.  The
// swizzle key of that row depends on w and l only (rkey is periodic in the row with period
// RPL * 4 / gcd), so each lane needs one row index and one swizzled chunk offset for every
// load of every tile; the rest of the address is uniform.
template <int ROWS, int D>
struct Tile {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 64 / CPR;
  static constexpr int LOADS = ROWS * CPR / 256;
  static_assert(ROWS * CPR % 256 == 0, "tile must be a whole number of loads per thread");
};

struct LaneStage {
  uint32_t row;    // the lane's row within each load's RPL rows
  uint32_t chunk;  // byte offset of the lane's swizzled 16-byte piece within its row
  uint32_t wofs;   // byte offset of the wave's 1 KB within each load's 4 KB of LDS (uniform)
};

template <int D>
__device__ __forceinline__ LaneStage lane_stage(int wave, int lane) {
  constexpr int CPR = D / 8, RPL = 64 / CPR;
  LaneStage ls;
  ls.row = static_cast<uint32_t>(lane / CPR);
  ls.chunk = static_cast<uint32_t>(((lane % CPR) ^ rkey<D>(wave * RPL + lane / CPR)) << 4);
  ls.wofs = __builtin_amdgcn_readfirstlane(wave * 1024);
  return ls;
}

typedef __attribute__((address_space(3))) char* lds_bytes;

// LDS destination of load i: each wave instruction fills 1 KB of contiguous LDS.  The address
// is built from scalar values only (the buffer's fixed LDS address, the load index and the
// wave's uniform offset), so it reaches M0 without a per-load vector-to-scalar move.
__device__ __forceinline__ lds_bytes lds_dst(uint16_t* lds, int i, const LaneStage& ls) {
  return (lds_bytes)lds + i * 4096 + ls.wofs;
}

// Stage rows row0 .. row0 + ROWS - 1 of a strided operand.  A whole tile inside the sequence
// is a uniform base plus one 32-bit lane offset (scalar-base loads, no per-load address
// arithmetic); a tile that crosses the end clamps each row to S - 1.
template <int ROWS, int D>
__device__ __forceinline__ void stage_strided(const HeadRows& hr, const LaneStage& ls, int row0,
                                              int S, uint16_t* lds, int wave) {
  using T = Tile<ROWS, D>;
  if (row0 + ROWS <= S) {
    // the wave's and lane's share of the offset is a VGPR; the load's and tile's share uniform
    uint32_t o = (wave * T::RPL + ls.row) * hr.rsb + ls.chunk;
    asm volatile("" : "+v"(o));  // opaque: kept as a 32-bit offset from the uniform base
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const char* base = hr.x + static_cast<int64_t>(row0 + i * 4 * T::RPL) * hr.rsb;
      __builtin_amdgcn_global_load_lds(base + o, lds_dst(lds, i, ls), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int row = min(row0 + (i * 4 + wave) * T::RPL + static_cast<int>(ls.row), S - 1);
      const char* g = hr.x + static_cast<int64_t>(row) * hr.rsb + ls.chunk;
      __builtin_amdgcn_global_load_lds(g, lds_dst(lds, i, ls), 16, 0, 0);
    }
    // (an empty statement after the loads: otherwise the compiler merges the last load of
    // both branches into one after them, on a per-lane 64-bit address)
    asm volatile("");
  }
}

// Row ids of the lane's loads of the tile whose ids sit in LDS ring slot `ring` (padding
// slots hold -1 and read row 0).
template <int ROWS, int D>
__device__ __forceinline__ void ids_of(const int32_t* ring, const LaneStage& ls, int wave,
                                       int (&id)[Tile<ROWS, D>::LOADS]) {
  using T = Tile<ROWS, D>;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) id[i] = max(ring[(i * 4 + wave) * T::RPL + ls.row], 0);
}

// Mapped rows, MODE 2: any pyramid size (64-bit address arithmetic per load).
template <int ROWS, int D>
__device__ __forceinline__ void stage_mapped(const HeadRows& hr, const LaneStage& ls,
                                             const int (&id)[Tile<ROWS, D>::LOADS], uint16_t* lds,
                                             int wave) {
#pragma unroll
  for (int i = 0; i < Tile<ROWS, D>::LOADS; ++i) {
    const uint64_t rel =
        static_cast<uint64_t>(static_cast<uint32_t>(id[i])) * hr.rsb + ls.chunk;
    const int64_t dp = id[i] >= hr.n0 ? hr.dp : 0;
    const char* g = hr.x + static_cast<int64_t>(rel) + dp;
    __builtin_amdgcn_global_load_lds(g, lds_dst(lds, i, ls), 16, 0, 0);
  }
}

// Mapped rows, MODE 1 (the pyramid's rows span less than 4 GiB): the lane's 32-bit offsets
// id * rsb + chunk, computed once per tile and shared by every operand with the same row
// stride; each load is issued from the raw base for offsets below n0 * rsb and from the
// moved pooled base otherwise.
template <int ROWS, int D>
__device__ __forceinline__ void mapped_offsets(const int* id, uint32_t rsb, const LaneStage& ls,
                                               uint32_t* o) {
#pragma unroll
  for (int i = 0; i < Tile<ROWS, D>::LOADS; ++i) {
    // ids and row strides below 2^24 (the launcher's condition for this mode): a 24-bit
    // multiply-add is exact here
    o[i] = __umul24(static_cast<uint32_t>(id[i]), rsb) + ls.chunk;
    asm volatile("" : "+v"(o[i]));
  }
}

template <int ROWS, int D, bool TWO = true>
__device__ __forceinline__ void stage_mapped32(const HeadRows& hr, const LaneStage& ls,
                                               const uint32_t* o, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < Tile<ROWS, D>::LOADS; ++i) {
    if constexpr (!TWO) {
      // one load on a per-lane 64-bit address (fewer live registers)
      const char* base = o[i] < hr.n0b ? hr.x : hr.pn;
      __builtin_amdgcn_global_load_lds(base + o[i], lds_dst(lds, i, ls), 16, 0, 0);
      continue;
    }
    // Each lane loads from one of two uniform bases: two exec-masked loads, each a scalar
    // base plus the 32-bit lane offset.  The opaque copies keep each address sum inside its
    // branch, and the empty statement after one load keeps the compiler from merging the two
    // into one load on a per-lane 64-bit address.  (The instruction offset of a direct
    // global->LDS load moves the LDS address too, so it stays 0 everywhere.)
    const lds_bytes dst = lds_dst(lds, i, ls);
    uint32_t oo = o[i];
    if (oo < hr.n0b) {
      asm volatile("" : "+v"(oo));
      __builtin_amdgcn_global_load_lds(hr.x + oo, dst, 16, 0, 0);
    } else {
      asm volatile("" : "+v"(oo));
      __builtin_amdgcn_global_load_lds(hr.pn + oo, dst, 16, 0, 0);
      asm volatile("");
    }
  }
}

// n (<= 64) int32 / float values into LDS with one direct load (4 bytes per lane).
__device__ __forceinline__ void stage_words(const void* g, void* lds, int lane, int n) {
  if (lane < n) {
    uint32_t boff = 4u * lane;
    asm volatile("" : "+v"(boff));
    __builtin_amdgcn_global_load_lds(static_cast<const char*>(g) + boff, lds, 4, 0, 0);
  }
}

// ------------------------------------------------------------------------ forward
struct FwdArgs {
  RowSrc q, k, v;
  const int32_t* gmap;        // mapped: [B*H, Sp] pyramid ids, -1 for padding
  float* o;                   // O rows at o + b osb + h osh + s oss
  int64_t osb, osh, oss;
  float* lse;                 // [B*H, Sp], base 2
  int64_t BH;
  int H, S, Sp, o_rows, causal;
  float sl2;                  // scale * log2(e)
};

// MODE: 0 = strided rows, 1 = mapped rows with 32-bit offsets, 2 = mapped rows, 64-bit.
template <int D, int MODE>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a) {
  constexpr bool MAPPED = MODE != 0;
  constexpr int BM = 128, BN = 64;
  using KT = Tile<BN, D>;
  constexpr int NL = KT::LOADS;
  __shared__ __attribute__((aligned(16))) uint16_t ks0[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t ks1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs1[BN * D];
  __shared__ __attribute__((aligned(16))) int32_t idr[4][BN];

  const int S = a.S, Sp = a.Sp;
  const int nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, a.BH * nqt);
  const int64_t bh = item / nqt;
  const int qt = nqt - 1 - static_cast<int>(item % nqt);  // far-from-diagonal (heavy) first
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int myq = qw + lq;
  const HeadRows hq = head_rows(a.q, b, h), hk = head_rows(a.k, b, h), hv = head_rows(a.v, b, h);
  const int32_t* gm = MAPPED ? a.gmap + bh * Sp : nullptr;
  const float sl2 = a.sl2;
  const bool causal = a.causal != 0;

  bf16x8 qreg[D / 16];
  {
    const int qid = MAPPED ? max(gm[myq], 0) : min(myq, S - 1);
    const uint16_t* qr = row_ptr(hq, qid);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qreg[kk] = ld_op16(qr + 16 * kk + hl * 8);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f, l_cmp = 0.f;

  const int kend = causal ? (S < q0 + BM ? S : q0 + BM) : S;
  const int nkt = (kend + BN - 1) / BN;

  // per-lane LDS byte offsets: K rows (16-byte operand reads), V^T (transposing reads)
  uint32_t toff[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) toff[db][sec] = tr_off<D>(lane, db, sec);

  const LaneStage ls = lane_stage<D>(wave, lane);
  auto load_ids = [&](int t) {
    if constexpr (MAPPED)
      if (wave == 0 && t < nkt) stage_words(gm + t * BN, idr[t & 3], lane, BN);
  };
  // row ids of tile t (mapped) -- read from LDS before the step issues any load
  auto get_ids = [&](int t, int (&id)[NL]) {
    if constexpr (MAPPED) ids_of<BN, D>(idr[t & 3], ls, wave, id);
    else
#pragma unroll
      for (int i = 0; i < NL; ++i) id[i] = 0;
  };
  auto stage_k = [&](int t, const int (&id)[NL], uint16_t* lds) {
    if constexpr (MODE == 2) stage_mapped<BN, D>(hk, ls, id, lds, wave);
    else stage_strided<BN, D>(hk, ls, t * BN, S, lds, wave);
  };
  auto stage_v = [&](int t, const int (&id)[NL], uint16_t* lds) {
    if constexpr (MODE == 2) stage_mapped<BN, D>(hv, ls, id, lds, wave);
    else stage_strided<BN, D>(hv, ls, t * BN, S, lds, wave);
  };
  auto mask = [&](int t, f32x16 (&sacc)[2]) {
    const int k0 = t * BN;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
        if ((causal && key > myq) || key >= S) sacc[b2][r] = -INFINITY;
      }
  };

  // Tile t: S^T = K Q^T, online softmax, O^T += V^T P^T (hi-lo P).
  auto plain_tile = [&](auto masked, int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    const uint16_t* ksb = B1 ? ks1 : ks0;
    const uint16_t* vsb = B1 ? vs1 : vs0;
    f32x16 sacc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) sacc[b2] = zero16();
    // at D = 64 (three waves per SIMD) the matrix products run at raised wave priority, so
    // that a wave with MFMAs to issue goes ahead of the other waves' softmax work
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
        sacc[b2] = mfma32(lds_at(ksb, b2 * 64 * D + op_off<D>(lq, hl, kk)), qreg[kk], sacc[b2]);
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
    if constexpr (decltype(masked)::value) mask(t, sacc);
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
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x8 ph, pl;
      c_to_op2(sacc[t4 >> 1], t4 & 1, ph, pl);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 av = tr_op(vsb, t4 * 32 * D + toff[db][0], t4 * 32 * D + toff[db][1]);
        oacc[db] = mfma32(av, pl, oacc[db]);
        oacc[db] = mfma32(av, ph, oacc[db]);
      }
    }
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
  };

  auto plain_step = [&](int t, auto bufc) {
    constexpr bool B1 = decltype(bufc)::value;
    int id[NL];
    const bool nx = t + 1 < nkt;
    if (nx) get_ids(t + 1, id);
    load_ids(t + 2);
    if (nx) {
      if constexpr (MODE == 1) {
        uint32_t o[NL];
        mapped_offsets<BN, D>(id, hk.rsb, ls, o);
        stage_mapped32<BN, D>(hk, ls, o, B1 ? ks0 : ks1);
        stage_mapped32<BN, D>(hv, ls, o, B1 ? vs0 : vs1);
      } else {
        stage_k(t + 1, id, B1 ? ks0 : ks1);
        stage_v(t + 1, id, B1 ? vs0 : vs1);
      }
    }
    const int k0 = t * BN;
    if ((causal && k0 + BN - 1 > qw) || k0 + BN > S)
      plain_tile(std::true_type{}, t, bufc);
    else
      plain_tile(std::false_type{}, t, bufc);
    wait_vmem();
    __syncthreads();
  };

  load_ids(0);
  load_ids(1);
  wait_vmem();
  __syncthreads();
  {
    int id0[NL];
    get_ids(0, id0);
    if constexpr (MODE == 1) {
      uint32_t o0[NL];
      mapped_offsets<BN, D>(id0, hk.rsb, ls, o0);
      stage_mapped32<BN, D>(hk, ls, o0, ks0);
      stage_mapped32<BN, D>(hv, ls, o0, vs0);
    } else {
      stage_k(0, id0, ks0);
      stage_v(0, id0, vs0);
    }
  }
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    plain_step(t, std::false_type{});
    if (t + 1 < nkt) plain_step(t + 1, std::true_type{});
  }

  const float l_own = l_run - l_cmp;
  const float l_tot = pair_sum(l_own);
  const float inv_l = 1.0f / l_tot;
  if (myq < a.o_rows) {
    float* orow = a.o + b * a.osb + h * a.osh + static_cast<int64_t>(myq) * a.oss;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 val = make_float4(oacc[db][4 * g] * inv_l, oacc[db][4 * g + 1] * inv_l,
                                       oacc[db][4 * g + 2] * inv_l, oacc[db][4 * g + 3] * inv_l);
        *reinterpret_cast<float4*>(orow + db * 32 + g * 8 + hl * 4) = val;
      }
  }
  if (hl == 0) a.lse[bh * Sp + myq] = m_run + log2f(l_tot);  // base-2 log-sum-exp
}

// Three waves per SIMD at D = 64 (about 145 registers), two at D = 128.
#define LH_FWD(NAME, D, MODE, W)                                                             \
  __global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W))) void NAME( \
      FwdArgs a) {                                                                          \
    attn_fwd_body<D, MODE>(a);                                                              \
  }
LH_FWD(attn_fwd_d64, 64, 0, 3)
LH_FWD(attn_fwd_d128, 128, 0, 2)
LH_FWD(attn_fwd_mapped_d64, 64, 1, 3)
LH_FWD(attn_fwd_mapped_d128, 128, 1, 2)
LH_FWD(attn_fwd_mapped64_d64, 64, 2, 3)
LH_FWD(attn_fwd_mapped64_d128, 128, 2, 2)
#undef LH_FWD

// ------------------------------------------------------------------------ backward
struct BwdArgs {
  RowSrc q, k, v;
  const int32_t* gmap;        // mapped: [B*H, Sp]
  const uint16_t* dout;       // dO rows at dout + b dsb + h dsh + s dss (bf16)
  int64_t dsb, dsh, dss;
  const float* lse;           // [B*H, Sp], base 2
  const float* delta;         // [B*H, Sp] (zero for padding)
  float* dq;                  // gradient rows at g + b gsb + h gsh + s gss
  float* dk;
  float* dv;
  int64_t gsb, gsh, gss;
  int64_t BH;
  int H, S, Sp, g_rows, causal;
  float scale, sl2;
};

// ---------------------------------------------------------------- key pass (dK, dV)
// Workgroup = 128 keys (4 waves x 32); loops over query tiles of BQ from the diagonal down.
// S = Q K^T and dP = dO V^T with keys as the C column, so P and dS leave the C registers as
// B operands of dV^T = dO^T P and dK^T = Q^T dS, whose A operands are transposing reads of
// the staged dO and Q row tiles.  V is negated once and the dP accumulator is seeded with
// Delta, so the product yields Delta - dP and dS costs one multiply (the sign is folded into
// the final dK scale).
template <int D, int BQ, int MODE>
__device__ __forceinline__ void attn_bwd_kv_body(const BwdArgs& a) {
  constexpr bool MAPPED = MODE != 0;
  constexpr int BK = 128, NB = BQ / 32;
  using QT = Tile<BQ, D>;
  constexpr int NL = QT::LOADS;
  // each buffer its own LDS object, named statically (the loop is unrolled by the number of
  // buffers): the compiler then does not make a tile's LDS reads wait for the next tile's
  // loads.  The pipelined D = 64 loop rotates three buffers, the others two.
  __shared__ __attribute__((aligned(16))) uint16_t qs0[BQ * D], qs1[BQ * D], qs2[BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t ds0[BQ * D], ds1[BQ * D], ds2[BQ * D];
  __shared__ __attribute__((aligned(16))) float ls0[BQ], ls1[BQ], ls2[BQ];
  __shared__ __attribute__((aligned(16))) float dl0[BQ], dl1[BQ], dl2[BQ];
  __shared__ __attribute__((aligned(16))) int32_t idr[4][BQ];

  const int S = a.S, Sp = a.Sp;
  const int nkt = Sp / BK;
  const int64_t item = xcd_item(blockIdx.x, a.BH * nkt);
  const int64_t bh = item / nkt;
  const int ktile = static_cast<int>(item % nkt);  // small key tiles have the most work: first
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int K0 = ktile * BK;
  const int kw = K0 + wave * 32;
  const int mykey = kw + lq;
  const bool causal = a.causal != 0;
  const HeadRows hq = head_rows(a.q, b, h), hk = head_rows(a.k, b, h), hv = head_rows(a.v, b, h);
  const int32_t* gm = MAPPED ? a.gmap + bh * Sp : nullptr;
  const uint16_t* dob = a.dout + b * a.dsb + h * a.dsh;
  const float* lb = a.lse + bh * Sp;
  const float* dlb = a.delta + bh * Sp;
  const float sl2 = a.sl2;

  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const int kid = MAPPED ? max(gm[mykey], 0) : min(mykey, S - 1);
    const uint16_t* kr = row_ptr(hk, kid);
    const uint16_t* vr = row_ptr(hv, kid);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kreg[kk] = ld_op16(kr + 16 * kk + hl * 8);
      // -V: the dP product then accumulates Delta - dP on top of Delta
      vreg[kk] = as_bf16x8(__builtin_bit_cast(u32x4, ld_op16(vr + 16 * kk + hl * 8)) ^ 0x80008000u);
    }
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) {
    dkacc[d2] = zero16();
    dvacc[d2] = zero16();
  }

  const int qt0 = causal ? K0 / BQ : 0;
  const int nqt = (S + BQ - 1) / BQ;

  HeadRows hd;  // dO rows (strided)
  hd.x = reinterpret_cast<const char*>(dob);
  hd.rsb = static_cast<uint32_t>(a.dss * 2);
  hd.n0 = int64_t(1) << 62;
  hd.dp = 0;
  const LaneStage ls = lane_stage<D>(wave, lane);
  auto load_ids = [&](int t) {
    if constexpr (MAPPED)
      if (wave == 0 && t < nqt) stage_words(gm + t * BQ, idr[t & 3], lane, BQ);
  };
  // buffer `bi` (a compile-time index) of each kind
  auto qbuf = [&](auto bi) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return qs0; else if constexpr (B == 1) return qs1; else return qs2;
  };
  auto dbuf = [&](auto bi) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return ds0; else if constexpr (B == 1) return ds1; else return ds2;
  };
  auto lbuf = [&](auto bi) -> float* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return ls0; else if constexpr (B == 1) return ls1; else return ls2;
  };
  auto dlbuf = [&](auto bi) -> float* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return dl0; else if constexpr (B == 1) return dl1; else return dl2;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // Tile t: Q rows (through the map), dO rows, lse and Delta into buffer bufc; the ids are read
  // from LDS before any load of this step is issued.
  auto stage = [&](int t, auto bufc) {
    const int q0 = t * BQ;
    int id[NL];
    if constexpr (MAPPED) ids_of<BQ, D>(idr[t & 3], ls, wave, id);
    load_ids(t + 1);
    if constexpr (MODE == 1) {
      uint32_t o[Tile<BQ, D>::LOADS];
      mapped_offsets<BQ, D>(id, hq.rsb, ls, o);
      stage_mapped32<BQ, D>(hq, ls, o, qbuf(bufc));
    } else if constexpr (MODE == 2) {
      stage_mapped<BQ, D>(hq, ls, id, qbuf(bufc), wave);
    } else {
      stage_strided<BQ, D>(hq, ls, q0, S, qbuf(bufc), wave);
    }
    stage_strided<BQ, D>(hd, ls, q0, S, dbuf(bufc), wave);
    if (wave == 0) stage_words(lb + q0, lbuf(bufc), lane, BQ);
    if (wave == 1) stage_words(dlb + q0, dlbuf(bufc), lane, BQ);
  };

  // generic tile (any D, BQ): S and dP per 32-query block, then dV and dK per 16-query chunk
  auto tile = [&](auto masked, int t, auto bufc) {
    const uint16_t* qsb = qbuf(bufc);
    const uint16_t* dsb = dbuf(bufc);
    const float* lsb = lbuf(bufc);
    const float* dlb_ = dlbuf(bufc);
    const int q0 = t * BQ;
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
        sacc[b2] = mfma32(lds_at(qsb, b2 * 64 * D + op_off<D>(lq, hl, kk)), kreg[kk], sacc[b2]);
        pacc[b2] = mfma32(lds_at(dsb, b2 * 64 * D + op_off<D>(lq, hl, kk)), vreg[kk], pacc[b2]);
      }
    }
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = b2 * 32 + g * 8 + hl * 4;
        const float4 l4 = *reinterpret_cast<const float4*>(&lsb[qi]);
        const float lv4[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -lv4[u]));
          if constexpr (decltype(masked)::value) {
            const int qa = q0 + qi + u;
            if ((causal && qa < mykey) || qa >= S) p = 0.f;
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
        // transposing-read offsets, computed per use to keep registers free
        const uint32_t o0 = t4 * 32 * D + tr_off<D>(lane, d2, 0);
        const uint32_t o1 = t4 * 32 * D + tr_off<D>(lane, d2, 1);
        const bf16x8 ao = tr_op(dsb, o0, o1);
        const bf16x8 aq = tr_op(qsb, o0, o1);
        dvacc[d2] = mfma32(ao, pl, dvacc[d2]);
        dvacc[d2] = mfma32(ao, ph, dvacc[d2]);
        dkacc[d2] = mfma32(aq, sl, dkacc[d2]);
        dkacc[d2] = mfma32(aq, sh, dkacc[d2]);
      }
    }
  };

  // D = 64, 64 queries, pipelined across tiles: twelve groups of four MFMAs, each carrying one
  // unit of vector work whose inputs are complete:
  //   A0 p3'   A1 d3'   V3' b0   K3' b1   A2 p0   A3 d0   V0 p1   K0 d1   V1 b2   K1 p2   V2 d2   K2 b3
  // (A0 .. A3: S and dP of one 32-query block, two k steps each; V / K: the dV or dK update of
  // one 16-query chunk; b = exp and dS of a chunk, p / d = hi-lo split of its P / dS; ' = the
  // previous tile).  The split and the dV / dK products of a tile's last chunk run in the next
  // tile's first four groups, so no group is left without vector work; that tile's Q and dO
  // rows are still in their LDS buffers then, because three buffers rotate (a buffer is
  // restaged only two steps after its tile).  Fixed with scheduling barriers; the LDS operands
  // of each group are read one group ahead.  S and dP stay in sacc / pacc across steps.
  uint32_t loff[4], tro[2][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) loff[j] = op_off<64>(lq, hl, j);
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) tro[d2][sec] = tr_off<64>(lane, d2, sec);
  f32x16 sacc[2], pacc[2];

  auto tile64p = [&](auto masked, int t, auto cur, auto prev, auto first) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool FIRST = decltype(first)::value;
    const int q0 = t * BQ;
    const uint16_t* qsb = qbuf(cur);
    const uint16_t* dsb = dbuf(cur);
    const uint16_t* qsp = qbuf(prev);
    const uint16_t* dsp = dbuf(prev);
    const float* lsb = lbuf(cur);
    const float* dlb_ = dlbuf(cur);
    bf16x8 op[12][4];
    float4 lsv[4][2];
    bf16x8 ph[3], pl[3], sh[3], sl[3], php, plp, shp, slp;
    // opaque copies: the address sums stay inside the loop and fold into instruction
    // offsets instead of being hoisted into dozens of live registers
    uint32_t lo[4], tr[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = loff[j];
      asm volatile("" : "+v"(lo[j]));
    }
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        tr[d2][sec] = tro[d2][sec];
        asm volatile("" : "+v"(tr[d2][sec]));
      }
    // group g's MFMA unit: A units at g = 0, 1, 4, 5; dV units at even g >= 2 and dK units at
    // odd g >= 3, for chunk 3 of the previous tile (g = 2, 3) or chunk (g - 6) / 2 of this one
    auto is_a = [](int g) { return g == 0 || g == 1 || g == 4 || g == 5; };
    auto load_ops = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g == 0 || g == 1 || g == 4 || g == 5) {
        constexpr int b2 = g >> 2, kh = g & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = 2 * kh + j;
          op[g][2 * j] = lds_at(qsb, 4096 * b2 + lo[kk]);
          op[g][2 * j + 1] = lds_at(dsb, 4096 * b2 + lo[kk]);
        }
      } else if constexpr (!(FIRST && (g == 2 || g == 3))) {
        constexpr int t4 = g < 4 ? 3 : (g - 6) >> 1;
        const uint16_t* src = (g & 1) ? (g < 4 ? qsp : qsb) : (g < 4 ? dsp : dsb);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
          op[g][d2] = tr_op(src, 2048 * t4 + tr[d2][0], 2048 * t4 + tr[d2][1]);
      }
    };
    auto mfma_unit = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g == 0 || g == 1 || g == 4 || g == 5) {
        constexpr int b2 = g >> 2, kh = g & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kk = 2 * kh + j;
          sacc[b2] = mfma32(op[g][2 * j], kreg[kk], sacc[b2]);
          pacc[b2] = mfma32(op[g][2 * j + 1], vreg[kk], pacc[b2]);
        }
      } else if constexpr (FIRST && (g == 2 || g == 3)) {
      } else if constexpr ((g & 1) == 0) {
        const bf16x8& h_ = g == 2 ? php : ph[g == 2 ? 0 : (g - 6) >> 1];
        const bf16x8& l_ = g == 2 ? plp : pl[g == 2 ? 0 : (g - 6) >> 1];
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dvacc[d2] = mfma32(op[g][d2], l_, dvacc[d2]);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dvacc[d2] = mfma32(op[g][d2], h_, dvacc[d2]);
      } else {
        const bf16x8& h_ = g == 3 ? shp : sh[g == 3 ? 0 : (g - 7) >> 1];
        const bf16x8& l_ = g == 3 ? slp : sl[g == 3 ? 0 : (g - 7) >> 1];
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dkacc[d2] = mfma32(op[g][d2], l_, dkacc[d2]);
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) dkacc[d2] = mfma32(op[g][d2], h_, dkacc[d2]);
      }
    };
    (void)is_a;
    // the lse values of chunk t4's queries, read one group before its b unit
    auto load_ls = [&](int t4) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        lsv[t4][gg] = *reinterpret_cast<const float4*>(
            &lsb[(t4 >> 1) * 32 + ((t4 & 1) * 2 + gg) * 8 + hl * 4]);
    };
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
    auto b_unit = [&](int t4) {
      const int b2 = t4 >> 1, half = t4 & 1;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * half + gg;
        const float lv4[4] = {lsv[t4][gg].x, lsv[t4][gg].y, lsv[t4][gg].z, lsv[t4][gg].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[b2][r], sl2, -lv4[u]));
          if constexpr (MASK) {
            const int qa = q0 + b2 * 32 + g * 8 + hl * 4 + u;
            if ((causal && qa < mykey) || qa >= S) p = 0.f;
          }
          sacc[b2][r] = p;
          pacc[b2][r] = p * pacc[b2][r];
        }
      }
    };
    auto sp_unit = [&](int t4) { c_to_op2(sacc[t4 >> 1], t4 & 1, ph[t4], pl[t4]); };
    auto sd_unit = [&](int t4) { c_to_op2(pacc[t4 >> 1], t4 & 1, sh[t4], sl[t4]); };
    // one group: nm MFMAs, each followed by nv vector instructions, with the group's LDS
    // reads (the next group's operands) right after its first MFMA: the wait that the first
    // MFMA needs then covers only reads issued a whole group earlier, and the new reads have
    // the rest of the group to land
    auto layout = [&](auto nmc, auto nvc) {
      constexpr int nm = decltype(nmc)::value, nv = decltype(nvc)::value;
      if constexpr (nm > 0) {
#pragma unroll
        for (int i = 0; i < nm; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
          if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, 1>;
    using G2 = std::integral_constant<int, 2>;
    using G3 = std::integral_constant<int, 3>;
    using G4 = std::integral_constant<int, 4>;
    using G5 = std::integral_constant<int, 5>;
    using G6 = std::integral_constant<int, 6>;
    using G7 = std::integral_constant<int, 7>;
    using G8 = std::integral_constant<int, 8>;
    using G9 = std::integral_constant<int, 9>;
    using G10 = std::integral_constant<int, 10>;
    using G11 = std::integral_constant<int, 11>;
    using M0 = std::integral_constant<int, 0>;
    using M4 = std::integral_constant<int, 4>;
    using V0 = std::integral_constant<int, 0>;
    using V6 = std::integral_constant<int, 6>;
    using MP = std::conditional_t<FIRST, M0, M4>;  // previous tile's MFMA groups
    using VP = std::conditional_t<FIRST, V0, V6>;  // previous tile's vector work
    seed(0);
    load_ops(G0{});
    __builtin_amdgcn_sched_barrier(0);
    // g0: A0 | p3'
    load_ops(G1{});
    mfma_unit(G0{});
    if constexpr (!FIRST) c_to_op2(sacc[1], 1, php, plp);
    layout(M4{}, VP{});
    // g1: A1 | d3'
    load_ops(G2{});
    load_ls(0);
    mfma_unit(G1{});
    if constexpr (!FIRST) c_to_op2(pacc[1], 1, shp, slp);
    layout(M4{}, VP{});
    // g2: V3' | b0   (block 1 of the previous tile is consumed: seed it for this tile)
    load_ops(G3{});
    load_ls(1);
    seed(1);
    mfma_unit(G2{});
    b_unit(0);
    layout(MP{}, V6{});
    // g3: K3' | b1
    load_ops(G4{});
    mfma_unit(G3{});
    b_unit(1);
    layout(MP{}, V6{});
    // g4: A2 | p0
    load_ops(G5{});
    mfma_unit(G4{});
    sp_unit(0);
    layout(M4{}, V6{});
    // g5: A3 | d0
    load_ops(G6{});
    mfma_unit(G5{});
    sd_unit(0);
    layout(M4{}, V6{});
    // g6: V0 | p1
    load_ops(G7{});
    mfma_unit(G6{});
    sp_unit(1);
    layout(M4{}, V6{});
    // g7: K0 | d1
    load_ops(G8{});
    load_ls(2);
    mfma_unit(G7{});
    sd_unit(1);
    layout(M4{}, V6{});
    // g8: V1 | b2
    load_ops(G9{});
    mfma_unit(G8{});
    b_unit(2);
    layout(M4{}, V6{});
    // g9: K1 | p2
    load_ops(G10{});
    mfma_unit(G9{});
    sp_unit(2);
    layout(M4{}, V6{});
    // g10: V2 | d2
    load_ops(G11{});
    load_ls(3);
    mfma_unit(G10{});
    sd_unit(2);
    layout(M4{}, V6{});
    // g11: K2 | b3   (chunk 3's split and products run in the next step, or in finish)
    mfma_unit(G11{});
    b_unit(3);
    layout(M4{}, V6{});
  };

  // D = 128, 32 queries (one wave per SIMD, so the wave's own instruction stream must keep
  // the MFMAs busy): the dV / dK products of a tile run in the next tile, beside that tile's
  // score products, exponentials and splits.  Twelve groups of four MFMAs:
  //   A0 c0'  A1 c1'  A2 c2'  A3 c3'  V0a' b0  V0b' b1  K0a' p0  K0b' d0  V1a' p1  V1b' d1  K1a'  K1b'
  // (A0 .. A3: S and dP, two k steps each; V / K: dV or dK of one 16-query chunk, two
  // 32-column blocks; b = exp and dS of a chunk, p / d = hi-lo split of its P / dS; c' = copy
  // of the previous tile's split operands, so this tile's splits can take their registers;
  // ' = the previous tile, whose Q and dO rows are still staged: three buffers rotate).
  uint32_t loff128[8], tro128[4][2];
  if constexpr (D == 128) {
#pragma unroll
    for (int j = 0; j < 8; ++j) loff128[j] = op_off<128>(lq, hl, j);
#pragma unroll
    for (int d2 = 0; d2 < 4; ++d2)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) tro128[d2][sec] = tr_off<128>(lane, d2, sec);
  }
  f32x16 sacc1, pacc1;
  bf16x8 phc[2], plc[2], shc[2], slc[2];  // this tile's split P and dS, chunks 0 and 1
  bf16x8 php[2], plp[2], shp[2], slp[2];  // the previous tile's

  auto tile128p = [&](auto masked, int t, auto cur, auto prev, auto first) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool FIRST = decltype(first)::value;
    const int q0 = t * BQ;
    const uint16_t* qsb = qbuf(cur);
    const uint16_t* dsb = dbuf(cur);
    const uint16_t* qsp = qbuf(prev);
    const uint16_t* dsp = dbuf(prev);
    const float* lsb = lbuf(cur);
    const float* dlb_ = dlbuf(cur);
    bf16x8 op[12][4];
    float4 lsv[2][2];
    uint32_t lo[8], tr[4][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = loff128[j];
      asm volatile("" : "+v"(lo[j]));
    }
#pragma unroll
    for (int d2 = 0; d2 < 4; ++d2)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        tr[d2][sec] = tro128[d2][sec];
        asm volatile("" : "+v"(tr[d2][sec]));
      }
    // group g: A units at g < 4 (k steps 2g, 2g + 1); at g >= 4, u = g - 4 picks chunk u / 4,
    // dV (u / 2 even) or dK, and the column blocks 0-1 or 2-3 (u odd)
    auto load_ops = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g < 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          op[g][2 * j] = lds_at(qsb, lo[2 * g + j]);
          op[g][2 * j + 1] = lds_at(dsb, lo[2 * g + j]);
        }
      } else if constexpr (!FIRST) {
        constexpr int u = g - 4, c = u >> 2, isk = (u >> 1) & 1, half = u & 1;
        const uint16_t* src = isk ? qsp : dsp;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int d2 = 2 * half + i;
          op[g][i] = tr_op(src, 4096 * c + tr[d2][0], 4096 * c + tr[d2][1]);
        }
      }
    };
    auto mfma_unit = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g < 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sacc1 = mfma32(op[g][2 * j], kreg[2 * g + j], sacc1);
          pacc1 = mfma32(op[g][2 * j + 1], vreg[2 * g + j], pacc1);
        }
      } else if constexpr (!FIRST) {
        constexpr int u = g - 4, c = u >> 2, isk = (u >> 1) & 1, half = u & 1;
        const bf16x8& h_ = isk ? shp[c] : php[c];
        const bf16x8& l_ = isk ? slp[c] : plp[c];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f32x16& acc = isk ? dkacc[2 * half + i] : dvacc[2 * half + i];
          acc = mfma32(op[g][i], l_, acc);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f32x16& acc = isk ? dkacc[2 * half + i] : dvacc[2 * half + i];
          acc = mfma32(op[g][i], h_, acc);
        }
      }
    };
    auto seed = [&]() {
      sacc1 = zero16();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *reinterpret_cast<const float4*>(&dlb_[g * 8 + hl * 4]);
        pacc1[4 * g] = d4.x;
        pacc1[4 * g + 1] = d4.y;
        pacc1[4 * g + 2] = d4.z;
        pacc1[4 * g + 3] = d4.w;
      }
    };
    auto load_ls = [&](int t4) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        lsv[t4][gg] = *reinterpret_cast<const float4*>(&lsb[(t4 * 2 + gg) * 8 + hl * 4]);
    };
    auto b_unit = [&](int t4) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * t4 + gg;
        const float lv4[4] = {lsv[t4][gg].x, lsv[t4][gg].y, lsv[t4][gg].z, lsv[t4][gg].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = g * 4 + u;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc1[r], sl2, -lv4[u]));
          if constexpr (MASK) {
            const int qa = q0 + g * 8 + hl * 4 + u;
            if ((causal && qa < mykey) || qa >= S) p = 0.f;
          }
          sacc1[r] = p;
          pacc1[r] = p * pacc1[r];
        }
      }
    };
    auto copy_unit = [&](int k) {  // the previous tile's split operands into their registers
      const int c = k >> 1;
      if (k & 1) {
        shp[c] = shc[c];
        slp[c] = slc[c];
      } else {
        php[c] = phc[c];
        plp[c] = plc[c];
      }
    };
    auto layout = [&](auto nmc, auto nvc) {
      constexpr int nm = decltype(nmc)::value, nv = decltype(nvc)::value;
      if constexpr (nm > 0) {
#pragma unroll
        for (int i = 0; i < nm; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
          if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, 1>;
    using G2 = std::integral_constant<int, 2>;
    using G3 = std::integral_constant<int, 3>;
    using G4 = std::integral_constant<int, 4>;
    using G5 = std::integral_constant<int, 5>;
    using G6 = std::integral_constant<int, 6>;
    using G7 = std::integral_constant<int, 7>;
    using G8 = std::integral_constant<int, 8>;
    using G9 = std::integral_constant<int, 9>;
    using G10 = std::integral_constant<int, 10>;
    using G11 = std::integral_constant<int, 11>;
    using M0 = std::integral_constant<int, 0>;
    using M4 = std::integral_constant<int, 4>;
    using V0 = std::integral_constant<int, 0>;
    using V2 = std::integral_constant<int, 2>;
    using V6 = std::integral_constant<int, 6>;
    using MP = std::conditional_t<FIRST, M0, M4>;  // previous tile's MFMA groups
    using VC = std::conditional_t<FIRST, V0, V2>;  // copies of the previous tile's operands
    seed();
    load_ops(G0{});
    __builtin_amdgcn_sched_barrier(0);
    load_ops(G1{});
    mfma_unit(G0{});
    if constexpr (!FIRST) copy_unit(0);
    layout(M4{}, VC{});
    load_ops(G2{});
    mfma_unit(G1{});
    if constexpr (!FIRST) copy_unit(1);
    layout(M4{}, VC{});
    load_ops(G3{});
    mfma_unit(G2{});
    if constexpr (!FIRST) copy_unit(2);
    layout(M4{}, VC{});
    load_ops(G4{});
    load_ls(0);
    mfma_unit(G3{});
    if constexpr (!FIRST) copy_unit(3);
    layout(M4{}, VC{});
    load_ops(G5{});
    load_ls(1);
    mfma_unit(G4{});
    b_unit(0);
    layout(MP{}, V6{});
    load_ops(G6{});
    mfma_unit(G5{});
    b_unit(1);
    layout(MP{}, V6{});
    load_ops(G7{});
    mfma_unit(G6{});
    c_to_op2(sacc1, 0, phc[0], plc[0]);
    layout(MP{}, V6{});
    load_ops(G8{});
    mfma_unit(G7{});
    c_to_op2(pacc1, 0, shc[0], slc[0]);
    layout(MP{}, V6{});
    load_ops(G9{});
    mfma_unit(G8{});
    c_to_op2(sacc1, 1, phc[1], plc[1]);
    layout(MP{}, V6{});
    load_ops(G10{});
    mfma_unit(G9{});
    c_to_op2(pacc1, 1, shc[1], slc[1]);
    layout(MP{}, V6{});
    load_ops(G11{});
    mfma_unit(G10{});
    layout(MP{}, V0{});
    mfma_unit(G11{});
    layout(MP{}, V0{});
  };

  // D = 128: the last tile's dV and dK products (its rows are still in buffer bi)
  auto finish128 = [&](auto bi) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int d2 = 0; d2 < 4; ++d2) {
        const bf16x8 ao = tr_op(dbuf(bi), 4096 * c + tro128[d2][0], 4096 * c + tro128[d2][1]);
        dvacc[d2] = mfma32(ao, plc[c], dvacc[d2]);
        dvacc[d2] = mfma32(ao, phc[c], dvacc[d2]);
        const bf16x8 aq = tr_op(qbuf(bi), 4096 * c + tro128[d2][0], 4096 * c + tro128[d2][1]);
        dkacc[d2] = mfma32(aq, slc[c], dkacc[d2]);
        dkacc[d2] = mfma32(aq, shc[c], dkacc[d2]);
      }
  };

  // the last tile's chunk 3: split, dV and dK (its rows are still in buffer bi)
  auto finish = [&](auto bi) {
    bf16x8 hi, lo_;
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      const bf16x8 ao = tr_op(dbuf(bi), 2048 * 3 + tro[d2][0], 2048 * 3 + tro[d2][1]);
      c_to_op2(sacc[1], 1, hi, lo_);
      dvacc[d2] = mfma32(ao, lo_, dvacc[d2]);
      dvacc[d2] = mfma32(ao, hi, dvacc[d2]);
    }
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      const bf16x8 aq = tr_op(qbuf(bi), 2048 * 3 + tro[d2][0], 2048 * 3 + tro[d2][1]);
      c_to_op2(pacc[1], 1, hi, lo_);
      dkacc[d2] = mfma32(aq, lo_, dkacc[d2]);
      dkacc[d2] = mfma32(aq, hi, dkacc[d2]);
    }
  };

  auto next_buf = [](auto bi) {
    return std::integral_constant<int, (decltype(bi)::value + 1) % 3>{};
  };
  // pipelined step t (D = 64): tile t in buffer cur, tile t - 1 in prev, tile t + 1 staged
  // into the third buffer
  auto step3 = [&](int t, auto cur, auto prev, auto first) {
    if (t + 1 < nqt) stage(t + 1, next_buf(cur));
    const int q0 = t * BQ;
    const bool msk = (causal && q0 < kw + 31) || q0 + BQ > S;
    if constexpr (D == 64) {
      if (msk)
        tile64p(std::true_type{}, t, cur, prev, first);
      else
        tile64p(std::false_type{}, t, cur, prev, first);
    } else {
      if (msk)
        tile128p(std::true_type{}, t, cur, prev, first);
      else
        tile128p(std::false_type{}, t, cur, prev, first);
    }
    wait_vmem();
    __syncthreads();
  };
  // generic step t: tile t in buffer bufc, tile t + 1 staged into the other of two buffers
  auto step = [&](int t, auto bufc) {
    if (t + 1 < nqt) stage(t + 1, std::integral_constant<int, 1 - decltype(bufc)::value>{});
    const int q0 = t * BQ;
    const bool msk = (causal && q0 < kw + 31) || q0 + BQ > S;
    if (msk)
      tile(std::true_type{}, t, bufc);
    else
      tile(std::false_type{}, t, bufc);
    wait_vmem();
    __syncthreads();
  };
  if (qt0 < nqt) {
    load_ids(qt0);
    wait_vmem();
    __syncthreads();
    stage(qt0, I0{});
  }
  wait_vmem();
  __syncthreads();
  if constexpr ((D == 64 && BQ == 64) || (D == 128 && BQ == 32)) {
    auto fin = [&](auto bi) {
      if constexpr (D == 64) finish(bi); else finish128(bi);
    };
    if (qt0 < nqt) {
      step3(qt0, I0{}, I2{}, std::true_type{});
      for (int t = qt0 + 1; t < nqt; t += 3) {
        step3(t, I1{}, I0{}, std::false_type{});
        if (t + 1 < nqt) step3(t + 1, I2{}, I1{}, std::false_type{});
        if (t + 2 < nqt) step3(t + 2, I0{}, I2{}, std::false_type{});
      }
      const int lastb = (nqt - 1 - qt0) % 3;
      if (lastb == 0)
        fin(I0{});
      else if (lastb == 1)
        fin(I1{});
      else
        fin(I2{});
    }
  } else {
    for (int t = qt0; t < nqt; t += 2) {
      step(t, I0{});
      if (t + 1 < nqt) step(t + 1, I1{});
    }
  }
  if (mykey < a.g_rows) {
    float* dkr = a.dk + b * a.gsb + h * a.gsh + static_cast<int64_t>(mykey) * a.gss;
    float* dvr = a.dv + b * a.gsb + h * a.gsh + static_cast<int64_t>(mykey) * a.gss;
    const bool live = mykey < S;
#pragma unroll
    for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float ns = -a.scale;  // dkacc holds -dS^T Q
        float4 x = make_float4(dkacc[d2][4 * g] * ns, dkacc[d2][4 * g + 1] * ns,
                               dkacc[d2][4 * g + 2] * ns, dkacc[d2][4 * g + 3] * ns);
        float4 y = make_float4(dvacc[d2][4 * g], dvacc[d2][4 * g + 1], dvacc[d2][4 * g + 2],
                               dvacc[d2][4 * g + 3]);
        if (!live) x = y = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dkr + d2 * 32 + g * 8 + hl * 4) = x;
        *reinterpret_cast<float4*>(dvr + d2 * 32 + g * 8 + hl * 4) = y;
      }
  }
}

// -------------------------------------------------------------- query pass (dQ)
// Workgroup = 128 queries (the forward's layout) over key tiles of BN: S^T = K Q^T and
// dP^T = V dO^T (K and V rows staged), dS^T feeds dQ^T = K^T dS^T as the B operand, with K^T
// read from the staged K rows by transposing reads.  One 32-key block at a time, so the
// kernel fits three waves per SIMD at D = 64.
template <int D, int BN, int MODE>
__device__ __forceinline__ void attn_bwd_q_body(const BwdArgs& a) {
  constexpr bool MAPPED = MODE != 0;
  constexpr int BM = 128, NBK = BN / 32;
  using KT = Tile<BN, D>;
  constexpr int NL = KT::LOADS;
  // each buffer its own LDS object, named statically (the loop is unrolled by two)
  __shared__ __attribute__((aligned(16))) uint16_t ks0[BN * D], ks1[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[BN * D], vs1[BN * D];
  __shared__ __attribute__((aligned(16))) int32_t idr[4][BN];

  const int S = a.S, Sp = a.Sp;
  const int nqt = Sp / BM;
  const int64_t item = xcd_item(blockIdx.x, a.BH * nqt);
  const int64_t bh = item / nqt;
  const int qtile = nqt - 1 - static_cast<int>(item % nqt);
  const int64_t b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int Q0 = qtile * BM;
  const int qw = Q0 + wave * 32;
  const int myq = qw + lq;
  const bool causal = a.causal != 0;
  const HeadRows hq = head_rows(a.q, b, h), hk = head_rows(a.k, b, h), hv = head_rows(a.v, b, h);
  const int32_t* gm = MAPPED ? a.gmap + bh * Sp : nullptr;
  const float sl2 = a.sl2;

  bf16x8 qreg[D / 16], oreg[D / 16];
  {
    const int qid = MAPPED ? max(gm[myq], 0) : min(myq, S - 1);
    const uint16_t* qr = row_ptr(hq, qid);
    const uint16_t* dr = a.dout + b * a.dsb + h * a.dsh + static_cast<int64_t>(min(myq, S - 1)) * a.dss;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qreg[kk] = ld_op16(qr + 16 * kk + hl * 8);
      // dO negated (sign bits flipped), so the dP^T product seeded with Delta yields Delta - dP
      const u32x4 u = *reinterpret_cast<const u32x4*>(dr + 16 * kk + hl * 8);
      oreg[kk] = as_bf16x8(u ^ 0x80008000u);
    }
  }
  const float l2 = a.lse[bh * Sp + myq];
  const float dlt = a.delta[bh * Sp + myq];

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int d2 = 0; d2 < D / 32; ++d2) dqacc[d2] = zero16();

  const int kend = causal ? (S < Q0 + BM ? S : Q0 + BM) : S;
  const int nkt = (kend + BN - 1) / BN;
  uint32_t koff[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) koff[j] = op_off<D>(lq, hl, j);

  const LaneStage ls = lane_stage<D>(wave, lane);
  auto load_ids = [&](int t) {
    if constexpr (MAPPED)
      if (wave == 0 && t < nkt) stage_words(gm + t * BN, idr[t & 3], lane, BN);
  };
  // buffer `bi` (a compile-time index) of each kind
  auto kbuf = [&](auto bi) -> uint16_t* {
    if constexpr (decltype(bi)::value == 0) return ks0; else return ks1;
  };
  auto vbuf = [&](auto bi) -> uint16_t* {
    if constexpr (decltype(bi)::value == 0) return vs0; else return vs1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto stage = [&](int t, auto bufc) {
    int id[NL];
    if constexpr (MAPPED) ids_of<BN, D>(idr[t & 3], ls, wave, id);
    load_ids(t + 1);
    if constexpr (MODE == 1) {
      uint32_t o[Tile<BN, D>::LOADS];
      mapped_offsets<BN, D>(id, hk.rsb, ls, o);
      // (D = 128: the two-base form would push this kernel past its register budget)
      stage_mapped32<BN, D, D == 64>(hk, ls, o, kbuf(bufc));
      stage_mapped32<BN, D, D == 64>(hv, ls, o, vbuf(bufc));
    } else if constexpr (MODE == 2) {
      stage_mapped<BN, D>(hk, ls, id, kbuf(bufc), wave);
      stage_mapped<BN, D>(hv, ls, id, vbuf(bufc), wave);
    } else {
      stage_strided<BN, D>(hk, ls, t * BN, S, kbuf(bufc), wave);
      stage_strided<BN, D>(hv, ls, t * BN, S, vbuf(bufc), wave);
    }
  };

  // Tile t, one 32-key block at a time: S^T and dP^T, then dS^T, then its hi-lo split and the
  // dQ^T update.  At D = 64 (three waves per SIMD) the matrix products run at raised wave
  // priority, so a wave with MFMAs to issue goes ahead of the other waves' vector work.
  auto tile = [&](auto masked, int t, auto bufc) {
    const uint16_t* ksb = kbuf(bufc);
    const uint16_t* vsb = vbuf(bufc);
    const int k0 = t * BN;
    uint32_t ko[D / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      ko[j] = koff[j];
      asm volatile("" : "+v"(ko[j]));
    }
#pragma unroll
    for (int b2 = 0; b2 < NBK; ++b2) {
      f32x16 sacc = zero16(), pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = dlt;  // every C register is this lane's query
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        sacc = mfma32(lds_at(ksb, b2 * 64 * D + ko[kk]), qreg[kk], sacc);
        pacc = mfma32(lds_at(vsb, b2 * 64 * D + ko[kk]), oreg[kk], pacc);
      }
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
      // pacc = Delta - dP, so P * pacc = -dS: one multiply; the sign goes into the final scale
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], sl2, -l2));
        if constexpr (decltype(masked)::value) {
          const int key = k0 + b2 * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if ((causal && key > myq) || key >= S) p = 0.f;
        }
        pacc[r] = p * pacc[r];
      }
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int t4 = 2 * b2 + hh;
        bf16x8 sh, sl;
        c_to_op2(pacc, hh, sh, sl);
#pragma unroll
        for (int d2 = 0; d2 < D / 32; ++d2) {
          const uint32_t o0 = t4 * 32 * D + tr_off<D>(lane, d2, 0);
          const uint32_t o1 = t4 * 32 * D + tr_off<D>(lane, d2, 1);
          const bf16x8 ak = tr_op(ksb, o0, o1);
          dqacc[d2] = mfma32(ak, sl, dqacc[d2]);
          dqacc[d2] = mfma32(ak, sh, dqacc[d2]);
        }
      }
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
    }
  };

  // step t: tile t in buffer bufc, tile t + 1 staged into the other of two buffers
  auto step = [&](int t, auto bufc) {
    if (t + 1 < nkt) stage(t + 1, std::integral_constant<int, 1 - decltype(bufc)::value>{});
    const int k0 = t * BN;
    if ((causal && k0 + BN - 1 > qw) || k0 + BN > S)
      tile(std::true_type{}, t, bufc);
    else
      tile(std::false_type{}, t, bufc);
    wait_vmem();
    __syncthreads();
  };
  load_ids(0);
  wait_vmem();
  __syncthreads();
  stage(0, I0{});
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    step(t, I0{});
    if (t + 1 < nkt) step(t + 1, I1{});
  }

  if (myq < a.g_rows) {
    float* dqr = a.dq + b * a.gsb + h * a.gsh + static_cast<int64_t>(myq) * a.gss;
    const bool live = myq < S;
    const float nsc = -a.scale;  // dqacc holds -dQ^T / scale
#pragma unroll
    for (int d2 = 0; d2 < D / 32; ++d2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(dqacc[d2][4 * g] * nsc, dqacc[d2][4 * g + 1] * nsc,
                               dqacc[d2][4 * g + 2] * nsc, dqacc[d2][4 * g + 3] * nsc);
        if (!live) x = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dqr + d2 * 32 + g * 8 + hl * 4) = x;
      }
  }
}

// Occupancy: at D = 64 the key pass runs two waves per SIMD and the query pass three; at
// D = 128 the query pass runs two waves with 32-key tiles, the key pass one wave (its
// accumulators live in AGPRs).
#define LH_KV(NAME, D, BQ, MODE, ATTR)                                    \
  __global__ __launch_bounds__(256) ATTR void NAME(BwdArgs a) {           \
    attn_bwd_kv_body<D, BQ, MODE>(a);                                     \
  }
#define LH_Q(NAME, D, BN, MODE, W)                                                         \
  __global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W, W))) void NAME( \
      BwdArgs a) {                                                                         \
    attn_bwd_q_body<D, BN, MODE>(a);                                                       \
  }
#define LH_TWO_WAVES __attribute__((amdgpu_waves_per_eu(2, 2)))
#define LH_ONE_WAVE
LH_KV(attn_bwd_kv_d64, 64, 64, 0, LH_TWO_WAVES)
LH_KV(attn_bwd_kv_d128, 128, 32, 0, LH_ONE_WAVE)
LH_KV(attn_bwd_kv_mapped_d64, 64, 64, 1, LH_TWO_WAVES)
LH_KV(attn_bwd_kv_mapped_d128, 128, 32, 1, LH_ONE_WAVE)
LH_KV(attn_bwd_kv_mapped64_d64, 64, 64, 2, LH_TWO_WAVES)
LH_KV(attn_bwd_kv_mapped64_d128, 128, 32, 2, LH_ONE_WAVE)
LH_Q(attn_bwd_q_d64, 64, 64, 0, 3)
LH_Q(attn_bwd_q_d128, 128, 32, 0, 2)
LH_Q(attn_bwd_q_mapped_d64, 64, 64, 1, 3)
LH_Q(attn_bwd_q_mapped_d128, 128, 32, 1, 2)
LH_Q(attn_bwd_q_mapped64_d64, 64, 64, 2, 3)
LH_Q(attn_bwd_q_mapped64_d128, 128, 32, 2, 2)
#undef LH_KV
#undef LH_Q
#undef LH_TWO_WAVES
#undef LH_ONE_WAVE

// Delta[b, h, s] = sum_d dO[s, d] O[s, d] for s < S, 0 for the padding up to Sp: one wave per
// row group, D / 8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ dout, int64_t dsb,
                                                   int64_t dsh, int64_t dss,
                                                   const float* __restrict__ o, int64_t osb,
                                                   int64_t osh, int64_t oss,
                                                   float* __restrict__ delta, int64_t BH, int H,
                                                   int S, int Sp) {
  constexpr int G = D / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gid / G;
  const int g = static_cast<int>(gid % G);
  if (row >= BH * Sp) return;
  const int64_t bh = row / Sp;
  const int s = static_cast<int>(row % Sp);
  const int64_t b = bh / H, h = bh % H;
  float part = 0.f;
  if (s < S) {
    const uint4 u = *reinterpret_cast<const uint4*>(dout + b * dsb + h * dsh + s * dss + g * 8);
    const float* orow = o + b * osb + h * osh + s * oss + g * 8;
    const float4 o0 = *reinterpret_cast<const float4*>(orow);
    const float4 o1 = *reinterpret_cast<const float4*>(orow + 4);
    const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part = fmaf(__uint_as_float(w[i] << 16), ov[2 * i], part);
      part = fmaf(__uint_as_float(w[i] & 0xffff0000u), ov[2 * i + 1], part);
    }
  }
  for (int m = 1; m < G; m <<= 1) part += __shfl_xor(part, m);
  if (g == 0) delta[bh * Sp + s] = part;
}

RowSrc strided_rows(const void* x, const int64_t st[3]) {
  RowSrc r;
  r.x = static_cast<const uint16_t*>(x);
  r.px = nullptr;
  r.sb = st[0];
  r.sh = st[1];
  r.ss = st[2];
  r.psb = 0;
  r.n0 = int64_t(1) << 62;
  return r;
}

// Rows of a [B, N, H, D] token tensor and its pooled levels [B, P1, H, D] addressed by
// pyramid id.
RowSrc mapped_rows(const Levels& lv, const void* x, const void* px) {
  RowSrc r;
  r.x = static_cast<const uint16_t*>(x);
  r.px = static_cast<const uint16_t*>(px);
  r.sb = lv.N * lv.H * lv.D;
  r.sh = lv.D;
  r.ss = static_cast<int64_t>(lv.H) * lv.D;
  r.psb = lv.P1 * lv.H * lv.D;
  r.n0 = lv.N;
  return r;
}

}  // namespace

// ------------------------------------------------------------------------ launchers
// Mapped calls use 32-bit row offsets when every pyramid row of a head (N + P1 rows of
// H * D bf16) lies within 4 GiB of the head's first raw row, and ids and the row stride stay
// below 2^24 (the offsets are 24-bit products).
int mapped_mode(const AttnCall& c) {
  if (!c.mapped) return 0;
  const int64_t rows = c.lv->N + c.lv->P1;
  const int64_t rsb = static_cast<int64_t>(c.lv->H) * c.lv->D * 2;
  const int64_t lim24 = int64_t(1) << 24;
  return rows * rsb < (int64_t(1) << 32) && rows <= lim24 && rsb < lim24 ? 1 : 2;
}

hipError_t launch_attn_fwd2(const AttnCall& c, const void* q, const void* k, const void* v,
                            float* o, float* lse, hipStream_t st) {
  FwdArgs a;
  if (c.mapped) {
    a.q = mapped_rows(*c.lv, q, c.pq);
    a.k = mapped_rows(*c.lv, k, c.pk);
    a.v = mapped_rows(*c.lv, v, c.pv);
  } else {
    a.q = strided_rows(q, c.q_stride);
    a.k = strided_rows(k, c.k_stride);
    a.v = strided_rows(v, c.v_stride);
  }
  a.gmap = c.gmap;
  a.o = o;
  a.osb = c.o_stride[0];
  a.osh = c.o_stride[1];
  a.oss = c.o_stride[2];
  a.lse = lse;
  a.BH = c.B * c.H;
  a.H = static_cast<int>(c.H);
  a.S = static_cast<int>(c.S);
  a.Sp = static_cast<int>(padded_len(c.S));
  a.o_rows = c.o_rows;
  a.causal = c.causal;
  a.sl2 = c.scale * kLog2e;
  const unsigned blocks = static_cast<unsigned>(a.BH * (a.Sp / 128));
  static void (*const kern[2][3])(FwdArgs) = {
      {attn_fwd_d64, attn_fwd_mapped_d64, attn_fwd_mapped64_d64},
      {attn_fwd_d128, attn_fwd_mapped_d128, attn_fwd_mapped64_d128}};
  hipLaunchKernelGGL(kern[c.D == 64 ? 0 : 1][mapped_mode(c)], dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd2(int pass, const AttnCall& c, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse,
                            const float* delta, float* dq, float* dk, float* dv, hipStream_t st) {
  BwdArgs a;
  if (c.mapped) {
    a.q = mapped_rows(*c.lv, q, c.pq);
    a.k = mapped_rows(*c.lv, k, c.pk);
    a.v = mapped_rows(*c.lv, v, c.pv);
  } else {
    a.q = strided_rows(q, c.q_stride);
    a.k = strided_rows(k, c.k_stride);
    a.v = strided_rows(v, c.v_stride);
  }
  a.gmap = c.gmap;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dsb = c.do_stride[0];
  a.dsh = c.do_stride[1];
  a.dss = c.do_stride[2];
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.gsb = c.g_stride[0];
  a.gsh = c.g_stride[1];
  a.gss = c.g_stride[2];
  a.BH = c.B * c.H;
  a.H = static_cast<int>(c.H);
  a.S = static_cast<int>(c.S);
  a.Sp = static_cast<int>(padded_len(c.S));
  a.g_rows = c.o_rows;
  a.causal = c.causal;
  a.scale = c.scale;
  a.sl2 = c.scale * kLog2e;
  const unsigned blocks = static_cast<unsigned>(a.BH * (a.Sp / 128));
  const int di = c.D == 64 ? 0 : 1, m = mapped_mode(c);
  static void (*const kv[2][3])(BwdArgs) = {
      {attn_bwd_kv_d64, attn_bwd_kv_mapped_d64, attn_bwd_kv_mapped64_d64},
      {attn_bwd_kv_d128, attn_bwd_kv_mapped_d128, attn_bwd_kv_mapped64_d128}};
  static void (*const qp[2][3])(BwdArgs) = {
      {attn_bwd_q_d64, attn_bwd_q_mapped_d64, attn_bwd_q_mapped64_d64},
      {attn_bwd_q_d128, attn_bwd_q_mapped_d128, attn_bwd_q_mapped64_d128}};
  if (pass & 1) {
    hipLaunchKernelGGL(kv[di][m], dim3(blocks), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pass & 2) hipLaunchKernelGGL(qp[di][m], dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_delta(const AttnCall& c, const void* dout, const float* o, float* delta,
                             hipStream_t st) {
  const int64_t BH = c.B * c.H, Sp = padded_len(c.S);
  const int64_t threads = BH * Sp * (c.D / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  const auto* d = static_cast<const uint16_t*>(dout);
  if (c.D == 64)
    hipLaunchKernelGGL(delta_kernel<64>, grid, dim3(256), 0, st, d, c.do_stride[0],
                       c.do_stride[1], c.do_stride[2], o, c.o_stride[0], c.o_stride[1],
                       c.o_stride[2], delta, BH, static_cast<int>(c.H), static_cast<int>(c.S),
                       static_cast<int>(Sp));
  else
    hipLaunchKernelGGL(delta_kernel<128>, grid, dim3(256), 0, st, d, c.do_stride[0],
                       c.do_stride[1], c.do_stride[2], o, c.o_stride[0], c.o_stride[1],
                       c.o_stride[2], delta, BH, static_cast<int>(c.H), static_cast<int>(c.S),
                       static_cast<int>(Sp));
  return hipGetLastError();
}

}  // namespace lh
