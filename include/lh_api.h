/*
 * lh_api.h -- C ABI of the Lighthouse attention layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (pages cited by title and section heading):
 *   [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复",
 *        section "核心方法：金字塔池化与“外部选择”" (pool, selector, attention call, figure).
 *   [EN] encorp.ai, "Услуги по внедряване на AI задават правилния въпрос за Lighthouse
 *        Attention", sections "Какво точно промени Nous Research в attention пътя?" and
 *        "Как four-stage pipeline остава бърз, без да чупи градиентите?".
 *   [CB] clawdbytes.com, "Lighthouse Attention: the training-time hierarchy that makes
 *        quadratic attention ...", section "Four-Stage Pipeline Wraps Standard FlashAttention".
 *
 *   1. pool   Q, K and V together into an L-level average pyramid, factor p   ([WS] item 1)
 *   2. score  each pooled entry by the l2 norm of its key row, per head       ([EN] four-stage)
 *   3. select per level, per chunk of C consecutive entries, the top entries;
 *             the coarsest level is always kept whole                         ([CB] four-stage)
 *   4. gather the kept entries into one dense sequence ordered by causal
 *             position and run causal softmax attention on it               ([WS] item 3)
 *   5. scatter the outputs back to token positions with a causal offset       ([EN] four-stage)
 *   Backward routes gradients through scatter, attention, gather and pool; the selection
 *   has no gradient ([EN] four-stage; [WS] "深度洞察").
 *
 * Readings of what the pages leave open (used by every entry point below):
 *   - levels l = 0..L-1, level 0 = raw tokens, n_l = N / p^l; p^(L-1) must divide N.
 *   - score = l2 norm of the pooled KEY row of a head (float32); lh_scorer offers two
 *     further readings.
 *   - REFINE (the default mode; DIRECT below is the literal alternative): selection runs at
 *     levels 1..L-1 with budget
 *     k_l = min(k[l], n_l); each kept entry enters the gathered sequence as its p children
 *     one level finer, the coarsest level enters whole, so
 *     S = n_{L-1} + p * sum_{l=1}^{L-1} k_l  (about 65K at N = 1e6, L = 4, p = 4, k = 4096).
 *   - a chunk is C consecutive entries of the level being selected (one chunk holding the
 *     whole level when n_l <= C); chunk c keeps floor(k_l / n_chunks) entries, plus one when
 *     c < k_l mod n_chunks; inside a chunk rank by (score desc, index asc), NaN last.
 *   - entry (l, j) sits at causal position e = (j+1) p^l - 1; gathered order is
 *     (e ascending, l ascending); attention is plain causal softmax, scale 1/sqrt(D).
 *   - scatter adds the output of entry (l, j) to tokens [e, e + p^l - 1] (clipped to N);
 *     tokens reached by no entry get 0.
 *   - gathered Q/K/V and the gathered output-gradient are bfloat16 (round to nearest even);
 *     pooled values and scores are computed in float32; Og, LSE and gathered gradients are
 *     float32; outputs Y, dQ, dK, dV are in the input dtype.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are caller-owned device memory of the current HIP device;
 *     pointers marked "host" are host memory.  The library keeps no pointer after a call
 *     returns and allocates nothing (lh_forward_noalloc uses a static array instead).
 *   - Every device pointer must be 16-byte aligned (LH_ERR_ALIGN otherwise).
 *   - All arguments are validated on the host before the first launch; a call that
 *     returns an error has launched nothing.  Kernel faults surface at the caller's next
 *     synchronisation (or inside the call when the environment sets LH_DEBUG_SYNC=1).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = null stream).
 *     No entry point synchronises the host.  Calls on different streams that touch
 *     different buffers may run concurrently; the library's only mutable global state is
 *     the static workspace of lh_forward_noalloc (see there).
 *   - Tensors are dense and row-major unless strides are given.  Token tensors are
 *     [B, N, H, D].  Gathered-domain tensors store Sp = S rounded up to a multiple of 128
 *     slots: rows [B, H, Sp, D], per-slot vectors [B, H, Sp].  Slots S..Sp-1 are padding;
 *     the library writes them as finite values (zeros for gradients and Delta).
 *   - The forward and backward are deterministic (no atomics, fixed reduction orders).
 */
#ifndef LH_API_H
#define LH_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LH_MAX_LEVELS 8
/* size of the static per-GPU workspace of lh_forward_noalloc (64 MiB) */
#define LH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef void* lh_stream_t; /* hipStream_t */

typedef enum lh_status {
  LH_OK = 0,
  LH_ERR_NULL = -1,        /* a required pointer is NULL                                  */
  LH_ERR_SHAPE = -2,       /* batch/tokens/heads out of range, gathered length S above
                              2^24, or p^(L-1) does not divide N */
  LH_ERR_LEVELS = -3,      /* levels outside [1, LH_MAX_LEVELS]                            */
  LH_ERR_POOL = -4,        /* pool factor outside [2, 16]                                  */
  LH_ERR_K = -5,           /* a budget k[l] < 0                                            */
  LH_ERR_CHUNK = -6,       /* chunk not a power of two in [16, 2048], or a level larger
                              than one chunk is not a whole number of chunks              */
  LH_ERR_DTYPE = -7,       /* dtype or head_dim not supported                              */
  LH_ERR_ALIGN = -8,       /* a device pointer is not 16-byte aligned                      */
  LH_ERR_WORKSPACE = -9,   /* workspace smaller than lh_plan reports                       */
  LH_ERR_LAUNCH = -10,     /* the HIP runtime refused a launch                             */
  LH_ERR_UNSUPPORTED = -11, /* an unknown select_mode or other option                     */
  LH_ERR_SCRATCH = -12     /* lh_forward_noalloc: the forward workspace of this config is
                              larger than LH_NOALLOC_SCRATCH_BYTES                         */
} lh_status;

typedef enum lh_dtype { LH_BF16 = 0, LH_F32 = 1 } lh_dtype;

/* Which entries the selection keeps and how they enter the gathered sequence.  REFINE: k_l
 * entries are kept at levels 1..L-1 and each enters as its p children one level finer
 * (S = n_{L-1} + p * sum k_l; the reading that reproduces the pages' ~65K at N = 1e6).
 * DIRECT: the literal reading -- k_l entries are kept at levels 0..L-2 and enter themselves
 * (S = n_{L-1} + sum k_l).  In both the coarsest level enters whole. */
typedef enum lh_select_mode { LH_SEL_REFINE = 0, LH_SEL_DIRECT = 1 } lh_select_mode;

/* What an entry's score is (the pages name a parameter-free per-head l2-norm scorer -- the
 * projection-norm scorer of [CB] "The Bottom Line" -- without naming the vector):
 * K   = ||k_bar||, the pooled key row's norm (the default reading);
 * QK  = ||q_bar|| * ||k_bar||;
 * QKV = ||[q_bar; k_bar; v_bar]|| = sqrt(||q_bar||^2 + ||k_bar||^2 + ||v_bar||^2).
 * Norms are per head, of the float32 pooled rows, summed in float64. */
typedef enum lh_scorer { LH_SCORE_K = 0, LH_SCORE_QK = 1, LH_SCORE_QKV = 2 } lh_scorer;

/* Problem statement of one layer call: the pages' N, heads, head_dim, L, p, per-level k and
   chunk size ([EN] attention-path section gives N, L, p, k; [WS] item 2 the chunked top-K). */
typedef struct lh_config {
  int64_t batch;          /* B >= 1                                                      */
  int64_t n_tokens;       /* N >= 1, p^(L-1) divides N, N <= 2^30                         */
  int32_t heads;          /* H >= 1 (queries and keys share heads)                        */
  int32_t head_dim;       /* D in {64, 128}                                               */
  int32_t levels;         /* L in [1, 8]; L = 1 is dense causal attention (S = N)         */
  int32_t pool;           /* p in [2, 16]                                                 */
  int32_t k[LH_MAX_LEVELS]; /* k[l] = kept entries at selected level l (REFINE l = 1..L-1,
                               DIRECT l = 0..L-2); other entries unused; k[l] >= n_l
                               keeps the whole level                                     */
  int32_t chunk;          /* C: power of two in [16, 2048]                                */
  int32_t dtype;          /* lh_dtype of Q, K, V, Y, dY, dQ, dK, dV                       */
  int32_t select_mode;    /* lh_select_mode                                               */
  float softmax_scale;    /* <= 0 selects 1/sqrt(D)                                       */
  int32_t scorer;         /* lh_scorer (0 = K, the l2 norm of the pooled key row)          */
} lh_config;

/* Sizes derived from a config by closed forms (host struct filled by lh_plan). */
typedef struct lh_plan_info {
  int64_t level_size[LH_MAX_LEVELS];   /* n_l                                             */
  int64_t level_offset[LH_MAX_LEVELS]; /* pyramid id of (l, j) = level_offset[l] + j      */
  int64_t pooled_offset[LH_MAX_LEVELS];/* row of level l (l >= 1) in the pooled tensors   */
  int64_t pyramid_total;               /* P = sum_l n_l                                   */
  int64_t pooled_rows;                 /* sum_{l>=1} n_l                                  */
  int64_t k_eff[LH_MAX_LEVELS];        /* min(k[l], n_l) at selected levels, else 0       */
  int64_t n_chunks[LH_MAX_LEVELS];     /* chunks at selected levels, else 0               */
  int64_t chunk_width[LH_MAX_LEVELS];  /* entries per chunk at selected levels            */
  int64_t quota_base[LH_MAX_LEVELS];   /* every chunk of level l keeps quota_base[l] ...  */
  int64_t quota_rem[LH_MAX_LEVELS];    /* ... plus one for chunks c < quota_rem[l]        */
  int64_t sel_offset[LH_MAX_LEVELS];   /* start of level l's kept indices in `sel`        */
  int64_t sel_total;                   /* sum_l k_eff[l]                                  */
  int64_t gathered_len;                /* S (the same for every batch and head)           */
  int64_t gathered_pad;                /* Sp = S rounded up to a multiple of 128: the
                                          stored length of every gathered-domain tensor  */
  /* byte offsets of the pieces of the `saved` blob written by lh_forward: the map (gmap
     [B,H,Sp] and inv [B,H,P] int32), the pooled levels of Q, K, V ([B, pooled_rows, H, D]
     bf16), the attention output Og ([B,H,Sp,D] float32) and its log-sum-exp ([B,H,Sp]) */
  size_t saved_gmap, saved_inv, saved_pq, saved_pk, saved_pv, saved_o, saved_lse;
  size_t saved_bytes;                  /* size of the `saved` blob                        */
  size_t ws_forward_bytes;             /* workspace lh_forward needs (scores, selection)  */
  size_t ws_backward_bytes;            /* workspace lh_backward needs                     */
  float softmax_scale;                 /* the scale actually used                         */
} lh_plan_info;

/* Validate `cfg` and fill `info` (host). Touches no device. */
lh_status lh_plan(const lh_config* cfg, lh_plan_info* info);

/* Static, NUL-terminated description of a status code (host). */
const char* lh_status_string(lh_status status);

/* ---------------------------------------------------------------------------------------
 * Stage entry points (each one stage of the path, for parity checks and per-stage timing)
 * ------------------------------------------------------------------------------------- */

/* Stage 1+2 ([WS] item 1; [EN] four-stage): pool Q, K, V into levels 1..L-1 and score.
 *   q, k, v  device [B, N, H, D] in cfg->dtype
 *   pq,pk,pv device [B, pooled_rows, H, D] in pooled_dtype; level l (l >= 1) occupies rows
 *            pooled_offset[l] .. pooled_offset[l] + n_l - 1; each is the mean of p entries of
 *            the level below (float32 arithmetic, one rounding if pooled_dtype is bf16)
 *   scores   device float32 [B, H, pyramid_total], indexed by pyramid id; levels 1..L-1 are
 *            written, and level 0 (the raw key rows) too in DIRECT; REFINE leaves level 0
 *            untouched
 *   Any of pq/pk/pv may be NULL to skip that stream's pooled output (scores are computed
 *   either way).  With L = 1 nothing is launched. */
lh_status lh_pool_score(const lh_config* cfg, const void* q, const void* k, const void* v,
                        void* pq, void* pk, void* pv, int32_t pooled_dtype, float* scores,
                        lh_stream_t stream);

/* Stage 3 ([WS] item 2; [CB] four-stage): chunked bitonic top-K per selected level.
 *   scores device float32 [B, H, pyramid_total] from lh_pool_score
 *   sel    device int32 [B, H, sel_total]; level l's kept level-local indices, ascending,
 *          at sel_offset[l] .. sel_offset[l] + k_eff[l] - 1 */
lh_status lh_topk(const lh_config* cfg, const float* scores, int32_t* sel, lh_stream_t stream);

/* Stages 1-3 as one call ([WS] item 1 and item 2): the pooled rows of lh_pool_score and the
 * selection of lh_topk, identical to calling the two in turn.  Where a chunk of the finest
 * selected level f covers a whole number of coarsest blocks (C p^f a multiple of p^(L-1)),
 * one workgroup per chunk pools its token span, keeps level f's scores on chip and selects
 * that chunk in place; scores[.., level f] are then NOT written (every other level's are),
 * and the coarser selected levels follow in a second launch.  Otherwise the two stages run
 * as separate launches and every score is written.  Arguments as in lh_pool_score and
 * lh_topk; sel may be NULL only when sel_total is 0.  (lh_forward runs the two stages as
 * separate launches, which measure faster on MI355X: the pooling is HBM-bound either way.) */
lh_status lh_pool_score_topk(const lh_config* cfg, const void* q, const void* k, const void* v,
                             void* pq, void* pk, void* pv, int32_t pooled_dtype, float* scores,
                             int32_t* sel, lh_stream_t stream);

/* Stage 4a ([EN] four-stage, [WS] item 3): the gathered order.
 *   sel  device int32 [B, H, sel_total] from lh_topk
 *   gmap device int32 [B, H, Sp]: pyramid id of each gathered slot, in (e, l) order;
 *        padding slots hold -1
 *   inv  device int32 [B, H, pyramid_total]: slot of each pyramid entry, or -1 */
lh_status lh_build_map(const lh_config* cfg, const int32_t* sel, int32_t* gmap, int32_t* inv,
                       lh_stream_t stream);

/* Stage 4 as one call: the map of lh_build_map, then the gathered rows.  Slot s of head
 * (b, h) receives the row of pyramid entry gmap[s] -- a raw token of q/k/v (level 0) or a
 * pooled row of pq/pk/pv (level >= 1) -- rounded to bfloat16; padding slots are zero rows.
 *   q, k, v  as in lh_pool_score; pq, pk, pv in pooled_dtype (may be NULL when L = 1)
 *   sel      device int32 [B, H, sel_total];  gmap, inv as in lh_build_map (written)
 *   qg,kg,vg device bf16 [B, H, Sp, D] (written)
 * lh_forward does not call this: its attention reads the same rows through gmap. */
lh_status lh_gather(const lh_config* cfg, const void* q, const void* k, const void* v,
                    const void* pq, const void* pk, const void* pv, int32_t pooled_dtype,
                    const int32_t* sel, int32_t* gmap, int32_t* inv, void* qg, void* kg,
                    void* vg, lh_stream_t stream);

/* Causal (or full) softmax attention ([WS] item 3; [HE] news.hamidun.com, "Nous Research
 * introduced Lighthouse Attention ...", section "How Lighthouse Attention Works": the layer
 * wraps ordinary scaled dot-product attention), over rows given by strides: element
 * (b, h, s, d) of q is q[b*q_stride[0] + h*q_stride[1] + s*q_stride[2] + d] (d contiguous),
 * likewise k, v and o.  Dense attention on [B, N, H, D] tensors uses strides
 * (N*H*D, D, H*D); a gathered [B, H, S, D] tensor (H*S*D, S*D, D). */
typedef struct lh_attn_desc {
  int64_t batch, heads, seq, head_dim; /* B, H, S, D; D in {64, 128}; 1 <= S <= 2^24       */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3]; /* elements, (b, h, s)   */
  int32_t causal;                      /* 1: key s' <= query s; 0: every key             */
  float scale;                         /* <= 0 selects 1/sqrt(D)                        */
} lh_attn_desc;

/* O[s] = sum_{s' <= s} softmax(scale * q[s].k[s']) v[s'] (all s' when causal = 0);
 * lse[s] = log2 of sum_{s'} 2^(scale * log2(e) * q[s].k[s']), the row's log-sum-exp in base 2
 * (the natural log-sum-exp times log2(e)).
 *   q, k, v device bf16 rows (16-byte aligned, every stride a multiple of 8)
 *   o       device float32 rows at o_stride; rows s < S are written
 *   lse     device float32 [B, H, Sp] (Sp = S rounded up to 128; padding entries finite) */
lh_status lh_attn_fwd(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                      float* o, float* lse, lh_stream_t stream);

/* Bytes of workspace lh_attn_bwd needs (Delta = rowsum(dO * O), float32 [B, H, Sp]). */
lh_status lh_attn_ws_bytes(const lh_attn_desc* desc, size_t* bytes);

/* Backward of lh_attn_fwd for the upstream gradient dout (bf16 rows at o_stride), from its
 * o and lse: dV = P^T dO, dP = dO V^T, dS = P (dP - Delta), dQ = scale dS K, dK = scale dS^T Q.
 *   dq, dk, dv device float32 rows at o_stride (rows s < S written); ws as above. */
lh_status lh_attn_bwd(const lh_attn_desc* desc, const void* q, const void* k, const void* v,
                      const float* o, const float* lse, const void* dout, float* dq, float* dk,
                      float* dv, void* ws, size_t ws_bytes, lh_stream_t stream);

/* The attention of the layer with its rows read through the map (no gathered copy): slot s
 * of head (b, h) is pyramid entry gmap[s] of q/k/v (level 0) or pq/pk/pv (pooled levels,
 * bf16, as written by lh_pool_score).  Causal, scale cfg->softmax_scale.
 *   og  device float32 [B, H, Sp, D] (every slot written; padding rows finite)
 *   lse device float32 [B, H, Sp] */
lh_status lh_attn_fwd_mapped(const lh_config* cfg, const void* q, const void* k, const void* v,
                             const void* pq, const void* pk, const void* pv,
                             const int32_t* gmap, float* og, float* lse, lh_stream_t stream);

/* Backward of lh_attn_fwd_mapped.  passes: 1 = key pass (dkg, dvg), 2 = query pass (dqg),
 * 3 = both; an argument a selected pass does not write may be NULL.
 *   lse, delta device float32 [B, H, Sp] (delta from lh_scatter_bwd)
 *   dog        device bf16 [B, H, Sp, D] (from lh_scatter_bwd)
 *   dqg, dkg, dvg device float32 [B, H, Sp, D] (padding rows zero) */
lh_status lh_attn_bwd_mapped(const lh_config* cfg, const void* q, const void* k, const void* v,
                             const void* pq, const void* pk, const void* pv,
                             const int32_t* gmap, const float* lse, const float* delta,
                             const void* dog, float* dqg, float* dkg, float* dvg, int32_t passes,
                             lh_stream_t stream);

/* Stage 5 ([EN] four-stage): Y[b, t, h] = sum_l og[b, h, inv(l, floor((t+1)/p^l) - 1)]
 * over gathered entries, one float32 sum, one rounding to cfg->dtype.
 *   inv device int32 [B, H, pyramid_total]; og device float32 [B, H, Sp, D]
 *   y   device [B, N, H, D] in cfg->dtype (fully overwritten) */
lh_status lh_scatter(const lh_config* cfg, const int32_t* inv, const float* og, void* y,
                     lh_stream_t stream);

/* Adjoint of lh_scatter: dOg[s] = sum of dY over the tokens slot s reached, rounded to
 * bf16; delta[s] = sum_d dOg[s, d] * og[s, d] (the attention backward's Delta, fused here).
 *   gmap device int32 [B, H, Sp]; og device float32 [B, H, Sp, D]
 *   dy device [B, N, H, D] in cfg->dtype
 *   dog device bf16 [B, H, Sp, D]; delta device float32 [B, H, Sp]; padding slots zero */
lh_status lh_scatter_bwd(const lh_config* cfg, const int32_t* gmap, const float* og,
                         const void* dy, void* dog, float* delta, lh_stream_t stream);

/* Adjoint of gather o pool ([EN] four-stage: gradients reach Q, K, V through the gathered
 * values only): dX[b, t, h] = sum_l [entry (l, floor(t/p^l)) gathered] dXg[slot] / p^l.
 *   inv device int32 [B, H, pyramid_total]; dqg, dkg, dvg device float32 [B, H, Sp, D]
 *   dq, dk, dv device [B, N, H, D] in cfg->dtype (fully overwritten) */
lh_status lh_gather_pool_bwd(const lh_config* cfg, const int32_t* inv, const float* dqg,
                             const float* dkg, const float* dvg, void* dq, void* dk, void* dv,
                             lh_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Whole layer
 * ------------------------------------------------------------------------------------- */

/* Forward: stages 1-5 (pool+score, top-K, map, attention through the map, scatter).
 *   q, k, v device [B, N, H, D] in cfg->dtype;  y device [B, N, H, D] in cfg->dtype
 *   saved   device blob of lh_plan_info.saved_bytes, written here and read by lh_backward
 *           (map, pooled levels, Og and LSE at the saved_* offsets)
 *   ws      device workspace of at least ws_forward_bytes (contents undefined after) */
lh_status lh_forward(const lh_config* cfg, const void* q, const void* k, const void* v,
                     void* y, void* saved, void* ws, size_t ws_bytes, lh_stream_t stream);

/* lh_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Identical kernels and results; the
 * forward workspace comes from a static array of LH_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends (looked up once per device with
 * hipGetSymbolAddress).  Configs with ws_forward_bytes above that size are rejected with
 * LH_ERR_SCRATCH before anything is launched.  It calls no allocating routine.  Every call on
 * one GPU shares that GPU's array (whose contents are whatever the last call left; nothing
 * in it needs to start at zero), so calls that overlap on one GPU -- on different streams or
 * from different threads -- race: serialise them.  Uses the current HIP device. */
lh_status lh_forward_noalloc(const lh_config* cfg, const void* q, const void* k, const void* v,
                             void* y, void* saved, lh_stream_t stream);

/* Backward with the selection frozen at what lh_forward saved.  The attention rows are read
 * again through the map, so the forward's inputs q, k, v are passed too (unchanged since
 * lh_forward, as an autograd framework keeps them).
 *   q, k, v device [B, N, H, D] in cfg->dtype; saved as written by lh_forward
 *   dy device [B, N, H, D] in cfg->dtype; dq, dk, dv device [B, N, H, D] in cfg->dtype
 *   ws device workspace of at least ws_backward_bytes */
lh_status lh_backward(const lh_config* cfg, const void* q, const void* k, const void* v,
                      const void* saved, const void* dy, void* dq, void* dk, void* dv, void* ws,
                      size_t ws_bytes, lh_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LH_API_H */
