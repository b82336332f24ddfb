"""Plain, slow CPU oracle of the Lighthouse attention layer (forward and backward).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and its Python
binding) never imports, links or calls it, and this module imports nothing from the product.

Everything here is NumPy float64, one (batch, head) at a time, written to be checked by eye
against the pages. Library routines used as steps: matmul, exp/log, sort/lexsort, fancy
indexing. There is no blocking, fusion or reordering beyond what the definitions state
(the attention loop walks query rows in groups; each row's softmax is exact and complete).

Pages cited (titles as published; sections by their headings):
  [WS] wispaper.ai, "Lighthouse Attention：预训练长文本的高速公路，训练提速 21 倍且无损恢复"
       section "核心方法：金字塔池化与“外部选择”" (items 1 pyramid pool, 2 hierarchical
       selector, 3 FlashAttention call, and the architecture figure caption), section
       "深度洞察" (gradient flow).
  [EN] encorp.ai, "Услуги по внедряване на AI задават правилния въпрос за Lighthouse
       Attention", sections "Какво точно промени Nous Research в attention пътя?" (the
       N = 1,000,000 worked size) and "Как four-stage pipeline остава бърз, без да чупи
       градиентите?" (the four stages, the causality-preserving scatter offset, the
       non-differentiable top-K).
  [CB] clawdbytes.com, "Lighthouse Attention: the training-time hierarchy that makes
       quadratic attention ...", sections "The Core Innovation: Symmetric Pyramid Pooling"
       and "Four-Stage Pipeline Wraps Standard FlashAttention" (stratified chunked top-K,
       coarsest level kept whole).
  [HE] news.hamidun.com, "Nous Research introduced Lighthouse Attention to accelerate LLM
       training", section "How Lighthouse Attention Works" (wraps ordinary SDPA).

Readings of what the pages leave open (each is restated where it is used):
  R1 levels l = 0..L-1, level 0 = the raw tokens, n_l = N / p**l, p**(L-1) must divide N.
  R2 pooling = non-overlapping mean of p consecutive entries of the level below.
  R3 score = l2 norm of the pooled KEY row of one head (scorer "k").  The pages name a
     per-head l2-norm (projection-norm) scorer without naming the vector; two further readings
     are kept as options: "qk" = ||q_bar|| * ||k_bar|| and "qkv" = the l2 norm of the
     concatenated row [q_bar; k_bar; v_bar].
  R4 REFINE selection: at levels l = 1..L-1 keep k_l = min(k[l], n_l) entries; each kept
     entry enters the gathered sequence as its p children one level finer; the coarsest
     level enters whole.  S = n_{L-1} + p * sum_l k_l (reproduces the pages' ~65K at
     N = 1e6, L = 4, p = 4, k = 4096).  DIRECT (the literal reading) keeps k entries at
     levels 0..L-2 and gathers them themselves.
  R5 chunks = C consecutive entries of the level being selected (one chunk if n_l <= C);
     quotas split k_l evenly, the first (k_l mod n_chunks) chunks take one more.
  R6 rank inside a chunk by (score descending, index ascending); NaN ranks last.
  R7 causal position of entry (l, j) is e = (j+1) * p**l - 1, the last token of its block;
     the gathered sequence is ordered by (e ascending, l ascending).
  R8 attention = plain causal softmax attention over the gathered order, scale 1/sqrt(D).
  R9 scatter: entry (l, j) is added to the tokens [e, e + p**l - 1] (clipped to N); tokens
     that receive nothing are 0.  Contributions of several levels are summed.
  R10 gathered Q/K/V and the gathered output-gradient are rounded to bfloat16 (round to
     nearest even) before attention when the attention runs in bf16.
  R11 backward: selection is frozen (no gradient into scores); pooling's adjoint gives each
     source token 1/p**l of its pooled entry's gradient.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

REFINE = "refine"
DIRECT = "direct"
SCORERS = ("k", "qk", "qkv")


# --------------------------------------------------------------------------------------
# configuration and sizes
# --------------------------------------------------------------------------------------
@dataclass
class Config:
    """Layer hyper-parameters: the pages' problem statement (N, L, p, per-level k, chunk).

    [EN] "Какво точно промени Nous Research в attention пътя?" names N, L, p and k;
    [WS] item 2 and [CB] "Four-Stage Pipeline" name the chunked top-K.
    """

    levels: int
    pool: int
    k: list  # k[l]; REFINE reads l = 1..L-1, DIRECT reads l = 0..L-2
    chunk: int
    mode: str = REFINE
    scale: float | None = None  # None -> 1/sqrt(D)   (reading R8)
    bf16_attention: bool = True  # reading R10
    scorer: str = "k"  # reading R3: "k", "qk" or "qkv"
    k_list: list = field(init=False)

    def __post_init__(self):
        if isinstance(self.k, int):
            self.k_list = [self.k] * self.levels
        else:
            self.k_list = list(self.k)
            if len(self.k_list) < self.levels:
                raise ValueError("k must give one budget per level")
        if self.levels < 1 or self.pool < 2 or self.chunk < 1:
            raise ValueError("need L >= 1, p >= 2, chunk >= 1")
        if self.mode not in (REFINE, DIRECT):
            raise ValueError("mode must be refine or direct")
        if self.scorer not in SCORERS:
            raise ValueError(f"scorer must be one of {SCORERS}")


def level_sizes(n_tokens: int, levels: int, pool: int) -> list:
    """n_l = N / p**l for l = 0..L-1 (reading R1)."""
    if n_tokens % pool ** (levels - 1):
        raise ValueError("p**(L-1) must divide N")
    return [n_tokens // pool**lv for lv in range(levels)]


def level_offsets(sizes: list) -> list:
    """Pyramid id of entry (l, j) is offsets[l] + j."""
    return [int(sum(sizes[:lv])) for lv in range(len(sizes))]


def selected_levels(cfg: Config) -> list:
    """Levels that selection runs on (reading R4)."""
    if cfg.mode == REFINE:
        return list(range(1, cfg.levels))
    return list(range(0, cfg.levels - 1))


def gathered_length(n_tokens: int, cfg: Config) -> int:
    """S, counted from the definition of the gathered set (reading R4)."""
    sizes = level_sizes(n_tokens, cfg.levels, cfg.pool)
    s = sizes[-1]
    for lv in selected_levels(cfg):
        kl = min(cfg.k_list[lv], sizes[lv])
        s += kl * (cfg.pool if cfg.mode == REFINE else 1)
    return s


# --------------------------------------------------------------------------------------
# bfloat16 rounding (reading R10), written from the format's definition
# --------------------------------------------------------------------------------------
_BF16_MAX = (2.0 - 2.0**-7) * 2.0**127


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even; returns float64.

    bfloat16 keeps 8 significant bits and float32's exponent range: for |x| in
    [2**(e-1), 2**e) the spacing is 2**(e-8); below the smallest normal 2**-126 the spacing
    is fixed at 2**-133. Values past the largest finite bf16 after rounding become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        quantum = np.ldexp(1.0, e - 8)
        r = np.rint(x / quantum) * quantum  # np.rint rounds half to even
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    return r


# --------------------------------------------------------------------------------------
# stage 1: symmetric pyramid pool   ([WS] item 1; [CB] "The Core Innovation")
# --------------------------------------------------------------------------------------
def pool_pyramid(x: np.ndarray, levels: int, pool: int) -> list:
    """Average-pool one head's rows [N, D] into levels 0..L-1 (readings R1, R2).

    The same operator is applied to Q, K and V: the pages pool all three together.
    """
    out = [np.asarray(x, dtype=np.float64)]
    for _ in range(1, levels):
        prev = out[-1]
        out.append(prev.reshape(prev.shape[0] // pool, pool, prev.shape[1]).mean(axis=1))
    return out


# --------------------------------------------------------------------------------------
# stage 2: parameter-free per-head l2 score   ([EN] four-stage section; [CB] "Four-Stage"
#          and "The Bottom Line" for the projection-norm scorer of the recommended recipe)
# --------------------------------------------------------------------------------------
def row_norms(levels: list) -> list:
    """l2 norm of every row of every level."""
    return [np.sqrt(np.sum(x * x, axis=1)) for x in levels]


def score_pyramid(k_levels: list, scorer: str = "k", q_levels=None, v_levels=None) -> list:
    """Score of each pooled entry of one head (reading R3).

    "k":   ||k_bar||, the norm of the pooled key row;
    "qk":  ||q_bar|| * ||k_bar||;
    "qkv": ||[q_bar; k_bar; v_bar]|| = sqrt(||q_bar||^2 + ||k_bar||^2 + ||v_bar||^2).
    """
    nk = row_norms(k_levels)
    if scorer == "k":
        return nk
    nq = row_norms(q_levels)
    if scorer == "qk":
        return [a * b for a, b in zip(nq, nk)]
    if scorer == "qkv":
        nv = row_norms(v_levels)
        return [np.sqrt(a * a + b * b + c * c) for a, b, c in zip(nq, nk, nv)]
    raise ValueError(f"unknown scorer {scorer}")


# --------------------------------------------------------------------------------------
# stage 3: chunked, stratified top-K   ([WS] item 2; [CB] "Four-Stage Pipeline")
# --------------------------------------------------------------------------------------
def chunk_layout(n: int, chunk: int) -> tuple:
    """(number of chunks, chunk width) for a level of n entries (reading R5)."""
    if n <= chunk:
        return 1, n
    if n % chunk:
        raise ValueError("a level larger than one chunk must be a whole number of chunks")
    return n // chunk, chunk


def chunk_quotas(k_eff: int, n_chunks: int) -> list:
    """Even split of the level budget over chunks, first chunks take the remainder (R5)."""
    base, rem = divmod(k_eff, n_chunks)
    return [base + (1 if c < rem else 0) for c in range(n_chunks)]


def select_level(scores: np.ndarray, k: int, chunk: int) -> np.ndarray:
    """Indices kept at one level, ascending (readings R5, R6).

    Inside each chunk the entries are ranked by score (high first), ties by lower index,
    NaN scores last, and the chunk keeps its quota.
    """
    n = scores.shape[0]
    k_eff = min(k, n)
    n_chunks, width = chunk_layout(n, chunk)
    quotas = chunk_quotas(k_eff, n_chunks)
    kept = []
    for c in range(n_chunks):
        idx = np.arange(c * width, (c + 1) * width)
        s = scores[idx]
        nan = np.isnan(s)
        order = np.lexsort((idx, np.where(nan, 0.0, -s), nan))
        kept.append(np.sort(idx[order[: quotas[c]]]))
    return np.concatenate(kept).astype(np.int64) if kept else np.zeros(0, np.int64)


# --------------------------------------------------------------------------------------
# stage 4a: the gathered set and its causal order   ([EN] four-stage section; [WS] item 3)
# --------------------------------------------------------------------------------------
def causal_position(level: np.ndarray, j: np.ndarray, pool: int) -> np.ndarray:
    """e(l, j) = (j+1) * p**l - 1: the last token the pooled entry summarises (R7)."""
    return (np.asarray(j, np.int64) + 1) * (pool ** np.asarray(level, np.int64)) - 1


def gathered_set(sel: dict, sizes: list, cfg: Config) -> tuple:
    """Levels and level-local indices of the gathered entries, in gathered order.

    REFINE (R4): every coarsest entry, plus the p children of each kept entry.
    DIRECT: every coarsest entry, plus the kept entries themselves.
    Order: causal position ascending, then level ascending (R7).
    """
    top = cfg.levels - 1
    lv = [np.full(sizes[top], top, np.int64)]
    jj = [np.arange(sizes[top], dtype=np.int64)]
    for level in selected_levels(cfg):
        kept = np.asarray(sel[level], np.int64)
        if cfg.mode == REFINE:
            children = (kept[:, None] * cfg.pool + np.arange(cfg.pool)[None, :]).reshape(-1)
            lv.append(np.full(children.shape[0], level - 1, np.int64))
            jj.append(children)
        else:
            lv.append(np.full(kept.shape[0], level, np.int64))
            jj.append(kept)
    lv = np.concatenate(lv)
    jj = np.concatenate(jj)
    e = causal_position(lv, jj, cfg.pool)
    order = np.lexsort((lv, e))
    return lv[order], jj[order]


def inverse_map(glev: np.ndarray, gidx: np.ndarray, sizes: list) -> list:
    """Per level, the gathered slot of each entry, or -1 when it is not gathered."""
    inv = [np.full(n, -1, np.int64) for n in sizes]
    for s, (lv, j) in enumerate(zip(glev.tolist(), gidx.tolist())):
        if inv[lv][j] != -1:
            raise AssertionError("entry gathered twice")
        inv[lv][j] = s
    return inv


# --------------------------------------------------------------------------------------
# stage 4b: causal attention on the gathered sequence   ([WS] item 3; [HE] "How ...")
# --------------------------------------------------------------------------------------
def causal_attention(q, k, v, scale, rows=512, causal=True):
    """O[s] = sum_{s' <= s} softmax_{s'}(scale * q[s].k[s']) v[s'], with the log-sum-exp.

    Plain softmax attention (reading R8): no dropout, bias, window or sink.  With
    causal=False every key is attended (the same softmax without the mask).
    """
    n = q.shape[0]
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        kend = r1 if causal else k.shape[0]
        logits = (q[r0:r1] @ k[:kend].T) * scale
        future = np.arange(kend)[None, :] > np.arange(r0, r1)[:, None]
        if causal:
            logits[future] = -np.inf
        m = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - m)
        z = w.sum(axis=1, keepdims=True)
        o[r0:r1] = (w / z) @ v[:kend]
        lse[r0:r1] = (m + np.log(z))[:, 0]
    return o, lse


def causal_attention_backward(q, k, v, o, lse, do, scale, rows=512, causal=True):
    """Gradients of causal_attention for upstream gradient do (selection frozen).

    With P the attention weights: dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dO*O));
    dQ = scale * dS K; dK = scale * dS^T Q.
    """
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.sum(do * o, axis=1)
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        kend = r1 if causal else k.shape[0]
        logits = (q[r0:r1] @ k[:kend].T) * scale
        future = np.arange(kend)[None, :] > np.arange(r0, r1)[:, None]
        if causal:
            logits[future] = -np.inf
        p = np.exp(logits - lse[r0:r1, None])
        dv[:kend] += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v[:kend].T
        ds = p * (dp - delta[r0:r1, None])
        dq[r0:r1] = scale * (ds @ k[:kend])
        dk[:kend] += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# stage 5: scatter back with the causality-preserving offset   ([EN] four-stage section)
# --------------------------------------------------------------------------------------
def scatter(og: np.ndarray, inv: list, n_tokens: int, pool: int) -> np.ndarray:
    """Y[t] = sum over levels l of Og[slot of (l, floor((t+1)/p**l) - 1)] (reading R9).

    Entry (l, j) reaches tokens t with floor((t+1)/p**l) - 1 == j, i.e. [e, e + p**l - 1].
    """
    y = np.zeros((n_tokens, og.shape[1]))
    t = np.arange(n_tokens, dtype=np.int64)
    for lv, inv_l in enumerate(inv):
        j = (t + 1) // pool**lv - 1
        ok = j >= 0
        slot = np.full(n_tokens, -1, np.int64)
        slot[ok] = inv_l[j[ok]]
        hit = slot >= 0
        y[hit] += og[slot[hit]]
    return y


def scatter_backward(dy: np.ndarray, glev, gidx, pool: int) -> np.ndarray:
    """dOg[s] = sum of dY over the tokens slot s was scattered to (adjoint of scatter)."""
    n = dy.shape[0]
    e = causal_position(glev, gidx, pool)
    span = pool ** np.asarray(glev, np.int64)
    dog = np.zeros((len(glev), dy.shape[1]))
    for s in range(len(glev)):
        lo = int(e[s])
        hi = min(n, lo + int(span[s]))
        dog[s] = dy[lo:hi].sum(axis=0)
    return dog


def gather_pool_backward(dxg: np.ndarray, inv: list, n_tokens: int, pool: int) -> np.ndarray:
    """dX[t] = sum_l [entry (l, floor(t/p**l)) gathered] * dXg[slot] / p**l  (reading R11).

    The adjoint of "gather the pooled entry" composed with "mean over its p**l tokens".
    """
    dx = np.zeros((n_tokens, dxg.shape[1]))
    t = np.arange(n_tokens, dtype=np.int64)
    for lv, inv_l in enumerate(inv):
        slot = inv_l[t // pool**lv]
        hit = slot >= 0
        dx[hit] += dxg[slot[hit]] / float(pool**lv)
    return dx


# --------------------------------------------------------------------------------------
# one (batch, head): the whole layer
# --------------------------------------------------------------------------------------
@dataclass
class HeadState:
    """What one head's forward produced (and its backward needs)."""

    sizes: list
    q_levels: list
    k_levels: list
    v_levels: list
    scores: list
    sel: dict
    glev: np.ndarray
    gidx: np.ndarray
    inv: list
    qg: np.ndarray
    kg: np.ndarray
    vg: np.ndarray
    og: np.ndarray
    lse: np.ndarray
    scale: float


def head_selection(k: np.ndarray, cfg: Config, sizes=None, q=None, v=None):
    """Pool, score and select (stages 1-3); q and v are needed by the "qk"/"qkv" scorers."""
    n = k.shape[0]
    sizes = sizes or level_sizes(n, cfg.levels, cfg.pool)
    k_levels = pool_pyramid(k, cfg.levels, cfg.pool)
    q_levels = pool_pyramid(q, cfg.levels, cfg.pool) if cfg.scorer != "k" else None
    v_levels = pool_pyramid(v, cfg.levels, cfg.pool) if cfg.scorer == "qkv" else None
    scores = score_pyramid(k_levels, cfg.scorer, q_levels, v_levels)
    sel = {lv: select_level(scores[lv], cfg.k_list[lv], cfg.chunk) for lv in selected_levels(cfg)}
    return k_levels, scores, sel


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, cfg: Config, sel=None) -> tuple:
    """Forward of one (batch, head); q, k, v are [N, D]. Returns (Y [N, D], HeadState).

    `sel` (optional, {level: ascending kept indices}) replaces the top-K step's result, so
    the remaining steps can be checked on a selection made elsewhere.
    """
    n, d = q.shape
    sizes = level_sizes(n, cfg.levels, cfg.pool)
    q_levels = pool_pyramid(q, cfg.levels, cfg.pool)
    v_levels = pool_pyramid(v, cfg.levels, cfg.pool)
    k_levels, scores, own_sel = head_selection(k, cfg, sizes, q=q, v=v)
    sel = own_sel if sel is None else {lv: np.asarray(sel[lv], np.int64) for lv in own_sel}
    glev, gidx = gathered_set(sel, sizes, cfg)
    inv = inverse_map(glev, gidx, sizes)
    rnd = round_bf16 if cfg.bf16_attention else (lambda a: a)
    qg = rnd(np.stack([q_levels[a][b] for a, b in zip(glev.tolist(), gidx.tolist())]))
    kg = rnd(np.stack([k_levels[a][b] for a, b in zip(glev.tolist(), gidx.tolist())]))
    vg = rnd(np.stack([v_levels[a][b] for a, b in zip(glev.tolist(), gidx.tolist())]))
    scale = cfg.scale if cfg.scale is not None else 1.0 / math.sqrt(d)
    og, lse = causal_attention(qg, kg, vg, scale)
    y = scatter(og, inv, n, cfg.pool)
    st = HeadState(sizes, q_levels, k_levels, v_levels, scores, sel, glev, gidx, inv,
                   qg, kg, vg, og, lse, scale)
    return y, st


def head_backward(dy: np.ndarray, st: HeadState, cfg: Config) -> tuple:
    """Backward of one (batch, head): returns dQ, dK, dV [N, D]. Selection stays frozen."""
    n = dy.shape[0]
    dog = scatter_backward(dy, st.glev, st.gidx, cfg.pool)
    if cfg.bf16_attention:
        dog = round_bf16(dog)
    dqg, dkg, dvg = causal_attention_backward(st.qg, st.kg, st.vg, st.og, st.lse, dog, st.scale)
    dq = gather_pool_backward(dqg, st.inv, n, cfg.pool)
    dk = gather_pool_backward(dkg, st.inv, n, cfg.pool)
    dv = gather_pool_backward(dvg, st.inv, n, cfg.pool)
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# whole layer on [B, N, H, D] arrays
# --------------------------------------------------------------------------------------
def forward(q, k, v, cfg: Config):
    """Layer forward on [B, N, H, D] inputs; returns (Y float64, states[b][h])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    b_, n, h_, d = q.shape
    y = np.zeros((b_, n, h_, d))
    states = []
    for b in range(b_):
        row = []
        for h in range(h_):
            y[b, :, h], st = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], cfg)
            row.append(st)
        states.append(row)
    return y, states


def backward(dy, states, cfg: Config):
    """Layer backward on a [B, N, H, D] upstream gradient; returns dQ, dK, dV float64."""
    dy = np.asarray(dy, np.float64)
    b_, n, h_, d = dy.shape
    dq = np.zeros((b_, n, h_, d))
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    for b in range(b_):
        for h in range(h_):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = head_backward(dy[b, :, h], states[b][h], cfg)
    return dq, dk, dv


def pyramid_ids(st: HeadState) -> np.ndarray:
    """The gathered map as pyramid ids (offsets[l] + j), in gathered order."""
    off = np.asarray(level_offsets(st.sizes), np.int64)
    return off[st.glev] + st.gidx
