"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Stage-isolated checks feed the GPU's own output of the previous stage into the oracle's next
stage, so one kernel's error never hides or cascades into another's; end-to-end checks run
lh_forward / lh_backward against the oracle's whole layer on the same seeded inputs.

Tolerances:
  pooled values (float32):   |d| <= 1e-4 * max(|ref|, ||row||_2 / sqrt(D))
  scores (float32):          |d| <= 1e-4 * |ref|
  selection, maps:           bit-exact on the GPU's own scores; against the oracle's float64
                             scores a swap is forgiven only if the two scores are within
                             1e-6 relative
  gathered rows (bf16):      equal to the oracle's bf16 rounding, except an element may sit
                             one bf16 step away when float32 pooling and float64 pooling land
                             on opposite sides of a rounding tie (counted, must be rare)
  attention Og (float32):    |d| <= 2^-13 * (P |V|) + 1e-6: P enters the product as a bf16
                             hi/lo pair (relative error <= 2^-16), bounded by the same
                             attention applied to |V|, plus float32 accumulation;
                             LSE: 1e-5 + 1e-6 |ref|
  Y, dQ, dK, dV (bf16/f32):  |d| <= 2e-2 + 2^-8 |ref| (2e-2 plus the half-step of the final
                             bf16 rounding)
"""

import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_lh_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(w, with_grad=True):
    x = synth.workload_inputs(w, with_grad=with_grad)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return {n: torch.from_numpy(a).to(DEV).to(dt) for n, a in x.items()}, x


def ocfg(w):
    return O.Config(w.levels, w.pool, w.k, w.chunk, mode=O.DIRECT if w.mode == "direct" else O.REFINE,
                    scorer=w.scorer)


def sel_levels(w):
    """Levels the selection runs on: 1..L-1 (REFINE) or 0..L-2 (DIRECT)."""
    return range(0, w.levels - 1) if w.mode == "direct" else range(1, w.levels)


def small(name, **kw):
    base = synth.WORKLOADS[name]
    d = base.__dict__.copy()
    d.update(kw)
    return synth.Workload(**d)


TINY = synth.WORKLOADS["tiny-4k"]
MEDIUM = synth.WORKLOADS["medium-32k"]
# ragged gathered length (S = 256 + 4 * (37 + 37) = 552, not a multiple of 128), bf16, D = 64
RAGGED = synth.Workload("ragged", 1, 4096, 2, 64, "bf16", 3, 4, 37, 64, 11, True)
# head_dim 128, batch 2, four levels, 3 chunks at level 1 with a remainder in the quotas
WIDE = synth.Workload("wide-d128", 2, 3072, 2, 128, "bf16", 4, 4, 50, 256, 12, True)
# dense causal attention: one level, S = N
DENSE = synth.Workload("dense", 1, 640, 2, 64, "bf16", 1, 4, 0, 64, 13, True)
# pool factor 2 with five levels (the wider prefetch bound of the token-walking kernels)
POOL2 = synth.Workload("pool2-l5", 1, 4096, 2, 64, "bf16", 5, 2, 100, 256, 14, True)
# a pool factor that is not a power of two (division instead of shifts), three chunks
POOL3 = synth.Workload("pool3", 1, 4608, 2, 64, "bf16", 3, 3, 100, 512, 15, True)
# the DIRECT selection reading: kept entries of levels 0..L-2 enter themselves
DIRECT = synth.Workload("direct", 1, 4096, 2, 64, "bf16", 3, 4, 100, 64, 16, True, "direct")
DIRECT_P2 = synth.Workload("direct-p2-d128", 1, 2048, 2, 128, "bf16", 4, 2, 64, 128, 17, True,
                           "direct")
# degenerate budgets: nothing selected (only the coarsest level is gathered, S = n_{L-1} = 128,
# the first 15 tokens receive nothing) and everything selected (k >= n_l at every level: the
# whole pyramid is gathered, S = 1024 + 256 + 64; level 2 is a single chunk of exactly C)
EMPTY_SEL = synth.Workload("empty-sel", 1, 2048, 2, 64, "bf16", 3, 4, 0, 64, 18, True)
FULL_BUDGET = synth.Workload("full-budget", 1, 1024, 2, 64, "bf16", 3, 4, 1000, 64, 19, True)
# the scorer readings: ||q_bar|| * ||k_bar|| and ||[q_bar; k_bar; v_bar]|| (also under DIRECT,
# where raw tokens are scored too, at D = 128 and p = 2, and with float32 inputs)
SCORER_QK = synth.Workload("scorer-qk", 1, 4096, 2, 64, "bf16", 3, 4, 100, 64, 20, True,
                           scorer="qk")
SCORER_QKV_DIRECT = synth.Workload("scorer-qkv-direct-d128", 1, 2048, 2, 128, "bf16", 4, 2, 64,
                                   128, 21, True, "direct", scorer="qkv")
SCORER_QKV_F32 = synth.Workload("scorer-qkv-f32", 1, 4096, 2, 64, "f32", 3, 4, 128, 64, 22, True,
                                scorer="qkv")
SCORER_CASES = [SCORER_QK, SCORER_QKV_DIRECT, SCORER_QKV_F32]
STAGE_CASES = [TINY, RAGGED, WIDE, POOL2, POOL3, DIRECT, DIRECT_P2, EMPTY_SEL, FULL_BUDGET] + SCORER_CASES
E2E_CASES = [TINY, RAGGED, WIDE, DENSE, POOL2, POOL3, DIRECT, DIRECT_P2, EMPTY_SEL, FULL_BUDGET] + SCORER_CASES


def pooled_rows_oracle(x, w):
    """Oracle pyramids of one tensor: [B][H] -> list of level arrays."""
    b_, n, h_, d = x.shape
    return [[O.pool_pyramid(x[b, :, h].astype(np.float64), w.levels, w.pool) for h in range(h_)]
            for b in range(b_)]


# ------------------------------------------------------------------------ stages 1+2
@pytest.mark.parametrize("w", STAGE_CASES, ids=lambda w: w.name)
def test_pool_score(w):
    t, x = inputs(w, with_grad=False)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    pq, pk, pv, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.float32)
    torch.cuda.synchronize()
    worst_rel = 0.0
    ref = {name: pooled_rows_oracle(x[name], w) for name in "qkv"}
    for name, p in (("q", pq), ("k", pk), ("v", pv)):
        got = f64(p)
        for b in range(w.batch):
            for h in range(w.heads):
                for lv in range(1, w.levels):
                    o = info.pooled_offset[lv]
                    g = got[b, o:o + info.level_size[lv], h]
                    r = ref[name][b][h][lv]
                    scale = np.maximum(np.abs(r), np.linalg.norm(r, axis=1, keepdims=True) / np.sqrt(w.head_dim))
                    assert np.all(np.abs(g - r) <= 1e-4 * scale + 1e-30), (name, b, h, lv)
    # scores of the scored levels (the raw tokens too under DIRECT) against the oracle's scorer
    first = 0 if w.mode == "direct" else 1
    for b in range(w.batch):
        for h in range(w.heads):
            s_ref = O.score_pyramid(ref["k"][b][h], w.scorer, ref["q"][b][h], ref["v"][b][h])
            for lv in range(first, w.levels):
                s_got = f64(sc[b, h, info.level_offset[lv]:info.level_offset[lv] + info.level_size[lv]])
                rel = np.abs(s_got - s_ref[lv]) / np.maximum(s_ref[lv], 1e-30)
                worst_rel = max(worst_rel, float(rel.max()))
                assert np.all(rel <= 1e-4), (b, h, lv)
    print(f"[{w.name}] worst score relative error {worst_rel:.3e}")
    # bf16 pooled output is the same float32 value rounded once
    pq16, pk16, pv16, sc16 = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    for a, b16 in ((pq, pq16), (pk, pk16), (pv, pv16)):
        assert torch.equal(a.to(torch.bfloat16), b16)
    lo = info.level_offset[min(sel_levels(w), default=1)]
    assert torch.equal(sc[:, :, lo:], sc16[:, :, lo:])


# ------------------------------------------------------------------------ stage 3
def _oracle_select(scores_np, w, info):
    return {lv: O.select_level(scores_np[info.level_offset[lv]:info.level_offset[lv] + info.level_size[lv]],
                               w.k, w.chunk) for lv in sel_levels(w)}


@pytest.mark.parametrize("w", STAGE_CASES + [MEDIUM], ids=lambda w: w.name)
def test_topk_exact_on_gpu_scores(w):
    t, x = inputs(w, with_grad=False)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    _, _, _, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc)
    sc_np = f64(sc)
    sel_np = sel.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.heads):
            want = _oracle_select(sc_np[b, h], w, info)
            for lv in sel_levels(w):
                o = info.sel_offset[lv]
                got = sel_np[b, h, o:o + info.k_eff[lv]]
                assert np.array_equal(got, want[lv]), (b, h, lv)


@pytest.mark.parametrize("w", [TINY, MEDIUM, SCORER_QK, SCORER_QKV_DIRECT], ids=lambda w: w.name)
def test_topk_against_float64_scores_with_near_ties(w):
    t, x = inputs(w, with_grad=False)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    _, _, _, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc).cpu().numpy()
    swaps = 0
    for b in range(w.batch):
        for h in range(w.heads):
            _, scores, want = O.head_selection(x["k"][b, :, h].astype(np.float64), ocfg(w),
                                               q=x["q"][b, :, h].astype(np.float64),
                                               v=x["v"][b, :, h].astype(np.float64))
            for lv in sel_levels(w):
                o = info.sel_offset[lv]
                got = set(sel[b, h, o:o + info.k_eff[lv]].tolist())
                ref = set(want[lv].tolist())
                s = scores[lv]
                extra, missing = sorted(got - ref), sorted(ref - got)
                assert len(extra) == len(missing)
                for a, m in zip(extra, missing):
                    gap = abs(s[a] - s[m])
                    assert gap <= 1e-6 * max(s[a], s[m]), (b, h, lv, a, m, gap)
                    swaps += 1
    print(f"[{w.name}] forgiven near-tie swaps: {swaps}")


# ------------------------------------------------------------------------ stages 1-3 fused
def _fusable(w, info):
    """The fused pool + score + top-K kernel runs when a chunk of the finest selected level
    covers a whole number of coarsest blocks."""
    f = min(sel_levels(w), default=None)
    if w.levels < 2 or info.sel_total == 0 or f is None:
        return False
    return info.chunk_width[f] * w.pool ** f % w.pool ** (w.levels - 1) == 0


# a 512K-shaped selection (L = 4, p = 4, C = 1024: a level-1 chunk spans 4096 tokens) at 32K
FUSED_C1024 = synth.Workload("fused-c1024", 1, 32768, 4, 64, "bf16", 4, 4, 700, 1024, 23, False)
# DIRECT, C = 2048 over raw tokens (R = 8 keys per thread), D = 128, batch 2
FUSED_DIRECT_C2048 = synth.Workload("fused-direct-c2048-d128", 2, 16384, 2, 128, "bf16", 3, 4,
                                    1500, 2048, 24, False, "direct")
# DIRECT with chunks narrower than a coarsest block: separate launches
SPLIT_DIRECT = synth.Workload("split-direct", 1, 4096, 2, 64, "bf16", 4, 4, 20, 16, 25, False,
                              "direct")
# p = 3 with one level-1 chunk of 1536 entries (not a power of two: a padded network), which
# spans all 4608 tokens, a whole number of coarsest blocks
FUSED_P3_ONE_CHUNK = synth.Workload("fused-p3-one-chunk", 1, 4608, 2, 64, "bf16", 3, 3, 100, 2048,
                                    26, False)
FUSED_CASES = STAGE_CASES + [MEDIUM, FUSED_C1024, FUSED_DIRECT_C2048, SPLIT_DIRECT,
                             FUSED_P3_ONE_CHUNK]


def _check_fused(w, t, info, cfg):
    pq, pk, pv, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc)
    fq, fk, fv, fsc, fsel = ops.lh_pool_score_topk(cfg, t["q"], t["k"], t["v"],
                                                   pooled_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for a, b in ((pq, fq), (pk, fk), (pv, fv)):
        assert torch.equal(a, b)
    if info.sel_total:
        assert torch.equal(sel[..., :info.sel_total], fsel[..., :info.sel_total])
    fused = _fusable(w, info)
    first = 0 if w.mode == "direct" else 1
    for lv in range(first, w.levels):
        o, n = info.level_offset[lv], info.level_size[lv]
        if fused and lv == min(sel_levels(w)):  # kept on chip: never written
            assert torch.isnan(fsc[:, :, o:o + n]).all(), lv
        else:
            assert torch.equal(sc[:, :, o:o + n], fsc[:, :, o:o + n]), lv
    return fused


@pytest.mark.parametrize("w", FUSED_CASES, ids=lambda w: w.name)
def test_pool_score_topk_matches_separate_stages(w):
    """One fused pass gives the pooled rows and the selection of lh_pool_score + lh_topk bit
    for bit (the separate stages are checked against the oracle above)."""
    t, _ = inputs(w, with_grad=False)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    fused = _check_fused(w, t, info, cfg)
    print(f"[{w.name}] fused kernel: {fused}")
    if w in (FUSED_C1024, FUSED_DIRECT_C2048, FUSED_P3_ONE_CHUNK):
        assert fused
    if w is SPLIT_DIRECT:
        assert not fused


def test_pool_score_topk_without_pooled_outputs():
    """Pooled outputs are optional: with pq and pv NULL (and pk NULL too) the fused pass keeps
    the same entries, and the rows it was asked for are identical."""
    import ctypes
    from hierarchical_sparse_attention_lh_amd import _lib
    for w in (FUSED_C1024, SCORER_QK):
        t, _ = inputs(w, with_grad=False)
        cfg = ops.config_for(w)
        info = ops.lh_plan(cfg)
        _, pk, _, _, sel = ops.lh_pool_score_topk(cfg, t["q"], t["k"], t["v"],
                                                  pooled_dtype=torch.bfloat16)
        for keep_k in (True, False):
            pk2 = torch.zeros_like(pk) if keep_k else None
            sc2 = torch.empty((w.batch, w.heads, info.pyramid_total), dtype=torch.float32,
                              device=DEV)
            sel2 = torch.empty_like(sel)
            code = _lib.load().lh_pool_score_topk(
                ctypes.byref(cfg), ops._p(t["q"]), ops._p(t["k"]), ops._p(t["v"]), None,
                ops._p(pk2) if keep_k else None, None, _lib.LH_BF16, ops._p(sc2), ops._p(sel2),
                ops._stream())
            assert code == 0
            torch.cuda.synchronize()
            assert torch.equal(sel2[..., :info.sel_total], sel[..., :info.sel_total]), (w.name, keep_k)
            if keep_k:
                assert torch.equal(pk2, pk), w.name


def test_pool_score_topk_exact_ties():
    """Whole runs of equal scores inside every chunk (key tokens repeated in blocks of 64, so
    16 consecutive level-1 and 4 consecutive level-2 entries tie exactly): both paths must keep
    the lower indices."""
    w = FUSED_C1024
    t, _ = inputs(w, with_grad=False)
    n = w.n_tokens
    idx = torch.arange(n, device=DEV) // 64 * 64
    t["k"] = t["k"][:, idx].contiguous()
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    assert _check_fused(w, t, info, cfg)
    _, _, _, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc).cpu().numpy()
    sc_np = f64(sc)
    for h in range(w.heads):
        for lv in sel_levels(w):
            o = info.level_offset[lv]
            want = O.select_level(sc_np[0, h, o:o + info.level_size[lv]], w.k, w.chunk)
            got = sel[0, h, info.sel_offset[lv]:info.sel_offset[lv] + info.k_eff[lv]]
            assert np.array_equal(got, want), (h, lv)


# ------------------------------------------------------------------------ stage 4
@pytest.mark.parametrize("w", STAGE_CASES + [MEDIUM], ids=lambda w: w.name)
def test_map_and_gather(w):
    t, x = inputs(w, with_grad=False)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    pq, pk, pv, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.float32)
    sel = ops.lh_topk(cfg, sc)
    gmap, inv = ops.lh_build_map(cfg, sel)
    gmap2, inv2, g = ops.lh_gather(cfg, t["q"], t["k"], t["v"], pq, pk, pv, sel)
    torch.cuda.synchronize()
    assert torch.equal(gmap, gmap2) and torch.equal(inv, inv2)
    sel_np, gmap_np, inv_np = sel.cpu().numpy(), gmap.cpu().numpy(), inv.cpu().numpy()
    S, Sp = info.gathered_len, info.gathered_pad
    sizes = [info.level_size[l] for l in range(w.levels)]
    offs = np.array([info.level_offset[l] for l in range(w.levels)])
    pooled = {"q": f64(pq), "k": f64(pk), "v": f64(pv)}
    near = 0
    for b in range(w.batch):
        for h in range(w.heads):
            s = {lv: sel_np[b, h, info.sel_offset[lv]:info.sel_offset[lv] + info.k_eff[lv]]
                 for lv in sel_levels(w)}
            glev, gidx = O.gathered_set(s, sizes, ocfg(w))
            ids = offs[glev] + gidx
            assert np.array_equal(gmap_np[b, h, :S], ids)
            assert np.all(gmap_np[b, h, S:] == -1)
            want_inv = np.full(info.pyramid_total, -1)
            want_inv[ids] = np.arange(S)
            assert np.array_equal(inv_np[b, h], want_inv)
            if b == 0 and h == 0:  # rows of one head against the oracle's bf16 rounding
                for name in ("q", "k", "v"):
                    rows = []
                    for lv, j in zip(glev, gidx):
                        if lv == 0:
                            rows.append(x[name][b, j, h].astype(np.float64))
                        else:
                            rows.append(pooled[name][b, info.pooled_offset[lv] + j, h])
                    want = O.round_bf16(np.stack(rows))
                    got = f64(g[name][b, h, :S])
                    diff = got != want
                    near += int(diff.sum())
                    if diff.any():  # only one bf16 step, only near a tie
                        step = np.abs(want[diff]) * 2.0**-7
                        assert np.all(np.abs(got[diff] - want[diff]) <= step * 1.001)
                    assert np.all(f64(g[name][b, h, S:]) == 0)
    print(f"[{w.name}] gathered elements one bf16 step off (ties): {near}")
    assert near <= 3


# ------------------------------------------------------------------------ attention
def _attn_case(seq, d, heads=2, seed=0, batch=1):
    """bf16 Q, K, V [B, H, S, D] with a lognormal per-position scale, exactly S rows."""
    rng = np.random.default_rng(seed)
    x = {}
    for n in "qkv":
        a = rng.standard_normal((batch, heads, seq, d)).astype(np.float32) * \
            np.exp(0.5 * rng.standard_normal((batch, 1, seq, 1))).astype(np.float32)
        x[n] = torch.from_numpy(a).to(torch.bfloat16)
    return x


def _check_fwd(o, lse, x, causal, bh_list, d):
    for b, h in bh_list:
        qq, kk, vv = (f64(x[n][b, h]) for n in "qkv")
        ro, rl = O.causal_attention(qq, kk, vv, d ** -0.5, causal=causal)
        bound, _ = O.causal_attention(qq, kk, np.abs(vv), d ** -0.5, causal=causal)
        seq = qq.shape[0]
        go, gl = f64(o[b, h]), f64(lse[b, h, :seq])
        rl = rl / np.log(2.0)  # the kernel reports the log-sum-exp in base 2
        # P enters as a bf16 hi/lo pair (relative error <= 2^-16): the rest is float32 rounding
        err = np.abs(go - ro)
        print(f"attn fwd S={seq} D={d} causal={causal} ({b},{h}): max |dO| {err.max():.2e}, "
              f"worst err/bound {(err / bound).max():.2e}, max |dLSE| {np.abs(gl - rl).max():.2e}")
        assert np.all(err <= 2.0**-13 * bound + 1e-6), (b, h, err.max())
        assert np.all(np.abs(gl - rl) <= 1e-5 + 1e-6 * np.abs(rl))
        assert np.all(np.isfinite(f64(lse[b, h])))


def _check_bwd(grads, x, dout, causal, bh_list, d):
    for b, h in bh_list:
        qq, kk, vv, dd = (f64(t[b, h]) for t in (x["q"], x["k"], x["v"], dout))
        ro, rl = O.causal_attention(qq, kk, vv, d ** -0.5, causal=causal)
        ref = O.causal_attention_backward(qq, kk, vv, ro, rl, dd, d ** -0.5, causal=causal)
        for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
            g = f64(got[b, h])
            err = np.abs(g - r)
            tol = 2e-2 + 2.0**-8 * np.abs(r)
            print(f"attn bwd S={qq.shape[0]} D={d} causal={causal} ({b},{h}) {name}: max err "
                  f"{err.max():.2e}, worst err/tol {(err / tol).max():.3f}")
            assert np.all(err <= tol), (name, b, h, err.max(), np.abs(r).max())


@pytest.mark.parametrize("seq,d", [(1, 64), (100, 64), (128, 64), (1000, 64), (777, 128), (2048, 128),
                                   (12000, 64), (8192, 128)])
def test_attention_forward(seq, d):
    x = _attn_case(seq, d, seed=seq + d)
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o, lse = ops.lh_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    _check_fwd(o, lse, x, True, [(0, 0), (0, 1)], d)


@pytest.mark.parametrize("d", [64, 128])
def test_attention_with_a_late_score_beyond_float_range(d):
    """Head 0: every query lies along e1 and one key in a later tile has a score of 1024, far
    above every score of the first tile (184 apart in base 2 after the scale, beyond float's
    exponent range): exponentials taken against an early row maximum would overflow, so the
    forward's running maximum must move.  Both passes of the backward use the saved
    log-sum-exp.  All against the float64 oracle."""
    seq = 300
    x = _attn_case(seq, d, seed=11 + d)
    q, k = x["q"].float(), x["k"].float()
    q[0, 0] = 0.0
    q[0, 0, :, 0] = 16.0 * (d / 64) ** 0.5  # about the same scaled score at both head sizes
    k[0, 0, 200] = 0.0
    k[0, 0, 200, 0] = 64.0
    x["q"], x["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    rng = np.random.default_rng(5)
    dout = torch.from_numpy(rng.standard_normal((1, 2, seq, d)).astype(np.float32)).to(torch.bfloat16)
    qd, kd, vd, dod = (t.to(DEV) for t in (x["q"], x["k"], x["v"], dout))
    o, lse = ops.lh_attn_fwd(qd, kd, vd)
    grads = ops.lh_attn_bwd(qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    _check_fwd(o, lse, x, True, [(0, 0), (0, 1)], d)
    _check_bwd(grads, x, dout, True, [(0, 0), (0, 1)], d)


@pytest.mark.parametrize("seq,d", [(100, 64), (1000, 64), (777, 128), (640, 64), (6000, 64)])
def test_attention_backward(seq, d):
    x = _attn_case(seq, d, seed=seq * 3 + d)
    rng = np.random.default_rng(seq)
    dout = torch.from_numpy(rng.standard_normal((1, 2, seq, d)).astype(np.float32)).to(torch.bfloat16)
    q, k, v, do = (t.to(DEV) for t in (x["q"], x["k"], x["v"], dout))
    o, lse = ops.lh_attn_fwd(q, k, v)
    grads = ops.lh_attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    _check_bwd(grads, x, dout, True, [(0, 0), (0, 1)], d)


@pytest.mark.parametrize("seq,d,causal", [(1000, 64, False), (333, 128, False), (2500, 64, True),
                                          (1111, 128, True)])
def test_attention_on_token_layout(seq, d, causal):
    """Dense attention straight on [B, N, H, D] token tensors (strides, no copy), batch 2,
    three heads, causal and not."""
    x = _attn_case(seq, d, heads=3, seed=seq + 7 * d, batch=2)
    tok = {n: a.transpose(1, 2).contiguous().to(DEV) for n, a in x.items()}  # [B, N, H, D]
    rng = np.random.default_rng(seq + 1)
    dout = torch.from_numpy(rng.standard_normal((2, 3, seq, d)).astype(np.float32)).to(torch.bfloat16)
    o, lse = ops.lh_attn_fwd(tok["q"], tok["k"], tok["v"], causal=causal, layout="bshd")
    do_tok = dout.transpose(1, 2).contiguous().to(DEV)
    grads = ops.lh_attn_bwd(tok["q"], tok["k"], tok["v"], o, lse, do_tok, causal=causal,
                            layout="bshd")
    torch.cuda.synchronize()
    bh = [(0, 0), (1, 2)]
    _check_fwd(o.transpose(1, 2), lse, x, causal, bh, d)
    _check_bwd([g.transpose(1, 2) for g in grads], x, dout, causal, bh, d)


@pytest.mark.parametrize("w", [TINY, RAGGED, WIDE, POOL3, DIRECT_P2, EMPTY_SEL, FULL_BUDGET],
                         ids=lambda w: w.name)
def test_attention_mapped(w):
    """The layer's attention reading rows through gmap, against the oracle on the gathered
    rows of the same (GPU) selection, forward and backward; and bit-identical to the strided
    attention over lh_gather's copies of those rows."""
    t, x = inputs(w)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    S, D = info.gathered_len, w.head_dim
    tb = {n: a.to(torch.bfloat16) for n, a in t.items()}  # bf16 token rows (f32 layers round)
    pq, pk, pv, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc)
    gmap, inv, g = ops.lh_gather(cfg, tb["q"], tb["k"], tb["v"], pq, pk, pv, sel) if w.dtype == "bf16" \
        else ops.lh_gather(cfg, t["q"], t["k"], t["v"], pq, pk, pv, sel)
    og, lse = ops.lh_attn_fwd_mapped(cfg, tb["q"], tb["k"], tb["v"], pq, pk, pv, gmap)
    dog, delta = ops.lh_scatter_bwd(cfg, gmap, og, t["dy"])
    dqg, dkg, dvg = ops.lh_attn_bwd_mapped(cfg, tb["q"], tb["k"], tb["v"], pq, pk, pv, gmap, lse,
                                           delta, dog)
    rows = {n: g[n][:, :, :S] for n in "qkv"}
    o2, lse2 = ops.lh_attn_fwd(rows["q"], rows["k"], rows["v"])
    torch.cuda.synchronize()
    assert torch.equal(og[:, :, :S], o2) and torch.equal(lse[:, :, :S], lse2[:, :, :S])
    assert torch.all(dqg[:, :, S:] == 0) and torch.all(dkg[:, :, S:] == 0)
    bh = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    xg = {n: rows[n] for n in "qkv"}
    _check_fwd(og[:, :, :S], lse, xg, True, bh, D)
    _check_bwd([a[:, :, :S] for a in (dqg, dkg, dvg)], xg, dog[:, :, :S], True, bh, D)


# ------------------------------------------------------------------------ stage 5
@pytest.mark.parametrize("w", STAGE_CASES, ids=lambda w: w.name)
def test_scatter_and_adjoints(w):
    t, x = inputs(w)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    S, Sp, D = info.gathered_len, info.gathered_pad, w.head_dim
    _, _, _, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc)
    gmap, inv = ops.lh_build_map(cfg, sel)
    rng = np.random.default_rng(5)
    og_np = np.zeros((w.batch, w.heads, Sp, D), np.float32)
    og_np[:, :, :S] = rng.standard_normal((w.batch, w.heads, S, D))
    og = torch.from_numpy(og_np).to(DEV)
    y = ops.lh_scatter(cfg, inv, og)
    dog, delta = ops.lh_scatter_bwd(cfg, gmap, og, t["dy"])
    g3 = [torch.from_numpy(np.ascontiguousarray(np.roll(og_np, i, axis=-1))).to(DEV) for i in range(3)]
    dq, dk, dv = ops.lh_gather_pool_bwd(cfg, inv, *g3)
    torch.cuda.synchronize()
    gmap_np = gmap.cpu().numpy()
    sizes = [info.level_size[l] for l in range(w.levels)]
    offs = np.array([info.level_offset[l] for l in range(w.levels)])
    for b in range(w.batch):
        for h in range(w.heads):
            ids = gmap_np[b, h, :S]
            glev = np.searchsorted(offs, ids, side="right") - 1
            gidx = ids - offs[glev]
            invl = O.inverse_map(glev, gidx, sizes)
            ref = O.scatter(og_np[b, h, :S].astype(np.float64), invl, w.n_tokens, w.pool)
            got = f64(y[b, :, h])
            assert np.all(np.abs(got - ref) <= 1e-5 + 2.0**-8 * np.abs(ref))
            rdog = O.round_bf16(O.scatter_backward(x["dy"][b, :, h].astype(np.float64), glev, gidx, w.pool))
            gd = f64(dog[b, h, :S])
            if w.dtype == "bf16":  # float32 sums of bf16 values are exact here
                assert np.array_equal(gd, rdog)
            else:  # float32 inputs: the float32 span sum rounds before the bf16 rounding, so
                # a result may sit one bf16 step away, or further under cancellation (bounded
                # by float32 summation error over the span's absolute values)
                off = gd != rdog
                assert off.mean() < 1e-3
                mag = O.scatter_backward(np.abs(x["dy"][b, :, h].astype(np.float64)), glev, gidx, w.pool)
                step = 2.0**-7 * np.maximum(np.abs(gd), np.abs(rdog))
                assert np.all(np.abs(gd - rdog) <= step + 64 * 2.0**-24 * mag)
            assert np.all(f64(dog[b, h, S:]) == 0)
            rdelta = np.sum(gd * og_np[b, h, :S], axis=1)  # Delta of the GPU's own dOg
            assert np.allclose(f64(delta[b, h, :S]), rdelta, rtol=1e-5, atol=1e-5)
            assert np.all(f64(delta[b, h, S:]) == 0)
            for i, got_t in enumerate((dq, dk, dv)):
                gsrc = np.roll(og_np, i, axis=-1)[b, h, :S].astype(np.float64)
                rx = O.gather_pool_backward(gsrc, invl, w.n_tokens, w.pool)
                gx = f64(got_t[b, :, h])
                assert np.all(np.abs(gx - rx) <= 1e-5 + 2.0**-8 * np.abs(rx))


# ------------------------------------------------------------------------ whole layer
def _oracle_layer(w, x):
    y, st = O.forward(x["q"], x["k"], x["v"], ocfg(w))
    grads = O.backward(x["dy"], st, ocfg(w))
    return y, st, grads


@pytest.mark.parametrize("w", E2E_CASES, ids=lambda w: w.name)
def test_layer_forward_backward(w):
    t, x = inputs(w)
    cfg = ops.config_for(w)
    y, bufs = ops.lh_forward(cfg, t["q"], t["k"], t["v"])
    dq, dk, dv = ops.lh_backward(cfg, t["q"], t["k"], t["v"], bufs, t["dy"])
    torch.cuda.synchronize()
    ry, st, (rq, rk, rv) = _oracle_layer(w, x)
    # the GPU's selection must be the oracle's (checked exactly: these inputs have no near ties)
    views = bufs.views()
    info = bufs.info
    offs = np.array([info.level_offset[l] for l in range(w.levels)])
    for b in range(w.batch):
        for h in range(w.heads):
            assert np.array_equal(views["gmap"][b, h, :info.gathered_len].cpu().numpy(),
                                  O.pyramid_ids(st[b][h]))
    for name, got, ref in (("y", y, ry), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = f64(got)
        err = np.abs(g - ref)
        tol = 2e-2 + 2.0**-8 * np.abs(ref)
        print(f"[{w.name}] {name}: max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}, "
              f"worst err/tol {(err / tol).max():.3f}")
        assert np.all(err <= tol), (name, err.max())


def test_layer_medium_forward_backward():
    w = MEDIUM
    t, x = inputs(w)
    cfg = ops.config_for(w)
    y, bufs = ops.lh_forward(cfg, t["q"], t["k"], t["v"])
    dq, dk, dv = ops.lh_backward(cfg, t["q"], t["k"], t["v"], bufs, t["dy"])
    torch.cuda.synchronize()
    # two heads through the oracle (each head is independent)
    sub = {n: a[:, :, [0, 5]] for n, a in x.items()}
    ry, st, (rq, rk, rv) = _oracle_layer(w, sub)
    for name, got, ref in (("y", y, ry), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = f64(got[:, :, [0, 5]])
        err = np.abs(g - ref)
        print(f"[medium] {name}: max abs err {err.max():.3e}")
        assert np.all(err <= 2e-2 + 2.0**-8 * np.abs(ref)), name


def test_forward_is_deterministic_and_ignores_stale_buffers():
    w = RAGGED
    t, x = inputs(w)
    cfg = ops.config_for(w)
    y1, b1 = ops.lh_forward(cfg, t["q"], t["k"], t["v"])
    g1 = ops.lh_backward(cfg, t["q"], t["k"], t["v"], b1, t["dy"])
    b2 = ops.Buffers(cfg)
    for buf in (b2.saved, b2.ws_fwd, b2.ws_bwd):
        buf.view(torch.uint8).fill_(0xFF)  # NaN patterns everywhere
    y2, _ = ops.lh_forward(cfg, t["q"], t["k"], t["v"], bufs=b2)
    g2 = ops.lh_backward(cfg, t["q"], t["k"], t["v"], b2, t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dense_attention_32k_token_layout():
    """Dense causal attention as its own operation at N = 32,768 (the stage-2 dense-resumption
    call): straight on [B, N, H, D] token tensors of the medium workload's shape and values,
    forward and backward, two of eight heads against the oracle."""
    w = MEDIUM
    t, x = inputs(w)
    o, lse = ops.lh_attn_fwd(t["q"], t["k"], t["v"], layout="bshd")
    grads = ops.lh_attn_bwd(t["q"], t["k"], t["v"], o, lse, t["dy"], layout="bshd")
    torch.cuda.synchronize()
    xb = {n: torch.from_numpy(x[n]).transpose(1, 2) for n in ("q", "k", "v", "dy")}  # [B, H, N, D]
    heads = [(0, 0), (0, 5)]
    _check_fwd(o.transpose(1, 2), lse, xb, True, heads, w.head_dim)
    _check_bwd([g.transpose(1, 2) for g in grads], xb, xb["dy"], True, heads, w.head_dim)
