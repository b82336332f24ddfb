"""GPU checks of what the pages fix, on the HIP path through the C ABI: causality of the whole
layer (bit-exact, forward and backward), exact chunked top-K at the wide chunks, and shapes at
the bounds the ABI accepts.

Causality (reading: chunk-causal selection; attention and scatter exactly causal):
  * Q or V changed at tokens >= t0, any t0, with the key-norm scorer (Q and V do not enter
    its scores): Y[:t0] is bit-identical.
  * Q, K and V changed at tokens >= t0, t0 a multiple of C * p^(L-1) (every chunk of every
    level then lies wholly before or wholly after t0), any scorer: Y[:t0] is bit-identical.
  * dY changed at tokens < t0 (inputs unchanged, so the selection is too): dQ, dK, dV at
    tokens >= t0 are bit-identical -- the backward only moves gradient from later tokens to
    earlier ones (a gathered entry that covers a token t >= t0 has causal position >= t0, so
    its scatter span, every query that attends it and every key it attends with a later
    query lie at or after t0).
Masked weights are exactly 0 in the kernels, so these hold bit for bit, not within a
tolerance.
"""

import numpy as np
import pytest
import torch

import oracle as O
from hierarchical_sparse_attention_lh_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(w):
    x = synth.workload_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return {n: torch.from_numpy(a).to(DEV).to(dt) for n, a in x.items()}, x


def _run(cfg, t):
    y, bufs = ops.lh_forward(cfg, t["q"], t["k"], t["v"])
    g = ops.lh_backward(cfg, t["q"], t["k"], t["v"], bufs, t["dy"])
    torch.cuda.synchronize()
    return y, g


# N = 16384 tokens, chunk 64, p = 4, L = 3: the chunk span C * p^(L-1) is 1024 tokens
CAUSAL = [
    synth.Workload("causal-refine", 1, 16384, 2, 64, "bf16", 3, 4, 120, 64, 31, True),
    synth.Workload("causal-direct", 1, 16384, 2, 64, "bf16", 3, 4, 120, 64, 32, True, "direct"),
    synth.Workload("causal-qkv", 1, 16384, 2, 64, "bf16", 3, 4, 120, 64, 33, True, scorer="qkv"),
    synth.Workload("causal-d128-p2", 1, 8192, 2, 128, "bf16", 4, 2, 90, 128, 34, True),
]


@pytest.mark.parametrize("w", CAUSAL, ids=lambda w: w.name)
def test_layer_is_causal_bit_exact(w):
    print(f"[causal] {w.name}", flush=True)
    t, _ = _inputs(w)
    cfg = ops.config_for(w)
    y0, g0 = _run(cfg, t)
    gen = torch.Generator(device="cpu").manual_seed(7)

    def noise(shape):
        return (torch.randn(shape, generator=gen) * 3).to(DEV).to(t["q"].dtype)

    span = w.chunk * w.pool ** (w.levels - 1)
    cases = []
    if w.scorer == "k":  # Q and V never enter the key-norm score: any t0
        for t0 in (1, 333, 5000, w.n_tokens - 77):
            cases.append((t0, ("q", "v")))
    for m in (1, 3):
        cases.append((m * span, ("q", "k", "v")))
    for t0, names in cases:
        z = dict(t)
        for n in names:
            a = t[n].clone()
            a[:, t0:] = noise(a[:, t0:].shape)
            z[n] = a
        y1, _ = ops.lh_forward(cfg, z["q"], z["k"], z["v"])
        torch.cuda.synchronize()
        assert torch.equal(y1[:, :t0], y0[:, :t0]), (t0, names)
        assert not torch.equal(y1[:, t0:], y0[:, t0:]), (t0, names)
    # backward: the gradient at tokens >= t0 ignores the upstream gradient before t0
    for t0 in (1, 517, 4096, w.n_tokens - 5):
        z = dict(t)
        a = t["dy"].clone()
        a[:, :t0] = noise(a[:, :t0].shape)
        z["dy"] = a
        _, g1 = _run(cfg, z)
        for a0, a1 in zip(g0, g1):
            assert torch.equal(a1[:, t0:], a0[:, t0:]), t0
        if t0 >= 100:  # (the first tokens may be reached by no gathered entry at all)
            assert any(not torch.equal(a1[:, :t0], a0[:, :t0]) for a0, a1 in zip(g0, g1)), t0


# ------------------------------------------------------------ top-K at the wide chunks
WIDE_CHUNKS = [
    # C = 1024: level 1 has 16 chunks (quotas 44/43), level 2 four
    synth.Workload("topk-c1024", 1, 65536, 2, 64, "bf16", 3, 4, 700, 1024, 41, False),
    # C = 2048 (the largest chunk): 16 and 4 chunks
    synth.Workload("topk-c2048", 1, 131072, 2, 64, "bf16", 3, 4, 1000, 2048, 42, False),
    # C = 2048 with level 3 (1536 entries) a single chunk narrower than C: a padded network
    synth.Workload("topk-c2048-pad", 1, 98304, 2, 64, "bf16", 4, 4, 1000, 2048, 43, False),
    # the same widths under DIRECT (raw tokens selected in 2048-wide chunks)
    synth.Workload("topk-c2048-direct", 1, 65536, 2, 64, "bf16", 3, 4, 3000, 2048, 44, False,
                   "direct"),
]


@pytest.mark.parametrize("w", WIDE_CHUNKS, ids=lambda w: w.name)
def test_topk_exact_at_wide_chunks(w):
    print(f"[topk] {w.name}", flush=True)
    t, _ = _inputs(w)
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    _, _, _, sc = ops.lh_pool_score(cfg, t["q"], t["k"], t["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc).cpu().numpy()
    sc_np = sc.double().cpu().numpy()
    levels = range(0, w.levels - 1) if w.mode == "direct" else range(1, w.levels)
    for h in range(w.heads):
        for lv in levels:
            o = info.level_offset[lv]
            want = O.select_level(sc_np[0, h, o:o + info.level_size[lv]], w.k, w.chunk)
            got = sel[0, h, info.sel_offset[lv]:info.sel_offset[lv] + info.k_eff[lv]]
            assert np.array_equal(got, want), (h, lv)
            nch, width = O.chunk_layout(info.level_size[lv], w.chunk)
            counts = np.bincount(got // width, minlength=nch)
            assert counts.tolist() == O.chunk_quotas(info.k_eff[lv], nch), (h, lv)


# ------------------------------------------------------------ shapes at the ABI bounds
BOUNDS = [
    # eight levels at p = 2 (the token-walking kernels' largest level count)
    synth.Workload("levels8-p2", 1, 4096, 2, 64, "bf16", 8, 2, 20, 64, 51, True),
    # the largest pool factor
    synth.Workload("pool16", 1, 8192, 2, 64, "bf16", 3, 16, 10, 64, 52, True),
    # the smallest chunk and the 16-token example: S = 4 + 4 = 8
    synth.Workload("n16", 1, 16, 2, 64, "bf16", 2, 4, 1, 16, 53, True),
    # the 16-token example under DIRECT at D = 128
    synth.Workload("n16-direct-d128", 1, 16, 2, 128, "bf16", 2, 4, 2, 16, 54, True, "direct"),
    # seven levels, p = 3 (a non-power-of-two factor with the longest walk; every level is one
    # chunk, since a level larger than a chunk must be a whole number of chunks)
    synth.Workload("levels7-p3", 1, 2187, 1, 64, "bf16", 7, 3, 9, 1024, 55, True),
]


@pytest.mark.parametrize("w", BOUNDS, ids=lambda w: w.name)
def test_layer_at_abi_bounds(w):
    print(f"[bounds] {w.name}", flush=True)
    t, x = _inputs(w)
    cfg = ops.config_for(w)
    y, g = _run(cfg, t)
    ocfg = O.Config(w.levels, w.pool, w.k, w.chunk,
                    mode=O.DIRECT if w.mode == "direct" else O.REFINE, scorer=w.scorer)
    ry, st = O.forward(x["q"], x["k"], x["v"], ocfg)
    rg = O.backward(x["dy"], st, ocfg)
    info = ops.lh_plan(cfg)
    assert info.gathered_len == O.gathered_length(w.n_tokens, ocfg)
    for name, got, ref in (("y", y, ry), ("dq", g[0], rg[0]), ("dk", g[1], rg[1]), ("dv", g[2], rg[2])):
        gg = got.float().cpu().numpy().astype(np.float64)
        err = np.abs(gg - ref)
        tol = 2e-2 + 2.0**-8 * np.abs(ref)
        print(f"[{w.name}] {name}: worst err/tol {(err / tol).max():.3f}")
        assert np.all(err <= tol), (name, float(err.max()))


# ------------------------------------------------- mapped rows beyond a 32-bit offset
# Mapped attention switches to 64-bit row addressing when a head's pyramid rows (N raw plus
# P1 pooled rows of H * D bf16) span 4 GiB or more.  These shapes cross that line (L = 2,
# p = 16, C = 1024: N + P1 = 539,648 rows of 8 KiB); the mapped kernels must then give exactly
# what the strided kernels give on the gathered copy of the same rows.
LARGE_ROWS = [(32, 128), (64, 64)]


@pytest.mark.parametrize("heads,d", LARGE_ROWS, ids=lambda v: str(v))
def test_mapped_attention_with_64bit_row_offsets(heads, d):
    n, levels, pool, k, chunk = 507904, 2, 16, 1024, 1024
    cfg = ops.make_config(1, n, heads, d, levels, pool, k, chunk)
    info = ops.lh_plan(cfg)
    assert (n + info.pooled_rows) * heads * d * 2 >= 1 << 32  # the 64-bit addressing path
    print(f"[rows64] H={heads} D={d} S={info.gathered_len}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(61 + d)
    x = {nm: torch.randn((1, n, heads, d), generator=gen, device=DEV, dtype=torch.bfloat16)
         for nm in ("q", "k", "v", "dy")}
    pq, pk, pv, sc = ops.lh_pool_score(cfg, x["q"], x["k"], x["v"], pooled_dtype=torch.bfloat16)
    sel = ops.lh_topk(cfg, sc)
    del sc
    gmap, inv, g = ops.lh_gather(cfg, x["q"], x["k"], x["v"], pq, pk, pv, sel)
    S = info.gathered_len
    og, lse = ops.lh_attn_fwd_mapped(cfg, x["q"], x["k"], x["v"], pq, pk, pv, gmap)
    dog, delta = ops.lh_scatter_bwd(cfg, gmap, og, x["dy"])
    del x["dy"]
    dqg, dkg, dvg = ops.lh_attn_bwd_mapped(cfg, x["q"], x["k"], x["v"], pq, pk, pv, gmap, lse,
                                           delta, dog)
    rows = {nm: g[nm][:, :, :S] for nm in "qkv"}
    o2, lse2 = ops.lh_attn_fwd(rows["q"], rows["k"], rows["v"])
    torch.cuda.synchronize()
    assert torch.equal(og[:, :, :S], o2) and torch.equal(lse[:, :, :S], lse2[:, :, :S])
    dq2, dk2, dv2 = ops.lh_attn_bwd(rows["q"], rows["k"], rows["v"], og[:, :, :S], lse,
                                    dog[:, :, :S])
    torch.cuda.synchronize()
    for a, b in ((dqg, dq2), (dkg, dk2), (dvg, dv2)):
        assert torch.equal(a[:, :, :S], b)
    del x, pq, pk, pv, g, rows, og, o2, dqg, dkg, dvg, dq2, dk2, dv2
    torch.cuda.empty_cache()
