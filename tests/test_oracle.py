"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a closed form, a value the
pages print, an invariant the pages state, brute force on tiny inputs, or a library routine
(torch CPU) that computes a special case.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(levels, pool, k, chunk, mode=O.REFINE, bf16=True):
    return O.Config(levels=levels, pool=pool, k=k, chunk=chunk, mode=mode, bf16_attention=bf16)


# ---------------------------------------------------------------- bf16 rounding
def test_round_bf16_matches_torch_on_float32_values(rng):
    # float32 inputs: torch's float32 -> bfloat16 cast rounds once, to nearest even.
    # magnitudes from bf16 subnormals (below 2**-126) up to 2**120
    x = np.ldexp(rng.standard_normal(200000), rng.integers(-140, 120, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_hand_cases():
    ulp = 2.0**-7  # spacing of bf16 in [1, 2)
    cases = {
        1.0 + ulp / 2: 1.0,                   # tie -> even (1.0)
        1.0 + 3 * ulp / 2: 1.0 + 2 * ulp,     # tie -> even
        1.0 + ulp / 2 + 2.0**-30: 1.0 + ulp,  # just above the tie
        -(1.0 + ulp / 2): -1.0,
        2.0**-133: 2.0**-133,                 # smallest subnormal
        2.0**-134 * 1.5: 2.0**-133,
        3.5e38: math.inf,
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.round_bf16(np.array([x]))[0] == want, x


# ---------------------------------------------------------------- pool and score
def test_pool_constant_one_hot_and_ramp():
    n, p, L = 256, 4, 4
    const = np.full((n, 3), 2.5)
    for lvl in O.pool_pyramid(const, L, p):
        assert np.all(lvl == 2.5)
    t0 = 137
    hot = np.zeros((n, 1))
    hot[t0] = 1.0
    for lv, lvl in enumerate(O.pool_pyramid(hot, L, p)):
        want = np.zeros(n // p**lv)
        want[t0 // p**lv] = 1.0 / p**lv
        assert np.array_equal(lvl[:, 0], want)
    ramp = np.arange(n, dtype=np.float64)[:, None]
    for lv, lvl in enumerate(O.pool_pyramid(ramp, L, p)):
        j = np.arange(n // p**lv)
        assert np.array_equal(lvl[:, 0], j * p**lv + (p**lv - 1) / 2.0)


def test_pool_equals_torch_avg_pool(rng):
    n, d, p, L = 1024, 8, 4, 4
    x = rng.standard_normal((n, d))
    levels = O.pool_pyramid(x, L, p)
    xt = torch.from_numpy(x).T[None]  # [1, D, N]
    for lv in range(L):
        w = p**lv
        ref = F.avg_pool1d(xt, kernel_size=w, stride=w)[0].T.numpy()
        assert np.allclose(levels[lv], ref, rtol=0, atol=1e-13)


def test_pool_nonpower_of_two_factor(rng):
    x = rng.standard_normal((27, 2))
    lv = O.pool_pyramid(x, 3, 3)
    assert np.allclose(lv[2], x.reshape(3, 9, 2).mean(axis=1), atol=1e-14)


def test_score_closed_forms(rng):
    k = np.zeros((4, 64))
    k[0, 0] = -3.0
    k[1, 5] = 4.0
    k[2, :] = 0.5
    got = O.score_pyramid([k])[0]
    assert got[0] == 3.0 and got[1] == 4.0 and got[2] == 4.0 and got[3] == 0.0
    r = rng.standard_normal((100, 64))
    assert np.allclose(O.score_pyramid([r])[0], np.linalg.norm(r, axis=1), rtol=1e-15)


# ---------------------------------------------------------------- chunked top-K
def _brute_select(scores, k, chunk):
    """Keep entry i iff fewer than its chunk's quota entries rank strictly before it."""
    n = len(scores)
    k_eff = min(k, n)
    if n <= chunk:
        chunks = [(0, n)]
    else:
        chunks = [(c * chunk, (c + 1) * chunk) for c in range(n // chunk)]
    nc = len(chunks)
    kept = []
    for c, (a, b) in enumerate(chunks):
        quota = k_eff // nc + (1 if c < k_eff % nc else 0)
        for i in range(a, b):
            better = 0
            for j in range(a, b):
                si, sj = scores[i], scores[j]
                if j == i:
                    continue
                if math.isnan(si) and not math.isnan(sj):
                    better += 1
                elif math.isnan(si) and math.isnan(sj):
                    better += j < i
                elif math.isnan(sj):
                    pass
                elif sj > si or (sj == si and j < i):
                    better += 1
            if better < quota:
                kept.append(i)
    return np.array(kept, dtype=np.int64)


@pytest.mark.parametrize("n,k,chunk", [(64, 8, 16), (64, 13, 16), (48, 7, 16), (16, 5, 64),
                                       (32, 32, 8), (32, 100, 8), (40, 3, 8)])
def test_topk_brute_force_with_ties(rng, n, k, chunk):
    for trial in range(20):
        s = rng.integers(0, 6, n).astype(np.float64)  # many exact ties
        if trial % 4 == 1:
            s[rng.integers(0, n, 3)] = np.nan
        if trial % 4 == 2:
            s = rng.standard_normal(n) ** 2
        got = O.select_level(s, k, chunk)
        assert np.array_equal(got, _brute_select(s, k, chunk))


def test_topk_matches_torch_topk_per_chunk(rng):
    n, k, chunk = 4096, 200, 512
    s = rng.random(n)
    got = O.select_level(s, k, chunk)
    nc = n // chunk
    want = []
    for c in range(nc):
        q = k // nc + (1 if c < k % nc else 0)
        idx = torch.topk(torch.from_numpy(s[c * chunk:(c + 1) * chunk]), q).indices.numpy()
        want.append(np.sort(idx + c * chunk))
    assert np.array_equal(got, np.concatenate(want))


def test_topk_quotas_and_clamp():
    # 98K-token workload, level 1: 24576 entries, chunk 512, k = 2048 -> 48 chunks,
    # 32 of them keep 43 and 16 keep 42; level 3: 1536 entries with k = 2048 keeps all.
    assert O.chunk_quotas(2048, 48) == [43] * 32 + [42] * 16
    assert O.chunk_quotas(2048, 12) == [171] * 8 + [170] * 4
    s = np.arange(1536, dtype=np.float64)
    assert np.array_equal(O.select_level(s, 2048, 512), np.arange(1536))
    s = np.random.default_rng(0).random(24576)
    sel = O.select_level(s, 2048, 512)
    counts = np.bincount(sel // 512, minlength=48)
    assert list(counts) == [43] * 32 + [42] * 16


def test_topk_rejects_ragged_chunks():
    with pytest.raises(ValueError):
        O.select_level(np.zeros(100), 10, 64)


# ---------------------------------------------------------------- gathered set and map
def _random_state(n, cfg, seed=0):
    rng = np.random.default_rng(seed)
    sizes = O.level_sizes(n, cfg.levels, cfg.pool)
    sel = {lv: O.select_level(rng.random(sizes[lv]), cfg.k_list[lv], cfg.chunk)
           for lv in O.selected_levels(cfg)}
    glev, gidx = O.gathered_set(sel, sizes, cfg)
    return sizes, sel, glev, gidx


@pytest.mark.parametrize("n,L,p,k,chunk,want", [
    (4096, 3, 4, 128, 64, 1280),          # tiny 4K workload
    (32768, 3, 4, 1024, 256, 10240),      # medium 32K
    (98304, 4, 4, 2048, 512, 24064),      # 98K layer
    (524288, 4, 4, 4096, 1024, 57344),    # 512K
    (1048576, 4, 4, 4096, 1024, 65536),   # 1M
])
def test_gathered_length_closed_form(n, L, p, k, chunk, want):
    cfg = _cfg(L, p, k, chunk)
    sizes, sel, glev, gidx = _random_state(n, cfg)
    closed = sizes[-1] + p * sum(min(k, sizes[lv]) for lv in range(1, L))
    assert len(glev) == closed == want == O.gathered_length(n, cfg)


def test_gathered_length_matches_pages_one_million():
    with open(os.path.join(GOLDEN, "gathered_length_1m.json")) as f:
        g = json.load(f)
    # chunk width 15625 divides every level of N = 1e6 (the oracle accepts any width).
    cfg = _cfg(g["levels"], g["pool"], g["k"], 15625)
    sizes, sel, glev, gidx = _random_state(g["n_tokens"], cfg)
    s = len(glev)
    assert round(s / 1000) == g["pages_value_thousands"]
    assert s == 64777
    # The literal reading (gather the selected entries themselves) misses the page value.
    direct = _cfg(g["levels"], g["pool"], g["k"], 15625, mode=O.DIRECT)
    _, _, dlev, _ = _random_state(g["n_tokens"], direct)
    assert len(dlev) == 27913 and round(len(dlev) / 1000) != g["pages_value_thousands"]


def test_worked_example_order_scatter_and_pool_backward():
    # N = 16, p = 4, L = 2, one level-1 entry kept: j = 2 (tokens 8..11).
    cfg = _cfg(2, 4, 1, 4)
    sizes = O.level_sizes(16, 2, 4)
    glev, gidx = O.gathered_set({1: np.array([2])}, sizes, cfg)
    assert list(zip(glev.tolist(), gidx.tolist())) == [
        (1, 0), (1, 1), (0, 8), (0, 9), (0, 10), (0, 11), (1, 2), (1, 3)]
    inv = O.inverse_map(glev, gidx, sizes)
    y = O.scatter(np.ones((8, 1)), inv, 16, 4)[:, 0]
    assert list(y) == [0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 2, 2, 1, 1, 1, 1]
    dxg = np.arange(8, dtype=np.float64)[:, None] + 1.0
    dx = O.gather_pool_backward(dxg, inv, 16, 4)[:, 0]
    assert dx[9] == dxg[3, 0] + dxg[6, 0] / 4  # own slot + the level-1 block containing 9
    assert dx[0] == dxg[0, 0] / 4


@pytest.mark.parametrize("n,L,p,k,chunk", [(4096, 3, 4, 128, 64), (2048, 4, 2, 37, 16),
                                           (729, 3, 3, 20, 27), (4096, 1, 4, 0, 64)])
def test_map_invariants_and_coverage(n, L, p, k, chunk):
    cfg = _cfg(L, p, k, chunk)
    sizes, sel, glev, gidx = _random_state(n, cfg, seed=3)
    e = O.causal_position(glev, gidx, p)
    key = list(zip(e.tolist(), glev.tolist()))
    assert all(a < b for a, b in zip(key, key[1:]))  # strictly increasing (e, level)
    inv = O.inverse_map(glev, gidx, sizes)
    for s, (lv, j) in enumerate(zip(glev, gidx)):
        assert inv[lv][j] == s
    assert sum(int((i >= 0).sum()) for i in inv) == len(glev)
    # input coverage: the gathered entries' token blocks cover every token
    covered = np.zeros(n, bool)
    for lv, j in zip(glev, gidx):
        covered[j * p**lv:(j + 1) * p**lv] = True
    assert covered.all()
    # output coverage: every token from p**(L-1) - 1 on gets exactly one coarsest entry
    ones = np.zeros((len(glev), 1))
    ones[glev == L - 1] = 1.0
    y = O.scatter(ones, inv, n, p)[:, 0]
    top = p ** (L - 1)
    assert np.all(y[top - 1:] == 1.0) and np.all(y[:top - 1] == 0.0)


def test_scatter_slot_codes_and_counts():
    n, L, p = 256, 3, 4
    cfg = _cfg(L, p, 10**6, 8)  # budgets cover every entry: the full pyramid is gathered
    sizes, sel, glev, gidx = _random_state(n, cfg)
    assert len(glev) == sum(sizes)
    inv = O.inverse_map(glev, gidx, sizes)
    y = O.scatter(np.ones((len(glev), 1)), inv, n, p)[:, 0]
    t = np.arange(n)
    assert np.array_equal(y, sum((t + 1 >= p**lv).astype(float) for lv in range(L)))
    # slot codes: only level 1 carries a code; each token must receive the code of entry
    # floor((t+1)/p) - 1 of level 1.
    code = np.zeros((len(glev), 1))
    code[glev == 1, 0] = 1000.0 + gidx[glev == 1]
    y = O.scatter(code, inv, n, p)[:, 0]
    j = (t + 1) // p - 1
    assert np.array_equal(y, np.where(j >= 0, 1000.0 + j, 0.0))


# ---------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa(rng):
    s, d = 300, 16
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    o, lse = O.causal_attention(q, k, v, 0.3, rows=64)
    qt, kt, vt = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.3)[0, 0].numpy()
    assert np.allclose(o, ref, atol=1e-12)
    logits = torch.from_numpy(q @ k.T * 0.3).masked_fill(
        torch.triu(torch.ones(s, s, dtype=torch.bool), 1), float("-inf"))
    assert np.allclose(lse, torch.logsumexp(logits, 1).numpy(), atol=1e-12)


def test_full_attention_matches_torch_sdpa_and_autograd(rng):
    # causal=False: the same softmax attention over every key
    s, d = 200, 8
    q, k, v, do = (rng.standard_normal((s, d)) for _ in range(4))
    o, lse = O.causal_attention(q, k, v, 0.4, rows=64, causal=False)
    ts = {a: torch.tensor(x, requires_grad=True) for a, x in (("q", q), ("k", k), ("v", v))}
    ref = F.scaled_dot_product_attention(ts["q"][None], ts["k"][None], ts["v"][None], scale=0.4)[0]
    assert np.allclose(o, ref.detach().numpy(), atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(q @ k.T * 0.4), 1).numpy(), atol=1e-12)
    ref.backward(torch.from_numpy(do))
    grads = O.causal_attention_backward(q, k, v, o, lse, do, 0.4, rows=64, causal=False)
    for a, g in zip("qkv", grads):
        assert np.allclose(g, ts[a].grad.numpy(), atol=1e-11), a


def test_causal_attention_backward_matches_torch_autograd(rng):
    s, d = 150, 8
    q, k, v, do = (rng.standard_normal((s, d)) for _ in range(4))
    o, lse = O.causal_attention(q, k, v, 0.3, rows=32)
    ts = {a: torch.tensor(x, requires_grad=True) for a, x in (("q", q), ("k", k), ("v", v))}
    ref = F.scaled_dot_product_attention(ts["q"][None], ts["k"][None], ts["v"][None],
                                         is_causal=True, scale=0.3)[0]
    ref.backward(torch.from_numpy(do))
    grads = O.causal_attention_backward(q, k, v, o, lse, do, 0.3, rows=32)
    for a, g in zip("qkv", grads):
        assert np.allclose(g, ts[a].grad.numpy(), atol=1e-11), a


def test_single_level_is_textbook_causal_sdpa(rng):
    n, h, d = 256, 2, 16
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    cfg = _cfg(1, 4, 0, 64)
    y, _ = O.forward(x["q"], x["k"], x["v"], cfg)
    for hh in range(h):
        t = [torch.from_numpy(O.round_bf16(x[w][0, :, hh]))[None, None] for w in "qkv"]
        ref = F.scaled_dot_product_attention(*t, is_causal=True)[0, 0].numpy()
        assert np.allclose(y[0, :, hh], ref, atol=1e-12)


def _full_pyramid_reference(q, k, v, L, p):
    """Lighthouse with every entry kept, from library routines: avg_pool1d pyramid,
    SDPA with a causal mask over the (e, level) order, and a 0/1 matrix for the scatter."""
    n, d = q.shape
    ents = sorted(((j + 1) * p**lv - 1, lv, j) for lv in range(L) for j in range(n // p**lv))

    def rows(x):
        xt = torch.from_numpy(x).T[None]
        lv_rows = [F.avg_pool1d(xt, p**lv, p**lv)[0].T for lv in range(L)]
        return torch.stack([lv_rows[lv][j] for _, lv, j in ents])

    qg, kg, vg = (torch.from_numpy(O.round_bf16(rows(x).numpy())) for x in (q, k, v))
    og = F.scaled_dot_product_attention(qg[None], kg[None], vg[None], is_causal=True)[0]
    m = torch.zeros(n, len(ents), dtype=torch.float64)
    for s, (e, lv, j) in enumerate(ents):
        m[e:min(n, e + p**lv), s] = 1.0
    return (m @ og).numpy()


def test_full_budget_equals_dense_attention_over_pyramid(rng):
    n, h, d, L, p = 128, 1, 8, 3, 4
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    cfg = _cfg(L, p, 10**6, 16)
    y, _ = O.forward(x["q"], x["k"], x["v"], cfg)
    ref = _full_pyramid_reference(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], L, p)
    assert np.allclose(y[0, :, 0], ref, atol=1e-12)


# ---------------------------------------------------------------- causality
def test_future_perturbation_leaves_past_unchanged(rng):
    n, h, d, L, p, k, chunk = 1024, 2, 8, 3, 4, 24, 16
    cfg = _cfg(L, p, k, chunk)
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    y0, _ = O.forward(x["q"], x["k"], x["v"], cfg)
    for t0 in (1, 100, 517, 1000):  # Q and V never enter the score: any t0
        z = {w: a.copy() for w, a in x.items()}
        z["q"][:, t0:] += rng.standard_normal(z["q"][:, t0:].shape)
        z["v"][:, t0:] *= -3.0
        y1, _ = O.forward(z["q"], z["k"], z["v"], cfg)
        assert np.array_equal(y1[:, :t0], y0[:, :t0])
        assert not np.array_equal(y1[:, t0:], y0[:, t0:])
    span = chunk * p ** (L - 1)  # K too: selection is causal at chunk granularity
    for t0 in (span, 2 * span, 3 * span):
        z = {w: a.copy() for w, a in x.items()}
        for w in "qkv":
            z[w][:, t0:] = rng.standard_normal(z[w][:, t0:].shape) * 5
        y1, _ = O.forward(z["q"], z["k"], z["v"], cfg)
        assert np.array_equal(y1[:, :t0], y0[:, :t0])


# ---------------------------------------------------------------- backward
def test_adjoint_identities(rng):
    n, d, L, p = 512, 4, 3, 4
    cfg = _cfg(L, p, 9, 16)
    sizes, sel, glev, gidx = _random_state(n, cfg, seed=7)
    inv = O.inverse_map(glev, gidx, sizes)
    og = rng.standard_normal((len(glev), d))
    dy = rng.standard_normal((n, d))
    lhs = np.sum(O.scatter(og, inv, n, p) * dy)
    rhs = np.sum(og * O.scatter_backward(dy, glev, gidx, p))
    assert abs(lhs - rhs) <= 1e-10 * abs(lhs)
    x = rng.standard_normal((n, d))
    lv = O.pool_pyramid(x, L, p)
    xg = np.stack([lv[a][b] for a, b in zip(glev, gidx)])
    g = rng.standard_normal(xg.shape)
    lhs = np.sum(xg * g)
    rhs = np.sum(x * O.gather_pool_backward(g, inv, n, p))
    assert abs(lhs - rhs) <= 1e-10 * abs(lhs)


def _loss(x, w, cfg):
    y, st = O.forward(x["q"], x["k"], x["v"], cfg)
    return float(np.sum(y * w)), st


def test_backward_finite_differences(rng):
    n, h, d, L, p, k, chunk = 256, 1, 4, 3, 4, 6, 16
    cfg = _cfg(L, p, k, chunk, bf16=False)
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    w = rng.standard_normal((1, n, h, d))
    _, st = _loss(x, w, cfg)
    grads = dict(zip("qkv", O.backward(w, st, cfg)))
    eps = 1e-6
    for name in "qkv":
        for _ in range(6):
            t, c = int(rng.integers(0, n)), int(rng.integers(0, d))
            xp = {a: b.copy() for a, b in x.items()}
            xm = {a: b.copy() for a, b in x.items()}
            xp[name][0, t, 0, c] += eps
            xm[name][0, t, 0, c] -= eps
            lp, sp = _loss(xp, w, cfg)
            lm, sm = _loss(xm, w, cfg)
            for a, b in ((sp, st), (sm, st)):  # the selection must not move
                assert all(np.array_equal(a[0][0].sel[lv], b[0][0].sel[lv]) for lv in b[0][0].sel)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[name][0, t, 0, c]) <= 1e-6 * (1 + abs(fd)), (name, t, c)


def test_backward_matches_torch_autograd(rng):
    n, h, d, L, p, k, chunk = 512, 2, 8, 3, 4, 10, 32
    cfg = _cfg(L, p, k, chunk, bf16=False)
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    dy = rng.standard_normal((1, n, h, d))
    y, states = O.forward(x["q"], x["k"], x["v"], cfg)
    dq, dk, dv = O.backward(dy, states, cfg)
    for hh in range(h):
        st = states[0][hh]
        ents = list(zip(st.glev.tolist(), st.gidx.tolist()))
        m = torch.zeros(n, len(ents), dtype=torch.float64)
        for s, (lv, j) in enumerate(ents):
            e = (j + 1) * p**lv - 1
            m[e:min(n, e + p**lv), s] = 1.0
        ts = {a: torch.tensor(x[a][0, :, hh], requires_grad=True) for a in "qkv"}

        def gathered(t):
            lv_rows = [F.avg_pool1d(t.T[None], p**lv, p**lv)[0].T for lv in range(L)]
            return torch.stack([lv_rows[lv][j] for lv, j in ents])

        og = F.scaled_dot_product_attention(*(gathered(ts[a])[None] for a in "qkv"), is_causal=True)[0]
        yt = m @ og
        assert np.allclose(yt.detach().numpy(), y[0, :, hh], atol=1e-12)
        yt.backward(torch.from_numpy(dy[0, :, hh]))
        for a, g in zip("qkv", (dq, dk, dv)):
            assert np.allclose(ts[a].grad.numpy(), g[0, :, hh], atol=1e-11), a


def test_no_gradient_path_into_scores(rng):
    # Scaling every key row of a chunk by a positive constant can change the scores but the
    # backward never looks at them: it is a function of the frozen gathered set only.
    n, d, L, p = 256, 4, 3, 4
    cfg = _cfg(L, p, 6, 16, bf16=False)
    x = {w: rng.standard_normal((1, n, 1, d)) for w in "qkv"}
    dy = rng.standard_normal((1, n, 1, d))
    _, st = O.forward(x["q"], x["k"], x["v"], cfg)
    g1 = O.backward(dy, st, cfg)
    st[0][0].scores = [np.full_like(s, np.nan) for s in st[0][0].scores]
    g2 = O.backward(dy, st, cfg)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def test_direct_mode_length():
    cfg = _cfg(3, 4, 128, 64, mode=O.DIRECT)
    sizes, sel, glev, gidx = _random_state(4096, cfg)
    assert len(glev) == 256 + 128 + 128 == O.gathered_length(4096, cfg)


def test_given_selection_reproduces_own_selection(rng):
    n, h, d = 1024, 1, 8
    cfg = _cfg(3, 4, 24, 16, bf16=False)
    x = {w: rng.standard_normal((n, d)) for w in "qkv"}
    y0, st0 = O.head_forward(x["q"], x["k"], x["v"], cfg)
    y1, st1 = O.head_forward(x["q"], x["k"], x["v"], cfg, sel=st0.sel)
    assert np.array_equal(y0, y1)
    # a different (valid) selection changes the gathered set but keeps its length
    other = {lv: np.sort(np.random.default_rng(1).permutation(len(st0.scores[lv]))[:len(s)])
             for lv, s in st0.sel.items()}
    y2, st2 = O.head_forward(x["q"], x["k"], x["v"], cfg, sel=other)
    assert len(st2.glev) == len(st0.glev) and not np.array_equal(y2, y0)


# ---------------------------------------------------------------- DIRECT selection reading
# DIRECT is the literal reading of the pages' selector: k entries are kept at levels 0..L-2
# and enter the gathered sequence themselves; the coarsest level enters whole.  Each pin
# below fails if the selected levels are shifted to 1..L-1.
def test_direct_length_separates_level_ranges():
    # N = 4096, L = 3, p = 4, k = 512: levels 0, 1 keep 512 + 512 (S = 256 + 1024 = 1280);
    # levels 1, 2 would keep 512 + 256 (S = 1024).
    cfg = _cfg(3, 4, 512, 64, mode=O.DIRECT)
    assert O.selected_levels(cfg) == [0, 1]
    sizes, sel, glev, gidx = _random_state(4096, cfg)
    assert sorted(sel) == [0, 1]
    assert len(glev) == O.gathered_length(4096, cfg) == 1280
    assert np.bincount(glev, minlength=3).tolist() == [512, 512, 256]


def test_direct_worked_example_two_levels():
    # N = 16, p = 4, L = 2: level 0 = tokens (selected), level 1 = 4 blocks (kept whole).
    # Kept tokens 5 and 9 (causal positions 5, 9); coarsest entries at e = 3, 7, 11, 15.
    cfg = _cfg(2, 4, 2, 16, mode=O.DIRECT)
    sizes = O.level_sizes(16, 2, 4)
    glev, gidx = O.gathered_set({0: np.array([5, 9])}, sizes, cfg)
    assert list(zip(glev.tolist(), gidx.tolist())) == [
        (1, 0), (0, 5), (1, 1), (0, 9), (1, 2), (1, 3)]
    inv = O.inverse_map(glev, gidx, sizes)
    # scatter of ones: block j of level 1 reaches tokens [4j + 3, 4j + 6]; tokens reach themselves
    y = O.scatter(np.ones((6, 1)), inv, 16, 4)[:, 0]
    assert list(y) == [0, 0, 0, 1, 1, 2, 1, 1, 1, 2, 1, 1, 1, 1, 1, 1]
    dxg = np.arange(6, dtype=np.float64)[:, None] + 1.0
    dx = O.gather_pool_backward(dxg, inv, 16, 4)[:, 0]
    assert dx[9] == dxg[3, 0] + dxg[4, 0] / 4   # token 9 itself + block 2 (tokens 8..11)
    assert dx[5] == dxg[1, 0] + dxg[2, 0] / 4   # token 5 itself + block 1
    assert dx[0] == dxg[0, 0] / 4
    assert dx[15] == dxg[5, 0] / 4


def test_direct_worked_example_three_levels():
    # N = 16, p = 2, L = 3: tokens (level 0) and pairs (level 1) are selected, the four
    # 4-token blocks (level 2) are kept whole.  Kept: token 6 (e = 6); pairs 2 (tokens 4-5,
    # e = 5) and 5 (tokens 10-11, e = 11).  Pair 5 and block 2 share e = 11: the finer first.
    cfg = _cfg(3, 2, [1, 2, 0], 16, mode=O.DIRECT)
    sizes = O.level_sizes(16, 3, 2)
    glev, gidx = O.gathered_set({0: np.array([6]), 1: np.array([2, 5])}, sizes, cfg)
    assert list(zip(glev.tolist(), gidx.tolist())) == [
        (2, 0), (1, 2), (0, 6), (2, 1), (1, 5), (2, 2), (2, 3)]
    inv = O.inverse_map(glev, gidx, sizes)
    y = O.scatter(np.ones((7, 1)), inv, 16, 2)[:, 0]
    # block 0 -> 3..6, pair 2 -> 5..6, token 6 -> 6, block 1 -> 7..10, pair 5 -> 11..12,
    # block 2 -> 11..14, block 3 -> 15
    assert list(y) == [0, 0, 0, 1, 1, 2, 3, 1, 1, 1, 1, 2, 2, 1, 1, 1]
    dxg = np.arange(7, dtype=np.float64)[:, None] + 1.0
    dx = O.gather_pool_backward(dxg, inv, 16, 2)[:, 0]
    assert dx[5] == dxg[1, 0] / 2 + dxg[3, 0] / 4
    assert dx[6] == dxg[2, 0] + dxg[3, 0] / 4
    assert dx[11] == dxg[4, 0] / 2 + dxg[5, 0] / 4
    assert dx[0] == dxg[0, 0] / 4


def test_direct_full_budget_equals_dense_attention_over_pyramid(rng):
    # every entry of levels 0..L-2 kept: the gathered set is the whole pyramid
    n, h, d, L, p = 128, 1, 8, 3, 4
    x = {w: rng.standard_normal((1, n, h, d)) for w in "qkv"}
    cfg = _cfg(L, p, 10**6, 16, mode=O.DIRECT)
    y, _ = O.forward(x["q"], x["k"], x["v"], cfg)
    ref = _full_pyramid_reference(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], L, p)
    assert np.allclose(y[0, :, 0], ref, atol=1e-12)


def _library_layer(q, k, v, L, p, chunk, kk, mode, scorer="k"):
    """One head of the layer rebuilt from library routines (torch avg_pool1d, vector_norm,
    SDPA) with the brute-force rank count as the selector, without bf16 rounding."""
    n, d = q.shape
    t = {a: torch.from_numpy(x).T[None] for a, x in (("q", q), ("k", k), ("v", v))}
    lv = {a: [F.avg_pool1d(t[a], p**l, p**l)[0].T for l in range(L)] for a in "qkv"}
    nrm = {a: [torch.linalg.vector_norm(r, dim=1).numpy() for r in lv[a]] for a in "qkv"}
    if scorer == "k":
        sc = nrm["k"]
    elif scorer == "qk":
        sc = [a * b for a, b in zip(nrm["q"], nrm["k"])]
    else:
        sc = [np.sqrt(a**2 + b**2 + c**2) for a, b, c in zip(nrm["q"], nrm["k"], nrm["v"])]
    levels = range(0, L - 1) if mode == O.DIRECT else range(1, L)
    ents = [((j + 1) * p ** (L - 1) - 1, L - 1, j) for j in range(n // p ** (L - 1))]
    for l in levels:
        for j in _brute_select(sc[l], kk, chunk).tolist():
            if mode == O.DIRECT:
                ents.append(((j + 1) * p**l - 1, l, j))
            else:
                ents += [((j * p + c + 1) * p ** (l - 1) - 1, l - 1, j * p + c) for c in range(p)]
    ents.sort()
    g = {a: torch.stack([lv[a][l][j] for _, l, j in ents]) for a in "qkv"}
    og = F.scaled_dot_product_attention(g["q"][None], g["k"][None], g["v"][None], is_causal=True)[0]
    m = torch.zeros(n, len(ents), dtype=torch.float64)
    for s, (e, l, j) in enumerate(ents):
        m[e:min(n, e + p**l), s] = 1.0
    return (m @ og).numpy(), ents


@pytest.mark.parametrize("mode", [O.DIRECT, O.REFINE])
@pytest.mark.parametrize("scorer", ["k", "qk", "qkv"])
def test_layer_matches_library_reconstruction(rng, mode, scorer):
    n, d, L, p, kk, chunk = 512, 8, 3, 4, 9, 32
    x = {w: rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal((n, 1))) for w in "qkv"}
    cfg = O.Config(L, p, kk, chunk, mode=mode, bf16_attention=False, scorer=scorer)
    y, st = O.head_forward(x["q"], x["k"], x["v"], cfg)
    ref, ents = _library_layer(x["q"], x["k"], x["v"], L, p, chunk, kk, mode, scorer)
    assert list(zip(st.glev.tolist(), st.gidx.tolist())) == [(l, j) for _, l, j in ents]
    assert np.allclose(y, ref, atol=1e-12)


# ---------------------------------------------------------------- scorer variants
def test_scorer_variants_closed_forms():
    # one entry per row: q = a e1, k = b e1, v = c e2
    a = np.array([2.0, -3.0, 0.0, 1.5])
    b = np.array([4.0, 0.5, 7.0, -2.0])
    c = np.array([1.0, 6.0, -2.0, 0.0])
    d = 16
    qr, kr, vr = (np.zeros((4, d)) for _ in range(3))
    qr[:, 0], kr[:, 0], vr[:, 1] = a, b, c
    k_only = O.score_pyramid([kr], "k")[0]
    qk = O.score_pyramid([kr], "qk", [qr], [vr])[0]
    qkv = O.score_pyramid([kr], "qkv", [qr], [vr])[0]
    assert np.array_equal(k_only, np.abs(b))
    assert np.array_equal(qk, np.abs(a) * np.abs(b))
    assert np.allclose(qkv, np.sqrt(a**2 + b**2 + c**2), rtol=1e-15)
    with pytest.raises(ValueError):
        O.Config(3, 4, 8, 16, scorer="dilated")


def test_scorer_variants_change_the_selection():
    # Two level-1 blocks: block 0 has the larger pooled key, block 1 the larger pooled query
    # (and value).  The key scorer keeps block 0, the query-key product keeps block 1.
    n, d, p = 8, 4, 4
    q, k, v = (np.zeros((n, d)) for _ in range(3))
    k[0:4, 0] = 3.0
    k[4:8, 0] = 2.0
    q[0:4, 1] = 1.0
    q[4:8, 1] = 5.0
    v[4:8, 2] = 1.0
    picks = {}
    for scorer in ("k", "qk", "qkv"):
        cfg = O.Config(2, p, 1, 16, bf16_attention=False, scorer=scorer)
        _, scores, sel = O.head_selection(k, cfg, q=q, v=v)
        picks[scorer] = sel[1].tolist()
    assert picks == {"k": [0], "qk": [1], "qkv": [1]}
