"""The C-ABI library on the host (no GPU): it loads, exports every declared symbol, binds to
the one HIP runtime torch mapped, plans sizes by the closed forms, and rejects every invalid
argument on the host before anything is launched."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle as O
from hierarchical_sparse_attention_lh_amd import _lib, ops, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lh_api.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lh_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (lh_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_single_hip_runtime_mapped():
    _lib.load()
    assert len(_lib.hip_runtimes_mapped()) == 1


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plan_matches_closed_forms(name):
    w = synth.WORKLOADS[name]
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    ocfg = O.Config(w.levels, w.pool, w.k, w.chunk)
    sizes = O.level_sizes(w.n_tokens, w.levels, w.pool)
    assert info.gathered_len == O.gathered_length(w.n_tokens, ocfg)
    assert info.gathered_pad % 128 == 0 and 0 <= info.gathered_pad - info.gathered_len < 128
    assert [info.level_size[l] for l in range(w.levels)] == sizes
    assert info.pyramid_total == sum(sizes)
    assert info.sel_total == sum(min(w.k, n) for n in sizes[1:])
    assert abs(info.softmax_scale - w.head_dim ** -0.5) < 1e-7
    offs = [info.saved_gmap, info.saved_inv, info.saved_pq, info.saved_pk, info.saved_pv,
            info.saved_o, info.saved_lse]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert info.saved_bytes > info.saved_lse
    # the saved blob holds no gathered copy of Q, K, V: map, pooled levels, Og and LSE only
    pooled = w.batch * info.pooled_rows * w.heads * w.head_dim * 2
    assert info.saved_pk - info.saved_pq >= pooled and info.saved_o - info.saved_pv >= pooled
    for lv in range(1, w.levels):
        nch = info.n_chunks[lv]
        assert info.quota_base[lv] * nch + info.quota_rem[lv] == info.k_eff[lv]
        assert 0 <= info.quota_rem[lv] < nch


def _cfg(**kw):
    base = dict(batch=1, n_tokens=4096, heads=2, head_dim=64, levels=3, pool=4, k=128, chunk=64,
                dtype="f32")
    base.update(kw)
    return ops.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), "LH_ERR_SHAPE"),
    (dict(n_tokens=4095), "LH_ERR_SHAPE"),        # p^(L-1) does not divide N
    (dict(n_tokens=2**31), "LH_ERR_SHAPE"),
    (dict(heads=0), "LH_ERR_SHAPE"),
    (dict(head_dim=96), "LH_ERR_DTYPE"),
    (dict(dtype=7), "LH_ERR_DTYPE"),
    (dict(levels=0), "LH_ERR_LEVELS"),
    (dict(levels=9), "LH_ERR_LEVELS"),
    (dict(pool=1), "LH_ERR_POOL"),
    (dict(pool=17), "LH_ERR_POOL"),
    (dict(k=-1), "LH_ERR_K"),
    (dict(chunk=48), "LH_ERR_CHUNK"),
    (dict(chunk=8), "LH_ERR_CHUNK"),
    (dict(chunk=4096), "LH_ERR_CHUNK"),
    (dict(n_tokens=12288, levels=2, chunk=2048), "LH_ERR_CHUNK"),  # level 1: 3072 entries
    # gathered length S = N + 1 above 2^24 (dense attention over every token, L = 1)
    (dict(n_tokens=2**24 + 1, levels=1, k=0), "LH_ERR_SHAPE"),
])
def test_plan_rejects(kw, code):
    with pytest.raises(_lib.LhError) as e:
        ops.lh_plan(_cfg(**kw))
    assert e.value.name == code


def test_unknown_select_mode_is_reported_unsupported():
    with pytest.raises(_lib.LhError) as e:
        ops.lh_plan(_cfg(select_mode=7))
    assert e.value.name == "LH_ERR_UNSUPPORTED"


@pytest.mark.parametrize("levels,pool,k,n", [(3, 4, 100, 4096), (4, 2, 64, 2048), (2, 4, 5000, 4096),
                                             (4, 4, 4096, 524288)])
def test_plan_direct_closed_forms(levels, pool, k, n):
    cfg = _cfg(select_mode=_lib.LH_SEL_DIRECT, levels=levels, pool=pool, k=k, n_tokens=n, chunk=64)
    info = ops.lh_plan(cfg)
    ocfg = O.Config(levels, pool, k, 64, mode=O.DIRECT)
    assert info.gathered_len == O.gathered_length(n, ocfg)
    sizes = O.level_sizes(n, levels, pool)
    assert info.gathered_len == sizes[-1] + sum(min(k, m) for m in sizes[:-1])
    assert [info.k_eff[l] for l in range(levels)] == [min(k, m) for m in sizes[:-1]] + [0]
    assert info.sel_total == sum(min(k, m) for m in sizes[:-1])


def _call(name, *args):
    return getattr(_lib.load(), name)(*args)


def _desc(seq=100, d=64, strides=None):
    desc = _lib.LhAttnDesc()
    desc.batch, desc.heads, desc.seq, desc.head_dim = 1, 1, seq, d
    st = strides or (seq * d, seq * d, d)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        for i in range(3):
            getattr(desc, name)[i] = st[i]
    desc.causal = 1
    return desc


def test_entry_points_reject_bad_pointers_before_launch():
    cfg = _cfg()
    c = ctypes.byref(cfg)
    ok = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
    bad = ctypes.c_void_p(0x10004)  # not 16-byte aligned
    null = None
    st = None
    L = _lib.CODE
    assert _call("lh_pool_score", None, ok, ok, ok, ok, ok, ok, 0, ok, st) == L["LH_ERR_NULL"]
    assert _call("lh_pool_score", c, null, ok, ok, ok, ok, ok, 0, ok, st) == L["LH_ERR_NULL"]
    assert _call("lh_pool_score", c, ok, bad, ok, ok, ok, ok, 0, ok, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_pool_score", c, ok, ok, ok, ok, ok, ok, 5, ok, st) == L["LH_ERR_DTYPE"]
    assert _call("lh_topk", c, null, ok, st) == L["LH_ERR_NULL"]
    assert _call("lh_pool_score_topk", c, ok, ok, ok, ok, ok, ok, 0, ok, null, st) == L["LH_ERR_NULL"]
    assert _call("lh_pool_score_topk", c, ok, ok, ok, ok, ok, ok, 5, ok, ok, st) == L["LH_ERR_DTYPE"]
    assert _call("lh_pool_score_topk", c, ok, ok, ok, null, ok, null, 0, bad, ok, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_build_map", c, ok, bad, ok, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_gather", c, ok, ok, ok, ok, ok, ok, 0, ok, ok, ok, ok, ok, null, st) == L["LH_ERR_NULL"]
    assert _call("lh_gather", c, ok, ok, ok, ok, ok, ok, 0, null, ok, ok, ok, ok, ok, st) == L["LH_ERR_NULL"]
    assert _call("lh_gather", c, ok, ok, ok, ok, ok, ok, 3, ok, ok, ok, ok, ok, ok, st) == L["LH_ERR_DTYPE"]
    d = _desc()
    dd = ctypes.byref(d)
    assert _call("lh_attn_fwd", dd, ok, ok, ok, ok, bad, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_attn_fwd", ctypes.byref(_desc(seq=0)), ok, ok, ok, ok, ok, st) == L["LH_ERR_SHAPE"]
    # above the attention length bound, and at it (reaches the pointer checks)
    assert _call("lh_attn_fwd", ctypes.byref(_desc(seq=2**24 + 1)), ok, ok, ok, ok, ok, st) == L["LH_ERR_SHAPE"]
    assert _call("lh_attn_fwd", ctypes.byref(_desc(seq=2**24)), ok, ok, ok, ok, bad, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_attn_fwd", ctypes.byref(_desc(d=32)), ok, ok, ok, ok, ok, st) == L["LH_ERR_DTYPE"]
    # a row stride that breaks 16-byte alignment of the rows
    assert _call("lh_attn_fwd", ctypes.byref(_desc(strides=(6400, 6400, 68))), ok, ok, ok, ok, ok,
                 st) == L["LH_ERR_ALIGN"]
    nbytes = ctypes.c_size_t(0)
    assert _call("lh_attn_ws_bytes", dd, ctypes.byref(nbytes)) == 0 and nbytes.value >= 128 * 4
    assert _call("lh_attn_bwd", dd, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, nbytes.value - 1, st) == \
        L["LH_ERR_WORKSPACE"]
    assert _call("lh_attn_bwd", dd, ok, ok, ok, null, ok, ok, ok, ok, ok, ok, nbytes.value, st) == \
        L["LH_ERR_NULL"]
    assert _call("lh_attn_fwd_mapped", c, ok, ok, ok, ok, ok, ok, null, ok, ok, st) == L["LH_ERR_NULL"]
    assert _call("lh_attn_bwd_mapped", c, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, 4,
                 st) == L["LH_ERR_UNSUPPORTED"]
    assert _call("lh_attn_bwd_mapped", c, ok, ok, ok, ok, ok, ok, ok, ok, ok, ok, null, ok, ok, 3,
                 st) == L["LH_ERR_NULL"]
    assert _call("lh_scatter", c, ok, ok, bad, st) == L["LH_ERR_ALIGN"]
    assert _call("lh_scatter_bwd", c, ok, ok, ok, ok, null, st) == L["LH_ERR_NULL"]
    assert _call("lh_gather_pool_bwd", c, ok, ok, ok, ok, ok, ok, bad, st) == L["LH_ERR_ALIGN"]
    info = ops.lh_plan(cfg)
    assert _call("lh_forward", c, ok, ok, ok, ok, ok, ok, info.ws_forward_bytes - 1, st) == L["LH_ERR_WORKSPACE"]
    assert _call("lh_backward", c, ok, ok, ok, ok, ok, ok, ok, ok, ok,
                 info.ws_backward_bytes - 1, st) == L["LH_ERR_WORKSPACE"]
    assert _call("lh_backward", c, null, ok, ok, ok, ok, ok, ok, ok, ok, 1 << 40, st) == L["LH_ERR_NULL"]
    assert _call("lh_forward", c, ok, ok, ok, null, ok, ok, 1 << 40, st) == L["LH_ERR_NULL"]


def test_status_strings():
    for code in _lib.STATUS:
        s = ops.lh_status_string(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert ops.lh_status_string(12345) == "unknown status"


def test_forward_noalloc_rejects_workspace_above_scratch_before_launch():
    # the benchmark workloads fit the static scratch; 2^20 tokens x 16 heads do not
    for w in synth.WORKLOADS.values():
        assert ops.lh_plan(ops.config_for(w)).ws_forward_bytes <= _lib.NOALLOC_SCRATCH_BYTES
    cfg = ops.make_config(1, 2**20, 16, 64, 4, 4, 4096, 1024)
    assert ops.lh_plan(cfg).ws_forward_bytes > _lib.NOALLOC_SCRATCH_BYTES
    ok = ctypes.c_void_p(0x10000)
    code = _call("lh_forward_noalloc", ctypes.byref(cfg), ok, ok, ok, ok, ok, None)
    assert code == _lib.CODE["LH_ERR_SCRATCH"]
    small = _cfg()
    assert _call("lh_forward_noalloc", ctypes.byref(small), ok, None, ok, ok, ok, None) == \
        _lib.CODE["LH_ERR_NULL"]
