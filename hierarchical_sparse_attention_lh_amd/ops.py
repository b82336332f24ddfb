"""Python binding of the C ABI (include/lh_api.h): argument marshalling only.

Every function has the name of the C entry point it calls.  torch supplies device memory
(outputs are allocated with torch.empty) and the current stream; every step of the layer runs
in liblh.so's HIP kernels.  Status codes other than LH_OK raise LhError.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LH_BF16, LH_F32, LH_SEL_DIRECT, LH_SEL_REFINE, LhAttnDesc, LhConfig, LhPlanInfo, check

_TORCH_DTYPE = {LH_BF16: torch.bfloat16, LH_F32: torch.float32}


def make_config(batch, n_tokens, heads, head_dim, levels, pool, k, chunk, dtype="bf16",
                scale=0.0, select_mode=LH_SEL_REFINE, scorer="k") -> LhConfig:
    """Fill an lh_config.  `k` is one budget for every level or a per-level list; `scorer`
    is "k", "qk" or "qkv" (or the lh_scorer code)."""
    cfg = LhConfig()
    cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim = batch, n_tokens, heads, head_dim
    cfg.levels, cfg.pool, cfg.chunk = levels, pool, chunk
    ks = [k] * _lib.MAX_LEVELS if isinstance(k, int) else list(k) + [0] * (_lib.MAX_LEVELS - len(k))
    for i in range(_lib.MAX_LEVELS):
        cfg.k[i] = int(ks[i])
    cfg.dtype = {"bf16": LH_BF16, "f32": LH_F32}.get(dtype, dtype)
    cfg.select_mode = select_mode
    cfg.softmax_scale = scale
    cfg.scorer = _lib.SCORERS.get(scorer, scorer)
    return cfg


def config_for(w) -> LhConfig:
    """lh_config of a synth.Workload."""
    return make_config(w.batch, w.n_tokens, w.heads, w.head_dim, w.levels, w.pool, w.k, w.chunk,
                       w.dtype, select_mode=LH_SEL_DIRECT if w.mode == "direct" else LH_SEL_REFINE,
                       scorer=w.scorer)


def torch_dtype(cfg: LhConfig):
    return _TORCH_DTYPE[cfg.dtype]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tokens(cfg, *ts):
    shape = (cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim)
    for t in ts:
        if t is None:
            continue
        if tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"expected a contiguous device tensor of shape {shape}")
        if t.dtype != torch_dtype(cfg):
            raise ValueError(f"expected dtype {torch_dtype(cfg)}, got {t.dtype}")


def lh_plan(cfg: LhConfig) -> LhPlanInfo:
    info = LhPlanInfo()
    check(_lib.load().lh_plan(ctypes.byref(cfg), ctypes.byref(info)))
    return info


def lh_status_string(code: int) -> str:
    return _lib.load().lh_status_string(code).decode()


def lh_pool_score(cfg, q, k, v, pooled_dtype=torch.float32):
    """Returns (pq, pk, pv, scores); pooled [B, pooled_rows, H, D], scores [B, H, P]."""
    _check_tokens(cfg, q, k, v)
    info = lh_plan(cfg)
    dev = q.device
    shape = (cfg.batch, max(1, info.pooled_rows), cfg.heads, cfg.head_dim)
    pq, pk, pv = (torch.empty(shape, dtype=pooled_dtype, device=dev) for _ in range(3))
    scores = torch.full((cfg.batch, cfg.heads, info.pyramid_total), float("nan"),
                        dtype=torch.float32, device=dev)
    code = LH_F32 if pooled_dtype == torch.float32 else LH_BF16
    check(_lib.load().lh_pool_score(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq), _p(pk),
                                    _p(pv), code, _p(scores), _stream()))
    return pq, pk, pv, scores


def lh_topk(cfg, scores):
    info = lh_plan(cfg)
    sel = torch.empty((cfg.batch, cfg.heads, max(1, info.sel_total)), dtype=torch.int32,
                      device=scores.device)
    check(_lib.load().lh_topk(ctypes.byref(cfg), _p(scores), _p(sel), _stream()))
    return sel


def lh_pool_score_topk(cfg, q, k, v, pooled_dtype=torch.float32):
    """Stages 1-3 in one call: returns (pq, pk, pv, scores, sel).  When the fused kernel runs,
    the scores of the finest selected level are left as NaN (never written)."""
    _check_tokens(cfg, q, k, v)
    info = lh_plan(cfg)
    dev = q.device
    shape = (cfg.batch, max(1, info.pooled_rows), cfg.heads, cfg.head_dim)
    pq, pk, pv = (torch.empty(shape, dtype=pooled_dtype, device=dev) for _ in range(3))
    scores = torch.full((cfg.batch, cfg.heads, info.pyramid_total), float("nan"),
                        dtype=torch.float32, device=dev)
    sel = torch.empty((cfg.batch, cfg.heads, max(1, info.sel_total)), dtype=torch.int32,
                      device=dev)
    code = LH_F32 if pooled_dtype == torch.float32 else LH_BF16
    check(_lib.load().lh_pool_score_topk(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq),
                                         _p(pk), _p(pv), code, _p(scores), _p(sel), _stream()))
    return pq, pk, pv, scores, sel


def lh_build_map(cfg, sel):
    info = lh_plan(cfg)
    dev = sel.device
    gmap = torch.empty((cfg.batch, cfg.heads, info.gathered_pad), dtype=torch.int32, device=dev)
    inv = torch.empty((cfg.batch, cfg.heads, info.pyramid_total), dtype=torch.int32, device=dev)
    check(_lib.load().lh_build_map(ctypes.byref(cfg), _p(sel), _p(gmap), _p(inv), _stream()))
    return gmap, inv


def lh_gather(cfg, q, k, v, pq, pk, pv, sel):
    """Map and gathered rows in one call: returns (gmap, inv, {"q", "k", "v": [B, H, Sp, D] bf16})."""
    _check_tokens(cfg, q, k, v)
    info = lh_plan(cfg)
    sp, d = info.gathered_pad, cfg.head_dim
    dev = q.device
    gmap = torch.empty((cfg.batch, cfg.heads, sp), dtype=torch.int32, device=dev)
    inv = torch.empty((cfg.batch, cfg.heads, info.pyramid_total), dtype=torch.int32, device=dev)
    out = {n: torch.empty((cfg.batch, cfg.heads, sp, d), dtype=torch.bfloat16, device=dev)
           for n in "qkv"}
    code = LH_BF16 if pq is None or pq.dtype == torch.bfloat16 else LH_F32
    check(_lib.load().lh_gather(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq), _p(pk), _p(pv),
                                code, _p(sel), _p(gmap), _p(inv), _p(out["q"]), _p(out["k"]),
                                _p(out["v"]), _stream()))
    return gmap, inv, out


_AXES = {"bhsd": (0, 1, 2), "bshd": (0, 2, 1)}  # tensor dims of (batch, head, position)


def attn_desc(q, k, v, o, causal=True, scale=0.0, layout="bhsd") -> LhAttnDesc:
    """lh_attn_desc of torch tensors laid out [B, H, S, D] ("bhsd") or [B, S, H, D] ("bshd",
    e.g. the layer's token tensors); strides come from the tensors themselves."""
    ax = _AXES[layout]
    b, h, s_, d = (q.shape[ax[0]], q.shape[ax[1]], q.shape[ax[2]], q.shape[3])
    desc = LhAttnDesc()
    desc.batch, desc.heads, desc.seq, desc.head_dim = b, h, s_, d
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        if t.stride(3) != 1:
            raise ValueError("the last dimension must be contiguous")
        st = getattr(desc, name)
        for i in range(3):
            st[i] = t.stride(ax[i])
    desc.causal = 1 if causal else 0
    desc.scale = scale
    return desc


def _lse_shape(desc):
    return (desc.batch, desc.heads, (desc.seq + 127) // 128 * 128)


def lh_attn_fwd(q, k, v, causal=True, scale=0.0, layout="bhsd"):
    """Softmax attention over strided bf16 rows; returns (o float32 shaped like q, lse
    [B, H, Sp] in base 2: the natural log-sum-exp times log2(e))."""
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    desc = attn_desc(q, k, v, o, causal, scale, layout)
    lse = torch.empty(_lse_shape(desc), dtype=torch.float32, device=q.device)
    check(_lib.load().lh_attn_fwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse),
                                  _stream()))
    return o, lse


def lh_attn_bwd(q, k, v, o, lse, dout, causal=True, scale=0.0, layout="bhsd"):
    """Backward of lh_attn_fwd (dout bf16 laid out like o); returns float32 dq, dk, dv."""
    desc = attn_desc(q, k, v, o, causal, scale, layout)
    if dout.stride() != o.stride():
        raise ValueError("dout must have the layout of o")
    lib = _lib.load()
    nbytes = ctypes.c_size_t(0)
    check(lib.lh_attn_ws_bytes(ctypes.byref(desc), ctypes.byref(nbytes)))
    ws = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty(o.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    check(lib.lh_attn_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse), _p(dout),
                          _p(dq), _p(dk), _p(dv), _p(ws), ws.numel(), _stream()))
    return dq, dk, dv


def lh_attn_fwd_mapped(cfg, q, k, v, pq, pk, pv, gmap):
    """The layer's attention with rows read through gmap: returns (og [B, H, Sp, D] float32,
    lse [B, H, Sp]).  q, k, v are bf16 token tensors; pq/pk/pv bf16 pooled levels."""
    info = lh_plan(cfg)
    sp, d = info.gathered_pad, cfg.head_dim
    og = torch.empty((cfg.batch, cfg.heads, sp, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((cfg.batch, cfg.heads, sp), dtype=torch.float32, device=q.device)
    check(_lib.load().lh_attn_fwd_mapped(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq), _p(pk),
                                         _p(pv), _p(gmap), _p(og), _p(lse), _stream()))
    return og, lse


def lh_attn_bwd_mapped(cfg, q, k, v, pq, pk, pv, gmap, lse, delta, dog, passes=3):
    """Backward of lh_attn_fwd_mapped; returns float32 dqg, dkg, dvg [B, H, Sp, D]."""
    shape = dog.shape
    dqg, dkg, dvg = (torch.empty(shape, dtype=torch.float32, device=dog.device) for _ in range(3))
    check(_lib.load().lh_attn_bwd_mapped(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq), _p(pk),
                                         _p(pv), _p(gmap), _p(lse), _p(delta), _p(dog), _p(dqg),
                                         _p(dkg), _p(dvg), passes, _stream()))
    return dqg, dkg, dvg


def lh_scatter(cfg, inv, og):
    y = torch.empty((cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim), dtype=torch_dtype(cfg),
                    device=og.device)
    check(_lib.load().lh_scatter(ctypes.byref(cfg), _p(inv), _p(og), _p(y), _stream()))
    return y


def lh_scatter_bwd(cfg, gmap, og, dy):
    """Returns (dog [B, H, Sp, D] bf16, delta [B, H, Sp] float32)."""
    _check_tokens(cfg, dy)
    info = lh_plan(cfg)
    sp, d = info.gathered_pad, cfg.head_dim
    dev = dy.device
    dog = torch.empty((cfg.batch, cfg.heads, sp, d), dtype=torch.bfloat16, device=dev)
    delta = torch.empty((cfg.batch, cfg.heads, sp), dtype=torch.float32, device=dev)
    check(_lib.load().lh_scatter_bwd(ctypes.byref(cfg), _p(gmap), _p(og), _p(dy), _p(dog),
                                     _p(delta), _stream()))
    return dog, delta


def lh_gather_pool_bwd(cfg, inv, dqg, dkg, dvg):
    shape = (cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim)
    dq, dk, dv = (torch.empty(shape, dtype=torch_dtype(cfg), device=dqg.device) for _ in range(3))
    check(_lib.load().lh_gather_pool_bwd(ctypes.byref(cfg), _p(inv), _p(dqg), _p(dkg), _p(dvg),
                                         _p(dq), _p(dk), _p(dv), _stream()))
    return dq, dk, dv


class Buffers:
    """Device buffers one layer call needs (saved blob and workspaces), sized by lh_plan."""

    def __init__(self, cfg: LhConfig, device="cuda"):
        self.cfg = cfg
        self.info = lh_plan(cfg)
        i = self.info
        self.saved = torch.empty(i.saved_bytes, dtype=torch.uint8, device=device)
        self.ws_fwd = torch.empty(max(256, i.ws_forward_bytes), dtype=torch.uint8, device=device)
        self.ws_bwd = torch.empty(max(256, i.ws_backward_bytes), dtype=torch.uint8, device=device)

    def views(self):
        """Typed views of the saved blob: gmap, inv, pq, pk, pv, o, lse."""
        i, c = self.info, self.cfg
        b, h, d, sp, p = c.batch, c.heads, c.head_dim, i.gathered_pad, i.pyramid_total

        def view(off, n, dtype, shape):
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return self.saved[off:off + nbytes].view(dtype).view(shape)

        pr = max(1, i.pooled_rows) if i.pooled_rows else 0
        out = {
            "gmap": view(i.saved_gmap, b * h * sp, torch.int32, (b, h, sp)),
            "inv": view(i.saved_inv, b * h * p, torch.int32, (b, h, p)),
            "o": view(i.saved_o, b * h * sp * d, torch.float32, (b, h, sp, d)),
            "lse": view(i.saved_lse, b * h * sp, torch.float32, (b, h, sp)),
        }
        for n in ("pq", "pk", "pv"):
            out[n] = view(getattr(i, "saved_" + n), b * pr * h * d, torch.bfloat16, (b, pr, h, d))
        return out


def lh_forward(cfg, q, k, v, bufs: Buffers | None = None, y=None):
    """Layer forward; returns (y, bufs).  `bufs.saved` feeds lh_backward."""
    _check_tokens(cfg, q, k, v, y)
    bufs = bufs or Buffers(cfg, q.device)
    if y is None:
        y = torch.empty_like(q)
    check(_lib.load().lh_forward(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(y), _p(bufs.saved),
                                 _p(bufs.ws_fwd), bufs.ws_fwd.numel(), _stream()))
    return y, bufs


def lh_forward_noalloc(cfg, q, k, v, y, saved):
    """lh_forward with the library's static per-GPU workspace; y and saved are caller-given
    (saved: a uint8 device tensor of lh_plan(cfg).saved_bytes).  Allocates nothing."""
    _check_tokens(cfg, q, k, v, y)
    check(_lib.load().lh_forward_noalloc(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(y),
                                         _p(saved), _stream()))
    return y


def lh_backward(cfg, q, k, v, bufs: Buffers, dy, dq=None, dk=None, dv=None):
    """Layer backward with the selection lh_forward saved in `bufs` (q, k, v: the forward's
    inputs); returns dq, dk, dv."""
    _check_tokens(cfg, q, k, v, dy, dq, dk, dv)
    dq = torch.empty_like(dy) if dq is None else dq
    dk = torch.empty_like(dy) if dk is None else dk
    dv = torch.empty_like(dy) if dv is None else dv
    check(_lib.load().lh_backward(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(bufs.saved), _p(dy),
                                  _p(dq), _p(dk), _p(dv), _p(bufs.ws_bwd), bufs.ws_bwd.numel(),
                                  _stream()))
    return dq, dk, dv


class StagedLayer:
    """The layer as its stage entry points, on preallocated buffers (no allocation per call).

    Runs exactly the kernels lh_forward / lh_backward run, in the same order, so a caller
    can put timing events between stages.  `stages_fwd` / `stages_bwd` are lists of
    (name, callable) pairs.  bf16 layers only (a float32 layer also rounds its inputs).
    """

    def __init__(self, cfg: LhConfig, q, k, v, dy, device="cuda"):
        if cfg.dtype != LH_BF16:
            raise ValueError("StagedLayer runs bf16 layers")
        self.cfg = cfg
        self.info = i = lh_plan(cfg)
        c = cfg
        self.q, self.k, self.v, self.dy = q, k, v, dy
        b, h, d, sp = c.batch, c.heads, c.head_dim, i.gathered_pad
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
        pooled = (b, max(1, i.pooled_rows), h, d)
        self.pq, self.pk, self.pv = (e(pooled, torch.bfloat16) for _ in range(3))
        self.scores = e((b, h, i.pyramid_total), torch.float32)
        self.sel = e((b, h, max(1, i.sel_total)), torch.int32)
        self.gmap = e((b, h, sp), torch.int32)
        self.inv = e((b, h, i.pyramid_total), torch.int32)
        self.og = e((b, h, sp, d), torch.float32)
        self.lse = e((b, h, sp), torch.float32)
        self.y = torch.empty_like(q)
        self.dog = e((b, h, sp, d), torch.bfloat16)
        self.delta = e((b, h, sp), torch.float32)
        self.dxg = [e((b, h, sp, d), torch.float32) for _ in range(3)]
        self.dx = [torch.empty_like(q) for _ in range(3)]
        lib = _lib.load()
        cr = ctypes.byref(cfg)
        P = _p
        st = _stream
        pools = (P(self.pq), P(self.pk), P(self.pv))
        self.stages_fwd = [
            ("pool_score", lambda: lib.lh_pool_score(cr, P(q), P(k), P(v), *pools, LH_BF16,
                                                     P(self.scores), st())),
            ("topk", lambda: lib.lh_topk(cr, P(self.scores), P(self.sel), st())),
            ("build_map", lambda: lib.lh_build_map(cr, P(self.sel), P(self.gmap), P(self.inv), st())),
            ("attn_fwd", lambda: lib.lh_attn_fwd_mapped(cr, P(q), P(k), P(v), *pools, P(self.gmap),
                                                        P(self.og), P(self.lse), st())),
            ("scatter", lambda: lib.lh_scatter(cr, P(self.inv), P(self.og), P(self.y), st())),
        ]

        def bwd(passes):
            return lambda: lib.lh_attn_bwd_mapped(cr, P(q), P(k), P(v), *pools, P(self.gmap),
                                                  P(self.lse), P(self.delta), P(self.dog),
                                                  P(self.dxg[0]), P(self.dxg[1]), P(self.dxg[2]),
                                                  passes, st())

        self.stages_bwd = [
            ("scatter_bwd", lambda: lib.lh_scatter_bwd(cr, P(self.gmap), P(self.og), P(dy),
                                                       P(self.dog), P(self.delta), st())),
            ("attn_bwd_dkdv", bwd(1)),
            ("attn_bwd_dq", bwd(2)),
            ("gather_pool_bwd", lambda: lib.lh_gather_pool_bwd(cr, P(self.inv), P(self.dxg[0]),
                                                               P(self.dxg[1]), P(self.dxg[2]),
                                                               P(self.dx[0]), P(self.dx[1]),
                                                               P(self.dx[2]), st())),
        ]

    def run(self, stages, between=None):
        for i, (name, fn) in enumerate(stages):
            check(fn())
            if between is not None:
                between(i, name)
