"""Python binding of the C ABI (include/lh_api.h): argument marshalling only.

Every function has the name of the C entry point it calls.  torch supplies device memory
(outputs are allocated with torch.empty) and the current stream; every step of the layer runs
in liblh.so's HIP kernels.  Status codes other than LH_OK raise LhError.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LH_BF16, LH_F32, LH_SEL_DIRECT, LH_SEL_REFINE, LhAttnDesc, LhConfig, LhGathered, LhPlanInfo, check

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


def lh_build_map(cfg, sel):
    info = lh_plan(cfg)
    dev = sel.device
    gmap = torch.empty((cfg.batch, cfg.heads, info.gathered_pad), dtype=torch.int32, device=dev)
    inv = torch.empty((cfg.batch, cfg.heads, info.pyramid_total), dtype=torch.int32, device=dev)
    check(_lib.load().lh_build_map(ctypes.byref(cfg), _p(sel), _p(gmap), _p(inv), _stream()))
    return gmap, inv


def lh_gather(cfg, q, k, v, pq, pk, pv, gmap, with_backward=True):
    """Returns dict q, k, v ([B, H, Sp, D]) and qt, kt, vt ([B, H, D, Sp]), all bf16."""
    _check_tokens(cfg, q, k, v)
    info = lh_plan(cfg)
    sp, d = info.gathered_pad, cfg.head_dim
    dev = q.device
    out = {}
    for n in ("q", "k", "v", "qt", "kt", "vt"):
        if not with_backward and n in ("v", "qt", "kt"):
            out[n] = None
            continue
        shape = (cfg.batch, cfg.heads, d, sp) if n.endswith("t") else (cfg.batch, cfg.heads, sp, d)
        out[n] = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    g = LhGathered(*[None if out[n] is None else out[n].data_ptr()
                     for n in ("q", "k", "v", "qt", "kt", "vt")])
    code = LH_BF16 if pq is None or pq.dtype == torch.bfloat16 else LH_F32
    check(_lib.load().lh_gather(ctypes.byref(cfg), _p(q), _p(k), _p(v), _p(pq), _p(pk), _p(pv),
                                code, _p(gmap), ctypes.byref(g), _stream()))
    return out


def swap23_index(n: int, device=None):
    """Column order of the library's transposed tensors: slot s sits at column swap23(s)
    (bits 2 and 3 of s exchanged; an involution, so the same index maps both ways)."""
    s = torch.arange(n, device=device)
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def to_transposed(x):
    """[..., Sp, D] -> [..., D, Sp] in the library's transposed layout (Sp a multiple of 16)."""
    return x.transpose(-1, -2)[..., swap23_index(x.shape[-2], x.device)].contiguous()


def from_transposed(xt):
    """Inverse of to_transposed."""
    return xt[..., swap23_index(xt.shape[-1], xt.device)].transpose(-1, -2).contiguous()


def attn_desc(batch, heads, seq, head_dim, scale=0.0) -> LhAttnDesc:
    return LhAttnDesc(batch, heads, seq, head_dim, scale)


def lh_attn_fwd(desc: LhAttnDesc, q, k, vt):
    """q, k [B, H, Sp, D] bf16, vt [B, H, D, Sp] bf16 -> (o [B, H, Sp, D] f32, lse [B, H, Sp]);
    lse is the base-2 log-sum-exp of each row (natural log-sum-exp times log2(e))."""
    b, h, sp, d = q.shape
    o = torch.empty((b, h, sp, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((b, h, sp), dtype=torch.float32, device=q.device)
    check(_lib.load().lh_attn_fwd(ctypes.byref(desc), _p(q), _p(k), _p(vt), _p(o), _p(lse),
                                  _stream()))
    return o, lse


def lh_attn_bwd(desc: LhAttnDesc, q, k, v, qt, kt, lse, delta, dout, doutt):
    b, h, sp, d = q.shape
    dq, dk, dv = (torch.empty((b, h, sp, d), dtype=torch.float32, device=q.device)
                  for _ in range(3))
    check(_lib.load().lh_attn_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(qt), _p(kt),
                                  _p(lse), _p(delta), _p(dout), _p(doutt), _p(dq), _p(dk),
                                  _p(dv), _stream()))
    return dq, dk, dv


def lh_scatter(cfg, inv, og):
    y = torch.empty((cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim), dtype=torch_dtype(cfg),
                    device=og.device)
    check(_lib.load().lh_scatter(ctypes.byref(cfg), _p(inv), _p(og), _p(y), _stream()))
    return y


def lh_scatter_bwd(cfg, gmap, og, dy):
    _check_tokens(cfg, dy)
    info = lh_plan(cfg)
    sp, d = info.gathered_pad, cfg.head_dim
    dev = dy.device
    dog = torch.empty((cfg.batch, cfg.heads, sp, d), dtype=torch.bfloat16, device=dev)
    dogt = torch.empty((cfg.batch, cfg.heads, d, sp), dtype=torch.bfloat16, device=dev)
    delta = torch.empty((cfg.batch, cfg.heads, sp), dtype=torch.float32, device=dev)
    check(_lib.load().lh_scatter_bwd(ctypes.byref(cfg), _p(gmap), _p(og), _p(dy), _p(dog),
                                     _p(dogt), _p(delta), _stream()))
    return dog, dogt, delta


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
        """Typed views of the saved blob: gmap, inv, q, k, v, qt, kt, vt, o, lse."""
        i, c = self.info, self.cfg
        b, h, d, sp, p = c.batch, c.heads, c.head_dim, i.gathered_pad, i.pyramid_total

        def view(off, n, dtype, shape):
            nbytes = n * torch.tensor([], dtype=dtype).element_size()
            return self.saved[off:off + nbytes].view(dtype).view(shape)

        out = {
            "gmap": view(i.saved_gmap, b * h * sp, torch.int32, (b, h, sp)),
            "inv": view(i.saved_inv, b * h * p, torch.int32, (b, h, p)),
            "o": view(i.saved_o, b * h * sp * d, torch.float32, (b, h, sp, d)),
            "lse": view(i.saved_lse, b * h * sp, torch.float32, (b, h, sp)),
        }
        for n in ("q", "k", "v"):
            out[n] = view(getattr(i, "saved_" + n), b * h * sp * d, torch.bfloat16, (b, h, sp, d))
            out[n + "t"] = view(getattr(i, "saved_" + n + "t"), b * h * sp * d, torch.bfloat16,
                                (b, h, d, sp))
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


def lh_backward(cfg, bufs: Buffers, dy, dq=None, dk=None, dv=None):
    """Layer backward with the selection lh_forward saved in `bufs`; returns dq, dk, dv."""
    _check_tokens(cfg, dy, dq, dk, dv)
    dq = torch.empty_like(dy) if dq is None else dq
    dk = torch.empty_like(dy) if dk is None else dk
    dv = torch.empty_like(dy) if dv is None else dv
    check(_lib.load().lh_backward(ctypes.byref(cfg), _p(bufs.saved), _p(dy), _p(dq), _p(dk),
                                  _p(dv), _p(bufs.ws_bwd), bufs.ws_bwd.numel(), _stream()))
    return dq, dk, dv


class StagedLayer:
    """The layer as its stage entry points, on preallocated buffers (no allocation per call).

    Runs exactly the kernels lh_forward / lh_backward run, in the same order, so a caller
    can put timing events between stages.  `stages_fwd` / `stages_bwd` are lists of
    (name, callable) pairs.
    """

    def __init__(self, cfg: LhConfig, q, k, v, dy, device="cuda"):
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
        self.g = {n: e((b, h, d, sp) if n.endswith("t") else (b, h, sp, d), torch.bfloat16)
                  for n in ("q", "k", "v", "qt", "kt", "vt")}
        self.og = e((b, h, sp, d), torch.float32)
        self.lse = e((b, h, sp), torch.float32)
        self.y = torch.empty_like(q)
        self.dog = e((b, h, sp, d), torch.bfloat16)
        self.dogt = e((b, h, d, sp), torch.bfloat16)
        self.delta = e((b, h, sp), torch.float32)
        self.dxg = [e((b, h, sp, d), torch.float32) for _ in range(3)]
        self.dx = [torch.empty_like(q) for _ in range(3)]
        self.desc = attn_desc(b, h, i.gathered_len, d)
        self.gathered = LhGathered(*[self.g[n].data_ptr() for n in ("q", "k", "v", "qt", "kt", "vt")])
        lib = _lib.load()
        cr = ctypes.byref(cfg)
        dr = ctypes.byref(self.desc)
        P = _p
        g = self.g
        st = _stream
        self.stages_fwd = [
            ("pool_score", lambda: lib.lh_pool_score(cr, P(q), P(k), P(v), P(self.pq), P(self.pk),
                                                     P(self.pv), LH_BF16, P(self.scores), st())),
            ("topk", lambda: lib.lh_topk(cr, P(self.scores), P(self.sel), st())),
            ("build_map", lambda: lib.lh_build_map(cr, P(self.sel), P(self.gmap), P(self.inv), st())),
            ("gather", lambda: lib.lh_gather(cr, P(q), P(k), P(v), P(self.pq), P(self.pk), P(self.pv),
                                             LH_BF16, P(self.gmap), ctypes.byref(self.gathered), st())),
            ("attn_fwd", lambda: lib.lh_attn_fwd(dr, P(g["q"]), P(g["k"]), P(g["vt"]), P(self.og),
                                                 P(self.lse), st())),
            ("scatter", lambda: lib.lh_scatter(cr, P(self.inv), P(self.og), P(self.y), st())),
        ]
        bwd_args = lambda: (dr, P(g["q"]), P(g["k"]), P(g["v"]), P(g["qt"]), P(g["kt"]),  # noqa: E731
                            P(self.lse), P(self.delta), P(self.dog), P(self.dogt),
                            P(self.dxg[0]), P(self.dxg[1]), P(self.dxg[2]), st())
        self.stages_bwd = [
            ("scatter_bwd", lambda: lib.lh_scatter_bwd(cr, P(self.gmap), P(self.og), P(dy), P(self.dog),
                                                       P(self.dogt), P(self.delta), st())),
            ("attn_bwd_dkdv", lambda: lib.lh_attn_bwd_dkdv(*bwd_args())),
            ("attn_bwd_dq", lambda: lib.lh_attn_bwd_dq(*bwd_args())),
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
