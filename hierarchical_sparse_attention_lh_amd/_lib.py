"""ctypes view of include/lh_api.h and the loader of liblh.so.

torch is imported before the library is opened so that liblh.so binds to the HIP runtime
torch already mapped (same soname): device pointers and streams from torch are then valid
in the library.  A missing library is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblh.so")
MAX_LEVELS = 8

LH_BF16, LH_F32 = 0, 1
LH_SEL_REFINE, LH_SEL_DIRECT = 0, 1
SCORERS = {"k": 0, "qk": 1, "qkv": 2}  # lh_scorer

STATUS = {
    0: "LH_OK", -1: "LH_ERR_NULL", -2: "LH_ERR_SHAPE", -3: "LH_ERR_LEVELS", -4: "LH_ERR_POOL",
    -5: "LH_ERR_K", -6: "LH_ERR_CHUNK", -7: "LH_ERR_DTYPE", -8: "LH_ERR_ALIGN",
    -9: "LH_ERR_WORKSPACE", -10: "LH_ERR_LAUNCH", -11: "LH_ERR_UNSUPPORTED",
    -12: "LH_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20
CODE = {v: k for k, v in STATUS.items()}


class LhConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("levels", ctypes.c_int32), ("pool", ctypes.c_int32),
        ("k", ctypes.c_int32 * MAX_LEVELS), ("chunk", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("select_mode", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("scorer", ctypes.c_int32),
    ]


_I64L = ctypes.c_int64 * MAX_LEVELS


class LhPlanInfo(ctypes.Structure):
    _fields_ = [
        ("level_size", _I64L), ("level_offset", _I64L), ("pooled_offset", _I64L),
        ("pyramid_total", ctypes.c_int64), ("pooled_rows", ctypes.c_int64),
        ("k_eff", _I64L), ("n_chunks", _I64L), ("chunk_width", _I64L),
        ("quota_base", _I64L), ("quota_rem", _I64L), ("sel_offset", _I64L),
        ("sel_total", ctypes.c_int64), ("gathered_len", ctypes.c_int64),
        ("gathered_pad", ctypes.c_int64),
        ("saved_gmap", ctypes.c_size_t), ("saved_inv", ctypes.c_size_t),
        ("saved_pq", ctypes.c_size_t), ("saved_pk", ctypes.c_size_t), ("saved_pv", ctypes.c_size_t),
        ("saved_o", ctypes.c_size_t), ("saved_lse", ctypes.c_size_t),
        ("saved_bytes", ctypes.c_size_t),
        ("ws_forward_bytes", ctypes.c_size_t), ("ws_backward_bytes", ctypes.c_size_t),
        ("softmax_scale", ctypes.c_float),
    ]


_I64x3 = ctypes.c_int64 * 3


class LhAttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seq", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("q_stride", _I64x3), ("k_stride", _I64x3),
                ("v_stride", _I64x3), ("o_stride", _I64x3), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float)]


P = ctypes.c_void_p
_CFG = ctypes.POINTER(LhConfig)
_DESC = ctypes.POINTER(LhAttnDesc)
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SIGS = {
    "lh_plan": [_CFG, ctypes.POINTER(LhPlanInfo)],
    "lh_status_string": [ctypes.c_int],
    "lh_pool_score": [_CFG, P, P, P, P, P, P, _I32, P, P],
    "lh_topk": [_CFG, P, P, P],
    "lh_pool_score_topk": [_CFG, P, P, P, P, P, P, _I32, P, P, P],
    "lh_build_map": [_CFG, P, P, P, P],
    "lh_gather": [_CFG, P, P, P, P, P, P, _I32, P, P, P, P, P, P, P],
    "lh_attn_fwd": [_DESC, P, P, P, P, P, P],
    "lh_attn_ws_bytes": [_DESC, ctypes.POINTER(_SZ)],
    "lh_attn_bwd": [_DESC, P, P, P, P, P, P, P, P, P, P, _SZ, P],
    "lh_attn_fwd_mapped": [_CFG, P, P, P, P, P, P, P, P, P, P],
    "lh_attn_bwd_mapped": [_CFG, P, P, P, P, P, P, P, P, P, P, P, P, P, _I32, P],
    "lh_scatter": [_CFG, P, P, P, P],
    "lh_scatter_bwd": [_CFG, P, P, P, P, P, P],
    "lh_gather_pool_bwd": [_CFG, P, P, P, P, P, P, P, P],
    "lh_forward": [_CFG, P, P, P, P, P, P, _SZ, P],
    "lh_forward_noalloc": [_CFG, P, P, P, P, P, P],
    "lh_backward": [_CFG, P, P, P, P, P, P, P, P, P, _SZ, P],
}
EXPORTS = tuple(_SIGS)

_lib = None


def load():
    """Open liblh.so once (after torch) and declare every signature."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- maps the HIP runtime liblh.so must share

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m hierarchical_sparse_attention_lh_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "lh_status_string" else ctypes.c_int
    _lib = lib
    return lib


def hip_runtimes_mapped() -> list:
    """Paths of every libamdhip64 mapped into this process (there must be exactly one)."""
    seen = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[5]:
                seen.add(os.path.realpath(parts[5]))
    return sorted(seen)


class LhError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        self.name = STATUS.get(code, str(code))
        msg = load().lh_status_string(code).decode()
        super().__init__(f"{self.name}: {msg}")


def check(code: int):
    if code != 0:
        raise LhError(code)
