"""lh_forward_noalloc (the forward for callers that cannot allocate) against lh_forward,
through the C ABI: two calls in a row on one GPU, the second with a smaller input, each
compared bit for bit with lh_forward on the same inputs (same kernels, same order), and the
saved state checked by running lh_backward from it."""

import pytest
import torch

from hierarchical_sparse_attention_lh_amd import _lib, ops, synth

pytestmark = pytest.mark.gpu

# a forward workspace of ~33 MB, then a small ragged case (S = 552)
CASES = [synth.WORKLOADS["medium-32k"],
         synth.Workload("ragged", 1, 4096, 2, 64, "bf16", 3, 4, 37, 64, 11, True)]


def _inputs(w):
    x = synth.workload_inputs(w)
    return {n: torch.from_numpy(a).to("cuda").to(torch.bfloat16) for n, a in x.items()}


def test_forward_noalloc_matches_forward_on_two_calls():
    for w in CASES:
        print(f"[noalloc] {w.name}", flush=True)
        t = _inputs(w)
        cfg = ops.config_for(w)
        info = ops.lh_plan(cfg)
        assert info.ws_forward_bytes <= _lib.NOALLOC_SCRATCH_BYTES
        y_ref, bufs = ops.lh_forward(cfg, t["q"], t["k"], t["v"])
        g_ref = ops.lh_backward(cfg, t["q"], t["k"], t["v"], bufs, t["dy"])
        b2 = ops.Buffers(cfg)
        b2.saved.fill_(0xFF)  # stale NaN patterns: everything read must be written first
        y = torch.full_like(t["q"], float("nan"))
        ops.lh_forward_noalloc(cfg, t["q"], t["k"], t["v"], y, b2.saved)
        g = ops.lh_backward(cfg, t["q"], t["k"], t["v"], b2, t["dy"])
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        va, vb = bufs.views(), b2.views()
        S = info.gathered_len
        for name in ("gmap", "inv"):
            assert torch.equal(va[name], vb[name]), name
        for name in ("o", "lse"):
            assert torch.equal(va[name][:, :, :S], vb[name][:, :, :S]), name
        for a, b in zip(g_ref, g):
            assert torch.equal(a, b)
