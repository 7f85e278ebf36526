"""lh_score_topk_noalloc: the selection with the library's own per-GPU scratch
array instead of a caller workspace, for callers that cannot allocate.  Its
maps must equal lh_score_topk's bit for bit, call after call (the array keeps
the previous call's contents), and sizes beyond the array are refused on the
host before any launch."""
import ctypes

import pytest
import torch

from long_context_pretraining_amd import inputs
from long_context_pretraining_amd import lighthouse as lh

W = inputs.Workload
FAKE = 0x100000   # aligned, never dereferenced: the size check fails before any device call


def test_oversize_refused_before_any_launch():
    lib = lh.load_library()
    w = inputs.WORKLOADS["extreme_512k"]   # B*H = 16, N = 524288: 78 MB from q and k
    desc = lh.make_desc(w.B, w.H, w.N, w.d, w.p, w.L, w.k, torch.bfloat16)
    D = ctypes.byref(desc)
    assert lib.lh_score_topk_noalloc(D, FAKE, FAKE, None, FAKE, FAKE, None) == lh.LH_E_WORKSPACE
    assert lib.lh_score_topk_noalloc(D, None, FAKE, FAKE, FAKE, FAKE, None) == lh.LH_E_ARG
    assert lib.lh_score_topk_noalloc(D, FAKE, FAKE, FAKE + 4, FAKE, FAKE, None) == lh.LH_E_ARG


def _maps(w, use_pyr, noalloc):
    dt = inputs.TORCH_DTYPE[w.dtype]
    q, k, v = (x.cuda() for x in inputs.make_qkv(w))
    layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, dt)
    if layer.pyr is not None:
        lh.lh_pyramid(layer.desc, q, k, v, layer.pyr)
    pyr = layer.pyr if use_pyr else None
    gidx, gpos = torch.full_like(layer.gidx, -7), torch.full_like(layer.gpos, -7)
    if noalloc:
        lh.lh_score_topk_noalloc(layer.desc, q, k, pyr, gidx, gpos)
    else:
        lh.lh_score_topk(layer.desc, q, k, pyr, gidx, gpos, layer.sel_ws)
    torch.cuda.synchronize()
    return gidx.cpu(), gpos.cpu()


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lh.load_library()
    big = W("noalloc_big", 1, 16, 98304, 64, "bf16", 4, 4, 1536, 3, True)     # the 98K layer: 15 MB of scratch
    small = W("noalloc_small", 2, 3, 1000, 64, "bf16", 2, 3, 13, 101, True)  # then a smaller input
    for w, use_pyr in ((big, False), (small, False), (big, True), (small, True)):
        print(f"[noalloc] {w.name} norms from {'pyramid' if use_pyr else 'q, k'}", flush=True)
        ref = _maps(w, use_pyr, noalloc=False)
        got = _maps(w, use_pyr, noalloc=True)
        assert torch.equal(ref[0], got[0]), f"{w.name}: gidx differs"
        assert torch.equal(ref[1], got[1]), f"{w.name}: gpos differs"
