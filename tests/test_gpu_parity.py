"""HIP path vs the oracle, through the C ABI, on seeded synthetic inputs.

Selection maps bit-exact; tensors within the stated tolerances (see
tests/gpu_support.check_close).  Sizes span several tiles and ragged tails."""
import numpy as np
import pytest
import torch

from long_context_pretraining_amd import inputs
from long_context_pretraining_amd import lighthouse as lh
from oracle import lighthouse_oracle as orc
from tests.gpu_support import (check_close, compare_head, compare_selection, head_np, run_layer, say, to_np)

pytestmark = pytest.mark.gpu

W = inputs.Workload
SMALL = [
    inputs.WORKLOADS["tiny_f32"],                                   # B1 H1 N4096 d64 f32 p4 L3 k64, S=768
    W("ragged_bf16", 2, 3, 1000, 64, "bf16", 2, 3, 13, 101, True),  # S = 302
    W("ragged_f32", 1, 2, 1000, 64, "f32", 2, 3, 13, 103, False),
    W("p3_d128_bf16", 1, 2, 729, 128, "bf16", 3, 4, 7, 102, True),  # generic p, d = 128, S = 90
    W("clamped_bf16", 1, 2, 4096, 64, "bf16", 4, 4, 100, 104, True),  # k > M_3: S = 1120 < formula
    W("all_levels_bf16", 1, 1, 256, 64, "bf16", 4, 3, 1000, 106, True),  # every level fully expanded
    W("minimal_bf16", 1, 1, 16, 64, "bf16", 4, 3, 1, 107, False),    # N = p^(L-1), S = 9
    W("L2_bf16", 1, 2, 512, 64, "bf16", 4, 2, 40, 105, True),
    W("p2_L8_bf16", 1, 1, 2048, 64, "bf16", 2, 8, 5, 108, True),     # deepest pyramid
    # p^(L-1) = 4096: the coarse levels of a scatter-backward chunk exceed the LDS, so the
    # scatter backward takes its slot-centric form and pooling slices rows
    W("p4_L7_bf16", 1, 1, 8192, 64, "bf16", 4, 7, 2, 109, True),
    # large k against small coarse levels, pyramid form of the scatter backward (f32: with the
    # transposed copy; p = 3, d = 128: a partial last chunk and idle lane groups)
    W("pyr_f32", 1, 2, 2048, 64, "f32", 4, 4, 256, 110, False),
    W("pyr_p3_d128_bf16", 1, 2, 1350, 128, "bf16", 3, 4, 200, 111, True),
    # p = 5: the scatter backward takes its slot-centric form (f32: with the transposed copy)
    W("p5_f32", 1, 2, 1250, 64, "f32", 5, 3, 9, 115, False),
    # pyramid form of the scatter backward with level 1 as the top (p = 3, f32, a partial last
    # chunk) and with levels 3 and 4 from LDS at d = 128 over two batches
    W("tree_p3_L2_f32", 1, 2, 999, 64, "f32", 3, 2, 50, 116, False),
    W("tree_p2_L5_d128_bf16", 2, 2, 2048, 128, "bf16", 2, 5, 37, 117, True),
    # p^(L-1) = 16384: no pass of the pooling chunk fits whole rows, so it takes passes of
    # p^2 tokens over rows sliced to 8 elements
    W("p4_L8_bf16", 1, 1, 16384, 64, "bf16", 4, 8, 3, 114, True),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lh.load_library()


def _data(w):
    q, k, v = inputs.make_qkv(w)
    return q, k, v, inputs.make_dout(w)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_layer_parity_small(w):
    say(f"[parity] {w}")
    q, k, v, dout = _data(w)
    r = run_layer(w, q, k, v, dout)
    compare_selection(w, q, k, r)
    for b in range(w.B):
        for h in range(w.H):
            compare_head(w, q, k, v, dout, r, b, h)


def test_layer_parity_mid_bf16():
    """B=1 H=8 N=32768 d=128 bf16, p=4 L=4 k=256 (S=3584), every head."""
    w = inputs.WORKLOADS["mid_bf16"]
    say(f"[parity] {w}")
    q, k, v, dout = _data(w)
    r = run_layer(w, q, k, v, dout)
    compare_selection(w, q, k, r)
    for h in range(w.H):
        compare_head(w, q, k, v, dout, r, 0, h)


def test_exact_ties_select_lower_index():
    """Duplicated aligned blocks make equal scores at every level."""
    w = W("ties_bf16", 1, 2, 4096, 64, "bf16", 4, 4, 20, 109, True)
    q, k, v, dout = _data(w)
    for src, dst in [(0, 5), (0, 17), (0, 40), (9, 33)]:
        for t in (q, k, v):
            t[:, :, dst * 64:(dst + 1) * 64] = t[:, :, src * 64:(src + 1) * 64]
    q[:, :, 2000:2004] = q[:, :, 1000:1004]
    k[:, :, 2000:2004] = k[:, :, 1000:1004]
    r = run_layer(w, q, k, v, dout)
    compare_selection(w, q, k, r)
    compare_head(w, q, k, v, dout, r, 0, 1)


def test_all_scores_tied_across_wave_ranges():
    """Every Q and K row equal, so every score of every level ties: each level's
    top-K must take its lowest k indices.  N = 16384, p = 4, L = 3, k = 700:
    the top-K kernel splits level 2 (1024 entries) into 64-entry and level 1
    (4096) into 256-entry ranges, one per wave, so the run of taken ties
    crosses several range boundaries at both levels."""
    w = W("all_tied_bf16", 1, 1, 16384, 64, "bf16", 4, 3, 700, 112, False)
    q, k, v, dout = _data(w)
    q[:] = q[:, :, :1, :].clone()
    k[:] = k[:, :, :1, :].clone()
    r = run_layer(w, q, k, v, dout)
    compare_selection(w, q, k, r)
    compare_head(w, q, k, v, dout, r, 0, 0)


def test_layer_on_a_side_stream():
    """Every call enqueues on the stream it is given: the layer run on a side
    stream (default priority), synchronised through that stream alone, gives
    the default stream's results bit for bit."""
    w = W("stream_bf16", 1, 2, 2048, 64, "bf16", 4, 3, 40, 113, True)
    q, k, v, dout = _data(w)
    dev = torch.device("cuda")

    def run(stream):
        layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, torch.bfloat16)
        qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
        o, dq, dk, dv = (torch.empty_like(qd) for _ in range(4))
        torch.cuda.synchronize()
        layer.forward(qd, kd, vd, o, stream)
        layer.backward(dod, dq, dk, dv, stream)
        stream.synchronize()
        return [t.cpu() for t in (o, dq, dk, dv, layer.gidx, layer.gpos)]

    say("[stream] default vs side stream")
    ref = run(torch.cuda.current_stream())
    got = run(torch.cuda.Stream())
    for name, a, b in zip(("o", "dq", "dk", "dv", "gidx", "gpos"), ref, got):
        assert torch.equal(a, b), f"{name} differs on a side stream"


FROM_QK = [SMALL[0], SMALL[1], SMALL[3], SMALL[9], inputs.WORKLOADS["mid_bf16"]]


@pytest.mark.parametrize("w", FROM_QK, ids=lambda w: w.name)
def test_scores_from_q_and_k(w):
    """lh_score_topk given q and k and no pyramid buffer computes the token
    norms itself: the selection matches the oracle bit for bit and equals the
    one scored from the norms lh_pyramid leaves."""
    say(f"[score from q, k] {w}")
    q, k, v, dout = _data(w)
    dt = inputs.TORCH_DTYPE[w.dtype]
    layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, dt)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    o1, o2 = torch.empty_like(qd), torch.empty_like(qd)
    layer.forward(qd, kd, vd, o1, norms_from_pyramid=False)
    torch.cuda.synchronize()
    g1, p1 = layer.gidx.clone(), layer.gpos.clone()
    layer.forward(qd, kd, vd, o2)
    torch.cuda.synchronize()
    assert torch.equal(g1, layer.gidx) and torch.equal(p1, layer.gpos) and torch.equal(o1, o2)
    r = type("R", (), {})()
    r.gidx, r.gpos = g1, p1
    compare_selection(w, q, k, r)


@pytest.mark.parametrize("dtype,N,d", [("f32", 256, 64), ("bf16", 1000, 64), ("bf16", 777, 128)])
def test_dense_parity(dtype, N, d):
    """dense_causal_attn(+backward) vs the oracle at L = 1."""
    w = W("dense", 1, 2, N, d, dtype, 4, 1, 1, 11, dtype == "bf16")
    q, k, v, dout = _data(w)
    dt = inputs.TORCH_DTYPE[dtype]
    desc = lh.make_desc(1, 2, N, d, 4, 1, 1, dt)
    plan = lh.lh_make_plan(desc)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, dout))
    o = torch.empty_like(qd)
    lse = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(plan.dense_fwd_ws_bytes, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(plan.dense_bwd_ws_bytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    lh.dense_causal_attn(desc, qd, kd, vd, o, lse, ws)
    lh.dense_causal_attn_backward(desc, qd, kd, vd, lse, ws, dod, dq, dk, dv, wsb)
    torch.cuda.synchronize()
    for h in range(2):
        st = orc.head_forward(head_np(q, 0, h), head_np(k, 0, h), head_np(v, 0, h), 4, 1, 1, dtype)
        bw = orc.head_backward(st, head_np(dout, 0, h))
        check_close(to_np(o[0, h]), st["O"], dtype, f"dense O h{h}")
        assert np.allclose(to_np(lse[0, h]), st["lse"], rtol=1e-4, atol=1e-4)
        check_close(to_np(dq[0, h]), bw["dq"], dtype, f"dense dQ h{h}")
        check_close(to_np(dk[0, h]), bw["dk"], dtype, f"dense dK h{h}")
        check_close(to_np(dv[0, h]), bw["dv"], dtype, f"dense dV h{h}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_L1_layer_equals_dense_bitwise(dtype):
    """Switching selection off (L = 1) gives dense attention exactly: the
    layer and dense_causal_attn agree bit for bit, forward and backward."""
    w = W("L1", 1, 2, 640, 64, dtype, 4, 1, 1, 12, False)
    q, k, v, dout = _data(w)
    r = run_layer(w, q, k, v, dout)
    dt = inputs.TORCH_DTYPE[dtype]
    desc = lh.make_desc(1, 2, 640, 64, 4, 1, 1, dt)
    plan = lh.lh_make_plan(desc)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, dout))
    o = torch.empty_like(qd)
    lse = torch.empty((1, 2, 640), dtype=torch.float32, device="cuda")
    lh.dense_causal_attn(desc, qd, kd, vd, o, lse, torch.empty(plan.dense_fwd_ws_bytes, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(r.gidx[0, 0].cpu(), torch.arange(640, dtype=torch.int32))
    assert torch.equal(o, r.o)
    assert torch.equal(lse, r.lse)


def test_deterministic_two_runs():
    w = W("det", 1, 4, 8192, 64, "bf16", 4, 4, 64, 110, True)
    q, k, v, dout = _data(w)
    r = run_layer(w, q, k, v, dout, runs=2)
    for a, b in zip(r.runs[0], r.runs[1]):
        assert torch.equal(a, b)


def test_frozen_selection_causality_on_gpu():
    """With gidx/gpos fixed, changing every token after t leaves o[<= t]
    bit-identical (left-to-right causality through the HIP path)."""
    w = W("causal", 1, 2, 2048, 64, "bf16", 4, 3, 16, 111, True)
    q, k, v, dout = _data(w)
    r = run_layer(w, q, k, v, dout)
    t = 1234
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for x in (q2, k2, v2):
        x[:, :, t + 1:] = inputs.make_random(x[:, :, t + 1:].shape, 999, "bf16")
    layer = r.layer
    qd, kd, vd = (x.cuda() for x in (q2, k2, v2))
    o2 = torch.empty_like(qd)
    layer.forward(qd, kd, vd, o2, select=False)
    torch.cuda.synchronize()
    assert torch.equal(o2[:, :, :t + 1], r.o[:, :, :t + 1])
