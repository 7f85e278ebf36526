"""Q, K, V projections and their gradients: the HIP library (lh_qkv_forward,
lh_qkv_backward, through the C ABI) against the oracle on seeded inputs.
bf16 outputs (q, k, v, dx) within 2e-2*max(1,|ref|) element-wise; dw (f32,
summed over every token) within 1e-4 of its largest magnitude.  Shapes span
single partial 256 x 256 tiles, several tiles with ragged row and column tails,
a batch boundary inside a row tile, dW k-splits of which some are empty, d = 64
and 128, and the headline layer (B=1 N=98304 Dm=1024 H=16 d=64) on sampled
rows and columns."""
import numpy as np
import pytest
import torch

from long_context_pretraining_amd import inputs
from long_context_pretraining_amd import lighthouse as lh
from oracle import lighthouse_oracle as orc
from tests.gpu_support import check_close, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lh.load_library()


def _run(B, N, Dm, H, d, seed, runs=1):
    x, w, (gq, gk, gv) = inputs.make_proj_inputs(B, N, Dm, H, d, seed)
    desc = lh.make_proj_desc(B, N, Dm, H, d)
    dev = torch.device("cuda")
    xd, wd, gqd, gkd, gvd = (t.to(dev) for t in (x, w, gq, gk, gv))
    ws = torch.empty(lh.lh_qkv_plan(desc), dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(runs):
        q, k, v = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
        dx = torch.empty((B, N, Dm), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((3 * H * d, Dm), dtype=torch.float32, device=dev)
        lh.lh_qkv_forward(desc, xd, wd, q, k, v)
        lh.lh_qkv_backward(desc, xd, wd, gqd, gkd, gvd, dx, dw, ws)
        torch.cuda.synchronize()
        outs.append((q, k, v, dx, dw))
    return (x, w, gq, gk, gv), outs


def _compare_full(data, out, H, d, tag):
    x, w, gq, gk, gv = (to_np(t) for t in data)
    q, k, v, dx, dw = out
    rq, rk, rv = orc.qkv_project(x, w, H, d, "bf16")
    rdx, rdw = orc.qkv_project_backward(x, w, gq, gk, gv, "bf16")
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("dx", dx, rdx)):
        check_close(to_np(got), ref, "bf16", f"{tag} {name}")
    check_close(to_np(dw), rdw, "f32", f"{tag} dw")


@pytest.mark.parametrize("B,N,Dm,H,d", [
    (2, 128, 128, 2, 64),    # exact tiles, two batches
    (1, 192, 192, 3, 64),    # ragged row and column tiles (192 = 1.5 tiles), 3 k-blocks
    (2, 320, 256, 1, 128),   # d = 128: a head spans two k-blocks
    (1, 64, 64, 1, 64),      # a single partial tile everywhere
    (1, 576, 320, 2, 64),    # 2.25 x 1.5 tiles forward, 1.25-tile dX columns, 9 one-block dW splits
    (2, 1088, 512, 4, 64),   # batch boundary inside a row tile; 16 dW splits of 3 k-blocks, the last ones empty
    (1, 640, 384, 2, 128),   # d = 128 over several tiles
])
def test_projection_parity_small(B, N, Dm, H, d):
    tag = f"proj B{B} N{N} Dm{Dm} H{H} d{d}"
    say(f"[proj] {tag}")
    data, outs = _run(B, N, Dm, H, d, seed=70 + N, runs=2)
    _compare_full(data, outs[0], H, d, tag)
    for a, b in zip(outs[0], outs[1]):   # deterministic: no atomics feed any output
        assert torch.equal(a, b), f"{tag}: two runs differ"


def test_projection_parity_headline_sampled():
    """B=1 N=98304 Dm=1024 H=16 d=64: q, k, v and dx on 96 sampled tokens, dw
    on 48 sampled input columns (every output row, all 98304 tokens summed)."""
    B, N, Dm, H, d = 1, 98304, 1024, 16, 64
    say(f"[proj] headline B{B} N{N} Dm{Dm} H{H} d{d}")
    data, outs = _run(B, N, Dm, H, d, seed=77)
    x, w, gq, gk, gv = data
    q, k, v, dx, dw = outs[0]
    rng = np.random.Generator(np.random.PCG64(78))
    toks = np.sort(np.concatenate([[0, 1, N - 1], rng.choice(N, 93, replace=False)]))
    cols = np.sort(np.concatenate([[0, Dm - 1], rng.choice(Dm, 46, replace=False)]))
    xs = to_np(x[:, toks])                                    # [1, T, Dm]
    rq, rk, rv = orc.qkv_project(xs, to_np(w), H, d, "bf16")  # [1, H, T, d]
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_close(to_np(got[:, :, toks]), ref, "bf16", f"headline {name}")
    gs = [to_np(t[:, :, toks]) for t in (gq, gk, gv)]
    rdx, _ = orc.qkv_project_backward(xs, to_np(w), *gs, "bf16")
    check_close(to_np(dx[:, toks]), rdx, "bf16", "headline dx")
    G = orc.qkv_features(*(to_np(t) for t in (gq, gk, gv)))   # [1, N, 3Hd]
    rdw = G.reshape(N, -1).T @ to_np(x)[0][:, cols]
    check_close(to_np(dw[:, cols]), rdw, "f32", "headline dw")
