"""The oracle's Q, K, V projections and their gradients against what the
mathematics fixes (no GPU): the definition by explicit loops on tiny inputs,
the head/feature order through structured weights, the adjoint identity, and
central finite differences."""
import numpy as np
import pytest

from oracle import lighthouse_oracle as orc
from tests import pins


def _data(B, N, Dm, H, d, seed):
    r = pins.rng(seed)
    x = r.standard_normal((B, N, Dm))
    w = r.standard_normal((3 * H * d, Dm)) / np.sqrt(Dm)
    g = [r.standard_normal((B, H, N, d)) for _ in range(3)]
    return x, w, g


def test_projection_matches_loops():
    """q[b,h,n,j] = sum_i x[b,n,i] w[h d + j, i] (K and V from the next H d rows)."""
    B, N, Dm, H, d = 2, 3, 5, 2, 3
    x, w, _ = _data(B, N, Dm, H, d, 1)
    q, k, v = orc.qkv_project(x, w, H, d, "f64")
    for which, t in enumerate((q, k, v)):
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    for j in range(d):
                        ref = sum(x[b, n, i] * w[which * H * d + h * d + j, i] for i in range(Dm))
                        assert abs(t[b, h, n, j] - ref) < 1e-12


def test_projection_head_order_with_selector_weights():
    """Weights that copy input features pick out the documented head layout."""
    B, N, H, d = 1, 4, 2, 3
    Dm = 3 * H * d
    x = pins.rng(2).standard_normal((B, N, Dm))
    w = np.eye(Dm)                        # feature f of the output = input feature f
    q, k, v = orc.qkv_project(x, w, H, d, "f64")
    for which, t in enumerate((q, k, v)):
        for h in range(H):
            assert np.array_equal(t[0, h], x[0, :, which * H * d + h * d: which * H * d + (h + 1) * d])


def test_backward_matches_loops():
    B, N, Dm, H, d = 2, 3, 4, 1, 2
    x, w, (dq, dk, dv) = _data(B, N, Dm, H, d, 3)
    dx, dw = orc.qkv_project_backward(x, w, dq, dk, dv, "f64")
    gs = (dq, dk, dv)
    for b in range(B):
        for n in range(N):
            for i in range(Dm):
                ref = sum(gs[c][b, h, n, j] * w[c * H * d + h * d + j, i]
                          for c in range(3) for h in range(H) for j in range(d))
                assert abs(dx[b, n, i] - ref) < 1e-12
    for c in range(3):
        for h in range(H):
            for j in range(d):
                for i in range(Dm):
                    ref = sum(gs[c][b, h, n, j] * x[b, n, i] for b in range(B) for n in range(N))
                    assert abs(dw[c * H * d + h * d + j, i] - ref) < 1e-12


def test_adjoint_identity():
    """<(q,k,v)(x,w), g> = <x, dx> = <w, dw> (the map is linear in x and in w)."""
    B, N, Dm, H, d = 2, 7, 6, 3, 4
    x, w, g = _data(B, N, Dm, H, d, 4)
    q, k, v = orc.qkv_project(x, w, H, d, "f64")
    dx, dw = orc.qkv_project_backward(x, w, *g, "f64")
    lhs = sum(float(np.sum(a * b)) for a, b in zip((q, k, v), g))
    assert lhs == pytest.approx(float(np.sum(x * dx)), rel=1e-12)
    assert lhs == pytest.approx(float(np.sum(w * dw)), rel=1e-12)


def test_finite_differences():
    B, N, Dm, H, d = 1, 3, 4, 2, 2
    x, w, g = _data(B, N, Dm, H, d, 5)

    def loss(xx, ww):
        return sum(float(np.sum(a * b)) for a, b in zip(orc.qkv_project(xx, ww, H, d, "f64"), g))

    dx, dw = orc.qkv_project_backward(x, w, *g, "f64")
    eps = 1e-6
    for idx in [(0, 0, 0), (0, 2, 3), (0, 1, 2)]:
        e = np.zeros_like(x)
        e[idx] = eps
        assert (loss(x + e, w) - loss(x - e, w)) / (2 * eps) == pytest.approx(dx[idx], rel=1e-6, abs=1e-9)
    for idx in [(0, 0), (5, 3), (11, 1)]:
        e = np.zeros_like(w)
        e[idx] = eps
        assert (loss(x, w + e) - loss(x, w - e)) / (2 * eps) == pytest.approx(dw[idx], rel=1e-6, abs=1e-9)


def test_rounding_is_applied_once():
    B, N, Dm, H, d = 1, 2, 8, 1, 8
    x, w, _ = _data(B, N, Dm, H, d, 6)
    q64 = orc.qkv_project(x, w, H, d, "f64")[0]
    q16 = orc.qkv_project(x, w, H, d, "bf16")[0]
    assert np.array_equal(q16, orc.round_to(q64, "bf16"))
