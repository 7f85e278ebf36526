"""The CPU oracle against what the pages and mathematics fix (no GPU)."""
import math

import numpy as np
import pytest

from oracle import lighthouse_oracle as orc
from tests import pins
from tests.conftest import read_golden


def rand_qkv(N, d, seed, dtype="f32", lognormal=True):
    r = pins.rng(seed)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    if lognormal:
        m = np.exp(0.5 * r.standard_normal((N, 1)))
        q, k, v = q * m, k * m, v * m
    if dtype in ("f32", "bf16"):
        q, k, v = (orc.round_to(a, dtype) for a in (q, k, v))
    return q, k, v


# ------------------------------------------------------------------ sizes
@pytest.mark.parametrize("N,p,L", [(4096, 4, 3), (98304, 4, 4), (524288, 4, 6), (64, 2, 3), (81, 3, 5), (256, 4, 1)])
def test_entry_count_bound(N, p, L):
    plan = orc.make_plan(N, p, L, 1)
    assert plan.M_total <= N * p / (p - 1)          # skill card, Stage 1
    assert plan.M == [N // p ** l for l in range(L)]


def test_s_formula_golden():
    for N, p, L, k, Sf, Sa in read_golden("s_formula.txt"):
        plan = orc.make_plan(int(N), int(p), int(L), int(k))
        assert plan.S_formula == int(Sf)
        assert plan.S == int(Sa)


def test_plan_rejects_bad_shapes():
    for args in [(100, 4, 3, 1), (64, 1, 2, 1), (64, 2, 0, 1), (64, 2, 2, 0)]:
        with pytest.raises(ValueError):
            orc.make_plan(*args)


# ------------------------------------------------------------------ rounding
def test_bf16_rounding_golden():
    for expr, hexv in read_golden("bf16_rounding.txt"):
        val = eval(expr, {"__builtins__": {}})
        got = orc.round_to(np.array([val]), "bf16").astype(np.float32).view(np.uint32)[0] >> 16
        assert got == int(hexv, 16), (expr, hex(got), hexv)


def test_round_to_is_identity_on_representable():
    r = pins.rng(1)
    x = orc.round_to(r.standard_normal(10000) * 100, "bf16")
    assert np.array_equal(orc.round_to(x, "bf16"), x)
    y = r.standard_normal(10000).astype(np.float32).astype(np.float64)
    assert np.array_equal(orc.round_to(y, "f32"), y)


# ------------------------------------------------------------------ pyramid
def test_pyramid_golden():
    rows = {r[0]: [float(x) for x in r[1:]] for r in read_golden("pyramid_tiny.txt")}
    x = np.array(rows["x"])[:, None]
    lv = orc.pyramid(x, 2, 3, "f64")
    assert lv[1][:, 0].tolist() == rows["level1"]
    assert lv[2][:, 0].tolist() == rows["level2"]


@pytest.mark.parametrize("p,L", [(2, 4), (4, 3), (3, 3)])
def test_pyramid_is_recursive_mean(p, L):
    """Each level summarises p consecutive entries of the level below
    (gist.science 2A) -- a characterisation different from the direct span
    mean the oracle computes."""
    N, d = p ** (L - 1) * 5, 6
    x = pins.rng(2).standard_normal((N, d))
    lv = orc.pyramid(x, p, L, "f64")
    for l in range(1, L):
        rec = lv[l - 1].reshape(-1, p, d).sum(axis=1) / p
        np.testing.assert_allclose(lv[l], rec, rtol=1e-14, atol=1e-14)


def test_pyramid_dyadic_exact_and_constant():
    r = pins.rng(3)
    x = r.integers(-8, 9, size=(256, 8)).astype(np.float64)
    lv = orc.pyramid(x, 4, 4, "bf16")
    for l in range(1, 4):
        n = 4 ** l
        # sums of <= 64 integers in [-8, 8] divided by a power of two: exact in bf16? only when
        # the mean fits 8 significant bits -- check exactness where it does
        exact = x.reshape(-1, n, 8).sum(axis=1) / n
        fits = orc.round_to(exact, "bf16") == exact
        assert np.array_equal(lv[l][fits], exact[fits])
    c = np.full((64, 4), 1.25)
    for a in orc.pyramid(c, 4, 3, "bf16"):
        assert np.all(a == 1.25)


# ------------------------------------------------------------------ scores
def test_scores_golden_pythagorean():
    q = np.zeros((3, 8), dtype=np.float32)
    k = np.zeros((3, 8), dtype=np.float32)
    q[0, :2] = [3, 4]; k[0, 6:] = [12, 5]          # 5 + 13
    q[1, :] = 0.5; k[1, :] = 1.0                  # 2*sqrt(8)*.. : |q| = sqrt(2), |k| = sqrt(8)
    q[2, 3] = -7.0                                # 7 + 0
    s = orc.token_scores(q, k)
    assert s[0] == 18.0
    assert s[1] == np.float32(np.sqrt(np.float32(2.0)) + np.sqrt(np.float32(8.0)))
    assert s[2] == 7.0
    q64 = np.full((1, 64), 0.5, dtype=np.float32); k64 = np.ones((1, 64), dtype=np.float32)
    assert orc.token_scores(q64, k64)[0] == 12.0


def test_norm_order_golden():
    pins.check_norm_order_golden(orc)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_scores_close_to_fp64_norms(d):
    r = pins.rng(d)
    q = (r.standard_normal((4000, d)) * np.exp(r.standard_normal((4000, 1)))).astype(np.float32)
    k = (r.standard_normal((4000, d)) * np.exp(r.standard_normal((4000, 1)))).astype(np.float32)
    s = orc.token_scores(q, k).astype(np.float64)
    ref = np.linalg.norm(q.astype(np.float64), axis=1) + np.linalg.norm(k.astype(np.float64), axis=1)
    assert np.all(np.abs(s - ref) <= 4 * 2.0 ** -24 * ref)


def test_scores_sign_invariant_bitwise():
    r = pins.rng(9)
    q = r.standard_normal((500, 64)).astype(np.float32)
    k = r.standard_normal((500, 64)).astype(np.float32)
    f = r.choice(np.array([-1, 1], dtype=np.float32), size=q.shape)
    assert np.array_equal(orc.token_scores(q, k), orc.token_scores(q * f, k * f[::-1]))


def test_level_scores_are_span_max_and_recursive():
    s = pins.rng(4).random(4 ** 4).astype(np.float32)
    sig = orc.level_scores(s, 4, 4)
    for l in range(1, 4):
        n = 4 ** l
        for j in range(sig[l].shape[0]):
            assert sig[l][j] == max(s[j * n:(j + 1) * n])
        assert np.array_equal(sig[l], sig[l - 1].reshape(-1, 4).max(axis=1))


# ------------------------------------------------------------------ top-K and gather
def test_topk_bruteforce():
    pins.check_topk_bruteforce(orc)


def test_topk_closed_forms():
    M, k = 50, 7
    assert orc.top_k_level(np.ones(M, np.float32), k).tolist() == list(range(k))
    assert orc.top_k_level(np.arange(M, 0, -1).astype(np.float32), k).tolist() == list(range(k))
    assert orc.top_k_level(np.arange(M).astype(np.float32), k).tolist() == list(range(M - k, M))
    assert orc.top_k_level(np.arange(M).astype(np.float32), M).tolist() == list(range(M))


def test_selection_golden():
    pins.check_selection_golden(orc)


def test_scatter_ranges_golden():
    pins.check_scatter_ranges_golden(orc)


@pytest.mark.parametrize("N,p,L,k", [(4096, 4, 3, 64), (256, 2, 5, 3), (243, 3, 3, 5), (1024, 4, 4, 100), (64, 4, 1, 1)])
def test_gather_order(N, p, L, k):
    q, kk, _ = rand_qkv(N, 16, N + k)
    pins.check_gather_order(orc, q.astype(np.float32), kk.astype(np.float32), orc.make_plan(N, p, L, k))


def test_gather_order_with_exact_ties():
    N, d = 1024, 16
    q, k, _ = rand_qkv(N, d, 77)
    q[256:320] = q[0:64]; k[256:320] = k[0:64]      # duplicated aligned blocks: ties at every level
    q[640:704] = q[0:64]; k[640:704] = k[0:64]
    pins.check_gather_order(orc, q.astype(np.float32), k.astype(np.float32), orc.make_plan(N, 4, 4, 5))


# ------------------------------------------------------------------ attention and scatter
def test_dense_equals_sdpa():
    pins.check_dense_vs_sdpa(orc)


def test_dense_equals_sdpa_in_row_groups():
    # S = 100 rows in groups of 16: the last group is ragged (4 rows)
    pins.check_dense_vs_sdpa(orc, N=100, row_block=16)


def test_attention_row_groups_agree():
    pins.check_row_blocks(orc)


def test_zero_queries_give_running_mean():
    q, k, v = rand_qkv(256, 8, 12, "f64")
    q[:] = 0.0
    st = orc.head_forward(q, k, v, 4, 3, 4, "f64")
    cm = np.cumsum(st["Vt"], axis=0) / np.arange(1, st["plan"].S + 1)[:, None]
    np.testing.assert_allclose(st["Ot"], cm, rtol=1e-12, atol=1e-12)


def test_first_row_copies_value():
    q, k, v = rand_qkv(512, 16, 13, "bf16")
    st = orc.head_forward(q, k, v, 4, 3, 8, "bf16")
    assert np.array_equal(st["Ot"][0], st["Vt"][0])


@pytest.mark.parametrize("N,p,L,k", [(1024, 4, 4, 20), (256, 2, 4, 8), (4096, 4, 3, 64)])
def test_constant_values_fanin(N, p, L, k):
    q, kk, _ = rand_qkv(N, 8, 21)
    f = pins.check_constant_v_fanin(orc, q, kk, orc.make_plan(N, p, L, k))
    assert f.max() == L or N < p ** L      # fan-in reaches L on these sizes


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("t", [0, 200, 777, 1022])
def test_causality_signflip(dtype, t):
    q, k, v = rand_qkv(1024, 16, 31, dtype)
    pins.check_causality_signflip(orc, q, k, v, orc.make_plan(1024, 4, 4, 16), t, dtype)


@pytest.mark.parametrize("t", [5, 300, 1000])
def test_causality_frozen_selection(t):
    q, k, v = rand_qkv(1024, 16, 32, "f64")
    pins.check_causality_frozen(orc, q, k, v, orc.make_plan(1024, 4, 4, 16), t)


def test_linear_in_values():
    q, k, v1 = rand_qkv(256, 8, 41, "f64")
    _, _, v2 = rand_qkv(256, 8, 42, "f64")
    plan = orc.make_plan(256, 2, 4, 6)
    st1 = orc.head_forward(q, k, v1, 2, 4, 6, "f64")
    sel = (st1["gidx"], st1["gpos"])
    st2 = orc.head_forward(q, k, v2, 2, 4, 6, "f64", selection=sel)
    st3 = orc.head_forward(q, k, 2 * v1 - v2, 2, 4, 6, "f64", selection=sel)
    np.testing.assert_allclose(st3["O"], 2 * st1["O"] - st2["O"], atol=1e-12)
    assert plan.S == st1["plan"].S


# ------------------------------------------------------------------ backward
@pytest.mark.parametrize("p,L,kk,seed", [(2, 3, 4, 1), (4, 3, 2, 2)])
def test_finite_differences(p, L, kk, seed):
    for h in range(2):
        pins.check_finite_differences(orc, 64, 8, p, L, kk, seed * 10 + h)


def test_finite_differences_in_row_groups():
    # S = 32 sub-sequence rows in groups of 8 (gradients summed over four groups)
    pins.check_finite_differences(orc, 64, 8, 2, 3, 4, 77, row_block=8)


def test_rejects_non_finite():
    q, k, v = rand_qkv(64, 8, 5, "f64")
    q[3, 2] = np.nan
    with pytest.raises(ValueError):
        orc.head_forward(q, k, v, 2, 3, 4, "f64")
