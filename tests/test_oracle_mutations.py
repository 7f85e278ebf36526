"""The pins have teeth: plant plausible mistakes in private copies of the
oracle (on the CPU) and check that some pin fails for each."""
import importlib.util
import os
import sys

import numpy as np
import pytest

from tests import pins
from tests.conftest import ROOT


_count = [0]


def fresh_oracle():
    _count[0] += 1
    name = f"oracle_mutant_{_count[0]}"
    path = os.path.join(ROOT, "oracle", "lighthouse_oracle.py")
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


def qkv(N=1024, d=16, seed=3):
    r = pins.rng(seed)
    return [r.standard_normal((N, d)).astype(np.float32).astype(np.float64) for _ in range(3)]


def expect_failure(fn, *args):
    with pytest.raises((AssertionError, IndexError, ValueError)):
        fn(*args)


def test_unshifted_scatter_breaks_causality():
    m = fresh_oracle()

    def scatter(Ot, gpos, plan):
        O = np.zeros((plan.N, Ot.shape[1]))
        t = np.arange(plan.N)
        for l in range(plan.L):
            g = gpos[plan.level_off[l] + t // plan.p ** l].astype(np.int64)   # no causal offset
            O[g >= 0] += Ot[g[g >= 0]]
        return O
    m.scatter = scatter
    q, k, v = qkv()
    expect_failure(pins.check_causality_signflip, m, q, k, v, m.make_plan(1024, 4, 4, 16), 500, "f32")


def test_high_index_tiebreak_fails_bruteforce():
    m = fresh_oracle()
    m.top_k_level = lambda sig, k: np.sort(np.argsort(-sig[::-1].astype(np.float64), kind="stable")[:k] * -1 + len(sig) - 1)
    expect_failure(pins.check_topk_bruteforce, m)


def test_coarse_first_order_fails():
    m = fresh_oracle()
    orig = m.gather_order

    def gather_order(sel, plan):
        p = plan.p
        ends, lev, idx = [], [], []
        for l, ids in enumerate(sel):
            ids = np.asarray(ids, dtype=np.int64)
            ends.append((ids + 1) * p ** l - 1); lev.append(np.full(ids.shape, -l)); idx.append(ids)
        ends, lev, idx = np.concatenate(ends), np.concatenate(lev), np.concatenate(idx)
        order = np.lexsort((lev, ends))                   # coarser level first at equal end
        flat = np.asarray(plan.level_off)[-lev] + idx
        gidx = flat[order].astype(np.int32)
        gpos = np.full(plan.M_total, -1, dtype=np.int32)
        gpos[gidx] = np.arange(gidx.shape[0], dtype=np.int32)
        return gidx, gpos
    m.gather_order = gather_order
    assert orig is not gather_order
    q, k, _ = qkv(N=1024)
    expect_failure(pins.check_gather_order, m, q.astype(np.float32), k.astype(np.float32), m.make_plan(1024, 4, 4, 16))
    expect_failure(pins.check_selection_golden, m)


def test_missing_pool_scale_fails_fd():
    m = fresh_oracle()

    def gpb(dXt, gpos, plan):
        dX = np.zeros((plan.N, dXt.shape[1]))
        t = np.arange(plan.N)
        for l in range(plan.L):
            g = gpos[plan.level_off[l] + t // plan.p ** l].astype(np.int64)
            dX[g >= 0] += dXt[g[g >= 0]]                    # forgot 1/p^l
        return dX
    m.gather_pool_backward = gpb
    expect_failure(pins.check_finite_differences, m, 64, 8, 2, 3, 4, 1)


def test_product_score_fails_golden():
    m = fresh_oracle()
    m.token_scores = lambda q, k: (np.sqrt(m._sumsq_f32(q)) * np.sqrt(m._sumsq_f32(k))).astype(np.float32)
    from tests.test_oracle import test_scores_golden_pythagorean
    import tests.test_oracle as t
    saved = t.orc
    t.orc = m
    try:
        with pytest.raises(AssertionError):
            test_scores_golden_pythagorean()
    finally:
        t.orc = saved


def test_missing_mask_fails_dense():
    m = fresh_oracle()

    def attn(Qt, Kt, Vt, scale, row_block=2048):
        Z = scale * Qt @ Kt.T
        mx = Z.max(axis=1, keepdims=True)
        P = np.exp(Z - mx)
        l = P.sum(axis=1, keepdims=True)
        return (P @ Vt) / l, (mx + np.log(l))[:, 0]
    m.attention_forward = attn
    expect_failure(pins.check_dense_vs_sdpa, m)


def test_unshifted_scatter_backward_fails_fd():
    m = fresh_oracle()
    m.scatter_ranges = lambda l, i, p, N: (i * p ** l, min(N - 1, (i + 1) * p ** l - 1))
    expect_failure(pins.check_finite_differences, m, 64, 8, 2, 3, 4, 1)


def test_strided_norm_order_fails_golden():
    m = fresh_oracle()

    def sumsq(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.zeros((x.shape[0], 8), dtype=np.float32)
        for j in range(x.shape[1]):                     # element j into partial sum j mod 8
            a[:, j % 8] = a[:, j % 8] + x[:, j] * x[:, j]
        t = a[:, 0:4] + a[:, 4:8]
        u = t[:, 0:2] + t[:, 2:4]
        return u[:, 0] + u[:, 1]
    m._sumsq_f32 = sumsq
    expect_failure(pins.check_norm_order_golden, m)


def test_sequential_norm_order_fails_golden():
    m = fresh_oracle()

    def sumsq(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.zeros(x.shape[0], dtype=np.float32)
        for j in range(x.shape[1]):
            a = a + x[:, j] * x[:, j]
        return a
    m._sumsq_f32 = sumsq
    expect_failure(pins.check_norm_order_golden, m)


def test_overwritten_row_group_gradients_fail():
    m = fresh_oracle()

    def attention_backward(Qt, Kt, Vt, Ot, dOt, lse, scale, row_block=2048):
        S, d = Qt.shape
        dQ, dK, dV = np.zeros_like(Qt), np.zeros_like(Kt), np.zeros_like(Vt)
        D = np.sum(dOt * Ot, axis=1)
        for r0 in range(0, S, row_block):
            r1 = min(S, r0 + row_block)
            Z = scale * (Qt[r0:r1] @ Kt[:r1].T)
            Z[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
            P = np.exp(Z - lse[r0:r1, None])
            dS = P * (dOt[r0:r1] @ Vt[:r1].T - D[r0:r1, None])
            dQ[r0:r1] = scale * (dS @ Kt[:r1])
            dK[:r1] = scale * (dS.T @ Qt[r0:r1])         # overwrites earlier groups' terms
            dV[:r1] = P.T @ dOt[r0:r1]
        return dQ, dK, dV
    m.attention_backward = attention_backward
    expect_failure(pins.check_row_blocks, m)
    expect_failure(pins.check_dense_vs_sdpa, m, 100, 16, 5, 16)
    expect_failure(pins.check_finite_differences, m, 64, 8, 2, 3, 4, 77, 24, 1e-6, 8)
