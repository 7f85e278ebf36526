"""Checks that pin the oracle to facts outside itself.

Each function raises AssertionError when the oracle (module ``orc``) breaks
a property fixed by the pages or by mathematics.  They take the oracle
module as an argument so that tests/test_oracle_mutations.py can run the
same checks on deliberately broken copies and show that they fail.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

from tests.conftest import read_golden


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- selection
def check_topk_bruteforce(orc, trials=300, seed=7):
    """Top-k under (score desc, index asc) equals the unique k-subset whose
    every member beats every non-member, found by enumerating all subsets."""
    r = rng(seed)
    for _ in range(trials):
        M = int(r.integers(1, 8))
        k = int(r.integers(1, M + 1))
        sig = r.choice(np.array([0.0, 1.0, 1.5, 2.0], dtype=np.float32), size=M)
        got = list(orc.top_k_level(sig, k))
        wins = []
        for sub in itertools.combinations(range(M), k):
            rest = [j for j in range(M) if j not in sub]
            beats = all((sig[a] > sig[b]) or (sig[a] == sig[b] and a < b) for a in sub for b in rest)
            if beats:
                wins.append(list(sub))
        assert len(wins) == 1
        assert got == wins[0], (sig, k, got, wins)


def check_selection_golden(orc):
    rows = {r[0]: r[1:] for r in read_golden("selection_tiny.txt")}
    s = np.array([float(x) for x in rows["scores"]], dtype=np.float32)
    plan = orc.make_plan(16, 2, 3, 1)
    assert plan.S == 8
    sel = orc.selected_sets(s, plan)
    gidx, gpos = orc.gather_order(sel, plan)
    assert [int(x) for x in gidx] == [int(x) for x in rows["gidx"]]
    # fan-in counted from the ranges of the selected entries
    f = np.zeros(16, dtype=int)
    for g in range(plan.S):
        l, i = orc.entry_of(int(gidx[g]), plan)
        lo, hi = orc.scatter_ranges(l, i, 2, 16)
        f[lo:hi + 1] += 1
    assert list(f) == [int(x) for x in rows["fanin"]]
    # and through the oracle's scatter with constant rows
    Ot = np.ones((plan.S, 1))
    assert list(orc.scatter(Ot, gpos, plan)[:, 0].astype(int)) == [int(x) for x in rows["fanin"]]


def check_scatter_ranges_golden(orc):
    for p, l, i, lo, hi in read_golden("scatter_ranges.txt"):
        assert orc.scatter_ranges(int(l), int(i), int(p), 10 ** 6) == (int(lo), int(hi))


def check_gather_order(orc, q, k, plan):
    """Sorted by (span end, level); every selected entry once; gpos inverts
    gidx; a child precedes its selected parent; slot positions equal the
    closed-form count of entries that come before each one."""
    gidx, gpos = orc.select(q, k, plan)
    p, L = plan.p, plan.L
    assert gidx.shape == (plan.S,)
    assert len(set(gidx.tolist())) == plan.S
    assert np.all(gpos[gidx] == np.arange(plan.S))
    assert int((gpos >= 0).sum()) == plan.S
    keys = []
    for f in gidx:
        l, i = orc.entry_of(int(f), plan)
        keys.append(((i + 1) * p ** l - 1, l))
    assert keys == sorted(keys)
    sel = [set() for _ in range(L)]
    for f in gidx:
        l, i = orc.entry_of(int(f), plan)
        sel[l].add(i)
    # counts: coarsest whole, p * k_l below
    assert len(sel[L - 1]) == plan.M[L - 1]
    for l in range(1, L):
        assert len(sel[l - 1]) == p * plan.k_eff[l]
    # children before parent
    for l in range(1, L):
        for i in sel[l]:
            for c in range(p):
                if p * i + c in sel[l - 1]:
                    assert gpos[plan.level_off[l - 1] + p * i + c] < gpos[plan.level_off[l] + i]
    # closed-form position: entries of every level whose (end, level) key is smaller
    pref = []
    for l in range(L):
        bits = np.zeros(plan.M[l] + 1, dtype=np.int64)
        for i in sel[l]:
            bits[i + 1] = 1
        pref.append(np.cumsum(bits))           # pref[l][x] = # selected among [0, x)
    for l in range(L):
        for i in sel[l]:
            pos = pref[l][i]
            for l2 in range(L):
                if l2 < l:
                    pos += pref[l2][min(plan.M[l2], (i + 1) * p ** (l - l2))]
                elif l2 > l:
                    pos += pref[l2][-(-(i + 1) // p ** (l2 - l)) - 1]
            assert gpos[plan.level_off[l] + i] == pos


def check_norm_order_golden(orc):
    """Reading R2's summation order against hand-worked float32 sums of rows
    whose result differs under other plausible orders (strided, sequential,
    adjacent-pair tree); see tests/golden/norm_order.txt."""
    for name, ones, r2, strided, seq, norm in read_golden("norm_order.txt"):
        x = np.zeros((1, 64), dtype=np.float32)
        x[0, 0] = 4096.0
        for j in ones.split(","):
            x[0, int(j)] = 1.0
        got = orc._sumsq_f32(x)
        assert got.dtype == np.float32
        assert float(got[0]) == float(r2), (name, float(got[0]), r2)
        assert float(r2) != float(strided) or float(r2) != float(seq)
        assert float(orc.token_norms(x)[0]) == float(norm), (name, float(orc.token_norms(x)[0]), norm)


# ---------------------------------------------------------------- scatter / causality
def check_constant_v_fanin(orc, q, k, plan):
    """V rows all equal to c: every sub-sequence output equals c, so O_t is c
    times the number of selected entries whose range R(l, i) holds t; that
    count is at most L and level l covers nothing before t = p^l - 1."""
    N, d = q.shape
    c = np.linspace(-1.0, 2.0, d)
    v = np.tile(c, (N, 1))
    st = orc.head_forward(q, k, v, plan.p, plan.L, plan.k, "f64")
    f = np.zeros(N, dtype=int)
    first = {}
    for g in range(plan.S):
        l, i = orc.entry_of(int(st["gidx"][g]), plan)
        lo, hi = orc.scatter_ranges(l, i, plan.p, N)
        f[lo:hi + 1] += 1
        first[l] = min(first.get(l, N), lo)
    assert f.max() <= plan.L
    for l, t0 in first.items():
        assert t0 >= plan.p ** l - 1
    np.testing.assert_allclose(st["O"], f[:, None] * c[None, :], rtol=0, atol=1e-12)
    return f


def check_causality_signflip(orc, q, k, v, plan, t, dtype, seed=3):
    """Global top-K makes selection depend on the whole sequence, so the
    test keeps every score bit-identical: it flips signs of q/k coordinates
    after t (squares unchanged) and replaces v after t.  Outputs at
    positions <= t must not change by a single bit (left-to-right causality,
    hotpaper.ai abstract; gist.science Contributions)."""
    r = rng(seed)
    st0 = orc.head_forward(q, k, v, plan.p, plan.L, plan.k, dtype)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    flip_q = r.choice([-1.0, 1.0], size=q2[t + 1:].shape)
    flip_k = r.choice([-1.0, 1.0], size=k2[t + 1:].shape)
    q2[t + 1:] *= flip_q
    k2[t + 1:] *= flip_k
    v2[t + 1:] = r.standard_normal(v2[t + 1:].shape).astype(np.float32)
    if dtype == "bf16":
        v2 = orc.round_to(v2, "bf16")
    st1 = orc.head_forward(q2, k2, v2, plan.p, plan.L, plan.k, dtype)
    assert np.array_equal(st0["gidx"], st1["gidx"])
    assert np.array_equal(st0["O"][:t + 1], st1["O"][:t + 1])
    return st0, st1


def check_causality_frozen(orc, q, k, v, plan, t, seed=4):
    r = rng(seed)
    st0 = orc.head_forward(q, k, v, plan.p, plan.L, plan.k, "f64")
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[t + 1:] = r.standard_normal(a[t + 1:].shape)
    st1 = orc.head_forward(q2, k2, v2, plan.p, plan.L, plan.k, "f64",
                           selection=(st0["gidx"], st0["gpos"]))
    assert np.array_equal(st0["O"][:t + 1], st1["O"][:t + 1])


# ---------------------------------------------------------------- attention
def check_dense_vs_sdpa(orc, N=64, d=16, seed=5, row_block=None):
    """L = 1 is dense causal attention (skill card, selection-attention
    decoupling): compare with torch's scaled_dot_product_attention in
    float64, forward and gradients.  A row_block below N runs the oracle's
    attention in several row groups."""
    r = rng(seed)
    q, k, v, g = (r.standard_normal((N, d)) for _ in range(4))
    st = orc.head_forward(q, k, v, 4, 1, 1, "f64", row_block=row_block)
    assert st["plan"].S == N and np.array_equal(st["gidx"], np.arange(N))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                         is_causal=True)[0, 0]
    (o * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(st["O"], o.detach().numpy(), rtol=1e-12, atol=1e-12)
    bw = orc.head_backward(st, g)
    np.testing.assert_allclose(bw["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bw["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bw["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_finite_differences(orc, N, d, p, L, kk, seed, ncoord=24, h=1e-6, row_block=None):
    """Central differences of sum(O * G) with the selection frozen (the
    selection is gradient-free: skill card, gradient flow)."""
    r = rng(seed)
    q, k, v = (r.standard_normal((N, d)) * np.exp(0.5 * r.standard_normal((N, 1))) for _ in range(3))
    G = r.standard_normal((N, d))
    st = orc.head_forward(q, k, v, p, L, kk, "f64", row_block=row_block)
    sel = (st["gidx"], st["gpos"])
    bw = orc.head_backward(st, G)
    grads = {"q": bw["dq"], "k": bw["dk"], "v": bw["dv"]}

    def loss(qq, kk_, vv):
        return float(np.sum(orc.head_forward(qq, kk_, vv, p, L, kk, "f64", selection=sel,
                                             row_block=row_block)["O"] * G))

    for name in ("q", "k", "v"):
        gmax = np.abs(grads[name]).max()
        for _ in range(ncoord):
            t, j = int(r.integers(N)), int(r.integers(d))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][t, j] += h
            lp = loss(args["q"], args["k"], args["v"])
            args[name][t, j] -= 2 * h
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[name][t, j]) <= 1e-6 * max(1.0, gmax), (name, t, j, fd, grads[name][t, j])


def check_row_blocks(orc, S=100, d=16, seed=6, row_block=16):
    """The attention's row groups bound memory only: groups of row_block < S
    rows give the same output, log-sum-exp and gradients as one group."""
    r = rng(seed)
    Qt, Kt, Vt, dOt = (r.standard_normal((S, d)) * np.exp(0.5 * r.standard_normal((S, 1))) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    O1, lse1 = orc.attention_forward(Qt, Kt, Vt, scale, S)
    O2, lse2 = orc.attention_forward(Qt, Kt, Vt, scale, row_block)
    np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse1, rtol=1e-12, atol=1e-12)
    g1 = orc.attention_backward(Qt, Kt, Vt, O1, dOt, lse1, scale, S)
    g2 = orc.attention_backward(Qt, Kt, Vt, O1, dOt, lse1, scale, row_block)
    for a, b in zip(g2, g1):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(b).max())
