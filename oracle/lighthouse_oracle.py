"""Lighthouse Attention: plain, slow CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path never calls it; the
HIP library shares no code, header, table or helper with it.

What it computes follows the pages on arXiv 2605.06554 ("Long Context
Pre-Training with Lighthouse Attention"), cited by page and section:

* [SK]  skillsmp.com ... lighthouse-attention (the skill card): sections
        "Stage 1 pyramid construction", "Stage 2 scoring and selection",
        "Stage 3 dense sub-sequence attention", "Stage 4 scatter-back",
        "gradient flow", "complexity", "selection-attention decoupling".
* [GE]  gist.science/paper/2605.06554, technical summary, section 2
        ("Methodology"), parts A-C.
* [GI]  gist.science/it/paper/2605.06554 (Italian summary), section 2 A-C.

Precision.  Everything is float64 except the token scores, which are float32
in one fixed order so that the integer decisions built on them (the selected
sets and the gather order) are reproducible bit for bit by any
implementation that follows the same order.  Where a tensor of the layer's
dtype is stored and reused (pyramid levels >= 1, the gradient of the
sub-sequence output, which feeds matrix products, and the final outputs and
gradients) the oracle rounds to that dtype once, with round-to-nearest-even,
exactly as a bf16/fp32 implementation stores it; the sub-sequence output
itself is an intermediate and stays unrounded.  The "f64" dtype turns every
rounding off (used by finite differences).

Readings of points the pages leave open (each is used below):
  R1 score of an entry = ||q||_2 + ||k||_2 (the pages name both norms but not
     how they combine);
  R2 squared norm summed in float32 in a fixed order: 8 contiguous chunks of
     d/8 elements, each summed left to right (product rounded, then added),
     then chunk sums combined as (a_r + a_{r+4}), then (t_r + t_{r+2}), then
     (u_0 + u_1); then a correctly rounded float32 sqrt;
  R4 per level l = 1..L-1 the top-k_l entries of that level (k_l = min(k, M_l))
     are expanded into their p children at level l-1; the coarsest level is
     kept whole; ties are broken toward the lower index;
  R5 gathered order = ascending (last token of the entry's span, level), so a
     child comes before its parent at equal span end;
  R6 softmax scale 1/sqrt(d) unless given; the causal mask includes the
     diagonal;
  R7 scatter ranges clipped at N-1, uncovered positions are 0, contributions
     summed over levels;
  R8 pyramid entry = exact mean of its p^l tokens, rounded once to the dtype;
  R9 backward = exact chain rule with the selection held fixed.

Parity pins: every function here is pinned by tests/test_oracle_*.py against
closed forms, brute force, library routines or the pages' formulas; none is
"parity unpinned" except agreement with the authors' own code, which is not
available (the readings R1, R4, R5, R8 cannot be confirmed by any printed value).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MAX_LEVELS = 8
# Rows of the sub-sequence attention taken per group (memory only: each row is
# computed whole, and the backward adds every group's dK, dV contributions).
ATTN_ROW_BLOCK = 2048


# --------------------------------------------------------------------------
# Sizes
# --------------------------------------------------------------------------
@dataclass
class Plan:
    """Level sizes and the sub-sequence length for one (N, p, L, k).

    [SK] Stage 1: level l has N / p^l entries, the total is at most
    N p/(p-1).  [SK] Stage 3: S = N/p^(L-1) + (L-1) p k.  Reading R4 clamps a
    level's budget to its size, so S is smaller than the formula when k
    exceeds the coarsest level (the formula's S is reported beside it).
    """
    N: int
    p: int
    L: int
    k: int
    M: list = field(default_factory=list)          # entries per level, l = 0..L-1
    k_eff: list = field(default_factory=list)      # k_eff[l] for l = 1..L-1 (index 0 unused: 0)
    level_off: list = field(default_factory=list)  # flat id of (l, i) = level_off[l] + i
    M_total: int = 0
    S: int = 0
    S_formula: int = 0


def make_plan(N: int, p: int, L: int, k: int) -> Plan:
    if p < 2 or L < 1 or k < 1 or N < 1 or L > MAX_LEVELS:
        raise ValueError("need p >= 2, 1 <= L <= 8, k >= 1, N >= 1")
    if N % (p ** (L - 1)) != 0:
        raise ValueError("N must be a multiple of p^(L-1)")
    M = [N // p ** l for l in range(L)]
    k_eff = [0] + [min(k, M[l]) for l in range(1, L)]
    off = [0]
    for l in range(L):
        off.append(off[-1] + M[l])
    S = M[L - 1] + p * sum(k_eff[1:])
    S_formula = N // p ** (L - 1) + (L - 1) * p * k
    return Plan(N, p, L, k, M, k_eff, off, off[-1], S, S_formula)


# --------------------------------------------------------------------------
# Rounding to the stored dtype
# --------------------------------------------------------------------------
def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 (or float32) values once, to nearest-even, into `dtype`.

    Returned as float64 holding the rounded values.  bf16 is done as a
    round-to-odd step to float32 followed by a nearest-even step to 8
    significand bits, which equals one direct rounding because float32 keeps
    more than two extra bits (the usual round-to-odd argument).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    f = x.astype(np.float32)
    # step back toward zero where float32 rounding went away from zero
    away = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(away, np.nextafter(f, np.float32(0)), f)
    inexact = f.astype(np.float64) != x
    u = f.view(np.uint32).copy()
    u |= inexact.astype(np.uint32)                       # sticky bit = round to odd
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _check_finite(*arrays):
    for a in arrays:
        if not np.all(np.isfinite(a)):
            raise ValueError("oracle inputs must be finite")


# --------------------------------------------------------------------------
# Stage 1: symmetric mean pyramid  ([SK] Stage 1; [GE] 2A; [GI] 2A)
# --------------------------------------------------------------------------
def pyramid(x: np.ndarray, p: int, L: int, dtype: str) -> list:
    """Levels 0..L-1 of one tensor x [N, d]; level l entry i is the mean of
    tokens [i p^l, (i+1) p^l) (reading R8: exact mean, one rounding)."""
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape
    levels = [x.copy()]
    for l in range(1, L):
        n = p ** l
        levels.append(round_to(x.reshape(N // n, n, d).mean(axis=1), dtype))
    return levels


# --------------------------------------------------------------------------
# Stage 2: scores, max-pool inheritance, per-level top-K  ([SK] Stage 2)
# --------------------------------------------------------------------------
def _sumsq_f32(x: np.ndarray) -> np.ndarray:
    """Reading R2: float32 squared norm of each row of x [N, d] in the fixed
    chunked order (8 chunks of d/8, left to right, then a 3-step tree)."""
    x = np.asarray(x, dtype=np.float32)
    N, d = x.shape
    if d % 8:
        raise ValueError("d must be a multiple of 8")
    c = d // 8
    xc = x.reshape(N, 8, c)
    a = np.zeros((N, 8), dtype=np.float32)
    for j in range(c):
        col = xc[:, :, j]
        a = a + col * col                  # float32 product, then float32 add
    t = a[:, 0:4] + a[:, 4:8]
    u = t[:, 0:2] + t[:, 2:4]
    return u[:, 0] + u[:, 1]


def token_norms(x: np.ndarray) -> np.ndarray:
    """||x_t|| of every row in float32 (reading R2: the fixed chunked order,
    then a correctly rounded float32 sqrt)."""
    return np.sqrt(_sumsq_f32(x))


def token_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Parameter-free score of every token: ||q_t|| + ||k_t|| in float32
    ([SK] Stage 2 names the two l2 norms; [GE] 2B; reading R1)."""
    return (token_norms(q) + token_norms(k)).astype(np.float32)


def level_scores(s: np.ndarray, p: int, L: int) -> list:
    """Coarser levels inherit the max of the level-0 scores over their span
    ([SK] Stage 2; [GE] 2B: a coarse span keeps its strongest token)."""
    s = np.asarray(s, dtype=np.float32)
    N = s.shape[0]
    return [s.reshape(N // p ** l, p ** l).max(axis=1) for l in range(L)]


def top_k_level(sig: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k entries first under (score descending, index
    ascending), returned in ascending index order.  A stable sort on the
    negated score keeps equal scores in index order (ties to the lower
    index)."""
    order = np.argsort(-sig.astype(np.float64), kind="stable")
    return np.sort(order[:k])


def selected_sets(s: np.ndarray, plan: Plan) -> list:
    """Sel[l] = sorted selected indices of level l (reading R4):
    the coarsest level is kept whole; level l-1 gets the p children of the
    top-k_l entries of level l."""
    p, L = plan.p, plan.L
    sig = level_scores(s, p, L)
    sel = [None] * L
    sel[L - 1] = np.arange(plan.M[L - 1])
    for l in range(1, L):
        T = top_k_level(sig[l], plan.k_eff[l])
        sel[l - 1] = (T[:, None] * p + np.arange(p)[None, :]).reshape(-1)
    return sel


def gather_order(sel: list, plan: Plan):
    """Gathered order (reading R5) and its inverse.

    Entries are sorted by the last token of their span, e = (i+1) p^l - 1,
    then by level ascending.  Returns gidx [S] (flat id level_off[l] + i of
    the entry in slot g) and gpos [M_total] (slot of each entry, -1 if not
    selected)."""
    p = plan.p
    ends, lev, idx = [], [], []
    for l, ids in enumerate(sel):
        ids = np.asarray(ids, dtype=np.int64)
        ends.append((ids + 1) * p ** l - 1)
        lev.append(np.full(ids.shape, l, dtype=np.int64))
        idx.append(ids)
    ends, lev, idx = np.concatenate(ends), np.concatenate(lev), np.concatenate(idx)
    order = np.lexsort((lev, ends))                 # primary key: ends
    flat = np.asarray(plan.level_off, dtype=np.int64)[lev] + idx
    gidx = flat[order].astype(np.int32)
    gpos = np.full(plan.M_total, -1, dtype=np.int32)
    gpos[gidx] = np.arange(gidx.shape[0], dtype=np.int32)
    return gidx, gpos


def select(q: np.ndarray, k: np.ndarray, plan: Plan):
    """Scores -> per-level top-K -> gather map for one head ([SK] Stage 2-3)."""
    _check_finite(q, k)
    s = token_scores(q, k)
    return gather_order(selected_sets(s, plan), plan)


def entry_of(flat: int, plan: Plan):
    """(level, index) of a flat pyramid id."""
    for l in range(plan.L):
        if flat < plan.level_off[l + 1]:
            return l, flat - plan.level_off[l]
    raise IndexError(flat)


# --------------------------------------------------------------------------
# Stage 3: gather and dense causal attention  ([SK] Stage 3; [GE] 2C)
# --------------------------------------------------------------------------
def gather(levels: list, gidx: np.ndarray, plan: Plan) -> np.ndarray:
    """Rows of the selected entries in gathered order, [S, d] float64."""
    allrows = np.concatenate(levels, axis=0)
    return allrows[np.asarray(gidx, dtype=np.int64)]


def attention_forward(Qt, Kt, Vt, scale: float, row_block: int = ATTN_ROW_BLOCK):
    """Causal softmax attention on the sub-sequence, float64.

    O_g = sum_{g' <= g} softmax_g'(scale q_g . k_g') v_g'; also returns the
    row log-sum-exp.  Rows are taken in groups only to bound memory; each row
    is computed whole."""
    S, d = Qt.shape
    O = np.empty((S, Vt.shape[1]), dtype=np.float64)
    lse = np.empty(S, dtype=np.float64)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        Z = scale * (Qt[r0:r1] @ Kt[:r1].T)
        rows = np.arange(r0, r1)[:, None]
        Z[np.arange(r1)[None, :] > rows] = -np.inf
        m = Z.max(axis=1, keepdims=True)
        P = np.exp(Z - m)
        l = P.sum(axis=1, keepdims=True)
        O[r0:r1] = (P @ Vt[:r1]) / l
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return O, lse


def attention_backward(Qt, Kt, Vt, Ot, dOt, lse, scale: float, row_block: int = ATTN_ROW_BLOCK):
    """Gradients of causal attention w.r.t. its three inputs, float64.

    P is recomputed from the logits and the row log-sum-exp;
    D_g = dO_g . O_g; dV = P^T dO; dS = P * (dO V^T - D); dQ = scale dS K;
    dK = scale dS^T Q.  Rows are grouped only to bound memory."""
    S, d = Qt.shape
    dQ = np.zeros_like(Qt, dtype=np.float64)
    dK = np.zeros_like(Kt, dtype=np.float64)
    dV = np.zeros_like(Vt, dtype=np.float64)
    D = np.sum(dOt * Ot, axis=1)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        Z = scale * (Qt[r0:r1] @ Kt[:r1].T)
        rows = np.arange(r0, r1)[:, None]
        Z[np.arange(r1)[None, :] > rows] = -np.inf    # causal mask before exponentiating
        P = np.exp(Z - lse[r0:r1, None])
        dP = dOt[r0:r1] @ Vt[:r1].T
        dS = P * (dP - D[r0:r1, None])
        dQ[r0:r1] = scale * (dS @ Kt[:r1])
        dK[:r1] += scale * (dS.T @ Qt[r0:r1])
        dV[:r1] += P.T @ dOt[r0:r1]
    return dQ, dK, dV


# --------------------------------------------------------------------------
# Stage 4: scatter-back  ([SK] Stage 4; [GE] 2C)
# --------------------------------------------------------------------------
def scatter_ranges(l: int, i: int, p: int, N: int):
    """R(l, i) = [i p^l + p^l - 1, i p^l + 2 p^l - 2], clipped at N-1."""
    n = p ** l
    lo = i * n + n - 1
    return lo, min(N - 1, i * n + 2 * n - 2)


def scatter(Ot: np.ndarray, gpos: np.ndarray, plan: Plan) -> np.ndarray:
    """O_t = sum over levels of the output of the level-l entry whose range
    R(l, i) holds t, i.e. i = floor((t+1)/p^l) - 1, when that entry is
    selected; 0 where nothing covers t (reading R7)."""
    N, p = plan.N, plan.p
    O = np.zeros((N, Ot.shape[1]), dtype=np.float64)
    t = np.arange(N)
    for l in range(plan.L):
        i = (t + 1) // p ** l - 1
        ok = i >= 0
        g = np.full(N, -1, dtype=np.int64)
        g[ok] = gpos[plan.level_off[l] + i[ok]]
        hit = g >= 0
        O[hit] += Ot[g[hit]]
    return O


def scatter_backward(dO: np.ndarray, gidx: np.ndarray, plan: Plan) -> np.ndarray:
    """dOt[g] = sum of dO_t over t in R(l, i) for the entry (l, i) in slot g
    ([SK] gradient flow: the gradient passes back through the scatter)."""
    S = gidx.shape[0]
    dOt = np.zeros((S, dO.shape[1]), dtype=np.float64)
    for g in range(S):
        l, i = entry_of(int(gidx[g]), plan)
        lo, hi = scatter_ranges(l, i, plan.p, plan.N)
        if lo <= hi:
            dOt[g] = dO[lo:hi + 1].sum(axis=0)
    return dOt


def gather_pool_backward(dXt: np.ndarray, gpos: np.ndarray, plan: Plan) -> np.ndarray:
    """dX_t = sum over levels of p^-l dXt[slot of entry (l, floor(t/p^l))]
    for selected entries: the transpose of gather followed by the mean over
    the entry's own span [i p^l, (i+1) p^l)."""
    N, p = plan.N, plan.p
    dX = np.zeros((N, dXt.shape[1]), dtype=np.float64)
    t = np.arange(N)
    for l in range(plan.L):
        i = t // p ** l
        g = gpos[plan.level_off[l] + i].astype(np.int64)
        hit = g >= 0
        dX[hit] += dXt[g[hit]] / float(p ** l)
    return dX


# --------------------------------------------------------------------------
# Whole layer, one head
# --------------------------------------------------------------------------
def head_forward(q, k, v, p, L, kk, dtype, scale=None, selection=None, row_block=None):
    """Forward of one head.  q, k, v: [N, d] values of `dtype`.
    `selection` = (gidx, gpos) freezes the selection (it is gradient-free);
    `row_block` sets the attention's row groups (memory only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check_finite(q, k, v)
    N, d = q.shape
    plan = make_plan(N, p, L, kk)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if selection is None:
        gidx, gpos = select(q.astype(np.float32), k.astype(np.float32), plan)
    else:
        gidx, gpos = selection
    lq, lk, lv = pyramid(q, p, L, dtype), pyramid(k, p, L, dtype), pyramid(v, p, L, dtype)
    Qt, Kt, Vt = gather(lq, gidx, plan), gather(lk, gidx, plan), gather(lv, gidx, plan)
    rb = ATTN_ROW_BLOCK if row_block is None else row_block
    Ot, lse = attention_forward(Qt, Kt, Vt, scale, rb)
    O = round_to(scatter(Ot, gpos, plan), dtype)
    return dict(plan=plan, scale=scale, gidx=gidx, gpos=gpos, levels=(lq, lk, lv),
                Qt=Qt, Kt=Kt, Vt=Vt, Ot=Ot, lse=lse, O=O, dtype=dtype, row_block=rb)

def head_backward(st: dict, dO):
    """Backward of one head from the forward state and dO [N, d]."""
    plan, dtype, scale = st["plan"], st["dtype"], st["scale"]
    dO = np.asarray(dO, dtype=np.float64)
    _check_finite(dO)
    dOt = round_to(scatter_backward(dO, st["gidx"], plan), dtype)
    dQt, dKt, dVt = attention_backward(st["Qt"], st["Kt"], st["Vt"], st["Ot"], dOt,
                                       st["lse"], scale, st["row_block"])
    dq = round_to(gather_pool_backward(dQt, st["gpos"], plan), dtype)
    dk = round_to(gather_pool_backward(dKt, st["gpos"], plan), dtype)
    dv = round_to(gather_pool_backward(dVt, st["gpos"], plan), dtype)
    return dict(dOt=dOt, dQt=dQt, dKt=dKt, dVt=dVt, dq=dq, dk=dk, dv=dv)


def layer_forward(q, k, v, p, L, kk, dtype, scale=None, heads=None):
    """[B,H,N,d] arrays -> dict of per-head states keyed by (b, h)."""
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    return {(b, h): head_forward(q[b, h], k[b, h], v[b, h], p, L, kk, dtype, scale)
            for (b, h) in heads}


def dense_forward(q, k, v, dtype, scale=None):
    """Dense causal attention of one head: the layer with L = 1 ([SK]
    selection-attention decoupling: switching selection off gives dense)."""
    N = q.shape[0]
    return head_forward(q, k, v, 2, 1, 1, dtype, scale)


# ------------------------------------------------------------------ projections
# [SK] "four-stage pipeline": the layer starts from the Q, K, V projections of
# its input X; "complexity": the projections are a GEMM of Theta(N d_model d);
# "gradient flow": the gradient reaches W_Q, W_K, W_V through gather (none
# through selection).  Reading: one weight matrix w [3 H d, Dm] in the
# out x in convention, rows Q then K then V, head h of each at rows h d ..
# (h+1) d - 1 (multi-head attention with H heads of size d for Q, K and V).

def qkv_project(x, w, H, d, dtype):
    """x [B,N,Dm], w [3Hd, Dm] -> q, k, v [B,H,N,d]: q[b,h,n] = x[b,n] . w[h d + j]
    for j < d (k and v from the next H d rows), in float64 (a library matrix
    product), each output rounded once to dtype."""
    B, N, Dm = x.shape
    if w.shape != (3 * H * d, Dm):
        raise ValueError("w must be [3*H*d, Dm]")
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T      # [B, N, 3Hd]
    y = y.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)                       # [3, B, H, N, d]
    return tuple(round_to(y[i], dtype) for i in range(3))


def qkv_features(dq, dk, dv):
    """[B,H,N,d] x 3 -> [B, N, 3Hd] with feature index (which, h, j) as in w's rows."""
    g = np.stack([np.asarray(a, dtype=np.float64) for a in (dq, dk, dv)])         # [3, B, H, N, d]
    three, B, H, N, d = g.shape
    return g.transpose(1, 3, 0, 2, 4).reshape(B, N, 3 * H * d)


def qkv_project_backward(x, w, dq, dk, dv, dtype):
    """Gradients of sum(q dq + k dk + v dv) for q, k, v = qkv_project(x, w):
    dx [B,N,Dm] = G w (rounded once to dtype) and dw [3Hd, Dm] = G^T x summed
    over all B N tokens (float64), where G [B,N,3Hd] = qkv_features(dq, dk, dv)."""
    G = qkv_features(dq, dk, dv)
    B, N, F = G.shape
    x64 = np.asarray(x, dtype=np.float64)
    dx = round_to(G @ np.asarray(w, dtype=np.float64), dtype)
    dw = G.reshape(B * N, F).T @ x64.reshape(B * N, -1)
    return dx, dw
