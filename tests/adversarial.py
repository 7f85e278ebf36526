"""Adversarial inputs for the 98K layer: clustered high-norm spans, exact-tie
subtrees and score ties straddling each top-K cut (test infrastructure; uses
the oracle's scores to place the ties, never the HIP path).

Recipe (on top of the seeded N(0,1) x lognormal(0,0.5) tensors):
 1. Boost: floor(0.01 N) tokens in 3 non-overlapping spans (lengths split as
    evenly as possible), starts drawn by the RNG and not aligned to p^l, the
    same for every head; their q and k rows are multiplied by 8 (exact in
    bf16: a power of two), v is left alone.
 2. Exact-tie subtrees: per head, one aligned block of p^(L-1) tokens from
    inside a boosted span is copied (q, k, v) over 4 other aligned blocks:
    identical subtrees, so equal scores at every level.
 3. Threshold ties: for l = L-2 down to 1, tau_l = the k_l-th largest level-l
    score; the q, k rows of a token scoring exactly tau_l are copied into one
    token of 16 level-l entries that score below tau_l and whose coarser
    ancestors score at least tau_l (so no coarser level changes).  The tie
    group then straddles the cut: #{> tau} < k_l < #{>= tau}.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import lighthouse_oracle as orc


def _level_scores_head(q, k, p, L):
    s = orc.token_scores(q[0].float().numpy(), k[0].float().numpy())
    return s, orc.level_scores(s, p, L)


def make_adversarial(w, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log=print):
    """Modifies q, k, v ([B,H,N,d] CPU tensors of the layer dtype) in place."""
    assert w.B == 1
    rng = np.random.Generator(np.random.PCG64(w.seed + 2000))
    N, p, L, H = w.N, w.p, w.L, w.H
    plan = orc.make_plan(N, p, L, w.k)
    blk = p ** (L - 1)

    # 1. boosted spans
    total = N // 100
    lens = [total // 3 + (1 if i < total % 3 else 0) for i in range(3)]
    seg = N // 3
    spans = []
    for i, ln in enumerate(lens):
        lo = i * seg
        start = int(rng.integers(lo + 1, lo + seg - ln - 1))
        if start % p == 0:
            start += 1
        spans.append((start, start + ln))
    for a, b in spans:
        q[:, :, a:b] *= 8
        k[:, :, a:b] *= 8
    boosted = np.zeros(N, dtype=bool)
    for a, b in spans:
        boosted[a:b] = True

    # 2. exact-tie subtrees
    for h in range(H):
        a, b = spans[int(rng.integers(3))]
        src = (a + blk - 1) // blk
        if (src + 1) * blk > b:
            src = a // blk
        dsts = []
        while len(dsts) < 4:
            dst = int(rng.integers(N // blk))
            if dst != src and dst not in dsts and not boosted[dst * blk:(dst + 1) * blk].any():
                dsts.append(dst)
        for dst in dsts:
            for t in (q, k, v):
                t[0, h, dst * blk:(dst + 1) * blk] = t[0, h, src * blk:(src + 1) * blk]

    # 3. threshold ties at every level with a cut
    sizes = {}
    for l in range(L - 2, 0, -1):
        kl = plan.k_eff[l]
        if kl >= plan.M[l]:
            continue
        for h in range(H):
            s, sig = _level_scores_head(q[:, h], k[:, h], p, L)
            order = np.argsort(-sig[l].astype(np.float64), kind="stable")
            tau = sig[l][order[kl - 1]]
            owner = int(order[kl - 1])
            n = p ** l
            tok = owner * n + int(np.flatnonzero(s[owner * n:(owner + 1) * n] == tau)[0])
            ok = sig[l] < tau
            for lc in range(l + 1, L):     # ancestors must already score >= tau
                ok &= np.repeat(sig[lc] >= tau, p ** (lc - l))
            cand = np.flatnonzero(ok)
            below = cand[cand < owner][-8:]
            above = cand[cand > owner][:8]
            chosen = np.concatenate([below, above])
            if len(chosen) < 16:
                extra = [c for c in cand if c not in set(chosen.tolist())]
                chosen = np.concatenate([chosen, np.array(extra[:16 - len(chosen)], dtype=np.int64)])
            for j in chosen[:16]:
                dst = int(j) * n + int(rng.integers(n))
                q[0, h, dst] = q[0, h, tok]
                k[0, h, dst] = k[0, h, tok]
            s2, sig2 = _level_scores_head(q[:, h], k[:, h], p, L)
            gt = int((sig2[l] > tau).sum())
            ge = int((sig2[l] >= tau).sum())
            assert gt < kl < ge, (l, h, gt, kl, ge)
            sizes[(l, h)] = ge - gt
    # fan-in reaches L somewhere in every head
    for h in range(H):
        gidx, gpos = orc.select(q[0, h].float().numpy(), k[0, h].float().numpy(), plan)
        fan = np.zeros(N + 1, dtype=np.int32)
        for l in range(L):
            sel = np.flatnonzero(gpos[plan.level_off[l]:plan.level_off[l + 1]] >= 0)
            lo = (sel + 1) * p ** l - 1
            hi = np.minimum(N - 1, lo + p ** l - 1)
            np.add.at(fan, lo, 1)
            np.add.at(fan, hi + 1, -1)
        assert np.cumsum(fan)[:N].max() == L, h
    log(f"adversarial: spans {spans}; tie-group sizes at the cuts (level, head) -> size: "
        f"min {min(sizes.values())}, max {max(sizes.values())}")
    return spans, sizes
