"""Helpers for the GPU parity tests: run the HIP library through the C ABI
on a workload and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from long_context_pretraining_amd import inputs
from long_context_pretraining_amd import lighthouse as lh
from oracle import lighthouse_oracle as orc


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, ref, dtype: str, what: str):
    """f32: max|a-b| <= 1e-4 max|b| over the tensor; bf16: |a-b| <= 2e-2 max(1,|b|)
    element-wise (one bf16 ulp at |b| >= 8 is 0.0625, so a pure 2e-2 bound
    cannot hold there)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = np.abs(got - ref)
    if dtype == "f32":
        bound = 1e-4 * max(float(np.abs(ref).max()), 1e-30)
        assert diff.max() <= bound, f"{what}: max abs err {diff.max():.3e} > {bound:.3e}"
    else:
        lim = 2e-2 * np.maximum(1.0, np.abs(ref))
        bad = diff > lim
        if bad.any():
            i = np.unravel_index(np.argmax(diff / lim), diff.shape)
            raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements beyond 2e-2*max(1,|ref|); "
                                 f"worst at {i}: got {got[i]:.6g} ref {ref[i]:.6g}")
    return float(diff.max())


class GpuResult:
    pass


def run_layer(w: inputs.Workload, q, k, v, dout, runs: int = 1) -> GpuResult:
    """Run pyramid, score/top-K, forward and backward once (or `runs` times,
    keeping every run's outputs for determinism checks)."""
    dt = inputs.TORCH_DTYPE[w.dtype]
    layer = lh.LighthouseLayer(w.B, w.H, w.N, w.d, w.p, w.L, w.k, dt)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, dout))
    outs = []
    for _ in range(runs):
        o = torch.empty_like(qd)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(qd), torch.empty_like(qd)
        layer.forward(qd, kd, vd, o)
        layer.backward(dod, dq, dk, dv)
        torch.cuda.synchronize()
        outs.append((o.clone(), dq.clone(), dk.clone(), dv.clone(), layer.gidx.clone(), layer.gpos.clone()))
    r = GpuResult()
    r.layer, r.plan = layer, layer.plan
    r.o, r.dq, r.dk, r.dv, r.gidx, r.gpos = outs[-1]
    r.runs = outs
    B, H, S, d = w.B, w.H, layer.plan.S, w.d
    Mu = layer.plan.M_total - w.N
    r.pyr = r.norms = None
    if layer.pyr is not None:   # the pooled levels, then the token norms of q and k ([2][B,H,N] f32)
        nlev = 3 * B * H * Mu * d
        r.pyr = layer.pyr[:nlev].view(3, B, H, Mu, d)
        r.norms = layer.pyr[nlev:].view(torch.float32).view(2, B, H, w.N)
    r.og = layer.fwd_view(lh.FWD_O, torch.float32, (B, H, S, d))
    r.lse = layer.fwd_view(lh.FWD_LSE, torch.float32, (B, H, S))
    r.qg = layer.fwd_view(lh.FWD_QG, dt, (B, H, S, d))
    r.dog = layer.bwd_view(lh.BWD_DO, dt, (B, H, S, d))
    return r


def head_np(t, b, h):
    return t[b, h].float().numpy().astype(np.float64)


def compare_selection(w, q, k, r, heads=None):
    plan = orc.make_plan(w.N, w.p, w.L, w.k)
    gidx, gpos = r.gidx.cpu().numpy(), r.gpos.cpu().numpy()
    heads = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        g_ref, p_ref = orc.select(head_np(q, b, h).astype(np.float32), head_np(k, b, h).astype(np.float32), plan)
        assert np.array_equal(gidx[b, h], g_ref), f"gidx differs at head ({b},{h}): first at {np.argmax(gidx[b, h] != g_ref)}"
        assert np.array_equal(gpos[b, h], p_ref), f"gpos differs at head ({b},{h})"


def error_ratio(got, ref, dtype):
    """Worst error as a fraction of the allowed error (<= 1 passes)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    if dtype == "f32":
        return float(diff.max() / (1e-4 * max(float(np.abs(ref).max()), 1e-30)))
    return float((diff / (2e-2 * np.maximum(1.0, np.abs(ref)))).max())


def compare_head(w, q, k, v, dout, r, b, h, scale=None, check_bwd=True):
    """Every tensor of one head against the oracle; all are checked and every
    failure is reported together."""
    st = orc.head_forward(head_np(q, b, h), head_np(k, b, h), head_np(v, b, h), w.p, w.L, w.k, w.dtype, scale)
    tag = f"{w.name}[{b},{h}]"
    assert np.array_equal(r.gidx[b, h].cpu().numpy(), st["gidx"]), f"{tag}: gidx"
    pairs = []
    if r.pyr is not None:
        plan = st["plan"]
        for zi, z in enumerate("qkv"):
            got = to_np(r.pyr[zi, b, h])
            for l in range(1, w.L):
                lo, hi = plan.level_off[l] - w.N, plan.level_off[l + 1] - w.N
                pairs.append((f"pyramid {z} level {l}", got[lo:hi], st["levels"][zi][l]))
    pairs += [("gathered Q", to_np(r.qg[b, h]), st["Qt"]), ("sub-sequence output", to_np(r.og[b, h]), st["Ot"]),
              ("output O", to_np(r.o[b, h]), st["O"])]
    lse = to_np(r.lse[b, h])
    lse_ok = bool(np.all(np.abs(lse - st["lse"]) <= 1e-4 * np.maximum(1.0, np.abs(st["lse"]))))
    if check_bwd:
        bw = orc.head_backward(st, head_np(dout, b, h))
        pairs += [("dO~", to_np(r.dog[b, h]), bw["dOt"]), ("dQ", to_np(r.dq[b, h]), bw["dq"]),
                  ("dK", to_np(r.dk[b, h]), bw["dk"]), ("dV", to_np(r.dv[b, h]), bw["dv"])]
    fails = []
    ratios = {}
    for name, got, ref in pairs:
        ratios[name] = error_ratio(got, ref, w.dtype)
        try:
            check_close(got, ref, w.dtype, f"{tag} {name}")
        except AssertionError as e:
            fails.append(str(e))
    say(f"  {tag} worst error / allowed: " + ", ".join(f"{n} {x:.3f}" for n, x in ratios.items()
                                                      if not n.startswith("pyramid")))
    if not lse_ok:
        fails.append(f"{tag}: lse")
    if r.norms is not None:   # the token norms the scores start from: bit for bit (reading R2)
        for zi, (z, x) in enumerate((("q", q), ("k", k))):
            ref = orc.token_norms(head_np(x, b, h).astype(np.float32))
            got = r.norms[zi, b, h].cpu().numpy()
            if not np.array_equal(got, ref):
                fails.append(f"{tag}: ||{z}_t|| differs from the oracle at {int(np.sum(got != ref))} tokens")
    assert not fails, "\n".join(fails)
    return st
