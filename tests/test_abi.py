"""The C ABI on the CPU: the library loads, exports what the header declares,
sizes problems like the oracle, and rejects bad arguments before launching
anything (no GPU needed: every check here fails before a launch)."""
import ctypes

import pytest

from long_context_pretraining_amd import lighthouse as lh
from oracle import lighthouse_oracle as orc
from tests.conftest import read_golden

FAKE = 0x100000          # aligned, never dereferenced: every call below fails validation first


def test_exports_every_header_function():
    lib = lh.load_library()
    names = lh.header_functions()
    assert set(names) == {"lh_make_plan", "lh_pyramid", "lh_score_topk", "lh_score_topk_noalloc",
                          "lh_forward", "lh_backward",
                          "dense_causal_attn", "dense_causal_attn_backward", "lh_status_string", "lh_set_probe",
                          "lh_set_probe_flush", "lh_peak_hbm", "lh_peak_mfma",
                          "lh_qkv_plan", "lh_qkv_forward", "lh_qkv_backward"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in (lh.LH_OK, lh.LH_E_ARG, lh.LH_E_UNSUPPORTED, lh.LH_E_WORKSPACE, lh.LH_E_DEVICE, 17):
        assert isinstance(lh.status_string(s), str) and lh.status_string(s)


@pytest.mark.parametrize("N,p,L,k,d,dt", [(4096, 4, 3, 64, 64, 0), (98304, 4, 4, 1536, 64, 1), (98304, 4, 4, 6144, 64, 1),
                                          (524288, 4, 6, 1536, 64, 1), (1000, 2, 3, 13, 128, 1), (729, 3, 4, 7, 64, 1),
                                          (256, 4, 1, 1, 64, 0)])
def test_plan_matches_oracle(N, p, L, k, d, dt):
    plan = lh.lh_make_plan(lh.make_desc(1, 2, N, d, p, L, k, dt))
    ref = orc.make_plan(N, p, L, k)
    assert list(plan.M)[:L] == ref.M
    assert list(plan.k_eff)[1:L] == ref.k_eff[1:]
    assert list(plan.level_off)[:L + 1] == ref.level_off
    assert plan.M_total == ref.M_total and plan.S == ref.S and plan.S_formula == ref.S_formula
    assert plan.S_pad % 64 == 0 and plan.S <= plan.S_pad < plan.S + 64
    e = 4 if dt == 0 else 2
    # pooled levels of q, k, v (B=1, H=2), then the token norms of q and k in f32 (L > 1)
    assert plan.pyr_bytes == 3 * 2 * (ref.M_total - N) * d * e + (2 * 2 * N * 4 if L > 1 else 0)
    offs = list(plan.fwd_off)
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and plan.fwd_ws_bytes > offs[-1]


def test_plan_golden_s():
    for N, p, L, k, Sf, Sa in read_golden("s_formula.txt"):
        plan = lh.lh_make_plan(lh.make_desc(1, 1, int(N), 64, int(p), int(L), int(k), 1))
        assert (plan.S_formula, plan.S) == (int(Sf), int(Sa))


@pytest.mark.parametrize("args,code", [
    ((1, 1, 100, 64, 4, 3, 1, 1), lh.LH_E_ARG),        # N not a multiple of p^(L-1)
    ((1, 1, 64, 64, 1, 2, 1, 1), lh.LH_E_ARG),         # p < 2
    ((1, 1, 64, 64, 2, 0, 1, 1), lh.LH_E_ARG),         # L < 1
    ((1, 1, 64, 64, 2, 9, 1, 1), lh.LH_E_ARG),         # L > 8
    ((1, 1, 64, 64, 2, 2, 0, 1), lh.LH_E_ARG),         # k < 1
    ((0, 1, 64, 64, 2, 2, 1, 1), lh.LH_E_ARG),         # B < 1
    ((1, 0, 64, 64, 2, 2, 1, 1), lh.LH_E_ARG),         # no heads
    ((1, 1, 0, 64, 2, 2, 1, 1), lh.LH_E_ARG),          # empty sequence
    ((1, 1, 64, 0, 2, 2, 1, 1), lh.LH_E_ARG),          # empty rows (d = 0)
    ((1, 1, 64, 64, 2, 2, 1, 7), lh.LH_E_ARG),         # unknown dtype
    ((1, 1, 64, 60, 2, 2, 1, 1), lh.LH_E_ARG),         # d not a multiple of 8
    ((1, 1, 64, 96, 2, 2, 1, 1), lh.LH_E_UNSUPPORTED), # d = 96 not built
    ((1, 1, 64, 128, 2, 2, 1, 0), lh.LH_E_UNSUPPORTED),  # f32 with d = 128 not built
    ((1, 1, 8, 64, 4, 3, 1, 1), lh.LH_E_ARG),          # p^(L-1) > N
    ((1, 1, 1 << 25, 64, 2, 1, 1, 1), lh.LH_E_UNSUPPORTED),  # L = 1: S = 2^25 rows of 128 B reach 2^32 bytes
    ((1, 1, 8 ** 5, 64, 8, 6, 1, 1), lh.LH_E_UNSUPPORTED),   # p^(L-1) = 32768: a score chunk exceeds the LDS
])
def test_plan_rejects(args, code):
    with pytest.raises(lh.LighthouseError) as e:
        lh.lh_make_plan(lh.make_desc(*args))
    assert e.value.status == code


def _call(name, *args):
    lib = lh.load_library()
    return getattr(lib, name)(*args)


def test_entry_points_validate_before_launch():
    desc = lh.make_desc(1, 2, 4096, 64, 4, 3, 64, 1)
    plan = lh.lh_make_plan(desc)
    D = ctypes.byref(desc)
    # null pointers
    assert _call("lh_pyramid", D, None, FAKE, FAKE, FAKE, plan.pyr_bytes, None) == lh.LH_E_ARG
    assert _call("lh_score_topk", D, FAKE, FAKE, FAKE, FAKE, None, FAKE, plan.sel_ws_bytes, None) == lh.LH_E_ARG
    assert _call("lh_score_topk", D, None, FAKE, FAKE, FAKE, FAKE, FAKE, plan.sel_ws_bytes, None) == lh.LH_E_ARG  # no q
    assert _call("lh_score_topk", D, FAKE, None, None, FAKE, FAKE, FAKE, plan.sel_ws_bytes, None) == lh.LH_E_ARG  # no k
    assert _call("lh_score_topk", D, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, plan.sel_ws_bytes,
                 None) == lh.LH_E_ARG   # misaligned (optional) pyramid
    assert _call("lh_forward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, plan.fwd_ws_bytes, None) == lh.LH_E_ARG
    assert _call("lh_backward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, plan.bwd_ws_bytes, None) == lh.LH_E_ARG
    # misaligned pointers
    assert _call("lh_pyramid", D, FAKE + 2, FAKE, FAKE, FAKE, plan.pyr_bytes, None) == lh.LH_E_ARG
    assert _call("dense_causal_attn", D, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, plan.dense_fwd_ws_bytes, None) == lh.LH_E_ARG
    # short workspaces
    assert _call("lh_pyramid", D, FAKE, FAKE, FAKE, FAKE, plan.pyr_bytes - 1, None) == lh.LH_E_WORKSPACE
    assert _call("lh_score_topk", D, FAKE, FAKE, None, FAKE, FAKE, FAKE, plan.sel_ws_bytes - 1,
                 None) == lh.LH_E_WORKSPACE
    assert _call("lh_forward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, plan.fwd_ws_bytes - 1, None) == lh.LH_E_WORKSPACE
    assert _call("lh_backward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, plan.bwd_ws_bytes - 1, None) == lh.LH_E_WORKSPACE
    assert _call("dense_causal_attn", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, plan.dense_fwd_ws_bytes - 1, None) == lh.LH_E_WORKSPACE
    assert _call("dense_causal_attn_backward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 plan.dense_bwd_ws_bytes - 1, None) == lh.LH_E_WORKSPACE
    # bad descriptor
    bad = lh.make_desc(1, 2, 4095, 64, 4, 3, 64, 1)
    assert _call("lh_forward", ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == lh.LH_E_ARG
    assert _call("lh_make_plan", None, None) == lh.LH_E_ARG


def test_row_offset_limit():
    """One head's rows must stay under 2^32 bytes (32-bit offsets in the
    attention kernels): the last size below passes, the first at the limit is
    refused, by the plan (sub-sequence S) and by the dense entry points (N)."""
    below = lh.lh_make_plan(lh.make_desc(1, 1, (1 << 25) - 64, 64, 2, 1, 1, 1))
    assert below.S == (1 << 25) - 64
    # S small (L = 4), N = 2^25 bf16 rows of 128 B: the layer plans, the dense path refuses
    desc = lh.make_desc(1, 1, 1 << 25, 64, 4, 4, 64, 1)
    plan = lh.lh_make_plan(desc)
    assert plan.S < (1 << 20)
    D = ctypes.byref(desc)
    assert _call("dense_causal_attn", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == lh.LH_E_UNSUPPORTED
    assert _call("dense_causal_attn_backward", D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 1 << 40, None) == lh.LH_E_UNSUPPORTED


def test_tensor_marshalling_rejects_host_tensors():
    import torch
    desc = lh.make_desc(1, 1, 64, 64, 2, 2, 1, 1)
    t = torch.zeros(10)
    with pytest.raises(ValueError):
        lh.lh_pyramid(desc, t, t, t, t)


@pytest.mark.parametrize("N,p,L,d,dt", [(4 ** 7, 4, 8, 64, 1), (4 ** 7, 4, 8, 128, 1), (4 ** 7, 4, 8, 64, 0),
                                         (3 ** 8, 3, 8, 64, 1), (2 ** 14, 128, 3, 64, 1), (8 ** 4, 8, 5, 128, 1)])
def test_deep_pyramids_plan(N, p, L, d, dt):
    """Deep pyramids up to p^(L-1) = 16384 plan (the pooling pass then takes
    short passes over sliced rows) and match the oracle's sizes."""
    plan = lh.lh_make_plan(lh.make_desc(1, 1, N, d, p, L, 1, dt))
    assert plan.S == orc.make_plan(N, p, L, 1).S


def test_probe_hook_validates_kernel_id():
    lib = lh.load_library()
    assert lib.lh_set_probe(-1, None, None) == lh.LH_OK
    assert lib.lh_set_probe(lh.KERNEL_NORM + 1, None, None) == lh.LH_E_ARG
    assert lib.lh_set_probe(-2, None, None) == lh.LH_E_ARG
    assert lib.lh_set_probe(lh.KERNEL_ATTN_DKDV, None, None) == lh.LH_OK   # null events: off
    assert lib.lh_set_probe_flush(None, 0) == lh.LH_OK
    assert lib.lh_set_probe_flush(FAKE + 4, 1 << 20) == lh.LH_E_ARG     # misaligned
    assert lib.lh_set_probe_flush(None, 1 << 20) == lh.LH_E_ARG         # no buffer
    assert lib.lh_peak_hbm(0, FAKE, FAKE, 17, None) == lh.LH_E_ARG          # not a multiple of 16
    assert lib.lh_peak_hbm(3, FAKE, FAKE, 16, None) == lh.LH_E_ARG          # unknown mode
    assert lib.lh_peak_hbm(0, FAKE, None, 16, None) == lh.LH_E_ARG          # copy without a source
    assert lib.lh_peak_mfma(None, 10, None) == lh.LH_E_ARG
    assert lib.lh_peak_mfma(FAKE, 0, None) == lh.LH_E_ARG


def test_projection_plan_and_argument_checks():
    """Projection calls: sizes on the host, shape/alignment checks before any launch."""
    lib = lh.load_library()
    B, N, Dm, H, d = 2, 128, 128, 2, 64
    n = lh.lh_qkv_plan(lh.make_proj_desc(B, N, Dm, H, d))
    Nc, M = 3 * H * d, B * N
    assert n >= Dm * Nc * 2 + 4 * Nc * Dm * 4   # W^T and at least 4 dW k-split partials (f32)
    for bad, status in [((B, 100, Dm, H, d), lh.LH_E_UNSUPPORTED),    # N not a multiple of 64
                        ((B, N, 96, H, d), lh.LH_E_UNSUPPORTED),      # Dm not a multiple of 64
                        ((B, N, Dm, H, 96), lh.LH_E_UNSUPPORTED),     # d not built
                        ((0, N, Dm, H, d), lh.LH_E_ARG),              # empty batch
                        ((B, 0, Dm, H, d), lh.LH_E_ARG),              # empty sequence
                        ((B, N, Dm, 0, d), lh.LH_E_ARG)]:             # no heads
        with pytest.raises(lh.LighthouseError) as e:
            lh.lh_qkv_plan(lh.make_proj_desc(*bad))
        assert e.value.status == status
    desc = lh.make_proj_desc(B, N, Dm, H, d)
    fake = 1 << 20   # aligned, never dereferenced: the checks fail before any launch
    assert lib.lh_qkv_forward(ctypes.byref(desc), None, fake, fake, fake, fake, None) == lh.LH_E_ARG
    assert lib.lh_qkv_forward(ctypes.byref(desc), fake + 2, fake, fake, fake, fake, None) == lh.LH_E_ARG
    assert lib.lh_qkv_backward(ctypes.byref(desc), fake, fake, fake, fake, fake, fake, fake, fake, n - 1,
                               None) == lh.LH_E_WORKSPACE
