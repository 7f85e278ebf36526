"""Python binding of liblighthouse.so (include/lighthouse.h), same names.

Argument marshalling only: every step runs in the HIP library.  torch is
used for device memory and the current stream.  Importing this module does
not load the library; the first call does, and fails loudly if it has not
been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblighthouse.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lighthouse.h")

LH_F32, LH_BF16 = 0, 1
LH_OK, LH_E_ARG, LH_E_UNSUPPORTED, LH_E_WORKSPACE, LH_E_DEVICE = 0, -1, -2, -3, -4
MAX_LEVELS = 8
FWD_QG, FWD_KG, FWD_VG, FWD_QT, FWD_KT, FWD_VT, FWD_O, FWD_LSE = range(8)
BWD_DO, BWD_DOT, BWD_NEG_D, BWD_DQ, BWD_DK, BWD_DV, BWD_NEG_LSE = range(7)

DTYPE_CODE = {torch.float32: LH_F32, torch.bfloat16: LH_BF16}


class LhDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64), ("d", ctypes.c_int64),
                ("p", ctypes.c_int32), ("L", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class LhPlan(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64 * MAX_LEVELS), ("k_eff", ctypes.c_int64 * MAX_LEVELS),
                ("level_off", ctypes.c_int64 * (MAX_LEVELS + 1)), ("M_total", ctypes.c_int64),
                ("S", ctypes.c_int64), ("S_formula", ctypes.c_int64), ("S_pad", ctypes.c_int64),
                ("pyr_bytes", ctypes.c_size_t), ("sel_ws_bytes", ctypes.c_size_t),
                ("fwd_ws_bytes", ctypes.c_size_t), ("bwd_ws_bytes", ctypes.c_size_t),
                ("dense_fwd_ws_bytes", ctypes.c_size_t), ("dense_bwd_ws_bytes", ctypes.c_size_t),
                ("fwd_off", ctypes.c_size_t * 8), ("bwd_off", ctypes.c_size_t * 7)]


class LhProjDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("Dm", ctypes.c_int64), ("H", ctypes.c_int64),
                ("d", ctypes.c_int64)]


class LighthouseError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SIGS = {
    "lh_make_plan": [ctypes.POINTER(LhDesc), ctypes.POINTER(LhPlan)],
    "lh_pyramid": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _SZ, _VP],
    "lh_score_topk": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "lh_score_topk_noalloc": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP],
    "lh_forward": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "lh_backward": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "dense_causal_attn": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "dense_causal_attn_backward": [ctypes.POINTER(LhDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                   _SZ, _VP],
    "lh_qkv_plan": [ctypes.POINTER(LhProjDesc), ctypes.POINTER(ctypes.c_size_t)],
    "lh_qkv_forward": [ctypes.POINTER(LhProjDesc), _VP, _VP, _VP, _VP, _VP, _VP],
    "lh_qkv_backward": [ctypes.POINTER(LhProjDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP],
    "lh_status_string": [ctypes.c_int],
    "lh_set_probe": [ctypes.c_int, _VP, _VP],
    "lh_set_probe_flush": [_VP, _SZ],
    "lh_peak_hbm": [ctypes.c_int, _VP, _VP, _SZ, _VP],
    "lh_peak_mfma": [_VP, ctypes.c_int, _VP],
}

(KERNEL_POOL, KERNEL_SCORE, KERNEL_TOPK, KERNEL_MAP, KERNEL_GATHER, KERNEL_ATTN_FWD, KERNEL_SCATTER_FWD,
 KERNEL_SCATTER_BWD, KERNEL_ATTN_DKDV, KERNEL_ATTN_DQ, KERNEL_GATHER_POOL_BWD, KERNEL_TRANSPOSE,
 KERNEL_DENSE_PREP, KERNEL_QKV_FWD, KERNEL_QKV_BWD, KERNEL_NORM) = range(16)


def header_functions() -> list:
    """Names of the functions include/lighthouse.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m long_context_pretraining_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "lh_status_string" else ctypes.c_int
    _lib = lib
    return lib


def lh_set_probe(kernel: int, start_event, stop_event):
    """Record raw hipEvent_t handles around every later launch of `kernel`
    (-1 switches the hook off)."""
    _check(load_library().lh_set_probe(kernel, start_event, stop_event), "lh_set_probe")


def lh_set_probe_flush(buffer, nbytes: int):
    """Before every later probed launch, read nbytes of the device tensor
    `buffer`, evicting the caches (0 switches it off)."""
    _check(load_library().lh_set_probe_flush(_p(buffer) if nbytes else None, nbytes), "lh_set_probe_flush")


PEAK_MFMA_FLOPS_PER_ITER = 256 * 8 * 4 * 32768


def lh_peak_hbm(mode: int, dst, src, nbytes: int, stream=None):
    """mode 0: copy src to dst; 1: read src; 2: write dst."""
    _check(load_library().lh_peak_hbm(mode, _p(dst), _p(src), nbytes, _stream(stream)), "lh_peak_hbm")


def lh_peak_mfma(out, iters: int, stream=None):
    _check(load_library().lh_peak_mfma(_p(out), iters, _stream(stream)), "lh_peak_mfma")


def status_string(status: int) -> str:
    return load_library().lh_status_string(status).decode()


def _check(status: int, where: str):
    if status != LH_OK:
        raise LighthouseError(status, where)


def make_desc(B, H, N, d, p, L, k, dtype, scale: float = 0.0) -> LhDesc:
    code = dtype if isinstance(dtype, int) else DTYPE_CODE[dtype]
    return LhDesc(B, H, N, d, p, L, k, code, scale)


def lh_make_plan(desc: LhDesc) -> LhPlan:
    plan = LhPlan()
    _check(load_library().lh_make_plan(ctypes.byref(desc), ctypes.byref(plan)), "lh_make_plan")
    return plan


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def lh_pyramid(desc, q, k, v, pyr, stream=None):
    _check(load_library().lh_pyramid(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(pyr), _nbytes(pyr),
                                     _stream(stream)), "lh_pyramid")


def lh_score_topk(desc, q, k, pyr, gidx, gpos, ws, stream=None):
    """pyr may be None: the token norms are then computed from q and k."""
    _check(load_library().lh_score_topk(ctypes.byref(desc), _p(q), _p(k), _p(pyr), _p(gidx), _p(gpos), _p(ws),
                                        _nbytes(ws), _stream(stream)), "lh_score_topk")


STATIC_SCRATCH_BYTES = 32 << 20


def lh_score_topk_noalloc(desc, q, k, pyr, gidx, gpos, stream=None):
    """lh_score_topk with the library's own per-GPU scratch array (no ws)."""
    _check(load_library().lh_score_topk_noalloc(ctypes.byref(desc), _p(q), _p(k), _p(pyr), _p(gidx), _p(gpos),
                                                _stream(stream)), "lh_score_topk_noalloc")


def lh_forward(desc, q, k, v, pyr, gidx, gpos, o, fwd_ws, stream=None):
    _check(load_library().lh_forward(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(pyr), _p(gidx), _p(gpos), _p(o),
                                     _p(fwd_ws), _nbytes(fwd_ws), _stream(stream)), "lh_forward")


def lh_backward(desc, gidx, gpos, fwd_ws, dout, dq, dk, dv, bwd_ws, stream=None):
    _check(load_library().lh_backward(ctypes.byref(desc), _p(gidx), _p(gpos), _p(fwd_ws), _p(dout), _p(dq), _p(dk),
                                      _p(dv), _p(bwd_ws), _nbytes(bwd_ws), _stream(stream)), "lh_backward")


def dense_causal_attn(desc, q, k, v, o, lse, ws, stream=None):
    _check(load_library().dense_causal_attn(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse), _p(ws),
                                            _nbytes(ws), _stream(stream)), "dense_causal_attn")


def dense_causal_attn_backward(desc, q, k, v, lse, fwd_ws, dout, dq, dk, dv, ws, stream=None):
    _check(load_library().dense_causal_attn_backward(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(lse),
                                                     _p(fwd_ws), _p(dout), _p(dq), _p(dk), _p(dv), _p(ws),
                                                     _nbytes(ws), _stream(stream)), "dense_causal_attn_backward")


def make_proj_desc(B, N, Dm, H, d) -> LhProjDesc:
    return LhProjDesc(B, N, Dm, H, d)


def lh_qkv_plan(desc: LhProjDesc) -> int:
    n = ctypes.c_size_t()
    _check(load_library().lh_qkv_plan(ctypes.byref(desc), ctypes.byref(n)), "lh_qkv_plan")
    return n.value


def lh_qkv_forward(desc, x, w, q, k, v, stream=None):
    _check(load_library().lh_qkv_forward(ctypes.byref(desc), _p(x), _p(w), _p(q), _p(k), _p(v), _stream(stream)),
           "lh_qkv_forward")


def lh_qkv_backward(desc, x, w, dq, dk, dv, dx, dw, ws, stream=None):
    _check(load_library().lh_qkv_backward(ctypes.byref(desc), _p(x), _p(w), _p(dq), _p(dk), _p(dv), _p(dx),
                                          _p(dw), _p(ws), _nbytes(ws), _stream(stream)), "lh_qkv_backward")


# ---------------------------------------------------------------------------
# Convenience: all buffers of one layer call, allocated once.
# ---------------------------------------------------------------------------
class LighthouseLayer:
    """Owns the device buffers for one shape and runs the four calls."""

    def __init__(self, B, H, N, d, p, L, k, dtype=torch.bfloat16, scale=0.0, device="cuda"):
        self.desc = make_desc(B, H, N, d, p, L, k, dtype, scale)
        self.plan = lh_make_plan(self.desc)
        self.dtype = dtype
        P = self.plan
        u8 = dict(dtype=torch.uint8, device=device)
        self.pyr = torch.empty(max(P.pyr_bytes // (2 if dtype == torch.bfloat16 else 4), 1), dtype=dtype,
                               device=device) if P.pyr_bytes else None
        self.sel_ws = torch.empty(max(P.sel_ws_bytes, 256), **u8)
        self.fwd_ws = torch.empty(P.fwd_ws_bytes, **u8)
        self.bwd_ws = torch.empty(P.bwd_ws_bytes, **u8)
        self.gidx = torch.empty((B, H, P.S), dtype=torch.int32, device=device)
        self.gpos = torch.empty((B, H, P.M_total), dtype=torch.int32, device=device)
        self.shape = (B, H, N, d)

    def forward(self, q, k, v, o, stream=None, select=True, norms_from_pyramid=True):
        """norms_from_pyramid=False scores straight from q and k (the token norms
        are then computed again rather than taken from the pyramid buffer)."""
        if self.pyr is not None:
            lh_pyramid(self.desc, q, k, v, self.pyr, stream)
        if select:
            lh_score_topk(self.desc, q, k, self.pyr if norms_from_pyramid else None, self.gidx, self.gpos,
                          self.sel_ws, stream)
        lh_forward(self.desc, q, k, v, self.pyr, self.gidx, self.gpos, o, self.fwd_ws, stream)

    def backward(self, dout, dq, dk, dv, stream=None):
        lh_backward(self.desc, self.gidx, self.gpos, self.fwd_ws, dout, dq, dk, dv, self.bwd_ws, stream)

    # views into the forward state (for tests)
    def fwd_view(self, which, dtype, shape):
        off = self.plan.fwd_off[which]
        n = 1
        for s in shape:
            n *= s
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.fwd_ws[off:off + n * esz].view(dtype).view(shape)

    def bwd_view(self, which, dtype, shape):
        off = self.plan.bwd_off[which]
        n = 1
        for s in shape:
            n *= s
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.bwd_ws[off:off + n * esz].view(dtype).view(shape)
