"""Thin Python binding of the C ABI in include/gdn.h (libgdn_hip.so).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the mixer runs in the library's gfx950 kernels. The
functions keep the ABI's names. There is no fallback: if the library is not
built, or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn_hip.so")

GDN_OK, GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, -1, -2, -3
GDN_FLAG_BAD_SLOT, GDN_FLAG_BAD_NTOK = 0x1, 0x2
EXPORTS = (
    "gdn_abi_version", "gdn_last_error", "gdn_state_pool_bytes", "gdn_state_pool_create",
    "gdn_state_pool_destroy", "gdn_state_pool_state", "gdn_state_pool_conv", "gdn_state_pool_flags",
    "gdn_state_pool_slots", "gdn_state_pool_zero", "gdn_conv_silu_norm", "gdn_decode_step",
    "gdn_decode_step_norm", "gdn_decode_fused", "gdn_verify_window", "gdn_commit", "gdn_commit_window",
    "gdn_gated_rmsnorm",
    "gdn_ab_project", "gdn_split_bf16_bytes", "gdn_pack_bf16_bytes", "gdn_split_bf16", "gdn_pack_bf16",
    "gdn_project_bf16", "gdn_project2_bf16", "gdn_project_workspace_bytes", "gdn_project_multi_bf16",
    "gdn_check_slots", "gdn_project_bf16_noalloc",
)


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class gdn_geom(ctypes.Structure):
    _fields_ = [("h_k", ctypes.c_int32), ("h_v", ctypes.c_int32), ("s", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("gate_silu", ctypes.c_int32), ("scale_after_readout", ctypes.c_int32)]


@dataclass(frozen=True)
class Geom:
    """GDN geometry; the defaults are the pages' model (16 qk heads, 48 value heads,
    sigmoid output gate, 1/sqrt(S) on q).  gate_silu: the earlier model's SiLU gate;
    scale_after_readout: the 1/sqrt(S) on the readout o instead of on q."""
    h_k: int = 16
    h_v: int = 48
    s: int = 128
    d_conv: int = 4
    gate_silu: bool = False
    scale_after_readout: bool = False

    @property
    def channels(self) -> int:
        return (2 * self.h_k + self.h_v) * self.s

    def c(self) -> gdn_geom:
        return gdn_geom(self.h_k, self.h_v, self.s, self.d_conv, int(self.gate_silu), int(self.scale_after_readout))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdn_hip.so. torch is imported first so the library binds to the HIP
    runtime torch already loaded (one runtime, one set of device pointers)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads libamdhip64 into the process)
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    G = ctypes.POINTER(gdn_geom)
    sig = {
        "gdn_abi_version": ([], ctypes.c_int),
        "gdn_last_error": ([], ctypes.c_char_p),
        "gdn_state_pool_bytes": ([G, i64], ctypes.c_size_t),
        "gdn_state_pool_create": ([G, i64, vp, ctypes.c_size_t, ctypes.POINTER(vp)], ctypes.c_int),
        "gdn_state_pool_destroy": ([vp], None),
        "gdn_check_slots": ([vp, i32, i64], ctypes.c_int),
        "gdn_state_pool_state": ([vp], vp),
        "gdn_state_pool_conv": ([vp], vp),
        "gdn_state_pool_flags": ([vp], vp),
        "gdn_state_pool_slots": ([vp], i64),
        "gdn_state_pool_zero": ([vp, vp, i32, vp], ctypes.c_int),
        "gdn_conv_silu_norm": ([vp, vp, vp, i32, i32, vp, vp, f32, vp, vp], ctypes.c_int),
        "gdn_decode_step": ([vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "gdn_decode_step_norm": ([vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp],
                                 ctypes.c_int),
        "gdn_decode_fused": ([vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp], ctypes.c_int),
        "gdn_verify_window": ([vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp],
                              ctypes.c_int),
        "gdn_commit": ([vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "gdn_commit_window": ([vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                               f32, vp, vp, vp], ctypes.c_int),
        "gdn_gated_rmsnorm": ([vp, vp, vp, f32, i64, i32, i32, vp, vp], ctypes.c_int),
        "gdn_ab_project": ([vp, vp, vp, i64, i32, i32, vp, vp, vp], ctypes.c_int),
        "gdn_split_bf16_bytes": ([i64, i32], ctypes.c_int64),
        "gdn_pack_bf16_bytes": ([i32, i32], ctypes.c_int64),
        "gdn_split_bf16": ([vp, i64, i32, vp, vp], ctypes.c_int),
        "gdn_pack_bf16": ([vp, i32, i32, vp, vp], ctypes.c_int),
        "gdn_project2_bf16": ([vp, vp, i64, i32, i32, vp, i32, vp, vp, i64, vp], ctypes.c_int),
        "gdn_project_bf16": ([vp, vp, i64, i32, i32, vp, vp, i64, vp], ctypes.c_int),
        "gdn_project_workspace_bytes": ([i64, i32, i32], ctypes.c_int64),
        "gdn_project_multi_bf16": ([vp, vp, i64, i32, i32, vp, vp, vp, i64, vp], ctypes.c_int),
        "gdn_project_bf16_noalloc": ([vp, vp, i64, i32, i32, vp, vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(rc: int):
    if rc != GDN_OK:
        raise GdnError(rc, load_library().gdn_last_error().decode())


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _f32(t, name: str, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _i32(t, name: str, n: int):
    import torch
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor of {n} elements")
    return t.data_ptr()


# Debug mode: when on, every call that takes a device slot list first copies it to the
# host and runs gdn_check_slots on it (a synchronising copy, so off by default).  Also
# switched on by the environment variable GDN_CHECK_SLOTS=1.
_check_slots_on = os.environ.get("GDN_CHECK_SLOTS", "") not in ("", "0")


def set_slot_checks(on: bool) -> None:
    """Switch the host-side slot validation of every mixer call on or off."""
    global _check_slots_on
    _check_slots_on = bool(on)


def gdn_check_slots(slots, n_slots: int) -> None:
    """Validate a slot list on the host (gdn_check_slots): every entry in [0, n_slots) and
    none repeated.  slots: an int32 torch tensor (any device) or array-like.  Raises
    GdnError (GDN_ERR_ARG) naming the first bad entry."""
    import numpy as np
    try:
        import torch
        if isinstance(slots, torch.Tensor):
            slots = slots.detach().cpu().numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(np.asarray(slots).reshape(-1))
    if a.size and (a.dtype.kind not in "iu" or a.min() < -2 ** 31 or a.max() >= 2 ** 31):
        raise ValueError("slots must hold 32-bit integers")
    a = a.astype(np.int32)
    _check(load_library().gdn_check_slots(a.ctypes.data if a.size else None, int(a.size), int(n_slots)))


def _slots(pool: "StatePool", slots, n: int):
    """The device pointer of a slot list (None: slot b for sequence b), validated on the
    host first when slot checks are on."""
    ptr = _i32(slots, "slots", n)
    if _check_slots_on and slots is not None:
        gdn_check_slots(slots, pool.n_slots)
    return ptr


def gdn_state_pool_bytes(n_slots: int, geom: Geom = Geom()) -> int:
    g = geom.c()
    n = load_library().gdn_state_pool_bytes(ctypes.byref(g), n_slots)
    if n == 0:
        raise GdnError(GDN_ERR_ARG, load_library().gdn_last_error().decode())
    return n


class StatePool:
    """A pool of recurrent-state slots in one torch-owned device buffer.

    .state  float32 [n_slots][h_v][s][s]  (row = key index, column = value index)
    .conv   float32 [n_slots][C][d_conv-1] (raw qkv history, oldest first)
    .flags  int32 [1] device flag word (GDN_FLAG_* bits)
    """

    def __init__(self, n_slots: int, geom: Geom = Geom(), device=None):
        import torch
        L = load_library()
        self.geom = geom
        self.n_slots = n_slots
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        nbytes = gdn_state_pool_bytes(n_slots, geom)
        with torch.cuda.device(self.device):
            self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            h = ctypes.c_void_p()
            g = geom.c()
            _check(L.gdn_state_pool_create(ctypes.byref(g), n_slots, self.buffer.data_ptr(), nbytes,
                                           ctypes.byref(h)))
        self.handle = h
        base = self.buffer.data_ptr()
        st = L.gdn_state_pool_state(h) - base
        cv = L.gdn_state_pool_conv(h) - base
        fl = L.gdn_state_pool_flags(h) - base
        n_st = n_slots * geom.h_v * geom.s * geom.s * 4
        n_cv = n_slots * geom.channels * (geom.d_conv - 1) * 4
        self.state = self.buffer[st:st + n_st].view(torch.float32).view(n_slots, geom.h_v, geom.s, geom.s)
        self.conv = self.buffer[cv:cv + n_cv].view(torch.float32).view(n_slots, geom.channels,
                                                                         geom.d_conv - 1)
        self.flags = self.buffer[fl:fl + 4].view(torch.int32)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.gdn_state_pool_destroy(h)
            self.handle = None

    def zero(self, slots=None):
        gdn_state_pool_zero(self, slots)


def gdn_state_pool_zero(pool: StatePool, slots=None):
    n = 0 if slots is None else slots.numel()
    ptr = _slots(pool, slots, n)
    _check(load_library().gdn_state_pool_zero(pool.handle, ptr, n, _stream(pool.buffer)))


def gdn_conv_silu_norm(pool: StatePool, qkv, conv_w, eps: float, h, slots=None, n_tok=None):
    """qkv, h [B][T][C]; conv_w [C][d_conv]; slots/n_tok int32 [B] or None."""
    B, T = qkv.shape[0], qkv.shape[1]
    C = pool.geom.channels
    args = (_f32(qkv, "qkv", (B, T, C)), _f32(conv_w, "conv_w", (C, pool.geom.d_conv)),
            _f32(h, "h", (B, T, C)))
    _check(load_library().gdn_conv_silu_norm(pool.handle, _slots(pool, slots, B), _i32(n_tok, "n_tok", B),
                                             B, T, args[0], args[1], float(eps), args[2], _stream(qkv)))


def gdn_decode_step(pool: StatePool, h, alpha, beta_logit, dt, ssm_a, o, slots=None, n_tok=None):
    """h [B][T][C]; alpha, beta_logit [B][T][h_v]; dt, ssm_a [h_v]; o [B][T][h_v][s]."""
    g = pool.geom
    B, T = h.shape[0], h.shape[1]
    ptrs = (_f32(h, "h", (B, T, g.channels)), _f32(alpha, "alpha", (B, T, g.h_v)),
            _f32(beta_logit, "beta_logit", (B, T, g.h_v)), _f32(dt, "dt", (g.h_v,)),
            _f32(ssm_a, "ssm_a", (g.h_v,)), _f32(o, "o", (B, T, g.h_v, g.s)))
    _check(load_library().gdn_decode_step(pool.handle, _slots(pool, slots, B), _i32(n_tok, "n_tok", B), B, T,
                                          *ptrs, _stream(h)))


def gdn_decode_step_norm(pool: StatePool, h, alpha, beta_logit, dt, ssm_a, z, norm_w, eps: float, y,
                         o=None, slots=None, n_tok=None):
    """gdn_decode_step with the gated RMSNorm fused in; y [B][T][h_v*s]; o optional."""
    g = pool.geom
    B, T = h.shape[0], h.shape[1]
    ptrs = (_f32(h, "h", (B, T, g.channels)), _f32(alpha, "alpha", (B, T, g.h_v)),
            _f32(beta_logit, "beta_logit", (B, T, g.h_v)), _f32(dt, "dt", (g.h_v,)),
            _f32(ssm_a, "ssm_a", (g.h_v,)), _f32(z, "z", (B, T, g.h_v * g.s)),
            _f32(norm_w, "norm_w", (g.s,)))
    o_ptr = None if o is None else _f32(o, "o", (B, T, g.h_v, g.s))
    _check(load_library().gdn_decode_step_norm(pool.handle, _slots(pool, slots, B), _i32(n_tok, "n_tok", B),
                                               B, T, *ptrs, float(eps), o_ptr,
                                               _f32(y, "y", (B, T, g.h_v * g.s)), _stream(h)))


def gdn_decode_fused(pool: StatePool, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w, eps: float, y,
                     h=None, slots=None, ys: Optional["SplitX"] = None):
    """One decode token of the whole mixer in one launch. qkv [B][C] (or [B][1][C]);
    alpha, beta_logit [B][h_v]; z, y [B][h_v*s]; h optional [B][C]; ys optional: y
    split for the out projection (a SplitX of B rows x h_v*s, as gdn_split_bf16 makes),
    written by the same launch; y may then be None."""
    g = pool.geom
    B = qkv.shape[0]

    def ptr(t, name, n):
        p_ = _f32(t, name)
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} elements, not {t.numel()}")
        return p_
    vdim = g.h_v * g.s
    if ys is not None and ((ys.rows, ys.k) != (B, vdim)
                           or ys.data.numel() * 2 < load_library().gdn_split_bf16_bytes(B, vdim)):
        raise ValueError(f"ys must be the split of a [{B}][{vdim}] activation")
    args = (ptr(qkv, "qkv", B * g.channels), _f32(conv_w, "conv_w", (g.channels, g.d_conv)),
            ptr(alpha, "alpha", B * g.h_v), ptr(beta_logit, "beta_logit", B * g.h_v),
            _f32(dt, "dt", (g.h_v,)), _f32(ssm_a, "ssm_a", (g.h_v,)), ptr(z, "z", B * vdim),
            _f32(norm_w, "norm_w", (g.s,)))
    _check(load_library().gdn_decode_fused(pool.handle, _slots(pool, slots, B), B, *args, float(eps),
                                           None if y is None else ptr(y, "y", B * vdim),
                                           None if h is None else ptr(h, "h", B * g.channels),
                                           None if ys is None else ys.data.data_ptr(), _stream(qkv)))


def gdn_verify_window(pool: StatePool, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w, eps: float, h, y,
                      slots=None, n_tok=None):
    """A speculative window of T tokens from the untouched pool: writes h [B][T][C] and
    y [B][T][h_v*s]; persists nothing."""
    g = pool.geom
    B, T = qkv.shape[0], qkv.shape[1]
    ptrs = (_f32(qkv, "qkv", (B, T, g.channels)), _f32(conv_w, "conv_w", (g.channels, g.d_conv)),
            _f32(alpha, "alpha", (B, T, g.h_v)), _f32(beta_logit, "beta_logit", (B, T, g.h_v)),
            _f32(dt, "dt", (g.h_v,)), _f32(ssm_a, "ssm_a", (g.h_v,)), _f32(z, "z", (B, T, g.h_v * g.s)),
            _f32(norm_w, "norm_w", (g.s,)))
    _check(load_library().gdn_verify_window(pool.handle, _slots(pool, slots, B), _i32(n_tok, "n_tok", B), B, T,
                                            *ptrs, float(eps), _f32(h, "h", (B, T, g.channels)),
                                            _f32(y, "y", (B, T, g.h_v * g.s)), _stream(qkv)))


def gdn_commit(pool: StatePool, qkv, h, alpha, beta_logit, dt, ssm_a, n_keep=None, slots=None):
    """Commit the first n_keep[b] tokens of a window: advance the conv history by their
    raw qkv rows and replay their recurrence from the window's h into the state."""
    g = pool.geom
    B, T = qkv.shape[0], qkv.shape[1]
    ptrs = (_f32(qkv, "qkv", (B, T, g.channels)), _f32(h, "h", (B, T, g.channels)),
            _f32(alpha, "alpha", (B, T, g.h_v)), _f32(beta_logit, "beta_logit", (B, T, g.h_v)),
            _f32(dt, "dt", (g.h_v,)), _f32(ssm_a, "ssm_a", (g.h_v,)))
    _check(load_library().gdn_commit(pool.handle, _slots(pool, slots, B), _i32(n_keep, "n_keep", B), B, T,
                                     *ptrs, _stream(qkv)))


def gdn_commit_window(pool: StatePool, prev, n_keep, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w,
                      eps: float, h, y, slots=None, n_tok=None):
    """One speculative round: gdn_commit of the previous window (prev = its
    (qkv, h, alpha, beta_logit), n_keep of its tokens) then gdn_verify_window of the
    next (qkv, alpha, beta_logit, z -> h, y), with each state tile read once."""
    g = pool.geom
    qkv0, h0, alpha0, beta0 = prev
    B, T0 = qkv0.shape[0], qkv0.shape[1]
    T1 = qkv.shape[1]
    if qkv.shape[0] != B:
        raise ValueError(f"the two windows have {B} and {qkv.shape[0]} sequences")
    p0 = (_f32(qkv0, "qkv0", (B, T0, g.channels)), _f32(h0, "h0", (B, T0, g.channels)),
          _f32(alpha0, "alpha0", (B, T0, g.h_v)), _f32(beta0, "beta_logit0", (B, T0, g.h_v)))
    p1 = (_f32(qkv, "qkv", (B, T1, g.channels)), _f32(conv_w, "conv_w", (g.channels, g.d_conv)),
          _f32(alpha, "alpha", (B, T1, g.h_v)), _f32(beta_logit, "beta_logit", (B, T1, g.h_v)),
          _f32(dt, "dt", (g.h_v,)), _f32(ssm_a, "ssm_a", (g.h_v,)), _f32(z, "z", (B, T1, g.h_v * g.s)),
          _f32(norm_w, "norm_w", (g.s,)))
    _check(load_library().gdn_commit_window(pool.handle, _slots(pool, slots, B), B, _i32(n_keep, "n_keep", B), T0,
                                            *p0, _i32(n_tok, "n_tok", B), T1, *p1, float(eps),
                                            _f32(h, "h", (B, T1, g.channels)), _f32(y, "y", (B, T1, g.h_v * g.s)),
                                            _stream(qkv)))


def gdn_gated_rmsnorm(o, z, w, eps: float, y, gate_silu: bool = False):
    """o, z, y: any contiguous float32 layout whose last axis is s = 128 rows; w [s].
    gate_silu: z * sigmoid(z) as the gate instead of sigmoid(z)."""
    s = w.shape[-1]
    rows = o.numel() // s
    ptrs = (_f32(o, "o"), _f32(z, "z"), _f32(w, "w", (s,)), _f32(y, "y"))
    if z.numel() != o.numel() or y.numel() != o.numel():
        raise ValueError("o, z and y must hold the same number of elements")
    _check(load_library().gdn_gated_rmsnorm(ptrs[0], ptrs[1], ptrs[2], float(eps), rows, s, int(bool(gate_silu)),
                                            ptrs[3], _stream(o)))


def gdn_mixer(pool: StatePool, qkv, alpha, beta_logit, z, conv_w, dt, ssm_a, norm_w, eps: float,
              h, o, y, slots=None, n_tok=None, fused: bool = False):
    """One pass of the whole mixer in the layer's order: three ABI calls, or two with
    the gated RMSNorm fused into the recurrence (o is then optional)."""
    gdn_conv_silu_norm(pool, qkv, conv_w, eps, h, slots, n_tok)
    if fused:
        gdn_decode_step_norm(pool, h, alpha, beta_logit, dt, ssm_a, z, norm_w, eps, y, o, slots, n_tok)
    else:
        gdn_decode_step(pool, h, alpha, beta_logit, dt, ssm_a, o, slots, n_tok)
        gdn_gated_rmsnorm(o, z, norm_w, eps, y, gate_silu=pool.geom.gate_silu)


def gdn_ab_project(x, w_alpha, w_beta, alpha, beta_logit):
    """x [.., n_embd] fp32; w_alpha, w_beta [h_v][n_embd] bf16 bits (torch.int16 or
    torch.uint16 tensors); alpha, beta_logit [.., h_v] fp32 outputs."""
    import torch
    n_embd = x.shape[-1]
    rows = x.numel() // n_embd
    h_v = w_alpha.shape[0]
    for t, name in ((w_alpha, "w_alpha"), (w_beta, "w_beta")):
        if t.dtype not in (torch.int16, torch.uint16) or not t.is_cuda or not t.is_contiguous() \
                or tuple(t.shape) != (h_v, n_embd):
            raise ValueError(f"{name} must be a contiguous 16-bit CUDA tensor of shape {(h_v, n_embd)}")
    for t, name in ((alpha, "alpha"), (beta_logit, "beta_logit")):
        if t.numel() != rows * h_v:
            raise ValueError(f"{name} must hold {rows * h_v} elements")
    _check(load_library().gdn_ab_project(_f32(x, "x"), w_alpha.data_ptr(), w_beta.data_ptr(), rows, n_embd, h_v,
                                         _f32(alpha, "alpha"), _f32(beta_logit, "beta_logit"), _stream(x)))


def _bits16(t, name: str, shape):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.int16, torch.uint16, torch.bfloat16) \
            or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous 16-bit CUDA tensor of shape {tuple(shape)}")
    return t.data_ptr()


class SplitX:
    """Split fp32 activations [rows][k] in the library's tiled layout (gdn_split_bf16)."""

    def __init__(self, data, rows: int, k: int):
        self.data, self.rows, self.k = data, rows, k


class PackedW:
    """A bf16 weight matrix [n][k] rearranged by gdn_pack_bf16."""

    def __init__(self, data, n: int, k: int):
        self.data, self.n, self.k = data, n, k


def gdn_split_bf16(x, xs: Optional[SplitX] = None) -> SplitX:
    """x [.., k] fp32 -> its bf16 (hi, lo) split in the tiled layout."""
    import torch
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    nbytes = load_library().gdn_split_bf16_bytes(rows, k)
    if nbytes < 0:
        raise ValueError(f"cannot split [{rows}][{k}]: k must be a positive multiple of 8")
    if xs is None:
        xs = SplitX(torch.empty(nbytes // 2, dtype=torch.int16, device=x.device), rows, k)
    elif (xs.rows, xs.k) != (rows, k) or xs.data.numel() * 2 < nbytes:
        raise ValueError("xs was made for another shape")
    _check(load_library().gdn_split_bf16(_f32(x, "x"), rows, k, xs.data.data_ptr(), _stream(x)))
    return xs


def gdn_pack_bf16(w) -> PackedW:
    """w [n][k] bf16 bits (int16 / uint16 / bfloat16 tensor) -> packed weights."""
    import torch
    n, k = w.shape
    nbytes = load_library().gdn_pack_bf16_bytes(n, k)
    if nbytes < 0:
        raise ValueError(f"cannot pack [{n}][{k}]: k must be a positive multiple of 8")
    wp = torch.empty(nbytes // 2, dtype=torch.int16, device=w.device)
    _check(load_library().gdn_pack_bf16(_bits16(w, "w", (n, k)), n, k, wp.data_ptr(), _stream(w)))
    return PackedW(wp, n, k)


def gdn_project_workspace_bytes(rows: int, k: int, n: int) -> int:
    """Device workspace the product rows x k x n needs (0 for most shapes)."""
    nbytes = load_library().gdn_project_workspace_bytes(rows, k, n)
    if nbytes < 0:
        raise ValueError(f"bad projection shape rows={rows} k={k} n={n}")
    return nbytes


def _workspace(rows, k, n, device, workspace):
    """(pointer, bytes, keep-alive) of the projection workspace: the caller's tensor, or
    a fresh one from torch's allocator when the shape needs one."""
    import torch
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    nbytes = gdn_project_workspace_bytes(rows, k, n)
    if nbytes == 0:
        return None, 0, None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws.data_ptr(), nbytes, ws


def gdn_project_bf16(xs: SplitX, wp: PackedW, out=None, workspace=None):
    """out [rows][n] fp32 = x @ w^T from the split activations and the packed weights.
    workspace: optional device tensor of gdn_project_workspace_bytes(rows, k, n) bytes
    (allocated here when the shape needs one and none is given)."""
    import torch
    if xs.k != wp.k:
        raise ValueError(f"x has k={xs.k}, w has k={wp.k}")
    if out is None:
        out = torch.empty(xs.rows, wp.n, dtype=torch.float32, device=xs.data.device)
    if out.numel() != xs.rows * wp.n:
        raise ValueError(f"out must hold {xs.rows * wp.n} elements")
    ws, ws_bytes, _keep = _workspace(xs.rows, xs.k, wp.n, xs.data.device, workspace)
    _check(load_library().gdn_project_bf16(xs.data.data_ptr(), wp.data.data_ptr(), xs.rows, xs.k, wp.n,
                                           _f32(out, "out"), ws, ws_bytes, _stream(xs.data)))
    return out


def gdn_project_bf16_noalloc(xs: SplitX, wp: PackedW, out):
    """gdn_project_bf16 without a workspace or any allocation: a k-split launch keeps its
    partial blocks in the library's own per-GPU scratch buffer (GDN_PROJECT_SCRATCH_BYTES;
    larger needs raise GdnError).  out [rows][n] fp32 must be given."""
    if xs.k != wp.k:
        raise ValueError(f"x has k={xs.k}, w has k={wp.k}")
    if out is None or out.numel() != xs.rows * wp.n:
        raise ValueError(f"out must be given and hold {xs.rows * wp.n} elements")
    _check(load_library().gdn_project_bf16_noalloc(xs.data.data_ptr(), wp.data.data_ptr(), xs.rows, xs.k, wp.n,
                                                   _f32(out, "out"), _stream(xs.data)))
    return out


def gdn_project2_bf16(xs: SplitX, wp: PackedW, n1: int, out1=None, out2=None, workspace=None):
    """Two projections of the same activations in one launch: wp packs the
    concatenation [w1; w2] (n1 + n2 rows); returns (out1 [rows][n1], out2 [rows][n2])."""
    import torch
    n2 = wp.n - n1
    if xs.k != wp.k or not 0 < n1 < wp.n:
        raise ValueError(f"x has k={xs.k}, w has k={wp.k} and {wp.n} rows, n1={n1}")
    dev = xs.data.device
    out1 = torch.empty(xs.rows, n1, device=dev) if out1 is None else out1
    out2 = torch.empty(xs.rows, n2, device=dev) if out2 is None else out2
    if out1.numel() != xs.rows * n1 or out2.numel() != xs.rows * n2:
        raise ValueError("out1 / out2 have the wrong size")
    ws, ws_bytes, _keep = _workspace(xs.rows, xs.k, wp.n, dev, workspace)
    _check(load_library().gdn_project2_bf16(xs.data.data_ptr(), wp.data.data_ptr(), xs.rows, xs.k, n1,
                                            _f32(out1, "out1"), n2, _f32(out2, "out2"), ws, ws_bytes,
                                            _stream(xs.data)))
    return out1, out2


def gdn_project_multi_bf16(xs: SplitX, wp: PackedW, cols, outs=None, workspace=None):
    """Up to 4 projections of the same activations in one launch: wp packs the weight
    matrices stacked row-wise, cols[o] rows each; returns the outputs [rows][cols[o]]."""
    import torch
    cols = [int(c) for c in cols]
    if xs.k != wp.k or sum(cols) != wp.n or not 1 <= len(cols) <= 4:
        raise ValueError(f"x has k={xs.k}, w has k={wp.k} and {wp.n} rows, cols={cols}")
    dev = xs.data.device
    outs = [torch.empty(xs.rows, c, device=dev) for c in cols] if outs is None else list(outs)
    if len(outs) != len(cols) or any(o.numel() != xs.rows * c for o, c in zip(outs, cols)):
        raise ValueError("outs do not match cols")
    ptrs = (ctypes.c_void_p * len(outs))(*[_f32(o, f"outs[{i}]") for i, o in enumerate(outs)])
    col_arr = (ctypes.c_int32 * len(cols))(*cols)
    ws, ws_bytes, _keep = _workspace(xs.rows, xs.k, wp.n, dev, workspace)
    _check(load_library().gdn_project_multi_bf16(xs.data.data_ptr(), wp.data.data_ptr(), xs.rows, xs.k, len(cols),
                                                 col_arr, ptrs, ws, ws_bytes, _stream(xs.data)))
    return outs


def gdn_project(x, wp: PackedW, out=None):
    """out [.., n] = x @ w^T for fp32 x [.., k] through a split and the product."""
    res = gdn_project_bf16(gdn_split_bf16(x), wp, out)
    return res.view(*x.shape[:-1], wp.n) if out is None else res
