"""fp64 CPU oracle of the Gated DeltaNet decode mixer (ctypes front end).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg use this module; the product path never imports,
links or runs it. It shares no code with the HIP library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, no
fusion or reordering beyond the op order of the GDN layer on the
``include/strata/core/layer.hpp`` page). This file only marshals numpy arrays,
gathers per-sequence state by slot index and runs independent sequences on a
thread pool (ctypes releases the GIL during each C call).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        # GDN_ORACLE_LIB: another build of this source to load instead (the mutation
        # tests load copies with one mistake planted, to show the pins catch it)
        path = os.environ.get("GDN_ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB_PATH):
                build()
            path = _LIB_PATH
        L = ctypes.CDLL(path)
        i, i64, d = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.gdn_oracle_sigmoid.argtypes = [d]
        L.gdn_oracle_sigmoid.restype = d
        L.gdn_oracle_softplus.argtypes = [d]
        L.gdn_oracle_softplus.restype = d
        L.gdn_oracle_conv_silu_norm.argtypes = [i, i, i, i, i, _D, _D, d, _D, _D, i]
        L.gdn_oracle_beta_gate.argtypes = [i, i, _D, _D, _D, _D, _D, _D]
        L.gdn_oracle_delta_rule.argtypes = [i, i, i, i, _D, _D, _D, _D, _D, d]
        L.gdn_oracle_gated_rmsnorm.argtypes = [i64, i, _D, _D, _D, d, _D, i]
        L.gdn_oracle_mixer.argtypes = [i, i, i, i, i] + [_D] * 8 + [d] + [_D] * 6 + [i, i]
        U16 = ctypes.POINTER(ctypes.c_uint16)
        L.gdn_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.gdn_oracle_bf16_value.restype = d
        L.gdn_oracle_ab_project.argtypes = [i64, i, i, _D, U16, U16, _D, _D]
        L.gdn_oracle_ab_project.restype = i
        L.gdn_oracle_project.argtypes = [i64, i, i, _D, U16, _D]
        L.gdn_oracle_project.restype = i
        for f in ("conv_silu_norm", "beta_gate", "delta_rule", "gated_rmsnorm", "mixer"):
            getattr(L, "gdn_oracle_" + f).restype = i
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_D)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def sigmoid(x: float) -> float:
    return lib().gdn_oracle_sigmoid(float(x))


def softplus(x: float) -> float:
    return lib().gdn_oracle_softplus(float(x))


def conv_silu_norm(geom, qkv, conv_w, eps, conv_state, scale_q: bool = True):
    """qkv [T][C], conv_w [C][d], conv_state [C][d-1] -> (h [T][C], new conv_state).
    scale_q=False leaves q unit-norm (the 1/sqrt(S) then goes on the readout)."""
    qkv, conv_w = _f64(qkv), _f64(conv_w)
    cs = _f64(conv_state).copy()
    T = qkv.shape[0]
    h = np.zeros_like(qkv)
    _check(lib().gdn_oracle_conv_silu_norm(geom.h_k, geom.h_v, geom.s, geom.d_conv, T, _p(qkv),
                                           _p(conv_w), float(eps), _p(cs), _p(h), int(bool(scale_q))),
           "conv_silu_norm")
    return h, cs


def beta_gate(alpha, beta_logit, dt, ssm_a):
    """alpha, beta_logit [T][h_v] -> (beta, gate) [T][h_v]."""
    alpha, beta_logit, dt, ssm_a = map(_f64, (alpha, beta_logit, dt, ssm_a))
    T, h_v = alpha.shape
    beta = np.zeros_like(alpha)
    gate = np.zeros_like(alpha)
    _check(lib().gdn_oracle_beta_gate(h_v, T, _p(alpha), _p(beta_logit), _p(dt), _p(ssm_a),
                                      _p(beta), _p(gate)), "beta_gate")
    return beta, gate


def delta_rule(geom, h, beta, gate, state, o_scale: float = 1.0):
    """h [T][C], beta/gate [T][h_v], state [h_v][s][s] -> (o [T][h_v][s], new state);
    o is multiplied by o_scale after the readout."""
    h, beta, gate = _f64(h), _f64(beta), _f64(gate)
    st = _f64(state).copy()
    T = h.shape[0]
    o = np.zeros((T, geom.h_v, geom.s))
    _check(lib().gdn_oracle_delta_rule(geom.h_k, geom.h_v, geom.s, T, _p(h), _p(beta), _p(gate),
                                       _p(st), _p(o), float(o_scale)), "delta_rule")
    return o, st


def gated_rmsnorm(o, z, w, eps, gate_silu: bool = False):
    """o, z [rows][s], w [s] -> y [rows][s]; gate_silu: z * sigmoid(z) instead of sigmoid(z)."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    s = o.shape[-1]
    rows = o.size // s
    y = np.zeros_like(o)
    _check(lib().gdn_oracle_gated_rmsnorm(rows, s, _p(o), _p(z), _p(w), float(eps), _p(y), int(bool(gate_silu))),
           "gated_rmsnorm")
    return y


def mixer(geom, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w, eps, conv_state, state,
          gate_silu: bool = False, scale_after_readout: bool = False):
    """Whole mixer for one sequence over T tokens; returns dict(h, o, y, state, conv_state).
    gate_silu / scale_after_readout select the two variants (SiLU output gate; 1/sqrt(S)
    on the readout instead of on q)."""
    qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w = map(
        _f64, (qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w))
    cs = _f64(conv_state).copy()
    st = _f64(state).copy()
    T = qkv.shape[0]
    h = np.zeros_like(qkv)
    o = np.zeros((T, geom.h_v, geom.s))
    y = np.zeros((T, geom.h_v * geom.s))
    scratch = np.zeros(2 * geom.h_v)
    _check(lib().gdn_oracle_mixer(geom.h_k, geom.h_v, geom.s, geom.d_conv, T, _p(qkv), _p(conv_w),
                                  _p(alpha), _p(beta_logit), _p(dt), _p(ssm_a), _p(z), _p(norm_w),
                                  float(eps), _p(cs), _p(st), _p(h), _p(o), _p(y), _p(scratch),
                                  int(bool(gate_silu)), int(bool(scale_after_readout))),
           "mixer")
    return {"h": h, "o": o, "y": y, "state": st, "conv_state": cs}


def bf16_value(bits: int) -> float:
    return lib().gdn_oracle_bf16_value(int(bits))


def ab_project(x, w_alpha_bits, w_beta_bits):
    """x [..][n_embd]; w_* [h_v][n_embd] uint16 bf16 bits -> (alpha, beta_logit) [..][h_v]."""
    x = _f64(x)
    shape = x.shape[:-1]
    n_embd = x.shape[-1]
    x2 = x.reshape(-1, n_embd)
    wa = np.ascontiguousarray(w_alpha_bits, dtype=np.uint16)
    wb = np.ascontiguousarray(w_beta_bits, dtype=np.uint16)
    h_v = wa.shape[0]
    alpha = np.zeros((x2.shape[0], h_v))
    beta = np.zeros((x2.shape[0], h_v))
    U16 = ctypes.POINTER(ctypes.c_uint16)
    _check(lib().gdn_oracle_ab_project(x2.shape[0], n_embd, h_v, _p(x2), wa.ctypes.data_as(U16),
                                       wb.ctypes.data_as(U16), _p(alpha), _p(beta)), "ab_project")
    return alpha.reshape(*shape, h_v), beta.reshape(*shape, h_v)


def project(x, w_bits, threads: Optional[int] = None):
    """x [..][k]; w [n][k] uint16 bf16 bits -> out [..][n] (rows split over threads)."""
    x = _f64(x)
    shape = x.shape[:-1]
    k = x.shape[-1]
    x2 = x.reshape(-1, k)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    n = w.shape[0]
    out = np.zeros((x2.shape[0], n))
    U16 = ctypes.POINTER(ctypes.c_uint16)
    rows = x2.shape[0]
    threads = max(1, min(threads or (os.cpu_count() or 1), rows))
    bounds = np.linspace(0, rows, threads + 1).astype(int)

    def part(i):
        a, b = bounds[i], bounds[i + 1]
        if b > a:
            xs, os_ = x2[a:b], out[a:b]
            _check(lib().gdn_oracle_project(b - a, k, n, _p(xs), w.ctypes.data_as(U16), _p(os_)), "project")
    lib()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(part, range(threads)))
    return out.reshape(*shape, n)


def run_sequence(wl, b: int, t0: int = 0, t1: Optional[int] = None, state=None, conv_state=None):
    """Advance sequence b of a workload over its tokens [t0, t1) (clipped to its token count),
    in the workload's model variant (wl.gate_silu, wl.scale_after_readout)."""
    n = wl.tokens_of(b)
    t1 = n if t1 is None else min(t1, n)
    slot = int(wl.slots[b])
    st0 = wl.state[slot] if state is None else state
    cs0 = wl.conv_state[slot] if conv_state is None else conv_state
    return mixer(wl.geom, wl.qkv[b, t0:t1], wl.conv_w, wl.alpha[b, t0:t1], wl.beta_logit[b, t0:t1],
                 wl.dt, wl.ssm_a, wl.z[b, t0:t1], wl.norm_w, wl.eps, cs0, st0,
                 gate_silu=getattr(wl, "gate_silu", False),
                 scale_after_readout=getattr(wl, "scale_after_readout", False))


def run_workload(wl, seqs: Optional[Iterable[int]] = None, threads: Optional[int] = None):
    """Run the oracle for the chosen sequences (default: all); list of per-sequence dicts."""
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    threads = threads or min(len(seqs), os.cpu_count() or 1) or 1
    lib()
    if threads <= 1:
        return [run_sequence(wl, b) for b in seqs]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda b: run_sequence(wl, b), seqs))
