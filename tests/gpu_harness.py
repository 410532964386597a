"""Helpers for the GPU parity tests: move a seeded workload onto the device, run the
HIP path through the C ABI, and compare against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

from parity import assert_close, assert_exact, assert_tokens, tol  # noqa: F401  (the tests import them from here too)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class GpuMixer:
    """The workload's tensors on the device plus a state pool filled from it."""

    def __init__(self, wl, pool=None):
        import torch
        import gated_deltanet_mixer_gdn_amd as G
        self.G = G
        self.wl = wl
        g = wl.geom
        self.geom = G.Geom(g.h_k, g.h_v, g.s, g.d_conv, gate_silu=getattr(wl, "gate_silu", False),
                           scale_after_readout=getattr(wl, "scale_after_readout", False))
        if pool is None:
            pool = G.StatePool(wl.n_slots, self.geom)
            pool.state.copy_(dev(wl.state))
            pool.conv.copy_(dev(wl.conv_state))
            pool.flags.zero_()
        self.pool = pool
        self.conv_w = dev(wl.conv_w)
        self.dt = dev(wl.dt)
        self.ssm_a = dev(wl.ssm_a)
        self.norm_w = dev(wl.norm_w)
        self.qkv = dev(wl.qkv)
        self.alpha = dev(wl.alpha)
        self.beta_logit = dev(wl.beta_logit)
        self.z = dev(wl.z)
        self.slots = dev(wl.slots)
        self.n_tok = dev(wl.n_tok) if wl.n_tok is not None else None
        B, T = wl.B, wl.T
        self.h = torch.empty(B, T, g.channels, device="cuda")
        self.o = torch.empty(B, T, g.h_v, g.s, device="cuda")
        self.y = torch.empty(B, T, g.h_v * g.s, device="cuda")

    def run(self, t0: int = 0, t1=None, slots=None, n_tok="default", fused=False):
        """One mixer pass over tokens [t0, t1) of every sequence.  fused: False = three
        calls; True or "norm" = conv + recurrence with the norm fused in; "one" = the
        single-launch decode (one token, every sequence)."""
        import torch
        t1 = self.wl.T if t1 is None else t1
        sl = lambda x: x[:, t0:t1].contiguous()
        qkv, alpha, bl, z = sl(self.qkv), sl(self.alpha), sl(self.beta_logit), sl(self.z)
        B, T = qkv.shape[0], qkv.shape[1]
        g = self.geom
        h = torch.empty(B, T, g.channels, device="cuda")
        o = torch.empty(B, T, g.h_v, g.s, device="cuda")
        y = torch.empty(B, T, g.h_v * g.s, device="cuda")
        slots = self.slots if slots is None else slots
        n_tok = self.n_tok if isinstance(n_tok, str) else n_tok
        if fused == "one":
            assert T == 1 and n_tok is None, "the single-launch decode takes one token per sequence"
            o.zero_()
            self.G.gdn_decode_fused(self.pool, qkv, self.conv_w, alpha, bl, self.dt, self.ssm_a, z, self.norm_w,
                                    self.wl.eps, y, h, slots)
        else:
            self.G.gdn_mixer(self.pool, qkv, alpha, bl, z, self.conv_w, self.dt, self.ssm_a, self.norm_w,
                             self.wl.eps, h, o, y, slots, n_tok, fused=bool(fused))
        self.h[:, t0:t1] = h
        self.o[:, t0:t1] = o
        self.y[:, t0:t1] = y
        return h, o, y

    def slot_state(self, b: int):
        return self.pool.state[int(self.wl.slots[b])].cpu().numpy()

    def slot_conv(self, b: int):
        return self.pool.conv[int(self.wl.slots[b])].cpu().numpy()
