"""Seeded synthetic inputs for the Gated DeltaNet decode mixer.

This module is the only code shared by the fp64 oracle's tests and the HIP path.
It draws random numbers and lays them out; it performs none of the mixer's
arithmetic (no convolution, activation, normalisation or recurrence).

Shapes follow the decode mixer of the GDN layer as composed on the
``src/core/layer.cpp`` page (``gdn_layer``, steps 3-7) and the buffer list on the
``include/strata/core/layer.hpp`` page (``GdnBuffers``):

* qkv / h        [B][T][C]        with C = 2*h_k*S + h_v*S (q | k | v runs)
* alpha, beta    [B][T][h_v]      (beta given as logits: the sigmoid is the method's)
* z, y           [B][T][h_v*S]
* conv_w         [C][d_conv]      (tap d_conv-1 multiplies the current input)
* dt, ssm_a      [h_v]
* norm_w         [S]              (shared by all value heads)
* state pool     [n_slots][h_v][S][S]   (row = key index, column = value index)
* conv pool      [n_slots][C][d_conv-1] (oldest first, raw qkv values)

Value recipes (N(mu, sigma) means mean mu and standard deviation sigma):
conv_w ~ N(0, 0.5); dt ~ N(0, 0.5); ssm_a = -exp(U(-1, 1)); norm_w ~ 1 + N(0, 0.1);
per-token qkv, alpha, beta logits and z ~ N(0, 1). All values are float32.
Draw order: conv_w, dt, ssm_a, norm_w, state, conv state, (slot list, token
counts), then per token t: qkv, alpha, beta logits, z.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# The GDN geometry of the pages' model: 16 qk heads, 48 value heads, 128-wide heads,
# a 4-tap short convolution ("ModelGeometry" GDN fields used by gdn_layer).
H_K, H_V, S, D_CONV = 16, 48, 128, 4


@dataclass
class Geom:
    h_k: int = H_K
    h_v: int = H_V
    s: int = S
    d_conv: int = D_CONV

    @property
    def channels(self) -> int:
        return 2 * self.h_k * self.s + self.h_v * self.s

    @property
    def value_dim(self) -> int:
        return self.h_v * self.s


@dataclass
class Workload:
    name: str
    geom: Geom
    B: int
    T: int
    n_slots: int
    conv_w: np.ndarray
    dt: np.ndarray
    ssm_a: np.ndarray
    norm_w: np.ndarray
    state: np.ndarray          # [n_slots][h_v][s][s]
    conv_state: np.ndarray     # [n_slots][C][d_conv-1]
    slots: np.ndarray          # int32 [B], unique
    n_tok: Optional[np.ndarray]  # int32 [B] in [0, T], or None = every sequence takes T tokens
    qkv: np.ndarray            # [B][T][C]
    alpha: np.ndarray          # [B][T][h_v]
    beta_logit: np.ndarray     # [B][T][h_v]
    z: np.ndarray              # [B][T][h_v*s]
    eps: float = 1e-6
    meta: dict = field(default_factory=dict)
    # model variants: the SiLU output gate z * sigmoid(z), and the 1/sqrt(S) on the
    # readout o instead of on q (both off = the pages' model)
    gate_silu: bool = False
    scale_after_readout: bool = False

    def tokens_of(self, b: int) -> int:
        return self.T if self.n_tok is None else int(self.n_tok[b])


def _normal(rng, shape, std=1.0, mean=0.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make(name: str, B: int, T: int, seed: int, *, geom: Optional[Geom] = None,
         n_slots: Optional[int] = None, state_std: float = 0.0, conv_std: float = 0.0,
         slot_choice: str = "identity", ragged_max: Optional[int] = None) -> Workload:
    """Draw one workload.

    state_std / conv_std = 0 means a zero-initialised state / conv state.
    slot_choice: "identity" uses slots 0..B-1; "random" draws B unique slots
    from the pool. ragged_max: when set, draws a per-sequence token count
    U{1..ragged_max} (T is then ragged_max).
    """
    g = geom or Geom()
    C = g.channels
    n_slots = B if n_slots is None else n_slots
    if n_slots < B:
        raise ValueError("pool smaller than the batch")
    rng = np.random.default_rng(seed)
    conv_w = _normal(rng, (C, g.d_conv), 0.5)
    dt = _normal(rng, (g.h_v,), 0.5)
    ssm_a = (-np.exp(rng.uniform(-1.0, 1.0, g.h_v))).astype(np.float32)
    norm_w = _normal(rng, (g.s,), 0.1, 1.0)
    sshape = (n_slots, g.h_v, g.s, g.s)
    state = _normal(rng, sshape, state_std) if state_std else np.zeros(sshape, np.float32)
    cshape = (n_slots, C, g.d_conv - 1)
    conv_state = _normal(rng, cshape, conv_std) if conv_std else np.zeros(cshape, np.float32)
    if slot_choice == "random":
        slots = rng.choice(n_slots, B, replace=False).astype(np.int32)
    else:
        slots = np.arange(B, dtype=np.int32)
    n_tok = None
    if ragged_max is not None:
        n_tok = rng.integers(1, ragged_max + 1, B).astype(np.int32)
        T = ragged_max
    qkv = np.empty((B, T, C), np.float32)
    alpha = np.empty((B, T, g.h_v), np.float32)
    beta_logit = np.empty((B, T, g.h_v), np.float32)
    z = np.empty((B, T, g.value_dim), np.float32)
    for t in range(T):
        qkv[:, t] = _normal(rng, (B, C))
        alpha[:, t] = _normal(rng, (B, g.h_v))
        beta_logit[:, t] = _normal(rng, (B, g.h_v))
        z[:, t] = _normal(rng, (B, g.value_dim))
    return Workload(name, g, B, T, n_slots, conv_w, dt, ssm_a, norm_w, state, conv_state,
                    slots, n_tok, qkv, alpha, beta_logit, z)


# The five synthetic workloads of the decode mixer, seeds 1-5 in this order.
def tiny(seed: int = 1) -> Workload:
    """One sequence, 8 sequential decode steps (one token per call), zero state."""
    return make("tiny_b1_t8", 1, 8, seed)


def decode_b64(seed: int = 2) -> Workload:
    """One decode step for 64 sequences; state ~ N(0, 0.02), conv state ~ N(0, 1)."""
    return make("decode_b64", 64, 1, seed, state_std=0.02, conv_std=1.0)


def decode_b256(seed: int = 3) -> Workload:
    """One decode step for 256 sequences: a 768 MiB fp32 state streamed from HBM."""
    return make("decode_b256", 256, 1, seed, state_std=0.02, conv_std=1.0)


def prefill_b16_t512(seed: int = 4) -> Workload:
    """16 sequences x 512 sequential tokens from a zero state."""
    return make("prefill_b16_t512", 16, 512, seed)


def ragged_pool(seed: int = 5, n_slots: int = 2048, B: int = 1024, max_steps: int = 8) -> Workload:
    """2048-slot pool, 1024 active sequences at random unique slots, U{1..8} tokens each."""
    return make("ragged_pool2048_b1024", B, max_steps, seed, n_slots=n_slots, state_std=0.02,
                conv_std=1.0, slot_choice="random", ragged_max=max_steps)


CONFIGS = {
    "tiny": tiny,
    "b64": decode_b64,
    "b256": decode_b256,
    "prefill": prefill_b16_t512,
    "ragged": ragged_pool,
}


# ------------------------------------------------------------------ the alpha / beta projections
N_EMBD = 2560   # hidden size of the pages' model (each of the 48 projection rows walks 2,560 elements)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (input generation only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclass
class AbWorkload:
    x: np.ndarray          # [B][T][n_embd] fp32 hidden states
    w_alpha: np.ndarray    # [h_v][n_embd] bf16 bits
    w_beta: np.ndarray     # [h_v][n_embd] bf16 bits


def make_ab(B: int, T: int, seed: int, n_embd: int = N_EMBD, h_v: int = H_V) -> AbWorkload:
    """x ~ N(0, 1); weights ~ N(0, 1/sqrt(n_embd)) rounded to bf16."""
    rng = np.random.default_rng(seed)
    std = 1.0 / np.sqrt(n_embd)
    w_alpha = bf16_bits(_normal(rng, (h_v, n_embd), std))
    w_beta = bf16_bits(_normal(rng, (h_v, n_embd), std))
    x = _normal(rng, (B, T, n_embd))
    return AbWorkload(x, w_alpha, w_beta)


# ------------------------------------------------------------------ the qkv / z / out projections
# (rows, k, n) of the three projections around the mixer at the pages' sizes
PROJECTIONS = {"qkv": (N_EMBD, 2 * H_K * S + H_V * S), "z": (N_EMBD, H_V * S), "out": (H_V * S, N_EMBD)}


def make_proj(rows: int, k: int, n: int, seed: int):
    """x [rows][k] ~ N(0, 1); w [n][k] ~ N(0, 1/sqrt(k)) rounded to bf16 bits."""
    rng = np.random.default_rng(seed)
    w = bf16_bits(_normal(rng, (n, k), 1.0 / np.sqrt(k)))
    x = _normal(rng, (rows, k))
    return x, w
