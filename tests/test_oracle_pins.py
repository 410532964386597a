"""Pins of the fp64 oracle against things other than itself.

The pages print no worked GDN example, so the oracle is pinned by: hand-worked
examples (tests/golden/hand_worked.json), closed forms, library routines
(scipy's expit, numpy's logaddexp / correlate / norm / matmul), an independent
dense-matrix formulation of the recurrence, and the invariants the method must
satisfy (unchanged state at beta = 0 and zero gate, exact recall at beta = 1,
unit norms, linearity, head independence, chunking invariance).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import gdn_workloads as W
from gdn_workloads import Geom, make

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))
SMALL = Geom(h_k=2, h_v=6, s=8, d_conv=4)


# ---------------------------------------------------------------- scalars
def test_scalar_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(-math.inf) == 0.0
    assert oracle.sigmoid(math.inf) == 1.0
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    assert oracle.softplus(-math.inf) == 0.0
    assert oracle.softplus(30.0) == pytest.approx(30.0 + math.exp(-30.0), rel=1e-15)
    assert oracle.softplus(800.0) == 800.0
    xs = np.linspace(-40, 40, 161)
    sp = np.array([oracle.softplus(x) for x in xs])
    np.testing.assert_allclose(sp, np.logaddexp(0.0, xs), rtol=1e-13, atol=1e-300)
    sg = np.array([oracle.sigmoid(x) for x in xs])
    np.testing.assert_allclose(sg, expit(xs), rtol=1e-13, atol=1e-300)


# ---------------------------------------------------------------- hand-worked golden values
def test_golden_delta_rule_hand_worked():
    g = GOLD["delta_rule"]
    geom = Geom(**g["geometry"], d_conv=4)
    state = np.array(g["state0"], float)[None]
    for tok in g["tokens"]:
        h = np.array(tok["q"] + tok["k"] + tok["v"], float)[None]
        beta = np.array([[tok["beta"]]])
        gate = np.array([[math.log(tok["decay"])]])
        o, state = oracle.delta_rule(geom, h, beta, gate, state)
        np.testing.assert_allclose(o[0, 0], tok["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(state[0], tok["state"], rtol=0, atol=1e-12)


def test_golden_gated_rmsnorm_hand_worked():
    g = GOLD["gated_rmsnorm"]
    y = oracle.gated_rmsnorm(np.array([g["o"]]), np.array([g["z"]]), np.array(g["w"]), g["eps"])
    np.testing.assert_allclose(y[0], g["y"], rtol=1e-15, atol=0)


def test_golden_conv_silu_norm_hand_worked():
    g = GOLD["conv_silu_norm"]
    geom = Geom(**g["geometry"])
    h, cs = oracle.conv_silu_norm(geom, np.array([g["x"]], float), np.array(g["conv_w"], float),
                                  g["eps"], np.array(g["conv_state0"], float))
    np.testing.assert_array_equal(cs, np.array(g["conv_state1"], float))
    u = np.array(g["u"])
    silu = u * expit(u)
    np.testing.assert_allclose(h[0, 0:2], g["q_tilde"], rtol=0, atol=1e-15)
    k = silu[2:4] / np.linalg.norm(silu[2:4])
    np.testing.assert_allclose(h[0, 2:4], k, rtol=1e-14, atol=0)
    np.testing.assert_allclose(h[0, 4:6], silu[4:6], rtol=1e-14, atol=0)


# ---------------------------------------------------------------- conv + SiLU + L2
def _numpy_conv_silu_norm(geom, qkv, conv_w, conv_state, eps):
    """Independent formulation: correlate the full (history ++ inputs) sequence of each
    channel with its taps, then SiLU by expit, then norms by numpy.linalg.norm."""
    T, C = qkv.shape
    seq = np.concatenate([conv_state.T, qkv], axis=0)          # [(d-1)+T][C]
    u = np.stack([np.correlate(seq[:, c], conv_w[c], mode="valid") for c in range(C)], axis=1)
    h = u * expit(u)
    s, hk = geom.s, geom.h_k
    for part in range(2):
        blk = h[:, part * hk * s:(part + 1) * hk * s].reshape(T, hk, s)
        n = np.sqrt(np.linalg.norm(blk, axis=-1, keepdims=True) ** 2 + eps)
        h[:, part * hk * s:(part + 1) * hk * s] = (blk / n).reshape(T, hk * s)
    h[:, :hk * s] /= math.sqrt(s)
    new_state = seq[-(geom.d_conv - 1):].T
    return h, new_state


@pytest.mark.parametrize("geom,T", [(SMALL, 1), (SMALL, 7), (Geom(), 2)])
def test_conv_silu_norm_matches_numpy_correlate(geom, T):
    wl = make("t", 1, T, seed=11, geom=geom, conv_std=1.0)
    h, cs = oracle.conv_silu_norm(geom, wl.qkv[0], wl.conv_w, wl.eps, wl.conv_state[0])
    h_ref, cs_ref = _numpy_conv_silu_norm(geom, wl.qkv[0].astype(float), wl.conv_w.astype(float),
                                          wl.conv_state[0].astype(float), wl.eps)
    np.testing.assert_allclose(h, h_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cs, cs_ref)


def test_conv_one_hot_current_tap_is_silu():
    geom = SMALL
    wl = make("t", 1, 3, seed=12, geom=geom, conv_std=1.0)
    W = np.zeros_like(wl.conv_w)
    W[:, 3] = 1.0
    h, _ = oracle.conv_silu_norm(geom, wl.qkv[0], W, wl.eps, wl.conv_state[0])
    v0 = 2 * geom.h_k * geom.s
    x = wl.qkv[0].astype(float)
    np.testing.assert_allclose(h[:, v0:], x[:, v0:] * expit(x[:, v0:]), rtol=1e-14, atol=0)


def test_conv_one_hot_oldest_tap_is_a_shift_register():
    geom = SMALL
    T = 6
    wl = make("t", 1, T, seed=13, geom=geom)
    W = np.zeros_like(wl.conv_w)
    W[:, 0] = 1.0
    h, cs = oracle.conv_silu_norm(geom, wl.qkv[0], W, wl.eps, np.zeros_like(wl.conv_state[0]))
    v0 = 2 * geom.h_k * geom.s
    x = wl.qkv[0].astype(float)[:, v0:]
    np.testing.assert_array_equal(h[:3, v0:], 0.0)          # zero history for three tokens
    np.testing.assert_allclose(h[3:, v0:], x[:T - 3] * expit(x[:T - 3]), rtol=1e-14, atol=0)
    np.testing.assert_array_equal(cs, wl.qkv[0].astype(float)[-3:].T)


def test_l2_norms_are_unit_and_q_is_scaled():
    geom = Geom()
    wl = make("t", 1, 2, seed=14, geom=geom, conv_std=1.0)
    h, _ = oracle.conv_silu_norm(geom, wl.qkv[0], wl.conv_w, 0.0, wl.conv_state[0])
    s, hk = geom.s, geom.h_k
    q = h[:, :hk * s].reshape(2, hk, s)
    k = h[:, hk * s:2 * hk * s].reshape(2, hk, s)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1 / math.sqrt(s), rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14)
    # with eps = 1e-6 the norm differs from 1 by about eps / (2 |x|^2)
    h2, _ = oracle.conv_silu_norm(geom, wl.qkv[0], wl.conv_w, 1e-6, wl.conv_state[0])
    k2 = h2[:, hk * s:2 * hk * s].reshape(2, hk, s)
    np.testing.assert_allclose(np.linalg.norm(k2, axis=-1), 1.0, rtol=1e-6)
    # v untouched by any norm: equals silu(conv) exactly as computed with eps = 0
    np.testing.assert_array_equal(h2[:, 2 * hk * s:], h[:, 2 * hk * s:])


def test_l2_norm_of_zero_head_is_zero():
    geom = SMALL
    qkv = np.zeros((1, geom.channels))
    h, _ = oracle.conv_silu_norm(geom, qkv, np.ones((geom.channels, 4)), 1e-6,
                                 np.zeros((geom.channels, 3)))
    np.testing.assert_array_equal(h, 0.0)


# ---------------------------------------------------------------- beta and gate
def test_beta_gate_against_library():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((5, 48)) * 3
    b = rng.standard_normal((5, 48)) * 3
    dt = rng.standard_normal(48)
    A = -np.exp(rng.uniform(-1, 1, 48))
    beta, gate = oracle.beta_gate(a, b, dt, A)
    np.testing.assert_allclose(beta, expit(b), rtol=1e-14)
    np.testing.assert_allclose(gate, np.logaddexp(0.0, a + dt) * A, rtol=1e-13)
    assert (gate <= 0).all()


# ---------------------------------------------------------------- the recurrence
def _dense_recurrence(geom, h, beta, gate, state):
    """Independent dense-matrix form: S_t = (I - b k k^T) e^g S_{t-1} + b k v^T, o_t = S_t^T q."""
    s, hk, hv = geom.s, geom.h_k, geom.h_v
    grp = hv // hk
    S = state.copy()
    T = h.shape[0]
    o = np.zeros((T, hv, s))
    I = np.eye(s)
    for t in range(T):
        for i in range(hv):
            j = i // grp
            q = h[t, j * s:(j + 1) * s]
            k = h[t, hk * s + j * s: hk * s + (j + 1) * s]
            v = h[t, 2 * hk * s + i * s: 2 * hk * s + (i + 1) * s]
            b = beta[t, i]
            S[i] = (I - b * np.outer(k, k)) @ (math.exp(gate[t, i]) * S[i]) + b * np.outer(k, v)
            o[t, i] = S[i].T @ q
    return o, S


def _random_step_inputs(geom, T, seed, unit_k=True):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, geom.channels))
    if unit_k:
        s, hk = geom.s, geom.h_k
        for part in range(2):
            blk = h[:, part * hk * s:(part + 1) * hk * s].reshape(T, hk, s)
            blk /= np.linalg.norm(blk, axis=-1, keepdims=True)
    beta = expit(rng.standard_normal((T, geom.h_v)))
    gate = -rng.uniform(0, 2, (T, geom.h_v))
    state = rng.standard_normal((geom.h_v, geom.s, geom.s)) * 0.1
    return h, beta, gate, state


@pytest.mark.parametrize("s,hk,T", [(4, 1, 1), (4, 2, 8), (8, 1, 5), (8, 2, 8)])
def test_recurrence_matches_dense_matrix_form(s, hk, T):
    geom = Geom(h_k=hk, h_v=3 * hk, s=s)
    h, beta, gate, state = _random_step_inputs(geom, T, seed=100 + s + hk + T)
    o, st = oracle.delta_rule(geom, h, beta, gate, state)
    o_ref, st_ref = _dense_recurrence(geom, h, beta, gate, state)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, st_ref, rtol=1e-12, atol=1e-13)


def test_beta0_gate0_leaves_state_bit_identical():
    geom = Geom()
    h, _, _, state = _random_step_inputs(geom, 2, seed=7)
    beta, gate = oracle.beta_gate(np.zeros((2, 48)), np.full((2, 48), -np.inf), np.zeros(48),
                                  np.zeros(48))
    assert (beta == 0).all() and (gate == 0).all()
    o, st = oracle.delta_rule(geom, h, beta, gate, state)
    np.testing.assert_array_equal(st, state)
    # and the readout is then the plain S^T q of the unchanged state
    q = h[1, :geom.h_k * geom.s].reshape(geom.h_k, geom.s)
    o_ref = np.einsum("irc,ir->ic", state, np.repeat(q, 3, axis=0))
    np.testing.assert_allclose(o[1], o_ref, rtol=1e-13, atol=1e-15)


def test_beta0_is_pure_decay():
    geom = SMALL
    h, _, gate, state = _random_step_inputs(geom, 1, seed=8)
    _, st = oracle.delta_rule(geom, h, np.zeros((1, geom.h_v)), gate, state)
    np.testing.assert_allclose(st, state * np.exp(gate[0])[:, None, None], rtol=1e-15)


def test_beta1_unit_k_recalls_v_exactly():
    geom = Geom()
    h, _, _, state = _random_step_inputs(geom, 1, seed=9)
    beta, gate = oracle.beta_gate(np.zeros((1, 48)), np.full((1, 48), np.inf), np.zeros(48),
                                  np.zeros(48))
    assert (beta == 1).all() and (gate == 0).all()
    _, st = oracle.delta_rule(geom, h, beta, gate, state)
    s, hk = geom.s, geom.h_k
    for i in range(geom.h_v):
        k = h[0, hk * s + (i // 3) * s: hk * s + (i // 3 + 1) * s]
        v = h[0, 2 * hk * s + i * s: 2 * hk * s + (i + 1) * s]
        np.testing.assert_allclose(st[i].T @ k, v, rtol=0, atol=1e-12)


def test_recurrence_is_linear_in_state_and_v():
    geom = SMALL
    h, beta, gate, state = _random_step_inputs(geom, 3, seed=10)
    o1, st1 = oracle.delta_rule(geom, h, beta, gate, state)
    h2 = h.copy()
    h2[:, 2 * geom.h_k * geom.s:] *= 2.0
    o2, st2 = oracle.delta_rule(geom, h2, beta, gate, 2.0 * state)
    np.testing.assert_array_equal(o2, 2.0 * o1)
    np.testing.assert_array_equal(st2, 2.0 * st1)


def test_value_heads_are_independent():
    geom = SMALL
    h, beta, gate, state = _random_step_inputs(geom, 2, seed=11)
    o1, st1 = oracle.delta_rule(geom, h, beta, gate, state)
    i = 4
    h2 = h.copy()
    v0 = 2 * geom.h_k * geom.s
    h2[:, v0 + i * geom.s: v0 + (i + 1) * geom.s] += 1.0
    o2, st2 = oracle.delta_rule(geom, h2, beta, gate, state)
    other = [x for x in range(geom.h_v) if x != i]
    np.testing.assert_array_equal(o2[:, other], o1[:, other])
    np.testing.assert_array_equal(st2[other], st1[other])
    assert not np.allclose(o2[:, i], o1[:, i])


def test_gqa_groups_share_q_and_k():
    """Reading: value head i reads qk head i // (h_v/h_k).  Parity unpinned by the pages;
    this pins only that the oracle implements that reading."""
    geom = SMALL
    h, beta, gate, state = _random_step_inputs(geom, 1, seed=12)
    state[:] = state[0]
    v0 = 2 * geom.h_k * geom.s
    for i in range(geom.h_v):
        h[:, v0 + i * geom.s: v0 + (i + 1) * geom.s] = h[:, v0: v0 + geom.s]
    beta[:] = beta[:, :1]
    gate[:] = gate[:, :1]
    o, _ = oracle.delta_rule(geom, h, beta, gate, state)
    np.testing.assert_array_equal(o[0, 0], o[0, 1])
    np.testing.assert_array_equal(o[0, 0], o[0, 2])
    assert not np.allclose(o[0, 0], o[0, 3])
    # perturbing q of qk head 1 moves value heads 3..5 only
    h2 = h.copy()
    h2[:, geom.s: 2 * geom.s] *= -1.0
    o2, _ = oracle.delta_rule(geom, h2, beta, gate, state)
    np.testing.assert_array_equal(o2[0, :3], o[0, :3])
    np.testing.assert_array_equal(o2[0, 3:], -o[0, 3:])


# ---------------------------------------------------------------- gated RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    s = 128
    rng = np.random.default_rng(4)
    w = 1 + 0.1 * rng.standard_normal(s)
    z = rng.standard_normal((3, s))
    cs = np.array([2.5, -0.01, 1e-4])
    o = cs[:, None] * np.ones((3, s))
    y = oracle.gated_rmsnorm(o, z, w, 1e-6)
    ref = (cs / np.sqrt(cs ** 2 + 1e-6))[:, None] * w[None] * expit(z)
    np.testing.assert_allclose(y, ref, rtol=1e-14)


def test_rmsnorm_scale_invariance_and_sigmoid_gate():
    s = 128
    rng = np.random.default_rng(5)
    o = rng.standard_normal((4, s))
    z = rng.standard_normal((4, s))
    w = rng.standard_normal(s)
    y1 = oracle.gated_rmsnorm(o, z, w, 0.0)
    y2 = oracle.gated_rmsnorm(1000.0 * o, z, w, 0.0)
    np.testing.assert_allclose(y2, y1, rtol=1e-13)
    rms = np.sqrt(np.mean(o ** 2, axis=-1, keepdims=True))
    np.testing.assert_allclose(y1, o / rms * w * expit(z), rtol=1e-13)
    # a SiLU gate instead of the sigmoid would differ by a factor z: make sure it is not that
    assert not np.allclose(y1, o / rms * w * z * expit(z))


# ---------------------------------------------------------------- composition
def test_mixer_equals_stages_in_order():
    geom = SMALL
    wl = make("t", 1, 5, seed=21, geom=geom, state_std=0.05, conv_std=1.0)
    r = oracle.run_sequence(wl, 0)
    h, cs = oracle.conv_silu_norm(geom, wl.qkv[0], wl.conv_w, wl.eps, wl.conv_state[0])
    beta, gate = oracle.beta_gate(wl.alpha[0], wl.beta_logit[0], wl.dt, wl.ssm_a)
    o, st = oracle.delta_rule(geom, h, beta, gate, wl.state[0])
    y = oracle.gated_rmsnorm(o.reshape(-1, geom.s), wl.z[0].reshape(-1, geom.s), wl.norm_w, wl.eps)
    np.testing.assert_array_equal(r["h"], h)
    np.testing.assert_array_equal(r["conv_state"], cs)
    np.testing.assert_array_equal(r["o"], o)
    np.testing.assert_array_equal(r["state"], st)
    np.testing.assert_array_equal(r["y"].reshape(-1, geom.s), y)


def test_mixer_chunked_equals_single_shot():
    """T tokens in one call equal the same tokens fed in several calls (conv history and
    state carried between calls)."""
    geom = SMALL
    wl = make("t", 1, 7, seed=22, geom=geom, state_std=0.05, conv_std=1.0)
    full = oracle.run_sequence(wl, 0)
    st, cs = wl.state[0], wl.conv_state[0]
    outs = []
    for (a, b) in [(0, 1), (1, 3), (3, 7)]:
        r = oracle.run_sequence(wl, 0, a, b, state=st, conv_state=cs)
        st, cs = r["state"], r["conv_state"]
        outs.append(r)
    np.testing.assert_array_equal(np.concatenate([r["o"] for r in outs]), full["o"])
    np.testing.assert_array_equal(np.concatenate([r["y"] for r in outs]), full["y"])
    np.testing.assert_array_equal(st, full["state"])
    np.testing.assert_array_equal(cs, full["conv_state"])


def test_run_workload_gathers_slots():
    geom = SMALL
    wl = make("t", 3, 2, seed=23, geom=geom, n_slots=7, state_std=0.05, conv_std=1.0,
              slot_choice="random")
    res = oracle.run_workload(wl, threads=2)
    for b in range(3):
        r = oracle.mixer(geom, wl.qkv[b], wl.conv_w, wl.alpha[b], wl.beta_logit[b], wl.dt, wl.ssm_a,
                         wl.z[b], wl.norm_w, wl.eps, wl.conv_state[wl.slots[b]], wl.state[wl.slots[b]])
        np.testing.assert_array_equal(res[b]["state"], r["state"])
        np.testing.assert_array_equal(res[b]["y"], r["y"])


def test_oracle_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.delta_rule(Geom(h_k=2, h_v=5, s=4), np.zeros((1, 2 * 2 * 4 + 5 * 4)), np.zeros((1, 5)),
                          np.zeros((1, 5)), np.zeros((5, 4, 4)))


# ---------------------------------------------------------------- alpha / beta projections
def test_bf16_values_of_known_bit_patterns():
    # sign | 8 exponent bits | 7 mantissa bits, bias 127 (the upper half of a binary32)
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC040) == -3.0
    assert oracle.bf16_value(0x4049) == 3.140625
    assert oracle.bf16_value(0x3E80) == 0.25
    assert oracle.bf16_value(0x0000) == 0.0
    assert math.copysign(1.0, oracle.bf16_value(0x8000)) == -1.0
    assert oracle.bf16_value(0x7F80) == math.inf
    assert oracle.bf16_value(0x0001) == 2.0 ** -133          # smallest subnormal
    assert oracle.bf16_value(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


def test_ab_project_hand_worked():
    # alpha = 0.5 * 1 + (-1) * 2 = -1.5 ;  beta = 0.25 * 1 + 3 * 2 = 6.25
    x = np.array([[1.0, 2.0]])
    wa = np.array([[0x3F00, 0xBF80]], np.uint16)     # 0.5, -1
    wb = np.array([[0x3E80, 0x4040]], np.uint16)     # 0.25, 3
    a, b = oracle.ab_project(x, wa, wb)
    assert a[0, 0] == -1.5 and b[0, 0] == 6.25


def test_ab_project_matches_numpy_matmul():
    wl = W.make_ab(3, 2, seed=31, n_embd=256, h_v=6)
    a, b = oracle.ab_project(wl.x, wl.w_alpha, wl.w_beta)
    dec = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(a, wl.x.astype(np.float64) @ dec(wl.w_alpha).T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b, wl.x.astype(np.float64) @ dec(wl.w_beta).T, rtol=1e-12, atol=1e-12)
    a2, _ = oracle.ab_project(2.0 * wl.x, wl.w_alpha, wl.w_beta)
    np.testing.assert_array_equal(a2, 2.0 * a)


def test_project_matches_numpy_and_hand_example():
    x = np.array([[1.0, 2.0, -1.0]])
    w = np.array([[0x3F00, 0xBF80, 0x4000], [0x0000, 0x3F80, 0x3F80]], np.uint16)   # [0.5,-1,2], [0,1,1]
    np.testing.assert_array_equal(oracle.project(x, w), [[0.5 - 2.0 - 2.0, 2.0 - 1.0]])
    xr, wr = W.make_proj(7, 64, 40, seed=33)
    dec = (wr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(oracle.project(xr, wr, threads=3), xr.astype(np.float64) @ dec.T, rtol=1e-12, atol=1e-12)


def test_silu_gate_closed_forms():
    """The earlier model's output gate is SiLU, z * sigmoid(z): zero at z = 0, (3/4) ln 3 at
    z = ln 3 (sigmoid(ln 3) = 3/4), and z itself to 1e-17 at z = 40; the norm part is
    unchanged: o = (3, 4) has mean square 12.5."""
    o = np.array([[3.0, 4.0], [3.0, 4.0]])
    w = np.array([1.0, 2.0])
    z = np.array([[0.0, np.log(3.0)], [40.0, -40.0]])
    y = oracle.gated_rmsnorm(o, z, w, 0.0, gate_silu=True)
    inv = 1.0 / np.sqrt(12.5)
    np.testing.assert_allclose(y[0], [0.0, 4.0 * inv * 2.0 * 0.75 * np.log(3.0)], rtol=1e-15, atol=0)
    np.testing.assert_allclose(y[1], [3.0 * inv * 40.0, 0.0], rtol=1e-15, atol=1e-15)
    ys = oracle.gated_rmsnorm(o, z, w, 0.0)
    np.testing.assert_allclose(ys[0], [3.0 * inv * 0.5, 4.0 * inv * 2.0 * 0.75], rtol=1e-15)


def test_readout_scale_placement_is_the_same_mixer():
    """1/sqrt(S) on the readout instead of on q: q in h is unit-norm (sqrt(S) times the
    default's), and o, y and the state agree with the default to rounding, because the
    recurrence is linear in q and q does not enter the state."""
    wl = W.make("v", 2, 5, seed=41, geom=W.Geom(h_k=2, h_v=4, s=16), state_std=0.02, conv_std=1.0)
    a = oracle.run_sequence(wl, 1)
    wl.scale_after_readout = True
    b = oracle.run_sequence(wl, 1)
    qn = wl.geom.h_k * wl.geom.s
    np.testing.assert_allclose(b["h"][:, :qn], a["h"][:, :qn] * np.sqrt(wl.geom.s), rtol=1e-14)
    np.testing.assert_array_equal(b["h"][:, qn:], a["h"][:, qn:])
    for key in ("o", "y", "state", "conv_state"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-14 * np.abs(a[key]).max())
    assert np.abs(b["o"]).max() > 0.1
