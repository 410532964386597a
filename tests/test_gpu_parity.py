"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

Every workload is seeded and synthetic. Every comparison uses the one bound of
tests/parity.py: tol(n) = 1e-4 + 9e-4 (n - 1) / 511 times max |ref| for a value n
sequential steps from the seeded inputs (o and y of token t: n = t + 1; a state after
n_b tokens: n = n_b; h: n = 1), so 1e-4 per decode step and 1e-3 after 512 steps.
The conv history (raw inputs, only moved), integer and placement results (untouched
slots, skipped tokens, flags) are compared bit for bit.
"""
import numpy as np
import pytest

import gdn_workloads as W
import oracle
from gpu_harness import GpuMixer, assert_close, assert_exact, assert_tokens, dev, log, tol

pytestmark = pytest.mark.gpu

_ORACLE = {}


def _workload_and_oracle(name):
    """The workload and the oracle's results for all its sequences, computed once."""
    if name not in _ORACLE:
        wl = W.CONFIGS[name]()
        _ORACLE[name] = (wl, oracle.run_workload(wl))
    return _ORACLE[name]

FUSED = pytest.mark.parametrize("fused", [False, True], ids=["3calls", "fused_norm"])
# single-token workloads also run through the single-launch decode
DECODE_MODES = pytest.mark.parametrize("fused", [False, True, "one"], ids=["3calls", "fused_norm", "one_launch"])


def _stack(results, key, n=None):
    return np.stack([r[key] if n is None else r[key][:n] for r in results])


def _compare_all(gm, wl, res, tag, keys=("o", "y", "h"), first_step=1):
    """o and y of every valid token at tol(first_step + t) per token index t, h at tol(1)
    at every token (first_step - 1 steps ran before this call), the final state of every
    slot at tol(first_step - 1 + the most tokens a sequence took), the conv history bit
    for bit.  Outputs of skipped tokens must be zero."""
    counts = [wl.tokens_of(b) for b in range(wl.B)]
    errs = {}
    for key in keys:
        arr = getattr(gm, key).cpu().numpy()
        errs[key] = assert_tokens(f"{tag} {key}", arr, [r[key] for r in res], counts, first_step,
                                  recurrent=key != "h")[0]
    st = gm.pool.state.cpu().numpy()
    cv = gm.pool.conv.cpu().numpy()
    sl = wl.slots
    errs["state"] = assert_close(f"{tag} state", st[sl], _stack(res, "state"), max(1, first_step - 1 + max(counts)))
    assert_exact(f"{tag} conv", cv[sl], _stack(res, "conv_state"))
    log(f"{tag}: rel errors " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()) + ", conv exact")
    return st, cv


# ------------------------------------------------------------------ the five workloads
@DECODE_MODES
def test_tiny_b1_t8_every_step(fused):
    """One sequence, 8 sequential single-token calls, parity after every step."""
    wl = W.tiny()
    log(f"tiny_b1_t8 fused={fused}: start")
    gm = GpuMixer(wl)
    st, cs = wl.state[0], wl.conv_state[0]
    for t in range(wl.T):
        h, o, y = gm.run(t, t + 1, fused=fused)
        r = oracle.run_sequence(wl, 0, t, t + 1, state=st, conv_state=cs)
        st, cs = r["state"], r["conv_state"]
        # token t has gone through t + 1 steps of the recurrence; h through none
        assert_close(f"step {t} h", h.cpu().numpy()[0], r["h"], 1)
        if fused != "one":
            assert_close(f"step {t} o", o.cpu().numpy()[0], r["o"], t + 1)
        assert_close(f"step {t} y", y.cpu().numpy()[0], r["y"], t + 1)
        assert_close(f"step {t} state", gm.slot_state(0), st, t + 1)
        assert_exact(f"step {t} conv", gm.slot_conv(0), cs)
    assert int(gm.pool.flags.item()) == 0


@DECODE_MODES
def test_decode_b64_one_step(fused):
    log(f"decode_b64 fused={fused}: start")
    wl, res = _workload_and_oracle("b64")
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    _compare_all(gm, wl, res, "decode_b64", keys=("y", "h") if fused == "one" else ("o", "y", "h"))
    assert int(gm.pool.flags.item()) == 0


@DECODE_MODES
def test_decode_b256_one_step(fused):
    """The bandwidth-bound decode: 256 sequences, 768 MiB of state, in the launch
    configuration the benchmark times."""
    log(f"decode_b256 fused={fused}: start")
    wl, res = _workload_and_oracle("b256")
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    _compare_all(gm, wl, res, "decode_b256", keys=("y", "h") if fused == "one" else ("o", "y", "h"))


@FUSED
def test_prefill_b16_t512_state_on_chip(fused):
    """16 sequences x 512 tokens in ONE call: the state stays in VGPRs across the tokens."""
    log(f"prefill_b16_t512 fused={fused}: start")
    wl, res = _workload_and_oracle("prefill")
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    # token t of o and y at tol(t + 1): 1e-4 for the first token, 1e-3 for the 512th
    _compare_all(gm, wl, res, "prefill_b16_t512")


def test_512_sequential_single_launch_decodes():
    """512 decode tokens as 512 calls of the single-launch decode (the benchmark's step),
    from a filled state, against the oracle for every token's y and the final state and
    conv history (the 512-step bound), and bit for bit against the same 512 tokens as
    one multi-token call of the two-launch form."""
    import torch
    T = 512
    wl = W.make("seq512", 4, T, seed=71, n_slots=6, state_std=0.02, conv_std=1.0, slot_choice="random")
    log("512 sequential single-launch decodes: oracle")
    res = oracle.run_workload(wl)
    one = GpuMixer(wl)
    for t in range(T):
        one.run(t, t + 1, fused="one")
    torch.cuda.synchronize()
    log("512 sequential single-launch decodes: compare")
    _compare_all(one, wl, res, "seq512", keys=("y", "h"))
    multi = GpuMixer(wl)
    multi.run(fused=True)
    assert torch.equal(one.pool.state, multi.pool.state)
    assert torch.equal(one.pool.conv, multi.pool.conv)
    assert torch.equal(one.y, multi.y) and torch.equal(one.h, multi.h)
    assert int(one.pool.flags.item()) == 0


@FUSED
def test_ragged_pool2048_b1024(fused):
    """2048-slot pool, 1024 sequences at random unique slots, U{1..8} tokens each, one call
    with per-sequence token counts. Untouched slots stay bit-identical."""
    import torch
    log(f"ragged fused={fused}: start")
    wl, res = _workload_and_oracle("ragged")
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    st, _ = _compare_all(gm, wl, res, "ragged")
    untouched = np.setdiff1d(np.arange(wl.n_slots), wl.slots)
    assert np.array_equal(st[untouched], wl.state[untouched]), "an untouched slot changed"
    assert np.array_equal(gm.pool.conv.cpu().numpy()[untouched], wl.conv_state[untouched])
    assert int(gm.pool.flags.item()) == 0

    # The same work as continuous batching: call t advances only the sequences that still
    # have a token t, gathered by slot.  Bitwise equal to the one-call form.
    log("ragged: continuous-batching form")
    gm2 = GpuMixer(wl)
    for t in range(wl.T):
        act = np.nonzero(wl.n_tok > t)[0]
        if act.size == 0:
            continue
        idx = dev(act.astype(np.int64))
        sub = lambda x: x[idx, t:t + 1].contiguous()
        B = act.size
        h = torch.empty(B, 1, wl.geom.channels, device="cuda")
        o = torch.empty(B, 1, wl.geom.h_v, wl.geom.s, device="cuda")
        y = torch.empty(B, 1, wl.geom.value_dim, device="cuda")
        gm2.G.gdn_mixer(gm2.pool, sub(gm2.qkv), sub(gm2.alpha), sub(gm2.beta_logit), sub(gm2.z),
                        gm2.conv_w, gm2.dt, gm2.ssm_a, gm2.norm_w, wl.eps, h, o, y, gm2.slots[idx].contiguous(),
                        fused=fused)
        gm2.o[idx, t:t + 1] = o
        gm2.y[idx, t:t + 1] = y
    assert torch.equal(gm2.pool.state, gm.pool.state)
    assert torch.equal(gm2.pool.conv, gm.pool.conv)
    mask = torch.arange(wl.T, device="cuda")[None, :] < gm.n_tok[:, None].long()
    assert torch.equal(gm2.o[mask], gm.o[mask])
    assert torch.equal(gm2.y[mask], gm.y[mask])


def test_pool_beyond_2g_floats_top_slots():
    """A pool of 2,800 slots (8.2 GiB of state: element offsets pass 2^31 from slot 2,731
    on, byte offsets pass 2^32 from slot 1,366 on).  Sequences sit on the top slots and
    on both sides of those boundaries; every call form must address them right and leave
    the other slots bit-identical."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    n_big = 2800
    g = W.Geom()
    assert (n_big - 1) * g.h_v * g.s * g.s > 2 ** 31
    log(f"big pool: {n_big} slots")
    big = G.StatePool(n_big)
    big.state.fill_(0.25)
    big.conv.fill_(-0.5)
    big.flags.zero_()
    forms = [("3calls", 3, False, [2799, 2731, 2730, 1366]), ("fused_norm", 3, True, [2798, 2732, 1365, 0]),
             ("one_launch", 1, "one", [2797, 2733, 2729, 1367])]
    used = []
    for k, (tag, T, fused, hi) in enumerate(forms):
        wl = W.make("bigpool", len(hi), T, seed=62 + k, n_slots=len(hi), state_std=0.02, conv_std=1.0)
        res = oracle.run_workload(wl)
        hi_d = dev(np.array(hi, np.int32))
        big.state[hi_d.long()] = dev(wl.state)
        big.conv[hi_d.long()] = dev(wl.conv_state)
        log(f"big pool {tag}: slots {hi}")
        gm = GpuMixer(wl, pool=big)
        gm.run(slots=hi_d, fused=fused)
        torch.cuda.synchronize()
        for key in ("o", "y", "h") if fused != "one" else ("y", "h"):
            assert_tokens(f"big pool {tag} {key}", getattr(gm, key).cpu().numpy(), [r[key] for r in res],
                          [T] * len(hi), recurrent=key != "h")
        assert_close(f"big pool {tag} state", big.state[hi_d.long()].cpu().numpy(), _stack(res, "state"), T)
        assert_exact(f"big pool {tag} conv", big.conv[hi_d.long()].cpu().numpy(), _stack(res, "conv_state"))
        used += hi
    assert int(big.flags.item()) == 0
    # untouched slots, among them the neighbours of every slot used
    probe = sorted({s + d for s in used for d in (-1, 1) if 0 <= s + d < n_big} - set(used))
    p_d = dev(np.array(probe, np.int64))
    assert bool((big.state[p_d] == 0.25).all()), "an untouched slot's state changed"
    assert bool((big.conv[p_d] == -0.5).all()), "an untouched slot's conv history changed"


# ------------------------------------------------------------------ properties and edges
SMALL_GEOMS =[W.Geom(h_k=1, h_v=3), W.Geom(h_k=2, h_v=4), W.Geom(h_k=2, h_v=6)]


@pytest.mark.parametrize("geom", SMALL_GEOMS, ids=lambda g: f"hk{g.h_k}hv{g.h_v}")
@pytest.mark.parametrize("B,T", [(1, 1), (5, 11), (3, 17)])
def test_small_geometries_several_tiles_ragged_tail(geom, B, T):
    """Other head counts of the family; T spans several 8-token conv blocks with a tail."""
    wl = W.make("small", B, T, seed=40 + B + T + geom.h_v, geom=geom, n_slots=B + 2, state_std=0.05,
                conv_std=1.0, slot_choice="random")
    log(f"small geometry h_k={geom.h_k} h_v={geom.h_v} B={B} T={T}")
    gm = GpuMixer(wl)
    gm.run()
    res = oracle.run_workload(wl)
    _compare_all(gm, wl, res, "small")


@FUSED
def test_chunked_calls_equal_one_call_bitwise(fused):
    """T tokens in one call equal the same tokens split over several calls, bit for bit
    (the multi-token path must reproduce the single-token decode exactly)."""
    import torch
    wl = W.make("chunk", 4, 20, seed=50, state_std=0.02, conv_std=1.0)
    log(f"chunked vs one call, fused={fused}")
    a = GpuMixer(wl)
    a.run(fused=fused)
    b = GpuMixer(wl)
    for t0, t1 in [(0, 1), (1, 8), (8, 9), (9, 20)]:
        b.run(t0, t1, fused=fused)
    assert torch.equal(a.pool.state, b.pool.state)
    assert torch.equal(a.pool.conv, b.pool.conv)
    assert torch.equal(a.o, b.o) and torch.equal(a.y, b.y) and torch.equal(a.h, b.h)


def test_batch_order_invariance():
    import torch
    wl = W.make("perm", 6, 3, seed=51, n_slots=9, state_std=0.02, conv_std=1.0, slot_choice="random")
    log("batch order invariance")
    a = GpuMixer(wl)
    a.run()
    perm = np.array([3, 0, 5, 1, 4, 2])
    wl2 = W.make("perm", 6, 3, seed=51, n_slots=9, state_std=0.02, conv_std=1.0, slot_choice="random")
    for f in ("qkv", "alpha", "beta_logit", "z", "slots"):
        setattr(wl2, f, getattr(wl2, f)[perm].copy())
    b = GpuMixer(wl2)
    b.run()
    assert torch.equal(a.pool.state, b.pool.state)
    assert torch.equal(a.o[dev(perm)], b.o)
    assert torch.equal(a.y[dev(perm)], b.y)


def test_beta0_gate0_leaves_state_bit_identical():
    """beta logit = -inf gives beta = 0 and ssm_a = 0 gives exp(g) = 1 exactly."""
    import torch
    wl = W.make("inv", 3, 2, seed=52, state_std=0.02, conv_std=1.0)
    wl.beta_logit[:] = -np.inf
    wl.ssm_a[:] = 0.0
    gm = GpuMixer(wl)
    before = gm.pool.state.clone()
    gm.run()
    assert torch.equal(gm.pool.state, before)
    res = oracle.run_workload(wl)
    _compare_all(gm, wl, res, "beta0")


def test_beta1_unit_k_recalls_v():
    """beta = 1, decay 1: after the step S^T k = v for the (unit) k of each head."""
    wl = W.make("recall", 2, 1, seed=53, state_std=0.02, conv_std=1.0)
    wl.beta_logit[:] = np.inf
    wl.ssm_a[:] = 0.0
    gm = GpuMixer(wl)
    gm.run()
    h = gm.h.cpu().numpy()
    st = gm.pool.state.cpu().numpy()
    g = wl.geom
    for b in range(2):
        for i in range(g.h_v):
            j = i // (g.h_v // g.h_k)
            k = h[b, 0, (g.h_k + j) * g.s:(g.h_k + j + 1) * g.s].astype(np.float64)
            v = h[b, 0, (2 * g.h_k + i) * g.s:(2 * g.h_k + i + 1) * g.s].astype(np.float64)
            kv = st[b, i].astype(np.float64).T @ k
            assert np.abs(kv - v).max() <= tol(1) * np.abs(v).max()


def test_zero_tokens_and_bad_counts():
    """n_tok = 0 leaves a slot untouched and writes zeros; counts outside [0, T] are
    clamped and flagged."""
    import torch
    wl = W.make("ntok", 4, 5, seed=54, n_slots=6, state_std=0.02, conv_std=1.0, slot_choice="random")
    wl.n_tok = np.array([0, 5, 2, 3], np.int32)
    gm = GpuMixer(wl)
    gm.run()
    assert int(gm.pool.flags.item()) == 0
    st = gm.pool.state.cpu().numpy()
    assert np.array_equal(st[wl.slots[0]], wl.state[wl.slots[0]])
    assert (gm.o[0] == 0).all() and (gm.h[0] == 0).all()
    res = oracle.run_workload(wl)
    _compare_all(gm, wl, res, "ntok")
    # out-of-range counts: 9 -> 5 (T) and -3 -> 0, with the flag raised
    wl2 = W.make("ntok", 2, 5, seed=55, state_std=0.02, conv_std=1.0)
    gm2 = GpuMixer(wl2)
    before = gm2.pool.state.clone()
    gm2.run(n_tok=dev(np.array([9, -3], np.int32)))
    assert int(gm2.pool.flags.item()) & gm2.G.GDN_FLAG_BAD_NTOK
    assert torch.equal(gm2.pool.state[1], before[1])
    wl2.n_tok = np.array([5, 0], np.int32)
    res2 = oracle.run_workload(wl2)
    _compare_all(gm2, wl2, res2, "ntok-clamped")


def test_bad_slot_is_skipped_and_flagged():
    import torch
    wl = W.make("badslot", 3, 2, seed=56, n_slots=4, state_std=0.02, conv_std=1.0)
    gm = GpuMixer(wl)
    before = gm.pool.state.clone()
    bad = dev(np.array([0, 7, -1], np.int32))
    gm.run(slots=bad)
    assert int(gm.pool.flags.item()) & gm.G.GDN_FLAG_BAD_SLOT
    assert (gm.o[1:] == 0).all() and (gm.y[1:] == 0).all() and (gm.h[1:] == 0).all()
    assert torch.equal(gm.pool.state[1:], before[1:])
    res = oracle.run_workload(wl, seqs=[0])
    assert_tokens("badslot o", gm.o[:1].cpu().numpy(), [res[0]["o"]], [wl.T])


def test_pool_zero():
    import torch
    wl = W.make("zero", 2, 1, seed=57, n_slots=5, state_std=0.02, conv_std=1.0)
    gm = GpuMixer(wl)
    gm.pool.flags.fill_(3)
    gm.pool.zero(dev(np.array([1, 3], np.int32)))
    st, cv = gm.pool.state.cpu().numpy(), gm.pool.conv.cpu().numpy()
    assert (st[[1, 3]] == 0).all() and (cv[[1, 3]] == 0).all()
    assert np.array_equal(st[[0, 2, 4]], wl.state[[0, 2, 4]])
    assert int(gm.pool.flags.item()) == 3
    gm.pool.zero()
    assert int(torch.count_nonzero(gm.pool.state)) == 0 and int(torch.count_nonzero(gm.pool.conv)) == 0
    assert int(gm.pool.flags.item()) == 0


def test_gated_rmsnorm_ragged_rows_and_in_place():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    rng = np.random.default_rng(58)
    for rows in (1, 7, 13, 1031):
        o = rng.standard_normal((rows, 128)).astype(np.float32) * rng.uniform(0.01, 10, (rows, 1)).astype(np.float32)
        z = rng.standard_normal((rows, 128)).astype(np.float32)
        w = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
        ref = oracle.gated_rmsnorm(o, z, w, 1e-6)
        od = dev(o)
        y = torch.empty_like(od)
        G.gdn_gated_rmsnorm(od, dev(z), dev(w), 1e-6, y)
        assert_close(f"rmsnorm rows={rows}", y.cpu().numpy(), ref, 1)
        G.gdn_gated_rmsnorm(od, dev(z), dev(w), 1e-6, od)   # y aliasing o
        assert torch.equal(od, y)


def test_empty_batch_is_a_no_op():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    pool = G.StatePool(2)
    pool.zero()
    e = torch.empty(0, 1, 10240, device="cuda")
    G.gdn_conv_silu_norm(pool, e, torch.zeros(10240, 4, device="cuda"), 1e-6, torch.empty_like(e))
    G.gdn_decode_step(pool, e, torch.empty(0, 1, 48, device="cuda"), torch.empty(0, 1, 48, device="cuda"),
                      torch.zeros(48, device="cuda"), torch.zeros(48, device="cuda"),
                      torch.empty(0, 1, 48, 128, device="cuda"))
    e1 = torch.empty(0, 10240, device="cuda")
    G.gdn_decode_fused(pool, e1, torch.zeros(10240, 4, device="cuda"), torch.empty(0, 48, device="cuda"),
                       torch.empty(0, 48, device="cuda"), torch.zeros(48, device="cuda"), torch.zeros(48, device="cuda"),
                       torch.empty(0, 6144, device="cuda"), torch.ones(128, device="cuda"), 1e-6,
                       torch.empty(0, 6144, device="cuda"))
    G.gdn_decode_step_norm(pool, e, torch.empty(0, 1, 48, device="cuda"), torch.empty(0, 1, 48, device="cuda"),
                           torch.zeros(48, device="cuda"), torch.zeros(48, device="cuda"),
                           torch.empty(0, 1, 6144, device="cuda"), torch.ones(128, device="cuda"), 1e-6,
                           torch.empty(0, 1, 6144, device="cuda"))
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(pool.state)) == 0 and int(torch.count_nonzero(pool.conv)) == 0


def test_abi_rejects_bad_arguments_on_device():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    pool = G.StatePool(2)
    x = torch.zeros(1, 1, 10240, device="cuda")
    with pytest.raises(G.GdnError) as e:
        G.gdn_conv_silu_norm(pool, x, torch.zeros(10240, 4, device="cuda"), 1e-6, x)   # h aliases qkv
    assert e.value.code == G.GDN_ERR_ARG and "overlaps" in str(e.value)
    with pytest.raises(G.GdnError):
        G.gdn_decode_step(pool, torch.zeros(3, 1, 10240, device="cuda"), torch.zeros(3, 1, 48, device="cuda"),
                          torch.zeros(3, 1, 48, device="cuda"), torch.zeros(48, device="cuda"),
                          torch.zeros(48, device="cuda"), torch.zeros(3, 1, 48, 128, device="cuda"))  # B > n_slots


@pytest.mark.parametrize("T", [1, 6, 19])
def test_fused_norm_equals_separate_norm(T):
    """The fused epilogue computes the same norm as gdn_gated_rmsnorm, bit for bit, in both
    the single-token and the multi-token kernel; o is optional."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("fuse", 5, T, seed=59 + T, n_slots=7, state_std=0.02, conv_std=1.0, slot_choice="random")
    wl.n_tok = np.minimum(np.array([6, 1, 0, 3, 19], np.int32), T).astype(np.int32)
    a = GpuMixer(wl)
    a.run()
    b = GpuMixer(wl)
    b.run(fused=True)
    assert torch.equal(a.pool.state, b.pool.state) and torch.equal(a.o, b.o)
    assert torch.equal(b.y, a.y)
    # o = None: same y and state, o untouched
    c = GpuMixer(wl)
    h = torch.empty_like(c.h)
    G.gdn_conv_silu_norm(c.pool, c.qkv, c.conv_w, wl.eps, h, c.slots, c.n_tok)
    y = torch.full_like(c.y, 7.0)
    G.gdn_decode_step_norm(c.pool, h, c.alpha, c.beta_logit, c.dt, c.ssm_a, c.z, c.norm_w, wl.eps, y,
                           None, c.slots, c.n_tok)
    assert torch.equal(y, b.y) and torch.equal(c.pool.state, b.pool.state)
    with pytest.raises(G.GdnError):
        G.gdn_decode_step_norm(c.pool, h, c.alpha, c.beta_logit, c.dt, c.ssm_a, c.z, c.norm_w, wl.eps, c.z,
                               None, c.slots, c.n_tok)   # y aliases z


@FUSED
@pytest.mark.parametrize("B", [6, 20])
def test_token_counts_across_conv_blocks(fused, B):
    """Ragged counts that end before, at and across the conv kernel's 8-token groups (the
    history of later groups comes from qkv, the stored history is read and written by
    group 0 only): 0, 1, 3, 4, 5, 32, 33, 64 and 70 of 70 tokens, at two batch sizes."""
    wl = W.make("blocks", B, 70, seed=60, n_slots=B + 3, state_std=0.02, conv_std=1.0, slot_choice="random")
    wl.n_tok = np.resize(np.array([0, 1, 3, 33, 64, 70, 4, 5, 32], np.int32), B)
    log(f"conv token blocks, B={B} fused={fused}")
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    res = oracle.run_workload(wl)
    _compare_all(gm, wl, res, "blocks")


@pytest.mark.parametrize("geom", [W.Geom(), W.Geom(h_k=2, h_v=6), W.Geom(h_k=2, h_v=4), W.Geom(h_k=2, h_v=2),
                                  W.Geom(h_k=1, h_v=4), W.Geom(h_k=1, h_v=14)],
                         ids=lambda g: f"hk{g.h_k}hv{g.h_v}")
def test_single_launch_decode_equals_two_calls_bitwise(geom):
    """gdn_decode_fused == gdn_conv_silu_norm + gdn_decode_step_norm, bit for bit, and
    matches the oracle; without h it writes the same y and state."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("one", 5, 1, seed=61 + geom.h_v, geom=geom, n_slots=8, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    log(f"single-launch decode h_k={geom.h_k} h_v={geom.h_v}")
    a = GpuMixer(wl)
    a.run(fused=True)
    b = GpuMixer(wl)
    b.run(fused="one")
    assert torch.equal(a.h, b.h) and torch.equal(a.y, b.y)
    assert torch.equal(a.pool.state, b.pool.state) and torch.equal(a.pool.conv, b.pool.conv)
    res = oracle.run_workload(wl)
    _compare_all(b, wl, res, "one-launch", keys=("y", "h"))
    c = GpuMixer(wl)
    y = torch.empty_like(c.y[:, 0])
    G.gdn_decode_fused(c.pool, c.qkv[:, 0].contiguous(), c.conv_w, c.alpha[:, 0].contiguous(),
                       c.beta_logit[:, 0].contiguous(), c.dt, c.ssm_a, c.z[:, 0].contiguous(), c.norm_w, wl.eps, y,
                       None, c.slots)
    assert torch.equal(y, b.y[:, 0]) and torch.equal(c.pool.state, b.pool.state)


def test_single_launch_decode_bad_slot():
    import torch
    wl = W.make("one-bad", 3, 1, seed=62, n_slots=4, state_std=0.02, conv_std=1.0)
    gm = GpuMixer(wl)
    before_s, before_c = gm.pool.state.clone(), gm.pool.conv.clone()
    gm.run(fused="one", slots=dev(np.array([2, 9, -4], np.int32)))
    assert int(gm.pool.flags.item()) & gm.G.GDN_FLAG_BAD_SLOT
    assert (gm.y[1:] == 0).all() and (gm.h[1:] == 0).all()
    keep = [0, 1, 3]
    assert torch.equal(gm.pool.state[keep], before_s[keep]) and torch.equal(gm.pool.conv[keep], before_c[keep])
    wl.slots = np.array([2, 0, 0], np.int32)
    res = oracle.run_workload(wl, seqs=[0])
    assert_close("one-bad y", gm.y[0].cpu().numpy(), res[0]["y"], 1)


@pytest.mark.parametrize("T", [1, 4, 37])
def test_verify_window_then_commit(T):
    """A window of T drafted tokens from the untouched state, then a commit of n_keep
    accepted tokens per sequence, equals decoding those tokens directly, bit for bit
    (the pages' speculative window and commit)."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("window", 5, T, seed=70 + T, n_slots=8, state_std=0.02, conv_std=1.0, slot_choice="random")
    n_keep = np.minimum(np.array([T, 0, 1, max(T - 1, 0), 2], np.int32), T).astype(np.int32)
    log(f"verify window T={T} n_keep={n_keep.tolist()}")
    win = GpuMixer(wl)
    before_s, before_c = win.pool.state.clone(), win.pool.conv.clone()
    h = torch.empty_like(win.h)
    y = torch.empty_like(win.y)
    G.gdn_verify_window(win.pool, win.qkv, win.conv_w, win.alpha, win.beta_logit, win.dt, win.ssm_a, win.z,
                        win.norm_w, wl.eps, h, y, win.slots)
    torch.cuda.synchronize()
    assert torch.equal(win.pool.state, before_s) and torch.equal(win.pool.conv, before_c), "window wrote the pool"
    direct = GpuMixer(wl)
    direct.run(fused=True)                        # all T tokens, persisted
    assert torch.equal(y, direct.y) and torch.equal(h, direct.h)
    res = oracle.run_workload(wl)
    assert_tokens("window y", y.cpu().numpy(), [r["y"] for r in res], [T] * wl.B)

    G.gdn_commit(win.pool, win.qkv, h, win.alpha, win.beta_logit, win.dt, win.ssm_a, dev(n_keep), win.slots)
    kept = GpuMixer(wl)
    kept.run(fused=True, n_tok=dev(n_keep))       # only the accepted tokens, persisted
    assert torch.equal(win.pool.state, kept.pool.state)
    assert torch.equal(win.pool.conv, kept.pool.conv)
    assert int(win.pool.flags.item()) == 0
    # the next decode token continues identically from both pools
    nxt = W.make("window-next", 5, 1, seed=90 + T, n_slots=8, state_std=0.02, conv_std=1.0)
    for gm in (win, kept):
        q, a_, b_, z_ = dev(nxt.qkv), dev(nxt.alpha), dev(nxt.beta_logit), dev(nxt.z)
        hh = torch.empty(5, 1, wl.geom.channels, device="cuda")
        yy = torch.empty(5, 1, wl.geom.value_dim, device="cuda")
        G.gdn_conv_silu_norm(gm.pool, q, gm.conv_w, wl.eps, hh, gm.slots)
        G.gdn_decode_step_norm(gm.pool, hh, a_, b_, gm.dt, gm.ssm_a, z_, gm.norm_w, wl.eps, yy, None, gm.slots)
        gm.next_y = yy
    assert torch.equal(win.next_y, kept.next_y)


@pytest.mark.parametrize("T", [6, 20])
def test_verify_window_ragged_with_an_unknown_slot(T):
    """A window with per-sequence token counts and one unknown slot (a short and a long
    window): y and h equal decoding the same tokens directly, bit for bit; the unknown
    slot's rows are zero and flagged; the pool is untouched."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("window-ragged", 4, T, seed=95 + T, n_slots=6, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    n_tok = np.array([T, 1, 0, max(T - 2, 1)], np.int32)
    slots = wl.slots.copy()
    slots[3] = 99                                    # outside the pool
    log(f"ragged window T={T} n_tok={n_tok.tolist()} slots={slots.tolist()}")
    win = GpuMixer(wl)
    before_s, before_c = win.pool.state.clone(), win.pool.conv.clone()
    h = torch.full_like(win.h, 3.0)
    y = torch.full_like(win.y, 3.0)
    G.gdn_verify_window(win.pool, win.qkv, win.conv_w, win.alpha, win.beta_logit, win.dt, win.ssm_a, win.z,
                        win.norm_w, wl.eps, h, y, dev(slots), dev(n_tok))
    torch.cuda.synchronize()
    assert torch.equal(win.pool.state, before_s) and torch.equal(win.pool.conv, before_c), "window wrote the pool"
    assert int(win.pool.flags.item()) & G.GDN_FLAG_BAD_SLOT
    assert not y[3].any() and not h[3].any()
    direct = GpuMixer(wl)
    direct.run(fused=True, slots=dev(slots), n_tok=dev(n_tok))
    assert torch.equal(y, direct.y) and torch.equal(h, direct.h)


@pytest.mark.parametrize("B,T,ragged", [(64, 4, False), (43, 3, True), (42, 5, True), (100, 8, True), (160, 2, True)])
def test_many_sequence_window_matches_direct_decode(B, T, ragged):
    """Windows over many sequences (thousands of workgroups, so every CU runs several):
    y and h equal decoding the same tokens directly, bit for bit, with ragged token
    counts (0 to T), unknown slots flagged with zero rows, and the pool untouched;
    sampled sequences against the oracle."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("window-many", B, T, seed=300 + B + T, n_slots=B + 7, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    rng = np.random.default_rng(400 + B)
    slots = wl.slots.copy()
    n_tok = np.full(B, T, np.int32)
    if ragged:
        n_tok = rng.integers(0, T + 1, B).astype(np.int32)
        n_tok[0] = T
        slots[[5, B - 1]] = [B + 7, -3]                  # outside the pool
    log(f"many-sequence window B={B} T={T} ragged={ragged} tokens={int(n_tok.sum())}")
    win = GpuMixer(wl)
    before_s, before_c = win.pool.state.clone(), win.pool.conv.clone()
    h = torch.full_like(win.h, 3.0)
    y = torch.full_like(win.y, 3.0)
    G.gdn_verify_window(win.pool, win.qkv, win.conv_w, win.alpha, win.beta_logit, win.dt, win.ssm_a, win.z,
                        win.norm_w, wl.eps, h, y, dev(slots), dev(n_tok))
    torch.cuda.synchronize()
    assert torch.equal(win.pool.state, before_s) and torch.equal(win.pool.conv, before_c), "window wrote the pool"
    flags = int(win.pool.flags.item())
    assert bool(flags & G.GDN_FLAG_BAD_SLOT) == ragged and not flags & G.GDN_FLAG_BAD_NTOK
    if ragged:
        assert not y[[5, B - 1]].any() and not h[[5, B - 1]].any()
    direct = GpuMixer(wl)
    direct.run(fused=True, slots=dev(slots), n_tok=dev(n_tok))
    assert torch.equal(y, direct.y) and torch.equal(h, direct.h)
    for b in (0, B // 2 + 1):
        k = int(n_tok[b])
        if k == 0 or not 0 <= slots[b] < B + 7:
            continue
        slot = int(slots[b])
        ref = oracle.mixer(wl.geom, wl.qkv[b, :k], wl.conv_w, wl.alpha[b, :k], wl.beta_logit[b, :k], wl.dt,
                           wl.ssm_a, wl.z[b, :k], wl.norm_w, wl.eps, wl.conv_state[slot], wl.state[slot])
        assert_tokens(f"window y seq {b}", y[b:b + 1, :k].cpu().numpy(), [ref["y"]], [k])


@pytest.mark.parametrize("T0,T1,ragged", [(4, 4, True), (6, 1, True), (20, 9, True), (4, 3, False)])
def test_commit_window_equals_commit_then_window(T0, T1, ragged):
    """gdn_commit_window (the commit of one window and the next window with each state
    tile read once) equals gdn_commit followed by gdn_verify_window bit for bit: state,
    conv history, h, y and flags.  Ragged: per-sequence n_keep (0, all, some) and window
    token counts (0 included) and one unknown slot.  With everything kept, the next
    window's y and h also equal decoding all T0 + T1 tokens directly, and the oracle."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    B = 5
    wl = W.make("round", B, T0 + T1, seed=170 + T0 + T1, n_slots=9, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    slots = wl.slots.copy()
    if ragged:
        n_keep = np.array([T0, 0, 1, max(T0 - 1, 0), 2], np.int32)
        n_tok = np.array([T1, max(T1 - 1, 0), 0, 1, T1], np.int32)
        slots[4] = 77                                 # outside the pool
        nk, nt = dev(n_keep), dev(n_tok)
    else:
        nk = nt = None
    log(f"commit window T0={T0} T1={T1} ragged={ragged}")
    sl = dev(slots)
    two, one = GpuMixer(wl), GpuMixer(wl)
    w0 = lambda gm, a: getattr(gm, a)[:, :T0].contiguous()
    w1 = lambda gm, a: getattr(gm, a)[:, T0:].contiguous()
    outs = {}
    for name, gm in (("two", two), ("one", one)):
        g = wl.geom
        h0 = torch.empty(B, T0, g.channels, device="cuda")
        y0 = torch.empty(B, T0, g.value_dim, device="cuda")
        G.gdn_verify_window(gm.pool, w0(gm, "qkv"), gm.conv_w, w0(gm, "alpha"), w0(gm, "beta_logit"), gm.dt,
                            gm.ssm_a, w0(gm, "z"), gm.norm_w, wl.eps, h0, y0, sl)
        h1 = torch.full((B, T1, g.channels), 3.0, device="cuda")
        y1 = torch.full((B, T1, g.value_dim), 3.0, device="cuda")
        prev = (w0(gm, "qkv"), h0, w0(gm, "alpha"), w0(gm, "beta_logit"))
        if name == "two":
            G.gdn_commit(gm.pool, prev[0], h0, prev[2], prev[3], gm.dt, gm.ssm_a, nk, sl)
            G.gdn_verify_window(gm.pool, w1(gm, "qkv"), gm.conv_w, w1(gm, "alpha"), w1(gm, "beta_logit"), gm.dt,
                                gm.ssm_a, w1(gm, "z"), gm.norm_w, wl.eps, h1, y1, sl, nt)
        else:
            G.gdn_commit_window(gm.pool, prev, nk, w1(gm, "qkv"), gm.conv_w, w1(gm, "alpha"), w1(gm, "beta_logit"),
                                gm.dt, gm.ssm_a, w1(gm, "z"), gm.norm_w, wl.eps, h1, y1, sl, nt)
        outs[name] = (h1, y1)
    torch.cuda.synchronize()
    for a, b_, what in ((two.pool.state, one.pool.state, "state"), (two.pool.conv, one.pool.conv, "conv history"),
                        (outs["two"][0], outs["one"][0], "h"), (outs["two"][1], outs["one"][1], "y"),
                        (two.pool.flags, one.pool.flags, "flags")):
        assert torch.equal(a, b_), f"{what} differs"
    h1, y1 = outs["one"]
    assert y1.abs().max().item() > 0
    if ragged:
        assert int(one.pool.flags.item()) & G.GDN_FLAG_BAD_SLOT
        assert not y1[4].any() and not h1[4].any()
        assert not y1[2].any()
    else:
        assert int(one.pool.flags.item()) == 0
        direct = GpuMixer(wl)
        direct.run(fused=True)
        assert torch.equal(y1, direct.y[:, T0:]) and torch.equal(h1, direct.h[:, T0:])
        res = oracle.run_workload(wl)
        # the next window's token t follows the T0 committed tokens: T0 + t + 1 steps
        assert_tokens("round y", y1.cpu().numpy(), [r["y"][T0:] for r in res], [T1] * B, first_step=T0 + 1)


def test_speculative_round_b256_t4_full_size():
    """The speculative round at the size the benchmark times (256 sequences, 768 MiB of
    state, windows of 4 drafted tokens, n_keep ~ U{1..4} from the benchmark's seed):
    gdn_verify_window, then gdn_commit_window with the next window.  The fused round
    equals gdn_commit + gdn_verify_window bit for bit on the whole pool, and sampled
    sequences match the oracle run over their kept tokens followed by the next window
    (y of the next window; the committed state)."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    B, T = 256, 4
    wl = W.make("round_b256", B, 2 * T, seed=31, state_std=0.02, conv_std=1.0)
    g = wl.geom
    n_keep = np.random.default_rng(32).integers(1, T + 1, B).astype(np.int32)
    log(f"round b256 t4: {int(n_keep.sum())} kept")
    fused, two = GpuMixer(wl), GpuMixer(wl)
    part = lambda gm, a, lo: getattr(gm, a)[:, lo:lo + T].contiguous()
    nk = dev(n_keep)
    res = {}
    for name, gm in (("fused", fused), ("two", two)):
        h0 = torch.empty(B, T, g.channels, device="cuda")
        y0 = torch.empty(B, T, g.value_dim, device="cuda")
        G.gdn_verify_window(gm.pool, part(gm, "qkv", 0), gm.conv_w, part(gm, "alpha", 0), part(gm, "beta_logit", 0),
                            gm.dt, gm.ssm_a, part(gm, "z", 0), gm.norm_w, wl.eps, h0, y0)
        prev = (part(gm, "qkv", 0), h0, part(gm, "alpha", 0), part(gm, "beta_logit", 0))
        h1 = torch.empty(B, T, g.channels, device="cuda")
        y1 = torch.empty(B, T, g.value_dim, device="cuda")
        nxt = [part(gm, a, T) for a in ("qkv", "alpha", "beta_logit", "z")]
        if name == "fused":
            G.gdn_commit_window(gm.pool, prev, nk, nxt[0], gm.conv_w, nxt[1], nxt[2], gm.dt, gm.ssm_a, nxt[3],
                                gm.norm_w, wl.eps, h1, y1)
        else:
            G.gdn_commit(gm.pool, prev[0], h0, prev[2], prev[3], gm.dt, gm.ssm_a, nk)
            G.gdn_verify_window(gm.pool, nxt[0], gm.conv_w, nxt[1], nxt[2], gm.dt, gm.ssm_a, nxt[3], gm.norm_w,
                                wl.eps, h1, y1)
        res[name] = (h1, y1)
    torch.cuda.synchronize()
    assert torch.equal(res["fused"][1], res["two"][1]) and torch.equal(res["fused"][0], res["two"][0])
    assert torch.equal(fused.pool.state, two.pool.state) and torch.equal(fused.pool.conv, two.pool.conv)
    assert int(fused.pool.flags.item()) == 0
    y1 = res["fused"][1]
    for b in (0, 97, 255):
        k = int(n_keep[b])
        idx = np.r_[0:k, T:2 * T]                     # the kept tokens, then the next window
        slot = int(wl.slots[b])
        ref = oracle.mixer(g, wl.qkv[b, idx], wl.conv_w, wl.alpha[b, idx], wl.beta_logit[b, idx], wl.dt, wl.ssm_a,
                           wl.z[b, idx], wl.norm_w, wl.eps, wl.conv_state[slot], wl.state[slot])
        assert_tokens(f"round y seq {b}", y1[b:b + 1].cpu().numpy(), [ref["y"][k:]], [T], first_step=k + 1)
        com = oracle.mixer(g, wl.qkv[b, :k], wl.conv_w, wl.alpha[b, :k], wl.beta_logit[b, :k], wl.dt, wl.ssm_a,
                           wl.z[b, :k], wl.norm_w, wl.eps, wl.conv_state[slot], wl.state[slot])
        assert_close(f"committed state seq {b}", fused.pool.state[slot].cpu().numpy(), com["state"], k)
        assert_exact(f"committed conv seq {b}", fused.pool.conv[slot].cpu().numpy(), com["conv_state"])


# ------------------------------------------------------------------ alpha / beta projections
@pytest.mark.parametrize("B,T,n_embd,h_v", [(1, 1, 2560, 48), (3, 1, 2560, 48), (256, 1, 2560, 48),
                                            (16, 512, 2560, 48), (5, 2, 260, 6), (2, 3, 4, 3)])
def test_ab_projection(B, T, n_embd, h_v):
    """alpha / beta logits from bf16 weights and fp32 activations vs the oracle; rows not a
    multiple of the 4-row block, a partial 8-column group and an n_embd tail included."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    ab = W.make_ab(B, T, seed=80 + B + T, n_embd=n_embd, h_v=h_v)
    log(f"ab projection B={B} T={T} n_embd={n_embd} h_v={h_v}")
    x = dev(ab.x)
    wa = torch.from_numpy(ab.w_alpha.view(np.int16)).cuda()
    wb = torch.from_numpy(ab.w_beta.view(np.int16)).cuda()
    alpha = torch.full((B, T, h_v), 7.0, device="cuda")
    beta = torch.full((B, T, h_v), 7.0, device="cuda")
    G.gdn_ab_project(x, wa, wb, alpha, beta)
    ra, rb = oracle.ab_project(ab.x, ab.w_alpha, ab.w_beta)
    assert_close("alpha", alpha.cpu().numpy(), ra, 1)
    assert_close("beta_logit", beta.cpu().numpy(), rb, 1)


def test_ab_projection_feeds_the_recurrence():
    """Projection -> gdn_decode_step_norm equals the oracle's projection -> mixer."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("proj", 4, 3, seed=85, state_std=0.02, conv_std=1.0)
    ab = W.make_ab(4, 3, seed=86)
    ra, rb = oracle.ab_project(ab.x, ab.w_alpha, ab.w_beta)
    wl.alpha, wl.beta_logit = ra.astype(np.float32), rb.astype(np.float32)
    gm = GpuMixer(wl)
    G.gdn_ab_project(dev(ab.x), torch.from_numpy(ab.w_alpha.view(np.int16)).cuda(),
                     torch.from_numpy(ab.w_beta.view(np.int16)).cuda(), gm.alpha, gm.beta_logit)
    gm.run(fused=True)
    res = oracle.run_workload(wl)
    # alpha and beta come out of one projection: the mixer's token t is t + 2 steps in
    _compare_all(gm, wl, res, "proj->mixer", keys=("y", "h"), first_step=2)


def test_ab_projection_empty_is_a_no_op():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    x = torch.empty(0, 2560, device="cuda")
    w = torch.zeros(48, 2560, dtype=torch.int16, device="cuda")
    G.gdn_ab_project(x, w, w, torch.empty(0, 48, device="cuda"), torch.empty(0, 48, device="cuda"))


# ------------------------------------------------------------------ model variants
VARIANTS = pytest.mark.parametrize("gate_silu,after", [(True, False), (False, True), (True, True)],
                                   ids=["silu_gate", "scale_after_readout", "both"])


@VARIANTS
@DECODE_MODES
def test_model_variants_decode(gate_silu, after, fused):
    """The SiLU output gate and the 1/sqrt(S) on the readout (geometry options) in every
    decode form, against the oracle in the same variant (h then holds the unit-norm q)."""
    wl = W.make("variant", 12, 1, seed=120, state_std=0.02, conv_std=1.0)
    wl.gate_silu, wl.scale_after_readout = gate_silu, after
    log(f"variant silu={gate_silu} after={after} fused={fused}")
    res = oracle.run_workload(wl)
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    _compare_all(gm, wl, res, "variant", keys=("y", "h") if fused == "one" else ("o", "y", "h"))


@VARIANTS
@FUSED
def test_model_variants_multi_token_ragged(gate_silu, after, fused):
    """The variants in the multi-token kernel with ragged counts (small geometry)."""
    wl = W.make("variant_ragged", 5, 11, seed=121, geom=W.Geom(h_k=2, h_v=6), state_std=0.02, conv_std=1.0,
                ragged_max=11)
    wl.gate_silu, wl.scale_after_readout = gate_silu, after
    log(f"variant ragged silu={gate_silu} after={after} fused={fused}")
    res = oracle.run_workload(wl)
    gm = GpuMixer(wl)
    gm.run(fused=fused)
    _compare_all(gm, wl, res, "variant ragged")


@VARIANTS
def test_model_variants_keep_the_bitwise_identities(gate_silu, after):
    """Within a variant, the single launch equals the two calls, the fused norm equals the
    separate norm, and a T-token call equals the same tokens one call at a time."""
    import torch
    wl = W.make("variant_bits", 6, 1, seed=122, geom=W.Geom(h_k=2, h_v=6), state_std=0.02, conv_std=1.0)
    wl.gate_silu, wl.scale_after_readout = gate_silu, after
    outs = {}
    for mode in (False, True, "one"):
        gm = GpuMixer(wl)
        gm.run(fused=mode)
        outs[mode] = (gm.y.clone(), gm.pool.state.clone())
    assert torch.equal(outs[False][0], outs[True][0]) and torch.equal(outs[True][0], outs["one"][0])
    assert torch.equal(outs[False][1], outs["one"][1])
    wl2 = W.make("variant_chunks", 3, 7, seed=123, geom=W.Geom(h_k=2, h_v=6), state_std=0.02, conv_std=1.0)
    wl2.gate_silu, wl2.scale_after_readout = gate_silu, after
    a, b = GpuMixer(wl2), GpuMixer(wl2)
    a.run(fused=True)
    for t0, t1 in ((0, 1), (1, 4), (4, 7)):
        b.run(t0, t1, fused=True)
    assert torch.equal(a.y, b.y) and torch.equal(a.pool.state, b.pool.state)
