"""A seeded sweep of shapes against the fp64 oracle: geometries of the family (qk heads
and GQA group sizes, including groups the single launch runs head by head), batch
sizes, token counts across several conv blocks with ragged tails, per-sequence token
counts (zero included), pools larger than the batch with random slots, zero and
filled states, and every call form.  Tolerance: the one bound of tests/parity.py (o and
y of token t at tol(t + 1), h at tol(1), states at tol(the most tokens a sequence took),
1e-4 for one step growing linearly to 1e-3 at 512); the conv history and untouched
slots bit for bit."""
import numpy as np
import pytest

import gdn_workloads as W
import oracle
from gpu_harness import GpuMixer, assert_close, assert_exact, assert_tokens, log

pytestmark = pytest.mark.gpu

GEOMS = [(1, 1), (1, 3), (2, 2), (2, 3), (3, 5), (4, 1), (4, 4), (2, 14), (16, 3)]


def _case(k):
    rng = np.random.default_rng(9000 + k)
    h_k, g = GEOMS[(k + k // 3) % len(GEOMS)]
    B = int(rng.integers(1, 10))
    T = 1 if k % 3 == 2 else int(rng.choice([1, 2, 3, 7, 9, 16, 33, 40]))
    ragged = bool(rng.integers(0, 2)) and T > 1
    form = "one" if k % 3 == 2 else str(rng.choice(["3calls", "fused_norm"]))
    return dict(h_k=h_k, h_v=h_k * g, B=B, T=T, ragged=ragged, form=form,
                n_slots=B + int(rng.integers(0, 6)), state_std=float(rng.choice([0.0, 0.02, 0.1])),
                conv_std=float(rng.choice([0.0, 1.0])), seed=int(rng.integers(1, 1 << 30)))


@pytest.mark.parametrize("k", range(27))
def test_random_shape_against_oracle(k):
    import torch
    c = _case(k)
    log(f"random shape {k}: {c}")
    geom = W.Geom(h_k=c["h_k"], h_v=c["h_v"])
    wl = W.make(f"rand{k}", c["B"], c["T"], c["seed"], geom=geom, n_slots=c["n_slots"], state_std=c["state_std"],
                conv_std=c["conv_std"], slot_choice="random", ragged_max=c["T"] if c["ragged"] else None)
    if c["ragged"]:
        # some sequences with no token at all
        wl.n_tok[np.random.default_rng(c["seed"]).random(c["B"]) < 0.2] = 0
    res = oracle.run_workload(wl)
    gm = GpuMixer(wl)
    fused = {"3calls": False, "fused_norm": True, "one": "one"}[c["form"]]
    gm.run(fused=fused)
    torch.cuda.synchronize()
    keys = ("y", "h") if fused == "one" else ("o", "y", "h")
    counts = [wl.tokens_of(b) for b in range(wl.B)]
    for key in keys:
        assert_tokens(f"rand{k} {key}", getattr(gm, key).cpu().numpy(), [r[key] for r in res], counts,
                      recurrent=key != "h")
    st = gm.pool.state.cpu().numpy()
    cv = gm.pool.conv.cpu().numpy()
    assert_close(f"rand{k} state", st[wl.slots], np.stack([r["state"] for r in res]), max(1, max(counts)))
    assert_exact(f"rand{k} conv", cv[wl.slots], np.stack([r["conv_state"] for r in res]))
    untouched = np.setdiff1d(np.arange(wl.n_slots), wl.slots)
    assert np.array_equal(st[untouched], wl.state[untouched])
    assert np.array_equal(cv[untouched], wl.conv_state[untouched])
    assert int(gm.pool.flags.item()) == 0
