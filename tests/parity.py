"""The one parity bound every GPU test applies, and the record of the margins achieved.

The bound comes from the decode mixer's stated tolerances: for each of o, y, the state
and the conv history, max |gpu - ref| <= 1e-4 x max |ref| per decode step, and
<= 1e-3 x max |ref| after 512 sequential steps.  It is read as one function of n, the
number of sequential steps between the seeded inputs and the value compared:

    tol(n) = 1e-4 + 9e-4 * (n - 1) / 511        (1e-4 at n = 1, 1e-3 at n = 512)

n is counted per compared value:
  * o and y of token t of a sequence (0-based, counted from the state the test seeded):
    n = t + 1, each token of the recurrence being one step;
  * the state of a sequence after it took n_b tokens: n = n_b;
  * h (conv + SiLU + L2 norm of raw inputs; no recurrence feeds it): n = 1 at every token;
  * a projection's output: n = 1; in a chain, every product before or after the mixer
    adds one step to what follows it (x -> qkv -> one mixer token -> out: n = 3 for out);
  * the conv history holds raw inputs that are only moved, so it is compared bit for bit.

The ratio is taken against max |ref| over the values compared together: every token
index of o and y on its own (the sequences that have that token), the states of one
call together, a projection's whole output.

Every comparison appends {test, what, steps, rel_err, tol} to the JSON-lines file named
by the environment variable GDN_PARITY_LOG (when it is set), failures included, so a
GPU run leaves the achieved margins behind.
"""
from __future__ import annotations

import json
import os

import numpy as np


def tol(n: int) -> float:
    """Relative bound for a value n sequential steps from the seeded inputs."""
    if n < 1:
        raise ValueError(f"steps must be >= 1, not {n}")
    return 1e-4 + 9e-4 * (n - 1) / 511


def _record(what: str, steps, rel_err: float, bound):
    path = os.environ.get("GDN_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps({"test": test, "what": what, "steps": steps, "rel_err": rel_err,
                            "tol": bound}) + "\n")


def assert_close(name: str, gpu, ref, steps: int = 1):
    """max |gpu - ref| <= tol(steps) x max |ref| over the whole array; returns the ratio
    max |gpu - ref| / max |ref|."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite values from the GPU"
    m = float(np.abs(r).max()) if r.size else 0.0
    err = float(np.abs(g - r).max()) if r.size else 0.0
    rel = err / m if m else 0.0
    bound = tol(steps)
    _record(name, steps, rel, bound)
    assert err <= bound * m, f"{name}: max abs err {err:.3e} > {bound:.3e} x max|ref| ({m:.3e}), {steps} steps"
    return rel


def assert_exact(name: str, gpu, ref):
    """Bit-for-bit equality of values that are only moved (the conv history)."""
    g = np.asarray(gpu)
    r = np.asarray(ref)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    equal = np.array_equal(g.astype(np.float64), r.astype(np.float64))
    _record(name, None, 0.0 if equal else float(np.abs(g.astype(np.float64) - r).max()), 0.0)
    assert equal, f"{name}: not bit for bit equal ({int((g != r).sum())} values differ)"


def assert_tokens(name: str, gpu, refs, counts, first_step: int = 1, recurrent: bool = True):
    """Per token index: gpu [B][T][...] against refs (one [n_b][...] array per sequence,
    n_b = counts[b] tokens), token t of every sequence that has it compared together at
    tol(first_step + t) (first_step - 1 steps ran before this call's token 0), or at
    tol(1) for every token when the value does not come out of the recurrence
    (recurrent=False: h).  Tokens past a sequence's count must be zero.  Returns the
    largest ratio over the tokens and the largest share of its bound any token used."""
    gpu = np.asarray(gpu)
    T = gpu.shape[1]
    worst_rel, worst_use, worst = 0.0, 0.0, None
    for b, n in enumerate(counts):
        assert (gpu[b, n:] == 0).all(), f"{name}: outputs of skipped tokens of sequence {b} are not zero"
    for t in range(T):
        seqs = [b for b, n in enumerate(counts) if n > t]
        if not seqs:
            continue
        g = gpu[seqs, t].astype(np.float64)
        r = np.stack([np.asarray(refs[b])[t] for b in seqs]).astype(np.float64)
        assert np.isfinite(g).all(), f"{name}: non-finite values from the GPU at token {t}"
        m = float(np.abs(r).max())
        err = float(np.abs(g - r).max())
        rel = err / m if m else 0.0
        steps = first_step + t if recurrent else 1
        bound = tol(steps)
        if rel >= worst_rel:
            worst_rel = rel
        if rel / bound >= worst_use:
            worst_use, worst = rel / bound, (t, rel, bound, steps)
        if not err <= bound * m:
            _record(f"{name} (token {t}, over its bound)", steps, rel, bound)
            raise AssertionError(f"{name}: token {t}: max abs err {err:.3e} > {bound:.3e} x max|ref| "
                                 f"({m:.3e}), {steps} steps")
    if worst is not None:
        _record(f"{name} (token {worst[0]}, the token closest to its bound)", worst[3], worst[1], worst[2])
    return worst_rel, worst_use
