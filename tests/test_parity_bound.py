"""The parity bound shared by the GPU tests (tests/parity.py), checked on the CPU: its
two anchor values, its shape, and that its helpers catch the mistakes they exist for."""
import numpy as np
import pytest

from parity import assert_close, assert_exact, assert_tokens, tol


def test_anchor_values_and_linearity():
    assert tol(1) == pytest.approx(1e-4, rel=1e-15)
    assert tol(512) == pytest.approx(1e-3, rel=1e-15)
    steps = np.arange(1, 513)
    vals = np.array([tol(int(n)) for n in steps])
    assert np.all(np.diff(vals) > 0)
    assert np.allclose(np.diff(vals), 9e-4 / 511, rtol=1e-9)
    with pytest.raises(ValueError):
        tol(0)


def test_assert_close_is_relative_to_max_ref():
    ref = np.array([1.0, -2.0, 0.5])
    assert_close("ok", ref + np.array([0.0, 1.9e-4, 0.0]), ref, 1)       # 0.95e-4 x 2
    with pytest.raises(AssertionError):
        assert_close("bad", ref + np.array([0.0, 2.1e-4, 0.0]), ref, 1)
    assert_close("two steps later", ref + np.array([0.0, 2.0035e-4, 0.0]), ref, 2)
    with pytest.raises(AssertionError):
        assert_close("nan", np.array([np.nan, 0, 0]), ref, 1)


def test_assert_tokens_uses_each_tokens_own_bound():
    """Token t is held to tol(t + 1) against its own max |ref|; an error that the last
    token's bound would hide is still caught at the first token; skipped tokens must be
    zero."""
    rng = np.random.default_rng(0)
    ref = [rng.standard_normal((6, 4)) for _ in range(3)]
    gpu = np.stack(ref).copy()
    assert_tokens("clean", gpu, ref, [6, 6, 6])
    bad = gpu.copy()
    bad[1, 0, 2] += 3e-4 * np.abs(np.stack(ref)[:, 0]).max()   # inside tol(6), outside tol(1)
    with pytest.raises(AssertionError, match="token 0"):
        assert_tokens("first token", bad, ref, [6, 6, 6])
    late = gpu.copy()
    late[1, 5, 2] += 1.0e-4 * np.abs(np.stack(ref)[:, 5]).max()   # inside tol(6)
    assert_tokens("last token", late, ref, [6, 6, 6])
    ragged = gpu.copy()
    ragged[2, 4:] = 0.0
    assert_tokens("ragged", ragged, [ref[0], ref[1], ref[2][:4]], [6, 6, 4])
    ragged[2, 5, 0] = 1.0
    with pytest.raises(AssertionError, match="skipped"):
        assert_tokens("ragged tail", ragged, [ref[0], ref[1], ref[2][:4]], [6, 6, 4])
    # h: no recurrence, every token at tol(1)
    with pytest.raises(AssertionError):
        assert_tokens("h", late, ref, [6, 6, 6], recurrent=False)


def test_assert_exact():
    a = np.arange(6, dtype=np.float32).reshape(2, 3)
    assert_exact("same", a, a.astype(np.float64))
    b = a.copy()
    b[1, 2] = np.nextafter(b[1, 2], np.float32(100))
    with pytest.raises(AssertionError):
        assert_exact("one ulp", b, a)
