"""Host-side checks of bench.py: the algorithmic byte counts behind roofline.achieved,
written out here from the tensor sizes, and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import gdn_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_decode_b256():
    import bench
    wl = W.make("b256_shape", 256, 1, seed=0)   # zero state: only the shapes matter here
    got, units = bench.algorithmic_bytes(wl)
    B, hv, S, C, K = 256, 48, 128, 10240, 3
    state = 2 * B * hv * S * S * 4                    # read + written once
    hist = 2 * B * C * K * 4                          # conv history read + written
    qkv = B * C * 4
    ab = 2 * B * hv * 4                               # alpha and beta logits
    z = y = B * hv * S * 4
    consts = C * 4 * 4 + 2 * hv * 4 + S * 4           # conv taps, dt and ssm_a, norm weight
    assert got["one"] == state + hist + qkv + ab + z + y + consts == 1_696_859_008
    h = B * C * 4
    assert got["conv"] == qkv + h + hist + C * 4 * 4 == 84_049_920
    assert got["step_norm"] == state + h + ab + 2 * hv * 4 + z + y + S * 4 == 1_633_780_608
    assert units == B * hv


def test_algorithmic_bytes_ragged_counts_only_live_tokens():
    import bench
    wl = W.make("ragged_shape", 6, 4, seed=3, n_slots=9, slot_choice="random", ragged_max=4)
    got, units = bench.algorithmic_bytes(wl)
    tok = int(wl.n_tok.sum())
    assert units == tok * 48
    full = W.make("full_shape", 6, 4, seed=3, n_slots=9, slot_choice="random")
    got_full, _ = bench.algorithmic_bytes(full)
    # fewer live tokens: less h, qkv and alpha/beta traffic; the state still once per sequence
    assert got["step"] < got_full["step"]
    dropped = (6 * 4 - tok) * (10240 * 4 + 2 * 48 * 4)
    assert got_full["step"] - got["step"] == dropped


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
