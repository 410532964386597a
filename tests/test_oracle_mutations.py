"""The oracle's pins against planted mistakes (CPU only).

Each case below plants one plausible mistake in a copy of ``oracle/gdn_oracle.c``
(a dropped term, a wrong sign, index or operand, a transposed read, a wrong
constant), builds that copy with the oracle's own gcc line, and runs the pin tests
(``tests/test_oracle_pins.py``) against it in a child process: some pin must fail.
The unmodified source, built the same way, must pass them all.  The source file
itself is never touched."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the source, its replacement); each text occurs exactly once
MUTATIONS = [
    ("sigmoid of -x", "return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    ("softplus growing tail", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("conv taps reversed", "for (int j = 0; j < hist; ++j) u += w[j] * X[j];\n            u += w[hist] * x[c];",
     "for (int j = 0; j < hist; ++j) u += w[hist - j] * X[j];\n            u += w[0] * x[c];"),
    ("history rolls the pre-activation", "if (hist > 0) X[hist - 1] = x[c];", "if (hist > 0) X[hist - 1] = u;"),
    ("history not rolled", "for (int j = 0; j + 1 < hist; ++j) X[j] = X[j + 1];", "(void) 0;"),
    ("v normalised too", "for (int part = 0; part < 2; ++part) {", "for (int part = 0; part < 3; ++part) {"),
    ("L2 norm without eps", "const double inv = 1.0 / sqrt(ss + eps);", "const double inv = 1.0 / sqrt(ss);"),
    ("q scale missing", "for (int64_t e = 0; e < (int64_t) h_k * s; ++e) out[e] *= qscale;", "(void) qscale;"),
    ("q scale before the norm",
     "const double qscale = 1.0 / sqrt((double) s);\n            for (int64_t e = 0; e < (int64_t) h_k * s; ++e) out[e] *= qscale;",
     "const double qscale = 1.0 / (double) s;\n            for (int64_t e = 0; e < (int64_t) h_k * s; ++e) out[e] *= qscale;"),
    ("dt dropped from the gate", "gate[e] = softplus(alpha[e] + dt[i]) * ssm_a[i];", "gate[e] = softplus(alpha[e]) * ssm_a[i];"),
    ("gate sign", "gate[e] = softplus(alpha[e] + dt[i]) * ssm_a[i];", "gate[e] = -softplus(alpha[e] + dt[i]) * ssm_a[i];"),
    ("head map i mod h_k", "const int j = i / group;", "const int j = i % h_k;"),
    ("k read from the q slot", "const double* k = ht + (int64_t) h_k * s + (int64_t) j * s;",
     "const double* k = ht + (int64_t) j * s;"),
    ("no decay", "St[e] *= decay;", "St[e] *= 1.0;"),
    ("decay after the read",
     "            /* decay */\n            for (int64_t e = 0; e < (int64_t) s * s; ++e) St[e] *= decay;\n",
     "            /* decay */\n"),
    ("read transposed", "m += St[(int64_t) r * s + c] * k[r];", "m += St[(int64_t) c * s + r] * k[r];"),
    ("delta sign", "d[c] = b * (v[c] - m);", "d[c] = b * (v[c] + m);"),
    ("beta dropped", "d[c] = b * (v[c] - m);", "d[c] = (v[c] - m);"),
    ("update subtracts", "St[(int64_t) r * s + c] += k[r] * d[c];", "St[(int64_t) r * s + c] -= k[r] * d[c];"),
    ("readout with k", "acc += St[(int64_t) r * s + c] * q[r];", "acc += St[(int64_t) r * s + c] * k[r];"),
    ("sum instead of mean", "ms /= (double) s;", "ms /= 1.0;"),
    ("RMS eps outside the root", "const double inv = 1.0 / sqrt(ms + eps);", "const double inv = 1.0 / (sqrt(ms) + eps);"),
    ("SiLU gate in the default model", "const double g = gate_silu ? zz * sigmoid(zz) : sigmoid(zz);",
     "const double g = zz * sigmoid(zz);"),
    ("sigmoid where the SiLU gate belongs", "const double g = gate_silu ? zz * sigmoid(zz) : sigmoid(zz);",
     "const double g = sigmoid(zz);"),
    ("z times sigmoid(-z)", "const double g = gate_silu ? zz * sigmoid(zz) : sigmoid(zz);",
     "const double g = gate_silu ? zz * sigmoid(-zz) : sigmoid(zz);"),
    ("norm weight dropped", "y[r * s + c] = x[c] * inv * w[c] * g;", "y[r * s + c] = x[c] * inv * g;"),
    ("q scaled although the scale moved to the readout", "conv_state, h + t * C, !scale_after_readout);",
     "conv_state, h + t * C, 1);"),
    ("readout scale 1/s", "scale_after_readout ? 1.0 / sqrt((double) s) : 1.0", "scale_after_readout ? 1.0 / (double) s : 1.0"),
    ("bf16 decoded one bit short", "const uint32_t u = (uint32_t) bits << 16;", "const uint32_t u = (uint32_t) bits << 15;"),
    ("alpha from the beta weights", "a += gdn_oracle_bf16_value(w_alpha[", "a += gdn_oracle_bf16_value(w_beta["),
    ("projection weight transposed", "acc += gdn_oracle_bf16_value(w[(int64_t) j * k + e]) * x[r * k + e];",
     "acc += gdn_oracle_bf16_value(w[(int64_t) e * n + j]) * x[r * k + e];"),
    ("projection drops its last term", "for (int e = 0; e < k; ++e) acc += gdn_oracle_bf16_value(",
     "for (int e = 0; e + 1 < k; ++e) acc += gdn_oracle_bf16_value("),
]


def _build(text: str, path: str):
    src = path[:-3] + ".c"
    with open(src, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-o", path, src, "-lm"])


def _pins_pass(lib_path: str) -> bool:
    env = dict(os.environ, GDN_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode == 0


def test_mutations_are_distinct_and_each_applies_once():
    text = open(SRC).read()
    assert len({(old, new) for _, old, new in MUTATIONS}) == len(MUTATIONS)
    for name, old, new in MUTATIONS:
        assert text.count(old) == 1, name
        assert old != new, name


def test_pins_pass_on_the_source_and_catch_every_planted_mistake(tmp_path):
    text = open(SRC).read()
    cases = [("unmodified", text)] + [(name, text.replace(old, new)) for name, old, new in MUTATIONS]
    libs = []
    for n, (name, src) in enumerate(cases):
        path = str(tmp_path / f"oracle_{n}.so")
        _build(src, path)
        libs.append((name, path))
    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(lambda c: (c[0], _pins_pass(c[1])), libs))
    assert results[0] == ("unmodified", True), "the pins fail on the unmodified oracle"
    missed = [name for name, passed in results[1:] if passed]
    assert not missed, f"no pin caught: {missed}"
