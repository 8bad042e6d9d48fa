"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that
the pins catch every one of them.

Each mutation is a textual replacement in oracle.c; the mutated copy is built
into a temporary shared library and every pin is run against it. A mutation
that no pin detects fails this test.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to find, replacement); the find text must occur exactly once.
MUTATIONS = [
    ("no decay in update (fwd)",
     "S[(size_t)i * d_v + j] = lam * S[(size_t)i * d_v + j] + kt[i] * vt[j];\n            }\n        }\n        /* o_t",
     "S[(size_t)i * d_v + j] = S[(size_t)i * d_v + j] + kt[i] * vt[j];\n            }\n        }\n        /* o_t"),
    ("readout uses k instead of q", "acc += S[(size_t)i * d_v + j] * qt[i];",
     "acc += S[(size_t)i * d_v + j] * kt[i];"),
    ("sigmoid sign flipped", "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    ("gate uses q twice", "z += a[i] * qt[i] * kt[i];", "z += a[i] * qt[i] * qt[i];"),
    ("aug term dropped (fwd)", "ot[j] = acc + g * vt[j];", "ot[j] = acc;"),
    ("outer product transposed index", "= lam * S[(size_t)i * d_v + j] + kt[i] * vt[j];\n            }\n        }\n        /* o_t",
     "= lam * S[(size_t)i * d_v + j] + kt[j % d_k] * vt[j];\n            }\n        }\n        /* o_t"),
    ("schedule exponent H instead of H-1", "(double)h / (double)(H - 1)", "(double)h / (double)H"),
    ("schedule base e instead of 2", "lam[h] = pow(2.0, -1.0 / half_life);", "lam[h] = exp(-1.0 / half_life);"),
    ("dq aug uses q", "dqt[i] = acc + ((a != NULL) ? c * a[i] * kt[i] : 0.0);",
     "dqt[i] = acc + ((a != NULL) ? c * a[i] * qt[i] : 0.0);"),
    ("no decay of G", "G[e] *= lam;", "G[e] *= 1.0;"),
    ("G accumulates k dO^T", "G[(size_t)i * d_v + j] += qt[i] * dot[j];", "G[(size_t)i * d_v + j] += kt[i] * dot[j];"),
    ("dS0 not decayed", "dS0[e] = (T > 0) ? lam * G[e] : G[e];", "dS0[e] = G[e];"),
    ("dv aug sigma' instead of sigma", "dvt[j] = acc + s * dot[j];", "dvt[j] = acc + s * (1.0 - s) * dot[j];"),
    ("da uses q twice", "da[i] += c * qt[i] * kt[i];", "da[i] += c * qt[i] * qt[i];"),
    ("da only when a is given", "da[i] += c * qt[i] * kt[i];",
     "if (a != NULL) da[i] += c * qt[i] * kt[i];"),
    ("gate argument at a = NULL is one", "    if (a == NULL) {\n        return 0.0;",
     "    if (a == NULL) {\n        return 1.0;"),
    ("dk aug sign", "dkt[i] = acc + ((a != NULL) ? c * a[i] * qt[i] : 0.0);",
     "dkt[i] = acc - ((a != NULL) ? c * a[i] * qt[i] : 0.0);"),
    ("dv reads G transposed wrong", "acc += G[(size_t)i * d_v + j] * kt[i];", "acc += G[(size_t)i * d_v + j] * qt[i];"),
    ("decode no decay", "S[(size_t)i * d_v + j] = lam * S[(size_t)i * d_v + j] + k[i] * v[j];",
     "S[(size_t)i * d_v + j] = S[(size_t)i * d_v + j] + k[i] * v[j];"),
    ("decode gate off", "o[j] = acc + g * v[j];", "o[j] = acc + 0.5 * v[j];"),
    ("conv taps reversed", "acc += w[(size_t)c * 4 + j] * x;", "acc += w[(size_t)c * 4 + (3 - j)] * x;"),
    ("conv bias dropped", "double acc = (b != NULL) ? b[c] : 0.0;\n            for (int j = 0; j < 4; ++j) {",
     "double acc = 0.0;\n            for (int j = 0; j < 4; ++j) {"),
    ("conv history ignored", "x = (st != NULL) ? st[(size_t)(3 + s) * D + c] : 0.0;\n                }\n                acc +=",
     "x = 0.0;\n                }\n                acc +="),
    ("silu is sigmoid", "return x * sigmoid(x);", "return sigmoid(x);"),
    ("conv final state one token early", "const int s = L - 3 + j;", "const int s = L - 4 + j;"),
    ("conv decode state not shifted", "st[c] = st[(size_t)D + c];", "st[c] = st[c];"),
    ("conv decode tap 2 reads x", "acc += w[(size_t)c * 4 + 2] * st[(size_t)2 * D + c];",
     "acc += w[(size_t)c * 4 + 2] * x[c];"),
    ("norm eps dropped", "inv_rms = 1.0 / sqrt(ss / d_v + eps)", "inv_rms = 1.0 / sqrt(ss / d_v)"),
    ("norm eps outside the root", "1.0 / sqrt(ss / d_v + eps)", "1.0 / (sqrt(ss / d_v) + eps)"),
    ("norm sums instead of averaging", "inv_rms = 1.0 / sqrt(ss / d_v + eps)", "inv_rms = 1.0 / sqrt(ss + eps)"),
    ("norm tier by head modulo", "const double inv_rms = 1.0 / sqrt(ss / d_v + eps);\n        const int tier = h / per_tier;",
     "const double inv_rms = 1.0 / sqrt(ss / d_v + eps);\n        const int tier = h % n_tiers;"),
    ("norm gamma transposed", "const double scale = (gamma != NULL) ? gamma[(size_t)tier * d_v + c] : 1.0;",
     "const double scale = (gamma != NULL) ? gamma[(size_t)c * n_tiers + tier] : 1.0;"),
    ("norm bwd tier by head modulo", "const double r = sqrt(ss / d_v + eps);\n        const int tier = h / per_tier;",
     "const double r = sqrt(ss / d_v + eps);\n        const int tier = h % n_tiers;"),
    ("norm gate sigmoid instead of silu", "out[(size_t)h * d_v + c] = silu(gc) *",
     "out[(size_t)h * d_v + c] = sigmoid(gc) *"),
    ("norm gate dropped", "out[(size_t)h * d_v + c] = silu(gc) *", "out[(size_t)h * d_v + c] = 1.0 *"),
    ("conv bwd silu' without the x term", "dpre[t] = dy[(size_t)t * D + c] * sg * (1.0 + pre * (1.0 - sg));",
     "dpre[t] = dy[(size_t)t * D + c] * sg * (1.0 - sg);"),
    ("conv bwd taps not flipped", "g += w[(size_t)c * 4 + j] * dpre[t];", "g += w[(size_t)c * 4 + (3 - j)] * dpre[t];"),
    ("conv bwd final-state gradient dropped", "g += d_st_out[(size_t)i * D + c];", "g += 0.0;"),
    ("conv bwd dw from the wrong input", "dw[(size_t)c * 4 + j] += dpre[t] * x[t + j];",
     "dw[(size_t)c * 4 + j] += dpre[t] * x[t + 3];"),
    ("conv bwd history ignored", "x[s + 3] = (s >= 0) ? u[(size_t)s * D + c] : ((st != NULL) ? st[(size_t)(3 + s) * D + c] : 0.0);",
     "x[s + 3] = (s >= 0) ? u[(size_t)s * D + c] : 0.0;"),
    ("norm bwd eps dropped", "const double r = sqrt(ss / d_v + eps);", "const double r = sqrt(ss / d_v);"),
    ("norm bwd silu' without the x term", "sg * (1.0 + g[i] * (1.0 - sg))", "sg * (1.0 - sg)"),
    ("norm bwd projection dropped", "d_o[i] = (w - (oh[c] / r) * (wy / d_v)) / r;", "d_o[i] = w / r;"),
    ("norm bwd dgamma without the gate", "dgamma[(size_t)tier * d_v + c] += dout[i] * s * y;",
     "dgamma[(size_t)tier * d_v + c] += dout[i] * y;"),
    ("norm bwd dg without gamma", "dg[i] = dout[i] * gm * y *", "dg[i] = dout[i] * y *"),
]


@pytest.mark.parametrize("name,find,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, find, repl, tmp_path):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for '{name}' not unique ({src.count(find)})"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(find, repl))
    hdr_dir = os.path.dirname(SRC)
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-I", hdr_dir,
                           "-o", str(so), str(mutated), "-lm"])
    good = oracle._load()
    bad = ctypes.CDLL(str(so))
    for fn in ("orc_decay_schedule", "orc_fwd", "orc_bwd", "orc_decode_step", "orc_conv_fwd",
               "orc_conv_decode_step", "orc_head_norm_gate", "orc_head_norm_gate_bwd", "orc_conv_bwd"):
        getattr(bad, fn).argtypes = getattr(good, fn).argtypes
        getattr(bad, fn).restype = None
    caught = []
    oracle._lib = bad
    try:
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except AssertionError:
                caught.append(check.__name__)
    finally:
        oracle._lib = good
    assert caught, f"no pin detects the planted mistake '{name}'"


# Mistakes in the Python batch wrappers of oracle/__init__.py (slicing of
# sequences, per-sequence states, the sum of da over sequences). The mutated
# module is loaded on its own and its functions replace the package's while
# the pins run.
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
PY_MUTATIONS = [
    ("packed conv: first sequence's state for every sequence",
     "s0 = None if st is None else st[n]", "s0 = None if st is None else st[0]"),
    ("packed conv: final state of the wrong sequence",
     "y[sp[0]:sp[1]], fin[n] = conv_fwd_unit(", "y[sp[0]:sp[1]], fin[max(n - 1, 0)] = conv_fwd_unit("),
    ("packed fwd: first sequence's initial state for every sequence",
     "None if a is None else a[h], None if S0 is None else S0[n, h])",
     "None if a is None else a[h], None if S0 is None else S0[0, h])"),
    ("packed bwd: first sequence's final-state gradient for every sequence",
     "None if dSf is None else dSf[n, h])", "None if dSf is None else dSf[0, h])"),
    ("packed bwd: da of the last sequence only",
     "da[h] += da_parts[(n, h)]", "da[h] = da_parts[(n, h)]"),
    ("packed bwd: sequence slice off by one",
     "out.append((n, h, 0, slice(cu[n], cu[n + 1])))", "out.append((n, h, 0, slice(cu[n], cu[n + 1] + 1)))"),
]


@pytest.mark.parametrize("name,find,repl", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_wrapper_mutation_is_caught(name, find, repl, monkeypatch):
    import types
    src = open(PY_SRC).read()
    assert src.count(find) == 1, f"mutation site for '{name}' not unique ({src.count(find)})"
    mod = types.ModuleType("oracle_mutated")
    mod.__file__ = PY_SRC
    exec(compile(src.replace(find, repl), PY_SRC, "exec"), mod.__dict__)
    for fn in ("fwd", "bwd", "conv_fwd", "head_norm_gate", "head_norm_gate_bwd"):
        monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin detects the planted mistake '{name}'"
