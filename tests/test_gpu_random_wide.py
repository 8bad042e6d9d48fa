"""GPU parity against the fp64 oracle over seeded random configurations with
wide magnitudes: the configurations of test_gpu_random_configs' generator
(its own seed), with the initial state, the final state's gradient and a
drawn over wider ranges (standard deviations up to 5, 5 and 2). A large a
puts the gate argument z over several units, where the gate terms of dq, dk
and da carry much of their RMS; such draws found the bf16 rounding of a and
a (.) q that the gate used to have. Each case runs the forward and backward
and, for bf16, the forward with the epilogue before the store."""
import numpy as np
import pytest

import tests.test_gpu_random_configs as RC

pytestmark = pytest.mark.gpu


def _wide_cases(n=64, seed=7310):
    cases = RC._cases(n, seed)
    rng = np.random.default_rng(seed + 99)
    for c in cases:
        c["s0_std"] = [None, 0.05, 1.0, 5.0][int(rng.integers(0, 4))]
        c["dsf_std"] = [None, 0.05, 1.0, 5.0][int(rng.integers(0, 4))]
        c["a_std"] = [None, 0.1, 1.0, 2.0][int(rng.integers(0, 4))]
    return cases


WIDE = _wide_cases()


def _wname(c):
    return f"{RC._name(c)}-s0{c['s0_std']}-dsf{c['dsf_std']}-a{c['a_std']}"


@pytest.mark.parametrize("case", WIDE, ids=[_wname(c) for c in WIDE])
def test_random_wide_fwd_bwd(case):
    RC.test_random_config_fwd_bwd(case)


WIDE_BF16 = [c for c in WIDE if c["dtype"] == "bf16"]


@pytest.mark.parametrize("case", WIDE_BF16, ids=[_wname(c) for c in WIDE_BF16])
def test_random_wide_fwd_norm_gate(case):
    RC.test_random_config_fwd_norm_gate(case)
