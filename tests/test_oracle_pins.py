"""CPU tests: the fp64 oracle against its pins (worked examples, closed forms,
brute force, invariants, chunked re-expressions). See tests/oracle_pins.py."""
import numpy as np
import pytest

import kda_synth
import oracle_pins as P


@pytest.mark.parametrize("case", P.golden_cases(), ids=lambda c: c["name"])
def test_golden_worked_example(ref, case):
    P.check_golden_case(ref, case)


@pytest.mark.parametrize("check", [c for c in P.ALL_CHECKS if c is not P.check_golden],
                         ids=lambda c: c.__name__)
def test_pin(ref, check):
    check(ref)


def test_scalar_decay_closed_form(ref):
    """0.9^20 exactly, beyond the page's two printed digits (ten-questions page, Q8)."""
    T = 20
    o, hT = ref(np.ones((T, 1, 1)), np.ones((T, 1, 1)), np.zeros((T, 1, 1)),
                np.full((T, 1, 1), np.log(0.9)), np.zeros((T, 1)), 1.0,
                h0=np.ones((1, 1, 1, 1)))
    assert abs(hT[0, 0, 0, 0] - 0.9 ** 20) < 1e-15
    assert abs(0.9 ** 20 - 0.12) < 0.005


def test_generator_squashing_matches_page_values():
    """The gate squashing used by the input recipes, against the values the
    ten-questions page prints in Q9 (to its printed precision)."""
    assert kda_synth.sigmoid(0.0) == 0.5
    assert abs(kda_synth.sigmoid(4.0) - 0.98) < 0.005
    assert abs(kda_synth.sigmoid(-4.0) - 0.02) < 0.005
    assert abs(kda_synth.softplus(-5.0) - 0.007) < 0.0005
    assert abs(kda_synth.softplus(5.0) - 5.007) < 0.0005


def test_generator_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties go to even
    ours = kda_synth.round_bf16(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), theirs.view(np.uint32))


def test_generator_is_seeded_and_normalised():
    a = kda_synth.gen_sequences((33, 7), 2, 8, 4, "bf16", "main", "normal", 5)
    b = kda_synth.gen_sequences((33, 7), 2, 8, 4, "bf16", "main", "normal", 5)
    for key in ("q", "k", "v", "log_alpha", "beta", "h0"):
        assert np.array_equal(a[key], b[key])
    assert list(a["cu_seqlens"]) == [0, 33, 40]
    assert np.allclose(np.linalg.norm(a["k"], axis=-1), 1.0, atol=1e-2)  # bf16-rounded unit keys
    assert np.all(a["log_alpha"] < 0) and np.all((a["beta"] > 0) & (a["beta"] < 1))
