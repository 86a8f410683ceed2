"""The CPU oracle against its pins (hand-worked values, brute force, torch float64,
closed forms, invariants). CPU only."""
import numpy as np
import pytest

import oracle
from pins import BLOCK_PINS, EXT_PINS, GN_PINS, TRAIN_PINS, block_brute_config0, _rand_block


@pytest.mark.parametrize("pin", BLOCK_PINS, ids=lambda f: f.__name__)
def test_block_pin(pin):
    ok, msg = pin(oracle.prenorm_block)
    assert ok, msg


def test_block_brute_config0():
    ok, msg = block_brute_config0(oracle.prenorm_block)
    assert ok, msg


@pytest.mark.parametrize("pin", EXT_PINS, ids=lambda f: f.__name__)
def test_external_bn_pin(pin):
    ok, msg = pin(oracle.relu_conv_residual)
    assert ok, msg


@pytest.mark.parametrize("pin", TRAIN_PINS, ids=lambda f: f.__name__)
def test_train_pin(pin):
    ok, msg = pin(oracle.prenorm_block_train)
    assert ok, msg


@pytest.mark.parametrize("pin", GN_PINS, ids=lambda f: f.__name__)
def test_gn_pin(pin):
    ok, msg = pin(oracle.conv_groupnorm)
    assert ok, msg


@pytest.mark.parametrize("d", [1, 3, 64, 127, 128, 200])
def test_points_match_full(d):
    """The point-wise evaluator (used at full sizes) agrees with the full oracle,
    including the first and last d outputs where the outer taps are padding."""
    p = _rand_block(2, 12, 200, 80 + d, beta_shift=0.3)
    full = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                p["beta"], p["eps"], p["W"], p["b"], d)
    rng = np.random.default_rng(d)
    pts = [(n, c, t) for n in range(2) for c in (0, 11) for t in (0, d - 1, d, 199 - d, 200 - d, 199)
           if 0 <= t < 200]
    pts += [tuple(rng.integers(0, s) for s in (2, 12, 200)) for _ in range(40)]
    got = oracle.prenorm_block_points(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                      p["beta"], p["eps"], p["W"], p["b"], d, pts)
    exp = np.array([full[n, c, t] for (n, c, t) in pts])
    assert np.max(np.abs(got - exp)) <= 1e-12


def test_output_length_formula():
    assert oracle.conv_output_length(4096, 128, 128) == 4096
    assert oracle.conv_output_length(1024, 1, 1) == 1024
    assert oracle.conv_output_length(10, 0, 2) == 6
    assert oracle.conv_output_length(10, 3, 1) == 14
