"""CPU pins of the fp64 attention oracle (see tests/pins.py for what each pin fixes)."""
import functools

import numpy as np
import pytest

from oracle import attention as A
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_reference_pins(pin):
    pin(A.reference)


@pytest.mark.parametrize("block", [1, 7, 64, 1000])
@pytest.mark.parametrize("pin", [pins.pin_golden, pins.pin_sdpa, pins.pin_constant_keys, pins.pin_zero_scale,
                                 pins.pin_first_row_and_single_token, pins.pin_key_shift],
                         ids=lambda p: p.__name__)
def test_online_pins(pin, block):
    pin(functools.partial(A.online, block=block))


def test_bruteforce_golden():
    pins.pin_golden(A.bruteforce)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 64, 129])
def test_online_equals_two_pass(causal, block):
    rng = np.random.Generator(np.random.PCG64(3))
    q, k, v = (rng.standard_normal((2, 2, 129, 16)) for _ in range(3))
    o1, l1 = A.reference(q, k, v, causal, 0.25)
    o2, l2 = A.online(q, k, v, causal, 0.25, block=block)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_rows_sum_to_one(causal):
    rng = np.random.Generator(np.random.PCG64(4))
    q, k, v = (rng.standard_normal((33, 8)) for _ in range(3))
    p = A.probabilities(q, k, causal, 0.7)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(p[np.triu_indices(33, 1)] == 0.0)
    o, _ = A.reference(q[None, None], k[None, None], v[None, None], causal, 0.7)
    assert np.max(np.abs(o[0, 0] - p @ v)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_matches_full(causal):
    rng = np.random.Generator(np.random.PCG64(5))
    q, k, v = (rng.standard_normal((1, 2, 50, 8)) for _ in range(3))
    o, l = A.reference(q, k, v, causal, 0.3)
    rows = np.array([0, 1, 17, 49])
    os_, ls = A.reference(q, k, v, causal, 0.3, rows=rows)
    assert np.array_equal(os_, o[:, :, rows]) and np.array_equal(ls, l[:, :, rows])


def test_bf16_inputs_are_consumed_exactly():
    import torch
    x = torch.randn(1, 1, 4, 8).to(torch.bfloat16)
    o, _ = A.reference(x, x, x, False, 0.0)
    # zero scale -> mean of V rows, computed from the exact bf16 values
    assert np.max(np.abs(o[0, 0] - x.float().double().numpy()[0, 0].mean(axis=0))) <= 1e-15
