"""CPU pins of the oracle's attention gradients (``oracle.attention.backward``).

Pinned against central finite differences of the reference forward (brute
force), against torch's float64 autograd through its own attention routine
(library), and against two invariants that a dropped term or a transposed
operand breaks: the key gradients of a head sum to zero (a shift of every key
by the same vector leaves the softmax unchanged), and the value gradients sum
to the output gradients summed over queries (each row of P sums to one)."""
import numpy as np
import pytest
import torch

from oracle import attention as A

RNG = np.random.default_rng(77)


def _case(n, d, b=1, h=2):
    return [RNG.standard_normal((b, h, n, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    q, k, v, do = _case(5, 3, b=1, h=1)
    scale, eps = 0.7, 1e-6
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)

    def loss(q_, k_, v_):
        return float((A.reference(q_, k_, v_, causal, scale)[0] * do).sum())

    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (which, idx, fd, g[idx])


def _torch_forward(q, k, v, causal, scale):
    """Attention as torch operations (autograd differentiates these mechanically)."""
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        n = q.shape[-2]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -float("inf"))
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.125, -0.3, 0.0])
def test_torch_autograd_float64(causal, scale):
    q, k, v, do = _case(37, 16)
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    ts = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
    _torch_forward(*ts, causal, scale).backward(torch.from_numpy(do))
    for g, t in zip((dq, dk, dv), ts):
        assert np.abs(g - t.grad.numpy()).max() < 1e-10
    if scale > 0:  # torch's own attention routine (its float64 path is reliable for positive scales)
        ts = [torch.from_numpy(x).requires_grad_(True) for x in (q, k, v)]
        torch.nn.functional.scaled_dot_product_attention(*ts, is_causal=causal, scale=scale).backward(
            torch.from_numpy(do))
        for g, t in zip((dq, dk, dv), ts):
            assert np.abs(g - t.grad.numpy()).max() < 1e-10


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    q, k, v, do = _case(64, 8)
    dq, dk, dv = A.backward(q, k, v, do, causal, 0.3)
    assert np.abs(dk.sum(axis=2)).max() < 1e-10
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() < 1e-10


@pytest.mark.parametrize("causal", [False, True])
def test_given_output_equals_the_definition(causal):
    """D from the exact output (sum_c dO_ic O_ic) is D from P and dP: the same gradients."""
    q, k, v, do = _case(40, 8)
    o, _ = A.reference(q, k, v, causal, 0.3)
    a = A.backward(q, k, v, do, causal, 0.3)
    b = A.backward(q, k, v, do, causal, 0.3, o=o)
    assert all(np.abs(x - y).max() < 1e-12 for x, y in zip(a, b))


def test_given_output_moves_only_dq_dk_by_the_closed_form():
    """Moving row i of the given output by e changes D_i by dO_i . e, hence dS_i by
    -P_i (dO_i . e): dQ_i by -scale (dO_i . e) P_i K, dK by -scale (dO_i . e) P_i^T q_i,
    every other row of dQ and all of dV unchanged."""
    q, k, v, do = _case(12, 5, b=1, h=1)
    scale, i = 0.4, 7
    o, _ = A.reference(q, k, v, False, scale)
    e = RNG.standard_normal(5)
    o2 = o.copy()
    o2[0, 0, i] += e
    dq1, dk1, dv1 = A.backward(q, k, v, do, False, scale, o=o)
    dq2, dk2, dv2 = A.backward(q, k, v, do, False, scale, o=o2)
    s = scale * q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dd = float(do[0, 0, i] @ e)
    want_dq = np.zeros_like(dq1[0, 0])
    want_dq[i] = -scale * dd * (p[i] @ k[0, 0])
    want_dk = -scale * dd * np.outer(p[i], q[0, 0, i])
    assert np.abs((dq2 - dq1)[0, 0] - want_dq).max() < 1e-12
    assert np.abs((dk2 - dk1)[0, 0] - want_dk).max() < 1e-12
    assert np.abs(dv2 - dv1).max() == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_keys_equal_the_full_backward(causal):
    """backward_sampled with the exact output and LSE reproduces the rows of dQ and the
    keys' rows of dK and dV of the full backward (D from the same given output)."""
    q, k, v, do = _case(40, 8, b=1, h=1)
    scale = 0.6
    o, lse = A.reference(q, k, v, causal, scale)
    dq, dk, dv = A.backward(q, k, v, do, causal, scale, o=o)
    rows, keys = np.array([0, 1, 17, 39]), np.array([0, 5, 38, 39])
    sq, sk, sv = A.backward_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], o[0, 0], lse[0, 0], causal, scale, rows, keys)
    assert np.abs(sq - dq[0, 0, rows]).max() < 1e-12
    assert np.abs(sk - dk[0, 0, keys]).max() < 1e-12
    assert np.abs(sv - dv[0, 0, keys]).max() < 1e-12
