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
