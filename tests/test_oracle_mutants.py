"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins in tests/pins.py reject every one of them."""
import numpy as np
import pytest

from tests import pins


def _make(score=None, mask=None, lse=None, out=None, norm_axis=1):
    """An oracle variant: the default arguments reproduce the correct definition."""
    score = score or (lambda q, k, scale: scale * (q @ k.T))
    mask = mask or (lambda n: np.triu(np.ones((n, n), dtype=bool), 1))
    lse = lse or (lambda m, l: m + np.log(l))
    out = out or (lambda p, v: p @ v)

    def attn(q, k, v, causal, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, d = q.shape
        o = np.empty((B, H, N, v.shape[-1]))
        ls = np.empty((B, H, N))
        for b in range(B):
            for h in range(H):
                s = score(q[b, h], k[b, h], scale)
                if causal:
                    s = np.where(mask(N), -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=norm_axis, keepdims=True)
                o[b, h] = out(e / l, v[b, h])
                ls[b, h] = lse(m, l)[:, 0] if np.ndim(lse(m, l)) == 2 else lse(m, l)
        return o, ls
    return attn


MUTANTS = {
    "correct": _make(),
    "mask_includes_diagonal": _make(mask=lambda n: np.triu(np.ones((n, n), dtype=bool), 0)),
    "mask_transposed": _make(mask=lambda n: np.tril(np.ones((n, n), dtype=bool), -1)),
    "mask_off_by_two": _make(mask=lambda n: np.triu(np.ones((n, n), dtype=bool), 2)),
    "scale_dropped": _make(score=lambda q, k, scale: q @ k.T),
    "scale_squared": _make(score=lambda q, k, scale: scale * scale * (q @ k.T)),
    "scale_sqrt": _make(score=lambda q, k, scale: np.sqrt(abs(scale)) * (q @ k.T)),
    "sign_flipped": _make(score=lambda q, k, scale: -scale * (q @ k.T)),
    "scores_transposed": _make(score=lambda q, k, scale: scale * (k @ q.T)),
    "normalised_over_queries": _make(norm_axis=0),
    "lse_missing_max": _make(lse=lambda m, l: np.log(l)),
    "lse_missing_log_sum": _make(lse=lambda m, l: m),
    "lse_base2": _make(lse=lambda m, l: m + np.log2(l)),
    "output_transposed_probs": _make(out=lambda p, v: p.T @ v),
    "output_unnormalised": _make(out=lambda p, v: (p / p.max(axis=1, keepdims=True)) @ v),
    "value_rows_reversed": _make(out=lambda p, v: p @ v[::-1]),
}


def test_correct_variant_passes_every_pin():
    assert pins.failing_pins(MUTANTS["correct"]) == []


@pytest.mark.parametrize("name", [n for n in MUTANTS if n != "correct"])
def test_planted_mistake_is_caught(name):
    assert pins.failing_pins(MUTANTS[name]), f"no pin rejects the planted mistake {name!r}"
