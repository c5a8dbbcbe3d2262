"""Checks that pin an attention implementation to facts other than its own code.

Each ``pin_*`` takes ``attn(q, k, v, causal, scale) -> (O, LSE)`` (float64
numpy arrays, inputs [B, H, N, d]) and raises AssertionError when the
implementation disagrees with

* a closed form (constant keys, zero scale, the first causal row, N = 1),
* an invariant (shift of K, joint permutation of K and V, linearity in V,
  the large-scale limit),
* a hand-derived worked example (tests/golden/attention_cases.json),
* an independent library routine (torch's float64 scaled-dot-product attention),
* a scalar brute-force loop on tiny inputs.

The same pins run against the oracle (they must pass) and against oracle
variants with planted mistakes (each must be caught by at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: max abs err {err} > {tol}"


def pin_golden(attn):
    with open(os.path.join(GOLDEN, "attention_cases.json")) as f:
        cases = json.load(f)["cases"]
    ev = lambda x: np.array(eval(x, {"math": math}) if isinstance(x, str) else [ev(y) for y in x],
                            dtype=np.float64)
    for c in cases:
        q, k, v = (ev(c[n])[None, None] for n in ("q", "k", "v"))
        o, lse = attn(q, k, v, c["causal"], float(ev(c["scale"])))
        _close(o[0, 0], ev(c["o"]), 1e-13, c["name"] + " O")
        _close(lse[0, 0], ev(c["lse"]), 1e-13, c["name"] + " LSE")


def pin_sdpa(attn):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU."""
    rng = _rng(11)
    for causal in (False, True):
        for (B, H, N, d, scale) in ((2, 3, 37, 16, 0.25), (1, 2, 64, 8, 1.3), (1, 1, 5, 3, 3.5)):  # positive scales only: torch float64 SDPA mishandles scale < 0
            q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
            o, lse = attn(q, k, v, causal, scale)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale)
            _close(o, ref.numpy(), 1e-12, f"sdpa causal={causal} N={N}")
            # LSE from torch.logsumexp over the scores torch computes with matmul
            s = scale * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
            if causal:
                s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, f"logsumexp causal={causal} N={N}")


def pin_bruteforce(attn):
    rng = _rng(12)
    for causal in (False, True):
        for (N, d, scale) in ((1, 1, 0.5), (3, 2, 1.0), (8, 4, 0.37), (7, 3, -1.1)):
            q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
            o, lse = attn(q, k, v, causal, scale)
            ob, lb = A.bruteforce(q, k, v, causal, scale)
            _close(o, ob, 1e-13, f"bruteforce O causal={causal} N={N}")
            _close(lse, lb, 1e-13, f"bruteforce LSE causal={causal} N={N}")


def pin_constant_keys(attn):
    """All keys equal: O_i = mean of the visible V rows, LSE_i = scale*q_i.k + ln(#visible)."""
    rng = _rng(13)
    B, H, N, d, scale = 1, 2, 19, 6, 0.3
    q = rng.standard_normal((B, H, N, d))
    krow = rng.standard_normal(d)
    k = np.broadcast_to(krow, (B, H, N, d)).copy()
    v = rng.standard_normal((B, H, N, d))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, scale)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(v, axis=2) / cnt[:, None] if causal else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        _close(o, mean, 1e-12, f"constant keys O causal={causal}")
        _close(lse, scale * (q @ krow) + np.log(cnt), 1e-12, f"constant keys LSE causal={causal}")


def pin_zero_scale(attn):
    rng = _rng(14)
    B, H, N, d = 2, 1, 11, 5
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.0)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        mean = np.cumsum(v, axis=2) / cnt[:, None] if causal else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        _close(o, mean, 1e-12, f"zero scale O causal={causal}")
        _close(lse, np.broadcast_to(np.log(cnt), lse.shape), 1e-12, f"zero scale LSE causal={causal}")


def pin_first_row_and_single_token(attn):
    """Causal row 0 sees key 0 only: O_0 = V_0, LSE_0 = scale*q_0.k_0; N = 1 likewise."""
    rng = _rng(15)
    q, k, v = (rng.standard_normal((2, 2, 9, 4)) for _ in range(3))
    o, lse = attn(q, k, v, True, 0.8)
    _close(o[:, :, 0], v[:, :, 0], 1e-14, "causal row 0 O")
    _close(lse[:, :, 0], 0.8 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-13, "causal row 0 LSE")
    for causal in (False, True):
        o, lse = attn(q[:, :, :1], k[:, :, :1], v[:, :, :1], causal, 0.8)
        _close(o, v[:, :, :1], 1e-14, "N=1 O")
        _close(lse[..., 0], 0.8 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-13, "N=1 LSE")


def pin_key_shift(attn):
    """K + 1 c^T leaves O unchanged and shifts LSE_i by scale * q_i . c."""
    rng = _rng(16)
    q, k, v = (rng.standard_normal((1, 2, 13, 6)) for _ in range(3))
    c = rng.standard_normal(6)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, causal, 0.6)
        o2, l2 = attn(q, k + c, v, causal, 0.6)
        _close(o2, o1, 1e-12, f"key shift O causal={causal}")
        _close(l2 - l1, 0.6 * (q @ c), 1e-12, f"key shift LSE causal={causal}")


def pin_permutation(attn):
    """Non-causal: permuting K and V rows jointly changes nothing; permuting Q permutes O."""
    rng = _rng(17)
    q, k, v = (rng.standard_normal((1, 1, 15, 5)) for _ in range(3))
    p = rng.permutation(15)
    o1, l1 = attn(q, k, v, False, 0.9)
    o2, l2 = attn(q, k[:, :, p], v[:, :, p], False, 0.9)
    _close(o2, o1, 1e-12, "KV permutation O")
    _close(l2, l1, 1e-12, "KV permutation LSE")
    o3, l3 = attn(q[:, :, p], k, v, False, 0.9)
    _close(o3, o1[:, :, p], 1e-12, "Q permutation O")
    _close(l3, l1[:, :, p], 1e-12, "Q permutation LSE")


def pin_linearity_in_v(attn):
    rng = _rng(18)
    q, k, v1, v2 = (rng.standard_normal((1, 2, 10, 4)) for _ in range(4))
    for causal in (False, True):
        oa, _ = attn(q, k, v1, causal, 0.5)
        ob, _ = attn(q, k, v2, causal, 0.5)
        oc, _ = attn(q, k, 2.0 * v1 - 3.0 * v2, causal, 0.5)
        _close(oc, 2.0 * oa - 3.0 * ob, 1e-12, f"linearity in V causal={causal}")


def pin_large_scale(attn):
    """scale -> large: O_i tends to V at the argmax of the visible scores."""
    rng = _rng(19)
    q, k, v = (rng.standard_normal((1, 1, 12, 8)) for _ in range(3))
    s = q[0, 0] @ k[0, 0].T
    for causal in (False, True):
        s2 = np.where(np.tril(np.ones_like(s)) > 0, s, -np.inf) if causal else s
        top = np.sort(s2, axis=1)
        gap = top[:, -1] - np.where(np.isfinite(top[:, -2]), top[:, -2], top[:, -1] - 10)
        assert gap.min() > 1e-3  # tie-free draw
        o, _ = attn(q, k, v, causal, 1e5)
        _close(o[0, 0], v[0, 0][np.argmax(s2, axis=1)], 1e-9, f"large scale causal={causal}")


ALL_PINS = [pin_golden, pin_sdpa, pin_bruteforce, pin_constant_keys, pin_zero_scale,
            pin_first_row_and_single_token, pin_key_shift, pin_permutation,
            pin_linearity_in_v, pin_large_scale]


def failing_pins(attn):
    """Names of the pins that reject ``attn`` (exceptions count as rejections)."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except Exception:  # noqa: BLE001 -- any failure is a detection
            bad.append(pin.__name__)
    return bad
