"""The attention forward pass, written out in float64 (test infrastructure only).

What is computed (the readings are listed in DESIGN.md under "Readings"):

  for every batch b and head h, with Q, K, V in R^{N x d}:
    S   = scale * Q K^T                           (N x N, materialised)
    S_ij = -inf for j > i                         (causal only; keys aligned with queries)
    m_i = max_j S_ij
    P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i)
    O   = P V,   LSE_i = m_i + ln sum_j exp(S_ij - m_i)

The pages describe the method only as a faster way to obtain *exactly* the
result of standard attention (FlashAttention-2 wiki page, introduction and
section "Leistung und Effizienz": identical results, exact and deterministic),
whose quadratic cost comes from the full score matrix (same page, section
"Hintergrund: Das Attention-Problem in Transformern").  So ``reference`` is
that standard definition, not the tiled algorithm.  ``online`` follows the
tiled algorithm's steps (running maximum, rescaling of the running sums,
division by the row sum only after the last key tile; page "FlashAttention-
Skalierung, Multi-GPU-Training und Gewichtsquantisierung", section 1, and the
wiki page's section "Technische Architektur", item 1) and serves as an
independent cross-check of the same result.  ``bruteforce`` is scalar Python
with math.fsum for tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (bf16 is widened exactly through float32)
        import torch

        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q, k, scale, causal, rows):
    """scale * q[rows] k^T with the causal mask applied (query index = row index)."""
    s = scale * (q[rows] @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s[keys[None, :] > rows[:, None]] = -np.inf
    return s


def probabilities(q, k, causal: bool, scale: float, rows=None) -> np.ndarray:
    """Softmax probabilities P for one head (q, k: [N, d]) -- rows of P sum to one."""
    q, k = _as_f64(q), _as_f64(k)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = _scores(q, k, scale, causal, rows)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def reference(q, k, v, causal: bool, scale: float, rows=None):
    """Plain definition of attention for [B, H, N, d] inputs.

    Returns (O, LSE) as float64 arrays of shapes [B, H, R, d] and [B, H, R],
    where R = N, or R = len(rows) when only the query rows ``rows`` are wanted
    (every key is still used; this is how full-size outputs are sampled).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((B, H, len(rows), v.shape[-1]))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal, rows)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            o[b, h] = (e / l) @ v[b, h]
            lse[b, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def online(q, k, v, causal: bool, scale: float, block: int = 64):
    """The tiled, single-pass formulation over key blocks of ``block`` keys.

    For each block of keys: new running max m' = max(m, rowmax S_blk); the
    running sum and the unnormalised output are multiplied by exp(m - m')
    before the block's exp(S_blk - m') terms are added; the division by the
    row sum (and the logsumexp) happens once, after the last block.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    o = np.empty(q.shape[:3] + (v.shape[-1],))
    lse = np.empty((B, H, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, v.shape[-1]))
            for j0 in range(0, N, block):
                kk = k[b, h, j0:j0 + block]
                s = scale * (q[b, h] @ kk.T)
                if causal:
                    keys = np.arange(j0, j0 + kk.shape[0])
                    s[keys[None, :] > rows[:, None]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                # rows that have seen no visible key yet keep m = -inf and zero sums
                alive = np.isfinite(m_new)
                alpha = np.where(alive, np.exp(np.where(alive, m - m_new, 0.0)), 1.0)
                p = np.where(alive[:, None], np.exp(s - np.where(alive, m_new, 0.0)[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j0 + block]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse


def bruteforce(q, k, v, causal: bool, scale: float):
    """Scalar triple loop with math.exp / math.fsum (tiny inputs only)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, N, dv))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                visible = range(i + 1) if causal else range(N)
                s = {j: scale * math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) for j in visible}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in visible}
                z = math.fsum(w.values())
                for c in range(dv):
                    o[b, h, i, c] = math.fsum(w[j] * v[b, h, j, c] for j in visible) / z
                lse[b, h, i] = m + math.log(z)
    return o, lse


def partial(q, k, v, causal: bool, scale: float, q_pos0: int, k_begin: int, k_end: int):
    """Attention of queries against one range of keys, for [B, H, Nq, d] queries and
    [B, H, Nk, d] keys and values.

    Query i sits at key position q_pos0 + i; it sees keys k_begin <= j < k_end and,
    when causal, only j <= q_pos0 + i.  Returns (O, LSE), float64 [B, H, Nq, d] and
    [B, H, Nq], with O normalised over the visible keys; a row that sees no key of
    the range gets O = 0 and LSE = -inf (the empty sum).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, _ = q.shape
    pos = q_pos0 + np.arange(Nq)
    keys = np.arange(k_begin, k_end)
    o = np.zeros((B, H, Nq, v.shape[-1]))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h, k_begin:k_end].T)
            if causal:
                s[keys[None, :] > pos[:, None]] = -np.inf
            seen = np.isfinite(s).any(axis=1)
            if not seen.any():
                continue
            s, vv = s[seen], v[b, h, k_begin:k_end]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            o[b, h, seen] = (e / l) @ vv
            lse[b, h, seen] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def merge(o_parts, lse_parts):
    """O and LSE over the union of disjoint key ranges from their partial results.

    The exponentials of the ranges add: LSE = log sum_s exp(LSE_s), and
    O = sum_s exp(LSE_s - LSE) O_s (the rescaling the online softmax applies per
    tile, here once per range).  Ranges with LSE_s = -inf contribute nothing; a row
    with every LSE_s = -inf gets O = 0, LSE = -inf.
    o_parts: [n, ..., d];  lse_parts: [n, ...].
    """
    o_parts, lse_parts = _as_f64(o_parts), _as_f64(lse_parts)
    m = lse_parts.max(axis=0)
    alive = np.isfinite(m)
    w = np.where(alive[None], np.exp(lse_parts - np.where(alive, m, 0.0)[None]), 0.0)
    z = w.sum(axis=0)
    lse = np.where(alive, np.where(alive, m, 0.0) + np.log(np.where(alive, z, 1.0)), -np.inf)
    o = np.where(alive[..., None], (w[..., None] * o_parts).sum(axis=0) / np.where(alive, z, 1.0)[..., None], 0.0)
    return o, lse


def backward(q, k, v, do, causal: bool, scale: float, o=None):
    """Gradients of attention for [B, H, N, d] inputs and output gradient dO.

    With S = scale * Q K^T (masked), P = softmax(S) row by row and O = P V, the
    chain rule gives, per head:
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij  (= sum_c dO_ic O_ic)
      dS = P * (dP - D)        (the softmax Jacobian applied row by row)
      dQ = scale * dS K,   dK = scale * dS^T Q.
    This is the quantity the pages' training use needs from the saved LSE
    (FlashAttention-2 wiki page, "Leistung und Effizienz": end-to-end training);
    here it is written from the plain definition, materialising P.
    With `o` given, D_i = sum_c dO_ic o_ic is taken from that output instead:
    the backward operation receives the forward's output as an input, and a
    rounded output (bf16) moves D by the rounding, which then enters dS.
    Returns (dQ, dK, dV) as float64 arrays.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    og = None if o is None else _as_f64(o)
    B, H, N, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            s = _scores(q[b, h], k[b, h], scale, causal, rows)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dd = (p * dp).sum(axis=1, keepdims=True) if og is None else (do[b, h] * og[b, h]).sum(axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_sampled(q, k, v, do, o, lse, causal: bool, scale: float, rows, keys):
    """Some rows of dQ and some keys' rows of dK and dV for one head (q, k, v, do, o:
    [N, d]; lse: [N]), by the formulas of ``backward`` with the forward's output O and
    logsumexp LSE taken as given: the backward operation receives both, and with them
    P_ij = exp(scale q_i . k_j - LSE_i) and D_i = sum_c dO_ic O_ic need no pass over a
    whole row of S.  Row i of dQ uses row i of P and dS, row j of dK and dV uses column
    j, so each costs O(N d) and long sequences can be sampled.  The gradients are
    those the pages' training use needs (FlashAttention-2 wiki page, "Leistung und
    Effizienz"), as in ``backward``.  Returns float64 (dQ[rows], dK[keys], dV[keys])."""
    q, k, v, do, o, lse = (_as_f64(x) for x in (q, k, v, do, o, lse))
    dd = (do * o).sum(axis=1)
    rows, keys = np.asarray(rows), np.asarray(keys)
    dq = np.zeros((len(rows), q.shape[1]))
    for n, i in enumerate(rows):
        s = scale * (k @ q[i])  # row i of S
        if causal:
            s[i + 1:] = -np.inf
        p = np.exp(s - lse[i])
        ds = p * (v @ do[i] - dd[i])  # dP_ij = dO_i . V_j
        dq[n] = scale * (ds @ k)
    dk = np.zeros((len(keys), k.shape[1]))
    dv = np.zeros((len(keys), v.shape[1]))
    for n, j in enumerate(keys):
        s = scale * (q @ k[j])  # column j of S
        if causal:
            s[:j] = -np.inf
        p = np.exp(s - lse)
        ds = p * (do @ v[j] - dd)
        dk[n] = scale * (ds @ q)
        dv[n] = p @ do
    return dq, dk, dv
