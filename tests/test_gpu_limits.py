"""The largest sequence length the C-ABI accepts, through split-KV, forward and backward.

The kernels form 32-bit byte offsets within a head, and the shape check admits N as long
as N * d * 4 bytes fit in an int32 (include/fa.h).  At d = 128 that is 4,194,303 tokens:
K and V hold 1.07 GB each, and tile offsets reach 2^30.  A few queries against all of
them is cheap on the GPU and within the fp64 oracle's reach, and it exercises both the
decode kernel (at most 32 queries) and the general kernel over key ranges, every output
compared (the same bounds as the split-KV tests).  The full forward and backward at that
length are checked on sampled rows, each computed by the oracle in O(N d)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_O, TOL_L = G.TOL["bf16"]


def test_split_kv_at_the_largest_key_count(fa):
    d = 128
    nk = (2 ** 31 - 1) // (4 * d)
    G.log(f"case largest key count: {nk} keys, d = {d}")
    _, k, v = synthetic.draw_qkv(1, 1, nk, d, seed=881, dtype="bf16")
    kd, vd = k.to(DEV), v.to(DEV)
    scale = d ** -0.5
    for nq, n_splits in ((16, 64), (40, 64)):  # decode kernel, then the general kernel
        q = synthetic.draw_qkv(1, 1, nq, d, seed=882 + nq, dtype="bf16")[0]
        G.log(f"  {nq} queries at the last positions, {n_splits} key ranges")
        o, lse = fa.split_kv_attention(q.to(DEV), kd, vd, n_splits, causal=True, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = A.partial(q, k, v, True, scale, nk - nq, 0, nk)
        eo = float(np.abs(o.float().cpu().numpy().astype(np.float64) - o_ref).max())
        el = float(np.abs(lse.cpu().numpy().astype(np.float64) - l_ref).max())
        G.log(f"  max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= TOL_O and el <= TOL_L


def test_forward_at_the_largest_sequence_length(fa):
    """fa_fwd on one head of 4,194,303 causal tokens: the query offsets reach the same
    bound (rows sampled: the first, the last, tile boundaries and random ones)."""
    d = 128
    n = (2 ** 31 - 1) // (4 * d)
    G.log(f"case largest sequence length: {n} tokens, d = {d}, causal")
    q, k, v = synthetic.draw_qkv(1, 1, n, d, seed=891, dtype="bf16")
    o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    rows = G.sample_rows(n, 24, seed=892)
    eo, el = G.compare_attention(o, lse, q, k, v, True, d ** -0.5, "bf16", rows=rows)
    G.log(f"  {len(rows)} rows: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
    assert eo <= TOL_O and el <= TOL_L


def test_backward_at_the_largest_sequence_length(fa):
    """fa_bwd on one causal head of 4,194,303 tokens: sampled rows of dQ and keys' rows of
    dK and dV (the first, the last, tile boundaries and random ones) against the oracle's
    backward_sampled, which takes the forward's O and LSE as given, as the backward
    operation does, and so costs O(N d) per row.  Each sampled row is held to the bf16
    budget relative to its own largest entry (the gradients of late keys are millions of
    times smaller than those of early ones); a row whose reference is exactly zero, to
    its absolute error."""
    d = 128
    n = (2 ** 31 - 1) // (4 * d)
    scale = d ** -0.5
    G.log(f"case backward at the largest sequence length: {n} tokens, d = {d}, causal")
    q, k, v = synthetic.draw_qkv(1, 1, n, d, seed=893, dtype="bf16")
    do = synthetic.draw_qkv(1, 1, n, d, seed=894, dtype="bf16")[0]
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = G.sample_rows(n, 8, seed=895)
    keys = G.sample_rows(n, 8, seed=896)
    ref = A.backward_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], o[0, 0], lse[0, 0], True, scale, rows, keys)
    got = [dq[0, 0, rows], dk[0, 0, keys], dv[0, 0, keys]]
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = g.float().cpu().numpy().astype(np.float64)
        # a row whose reference is exactly zero (dQ of row 0: one visible key, so dS = 0)
        # is held to its absolute error instead
        den = np.abs(r).max(axis=1)
        e = float(np.where(den > 0, np.abs(g - r).max(axis=1) / np.where(den > 0, den, 1.0), np.abs(g).max(axis=1)).max())
        G.log(f"  {name}: {len(r)} sampled rows, worst error relative to the row's largest entry {e:.2e}")
        assert e <= TOL_O
