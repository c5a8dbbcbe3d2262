"""The largest key count the C-ABI accepts, run through the split-KV path.

The kernels form 32-bit byte offsets within a head, and the shape check admits N as long
as N * d * 4 bytes fit in an int32 (include/fa.h).  At d = 128 that is 4,194,303 keys:
K and V hold 1.07 GB each, and tile offsets reach 2^30.  A few queries against all of
them is cheap on the GPU and within the fp64 oracle's reach, and it exercises both the
decode kernel (at most 32 queries) and the general kernel over key ranges, every output
compared (the same bounds as the split-KV tests)."""
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
