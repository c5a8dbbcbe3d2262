"""GPU parity of the split-KV path: fa_fwd_partial and fa_merge against the oracle.

fa_fwd_partial runs the bf16 forward kernel on one key range with queries at an
offset position (fa_fwd_split on several consecutive ranges in one launch; at
most 32 queries take the decode kernel, which splits each range over four
wavefronts); its O is fp32 but the probabilities feeding P V are rounded to
bf16 as in fa_fwd, so O carries the bf16 bound (2e-2) and LSE the 1e-3 one.
Rows that see no key of the range must come back exactly O = 0, LSE = -inf.
fa_merge is pure fp32 arithmetic: O within 1e-5 (fp32 output; bf16 output
within its rounding), LSE within 1e-5."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_O, TOL_L = 2e-2, 1e-3

# (Nq, Nk, q_pos0, k_begin, k_end, causal, d)
CASES = [
    (128, 128, 0, 0, 128, True, 128),      # the square problem over its full range
    (16, 1000, 984, 0, 1000, True, 128),   # decode: the last 16 positions of 1000
    (300, 700, 400, 256, 641, True, 128),  # offset queries, a range ending mid-tile
    (300, 700, 400, 256, 641, False, 64),
    (64, 64, 0, 10, 10, False, 128),       # empty range
    (32, 600, 0, 500, 600, True, 64),      # every query before the range: nothing visible
    (100, 333, 0, 17, 333, False, 64),     # ragged range
    (257, 513, 100, 0, 290, True, 128),    # some rows see nothing, others part of the range
    (1, 5000, 4999, 1234, 4999, True, 128),
    (32, 3000, 0, 0, 3000, False, 128),    # decode kernel, non-causal, 94 tiles over four wavefronts
    (17, 70, 53, 0, 70, True, 64),         # decode kernel, three tiles: one wavefront has none
    (33, 900, 867, 0, 900, True, 128),     # one query past the decode kernel's limit
]


def _inputs(nq, nk, d, seed):
    q, _, _ = synthetic.draw_qkv(2, 3, nq, d, seed=seed, dtype="bf16")
    _, k, v = synthetic.draw_qkv(2, 3, nk, d, seed=seed + 1, dtype="bf16")
    return q, k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: "q{}k{}p{}r{}-{}{}d{}".format(c[0], c[1], c[2], c[3], c[4],
                                                                                     "c" if c[5] else "", c[6]))
def test_partial(fa, case):
    nq, nk, pos0, kb, ke, causal, d = case
    G.log(f"case partial {case}")
    q, k, v = _inputs(nq, nk, d, seed=nq + nk + d)
    scale = d ** -0.5
    o, lse = fa.fa_fwd_partial(q.to(DEV), k.to(DEV), v.to(DEV), pos0, kb, ke, causal, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = A.partial(q, k, v, causal, scale, pos0, kb, ke)
    o, lse = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    empty = ~np.isfinite(l_ref)
    assert np.array_equal(~np.isfinite(lse), empty)
    assert np.all(lse[empty] == -np.inf) and not o[empty].any()
    live = ~empty
    eo = np.abs(o[live] - o_ref[live]).max() if live.any() else 0.0
    el = np.abs(lse[live] - l_ref[live]).max() if live.any() else 0.0
    G.log(f"  max|dO| {eo:.3e}  max|dLSE| {el:.3e}  empty rows {int(empty.sum())}")
    assert eo <= TOL_O and el <= TOL_L


# (Nq, Nk, q_pos0, k_begin, k_end, n_splits, causal, d)
SPLIT_CASES = [
    (16, 4096, 4080, 0, 4096, 8, True, 128),   # decode: the last 16 positions, 8 ranges
    (16, 1000, 984, 0, 1000, 7, True, 64),     # ragged ranges
    (300, 700, 400, 100, 650, 3, True, 128),
    (64, 100, 0, 0, 100, 16, False, 128),      # ranges of 6 or 7 keys
    (32, 600, 0, 500, 600, 4, True, 64),       # nothing visible in any range
    (8, 20, 12, 0, 20, 40, True, 128),         # more ranges than keys: empty ranges
    (1, 16384, 16383, 0, 16384, 8, True, 128),  # one new token
    (32, 2000, 0, 0, 2000, 5, False, 64),
    (20, 4133, 4113, 0, 4133, 6, True, 128),    # ranges ending mid-tile
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "q{}k{}p{}r{}-{}x{}{}d{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else "", c[7]))
def test_split_ranges_in_one_launch(fa, case):
    """fa_fwd_split: slice s equals the oracle's partial over the s-th range."""
    nq, nk, pos0, kb, ke, n, causal, d = case
    G.log(f"case split {case}")
    q, k, v = _inputs(nq, nk, d, seed=nq + nk + n)
    scale = d ** -0.5
    op, lp = fa.fa_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), n, pos0, kb, ke, causal, scale)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy().astype(np.float64), lp.cpu().numpy().astype(np.float64)
    eo = el = 0.0
    for s in range(n):
        b0, b1 = kb + (ke - kb) * s // n, kb + (ke - kb) * (s + 1) // n
        o_ref, l_ref = A.partial(q, k, v, causal, scale, pos0, b0, b1)
        empty = ~np.isfinite(l_ref)
        assert np.array_equal(~np.isfinite(lp[s]), empty), s
        assert np.all(lp[s][empty] == -np.inf) and not op[s][empty].any(), s
        live = ~empty
        if live.any():
            eo = max(eo, float(np.abs(op[s][live] - o_ref[live]).max()))
            el = max(el, float(np.abs(lp[s][live] - l_ref[live]).max()))
    G.log(f"  max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
    assert eo <= TOL_O and el <= TOL_L


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9])
@pytest.mark.parametrize("nq", [16, 100])
def test_split_scales(fa, scale, nq):
    """Negative, zero and large scales through both the decode kernel (16 queries)
    and the general one (100 queries)."""
    G.log(f"case split scale={scale} nq={nq}")
    nk, d, n = 1500, 128, 4
    q, k, v = _inputs(nq, nk, d, seed=4242)
    op, lp = fa.fa_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), n, nk - nq, 0, nk, True, scale)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy().astype(np.float64), lp.cpu().numpy().astype(np.float64)
    for s in range(n):
        o_ref, l_ref = A.partial(q, k, v, True, scale, nk - nq, nk * s // n, nk * (s + 1) // n)
        assert np.isfinite(l_ref).all()
        eo, el = np.abs(op[s] - o_ref).max(), np.abs(lp[s] - l_ref).max()
        G.log(f"  range {s}: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= TOL_O and el <= TOL_L


@pytest.mark.parametrize("n", [5, 64, 70])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_merge(fa, d, dtype, n):
    """n = 64 and 70: a row's range LSEs are read 64 at a time (one per lane)."""
    G.log(f"case merge d={d} {dtype} n={n}")
    rng = np.random.default_rng(d + n)
    B, H, N = 2, 3, 77
    o_parts = rng.standard_normal((n, B, H, N, d)).astype(np.float32)
    lse_parts = (3.0 * rng.standard_normal((n, B, H, N))).astype(np.float32)
    lse_parts[rng.random((n, B, H, N)) < 0.3] = -np.inf   # ranges a row does not see
    lse_parts[:, 0, 0, :5] = -np.inf                       # rows that see nothing at all
    o, lse = fa.fa_merge(torch.from_numpy(o_parts).to(DEV), torch.from_numpy(lse_parts).to(DEV), dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = A.merge(o_parts, lse_parts)
    o, lse = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.all(lse[0, 0, :5] == -np.inf) and not o[0, 0, :5].any()
    live = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), live)
    tol_o = 1e-5 if dtype == torch.float32 else 2.0 ** -8 * (1.0 + np.abs(o_ref[live]))
    assert np.all(np.abs(o[live] - o_ref[live]) <= tol_o)
    assert np.abs(lse[live] - l_ref[live]).max() <= 1e-5


@pytest.mark.parametrize("n_splits", [1, 3, 8])
def test_split_kv_decode(fa, n_splits):
    """Decode-shaped split-KV forward: 16 new queries against 4096 cached keys."""
    G.log(f"case split-KV decode n_splits={n_splits}")
    nq, nk, d = 16, 4096, 128
    q, k, v = _inputs(nq, nk, d, seed=99)
    o, lse = fa.split_kv_attention(q.to(DEV), k.to(DEV), v.to(DEV), n_splits, causal=True, scale=d ** -0.5)
    torch.cuda.synchronize()
    o_ref, l_ref = A.partial(q, k, v, True, d ** -0.5, nk - nq, 0, nk)
    eo = np.abs(o.float().cpu().numpy() - o_ref).max()
    el = np.abs(lse.cpu().numpy() - l_ref).max()
    G.log(f"  max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
    assert eo <= TOL_O and el <= TOL_L


def test_split_kv_decode_bench_shape(fa):
    """The split-KV bench's workload (B4 H16, the last 16 of 16384 causal positions,
    d = 128, 8 ranges) in its launch configuration: fa_fwd_split then fa_merge, with
    three heads checked against the oracle, each range's partial and the merged row."""
    import bench
    c = bench.DECODE
    B, H, Nq, Nk, d, n = c["B"], c["H"], c["Nq"], c["Nk"], c["d"], c["n_splits"]
    G.log(f"case split-KV decode bench shape {c}")
    q = synthetic.draw_qkv(B, H, Nq, d, seed=c["seed"], dtype="bf16")[0]
    _, k, v = synthetic.draw_qkv(B, H, Nk, d, seed=c["seed"] + 1, dtype="bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = d ** -0.5
    op, lp = fa.fa_fwd_split(qd, kd, vd, n, Nk - Nq, 0, Nk, True, scale)
    o, lse = fa.fa_merge(op, lp, torch.bfloat16)
    torch.cuda.synchronize()
    op, lp = op.cpu().numpy().astype(np.float64), lp.cpu().numpy().astype(np.float64)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b, h in ((0, 0), (1, 7), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        for s in range(n):
            o_ref, l_ref = A.partial(q[sl], k[sl], v[sl], True, scale, Nk - Nq, Nk * s // n, Nk * (s + 1) // n)
            assert np.abs(op[s][sl] - o_ref).max() <= TOL_O and np.abs(lp[s][sl] - l_ref).max() <= TOL_L
        o_ref, l_ref = A.partial(q[sl], k[sl], v[sl], True, scale, Nk - Nq, 0, Nk)
        eo, el = np.abs(o[sl] - o_ref).max(), np.abs(lse[sl] - l_ref).max()
        G.log(f"  head ({b},{h}) merged: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= TOL_O and el <= TOL_L


def test_split_kv_square_matches_full_forward(fa):
    """The square causal problem split in four key ranges equals fa_fwd within bf16 rounding."""
    q, k, v = _inputs(1024, 1024, 128, seed=5)
    k, v = synthetic.draw_qkv(2, 3, 1024, 128, seed=6, dtype="bf16")[1:]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_s, l_s = fa.split_kv_attention(qd, kd, vd, 4, causal=True)
    o_f, l_f = fa.fa_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = A.reference(q, k, v, True, 128 ** -0.5, rows=np.arange(0, 1024, 37))
    for o, l in ((o_s, l_s), (o_f, l_f)):
        o = o.float().cpu().numpy()[:, :, ::37]
        l = l.cpu().numpy()[:, :, ::37]
        assert np.abs(o - o_ref).max() <= TOL_O and np.abs(l - l_ref).max() <= TOL_L
