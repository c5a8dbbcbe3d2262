"""The pipelined bf16 forward against its serial debug build, bit for bit.

libfa_serial.so is libfa.so with the bf16 forward's loop in its serial form:
one key tile at a time through a single LDS slot, a full workgroup barrier on
each side of every copy, no overlap of copies, score products, softmax and
output products.  The arithmetic of each row is the same in both (the same
instructions in the same order), so any difference exposes a hazard in the
pipelined schedule: a slot overwritten while a wavefront still reads it, a
missing wait, a prefetch of the wrong tile.  This is the check for races that
a comparison against the oracle, within a tolerance, could miss.
"""
import ctypes

import pytest
import torch

import synthetic
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, N, d, causal): ragged tails, one tile, several tiles, several query blocks
    (1, 2, 1, 128, True),
    (1, 2, 33, 128, False),
    (1, 3, 300, 128, True),
    (2, 2, 700, 128, False),
    (1, 2, 1000, 64, True),
    (1, 3, 513, 64, False),
]


def _fwd(lib, q, k, v, causal, scale):
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, int(causal),
                    scale, 1, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return o, lse


def _split(lib, q, k, v, causal, scale, n_splits):
    B, H, N, d = q.shape
    o = torch.empty((n_splits, B, H, N, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((n_splits, B, H, N), dtype=torch.float32, device=q.device)
    st = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, N, d, 0,
                          0, N, n_splits, int(causal), scale, 1,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return o, lse


@pytest.fixture(scope="module")
def libs(fa):
    return fa.load_library(), fa.load_serial_library()


def _same(name, a, b):
    oa, la = a
    ob, lb = b
    torch.cuda.synchronize()
    eq_o = torch.equal(oa, ob)
    eq_l = torch.equal(la, lb)
    if not (eq_o and eq_l):
        G.log(f"  {name}: max|dO| {(oa.float() - ob.float()).abs().max().item():.3e} "
              f"max|dLSE| {(la - lb).abs().max().item():.3e}")
    assert eq_o and eq_l, name


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}d{}{}".format(*c[:4], "c" if c[4] else ""))
def test_pipelined_equals_serial(libs, case):
    B, H, N, d, causal = case
    G.log(f"case serial-vs-pipelined B{B} H{H} N{N} d{d} causal={causal}")
    q, k, v = (x.cuda() for x in synthetic.draw_qkv(B, H, N, d, seed=500 + N, dtype="bf16"))
    for scale in (d ** -0.5, 0.5, -0.15):
        _same(f"scale {scale}", _fwd(libs[0], q, k, v, causal, scale), _fwd(libs[1], q, k, v, causal, scale))


@pytest.mark.parametrize("name", ["bf16_causal_b4h16n2048d128", "bf16_b16h16n1024d64"])
def test_pipelined_equals_serial_workload(libs, name):
    """Whole launches of the bench workloads, every output compared."""
    w = synthetic.workload(name)
    G.log(f"case serial-vs-pipelined {w.name}")
    q, k, v, _ = synthetic.workload_inputs(w)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    _same(w.name, _fwd(libs[0], q, k, v, w.causal, w.scale), _fwd(libs[1], q, k, v, w.causal, w.scale))


def test_pipelined_equals_serial_split(libs):
    """The key-range (split) form of the same kernel: 200 queries, 4 ranges."""
    B, H, N, d = 1, 2, 600, 128
    G.log(f"case serial-vs-pipelined split B{B} H{H} N{N} d{d}")
    q, k, v = (x.cuda() for x in synthetic.draw_qkv(B, H, N, d, seed=611, dtype="bf16"))
    for causal in (False, True):
        _same(f"split causal={causal}", _split(libs[0], q, k, v, causal, d ** -0.5, 4),
              _split(libs[1], q, k, v, causal, d ** -0.5, 4))


def _growing_keys(B, H, N, d, seed, growth):
    """K rows scaled by 1 + growth * j / N: the row maxima keep rising along the keys, so the
    steady steps keep finding scores above their shift (the path that recomputes the step)."""
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=seed, dtype="bf16")
    ramp = 1.0 + growth * torch.arange(N, dtype=torch.float32) / N
    k = (k.float() * ramp[None, None, :, None]).to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("d", [64, 128])
def test_rising_maxima_take_the_full_step(libs, d):
    """Scores that keep exceeding the running shift in unmasked steps: the steps that skip
    the maximum must detect it and redo the step, bit-identical to the serial build and
    within the bf16 bounds of the oracle."""
    B, H, N = 1, 2, 1024
    G.log(f"case rising maxima d={d}")
    q, k, v = _growing_keys(B, H, N, d, seed=620 + d, growth=6.0)
    for causal in (False, True):
        for scale in (d ** -0.5, 0.5):
            got = _fwd(libs[0], q.cuda(), k.cuda(), v.cuda(), causal, scale)
            _same(f"rising causal={causal} scale={scale}", got, _fwd(libs[1], q.cuda(), k.cuda(), v.cuda(), causal, scale))
            eo, el = G.compare_attention(got[0], got[1], q, k, v, causal, scale, "bf16")
            G.log(f"  causal={causal} scale={scale}: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
            assert eo <= G.TOL["bf16"][0] and el <= G.TOL["bf16"][1]


def test_overflowing_jump_takes_the_full_step(libs):
    """One late key whose score exceeds every earlier one by far more than 128 (log2 units):
    under the old shift its probability overflows to +inf, which must send the step down the
    full path; rows that see the key then weight it alone."""
    B, H, N, d = 1, 1, 700, 128
    G.log("case overflowing jump")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=640, dtype="bf16")
    j, i0 = 600, 650
    k = k.clone()
    k[0, 0, j] = (q[0, 0, i0].float() * 1.5).to(torch.bfloat16)  # row i0 scores about 1.5 * |q|^2 = 190 on key j
    for causal in (False, True):
        got = _fwd(libs[0], q.cuda(), k.cuda(), v.cuda(), causal, 1.0)
        _same(f"jump causal={causal}", got, _fwd(libs[1], q.cuda(), k.cuda(), v.cuda(), causal, 1.0))
        assert torch.isfinite(got[0].float()).all() and torch.isfinite(got[1]).all()
        eo, el = G.compare_attention(got[0], got[1], q, k, v, causal, 1.0, "bf16")
        G.log(f"  causal={causal}: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= G.TOL["bf16"][0] and el <= G.TOL["bf16"][1]
