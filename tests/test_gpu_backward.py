"""GPU parity of the backward pass: fa_bwd against the oracle's fp64 gradients.

The kernel recomputes P from the forward's fp32 LSE, takes D = rowsum(dO * O)
from the bf16 O it is given, rounds P and dS to bf16 for the products that use
them and rounds the gradients to bf16 once.  Two bounds, both the bf16 budget
of the forward output (2e-2):
  * element by element, |g - g_ref| against the sum of the magnitudes of the
    terms that make up that element (tests/gpu_checks.py, bwd_term_scales), the
    analogue of the FP8 forward's G5b gate;
  * normwise, max |g - g_ref| / max(1, max |g_ref|) per gradient tensor of a head
    (gradient magnitudes scale with the scale, N and the inputs; with one key,
    dQ and dK vanish exactly and only rounding remains).

Each case checks against the oracle with D taken from the same bf16 O (the
kernel's own arithmetic) and, where stated, against the exact oracle (end to
end, including the rounding of O).  The two differ by scale * P (dO . dO_err)
terms: with O rounded to bf16, D moves by up to 2^-9 sum_c |dO_c O_c|, which
for a row with few keys and a large scale is comparable to dQ itself."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def _grads(fa, q, k, v, do, causal, scale, with_o=False):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return ((dq, dk, dv), o.cpu()) if with_o else (dq, dk, dv)


def _errors(got, ref):
    out = []
    for g, r in zip(got, ref):
        g = g.float().cpu().numpy().astype(np.float64)
        den = max(np.abs(r).max(), 1.0)
        out.append(float(np.abs(g - r).max() / den))
    return out


def _elem(got, ref, q, k, v, do, o, causal, scale):
    """Element-wise errors against the term scales (D from the given O, like ref)."""
    e = G.bwd_elem_errors(got, ref, G.bwd_term_scales(q, k, v, do, o, causal, scale))
    G.log(f"  element-wise errors dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
    return e


# B*H a multiple of 8 takes the grouped block order of non-causal launches
SMALL = [(1, 2, n, d) for n in (1, 7, 64, 100, 129, 300, 513) for d in (64, 128)] + [(2, 4, 300, 128), (2, 8, 129, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}N{}d{}".format(*s))
def test_backward_small(fa, shape, causal):
    B, H, N, d = shape
    G.log(f"case backward {shape} causal={causal}")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=N * 7 + d, dtype="bf16")
    do = synthetic.draw_qkv(B, H, N, d, seed=N * 7 + d + 1, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, causal, d ** -0.5, with_o=True)
    ref = A.backward(q, k, v, do, causal, d ** -0.5, o=o)
    e = _errors(got, ref)
    x = _errors(got, A.backward(q, k, v, do, causal, d ** -0.5))
    G.log(f"  normwise errors dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e} (exact O: {max(x):.2e})")
    assert max(e) <= TOL and max(x) <= TOL
    assert max(_elem(got, ref, q, k, v, do, o, causal, d ** -0.5)) <= G.BWD_ELEM_TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [0.0, -0.15, 0.5])
def test_backward_scales(fa, scale, d, causal):
    """Zero, negative and large scales, both head sizes (the d = 64 kernels flip or zero
    Q's bits, the pipelined d = 128 dK/dV kernel takes a signed multiplier)."""
    B, H, N = 1, 2, 200
    G.log(f"case backward scale={scale} d={d} causal={causal}")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=31, dtype="bf16")
    do = synthetic.draw_qkv(B, H, N, d, seed=32, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, causal, scale, with_o=True)
    ref = A.backward(q, k, v, do, causal, scale, o=o)
    if scale == 0.0:  # S does not depend on Q or K: their gradients vanish
        assert not got[0].float().abs().max().item() and not got[1].float().abs().max().item()
        e = _errors(got[2:], ref[2:])
    else:
        e = _errors(got, ref)
    G.log(f"  normwise errors {['%.2e' % x for x in e]}")
    assert max(e) <= TOL
    assert max(_elem(got, ref, q, k, v, do, o, causal, scale)) <= G.BWD_ELEM_TOL


@pytest.mark.parametrize("d", [64, 128])
def test_backward_zero_scale_overflowing_scores(fa, d):
    """scale 0 with |Q K^T| beyond the fp32 range: the scores are 0 by definition, so
    every gradient is finite, dQ = dK = 0 and dV = P^T dO with uniform P."""
    G.log(f"case backward zero scale, overflowing Q K^T, d={d}")
    q, k, v = synthetic.draw_qkv(1, 2, 100, d, seed=33, dtype="bf16")
    q, k = (q.float() * 2.0 ** 70).to(torch.bfloat16), (k.float() * 2.0 ** 70).to(torch.bfloat16)
    do = synthetic.draw_qkv(1, 2, 100, d, seed=34, dtype="bf16")[0]
    for causal in (False, True):
        got, o = _grads(fa, q, k, v, do, causal, 0.0, with_o=True)
        assert all(bool(torch.isfinite(g.float()).all()) for g in got)
        assert not got[0].float().abs().max().item() and not got[1].float().abs().max().item()
        e = _errors(got[2:], A.backward(q, k, v, do, causal, 0.0, o=o)[2:])
        G.log(f"  causal={causal} dV normwise error {e[0]:.2e}")
        assert max(e) <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_backward_few_keys_large_scale(fa, d):
    """Two keys and scale 0.3: dQ is small (|dQ| < 1) while dP and D are not, so the
    bf16 rounding of O moves dQ by about 3e-2 against the exact oracle; against D
    from the given O the kernel stays within the bound."""
    G.log(f"case backward few keys d={d}")
    q, k, v = synthetic.draw_qkv(1, 1, 2, d, seed=578167, dtype="bf16")
    do = synthetic.draw_qkv(1, 1, 2, d, seed=578169, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, False, 0.3, with_o=True)
    ref = A.backward(q, k, v, do, False, 0.3, o=o)
    e = _errors(got, ref)
    x = _errors(got, A.backward(q, k, v, do, False, 0.3))
    G.log(f"  normwise errors against D from the given O {max(e):.2e}, against the exact O {max(x):.2e}")
    assert max(e) <= TOL
    assert max(_elem(got, ref, q, k, v, do, o, False, 0.3)) <= G.BWD_ELEM_TOL


def test_backward_full_size_heads(fa):
    """The bench's bf16 workload (B4 H16 N2048 d128 causal) in its launch configuration, two heads checked."""
    w = synthetic.workload("bf16_causal_b4h16n2048d128")
    G.log(f"case backward {w.name}")
    q, k, v, _ = synthetic.workload_inputs(w)
    do = synthetic.draw_qkv(w.B, w.H, w.N, w.d, seed=w.seed + 100, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, w.causal, w.scale, with_o=True)
    for b, h in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = A.backward(q[sl], k[sl], v[sl], do[sl], w.causal, w.scale, o=o[sl])
        e = _errors([x[sl] for x in got], ref)
        G.log(f"  head ({b},{h}) normwise errors dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
        assert max(e) <= TOL
        assert max(_elem([x[sl] for x in got], ref, q[sl], k[sl], v[sl], do[sl], o[sl], w.causal, w.scale)) <= \
            G.BWD_ELEM_TOL
    for _ in range(2):  # no atomics: bitwise reproducible
        again = _grads(fa, q, k, v, do, w.causal, w.scale)
        assert all(torch.equal(x, y) for x, y in zip(got, again))


def test_backward_d64_workload_heads(fa):
    """The d = 64 workload (B16 H16 N1024 non-causal) in its launch configuration (the
    plain dK/dV loop and the pipelined dQ kernel at d = 64), two whole heads checked."""
    w = synthetic.workload("bf16_b16h16n1024d64")
    G.log(f"case backward {w.name}")
    q, k, v, _ = synthetic.workload_inputs(w)
    do = synthetic.draw_qkv(w.B, w.H, w.N, w.d, seed=w.seed + 100, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, w.causal, w.scale, with_o=True)
    for b, h in ((0, 0), (15, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = A.backward(q[sl], k[sl], v[sl], do[sl], w.causal, w.scale, o=o[sl])
        e = _errors([x[sl] for x in got], ref)
        G.log(f"  head ({b},{h}) normwise errors dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
        assert max(e) <= TOL
        assert max(_elem([x[sl] for x in got], ref, q[sl], k[sl], v[sl], do[sl], o[sl], w.causal, w.scale)) <= \
            G.BWD_ELEM_TOL


def test_backward_long_sequence_head(fa):
    """The long-sequence workload (B1 H32 N16384 d128 causal) in its launch configuration;
    one whole head against the fp64 gradient oracle (every N x N product materialised)."""
    w = synthetic.workload("bf16_causal_b1h32n16384d128")
    G.log(f"case backward {w.name}")
    q, k, v, _ = synthetic.workload_inputs(w)
    do = synthetic.draw_qkv(w.B, w.H, w.N, w.d, seed=w.seed + 100, dtype="bf16")[0]
    got, o = _grads(fa, q, k, v, do, w.causal, w.scale, with_o=True)
    b, h = 0, 21
    sl = (slice(b, b + 1), slice(h, h + 1))
    ref = A.backward(q[sl], k[sl], v[sl], do[sl], w.causal, w.scale, o=o[sl])
    e = _errors([x[sl] for x in got], ref)
    G.log(f"  head ({b},{h}) normwise errors dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
    assert max(e) <= TOL
    assert max(_elem([x[sl] for x in got], ref, q[sl], k[sl], v[sl], do[sl], o[sl], w.causal, w.scale)) <= \
        G.BWD_ELEM_TOL
