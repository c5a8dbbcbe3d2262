"""Randomised parity sweep: many small problems of random shape against the oracle.

The other GPU tests fix their shapes; this one draws them (seeded, so every run sees
the same cases): batch and head counts, ragged sequence lengths from 1 to 1600, both
head sizes, causal or not, and scales of either sign including zero.  Each case
runs one entry point of the library and is held to the same gates as the fixed
tests:
  * bf16 and fp32 forward (fa_fwd) against the fp64 definition, every output;
  * split-KV (one fa_fwd_split launch over 1-8 key ranges, then fa_merge) against
    the same definition, as the ranges together cover every key;
  * backward (fa_bwd) against the fp64 gradients with D from the bf16 O, normwise;
  * FP8 (pre-pass + fa_fwd_fp8) against the oracle of its own dequantised codes.
Every case is logged before it runs, so a failure names it."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BWD_TOL = 2e-2  # normwise, the bf16 budget of the forward output
CASES_PER_SEED = 60


def _case(rng):
    d = int(rng.choice([64, 128]))
    kind = str(rng.choice(["fwd", "fwd", "bwd", "split", "f32", "fp8"]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    N = int(rng.choice([rng.integers(1, 80), rng.integers(80, 700), rng.integers(700, 1600)]))
    scale = float(rng.choice([d ** -0.5, rng.uniform(-0.6, 0.6), 0.0, rng.uniform(0.05, 1.0)]))
    causal = bool(rng.integers(2))
    if kind == "f32":
        N = min(N, 900)
    if kind == "bwd":
        N = min(N, 600)
    if kind == "fp8":
        d = 128
    return kind, B, H, N, d, causal, scale


def _normwise(got, ref):
    out = []
    for g, r in zip(got, ref):
        g = g.float().cpu().numpy().astype(np.float64)
        out.append(float(np.abs(g - r).max() / max(np.abs(r).max(), 1.0)))
    return out


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_random_shapes(fa, seed):
    rng = np.random.default_rng(seed)
    for i in range(CASES_PER_SEED):
        kind, B, H, N, d, causal, scale = _case(rng)
        s = 50000 + 1000 * seed + i
        G.log(f"case sweep seed={seed} #{i} {kind} B{B} H{H} N{N} d{d} causal={causal} scale={scale:.4f}")
        if kind in ("fwd", "f32"):
            dt = "f32" if kind == "f32" else "bf16"
            q, k, v = synthetic.draw_qkv(B, H, N, d, seed=s, dtype=dt)
            o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
            eo, el = G.compare_attention(o, lse, q, k, v, causal, scale, dt)
            G.log(f"  max|dO| {eo:.2e}  max|dLSE| {el:.2e}")
            assert eo <= G.TOL[dt][0] and el <= G.TOL[dt][1]
        elif kind == "split":
            n_splits = int(rng.integers(1, 9))
            q, k, v = synthetic.draw_qkv(B, H, N, d, seed=s, dtype="bf16")
            o, lse = fa.split_kv_attention(q.to(DEV), k.to(DEV), v.to(DEV), n_splits, causal=causal, scale=scale)
            eo, el = G.compare_attention(o, lse, q, k, v, causal, scale, "bf16")
            G.log(f"  {n_splits} ranges: max|dO| {eo:.2e}  max|dLSE| {el:.2e}")
            assert eo <= G.TOL["bf16"][0] and el <= G.TOL["bf16"][1]
        elif kind == "bwd":
            q, k, v = synthetic.draw_qkv(B, H, N, d, seed=s, dtype="bf16")
            do = synthetic.draw_qkv(B, H, N, d, seed=s + 1, dtype="bf16")[0]
            qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
            o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, scale=scale)
            got = fa.fa_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
            torch.cuda.synchronize()
            ref = A.backward(q, k, v, do, causal, scale, o=o.cpu())
            if scale == 0.0:  # dQ and dK vanish exactly
                assert not got[0].float().abs().max().item() and not got[1].float().abs().max().item()
                e = _normwise(got[2:], ref[2:])
            else:
                e = _normwise(got, ref)
            G.log(f"  normwise {['%.2e' % x for x in e]}")
            assert max(e) <= BWD_TOL
        else:
            q, k, v = synthetic.draw_qkv(B, H, N, d, seed=s, dtype="bf16")
            signs = torch.from_numpy(synthetic.draw_signs(d, s)).to(DEV)
            o, lse, (q8, k8, v8t, qs, ks, vs) = fa.fp8_attention(q.to(DEV), k.to(DEV), v.to(DEV), signs,
                                                                 causal=causal, scale=scale)
            torch.cuda.synchronize()
            heads = [(b, h) for b in range(B) for h in range(H)]
            rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, causal, scale, heads=heads)
            G.log(f"  vs dequantised oracle: scaled err {rel:.2e}  LSE rel {el:.2e}")
            assert rel <= G.FP8_O_TOL and el <= G.FP8_LSE_TOL
