"""FP8 accuracy ablation: what block quantisation and incoherent processing buy.

The pages name two measures that keep FP8 attention accurate with outlier
activations (page "FlashAttention-Skalierung, Multi-GPU-Training und
Gewichtsquantisierung", section 1, FlashAttention-3 FP8 item): small tiles
with their own scales, and a random orthogonal rotation of Q and K.  These
tests measure both against the exact fp64 attention of the un-quantised
inputs:

* at the level of the method, with the oracle's quantiser and the fp64
  attention of the dequantised operands (CPU);
* through the HIP path, with and without the rotation (GPU).

Findings pinned here:
  - the rotation lowers the error when Q and K carry outliers (x10 and x50,
    0.1 %);
  - per-tile scales matter for e4m3 only once tile magnitudes differ by more
    than the format's ~15 binades of normal range can absorb: a 100x
    difference gives the same error as one scale per tensor, a 10^4x
    difference does not;
  - rounding the probabilities to e4m3 (rather than bf16) is the kernel's own
    share of the error: against the fp64 attention of the same dequantised
    operands, P in bf16 stays within the bf16 budget (2e-2 in the G5b metric)
    and below P in e4m3.

Through the HIP path the variants are fa_quant_rotate_fp8 with and without
signs, fa_quant_rotate_fp8_tensor (one scale per tensor) and
fa_fwd_fp8_pbf16 (probabilities in bf16), each against the exact oracle of
the un-quantised inputs and against the oracle of its own dequantised codes.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import attention as A
from oracle import fp8 as F

D = 128
SCALE = D ** -0.5


def _f64(*xs):
    return [x.float().numpy().astype(np.float64) for x in xs]


def _method_error(q, k, v, signs, tile, rows=None):
    """O of the dequantised operands (fp64, P not rounded) minus the exact O."""
    o_ref, _ = A.reference(q, k, v, True, SCALE)
    q8, qs, _ = F.quantize_rotate(q, signs, tile=tile)
    k8, ks, _ = F.quantize_rotate(k, signs, tile=tile)
    v8, vs, _ = F.quantize_tiles(v, tile=tile)
    o_m, _ = F.mirrored_attention(q8, k8, v8, qs, ks, vs, True, SCALE, tile=tile)
    if rows is not None:
        return o_m[0, 0, rows], o_ref[0, 0, rows]
    return o_m, o_ref


def _rmse(a, b):
    return float(np.sqrt(np.mean((a - b) ** 2)))


def test_rotation_lowers_error_with_outliers():
    """Q, K, V with 0.1 % of entries x10: error with the rotation below 0.9x the error without."""
    ratios = []
    for seed in (11, 12, 13):
        q, k, v = _f64(*synthetic.draw_qkv(1, 1, 1024, D, seed=seed, dtype="bf16", outlier_rate=1e-3,
                                           outlier_scale=10.0))
        signs = synthetic.draw_signs(D, seed)
        e_rot = _rmse(*_method_error(q, k, v, signs, 128))
        e_none = _rmse(*_method_error(q, k, v, None, 128))
        print(f"seed {seed}: rmse rotated {e_rot:.5f}  unrotated {e_none:.5f}")
        ratios.append(e_rot / e_none)
    assert np.mean(ratios) < 0.9, ratios


@pytest.mark.parametrize("factor, expect_gain", [(1e-2, False), (1e-4, True)])
def test_tile_scales_against_one_scale_per_tensor(factor, expect_gain):
    """The first half of V scaled by `factor`; causal rows 0 .. N/2-1 see only that half."""
    n = 1024
    rows = slice(0, n // 2)
    ratios = []
    for seed in (11, 12):
        q, k, v = _f64(*synthetic.draw_qkv(1, 1, n, D, seed=seed, dtype="bf16"))
        v[0, 0, : n // 2] *= factor
        signs = synthetic.draw_signs(D, seed)
        rel = {}
        for tile in (128, n):
            a, b = _method_error(q, k, v, signs, tile, rows=rows)
            rel[tile] = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        print(f"factor {factor:g} seed {seed}: relative error per-tile {rel[128]:.4f}  per-tensor {rel[n]:.4f}")
        ratios.append(rel[128] / rel[n])
    if expect_gain:
        assert max(ratios) < 0.8, ratios
    else:
        assert all(0.8 < r < 1.25 for r in ratios), ratios


@pytest.mark.gpu
def test_gpu_rotation_lowers_error_with_outliers(fa):
    """The HIP path (pre-pass + fp8 attention) with and without the rotation of Q and K."""
    B, H, N = 1, 4, 2048
    q, k, v = synthetic.draw_qkv(B, H, N, D, seed=77, dtype="bf16", outlier_rate=1e-3, outlier_scale=10.0)
    signs = torch.from_numpy(synthetic.draw_signs(D, 77)).cuda()
    o_ref, _ = A.reference(*_f64(q, k, v), True, SCALE)
    err = {}
    for name, sg in (("rotated", signs), ("unrotated", None)):
        o, _, _ = fa.fp8_attention(q.cuda(), k.cuda(), v.cuda(), sg, causal=True, scale=SCALE)
        torch.cuda.synchronize()
        e = o.float().cpu().numpy().astype(np.float64) - o_ref
        err[name] = (float(np.sqrt(np.mean(e ** 2))), float(np.abs(e).max()))
        print(f"GPU fp8 {name}: rmse {err[name][0]:.5f}  max abs {err[name][1]:.4f}", flush=True)
    assert err["rotated"][0] < 0.9 * err["unrotated"][0], err


def _gpu_variant(fa, q, k, v, signs, per_tensor=False, p_bf16=False):
    o, _, (q8, k8, v8t, qs, ks, vs) = fa.fp8_attention(q.cuda(), k.cuda(), v.cuda(), signs, causal=True, scale=SCALE,
                                                        per_tensor=per_tensor, p_bf16=p_bf16)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy().astype(np.float64)
    v8 = v8t.cpu()[..., :q.shape[-2]].transpose(-1, -2).contiguous().numpy()
    deq = [F.dequantize(x8, xs) for x8, xs in ((q8.cpu().numpy(), qs.cpu().numpy()), (k8.cpu().numpy(), ks.cpu().numpy()),
                                                (v8, vs.cpu().numpy()))]
    return og, deq


def _mirrored_scaled_error(og, deq):
    """max |O_gpu - O_hat| / max(1, sum_j P_hat |V_hat|) over the heads (the G5b metric)."""
    worst = 0.0
    qd, kd, vd = deq
    o_hat, _ = A.reference(qd, kd, vd, True, SCALE)
    for h in range(qd.shape[1]):
        p = A.probabilities(qd[0, h], kd[0, h], True, SCALE)
        mass = p @ np.abs(vd[0, h])
        worst = max(worst, float((np.abs(og[0, h] - o_hat[0, h]) / np.maximum(1.0, mass)).max()))
    return worst


@pytest.mark.gpu
@pytest.mark.parametrize("outlier", [10.0, 50.0])
def test_gpu_fp8_ablation(fa, outlier):
    """B1 H4 N2048 causal, 0.1 % of Q, K, V entries x`outlier`: the shipped FP8 path (rotation,
    per-tile scales, P in e4m3) against each measure taken away or replaced."""
    B, H, N = 1, 4, 2048
    q, k, v = synthetic.draw_qkv(B, H, N, D, seed=77, dtype="bf16", outlier_rate=1e-3, outlier_scale=outlier)
    signs = torch.from_numpy(synthetic.draw_signs(D, 77)).cuda()
    o_ref, _ = A.reference(*_f64(q, k, v), True, SCALE)
    res = {}
    for name, sg, pt, pb in (("shipped", signs, False, False), ("no rotation", None, False, False),
                             ("per-tensor scales", signs, True, False), ("P in bf16", signs, False, True)):
        og, deq = _gpu_variant(fa, q, k, v, sg, per_tensor=pt, p_bf16=pb)
        e = og - o_ref
        res[name] = {"rmse": float(np.sqrt(np.mean(e ** 2))), "max": float(np.abs(e).max()),
                     "fro": float(np.linalg.norm(e) / np.linalg.norm(o_ref)),
                     "g5b": _mirrored_scaled_error(og, deq)}
        r = res[name]
        print(f"x{outlier:g} {name:18s}: vs exact rmse {r['rmse']:.5f} max {r['max']:.4f} rel-Frobenius {r['fro']:.4f}"
              f" | vs own dequantised operands (scaled) {r['g5b']:.4f}", flush=True)
    # incoherent processing: the rotation lowers the error against the exact output
    assert res["shipped"]["rmse"] < 0.9 * res["no rotation"]["rmse"], res
    # with these outliers one scale per tensor is no better than one per tile
    assert res["shipped"]["rmse"] <= 1.1 * res["per-tensor scales"]["rmse"], res
    # the kernel's own error comes from rounding P: in bf16 it stays within the bf16 budget,
    # below the e4m3 one, which stays within G5b
    assert res["P in bf16"]["g5b"] <= 2e-2 and res["P in bf16"]["g5b"] < res["shipped"]["g5b"] <= 8e-2, res
    assert res["P in bf16"]["rmse"] <= res["shipped"]["rmse"], res


@pytest.mark.gpu
def test_gpu_tile_scales_with_magnitude_spread(fa):
    """The first half of V scaled by 1e-4 (causal rows 0 .. N/2-1 see only that half): one
    scale per tensor pushes that half into e4m3's subnormals, per-tile scales do not."""
    n = 1024
    q, k, v = synthetic.draw_qkv(1, 2, n, D, seed=78, dtype="bf16")
    v = v.float()
    v[:, :, : n // 2] *= 1e-4
    v = v.to(torch.bfloat16)
    signs = torch.from_numpy(synthetic.draw_signs(D, 78)).cuda()
    o_ref, _ = A.reference(*_f64(q, k, v), True, SCALE)
    rel = {}
    for name, pt in (("per-tile", False), ("per-tensor", True)):
        og, _ = _gpu_variant(fa, q, k, v, signs, per_tensor=pt)
        a, b = og[:, :, : n // 2], o_ref[:, :, : n // 2]
        rel[name] = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        print(f"V half x1e-4, {name}: relative error of the rows that see only that half {rel[name]:.4f}", flush=True)
    assert rel["per-tile"] < 0.8 * rel["per-tensor"], rel

