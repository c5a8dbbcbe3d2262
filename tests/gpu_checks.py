"""Comparison helpers for the GPU parity tests (CPU-side arithmetic only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention as A
from oracle import fp8 as F

# Gates.  fp32: 1e-5 on O and LSE.  bf16: 2e-2 on O against the unrounded
# fp64 output, 1e-3 on LSE.  fp8: against the oracle of the dequantised
# operands, the error of O_ic relative to max(1, sum_j P_ij |V_jc|) at most
# 8e-2, LSE within 1e-3 * max(1, |LSE|).
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}
FP8_O_TOL = 8e-2
FP8_LSE_TOL = 1e-3
# fp8 operands with the probabilities kept in bf16 (fa_fwd_fp8_pbf16): the bf16 budget
FP8_PBF16_O_TOL = 2e-2
# fp8 workload against the un-quantised inputs, relative Frobenius error per head: the
# method's own error on the checked heads (0.095-0.111, the oracle's quantiser and fp64
# attention of its operands) with room for the device's rounding of P and O
FP8_REL_FRO_BUDGET = 0.125


def log(msg: str):
    print(msg, flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """Rows that include the first, last and tile-boundary rows plus random ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [r for r in (0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 2, N - 1)
             if 0 <= r < N]
    rnd = rng.choice(N, size=min(N, n), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), rnd]))


def compare_attention(o_gpu, lse_gpu, q, k, v, causal, scale, dtype, heads=None, rows=None, chunk=4096):
    """max |dO|, max |dLSE| over the selected (b, h) heads and query rows (all rows when
    rows is None); the oracle runs on at most `chunk` rows at a time (each against all keys)."""
    o_gpu, lse_gpu = to_np(o_gpu), to_np(lse_gpu)
    B, H, N, d = q.shape
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    eo = el = 0.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        for c0 in range(0, len(rows), chunk):
            rr = rows[c0:c0 + chunk]
            o_ref, l_ref = A.reference(q[sl], k[sl], v[sl], causal, scale, rows=rr)
            og, lg = o_gpu[sl][:, :, rr], lse_gpu[sl][:, :, rr]
            assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), (b, h)
            eo = max(eo, float(np.abs(og - o_ref).max()))
            el = max(el, float(np.abs(lg - l_ref).max()))
    return eo, el


def rel_frobenius(o_gpu, q, k, v, causal, scale, heads, chunk=4096):
    """Per head ||O_gpu - O||_F / ||O||_F against the exact oracle of q, k, v."""
    o_gpu = to_np(o_gpu)
    N = q.shape[2]
    out = []
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        num = den = 0.0
        for c0 in range(0, N, chunk):
            rr = np.arange(c0, min(N, c0 + chunk))
            o_ref, _ = A.reference(q[sl], k[sl], v[sl], causal, scale, rows=rr)
            num += float(((o_gpu[sl][:, :, rr] - o_ref) ** 2).sum())
            den += float((o_ref ** 2).sum())
        out.append(np.sqrt(num / den))
    return out


def check_codes(codes_gpu, scale_gpu, x, signs, transposed=False, per_tensor=False):
    """Quantiser parity against the oracle's exact (fp64) rotation and scaling.

    The device computes the rotation as a fast Walsh-Hadamard transform in
    fp32 (log2(d) rounded additions per output) and the scaled value as one
    fp32 product, so its scaled value t differs from the exact one by at most
      delta = mult * log2(d) * u * sum_j |x_j|  +  |t| * (log2(d) * u * S / amax + 3u)
    (u = 2^-24, sum over the row's inputs, S = the largest such row sum in
    the tile; the second term covers the rounded tile amax and multiplier;
    without rotation log2(d) is 0).  A code may differ from the oracle's only
    where rounding some value within 2 * delta of the exact one gives the
    device's code -- both codes are then correct roundings of values the
    arithmetic cannot tell apart.  Rounding is monotone, so that holds exactly
    when the device's code value lies between the values of the codes of
    t - 2 delta and t + 2 delta.  Codes are compared by value: +0 and -0 (0x00,
    0x80) are the same zero, whose sign the oracle's fp64 rotation can get
    from a rounding residue where the exact transform is 0.  Scales must agree
    within the same relative bound.  per_tensor: one scale for the whole tensor
    (fa_quant_rotate_fp8_tensor), against the oracle's quantize_rotate_tensor;
    the bounds then use the tensor's largest row sum.  Returns (n_mismatch,
    n_total)."""
    u = 2.0 ** -24
    codes_gpu = codes_gpu.cpu()
    if transposed:
        # [B, H, d, N64]: the rows past N are padding and must hold code 0
        n = x.shape[-2]
        assert codes_gpu.shape[-1] == (n + 63) // 64 * 64, codes_gpu.shape
        assert int(codes_gpu[..., n:].abs().sum()) == 0 if codes_gpu.shape[-1] > n else True
        codes_gpu = codes_gpu[..., :n].transpose(-1, -2)
    codes_gpu = codes_gpu.contiguous().numpy()
    sg = None if signs is None else np.asarray(signs.cpu() if hasattr(signs, "cpu") else signs)
    xf = to_np(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    c_ref, s_ref, t = (F.quantize_rotate_tensor if per_tensor else F.quantize_rotate)(xf, sg)
    B, H, N, d = xf.shape
    depth = 0 if sg is None else int(np.log2(d))
    rowsum = np.abs(xf).sum(axis=-1)                       # [B, H, N]
    nt = s_ref.shape[-1]
    pad = nt * F.TILE_ROWS - N
    tile_max_rowsum = np.pad(rowsum, ((0, 0), (0, 0), (0, pad))).reshape(B, H, nt, F.TILE_ROWS).max(-1)
    if per_tensor:
        tile_max_rowsum = np.full_like(tile_max_rowsum, rowsum.max())
    amax = s_ref * F.E4M3_MAX * (np.sqrt(d) if sg is not None else 1.0)   # exact amax of the transform
    rel_tile = depth * u * tile_max_rowsum / np.where(amax > 0, amax, 1.0) + 3 * u  # [B, H, nt]
    s_gpu = scale_gpu.cpu().numpy().astype(np.float64)
    rel = np.abs(s_gpu - s_ref) / s_ref
    assert np.all(rel <= 2 * rel_tile + 4 * u), f"scale mismatch {rel.max()}"
    g_val = F.e4m3_decode(codes_gpu)
    assert not np.isnan(g_val).any(), "NaN code from the device"
    bad = g_val != F.e4m3_decode(c_ref)
    n_bad = int(bad.sum())
    if n_bad:
        mult = F.E4M3_MAX / np.where(amax > 0, amax, 1.0)
        rel_e = np.repeat(rel_tile, F.TILE_ROWS, axis=2)[:, :, :N, None]
        mult_e = np.repeat(mult, F.TILE_ROWS, axis=2)[:, :, :N, None]
        delta = 2 * (mult_e * depth * u * rowsum[..., None] + np.abs(t) * rel_e)
        tb, db_ = t[bad], np.broadcast_to(delta, t.shape)[bad]
        lo, hi = F.e4m3_decode(F.e4m3_encode(tb - db_)), F.e4m3_decode(F.e4m3_encode(tb + db_))
        ok = (g_val[bad] >= lo) & (g_val[bad] <= hi)
        assert ok.all(), f"{int((~ok).sum())} of {n_bad} differing codes are not explained by fp32 rounding"
    return n_bad, codes_gpu.size


def fp8_errors(o_gpu, lse_gpu, q8, k8, v8t, qs, ks, vs, causal, scale, heads, rows=None):
    """Errors of the fp8 kernel against the oracle of its own dequantised operands."""
    o_gpu, lse_gpu = to_np(o_gpu), to_np(lse_gpu)
    q8, k8 = q8.cpu().numpy(), k8.cpu().numpy()
    v8 = v8t.cpu()[..., :q8.shape[-2]].transpose(-1, -2).contiguous().numpy()
    qs, ks, vs = qs.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()
    worst_rel = worst_abs = worst_lse = 0.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qd, kd, vd = F.dequantize(q8[sl], qs[sl]), F.dequantize(k8[sl], ks[sl]), F.dequantize(v8[sl], vs[sl])
        o_ref, l_ref = A.reference(qd, kd, vd, causal, scale, rows=rows)
        p = A.probabilities(qd[0, 0], kd[0, 0], causal, scale, rows=rows)
        mass = p @ np.abs(vd[0, 0])
        og = o_gpu[sl][0, 0] if rows is None else o_gpu[sl][0, 0][rows]
        lg = lse_gpu[sl][0, 0] if rows is None else lse_gpu[sl][0, 0][rows]
        assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg)), (b, h)
        err = np.abs(og - o_ref[0, 0])
        worst_rel = max(worst_rel, float((err / np.maximum(1.0, mass)).max()))
        worst_abs = max(worst_abs, float(err.max()))
        worst_lse = max(worst_lse, float((np.abs(lg - l_ref[0, 0]) / np.maximum(1.0, np.abs(l_ref[0, 0]))).max()))
    return worst_rel, worst_abs, worst_lse


# Backward, element by element: each gradient element is a sum of terms, and rounding
# P and dS to bf16, the fp32 accumulations and the final bf16 rounding each move it by
# a fraction of the sum of the magnitudes of its terms:
#   dV_jc = sum_i P_ij dO_ic                -> sum_i P_ij |dO_ic|
#   dQ_ic = scale sum_j dS_ij K_jc          -> |scale| sum_j |dS_ij| |K_jc|
#   dK_jc = scale sum_i dS_ij Q_ic          -> |scale| sum_i |dS_ij| |Q_ic|
# (the same construction as the FP8 G5b gate).  The floor, 1e-3 of the tensor's largest
# such sum (at least 1e-3), covers the fp32 cancellation in dP - D, whose rounding does
# not shrink with |dP - D|.  The bound is the forward's bf16 budget.
BWD_ELEM_TOL = 2e-2


def bwd_term_scales(q, k, v, do, o, causal: bool, scale: float, chunk: int = 2048):
    """(mQ, mK, mV): the sums of term magnitudes above, float64 [B, H, N, d], with D
    from the given output o; query rows in chunks of `chunk` (bounded memory)."""
    q, k, v, do, o = (to_np(x) for x in (q, k, v, do, o))
    B, H, N, d = q.shape
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                p = A.probabilities(q[b, h], k[b, h], causal, scale, rows=rows)
                dp = do[b, h, rows] @ v[b, h].T
                dd = (do[b, h, rows] * o[b, h, rows]).sum(axis=1, keepdims=True)
                ds = np.abs(p * (dp - dd))
                mv[b, h] += p.T @ np.abs(do[b, h, rows])
                mq[b, h, rows] = abs(scale) * (ds @ np.abs(k[b, h]))
                mk[b, h] += abs(scale) * (ds.T @ np.abs(q[b, h, rows]))
    return mq, mk, mv


def bwd_elem_errors(got, ref, scales) -> list:
    """max over elements of |g - g_ref| / (term scale + floor), per gradient tensor."""
    out = []
    for g, r, m in zip(got, ref, scales):
        g = to_np(g)
        floor = 1e-3 * max(1.0, float(m.max()))
        out.append(float((np.abs(g - r) / (m + floor)).max()))
    return out
