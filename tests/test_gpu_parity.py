"""GPU parity: the HIP kernels (through the C-ABI) against the fp64 oracle.

Small shapes are compared element by element over every output; the five
full-size workloads are run in the exact launch configuration the benchmark
times and compared on sampled heads and rows (which the oracle computes one
by one, against all keys)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import fp8 as F
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(fa, q, k, v, causal, scale):
    o, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# --------------------------------------------------------------------------- small shapes, every output
# B*H a multiple of 8 takes the grouped block order of non-causal launches
SMALL = [(1, 2, n, d) for n in (1, 7, 64, 100, 128, 129, 255, 300, 513) for d in (64, 128)] + [
    (2, 3, 257, 64), (2, 4, 300, 128), (2, 8, 129, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}N{}d{}".format(*s))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_shapes(fa, dtype, shape, causal):
    B, H, N, d = shape
    G.log(f"case {dtype} {shape} causal={causal}")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=N * 7 + d + causal, dtype=dtype)
    o, lse = _run(fa, q, k, v, causal, d ** -0.5)
    assert o.dtype == q.dtype and lse.shape == (B, H, N)
    eo, el = G.compare_attention(o, lse, q, k, v, causal, d ** -0.5, dtype)
    tol_o, tol_l = G.TOL[dtype]
    G.log(f"  max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
    assert eo <= tol_o and el <= tol_l


@pytest.mark.parametrize("scale", [0.0, -0.15, 0.5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scale_edge_cases(fa, dtype, scale):
    """scale 0 (uniform weights), a negative scale (max/min swap), a large one."""
    G.log(f"case {dtype} scale={scale}")
    q, k, v = synthetic.draw_qkv(1, 2, 300, 128, seed=99, dtype=dtype)
    for causal in (False, True):
        o, lse = _run(fa, q, k, v, causal, scale)
        eo, el = G.compare_attention(o, lse, q, k, v, causal, scale, dtype)
        G.log(f"  causal={causal} max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= G.TOL[dtype][0] and el <= G.TOL[dtype][1]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("where", ["k", "v"])
def test_nan_input_propagates(fa, where, causal, d):
    """A NaN in one element of key row j (of K or of V, head 1) reaches exactly the
    query rows that see key j: their whole O row and LSE (K) or their O column (V)
    are NaN. Every other output is finite and matches the oracle on the same inputs
    with that element set to zero (a key a row does not see cannot change it)."""
    B, H, N, j, c = 1, 2, 200, 77, 3
    G.log(f"case nan in {where} causal={causal} d={d}")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=500 + d, dtype="bf16")
    clean = {"k": k, "v": v}
    bad = clean[where].clone()
    bad[0, 1, j, c] = float("nan")
    clean[where] = clean[where].clone()
    clean[where][0, 1, j, c] = 0.0
    args = {"k": k, "v": v}
    args[where] = bad
    o, lse = _run(fa, q, args["k"], args["v"], causal, d ** -0.5)
    og, lg = G.to_np(o), G.to_np(lse)
    sees = np.arange(N) >= j if causal else np.ones(N, dtype=bool)
    if where == "k":
        assert np.all(np.isnan(og[0, 1, sees])) and np.all(np.isnan(lg[0, 1, sees]))
        finite_rows = np.nonzero(~sees)[0]
    else:
        assert np.all(np.isnan(og[0, 1, sees, c]))
        assert np.all(np.isfinite(np.delete(og[0, 1, sees], c, axis=1))) and np.all(np.isfinite(lg[0, 1, sees]))
        finite_rows = np.arange(N)
    # head 0 entirely, and head 1 outside the NaN's reach, against the oracle
    eo, el = G.compare_attention(o[:, :1], lse[:, :1], q[:, :1], clean["k"][:, :1], clean["v"][:, :1], causal,
                                 d ** -0.5, "bf16")
    assert eo <= G.TOL["bf16"][0] and el <= G.TOL["bf16"][1]
    if len(finite_rows):
        if where == "v":  # compare head 1 without column c
            keep = [x for x in range(d) if x != c]
            eo1, el1 = G.compare_attention(o[:, 1:, :, keep], lse[:, 1:], q[:, 1:], clean["k"][:, 1:],
                                           clean["v"][:, 1:, :, keep], causal, d ** -0.5, "bf16", rows=finite_rows)
        else:
            eo1, el1 = G.compare_attention(o[:, 1:], lse[:, 1:], q[:, 1:], clean["k"][:, 1:], clean["v"][:, 1:],
                                           causal, d ** -0.5, "bf16", rows=finite_rows)
        G.log(f"  finite part: max|dO| {max(eo, eo1):.3e}  max|dLSE| {max(el, el1):.3e}")
        assert eo1 <= G.TOL["bf16"][0] and el1 <= G.TOL["bf16"][1]


def test_empty_problem_launches_nothing(fa):
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = fa.fa_fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (2, 3, 0)


def test_unsupported_head_dim_raises(fa):
    q = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------- the five workloads at full size
def _heads(B, H, n):
    idx = np.linspace(0, B * H - 1, n).round().astype(int)
    return [(int(i) // H, int(i) % H) for i in np.unique(idx)]


@pytest.mark.parametrize("wi", [0, 1, 2, 3])
def test_workload_full_size(fa, wi):
    w = synthetic.WORKLOADS[wi]
    G.log(f"case workload {w.name}")
    q, k, v, _ = synthetic.workload_inputs(w)
    o, lse = _run(fa, q, k, v, w.causal, w.scale)
    tol_o, tol_l = G.TOL[w.dtype]
    if w.N <= 2048:  # whole heads (every row of 8 heads, spread over the batch and the block order)
        eo, el = G.compare_attention(o, lse, q, k, v, w.causal, w.scale, w.dtype, heads=_heads(w.B, w.H, 8))
        G.log(f"  whole heads: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= tol_o and el <= tol_l
    else:  # N = 16384: two whole heads, every row against every key (the oracle in row chunks)
        eo, el = G.compare_attention(o, lse, q, k, v, w.causal, w.scale, w.dtype, heads=[(0, 0), (0, w.H - 1)])
        G.log(f"  whole heads (0,0), (0,{w.H - 1}): max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
        assert eo <= tol_o and el <= tol_l
    rows = G.sample_rows(w.N, 96, seed=wi)
    eo, el = G.compare_attention(o, lse, q, k, v, w.causal, w.scale, w.dtype,
                                 heads=_heads(w.B, w.H, 16 if w.N > 2048 else 64), rows=rows)
    G.log(f"  sampled rows: max|dO| {eo:.3e}  max|dLSE| {el:.3e}")
    assert eo <= tol_o and el <= tol_l
    # deterministic: two more launches reproduce every bit
    for _ in range(2):
        o2, lse2 = _run(fa, q, k, v, w.causal, w.scale)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)


# --------------------------------------------------------------------------- fp8
def _fp8_case(fa, q, k, v, signs, causal, scale, p_bf16=False, per_tensor=False):
    sg = None if signs is None else torch.from_numpy(signs).to(DEV)
    o, lse, aux = fa.fp8_attention(q.to(DEV), k.to(DEV), v.to(DEV), sg, causal=causal, scale=scale, p_bf16=p_bf16,
                                   per_tensor=per_tensor)
    torch.cuda.synchronize()
    return o, lse, aux


@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("N", [1, 100, 128, 200, 256, 640])
@pytest.mark.parametrize("d", [64, 128])
def test_quantizer_small(fa, N, d, per_tensor):
    G.log(f"case quantizer N={N} d={d} per_tensor={per_tensor}")
    q, _, _ = synthetic.draw_qkv(2, 2, N, d, seed=N + d, dtype="bf16", outlier_rate=0.01, outlier_scale=50.0)
    signs = synthetic.draw_signs(d, N)
    sg = torch.from_numpy(signs).to(DEV)
    for rot in (True, False):
        for tr in (False, True):
            x8, xs = fa.fa_quant_rotate_fp8(q.to(DEV), sg if rot else None, tr, per_tensor=per_tensor)
            torch.cuda.synchronize()
            if per_tensor:
                assert bool((xs == xs.flatten()[0]).all())  # one scale in every tile entry
            nb, nt = G.check_codes(x8, xs, q, signs if rot else None, transposed=tr, per_tensor=per_tensor)
            G.log(f"  rotate={rot} transposed={tr}: {nb} of {nt} codes at rounding ties")
            assert nb <= 1e-2 * nt


@pytest.mark.parametrize("N", [1, 200, 640])
@pytest.mark.parametrize("d", [64, 128])
def test_quantizer_fused_qkv_matches_separate_calls(fa, d, N):
    """The one-launch pre-pass equals the three fa_quant_rotate_fp8 calls bit for bit."""
    G.log(f"case fused pre-pass d={d} N={N}")
    q, k, v = (x.to(DEV) for x in synthetic.draw_qkv(2, 3, N, d, seed=N + 5 * d, dtype="bf16", outlier_rate=0.01,
                                                        outlier_scale=50.0))
    for sg in (torch.from_numpy(synthetic.draw_signs(d, N)).to(DEV), None):
        fused = fa.fa_quant_rotate_fp8_qkv(q, k, v, sg)
        q8, qs = fa.fa_quant_rotate_fp8(q, sg, False)
        k8, ks = fa.fa_quant_rotate_fp8(k, sg, False)
        v8t, vs = fa.fa_quant_rotate_fp8(v, None, True)
        torch.cuda.synchronize()
        for a, b in zip(fused, (q8, k8, v8t, qs, ks, vs)):
            assert torch.equal(a, b)


@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_quantizer_tiny_tile(fa, d, rot):
    """A tile of bf16 subnormals (magnitudes below 2^-96) quantises as an all-zero tile
    (scale 1, codes of zero, no NaN codes); the next tile, at 2^-90, keeps the amax rule."""
    G.log(f"case quantizer tiny tile d={d} rotate={rot}")
    x = torch.linspace(-1, 1, 256 * d, dtype=torch.float64).reshape(1, 1, 256, d)
    x[:, :, :128] *= 2.0 ** -130
    x[:, :, 128:] *= 2.0 ** -90
    x = x.to(torch.bfloat16)
    signs = synthetic.draw_signs(d, 5)
    sg = torch.from_numpy(signs).to(DEV) if rot else None
    for tr in (False, True):
        x8, xs = fa.fa_quant_rotate_fp8(x.to(DEV), sg, tr)
        torch.cuda.synchronize()
        c = x8.cpu()
        c = c[..., :256].transpose(-1, -2) if tr else c
        assert float(xs[0, 0, 0]) == 1.0 and bool(((c[0, 0, :128] & 0x7F) == 0).all())
        assert not bool(((c & 0x7F) == 0x7F).any())  # no NaN code anywhere
        assert 0.0 < float(xs[0, 0, 1]) < 1e-20
        live = (x8[..., 128:256].contiguous(), x8[:, :, 128:]) [0 if tr else 1]
        nb, nt = G.check_codes(live, xs[:, :, 1:], x[:, :, 128:], signs if rot else None, transposed=tr)
        assert nb <= 1e-2 * nt


@pytest.mark.parametrize("p_bf16", [False, True])
@pytest.mark.parametrize("outliers", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 128, 200, 256, 640])
def test_fp8_small(fa, N, causal, outliers, p_bf16):
    """G5b on every output; the P-in-bf16 variant rounds P to bf16, so it is held to the
    bf16 budget (2e-2) in the same scaled metric."""
    G.log(f"case fp8 N={N} causal={causal} outliers={outliers} p_bf16={p_bf16}")
    d = 128
    q, k, v = synthetic.draw_qkv(1, 2, N, d, seed=3 * N + causal, dtype="bf16",
                                 outlier_rate=1e-3 if outliers else 0.0, outlier_scale=50.0)
    signs = synthetic.draw_signs(d, N + 1)
    o, lse, (q8, k8, v8t, qs, ks, vs) = _fp8_case(fa, q, k, v, signs, causal, d ** -0.5, p_bf16=p_bf16)
    rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, causal, d ** -0.5, heads=[(0, 0), (0, 1)])
    G.log(f"  vs dequantised oracle: scaled err {rel:.3e} (abs {ab:.3e})  LSE rel {el:.3e}")
    assert rel <= (G.FP8_PBF16_O_TOL if p_bf16 else G.FP8_O_TOL) and el <= G.FP8_LSE_TOL


@pytest.mark.parametrize("p_bf16", [False, True])
@pytest.mark.parametrize("scale", [0.0, -0.15, 0.5])
def test_fp8_scales(fa, scale, p_bf16):
    """Negative scale (every Q code's sign bit flipped), zero scale (Q zeroed), large scale."""
    G.log(f"case fp8 scale={scale} p_bf16={p_bf16}")
    d, N = 128, 300
    q, k, v = synthetic.draw_qkv(1, 2, N, d, seed=41, dtype="bf16")
    signs = synthetic.draw_signs(d, 42)
    o, lse, (q8, k8, v8t, qs, ks, vs) = _fp8_case(fa, q, k, v, signs, True, scale, p_bf16=p_bf16)
    rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, True, scale, heads=[(0, 0), (0, 1)])
    G.log(f"  vs dequantised oracle: scaled err {rel:.3e} (abs {ab:.3e})  LSE rel {el:.3e}")
    assert rel <= (G.FP8_PBF16_O_TOL if p_bf16 else G.FP8_O_TOL) and el <= G.FP8_LSE_TOL


def _steady_shift_moves(q8, k8, qs, ks, causal, scale):
    """How many times the lazy shift (moved to a 64-key tile's row maximum when that
    exceeds it by more than 2, in log2 units) moves in the unmasked steps after a row
    block's first tile, replayed in fp64 on the dequantised codes of head (0, 0).  A
    256-query block's unmasked tiles are those wholly before its first query."""
    qd = F.dequantize(q8.cpu().numpy(), qs.cpu().numpy())[0, 0]
    kd = F.dequantize(k8.cpu().numpy(), ks.cpu().numpy())[0, 0]
    n = qd.shape[0]
    s = (qd @ kd.T) * scale * np.log2(np.e)
    moves = 0
    for i in range(n):
        q0 = i // 256 * 256
        n_full = (min(n, q0 + 1) if causal else n) // 64
        m = -np.inf
        for t in range((n + 63) // 64):
            hi = min(n, 64 * t + 64, i + 1 if causal else n)
            if 64 * t >= hi:
                break
            mt = s[i, 64 * t:hi].max()
            if mt > m + 2.0:
                m = mt
                moves += int(1 <= t < n_full)
    return moves


@pytest.mark.parametrize("p_bf16", [False, True])
def test_fp8_rising_maxima(fa, p_bf16):
    """K rows scaled by 1 + 6 j / N, so the row maxima keep rising along the keys: the lazy
    shift moves in unmasked steps (counted on the dequantised codes), and O and the rounded
    row sum are carried to the new shift.  G5b on every output of both heads."""
    B, H, N, d = 1, 2, 1100, 128
    G.log(f"case fp8 rising maxima p_bf16={p_bf16}")
    q, k, v = synthetic.draw_qkv(B, H, N, d, seed=651, dtype="bf16")
    ramp = 1.0 + 6.0 * torch.arange(N, dtype=torch.float32) / N
    k = (k.float() * ramp[None, None, :, None]).to(torch.bfloat16)
    signs = synthetic.draw_signs(d, 652)
    for causal in (False, True):
        for scale in (d ** -0.5, 0.5):
            o, lse, (q8, k8, v8t, qs, ks, vs) = _fp8_case(fa, q, k, v, signs, causal, scale, p_bf16=p_bf16)
            moves = _steady_shift_moves(q8, k8, qs, ks, causal, scale)
            rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, causal, scale, heads=[(0, 0), (0, 1)])
            G.log(f"  causal={causal} scale={scale:.4f}: {moves} shift moves in unmasked steps of head 0; "
                  f"scaled err {rel:.3e} (abs {ab:.3e})  LSE rel {el:.3e}")
            assert moves > 100
            assert rel <= (G.FP8_PBF16_O_TOL if p_bf16 else G.FP8_O_TOL) and el <= G.FP8_LSE_TOL


def test_fp8_workload_full_size(fa):
    """The fp8 workload (B2 H16 N8192, x50 outliers) in the bench's launch configuration.
    G5a on three whole heads; G5b on two whole heads (all 8192 rows) and sampled rows of a
    third; the whole-tensor error against the un-quantised inputs gated per head; the
    P-in-bf16 variant on the same operands; three launches bitwise equal."""
    w = synthetic.WORKLOADS[4]
    G.log(f"case workload {w.name}")
    q, k, v, signs = synthetic.workload_inputs(w)
    o, lse, (q8, k8, v8t, qs, ks, vs) = _fp8_case(fa, q, k, v, signs, w.causal, w.scale)
    heads = _heads(w.B, w.H, 3)
    # G5a: the pre-pass against the oracle quantiser on whole heads
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        for x, x8, xs, sg, tr in ((q, q8, qs, signs, False), (k, k8, ks, signs, False), (v, v8t, vs, None, True)):
            nb, nt = G.check_codes(x8[sl], xs[sl], x[sl], sg, tr)
            G.log(f"  head {(b, h)}: {nb} of {nt} codes at rounding ties")
            assert nb <= 1e-2 * nt
    # G5b: the attention kernel against the oracle of its dequantised operands, whole heads
    rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, w.causal, w.scale, heads=heads[:2])
    G.log(f"  whole heads {heads[:2]} vs dequantised oracle: scaled err {rel:.3e} (abs {ab:.3e})  LSE rel {el:.3e}")
    assert rel <= G.FP8_O_TOL and el <= G.FP8_LSE_TOL
    rows = G.sample_rows(w.N, 128, seed=4)
    rel, ab, el = G.fp8_errors(o, lse, q8, k8, v8t, qs, ks, vs, w.causal, w.scale, heads=heads[2:], rows=rows)
    G.log(f"  sampled rows of {heads[2:]}: scaled err {rel:.3e} (abs {ab:.3e})  LSE rel {el:.3e}")
    assert rel <= G.FP8_O_TOL and el <= G.FP8_LSE_TOL
    # against the un-quantised inputs: the method's own error (fp64 attention of the oracle's
    # quantised operands) is 0.095-0.111 in relative Frobenius norm on these heads; the
    # device path may add little to it
    fro = G.rel_frobenius(o, q, k, v, w.causal, w.scale, heads)
    G.log(f"  vs un-quantised oracle: relative Frobenius error per head {['%.4f' % x for x in fro]}")
    assert max(fro) <= G.FP8_REL_FRO_BUDGET
    # the P-in-bf16 variant on the same operands, against the same dequantised oracle
    o16, l16 = fa.fa_fwd_fp8(q8, k8, v8t, qs, ks, vs, causal=w.causal, scale=w.scale, p_bf16=True)
    torch.cuda.synchronize()
    rel16, ab16, el16 = G.fp8_errors(o16, l16, q8, k8, v8t, qs, ks, vs, w.causal, w.scale, heads=heads[:1])
    G.log(f"  P in bf16, whole head {heads[0]}: scaled err {rel16:.3e} (abs {ab16:.3e})  LSE rel {el16:.3e}")
    assert rel16 <= G.FP8_PBF16_O_TOL and el16 <= G.FP8_LSE_TOL
    for _ in range(2):
        o2, lse2, _ = _fp8_case(fa, q, k, v, signs, w.causal, w.scale)
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
