"""CPU pins of the fp8 half of the oracle: e4m3 codec, rotation, block quantisation."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import attention as A
from oracle import fp8 as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- codec
def test_decode_spec_anchors():
    with open(os.path.join(GOLDEN, "e4m3_anchors.json")) as f:
        anchors = json.load(f)["anchors"]
    for a in anchors:
        got = F.e4m3_decode([int(a["code"], 16)])[0]
        want = float(eval(a["value"], {"nan": float("nan")})) if a["value"] != "nan" else float("nan")
        if math.isnan(want):
            assert math.isnan(got), a
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), a


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = F.e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_encode_decode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.Generator(np.random.PCG64(21))
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448)
    # also every midpoint between adjacent finite codes (exact ties)
    vals = np.unique(F.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids, vals, -vals])
    assert np.array_equal(F.e4m3_encode(x), _torch_encode(x))


def test_ties_go_to_even_and_saturation():
    # 1.0625 lies halfway between 1.0 (0x38, even mantissa) and 1.125 (0x39)
    assert F.e4m3_encode([1.0625])[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert F.e4m3_encode([1.1875])[0] == 0x3A
    # half of the smallest subnormal rounds to zero (even), 1.5 of it to 2 steps
    assert F.e4m3_encode([2.0 ** -10])[0] == 0x00
    assert F.e4m3_encode([1.5 * 2.0 ** -9])[0] == 0x02
    for big in (449.0, 464.0, 500.0, 1e30, np.inf):
        assert F.e4m3_encode([big])[0] == 0x7E
        assert F.e4m3_encode([-big])[0] == 0xFE
    assert F.e4m3_encode([np.nan])[0] & 0x7F == 0x7F


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_sylvester_matches_scipy(d):
    assert np.array_equal(F.sylvester_hadamard(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthogonal_and_preserves_scores(d):
    rng = np.random.Generator(np.random.PCG64(22))
    s = (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)
    R = F.rotation_matrix(s)
    assert np.max(np.abs(R @ R.T - np.eye(d))) <= 1e-14
    q, k, v = (rng.standard_normal((1, 2, 40, d)) for _ in range(3))
    qr, kr = F.rotate(q, s), F.rotate(k, s)
    assert np.max(np.abs(qr @ np.swapaxes(kr, -1, -2) - q @ np.swapaxes(k, -1, -2))) <= 1e-12
    for causal in (False, True):
        o1, l1 = A.reference(q, k, v, causal, 1 / np.sqrt(d))
        o2, l2 = A.reference(qr, kr, v, causal, 1 / np.sqrt(d))
        assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12
    # a rotation spreads a single outlier over all d coordinates with equal magnitude
    e = np.zeros((1, 1, 1, d)); e[..., 3] = 50.0
    assert np.allclose(np.abs(F.rotate(e, s)), 50.0 / np.sqrt(d))


# ---------------------------------------------------------------- quantisation
@pytest.mark.parametrize("N", [128, 300, 1])
def test_quantizer_bounds(N):
    rng = np.random.Generator(np.random.PCG64(23))
    y = rng.standard_normal((2, 3, N, 16)) * np.exp(rng.standard_normal((2, 3, N, 16)) * 2)
    codes, scales, t = F.quantize_tiles(y)
    nt = -(-N // 128)
    assert scales.shape == (2, 3, nt)
    deq = F.dequantize(codes, scales)
    for i in range(nt):
        blk = y[:, :, i * 128:(i + 1) * 128]
        amax = np.abs(blk).max(axis=(2, 3))
        assert np.allclose(scales[:, :, i], amax / 448.0, rtol=0, atol=0)
        # the tile's largest entry maps to +-448 exactly
        flat = np.abs(blk).reshape(2, 3, -1).argmax(axis=-1)
        c = codes[:, :, i * 128:(i + 1) * 128].reshape(2, 3, -1)
        top = np.take_along_axis(c, flat[..., None], axis=-1)
        assert np.all((top & 0x7F) == 0x7E)
    sc = np.repeat(scales, 128, axis=2)[:, :, :N, None]
    err = np.abs(deq - y)
    normal = np.abs(y) >= 2.0 ** -6 * sc
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y)[normal] * (1 + 1e-12))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(sc, y.shape)[~normal] * (1 + 1e-12))
    # codes agree with torch's float8_e4m3fn cast of the same scaled values
    assert np.array_equal(codes, _torch_encode(t))


def test_zero_tile_gets_unit_scale():
    y = np.zeros((1, 1, 256, 8)); y[0, 0, 200, 1] = 3.0
    codes, scales, _ = F.quantize_tiles(y)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, :128] == 0)
    assert scales[0, 0, 1] == 3.0 / 448


def test_tiny_tile_counts_as_zero():
    """A tile of magnitudes below 2^-96 (bf16 subnormals here) gets scale 1 and codes of
    zero (448 / amax would overflow fp32); one just above keeps the amax / 448 rule."""
    y = np.zeros((1, 1, 256, 8))
    y[0, 0, :128] = np.linspace(-1, 1, 128 * 8).reshape(128, 8) * 2.0 ** -130
    y[0, 0, 128:] = np.linspace(-1, 1, 128 * 8).reshape(128, 8) * 2.0 ** -90
    codes, scales, _ = F.quantize_tiles(y)
    assert scales[0, 0, 0] == 1.0 and np.all((codes[0, 0, :128] & 0x7F) == 0)
    assert scales[0, 0, 1] == 2.0 ** -90 / 448 and np.isfinite(448 / (2.0 ** -90))
    assert np.all(np.isfinite(F.dequantize(codes, scales)))
    assert (codes[0, 0, 255, 7] & 0x7F) == 0x7E  # the amax element still maps to 448
    # the rotated path applies the bound to the unnormalised transform (sqrt(d) x larger)
    s = np.ones(8, dtype=np.int8)
    x = np.zeros((1, 1, 128, 8)); x[0, 0, 0, 0] = 2.0 ** -97  # transform amax 2^-97 < 2^-96
    c, sc, _ = F.quantize_rotate(x, s)
    assert sc[0, 0, 0] == 1.0 and np.all((c & 0x7F) == 0)
    x[0, 0, 0, 0] = 2.0 ** -95
    c, sc, _ = F.quantize_rotate(x, s)
    assert sc[0, 0, 0] == pytest.approx(2.0 ** -95 / np.sqrt(8) / 448, rel=1e-12)


def test_tensor_scale():
    """One scale for the whole tensor: amax over every (b, h, row, column) / 448, in every
    tile entry; the amax element maps to 448; one tile of one head is the tile rule; the
    dequantisation error obeys the same bounds as the tile quantiser, against that scale."""
    rng = np.random.Generator(np.random.PCG64(29))
    y = rng.standard_normal((2, 3, 300, 16)) * np.exp(rng.standard_normal((2, 3, 300, 16)))
    y[1, 2, 77, 5] = -400.0  # the tensor's amax
    codes, scales, t = F.quantize_tensor(y)
    assert np.abs(y).max() == 400.0
    assert scales.shape == (2, 3, 3) and np.all(scales == 400.0 / 448)
    assert codes[1, 2, 77, 5] == 0xFE  # -448
    assert np.count_nonzero((codes & 0x7F) == 0x7E) == 1
    deq = F.dequantize(codes, scales)
    err = np.abs(deq - y)
    normal = np.abs(y) >= 2.0 ** -6 * (400.0 / 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y)[normal] * (1 + 1e-12))
    assert np.all(err[~normal] <= 2.0 ** -10 * (400.0 / 448) * (1 + 1e-12))
    one = y[:1, :1, :128]
    c1, s1, _ = F.quantize_tensor(one)
    c2, s2, _ = F.quantize_tiles(one)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # rotated: the same rotation as the tile quantiser, one scale over the rotated tensor
    s = (rng.integers(0, 2, 16) * 2 - 1).astype(np.int8)
    c3, s3, _ = F.quantize_rotate_tensor(y, s)
    c4, s4, _ = F.quantize_tensor(y @ F.rotation_matrix(s))
    assert np.array_equal(c3, c4) and np.array_equal(s3, s4)
    assert np.all(F.quantize_tensor(np.zeros((1, 1, 5, 4)))[1] == 1.0)


def test_mirrored_oracle_is_exact_on_representable_inputs():
    """Inputs that are e4m3 values times a tile scale quantise losslessly,
    so the mirrored oracle must equal the exact one there."""
    rng = np.random.Generator(np.random.PCG64(24))
    codes = rng.integers(0, 0x7E, size=(3, 1, 2, 256, 16)).astype(np.uint8)
    codes[..., 0, 0] = 0x7E  # each tile's amax is the code 448 -> scale recovered exactly
    codes[..., 128, 0] = 0x7E
    sign = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    vals = F.e4m3_decode(codes | sign)
    tile_scale = np.array([0.5, 0.125])[None, None, None, :, None, None]
    x = (vals.reshape(3, 1, 2, 2, 128, 16) * tile_scale).reshape(3, 1, 2, 256, 16)
    q, k, v = x
    qc, qs, _ = F.quantize_tiles(q)
    kc, ks, _ = F.quantize_tiles(k)
    vc, vs, _ = F.quantize_tiles(v)
    assert np.array_equal(F.dequantize(qc, qs), q)
    for causal in (False, True):
        o1, l1 = F.mirrored_attention(qc, kc, vc, qs, ks, vs, causal, 0.1)
        o2, l2 = A.reference(q, k, v, causal, 0.1)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_quantize_rotate_uses_the_shared_rotation():
    rng = np.random.Generator(np.random.PCG64(25))
    s = (rng.integers(0, 2, 64) * 2 - 1).astype(np.int8)
    x = rng.standard_normal((1, 2, 130, 64))
    c1, s1, t1 = F.quantize_rotate(x, s)
    c2, s2, t2 = F.quantize_tiles(x @ F.rotation_matrix(s))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    c3, s3, _ = F.quantize_rotate(x, None)
    c4, s4, _ = F.quantize_tiles(x)
    assert np.array_equal(c3, c4) and np.array_equal(s3, s4)
