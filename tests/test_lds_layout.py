"""The LDS tile layout of the gradient kernels, modelled on the CPU.

The dQ and dK/dV kernels keep each streamed tile (32 rows of d bf16 values) in LDS and
read it two ways: as rows (each lane 16 bytes of one row, `ds_read_b128`) and transposed
(`ds_read_b64_tr_b16`, each lane 8 bytes).  The rows are 2 d + 64 bytes apart and the
16-byte piece p of row R sits at piece p ^ ((R >> 2) & 3).  This test restates the
address arithmetic of the kernels' helpers (`piece_off`, `row_reader`, `tr_reader`) and
checks, for every lane:

* that the row readers' two per-lane bases with constant offsets reach the swizzled
  position of the piece they mean, for every chunk;
* that no access touches a 4-byte bank twice within one pass of the LDS (64 banks;
  16 lanes at a time for 16-byte accesses, 32 for 8-byte ones), so that neither read
  kind has bank conflicts (the SQ_LDS_BANK_CONFLICT counter reads 0 on the GPU).
"""
from collections import Counter

import pytest

KT = 32  # rows per tile


def stride(d):
    return 2 * d + 64


def swz(row):
    return (row >> 2) & 3


def piece_off(d, row, piece):
    return row * stride(d) + ((piece ^ swz(row)) << 4)


def permuted_row(i):
    return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC)


def row_reader(d, row, g):
    c = swz(row)
    b = row * stride(d) + 16 * (g ^ (c & 1))
    return b + 32 * (c >> 1), b - 32 * (c >> 1)


def row_read_addr(d, lane, ks):
    li, g = lane & 31, lane >> 5
    even, odd = row_reader(d, permuted_row(li), g)
    return (odd if ks & 1 else even) + ks * 32


def tr_reader(d, lane):
    grp16, l16 = lane >> 4, lane & 15
    r = 8 * (grp16 >> 1) + (l16 >> 2)
    q = 2 * (grp16 & 1) + ((l16 & 3) >> 1)
    h = 8 * (l16 & 1)
    lo = r * stride(d) + 16 * (q ^ swz(r)) + h
    hi = (r + 4) * stride(d) + 16 * (q ^ swz(r + 4)) + h
    return lo, hi


def worst_multiplicity(addrs, width, group):
    """Largest number of distinct addresses sharing a 4-byte bank within one pass."""
    worst = 1
    for g0 in range(0, len(addrs), group):
        banks = Counter()
        for a in set(addrs[g0:g0 + group]):
            for w in range(a // 4, (a + width) // 4):
                banks[w % 64] += 1
        worst = max(worst, max(banks.values()))
    return worst


@pytest.mark.parametrize("d", [64, 128])
def test_row_reads_reach_their_pieces(d):
    for lane in range(64):
        li, g = lane & 31, lane >> 5
        row = permuted_row(li)
        for ks in range(d // 16):
            assert row_read_addr(d, lane, ks) == piece_off(d, row, 2 * ks + g), (lane, ks)


@pytest.mark.parametrize("d", [64, 128])
def test_row_reads_are_conflict_free(d):
    for ks in range(d // 16):
        addrs = [row_read_addr(d, lane, ks) for lane in range(64)]
        assert worst_multiplicity(addrs, 16, 16) == 1, ks


@pytest.mark.parametrize("d", [64, 128])
def test_transposed_reads_stay_in_their_window_and_are_conflict_free(d):
    for db in range(d // 32):
        for mm in range(2):
            base = mm * 16 * stride(d) + db * 64
            for half in range(2):
                addrs = [base + tr_reader(d, lane)[half] for lane in range(64)]
                for a in addrs:
                    row, col = divmod(a, stride(d))
                    # 8 bytes inside the 64-byte window of d-block db, on one of the tile's rows
                    assert 0 <= row < KT and db * 64 <= col and col + 8 <= db * 64 + 64
                assert worst_multiplicity(addrs, 8, 32) == 1, (db, mm, half)


@pytest.mark.parametrize("d", [64, 128])
def test_swizzle_is_a_permutation_within_each_window(d):
    """Every (row, piece) has its own 16 bytes, inside the 64-byte window of its piece."""
    seen = set()
    for row in range(KT):
        for piece in range(d // 8):
            off = piece_off(d, row, piece)
            assert off not in seen
            seen.add(off)
            assert (off - row * stride(d)) // 64 == piece // 4
