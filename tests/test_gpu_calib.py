"""The calibration kernels that the measurements use (include/fa_calib.h)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_copy_kernel_copies_every_byte(fa):
    for nbytes in (16, 4096 + 48, 3 << 20):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
        dst = torch.zeros_like(src)
        fa.fa_calib_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), nbytes


def test_mfma_kernels_run(fa):
    """Each thread's sum is the same closed form in every workgroup (same operands)."""
    for kind in ("bf16", "fp8"):
        out, flop = fa.fa_calib_mfma(kind, 8, 3)
        torch.cuda.synchronize()
        assert flop == 8 * 4 * 3 * 4 * fa.CALIB_MFMA_FLOP[kind]
        per_wg = out.view(8, 256)
        assert torch.isfinite(out).all() and (out != 0).any(), kind
        assert torch.equal(per_wg, per_wg[:1].expand(8, 256)), kind


def test_calib_arguments_rejected(fa):
    x = torch.zeros(32, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError):
        fa.fa_calib_copy(x[:20], torch.zeros(20, dtype=torch.uint8, device="cuda"))  # not a multiple of 16
    with pytest.raises(fa.FAError):
        fa.fa_calib_mfma("bf16", 0, 1)


def test_read_kernel_reads_every_byte(fa):
    """The XOR of the per-thread XORs is the XOR of every 32-bit word of the input."""
    for nbytes in (16, 4096 + 48, 3 << 20):
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
        out = fa.fa_calib_read(src)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
        grid = min(-(-nbytes // 16384), 16384)
        got = np.bitwise_xor.reduce(out[: grid * 256].cpu().numpy().view(np.uint32))
        assert got == want, nbytes
