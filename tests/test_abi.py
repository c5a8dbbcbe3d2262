"""CPU checks of the C-ABI library: it loads, exports every function fa.h
declares, and rejects invalid arguments with the documented status before
any GPU work (these calls return from validation; none reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def fa():
    import exact_tiled_attention_18_amd as fa
    if not os.path.exists(fa.LIB_PATH):
        from exact_tiled_attention_18_amd import _build
        _build.build(verbose=False)
    fa.load_library()
    return fa


def test_header_declares_the_api():
    assert _declared_functions() == ["fa_abi_version", "fa_bwd", "fa_bwd_noalloc", "fa_fwd", "fa_fwd_fp8",
                                     "fa_fwd_fp8_pbf16", "fa_fwd_partial", "fa_fwd_split", "fa_merge",
                                     "fa_quant_rotate_fp8", "fa_quant_rotate_fp8_qkv", "fa_quant_rotate_fp8_tensor",
                                     "fa_status_string"]


def test_library_exports_every_declared_symbol(fa):
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(fa):
    assert fa.fa_abi_version() == 4
    assert fa.fa_status_string(0) == "ok"
    assert fa.fa_status_string(fa.FA_ERR_SCRATCH) == "problem exceeds the library's static scratch"
    assert fa.fa_status_string(3) == "unsupported argument"
    assert fa.fa_status_string(99) == "unknown status"


P = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
P2 = ctypes.c_void_p(0x20000000)
P3 = ctypes.c_void_p(0x40000000)
P4 = ctypes.c_void_p(0x60000000)
P5 = ctypes.c_void_p(0x70000000)


def _fwd(fa, q=P, k=P2, v=P3, o=P4, lse=P5, B=1, H=1, N=128, d=64, causal=0, scale=0.125, dtype=1):
    return fa.load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


def test_fwd_validation(fa):
    assert _fwd(fa, B=-1) == fa.FA_ERR_SHAPE
    assert _fwd(fa, N=-5) == fa.FA_ERR_SHAPE
    assert _fwd(fa, B=1 << 40, H=1 << 30) == fa.FA_ERR_SHAPE  # element count overflows int64
    # one head's fp32 bytes N * d * 4 must fit the kernels' 32-bit offsets
    assert _fwd(fa, N=(2 ** 31 - 1) // (4 * 64) + 1) == fa.FA_ERR_SHAPE
    # one launch holds at most 2^32 work-items: B*H*ceil(N/16) workgroups of up to 512 threads
    assert _fwd(fa, B=1 << 10, H=1 << 10, N=160) == fa.FA_ERR_SHAPE
    assert fa.vt_cols(1) == 64 and fa.vt_cols(64) == 64 and fa.vt_cols(65) == 128
    assert _fwd(fa, d=96) == fa.FA_ERR_UNSUPPORTED
    assert _fwd(fa, dtype=7) == fa.FA_ERR_UNSUPPORTED
    assert _fwd(fa, causal=2) == fa.FA_ERR_UNSUPPORTED
    assert _fwd(fa, scale=float("nan")) == fa.FA_ERR_SCALE
    assert _fwd(fa, scale=float("inf")) == fa.FA_ERR_SCALE
    assert _fwd(fa, q=None) == fa.FA_ERR_NULL
    assert _fwd(fa, lse=None) == fa.FA_ERR_NULL
    assert _fwd(fa, o=ctypes.c_void_p(0x10008)) == fa.FA_ERR_UNSUPPORTED  # misaligned
    assert _fwd(fa, o=ctypes.c_void_p(0x10000 + 64)) == fa.FA_ERR_ALIAS  # o overlaps q
    assert _fwd(fa, lse=ctypes.c_void_p(0x60000000 + 128)) == fa.FA_ERR_ALIAS  # lse inside o
    # empty problems succeed without launching anything (null pointers are fine then)
    assert _fwd(fa, q=None, k=None, v=None, o=None, lse=None, N=0) == fa.FA_OK
    assert _fwd(fa, q=None, k=None, v=None, o=None, lse=None, B=0) == fa.FA_OK


@pytest.mark.parametrize("entry", ["fa_quant_rotate_fp8", "fa_quant_rotate_fp8_tensor"])
def test_quant_validation(fa, entry):
    fn = getattr(fa.load_library(), entry)
    f = lambda x=P, x8=P2, s=P3, sg=None, B=1, H=1, N=128, d=128, t=0: fn(x, x8, s, sg, B, H, N, d, t, None)
    assert f(d=32) == fa.FA_ERR_UNSUPPORTED
    assert f(t=2) == fa.FA_ERR_UNSUPPORTED
    assert f(x=None) == fa.FA_ERR_NULL
    assert f(N=-1) == fa.FA_ERR_SHAPE
    assert f(x8=ctypes.c_void_p(0x10000 + 32)) == fa.FA_ERR_ALIAS
    assert f(x=None, x8=None, s=None, N=0) == fa.FA_OK


@pytest.mark.parametrize("entry", ["fa_fwd_fp8", "fa_fwd_fp8_pbf16"])
def test_fp8_validation(fa, entry):
    fn = getattr(fa.load_library(), entry)
    f = lambda vt=1, d=128, causal=0, scale=0.1, q=P, o=P4: fn(
        q, P2, P3, ctypes.c_void_p(0x50000000), ctypes.c_void_p(0x50001000), ctypes.c_void_p(0x50002000), vt,
        o, P5, 1, 1, 256, d, causal, scale, None)
    assert f(vt=0) == fa.FA_ERR_UNSUPPORTED
    assert f(d=64) == fa.FA_ERR_UNSUPPORTED
    assert f(causal=3) == fa.FA_ERR_UNSUPPORTED
    assert f(scale=float("-inf")) == fa.FA_ERR_SCALE
    assert f(q=None) == fa.FA_ERR_NULL
    assert f(o=ctypes.c_void_p(0x20000000 + 16)) == fa.FA_ERR_ALIAS


def test_product_path_has_no_cpu_fallback():
    """The package must not import the oracle or any CPU attention path."""
    pkg = os.path.join(ROOT, "exact_tiled_attention_18_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle_", ""), fn
            assert "scaled_dot_product_attention" not in src and "softmax" not in src, fn


def _partial(fa, q=P, k=P2, v=P3, o=P4, lse=P5, B=1, H=1, Nq=64, Nk=128, d=64, pos0=0, kb=0, ke=128, causal=1,
             scale=0.125, dtype=1):
    return fa.load_library().fa_fwd_partial(q, k, v, o, lse, B, H, Nq, Nk, d, pos0, kb, ke, causal, scale, dtype,
                                            None)


def test_partial_validation(fa):
    assert _partial(fa, kb=-1) == fa.FA_ERR_SHAPE
    assert _partial(fa, kb=50, ke=40) == fa.FA_ERR_SHAPE       # reversed range
    assert _partial(fa, ke=129) == fa.FA_ERR_SHAPE             # past the keys
    assert _partial(fa, pos0=-1) == fa.FA_ERR_SHAPE
    assert _partial(fa, pos0=2 ** 30) == fa.FA_ERR_SHAPE       # positions beyond 32-bit arithmetic
    assert _partial(fa, dtype=0) == fa.FA_ERR_UNSUPPORTED      # bf16 only
    assert _partial(fa, d=96) == fa.FA_ERR_UNSUPPORTED
    assert _partial(fa, causal=3) == fa.FA_ERR_UNSUPPORTED
    assert _partial(fa, scale=float("nan")) == fa.FA_ERR_SCALE
    assert _partial(fa, o=None) == fa.FA_ERR_NULL
    assert _partial(fa, o=ctypes.c_void_p(0x10000 + 32)) == fa.FA_ERR_ALIAS  # o_part overlaps q
    assert _partial(fa, q=None, k=None, v=None, o=None, lse=None, Nq=0) == fa.FA_OK


def _split(fa, q=P, k=P2, v=P3, o=P4, lse=P5, B=1, H=1, Nq=64, Nk=128, d=64, pos0=0, kb=0, ke=128, n=4, causal=1,
           scale=0.125, dtype=1):
    return fa.load_library().fa_fwd_split(q, k, v, o, lse, B, H, Nq, Nk, d, pos0, kb, ke, n, causal, scale, dtype,
                                          None)


def test_split_validation(fa):
    assert _split(fa, n=0) == fa.FA_ERR_SHAPE
    assert _split(fa, n=65536) == fa.FA_ERR_SHAPE              # one grid row per range
    assert _split(fa, kb=50, ke=40) == fa.FA_ERR_SHAPE
    assert _split(fa, pos0=2 ** 30) == fa.FA_ERR_SHAPE
    assert _split(fa, dtype=0) == fa.FA_ERR_UNSUPPORTED
    assert _split(fa, d=96) == fa.FA_ERR_UNSUPPORTED
    assert _split(fa, scale=float("inf")) == fa.FA_ERR_SCALE
    assert _split(fa, lse=None) == fa.FA_ERR_NULL
    # the n slices of o_parts reach past q's start: overlap detected over all of them
    assert _split(fa, o=ctypes.c_void_p(0x10000 - 3 * 64 * 64 * 4)) == fa.FA_ERR_ALIAS
    assert _split(fa, q=None, k=None, v=None, o=None, lse=None, Nq=0) == fa.FA_OK


def _merge(fa, op=P, lp=P2, n=3, o=P3, lse=P4, B=1, H=1, N=64, d=64, dtype=1):
    return fa.load_library().fa_merge(op, lp, n, o, lse, B, H, N, d, dtype, None)


def test_merge_validation(fa):
    assert _merge(fa, n=0) == fa.FA_ERR_SHAPE
    assert _merge(fa, N=-1) == fa.FA_ERR_SHAPE
    assert _merge(fa, d=32) == fa.FA_ERR_UNSUPPORTED
    assert _merge(fa, dtype=5) == fa.FA_ERR_UNSUPPORTED
    assert _merge(fa, op=None) == fa.FA_ERR_NULL
    assert _merge(fa, o=ctypes.c_void_p(0x10000 + 64)) == fa.FA_ERR_ALIAS  # o inside o_parts
    assert _merge(fa, op=None, lp=None, o=None, lse=None, N=0) == fa.FA_OK


def _bwd(fa, q=P, k=P2, v=P3, o=P4, do=P5, lse=ctypes.c_void_p(0x7A000000), dq=ctypes.c_void_p(0x7C000000),
         dk=ctypes.c_void_p(0x7E000000), dv=ctypes.c_void_p(0x80000000), delta=ctypes.c_void_p(0x82000000),
         B=1, H=1, N=128, d=64, causal=1, scale=0.125, dtype=1):
    return fa.load_library().fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, dtype, None)


def test_bwd_validation(fa):
    assert _bwd(fa, N=-1) == fa.FA_ERR_SHAPE
    assert _bwd(fa, d=32) == fa.FA_ERR_UNSUPPORTED
    assert _bwd(fa, dtype=0) == fa.FA_ERR_UNSUPPORTED
    assert _bwd(fa, causal=2) == fa.FA_ERR_UNSUPPORTED
    assert _bwd(fa, scale=float("inf")) == fa.FA_ERR_SCALE
    assert _bwd(fa, delta=None) == fa.FA_ERR_NULL
    assert _bwd(fa, dq=ctypes.c_void_p(0x10000 + 64)) == fa.FA_ERR_ALIAS  # dq overlaps q
    assert _bwd(fa, dk=ctypes.c_void_p(0x7C000000 + 32)) == fa.FA_ERR_ALIAS  # dk overlaps dq
    assert _bwd(fa, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None, delta=None,
                N=0) == fa.FA_OK


def _bwd_noalloc(fa, q=P, k=P2, v=P3, o=P4, do=P5, lse=ctypes.c_void_p(0x7A000000), dq=ctypes.c_void_p(0x7C000000),
                 dk=ctypes.c_void_p(0x7E000000), dv=ctypes.c_void_p(0x80000000), B=1, H=1, N=128, d=64, causal=1,
                 scale=0.125, dtype=1):
    return fa.load_library().fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, None)


def test_bwd_noalloc_validation(fa):
    """Rejected before the device or any pointer is touched: a problem beyond the static
    workspace (even with null pointers), and every argument error fa_bwd reports."""
    rows = fa.FA_BWD_NOALLOC_MAX_ROWS
    none = dict(q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None)
    assert _bwd_noalloc(fa, B=1, H=1, N=rows + 1, **none) == fa.FA_ERR_SCRATCH
    assert _bwd_noalloc(fa, B=4, H=32, N=rows // 64, **none) == fa.FA_ERR_SCRATCH
    assert _bwd_noalloc(fa, N=-1) == fa.FA_ERR_SHAPE
    assert _bwd_noalloc(fa, d=32) == fa.FA_ERR_UNSUPPORTED
    assert _bwd_noalloc(fa, dtype=0) == fa.FA_ERR_UNSUPPORTED
    assert _bwd_noalloc(fa, causal=2) == fa.FA_ERR_UNSUPPORTED
    assert _bwd_noalloc(fa, scale=float("nan")) == fa.FA_ERR_SCALE
    assert _bwd_noalloc(fa, dv=None) == fa.FA_ERR_NULL
    assert _bwd_noalloc(fa, N=0, **none) == fa.FA_OK


def test_quant_qkv_validation(fa):
    lib = fa.load_library()
    A = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(9)]  # q, k, v, q8, k8, v8t, scales: disjoint

    def f(i=None, val=None, d=128, N=256, sg=None):
        args = list(A)
        if i is not None:
            args[i] = val
        return lib.fa_quant_rotate_fp8_qkv(*args, sg, 1, 2, N, d, None)
    assert f(d=32) == fa.FA_ERR_UNSUPPORTED
    assert f(N=-1) == fa.FA_ERR_SHAPE
    assert f(0, None) == fa.FA_ERR_NULL and f(8, None) == fa.FA_ERR_NULL
    assert f(4, ctypes.c_void_p(0x10000000 * 4 + 64)) == fa.FA_ERR_ALIAS   # k8 inside q8
    assert f(5, ctypes.c_void_p(0x10000000 * 2 + 32)) == fa.FA_ERR_ALIAS   # v8t inside k
    assert f(7, ctypes.c_void_p(0x10000000 * 7 + 8)) == fa.FA_ERR_ALIAS    # k_scale inside q_scale (16 bytes)
    assert f(3, ctypes.c_void_p(0x10000000 * 4 + 8)) == fa.FA_ERR_UNSUPPORTED  # misaligned q8
    assert lib.fa_quant_rotate_fp8_qkv(*([None] * 9), None, 1, 2, 0, 128, None) == fa.FA_OK

