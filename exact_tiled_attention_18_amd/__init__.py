"""Exact tiled attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C-ABI library ``libfa.so`` (declared in
``include/fa.h``).  The functions keep the C names and only marshal
arguments: torch tensors supply device pointers, ``torch.cuda.current_stream()``
supplies the stream, and output tensors are allocated here when the caller
does not pass them.  Every step of the computation runs in the library's
HIP kernels; there is no fallback -- if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
# debug build: the bf16 forward's loop in its serial form (one tile at a time, one LDS
# slot, full barriers); it must agree with libfa.so bit for bit
SERIAL_LIB_PATH = os.path.join(_HERE, "libfa_serial.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_SCALE, FA_ERR_ALIAS, FA_ERR_HIP, FA_ERR_SCRATCH = range(8)
FA_BWD_NOALLOC_MAX_ROWS = 1 << 22  # rows (B * H * N) of fa_bwd_noalloc's static workspace
FA_F32, FA_BF16 = 0, 1
TILE_ROWS = 128  # rows per fp8 quantisation tile


def vt_cols(n: int) -> int:
    """Row length of transposed V codes: n rounded up to a multiple of 64 (FA_FP8_VT_COLS)."""
    return (n + 63) // 64 * 64

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"fa status {status}: {fa_status_string(status)}")


def load_library():
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_serial_library():
    """Load the debug build libfa_serial.so (same C-ABI; raises if it has not been built)."""
    return _open(SERIAL_LIB_PATH)


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.fa_abi_version.restype = i32
    lib.fa_abi_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i32]
    lib.fa_fwd.restype = i32
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.fa_quant_rotate_fp8.restype = i32
    lib.fa_quant_rotate_fp8.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.fa_quant_rotate_fp8_qkv.restype = i32
    lib.fa_quant_rotate_fp8_qkv.argtypes = [vp] * 10 + [i64, i64, i64, i64, vp]
    lib.fa_quant_rotate_fp8_tensor.restype = i32
    lib.fa_quant_rotate_fp8_tensor.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i32, f32, vp]
    lib.fa_fwd_fp8_pbf16.restype = i32
    lib.fa_fwd_fp8_pbf16.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i64, i64, i32, f32, vp]
    lib.fa_fwd_partial.restype = i32
    lib.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.fa_fwd_split.restype = i32
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, i32, f32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd.argtypes = [vp] * 10 + [i64, i64, i64, i64, i32, f32, i32, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, i32, f32, i32, vp]
    lib.fa_merge.restype = i32
    lib.fa_merge.argtypes = [vp, vp, i64, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.fa_calib_mfma.restype = i32
    lib.fa_calib_mfma.argtypes = [i32, i64, i64, vp, vp]
    lib.fa_calib_copy.restype = i32
    lib.fa_calib_copy.argtypes = [vp, vp, i64, vp]
    lib.fa_calib_read.restype = i32
    lib.fa_calib_read.argtypes = [vp, i64, vp, vp]
    return lib


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int):
    if status != FA_OK:
        raise FAError(status)


def _check_dense(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _expect(t, shape, dtype, name):
    """The library trusts the sizes it is given: every buffer must have exactly this shape."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def fa_fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None, stream=None):
    """O, LSE = attention(q, k, v) for [B, H, N, d] float32 or bfloat16 tensors."""
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    dtype = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(q.dtype, -1)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_dense(q, k, v, o, lse)
    for t, name in ((k, "k"), (v, "v"), (o, "o")):
        _expect(t, q.shape, q.dtype, name)
    _expect(lse, (B, H, N), torch.float32, "lse")
    lib = load_library()
    _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(causal),
                      float(scale), dtype, _stream(stream)))
    return o, lse


def fa_quant_rotate_fp8(x, signs=None, transpose_out: bool = False, x8=None, x_scale=None, stream=None,
                        per_tensor: bool = False):
    """e4m3 codes (uint8) and per-128-row-tile scales of x (bfloat16 [B, H, N, d]); with
    per_tensor, one scale for the whole tensor, repeated in every tile entry
    (fa_quant_rotate_fp8_tensor)."""
    B, H, N, d = x.shape
    x8_shape = (B, H, d, vt_cols(N)) if transpose_out else (B, H, N, d)
    if x8 is None:
        x8 = torch.empty(x8_shape, dtype=torch.uint8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((B, H, (N + TILE_ROWS - 1) // TILE_ROWS), dtype=torch.float32, device=x.device)
    _check_dense(x, signs, x8, x_scale)
    _expect(x, (B, H, N, d), torch.bfloat16, "x")
    _expect(x8, x8_shape, torch.uint8, "x8")
    _expect(x_scale, (B, H, (N + TILE_ROWS - 1) // TILE_ROWS), torch.float32, "x_scale")
    if signs is not None:
        _expect(signs, (d,), torch.int8, "signs")
    lib = load_library()
    fn = lib.fa_quant_rotate_fp8_tensor if per_tensor else lib.fa_quant_rotate_fp8
    _check(fn(_ptr(x), _ptr(x8), _ptr(x_scale), _ptr(signs), B, H, N, d, int(transpose_out), _stream(stream)))
    return x8, x_scale


def fa_quant_rotate_fp8_qkv(q, k, v, signs=None, out=None, stream=None):
    """The FP8 pre-pass of q, k, v (bfloat16 [B, H, N, d]) in one launch: returns
    (q8, k8, v8t, q_scale, k_scale, v_scale) as three fa_quant_rotate_fp8 calls would
    (Q and K with signs, V transposed); `out` may supply those six buffers."""
    B, H, N, d = q.shape
    nt = (N + TILE_ROWS - 1) // TILE_ROWS
    if out is None:
        q8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device)
        out = (q8, torch.empty_like(q8), torch.empty((B, H, d, vt_cols(N)), dtype=torch.uint8, device=q.device),
               *(torch.empty((B, H, nt), dtype=torch.float32, device=q.device) for _ in range(3)))
    q8, k8, v8t, qs, ks, vs = out
    _check_dense(q, k, v, signs, *out)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, (B, H, N, d), torch.bfloat16, name)
    _expect(q8, (B, H, N, d), torch.uint8, "q8")
    _expect(k8, (B, H, N, d), torch.uint8, "k8")
    _expect(v8t, (B, H, d, vt_cols(N)), torch.uint8, "v8t")
    for t, name in ((qs, "q_scale"), (ks, "k_scale"), (vs, "v_scale")):
        _expect(t, (B, H, nt), torch.float32, name)
    if signs is not None:
        _expect(signs, (d,), torch.int8, "signs")
    lib = load_library()
    _check(lib.fa_quant_rotate_fp8_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(qs), _ptr(ks),
                                       _ptr(vs), _ptr(signs), B, H, N, d, _stream(stream)))
    return out


def fa_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None,
               o=None, lse=None, stream=None, p_bf16: bool = False):
    """O (bfloat16), LSE from e4m3 Q, K ([B, H, N, d]) and transposed V ([B, H, d, vt_cols(N)]);
    with p_bf16, the probabilities stay in bf16 for P V (fa_fwd_fp8_pbf16)."""
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_dense(q8, k8, v8t, q_scale, k_scale, v_scale, o, lse)
    _expect(q8, q8.shape, torch.uint8, "q8")
    _expect(k8, q8.shape, torch.uint8, "k8")
    _expect(v8t, (B, H, d, vt_cols(N)), torch.uint8, "v8t")
    nt = (N + TILE_ROWS - 1) // TILE_ROWS
    for t, name in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _expect(t, (B, H, nt), torch.float32, name)
    _expect(o, (B, H, N, d), torch.bfloat16, "o")
    _expect(lse, (B, H, N), torch.float32, "lse")
    lib = load_library()
    fn = lib.fa_fwd_fp8_pbf16 if p_bf16 else lib.fa_fwd_fp8
    _check(fn(_ptr(q8), _ptr(k8), _ptr(v8t), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), 1, _ptr(o), _ptr(lse),
              B, H, N, d, int(causal), float(scale), _stream(stream)))
    return o, lse


def fp8_attention(q, k, v, signs, causal: bool = False, scale: float | None = None, stream=None,
                  per_tensor: bool = False, p_bf16: bool = False):
    """The FP8 path end to end: the pre-pass (Q and K rotated with the same signs, V
    not rotated and written transposed; one fused launch) and the fp8 forward.
    per_tensor and p_bf16 select the ablation variants (one scale per tensor, three
    pre-pass calls; probabilities in bf16).  Returns (o, lse, (q8, k8, v8t, q_scale,
    k_scale, v_scale))."""
    if per_tensor:
        q8, qs = fa_quant_rotate_fp8(q, signs, False, stream=stream, per_tensor=True)
        k8, ks = fa_quant_rotate_fp8(k, signs, False, stream=stream, per_tensor=True)
        v8t, vs = fa_quant_rotate_fp8(v, None, True, stream=stream, per_tensor=True)
    else:
        q8, k8, v8t, qs, ks, vs = fa_quant_rotate_fp8_qkv(q, k, v, signs, stream=stream)
    o, lse = fa_fwd_fp8(q8, k8, v8t, qs, ks, vs, causal, scale, stream=stream, p_bf16=p_bf16)
    return o, lse, (q8, k8, v8t, qs, ks, vs)


def fa_fwd_partial(q, k, v, q_pos0: int, k_begin: int, k_end: int, causal: bool = False,
                   scale: float | None = None, o_part=None, lse_part=None, stream=None):
    """O (float32, normalised over the range) and LSE of bfloat16 queries q [B, H, Nq, d]
    (query i at key position q_pos0 + i) against keys k_begin <= j < k_end of k, v [B, H, Nk, d]."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / d ** 0.5
    if o_part is None:
        o_part = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_dense(q, k, v, o_part, lse_part)
    _expect(q, (B, H, Nq, d), torch.bfloat16, "q")
    _expect(k, (B, H, Nk, d), torch.bfloat16, "k")
    _expect(v, (B, H, Nk, d), torch.bfloat16, "v")
    _expect(o_part, (B, H, Nq, d), torch.float32, "o_part")
    _expect(lse_part, (B, H, Nq), torch.float32, "lse_part")
    lib = load_library()
    _check(lib.fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, H, Nq, Nk, d,
                              int(q_pos0), int(k_begin), int(k_end), int(causal), float(scale), FA_BF16,
                              _stream(stream)))
    return o_part, lse_part


def fa_fwd_split(q, k, v, n_splits: int, q_pos0: int, k_begin: int, k_end: int, causal: bool = False,
                 scale: float | None = None, o_parts=None, lse_parts=None, stream=None):
    """fa_fwd_partial over n_splits consecutive ranges of [k_begin, k_end) in one launch:
    float32 o_parts [n_splits, B, H, Nq, d] and lse_parts [n_splits, B, H, Nq]; range s is
    [k_begin + (k_end - k_begin) * s // n_splits, k_begin + (k_end - k_begin) * (s + 1) // n_splits)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / d ** 0.5
    if o_parts is None:
        o_parts = torch.empty((n_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((n_splits, B, H, Nq), dtype=torch.float32, device=q.device)
    _check_dense(q, k, v, o_parts, lse_parts)
    _expect(q, (B, H, Nq, d), torch.bfloat16, "q")
    _expect(k, (B, H, Nk, d), torch.bfloat16, "k")
    _expect(v, (B, H, Nk, d), torch.bfloat16, "v")
    _expect(o_parts, (n_splits, B, H, Nq, d), torch.float32, "o_parts")
    _expect(lse_parts, (n_splits, B, H, Nq), torch.float32, "lse_parts")
    lib = load_library()
    _check(lib.fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o_parts), _ptr(lse_parts), B, H, Nq, Nk, d,
                            int(q_pos0), int(k_begin), int(k_end), int(n_splits), int(causal), float(scale), FA_BF16,
                            _stream(stream)))
    return o_parts, lse_parts


def fa_merge(o_parts, lse_parts, dtype=torch.bfloat16, o=None, lse=None, stream=None):
    """O [B, H, N, d] (dtype) and LSE [B, H, N] over the union of the key ranges of
    o_parts (float32 [n, B, H, N, d]) and lse_parts (float32 [n, B, H, N])."""
    n, B, H, N, d = o_parts.shape
    code = {torch.float32: FA_F32, torch.bfloat16: FA_BF16}.get(dtype, -1)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    _check_dense(o_parts, lse_parts, o, lse)
    _expect(lse_parts, (n, B, H, N), torch.float32, "lse_parts")
    _expect(o_parts, (n, B, H, N, d), torch.float32, "o_parts")
    _expect(o, (B, H, N, d), dtype, "o")
    _expect(lse, (B, H, N), torch.float32, "lse")
    lib = load_library()
    _check(lib.fa_merge(_ptr(o_parts), _ptr(lse_parts), n, _ptr(o), _ptr(lse), B, H, N, d, code, _stream(stream)))
    return o, lse


def split_kv_attention(q, k, v, n_splits: int, causal: bool = False, scale: float | None = None,
                       q_pos0: int | None = None, stream=None):
    """Split-KV forward: the keys [0, Nk) cut into n_splits contiguous ranges, all
    computed by one fa_fwd_split launch, then fa_merge.  By default the queries are
    the last Nq positions of the key sequence (q_pos0 = Nk - Nq)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if q_pos0 is None:
        q_pos0 = Nk - Nq
    o_parts, lse_parts = fa_fwd_split(q, k, v, n_splits, q_pos0, 0, Nk, causal, scale, stream=stream)
    return fa_merge(o_parts, lse_parts, q.dtype, stream=stream)


def fa_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
           delta=None, stream=None):
    """dQ, dK, dV (bfloat16 [B, H, N, d]) for bfloat16 q, k, v, the forward's o and lse,
    and the output gradient dout.  delta (float32 [B, H, N]) is a workspace."""
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_dense(q, k, v, o, dout, lse, dq, dk, dv, delta)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, (B, H, N, d), torch.bfloat16, name)
    _expect(lse, (B, H, N), torch.float32, "lse")
    _expect(delta, (B, H, N), torch.float32, "delta")
    lib = load_library()
    _check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      _ptr(delta), B, H, N, d, int(causal), float(scale), FA_BF16, _stream(stream)))
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, dq=None, dk=None,
                   dv=None, stream=None):
    """fa_bwd with the library's static workspace instead of a delta argument (the C call
    allocates nothing; outputs are allocated here unless passed).  Calls that overlap on
    one GPU share that workspace and race."""
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_dense(q, k, v, o, dout, lse, dq, dk, dv)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, (B, H, N, d), torch.bfloat16, name)
    _expect(lse, (B, H, N), torch.float32, "lse")
    lib = load_library()
    _check(lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, H, N, d, int(causal), float(scale), FA_BF16, _stream(stream)))
    return dq, dk, dv


# ---- calibration kernels (include/fa_calib.h): not part of the method; they measure
# what the chip sustains for the resources the attention kernels are priced against

CALIB_MFMA_FLOP = {"bf16": 32768, "fp8": 131072}  # per instruction


def fa_calib_mfma(kind: str, workgroups: int, iters: int, out=None, stream=None):
    """Launches the MFMA-only kernel (kind "bf16" or "fp8"); returns (out, FLOP per launch)."""
    code = {"bf16": 0, "fp8": 1}[kind]
    if out is None:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    _expect(out, (workgroups * 256,), torch.float32, "out")
    _check(load_library().fa_calib_mfma(code, workgroups, iters, _ptr(out), _stream(stream)))
    return out, workgroups * 4 * iters * 4 * CALIB_MFMA_FLOP[kind]


def fa_calib_copy(src, dst, stream=None):
    """dst[:] = src[:] (contiguous device tensors of the same byte size, a multiple of 16)."""
    _check_dense(src, dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check(load_library().fa_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
    return dst


CALIB_READ_OUT_WORDS = 16384 * 256


def fa_calib_read(src, out=None, stream=None):
    """Reads every byte of src (a contiguous device tensor, size a multiple of 16) once;
    out (int32 [CALIB_READ_OUT_WORDS]) receives per-thread XORs."""
    if out is None:
        out = torch.empty(CALIB_READ_OUT_WORDS, dtype=torch.int32, device=src.device)
    _check_dense(src, out)
    _expect(out, (CALIB_READ_OUT_WORDS,), torch.int32, "out")
    _check(load_library().fa_calib_read(_ptr(src), src.numel() * src.element_size(), _ptr(out), _stream(stream)))
    return out
