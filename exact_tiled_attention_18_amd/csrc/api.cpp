// C-ABI entry points: argument validation, then one enqueue per kernel.
// Validation never touches the GPU, so a rejected call has no side effect.
// Plain host C++: every GPU action goes through the launchers of launch.h, so
// this file also builds with a host compiler against a recording stand-in for
// them (the sanitizer build of the validation code).
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "launch.h"

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Element count B*H*N*d without int64 overflow; also bounds the kernels'
// 32-bit row indices and the size of a single launch.
int shape_status(int64_t B, int64_t H, int64_t N, int64_t d, int64_t* count) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
  int64_t bh, bhn, n;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &bhn) || !mul_ok(bhn, d, &n)) return FA_ERR_SHAPE;
  // per-head byte offsets are 32-bit in the kernels: N * d * 4 (fp32) must fit
  if (d > 0 && N > INT32_MAX / (4 * d)) return FA_ERR_SHAPE;
  // one launch: at most 2^32 work-items; the finest grid is the fp32 kernel's, one
  // workgroup of up to 512 threads per 16 queries
  if (bh > 0 && (N + 15) / 16 > (int64_t(1) << 23) / bh) return FA_ERR_SHAPE;
  *count = n;
  return FA_OK;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape";
    case FA_ERR_UNSUPPORTED: return "unsupported argument";
    case FA_ERR_SCALE: return "non-finite scale";
    case FA_ERR_ALIAS: return "output overlaps input";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_SCRATCH: return "problem exceeds the library's static scratch";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
           int64_t N, int64_t d, int causal, float scale, int dtype, void* stream) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (n == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t tb = n * (dtype == FA_F32 ? 4 : 2), lb = B * H * N * 4;
  for (const void* in : {q, k, v})
    if (overlaps(o, tb, in, tb) || overlaps(lse, lb, in, tb)) return FA_ERR_ALIAS;
  if (overlaps(o, tb, lse, lb)) return FA_ERR_ALIAS;

  const fa::AttnArgs a{q, k, v, o, lse, B, H, N, d, causal, scale, static_cast<hipStream_t>(stream)};
  return hip_status(dtype == FA_F32 ? fa::launch_attn_f32(a) : fa::launch_attn_bf16(a));
}

}  // extern "C"

namespace {
int quant_rotate(const void* x, uint8_t* x8, float* x_scale, const int8_t* signs, int64_t B, int64_t H, int64_t N,
                 int64_t d, int transpose_out, void* stream, int per_tensor) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (transpose_out != 0 && transpose_out != 1) return FA_ERR_UNSUPPORTED;
  if (n == 0) return FA_OK;
  if (!x || !x8 || !x_scale) return FA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(x_scale, 4)) return FA_ERR_UNSUPPORTED;
  const int64_t sb = B * H * ((N + 127) / 128) * 4;
  const int64_t xb = transpose_out ? B * H * d * FA_FP8_VT_COLS(N) : n;  // bytes of x8
  if (overlaps(x8, xb, x, 2 * n) || overlaps(x_scale, sb, x, 2 * n) || overlaps(x8, xb, x_scale, sb))
    return FA_ERR_ALIAS;
  if (signs && (overlaps(x8, xb, signs, d) || overlaps(x_scale, sb, signs, d))) return FA_ERR_ALIAS;

  const fa::QuantArgs a{x, x8, x_scale, signs, B, H, N, d, transpose_out, static_cast<hipStream_t>(stream),
                        per_tensor};
  return hip_status(fa::launch_quant_rotate_fp8(a));
}
}  // namespace

extern "C" {

int fa_quant_rotate_fp8(const void* x, uint8_t* x8, float* x_scale, const int8_t* signs, int64_t B,
                        int64_t H, int64_t N, int64_t d, int transpose_out, void* stream) {
  return quant_rotate(x, x8, x_scale, signs, B, H, N, d, transpose_out, stream, 0);
}

int fa_quant_rotate_fp8_tensor(const void* x, uint8_t* x8, float* x_scale, const int8_t* signs, int64_t B,
                               int64_t H, int64_t N, int64_t d, int transpose_out, void* stream) {
  return quant_rotate(x, x8, x_scale, signs, B, H, N, d, transpose_out, stream, 1);
}

int fa_quant_rotate_fp8_qkv(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                            float* q_scale, float* k_scale, float* v_scale, const int8_t* signs, int64_t B,
                            int64_t H, int64_t N, int64_t d, void* stream) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (n == 0) return FA_OK;
  const void* in[3] = {q, k, v};
  uint8_t* out[3] = {q8, k8, v8t};
  float* sc[3] = {q_scale, k_scale, v_scale};
  for (int i = 0; i < 3; ++i) {
    if (!in[i] || !out[i] || !sc[i]) return FA_ERR_NULL;
    if (!aligned(in[i], 16) || !aligned(out[i], 16) || !aligned(sc[i], 4)) return FA_ERR_UNSUPPORTED;
  }
  const int64_t sb = B * H * ((N + 127) / 128) * 4;
  const int64_t ob[3] = {n, n, B * H * d * FA_FP8_VT_COLS(N)};
  // no output may overlap an input, the signs or another output
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(out[i], ob[i], in[j], 2 * n) || overlaps(sc[i], sb, in[j], 2 * n)) return FA_ERR_ALIAS;
    if (signs && (overlaps(out[i], ob[i], signs, d) || overlaps(sc[i], sb, signs, d))) return FA_ERR_ALIAS;
    for (int j = 0; j < 3; ++j) {
      if (overlaps(out[i], ob[i], sc[j], sb)) return FA_ERR_ALIAS;
      if (j != i && (overlaps(out[i], ob[i], out[j], ob[j]) || overlaps(sc[i], sb, sc[j], sb))) return FA_ERR_ALIAS;
    }
  }
  const fa::QkvQuantArgs a{{q, k, v}, {q8, k8, v8t}, {q_scale, k_scale, v_scale}, signs, B, H, N, d,
                           static_cast<hipStream_t>(stream)};
  return hip_status(fa::launch_quant_qkv_fp8(a));
}

}  // extern "C"

namespace {
int fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale, const float* k_scale,
            const float* v_scale, int v_transposed, void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
            int causal, float scale, void* stream, int p_bf16) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (d != 128 || v_transposed != 1) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (n == 0) return FA_OK;
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t ob = 2 * n, lb = B * H * N * 4, sb = B * H * ((N + 127) / 128) * 4;
  const void* ins[] = {q8, k8, v8};
  const int64_t inb[] = {n, n, B * H * d * FA_FP8_VT_COLS(N)};
  const void* scs[] = {q_scale, k_scale, v_scale};
  for (int i = 0; i < 3; ++i)
    if (overlaps(o, ob, ins[i], inb[i]) || overlaps(lse, lb, ins[i], inb[i]) || overlaps(o, ob, scs[i], sb) ||
        overlaps(lse, lb, scs[i], sb))
      return FA_ERR_ALIAS;
  if (overlaps(o, ob, lse, lb)) return FA_ERR_ALIAS;

  const fa::Fp8AttnArgs a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, causal, scale,
                          static_cast<hipStream_t>(stream), p_bf16};
  return hip_status(fa::launch_attn_fp8(a));
}
}  // namespace

extern "C" {

int fa_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, int v_transposed, void* o, float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale, void* stream) {
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, v_transposed, o, lse, B, H, N, d, causal, scale, stream, 0);
}

int fa_fwd_fp8_pbf16(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                     const float* k_scale, const float* v_scale, int v_transposed, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale, void* stream) {
  return fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, v_transposed, o, lse, B, H, N, d, causal, scale, stream, 1);
}

int fa_fwd_split(const void* q, const void* k, const void* v, float* o_parts, float* lse_parts, int64_t B,
                 int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t q_pos0, int64_t k_begin, int64_t k_end,
                 int64_t n_splits, int causal, float scale, int dtype, void* stream) {
  int64_t nq = 0, nk = 0, tot = 0;
  if (int st = shape_status(B, H, Nq, d, &nq)) return st;
  if (int st = shape_status(B, H, Nk, d, &nk)) return st;
  if (k_begin < 0 || k_end < k_begin || k_end > Nk) return FA_ERR_SHAPE;
  if (n_splits < 1 || n_splits > 65535 || !mul_ok(nq, n_splits, &tot)) return FA_ERR_SHAPE;
  // relative positions (q_pos0 + i - k_begin) must fit the kernels' 32-bit arithmetic
  if (q_pos0 < 0 || q_pos0 > INT32_MAX / 2 - Nq) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (nq == 0) return FA_OK;
  if (!q || !k || !v || !o_parts || !lse_parts) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_parts, 16) || !aligned(lse_parts, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t qb = 2 * nq, kb = 2 * nk, ob = 4 * tot, lb = B * H * Nq * 4 * n_splits;
  if (overlaps(o_parts, ob, q, qb) || overlaps(o_parts, ob, k, kb) || overlaps(o_parts, ob, v, kb) ||
      overlaps(lse_parts, lb, q, qb) || overlaps(lse_parts, lb, k, kb) || overlaps(lse_parts, lb, v, kb) ||
      overlaps(o_parts, ob, lse_parts, lb))
    return FA_ERR_ALIAS;
  const fa::AttnArgs a{q, k, v, o_parts, lse_parts, B, H, Nq, d, causal, scale, static_cast<hipStream_t>(stream)};
  const fa::PartialArgs p{Nk, q_pos0, k_begin, k_end, n_splits};
  return hip_status(fa::launch_attn_bf16_partial(a, p));
}

int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int64_t B,
                   int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t q_pos0, int64_t k_begin, int64_t k_end,
                   int causal, float scale, int dtype, void* stream) {
  return fa_fwd_split(q, k, v, o_part, lse_part, B, H, Nq, Nk, d, q_pos0, k_begin, k_end, 1, causal, scale, dtype,
                      stream);
}

int fa_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse, int64_t B,
             int64_t H, int64_t N, int64_t d, int dtype, void* stream) {
  int64_t n = 0, tot = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (n_parts < 1 || !mul_ok(n, n_parts, &tot) || n_parts > INT32_MAX) return FA_ERR_SHAPE;
  if (B * H * N > (int64_t(INT32_MAX) - 3) * 4) return FA_ERR_SHAPE;  // one wavefront per row, 4 per block
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (n == 0) return FA_OK;
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (!aligned(o_parts, 8) || !aligned(lse_parts, 4) || !aligned(o, 4) || !aligned(lse, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t pb = 4 * tot, plb = 4 * B * H * N * n_parts, ob = (dtype == FA_F32 ? 4 : 2) * n,
                lb = 4 * B * H * N;
  if (overlaps(o, ob, o_parts, pb) || overlaps(o, ob, lse_parts, plb) || overlaps(lse, lb, o_parts, pb) ||
      overlaps(lse, lb, lse_parts, plb) || overlaps(o, ob, lse, lb))
    return FA_ERR_ALIAS;
  const fa::MergeArgs a{o_parts, lse_parts, n_parts, o, lse, B, H, N, d, dtype, static_cast<hipStream_t>(stream)};
  return hip_status(fa::launch_merge(a));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
           float scale, int dtype, void* stream) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (n == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  const void* in16[] = {q, k, v, o, dout};
  for (const void* p : in16)
    if (!aligned(p, 16)) return FA_ERR_UNSUPPORTED;
  if (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t tb = 2 * n, rb = 4 * B * H * N;
  void* outs[] = {dq, dk, dv};
  for (void* out : outs) {
    for (const void* in : in16)
      if (overlaps(out, tb, in, tb)) return FA_ERR_ALIAS;
    if (overlaps(out, tb, lse, rb) || overlaps(out, tb, delta, rb)) return FA_ERR_ALIAS;
  }
  if (overlaps(dq, tb, dk, tb) || overlaps(dq, tb, dv, tb) || overlaps(dk, tb, dv, tb)) return FA_ERR_ALIAS;
  for (const void* in : in16)
    if (overlaps(delta, rb, in, tb)) return FA_ERR_ALIAS;
  if (overlaps(delta, rb, lse, rb)) return FA_ERR_ALIAS;
  const fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale,
                      static_cast<hipStream_t>(stream)};
  return hip_status(fa::launch_attn_bwd(a));
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                   int causal, float scale, int dtype, void* stream) {
  int64_t n = 0;
  if (int st = shape_status(B, H, N, d, &n)) return st;
  if (B * H * N > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  // the argument checks that need no workspace, before the device is touched
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (n == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  void* ws = nullptr;
  if (fa::scratch_address(&ws) != hipSuccess || !ws) return FA_ERR_HIP;
  // the workspace is library memory, so it overlaps none of the caller's buffers
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(ws), B, H, N, d, causal, scale, dtype,
                stream);
}

}  // extern "C"
