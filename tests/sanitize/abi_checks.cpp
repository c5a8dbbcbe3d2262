// Host-side checks of the C-ABI's validation (api.cpp) against recording
// launchers (fake_launch.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every rejected call must return its documented
// status and launch nothing; every accepted call must reach exactly one
// launcher with the caller's sizes; a failing launch must come back as
// FA_ERR_HIP.  Host buffers stand in for device memory: the validation code
// compares and offsets pointers but never dereferences them.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "fa.h"
#include "fake_launch.h"

namespace {

int g_failures = 0, g_checks = 0;

void check(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::printf("FAIL line %d: %s\n", line, what);
  }
}
#define CHECK(cond) check((cond), #cond, __LINE__)

// a call that must be rejected with `want` and launch nothing
#define REJECT(want, call)                 \
  do {                                     \
    fake::launches = 0;                    \
    const int st_ = (call);                \
    check(st_ == (want), #call, __LINE__); \
    check(fake::launches == 0, "no launch: " #call, __LINE__); \
  } while (0)

// a call that must succeed with exactly one launch of `launcher`
#define ACCEPT(launcher, call)                                              \
  do {                                                                      \
    fake::launches = 0;                                                     \
    const int st_ = (call);                                                 \
    check(st_ == FA_OK, #call, __LINE__);                                   \
    check(fake::launches == 1 && std::strcmp(fake::last, launcher) == 0,    \
          "one launch of " launcher ": " #call, __LINE__);                  \
  } while (0)

// a call that must succeed without any launch (an empty problem)
#define NOOP(call)                                          \
  do {                                                      \
    fake::launches = 0;                                     \
    check((call) == FA_OK, #call, __LINE__);                \
    check(fake::launches == 0, "no launch: " #call, __LINE__); \
  } while (0)

// a call whose launch fails
#define LAUNCH_FAILS(call)                                    \
  do {                                                        \
    fake::next_status = hipErrorLaunchFailure;                \
    check((call) == FA_ERR_HIP, #call, __LINE__);             \
    fake::next_status = hipSuccess;                           \
  } while (0)

// 256-byte aligned host buffers, released at exit
struct Pool {
  std::vector<void*> held;
  char* get(size_t bytes) {
    void* p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
    held.push_back(p);
    return static_cast<char*>(p);
  }
  ~Pool() {
    for (void* p : held) std::free(p);
  }
};

const float kNaN = std::numeric_limits<float>::quiet_NaN();
const float kInfF = std::numeric_limits<float>::infinity();

void forward(Pool& pool) {
  const int64_t B = 2, H = 3, N = 100, d = 64;
  const size_t tb = B * H * N * d * 2, lb = B * H * N * 4;
  char *q = pool.get(tb), *k = pool.get(tb), *v = pool.get(tb), *o = pool.get(tb);
  float* lse = reinterpret_cast<float*>(pool.get(lb));
  const float sc = 0.125f;
  ACCEPT("attn_bf16", fa_fwd(q, k, v, o, lse, B, H, N, d, 1, sc, FA_BF16, nullptr));
  CHECK(fake::last_B == B && fake::last_H == H && fake::last_N == N && fake::last_d == d);
  char* o32 = pool.get(2 * tb);
  ACCEPT("attn_f32", fa_fwd(q, k, v, o32, lse, B, H, N, d, 0, sc, FA_F32, nullptr));
  char *q2 = pool.get(2 * tb), *k2 = pool.get(2 * tb), *v2 = pool.get(2 * tb), *o2 = pool.get(2 * tb);
  ACCEPT("attn_bf16", fa_fwd(q2, k2, v2, o2, lse, B, H, N, 128, 0, -0.5f, FA_BF16, nullptr));
  // d = 128 on buffers sized for d = 64: each output then reaches into the next buffer
  REJECT(FA_ERR_ALIAS, fa_fwd(q, k, v, o, lse, B, H, N, 128, 0, 0.5f, FA_BF16, nullptr));
  NOOP(fa_fwd(q, k, v, o, lse, B, H, 0, d, 1, sc, FA_BF16, nullptr));
  NOOP(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_NULL, fa_fwd(nullptr, k, v, o, lse, B, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_NULL, fa_fwd(q, k, v, o, nullptr, B, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd(q, k, v, o, lse, -1, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd(q, k, v, o, lse, B, H, INT64_MAX / 2, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd(q, k, v, o, lse, INT64_MAX, INT64_MAX, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd(q, k, v, o, lse, 1 << 20, 1 << 20, 1 << 20, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd(q, k, v, o, lse, B, H, N, 96, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd(q, k, v, o, lse, B, H, N, d, 1, sc, 7, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd(q, k, v, o, lse, B, H, N, d, 2, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd(q + 2, k, v, o, lse, B, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_SCALE, fa_fwd(q, k, v, o, lse, B, H, N, d, 1, kNaN, FA_BF16, nullptr));
  REJECT(FA_ERR_SCALE, fa_fwd(q, k, v, o, lse, B, H, N, d, 1, -kInfF, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd(q, k, v, q, lse, B, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd(q, k, v, o, reinterpret_cast<float*>(v + 64), B, H, N, d, 1, sc, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd(q, k, v, o, reinterpret_cast<float*>(o + 16), B, H, N, d, 1, sc, FA_BF16, nullptr));
  LAUNCH_FAILS(fa_fwd(q, k, v, o, lse, B, H, N, d, 1, sc, FA_BF16, nullptr));
}

void fp8(Pool& pool) {
  const int64_t B = 1, H = 2, N = 300, d = 128, nt = (N + 127) / 128;
  const size_t n = B * H * N * d, vt = B * H * d * FA_FP8_VT_COLS(N), sb = B * H * nt * 4;
  char *q = pool.get(2 * n), *k = pool.get(2 * n), *v = pool.get(2 * n);
  auto* q8 = reinterpret_cast<uint8_t*>(pool.get(n));
  auto* k8 = reinterpret_cast<uint8_t*>(pool.get(n));
  auto* v8 = reinterpret_cast<uint8_t*>(pool.get(vt));
  auto* qs = reinterpret_cast<float*>(pool.get(sb));
  auto* ks = reinterpret_cast<float*>(pool.get(sb));
  auto* vs = reinterpret_cast<float*>(pool.get(sb));
  auto* signs = reinterpret_cast<int8_t*>(pool.get(d));
  char* o = pool.get(2 * n);
  auto* lse = reinterpret_cast<float*>(pool.get(B * H * N * 4));
  // pre-pass, one tensor
  ACCEPT("quant_tile", fa_quant_rotate_fp8(q, q8, qs, signs, B, H, N, d, 0, nullptr));
  ACCEPT("quant_tile", fa_quant_rotate_fp8(v, v8, vs, nullptr, B, H, N, d, 1, nullptr));
  ACCEPT("quant_tensor", fa_quant_rotate_fp8_tensor(q, q8, qs, signs, B, H, N, d, 0, nullptr));
  NOOP(fa_quant_rotate_fp8(q, q8, qs, signs, B, H, 0, d, 0, nullptr));
  REJECT(FA_ERR_NULL, fa_quant_rotate_fp8(q, nullptr, qs, signs, B, H, N, d, 0, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_quant_rotate_fp8(q, q8, qs, signs, B, H, N, 32, 0, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_quant_rotate_fp8(q, q8, qs, signs, B, H, N, d, 2, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8(q, reinterpret_cast<uint8_t*>(q), qs, signs, B, H, N, d, 0, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8(q, q8, reinterpret_cast<float*>(q8 + 16), signs, B, H, N, d, 0, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8(q, q8, qs, reinterpret_cast<int8_t*>(qs), B, H, N, d, 0, nullptr));
  LAUNCH_FAILS(fa_quant_rotate_fp8(q, q8, qs, signs, B, H, N, d, 0, nullptr));
  // pre-pass, one launch for Q, K and V
  ACCEPT("quant_qkv", fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, v8, qs, ks, vs, signs, B, H, N, d, nullptr));
  ACCEPT("quant_qkv", fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, v8, qs, ks, vs, nullptr, B, H, N, d, nullptr));
  NOOP(fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, v8, qs, ks, vs, signs, 0, H, N, d, nullptr));
  REJECT(FA_ERR_NULL, fa_quant_rotate_fp8_qkv(q, k, nullptr, q8, k8, v8, qs, ks, vs, signs, B, H, N, d, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8_qkv(q, k, v, q8, q8, v8, qs, ks, vs, signs, B, H, N, d, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, v8, qs, qs + 2, vs, signs, B, H, N, d, nullptr));
  REJECT(FA_ERR_ALIAS, fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, reinterpret_cast<uint8_t*>(k), qs, ks, vs, signs, B,
                                               H, N, d, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_quant_rotate_fp8_qkv(q, k, v, q8 + 1, k8, v8, qs, ks, vs, signs, B, H, N, d, nullptr));
  LAUNCH_FAILS(fa_quant_rotate_fp8_qkv(q, k, v, q8, k8, v8, qs, ks, vs, signs, B, H, N, d, nullptr));
  // attention on the codes
  ACCEPT("attn_fp8", fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, lse, B, H, N, d, 1, 0.08f, nullptr));
  ACCEPT("attn_fp8_pbf16", fa_fwd_fp8_pbf16(q8, k8, v8, qs, ks, vs, 1, o, lse, B, H, N, d, 0, 0.08f, nullptr));
  NOOP(fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, lse, B, 0, N, d, 1, 0.08f, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 0, o, lse, B, H, N, d, 1, 0.08f, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, lse, B, H, N, 64, 1, 0.08f, nullptr));
  REJECT(FA_ERR_SCALE, fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, lse, B, H, N, d, 1, kInfF, nullptr));
  REJECT(FA_ERR_NULL, fa_fwd_fp8(q8, k8, v8, nullptr, ks, vs, 1, o, lse, B, H, N, d, 1, 0.08f, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, v8, lse, B, H, N, d, 1, 0.08f, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, ks, B, H, N, d, 1, 0.08f, nullptr));
  LAUNCH_FAILS(fa_fwd_fp8(q8, k8, v8, qs, ks, vs, 1, o, lse, B, H, N, d, 1, 0.08f, nullptr));
}

void split_and_merge(Pool& pool) {
  const int64_t B = 1, H = 2, Nq = 16, Nk = 1000, d = 128, S = 4;
  char *q = pool.get(B * H * Nq * d * 2), *k = pool.get(B * H * Nk * d * 2), *v = pool.get(B * H * Nk * d * 2);
  auto* op = reinterpret_cast<float*>(pool.get(S * B * H * Nq * d * 4));
  auto* lp = reinterpret_cast<float*>(pool.get(S * B * H * Nq * 4));
  char* o = pool.get(B * H * Nq * d * 2);
  auto* lse = reinterpret_cast<float*>(pool.get(B * H * Nq * 4));
  ACCEPT("attn_bf16_partial", fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, Nk - Nq, 0, Nk, S, 1, 0.1f, FA_BF16, nullptr));
  ACCEPT("attn_bf16_partial", fa_fwd_partial(q, k, v, op, lp, B, H, Nq, Nk, d, Nk - Nq, 10, 500, 1, 0.1f, FA_BF16, nullptr));
  NOOP(fa_fwd_split(q, k, v, op, lp, B, H, 0, Nk, d, 0, 0, Nk, S, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, 0, 10, 5, S, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, 0, 0, Nk + 1, S, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, 0, 0, Nk, 0, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, -1, 0, Nk, S, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, INT64_MAX, 0, Nk, S, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, 0, 0, Nk, S, 1, 0.1f, FA_F32, nullptr));
  REJECT(FA_ERR_ALIAS, fa_fwd_split(q, k, v, reinterpret_cast<float*>(k), lp, B, H, Nq, Nk, d, 0, 0, Nk, S, 1, 0.1f,
                                    FA_BF16, nullptr));
  LAUNCH_FAILS(fa_fwd_split(q, k, v, op, lp, B, H, Nq, Nk, d, 0, 0, Nk, S, 1, 0.1f, FA_BF16, nullptr));
  ACCEPT("merge", fa_merge(op, lp, S, o, lse, B, H, Nq, d, FA_BF16, nullptr));
  NOOP(fa_merge(op, lp, S, o, lse, B, H, 0, d, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_merge(op, lp, 0, o, lse, B, H, Nq, d, FA_BF16, nullptr));
  REJECT(FA_ERR_SHAPE, fa_merge(op, lp, INT64_MAX, o, lse, B, H, Nq, d, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_merge(op, lp, S, o, lse, B, H, Nq, d, 5, nullptr));
  REJECT(FA_ERR_ALIAS, fa_merge(op, lp, S, op + 8, lse, B, H, Nq, d, FA_BF16, nullptr));
  LAUNCH_FAILS(fa_merge(op, lp, S, o, lse, B, H, Nq, d, FA_BF16, nullptr));
}

void backward(Pool& pool) {
  const int64_t B = 1, H = 2, N = 200, d = 64;
  const size_t tb = B * H * N * d * 2, rb = B * H * N * 4;
  char *q = pool.get(tb), *k = pool.get(tb), *v = pool.get(tb), *o = pool.get(tb), *dout = pool.get(tb);
  char *dq = pool.get(tb), *dk = pool.get(tb), *dv = pool.get(tb);
  auto* lse = reinterpret_cast<float*>(pool.get(rb));
  auto* delta = reinterpret_cast<float*>(pool.get(rb));
  ACCEPT("attn_bwd", fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  CHECK(fake::last_ws == delta);
  NOOP(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, 0, d, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_UNSUPPORTED, fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, 1, 0.1f, FA_F32, nullptr));
  REJECT(FA_ERR_NULL, fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_bwd(q, k, v, o, dout, lse, dq, dq, dv, delta, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, lse, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_ALIAS, fa_bwd(q, k, v, o, dout, lse, dq, dk, o, delta, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_SCALE, fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, 1, kNaN, FA_BF16, nullptr));
  LAUNCH_FAILS(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  // the entry point that allocates nothing: the workspace is the library's own
  ACCEPT("attn_bwd", fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  CHECK(fake::last_ws == fake::scratch_stand_in);
  REJECT(FA_ERR_SCRATCH, fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, 1, 1, FA_BWD_NOALLOC_MAX_ROWS + 1, d, 1,
                                        0.1f, FA_BF16, nullptr));
  REJECT(FA_ERR_NULL, fa_bwd_noalloc(q, k, v, o, nullptr, lse, dq, dk, dv, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  fake::scratch_status = hipErrorInvalidSymbol;
  REJECT(FA_ERR_HIP, fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
  fake::scratch_status = hipSuccess;
  LAUNCH_FAILS(fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, 1, 0.1f, FA_BF16, nullptr));
}

}  // namespace

int main() {
  Pool pool;
  CHECK(fa_abi_version() == FA_ABI_VERSION);
  for (int st = -2; st < 12; ++st) CHECK(fa_status_string(st) != nullptr);
  forward(pool);
  fp8(pool);
  split_and_merge(pool);
  backward(pool);
  std::printf("%d of %d checks passed\n", g_checks - g_failures, g_checks);
  return g_failures == 0 ? 0 : 1;
}
