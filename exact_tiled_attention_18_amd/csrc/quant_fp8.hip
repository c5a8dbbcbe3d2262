// FP8 pre-pass: random-sign Hadamard rotation + per-tile e4m3 quantisation.
//
// The pages keep FP8 accurate in the presence of outlier activations with two
// measures (page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1, FlashAttention-3 FP8 item): block
// quantisation, where each small tile has its own scale, and incoherent
// processing, where Q and K are multiplied by a random orthogonal matrix so
// that an outlier is spread over all coordinates before rounding.  Here the
// orthogonal matrix is R = diag(s) H_d / sqrt(d) (s a +-1 vector, H_d the
// Sylvester Hadamard matrix), applied as a fast Walsh-Hadamard transform in
// fp32 registers; the 1/sqrt(d) factor is folded into the tile scale.  A tile
// is 128 consecutive rows of one (batch, head) with all d columns; its scale
// is amax / 448 and every value is divided by it and rounded to the nearest
// e4m3 code (ties to even, saturating at +-448).
//
// One workgroup quantises one tile: it reads the tile once (bf16), keeps it
// in registers through the transform and the amax reduction, and writes the
// codes once -- the kernel moves each byte of HBM exactly once, which is its
// bound.  For V the codes can be written transposed, [B, H, d, N64] with N64
// = N rounded up to a multiple of 64 and zero codes in the padding, so the
// attention kernel's P V product reads whole aligned 64-key rows.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;

// fp32 -> OCP e4m3 code, round to nearest even, saturating at +-448, from the
// format definition (bias 7, 3 mantissa bits, subnormal step 2^-9).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  const uint32_t u = __float_as_uint(t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;  // NaN
  const float af = __uint_as_float(a);
  if (af < 0.015625f) {  // below 2^-6: subnormal grid m * 2^-9, m = 0..8
    return sign | (uint32_t)__builtin_rintf(af * 512.0f);
  }
  // keep 3 mantissa bits with round-to-nearest-even on the fp32 pattern,
  // then move the exponent bias from 127 to 7
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  r -= (127u - 7u) << 3;
  return sign | (r > 0x7Eu ? 0x7Eu : r);
}

template <int D, bool ROTATE, bool TRANSPOSE>
__global__ __launch_bounds__(kThreads) void quant_rotate_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8, float* __restrict__ x_scale,
    const int8_t* __restrict__ signs, int N, int nTiles) {
  constexpr int TPR = D / 8;                 // threads per row (8 values each)
  constexpr int RPP = kThreads / TPR;        // rows per pass
  constexpr int PASSES = kTileRows / RPP;
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tr[TRANSPOSE ? D * (kTileRows + 16) : 1];

  const int tile = blockIdx.x % nTiles;
  const int bh = blockIdx.x / nTiles;
  const int tid = threadIdx.x;
  const int cg = tid % TPR;  // column group: columns 8*cg .. 8*cg+7
  const int r0 = tile * kTileRows;
  const size_t base = (size_t)bh * N * D;

  float z[PASSES][8];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP + tid / TPR;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row < N) w = *reinterpret_cast<const uint4*>(x + base + (size_t)row * D + cg * 8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (e & 1) ? (ww[e >> 1] & 0xFFFF0000u) : (ww[e >> 1] << 16);
      z[p][e] = __uint_as_float(h);  // bf16 -> fp32 is exact
    }
  }

  if constexpr (ROTATE) {
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)signs[cg * 8 + e];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
#pragma unroll
      for (int e = 0; e < 8; ++e) z[p][e] *= sg[e];
      // Walsh-Hadamard butterflies, natural (Sylvester) order: for span h the
      // pair (i, i+h) becomes (a+b, a-b).  Spans 1, 2, 4 are inside a thread.
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & h) == 0) {
            const float a = z[p][e], b = z[p][e + h];
            z[p][e] = a + b;
            z[p][e + h] = a - b;
          }
      // spans 8 .. D/2 pair this thread with the one whose column group differs in one bit
#pragma unroll
      for (int hm = 1; hm < TPR; hm <<= 1) {
        const bool hi = (cg & hm) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float other = __shfl_xor(z[p][e], hm);
          z[p][e] = hi ? (other - z[p][e]) : (z[p][e] + other);
        }
      }
    }
  }

  // amax over the tile
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(z[p][e]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // value / scale = z * 448 / amax(z): the rotation's 1/sqrt(d) cancels here
  const float mult = amax > 0.f ? 448.0f / amax : 1.0f;
  if (tid == 0) {
    const float den = ROTATE ? 448.0f * __builtin_sqrtf((float)D) : 448.0f;
    x_scale[(size_t)bh * nTiles + tile] = amax > 0.f ? amax / den : 1.0f;
  }

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int lrow = p * RPP + tid / TPR;
    const int row = r0 + lrow;
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = row < N ? e4m3_code(z[p][e] * mult) : 0u;  // padding: code 0 (not -0)
    const uint32_t lo = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    const uint32_t hi = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    if constexpr (!TRANSPOSE) {
      if (row < N) *reinterpret_cast<uint2*>(x8 + base + (size_t)row * D + cg * 8) = make_uint2(lo, hi);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tr[(cg * 8 + e) * (kTileRows + 16) + lrow] = (uint8_t)c[e];
    }
  }
  if constexpr (TRANSPOSE) {
    __syncthreads();
    // x8 is [B, H, D, N64]: row `col` of this head holds the codes of all N rows,
    // then code 0 up to N64
    const int ldv = (N + 63) / 64 * 64;
    const int chunks = min(kTileRows, ldv - r0) / 16;
    uint8_t* dst = x8 + (size_t)bh * D * ldv + r0;
    for (int i = tid; i < D * chunks; i += kThreads) {
      const int col = i / chunks, ch = i % chunks;
      *reinterpret_cast<uint4*>(dst + (size_t)col * ldv + ch * 16) =
          *reinterpret_cast<const uint4*>(&tr[col * (kTileRows + 16) + ch * 16]);
    }
  }
}

template <int D>
hipError_t launch_d(const QuantArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nTiles = (N + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)(BH * nTiles)), block(kThreads);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.signs) {
    if (a.transpose_out)
      hipLaunchKernelGGL((quant_rotate_kernel<D, true, true>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
    else
      hipLaunchKernelGGL((quant_rotate_kernel<D, true, false>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
  } else {
    if (a.transpose_out)
      hipLaunchKernelGGL((quant_rotate_kernel<D, false, true>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
    else
      hipLaunchKernelGGL((quant_rotate_kernel<D, false, false>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rotate_fp8(const QuantArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

}  // namespace fa
