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
// e4m3 code (ties to even; the largest magnitude maps to 448); a tile of
// magnitudes below 2^-96 counts as all-zero (scale 1).
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
// A tile whose largest magnitude (after the unnormalised transform) is below 2^-96
// is quantised as an all-zero tile: scale 1, every code +-0.  Above it, 448 / amax
// stays finite (below 2^105) and the scale amax / (448 sqrt(d)) a normal fp32 value;
// without the bound a tile of tiny values (bf16 subnormals, say) would get an
// infinite multiplier and turn its zero entries into NaN codes.
constexpr float kMinAmax = 0x1p-96f;

// Scale granularity (template MODE of the kernels below).  PER_TILE: each workgroup
// quantises its tile with the tile's own amax.  AMAX: it only writes the tile's amax
// into x_scale.  GIVEN: it quantises with the amax found in its x_scale entry (the
// whole tensor's, spread there by reduce_amax_kernel) and replaces it by the scale.
// AMAX, reduce, GIVEN is the per-tensor quantisation the block scales are compared
// against.
enum { PER_TILE = 0, AMAX = 1, GIVEN = 2 };

// four fp32 -> four OCP e4m3 codes packed in 32 bits (v_cvt_pk_fp8_f32: round to
// nearest even).  The scaled values here satisfy |t| <= 448 up to one rounding
// of the multiplier, far below 464, the first value that would not round to
// the largest finite code 448.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// DPP move of x over the whole wave (every lane written, so no old value is needed)
template <int CTRL>
__device__ __forceinline__ float dpp_all(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// value held by the lane whose index differs in bit HM (HM = 1, 2, 4, 8; inside 16-lane rows)
template <int HM>
__device__ __forceinline__ float partner(float x) {
  if constexpr (HM == 1) return dpp_all<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  if constexpr (HM == 2) return dpp_all<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  if constexpr (HM == 4) {
    // row_shl:4 into lanes 0-3 and 8-11 of each row (the other lanes are written next),
    // then row_shr:4 into lanes 4-7 and 12-15
    const float up = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x104, 0xF, 0x5, false));
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(up), __float_as_int(x), 0x114, 0xF, 0xA, false));
  }
  return dpp_all<0x128>(x);                          // row_ror:8
}

template <int HM>
__device__ __forceinline__ void butterfly(float (&z)[8], int cg) {
  const float sgn = (cg & HM) ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = fmaf(z[e], sgn, partner<HM>(z[e]));
}

// One 128-row tile (work item `item` = bh * nTiles + tile) of one tensor, row by row:
// optional sign flip and Hadamard transform, amax, codes row-major or transposed.
template <int D, bool ROTATE, bool TRANSPOSE, int MODE>
__device__ __forceinline__ void rotate_tile(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                            float* __restrict__ x_scale, const int8_t* __restrict__ signs, int N,
                                            int nTiles, int item) {
  constexpr int TPR = D / 8;                 // threads per row (8 values each)
  static_assert(TPR == 8 || TPR == 16, "row groups of 8 or 16 lanes");
  constexpr int RPP = kThreads / TPR;        // rows per pass
  constexpr int PASSES = kTileRows / RPP;
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tr[TRANSPOSE ? D * (kTileRows + 16) : 1];

  const int tile = item % nTiles;
  const int bh = item / nTiles;
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
      // spans 8 .. D/2 pair this thread with the one whose column group differs in one
      // bit (TPR consecutive lanes hold a row): (a, b) -> (a + b, a - b), the upper
      // lane computing b * -1 + a exactly as a - b
      butterfly<1>(z[p], cg);
      butterfly<2>(z[p], cg);
      butterfly<4>(z[p], cg);
      if constexpr (TPR == 16) butterfly<8>(z[p], cg);
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
  if constexpr (MODE == GIVEN) amax = x_scale[(size_t)bh * nTiles + tile];  // the tensor's amax
  __syncthreads();
  if constexpr (MODE != GIVEN) amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if constexpr (MODE == AMAX) {
    if (tid == 0) x_scale[(size_t)bh * nTiles + tile] = amax;
    return;
  }

  // value / scale = z * 448 / amax(z): the rotation's 1/sqrt(d) cancels here
  const bool live = amax >= kMinAmax;
  const float mult = live ? 448.0f / amax : 1.0f;
  if (tid == 0) {
    const float den = ROTATE ? 448.0f * __builtin_sqrtf((float)D) : 448.0f;
    x_scale[(size_t)bh * nTiles + tile] = live ? amax / den : 1.0f;
  }

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int lrow = p * RPP + tid / TPR;
    const int row = r0 + lrow;
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = z[p][e] * mult;
    // rows past N: code 0 (a sign flip of zero would otherwise give -0)
    const uint32_t lo = row < N ? e4m3x4(t[0], t[1], t[2], t[3]) : 0u;
    const uint32_t hi = row < N ? e4m3x4(t[4], t[5], t[6], t[7]) : 0u;
    if constexpr (!TRANSPOSE) {
      if (row < N) *reinterpret_cast<uint2*>(x8 + base + (size_t)row * D + cg * 8) = make_uint2(lo, hi);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tr[(cg * 8 + e) * (kTileRows + 16) + lrow] = (uint8_t)((e < 4 ? lo : hi) >> (8 * (e & 3)));
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

// Transposed output without rotation (the V operand): thread (cg, j) loads the R
// consecutive rows R*j .. R*j+R-1 of the tile in columns 8cg .. 8cg+7 (R = 8 at
// d = 128, 4 at d = 64), so for each of its columns it holds R codes that go to
// LDS as one R-byte word, in 16-byte chunks of a column row whose order is
// XOR-swizzled by the column group (the column groups of a wavefront would
// otherwise write the same banks).
template <int D, int MODE>
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                               float* __restrict__ x_scale, int N, int nTiles, int item) {
  constexpr int CG = D / 8;                      // column groups
  constexpr int R = kTileRows * CG / kThreads;   // rows per thread
  static_assert(R == 4 || R == 8, "4 or 8 rows per thread");
  constexpr int LD = kTileRows + 16;             // LDS bytes per column row (16-byte aligned)
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tr[D * LD];

  const int tile = item % nTiles;
  const int bh = item / nTiles;
  const int tid = threadIdx.x;
  const int cg = tid % CG, j = tid / CG;
  const int r0 = tile * kTileRows;
  const size_t base = (size_t)bh * N * D;

  float z[R][8];  // [row][column]
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = r0 + R * j + i;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row < N) w = *reinterpret_cast<const uint4*>(x + base + (size_t)row * D + cg * 8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) z[i][e] = __uint_as_float((e & 1) ? (ww[e >> 1] & 0xFFFF0000u) : (ww[e >> 1] << 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(z[i][e]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  if constexpr (MODE == GIVEN) amax = x_scale[(size_t)bh * nTiles + tile];  // the tensor's amax
  __syncthreads();
  if constexpr (MODE != GIVEN) amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if constexpr (MODE == AMAX) {
    if (tid == 0) x_scale[(size_t)bh * nTiles + tile] = amax;
    return;
  }
  const bool live = amax >= kMinAmax;
  const float mult = live ? 448.0f / amax : 1.0f;
  if (tid == 0) x_scale[(size_t)bh * nTiles + tile] = live ? amax / 448.0f : 1.0f;

  const int pos = R * j;  // byte position of this thread's rows in a column row
  const int off = (((pos >> 4) ^ (cg & 7)) << 4) + (pos & 15);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint8_t* t = &tr[(cg * 8 + e) * LD + off];
    // rows past N hold zeros, whose code is 0
    const uint32_t lo = e4m3x4(z[0][e] * mult, z[1][e] * mult, z[2][e] * mult, z[3][e] * mult);
    if constexpr (R == 8) {
      const uint32_t hi = e4m3x4(z[4][e] * mult, z[5][e] * mult, z[6][e] * mult, z[7][e] * mult);
      *reinterpret_cast<uint2*>(t) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<uint32_t*>(t) = lo;
    }
  }
  __syncthreads();
  // x8 is [B, H, D, N64]: row `col` of this head holds the codes of all N rows,
  // then code 0 up to N64
  const int ldv = (N + 63) / 64 * 64;
  const int chunks = min(kTileRows, ldv - r0) / 16;
  uint8_t* dst = x8 + (size_t)bh * D * ldv + r0;
  for (int i = tid; i < D * chunks; i += kThreads) {
    const int col = i / chunks, ch = i % chunks;
    *reinterpret_cast<uint4*>(dst + (size_t)col * ldv + ch * 16) =
        *reinterpret_cast<const uint4*>(&tr[col * LD + ((ch ^ ((col >> 3) & 7)) << 4)]);
  }
}

template <int D, bool ROTATE, bool TRANSPOSE, int MODE>
__global__ __launch_bounds__(kThreads) void quant_rotate_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                                float* __restrict__ x_scale,
                                                                const int8_t* __restrict__ signs, int N, int nTiles) {
  rotate_tile<D, ROTATE, TRANSPOSE, MODE>(x, x8, x_scale, signs, N, nTiles, blockIdx.x);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void quant_transpose_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ x8,
                                                                   float* __restrict__ x_scale, int N, int nTiles) {
  transpose_tile<D, MODE>(x, x8, x_scale, N, nTiles, blockIdx.x);
}

// The whole pre-pass of the FP8 path in one launch: work items [0, T) are Q's tiles,
// [T, 2T) K's (both rotated when ROTATE), [2T, 3T) V's (codes transposed), T = B*H*nTiles.
struct QkvPtrs {
  const uint16_t* x[3];
  uint8_t* x8[3];
  float* scale[3];
};
template <int D, bool ROTATE>
__global__ __launch_bounds__(kThreads) void quant_qkv_kernel(QkvPtrs p, const int8_t* __restrict__ signs, int N,
                                                             int nTiles, int T) {
  const int item = blockIdx.x;
  if (item < T)
    rotate_tile<D, ROTATE, false, PER_TILE>(p.x[0], p.x8[0], p.scale[0], signs, N, nTiles, item);
  else if (item < 2 * T)
    rotate_tile<D, ROTATE, false, PER_TILE>(p.x[1], p.x8[1], p.scale[1], signs, N, nTiles, item - T);
  else
    transpose_tile<D, PER_TILE>(p.x[2], p.x8[2], p.scale[2], N, nTiles, item - 2 * T);
}

// The largest of the n amaxes in x_scale, written back into every entry (one
// workgroup; every read completes before the first write).
__global__ __launch_bounds__(kThreads) void reduce_amax_kernel(float* __restrict__ x_scale, int n) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  float amax = 0.f;
  for (int i = tid; i < n; i += kThreads) amax = fmaxf(amax, x_scale[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int i = tid; i < n; i += kThreads) x_scale[i] = amax;
}

template <int D, int MODE>
void launch_mode(const QuantArgs& a, int N, int nTiles, dim3 grid, dim3 block) {
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  if (a.signs) {
    if (a.transpose_out)
      hipLaunchKernelGGL((quant_rotate_kernel<D, true, true, MODE>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
    else
      hipLaunchKernelGGL((quant_rotate_kernel<D, true, false, MODE>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
  } else {
    if (a.transpose_out)
      hipLaunchKernelGGL((quant_transpose_kernel<D, MODE>), grid, block, 0, a.stream, x, a.x8, a.x_scale, N, nTiles);
    else
      hipLaunchKernelGGL((quant_rotate_kernel<D, false, false, MODE>), grid, block, 0, a.stream, x, a.x8, a.x_scale, a.signs, N, nTiles);
  }
}

template <int D>
hipError_t launch_d(const QuantArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nTiles = (N + kTileRows - 1) / kTileRows;
  const dim3 grid((unsigned)(BH * nTiles)), block(kThreads);
  if (!a.per_tensor) {
    launch_mode<D, PER_TILE>(a, N, nTiles, grid, block);
  } else {
    launch_mode<D, AMAX>(a, N, nTiles, grid, block);
    hipLaunchKernelGGL(reduce_amax_kernel, dim3(1), block, 0, a.stream, a.x_scale, BH * nTiles);
    launch_mode<D, GIVEN>(a, N, nTiles, grid, block);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_qkv_d(const QkvQuantArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nTiles = (N + kTileRows - 1) / kTileRows;
  const int T = BH * nTiles;
  QkvPtrs p;
  for (int i = 0; i < 3; ++i) {
    p.x[i] = static_cast<const uint16_t*>(a.x[i]);
    p.x8[i] = a.x8[i];
    p.scale[i] = a.scale[i];
  }
  const dim3 grid((unsigned)(3 * T)), block(kThreads);
  if (a.signs)
    hipLaunchKernelGGL((quant_qkv_kernel<D, true>), grid, block, 0, a.stream, p, a.signs, N, nTiles, T);
  else
    hipLaunchKernelGGL((quant_qkv_kernel<D, false>), grid, block, 0, a.stream, p, a.signs, N, nTiles, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rotate_fp8(const QuantArgs& a) {
  return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a);
}

hipError_t launch_quant_qkv_fp8(const QkvQuantArgs& a) {
  return a.d == 64 ? launch_qkv_d<64>(a) : launch_qkv_d<128>(a);
}

}  // namespace fa
