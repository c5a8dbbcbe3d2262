// Calibration kernels for the measurements (declared in include/fa_calib.h):
// what the chip sustains on its own for the two resources the attention kernels
// are priced against, under the same clock and power conditions.
//  * matrix cores: every wavefront runs a long chain of MFMAs on four independent
//    accumulators (32x32 blocks), nothing else -- the sustained dense rate, and
//    the reading of the MFMA-busy counter at a known full load;
//  * HBM: a streaming copy of known size (16-byte loads and stores, one pass) --
//    the sustained bandwidth, and the factor that turns the FETCH_SIZE and
//    WRITE_SIZE counters into bytes; and a streaming read (the decode kernels'
//    traffic is almost all reads).
#include "fa_calib.h"
#include "fa_device.h"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kAcc = 4;  // independent accumulators per wavefront

// kind 0: v_mfma_f32_32x32x16_bf16 (32768 FLOP each); kind 1:
// v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands and unit scales (131072 FLOP)
template <int KIND>
__global__ __launch_bounds__(256) void mfma_chain_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
      b[i] = (__bf16)(0.001f * (float)((lane * 3 + i) & 7));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  } else {
    i32x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x38383838 + ((lane + i) & 3);  // e4m3 values near 1
      b[i] = 0x30303030 + ((lane * 3 + i) & 3);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < kAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kUnroll = 4;           // 16-byte words in flight per thread
constexpr int kStreamGrid = 64 * 256;  // workgroups of the streaming kernels (64 per compute unit)

// dst[i] = src[i] for n16 16-byte words: each thread loads kUnroll words (256
// apart), then stores them; grid-stride over the array
__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n16; base += stride) {
    if (base + (kUnroll - 1) * 256 < n16) {
      uint4 w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) w[u] = src[base + u * 256];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[base + u * 256] = w[u];
    } else {
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * 256 < n16) dst[base + u * 256] = src[base + u * 256];
    }
  }
}

// out[thread] = XOR of the 16-byte words the thread reads (every word read once)
__global__ __launch_bounds__(256) void read16_kernel(const uint4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kUnroll;
  uint4 x = make_uint4(0, 0, 0, 0);
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; base < n16; base += stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * 256 < n16) {
        const uint4 w = src[base + u * 256];
        x.x ^= w.x, x.y ^= w.y, x.z ^= w.z, x.w ^= w.w;
      }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

unsigned stream_grid(int64_t n16) {
  const int64_t want = (n16 + 256 * kUnroll - 1) / (256 * kUnroll);
  return (unsigned)(want < kStreamGrid ? want : kStreamGrid);
}

}  // namespace
}  // namespace fa

extern "C" {

int fa_calib_mfma(int kind, int64_t workgroups, int64_t iters, float* out, void* stream) {
  if (kind != 0 && kind != 1) return FA_ERR_UNSUPPORTED;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return FA_ERR_SHAPE;
  if (!out) return FA_ERR_NULL;
  const dim3 grid((unsigned)workgroups), block(256);
  if (kind == 0)
    hipLaunchKernelGGL(fa::mfma_chain_kernel<0>, grid, block, 0, static_cast<hipStream_t>(stream), (int)iters, out);
  else
    hipLaunchKernelGGL(fa::mfma_chain_kernel<1>, grid, block, 0, static_cast<hipStream_t>(stream), (int)iters, out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_calib_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return FA_ERR_SHAPE;
  if (bytes == 0) return FA_OK;
  if (!src || !dst) return FA_ERR_NULL;
  if ((uintptr_t)src % 16 || (uintptr_t)dst % 16) return FA_ERR_UNSUPPORTED;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes) return FA_ERR_ALIAS;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(fa::copy16_kernel, dim3(fa::stream_grid(n16)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_calib_read(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return FA_ERR_SHAPE;
  if (bytes == 0) return FA_OK;
  if (!src || !out) return FA_ERR_NULL;
  if ((uintptr_t)src % 16 || (uintptr_t)out % 4) return FA_ERR_UNSUPPORTED;
  const int64_t n16 = bytes / 16;
  const unsigned grid = fa::stream_grid(n16);
  const uintptr_t s = (uintptr_t)src, o = (uintptr_t)out, ob = (uintptr_t)grid * 256 * 4;
  if (s < o + ob && o < s + (uintptr_t)bytes) return FA_ERR_ALIAS;
  hipLaunchKernelGGL(fa::read16_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), n16, out);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
