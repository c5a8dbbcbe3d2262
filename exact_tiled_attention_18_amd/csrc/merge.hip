// Merge of partial attention results over disjoint key ranges.
//
// A row's softmax over a union of key ranges follows from the ranges' own
// results, because the exponentials add: with L_s the logsumexp of range s and
// O_s its normalised output, the union has L = log(sum_s exp(L_s)) and
// O = sum_s exp(L_s - L) O_s.  This is the rescaling identity behind the
// pages' online softmax (FlashAttention-2 wiki page, "Technische Architektur",
// item 1; page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1) applied once to whole blocks: the step
// that lets one row be split over key ranges (split-KV) or over devices.
//
// One wavefront per row; the kernel reads each partial once and writes O and
// LSE once, with the loads of a row issued together so that it is bound by
// HBM rather than by one memory round trip per range.  Ranges in which a row sees no key carry
// L_s = -inf and contribute nothing; a row that sees no key at all gets
// O = 0, L = -inf.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kRowsPerBlock = 4;  // wavefronts per workgroup
constexpr int kUnroll = 8;        // partial rows whose loads are in flight together

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Lane j holds the LSE of range s0 + j, so a row's LSEs arrive in one load per 64
// ranges and the maximum and the sum of the weights are wave reductions; the
// partial rows are read kUnroll at a time, each weighted by its range's factor
// taken from the lane that holds it.  The first batch of partial rows does not
// depend on the weights and is loaded together with the LSEs, so up to kUnroll
// ranges cost one memory round trip.
template <int D, bool BF16>
__global__ __launch_bounds__(kRowsPerBlock * 64) void merge_kernel(const float* __restrict__ o_parts,
                                                                   const float* __restrict__ lse_parts, int n,
                                                                   void* __restrict__ o, float* __restrict__ lse,
                                                                   int64_t rows) {
  constexpr int C = D / 64;  // columns per lane
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  float x[kUnroll][C];
  // rows s0 + j0 .. s0 + j0 + kUnroll - 1 of the partials (indices past cnt repeat the
  // last range, whose weight there is 0)
  auto load_batch = [&](int s0, int j0, int cnt) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + (j0 + u < cnt ? j0 + u : cnt - 1);
      const float* src = o_parts + ((int64_t)s * rows + row) * D + lane * C;
      if constexpr (C == 2) {
        const float2 v2 = *reinterpret_cast<const float2*>(src);
        x[u][0] = v2.x;
        x[u][1] = v2.y;
      } else {
        x[u][0] = src[0];
      }
    }
  };
  const int cnt0 = n < 64 ? n : 64;
  const float ls0 = lane < cnt0 ? lse_parts[(int64_t)lane * rows + row] : -kInf;
  if (n > 0) load_batch(0, 0, cnt0);
  float mx = ls0;
  for (int s0 = 64; s0 < n; s0 += 64)
    if (s0 + lane < n) mx = fmaxf(mx, lse_parts[(int64_t)(s0 + lane) * rows + row]);
  mx = wave_max(mx);
  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;
  float sum = 0.f;
  if (mx != -kInf) {
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int cnt = n - s0 < 64 ? n - s0 : 64;
      const float ls = s0 == 0 ? ls0 : (lane < cnt ? lse_parts[(int64_t)(s0 + lane) * rows + row] : -kInf);
      // weight of range s0 + lane: exp(L_s - max), 0 for a range the row does not see
      const float ws = lane < cnt ? exp2_fast((ls - mx) * kLog2e) : 0.f;
      sum += wave_sum(ws);
      for (int j0 = 0; j0 < cnt; j0 += kUnroll) {
        if (s0 > 0 || j0 > 0) load_batch(s0, j0, cnt);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int j = j0 + u < cnt ? j0 + u : 0;
          const float w = j0 + u < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws), j)) : 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) acc[c] = fmaf(w, x[u][c], acc[c]);
        }
      }
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  if constexpr (BF16) {
    uint16_t* dst = static_cast<uint16_t*>(o) + row * D + lane * C;
    if constexpr (C == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      dst[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xFFFFu);
    }
  } else {
    float* dst = static_cast<float*>(o) + row * D + lane * C;
#pragma unroll
    for (int j = 0; j < C; ++j) dst[j] = acc[j] * inv;
  }
  if (lane == 0) lse[row] = sum > 0.f ? mx + log2_fast(sum) * kLn2 : -kInf;
}

template <int D>
hipError_t launch_d(const MergeArgs& a) {
  const int64_t rows = a.B * a.H * a.N;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
  if (a.dtype == 1)
    hipLaunchKernelGGL((merge_kernel<D, true>), grid, block, 0, a.stream, a.o_parts, a.lse_parts, (int)a.n, a.o,
                       a.lse, rows);
  else
    hipLaunchKernelGGL((merge_kernel<D, false>), grid, block, 0, a.stream, a.o_parts, a.lse_parts, (int)a.n, a.o,
                       a.lse, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a) { return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a); }

}  // namespace fa
