// fp32 attention forward (VALU).
//
// The fp32 problem this path serves is tiny (the whole workload is a few
// dozen MFLOP) and latency-bound, and gfx950 has no reduced-precision fp32
// matrix mode that would keep the 1e-5 accuracy, so the products run as
// plain fp32 FMAs on the vector ALUs.  The structure is the one of the bf16
// kernel: one workgroup owns a block of queries (outer loop), K/V tiles are
// staged through LDS (inner loop), and each query keeps a running maximum,
// a running sum and an unnormalised output, divided by the sum only after
// the last tile (page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1; FlashAttention-2 wiki page, section
// "Technische Architektur", items 1-2).
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kQueriesPerBlock = 64;
constexpr int kKeysPerTile = 32;
constexpr int kDimsPerThread = 64;

// One query is owned by D/64 adjacent threads, each holding 64 of its d
// columns in registers.  Work item (linear block id) -> (query block, head):
// causal grids start with the heaviest query blocks.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kQueriesPerBlock * (D / kDimsPerThread)) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c) {
  constexpr int TPQ = D / kDimsPerThread;
  constexpr int NT = kQueriesPerBlock * TPQ;
  __shared__ __attribute__((aligned(16))) float Ks[kKeysPerTile][D];
  __shared__ __attribute__((aligned(16))) float Vs[kKeysPerTile][D];

  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x;
  const int sub = tid % TPQ;
  const int qi = qblk * kQueriesPerBlock + tid / TPQ;
  const int d0 = sub * kDimsPerThread;

  float qr[kDimsPerThread], acc[kDimsPerThread];
#pragma unroll
  for (int e = 0; e < kDimsPerThread; ++e) {
    qr[e] = qi < N ? q[base + (size_t)qi * D + d0 + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -kInf, l = 0.f;

  const int q_last = min(N - 1, qblk * kQueriesPerBlock + kQueriesPerBlock - 1);
  const int kv_end = CAUSAL ? q_last + 1 : N;
  for (int k0 = 0; k0 < kv_end; k0 += kKeysPerTile) {
    __syncthreads();
    for (int i = tid; i < kKeysPerTile * D / 4; i += NT) {
      const int row = i / (D / 4), col = (i % (D / 4)) * 4;
      float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
      if (k0 + row < N) {
        kv4 = *reinterpret_cast<const float4*>(k + base + (size_t)(k0 + row) * D + col);
        vv4 = *reinterpret_cast<const float4*>(v + base + (size_t)(k0 + row) * D + col);
      }
      *reinterpret_cast<float4*>(&Ks[row][col]) = kv4;
      *reinterpret_cast<float4*>(&Vs[row][col]) = vv4;
    }
    __syncthreads();

    // scores of this query against the tile's keys, in log2 units
    float t[kKeysPerTile];
    float mt = -kInf;
#pragma unroll
    for (int j = 0; j < kKeysPerTile; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < kDimsPerThread; ++e) s = fmaf(qr[e], Ks[j][d0 + e], s);
      if (TPQ == 2) s += __shfl_xor(s, 1);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= qi);
      t[j] = vis ? s * c : -kInf;
      mt = fmaxf(mt, t[j]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -kInf) continue;  // no visible key for this query yet
    const float alpha = exp2_fast(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kKeysPerTile; ++j) {
      t[j] = exp2_fast(t[j] - m_new);
      rs += t[j];
    }
    l = alpha * l + rs;
    m = m_new;
#pragma unroll
    for (int e = 0; e < kDimsPerThread; ++e) {
      float a = alpha * acc[e];
#pragma unroll
      for (int j = 0; j < kKeysPerTile; ++j) a = fmaf(t[j], Vs[j][d0 + e], a);
      acc[e] = a;
    }
  }

  if (qi < N) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < kDimsPerThread; e += 4) {
      float4 r = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
      *reinterpret_cast<float4*>(o + base + (size_t)qi * D + d0 + e) = r;
    }
    if (sub == 0) lse[(size_t)bh * N + qi] = (m + log2_fast(l)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nQB = (N + kQueriesPerBlock - 1) / kQueriesPerBlock;
  const dim3 grid((unsigned)(nQB * BH)), block(kQueriesPerBlock * (D / kDimsPerThread));
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), grid, block, 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, BH, N, nQB,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
