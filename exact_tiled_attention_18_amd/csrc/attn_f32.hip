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

constexpr int kQueriesPerBlock = 16;
constexpr int kKeysPerTile = 32;
constexpr int kDimsPerThread = 64;
constexpr int kKeySplits = 16;  // threads sharing one query's keys (every 16th key of a tile each)

// A query is owned by D/64 x kKeySplits adjacent threads: D/64 of them split
// its d columns (64 each, in registers), and kKeySplits groups of those split
// each tile's keys (key j goes to group j % kKeySplits), each group keeping its
// own running maximum, sum and unnormalised output.  After the last tile the
// partial states merge with the same rescaling rule (a butterfly over lanes).
// Work item (linear block id) -> (query block, head): causal grids start with
// the heaviest query blocks.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kQueriesPerBlock * kKeySplits * (D / kDimsPerThread)) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c) {
  constexpr int TPQ = D / kDimsPerThread;  // threads per query and key group
  constexpr int TQ = TPQ * kKeySplits;     // threads per query
  constexpr int NT = kQueriesPerBlock * TQ;
  constexpr int KPT = kKeysPerTile / kKeySplits;  // keys per thread and tile
  static_assert(TQ <= 64, "a query's threads share a wavefront");
  // rows padded by 16 bytes: the key groups of a wavefront read as many different
  // rows at once, which would otherwise all fall on the same LDS banks
  __shared__ __attribute__((aligned(16))) float Ks[kKeysPerTile][D + 4];
  __shared__ __attribute__((aligned(16))) float Vs[kKeysPerTile][D + 4];

  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x;
  const int sub = tid % TPQ;
  const int split = (tid / TPQ) % kKeySplits;
  const int qi = qblk * kQueriesPerBlock + tid / TQ;
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
  // tile copies: each thread moves P float4 pieces of K and of V, loaded one tile ahead
  constexpr int P = (kKeysPerTile * D / 4 + NT - 1) / NT;
  float4 kst[P], vst[P];
  auto load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = tid + p * NT, row = i / (D / 4), col = (i % (D / 4)) * 4;
      kst[p] = vst[p] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < kKeysPerTile * D / 4 && k0 + row < N) {
        kst[p] = *reinterpret_cast<const float4*>(k + base + (size_t)(k0 + row) * D + col);
        vst[p] = *reinterpret_cast<const float4*>(v + base + (size_t)(k0 + row) * D + col);
      }
    }
  };
  load(0);
  for (int k0 = 0; k0 < kv_end; k0 += kKeysPerTile) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = tid + p * NT, row = i / (D / 4), col = (i % (D / 4)) * 4;
      if (i < kKeysPerTile * D / 4) {
        *reinterpret_cast<float4*>(&Ks[row][col]) = kst[p];
        *reinterpret_cast<float4*>(&Vs[row][col]) = vst[p];
      }
    }
    __syncthreads();
    if (k0 + kKeysPerTile < kv_end) load(k0 + kKeysPerTile);

    // scores of this query against this thread's keys of the tile, in log2 units
    float t[KPT];
    float mt = -kInf;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = split + kKeySplits * i;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < kDimsPerThread; ++e) s = fmaf(qr[e], Ks[j][d0 + e], s);
      if (TPQ == 2) s += __shfl_xor(s, 1);
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= qi);
      t[i] = vis ? s * c : -kInf;
      mt = fmaxf(mt, t[i]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -kInf) continue;  // no visible key for this thread yet
    const float alpha = exp2_fast(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      t[i] = exp2_fast(t[i] - m_new);
      rs += t[i];
    }
    l = alpha * l + rs;
    m = m_new;
#pragma unroll
    for (int e = 0; e < kDimsPerThread; ++e) {
      float a = alpha * acc[e];
#pragma unroll
      for (int i = 0; i < KPT; ++i) a = fmaf(t[i], Vs[split + kKeySplits * i][d0 + e], a);
      acc[e] = a;
    }
  }

  // merge the key groups' partial states: M = max of the maxima, every part
  // rescaled by exp2(m_g - M) (0 for a group that saw no key)
#pragma unroll
  for (int off = TPQ; off < TQ; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    const float mm = fmaxf(m, m2);
    const float a1 = m == -kInf ? 0.f : exp2_fast(m - mm);
    const float a2 = m2 == -kInf ? 0.f : exp2_fast(m2 - mm);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < kDimsPerThread; ++e) acc[e] = acc[e] * a1 + __shfl_xor(acc[e], off) * a2;
    m = mm;
  }

  if (qi < N && split == 0) {
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
  const dim3 grid((unsigned)(nQB * BH)), block(kQueriesPerBlock * kKeySplits * (D / kDimsPerThread));
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
