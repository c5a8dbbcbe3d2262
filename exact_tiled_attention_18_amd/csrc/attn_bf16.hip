// bf16 attention forward on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Method (page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1; FlashAttention-2 wiki page, sections
// "Hintergrund" and "Technische Architektur", items 1-3):
//   * outer loop over query blocks -- one workgroup per (query block, head,
//     batch), so a single head is spread over many compute units;
//   * inner loop over key/value tiles staged through LDS;
//   * online softmax: running row maximum, exp2 of the shifted scores,
//     correction of the running sum and the unnormalised output by
//     exp2(m_old - m_new), and a single division by the row sum after the
//     last tile;
//   * every wavefront owns whole query rows, so row maxima and sums never
//     go through LDS.
//
// MI355X mapping.  A wavefront owns 32*QB queries.  Scores are computed
// transposed, S^T = K Q^T, with K as the MFMA A operand (from LDS) and Q as
// the B operand (registers, loaded once).  In the 32x32 accumulator layout a
// lane then holds one query column (lane % 32) and 16 of the 32 keys of the
// block, so the row statistics of a query live in one lane plus its partner
// 32 lanes away: the row max needs one cross-half exchange per tile and the
// row sum is kept per lane until the epilogue.  The K rows fed to the A
// operand are permuted (bits 2 and 3 of the row index swapped) so that a
// lane's 16 keys come out as two runs of 8 consecutive keys, which is exactly
// the operand layout the second product O^T += V^T P^T needs for P^T as its
// B operand: the probabilities go from accumulator registers to operand
// registers with one bf16 conversion and no data movement.  O^T is kept in
// the same column-per-query layout, so the per-tile correction factor is a
// lane-local multiply.  V is transposed into LDS on its way in (keys
// contiguous) for the A operand of the second product.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kBc = 64;  // keys per tile

template <int D>
struct Smem {
  static constexpr int KS = D + 8;    // K tile row stride (bf16 elements), 16-byte aligned rows
  static constexpr int VS = kBc + 8;  // V^T tile row stride
  uint16_t k[kBc * KS];
  uint16_t vt[D * VS];
};

__device__ __forceinline__ int permuted_row(int i) {  // swap bits 2 and 3
  return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC);
}
// key offset (within a 32-key block) of accumulator register r in lane half g
__device__ __forceinline__ int key_of_reg(int r, int g) { return (r & 7) + g * 8 + (r & 8) * 2; }

template <int D, bool CAUSAL, int QB>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c) {
  constexpr int W = 32 * QB;    // queries per wavefront
  constexpr int BR = kWaves * W;  // queries per workgroup
  constexpr int KB = kBc / 32;  // 32-key blocks per tile
  constexpr int DK = D / 16;    // k-steps of the first product
  constexpr int DB = D / 32;    // 32-column blocks of O^T
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) S sm;

  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, li = lane & 31;
  const int q0 = qblk * BR;
  const int qw0 = q0 + wave * W;
  const bool cpos = c >= 0.f;

  // Q^T as B operand: lane holds 8 consecutive d of its query per k-step.
  bf16x8 qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw0 + qb * 32 + li;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      uint4 val = make_uint4(0, 0, 0, 0);
      if (row < N) val = *reinterpret_cast<const uint4*>(q + base + (size_t)row * D + ks * 16 + g * 8);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, val);
    }
  }

  f32x16 oacc[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m[qb] = -kInf; l[qb] = 0.f; }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int nT = (kv_end + kBc - 1) / kBc;
  for (int t = 0; t < nT; ++t) {
    const int k0 = t * kBc;
    __syncthreads();
    // ---- K tile -> LDS (rows of d, 16-byte chunks)
#pragma unroll
    for (int i = 0; i < kBc * D / 8 / (kWaves * 64); ++i) {
      const int cidx = tid + i * kWaves * 64;
      const int row = cidx / (D / 8), col = (cidx % (D / 8)) * 8;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (k0 + row < N) val = *reinterpret_cast<const uint4*>(k + base + (size_t)(k0 + row) * D + col);
      *reinterpret_cast<uint4*>(&sm.k[row * S::KS + col]) = val;
    }
    // ---- V tile -> LDS transposed (V^T: rows of keys)
    {
      constexpr int KPT = kBc * D / 8 / (kWaves * 64);  // keys per thread (4 for d=128, 2 for d=64)
      const int dc = tid % (D / 8), kg = tid / (D / 8);
      uint4 vv[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int key = k0 + kg * KPT + j;
        vv[j] = make_uint4(0, 0, 0, 0);
        if (key < N) vv[j] = *reinterpret_cast<const uint4*>(v + base + (size_t)key * D + dc * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t h[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t w = (&vv[j].x)[e >> 1];
          h[j] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFF));
        }
        uint16_t* dst = &sm.vt[(dc * 8 + e) * S::VS + kg * KPT];
        if constexpr (KPT == 4) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
        } else {
          *reinterpret_cast<uint32_t*>(dst) = h[0] | ((uint32_t)h[1] << 16);
        }
      }
    }
    __syncthreads();
    if (CAUSAL && k0 > qw0 + W - 1) continue;  // every key of the tile is in this wave's future

    // ---- S^T = K Q^T
    f32x16 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = kb * 32 + permuted_row(li);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[row * S::KS + ks * 16 + g * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 domain: t = c * s, c = scale * log2(e))
    const bool masked = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    bf16x8 pf[QB][kBc / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qw0 + qb * 32 + li;
      // the max of c*s is c*max(s) for c >= 0 and c*min(s) for c < 0 (rounding is monotone)
      float mx = cpos ? -kInf : kInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][qb][r];
          if (masked) {
            const int key = k0 + kb * 32 + key_of_reg(r, g);
            if (key >= N || (CAUSAL && key > qi)) x = cpos ? -kInf : kInf;
          }
          mx = cpos ? fmaxf(mx, x) : fminf(mx, x);
        }
      const float mo = xor32(mx);
      mx = cpos ? fmaxf(mx, mo) : fminf(mx, mo);
      const float mt = (mx == kInf || mx == -kInf) ? -kInf : c * mx;
      const float m_new = fmaxf(m[qb], mt);
      const float alpha = m_new == -kInf ? 1.f : exp2_fast(m[qb] - m_new);
      const float msub = m_new == -kInf ? 0.f : m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_fast(fmaf(s[kb][qb][r], c, -msub));
          if (masked) {
            const int key = k0 + kb * 32 + key_of_reg(r, g);
            if (key >= N || (CAUSAL && key > qi)) p = 0.f;
          }
          s[kb][qb][r] = p;
          rs += p;
        }
      l[qb] = alpha * l[qb] + rs;
      m[qb] = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 w;
          w.x = pack_bf16x2(s[kb][qb][8 * h + 0], s[kb][qb][8 * h + 1]);
          w.y = pack_bf16x2(s[kb][qb][8 * h + 2], s[kb][qb][8 * h + 3]);
          w.z = pack_bf16x2(s[kb][qb][8 * h + 4], s[kb][qb][8 * h + 5]);
          w.w = pack_bf16x2(s[kb][qb][8 * h + 6], s[kb][qb][8 * h + 7]);
          pf[qb][kb * 2 + h] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int mm = 0; mm < kBc / 16; ++mm) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.vt[(db * 32 + li) * S::VS + mm * 16 + g * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][mm], oacc[db][qb], 0, 0, 0);
      }
  }

  // ---- epilogue: the single division by the row sum, LSE, stores
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + xor32(l[qb]);
    const int qi = qw0 + qb * 32 + li;
    if (qi < N) {
      const float inv = 1.f / lt;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dcol = db * 32 + 8 * a4 + 4 * g;
          uint2 w;
          w.x = pack_bf16x2(oacc[db][qb][4 * a4 + 0] * inv, oacc[db][qb][4 * a4 + 1] * inv);
          w.y = pack_bf16x2(oacc[db][qb][4 * a4 + 2] * inv, oacc[db][qb][4 * a4 + 3] * inv);
          *reinterpret_cast<uint2*>(o + base + (size_t)qi * D + dcol) = w;
        }
      if (g == 0) lse[(size_t)bh * N + qi] = (m[qb] + log2_fast(lt)) * kLn2;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnArgs& a) {
  constexpr int QB = 1;
  constexpr int BR = kWaves * 32 * QB;
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nQB = (N + BR - 1) / BR;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, QB>), dim3((unsigned)(nQB * BH)), dim3(kWaves * 64), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, BH, N, nQB,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
