// FP8 (OCP e4m3) attention forward on gfx950 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).
//
// Same structure as the bf16 kernel (query block per workgroup, key/value
// tiles through LDS, online softmax with one final division, transposed
// scores so that each lane owns a query), on operands produced by the
// quantise+rotate pre-pass.  The FP8 variant of the pages doubles the matrix
// throughput and relies on per-tile scales and the random rotation of Q and K
// for accuracy (page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1, FlashAttention-3 FP8 item).
//
// Scales.  A workgroup's 128 queries are exactly one quantisation tile of Q,
// and a 64-key tile lies inside one 128-row tile of K and of V, so every
// score of a (query tile, key tile) pair shares the factor
// scale * q_scale * k_scale, folded into the softmax multiplier.  The
// probabilities are multiplied by 256 and rounded to e4m3 for the second
// product; the accumulator is kept in units of the current V tile's scale
// (the correction factor of the online softmax also carries the ratio of
// consecutive V scales), and the epilogue multiplies by the last V scale and
// divides by 256 and by the row sum, which is accumulated from the unrounded
// fp32 probabilities.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kBc = 64;
constexpr int kD = 128;
constexpr int kTile = 128;  // quantisation tile rows
constexpr int kKS = kD + 16;   // K8 tile row stride (bytes)
constexpr int kVS = kBc + 16;  // V8^T tile row stride (bytes)

__device__ __forceinline__ int permuted_row(int i) { return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC); }
__device__ __forceinline__ int key_of_reg(int r, int g) { return (r & 7) + g * 8 + (r & 8) * 2; }

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 = fp8 e4m3 for both operands; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
    uint16_t* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c) {
  constexpr int BR = kWaves * 32;  // = kTile: one Q quantisation tile per workgroup
  constexpr int KB = kBc / 32;
  constexpr int DB = kD / 32;
  __shared__ __attribute__((aligned(16))) uint8_t ksm[kBc * kKS];
  __shared__ __attribute__((aligned(16))) uint8_t vsm[kD * kVS];

  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const int nTiles = (N + kTile - 1) / kTile;
  const size_t base = (size_t)bh * N * kD;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, li = lane & 31;
  const int q0 = qblk * BR;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + li;
  const float cq = c * qs[(size_t)bh * nTiles + qblk];
  const bool cpos = c >= 0.f;

  // Q8 as B operand: per k-step of 64 columns, lane half g holds 32 consecutive columns
  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (qi < N) {
      const uint8_t* p = q8 + base + (size_t)qi * kD + kk * 64 + g * 32;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 16);
    }
    qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -kInf, l = 0.f, sv_prev = 1.f;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int nT = (kv_end + kBc - 1) / kBc;
  for (int t = 0; t < nT; ++t) {
    const int k0 = t * kBc;
    __syncthreads();
    // K8 tile: 64 rows of 128 bytes
#pragma unroll
    for (int i = 0; i < kBc * kD / 16 / (kWaves * 64); ++i) {
      const int cidx = tid + i * kWaves * 64;
      const int row = cidx / (kD / 16), col = (cidx % (kD / 16)) * 16;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (k0 + row < N) val = *reinterpret_cast<const uint4*>(k8 + base + (size_t)(k0 + row) * kD + col);
      *reinterpret_cast<uint4*>(&ksm[row * kKS + col]) = val;
    }
    // V8^T tile: 128 rows (d) of 64 key bytes, from the [d][N] layout
    {
      const uint8_t* vbase = v8t + (size_t)bh * kD * N;
      if ((N & 15) == 0 && k0 + kBc <= N) {
#pragma unroll
        for (int i = 0; i < kD * kBc / 16 / (kWaves * 64); ++i) {
          const int cidx = tid + i * kWaves * 64;
          const int row = cidx / (kBc / 16), col = (cidx % (kBc / 16)) * 16;
          *reinterpret_cast<uint4*>(&vsm[row * kVS + col]) =
              *reinterpret_cast<const uint4*>(vbase + (size_t)row * N + k0 + col);
        }
      } else {
        for (int i = tid; i < kD * kBc; i += kWaves * 64) {
          const int row = i / kBc, col = i % kBc;
          vsm[row * kVS + col] = (k0 + col < N) ? vbase[(size_t)row * N + k0 + col] : (uint8_t)0;
        }
      }
    }
    __syncthreads();
    if (CAUSAL && k0 > qw0 + 31) continue;

    const float cst = cq * ks[(size_t)bh * nTiles + k0 / kTile];
    const float sv = vs[(size_t)bh * nTiles + k0 / kTile];

    // S^T = K8 Q8^T
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int row = kb * 32 + permuted_row(li);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 lo = *reinterpret_cast<const uint4*>(&ksm[row * kKS + kk * 64 + g * 32]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&ksm[row * kKS + kk * 64 + g * 32 + 16]);
        const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        s[kb] = mfma_fp8(a, qf[kk], s[kb]);
      }
    }

    const bool masked = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    float mx = cpos ? -kInf : kInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r];
        if (masked) {
          const int key = k0 + kb * 32 + key_of_reg(r, g);
          if (key >= N || (CAUSAL && key > qi)) x = cpos ? -kInf : kInf;
        }
        mx = cpos ? fmaxf(mx, x) : fminf(mx, x);
      }
    const float mo = xor32(mx);
    mx = cpos ? fmaxf(mx, mo) : fminf(mx, mo);
    const float mt = (mx == kInf || mx == -kInf) ? -kInf : cst * mx;
    const float m_new = fmaxf(m, mt);
    const float alpha = m_new == -kInf ? 1.f : exp2_fast(m - m_new);
    const float msub = m_new == -kInf ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2_fast(fmaf(s[kb][r], cst, -msub));
        if (masked) {
          const int key = k0 + kb * 32 + key_of_reg(r, g);
          if (key >= N || (CAUSAL && key > qi)) p = 0.f;
        }
        s[kb][r] = p;
        rs += p;
      }
    l = alpha * l + rs;
    m = m_new;
    const float fac = alpha * (sv_prev / sv);
    sv_prev = sv;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= fac;

    // P8^T as B operand: keys [8g, 8g+8), [16+8g, ...), [32+8g, ...), [48+8g, ...)
    i32x8 pf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b0 = 8 * h;
        pf[kb * 4 + h * 2 + 0] = (int)pack_fp8x4(s[kb][b0 + 0] * 256.f, s[kb][b0 + 1] * 256.f,
                                                 s[kb][b0 + 2] * 256.f, s[kb][b0 + 3] * 256.f);
        pf[kb * 4 + h * 2 + 1] = (int)pack_fp8x4(s[kb][b0 + 4] * 256.f, s[kb][b0 + 5] * 256.f,
                                                 s[kb][b0 + 6] * 256.f, s[kb][b0 + 7] * 256.f);
      }

    // O^T += V8^T P8^T (accumulated in units of sv / 256)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint8_t* vr = &vsm[(db * 32 + li) * kVS + g * 8];
      const uint2 a0 = *reinterpret_cast<const uint2*>(vr + 0);
      const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 16);
      const uint2 a2 = *reinterpret_cast<const uint2*>(vr + 32);
      const uint2 a3 = *reinterpret_cast<const uint2*>(vr + 48);
      const i32x8 a = {(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, (int)a3.x, (int)a3.y};
      oacc[db] = mfma_fp8(a, pf, oacc[db]);
    }
  }

  const float lt = l + xor32(l);
  if (qi < N) {
    const float inv = sv_prev / (256.f * lt);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int dcol = db * 32 + 8 * a4 + 4 * g;
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv);
        *reinterpret_cast<uint2*>(o + base + (size_t)qi * kD + dcol) = w;
      }
    if (g == 0) lse[(size_t)bh * N + qi] = (m + log2_fast(lt)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_fp8(const Fp8AttnArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nQB = (N + kTile - 1) / kTile;
  const dim3 grid((unsigned)(nQB * BH)), block(kWaves * 64);
  const float c = a.scale * kLog2e;
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<true>), grid, block, 0, a.stream, a.q8, a.k8, a.v8t, a.q_scale,
                       a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o), a.lse, BH, N, nQB, c);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false>), grid, block, 0, a.stream, a.q8, a.k8, a.v8t, a.q_scale,
                       a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o), a.lse, BH, N, nQB, c);
  return hipGetLastError();
}

}  // namespace fa
