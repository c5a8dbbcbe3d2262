// fp32 attention forward on the matrix cores.
//
// The fp32 path serves small problems (its workload is a few dozen MFLOP) and
// is bound by latency, not throughput: what matters is how many compute units
// share the work and how few dependent steps each takes.  The products run on
// the matrix cores, which read their operands from registers, so no tile is
// staged through LDS.  The scores are the accuracy-critical product: a score
// of magnitude |s| accumulated in fp32 carries a rounding error of several
// u |s|, which at scale 0.5 and d = 128 (|s| up to ~50) moves the LSE by
// about 1e-5, the whole fp32 budget.  So S = Q K^T runs on the fp64 matrix
// core (v_mfma_f64_16x16x4_f64: fp32 inputs widen exactly, the products are
// exact and the sums carry 2^-53 relative error) and is rounded to fp32 once,
// after the scaling.  P V runs on v_mfma_f32_16x16x4_f32 (fp32 operands and
// accumulation; the output is a convex combination of V rows, so its error
// stays at a few u |V|).
//
// Decomposition.  A workgroup owns 16 queries of one head; its W wavefronts
// split the keys, wavefront w taking the 32-key blocks w, w + W, w + 2W, ...
// (W = 8 at d = 64, two wavefronts per SIMD, so that one's score products run
// while the other waits on its loads or its softmax; W = 4 at d = 128, whose
// registers fit one wavefront per SIMD).
// Each wavefront keeps its own running maximum, sum and unnormalised output
// over its blocks (the online softmax of page "FlashAttention-Skalierung,
// Multi-GPU-Training und Gewichtsquantisierung", section 1, and of the
// FlashAttention-2 wiki page, section "Technische Architektur", items 1-2);
// after the last block the W partial states merge through LDS by the
// rescaling rule (each part times exp2 of its maximum minus the largest), and
// the output is divided by the merged sum once.
//
// Layouts (16x16x4 MFMAs: lane l = 16 g + i holds A[i][g] and B[g][i]; the fp32
// form holds C[4 g + r][i] in register r, the fp64 form C[4 r + g][i]):
//  * scores transposed, S^T = K Q^T (fp64 form), in two 16-key halves of a
//    block: A = K rows, B = Q^T; the k-step s pairs the dimensions g * D/4 + s,
//    so a lane's K and Q operands are D/4 consecutive floats of one row;
//  * lane (i, g) then holds query i's scores of keys 16 h + 4 r + g (half h,
//    register r), and these are exactly the B operand P^T of the k-step (h, r)
//    in O^T += V^T P^T (fp32 form); the A operand V^T of that step is
//    V[16 h + 4 r + g][16 b + i] for the 16-dimension block b, one float per lane;
//  * O^T in lane (i, g), block b, register r: dimension 16 b + 4 g + r of query i.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kQ = 16;        // queries per workgroup
constexpr int kKB = 32;       // keys per block (two 16-key halves)
template <int D>
constexpr int waves() { return D == 64 ? 8 : 4; }  // wavefronts per workgroup, splitting the keys

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mfma4d(double a, double b, const f64x4& c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// the maximum and the sum over the four lanes that hold one query (lanes i, i+16, i+32, i+48)
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int D>
struct Block {
  static constexpr int KS = D / 4;  // k-steps of a score product = floats per lane of a K or Q row
  static constexpr int DB = D / 16; // 16-dimension blocks of O^T
  float kf[2][KS];                  // K operands of the two halves
  float vf[2][4][DB];               // V^T operands: half, register r, dimension block
};

template <int D>
__device__ __forceinline__ void load_block(Block<D>& blk, const float* __restrict__ k, const float* __restrict__ v,
                                           int kb, int N, int i, int g) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = kb * kKB + 16 * h + i;
    if (key < N) {
      const float4* src = reinterpret_cast<const float4*>(k + (size_t)key * D + g * Block<D>::KS);
#pragma unroll
      for (int s = 0; s < Block<D>::KS / 4; ++s) {
        const float4 w = src[s];
        blk.kf[h][4 * s] = w.x, blk.kf[h][4 * s + 1] = w.y, blk.kf[h][4 * s + 2] = w.z, blk.kf[h][4 * s + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < Block<D>::KS; ++s) blk.kf[h][s] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vkey = kb * kKB + 16 * h + 4 * g + r;
#pragma unroll
      for (int b = 0; b < Block<D>::DB; ++b) blk.vf[h][r][b] = vkey < N ? v[(size_t)vkey * D + 16 * b + i] : 0.f;
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(waves<D>() * 64) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, double c) {
  using Blk = Block<D>;
  constexpr int KS = Blk::KS, DB = Blk::DB, kWaves = waves<D>();
  constexpr int OS = D + 4;  // LDS row stride of the merge (floats)
  __shared__ float s_m[kWaves][kQ], s_l[kWaves][kQ];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][kQ][OS];

  // work item -> (query block, head); causal grids start with the heaviest blocks
  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  q += base, k += base, v += base;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const int q0 = qblk * kQ, qi = q0 + i;
  const int kv_end = CAUSAL ? min(N, q0 + kQ) : N;
  const int nKB = (kv_end + kKB - 1) / kKB;

  // Q^T operands (widened to fp64): query q0 + i, dimensions g * D/4 .. + D/4 (zeros past N)
  float qf[KS];
  if (qi < N) {
    const float4* src = reinterpret_cast<const float4*>(q + (size_t)qi * D + g * KS);
#pragma unroll
    for (int s = 0; s < KS / 4; ++s) {
      const float4 x = src[s];
      qf[4 * s] = x.x, qf[4 * s + 1] = x.y, qf[4 * s + 2] = x.z, qf[4 * s + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = 0.f;
  }

  f32x4 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -kInf, l = 0.f;

  Blk cur, nxt;
  if (w < nKB) load_block<D>(cur, k, v, w, N, i, g);
  for (int kb = w; kb < nKB; kb += kWaves) {
    if (kb + kWaves < nKB) load_block<D>(nxt, k, v, kb + kWaves, N, i, g);  // next block in flight
    // S^T of the two 16-key halves: fp32 products in chunks of 4 k-steps (16
    // dimensions), each chunk accumulated from zero, the chunks added in fp64
    f64x4 sd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sd[h] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s0 = 0; s0 < KS; s0 += 4) {
        f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = s0; s < s0 + 4; ++s) part = mfma4(cur.kf[h][s], qf[s], part);
#pragma unroll
        for (int r = 0; r < 4; ++r) sd[h][r] += (double)part[r];
      }
    }
    // mask (keys past N; causal: keys after the query), scale to log2 units and round
    // to fp32 once, row maximum
    float st[2][4];
    float mt = -kInf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * kKB + 16 * h + 4 * g + r;
        const bool vis = key < N && (!CAUSAL || key <= qi);
        st[h][r] = vis ? (float)(sd[h][r] * c) : -kInf;
        mt = fmaxf(mt, st[h][r]);
      }
    mt = max4(mt);
    const float m_new = fmaxf(m, mt);
    // a row with no visible key so far keeps m = -inf, l = 0, O = 0
    const float alpha = m_new == -kInf ? 1.f : exp2_fast(m - m_new);
    const float sub = m_new == -kInf ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[h][r] = exp2_fast(st[h][r] - sub);  // masked: exp2(-inf) = 0
        rs += st[h][r];
      }
    l = l * alpha + sum4(rs);
    m = m_new;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      acc[b] *= alpha;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[b] = mfma4(cur.vf[h][r][b], st[h][r], acc[b]);
    }
    cur = nxt;
  }

  // ---- merge the four wavefronts' partial states
  if (g == 0) {
    s_m[w][i] = m;
    s_l[w][i] = l;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[w][i][16 * b + 4 * g + r] = acc[b][r];
  __syncthreads();
  // thread t: query t / 16, dimensions (t % 16) * D/16 .. + D/16 (the first 256 threads)
  const int tq = threadIdx.x / 16, td = (threadIdx.x % 16) * (D / 16);
  const int row = q0 + tq;
  if (tq < kQ && row < N) {
    float mm = -kInf;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) mm = fmaxf(mm, s_m[u][tq]);
    float a[kWaves], lt = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      a[u] = s_m[u][tq] == -kInf ? 0.f : exp2_fast(s_m[u][tq] - mm);
      lt = fmaf(a[u], s_l[u][tq], lt);
    }
    const float inv = 1.f / lt;
#pragma unroll
    for (int e = 0; e < D / 16; e += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        const float4 y = *reinterpret_cast<const float4*>(&s_o[u][tq][td + e]);
        x.x = fmaf(a[u], y.x, x.x), x.y = fmaf(a[u], y.y, x.y), x.z = fmaf(a[u], y.z, x.z), x.w = fmaf(a[u], y.w, x.w);
      }
      *reinterpret_cast<float4*>(o + base + (size_t)row * D + td + e) =
          make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
    }
    if (td == 0) lse[(size_t)bh * N + row] = (mm + log2_fast(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int nQB = (N + kQ - 1) / kQ;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(nQB * BH)), dim3(waves<D>() * 64), 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                     static_cast<float*>(a.o), a.lse, BH, N, nQB, (double)a.scale * 1.4426950408889634);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a) {
  if (a.d == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
