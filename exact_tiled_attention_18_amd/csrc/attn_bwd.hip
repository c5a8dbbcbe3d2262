// bf16 attention backward on gfx950 matrix cores: dQ, dK, dV from the saved LSE.
//
// The pages' motivating use is training (FlashAttention-2 wiki page,
// "Leistung und Effizienz": end-to-end training throughput; 16k-context
// training in the time of 8k), which needs the gradient of the attention
// output.  With S = scale * Q K^T, P = softmax(S) and O = P V, the gradients
// for an output gradient dO are
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// As in the forward pass, no N x N matrix is stored: P is recomputed tile by
// tile from the scores and the saved LSE, P = exp(scale * q.k - LSE).
//
// Three kernels, no atomics (the result is bitwise reproducible):
//   * delta:   D_i = rowsum(dO * O) in fp32 (one read of O and dO);
//   * dQ:      one workgroup per (256-query block, head), 8 wavefronts of 32
//              queries; K and V tiles of 32 keys through LDS.  As in the
//              forward kernel the scores are transposed (S^T = K Q^T, one query
//              per lane), with K's and V's rows permuted so that dS^T comes
//              out in the B-operand layout of dQ^T += K^T dS^T, K^T being read
//              with the transposing LDS read;
//   * dK, dV:  one workgroup per (128-key block, head), 4 wavefronts of 32
//              keys, the block's K and V held in registers; query tiles (Q,
//              dO, LSE, D) of 32 rows through LDS.  Here S = Q K^T keeps one
//              key per lane, with Q's and dO's rows permuted, so P and dS come
//              out as B operands of dV^T += dO^T P and dK^T += Q^T dS.
// Tiles are double-buffered: the next tile is loaded into registers while the
// current one is used, then written to the other buffer before the step's
// single barrier.
//
// A negative scale flips every sign bit of Q, a zero scale zeroes Q (the
// kernels then use the positive multiplier |scale| * log2(e)): dQ = scale *
// (dS K) and dK = |scale| * (dS^T Q') for the flipped Q', which are the
// gradients of the original problem.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kT = 32;  // rows per streamed tile (keys in dQ, queries in dK/dV)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ int permuted_row(int i) { return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC); }

__device__ __forceinline__ v4i16 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// register r of lane half g of a 32x32 accumulator computed with permuted A rows
// holds row (r & 7) + 8 g + 2 (r & 8) of the unpermuted operand
__device__ __forceinline__ int row_of_reg(int r, int g) { return (r & 7) + 8 * g + 2 * (r & 8); }

template <int D>
struct Tile {
  static constexpr int S = D * 2 + 64;         // row stride (bytes): conflict-free transposing reads
  static constexpr int BYTES = kT * S;
  static constexpr int PIECES = kT * D * 2 / 16;  // 16-byte pieces per tile
};

// 8 bf16 of row `row` of a tile, columns 16 ks + 8 g .. +7 (an A operand with
// permuted rows, or a row-major B operand)
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* tile, int row, int ks, int g) {
  return *reinterpret_cast<const bf16x8*>(tile + row * Tile<D>::S + ks * 32 + g * 16);
}

// the transposed A operand: rows d of block db, k = tile rows 16 mm + 8 g' .. +7
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, int tr_off, int db, int mm) {
  const char* pa = tile + tr_off + (mm * 16) * Tile<D>::S + db * 64;
  const v4i16 lo = tr_read(pa), hi = tr_read(pa + 4 * Tile<D>::S);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__device__ __forceinline__ int tr_offset(int lane) {
  const int grp16 = lane >> 4, l16 = lane & 15;
  return (8 * (grp16 >> 1) + (l16 >> 2)) * Tile<D>::S + (16 * (grp16 & 1) + 4 * (l16 & 3)) * 2;
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  uint4 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  w.z = pack_bf16x2(x[4], x[5]);
  w.w = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, w);
}

// stores of a transposed 32 x 32 accumulator block: lane (row l % 32) receives
// columns db * 32 + 8 a4 + 4 g .. +3 of its row
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* dst_row, const f32x16 (&acc)[D / 32], float mul, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      uint2 w;
      w.x = pack_bf16x2(acc[db][4 * a4 + 0] * mul, acc[db][4 * a4 + 1] * mul);
      w.y = pack_bf16x2(acc[db][4 * a4 + 2] * mul, acc[db][4 * a4 + 3] * mul);
      *reinterpret_cast<uint2*>(dst_row + db * 32 + 8 * a4 + 4 * g) = w;
    }
}

// ---------------------------------------------------------------- D = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
  constexpr int C = D / 4;  // columns per thread, four threads per row
  const int64_t row = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* po = o + row * D + part * C;
    const uint16_t* pd = dout + row * D + part * C;
#pragma unroll
    for (int i = 0; i < C; i += 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(po + i), b = *reinterpret_cast<const uint4*>(pd + i);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(bf16_lo(aw[j]), bf16_lo(bw[j]), acc);
        acc = fmaf(bf16_hi(aw[j]), bf16_hi(bw[j]), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v,
                                                     const uint16_t* __restrict__ dout,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     uint16_t* __restrict__ dq, int BH, int N, int nQB, float c,
                                                     float dq_mul, uint32_t qxor, uint32_t qand) {
  using T = Tile<D>;
  constexpr int DK = D / 16, DB = D / 32, kBr = 256;
  __shared__ __attribute__((aligned(16))) char smem[4 * T::BYTES];  // K and V, two buffers each
  // K buffers at 0 and BYTES, V buffers at 2 * BYTES and 3 * BYTES
  auto kbuf = [&](int b) { return smem + b * T::BYTES; };
  auto vbuf = [&](int b) { return smem + (2 + b) * T::BYTES; };

  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q0 = qblk * kBr;
  const int qi = q0 + (tid >> 6) * 32 + li;  // this lane's query

  constexpr int kRsrcWord3 = 0x00020000;
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k + base), (short)0, N * D * 2, kRsrcWord3);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v + base), (short)0, N * D * 2, kRsrcWord3);
  const bool copier = tid < T::PIECES;
  const int prow = (tid % T::PIECES) / (D / 8), pcol = (tid % (D / 8)) * 16;
  const int ld_off = prow * D * 2 + pcol, st_off = prow * T::S + pcol;
  const int krow = permuted_row(li);
  const int tr_off = tr_offset<D>(lane);

  bf16x8 qf[DK], df[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (qi < N) {
      a = *reinterpret_cast<const uint4*>(q + base + (size_t)qi * D + ks * 16 + g * 8);
      b = *reinterpret_cast<const uint4*>(dout + base + (size_t)qi * D + ks * 16 + g * 8);
    }
    a = make_uint4((a.x ^ qxor) & qand, (a.y ^ qxor) & qand, (a.z ^ qxor) & qand, (a.w ^ qxor) & qand);
    qf[ks] = __builtin_bit_cast(bf16x8, a);
    df[ks] = __builtin_bit_cast(bf16x8, b);
  }
  const float lse2 = qi < N ? lse[(size_t)bh * N + qi] * kLog2e : 0.f;
  const float dd = qi < N ? delta[(size_t)bh * N + qi] : 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
  const int nT = (kv_end + kT - 1) / kT;
  uint4 sk = make_uint4(0, 0, 0, 0), sv = sk;
  if (copier) {
    sk = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, ld_off, 0, 0));
    sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, ld_off, 0, 0));
    *reinterpret_cast<uint4*>(kbuf(0) + st_off) = sk;
    *reinterpret_cast<uint4*>(vbuf(0) + st_off) = sv;
  }
  __syncthreads();
  for (int t = 0; t < nT; ++t) {
    const int cur = t & 1;
    if (copier && t + 1 < nT) {
      sk = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, ld_off + (t + 1) * kT * D * 2, 0, 0));
      sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, ld_off + (t + 1) * kT * D * 2, 0, 0));
    }
    // S^T = K Q'^T and dP^T = V dO^T, one query per lane
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      st = mfma(read_row<D>(kbuf(cur), krow, ks, g), qf[ks], st);
      dpt = mfma(read_row<D>(vbuf(cur), krow, ks, g), df[ks], dpt);
    }
    // dS^T = P^T * (dP^T - D), keys masked where not visible
    float ds[16];
    const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - t * kT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = row_of_reg(r, g) <= lim ? exp2_fast(fmaf(st[r], c, -lse2)) : 0.f;
      ds[r] = p * (dpt[r] - dd);
    }
    const bf16x8 db0 = pack8(ds), db1 = pack8(ds + 8);
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = mfma(read_tr<D>(kbuf(cur), tr_off, db, 0), db0, acc[db]);
      acc[db] = mfma(read_tr<D>(kbuf(cur), tr_off, db, 1), db1, acc[db]);
    }
    if (copier && t + 1 < nT) {
      *reinterpret_cast<uint4*>(kbuf(cur ^ 1) + st_off) = sk;
      *reinterpret_cast<uint4*>(vbuf(cur ^ 1) + st_off) = sv;
    }
    __syncthreads();
  }
  if (qi < N) store_rows<D>(dq + base + (size_t)qi * D, acc, dq_mul, g);
}

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int BH, int N, float c, float dk_mul, uint32_t qxor,
    uint32_t qand) {
  using T = Tile<D>;
  constexpr int DK = D / 16, DB = D / 32, kBk = 128;
  constexpr int kPer = T::PIECES / 256;  // 16-byte pieces per thread and operand tile (1 or 2)
  __shared__ __attribute__((aligned(16))) char smem[4 * T::BYTES];          // Q' and dO, two buffers each
  __shared__ __attribute__((aligned(16))) float stat[2][2][kT];              // [buffer][LSE*log2e, D][row]
  // Q' buffers at 0 and BYTES, dO buffers at 2 * BYTES and 3 * BYTES
  auto qbuf = [&](int b) { return smem + b * T::BYTES; };
  auto dbuf = [&](int b) { return smem + (2 + b) * T::BYTES; };

  const int L = blockIdx.x;
  const int kblk = L / BH;  // smallest key blocks (most causal work) first
  const int bh = L % BH;
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int k0 = kblk * kBk;
  const int kj = k0 + (tid >> 6) * 32 + li;  // this lane's key

  constexpr int kRsrcWord3 = 0x00020000;
  const auto qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(q + base), (short)0, N * D * 2, kRsrcWord3);
  const auto drs = __builtin_amdgcn_make_buffer_rsrc((void*)(dout + base), (short)0, N * D * 2, kRsrcWord3);
  int ld_off[kPer], st_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int piece = tid + 256 * i;
    const int prow = piece / (D / 8), pcol = (piece % (D / 8)) * 16;
    ld_off[i] = prow * D * 2 + pcol;
    st_off[i] = prow * T::S + pcol;
  }
  const int qrow = permuted_row(li);
  const int tr_off = tr_offset<D>(lane);

  bf16x8 kf[DK], vf[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (kj < N) {
      a = *reinterpret_cast<const uint4*>(k + base + (size_t)kj * D + ks * 16 + g * 8);
      b = *reinterpret_cast<const uint4*>(v + base + (size_t)kj * D + ks * 16 + g * 8);
    }
    kf[ks] = __builtin_bit_cast(bf16x8, a);
    vf[ks] = __builtin_bit_cast(bf16x8, b);
  }
  f32x16 dva[DB], dka[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dva[db][r] = dka[db][r] = 0.f;

  // query tiles that see any key of the block
  const int t0 = CAUSAL ? k0 / kT : 0;
  const int nQT = (N + kT - 1) / kT;
  uint4 sq[kPer], sd[kPer];
  float sstat = 0.f;
  auto load = [&](int t) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qrs, ld_off[i] + t * kT * D * 2, 0, 0));
      sq[i] = make_uint4((a.x ^ qxor) & qand, (a.y ^ qxor) & qand, (a.z ^ qxor) & qand, (a.w ^ qxor) & qand);
      sd[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(drs, ld_off[i] + t * kT * D * 2, 0, 0));
    }
    if (tid < 2 * kT) {
      const int row = t * kT + (tid & (kT - 1));
      sstat = row < N ? (tid < kT ? lse[(size_t)bh * N + row] * kLog2e : delta[(size_t)bh * N + row]) : 0.f;
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      *reinterpret_cast<uint4*>(qbuf(b) + st_off[i]) = sq[i];
      *reinterpret_cast<uint4*>(dbuf(b) + st_off[i]) = sd[i];
    }
    if (tid < 2 * kT) stat[b][tid / kT][tid & (kT - 1)] = sstat;
  };
  if (t0 < nQT) {
    load(t0);
    store(0);
  }
  __syncthreads();
  for (int t = t0; t < nQT; ++t) {
    const int cur = (t - t0) & 1;
    if (t + 1 < nQT) load(t + 1);
    // S = Q' K^T and dP = dO V^T, one key per lane
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      s = mfma(read_row<D>(qbuf(cur), qrow, ks, g), kf[ks], s);
      dp = mfma(read_row<D>(dbuf(cur), qrow, ks, g), vf[ks], dp);
    }
    // LSE and D of this lane's 16 queries (two runs of 8)
    float ls[16], dl[16];
    {
      const float4* sl = reinterpret_cast<const float4*>(&stat[cur][0][0]);
      const float4* sdl = reinterpret_cast<const float4*>(&stat[cur][1][0]);
      const float4 a0 = sl[2 * g], a1 = sl[2 * g + 1], a2 = sl[4 + 2 * g], a3 = sl[5 + 2 * g];
      const float4 b0 = sdl[2 * g], b1 = sdl[2 * g + 1], b2 = sdl[4 + 2 * g], b3 = sdl[5 + 2 * g];
      const float av[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                            a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
      const float bv[16] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w,
                            b2.x, b2.y, b2.z, b2.w, b3.x, b3.y, b3.z, b3.w};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        ls[r] = av[r];
        dl[r] = bv[r];
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = t * kT + row_of_reg(r, g);
      const bool vis = qr < N && kj < N && (!CAUSAL || kj <= qr);
      p[r] = vis ? exp2_fast(fmaf(s[r], c, -ls[r])) : 0.f;
      ds[r] = p[r] * (dp[r] - dl[r]);
    }
    const bf16x8 pb0 = pack8(p), pb1 = pack8(p + 8), sb0 = pack8(ds), sb1 = pack8(ds + 8);
    // dV^T += dO^T P and dK^T += Q'^T dS
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dva[db] = mfma(read_tr<D>(dbuf(cur), tr_off, db, 0), pb0, dva[db]);
      dva[db] = mfma(read_tr<D>(dbuf(cur), tr_off, db, 1), pb1, dva[db]);
      dka[db] = mfma(read_tr<D>(qbuf(cur), tr_off, db, 0), sb0, dka[db]);
      dka[db] = mfma(read_tr<D>(qbuf(cur), tr_off, db, 1), sb1, dka[db]);
    }
    if (t + 1 < nQT) store(cur ^ 1);
    __syncthreads();
  }
  if (kj < N) {
    store_rows<D>(dv + base + (size_t)kj * D, dva, 1.f, g);
    store_rows<D>(dk + base + (size_t)kj * D, dka, dk_mul, g);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const BwdArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const int64_t rows = (int64_t)BH * N;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* o = static_cast<const uint16_t*>(a.o);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, a.stream, o, dout,
                     a.delta, rows);
  const float c = a.scale == 0.f ? 1.f : fabsf(a.scale) * kLog2e;
  const uint32_t qxor = a.scale < 0.f ? 0x80008000u : 0u;
  const uint32_t qand = a.scale == 0.f ? 0u : 0xFFFFFFFFu;
  const int nQB = (N + 255) / 256;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nQB * BH)), dim3(512), 0, a.stream, q, k, v, dout,
                     a.lse, a.delta, static_cast<uint16_t*>(a.dq), BH, N, nQB, c, a.scale, qxor, qand);
  const int nKB = (N + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nKB * BH)), dim3(256), 0, a.stream, q, k, v,
                     dout, a.lse, a.delta, static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), BH, N, c,
                     fabsf(a.scale), qxor, qand);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_d<64, true>(a) : launch_d<64, false>(a);
  return a.causal ? launch_d<128, true>(a) : launch_d<128, false>(a);
}

}  // namespace fa
