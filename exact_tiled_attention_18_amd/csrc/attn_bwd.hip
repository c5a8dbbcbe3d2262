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
// Two kernels, no atomics (the result is bitwise reproducible):
//   * dQ:      one workgroup per (256-query block, head), 8 wavefronts of 32
//              queries; K and V tiles of 32 keys through LDS.  Its prologue also
//              forms D_i = rowsum(dO * O) in fp32 for its queries, from the dO
//              row it loads anyway and one read of the O row, and writes D for
//              the dK/dV kernel, which runs after it.  As in the
//              forward kernel the scores are transposed (S^T = K Q^T, one query
//              per lane), with K's and V's rows permuted so that dS^T comes
//              out in the B-operand layout of dQ^T += K^T dS^T, K^T being read
//              with the transposing LDS read;
//   * dK, dV:  one workgroup per (128-key block, head), the block's K and V held
//              in registers, 32 keys per wavefront; query tiles (Q, dO, LSE, D)
//              of 32 rows through LDS.  Here S = Q K^T keeps one key per lane,
//              with Q's and dO's rows permuted, so P and dS come out as B
//              operands of dV^T += dO^T P and dK^T += Q^T dS.
// The dQ kernel, and the dK/dV kernel at d = 128, are software-pipelined: each step
// interleaves the score MFMAs of the next tile, the gradient MFMAs of an earlier one
// and the vector work of the current one.  At d = 128 the dK/dV work of each 32
// keys is split between two wavefronts on one SIMD (K, S, P, dV on one side; V, dP,
// dS, dK on the other, P passed through LDS).  At d = 64 the dK/dV kernel is the
// plain loop of 4 wavefronts, two per SIMD: tiles double-buffered, the next one
// loaded into registers while the current one is used, then written to the other
// buffer before the step's single barrier.
//
// A negative scale flips every sign bit of Q, a zero scale zeroes Q (the
// kernels then use the positive multiplier |scale| * log2(e)): dQ = scale *
// (dS K) and dK = |scale| * (dS^T Q') for the flipped Q', which are the
// gradients of the original problem.  The d = 128 dK/dV kernel instead takes Q
// unchanged with the signed multiplier scale * log2(e) and dK = scale * (dS^T Q),
// the same products with the sign moved out of the operand.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kT = 32;  // rows per streamed tile (keys in dQ, queries in dK/dV)

// Work item L -> (block, head) when every block of a launch costs the same (non-causal,
// B*H a multiple of 8): workgroup ids go to the 8 XCDs in turn, and within an XCD the
// blocks of a head are consecutive, so they run together and share the head's data in
// that XCD's L2.
__device__ __forceinline__ void grouped_item(int L, int BH, int nblk, int& blk, int& bh) {
  const int slot = L / 8;
  blk = slot % nblk;
  bh = (slot / nblk) * 8 + L % 8;
}

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

// LDS operand tiles: kT rows of S bytes.  A tile is read both ways: as rows
// (16-byte reads, 16 lanes on 16 different rows) and transposed (ds_read_b64_tr_b16,
// 8 lanes on each of 4 consecutive rows, 64 bytes of each).  The stride S = 2 D + 64
// puts 4 consecutive rows in 4 different 16-bank windows, which the transposed reads
// need; rows 4 apart then share a window, so the 16-byte piece p of row R is stored
// at piece p ^ swz(R), swz(R) = (R >> 2) & 3: the 4 rows that share a window use 4
// different 4-bank slots of it, and both kinds of read are free of bank conflicts.
// (The plain layout had 4-way conflicts on every row read: 2.8e7 conflict cycles per
// launch in each of the d = 128 gradient kernels at B4 H16 N2048.)
template <int D>
struct Tile {
  static constexpr int S = D * 2 + 64;         // row stride (bytes)
  static constexpr int BYTES = kT * S;
  static constexpr int PIECES = kT * D * 2 / 16;  // 16-byte pieces per tile
};

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// byte offset of 16-byte piece `piece` of row `row`
template <int D>
__device__ __forceinline__ int piece_off(int row, int piece) {
  return row * Tile<D>::S + ((piece ^ swz(row)) << 4);
}

// A lane's row reads: pieces 2 ks + g of one row.  With c = swz(row), piece
// (2 ks + g) ^ c lies at byte 32 ks + 32 c1 + 16 (g ^ c0) for even ks and at
// 32 ks - 32 c1 + 16 (g ^ c0) for odd ks (c = 2 c1 + c0), so each parity has a
// per-lane base and ks stays a constant offset.
struct RowRd {
  int even, odd;
};
template <int D>
__device__ __forceinline__ RowRd row_reader(int row, int g) {
  const int c = swz(row), b = row * Tile<D>::S + 16 * (g ^ (c & 1));
  return RowRd{b + 32 * (c >> 1), b - 32 * (c >> 1)};
}

// 8 bf16 of the lane's row, columns 16 ks + 8 g .. +7 (an A operand with permuted
// rows, or a row-major B operand)
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* tile, const RowRd& rr, int ks) {
  return *reinterpret_cast<const bf16x8*>(tile + ((ks & 1) ? rr.odd : rr.even) + ks * 32);
}

// A lane's transposed reads: lane k of each 16-lane group points at row
// 8 (group / 2) + k / 4 (and 4 rows further for the second half), 8 bytes at column
// byte 32 (group % 2) + 8 (k % 4) of a 64-byte window; the swizzle moves pieces
// within the window only, so the window (db) and the 16-row step (mm) stay
// constant offsets.
struct TrRd {
  int lo, hi;
};
template <int D>
__device__ __forceinline__ TrRd tr_reader(int lane) {
  const int grp16 = lane >> 4, l16 = lane & 15;
  const int r = 8 * (grp16 >> 1) + (l16 >> 2), q = 2 * (grp16 & 1) + ((l16 & 3) >> 1), h = 8 * (l16 & 1);
  return TrRd{r * Tile<D>::S + 16 * (q ^ swz(r)) + h, (r + 4) * Tile<D>::S + 16 * (q ^ swz(r + 4)) + h};
}

// the transposed A operand: rows d of block db, k = tile rows 16 mm + 8 g' .. +7
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, const TrRd& tr, int db, int mm) {
  const char* pa = tile + (mm * 16) * Tile<D>::S + db * 64;
  const v4i16 lo = tr_read(pa + tr.lo), hi = tr_read(pa + tr.hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  uint4 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  w.z = pack_bf16x2(x[4], x[5]);
  w.w = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, w);
}

// stores of transposed 32 x 32 accumulator blocks: lane (row l % 32) receives
// columns db * 32 .. db * 32 + 31 of its row
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* dst_row, const f32x16 (&acc)[D / 32], float mul, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) store_row_bf16(dst_row + db * 32, acc[db], mul, g);
}

// ---------------------------------------------------------------- dQ
// Software pipeline over key tiles: step t issues the MFMAs
// of S^T_{t+1} = K_{t+1} Q'^T and dP^T_{t+1} = V_{t+1} dO^T, the MFMAs of
// dQ^T += K_{t-1}^T dS^T_{t-1}, and the vector work that turns S^T_t, dP^T_t into
// dS^T_t.  Four K/V buffers hold tiles t-1 .. t+2.  To stay within two wavefronts
// per SIMD, dO (the B operand of dP^T, the same for every tile) is kept in LDS
// for the whole workgroup instead of in registers.
template <int D, bool CAUSAL>
struct DqPipe {
  using T = Tile<D>;
  static constexpr int DK = D / 16, DB = D / 32, NB = 4;
  static constexpr int EPC = 16 / DK;     // score elements per chunk (2)
  static constexpr int DS = D * 2 + 16;   // dO row stride (bytes): conflict-free 16-byte row reads
  static_assert(DK == 2 * DB, "one dQ operand per chunk");

  bf16x8 qf[DK];
  f32x16 acc[DB];
  f32x16 st[2], dpt[2];     // S^T and dP^T of tiles t (parity B) and t+1
  uint32_t dsw[2][8];       // dS^T (bf16 pairs) of tiles t (parity B) and t-1
  bf16x8 opk[2], opv[2], opd[2], opt[2];  // operands of the next chunk
  uint4 sk, sv;
  char* kv;     // K buffers at 0 .. NB-1, V buffers at NB .. 2 NB - 1 (BYTES each)
  char* dos;    // dO rows of the workgroup's queries, stride DS
  __amdgpu_buffer_rsrc_t krs, vrs;
  int N, g, li, qi, qloc, ld_off, st_off;
  RowRd krow;
  TrRd tr_off;
  bool copier;
  float c, lse2, dd;

  __device__ __forceinline__ char* kbuf(int b) const { return kv + b * T::BYTES; }
  __device__ __forceinline__ char* vbuf(int b) const { return kv + (NB + b) * T::BYTES; }
  __device__ __forceinline__ void load(int t) {
    if (!copier) return;
    sk = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, ld_off + t * kT * D * 2, 0, 0));
    sv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, ld_off + t * kT * D * 2, 0, 0));
  }
  __device__ __forceinline__ void store(int b) {
    if (!copier) return;
    *reinterpret_cast<uint4*>(kbuf(b) + st_off) = sk;
    *reinterpret_cast<uint4*>(vbuf(b) + st_off) = sv;
  }
  __device__ __forceinline__ void read_sdp(int slot, int ch, int bn) {
    opk[slot] = read_row<D>(kbuf(bn), krow, ch);
    opv[slot] = read_row<D>(vbuf(bn), krow, ch);
    opd[slot] = *reinterpret_cast<const bf16x8*>(dos + qloc * DS + ch * 32 + g * 16);
  }
  __device__ __forceinline__ void read_kt(int slot, int ch, int bo) {
    opt[slot] = read_tr<D>(kbuf(bo), tr_off, ch % DB, ch / DB);
  }
  __device__ __forceinline__ bf16x8 word8(const uint32_t (&w)[8], int mm) const {
    return __builtin_bit_cast(bf16x8, make_uint4(w[4 * mm], w[4 * mm + 1], w[4 * mm + 2], w[4 * mm + 3]));
  }
  // dS^T of score elements [e0, e0 + EPC) of tile t (parity B); without G every key
  // of the tile is visible to every query of the workgroup
  template <int B, bool G>
  __device__ __forceinline__ void grad_slice(int lim, int e0) {
#pragma unroll
    for (int e = e0; e < e0 + EPC; e += 2) {
      float d2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = e + h;
        const float pr = !G || row_of_reg(r, g) <= lim ? exp2_fast(fmaf(st[B][r], c, -lse2)) : 0.f;
        d2[h] = pr * (dpt[B][r] - dd);
      }
      dsw[B][e >> 1] = pack_bf16x2(d2[0], d2[1]);
      // a use of the packed result in this chunk, so that the compiler does not sink the
      // work towards its use in the next step (and spill on the way)
      asm volatile("" ::"v"(dsw[B][e >> 1]));
    }
  }
  template <int B, bool G = true>
  __device__ __forceinline__ void step(int t, int cur, int qlim) {
    const int bn = (cur + 1) % NB, bo = (cur + NB - 1) % NB, bw = (cur + 2) % NB;
    const int lim = qlim - t * kT;  // last visible key of this lane's query, relative to tile t
    read_sdp(0, 0, bn);
#pragma unroll
    for (int r = 0; r < 16; ++r) st[B ^ 1][r] = dpt[B ^ 1][r] = 0.f;
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      if (ch + 1 < DK) {
        read_sdp((ch + 1) & 1, ch + 1, bn);
        read_kt((ch + 1) & 1, ch + 1, bo);
      } else {
        read_kt(0, 0, cur);  // the next step's chunk 0: K^T of tile t
      }
      const int sl = ch & 1, db = ch % DB, mm = ch / DB;
      acc[db] = mfma(opt[sl], word8(dsw[B ^ 1], mm), acc[db]);
      st[B ^ 1] = mfma(opk[sl], qf[ch], st[B ^ 1]);
      dpt[B ^ 1] = mfma(opv[sl], opd[sl], dpt[B ^ 1]);
      grad_slice<B, G>(lim, ch * EPC);
      if (ch == 1) store(bw);
      if (ch == 2) load(t + 3);  // past the last tile: zeros or unused keys, never read
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 100, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);  // DS writes
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);  // VMEM reads
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
  template <int B>
  __device__ __forceinline__ void last(int b) {
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      const int db = ch % DB, mm = ch / DB;
      const bf16x8 a = ch == 0 ? opt[0] : read_tr<D>(kbuf(b), tr_off, db, mm);
      acc[db] = mfma(a, word8(dsw[B], mm), acc[db]);
    }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dq_pipe_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const uint16_t* __restrict__ o,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ delta,
                                                          uint16_t* __restrict__ dq, int BH, int N, int nQB, float c,
                                                          float dq_mul, uint32_t qxor, uint32_t qand) {
  using W = DqPipe<D, CAUSAL>;
  using T = Tile<D>;
  constexpr int DK = W::DK, NB = W::NB, kBr = 256;
  __shared__ __attribute__((aligned(16))) char kv[2 * NB * T::BYTES];
  __shared__ __attribute__((aligned(16))) char dos[kBr * W::DS];

  W w;
  const int L = blockIdx.x;
  int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  int bh = L % BH;
  if (!CAUSAL && BH % 8 == 0) grouped_item(L, BH, nQB, qblk, bh);
  const size_t base = (size_t)bh * N * D;
  const int tid = threadIdx.x, lane = tid & 63;
  w.g = lane >> 5;
  w.li = lane & 31;
  const int q0 = qblk * kBr;
  w.qloc = (tid >> 6) * 32 + w.li;
  w.qi = q0 + w.qloc;  // this lane's query
  w.N = N;
  w.c = c;
  w.kv = kv;
  w.dos = dos;
  constexpr int kRsrcWord3 = 0x00020000;
  w.krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k + base), (short)0, N * D * 2, kRsrcWord3);
  w.vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v + base), (short)0, N * D * 2, kRsrcWord3);
  w.copier = tid < T::PIECES;
  const int prow = (tid % T::PIECES) / (D / 8), pcol = (tid % (D / 8)) * 16;
  w.ld_off = prow * D * 2 + pcol;
  w.st_off = piece_off<D>(prow, pcol / 16);
  w.krow = row_reader<D>(permuted_row(w.li), w.g);
  w.tr_off = tr_reader<D>(lane);

  // this lane's query: Q' fragments in registers, its dO row halves into LDS, and
  // D = rowsum(dO * O) over the lane's half of the row (the columns of its Q and dO
  // fragments) plus the partner lane's half
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), b = a, ov = a;
    if (w.qi < N) {
      a = *reinterpret_cast<const uint4*>(q + base + (size_t)w.qi * D + ks * 16 + w.g * 8);
      b = *reinterpret_cast<const uint4*>(dout + base + (size_t)w.qi * D + ks * 16 + w.g * 8);
      ov = *reinterpret_cast<const uint4*>(o + base + (size_t)w.qi * D + ks * 16 + w.g * 8);
    }
    a = make_uint4((a.x ^ qxor) & qand, (a.y ^ qxor) & qand, (a.z ^ qxor) & qand, (a.w ^ qxor) & qand);
    w.qf[ks] = __builtin_bit_cast(bf16x8, a);
    *reinterpret_cast<uint4*>(dos + w.qloc * W::DS + ks * 32 + w.g * 16) = b;
    const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dpart = fmaf(bf16_lo(ow[j]), bf16_lo(bw[j]), dpart);
      dpart = fmaf(bf16_hi(ow[j]), bf16_hi(bw[j]), dpart);
    }
  }
  w.dd = sum_pair(dpart);  // 0 for rows past N
  if (w.qi < N && w.g == 0) delta[(size_t)bh * N + w.qi] = w.dd;
  w.lse2 = w.qi < N ? lse[(size_t)bh * N + w.qi] * kLog2e : 0.f;
#pragma unroll
  for (int db = 0; db < W::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.acc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
  const int nT = (kv_end + kT - 1) / kT;
  const int qlim = CAUSAL ? min(w.qi, N - 1) : N - 1;
  if (nT > 0) {
    // prologue: tiles 0 and 1 into buffers 0 and 1; K buffer 3 (tile -1 of the first
    // step's dQ products) zeroed along with dS^T_{-1}; S^T_0, dP^T_0
    w.load(0);
    w.store(0);
    w.load(1);
    w.store(1);
    for (int i = tid; i < T::BYTES / 16; i += 512) *reinterpret_cast<uint4*>(w.kbuf(3) + 16 * i) = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) w.dsw[1][i] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) w.st[0][r] = w.dpt[0][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      w.st[0] = mfma(read_row<D>(w.kbuf(0), w.krow, ks), w.qf[ks], w.st[0]);
      w.dpt[0] = mfma(read_row<D>(w.vbuf(0), w.krow, ks),
                      *reinterpret_cast<const bf16x8*>(dos + w.qloc * W::DS + ks * 32 + w.g * 16), w.dpt[0]);
    }
    w.load(2);
    w.read_kt(0, 0, 3);
    int t = 0;
    // four steps per iteration (two parities times the four buffers): buffer indices
    // are constants, so LDS addresses fold into instruction offsets
    // key tiles [0, tf) lie wholly at or before the workgroup's first query (and below
    // N): they skip the per-element visibility test
    const int tf = ((CAUSAL ? min(q0, N - 1) : N - 1) + 1) / kT;
    auto quad = [&](auto guard) {
      constexpr bool G = decltype(guard)::value;
      w.template step<0, G>(t, 0, qlim);
      w.template step<1, G>(t + 1, 1, qlim);
      w.template step<0, G>(t + 2, 2, qlim);
      w.template step<1, G>(t + 3, 3, qlim);
    };
    for (; t + 3 < tf; t += 4) quad(std::false_type{});
    for (; t + 3 < nT; t += 4) quad(std::true_type{});
    for (; t + 1 < nT; t += 2) {
      w.template step<0>(t, t % NB, qlim);
      w.template step<1>(t + 1, (t + 1) % NB, qlim);
    }
    if (t < nT) {
      w.template step<0>(t, t % NB, qlim);
      w.template last<0>(t % NB);
    } else {
      w.template last<1>((t - 1) % NB);
    }
  }
  if (w.qi < N) store_rows<D>(dq + base + (size_t)w.qi * D, w.acc, dq_mul, w.g);
}

// ---------------------------------------------------------------- dK, dV
// two wavefronts per SIMD (stated, so that the compiler budgets 256 registers per
// wavefront): it then keeps every accumulator in VGPRs and uses the VGPR forms of the
// MFMAs.  Without the bound it put S, dP, dK and dV in accumulation registers and
// copied them out and back, 96 of the step's 330 vector instructions.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
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
  int kblk = L / BH;  // smallest key blocks (most causal work) first
  int bh = L % BH;
  if (!CAUSAL && BH % 8 == 0) grouped_item(L, BH, (int)(gridDim.x / BH), kblk, bh);
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
    st_off[i] = piece_off<D>(prow, pcol / 16);
  }
  const RowRd qrow = row_reader<D>(permuted_row(li), g);
  const TrRd tr_off = tr_reader<D>(lane);

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
    // every wavefront loads the tile's 2 kT statistics (lane i: LSE for i < kT, D
    // otherwise); rows past N repeat row N - 1, which only invisible queries use
    const int i = tid & (2 * kT - 1);
    const int row = min(t * kT + (i & (kT - 1)), N - 1);
    const float* src = (i < kT ? lse : delta) + (size_t)bh * N;
    sstat = src[row] * (i < kT ? kLog2e : 1.f);
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      *reinterpret_cast<uint4*>(qbuf(b) + st_off[i]) = sq[i];
      *reinterpret_cast<uint4*>(dbuf(b) + st_off[i]) = sd[i];
    }
    const int i = tid & (2 * kT - 1);  // the four wavefronts store the same values
    stat[b][i / kT][i & (kT - 1)] = sstat;
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
      s = mfma(read_row<D>(qbuf(cur), qrow, ks), kf[ks], s);
      dp = mfma(read_row<D>(dbuf(cur), qrow, ks), vf[ks], dp);
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
    // a tile below N that lies wholly after every key of a block below N sees all of them
    const bool full = (t + 1) * kT <= N && k0 + kBk <= N && (!CAUSAL || k0 + kBk <= t * kT + 1);
    if (full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2_fast(fmaf(s[r], c, -ls[r]));
        ds[r] = p[r] * (dp[r] - dl[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = t * kT + row_of_reg(r, g);
        const bool vis = qr < N && kj < N && (!CAUSAL || kj <= qr);
        p[r] = vis ? exp2_fast(fmaf(s[r], c, -ls[r])) : 0.f;
        ds[r] = p[r] * (dp[r] - dl[r]);
      }
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

// ---------------------------------------------------------------- dK, dV (d = 128): wavefront pairs
// Eight wavefronts, two per SIMD.  Wavefront w < 4 (the P side) and wavefront w + 4 (the
// dS side) share the 32 keys 32 w .. 32 w + 31 of the block.  The P side holds K and dV:
// it computes S = Q K^T, turns S into P and accumulates dV^T += dO^T P.  The dS side holds
// V and dK: it computes dP = dO V^T, takes P from the P side through LDS in fp32 (the
// values the P side rounds to bf16 for dV, so dS is what one wavefront doing both would
// form), forms dS = P (dP - D) and accumulates dK^T += Q^T dS.  Each side keeps about half the state of one wavefront doing
// both, so each fits the 256 registers that two wavefronts per SIMD allow, and every SIMD
// runs one wavefront of each side, whose MFMAs and vector work overlap.  Step t:
//   P side:  MFMAs of S_{t+1} = Q_{t+1} K^T and dV += dO_{t-1}^T P_{t-1}; vector work
//            P_t from S_t, written to LDS;
//   dS side: MFMAs of dP_t = dO_t V^T and dK += Q_{t-2}^T dS_{t-2}; vector work dS_{t-1}
//            from P_{t-1} (written in step t-1) and dP_{t-1}.
// Six LDS buffers hold tiles t-2 .. t+3 (tile t+2 is written in step t).  After the last
// step each side finishes the products it still owes (dV of the last tile; dS of the last
// tile and dK of the last two), without further barriers.
template <int D, bool CAUSAL>
struct DkDvPair {
  using T = Tile<D>;
  static constexpr int DK = D / 16, DB = D / 32, NB = 6;
  static constexpr int EPC = 16 / DK;  // score elements per chunk
  static_assert(DK == 8 && EPC == 2, "written for d = 128");
  static_assert(T::PIECES == 512, "one 16-byte piece per thread and operand tile");

  // both sides
  char* smem;
  float* stat;  // [NB][2][kT]: LSE * log2(e), D
  float4* xp;   // [4 key groups][2 parities][4][64 lanes]: P of one tile, fp32
  __amdgpu_buffer_rsrc_t qrs, drs;
  const float* lse_h;
  const float* delta_h;
  int N, tid, g, li, kj, kg, lane;
  RowRd qrow;
  TrRd tr_off;
  int ld_off, st_off;
  uint4 sq, sd;
  float sstat;
  float c;  // scale * log2(e), signed: Q enters unchanged
  // P side
  bf16x8 kf[DK];
  f32x16 dva[DB];
  f32x16 s[2];          // S of tiles t (parity B) and t+1
  uint32_t pw[2][8];    // P (bf16 pairs) of tiles t (parity B) and t-1
  bf16x8 opq[2], opv[2];
  float ls[16];
  float4 pout;          // four P values on their way to LDS
  // dS side
  bf16x8 vf[DK];
  f32x16 dka[DB];
  f32x16 dp[2];         // dP of tiles t (parity B) and t-1
  uint32_t sw[2][8];    // dS (bf16 pairs) of tiles t-1 (parity B) and t-2
  bf16x8 opd[2], opk[2];
  float dl[16];
  float4 pin[4];        // P of tile t-1, from LDS

  __device__ __forceinline__ char* qbuf(int b) const { return smem + b * T::BYTES; }
  __device__ __forceinline__ char* dbuf(int b) const { return smem + (NB + b) * T::BYTES; }
  __device__ __forceinline__ float4* xslot(int par, int i) const { return xp + ((kg * 2 + par) * 4 + i) * 64 + lane; }

  __device__ __forceinline__ void load(int t) {
    sq = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qrs, ld_off + t * kT * D * 2, 0, 0));
    sd = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(drs, ld_off + t * kT * D * 2, 0, 0));
    // every wavefront loads the tile's 2 kT statistics (lane i: LSE for i < kT, D
    // otherwise); rows past N repeat row N - 1, which only invisible queries use
    const int i = tid & (2 * kT - 1);
    const int row = min(t * kT + (i & (kT - 1)), N - 1);
    const float* src = i < kT ? lse_h : delta_h;
    sstat = src[row] * (i < kT ? kLog2e : 1.f);
  }
  __device__ __forceinline__ void store(int b) {
    *reinterpret_cast<uint4*>(qbuf(b) + st_off) = sq;
    *reinterpret_cast<uint4*>(dbuf(b) + st_off) = sd;
    const int i = tid & (2 * kT - 1);  // the eight wavefronts store the same values
    stat[(b * 2 + i / kT) * kT + (i & (kT - 1))] = sstat;
  }
  // statistic st (0: LSE, 1: D) of half h of this lane's 16 queries (the queries
  // 8 h .. 8 h + 7 of each of its two runs of 8) of the tile in buffer b
  __device__ __forceinline__ void read_stat_half(float (&dst)[16], int b, int st, int h) const {
    const float4* sl = reinterpret_cast<const float4*>(stat + (b * 2 + st) * kT);
    const float4 a0 = sl[4 * h + 2 * g], a1 = sl[4 * h + 2 * g + 1];
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int r = 0; r < 8; ++r) dst[8 * h + r] = av[r];
  }
  __device__ __forceinline__ bf16x8 word8(const uint32_t (&w)[8], int mm) const {
    return __builtin_bit_cast(bf16x8, make_uint4(w[4 * mm], w[4 * mm + 1], w[4 * mm + 2], w[4 * mm + 3]));
  }
  __device__ __forceinline__ void chunk_schedule() const {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 100, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);  // DS writes
    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);  // VMEM reads
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- P side, step t (tile t in buffer cur, parity B = (t - t0) & 1); the dV operand
  // of chunk 0 was read by the previous step, S_{t+1}'s after the barrier
  template <int B, bool G>
  __device__ __forceinline__ void step_p(int t, int cur) {
    const int bn = (cur + 1) % NB, bo = (cur + NB - 1) % NB, bw = (cur + 2) % NB;
    opq[0] = read_row<D>(qbuf(bn), qrow, 0);
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      if (ch + 1 < DK) {
        opq[(ch + 1) & 1] = read_row<D>(qbuf(bn), qrow, ch + 1);
        opv[(ch + 1) & 1] = read_tr<D>(dbuf(bo), tr_off, (ch + 1) % DB, (ch + 1) / DB);
      } else {
        opv[0] = read_tr<D>(dbuf(cur), tr_off, 0, 0);  // the next step's chunk 0: dO^T of tile t
      }
      const int sl = ch & 1, db = ch % DB, mm = ch / DB;
      dva[db] = mfma(opv[sl], word8(pw[B ^ 1], mm), dva[db]);
      s[B ^ 1] = mfma(opq[sl], kf[ch], ch == 0 ? f32x16{} : s[B ^ 1]);
      // P of score elements 2 ch, 2 ch + 1 of tile t
      float p2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * ch + h;
        const int qr = t * kT + row_of_reg(r, g);
        const bool vis = !G || (qr < N && kj < N && (!CAUSAL || kj <= qr));
        float sv = s[B][r];
        asm volatile("" : "+v"(sv));  // keeps this element's work in its chunk
        p2[h] = vis ? exp2_fast(fmaf(sv, c, -ls[r])) : 0.f;
      }
      pw[B][ch] = pack_bf16x2(p2[0], p2[1]);
      if (ch & 1) {
        pout.z = p2[0];
        pout.w = p2[1];
        *xslot(B, ch >> 1) = pout;
      } else {
        pout.x = p2[0];
        pout.y = p2[1];
      }
      asm volatile("" ::"v"(pw[B][ch]));  // a use in this chunk: no sinking into the next step
      // the next tile's LSE, into the halves this step has finished with
      if (ch == DK / 2) read_stat_half(ls, bn, 0, 0);
      if (ch == DK - 1) read_stat_half(ls, bn, 0, 1);
      if (ch == 1) store(bw);
      if (ch == 2) load(t + 3);
      chunk_schedule();
    }
    __syncthreads();
  }

  // ---- dS side, step t: dP_t from the tile in buffer cur, dS_{t-1} (tile in cur - 1),
  // dK products with dS_{t-2} (tile in cur - 2); chunk 0's operands were read by the
  // previous step (all these tiles were in LDS before its barrier)
  template <int B>
  __device__ __forceinline__ void step_d(int t, int cur) {
    const int bn = (cur + 1) % NB, bo = (cur + NB - 1) % NB, bo2 = (cur + NB - 2) % NB, bw = (cur + 2) % NB;
    pin[0] = *xslot(B ^ 1, 0);
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      if (ch + 1 < DK) {
        opd[(ch + 1) & 1] = read_row<D>(dbuf(cur), qrow, ch + 1);
        opk[(ch + 1) & 1] = read_tr<D>(qbuf(bo2), tr_off, (ch + 1) % DB, (ch + 1) / DB);
      } else {
        opd[0] = read_row<D>(dbuf(bn), qrow, 0);         // the next step's chunk 0: dO of tile t+1
        opk[0] = read_tr<D>(qbuf(bo), tr_off, 0, 0);     // and Q^T of tile t-1
      }
      if ((ch & 1) && ch + 1 < DK) pin[(ch + 1) >> 1] = *xslot(B ^ 1, (ch + 1) >> 1);
      const int sl = ch & 1, db = ch % DB, mm = ch / DB;
      dka[db] = mfma(opk[sl], word8(sw[B ^ 1], mm), dka[db]);
      dp[B] = mfma(opd[sl], vf[ch], ch == 0 ? f32x16{} : dp[B]);
      // dS of score elements 2 ch, 2 ch + 1 of tile t-1
      float d2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * ch + h;
        float dv = dp[B ^ 1][r];
        asm volatile("" : "+v"(dv));
        const float4 pq = pin[r >> 2];
        const float p = (r & 3) == 0 ? pq.x : (r & 3) == 1 ? pq.y : (r & 3) == 2 ? pq.z : pq.w;
        d2[h] = p * (dv - dl[r]);
      }
      sw[B][ch] = pack_bf16x2(d2[0], d2[1]);
      asm volatile("" ::"v"(sw[B][ch]));
      // D of tile t, for the next step
      if (ch == DK / 2) read_stat_half(dl, cur, 1, 0);
      if (ch == DK - 1) read_stat_half(dl, cur, 1, 1);
      if (ch == 1) store(bw);
      if (ch == 2) load(t + 3);
      chunk_schedule();
    }
    __syncthreads();
  }

  // ---- after the last step (parity B, tile in buffer cur): the products still owed,
  // with no barrier (they read only tiles already in LDS and the P slot of the last tile)
  template <int B>
  __device__ __forceinline__ void tail_p(int cur) {
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {  // dV += dO^T P of the last tile
      const int db = ch % DB, mm = ch / DB;
      const bf16x8 av = ch == 0 ? opv[0] : read_tr<D>(dbuf(cur), tr_off, db, mm);
      dva[db] = mfma(av, word8(pw[B], mm), dva[db]);
    }
  }
  template <int B>
  __device__ __forceinline__ void tail_d(int cur) {
    const int bo = (cur + NB - 1) % NB;
    // dS of the last tile, into the free dS buffer
#pragma unroll
    for (int i = 0; i < 4; ++i) pin[i] = *xslot(B, i);
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      float d2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 2 * ch + h;
        const float4 pq = pin[r >> 2];
        const float p = (r & 3) == 0 ? pq.x : (r & 3) == 1 ? pq.y : (r & 3) == 2 ? pq.z : pq.w;
        d2[h] = p * (dp[B][r] - dl[r]);
      }
      sw[B ^ 1][ch] = pack_bf16x2(d2[0], d2[1]);
    }
    // dK += Q^T dS of the last two tiles
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      const int db = ch % DB, mm = ch / DB;
      const bf16x8 ak = ch == 0 ? opk[0] : read_tr<D>(qbuf(bo), tr_off, db, mm);
      dka[db] = mfma(ak, word8(sw[B], mm), dka[db]);
    }
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      const int db = ch % DB, mm = ch / DB;
      dka[db] = mfma(read_tr<D>(qbuf(cur), tr_off, db, mm), word8(sw[B ^ 1], mm), dka[db]);
    }
  }

  // all steps of one side, tiles t0 .. nQT - 1, then the tail; the P side's steps on
  // tiles [t0 + 4, tf) (causal; [0, tf) otherwise) skip the visibility test
  template <bool PSIDE>
  __device__ __forceinline__ void run(int t0, int nQT, int tf) {
    const int tend = nQT;
    int t = t0;
    auto six = [&](auto guard) {
      constexpr bool G = decltype(guard)::value;
      if constexpr (PSIDE) {
        step_p<0, G>(t, 0);
        step_p<1, G>(t + 1, 1);
        step_p<0, G>(t + 2, 2);
        step_p<1, G>(t + 3, 3);
        step_p<0, G>(t + 4, 4);
        step_p<1, G>(t + 5, 5);
      } else {
        step_d<0>(t, 0);
        step_d<1>(t + 1, 1);
        step_d<0>(t + 2, 2);
        step_d<1>(t + 3, 3);
        step_d<0>(t + 4, 4);
        step_d<1>(t + 5, 5);
      }
    };
    if (CAUSAL && t + 6 <= tend) {
      six(std::true_type{});
      t += 6;
    }
    for (; t + 6 <= tf; t += 6) six(std::false_type{});
    for (; t + 6 <= tend; t += 6) six(std::true_type{});
    for (; t + 2 <= tend; t += 2) {
      if constexpr (PSIDE) {
        step_p<0, true>(t, (t - t0) % NB);
        step_p<1, true>(t + 1, (t + 1 - t0) % NB);
      } else {
        step_d<0>(t, (t - t0) % NB);
        step_d<1>(t + 1, (t + 1 - t0) % NB);
      }
    }
    if (t < tend) {
      if constexpr (PSIDE)
        step_p<0, true>(t, (t - t0) % NB);
      else
        step_d<0>(t, (t - t0) % NB);
      ++t;
    }
    // the last step was t - 1
    const int last = (t - 1 - t0) % NB;
    if ((t - 1 - t0) & 1) {
      if constexpr (PSIDE) tail_p<1>(last); else tail_d<1>(last);
    } else {
      if constexpr (PSIDE) tail_p<0>(last); else tail_d<0>(last);
    }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dkdv_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int BH, int N, float c, float dk_mul) {
  using W = DkDvPair<D, CAUSAL>;
  using T = Tile<D>;
  constexpr int DK = W::DK, DB = W::DB, NB = W::NB, kBk = 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * NB * T::BYTES];  // Q' buffers, then dO buffers
  __shared__ __attribute__((aligned(16))) float stat[NB * 2 * kT];
  __shared__ __attribute__((aligned(16))) float4 xp[4 * 2 * 4 * 64];

  W w;
  const int L = blockIdx.x;
  int kblk = L / BH;  // smallest key blocks (most causal work) first
  int bh = L % BH;
  if (!CAUSAL && BH % 8 == 0) grouped_item(L, BH, (int)(gridDim.x / BH), kblk, bh);
  const size_t base = (size_t)bh * N * D;
  w.tid = threadIdx.x;
  w.lane = w.tid & 63;
  w.g = w.lane >> 5;
  w.li = w.lane & 31;
  w.kg = (w.tid >> 6) & 3;
  const bool pside = w.tid < 256;
  const int k0 = kblk * kBk;
  w.kj = k0 + w.kg * 32 + w.li;  // this lane's key
  w.N = N;
  w.c = c;
  w.smem = smem;
  w.stat = stat;
  w.xp = xp;
  w.lse_h = lse + (size_t)bh * N;
  w.delta_h = delta + (size_t)bh * N;
  constexpr int kRsrcWord3 = 0x00020000;
  // a zero scale reads Q as zeros (a buffer of no bytes): the scores are then exactly 0
  // even where Q K^T would overflow, as in the forward, which zeroes Q
  w.qrs = __builtin_amdgcn_make_buffer_rsrc((void*)(q + base), (short)0, c == 0.f ? 0 : N * D * 2, kRsrcWord3);
  w.drs = __builtin_amdgcn_make_buffer_rsrc((void*)(dout + base), (short)0, N * D * 2, kRsrcWord3);
  {
    const int prow = w.tid / (D / 8), pcol = (w.tid % (D / 8)) * 16;
    w.ld_off = prow * D * 2 + pcol;
    w.st_off = piece_off<D>(prow, pcol / 16);
  }
  w.qrow = row_reader<D>(permuted_row(w.li), w.g);
  w.tr_off = tr_reader<D>(w.lane);

  // the side's operand rows of the block: K (P side) or V (dS side)
  {
    const uint16_t* src = pside ? k : v;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      uint4 a = make_uint4(0, 0, 0, 0);
      if (w.kj < N) a = *reinterpret_cast<const uint4*>(src + base + (size_t)w.kj * D + ks * 16 + w.g * 8);
      if (pside)
        w.kf[ks] = __builtin_bit_cast(bf16x8, a);
      else
        w.vf[ks] = __builtin_bit_cast(bf16x8, a);
    }
  }
  const int t0 = CAUSAL ? k0 / kT : 0;
  const int nQT = (N + kT - 1) / kT;
  if (t0 < nQT) {
    // prologue: tiles t0 and t0+1 into buffers 0 and 1; buffers 4 and 5 (tiles t0-2 and
    // t0-1 of the first steps' products) zeroed with their statistics, and the P slot of
    // tile t0-1; tile t0+2 loaded for the first step
    w.load(t0);
    w.store(0);
    w.load(t0 + 1);
    w.store(1);
    for (int i = w.tid; i < 2 * T::BYTES / 16; i += 512) {
      *reinterpret_cast<uint4*>(w.qbuf(4) + 16 * i) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(w.dbuf(4) + 16 * i) = make_uint4(0, 0, 0, 0);
    }
    for (int i = w.tid; i < 2 * 2 * kT; i += 512) stat[4 * 2 * kT + i] = 0.f;
    for (int i = w.tid; i < 4 * 4 * 64; i += 512) xp[((i >> 8) * 2 + 1) * 256 + (i & 255)] = make_float4(0.f, 0.f, 0.f, 0.f);
    w.load(t0 + 2);
    __syncthreads();
    if (pside) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.dva[db][r] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) w.pw[1][i] = 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) w.read_stat_half(w.ls, 0, 0, h);
      w.s[0] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) w.s[0] = mfma(read_row<D>(w.qbuf(0), w.qrow, ks), w.kf[ks], w.s[0]);
      w.opv[0] = read_tr<D>(w.dbuf(5), w.tr_off, 0, 0);
      w.template run<true>(t0, nQT, k0 + kBk <= N ? N / kT : 0);
      if (w.kj < N) store_rows<D>(dv + base + (size_t)w.kj * D, w.dva, 1.f, w.g);
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.dka[db][r] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) w.sw[1][i] = 0u;
      w.dp[1] = f32x16{};
#pragma unroll
      for (int h = 0; h < 2; ++h) w.read_stat_half(w.dl, 5, 1, h);
      w.opd[0] = read_row<D>(w.dbuf(0), w.qrow, 0);
      w.opk[0] = read_tr<D>(w.qbuf(4), w.tr_off, 0, 0);
      w.template run<false>(t0, nQT, 0);
      if (w.kj < N) store_rows<D>(dk + base + (size_t)w.kj * D, w.dka, dk_mul, w.g);
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const BwdArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* o = static_cast<const uint16_t*>(a.o);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
  const float c = a.scale == 0.f ? 1.f : fabsf(a.scale) * kLog2e;
  const uint32_t qxor = a.scale < 0.f ? 0x80008000u : 0u;
  const uint32_t qand = a.scale == 0.f ? 0u : 0xFFFFFFFFu;
  const int nQB = (N + 255) / 256;
  // dQ first: it writes D, which the dK/dV kernel reads
  hipLaunchKernelGGL((bwd_dq_pipe_kernel<D, CAUSAL>), dim3((unsigned)(nQB * BH)), dim3(512), 0, a.stream, q, k, v, o,
                     dout, a.lse, a.delta, static_cast<uint16_t*>(a.dq), BH, N, nQB, c, a.scale, qxor, qand);
  const int nKB = (N + 127) / 128;
  // d = 128: wavefront pairs, 8 wavefronts; d = 64: the plain loop, 4 wavefronts (the
  // pairs at d = 64 were bit-identical but 11 % slower on B16 H16 N1024)
  if constexpr (D == 128)
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)(nKB * BH)), dim3(512), 0, a.stream, q, k,
                       v, dout, a.lse, a.delta, static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), BH, N,
                       a.scale * kLog2e, a.scale);
  else
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
