// FP8 (OCP e4m3) attention forward on gfx950 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).
//
// The FP8 variant of the pages doubles the matrix throughput and keeps the
// result accurate with per-tile scales and a random rotation of Q and K (page
// "FlashAttention-Skalierung, Multi-GPU-Training und Gewichtsquantisierung",
// section 1, FlashAttention-3 FP8 item).  Its operands come from the
// quantise+rotate pre-pass: Q8, K8 as [B, H, N, 128] codes and V8 transposed
// as [B, H, 128, N64] (rows padded with zero codes to a multiple of 64 keys),
// each with one fp32 scale per 128-row tile.
//
// Structure (the bf16 kernel's, adapted to the fp8 instruction shape):
//   * one workgroup per (256-query block, head, batch), 8 wavefronts of 32
//     queries, heaviest causal blocks first;
//   * 64-key tiles, the K extent of one P V matrix instruction; K8 and V8^T
//     tiles go HBM -> registers (buffer loads, zero past the end) -> three
//     rotating LDS slots, one step ahead;
//   * scores transposed, S^T = K8 Q8^T, so a lane owns one query: for each
//     32-key half of the tile the K rows are permuted (bits 2 and 3 of the
//     row index swapped) and lane half g receives keys 8g..8g+7 and
//     16+8g..16+8g+7;
//   * the P V product contracts over the 64 keys in the order in which the
//     probabilities already sit in the lanes (keys 8g, 16+8g, 32+8g, 48+8g,
//     eight each): the V8^T tile is stored in LDS with its key columns in
//     that order, so both operands of the product are read with two 16-byte
//     LDS reads per lane and no data moves between lanes;
//   * software pipeline: step t issues S_{t+1}, O += P_{t-1} V_{t-1} and the
//     softmax of S_t in four chunks of one score and one output instruction
//     each, with the vector work of the softmax between them.
//
// Scales.  Every score of a (query tile, key tile) pair shares the factor
// scale * q_scale * k_scale, folded into the softmax multiplier.  V's tile
// scale enters through the probabilities: with r = v_scale / v_scale_max
// (v_scale_max: largest V scale of the head) written as r = 2^(e+1) * f,
// f in [1/2, 1), the probabilities of the tile are multiplied by 2^6 * f
// before rounding to e4m3 -- a shift of the exponent, at no cost -- and the
// power of two 2^(e+1) goes exactly into the E8M0 block scale of the P
// operand of the P V instruction.  The accumulator is then in units of
// v_scale_max / 2^6 for every tile (no per-tile rescaling), and the rounding
// of P keeps the same relative precision whatever V's scales are.  The
// running row sums add the probabilities times 2^6, so O = acc *
// v_scale_max / (rounded sum) and LSE follows from the fp32 sum.  The softmax shift
// moves lazily, only when a row maximum exceeds it by more than 2 (log2
// units): probabilities stay below 4, so the rounded values stay below 256,
// inside the e4m3 range (448).
//
// Two row sums, as in the bf16 kernel.  l adds the fp32 probabilities and gives
// LSE.  lh adds the e4m3-rounded probabilities that actually enter P V and
// normalises O, which makes O an exact weighted mean of the dequantised V rows
// under the weights used (with l, a row dominated by one key would carry that
// key's rounding error, up to 2^-4 of |v|).  The rounded sum of a tile is taken
// on the matrix core: four v_mfma_f32_16x16x32_fp8_fp8 against a constant
// selector of ones, whose rows pick, for every lane, the two lane groups that
// hold its own query (lanes l and l + 32), so that accumulator register 0 of
// lane l ends up holding the sum of the tile's 64 codes of query l % 32.
//
// A negative scale flips the sign bit of every Q code (exact), a zero scale
// zeroes Q; the kernel always works with a positive multiplier.
#include "fa_device.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kBc = 64;                 // keys per tile
constexpr int kTile = 128;              // quantisation tile rows
constexpr int kSlots = 3;               // LDS slots per operand
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBr = kWaves * 32;        // queries per workgroup
constexpr int kKS = kD + 16;            // K8 tile row stride (bytes)
constexpr int kVS = kBc + 16;           // V8^T tile row stride (bytes)
constexpr int kKSlot = kBc * kKS;
constexpr int kVSlot = kD * kVS;
constexpr int kLdsBytes = kSlots * (kKSlot + kVSlot);
constexpr float kSlack = 2.f;           // lazy shift slack (log2 units)
constexpr float kPShift = 6.f;          // probabilities enter e4m3 times 2^6
constexpr int NCH = 4;                  // chunks per step
static_assert(kBc * kD / 16 == kThreads && kD * kBc / 16 == kThreads, "one 16-byte piece per thread");

__device__ __forceinline__ int permuted_row(int i) { return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC); }

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  // the conversion writes one half of its destination and keeps the other; the second
  // one overwrites the kept half, so the first may keep any bits -- a's own, which
  // spares zeroing a register for it
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 = e4m3 for both operands; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// the same with B scaled by 2^(bscale - 127) (E8M0 block scale, exact)
__device__ __forceinline__ f32x16 mfma_fp8_bs(const i32x8& a, const i32x8& b, const f32x16& c, int bscale) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, bscale);
}

__device__ __forceinline__ i32x8 lds_read32(const char* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// a wave-uniform value, kept in a scalar register
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}


template <bool CAUSAL>
struct Attn8 {
  // ---- per-thread state
  i32x8 qf[2];          // Q8 as B operand, one per 64-column half of d
  f32x16 oacc[4];       // O^T, 32 rows of d each
  f32x16 sbuf[2][2];    // S^T of two consecutive tiles, two 32-key halves each
  i32x8 pbuf[2];        // P8^T of two consecutive tiles
  int pscale[2];        // their E8M0 block scales
  float pinvf[2];       // and the 1 / f of their tiles (for the rounded row sum)
  long sel;             // selector of ones for the rounded row sums (A operand, 8 codes)
  i32x8 kop[2], vop[2]; // operand prefetch, by chunk parity
  uint4 stg_k, stg_v;   // this thread's piece of the next K8 / V8^T tiles
  float m, l, lh, alpha, msub, rs;
  float cst, inv_frac;  // softmax multiplier and 1 / f of the tile being softmaxed
  int psc;               // its E8M0 scale 127 + e + 1
  float lfac;            // and log2 f
  float ks_n, vs_n;      // raw K and V tile scales of the next tile (loaded one step ahead)
  float msub_q;

  // ---- per-workgroup constants
  __amdgpu_buffer_rsrc_t krs, vrs, ksrs, vsrs;
  char* kslot;
  char* vslot;
  const float* ks_head;
  const float* vs_head;
  int N, nTiles, qw0, lane, g, li;
  int ldv;          // V8^T row length (keys, a multiple of 64)
  int kst_off, vst_off;
  int krd_off, vrd_off;
  int vld_row;      // this thread's V8^T row (d) in a tile copy
  int vld_col;      // ... and key offset inside the tile
  float cq, log2_svmax, svmax;

  __device__ __forceinline__ i32x8 read_k(int slot, int ch) const {
    const int kb = ch & 1, kk = ch >> 1;
    return lds_read32(kslot + slot * kKSlot + krd_off + kb * 32 * kKS + kk * 64);
  }
  __device__ __forceinline__ i32x8 read_v(int slot, int ch) const {
    return lds_read32(vslot + slot * kVSlot + vrd_off + ch * 32 * kVS);
  }
  // sum of the 64 rounded probabilities (codes) of this lane's query in P8^T p, in
  // lane register 0 of a 16x16 accumulator: lane l holds keys of query l % 32, and
  // lane group G = l / 16 of the A operand selects, for output row 4 G', the lane
  // groups holding query 16 (G' % 2) + (l % 16), namely G' % 2 and G' % 2 + 2
  __device__ __forceinline__ float rounded_sum(const i32x8& p) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long b = (long)(((unsigned long)(uint32_t)p[2 * i + 1] << 32) | (uint32_t)p[2 * i]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(sel, b, acc, 0, 0, 0);
    }
    return acc[0];
  }
  // this thread's 16-byte pieces of K8 tile t (row-major) and V8^T tile t (row d, 16 keys);
  // buffer loads return zeros past the end of the head's data
  __device__ __forceinline__ uint4 load_k(int t) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, t * kBc * kD + (int)threadIdx.x * 16, 0, 0));
  }
  __device__ __forceinline__ uint4 load_v(int t) const {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vld_row * ldv + t * kBc + vld_col, 0, 0));
  }
  __device__ __forceinline__ void store_k(int slot, const uint4& x) const {
    *reinterpret_cast<uint4*>(kslot + slot * kKSlot + kst_off) = x;
  }
  __device__ __forceinline__ void store_v(int slot, const uint4& x) const {
    // keys 16j..16j+7 and 16j+8..16j+15 of this row go to positions 8j and 32+8j
    char* pv = vslot + slot * kVSlot + vst_off;
    *reinterpret_cast<uint2*>(pv) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2*>(pv + 32) = make_uint2(x.z, x.w);
  }
  // K and V scales of key tile t (its 128-row quantisation tile), one step before its
  // softmax; vector-memory loads, so waiting for them never waits for LDS traffic
  __device__ __forceinline__ void load_scales(int t) {
    const int off = min(t * kBc / kTile, nTiles - 1) * 4;
    ks_n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksrs, off, 0, 0));
    vs_n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vsrs, off, 0, 0));
  }

  __device__ __forceinline__ void mask_scores(int B, int t) {
    const int qi = qw0 + li;
    const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - t * kBc - g * 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r & 7) + (r & 8) * 2 > lim) sbuf[B][kb][r] = -kInf;
  }
  // +inf from a register the compiler cannot see through: against the literal it folds
  // the median back into a canonicalising maximum
  float pinf;
  __device__ __forceinline__ float max2(float a, float b) const { return __builtin_amdgcn_fmed3f(a, b, pinf); }
  __device__ __forceinline__ void softmax_slice(int ch, int B, int t, bool guard) {
    if (ch == 0) {
      // this tile's factors: multiplier, r = sv / svmax = 2^(e+1) f, 1 / f, E8M0 scale.
      // A 128-row quantisation tile holds key tiles 2u and 2u + 1, so the odd steps (B
      // = 1) keep the factors of the step before
      if (B == 0) {
        cst = uniform(cq * ks_n);
        const float lr = log2_fast(vs_n) - log2_svmax;        // log2 r <= 0
        const float e = fmaxf(__builtin_floorf(lr), -120.f);  // E8M0 stays in range
        lfac = uniform(lr - e - 1.f);                         // log2 f, in [-1, 0) unless clamped
        inv_frac = uniform(exp2_fast(-lfac));
        psc = __builtin_amdgcn_readfirstlane(128 + (int)e);
      }
      const float lf = lfac;
      if (guard) mask_scores(B, t);
      const f32x16& s0 = sbuf[B][0];
      const f32x16& s1 = sbuf[B][1];
      // row maximum over the 32 scores: two chains of three-input maxima, each started
      // by a median against +inf (max of its two operands; fmaxf on MFMA results
      // would first canonicalise each operand), joined the same way across the lanes
      float ma = max2(s0[0], s0[1]), mb = max2(s1[0], s1[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) {
        ma = fmaxf(ma, s0[r]);
        mb = fmaxf(mb, s1[r]);
      }
      const float mx = fmaxf(ma, mb);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      const float mt = cst * max2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // -inf when no key is visible
      const float m_new = mt > m + kSlack ? mt : m;
      // unmasked steps come after step 0, in which every row sees key 0: the shift is
      // finite there and needs no test for an empty row
      alpha = guard && m_new == -kInf ? 1.f : exp2_fast(m - m_new);
      m = m_new;
      l *= alpha;
      // 2^(cst*s - m + 6 + log2 f): the scaled probability that enters e4m3
      msub_q = guard && m_new == -kInf ? 0.f : m_new - kPShift - lf;
      rs = 0.f;
    } else if (ch == 1 || ch == 2) {
      f32x16& s = sbuf[B][ch - 1];
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = exp2_fast(fmaf(s[r], cst, -msub_q));
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (s[i] + s[i + 4]) + (s[i + 8] + s[i + 12]);
      rs += (h[0] + h[1]) + (h[2] + h[3]);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x16& s = sbuf[B][kb];
          const int b0 = 8 * hh;
          pbuf[B][kb * 4 + hh * 2 + 0] = (int)pack_fp8x4(s[b0 + 0], s[b0 + 1], s[b0 + 2], s[b0 + 3]);
          pbuf[B][kb * 4 + hh * 2 + 1] = (int)pack_fp8x4(s[b0 + 4], s[b0 + 5], s[b0 + 6], s[b0 + 7]);
        }
      pscale[B] = psc;
      pinvf[B] = inv_frac;
      l += rs * inv_frac;
    }
  }

  template <bool GUARD, int B>
  __device__ __forceinline__ void step(int t, int sk_next, int sk_w, int sv_pv, int sv_next, int sv_w) {
    f32x16(&snext)[2] = sbuf[B ^ 1];
    const i32x8& pold = pbuf[B ^ 1];
    const int psold = pscale[B ^ 1];
    float rsum = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch + 1 < NCH) {
        kop[(ch + 1) & 1] = read_k(sk_next, ch + 1);
        vop[(ch + 1) & 1] = read_v(sv_pv, ch + 1);
      } else {
        kop[0] = read_k(sk_next == kSlots - 1 ? 0 : sk_next + 1, 0);
        vop[0] = read_v(sv_next, 0);
      }
      // P V first: V's operand is the chunk's newest LDS read, so the one wait before
      // it also covers the K read of the score MFMA after it
      oacc[ch] = mfma_fp8_bs(vop[ch & 1], pold, oacc[ch], psold);
      if (ch == 0) rsum = rounded_sum(pold);
      {
        const int kb = ch & 1, kk = ch >> 1;
        if (kk == 0) {
          const f32x16 z = {};
          snext[kb] = mfma_fp8(kop[ch & 1], qf[0], z);
        } else {
          snext[kb] = mfma_fp8(kop[ch & 1], qf[1], snext[kb]);
        }
      }
      softmax_slice(ch, B, t, GUARD);
      if (ch == 1) {  // V's piece was loaded last: waiting for it covers K's too
        store_v(sv_w, stg_v);
        store_k(sk_w, stg_k);
      }
      if (ch == 2) {
        if (B == 1) load_scales(t + 1);  // an even tile next: a new quantisation tile
        stg_k = load_k(t + 4);
        stg_v = load_v(t + 2);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0); // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 200, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);  // DS writes
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);  // VMEM reads
      __builtin_amdgcn_sched_barrier(0);
    }
    // rounded sum of tile t-1 (shift of step t-1), then both it and O move to this step's shift
    lh = fmaf(rsum, pinvf[B ^ 1], lh) * alpha;
    // deferred correction of O for rows whose shift moved
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    __syncthreads();
  }

  template <int B>
  __device__ __forceinline__ void last_pv(int slot) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const i32x8 a = ch == 0 ? vop[0] : read_v(slot, ch);
      oacc[ch] = mfma_fp8_bs(a, pbuf[B], oacc[ch], pscale[B]);
    }
    lh = fmaf(rounded_sum(pbuf[B]), pinvf[B], lh);
  }
};

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
    uint16_t* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c, uint32_t qxor,
    uint32_t qand) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  Attn8<CAUSAL> s;
  // work item -> (query block, head): heaviest causal blocks first, heads interleaved
  // (longest first balances the compute units; grouping each XCD's heads one after
  // another read only the algorithmic HBM bytes but ran 7 % slower)
  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const int nTiles = (N + kTile - 1) / kTile;
  const int ldv = (N + kBc - 1) / kBc * kBc;
  const size_t base = (size_t)bh * N * kD;
  constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access on gfx9-class GPUs
  s.krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k8 + base), (short)0, N * kD, kRsrcWord3);
  s.vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v8t + (size_t)bh * kD * ldv), (short)0, kD * ldv, kRsrcWord3);
  s.kslot = smem;
  s.vslot = smem + kSlots * kKSlot;
  s.ks_head = ks + (size_t)bh * nTiles;
  s.vs_head = vs + (size_t)bh * nTiles;
  s.ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)s.ks_head, (short)0, nTiles * 4, kRsrcWord3);
  s.vsrs = __builtin_amdgcn_make_buffer_rsrc((void*)s.vs_head, (short)0, nTiles * 4, kRsrcWord3);
  s.N = N;
  s.pinf = kInf;
  asm volatile("" : "+v"(s.pinf));
  s.nTiles = nTiles;
  s.ldv = ldv;
  const int tid = threadIdx.x;
  s.lane = tid & 63;
  s.g = s.lane >> 5;
  s.li = s.lane & 31;
  {
    const int krow = tid >> 3, kcol = (tid & 7) * 16;
    s.kst_off = krow * kKS + kcol;
    s.vld_row = tid >> 2;
    s.vld_col = (tid & 3) * 16;
    s.vst_off = s.vld_row * kVS + (tid & 3) * 8;
    s.krd_off = permuted_row(s.li) * kKS + s.g * 32;
    s.vrd_off = s.li * kVS + s.g * 32;
  }
  const int q0 = qblk * kBr;
  s.qw0 = q0 + (tid >> 6) * 32;
  const int qi = s.qw0 + s.li;
  const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
  const int nT = (kv_end + kBc - 1) / kBc;
  const int nFull = (CAUSAL ? min(N, q0 + 1) : N) / kBc;

  // largest V scale of the head
  {
    float mx = 0.f;
    for (int i = s.lane; i < nTiles; i += 64) mx = fmaxf(mx, s.vs_head[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    s.svmax = uniform(mx);
    s.log2_svmax = uniform(log2_fast(mx));
  }
  s.cq = uniform(c * qs[(size_t)bh * nTiles + min(s.qw0 / kTile, nTiles - 1)]);

#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (qi < N) {
      const uint8_t* p = q8 + base + (size_t)qi * kD + kk * 64 + s.g * 32;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 16);
    }
    lo = make_uint4((lo.x ^ qxor) & qand, (lo.y ^ qxor) & qand, (lo.z ^ qxor) & qand, (lo.w ^ qxor) & qand);
    hi = make_uint4((hi.x ^ qxor) & qand, (hi.y ^ qxor) & qand, (hi.z ^ qxor) & qand, (hi.w ^ qxor) & qand);
    s.qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  s.m = -kInf;
  s.l = 0.f;
  s.lh = 0.f;
  s.alpha = 1.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) s.oacc[db][r] = 0.f;

  // ---- prologue: K_0..K_2 and V_0 into LDS, V slot 2 (standing for V_{-1}) and P_{-1}
  // zero; S_0; stage K_3 and V_1; scales of tile 0; operands of step 0's first chunk
  {
    const uint4 k0 = s.load_k(0), k1 = s.load_k(1), k2 = s.load_k(2), v0 = s.load_v(0);
    s.stg_k = s.load_k(3);
    s.stg_v = s.load_v(1);
    s.store_k(0, k0);
    s.store_k(1, k1);
    s.store_k(2, k2);
    s.store_v(0, v0);
    s.store_v(2, make_uint4(0, 0, 0, 0));
  }
  s.pbuf[1] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  s.pscale[1] = 127;
  s.pinvf[1] = 0.f;
  {
    // selector: lane l supplies A row l % 16, codes 8 (l / 16) .. + 7; row 4 G' is one
    // (e4m3 0x38) in the lane groups G with G % 2 == G' % 2
    const int row = s.lane & 15, grp = s.lane >> 4;
    s.sel = (row % 4 == 0 && (row / 4) % 2 == grp % 2) ? (long)0x3838383838383838ull : 0l;
  }
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const f32x16 z = {};
    s.sbuf[0][kb] = mfma_fp8(s.read_k(0, kb), s.qf[0], z);
    s.sbuf[0][kb] = mfma_fp8(s.read_k(0, kb + 2), s.qf[1], s.sbuf[0][kb]);
  }
  s.load_scales(0);
  s.kop[0] = s.read_k(1, 0);
  s.vop[0] = s.read_v(2, 0);

  int sk_next = 1, sk_w = 0, sv_pv = 2, sv_next = 0, sv_w = 1;  // for t = 0
  auto advance = [&]() {
    sk_next = sk_next == 2 ? 0 : sk_next + 1;
    sk_w = sk_w == 2 ? 0 : sk_w + 1;
    sv_pv = sv_pv == 2 ? 0 : sv_pv + 1;
    sv_next = sv_next == 2 ? 0 : sv_next + 1;
    sv_w = sv_w == 2 ? 0 : sv_w + 1;
  };
  s.template step<true, 0>(0, sk_next, sk_w, sv_pv, sv_next, sv_w);
  advance();
  int t = 1;
  for (; t + 1 < nFull; t += 2) {
    s.template step<false, 1>(t, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
    s.template step<false, 0>(t + 1, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
  }
  for (; t < nT; t += 2) {
    s.template step<true, 1>(t, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
    if (t + 1 < nT) {
      s.template step<true, 0>(t + 1, sk_next, sk_w, sv_pv, sv_next, sv_w);
      advance();
    }
  }
  if ((nT - 1) & 1) s.template last_pv<1>((nT - 1) % kSlots);
  else s.template last_pv<0>((nT - 1) % kSlots);

  // ---- epilogue: O = acc * svmax / (rounded sum), LSE = ln 2 * (m + log2(sum) - 6).  The
  // rounded sum already covers both lanes of a query; l is this lane's half of the sum.
  const float lt = sum_pair(s.l);
  if (qi < N) {
    const float inv = s.svmax / s.lh;
#pragma unroll
    for (int db = 0; db < 4; ++db) store_row_bf16(o + base + (size_t)qi * kD + db * 32, s.oacc[db], inv, s.g);
    if (s.g == 0) lse[(size_t)bh * N + qi] = (s.m + log2_fast(lt) - kPShift) * kLn2;
  }
}

// ---- The same attention with the probabilities kept in bf16: S = Q8 K8^T on the fp8
// matrix core as above, but P is rounded to bf16 and O += P V runs on the bf16 matrix
// core (v_mfma_f32_32x32x16_bf16), with V's e4m3 codes widened to bf16 -- exactly, as
// every e4m3 value is a bf16 value -- when its tile is staged into LDS.  This is the
// accuracy reference for the rounding of P to e4m3: the two kernels differ only
// there (and in the P V instruction).  It is written plainly, without the software
// pipeline: one 64-key tile per step, two barriers per step, K8 and V8^T tiles
// loaded one step ahead into registers.
//
// Layouts.  The scores come out as in Attn8 (lane half g holds keys 8g..8g+7 and
// 16+8g..16+8g+7 of each 32-key half kb), which for k-step j = 2 kb + h of the bf16
// product (keys 16 j .. 16 j + 15) is exactly the B-operand layout of P^T: lane
// half g needs keys 16 j + 8 g .. + 7, i.e. registers 8 h .. 8 h + 7 of half kb.
// V^T is kept row-major in LDS, one d-row of 64 keys (bf16) per row, so the A
// operand of a k-step (d-row 32 db + l % 32, keys 16 j + 8 (l / 32) .. + 7) is one
// 16-byte read.  V's tile scale ratio r = v_scale / v_scale_max goes wholly into
// the exponent shift: P = bf16(2^6 r p), so O accumulates in units of
// v_scale_max / 2^6 as in the fp8 kernel.  O is normalised by the sum of the
// bf16-rounded probabilities (divided by r per tile), LSE by the fp32 sum.
namespace pbf16 {
constexpr int kVS16 = kBc * 2 + 16;  // bf16 V^T row stride (bytes)
constexpr int kVBytes = kD * kVS16;
constexpr float kSlack16 = 2.f;

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
}  // namespace pbf16

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_pbf16_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8t,
    const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vs,
    uint16_t* __restrict__ o, float* __restrict__ lse, int BH, int N, int nQB, float c, uint32_t qxor,
    uint32_t qand) {
  using namespace pbf16;
  __shared__ __attribute__((aligned(16))) char kt[kKSlot];
  __shared__ __attribute__((aligned(16))) char vt[kVBytes];
  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const int nTiles = (N + kTile - 1) / kTile;
  const int ldv = (N + kBc - 1) / kBc * kBc;
  const size_t base = (size_t)bh * N * kD;
  constexpr int kRsrcWord3 = 0x00020000;  // raw buffer access: reads past the end return zeros
  const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k8 + base), (short)0, N * kD, kRsrcWord3);
  const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v8t + (size_t)bh * kD * ldv), (short)0, kD * ldv, kRsrcWord3);
  const float* ks_head = ks + (size_t)bh * nTiles;
  const float* vs_head = vs + (size_t)bh * nTiles;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q0 = qblk * kBr, qw0 = q0 + (tid >> 6) * 32, qi = qw0 + li;
  const int kv_end = CAUSAL ? min(N, q0 + kBr) : N;
  const int nT = (kv_end + kBc - 1) / kBc;
  // the wavefront's last tile holding a key one of its rows sees (wave-uniform)
  const int last_w = __builtin_amdgcn_readfirstlane(
      qw0 >= N ? -1 : (CAUSAL ? min(qw0 + 31, N - 1) : N - 1) / kBc);

  float svmax;
  {
    float mx = 0.f;
    for (int i = lane; i < nTiles; i += 64) mx = fmaxf(mx, vs_head[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    svmax = uniform(mx);
  }
  const float log2_svmax = uniform(log2_fast(svmax));
  const float cq = uniform(c * qs[(size_t)bh * nTiles + min(qw0 / kTile, nTiles - 1)]);

  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (qi < N) {
      const uint8_t* p = q8 + base + (size_t)qi * kD + kk * 64 + g * 32;
      lo = *reinterpret_cast<const uint4*>(p);
      hi = *reinterpret_cast<const uint4*>(p + 16);
    }
    lo = make_uint4((lo.x ^ qxor) & qand, (lo.y ^ qxor) & qand, (lo.z ^ qxor) & qand, (lo.w ^ qxor) & qand);
    hi = make_uint4((hi.x ^ qxor) & qand, (hi.y ^ qxor) & qand, (hi.z ^ qxor) & qand, (hi.w ^ qxor) & qand);
    qf[kk] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -kInf, l = 0.f, lh = 0.f;

  // this thread's 16-byte pieces: K8 row tid/8, bytes 16 (tid%8); V8^T row tid/4, keys 16 (tid%4)
  const int kst_off = (tid >> 3) * kKS + (tid & 7) * 16;
  const int vrow = tid >> 2, vcol = (tid & 3) * 16;
  const int krd_off = permuted_row(li) * kKS + g * 32;
  auto load_k = [&](int t) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, t * kBc * kD + tid * 16, 0, 0));
  };
  auto load_v = [&](int t) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, vrow * ldv + t * kBc + vcol, 0, 0));
  };
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  uint4 sk = load_k(0), sv = load_v(0);
  for (int t = 0; t < nT; ++t) {
    __syncthreads();  // every wavefront is done with tile t-1
    *reinterpret_cast<uint4*>(kt + kst_off) = sk;
    {
      // 16 codes -> 16 bf16 (exact), natural key order
      const uint32_t c4[4] = {sv.x, sv.y, sv.z, sv.w};
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c4[i], 1.0f, false));
        b[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c4[i], 1.0f, true));
      }
      char* pv = vt + vrow * kVS16 + vcol * 2;
      *reinterpret_cast<uint4*>(pv) = make_uint4(b[0], b[1], b[2], b[3]);
      *reinterpret_cast<uint4*>(pv + 16) = make_uint4(b[4], b[5], b[6], b[7]);
    }
    __syncthreads();
    if (t + 1 < nT) {
      sk = load_k(t + 1);
      sv = load_v(t + 1);
    }
    if (t > last_w) continue;  // no key of this tile is visible to the wavefront's rows
    // S^T of the tile: two 32-key halves kb, two 64-byte halves of d
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x16 z = {};
      sc[kb] = mfma_fp8(lds_read32(kt + krd_off + kb * 32 * kKS), qf[0], z);
      sc[kb] = mfma_fp8(lds_read32(kt + krd_off + kb * 32 * kKS + 64), qf[1], sc[kb]);
    }
    // mask: register r of half kb holds key t*64 + 32 kb + (r & 7) + 8 g + 2 (r & 8)
    const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - t * kBc - g * 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r & 7) + (r & 8) * 2 > lim) sc[kb][r] = -kInf;
    // tile factors: multiplier, log2 of r = v_scale / v_scale_max
    const int st = min(t * kBc / kTile, nTiles - 1);
    const float cst = uniform(cq * ks_head[st]);
    const float lr = uniform(log2_fast(vs_head[st]) - log2_svmax);
    const float inv_r = uniform(exp2_fast(-lr));
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    const float mt = cst * max_pair(mx);  // -inf when the row sees no key of the tile
    const float m_new = mt > m + kSlack16 ? mt : m;
    const float alpha = m_new == -kInf ? 1.f : exp2_fast(m - m_new);
    m = m_new;
    // 2^(cst s - m + 6 + log2 r): the scaled probability that enters bf16
    const float msub = m_new == -kInf ? 0.f : m_new - kPShift - lr;
    float rs = 0.f, hs = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[kb][r] = exp2_fast(fmaf(sc[kb][r], cst, -msub));
        rs += sc[kb][r];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4 wv;
        wv.x = pack_bf16x2(sc[kb][8 * h + 0], sc[kb][8 * h + 1]);
        wv.y = pack_bf16x2(sc[kb][8 * h + 2], sc[kb][8 * h + 3]);
        wv.z = pack_bf16x2(sc[kb][8 * h + 4], sc[kb][8 * h + 5]);
        wv.w = pack_bf16x2(sc[kb][8 * h + 6], sc[kb][8 * h + 7]);
        pb[kb][h] = __builtin_bit_cast(bf16x8, wv);
        hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.x), ones, hs, false);
        hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.y), ones, hs, false);
        hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.z), ones, hs, false);
        hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.w), ones, hs, false);
      }
    }
    l = l * alpha + rs * inv_r;
    lh = lh * alpha + hs * inv_r;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // O^T += V^T P^T over the tile's four 16-key steps
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * db + li) * kVS16 + (16 * j + 8 * g) * 2);
        oacc[db] = mfma_bf16(a, pb[j >> 1][j & 1], oacc[db]);
      }
  }

  // ---- epilogue: O = acc * svmax / (rounded sum), LSE = ln 2 * (m + log2(sum) - 6)
  const float lt = sum_pair(l), lht = sum_pair(lh);
  if (qi < N) {
    const float inv = svmax / lht;
#pragma unroll
    for (int db = 0; db < 4; ++db) store_row_bf16(o + base + (size_t)qi * kD + db * 32, oacc[db], inv, g);
    if (g == 0) lse[(size_t)bh * N + qi] = (m + log2_fast(lt) - kPShift) * kLn2;
  }
}

}  // namespace

hipError_t launch_attn_fp8(const Fp8AttnArgs& a) {
  const int BH = (int)(a.B * a.H), N = (int)a.N;
  if (a.p_bf16) {
    const int nQB = (N + kBr - 1) / kBr;
    const float c = a.scale == 0.f ? 1.f : fabsf(a.scale) * kLog2e;
    const uint32_t qxor = a.scale < 0.f ? 0x80808080u : 0u;
    const uint32_t qand = a.scale == 0.f ? 0u : 0xFFFFFFFFu;
    if (a.causal)
      hipLaunchKernelGGL((attn_fwd_fp8_pbf16_kernel<true>), dim3((unsigned)(nQB * BH)), dim3(kThreads), 0, a.stream,
                         a.q8, a.k8, a.v8t, a.q_scale, a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o), a.lse, BH,
                         N, nQB, c, qxor, qand);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_pbf16_kernel<false>), dim3((unsigned)(nQB * BH)), dim3(kThreads), 0,
                         a.stream, a.q8, a.k8, a.v8t, a.q_scale, a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o),
                         a.lse, BH, N, nQB, c, qxor, qand);
    return hipGetLastError();
  }
  const int nQB = (N + kBr - 1) / kBr;
  const dim3 grid((unsigned)(nQB * BH)), block(kThreads);
  // positive multiplier: negate Q (flip every code's sign bit) for a negative scale,
  // zero Q for a zero scale
  const float c = a.scale == 0.f ? 1.f : fabsf(a.scale) * kLog2e;
  const uint32_t qxor = a.scale < 0.f ? 0x80808080u : 0u;
  const uint32_t qand = a.scale == 0.f ? 0u : 0xFFFFFFFFu;
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<true>), grid, block, 0, a.stream, a.q8, a.k8, a.v8t, a.q_scale,
                       a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o), a.lse, BH, N, nQB, c, qxor, qand);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<false>), grid, block, 0, a.stream, a.q8, a.k8, a.v8t, a.q_scale,
                       a.k_scale, a.v_scale, static_cast<uint16_t*>(a.o), a.lse, BH, N, nQB, c, qxor, qand);
  return hipGetLastError();
}

}  // namespace fa
