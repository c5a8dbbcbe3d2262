// bf16 attention forward on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Method (page "FlashAttention-Skalierung, Multi-GPU-Training und
// Gewichtsquantisierung", section 1; FlashAttention-2 wiki page, sections
// "Hintergrund" and "Technische Architektur", items 1-3):
//   * outer loop over query blocks -- one workgroup per (query block, head,
//     batch), so a single head is spread over many compute units;
//   * inner loop over key/value tiles staged through LDS;
//   * online softmax: running row maximum, exp2 of the shifted scores,
//     correction of the running sums and of the unnormalised output, and a
//     single division by the row sum after the last tile;
//   * every wavefront owns whole query rows, so row maxima and sums never go
//     through LDS.
// The overlap of the matrix products with the softmax and with data movement
// follows the FlashAttention-3 ideas (same page, section 1; news page on
// FlashAttention-3, section "Innovationen"), rebuilt for CDNA4 below.
//
// Wavefront layout.  A wavefront owns 32 * QB queries (QB blocks of 32).  Scores
// are computed transposed, S^T = K Q^T, with K as the MFMA A operand (from
// LDS) and Q as the B operand (registers, loaded once).  In the 32x32
// accumulator layout a lane then holds one query (lane % 32) and 16 of the 32
// keys of a tile, so a query's statistics live in one lane plus its partner
// 32 lanes away.  The K rows fed to the A operand are permuted (bits 2 and 3
// of the row index swapped) so that a lane's 16 keys come out as two runs of
// 8 consecutive keys: exactly the B-operand layout of P^T in the second
// product O^T += V^T P^T, so the probabilities go from accumulators to
// operand registers with one bf16 conversion.  O^T keeps the query-per-lane
// layout, so rescaling it is lane-local.  V stays row-major in LDS; its
// transposed A operand comes from the transposing read ds_read_b64_tr_b16.
// The default is QB = 1 with two wavefronts per SIMD: one wavefront alone
// issues dependent vector instructions at about a third of the SIMD's rate,
// and the second one's stream fills the gaps.  QB = 2 (one wavefront per
// SIMD, 64 queries) halves the LDS bytes per MFMA instead; it measured slower.
//
// Software pipeline.  With QB = 1 the kernel fits in 256 architectural VGPRs
// (two wavefronts per SIMD), so no value is pinned to the accumulation
// registers: the compiler then selects the VGPR forms of the MFMAs and gives
// the whole budget to VGPRs, with no copies between the two register files.
// Step t (one 32-key
// tile) issues the 16 MFMAs of S_{t+1} = K_{t+1} Q^T, the 16 MFMAs of
// O^T += V_{t-1}^T P_{t-1}^T and the vector work of the softmax of S_t.  None
// depends on another, so the step is cut into D/16 chunks, each holding 2 + 2
// MFMAs, one slice of the softmax and the LDS reads of the next chunk's
// operands; scheduling barriers keep that order, so the matrix core runs
// while the vector unit computes exponentials, and LDS latency is hidden one
// chunk ahead -- the interleaving of matmul and softmax the pages describe
// for Hopper, inside one wavefront.  Every step issues the same instructions
// (no data-dependent branches): at t = 0 the P V product multiplies zero
// probabilities with a zeroed V slot, and past the last tile the scores of a
// stale K slot are computed and never used.  K/V tiles go HBM -> registers one
// step ahead and registers -> LDS into three rotating slots per operand
// (written two steps before use), so one workgroup barrier per step suffices
// although the next step's first operands are read before it.
//
// Lazy rescaling.  The softmax shift m of a row only moves when the row
// maximum exceeds it by more than 8 (log2 units); otherwise probabilities are
// exp2(c*s - m) <= 2^8 and the running sums and output keep their scale.  The
// shift cancels in O = acc / l and is added back in LSE = m + log2(l), so the
// result is unchanged while the rescale of O runs on only a few tiles; it is
// applied at the end of the step, after the step's products are issued.
//
// Two row sums.  l sums the fp32 probabilities and gives LSE; lh sums the
// bf16-rounded probabilities that actually enter P V (v_dot2_f32_bf16 against
// (1, 1)) and normalises O, which makes O an exact weighted mean of V under
// the rounded weights.
#include "fa_device.h"
#include "launch.h"

#ifndef FA_BF16_QB
#define FA_BF16_QB 1
#endif
// FA_SERIAL_PIPELINE=1 builds the debug form of the forward loop (see serial_steps)
#ifndef FA_SERIAL_PIPELINE
#define FA_SERIAL_PIPELINE 0
#endif

namespace fa {
namespace {

constexpr int kBc = 32;           // keys per tile
constexpr int kSlots = 3;         // LDS slots per operand
constexpr float kRescaleSlack = 8.f;
constexpr float kSumBound = 256.f;  // 2^kRescaleSlack

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D, int kThreads>
struct Layout {
  static constexpr int KS = D * 2 + 16;  // K row stride (bytes): conflict-free 16-byte row reads
  static constexpr int VS = D * 2 + 64;  // V row stride (bytes): conflict-free transposing reads
  static constexpr int KSLOT = kBc * KS;
  static constexpr int VSLOT = kBc * VS;
  static constexpr int BYTES = kSlots * (KSLOT + VSLOT);
  static constexpr int PIECES = kBc * D * 2 / 16;                      // 16-byte pieces per operand tile
  static constexpr int CHUNKS = PIECES >= kThreads ? PIECES / kThreads : 1;  // pieces per thread
  static constexpr bool PARTIAL = PIECES < kThreads;  // only the first PIECES threads copy
};

__device__ __forceinline__ int permuted_row(int i) { return i ^ ((((i >> 2) ^ (i >> 3)) & 1) * 0xC); }

// 4 bf16 of V^T: lane l of each 16-lane group receives V[K0 + j][D0 + l], j = 0..3,
// when lane k of the group points at V[K0 + k/4][D0 + 4*(k%4)].
__device__ __forceinline__ v4i16 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// QB = 32-query blocks per wavefront.  QB = 1: at d = 128, 8 wavefronts (256
// queries), two per SIMD, whose instruction streams the SIMD interleaves (one
// wavefront alone issues vector instructions at about a third of the SIMD's
// rate); at d = 64, 4 wavefronts (128 queries) in about 150 VGPRs, so three
// workgroups share a compute unit (three wavefronts per SIMD, from workgroups
// whose barriers are independent), which measured 9 % faster non-causal and
// 28 % faster causal than one 8-wavefront workgroup.  QB = 2: 4 wavefronts, one
// per SIMD, each with the whole register file, 256 queries.
template <int D, bool CAUSAL, int QB, int WAVES>
struct Attn {
  static constexpr int kQB = QB;
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kW = 32 * kQB;
  static constexpr int kBr = kWaves * kW;
  using Ly = Layout<D, kThreads>;
  static constexpr int DK = D / 16;  // k-steps of S = chunks per step
  static constexpr int DB = D / 32;  // 32-row blocks of O^T
  static constexpr int NCH = DK;     // chunks per step; PV chunk ch is (db, mm) = (ch % DB, ch / DB)
  static_assert(DB * 2 == NCH, "one PV operand per chunk");

  // ---- per-thread state
  bf16x8 qf[kQB][DK];
  f32x16 oacc[DB][kQB];
  f32x16 sbuf[2][kQB];     // S^T of two consecutive tiles
  bf16x8 pbuf[2][kQB][2];  // P^T (bf16) of two consecutive tiles
  bf16x8 kop[2], vop[2];   // operand prefetch, by chunk parity
  uint4 stg_k[Ly::CHUNKS], stg_v[Ly::CHUNKS];
  float m[kQB], l[kQB], lh[kQB], alpha[kQB], msub[kQB], mx[kQB], rs[kQB];
  float ex[kQB][16];       // probabilities of the tile being softmaxed (its scores stay in sbuf)

  // ---- per-workgroup constants
  __amdgpu_buffer_rsrc_t krs, vrs;  // this head's K and V; reads past N return zeros
  char* kslot;
  char* vslot;
  int kn;    // keys used: rows k0 .. k0 + kn - 1 of this head's K and V
  int qpos;  // position of query 0 relative to key k0 (causal: query i sees keys j <= qpos + i)
  int qw0, lane, g, li;
  int ld_off;   // byte offset of this thread's first 16-byte piece inside a tile
  int kst_off;  // LDS byte offset of that piece in a K slot
  int vst_off;  // ... in a V slot
  int krd_off;  // LDS byte offset of this lane's K operand row (k-step 0) in a slot
  int vrd_off;  // LDS byte offset of this lane's V^T operand (chunk 0) in a slot
  bool copier;  // this thread moves tile pieces (all threads unless a tile has fewer pieces)
  float c;      // > 0: scale * log2(e) in magnitude
  static constexpr int kRowsPerPiece = kThreads / (D / 8);  // rows between a thread's pieces (CHUNKS > 1)

  __device__ __forceinline__ bf16x8 read_k(int slot, int ks) const {
    return *reinterpret_cast<const bf16x8*>(kslot + slot * Ly::KSLOT + krd_off + ks * 32);
  }
  __device__ __forceinline__ bf16x8 read_v(int slot, int ch) const {
    const int db = ch % DB, mm = ch / DB;
    const char* pa = vslot + slot * Ly::VSLOT + vrd_off + (mm * 16) * Ly::VS + db * 64;
    const v4i16 lo = tr_read(pa), hi = tr_read(pa + 4 * Ly::VS);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // ---- HBM -> registers -> LDS copies of one operand tile: 16-byte pieces, rows read
  // whole (coalesced); piece i of a thread is row tid/(D/8) + i*kRowsPerPiece.
  // Buffer loads return zeros for rows past N (the whole offset is in the VGPR
  // operand, which the hardware bounds check covers).
  __device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, int t, uint4 (&stg)[Ly::CHUNKS]) const {
    if (Ly::PARTIAL && !copier) return;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS; ++i)
      stg[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, ld_off + (t * kBc + i * kRowsPerPiece) * D * 2, 0, 0));
  }
  __device__ __forceinline__ void store_tile(char* slot_base, int off, int stride,
                                             const uint4 (&stg)[Ly::CHUNKS]) const {
    if (Ly::PARTIAL && !copier) return;
    char* p = slot_base + off;
#pragma unroll
    for (int i = 0; i < Ly::CHUNKS; ++i) *reinterpret_cast<uint4*>(p + i * kRowsPerPiece * stride) = stg[i];
  }

  // ---- softmax of the scores in sbuf[B] (tile t) -> pbuf[B].  The launcher
  // guarantees c > 0 (a negative scale negates Q, a zero scale zeroes Q), so
  // the row maximum of c*s is c*max(s) and -inf marks a masked score.
  __device__ __forceinline__ void mask_scores(int B, int t) {
    // register r of lane half g holds key t*kBc + (r & 7) + 8*g + 2*(r & 8),
    // visible to query qi iff that key < kn and (causal) <= qpos + qi
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int qi = qw0 + qb * 32 + li;
      const int lim = (CAUSAL ? min(qpos + qi, kn - 1) : kn - 1) - t * kBc - g * 8;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((r & 7) + (r & 8) * 2 > lim) sbuf[B][qb][r] = -kInf;
    }
  }
  // maxima as v_med3_f32 against +inf (the median of a, b and +inf is max(a, b)): the
  // scores come straight from MFMAs and the partner's value from a lane swap, and
  // fmaxf on such values costs an extra canonicalising instruction per operand
  // (+inf comes from a register the compiler cannot see through: against the
  // literal it folds the median back into a canonicalising maximum)
  float pinf;
  __device__ __forceinline__ float max2(float a, float b) const { return __builtin_amdgcn_fmed3f(a, b, pinf); }
  __device__ __forceinline__ void row_max(int B, int qb) {
    float a = max2(sbuf[B][qb][0], sbuf[B][qb][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) a = fmaxf(a, sbuf[B][qb][r]);
    mx[qb] = a;
  }
  // GUARD: a row may have seen no key yet (m = -inf).  Unmasked steady steps come
  // after tile 0, which every row of the workgroup sees, so there m is finite and
  // the infinite cases need no test.
  template <bool GUARD>
  __device__ __forceinline__ void new_shift(int qb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[qb]), __float_as_uint(mx[qb]), false, false);
    const float mt = c * max2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // -inf when no key is visible
    const float m_new = mt > m[qb] + kRescaleSlack ? mt : m[qb];
    // 0 when m was -inf, exactly 1 when unchanged (also for rows with no visible key yet)
    alpha[qb] = GUARD && m_new == -kInf ? 1.f : exp2_fast(m[qb] - m_new);
    m[qb] = m_new;
    lh[qb] *= alpha[qb];  // (l takes its factor with the tile's sum, in pack)
    msub[qb] = GUARD && m_new == -kInf ? 0.f : m_new;
  }
  // exponentials of scores e0 .. e0 + n - 1 (n a power of two dividing 16, so one
  // query block), added to the row sum as a pairwise tree (short dependency chains)
  template <int n>
  __device__ __forceinline__ void exps(int B, int e0) {
    const int qb = e0 / 16, r0 = e0 % 16;
    float t[n];
#pragma unroll
    for (int i = 0; i < n; ++i) {
      t[i] = exp2_fast(fmaf(sbuf[B][qb][r0 + i], c, -msub[qb]));  // masked: exp2(-inf) = 0
      ex[qb][r0 + i] = t[i];
    }
#pragma unroll
    for (int w = n / 2; w >= 1; w /= 2)
#pragma unroll
      for (int i = 0; i < w; ++i) t[i] += t[i + w];
    rs[qb] = e0 % 16 == 0 ? t[0] : rs[qb] + t[0];  // the first run starts the tile's sum
  }
  __device__ __forceinline__ void pack(int B, int qb) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float h_acc[2] = {lh[qb], 0.f};  // one dot-product chain per half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 wv;
      wv.x = pack_bf16x2(ex[qb][8 * h + 0], ex[qb][8 * h + 1]);
      wv.y = pack_bf16x2(ex[qb][8 * h + 2], ex[qb][8 * h + 3]);
      wv.z = pack_bf16x2(ex[qb][8 * h + 4], ex[qb][8 * h + 5]);
      wv.w = pack_bf16x2(ex[qb][8 * h + 6], ex[qb][8 * h + 7]);
      pbuf[B][qb][h] = __builtin_bit_cast(bf16x8, wv);
      h_acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.x), ones, h_acc[h], false);
      h_acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.y), ones, h_acc[h], false);
      h_acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.z), ones, h_acc[h], false);
      h_acc[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.w), ones, h_acc[h], false);
    }
    lh[qb] = h_acc[0] + h_acc[1];
    // one explicit fused step, so that every path (pipelined, serial, and the
    // steady steps that skip the maximum) rounds the fp32 sum the same way
    l[qb] = fmaf(l[qb], alpha[qb], rs[qb]);
    // The probabilities and sums are next read after the step's conditional rescale
    // of O; without a use here the compiler's IR sinking moves the whole softmax
    // (exponentials included) past that branch, out of reach of the step's MFMAs.
    // An empty volatile asm reading them keeps the work in its chunks.
    const i32x4 p0 = __builtin_bit_cast(i32x4, pbuf[B][qb][0]), p1 = __builtin_bit_cast(i32x4, pbuf[B][qb][1]);
    asm volatile("" ::"v"(p0), "v"(p1), "v"(lh[qb]), "v"(l[qb]));
  }
  // slice ch of the softmax work: mask and row max, shift, the 16*kQB exponentials
  // spread over the middle chunks, packing at the end.
  // Unmasked steady steps (GUARD false) first take the exponentials under the
  // current shift, without the row maximum: the shift would move only if a score
  // exceeded it by more than kRescaleSlack, i.e. only if a probability exceeded
  // 2^kRescaleSlack, and a lane's probabilities are bounded by their sum.  So when
  // every lane's sum stays within 2^kRescaleSlack the shift stays, the correction
  // factor is 1 and the step is exactly the one the maximum would have given; when
  // some sum exceeds it (rare once the shift has settled; also +inf and NaN sums),
  // the wavefront takes the full path: the row maximum of the scores (still in
  // sbuf), the shift rule, and the exponentials again.
  template <bool GUARD>
  __device__ __forceinline__ void softmax_slice(int ch, int B, int t) {
    constexpr bool FAST = !GUARD;
    constexpr int E = 16 * kQB;
    // chunks [first_exp, last_exp) hold the exponentials, chunk pack_ch the packing; the
    // steps that skip the maximum start one chunk earlier at d = 128 (chunk 0 still
    // waits for the last score product of the previous step) and pack one chunk later
    // at d = 64: 1.2-1.9 % faster than the full steps' placement
    constexpr int first_exp = NCH == 8 ? (FAST ? 1 : 2) : 1;
    constexpr int last_exp = NCH == 8 ? (FAST ? 5 : 6) : 3;
    constexpr int pack_ch = FAST ? (NCH == 8 ? 5 : 3) : NCH - 2;
    constexpr int per = (E + (last_exp - first_exp) - 1) / (last_exp - first_exp);
    if (ch == 0 && !FAST) {
      if (GUARD) mask_scores(B, t);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) row_max(B, qb);
      if (NCH != 8) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) new_shift<GUARD>(qb);
      }
    }
    if (NCH == 8 && ch == 1 && !FAST) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) new_shift<GUARD>(qb);
    }
    if (FAST && ch == (NCH == 8 ? 1 : 0)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) alpha[qb] = 1.f;
    }
    static_assert(per * (last_exp - first_exp) == E && 16 % per == 0, "whole power-of-two runs of one query block");
    if (ch >= first_exp && ch < last_exp) exps<per>(B, (ch - first_exp) * per);
    if (FAST && ch == pack_ch) {
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) big |= !(rs[qb] <= kSumBound);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(big) != 0, 0)) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          row_max(B, qb);
          new_shift<false>(qb);
        }
        // the exponentials again, in the same runs (the same order of the row sum)
#pragma unroll
        for (int e0 = 0; e0 < E; e0 += per) exps<per>(B, e0);
      }
      // keep the probabilities where the fast path left them (no copies on that path)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) asm volatile("" : "+v"(ex[qb][r]), "+v"(ex[qb][r + 1]), "+v"(ex[qb][r + 2]), "+v"(ex[qb][r + 3]));
    }
    if (ch == pack_ch) pack(B, 0);
    if (ch == NCH - 1 && kQB == 2) pack(B, 1);
  }

  template <int B>
  __device__ __forceinline__ void last_pv(int slot) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const bf16x8 a = ch == 0 ? vop[0] : read_v(slot, ch);
      const int db = ch % DB, mm = ch / DB;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) oacc[db][qb] = mfma(a, pbuf[B][qb][mm], oacc[db][qb]);
    }
  }

  // ---- one pipeline step for tile t: S_{t+1} into sbuf[B^1], O += P_{t-1} V_{t-1},
  // softmax of sbuf[B] -> pbuf[B]; LDS writes of K_{t+3}, V_{t+1}; loads of K_{t+4}, V_{t+2}.
  // GUARD steps (the first, the causal diagonal and the tail) mask scores; the
  // others (1 <= t, tiles t and t+1 unmasked) need no mask.
  template <bool GUARD, int B>
  __device__ __forceinline__ void step(int t, int sk_next, int sk_w, int sv_pv, int sv_next, int sv_w) {
    f32x16 (&snext)[kQB] = sbuf[B ^ 1];
    const bf16x8 (&pold)[kQB][2] = pbuf[B ^ 1];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) snext[qb][r] = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // operands of the next chunk (or of the next step's first chunk)
      if (ch + 1 < NCH) {
        kop[(ch + 1) & 1] = read_k(sk_next, ch + 1);
        vop[(ch + 1) & 1] = read_v(sv_pv, ch + 1);
      } else {
        kop[0] = read_k(sk_next == kSlots - 1 ? 0 : sk_next + 1, 0);
        vop[0] = read_v(sv_next, 0);
      }
      // P V first: its operands (V^T) are the chunk's newest LDS reads, so the one
      // wait before it also covers the older K read of the score MFMA after it
      {
        const int db = ch % DB, mm = ch / DB;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) oacc[db][qb] = mfma(vop[ch & 1], pold[qb][mm], oacc[db][qb]);
      }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) snext[qb] = mfma(kop[ch & 1], qf[qb][ch], snext[qb]);
      softmax_slice<GUARD>(ch, B, t);
      if (ch == 1) {  // V's piece was loaded last: waiting for it covers K's too
        store_tile(vslot + sv_w * Ly::VSLOT, vst_off, Ly::VS, stg_v);
        store_tile(kslot + sk_w * Ly::KSLOT, kst_off, Ly::KS, stg_k);
      }
      if (ch == 2) {
        load_tile(krs, t + 4, stg_k);
        load_tile(vrs, t + 2, stg_v);
      }
      // issue order inside the chunk: the next chunk's LDS reads, then each MFMA
      // followed by a run of vector instructions (in-order issue would otherwise
      // stall the vector work behind back-to-back MFMAs), then memory copies
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 200, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);  // DS writes
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);  // VMEM reads
      __builtin_amdgcn_sched_barrier(0);
    }
    // deferred correction of O for rows whose shift moved
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) any |= alpha[qb] != 1.f;
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha[qb];
    }
    __syncthreads();
  }

  // ---- steps of a wavefront whose rows see no key of tile t or later (the causal
  // diagonal of its workgroup): O += P_{t-1} V_{t-1} once, then only the workgroup's
  // shared tile copies and the barrier, so that every wavefront passes the same barriers
  template <int B>
  __device__ __forceinline__ void step_pv(int t, int sk_w, int sv_pv, int sv_w) {
    const bf16x8 (&pold)[kQB][2] = pbuf[B ^ 1];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch + 1 < NCH) vop[(ch + 1) & 1] = read_v(sv_pv, ch + 1);
      const int db = ch % DB, mm = ch / DB;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) oacc[db][qb] = mfma(vop[ch & 1], pold[qb][mm], oacc[db][qb]);
    }
    step_idle(t, sk_w, sv_w);
  }
  __device__ __forceinline__ void step_idle(int t, int sk_w, int sv_w) {
    store_tile(kslot + sk_w * Ly::KSLOT, kst_off, Ly::KS, stg_k);
    store_tile(vslot + sv_w * Ly::VSLOT, vst_off, Ly::VS, stg_v);
    load_tile(krs, t + 4, stg_k);
    load_tile(vrs, t + 2, stg_v);
    __syncthreads();
  }

  // ---- debug form of the loop (FA_SERIAL_PIPELINE builds): one tile at a time
  // through a single LDS slot, a full barrier on each side of every copy, nothing
  // overlapped.  Scores, softmax, rescale and products are the same operations in
  // the same order as in the pipelined steps (the pipeline applies the correction
  // factor of tile t after adding P_{t-1} V_{t-1}, which is this loop's
  // "rescale, then add P_t V_t" one tile later), so the two builds agree bit for
  // bit, and a difference points at a hazard in the pipelined schedule.
  __device__ void serial_steps(int nT, int last_w) {
    for (int t = 0; t < nT; ++t) {
      load_tile(krs, t, stg_k);
      load_tile(vrs, t, stg_v);
      __syncthreads();  // every wavefront is done with tile t - 1
      store_tile(kslot, kst_off, Ly::KS, stg_k);
      store_tile(vslot, vst_off, Ly::VS, stg_v);
      __syncthreads();
      if (t > last_w) continue;  // no row of this wavefront sees tile t (uniform)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sbuf[0][qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const bf16x8 a = read_k(0, ks);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) sbuf[0][qb] = mfma(a, qf[qb][ks], sbuf[0][qb]);
      }
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) softmax_slice<true>(ch, 0, t);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha[qb];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const bf16x8 a = read_v(0, ch);
        const int db = ch % DB, mm = ch / DB;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) oacc[db][qb] = mfma(a, pbuf[0][qb][mm], oacc[db][qb]);
      }
    }
  }
};

// Rows of one launch: queries 0 .. nq-1 of each head against keys k0 .. k0+kn-1 of
// its nk rows of K and V; query i sits at key position qpos + i (relative to k0).
// The plain forward has nq = nk = kn = N, k0 = qpos = 0.
struct Geom {
  int nq, nk, k0, kn, qpos;
  int nsplit;  // PART: grid row s takes the s-th of nsplit consecutive sub-ranges of [k0, k0 + kn)
};

// PART: partial result over a key range -- O in fp32 (normalised over the range)
// and rows that see no key written as O = 0, LSE = -inf.
template <int D, bool CAUSAL, int QB, bool PART, int WAVES>
__global__ __launch_bounds__(WAVES * 64, D == 128 ? 2 : 3) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    void* __restrict__ o, float* __restrict__ lse, int BH, Geom gm, int nQB, float c, uint32_t qxor,
    uint32_t qand) {
  using A = Attn<D, CAUSAL, QB, WAVES>;
  using Ly = typename A::Ly;
  constexpr int DK = A::DK, DB = A::DB, kQB = A::kQB, kW = A::kW, kBr = A::kBr, kThreads = A::kThreads;
  __shared__ __attribute__((aligned(16))) char smem[Ly::BYTES];

  A s;
  if constexpr (PART) {
    // sub-range s of the keys, and slice s of the partial outputs
    const int sp = blockIdx.y;
    const int b0 = (int)((int64_t)gm.kn * sp / gm.nsplit), b1 = (int)((int64_t)gm.kn * (sp + 1) / gm.nsplit);
    gm.k0 += b0;
    gm.qpos -= b0;
    gm.kn = b1 - b0;
    o = static_cast<float*>(o) + (size_t)sp * BH * gm.nq * D;
    lse += (size_t)sp * BH * gm.nq;
  }
  // work item -> (query block, head).  Workgroup ids go to the 8 XCDs in turn, so
  // with B*H a multiple of 8 every block of a head runs on one XCD.  Causal: the
  // heaviest blocks first, heads interleaved -- longest first keeps the compute
  // units evenly loaded to the end.  (Giving each XCD its heads one after another,
  // heaviest first within a head, read only the algorithmic bytes from HBM at
  // B4 H16 N2048 instead of 1.37 times them, but its first wave held four copies of
  // every block length and the launch took 109 instead of 83 us.)  Otherwise the
  // blocks of a head are consecutive within their XCD, so they run together and
  // read the head's K/V through that XCD's L2 (interleaved heads would spread each
  // XCD's concurrent workgroups over more heads' K/V than its L2 holds).
  const int L = blockIdx.x;
  int qblk, bh;
  if (CAUSAL || PART || BH % 8 != 0) {
    qblk = CAUSAL ? (nQB - 1 - L / BH) : (L / BH);
    bh = L % BH;
  } else {
    const int slot = L / 8;
    qblk = slot % nQB;
    bh = (slot / nQB) * 8 + L % 8;
  }
  const int N = gm.nq;  // query rows
  const size_t base = (size_t)bh * N * D;
  const size_t kbase = ((size_t)bh * gm.nk + gm.k0) * D;
  constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access on gfx9-class GPUs
  s.krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k + kbase), (short)0, gm.kn * D * 2, kRsrcWord3);
  s.vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v + kbase), (short)0, gm.kn * D * 2, kRsrcWord3);
  s.kslot = smem;
  s.vslot = smem + kSlots * Ly::KSLOT;
  s.kn = gm.kn;
  s.qpos = gm.qpos;
  const int tid = threadIdx.x;
  s.lane = tid & 63;
  s.g = s.lane >> 5;
  s.li = s.lane & 31;
  {
    s.copier = tid < Ly::PIECES;
    const int prow = (tid % Ly::PIECES) / (D / 8), pcol = (tid % (D / 8)) * 16;  // first piece: row, byte column
    s.ld_off = prow * D * 2 + pcol;
    s.kst_off = prow * Ly::KS + pcol;
    s.vst_off = prow * Ly::VS + pcol;
    s.krd_off = permuted_row(s.li) * Ly::KS + s.g * 16;
    const int grp16 = s.lane >> 4, l16 = s.lane & 15;
    s.vrd_off = (8 * (grp16 >> 1) + (l16 >> 2)) * Ly::VS + (16 * (grp16 & 1) + 4 * (l16 & 3)) * 2;
  }
  const int q0 = qblk * kBr;
  s.qw0 = q0 + (tid >> 6) * kW;
  s.c = c;
  s.pinf = kInf;
  asm volatile("" : "+v"(s.pinf));
  const int kv_end = CAUSAL ? min(gm.kn, gm.qpos + q0 + kBr) : gm.kn;
  const int nT = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;
  // tiles 0 .. nFull-1 hold only keys that every query of the workgroup sees
  const int nFull = max(0, CAUSAL ? min(gm.kn, gm.qpos + q0 + 1) : gm.kn) / kBc;
  if (PART && nT == 0) {  // no key visible to any query of the block (uniform: before any barrier)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int qi = s.qw0 + qb * 32 + s.li;
      if (qi < N) {
        float* op = static_cast<float*>(o) + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
            *reinterpret_cast<float4*>(op + db * 32 + 8 * a4 + 4 * s.g) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s.g == 0) lse[(size_t)bh * N + qi] = -kInf;
      }
    }
    return;
  }

  // the first tiles' loads go out together, ahead of the Q loads: each would
  // otherwise wait for its own memory round trip before the next is issued
  uint4 pro_k[3][Ly::CHUNKS], pro_v[Ly::CHUNKS];
  if constexpr (!FA_SERIAL_PIPELINE) {
#pragma unroll
    for (int j = 0; j < 3; ++j) s.load_tile(s.krs, j, pro_k[j]);
    s.load_tile(s.vrs, 0, pro_v);
  }

#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int row = s.qw0 + qb * 32 + s.li;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      uint4 val = make_uint4(0, 0, 0, 0);
      if (row < N) val = *reinterpret_cast<const uint4*>(q + base + (size_t)row * D + ks * 16 + s.g * 8);
      // scale < 0: every sign bit flipped; scale == 0: zeros (c is then 1)
      val = make_uint4((val.x ^ qxor) & qand, (val.y ^ qxor) & qand, (val.z ^ qxor) & qand,
                       (val.w ^ qxor) & qand);
      s.qf[qb][ks] = __builtin_bit_cast(bf16x8, val);
    }
    s.m[qb] = -kInf;
    s.l[qb] = 0.f;
    s.lh[qb] = 0.f;
    s.alpha[qb] = 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) s.oacc[db][qb][r] = 0.f;
  }

  // the wavefront's own last tile: the last one holding a key visible to one of its
  // rows (wavefront-uniform; tiles up to nFull - 1 are visible to every row); -1 for
  // a wavefront whose rows all lie past N (a short last block, decode), which then
  // only helps with the tile copies
  const auto wave_last_tile = [&]() {
    const int lw = CAUSAL ? min(gm.qpos + s.qw0 + kW - 1, gm.kn - 1) : gm.kn - 1;
    return __builtin_amdgcn_readfirstlane(s.qw0 >= N || lw < 0 ? -1 : lw / kBc);
  };

  if constexpr (FA_SERIAL_PIPELINE) {
    s.serial_steps(nT, wave_last_tile());
  } else {
  // ---- prologue: K_0, K_1, K_2 and V_0 into LDS, V slot 2 (standing for V_{-1}) and
  // P_{-1} zero; S_0; stage K_3 and V_1; operands of step 0's first chunk
#pragma unroll
  for (int j = 0; j < 3; ++j) s.store_tile(s.kslot + j * Ly::KSLOT, s.kst_off, Ly::KS, pro_k[j]);
  s.store_tile(s.vslot, s.vst_off, Ly::VS, pro_v);
#pragma unroll
  for (int i = 0; i < Ly::CHUNKS; ++i) s.stg_v[i] = make_uint4(0, 0, 0, 0);
  s.store_tile(s.vslot + 2 * Ly::VSLOT, s.vst_off, Ly::VS, s.stg_v);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int h = 0; h < 2; ++h) s.pbuf[1][qb][h] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s.sbuf[0][qb][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    const bf16x8 a = s.read_k(0, ks);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) s.sbuf[0][qb] = mfma(a, s.qf[qb][ks], s.sbuf[0][qb]);
  }
  s.load_tile(s.krs, 3, s.stg_k);
  s.load_tile(s.vrs, 1, s.stg_v);
  s.kop[0] = s.read_k(1, 0);
  s.vop[0] = s.read_v(2, 0);
  // step 0 stores K_3 into slot 0, so every wavefront must have read K_0 for S_0 first
  // (in practice its reads finish long before the K_3 load returns; the barrier makes
  // the order certain)
  __syncthreads();

  // ---- steps; the slot of tile j is j % 3
  int sk_next = 1, sk_w = 0, sv_pv = 2, sv_next = 0, sv_w = 1;  // for t = 0
  auto advance = [&]() {
    sk_next = sk_next == 2 ? 0 : sk_next + 1;
    sk_w = sk_w == 2 ? 0 : sk_w + 1;
    sv_pv = sv_pv == 2 ? 0 : sv_pv + 1;
    sv_next = sv_next == 2 ? 0 : sv_next + 1;
    sv_w = sv_w == 2 ? 0 : sv_w + 1;
  };
  // steps with 1 <= t and tiles t, t+1 unmasked need no mask.  Buffer parity
  // B = t % 2 is static: every loop below starts at an odd t and advances by two.
  const int last_w = wave_last_tile();
  const int steady_end = min(nFull - 1, last_w + 1);
  s.template step<true, 0>(0, sk_next, sk_w, sv_pv, sv_next, sv_w);
  advance();
  int t = 1;
  // six steps per iteration (both buffer parities times the three slot phases), so
  // every slot is a constant and LDS addresses fold into instruction offsets; the
  // slot of tile j is j % 3, and the iteration starts at t = 1 mod 6
  for (; t + 5 < steady_end; t += 6) {
    s.template step<false, 1>(t, 2, 1, 0, 1, 2);
    s.template step<false, 0>(t + 1, 0, 2, 1, 2, 0);
    s.template step<false, 1>(t + 2, 1, 0, 2, 0, 1);
    s.template step<false, 0>(t + 3, 2, 1, 0, 1, 2);
    s.template step<false, 1>(t + 4, 0, 2, 1, 2, 0);
    s.template step<false, 0>(t + 5, 1, 0, 2, 0, 1);
  }
  sk_next = (t + 1) % 3, sk_w = t % 3, sv_pv = (t + 2) % 3, sv_next = t % 3, sv_w = (t + 1) % 3;
  for (; t + 1 < steady_end; t += 2) {
    s.template step<false, 1>(t, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
    s.template step<false, 0>(t + 1, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
  }
  const int t_end = min(nT, last_w + 1);
  int tn = t;  // next tile
  for (; t < t_end; t += 2) {
    s.template step<true, 1>(t, sk_next, sk_w, sv_pv, sv_next, sv_w);
    advance();
    tn = t + 1;
    if (t + 1 < t_end) {
      s.template step<true, 0>(t + 1, sk_next, sk_w, sv_pv, sv_next, sv_w);
      advance();
      tn = t + 2;
    }
  }
  if (tn < nT) {
    // tiles tn .. nT-1 hold no key this wavefront's rows see: the product of its last
    // tile (operands of its first chunk read by the last step), then copies only
    if (tn & 1) s.template step_pv<1>(tn, sk_w, sv_pv, sv_w);
    else s.template step_pv<0>(tn, sk_w, sv_pv, sv_w);
    advance();
    for (int u = tn + 1; u < nT; ++u) {
      s.step_idle(u, sk_w, sv_w);
      advance();
    }
  } else {
    // last product: O += P_{nT-1} V_{nT-1} (operands of its first chunk read by the last step)
    if ((nT - 1) & 1) s.template last_pv<1>((nT - 1) % kSlots);
    else s.template last_pv<0>((nT - 1) % kSlots);
  }
  }  // pipelined loop

  // ---- epilogue: the single division by the row sum, LSE, stores
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float lt = sum_pair(s.l[qb]);
    const float lht = sum_pair(s.lh[qb]);
    const int qi = s.qw0 + qb * 32 + s.li;
    if (qi < N) {
      if constexpr (PART) {
        // a row with no visible key in the range has l = 0: O = 0, LSE = -inf
        const float inv = lht > 0.f ? 1.f / lht : 0.f;
        float* op = static_cast<float*>(o) + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4)
            *reinterpret_cast<float4*>(op + db * 32 + 8 * a4 + 4 * s.g) =
                make_float4(s.oacc[db][qb][4 * a4 + 0] * inv, s.oacc[db][qb][4 * a4 + 1] * inv,
                            s.oacc[db][qb][4 * a4 + 2] * inv, s.oacc[db][qb][4 * a4 + 3] * inv);
        if (s.g == 0) lse[(size_t)bh * N + qi] = lt > 0.f ? (s.m[qb] + log2_fast(lt)) * kLn2 : -kInf;
      } else {
        const float inv = 1.f / lht;
        uint16_t* op = static_cast<uint16_t*>(o) + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) store_row_bf16(op + db * 32, s.oacc[db][qb], inv, s.g);
        if (s.g == 0) lse[(size_t)bh * N + qi] = (s.m[qb] + log2_fast(lt)) * kLn2;
      }
    }
  }
}

// The kernels need a positive multiplier c: scale * (q . k) = |scale| * ((-q) . k) for
// scale < 0 (negating bf16 is exact), and a zero scale is the same as zero queries.
struct ScaleArgs {
  float c;
  uint32_t qxor, qand;
};
inline ScaleArgs scale_args(float scale) {
  return ScaleArgs{scale == 0.f ? 1.f : fabsf(scale) * kLog2e, scale < 0.f ? 0x80008000u : 0u,
                   scale == 0.f ? 0u : 0xFFFFFFFFu};
}

template <int D, bool CAUSAL, int QB, bool PART, int WAVES>
hipError_t launch(const AttnArgs& a, const Geom& gm) {
  constexpr int kBr = Attn<D, CAUSAL, QB, WAVES>::kBr;
  constexpr int kThreads = Attn<D, CAUSAL, QB, WAVES>::kThreads;
  const int BH = (int)(a.B * a.H);
  const int nQB = (gm.nq + kBr - 1) / kBr;
  const ScaleArgs sc = scale_args(a.scale);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, QB, PART, WAVES>), dim3((unsigned)(nQB * BH), (unsigned)gm.nsplit),
                     dim3(kThreads), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.o, a.lse, BH, gm, nQB, sc.c, sc.qxor, sc.qand);
  return hipGetLastError();
}

// ---- split-KV decode: at most 32 queries against each key range of a split
// launch.  The general kernel gives every 32 queries a wavefront and shares each
// tile between them, so with one query block a single wavefront per workgroup
// computes and the range streams at its pace.  Here the workgroup's four
// wavefronts hold the same queries and take every fourth 32-key tile of the
// range, each with its own shift, sums and unnormalised output; the four parts
// are combined through LDS at the end by the same rule as parts over key ranges
// (scale each by exp2 of its shift minus the largest, then add).  No tile is
// shared, so K goes from HBM straight into the A-operand registers, one tile
// ahead; V goes through two LDS slots of the wavefront's own for the
// transposing read (a wavefront's LDS accesses take effect in issue order, so
// no barrier is needed until the final combination).
template <int D>
struct Decode {
  static constexpr int kWaves = 4;
  static constexpr int DK = D / 16, DB = D / 32;
  static constexpr int VS = D * 2 + 64;                     // V row stride (bytes), as in the general kernel
  static constexpr int VSLOT = kBc * VS;
  static constexpr int PIECES = kBc * D * 2 / 16 / 64;      // 16-byte pieces of a V tile per lane
  static constexpr int kRowsPerPiece = 64 / (D / 8);        // rows between a lane's pieces
  static constexpr int OS = D + 4;                          // row stride (floats) of a part's O^T
  static constexpr int PART_FLOATS = 32 * OS + 3 * 32;      // O^T, then shift, l and lh per query
  static constexpr int SLOTS_BYTES = kWaves * 2 * VSLOT;
  static constexpr int MERGE_BYTES = kWaves * PART_FLOATS * 4;
  static constexpr int BYTES = SLOTS_BYTES > MERGE_BYTES ? SLOTS_BYTES : MERGE_BYTES;
  static_assert(DB <= kWaves, "one d-block of the combination per wavefront");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D == 128 ? 2 : 3) void attn_decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int BH, Geom gm, float c, uint32_t qxor, uint32_t qand) {
  using Dc = Decode<D>;
  constexpr int DK = Dc::DK, DB = Dc::DB, VS = Dc::VS, PIECES = Dc::PIECES, kWaves = Dc::kWaves;
  __shared__ __attribute__((aligned(16))) char smem[Dc::BYTES];

  // range sp of the head's keys; slice sp of the partial outputs
  const int sp = blockIdx.y, bh = blockIdx.x;
  const int b0 = (int)((int64_t)gm.kn * sp / gm.nsplit), b1 = (int)((int64_t)gm.kn * (sp + 1) / gm.nsplit);
  const int kn = b1 - b0, qpos = gm.qpos - b0, N = gm.nq;
  o += ((size_t)sp * BH + bh) * N * D;
  lse += ((size_t)sp * BH + bh) * N;
  const size_t kbase = ((size_t)bh * gm.nk + gm.k0 + b0) * D;
  constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer access; reads past the range return zeros
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(k + kbase), (short)0, kn * D * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(v + kbase), (short)0, kn * D * 2, kRsrcWord3);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int kv_end = CAUSAL ? min(kn, qpos + N) : kn;  // keys past this are visible to no query
  const int nT = kv_end > 0 ? (kv_end + kBc - 1) / kBc : 0;

  // queries as the B operand (query li, dims 16 ks + 8 g ..), sign-flipped or zeroed for the scale
  bf16x8 qf[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    uint4 val = make_uint4(0, 0, 0, 0);
    if (li < N) val = *reinterpret_cast<const uint4*>(q + ((size_t)bh * N + li) * D + ks * 16 + g * 8);
    val = make_uint4((val.x ^ qxor) & qand, (val.y ^ qxor) & qand, (val.z ^ qxor) & qand, (val.w ^ qxor) & qand);
    qf[ks] = __builtin_bit_cast(bf16x8, val);
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -kInf, l = 0.f, lh = 0.f;

  // K: this lane's operand row (permuted, as in the general kernel), dims 16 ks + 8 g ..
  const int krow_off = permuted_row(li) * D * 2 + g * 16;
  // V: row-major 16-byte pieces into the wavefront's slots; transposing-read offsets
  const int vrow = lane / (D / 8), vcol = (lane % (D / 8)) * 16;
  const int grp16 = lane >> 4, l16 = lane & 15;
  const int vrd_off = (8 * (grp16 >> 1) + (l16 >> 2)) * VS + (16 * (grp16 & 1) + 4 * (l16 & 3)) * 2;
  char* const vbase = smem + w * 2 * Dc::VSLOT;
  auto load_k = [&](int t, bf16x8 (&kr)[DK]) {
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      kr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, t * kBc * D * 2 + krow_off + ks * 32, 0, 0));
  };
  auto load_v = [&](int t, uint4 (&st)[PIECES]) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i)
      st[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (t * kBc + vrow + i * Dc::kRowsPerPiece) * D * 2 + vcol, 0, 0));
  };

  bf16x8 kc[DK], kx[DK];
  uint4 vst[PIECES];
  int t = w;
  if (t < nT) {
    load_k(t, kc);
    load_v(t, vst);
  }
#pragma unroll 1
  for (int it = 0; t < nT; t += kWaves, ++it) {
    char* const slot = vbase + (it & 1) * Dc::VSLOT;
#pragma unroll
    for (int i = 0; i < PIECES; ++i)
      *reinterpret_cast<uint4*>(slot + (vrow + i * Dc::kRowsPerPiece) * VS + vcol) = vst[i];
    const bool more = t + kWaves < nT;
    if (more) {
      load_k(t + kWaves, kx);
      load_v(t + kWaves, vst);
    }
    // S^T of tile t: lane half g holds keys t*32 + (r & 7) + 8 g + 2 (r & 8) of query li
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) sc = mfma(kc[ks], qf[ks], sc);
    const int lim = (CAUSAL ? min(qpos + li, kn - 1) : kn - 1) - t * kBc - g * 8;
    float mx = -kInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if ((r & 7) + (r & 8) * 2 > lim) sc[r] = -kInf;
      mx = fmaxf(mx, sc[r]);
    }
    // online softmax with the lazy shift (moves only when the maximum exceeds it by the slack)
    const float mt = c * max_pair(mx);
    const float m_new = mt > m + kRescaleSlack ? mt : m;
    const float alpha = m_new == -kInf ? 1.f : exp2_fast(m - m_new);
    m = m_new;
    const float msub = m_new == -kInf ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = exp2_fast(fmaf(sc[r], c, -msub));
      rs += sc[r];
    }
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float hs = lh * alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 wv;
      wv.x = pack_bf16x2(sc[8 * h + 0], sc[8 * h + 1]);
      wv.y = pack_bf16x2(sc[8 * h + 2], sc[8 * h + 3]);
      wv.z = pack_bf16x2(sc[8 * h + 4], sc[8 * h + 5]);
      wv.w = pack_bf16x2(sc[8 * h + 6], sc[8 * h + 7]);
      pb[h] = __builtin_bit_cast(bf16x8, wv);
      hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.x), ones, hs, false);
      hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.y), ones, hs, false);
      hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.z), ones, hs, false);
      hs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv.w), ones, hs, false);
    }
    lh = hs;
    l = l * alpha + rs;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // O^T += V_t^T P_t^T
#pragma unroll
    for (int ch = 0; ch < DK; ++ch) {
      const int db = ch % DB, mm = ch / DB;
      const char* pa = slot + vrd_off + (mm * 16) * VS + db * 64;
      const v4i16 lo = tr_read(pa), hi = tr_read(pa + 4 * VS);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = mfma(a, pb[mm], oacc[db]);
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) kc[ks] = kx[ks];
    }
  }

  // ---- combination of the four parts (LDS reused once every wavefront is done with its slots)
  __syncthreads();
  float* const mine = reinterpret_cast<float*>(smem) + w * Dc::PART_FLOATS;
  {
    const float lt = sum_pair(l), lht = sum_pair(lh);
    if (g == 0) {
      mine[32 * Dc::OS + li] = m;
      mine[32 * Dc::OS + 32 + li] = lt;
      mine[32 * Dc::OS + 64 + li] = lht;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *reinterpret_cast<float4*>(mine + li * Dc::OS + db * 32 + 8 * a4 + 4 * g) =
            make_float4(oacc[db][4 * a4], oacc[db][4 * a4 + 1], oacc[db][4 * a4 + 2], oacc[db][4 * a4 + 3]);
  }
  __syncthreads();
  if (w < DB && li < N) {  // wavefront w writes dims 32 w .. 32 w + 31 of every query
    const float* part = reinterpret_cast<const float*>(smem);
    float mu[kWaves], f[kWaves];
    float M = -kInf;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      mu[u] = part[u * Dc::PART_FLOATS + 32 * Dc::OS + li];
      M = fmaxf(M, mu[u]);
    }
    float L = 0.f, LH = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      f[u] = mu[u] == -kInf ? 0.f : exp2_fast(mu[u] - M);
      L += f[u] * part[u * Dc::PART_FLOATS + 32 * Dc::OS + 32 + li];
      LH += f[u] * part[u * Dc::PART_FLOATS + 32 * Dc::OS + 64 + li];
    }
    // a row with no visible key in the range has l = 0: O = 0, LSE = -inf
    const float inv = LH > 0.f ? 1.f / LH : 0.f;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dcol = w * 32 + 8 * a4 + 4 * g;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < kWaves; ++u) {
        const float4 x = *reinterpret_cast<const float4*>(part + u * Dc::PART_FLOATS + li * Dc::OS + dcol);
        acc.x = fmaf(f[u], x.x, acc.x);
        acc.y = fmaf(f[u], x.y, acc.y);
        acc.z = fmaf(f[u], x.z, acc.z);
        acc.w = fmaf(f[u], x.w, acc.w);
      }
      *reinterpret_cast<float4*>(o + (size_t)li * D + dcol) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (w == 0 && g == 0) lse[li] = L > 0.f ? (M + log2_fast(L)) * kLn2 : -kInf;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_decode(const AttnArgs& a, const Geom& gm) {
  const int BH = (int)(a.B * a.H);
  const ScaleArgs sc = scale_args(a.scale);
  hipLaunchKernelGGL((attn_decode_bf16_kernel<D, CAUSAL>), dim3((unsigned)BH, (unsigned)gm.nsplit), dim3(256), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<float*>(a.o), a.lse, BH, gm, sc.c, sc.qxor,
                     sc.qand);
  return hipGetLastError();
}

// Wavefronts per workgroup (32 queries each with QB = 1): 8 at d = 128, 4 at d = 64
// (three workgroups per compute unit).  Key ranges for at most 32 queries (decode)
// go to the decode kernel above; for at most 128 queries d = 128 takes 4 as well:
// the workgroup's query block is then mostly empty rows, and smaller workgroups,
// two per compute unit, waste half as much.
template <bool PART>
hipError_t dispatch(const AttnArgs& a, const Geom& gm) {
  constexpr int QB = FA_BF16_QB;
  constexpr int W128 = QB == 1 ? 8 : 4;
  if constexpr (PART) {
    if (gm.nq <= 32) {
      if (a.d == 64) return a.causal ? launch_decode<64, true>(a, gm) : launch_decode<64, false>(a, gm);
      return a.causal ? launch_decode<128, true>(a, gm) : launch_decode<128, false>(a, gm);
    }
  }
  if (a.d == 64) return a.causal ? launch<64, true, QB, PART, 4>(a, gm) : launch<64, false, QB, PART, 4>(a, gm);
  if constexpr (PART) {
    if (gm.nq <= 128)
      return a.causal ? launch<128, true, QB, PART, 4>(a, gm) : launch<128, false, QB, PART, 4>(a, gm);
  }
  return a.causal ? launch<128, true, QB, PART, W128>(a, gm) : launch<128, false, QB, PART, W128>(a, gm);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a) {
  const int n = (int)a.N;
  return dispatch<false>(a, Geom{n, n, 0, n, 0, 1});
}

hipError_t launch_attn_bf16_partial(const AttnArgs& a, const PartialArgs& p) {
  const Geom gm{(int)a.N, (int)p.nk, (int)p.k_begin, (int)(p.k_end - p.k_begin), (int)(p.q_pos0 - p.k_begin),
                (int)p.n_splits};
  return dispatch<true>(a, gm);
}

}  // namespace fa
