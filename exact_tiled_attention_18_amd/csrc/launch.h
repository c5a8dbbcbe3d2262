// Host-side launchers, one per kernel family.  Each validates nothing (the
// C-ABI entry points in api.cpp do that) and returns the hipError_t of its
// launch.  Only runtime API types appear here, so host C++ can include it.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, H, N, d;
  int causal;
  float scale;
  hipStream_t stream;
};

hipError_t launch_attn_f32(const AttnArgs& a);
hipError_t launch_attn_bf16(const AttnArgs& a);

// Partial forward over a key range (AttnArgs.N = query rows, AttnArgs.o = float32 O).
struct PartialArgs {
  int64_t nk;       // key rows per head in k and v
  int64_t q_pos0;   // key position of query 0
  int64_t k_begin;  // first key used
  int64_t k_end;    // one past the last key used
  int64_t n_splits; // consecutive sub-ranges of [k_begin, k_end), one grid row each
};
hipError_t launch_attn_bf16_partial(const AttnArgs& a, const PartialArgs& p);

// O, LSE of the union of key ranges from n partial results.
struct MergeArgs {
  const float* o_parts;    // [n, B, H, N, d]
  const float* lse_parts;  // [n, B, H, N]
  int64_t n;
  void* o;                 // [B, H, N, d] of dtype
  float* lse;              // [B, H, N]
  int64_t B, H, N, d;
  int dtype;               // FA_F32 or FA_BF16
  hipStream_t stream;
};
hipError_t launch_merge(const MergeArgs& a);

// Backward pass (bf16): dQ, dK, dV from Q, K, V, O, dO and the saved LSE.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [B, H, N] workspace: rowsum(dO * O)
  int64_t B, H, N, d;
  int causal;
  float scale;
  hipStream_t stream;
};
hipError_t launch_attn_bwd(const BwdArgs& a);

struct QuantArgs {
  const void* x;
  uint8_t* x8;
  float* x_scale;
  const int8_t* signs;
  int64_t B, H, N, d;
  int transpose_out;
  hipStream_t stream;
  int per_tensor;  // 1: one scale (the whole tensor's amax) in every tile entry
};
hipError_t launch_quant_rotate_fp8(const QuantArgs& a);

// Q and K (rotated when signs is set) and V (transposed codes) in one launch.
struct QkvQuantArgs {
  const void* x[3];   // q, k, v
  uint8_t* x8[3];     // q8, k8 ([B, H, N, d]), v8t ([B, H, d, N64])
  float* scale[3];
  const int8_t* signs;
  int64_t B, H, N, d;
  hipStream_t stream;
};
hipError_t launch_quant_qkv_fp8(const QkvQuantArgs& a);

struct Fp8AttnArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  void* o;
  float* lse;
  int64_t B, H, N, d;
  int causal;
  float scale;
  hipStream_t stream;
  int p_bf16;  // 1: probabilities in bf16, P V on the bf16 matrix core
};
hipError_t launch_attn_fp8(const Fp8AttnArgs& a);

// Device address of fa_bwd_noalloc's static workspace on the current device
// (FA_BWD_NOALLOC_MAX_ROWS floats; looked up once per device, then cached).
hipError_t scratch_address(void** out);

}  // namespace fa
