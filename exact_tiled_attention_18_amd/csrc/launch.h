// Host-side launchers, one per kernel family.  Each validates nothing (the
// C-ABI entry points in api.hip do that) and returns the hipError_t of its
// launch.
#pragma once

#include <hip/hip_runtime.h>
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

struct QuantArgs {
  const void* x;
  uint8_t* x8;
  float* x_scale;
  const int8_t* signs;
  int64_t B, H, N, d;
  int transpose_out;
  hipStream_t stream;
};
hipError_t launch_quant_rotate_fp8(const QuantArgs& a);

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
};
hipError_t launch_attn_fp8(const Fp8AttnArgs& a);

}  // namespace fa
