// Recording stand-ins for the launchers of launch.h: the C-ABI validation code
// (api.cpp) links against these in the host sanitizer build, so every entry point
// can be driven on a machine without a GPU and every launch it would make counted.
#include "fake_launch.h"

namespace fake {
int launches = 0;
const char* last = "";
int64_t last_B = -1, last_H = -1, last_N = -1, last_d = -1;
const void* last_ws = nullptr;
hipError_t next_status = hipSuccess;
hipError_t scratch_status = hipSuccess;
alignas(256) float scratch_stand_in[64];

static hipError_t record(const char* name, int64_t B, int64_t H, int64_t N, int64_t d) {
  ++launches;
  last = name;
  last_B = B, last_H = H, last_N = N, last_d = d;
  return next_status;
}
}  // namespace fake

namespace fa {
hipError_t launch_attn_f32(const AttnArgs& a) { return fake::record("attn_f32", a.B, a.H, a.N, a.d); }
hipError_t launch_attn_bf16(const AttnArgs& a) { return fake::record("attn_bf16", a.B, a.H, a.N, a.d); }
hipError_t launch_attn_bf16_partial(const AttnArgs& a, const PartialArgs&) {
  return fake::record("attn_bf16_partial", a.B, a.H, a.N, a.d);
}
hipError_t launch_merge(const MergeArgs& a) { return fake::record("merge", a.B, a.H, a.N, a.d); }
hipError_t launch_attn_bwd(const BwdArgs& a) {
  fake::last_ws = a.delta;
  return fake::record("attn_bwd", a.B, a.H, a.N, a.d);
}
hipError_t launch_quant_rotate_fp8(const QuantArgs& a) {
  return fake::record(a.per_tensor ? "quant_tensor" : "quant_tile", a.B, a.H, a.N, a.d);
}
hipError_t launch_quant_qkv_fp8(const QkvQuantArgs& a) { return fake::record("quant_qkv", a.B, a.H, a.N, a.d); }
hipError_t launch_attn_fp8(const Fp8AttnArgs& a) {
  return fake::record(a.p_bf16 ? "attn_fp8_pbf16" : "attn_fp8", a.B, a.H, a.N, a.d);
}
hipError_t scratch_address(void** out) {
  if (fake::scratch_status != hipSuccess) return fake::scratch_status;
  *out = fake::scratch_stand_in;
  return hipSuccess;
}
}  // namespace fa
