// Internal device/host helpers of libmoe_ep (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_ep.h"

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8]).
#define MOE_WAIT_VMCNT0 0x0F70

MOE_DEV int lane_id() { return (int)__lane_id(); }

// gfx950 builtins behind plain device functions: templates call these, so the host compilation pass of a
// template kernel never sees a target-specific builtin.
MOE_DEV f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
MOE_DEV f32x16_t mfma_32x32x2_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// OCP e4m3 x OCP e4m3 (format code 0 for both operands), unit E8M0 scales (127 = 2^0)
MOE_DEV f32x16_t mfma_32x32x64_e4m3(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// Direct global -> LDS loads: lane L's bytes land at lds + L * bytes.
MOE_DEV void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}
MOE_DEV void load_lds4(const void* g, void* lds) { __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 4, 0, 0); }
MOE_DEV void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(MOE_WAIT_VMCNT0); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion).
MOE_DEV uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Two fp32 -> two OCP e4m3 codes (round to nearest even).  The hardware conversion does not saturate, so
// values are clamped to the largest finite magnitude first.
MOE_DEV uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

MOE_DEV float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Host-side launch bookkeeping shared by the entry points.
namespace moe {
void set_error(const char* fmt, ...);
moe_status launch_status(const char* what);
}  // namespace moe
