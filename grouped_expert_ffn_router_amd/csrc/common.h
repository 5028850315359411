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
// 16 x 16 x 128 form: lane l holds row (A) / column (B) l % 16 and 32 of the 128 reduction bytes (group l / 16);
// result element u of lane l is row 4 (l / 16) + u, column l % 16.
MOE_DEV f32x4_t mfma_16x16x128_e4m3(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// Direct global -> LDS loads: lane L's bytes land at lds + L * bytes (lds must be the same for the whole
// wavefront).  Written as inline assembly so the compiler does not treat them as LDS writes that later LDS
// reads of the other pipeline buffer must wait for; they have no register outputs, and every consumer waits
// for them explicitly (s_waitcnt vmcnt(0) then a workgroup barrier) before reading the buffer they fill.
MOE_DEV uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
}
// Source address = a wavefront-uniform 64-bit base (scalar registers) + this lane's 32-bit byte offset, so a
// load keeps one vector register per lane instead of a 64-bit pointer.
MOE_DEV int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
MOE_DEV const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
MOE_DEV void load_lds16(const void* base, uint32_t off, void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_addr(lds)));
}
MOE_DEV void load_lds4(const void* base, uint32_t off, void* lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_addr(lds)));
}
MOE_DEV void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(MOE_WAIT_VMCNT0); }
// Wait until at most N vector-memory loads of this wavefront are outstanding.  gfx9 s_waitcnt encoding: vmcnt[3:0]
// in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt (bits 6:4) and lgkmcnt (bits 11:8) left at their maxima.
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// No instruction moves across this point during scheduling.
MOE_DEV void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Scheduling groups (masks: 0x008 MFMA, 0x100 LDS read): one LDS read followed by n MFMAs.
MOE_DEV void sched_ds1_mfma1() {
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}
MOE_DEV void sched_ds1_mfma2() {
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}
MOE_DEV void sched_ds1_mfma4() {
  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

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

// Inclusive scan of one value per lane across a wavefront.
MOE_DEV int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
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
