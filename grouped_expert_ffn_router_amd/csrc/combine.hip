// Combine: the weighted, un-permuted sum of each token's expert outputs.
//
// Method: page "Expert parallelism and all-to-all", section "Walking through one MoE layer", step 4 (the
// expert outputs return to their token, which takes a weighted sum), and page "Expert Parallelism"
// (aiwiki), section "Implementation" (the inverse permutation restores token order).
//
// Also the pair-major form of the fused path (page "Expert parallelism and all-to-all", section "Walking through
// one MoE layer", step 4, with the routing weight already applied by the down product's epilogue): a token's k
// rows are adjacent, so the gather becomes a contiguous k-row reduction.
//
// One workgroup per token (for small batches, per span of a token's row) gathers the token's (at most k)
// expert-output rows through row_of_pair and writes its part of the output row once: no atomics, fixed slot
// order, deterministic.  Consecutive lanes take consecutive 16-byte units (4 fp32 columns), two units per
// thread and pass, with all 2k row reads issued before the first FMA (k <= 8); fp32 FMAs in slot order, one
// rounding, nontemporal stores.  128, 256 or 1024 threads per workgroup by batch size.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// Output of 4 consecutive columns starting at column c: one rounding to bf16 (8-byte store) or fp32 (16 bytes).
template <bool OUT_BF16>
MOE_DEV void store4(void* __restrict__ out, int64_t t, int H, int c, const f32x4_t& a) {
  if (OUT_BF16) {
    uint2 o;
    o.x = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
    o.y = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
    __builtin_nontemporal_store(o.x, reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + t * H + c));
    __builtin_nontemporal_store(o.y, reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + t * H + c) + 1);
  } else {
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + t * H + c));
  }
}

// Output of one 8-column unit: one rounding to bf16 (16-byte store) or an fp32 32-byte store.
template <bool OUT_BF16>
MOE_DEV void store_unit(void* __restrict__ out, int64_t t, int H, int u, const f32x4_t& a0, const f32x4_t& a1) {
  if (OUT_BF16) {
    i32x4_t o;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      o[q] = (int)f32_to_bf16_bits(a0[2 * q]) | ((int)f32_to_bf16_bits(a0[2 * q + 1]) << 16);
      o[q + 2] = (int)f32_to_bf16_bits(a1[2 * q]) | ((int)f32_to_bf16_bits(a1[2 * q + 1]) << 16);
    }
    __builtin_nontemporal_store(o, reinterpret_cast<i32x4_t*>(reinterpret_cast<uint16_t*>(out) + t * H) + u);
  } else {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + t * H + u * 8);
    __builtin_nontemporal_store(a0, dst);
    __builtin_nontemporal_store(a1, dst + 1);
  }
}

// KC > 0: k <= KC slots, unrolled so that a thread issues all of a unit's row reads before its first FMA.  Slots
// past k, and picks outside the window, read a row this token does have (weight 0, so they add an exact zero);
// a token with no pick in the window gets a zero row.  KC == 0: any k (up to 32), one slot at a time.
// SLOTS: y holds pair-major rows already multiplied by their routing weights (row t*k + j, weight 1).
template <bool OUT_BF16, int KC, bool SLOTS = false, int CT = 128>
__global__ __launch_bounds__(CT) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ rop,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      int64_t T, int k, int H, int e_lo, int E_local,
                                                      void* __restrict__ out, int slices) {
  __shared__ int s_row[32];
  __shared__ float s_w[32];
  // `slices` workgroups per token (KC > 0 only), each covering one span of the row's 16-byte units
  const int64_t t = blockIdx.x / slices;
  const int sl = blockIdx.x % slices;
  const int tid = threadIdx.x;
  if (tid < k) {
    const int e = idx[t * k + tid];
    const bool local = (unsigned)(e - e_lo) < (unsigned)E_local;
    // slots: a pair dropped by a fixed capacity (row_of_pair -1, when given) has no slot
    const bool kept = !SLOTS || rop == nullptr || rop[t * k + tid] >= 0;
    s_row[tid] = local && kept ? (SLOTS ? (int)(t * k + tid) : rop[t * k + tid]) : -1;
    s_w[tid] = SLOTS ? 1.0f : w[t * k + tid];
  }
  __syncthreads();
  const int units = H >> 3;
  if constexpr (KC > 0) {
    int safe = -1;
    for (int j = k - 1; j >= 0; --j)
      if (s_row[j] >= 0) safe = s_row[j];
    const f32x4_t* src[KC];
    float wt[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bool use = j < k && s_row[j] >= 0;
      src[j] = reinterpret_cast<const f32x4_t*>(y + (int64_t)(use ? s_row[j] : (safe < 0 ? 0 : safe)) * H);
      wt[j] = use ? s_w[j] : 0.0f;
    }
    // 16-byte units, consecutive lanes on consecutive units (each load instruction covers whole cache lines);
    // a thread takes units u and u + CT per pass, all 2 KC loads issued before the first FMA
    const int units4 = H >> 2;
    const int span = (units4 + slices - 1) / slices;
    const int ubeg = sl * span, uend = min(units4, ubeg + span);
    constexpr int NU = 2;
    for (int u0 = ubeg + tid; u0 < uend; u0 += NU * CT) {
      f32x4_t a[NU];
      bool ok[NU];
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        a[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        ok[i] = u0 + i * CT < uend;
      }
      if (safe >= 0) {
        f32x4_t v[NU][KC];
#pragma unroll
        for (int j = 0; j < KC; ++j)
#pragma unroll
          for (int i = 0; i < NU; ++i)
            v[i][j] = ok[i] ? __builtin_nontemporal_load(src[j] + u0 + i * CT) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KC; ++j)
#pragma unroll
          for (int i = 0; i < NU; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) a[i][q] = __builtin_fmaf(wt[j], v[i][j][q], a[i][q]);
      }
#pragma unroll
      for (int i = 0; i < NU; ++i)
        if (ok[i]) store4<OUT_BF16>(out, t, H, 4 * (u0 + i * CT), a[i]);
    }
  } else {
    for (int u = tid; u < units; u += blockDim.x) {
      f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int r = s_row[j];
        if (r < 0) continue;
        const float wj = s_w[j];
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(y + (int64_t)r * H + u * 8);
        const f32x4_t v0 = __builtin_nontemporal_load(src);
        const f32x4_t v1 = __builtin_nontemporal_load(src + 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a0[q] = __builtin_fmaf(wj, v0[q], a0[q]);
          a1[q] = __builtin_fmaf(wj, v1[q], a1[q]);
        }
      }
      store_unit<OUT_BF16>(out, t, H, u, a0, a1);
    }
  }
}

template <bool OUT_BF16, bool SLOTS>
static void launch_combine_k(const float* y, const int32_t* rop, const int32_t* idx, const float* w, int64_t T,
                             int k, int H, int e_lo, int E_local, void* out, hipStream_t s) {
  // Few tokens (decode-sized batches): split each row into column spans of at least 256 16-byte units so that
  // about 2048 workgroups are in flight; the one-slot-at-a-time form (k > 8) keeps one workgroup per token.
  int sl = 1;
  if (k <= 8 && T < 2048) {
    const int64_t want = (2048 + T - 1) / T;
    const int64_t most = (H / 4) / 256;
    sl = (int)(want < most ? want : most);
    if (sl < 1) sl = 1;
  }
  // Workgroup size (measured on MI355X): large batches stream best with 1024-thread workgroups (a whole
  // 4096-column row per pass: 5.9-6.2 TB/s against 5.1-5.2 with 128), column-split small batches with 256;
  // mid-sized ones keep 128.
  const dim3 g((unsigned)(T * sl));
  auto go = [&](auto kc, auto ct) {
    constexpr int KC_ = decltype(kc)::value, CT_ = decltype(ct)::value;
    hipLaunchKernelGGL((combine_kernel<OUT_BF16, KC_, SLOTS, CT_>), g, dim3(CT_), 0, s, y, rop, idx, w, T, k, H,
                       e_lo, E_local, out, KC_ == 0 ? 1 : sl);
  };
  auto by_ct = [&](auto kc) {
    if (T >= 4096)
      go(kc, std::integral_constant<int, 1024>{});
    else if (sl > 1)
      go(kc, std::integral_constant<int, 256>{});
    else
      go(kc, std::integral_constant<int, 128>{});
  };
  if (k == 1)
    by_ct(std::integral_constant<int, 1>{});
  else if (k == 2)
    by_ct(std::integral_constant<int, 2>{});
  else if (k <= 4)
    by_ct(std::integral_constant<int, 4>{});
  else if (k <= 8)
    by_ct(std::integral_constant<int, 8>{});
  else
    go(std::integral_constant<int, 0>{}, std::integral_constant<int, 128>{});
}

void launch_combine(const float* y, const int32_t* rop, const int32_t* idx, const float* w, int64_t T, int k, int H,
                    int e_lo, int E_local, void* out, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    launch_combine_k<true, false>(y, rop, idx, w, T, k, H, e_lo, E_local, out, s);
  else
    launch_combine_k<false, false>(y, rop, idx, w, T, k, H, e_lo, E_local, out, s);
}

void launch_combine_slots(const float* y_slot, const int32_t* rop, const int32_t* idx, int64_t T, int k, int H,
                          int e_lo, int E_local, void* out, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    launch_combine_k<true, true>(y_slot, rop, idx, nullptr, T, k, H, e_lo, E_local, out, s);
  else
    launch_combine_k<false, true>(y_slot, rop, idx, nullptr, T, k, H, e_lo, E_local, out, s);
}

}  // namespace moe
