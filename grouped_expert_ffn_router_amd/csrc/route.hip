// Routing: softmax top-k over each token's router logits (one token per group of G lanes of a wavefront).
//
// Method: page "Expert parallelism and all-to-all", section "Walking through one MoE layer", step 1 (every
// token gets (expert, weight) picks); the selection rule is logit descending with ties to the lower expert
// id, on the fp32 logits, and the weights are the softmax restricted to the k picks, renormalised.
//
// Each lane of a G-lane group holds VPL logits (experts g, g + G, g + 2G, ...).  k rounds of a group-wide
// arg-max under the key (value desc, id asc) pick the experts in slot order; the lane that owns the winner
// marks it taken.  Slot r's pick ends in lane r of the group (k <= G always holds: G >= E for E <= 64, and
// G = 64 >= 32 >= k otherwise).  Weights: exp(l_r - l_0) in fp64, a butterfly sum (every lane ends with the
// same bits), one fp64 division, one rounding to fp32.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moe {

template <int G, int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                         int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int g = lane % G;
  const int64_t t = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const bool valid = t < T;

  float v[VPL];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = g + j * G;
    const bool real = valid && e < E;
    v[j] = real ? logits[t * E + e] : -INFINITY;
    if (!real) taken |= 1u << j;
  }

  float my_v = 0.0f, v0 = 0.0f;
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = INT_MAX;  // sentinel: loses to every real entry, including a real -inf logit
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = g + j * G;
      if (!((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < be))) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be != INT_MAX && be % G == g) taken |= 1u << (be / G);
    if (r == 0) v0 = bv;
    if (g == r) {
      my_v = bv;
      my_e = be;
    }
  }

  const double ex = (g < k) ? exp((double)my_v - (double)v0) : 0.0;
  double s = ex;
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (valid && g < k) {
    topk_idx[t * k + g] = my_e;
    topk_w[t * k + g] = (float)(ex / s);
  }
}

template <int G, int VPL>
static void launch_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const int64_t tok_per_block = 4 * (64 / G);
  const int64_t blocks = (T + tok_per_block - 1) / tok_per_block;
  hipLaunchKernelGGL((route_topk_kernel<G, VPL>), dim3((unsigned)blocks), dim3(256), 0, s, logits, T, E, k, idx, w);
}

void launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  if (E <= 1)
    launch_route<1, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 2)
    launch_route<2, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 4)
    launch_route<4, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 8)
    launch_route<8, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 16)
    launch_route<16, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 32)
    launch_route<32, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 64)
    launch_route<64, 1>(logits, T, E, k, idx, w, s);
  else if (E <= 128)
    launch_route<64, 2>(logits, T, E, k, idx, w, s);
  else if (E <= 256)
    launch_route<64, 4>(logits, T, E, k, idx, w, s);
  else if (E <= 512)
    launch_route<64, 8>(logits, T, E, k, idx, w, s);
  else
    launch_route<64, 16>(logits, T, E, k, idx, w, s);
}

}  // namespace moe
