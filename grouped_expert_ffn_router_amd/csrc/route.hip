// Routing: softmax top-k over each token's router logits (one token per group of G lanes of a wavefront), and
// the router's linear map x W_r in front of it (one kernel with the selection up to 64 experts; above, a tiled
// logits kernel followed by the selection).
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// k rounds of a group-wide arg-max under (value desc, id asc) over the lanes' VPL values (expert of value j in
// lane g: g + j*G; taken bit j set for entries that do not exist); slot r's pick and weight end in lane r.
template <int G, int VPL>
MOE_DEV void group_topk(const float (&v)[VPL], uint32_t taken, int g, int k, int& my_e, float& my_w) {
  float my_v = 0.0f, v0 = 0.0f;
  my_e = 0;
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
  my_w = (float)(ex / s);
}

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
  int my_e;
  float my_w;
  group_topk<G, VPL>(v, taken, g, k, my_e, my_w);
  if (valid && g < k) {
    topk_idx[t * k + g] = my_e;
    topk_w[t * k + g] = my_w;
  }
}

// OCP e4m3 code -> value, from the format: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, exponent field 0
// holding the subnormals m * 2^-9 (the quantiser never writes the NaN codes).  Exact in fp32.
MOE_DEV float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u, sg = (c & 0x80u) << 24;
  const float mag = ex ? __uint_as_float(((ex + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | sg);
}

// 8 consecutive x values of one token in their stored form (f32, bf16, or e4m3 codes with the block scale);
// value(j) decodes the j-th exactly (j a compile-time constant after unrolling)
template <int DT>
struct XRaw;
template <>
struct XRaw<0> {
  float4 u0, u1;
  MOE_DEV void load(const uint8_t* x, const float*, int64_t t, int H, int h) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + t * H + h);
    u0 = p[0];
    u1 = p[1];
  }
  MOE_DEV float value(int j) const {  // selects between copies, not between members, so x stays in registers
    const float a = u0.x, b = u0.y, c = u0.z, d = u0.w, e = u1.x, f = u1.y, g = u1.z, i = u1.w;
    const float lo = (j & 3) == 0 ? a : ((j & 3) == 1 ? b : ((j & 3) == 2 ? c : d));
    const float hi = (j & 3) == 0 ? e : ((j & 3) == 1 ? f : ((j & 3) == 2 ? g : i));
    return j < 4 ? lo : hi;
  }
};
template <>
struct XRaw<1> {
  uint4 u;
  MOE_DEV void load(const uint8_t* x, const float*, int64_t t, int H, int h) {
    u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + t * H + h);
  }
  MOE_DEV float value(int j) const {
    const uint32_t a = u.x, b = u.y, c = u.z, e = u.w;
    const uint32_t d = j < 2 ? a : (j < 4 ? b : (j < 6 ? c : e));
    return __uint_as_float((j & 1) ? (d & 0xffff0000u) : (d << 16));
  }
};
template <>
struct XRaw<2> {
  uint2 u;
  float sc;
  MOE_DEV void load(const uint8_t* x, const float* xs, int64_t t, int H, int h) {
    u = *reinterpret_cast<const uint2*>(x + t * H + h);
    sc = xs[t * (H >> 7) + (h >> 7)];
  }
  MOE_DEV float value(int j) const {
    const uint32_t a = u.x, b = u.y;
    return e4m3_value(((j < 4 ? a : b) >> (8 * (j & 3))) & 0xffu) * sc;
  }
};

// Sum over the 16 lanes of each row of the wavefront, by DPP (xor 1, xor 2, half-row mirror, row mirror).  Every
// lane of a row ends with the same bits: each step adds two equal-shaped partial sums, and fp32 addition commutes.
MOE_DEV float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// Router logits x W_r fused with the top-k (E <= EP <= 64).  A workgroup owns TPL = 64 / EP tokens (at least 1)
// and NW waves; H is cut into 512-column chunks, chunk c going to wave c % NW, and lane l of a wave takes
// columns 8l .. 8l+7 of each of its chunks for all TPL tokens, so W_r rows are loaded once per workgroup and
// a token's load instruction covers 1 KiB of its row.  Each lane runs fp32 FMAs over its columns in ascending
// order; the 64 lanes are summed as four 16-lane rows (DPP), and the 4 NW row sums in (wave, row) order through
// LDS.  Any summation order keeps the |error| <= (H+2) 2^-24 sum|x w| bound of an fp32 dot product; this one is
// fixed, so a token's logits do not depend on T or on where the token sits.  The selection is
// route_topk_kernel's (one wave per token), so the routing equals moe_route_topk's on the returned logits.
template <int DT, int EP, int NW, bool FULL>
__global__ __launch_bounds__(64 * NW) void router_topk_kernel(const uint8_t* __restrict__ x,
                                                              const float* __restrict__ xs, int64_t T, int H,
                                                              const float* __restrict__ W, int E, int k,
                                                              float* __restrict__ logits,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_w) {
  constexpr int TPL = EP >= 64 ? 1 : 64 / EP;
  constexpr int NV = TPL * EP;  // partial sums per lane, token-major
  __shared__ float s_p[NW * 4 * NV];  // [wave][row][token][expert]
  const int lane = threadIdx.x & 63;
  const int wv = uniform_int(threadIdx.x >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * TPL;
  int64_t tr[TPL];  // tail tokens recompute the last token and store nothing
#pragma unroll
  for (int q = 0; q < TPL; ++q) tr[q] = t0 + q < T ? t0 + q : T - 1;
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
  for (int h = wv * 512 + lane * 8; h < H; h += NW * 512) {
    XRaw<DT> xr[TPL];
#pragma unroll
    for (int q = 0; q < TPL; ++q) xr[q].load(x, xs, tr[q], H, h);
    // whole rows of 16-byte W_r loads: all 8 columns at once; otherwise 2 at a time (register pressure)
    constexpr int JU = (FULL && DT != 2) ? 8 : 2;
#pragma unroll JU
    for (int j = 0; j < 8; ++j) {
      const float* wr = W + (int64_t)(h + j) * E;
      float wrow[EP];
      if constexpr (FULL) {
#pragma unroll
        for (int e = 0; e < EP; e += 4) {
          const float4 w4 = *reinterpret_cast<const float4*>(wr + e);
          wrow[e] = w4.x, wrow[e + 1] = w4.y, wrow[e + 2] = w4.z, wrow[e + 3] = w4.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) wrow[e] = e < E ? wr[e] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < TPL; ++q) {
        const float xj = xr[q].value(j);
#pragma unroll
        for (int e = 0; e < EP; ++e) acc[q * EP + e] = __builtin_fmaf(xj, wrow[e], acc[q * EP + e]);
      }
    }
  }
  // 16-lane row sums; lane c of row r stores the values v = c (mod 16)
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const float sv = row16_sum(acc[v]);
    if ((v & 15) == c) s_p[(wv * 4 + r) * NV + v] = sv;
  }
  __syncthreads();
  // the 4 NW row sums in (wave, row) order
  constexpr int NL = (NV + 64 * NW - 1) / (64 * NW);
  float lg[NL];
#pragma unroll
  for (int i2 = 0; i2 < NL; ++i2) {
    const int v = threadIdx.x + i2 * 64 * NW;
    if (v < NV) {
      float sum = s_p[v];
      for (int p = 1; p < 4 * NW; ++p) sum += s_p[p * NV + v];
      lg[i2] = sum;
      const int q = v / EP, e = v % EP;
      if (logits != nullptr && e < E && t0 + q < T) logits[(t0 + q) * E + e] = sum;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i2 = 0; i2 < NL; ++i2) {
    const int v = threadIdx.x + i2 * 64 * NW;
    if (v < NV) s_p[v] = lg[i2];
  }
  __syncthreads();
  // selection: wave w routes the workgroup's tokens w, w + NW, ...; lane g holds expert g
  for (int q = wv; q < TPL && t0 + q < T; q += NW) {
    const bool real = lane < E;
    const float v[1] = {real ? s_p[q * EP + lane] : -INFINITY};
    int my_e;
    float my_w;
    group_topk<64, 1>(v, real ? 0u : 1u, lane, k, my_e, my_w);
    if (lane < k) {
      topk_idx[(t0 + q) * k + lane] = my_e;
      topk_w[(t0 + q) * k + lane] = my_w;
    }
  }
}

template <int DT, int EP>
static void launch_router_ep(const void* x, const float* xs, int64_t T, int H, const float* W, int E, int k,
                             float* logits, int32_t* idx, float* w, hipStream_t s) {
  constexpr int NW = 8;
  constexpr int TPL = EP >= 64 ? 1 : 64 / EP;
  const int64_t blocks = (T + TPL - 1) / TPL;
  // E == EP with a 16-byte aligned W_r: whole rows read as 16-byte vectors
  if (E == EP && (reinterpret_cast<uintptr_t>(W) & 15) == 0)
    hipLaunchKernelGGL((router_topk_kernel<DT, EP, NW, true>), dim3((unsigned)blocks), dim3(64 * NW), 0, s,
                       reinterpret_cast<const uint8_t*>(x), xs, T, H, W, E, k, logits, idx, w);
  else
    hipLaunchKernelGGL((router_topk_kernel<DT, EP, NW, false>), dim3((unsigned)blocks), dim3(64 * NW), 0, s,
                       reinterpret_cast<const uint8_t*>(x), xs, T, H, W, E, k, logits, idx, w);
}

// Router logits for any E (used above 64 experts, followed by route_topk_kernel): a workgroup computes a tile of
// 16 TPT tokens x RL_TE experts, each thread TPT tokens x 4 experts; 32-column chunks of x (decoded to fp32) and
// of W_r are staged in LDS and every output runs its fp32 FMAs in ascending h, so a token's logits do not depend
// on T, its position or the tile it falls in, and |error| <= (H+2) 2^-24 sum|x w|.
constexpr int RL_TE = 64, RL_HC = 32;
template <int DT, int TPT>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint8_t* __restrict__ x, const float* __restrict__ xs,
                                                            int64_t T, int H, const float* __restrict__ W, int E,
                                                            float* __restrict__ logits) {
  constexpr int RL_TT = 16 * TPT;
  __shared__ float s_x[RL_TT][RL_HC + 1];
  __shared__ float s_w[RL_HC][RL_TE + 4];
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;  // tokens TPT ty .. +TPT, experts 4 tx .. +4 of the tile
  const int64_t t0 = (int64_t)blockIdx.x * RL_TT;
  const int e0 = blockIdx.y * RL_TE;
  float acc[TPT][4];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  // the next chunk's x groups (8 consecutive columns, TPT / 4 per thread) and W_r values (8 per thread) are
  // loaded into registers while the current chunk is multiplied out of LDS
  constexpr int NG = TPT / 4;
  XRaw<DT> xr[NG];
  bool xok[NG];
  float wreg[8];
  auto fetch = [&](int h0) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int idx = tid + g * 256;
      const int64_t t = t0 + (idx >> 2);
      const int h = h0 + (idx & 3) * 8;
      xok[g] = t < T && h < H;  // H % 8 == 0: a group is whole or absent
      if (xok[g]) xr[g].load(x, xs, t, H, h);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int idx = tid + g * 256;
      const int h = h0 + (idx >> 6), e = e0 + (idx & 63);
      wreg[g] = (h < H && e < E) ? W[(int64_t)h * E + e] : 0.0f;
    }
  };
  fetch(0);
  for (int h0 = 0; h0 < H; h0 += RL_HC) {
    __syncthreads();  // the previous chunk's reads of LDS are done
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int idx = tid + g * 256;
      const int tq = idx >> 2, c8 = (idx & 3) * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) s_x[tq][c8 + q] = xok[g] ? xr[g].value(q) : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int idx = tid + g * 256;
      s_w[idx >> 6][idx & 63] = wreg[g];
    }
    __syncthreads();
    if (h0 + RL_HC < H) fetch(h0 + RL_HC);
#pragma unroll 4
    for (int kk = 0; kk < RL_HC; ++kk) {
      float a[TPT], b[4];
#pragma unroll
      for (int i = 0; i < TPT; ++i) a[i] = s_x[ty * TPT + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = s_w[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = t0 + ty * TPT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[t * E + e] = acc[i][j];
    }
  }
}

template <int DT>
static void launch_router_dt(const void* x, const float* xs, int64_t T, int H, const float* W, int E, int k,
                             float* logits, int32_t* idx, float* w, hipStream_t s) {
  if (E <= 8)
    launch_router_ep<DT, 8>(x, xs, T, H, W, E, k, logits, idx, w, s);
  else if (E <= 16)
    launch_router_ep<DT, 16>(x, xs, T, H, W, E, k, logits, idx, w, s);
  else if (E <= 32)
    launch_router_ep<DT, 32>(x, xs, T, H, W, E, k, logits, idx, w, s);
  else
    launch_router_ep<DT, 64>(x, xs, T, H, W, E, k, logits, idx, w, s);
}

void launch_router_topk(const void* x, const float* xs, int esize_code, int64_t T, int H, const float* W, int E, int k,
                        float* logits, int32_t* idx, float* w, hipStream_t s) {
  if (E > 64) {  // logits (given) from the tiled kernel, then the selection of moe_route_topk
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    const unsigned ge = (unsigned)((E + RL_TE - 1) / RL_TE);
    // 128-token tiles when they give a few hundred workgroups, 64-token tiles (twice as many) otherwise
    const bool big = ((T + 127) / 128) * ge >= 256;
    auto go = [&](auto tpt) {
      constexpr int TPT = decltype(tpt)::value;
      const dim3 grid((unsigned)((T + 16 * TPT - 1) / (16 * TPT)), ge);
      if (esize_code == 0)
        hipLaunchKernelGGL((router_logits_kernel<0, TPT>), grid, dim3(256), 0, s, xb, xs, T, H, W, E, logits);
      else if (esize_code == 1)
        hipLaunchKernelGGL((router_logits_kernel<1, TPT>), grid, dim3(256), 0, s, xb, xs, T, H, W, E, logits);
      else
        hipLaunchKernelGGL((router_logits_kernel<2, TPT>), grid, dim3(256), 0, s, xb, xs, T, H, W, E, logits);
    };
    if (big)
      go(std::integral_constant<int, 8>{});
    else
      go(std::integral_constant<int, 4>{});
    launch_route_topk(logits, T, E, k, idx, w, s);
    return;
  }
  if (esize_code == 0)
    launch_router_dt<0>(x, xs, T, H, W, E, k, logits, idx, w, s);
  else if (esize_code == 1)
    launch_router_dt<1>(x, xs, T, H, W, E, k, logits, idx, w, s);
  else
    launch_router_dt<2>(x, xs, T, H, W, E, k, logits, idx, w, s);
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
