// Launchers of the device kernels (internal to libmoe_ep).  Arguments are validated by the entry points.
#pragma once
#include "common.h"

namespace moe {

void launch_route_topk(const float* logits, int64_t T, int E, int k, int32_t* idx, float* w, hipStream_t s);

int64_t dispatch_tiles(int64_t T);  // count tiles of the multi-workgroup dispatch form (128 tokens each)
// Largest dispatch workspace moe_dispatch_permute_noalloc serves from its fixed per-device scratch array.
constexpr size_t DISPATCH_SCRATCH_BYTES = (size_t)1 << 20;
// Device address of this library's dispatch scratch on the device of stream s (looked up once per device).
hipError_t dispatch_scratch(hipStream_t s, void** out);
void launch_dispatch(const void* x, const float* x_scales, int esize, int64_t T, int H, const int32_t* topk_idx, int k,
                     int E, int32_t* counts, int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row,
                     void* x_perm, float* x_perm_scales, void* workspace, int capacity, hipStream_t s);

struct FfnLaunch {
  moe_dtype dtype;
  const void* x_perm;
  const float* x_perm_scales;
  const int32_t* offsets;
  int e_lo, E_local, H, F;
  int64_t R_max;
  const void *w_gate, *w_up, *w_down;  // packed
  const float *s_gate, *s_up, *s_down;
  void* h;          // [R_max][F] layer dtype
  float* h_scales;  // fp8: [R_max][F/128]
  float* y_perm;    // [R_max][H]
  float* y_part;    // down GEMM split over K: [ksplit-1][R_max][H] partial sums (workspace)
  int ksplit;
  const int32_t* gather_rows;  // gate/up gather form: token_of_row, x_perm/x_perm_scales are then x/x_scales
  float* y_slot;               // down scatter form: [T*k][H] pair-major, weighted by topk_w
  const int32_t* token_of_row;
  const int32_t* row_of_pair;
  const float* topk_w;
  int k;
  float* gu;  // gate/up training form: pre-activations [R_max][2F] (g then u), fp32
};
int ffn_down_ksplit(int64_t R_max, int E_local, int H, int F, moe_dtype dtype);
void launch_ffn_gemm1(const FfnLaunch& p, hipStream_t s);  // x_perm -> h
void launch_ffn_gemm2(const FfnLaunch& p, hipStream_t s);  // h -> y_perm

// Backward of the grouped FFN and of the routing weights (fp32 / bf16 layers); weights in natural layouts.
struct BwdLaunch {
  moe_dtype dtype;
  int64_t T, R_max;
  int H, F, k, E, e_lo, E_local;
  const void* dout;  // [T][H] layer dtype
  const int32_t *topk_idx, *offsets, *row_of_pair, *token_of_row;
  const float* topk_w;
  const void *x_perm, *h;       // forward's permuted rows and SwiGLU output (layer dtype)
  const float* gu;              // forward's pre-activations [R_max][2F] fp32
  const float* y_perm;          // forward's expert outputs [R_max][H]
  const void *w_gate, *w_up, *w_down;
  void* dx;                     // [T][H] layer dtype
  float *dw_gate, *dw_up, *dw_down, *d_topk_w, *d_logits;
  // workspace
  int32_t *por, *poff;
  float* rw;                    // routing weight of each row
  void *dO, *dgu, *whT, *dOT, *xT, *dguT;
  float* dX;
};
void launch_ffn_backward(const BwdLaunch& p, hipStream_t s);

void launch_transpose(const void* src, void* dst, int esize, int E, int K, int N, hipStream_t s);

// router logits x W_r with the top-k (one fused kernel for E <= 64; above, logits then route_topk, logits given);
// dtype code 0 f32, 1 bf16, 2 fp8 (x_scales per 128 columns)
void launch_router_topk(const void* x, const float* xs, int esize_code, int64_t T, int H, const float* W, int E, int k,
                        float* logits, int32_t* idx, float* w, hipStream_t s);
void launch_combine(const float* y, const int32_t* rop, const int32_t* idx, const float* w, int64_t T, int k, int H,
                    int e_lo, int E_local, void* out, bool out_bf16, hipStream_t s);
// pair-major slots (already weighted): out[t] = sum over local picks j of y_slot[t*k + j]
void launch_combine_slots(const float* y_slot, const int32_t* rop, const int32_t* idx, int64_t T, int k, int H,
                          int e_lo, int E_local, void* out, bool out_bf16, hipStream_t s);

}  // namespace moe
