// C-ABI entry points of libmoe_ep: argument validation on the host (nothing is enqueued unless every
// argument is valid), then kernel launches on the caller's stream.  No entry point synchronises, allocates or
// reads device memory on the host.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"
#include "kernels.h"

namespace moe {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

moe_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static int dtype_bytes(moe_dtype d) { return d == MOE_DTYPE_F32 ? 4 : d == MOE_DTYPE_BF16 ? 2 : 1; }
static bool dtype_ok(int d) { return d == MOE_DTYPE_F32 || d == MOE_DTYPE_BF16 || d == MOE_DTYPE_FP8_E4M3; }

#define FAIL(code, ...)      \
  do {                       \
    set_error(__VA_ARGS__);  \
    return code;             \
  } while (0)
#define REQ_PTR(p, align, name)                                                          \
  do {                                                                                   \
    if ((p) == nullptr) FAIL(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);           \
    if (!aligned((p), (align))) FAIL(MOE_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, name, (int)(align)); \
  } while (0)

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

int moe_abi_version(void) { return MOE_EP_ABI_VERSION; }

const char* moe_last_error(void) { return g_err; }

uint64_t moe_payload_bytes(int64_t tokens, int32_t k, int32_t H, int32_t bytes_per_elem) {
  if (tokens < 0 || k < 0 || H < 0 || bytes_per_elem < 0) return 0;
  return 2ull * (uint64_t)k * (uint64_t)H * (uint64_t)bytes_per_elem * (uint64_t)tokens;
}

moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w,
                          moe_stream stream) {
  const char* fn = "moe_route_topk";
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (E < 1 || E > 1024) FAIL(MOE_ERR_INVALID_ARG, "%s: E = %d outside [1, 1024]", fn, E);
  if (k < 1 || k > E || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, min(E, 32)]", fn, k);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (T == 0) return MOE_OK;
  REQ_PTR(logits, 4, "logits");
  REQ_PTR(topk_idx, 4, "topk_idx");
  REQ_PTR(topk_w, 4, "topk_w");
  launch_route_topk(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_router_topk(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                           const float* w_router, int32_t E, int32_t k, float* logits, int32_t* topk_idx,
                           float* topk_w, moe_stream stream) {
  const char* fn = "moe_router_topk";
  if (!dtype_ok(x_dtype)) FAIL(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)x_dtype);
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (E < 1 || E > 1024) FAIL(MOE_ERR_INVALID_ARG, "%s: E = %d outside [1, 1024]", fn, E);
  if (E > 64 && T > 0 && logits == nullptr)
    FAIL(MOE_ERR_INVALID_ARG, "%s: E = %d > 64 needs the logits buffer (the selection reads it back)", fn, E);
  if (k < 1 || k > E || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, min(E, 32)]", fn, k);
  const bool fp8 = x_dtype == MOE_DTYPE_FP8_E4M3;
  if (H <= 0 || H % (fp8 ? 128 : 8))
    FAIL(MOE_ERR_INVALID_ARG, "%s: H = %d must be a positive multiple of %d", fn, H, fp8 ? 128 : 8);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (T == 0) return MOE_OK;
  REQ_PTR(x, 16, "x");
  if (fp8) REQ_PTR(x_scales, 4, "x_scales");
  REQ_PTR(w_router, 4, "w_router");
  if (logits != nullptr && !aligned(logits, 4)) FAIL(MOE_ERR_INVALID_ARG, "%s: logits is not 4-byte aligned", fn);
  REQ_PTR(topk_idx, 4, "topk_idx");
  REQ_PTR(topk_w, 4, "topk_w");
  const int code = x_dtype == MOE_DTYPE_F32 ? 0 : (x_dtype == MOE_DTYPE_BF16 ? 1 : 2);
  launch_router_topk(x, fp8 ? x_scales : nullptr, code, T, H, w_router, E, k, logits, topk_idx, topk_w,
                     (hipStream_t)stream);
  return launch_status(fn);
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return align256((size_t)E * (size_t)dispatch_tiles(T) * sizeof(int32_t)) +
         align256((size_t)(E + 1) * sizeof(int32_t)) + 256;
}

static moe_status dispatch_impl(const char* fn, const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T,
                                int32_t H, const int32_t* topk_idx, int32_t k, int32_t E, int32_t capacity,
                                int32_t* counts, int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row,
                                void* x_perm, float* x_perm_scales, void* workspace, size_t workspace_bytes,
                                moe_stream stream) {
  if (!dtype_ok(x_dtype)) FAIL(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)x_dtype);
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (E < 1 || E > 1024) FAIL(MOE_ERR_INVALID_ARG, "%s: E = %d outside [1, 1024]", fn, E);
  if (k < 1 || k > E || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, min(E, 32)]", fn, k);
  if (H <= 0 || H % 128) FAIL(MOE_ERR_INVALID_ARG, "%s: H = %d must be a positive multiple of 128", fn, H);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  REQ_PTR(counts, 4, "counts");
  REQ_PTR(offsets, 4, "offsets");
  const bool fp8 = x_dtype == MOE_DTYPE_FP8_E4M3;
  const bool gather = x_perm != nullptr;  // NULL: counts, offsets and the permutation only
  if (T > 0) {
    REQ_PTR(topk_idx, 4, "topk_idx");
    REQ_PTR(row_of_pair, 4, "row_of_pair");
    REQ_PTR(token_of_row, 4, "token_of_row");
    if (gather) {
      REQ_PTR(x, 16, "x");
      REQ_PTR(x_perm, 16, "x_perm");
      if (fp8) {
        REQ_PTR(x_scales, 4, "x_scales");
        REQ_PTR(x_perm_scales, 4, "x_perm_scales");
      }
    }
  }
  const size_t need = moe_dispatch_workspace_bytes(T, k, E);
  if (workspace == nullptr) {  // the fixed scratch of moe_dispatch_permute_noalloc
    if (need > DISPATCH_SCRATCH_BYTES)
      FAIL(MOE_ERR_WORKSPACE, "%s: T = %lld, k = %d, E = %d need %zu bytes of scratch, more than the fixed %zu", fn,
           (long long)T, k, E, need, DISPATCH_SCRATCH_BYTES);
    const hipError_t e = dispatch_scratch((hipStream_t)stream, &workspace);
    if (e != hipSuccess) FAIL(MOE_ERR_DEVICE, "%s: scratch address lookup failed: %s", fn, hipGetErrorString(e));
  } else if (workspace_bytes < need || !aligned(workspace, 256)) {
    FAIL(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, need, workspace_bytes);
  }
  launch_dispatch(x, fp8 && gather ? x_scales : nullptr, dtype_bytes(x_dtype), T, H, topk_idx, k, E, counts, offsets,
                  row_of_pair, token_of_row, x_perm, fp8 && gather ? x_perm_scales : nullptr, workspace, capacity,
                  (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_dispatch_permute(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                                const int32_t* topk_idx, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                                int32_t* row_of_pair, int32_t* token_of_row, void* x_perm, float* x_perm_scales,
                                void* workspace, size_t workspace_bytes, moe_stream stream) {
  if (workspace == nullptr)
    FAIL(MOE_ERR_WORKSPACE, "moe_dispatch_permute: workspace is NULL (needs %zu bytes)",
         moe_dispatch_workspace_bytes(T, k, E));
  return dispatch_impl("moe_dispatch_permute", x, x_scales, x_dtype, T, H, topk_idx, k, E, 0, counts, offsets,
                       row_of_pair, token_of_row, x_perm, x_perm_scales, workspace, workspace_bytes, stream);
}

moe_status moe_dispatch_permute_noalloc(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                                        const int32_t* topk_idx, int32_t k, int32_t E, int32_t* counts,
                                        int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row, void* x_perm,
                                        float* x_perm_scales, moe_stream stream) {
  // workspace NULL: every argument is validated first, then the size against the fixed scratch, then the
  // scratch's device address is looked up (once per device)
  return dispatch_impl("moe_dispatch_permute_noalloc", x, x_scales, x_dtype, T, H, topk_idx, k, E, 0, counts,
                       offsets, row_of_pair, token_of_row, x_perm, x_perm_scales, nullptr, 0, stream);
}

moe_status moe_dispatch_permute_capacity(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T,
                                         int32_t H, const int32_t* topk_idx, int32_t k, int32_t E, int32_t capacity,
                                         int32_t* counts, int32_t* offsets, int32_t* row_of_pair,
                                         int32_t* token_of_row, void* x_perm, float* x_perm_scales, void* workspace,
                                         size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_dispatch_permute_capacity";
  if (capacity < 1) FAIL(MOE_ERR_INVALID_ARG, "%s: capacity = %d < 1", fn, capacity);
  if (workspace == nullptr)
    FAIL(MOE_ERR_WORKSPACE, "%s: workspace is NULL (needs %zu bytes)", fn, moe_dispatch_workspace_bytes(T, k, E));
  return dispatch_impl(fn, x, x_scales, x_dtype, T, H, topk_idx, k, E, capacity, counts, offsets, row_of_pair,
                       token_of_row, x_perm, x_perm_scales, workspace, workspace_bytes, stream);
}

static size_t ffn_matrix_bytes(const moe_ffn_weights* w) {
  return (size_t)w->E_local * (size_t)w->H * (size_t)w->F * (size_t)dtype_bytes(w->dtype);
}

static moe_status check_weights(const char* fn, const moe_ffn_weights* w) {
  if (w == nullptr) FAIL(MOE_ERR_INVALID_ARG, "%s: weights descriptor is NULL", fn);
  if (!dtype_ok(w->dtype)) FAIL(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)w->dtype);
  if (w->layout != MOE_LAYOUT_NATURAL && w->layout != MOE_LAYOUT_PACKED)
    FAIL(MOE_ERR_INVALID_ARG, "%s: unknown layout %d", fn, (int)w->layout);
  if (w->E_local < 1) FAIL(MOE_ERR_INVALID_ARG, "%s: E_local = %d < 1", fn, w->E_local);
  if (w->H <= 0 || w->H % 128 || w->F <= 0 || w->F % 128 || w->H > 65536 || w->F > 65536)
    FAIL(MOE_ERR_INVALID_ARG, "%s: H = %d and F = %d must be multiples of 128 in [128, 65536]", fn, w->H, w->F);
  REQ_PTR(w->w_gate, 16, "w_gate");
  REQ_PTR(w->w_up, 16, "w_up");
  REQ_PTR(w->w_down, 16, "w_down");
  if (w->dtype == MOE_DTYPE_FP8_E4M3) {
    REQ_PTR(w->s_gate, 4, "s_gate");
    REQ_PTR(w->s_up, 4, "s_up");
    REQ_PTR(w->s_down, 4, "s_down");
  }
  return MOE_OK;
}

size_t moe_pack_ffn_weights_bytes(const moe_ffn_weights* src) {
  if (src == nullptr || src->E_local < 1 || src->H < 1 || src->F < 1 || !dtype_ok(src->dtype)) return 0;
  return 3 * align256(ffn_matrix_bytes(src));
}

moe_status moe_pack_ffn_weights(const moe_ffn_weights* src, void* dst, size_t dst_bytes, moe_ffn_weights* packed,
                                moe_stream stream) {
  const char* fn = "moe_pack_ffn_weights";
  const moe_status st = check_weights(fn, src);
  if (st != MOE_OK) return st;
  if (src->layout != MOE_LAYOUT_NATURAL) FAIL(MOE_ERR_INVALID_ARG, "%s: source must be MOE_LAYOUT_NATURAL", fn);
  if (packed == nullptr) FAIL(MOE_ERR_INVALID_ARG, "%s: packed descriptor is NULL", fn);
  const size_t need = moe_pack_ffn_weights_bytes(src);
  if (dst == nullptr || dst_bytes < need || !aligned(dst, 256))
    FAIL(MOE_ERR_INVALID_ARG, "%s: dst needs %zu bytes, 256-byte aligned (got %zu)", fn, need, dst_bytes);
  const size_t mb = align256(ffn_matrix_bytes(src));
  uint8_t* d = reinterpret_cast<uint8_t*>(dst);
  const int es = dtype_bytes(src->dtype);
  hipStream_t s = (hipStream_t)stream;
  launch_transpose(src->w_gate, d, es, src->E_local, src->H, src->F, s);
  launch_transpose(src->w_up, d + mb, es, src->E_local, src->H, src->F, s);
  launch_transpose(src->w_down, d + 2 * mb, es, src->E_local, src->F, src->H, s);
  *packed = *src;
  packed->layout = MOE_LAYOUT_PACKED;
  packed->w_gate = d;
  packed->w_up = d + mb;
  packed->w_down = d + 2 * mb;
  return launch_status(fn);
}

// Workspace layout: h [R_max][F] in the layer dtype | fp8: h scales [R_max][F/128] fp32 | down-GEMM partial sums
// [ksplit-1][R_max][H] fp32 (only when the reduction dimension is split), each part 256-byte aligned.
static size_t ffn_h_bytes(int64_t R_max, const moe_ffn_weights* w) {
  return align256((size_t)R_max * (size_t)w->F * (size_t)dtype_bytes(w->dtype));
}
static size_t ffn_hs_bytes(int64_t R_max, const moe_ffn_weights* w) {
  return w->dtype == MOE_DTYPE_FP8_E4M3 ? align256((size_t)R_max * (size_t)(w->F / 128) * sizeof(float)) : 0;
}

size_t moe_grouped_ffn_workspace_bytes(const moe_ffn_weights* w, int64_t R_max) {
  if (w == nullptr || R_max < 0 || w->F < 128 || w->H < 128 || w->E_local < 1 || !dtype_ok(w->dtype)) return 0;
  const int ks = ffn_down_ksplit(R_max, w->E_local, w->H, w->F, w->dtype);
  return ffn_h_bytes(R_max, w) + ffn_hs_bytes(R_max, w) +
         (size_t)(ks - 1) * align256((size_t)R_max * (size_t)w->H * sizeof(float)) + 256;
}

// Shared validation of the grouped-FFN entry points; fills the launch description.
static moe_status ffn_prepare(const char* fn, const void* x_perm, const float* x_perm_scales, const int32_t* offsets,
                              int32_t e_lo, int64_t R_max, const moe_ffn_weights* w, float* y_perm, bool need_x,
                              bool need_y, void* workspace, size_t workspace_bytes, FfnLaunch* p) {
  const moe_status st = check_weights(fn, w);
  if (st != MOE_OK) return st;
  if (w->layout != MOE_LAYOUT_PACKED)
    FAIL(MOE_ERR_UNSUPPORTED, "%s: weights must be MOE_LAYOUT_PACKED (see moe_pack_ffn_weights)", fn);
  if (R_max < 0 || R_max >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: R_max = %lld outside [0, 2^31)", fn, (long long)R_max);
  if (e_lo < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: e_lo = %d < 0", fn, e_lo);
  REQ_PTR(offsets, 4, "offsets");
  const bool fp8 = w->dtype == MOE_DTYPE_FP8_E4M3;
  if (R_max > 0) {
    if (need_x) {
      REQ_PTR(x_perm, 16, "x_perm");
      if (fp8) REQ_PTR(x_perm_scales, 4, "x_perm_scales");
    }
    if (need_y) REQ_PTR(y_perm, 16, "y_perm");
  }
  const size_t need = moe_grouped_ffn_workspace_bytes(w, R_max);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    FAIL(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, need, workspace_bytes);
  *p = FfnLaunch{};
  p->dtype = w->dtype;
  p->x_perm = x_perm;
  p->x_perm_scales = fp8 ? x_perm_scales : nullptr;
  p->offsets = offsets;
  p->e_lo = e_lo;
  p->E_local = w->E_local;
  p->H = w->H;
  p->F = w->F;
  p->R_max = R_max;
  p->w_gate = w->w_gate;
  p->w_up = w->w_up;
  p->w_down = w->w_down;
  p->s_gate = w->s_gate;
  p->s_up = w->s_up;
  p->s_down = w->s_down;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  p->h = ws;
  p->h_scales = fp8 ? reinterpret_cast<float*>(ws + ffn_h_bytes(R_max, w)) : nullptr;
  p->ksplit = ffn_down_ksplit(R_max, w->E_local, w->H, w->F, w->dtype);
  p->y_part = reinterpret_cast<float*>(ws + ffn_h_bytes(R_max, w) + ffn_hs_bytes(R_max, w));
  p->y_perm = y_perm;
  return MOE_OK;
}

moe_status moe_grouped_ffn(const void* x_perm, const float* x_perm_scales, const int32_t* offsets, int32_t e_lo,
                           int64_t R_max, const moe_ffn_weights* w, float* y_perm, void* workspace,
                           size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn";
  FfnLaunch p;
  const moe_status st = ffn_prepare(fn, x_perm, x_perm_scales, offsets, e_lo, R_max, w, y_perm, true, true, workspace,
                                    workspace_bytes, &p);
  if (st != MOE_OK || R_max == 0) return st;
  launch_ffn_gemm1(p, (hipStream_t)stream);
  launch_ffn_gemm2(p, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_grouped_ffn_gate_up(const void* x_perm, const float* x_perm_scales, const int32_t* offsets,
                                   int32_t e_lo, int64_t R_max, const moe_ffn_weights* w, void* workspace,
                                   size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_gate_up";
  FfnLaunch p;
  const moe_status st = ffn_prepare(fn, x_perm, x_perm_scales, offsets, e_lo, R_max, w, nullptr, true, false,
                                    workspace, workspace_bytes, &p);
  if (st != MOE_OK || R_max == 0) return st;
  launch_ffn_gemm1(p, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_grouped_ffn_down(const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                float* y_perm, void* workspace, size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_down";
  FfnLaunch p;
  const moe_status st = ffn_prepare(fn, nullptr, nullptr, offsets, e_lo, R_max, w, y_perm, false, true, workspace,
                                    workspace_bytes, &p);
  if (st != MOE_OK || R_max == 0) return st;
  launch_ffn_gemm2(p, (hipStream_t)stream);
  return launch_status(fn);
}

// ---------------------------------------------------------------------------------------------------------
// Training: the forward with its saved activations, and the backward pass.
// ---------------------------------------------------------------------------------------------------------
moe_status moe_grouped_ffn_train(const void* x_perm, const int32_t* offsets, int32_t e_lo, int64_t R_max,
                                 const moe_ffn_weights* w, void* h, float* gu, float* y_perm, void* workspace,
                                 size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_train";
  FfnLaunch p;
  const moe_status st = ffn_prepare(fn, x_perm, nullptr, offsets, e_lo, R_max, w, y_perm, true, true, workspace,
                                    workspace_bytes, &p);
  if (st != MOE_OK) return st;
  if (w->dtype == MOE_DTYPE_FP8_E4M3) FAIL(MOE_ERR_UNSUPPORTED, "%s: fp8 layers have no training form", fn);
  if (R_max == 0) return MOE_OK;
  REQ_PTR(h, 16, "h");
  REQ_PTR(gu, 16, "gu");
  p.h = h;
  p.gu = gu;
  launch_ffn_gemm1(p, (hipStream_t)stream);
  launch_ffn_gemm2(p, (hipStream_t)stream);
  return launch_status(fn);
}

namespace {
struct BwdSizes {
  int64_t Rpad;
  size_t por, poff, rw, dO, dgu, dX, whT, dOT, xT, dguT, total;
};
BwdSizes bwd_sizes(const moe_ffn_weights* w, int64_t R_max) {
  BwdSizes z{};
  const size_t b = (size_t)dtype_bytes(w->dtype), H = (size_t)w->H, F = (size_t)w->F, R = (size_t)R_max;
  z.Rpad = (R_max + 63) / 64 * 64 + (int64_t)w->E_local * 64;
  const size_t Rp = (size_t)z.Rpad;
  z.por = align256(R * 4);
  z.poff = align256(((size_t)w->E_local + 1) * 4);
  z.rw = align256(R * 4);
  z.dO = align256(R * H * b);
  z.dgu = align256(R * 2 * F * b);
  z.dX = align256(R * H * 4);
  z.whT = align256(F * Rp * b);
  z.dOT = align256(H * Rp * b);
  z.xT = align256(H * Rp * b);
  z.dguT = align256(2 * F * Rp * b);
  z.total = z.por + z.poff + z.rw + z.dO + z.dgu + z.dX + z.whT + z.dOT + z.xT + z.dguT + 256;
  return z;
}
}  // namespace

size_t moe_grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int64_t R_max) {
  if (w == nullptr || R_max < 0 || w->F < 128 || w->H < 128 || w->E_local < 1 ||
      (w->dtype != MOE_DTYPE_F32 && w->dtype != MOE_DTYPE_BF16))
    return 0;
  return bwd_sizes(w, R_max).total;
}

moe_status moe_grouped_ffn_backward(const void* dout, int64_t T, int32_t k, int32_t E, const int32_t* topk_idx,
                                    const float* topk_w, const int32_t* row_of_pair, const int32_t* token_of_row,
                                    const int32_t* offsets, int32_t e_lo, int64_t R_max, const void* x_perm,
                                    const void* h, const float* gu, const float* y_perm, const moe_ffn_weights* w,
                                    void* dx, float* dw_gate, float* dw_up, float* dw_down, float* d_topk_w,
                                    float* d_logits, void* workspace, size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_backward";
  const moe_status st = check_weights(fn, w);
  if (st != MOE_OK) return st;
  if (w->layout != MOE_LAYOUT_NATURAL)
    FAIL(MOE_ERR_UNSUPPORTED, "%s: the backward takes the weights in MOE_LAYOUT_NATURAL", fn);
  if (w->dtype == MOE_DTYPE_FP8_E4M3) FAIL(MOE_ERR_UNSUPPORTED, "%s: fp8 layers have no training form", fn);
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (k < 1 || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, 32]", fn, k);
  if (e_lo < 0 || E < k || (int64_t)e_lo + w->E_local > E)
    FAIL(MOE_ERR_INVALID_ARG, "%s: experts [e_lo, e_lo + E_local) = [%d, %d) must lie in [0, E = %d), E >= k", fn,
         e_lo, e_lo + w->E_local, E);
  if (E > 1024) FAIL(MOE_ERR_INVALID_ARG, "%s: E = %d > 1024", fn, E);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (R_max < 0 || R_max > T * (int64_t)k)
    FAIL(MOE_ERR_INVALID_ARG, "%s: R_max = %lld outside [0, T * k]", fn, (long long)R_max);
  const BwdSizes z = bwd_sizes(w, R_max);
  // transposed operands: a 256-row tile of [C][Rpad] stays inside 32-bit offsets
  if ((int64_t)z.Rpad * dtype_bytes(w->dtype) * 256 >= (1ll << 32))
    FAIL(MOE_ERR_INVALID_ARG, "%s: R_max = %lld is too large for the weight-gradient operands", fn,
         (long long)R_max);
  REQ_PTR(offsets, 4, "offsets");
  REQ_PTR(dw_gate, 16, "dw_gate");
  REQ_PTR(dw_up, 16, "dw_up");
  REQ_PTR(dw_down, 16, "dw_down");
  if (T > 0) {
    REQ_PTR(dout, 16, "dout");
    REQ_PTR(topk_idx, 4, "topk_idx");
    REQ_PTR(topk_w, 4, "topk_w");
    REQ_PTR(row_of_pair, 4, "row_of_pair");
    REQ_PTR(dx, 16, "dx");
    REQ_PTR(d_topk_w, 4, "d_topk_w");
    if (d_logits != nullptr && !aligned(d_logits, 4)) FAIL(MOE_ERR_INVALID_ARG, "%s: d_logits is not 4-byte aligned", fn);
  }
  if (R_max > 0) {
    REQ_PTR(token_of_row, 4, "token_of_row");
    REQ_PTR(x_perm, 16, "x_perm");
    REQ_PTR(h, 16, "h");
    REQ_PTR(gu, 16, "gu");
    REQ_PTR(y_perm, 16, "y_perm");
  }
  if (workspace == nullptr || workspace_bytes < z.total || !aligned(workspace, 256))
    FAIL(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", fn, z.total, workspace_bytes);
  BwdLaunch p{};
  p.dtype = w->dtype;
  p.T = T;
  p.R_max = R_max;
  p.H = w->H;
  p.F = w->F;
  p.k = k;
  p.E = E;
  p.e_lo = e_lo;
  p.E_local = w->E_local;
  p.dout = dout;
  p.topk_idx = topk_idx;
  p.offsets = offsets;
  p.row_of_pair = row_of_pair;
  p.token_of_row = token_of_row;
  p.topk_w = topk_w;
  p.x_perm = x_perm;
  p.h = h;
  p.gu = gu;
  p.y_perm = y_perm;
  p.w_gate = w->w_gate;
  p.w_up = w->w_up;
  p.w_down = w->w_down;
  p.dx = dx;
  p.dw_gate = dw_gate;
  p.dw_up = dw_up;
  p.dw_down = dw_down;
  p.d_topk_w = d_topk_w;
  p.d_logits = d_logits;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  p.por = reinterpret_cast<int32_t*>(ws);
  ws += z.por;
  p.poff = reinterpret_cast<int32_t*>(ws);
  ws += z.poff;
  p.rw = reinterpret_cast<float*>(ws);
  ws += z.rw;
  p.dO = ws;
  ws += z.dO;
  p.dgu = ws;
  ws += z.dgu;
  p.dX = reinterpret_cast<float*>(ws);
  ws += z.dX;
  p.whT = ws;
  ws += z.whT;
  p.dOT = ws;
  ws += z.dOT;
  p.xT = ws;
  ws += z.xT;
  p.dguT = ws;
  launch_ffn_backward(p, (hipStream_t)stream);
  return launch_status(fn);
}

// Gather / scatter form (no x_perm, pair-major output).  Validates what the permuted form does, plus the token
// tables; the activations' byte span must fit the kernels' 32-bit offsets.
static moe_status fused_prepare(const char* fn, const void* x, const float* x_scales, const int32_t* token_of_row,
                                const int32_t* row_of_pair, const float* topk_w, int64_t T, int32_t k,
                                bool need_x, bool need_y, float* y_slot, FfnLaunch* p) {
  const bool fp8 = p->dtype == MOE_DTYPE_FP8_E4M3;
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (k < 1 || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, 32]", fn, k);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (need_y && p->R_max > T * (int64_t)k)
    FAIL(MOE_ERR_INVALID_ARG, "%s: R_max = %lld exceeds T * k = %lld", fn, (long long)p->R_max, (long long)(T * k));
  if (T * (int64_t)p->H * dtype_bytes(p->dtype) >= (1ll << 32))
    FAIL(MOE_ERR_INVALID_ARG, "%s: T * H * element bytes must be < 2^32", fn);
  if (p->R_max > 0) {
    REQ_PTR(token_of_row, 4, "token_of_row");
    if (need_x) {
      REQ_PTR(x, 16, "x");
      if (fp8) REQ_PTR(x_scales, 4, "x_scales");
    }
    if (need_y) {
      REQ_PTR(row_of_pair, 4, "row_of_pair");
      REQ_PTR(topk_w, 4, "topk_w");
      REQ_PTR(y_slot, 16, "y_slot");
    }
  }
  p->x_perm = x;
  p->x_perm_scales = fp8 ? x_scales : nullptr;
  p->gather_rows = token_of_row;
  p->token_of_row = token_of_row;
  p->row_of_pair = row_of_pair;
  p->topk_w = topk_w;
  p->k = k;
  p->y_slot = y_slot;
  p->y_perm = nullptr;
  return MOE_OK;
}

moe_status moe_grouped_ffn_gate_up_gather(const void* x, const float* x_scales, const int32_t* token_of_row,
                                          int64_t T, const int32_t* offsets, int32_t e_lo, int64_t R_max,
                                          const moe_ffn_weights* w, void* workspace, size_t workspace_bytes,
                                          moe_stream stream) {
  const char* fn = "moe_grouped_ffn_gate_up_gather";
  FfnLaunch p;
  moe_status st = ffn_prepare(fn, nullptr, nullptr, offsets, e_lo, R_max, w, nullptr, false, false, workspace,
                              workspace_bytes, &p);
  if (st != MOE_OK) return st;
  st = fused_prepare(fn, x, x_scales, token_of_row, nullptr, nullptr, T, 1, true, false, nullptr, &p);
  if (st != MOE_OK || R_max == 0) return st;
  launch_ffn_gemm1(p, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_grouped_ffn_down_scatter(const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                        const int32_t* token_of_row, const int32_t* row_of_pair,
                                        const float* topk_w, int64_t T, int32_t k, float* y_slot, void* workspace,
                                        size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_down_scatter";
  FfnLaunch p;
  moe_status st = ffn_prepare(fn, nullptr, nullptr, offsets, e_lo, R_max, w, nullptr, false, false, workspace,
                              workspace_bytes, &p);
  if (st != MOE_OK) return st;
  st = fused_prepare(fn, nullptr, nullptr, token_of_row, row_of_pair, topk_w, T, k, false, true, y_slot, &p);
  if (st != MOE_OK || R_max == 0) return st;
  p.gather_rows = nullptr;
  launch_ffn_gemm2(p, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_grouped_ffn_fused(const void* x, const float* x_scales, const int32_t* token_of_row,
                                 const int32_t* row_of_pair, const float* topk_w, int64_t T, int32_t k,
                                 const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                 float* y_slot, void* workspace, size_t workspace_bytes, moe_stream stream) {
  const char* fn = "moe_grouped_ffn_fused";
  FfnLaunch p;
  moe_status st = ffn_prepare(fn, nullptr, nullptr, offsets, e_lo, R_max, w, nullptr, false, false, workspace,
                              workspace_bytes, &p);
  if (st != MOE_OK) return st;
  st = fused_prepare(fn, x, x_scales, token_of_row, row_of_pair, topk_w, T, k, true, true, y_slot, &p);
  if (st != MOE_OK || R_max == 0) return st;
  launch_ffn_gemm1(p, (hipStream_t)stream);
  p.gather_rows = nullptr;
  launch_ffn_gemm2(p, (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_combine_slots(const float* y_slot, const int32_t* row_of_pair, const int32_t* topk_idx, int64_t T,
                             int32_t k, int32_t H, int32_t e_lo, int32_t E_local, void* out, moe_dtype out_dtype,
                             moe_stream stream) {
  const char* fn = "moe_combine_slots";
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (k < 1 || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, 32]", fn, k);
  if (H <= 0 || H % 128) FAIL(MOE_ERR_INVALID_ARG, "%s: H = %d must be a positive multiple of 128", fn, H);
  if (e_lo < 0 || E_local < 1) FAIL(MOE_ERR_INVALID_ARG, "%s: window [%d, %d + %d) is empty or negative", fn, e_lo, e_lo, E_local);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (!dtype_ok(out_dtype)) FAIL(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)out_dtype);
  if (out_dtype == MOE_DTYPE_FP8_E4M3) FAIL(MOE_ERR_UNSUPPORTED, "%s: out_dtype must be F32 or BF16", fn);
  if (T == 0) return MOE_OK;
  REQ_PTR(y_slot, 16, "y_slot");
  REQ_PTR(topk_idx, 4, "topk_idx");
  REQ_PTR(out, 16, "out");
  if (row_of_pair != nullptr) REQ_PTR(row_of_pair, 4, "row_of_pair");
  launch_combine_slots(y_slot, row_of_pair, topk_idx, T, k, H, e_lo, E_local, out, out_dtype == MOE_DTYPE_BF16,
                       (hipStream_t)stream);
  return launch_status(fn);
}

moe_status moe_combine(const float* y_perm, const int32_t* row_of_pair, const int32_t* topk_idx, const float* topk_w,
                       int64_t T, int32_t k, int32_t H, int32_t e_lo, int32_t E_local, void* out,
                       moe_dtype out_dtype, moe_stream stream) {
  const char* fn = "moe_combine";
  if (T < 0) FAIL(MOE_ERR_INVALID_ARG, "%s: T = %lld < 0", fn, (long long)T);
  if (k < 1 || k > 32) FAIL(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, 32]", fn, k);
  if (H <= 0 || H % 128) FAIL(MOE_ERR_INVALID_ARG, "%s: H = %d must be a positive multiple of 128", fn, H);
  if (e_lo < 0 || E_local < 1) FAIL(MOE_ERR_INVALID_ARG, "%s: window [%d, %d + %d) is empty or negative", fn, e_lo, e_lo, E_local);
  if (T * (int64_t)k >= (1ll << 31)) FAIL(MOE_ERR_INVALID_ARG, "%s: T * k must be < 2^31", fn);
  if (!dtype_ok(out_dtype)) FAIL(MOE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)out_dtype);
  if (out_dtype == MOE_DTYPE_FP8_E4M3) FAIL(MOE_ERR_UNSUPPORTED, "%s: out_dtype must be F32 or BF16", fn);
  if (T == 0) return MOE_OK;
  REQ_PTR(y_perm, 16, "y_perm");
  REQ_PTR(row_of_pair, 4, "row_of_pair");
  REQ_PTR(topk_idx, 4, "topk_idx");
  REQ_PTR(topk_w, 4, "topk_w");
  REQ_PTR(out, 16, "out");
  launch_combine(y_perm, row_of_pair, topk_idx, topk_w, T, k, H, e_lo, E_local, out, out_dtype == MOE_DTYPE_BF16,
                 (hipStream_t)stream);
  return launch_status(fn);
}

}  // extern "C"
