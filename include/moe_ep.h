/*
 * moe_ep.h -- C ABI of libmoe_ep.so: one GPU's share of an expert-parallel mixture-of-experts layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (page "Expert parallelism and all-to-all", section "Walking through one MoE layer"):
 *   1. the router gives every token a list of (expert, weight) picks               -> moe_route_topk
 *      (with the router's x W_r in front)                                        -> moe_router_topk
 *   2. dispatch: each token's row goes to the experts it picked; locally this is a
 *      sort of the (token, pick) pairs into one contiguous slab per expert          -> moe_dispatch_permute
 *   3. every local expert runs on the rows it received, as one grouped matrix
 *      multiply (here a SwiGLU FFN: silu(x Wg) * (x Wu), then Wd)                    -> moe_grouped_ffn
 *   4. combine: each expert output goes back to its token, which takes the weighted
 *      sum of its picks                                                            -> moe_combine
 *   fused form: gather inside the gate/up product, weighted un-permute in the down product's epilogue
 *                                       -> moe_grouped_ffn_gate_up_gather / _down_scatter / _fused, moe_combine_slots
 *   fixed capacity per expert (pairs past it dropped)                             -> moe_dispatch_permute_capacity
 *   training: the forward keeping its activations, then the gradients of x, the expert weights, the routing
 *   weights and the logits                        -> moe_grouped_ffn_train, moe_grouped_ffn_backward
 * Between ranks, steps 2 and 4 are all-to-all exchanges; on one GPU they are the local permutation and its
 * inverse, and the exchange itself is not part of this library.
 *
 * Conventions common to every call:
 *  - Pointers marked (device) point to GPU memory; the caller allocates and owns every buffer.  The library
 *    allocates nothing and keeps no per-call state.  Buffers must be 16-byte aligned unless an entry point
 *    states otherwise (index and weight arrays: 4 bytes).
 *  - Calls are asynchronous: they validate their arguments on the host, then enqueue kernels on `stream`
 *    (NULL = the null stream) and return.  They never synchronise and never read device memory on the host,
 *    so a sequence of calls can be captured in a HIP graph.
 *  - Argument errors are reported before anything is enqueued: the call returns a non-zero moe_status and
 *    launches nothing (no silent fallback, no CPU path, no dtype downgrade).  moe_last_error() describes the
 *    failure.  Faults inside kernels surface as HIP errors at the caller's next synchronisation.
 *  - Data-dependent values (counts, offsets) stay on the device.  T = 0 is a successful no-op.
 *  - Indices are int32: T * k < 2^31.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_EP_ABI_VERSION 1

/* A hipStream_t (HIP's stream handle is a pointer to this opaque struct); NULL is the null stream. */
struct ihipStream_t;
typedef struct ihipStream_t* moe_stream;

typedef enum {
  MOE_DTYPE_F32 = 0,      /* IEEE binary32 */
  MOE_DTYPE_BF16 = 1,     /* bfloat16 */
  MOE_DTYPE_FP8_E4M3 = 2  /* OCP fp8 E4M3 (max 448, no infinities), always paired with fp32 scales */
} moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a size, pointer, alignment or window is out of range */
  MOE_ERR_UNSUPPORTED = 2, /* a valid request this library does not implement (dtype combination, layout) */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the matching *_workspace_bytes() */
  MOE_ERR_DEVICE = 4       /* a HIP launch or runtime call failed */
} moe_status;

/* Name of a status code (static string). */
const char* moe_status_string(moe_status s);
/* MOE_EP_ABI_VERSION of the loaded library. */
int moe_abi_version(void);
/* Message describing the last non-OK status returned on the calling thread (static per-thread buffer). */
const char* moe_last_error(void);

/*
 * Step 1 -- routing (page "Expert parallelism and all-to-all", section "Walking through one MoE layer",
 * step 1: every token gets a list of (expert, weight) picks; page "Expert parallelism", section "Adding an
 * implementation": the picks carry global expert ids and their weights).
 * For each token t: the k experts with the largest logits, ordered by logit descending, equal logits in
 * ascending expert id (selection compares the fp32 logits exactly); slot j holds the j-th pick.  The weights
 * are the softmax over all E logits restricted to the picks and renormalised, i.e.
 *   w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0),
 * evaluated in fp64 and rounded once to fp32.
 *   logits   (device) [T, E] fp32 row-major; finite or -inf (a -inf pick gets weight 0); each row needs at
 *            least one finite logit; NaN is not supported.
 *   topk_idx (device) [T, k] int32 out: global expert ids.
 *   topk_w   (device) [T, k] fp32 out.
 * Domain: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 32).
 */
moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w,
                          moe_stream stream);

/*
 * Step 1 with the router's linear map in front (page "Expert parallelism and all-to-all", section "Walking
 * through one MoE layer", step 1: the router runs on each GPU beside attention; the router logits of a token are
 * its hidden row times the router matrix W_r).  For each token t and expert e:
 *   logits[t][e] = sum_h x^[t][h] * W_r[h][e],
 * x^ being x decoded to real values (fp8: the e4m3 code's value times its column block's scale), computed with
 * fp32 multiply-adds in a fixed order that depends only on H, so |logits - exact| <= (H + 2) 2^-24 sum_h |x^ W_r|
 * and a token's logits do not depend on T or its position.  The picks and weights are then those of
 * moe_route_topk on these fp32 logits, bit for bit.
 *   x        (device) [T, H] row-major in x_dtype, 16-byte aligned.
 *   x_scales (device) fp8 only: [T, H/128] fp32, one scale per token and 128-column block; NULL otherwise.
 *   w_router (device) [H, E] fp32 row-major, 4-byte aligned.
 *   logits   (device) [T, E] fp32 out; may be NULL for E <= 64 when only the picks are wanted (the logits and
 *            the selection are then one kernel); required above 64 experts, where the selection reads it back.
 *   topk_idx, topk_w: as for moe_route_topk.
 * Domain: T >= 0, H a positive multiple of 8 (of 128 for fp8), 1 <= E <= 1024, 1 <= k <= min(E, 32).
 */
moe_status moe_router_topk(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                           const float* w_router, int32_t E, int32_t k, float* logits, int32_t* topk_idx,
                           float* topk_w, moe_stream stream);

/*
 * Steps 2-3 -- counts, offsets, permutation and gather (page "Expert Parallelism" (aiwiki), section
 * "Implementation": sort the tokens by destination so every destination's rows are one contiguous slab, and
 * count the rows per destination; section "The two all-to-alls": the sort precedes the dispatch exchange).
 * Pair p = t*k + j carries expert topk_idx[p].  Outputs:
 *   counts[e]       number of pairs with expert e;
 *   offsets[e]      exclusive prefix sum of counts; offsets[E] = T*k;
 *   row_of_pair[p]  offsets[e] + number of pairs p' < p with the same expert (a stable sort: inside an
 *                   expert slab, rows are in ascending token order);
 *   token_of_row[r] the token whose row sits at r (token_of_row[row_of_pair[p]] = p / k);
 *   x_perm[r, :]    = x[token_of_row[r], :], byte for byte; for fp8, x_perm_scales[r, :] =
 *                   x_scales[token_of_row[r], :] too.
 * All results are deterministic (no order-dependent atomics) and bit-exact.
 *   x             (device) [T, H] in x_dtype; fp8 rows come with x_scales (device) [T, H/128] fp32, one scale
 *                 per row per 128 columns (x = code * scale); NULL for other dtypes.
 *   topk_idx      (device) [T, k] int32, each in [0, E).
 *   counts        (device) [E] int32 out;  offsets (device) [E+1] int32 out.
 *   row_of_pair   (device) [T*k] int32 out;  token_of_row (device) [T*k] int32 out.
 *   x_perm        (device) [T*k, H] out, x_dtype;  x_perm_scales (device) [T*k, H/128] fp32 out (fp8 only).
 *                 x_perm = NULL: counts, offsets and the permutation only (x, x_scales, x_perm_scales unused);
 *                 the fused form below reads x through token_of_row instead.
 *   workspace     (device) at least moe_dispatch_workspace_bytes(T, k, E) bytes, 256-byte aligned.
 * Domain: T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 32), H > 0 and H % 128 == 0.
 */
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t E);
moe_status moe_dispatch_permute(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                                const int32_t* topk_idx, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                                int32_t* row_of_pair, int32_t* token_of_row, void* x_perm, float* x_perm_scales,
                                void* workspace, size_t workspace_bytes, moe_stream stream);

/*
 * moe_dispatch_permute without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Arguments, results and domain as
 * moe_dispatch_permute.  The scratch the multi-workgroup counting form needs (moe_dispatch_workspace_bytes(T, k,
 * E) bytes, about E * T / 32) comes from a fixed array of 1 MiB inside the library, one per GPU, held until the
 * process ends; a larger request (e.g. E = 256 with more than 130816 tokens) returns MOE_ERR_WORKSPACE and
 * enqueues nothing.
 * The kernels write every scratch word before they read it, so nothing is cleared between calls.  Calls that
 * overlap on one GPU (different streams, or graphs replayed concurrently) share the array and race; calls on one
 * stream are ordered and safe.  The first call on a device looks the array's address up (no allocation).
 */
moe_status moe_dispatch_permute_noalloc(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T, int32_t H,
                                        const int32_t* topk_idx, int32_t k, int32_t E, int32_t* counts,
                                        int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row, void* x_perm,
                                        float* x_perm_scales, moe_stream stream);

/*
 * Step 2 with a fixed capacity (page "Expert Parallelism" (aiwiki), section "Implementation", the note after
 * the sketch: fixed-size buffers let every rank know every size in advance, which removes the count exchange;
 * the price is that tokens beyond a buffer are dropped).  Expert e keeps the first `capacity` of its pairs in
 * ascending pair order p = t*k + j; its other pairs are dropped: row_of_pair[p] = -1, and they contribute
 * nothing in moe_combine (and in moe_combine_slots when it is given row_of_pair).  Kept weights are not
 * renormalised.  Outputs as moe_dispatch_permute with
 *   counts[e]  = min(number of pairs of e, capacity);  offsets = exclusive prefix sums of these counts;
 *   row_of_pair[p] = offsets[e] + (rank of p among the pairs of e) for kept pairs;
 *   token_of_row, x_perm, x_perm_scales: offsets[E] <= min(T*k, E*capacity) rows, which bounds every
 *   downstream buffer (a fixed worst case known before the call).
 * Bit-exact and deterministic.  Domain as moe_dispatch_permute, plus capacity >= 1.
 */
moe_status moe_dispatch_permute_capacity(const void* x, const float* x_scales, moe_dtype x_dtype, int64_t T,
                                         int32_t H, const int32_t* topk_idx, int32_t k, int32_t E, int32_t capacity,
                                         int32_t* counts, int32_t* offsets, int32_t* row_of_pair,
                                         int32_t* token_of_row, void* x_perm, float* x_perm_scales, void* workspace,
                                         size_t workspace_bytes, moe_stream stream);

/* Expert weights of the E_local experts this GPU holds (page "Expert parallelism", section "Expert
 * parallelism" plans: the expert weights are split along the expert dimension so each rank holds only its
 * local experts). */
typedef enum {
  /* w_gate, w_up [E_local][H][F]; w_down [E_local][F][H]  (row-major, as x @ W) */
  MOE_LAYOUT_NATURAL = 0,
  /* the same matrices transposed per expert, reduction dimension contiguous:
     w_gate, w_up [E_local][F][H]; w_down [E_local][H][F].  Produced by moe_pack_ffn_weights. */
  MOE_LAYOUT_PACKED = 1
} moe_weight_layout;

typedef struct {
  moe_dtype dtype;          /* F32, BF16, or FP8_E4M3 (then the three scale arrays are required) */
  moe_weight_layout layout;
  int32_t E_local, H, F;    /* H % 128 == 0, F % 128 == 0, both in [128, 65536] */
  const void* w_gate;       /* (device) see layout */
  const void* w_up;         /* (device) */
  const void* w_down;       /* (device) */
  /* fp8 only: one fp32 scale per 128 x 128 block, indexed [expert][reduction block][output block] in both
     layouts: s_gate, s_up [E_local][H/128][F/128]; s_down [E_local][F/128][H/128].  NULL otherwise. */
  const float* s_gate;
  const float* s_up;
  const float* s_down;
} moe_ffn_weights;

/*
 * Init-time weight repacking for moe_grouped_ffn: transposes each expert's matrices so the reduction
 * dimension is contiguous.  `src` must be MOE_LAYOUT_NATURAL.  `dst` (device) receives the three packed
 * matrices (at least moe_pack_ffn_weights_bytes(src) bytes, 256-byte aligned); `packed` (host) is filled
 * with a MOE_LAYOUT_PACKED description whose matrix pointers point into `dst` and whose scale pointers are
 * src's.  Weights are static, so this runs once per model load, never per layer call.
 */
size_t moe_pack_ffn_weights_bytes(const moe_ffn_weights* src);
moe_status moe_pack_ffn_weights(const moe_ffn_weights* src, void* dst, size_t dst_bytes, moe_ffn_weights* packed,
                                moe_stream stream);

/*
 * Steps 4-5 -- the local experts as one grouped matrix multiply (page "Expert parallelism and all-to-all",
 * section "Walking through one MoE layer", step 3: each GPU runs its local experts on the tokens it
 * received, as one grouped matrix multiply).
 * For every local expert i in [0, E_local), with global id e = e_lo + i and rows r in
 * [offsets[e], offsets[e+1]) of x_perm:
 *   G = x_perm[r] @ Wg_i,  U = x_perm[r] @ Wu_i        (fp32 accumulation)
 *   h = silu(G) * U                                   stored in the layer dtype: fp32, bf16 (round to
 *                                                     nearest even), or fp8 E4M3 with one fp32 scale per row
 *                                                     per 128 columns, scale = amax / 448 (1 if all zero)
 *   y_perm[r] = h @ Wd_i                              fp32, not rounded further
 * Rows of x_perm outside [offsets[e_lo], offsets[e_lo + E_local]) are not read, and the same rows of y_perm
 * are left untouched.  Experts with no rows cost nothing.
 *   x_perm        (device) [R_max, H] in w->dtype (the dispatch output);  x_perm_scales (device)
 *                 [R_max, H/128] fp32 for fp8, else NULL.
 *   offsets       (device) [e_lo + E_local + 1] int32, non-decreasing, offsets[e_lo + E_local] <= R_max.
 *   w             (host struct, device pointers) MOE_LAYOUT_PACKED weights (MOE_LAYOUT_NATURAL returns
 *                 MOE_ERR_UNSUPPORTED: call moe_pack_ffn_weights once at load time).
 *   y_perm        (device) [R_max, H] fp32 out.
 *   workspace     (device) at least moe_grouped_ffn_workspace_bytes(w, R_max) bytes, 256-byte aligned: it
 *                 holds h at byte 0 as [R_max][F] in the layer dtype (row r = row r of x_perm), for fp8 its scales
 *                 [R_max][F/128] fp32 from the next 256-byte boundary, and, when the down product's reduction
 *                 dimension is split to fill the GPU, the fp32 partial sums, which are added into y_perm in a
 *                 fixed order.
 * Precision: G and U accumulate in fp32 (fp8: each 128-wide block's products summed by the fp8 matrix
 * instruction, whose own error was measured at up to about 1e-5 of the sum of the products' magnitudes, then
 * scaled and accumulated in fp32), and h is the storage of silu(G) * U computed in fp32.  An h element whose exact value lies within that error of a
 * rounding midpoint of the storage format may take either neighbour.  For fp8 one such element moves its
 * token's outputs by one e4m3 step of h times its W_down row, about 0.08 RMS(out) sqrt(384 / F) at most: from
 * F = 2048 up the layer output stays within max|err| / RMS <= 6e-2 of the exact layer with these roundings;
 * below, within that bar plus such steps.  bf16 and fp32 layers: max|err| / RMS <= 2e-2 and 1e-4.
 * Domain: R_max >= 0, e_lo >= 0, 1 <= E_local.
 */
size_t moe_grouped_ffn_workspace_bytes(const moe_ffn_weights* w, int64_t R_max);
moe_status moe_grouped_ffn(const void* x_perm, const float* x_perm_scales, const int32_t* offsets, int32_t e_lo,
                           int64_t R_max, const moe_ffn_weights* w, float* y_perm, void* workspace,
                           size_t workspace_bytes, moe_stream stream);

/*
 * The two halves of moe_grouped_ffn, for callers that schedule or time them separately (same arguments,
 * same workspace; moe_grouped_ffn == gate_up followed by down on one stream):
 *   moe_grouped_ffn_gate_up  h = silu(x_perm Wg) * (x_perm Wu) in the layer dtype, into the workspace
 *   moe_grouped_ffn_down     y_perm = h Wd, reading h from the same workspace
 * The down half also follows moe_grouped_ffn_gate_up_gather (below): the gather form, the permuted result
 * without x_perm.  Whichever gate/up half is used, both halves take the same R_max (the workspace holds h and,
 * for fp8, its scales in a layout set by R_max).
 */
moe_status moe_grouped_ffn_gate_up(const void* x_perm, const float* x_perm_scales, const int32_t* offsets,
                                   int32_t e_lo, int64_t R_max, const moe_ffn_weights* w, void* workspace,
                                   size_t workspace_bytes, moe_stream stream);
moe_status moe_grouped_ffn_down(const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                float* y_perm, void* workspace, size_t workspace_bytes, moe_stream stream);

/*
 * Step 6 -- combine (page "Expert parallelism and all-to-all", section "Walking through one MoE layer",
 * step 4: each expert output returns to its token, and the token takes the weighted sum; page "Expert
 * Parallelism" (aiwiki), section "Implementation": the inverse permutation undoes the sort).
 *   out[t, :] = sum over slots j = 0..k-1 whose expert lies in [e_lo, e_lo + E_local) of
 *               topk_w[t, j] * y_perm[row_of_pair[t*k + j], :]
 * accumulated in fp32 in slot order and rounded once to out_dtype; a token with no local pick gets zeros.
 * Each output row is written by exactly one workgroup: no atomics, deterministic.
 *   y_perm (device) [R, H] fp32;  row_of_pair, topk_idx (device) [T*k] int32;  topk_w (device) [T*k] fp32.
 *   out    (device) [T, H] out, out_dtype F32 or BF16.
 * Domain: T >= 0, 1 <= k <= 32, H > 0 and H % 128 == 0, e_lo >= 0, E_local >= 1.
 */
moe_status moe_combine(const float* y_perm, const int32_t* row_of_pair, const int32_t* topk_idx, const float* topk_w,
                       int64_t T, int32_t k, int32_t H, int32_t e_lo, int32_t E_local, void* out,
                       moe_dtype out_dtype, moe_stream stream);

/*
 * Fused form of steps 3-6 on one GPU (page "Expert parallelism" (transformers docs), section "Choosing an
 * implementation": one of the listed implementations runs dispatch, experts and combine in a single kernel).
 * Here the gather moves into the gate/up product's loads and the weighted un-permute into the down product's
 * epilogue, so neither x_perm nor a permuted y is written:
 *   moe_grouped_ffn_gate_up_gather  h as moe_grouped_ffn_gate_up, reading row r of the slab as
 *                                   x[token_of_row[r], :] (and x_scales[token_of_row[r], :] for fp8)
 *   moe_grouped_ffn_down_scatter    for each window row r and the pair p with row_of_pair[p] = r:
 *                                   y_slot[p, :] = topk_w[p] * (h[r, :] Wd_e), reading h from the workspace
 *   moe_grouped_ffn_fused           both in order
 *   moe_combine_slots               out[t, :] = sum over slots j = 0..k-1 with topk_idx[t*k+j] in
 *                                   [e_lo, e_lo + E_local) (and, if row_of_pair is given, row_of_pair[t*k+j] >= 0:
 *                                   not dropped by a capacity) of y_slot[t*k + j, :], fp32 in slot order, one
 *                                   rounding
 * The layer output equals the permuted path's up to fp32 rounding order (the weight is applied before the sum).
 * Slots of pairs outside the window are neither written nor read.
 *   x, x_scales      (device) as moe_dispatch_permute's inputs;  token_of_row, row_of_pair (device) [T*k] int32
 *                    from moe_dispatch_permute (x_perm may be NULL there);  topk_w (device) [T*k] fp32.
 *   y_slot           (device) [T*k, H] fp32 out, pair-major.  workspace as moe_grouped_ffn (same size query).
 * Domain: as the permuted calls, plus 1 <= k <= 32, R_max <= T*k and T * H * element bytes < 2^32.
 */
moe_status moe_grouped_ffn_gate_up_gather(const void* x, const float* x_scales, const int32_t* token_of_row,
                                          int64_t T, const int32_t* offsets, int32_t e_lo, int64_t R_max,
                                          const moe_ffn_weights* w, void* workspace, size_t workspace_bytes,
                                          moe_stream stream);
moe_status moe_grouped_ffn_down_scatter(const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                        const int32_t* token_of_row, const int32_t* row_of_pair,
                                        const float* topk_w, int64_t T, int32_t k, float* y_slot, void* workspace,
                                        size_t workspace_bytes, moe_stream stream);
moe_status moe_grouped_ffn_fused(const void* x, const float* x_scales, const int32_t* token_of_row,
                                 const int32_t* row_of_pair, const float* topk_w, int64_t T, int32_t k,
                                 const int32_t* offsets, int32_t e_lo, int64_t R_max, const moe_ffn_weights* w,
                                 float* y_slot, void* workspace, size_t workspace_bytes, moe_stream stream);
moe_status moe_combine_slots(const float* y_slot, const int32_t* row_of_pair /* NULL: no dropped pairs */,
                             const int32_t* topk_idx, int64_t T, int32_t k, int32_t H, int32_t e_lo,
                             int32_t E_local, void* out, moe_dtype out_dtype, moe_stream stream);

/*
 * Training (page "Expert parallelism" (transformers docs), section "Adding an implementation": the gradients,
 * the routing weights' included, must reach every token; page "Expert parallelism and all-to-all", section
 * "Walking through one MoE layer": the layer whose calculus this is).  fp32 and bf16 layers; fp8 layers return
 * MOE_ERR_UNSUPPORTED.
 *
 * moe_grouped_ffn_train: moe_grouped_ffn that also keeps what the backward needs, in caller buffers:
 *   h  (device) [R_max, F]  layer dtype out: silu(g) * u as stored between the two products
 *   gu (device) [R_max, 2F] fp32 out: row r holds g = x_perm[r] Wg_e in columns [0, F) and
 *                           u = x_perm[r] Wu_e in [F, 2F), the products' fp32 accumulators
 *   other arguments, y_perm and the workspace as moe_grouped_ffn (packed weights, no scales).
 *
 * moe_grouped_ffn_backward: for dout = dL/dout [T, H] (layer dtype) of the layer output, with the routing and
 * dispatch tables and the saved activations of the same forward (x_perm, h, gu, y_perm), and the weights in
 * MOE_LAYOUT_NATURAL:
 *   dx       (device) [T, H] layer dtype out: dL/dx, each token's rows summed in slot order in fp32
 *   dw_gate, dw_up (device) [E_local, H, F] fp32 out; dw_down (device) [E_local, F, H] fp32 out
 *            (an expert without rows gets zeros)
 *   d_topk_w (device) [T, k] fp32 out: <dout[t], y of pick j>; 0 for picks that are not local or were dropped
 *   d_logits (device) [T, E] fp32 out, or NULL: w_m (d_topk_w_m - sum_j w_j d_topk_w_j) at each pick m (the
 *            Jacobian of the softmax renormalised over the k picks), 0 for the other experts; with a window of
 *            local experts this is this share's term of a sum over shares.
 * The storage of h in the layer dtype is differentiated as the identity.  Rounding: [dg | du] and w h are
 * stored in the layer dtype as matrix operands (dh itself is w (dout Wd^T), w applied in fp32); every product
 * accumulates in fp32.
 * Weight layouts: the backward's data products reduce along the rows of the natural matrices (dh over H with
 * Wd_e [F][H], dX over F with Wg_e, Wu_e [H][F]), the forward's along the rows of the packed ones, so a training
 * caller keeps both copies: 3 E_local H F bytes per element size beyond the forward's (2.82 GB for E_local = 8,
 * H = 4096, F = 14336 in bf16).
 * Results do not depend on run or launch order (no atomics).  Workspace: at least
 * moe_grouped_ffn_backward_workspace_bytes(w, R_max) bytes, 256-byte aligned.
 * Domain: as moe_grouped_ffn, plus 1 <= k <= 32, E >= k, [e_lo, e_lo + E_local) inside [0, E), E <= 1024,
 * R_max <= T * k, and R_max small enough that 256 rows of the transposed [C, R_max + 64 E_local] operands span
 * < 2^32 bytes.
 */
moe_status moe_grouped_ffn_train(const void* x_perm, const int32_t* offsets, int32_t e_lo, int64_t R_max,
                                 const moe_ffn_weights* w, void* h, float* gu, float* y_perm, void* workspace,
                                 size_t workspace_bytes, moe_stream stream);
size_t moe_grouped_ffn_backward_workspace_bytes(const moe_ffn_weights* w, int64_t R_max);
moe_status moe_grouped_ffn_backward(const void* dout, int64_t T, int32_t k, int32_t E, const int32_t* topk_idx,
                                    const float* topk_w, const int32_t* row_of_pair, const int32_t* token_of_row,
                                    const int32_t* offsets, int32_t e_lo, int64_t R_max, const void* x_perm,
                                    const void* h, const float* gu, const float* y_perm, const moe_ffn_weights* w,
                                    void* dx, float* dw_gate, float* dw_up, float* dw_down, float* d_topk_w,
                                    float* d_logits, void* workspace, size_t workspace_bytes, moe_stream stream);

/*
 * Host-only helper: the dispatch + combine payload in bytes of `tokens` tokens for one MoE layer, the closed
 * form 2 * k * H * bytes_per_elem * tokens (page "Expert parallelism and all-to-all", section "Traffic
 * math"; the 2 counts the dispatch and the combine).  Returns 0 for negative arguments.
 */
uint64_t moe_payload_bytes(int64_t tokens, int32_t k, int32_t H, int32_t bytes_per_elem);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EP_H */
