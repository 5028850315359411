/*
 * moe_oracle.c -- plain, slow CPU oracle for one GPU's share of an expert-parallel MoE layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline leg load this file's
 * library.  It shares no code, header, table or helper with the HIP library; it is written from the pages'
 * description of the layer and from the definitions of the number formats.
 *
 * What it follows (page titles and sections of the source pages):
 *  - "Expert parallelism and all-to-all", section "Walking through one MoE layer", steps 1-4: the router gives
 *    every token a list of (expert, weight) picks; the local experts run on the rows they receive; the home
 *    GPU takes the weighted sum of the expert outputs.
 *  - "Expert parallelism" (transformers docs), section "Token dispatch": route, send each (token, expert)
 *    pair to its expert, run the local experts, combine with the routing weights.
 *  - "Expert Parallelism" (aiwiki), section "Implementation": sort the tokens by destination expert so each
 *    destination's rows are contiguous, count rows per destination, and undo the sort afterwards.
 *  - The routing rule (softmax over the router logits, top-k, weights renormalised over the k picks, ties to
 *    the lower expert id on the fp32 logits) and the expert FFN (SwiGLU: silu(x Wg) * (x Wu), then Wd) define
 *    the layer checked here; the pages describe the picks only as pairs of an expert and a weight.
 *
 * Arithmetic: fp64 throughout.  Stored inputs (fp32, bf16, OCP fp8 e4m3 with fp32 scales) are decoded
 * exactly.  The one rounding the oracle copies from the method is the storage of the SwiGLU intermediate h in
 * the layer's dtype (fp32; bf16 round-to-nearest-even; fp8 e4m3 with one fp32 scale per row per 128 columns),
 * because the layer stores h in that dtype between its two expert matrix products.  The expert outputs and
 * the weighted sum stay in fp64 and are returned unrounded.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC moe_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2

/* ---------------------------------------------------------------------------------------------------------
 * Number formats, from their definitions.
 * bf16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent, 7 fraction bits).
 * OCP fp8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds subnormals
 * m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
 * ------------------------------------------------------------------------------------------------------- */

double orc_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a real value to the nearest bf16 (ties to even) and return its bit pattern.  Works from the value's
 * binade: a normal bf16 in [2^e, 2^(e+1)) has quantum 2^(e-7); below 2^-126 the quantum is 2^-133. */
uint16_t orc_bf16_encode(double v) {
  if (isnan(v)) return 0x7FC0;
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int e;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): leading bit is 2^(e-1) */
    int lead = e - 1;
    if (lead < -126) lead = -126;
    double q = ldexp(1.0, lead - 7);
    r = nearbyint(a / q) * q; /* default rounding mode: nearest, ties to even */
    double max_finite = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
    if (r > max_finite) r = INFINITY;
  }
  float f = (float)r; /* r is exactly representable: the conversion is exact */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t bits = (uint16_t)(u >> 16);
  if (neg) bits |= 0x8000;
  return bits;
}

double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Round to the nearest e4m3 value (ties to even), saturating at +-448.  The rounded magnitude is found from
 * its binade (quantum 2^(e-3) for normals, 2^-9 below 2^-6), and its code by searching the 127 non-negative
 * finite codes for the one that decodes to it. */
uint8_t orc_e4m3_encode(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  double r;
  if (a >= 448.0) {
    r = 448.0;
  } else if (a == 0.0) {
    r = 0.0;
  } else {
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -6) lead = -6;
    double q = ldexp(1.0, lead - 3);
    r = nearbyint(a / q) * q;
    if (r > 448.0) r = 448.0;
  }
  for (int c = 0; c < 127; ++c)
    if (orc_e4m3_decode((uint8_t)c) == r) return (uint8_t)(c | (neg ? 0x80 : 0));
  return 0x7F; /* unreachable for finite input */
}

/* ---------------------------------------------------------------------------------------------------------
 * Closed form of the dispatch + combine payload ("Expert parallelism and all-to-all", section "Traffic
 * math"): about 2 * k * H * bytes per token per MoE layer, the 2 counting the dispatch and the combine.
 * ------------------------------------------------------------------------------------------------------- */
uint64_t orc_payload_bytes(int64_t tokens, int32_t k, int32_t H, int32_t bytes_per_elem) {
  return (uint64_t)2 * (uint64_t)k * (uint64_t)H * (uint64_t)bytes_per_elem * (uint64_t)tokens;
}

/* ---------------------------------------------------------------------------------------------------------
 * Step 1: routing.  Each token's experts are ordered by (logit descending, expert id ascending), a full sort
 * of all E ids; slot j holds the j-th expert of that order.  The softmax over all E logits, restricted to the
 * k picks and divided by their sum, equals exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0), computed in fp64.
 * ------------------------------------------------------------------------------------------------------- */
typedef struct {
  float v;
  int32_t id;
} orc_key;

static int orc_key_cmp(const void* pa, const void* pb) {
  const orc_key* a = (const orc_key*)pa;
  const orc_key* b = (const orc_key*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

int orc_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx, double* topk_w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return 1;
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    orc_key* keys = (orc_key*)malloc(sizeof(orc_key) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) {
      keys[e].v = logits[t * E + e];
      keys[e].id = e;
    }
    qsort(keys, (size_t)E, sizeof(orc_key), orc_key_cmp);
    double l0 = (double)keys[0].v;
    double denom = 0.0;
    for (int32_t j = 0; j < k; ++j) denom += exp((double)keys[j].v - l0);
    for (int32_t j = 0; j < k; ++j) {
      topk_idx[t * k + j] = keys[j].id;
      topk_w[t * k + j] = exp((double)keys[j].v - l0) / denom;
    }
    free(keys);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------------------
 * Steps 2-3: counts, offsets and the permutation, from their definitions ("Expert Parallelism", aiwiki,
 * section "Implementation": sort by destination so each destination is one contiguous slab; count the rows
 * per destination; the inverse permutation undoes the sort).
 *   pair p = t*k + j carries expert topk_idx[p];
 *   counts[e]  = number of pairs with expert e;  offsets = exclusive prefix sum, offsets[E] = T*k;
 *   row_of_pair[p] = offsets[e] + number of earlier pairs (smaller p) with the same expert (a stable sort);
 *   token_of_row[row_of_pair[p]] = p / k.
 * ------------------------------------------------------------------------------------------------------- */
int orc_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                 int32_t* row_of_pair, int32_t* token_of_row) {
  if (T < 0 || k < 1 || E < 1) return 1;
  int64_t R = T * (int64_t)k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < R; ++p) {
    int32_t e = topk_idx[p];
    if (e < 0 || e >= E) return 1;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < R; ++p) {
    int32_t e = topk_idx[p];
    int32_t row = offsets[e] + seen[e];
    seen[e] += 1;
    row_of_pair[p] = row;
    token_of_row[row] = (int32_t)(p / k);
  }
  free(seen);
  return 0;
}

/* ---------------------------------------------------------------------------------------------------------
 * Step 4: the expert FFN of one (token, expert) pair and the weighted sum over the token's local picks.
 * Weights arrive in their natural layouts: w_gate, w_up [E_local][H][F], w_down [E_local][F][H]; fp8
 * weights carry one fp32 scale per 128 x 128 block: s_gate, s_up [E_local][H/128][F/128],
 * s_down [E_local][F/128][H/128].  fp8 x carries one fp32 scale per row per 128 columns.
 * ------------------------------------------------------------------------------------------------------- */
/* Fixed capacity (page "Expert Parallelism" (aiwiki), section "Implementation", the note after the sketch:
 * fixed-size buffers let every rank know every size in advance and remove the count exchange; the price is
 * that tokens beyond the buffer are dropped).  Reading taken: expert e keeps the first `capacity` of its
 * pairs in ascending pair order p = t*k + j; every other pair of e is dropped and contributes nothing to its
 * token; the kept weights are not renormalised.  Kept rows are packed: offsets are the prefix sums of the
 * kept counts and a kept pair's row is its expert's offset plus its rank among the expert's pairs.
 * keep[p] = 1 for kept pairs, 0 for dropped ones; row_of_pair[p] = -1 for dropped pairs. */
int orc_dispatch_capacity(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t capacity,
                          int32_t* counts, int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row,
                          uint8_t* keep) {
  if (T < 0 || k < 1 || E < 1 || capacity < 1) return 1;
  const int64_t R = T * (int64_t)k;
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (seen == NULL) return 1;
  /* pass 1: which pairs each expert keeps (its first `capacity`, scanning pairs in ascending order) */
  for (int64_t p = 0; p < R; ++p) {
    const int32_t e = topk_idx[p];
    if (e < 0 || e >= E) {
      free(seen);
      return 1;
    }
    keep[p] = seen[e] < capacity ? 1 : 0;
    seen[e] += 1;
  }
  /* kept counts and their prefix sums */
  for (int32_t e = 0; e < E; ++e) counts[e] = seen[e] < capacity ? seen[e] : capacity;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* pass 2: rows of the kept pairs */
  for (int32_t e = 0; e < E; ++e) seen[e] = 0;
  for (int64_t p = 0; p < R; ++p) {
    if (!keep[p]) {
      row_of_pair[p] = -1;
      continue;
    }
    const int32_t e = topk_idx[p];
    const int32_t row = offsets[e] + seen[e];
    seen[e] += 1;
    row_of_pair[p] = row;
    token_of_row[row] = (int32_t)(p / k);
  }
  free(seen);
  return 0;
}

static double orc_elem(int dtype, const void* base, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_BF16) return orc_bf16_decode(((const uint16_t*)base)[i]);
  return orc_e4m3_decode(((const uint8_t*)base)[i]);
}

/* Storage of the SwiGLU intermediate h in the layer dtype. */
static void orc_store_h(int dtype, double* a, int32_t F) {
  if (dtype == ORC_F32) {
    for (int32_t f = 0; f < F; ++f) a[f] = (double)(float)a[f];
  } else if (dtype == ORC_BF16) {
    for (int32_t f = 0; f < F; ++f) a[f] = orc_bf16_decode(orc_bf16_encode(a[f]));
  } else {
    /* one fp32 scale per 128 columns: scale = amax / 448 (1 if the group is zero); code = RNE(a / scale) */
    for (int32_t g0 = 0; g0 < F; g0 += 128) {
      double amax = 0.0;
      for (int32_t f = g0; f < g0 + 128; ++f)
        if (fabs(a[f]) > amax) amax = fabs(a[f]);
      float s = (amax == 0.0) ? 1.0f : (float)(amax / 448.0);
      for (int32_t f = g0; f < g0 + 128; ++f) a[f] = orc_e4m3_decode(orc_e4m3_encode(a[f] / (double)s)) * (double)s;
    }
  }
}

/* Router logits (page "Expert parallelism and all-to-all", section "Walking through one MoE layer", step 1:
 * the router runs on each GPU and gives every token its picks; here the router is the linear map x W_r that
 * the router-logit workloads define).  logits[t][e] = sum over h of x[t][h] W_r[h][e], in fp64 from the stored
 * x values decoded exactly; absdot[t][e] = sum over h of |x[t][h] W_r[h][e]| (for error bounds). */
int orc_router_logits(int32_t dtype, const void* x, const float* x_scales, int64_t T, int32_t H,
                      const float* w_router, int32_t E, double* logits, double* absdot) {
  if (dtype < 0 || dtype > 2 || H < 1 || E < 1 || T < 0) return 1;
  const int32_t HB = (H + 127) / 128;
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double s = 0.0, a = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        double xv = orc_elem(dtype, x, t * (int64_t)H + h);
        if (dtype == ORC_FP8) xv *= (double)x_scales[t * HB + h / 128];
        const double p = xv * (double)w_router[(int64_t)h * E + e];
        s += p;
        a += fabs(p);
      }
      logits[t * E + e] = s;
      absdot[t * E + e] = a;
    }
  }
  return 0;
}

int orc_moe_tokens(int32_t dtype, const void* x, const float* x_scales, int64_t T, int32_t H,
                   const int32_t* topk_idx, const double* topk_w, int32_t k, int32_t e_lo, int32_t E_local,
                   int32_t F, const void* w_gate, const void* w_up, const void* w_down, const float* s_gate,
                   const float* s_up, const float* s_down, const int64_t* tokens, int64_t n_tokens, double* out,
                   const uint8_t* keep) {
  if (dtype < 0 || dtype > 2 || H % 128 || F % 128 || k < 1) return 1;
  const int32_t HB = H / 128, FB = F / 128;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n_tokens; ++i) {
    int64_t t = tokens[i];
    double* o = out + i * (int64_t)H;
    for (int32_t c = 0; c < H; ++c) o[c] = 0.0;
    if (t < 0 || t >= T) continue;
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)F);
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    /* stored activation row, decoded exactly */
    for (int32_t c = 0; c < H; ++c) {
      xh[c] = orc_elem(dtype, x, t * (int64_t)H + c);
      if (dtype == ORC_FP8) xh[c] *= (double)x_scales[t * HB + c / 128];
    }
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j] - e_lo;
      if (e < 0 || e >= E_local) continue; /* not a local expert: contributes nothing here */
      if (keep != NULL && !keep[t * k + j]) continue; /* dropped by a fixed capacity: contributes nothing */
      const int64_t wo = (int64_t)e * H * F;
      /* g_f = sum_c x_c Wg[c][f], u_f = sum_c x_c Wu[c][f]  (ascending c for every f) */
      for (int32_t f = 0; f < F; ++f) g[f] = u[f] = 0.0;
      for (int32_t c = 0; c < H; ++c) {
        const double xc = xh[c];
        for (int32_t f = 0; f < F; ++f) {
          double wg = orc_elem(dtype, w_gate, wo + (int64_t)c * F + f);
          double wu = orc_elem(dtype, w_up, wo + (int64_t)c * F + f);
          if (dtype == ORC_FP8) {
            const int64_t sb = (int64_t)e * HB * FB + (int64_t)(c / 128) * FB + f / 128;
            wg *= (double)s_gate[sb];
            wu *= (double)s_up[sb];
          }
          g[f] += xc * wg;
          u[f] += xc * wu;
        }
      }
      /* SwiGLU: a_f = silu(g_f) * u_f, silu(z) = z / (1 + exp(-z)); then h is stored in the layer dtype */
      for (int32_t f = 0; f < F; ++f) g[f] = g[f] / (1.0 + exp(-g[f])) * u[f];
      orc_store_h(dtype, g, F);
      /* y_c = sum_f h_f Wd[f][c]  (ascending f for every c) */
      for (int32_t c = 0; c < H; ++c) y[c] = 0.0;
      for (int32_t f = 0; f < F; ++f) {
        const double hf = g[f];
        for (int32_t c = 0; c < H; ++c) {
          double wd = orc_elem(dtype, w_down, wo + (int64_t)f * H + c);
          if (dtype == ORC_FP8) wd *= (double)s_down[(int64_t)e * FB * HB + (int64_t)(f / 128) * HB + c / 128];
          y[c] += hf * wd;
        }
      }
      /* weighted sum in slot order */
      const double w = topk_w[t * k + j];
      for (int32_t c = 0; c < H; ++c) o[c] += w * y[c];
    }
    free(xh);
    free(g);
    free(u);
    free(y);
  }
  return 0;
}

/* The combine alone: out[t] = sum over local slots j (in slot order) of w[t][j] * y[row_of_pair[t*k+j]],
 * for expert outputs y [R][H] given in fp64.  Rows with no local pick are zero. */
int orc_combine(const double* y, const int32_t* row_of_pair, const int32_t* topk_idx, const double* topk_w,
                int64_t T, int32_t k, int32_t H, int32_t e_lo, int32_t E_local, double* out) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    double* o = out + t * (int64_t)H;
    for (int32_t c = 0; c < H; ++c) o[c] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < e_lo || e >= e_lo + E_local) continue;
      const double* yr = y + (int64_t)row_of_pair[t * k + j] * H;
      for (int32_t c = 0; c < H; ++c) o[c] += topk_w[t * k + j] * yr[c];
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------------------
 * The SwiGLU intermediate of chosen (token, pick) pairs, before and after its storage in the layer dtype
 * ("Expert parallelism and all-to-all", section "Walking through one MoE layer", step 3: the local experts'
 * products; h is the one value the method stores between the expert's two matrix products).  For each listed
 * pair p = t*k + j with local expert e = topk_idx[p] - e_lo, in fp64 from the exactly decoded inputs:
 *   g[i][f] = sum_c x_c Wg[c][f],  u[i][f] = sum_c x_c Wu[c][f],
 *   gabs[i][f] = sum_c |x_c Wg[c][f]|,  uabs[i][f] = sum_c |x_c Wu[c][f]|  (for error bounds),
 *   a[i][f] = silu(g_f) u_f,
 *   h_bits[i][f] the stored element: the fp32 bit pattern of a rounded to nearest even (fp32 layers), the bf16
 *                bit pattern (bf16), or the e4m3 code of a / scale (fp8),
 *   h_scales[i][f/128] (fp8 only) the group's fp32 scale: max |a| over the 128 columns / 448 rounded to fp32,
 *                1 if the group is all zero.
 * The storage rule is the one orc_moe_tokens applies to h.  A pair whose expert is not local gets zeros.
 * ------------------------------------------------------------------------------------------------------- */
int orc_pair_h(int32_t dtype, const void* x, const float* x_scales, int64_t T, int32_t H, const int32_t* topk_idx,
               int32_t k, int32_t e_lo, int32_t E_local, int32_t F, const void* w_gate, const void* w_up,
               const float* s_gate, const float* s_up, const int64_t* pairs, int64_t n, double* g, double* u,
               double* gabs, double* uabs, double* a, uint32_t* h_bits, float* h_scales) {
  if (dtype < 0 || dtype > 2 || H % 128 || F % 128 || k < 1 || T < 0) return 1;
  const int32_t HB = H / 128, FB = F / 128;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n; ++i) {
    double* gi = g + i * (int64_t)F;
    double* ui = u + i * (int64_t)F;
    double* ga = gabs + i * (int64_t)F;
    double* ua = uabs + i * (int64_t)F;
    double* ai = a + i * (int64_t)F;
    uint32_t* hb = h_bits + i * (int64_t)F;
    for (int32_t f = 0; f < F; ++f) gi[f] = ui[f] = ga[f] = ua[f] = ai[f] = 0.0, hb[f] = 0;
    if (h_scales != NULL)
      for (int32_t b = 0; b < FB; ++b) h_scales[i * FB + b] = 0.0f;
    const int64_t p = pairs[i];
    if (p < 0 || p >= T * k) continue;
    const int64_t t = p / k;
    const int32_t e = topk_idx[p] - e_lo;
    if (e < 0 || e >= E_local) continue;
    const int64_t wo = (int64_t)e * H * F;
    for (int32_t c = 0; c < H; ++c) {
      double xc = orc_elem(dtype, x, t * (int64_t)H + c);
      if (dtype == ORC_FP8) xc *= (double)x_scales[t * HB + c / 128];
      for (int32_t f = 0; f < F; ++f) {
        double wg = orc_elem(dtype, w_gate, wo + (int64_t)c * F + f);
        double wu = orc_elem(dtype, w_up, wo + (int64_t)c * F + f);
        if (dtype == ORC_FP8) {
          const int64_t sb = (int64_t)e * HB * FB + (int64_t)(c / 128) * FB + f / 128;
          wg *= (double)s_gate[sb];
          wu *= (double)s_up[sb];
        }
        gi[f] += xc * wg;
        ui[f] += xc * wu;
        ga[f] += fabs(xc * wg);
        ua[f] += fabs(xc * wu);
      }
    }
    for (int32_t f = 0; f < F; ++f) ai[f] = gi[f] / (1.0 + exp(-gi[f])) * ui[f];
    if (dtype == ORC_F32) {
      for (int32_t f = 0; f < F; ++f) {
        const float v = (float)ai[f];
        memcpy(&hb[f], &v, 4);
      }
    } else if (dtype == ORC_BF16) {
      for (int32_t f = 0; f < F; ++f) hb[f] = orc_bf16_encode(ai[f]);
    } else {
      for (int32_t g0 = 0; g0 < F; g0 += 128) {
        double amax = 0.0;
        for (int32_t f = g0; f < g0 + 128; ++f)
          if (fabs(ai[f]) > amax) amax = fabs(ai[f]);
        const float sc = (amax == 0.0) ? 1.0f : (float)(amax / 448.0);
        for (int32_t f = g0; f < g0 + 128; ++f) hb[f] = orc_e4m3_encode(ai[f] / (double)sc);
        if (h_scales != NULL) h_scales[i * FB + g0 / 128] = sc;
      }
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------------------------
 * Backward pass (training).  The pages ask only that the gradients, those of the routing weights included,
 * reach every token ("Expert parallelism" (transformers docs), section "Adding an implementation": the
 * collectives are wrapped so that autograd carries gradients back); the rest is the calculus of the forward
 * layer above.  For a kept local pair (t, j) of expert e with routing weight w and loss gradient dout_t:
 *   forward:  g = x Wg_e, u = x Wu_e, a = silu(g) * u, h = a stored in the layer dtype, y = h Wd_e
 *   dw[t][j]  = <dout_t, y>                  (the gradient of the routing weight)
 *   dy        = w dout_t
 *   dWd_e    += h^T dy                        (h as stored: y was computed from it)
 *   dh        = dy Wd_e^T
 *   dg        = dh * u * silu'(g),  silu'(z) = s (1 + z (1 - s)),  s = 1 / (1 + exp(-z))
 *   du        = dh * silu(g)
 *   dWg_e    += x^T dg,   dWu_e += x^T du,   dx_t += dg Wg_e^T + du Wu_e^T
 * The storage of h is differentiated as the identity (straight through).  Routing weights are the softmax over
 * the k picks, w_j = exp(l_j) / sum_i exp(l_i), whose Jacobian gives
 *   dlogits[t][idx_m] = w_m (dw_m - sum_i w_i dw_i)   for every pick m, and 0 for the other experts;
 * picks that are not local (or dropped by a capacity) have dw = 0 here, so this is this share's part of a sum.
 * fp8 layers are not covered (returns 1).
 * ------------------------------------------------------------------------------------------------------- */
static double orc_round_h(int dtype, double v) {
  if (dtype == ORC_F32) return (double)(float)v;
  return orc_bf16_decode(orc_bf16_encode(v));
}

/* g, u of one pair (ascending c for every f) */
static void orc_pair_gu(int dtype, const double* xh, int32_t H, int32_t F, const void* w_gate, const void* w_up,
                        int64_t wo, double* g, double* u) {
  for (int32_t f = 0; f < F; ++f) g[f] = u[f] = 0.0;
  for (int32_t c = 0; c < H; ++c) {
    const double xc = xh[c];
    for (int32_t f = 0; f < F; ++f) {
      g[f] += xc * orc_elem(dtype, w_gate, wo + (int64_t)c * F + f);
      u[f] += xc * orc_elem(dtype, w_up, wo + (int64_t)c * F + f);
    }
  }
}

static void orc_decode_row(int dtype, const void* x, int64_t t, int32_t H, double* xh) {
  for (int32_t c = 0; c < H; ++c) xh[c] = orc_elem(dtype, x, t * (int64_t)H + c);
}

static int orc_bwd_args_ok(int32_t dtype, int32_t H, int32_t F, int32_t k, int32_t E, int32_t e_lo,
                           int32_t E_local) {
  return (dtype == ORC_F32 || dtype == ORC_BF16) && H > 0 && F > 0 && k >= 1 && k <= E && e_lo >= 0 &&
         E_local >= 1 && e_lo + E_local <= E;
}

/* Per-token gradients for the listed tokens: dx rows [n][H], dw rows [n][k], dlogits rows [n][E] (each output
 * may be NULL).  dx_abs (may be NULL) [n][H]: the sum of the absolute values of dx's terms,
 * sum over pairs and f of |Wg[c][f] dg_f| + |Wu[c][f] du_f| (for rounding-error bounds); dx_sq (may be NULL):
 * the sum of their squares (for rounding-noise estimates). */
int orc_bwd_rows(int32_t dtype, const void* x, int64_t T, int32_t H, const int32_t* topk_idx, const double* topk_w,
                 int32_t k, int32_t E, int32_t e_lo, int32_t E_local, int32_t F, const void* w_gate, const void* w_up,
                 const void* w_down, const double* dout, const uint8_t* keep, const int64_t* tokens, int64_t n,
                 double* dx, double* dtw, double* dlogits, double* dx_abs, double* dx_sq) {
  if (!orc_bwd_args_ok(dtype, H, F, k, E, e_lo, E_local)) return 1;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n; ++i) {
    const int64_t t = tokens[i];
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)F);
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* hst = (double*)malloc(sizeof(double) * (size_t)F);
    double* dh = (double*)malloc(sizeof(double) * (size_t)F);
    double* dwv = (double*)malloc(sizeof(double) * (size_t)k);
    if (dx) for (int32_t c = 0; c < H; ++c) dx[i * H + c] = 0.0;
    if (dx_abs) for (int32_t c = 0; c < H; ++c) dx_abs[i * H + c] = 0.0;
    if (dx_sq) for (int32_t c = 0; c < H; ++c) dx_sq[i * H + c] = 0.0;
    for (int32_t j = 0; j < k; ++j) dwv[j] = 0.0;
    if (t >= 0 && t < T) {
      orc_decode_row(dtype, x, t, H, xh);
      const double* dt = dout + t * (int64_t)H;
      for (int32_t j = 0; j < k; ++j) {
        const int32_t e = topk_idx[t * k + j] - e_lo;
        if (e < 0 || e >= E_local) continue;
        if (keep != NULL && !keep[t * k + j]) continue;
        const int64_t wo = (int64_t)e * H * F;
        const double w = topk_w[t * k + j];
        orc_pair_gu(dtype, xh, H, F, w_gate, w_up, wo, g, u);
        for (int32_t f = 0; f < F; ++f) hst[f] = orc_round_h(dtype, g[f] / (1.0 + exp(-g[f])) * u[f]);
        /* dw = <dout_t, y> with y_c = sum_f h_f Wd[f][c]; dh_f = sum_c (w dout_c) Wd[f][c] */
        double dws = 0.0;
        for (int32_t f = 0; f < F; ++f) {
          double d = 0.0;
          for (int32_t c = 0; c < H; ++c) {
            const double wd = orc_elem(dtype, w_down, wo + (int64_t)f * H + c);
            d += w * dt[c] * wd;
            dws += hst[f] * wd * dt[c];
          }
          dh[f] = d;
        }
        dwv[j] = dws;
        if (dx) {
          for (int32_t f = 0; f < F; ++f) {
            const double s = 1.0 / (1.0 + exp(-g[f]));
            const double dg = dh[f] * u[f] * s * (1.0 + g[f] * (1.0 - s));
            const double du = dh[f] * g[f] * s;
            g[f] = dg; /* reuse: dg */
            u[f] = du; /* reuse: du */
          }
          for (int32_t c = 0; c < H; ++c) {
            double acc = 0.0, aab = 0.0, asq = 0.0;
            for (int32_t f = 0; f < F; ++f) {
              const double tg = orc_elem(dtype, w_gate, wo + (int64_t)c * F + f) * g[f];
              const double tu = orc_elem(dtype, w_up, wo + (int64_t)c * F + f) * u[f];
              acc += tg + tu;
              aab += fabs(tg) + fabs(tu);
              asq += tg * tg + tu * tu;
            }
            dx[i * H + c] += acc;
            if (dx_abs) dx_abs[i * H + c] += aab;
            if (dx_sq) dx_sq[i * H + c] += asq;
          }
        }
      }
    }
    if (dtw) for (int32_t j = 0; j < k; ++j) dtw[i * k + j] = dwv[j];
    if (dlogits) {
      double* dl = dlogits + i * (int64_t)E;
      for (int32_t e = 0; e < E; ++e) dl[e] = 0.0;
      if (t >= 0 && t < T) {
        double sw = 0.0;
        for (int32_t j = 0; j < k; ++j) sw += topk_w[t * k + j] * dwv[j];
        for (int32_t j = 0; j < k; ++j) dl[topk_idx[t * k + j]] = topk_w[t * k + j] * (dwv[j] - sw);
      }
    }
    free(xh);
    free(g);
    free(u);
    free(hst);
    free(dh);
    free(dwv);
  }
  return 0;
}

/* One weight-gradient element: which = 0 dWg[e][c][f], 1 dWu[e][c][f] (ii = c, jj = f), 2 dWd[e][f][c]
 * (ii = f, jj = c); e is the local expert index.  Sum over the expert's kept pairs in ascending pair order. */
static double orc_bwd_weight_elem(int32_t dtype, const void* x, int64_t T, int32_t H, const int32_t* topk_idx,
                                  const double* topk_w, int32_t k, int32_t e_lo, int32_t F, const void* w_gate,
                                  const void* w_up, const void* w_down, const double* dout, const uint8_t* keep,
                                  int32_t which, int32_t e, int32_t ii, int32_t jj, double* xh, double* absacc,
                                  double* sqacc) {
  const int64_t wo = (int64_t)e * H * F;
  const int32_t f = which == 2 ? ii : jj, c0 = which == 2 ? jj : ii;
  double acc = 0.0, aab = 0.0, asq = 0.0;
  for (int64_t p = 0; p < T * (int64_t)k; ++p) {
    if (topk_idx[p] != e_lo + e) continue;
    if (keep != NULL && !keep[p]) continue;
    const int64_t t = p / k;
    const double w = topk_w[p];
    orc_decode_row(dtype, x, t, H, xh);
    double g = 0.0, u = 0.0;
    for (int32_t c = 0; c < H; ++c) {
      g += xh[c] * orc_elem(dtype, w_gate, wo + (int64_t)c * F + f);
      u += xh[c] * orc_elem(dtype, w_up, wo + (int64_t)c * F + f);
    }
    const double* dt = dout + t * (int64_t)H;
    if (which == 2) {
      const double hf = orc_round_h(dtype, g / (1.0 + exp(-g)) * u);
      acc += hf * (w * dt[c0]);
      aab += fabs(hf * (w * dt[c0]));
      asq += (hf * (w * dt[c0])) * (hf * (w * dt[c0]));
    } else {
      double dh = 0.0;
      for (int32_t c = 0; c < H; ++c) dh += w * dt[c] * orc_elem(dtype, w_down, wo + (int64_t)f * H + c);
      const double s = 1.0 / (1.0 + exp(-g));
      const double d = which == 0 ? dh * u * s * (1.0 + g * (1.0 - s)) : dh * g * s;
      acc += xh[c0] * d;
      aab += fabs(xh[c0] * d);
      asq += (xh[c0] * d) * (xh[c0] * d);
    }
  }
  *absacc = aab;
  *sqacc = asq;
  return acc;
}

int orc_bwd_weight_elems(int32_t dtype, const void* x, int64_t T, int32_t H, const int32_t* topk_idx,
                         const double* topk_w, int32_t k, int32_t E, int32_t e_lo, int32_t E_local, int32_t F,
                         const void* w_gate, const void* w_up, const void* w_down, const double* dout,
                         const uint8_t* keep, const int32_t* which, const int32_t* ex, const int32_t* ii,
                         const int32_t* jj, int64_t n, double* out, double* out_abs, double* out_sq) {
  if (!orc_bwd_args_ok(dtype, H, F, k, E, e_lo, E_local)) return 1;
  int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < n; ++i) {
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double ab = 0.0, sq = 0.0;
    out[i] = orc_bwd_weight_elem(dtype, x, T, H, topk_idx, topk_w, k, e_lo, F, w_gate, w_up, w_down, dout, keep,
                                 which[i], ex[i], ii[i], jj[i], xh, &ab, &sq);
    if (out_abs) out_abs[i] = ab;
    if (out_sq) out_sq[i] = sq;
    free(xh);
  }
  return 0;
}

/* All weight gradients: dw_gate, dw_up [E_local][H][F], dw_down [E_local][F][H] (small layers).  The *_abs
 * outputs (may be NULL) hold the sums of the absolute values of the terms, for rounding-error bounds, the *_sq
 * outputs (may be NULL) the sums of their squares, for rounding-noise estimates. */
int orc_bwd_weights(int32_t dtype, const void* x, int64_t T, int32_t H, const int32_t* topk_idx,
                    const double* topk_w, int32_t k, int32_t E, int32_t e_lo, int32_t E_local, int32_t F,
                    const void* w_gate, const void* w_up, const void* w_down, const double* dout,
                    const uint8_t* keep, double* dw_gate, double* dw_up, double* dw_down, double* ab_gate,
                    double* ab_up, double* ab_down, double* sq_gate, double* sq_up, double* sq_down) {
  if (!orc_bwd_args_ok(dtype, H, F, k, E, e_lo, E_local)) return 1;
  int32_t e;
#pragma omp parallel for schedule(dynamic, 1)
  for (e = 0; e < E_local; ++e) {
    const int64_t wo = (int64_t)e * H * F;
    double* xh = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)F);
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* dh = (double*)malloc(sizeof(double) * (size_t)F);
    double* dy = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t q = 0; q < (int64_t)H * F; ++q) dw_gate[wo + q] = dw_up[wo + q] = dw_down[wo + q] = 0.0;
    if (ab_gate)
      for (int64_t q = 0; q < (int64_t)H * F; ++q) ab_gate[wo + q] = ab_up[wo + q] = ab_down[wo + q] = 0.0;
    if (sq_gate)
      for (int64_t q = 0; q < (int64_t)H * F; ++q) sq_gate[wo + q] = sq_up[wo + q] = sq_down[wo + q] = 0.0;
    for (int64_t p = 0; p < T * (int64_t)k; ++p) {
      if (topk_idx[p] != e_lo + e) continue;
      if (keep != NULL && !keep[p]) continue;
      const int64_t t = p / k;
      orc_decode_row(dtype, x, t, H, xh);
      orc_pair_gu(dtype, xh, H, F, w_gate, w_up, wo, g, u);
      for (int32_t c = 0; c < H; ++c) dy[c] = topk_w[p] * dout[t * (int64_t)H + c];
      for (int32_t f = 0; f < F; ++f) {
        const double hf = orc_round_h(dtype, g[f] / (1.0 + exp(-g[f])) * u[f]);
        double d = 0.0;
        for (int32_t c = 0; c < H; ++c) {
          dw_down[wo + (int64_t)f * H + c] += hf * dy[c];
          if (ab_down) ab_down[wo + (int64_t)f * H + c] += fabs(hf * dy[c]);
          if (sq_down) sq_down[wo + (int64_t)f * H + c] += (hf * dy[c]) * (hf * dy[c]);
          d += dy[c] * orc_elem(dtype, w_down, wo + (int64_t)f * H + c);
        }
        dh[f] = d;
      }
      for (int32_t f = 0; f < F; ++f) {
        const double s = 1.0 / (1.0 + exp(-g[f]));
        const double dg = dh[f] * u[f] * s * (1.0 + g[f] * (1.0 - s));
        const double du = dh[f] * g[f] * s;
        for (int32_t c = 0; c < H; ++c) {
          dw_gate[wo + (int64_t)c * F + f] += xh[c] * dg;
          dw_up[wo + (int64_t)c * F + f] += xh[c] * du;
          if (ab_gate) {
            ab_gate[wo + (int64_t)c * F + f] += fabs(xh[c] * dg);
            ab_up[wo + (int64_t)c * F + f] += fabs(xh[c] * du);
          }
          if (sq_gate) {
            sq_gate[wo + (int64_t)c * F + f] += (xh[c] * dg) * (xh[c] * dg);
            sq_up[wo + (int64_t)c * F + f] += (xh[c] * du) * (xh[c] * du);
          }
        }
      }
    }
    free(xh);
    free(g);
    free(u);
    free(dh);
    free(dy);
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
