// Backward pass of the grouped SwiGLU expert FFN and of the routing weights (training).
//
// Method: page "Expert parallelism" (transformers docs), section "Adding an implementation": gradients, those of
// the routing weights included, have to reach every token.  The arithmetic is the calculus of the forward layer
// (route, dispatch, h = silu(x Wg) * (x Wu), y = h Wd, out = sum_j w_j y_j).  For a pair row r of expert e with
// token t and weight w, and dout = dL/dout:
//   dO[r]   = dout[t]                                       gather (a copy: no rounding)
//   dh      = w * (dO Wd_e^T) -> dg = dh * u * silu'(g), du = dh * silu(g)     (MODE_DH, fused epilogue; g, u
//                                                            are the forward's fp32 pre-activations)
//   dX[r]   = dg Wg_e^T + du Wu_e^T                         (MODE_DX: one reduction over [dg | du])
//   dx[t]   = sum over the token's rows of dX                (un-permute, fp32 sums in slot order)
//   dWd_e   = (w h)_e^T dO_e, dWg_e = X_e^T dg_e, dWu_e = X_e^T du_e           (MODE_WG: reduction over rows)
//   dw[t,j] = <dout[t], y[r]>;  dlogits = w (dw - sum_i w_i dw_i) on the picks
//
// Design (gfx950):
//  * One grouped GEMM kernel, C[m][n] = sum_k A[m][k] B[n][k] with both operands' reduction dimension contiguous,
//    stages of each row's reduction slice moved global -> LDS with direct 16-byte loads and counted waits, and
//    the forward products' swizzled LDS layout and stage MFMA work (gemm_tile.h): bf16 on
//    v_mfma_f32_32x32x16_bf16 with double-buffered fragments, fp32 on v_mfma_f32_32x32x2f32, fp32 accumulation.
//    bf16 shapes that divide 256 use 8 wavefronts (320 x 256 tiles for the ragged data products, 256 x 256 for
//    the weight products); the rest 128 x 128 over 4.
//  * Tile order (gemm_tile.h, shared with the forward products): the data products go expert by expert, row
//    tiles fastest inside each column tile, or column tiles fastest for an expert with more rows than the
//    product has weight rows, with the 8 XCDs each taking one contiguous range (an expert's rows stay in one L2
//    across its column tiles); the weight products go in groups of 4 row tiles, column tiles next, row tiles
//    fastest inside a group, XCD-contiguous too.
//  * The data products (dh, dX) use the weights in their natural layouts, whose rows already have the reduction
//    dimension contiguous: Wd_e [F][H] for dh, the rows of Wg_e and Wu_e [H][F] back to back for dX.  Ragged M
//    per expert comes from the device-resident offsets, as in the forward kernel.
//  * The weight products reduce over an expert's rows, so their operands are transposed first into [C][Rpad]
//    buffers in which expert e owns columns [poff[e], poff[e+1]) (its row count rounded up to 64, zero-filled):
//    every expert's reduction range is then whole stages, and an expert with no rows gets a zero gradient.
//  * Roundings (bf16 layers): [dg | du] and w * h are stored in bf16 as matrix operands; dout and x_perm are
//    already bf16, and the routing weight of dh is applied in fp32, so every gradient term carries one.
#include <type_traits>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace moe {
namespace bwd {

constexpr int PADC = 64;  // reduction-column granularity of the transposed operands

enum Mode { MODE_DH = 0, MODE_DX = 1, MODE_WG = 2 };

// Tile shapes: 256 x 256 over 8 wavefronts (2 x 4, 128 x 64 each) with two 128-byte stages, where the shape
// divides; otherwise 128 x 128 over 4 wavefronts.  bf16 128-row tiles stream 64-byte slices through 4 stages;
// fp32 keeps 128-byte slices (32 values) and 2 stages.
template <int DT, int BIG>
struct Cfg;
template <>
struct Cfg<0, 0> {
  static constexpr int ESZ = 4, RB = 128, NS = 2, BM = 128, BN = 128, WM = 2, WN = 2;
};
template <>
struct Cfg<1, 0> {
  static constexpr int ESZ = 2, RB = 64, NS = 4, BM = 128, BN = 128, WM = 2, WN = 2;
};
template <>
struct Cfg<1, 1> {
  static constexpr int ESZ = 2, RB = 128, NS = 2, BM = 256, BN = 256, WM = 2, WN = 4;
};
// ragged row blocks of ~2 x 256 rows per expert: 320 rows avoid a nearly empty third block
template <>
struct Cfg<1, 2> {
  static constexpr int ESZ = 2, RB = 128, NS = 2, BM = 320, BN = 256, WM = 2, WN = 4;
};

using tile::swz;

struct GemmArgs {
  const uint8_t* A;        // DH: dO (dout rows) [R][H]; DX: dGU [R][2F]; WG: A^T [M][Rpad]
  const uint8_t* B0;       // DH: Wd natural [E][F][H]; DX: Wg natural [E][H][F]; WG: B^T [N][Rpad]
  const uint8_t* B1;       // DX: Wu natural [E][H][F]
  const int32_t* offsets;  // global expert offsets (DH, DX)
  const int32_t* poff;     // WG: padded column offsets [E_local + 1]
  int e_lo, E_local;
  int M, N;                // WG: per-expert output shape; DH, DX: N = output columns
  int K;                   // DH: H, DX: 2F (reduction length, values); WG: Rpad (row length of A^T and B^T)
  int F;                   // DH: F (epilogue), DX: F (the [Wg | Wu] split)
  int n_tiles, m_tiles;    // WG: m_tiles = M / BM; DH, DX: worst-case m-tiles
  const float* GU;         // DH: saved pre-activations [R][2F] fp32
  const float* rw;         // DH: routing weight of each row
  uint8_t* DGU;            // DH: out [R][2F] (layer dtype)
  float* C;                // DX: [R][N] fp32; WG: [E_local][M][N] fp32
};

template <int DT>
MOE_DEV float load_val(const uint8_t* p, int64_t i) {
  if constexpr (DT == 0) return reinterpret_cast<const float*>(p)[i];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}
template <int DT>
MOE_DEV void store_val(uint8_t* p, int64_t i, float v) {
  if constexpr (DT == 0)
    reinterpret_cast<float*>(p)[i] = v;
  else
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
}

template <int DT, int MODE, int BIG>
__global__ __launch_bounds__((64 * Cfg<DT, BIG>::WM * Cfg<DT, BIG>::WN)) void bwd_gemm_kernel(const GemmArgs a) {
  using C_ = Cfg<DT, BIG>;
  constexpr int RB = C_::RB, NS = C_::NS, ESZ = C_::ESZ;
  constexpr int BM = C_::BM, BN = C_::BN, WM = C_::WM, WN = C_::WN, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN, MB = WTM / 32, NB = WTN / 32;
  constexpr int RPI = 1024 / RB;  // rows one wavefront direct-load instruction fills
  constexpr int A_INS = BM / (NW * RPI), B_INS = BN / (NW * RPI);
  constexpr int NL = A_INS + B_INS;
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int CPR = RB / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  __shared__ int s_tile[4];

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform_int(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const int lr = lane & 31, lh = lane >> 5;

  // ---- tile -> (expert, rows, columns, reduction range)
  int e, m0, m_end, n0, k0v, kv;  // k0v, kv: first reduction value and count
  if constexpr (MODE == MODE_WG) {
    // (expert, group of 4 row tiles, column tile, row tile): the 32 tiles an XCD runs at once cover 4 row tiles
    // x 8 column tiles, whose operand slices fit its L2 together (measured on the Mixtral shape: backward 4229
    // -> 4046 us against row tiles fastest, whose 32 tiles span an expert's whole A operand; groups of 1, 2 or 8
    // gain less); the 8 XCDs (dealt workgroup ids round-robin) each take one contiguous range
    const int per = a.m_tiles * a.n_tiles;
    const int L = tile::xcd_tile_index(gridDim.x, blockIdx.x);
    e = L / per;
    const int rem = L % per;
    const int gm = a.m_tiles % 4 == 0 ? 4 : a.m_tiles;
    const int g = rem / (gm * a.n_tiles), r2 = rem % (gm * a.n_tiles);
    n0 = (r2 / gm) * BN;
    m0 = (g * gm + r2 % gm) * BM;
    m_end = a.M;
    k0v = a.poff[e];
    kv = a.poff[e + 1] - k0v;
  } else {
    // the forward products' ragged schedule (tile::expert_tile): expert by expert, row tiles fastest so the row
    // tiles sharing a weight tile are consecutive and an expert's rows stay in L2 across its column tiles;
    // column tiles fastest for an expert with more rows than weight rows (its rows stream once); each XCD
    // takes one contiguous range of the valid tiles; surplus workgroups of the worst-case grid exit at once.
    if (wid == 0) {
      const tile::ExpertTile t = tile::workgroup_tile<BM>(a.offsets, a.e_lo, a.E_local, a.n_tiles, 1, a.N,
                                                           blockIdx.x);
      if (lane == 0) {
        s_tile[0] = t.e;
        s_tile[1] = t.m0;
        s_tile[2] = t.m_end;
        s_tile[3] = t.ni * BN;
      }
    }
    __syncthreads();
    e = uniform_int(s_tile[0]);  // uniform: scalar registers for the addresses and loop bounds
    if (e < 0) return;
    m0 = uniform_int(s_tile[1]);
    m_end = uniform_int(s_tile[2]);
    n0 = uniform_int(s_tile[3]);
    k0v = 0;
    kv = a.K;
  }
  const int nk = kv * ESZ / RB;  // stages
  const int64_t Kb = (int64_t)a.K * ESZ;  // bytes per A row (and per B row, except DX)

  // ---- operand addressing: uniform 64-bit bases, 32-bit per-lane offsets
  const int uwid = uniform_int(wid);
  const uint8_t* a_base;
  const uint8_t* b_base0;
  const uint8_t* b_base1 = nullptr;
  int64_t b_row_bytes = Kb;
  int nk_split = nk;  // DX: stages of the first operand pair (dg with Wg); later stages use du with Wu
  if constexpr (MODE == MODE_WG) {
    a_base = uniform_ptr(a.A + (int64_t)m0 * Kb + (int64_t)k0v * ESZ);
    b_base0 = uniform_ptr(a.B0 + (int64_t)n0 * Kb + (int64_t)k0v * ESZ);
  } else if constexpr (MODE == MODE_DH) {
    a_base = uniform_ptr(a.A + (int64_t)m0 * Kb);
    b_base0 = uniform_ptr(a.B0 + ((int64_t)e * a.N + n0) * Kb);  // Wd_e rows f (N = F), H values each
  } else {
    a_base = uniform_ptr(a.A + (int64_t)m0 * Kb);
    b_row_bytes = (int64_t)a.F * ESZ;
    b_base0 = uniform_ptr(a.B0 + ((int64_t)e * a.N + n0) * b_row_bytes);  // Wg_e rows h (N = H), F values each
    b_base1 = uniform_ptr(a.B1 + ((int64_t)e * a.N + n0) * b_row_bytes);
    nk_split = (int)(b_row_bytes / RB);
  }
  uint32_t a_off[A_INS], b_off[B_INS];
#pragma unroll
  for (int q = 0; q < A_INS; ++q) {
    const int r = (uwid * A_INS + q) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<RB>(r);
    const int gr = MODE == MODE_WG ? r : min(m0 + r, m_end - 1) - m0;
    a_off[q] = (uint32_t)(gr * Kb + c * 16);
  }
#pragma unroll
  for (int q = 0; q < B_INS; ++q) {
    const int r = (uwid * B_INS + q) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<RB>(r);
    b_off[q] = (uint32_t)(r * b_row_bytes + c * 16);
  }
  auto load_stage = [&](uint8_t* dst, int kt) {
    const uint8_t* ab = uniform_ptr(a_base + (int64_t)kt * RB);
    const uint8_t* bb = uniform_ptr((MODE == MODE_DX && kt >= nk_split) ? b_base1 + (int64_t)(kt - nk_split) * RB
                                                                         : b_base0 + (int64_t)kt * RB);
#pragma unroll
    for (int q = 0; q < A_INS; ++q) load_lds16(ab, a_off[q], dst + (wid * A_INS + q) * 1024);
#pragma unroll
    for (int q = 0; q < B_INS; ++q) load_lds16(bb, b_off[q], dst + BM * RB + (wid * B_INS + q) * 1024);
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  int arow[MB], brow[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) arow[i] = wm * WTM + i * 32 + lr;
#pragma unroll
  for (int j = 0; j < NB; ++j) brow[j] = wn * WTN + j * 32 + lr;
  const tile::FragOff ao = tile::frag_offsets<RB, RB / 32>(arow[0], lh, 2);
  const tile::FragOff bo = tile::frag_offsets<RB, RB / 32>(brow[0], lh, 2);

  if (nk > 0) {
    // slices 0 .. NS-2 in flight; each iteration waits for its own slice, meets the other wavefronts (the buffer
    // read last iteration is then free), refills it with slice kt + NS - 1 (clamped: loaded, never read) and
    // computes slice kt
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) load_stage(smem + s * STAGE, min(s, nk - 1));
    int cb = 0, fb = NS - 1;
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NS - 2) * NL>();
      __syncthreads();
      load_stage(smem + fb * STAGE, min(kt + NS - 1, nk - 1));
      const uint8_t* As = smem + cb * STAGE;
      const uint8_t* Bs = As + BM * RB;
      if constexpr (DT == 1)
        tile::mma_stage_bf16<RB, MB, NB>(As, Bs, arow, brow, ao, bo, acc);
      else
        tile::mma_stage_f32<MB, NB>(As, Bs, arow, brow, ao, bo, acc, MB);
      cb = cb + 1 == NS ? 0 : cb + 1;
      fb = fb + 1 == NS ? 0 : fb + 1;
    }
    wait_vmcnt0();
  }

  // ---- epilogues; accumulator element v of a lane: row (v/4)*8 + 4*(lane/32) + v%4, column lane%32
  if constexpr (MODE == MODE_DH) {
    // SwiGLU backward at (row gm, column f), dh = w * d: the saved g, u and routing weights of 8 accumulator
    // values are loaded before any of their results is stored (restrict-qualified, so the loads are not held
    // behind the stores; rows past the slab read the slab's last row and store nothing)
    const float* __restrict__ GU = a.GU;
    const float* __restrict__ RW = a.rw;
    uint8_t* __restrict__ DGU = a.DGU;
    const int64_t F = a.F;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v0 = 0; v0 < 16; v0 += 8) {
        float gv[8][NB], uv[8][NB], wv[8];
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
          const int v = v0 + vv;
          const int gm = min(m0 + wm * WTM + i * 32 + (v >> 2) * 8 + 4 * lh + (v & 3), m_end - 1);
          wv[vv] = RW[gm];
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int64_t o = (int64_t)gm * 2 * F + n0 + wn * WTN + j * 32 + lr;
            gv[vv][j] = GU[o];
            uv[vv][j] = GU[o + F];
          }
        }
#pragma unroll
        for (int vv = 0; vv < 8; ++vv) {
          const int v = v0 + vv;
          const int gm = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + 4 * lh + (v & 3);
          if (gm >= m_end) continue;
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int64_t o = (int64_t)gm * 2 * F + n0 + wn * WTN + j * 32 + lr;
            const float g = gv[vv][j], u = uv[vv][j];
            const float dh = wv[vv] * acc[i][j][v];
            const float sg = 1.0f / (1.0f + __expf(-g));
            store_val<DT>(DGU, o, dh * u * sg * (1.0f + g * (1.0f - sg)));
            store_val<DT>(DGU, o + F, dh * g * sg);
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WTM + i * 32 + (v >> 2) * 8 + 4 * lh + (v & 3);
        const int gm = m0 + row;
        if (gm >= m_end) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = n0 + wn * WTN + j * 32 + lr;
          const float d = acc[i][j][v];
          if constexpr (MODE == MODE_DX) {
            a.C[(int64_t)gm * a.N + col] = d;
          } else {
            // the fp32 weight gradient (1.88 GB per launch on the Mixtral shape) is read by nothing in this
            // pass: streaming stores keep it from evicting the operand slices the other tiles share in L2
            // (backward 4090 -> 3867 us measured)
            __builtin_nontemporal_store(d, &a.C[((int64_t)e * a.M + gm) * a.N + col]);
          }
        }
      }
  }
}

// poff[0] = 0, poff[e + 1] = poff[e] + (count of local expert e rounded up to PADC)
__global__ void pad_offsets_kernel(const int32_t* __restrict__ offsets, int e_lo, int E_local,
                                   int32_t* __restrict__ poff) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  poff[0] = 0;
  for (int e = 0; e < E_local; ++e) {
    const int cnt = offsets[e_lo + e + 1] - offsets[e_lo + e];
    acc += (cnt + PADC - 1) / PADC * PADC;
    poff[e + 1] = acc;
  }
}

// pair of each row of the window: por[r] = t*k + j with row_of_pair[t*k + j] == r
__global__ __launch_bounds__(256) void pair_of_row_kernel(const int32_t* __restrict__ tok,
                                                          const int32_t* __restrict__ rop, int k,
                                                          const int32_t* __restrict__ offsets, int e_lo, int e_hi,
                                                          int32_t* __restrict__ por) {
  const int64_t r = offsets[e_lo] + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= offsets[e_hi]) return;
  const int t = tok[r];
  int p = -1;
  for (int j = 0; j < k; ++j)
    if (rop[(int64_t)t * k + j] == r) p = t * k + j;
  por[r] = p;
}

// dO[r] = dout[token(r)] (16-byte copies) and rw[r] = w[pair(r)]; one workgroup per row
__global__ __launch_bounds__(256) void dout_gather_kernel(const uint8_t* __restrict__ dout, int64_t row_bytes,
                                                          const int32_t* __restrict__ tok,
                                                          const int32_t* __restrict__ por,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ offsets, int e_lo, int e_hi,
                                                          uint8_t* __restrict__ dO, float* __restrict__ rw) {
  const int64_t r = offsets[e_lo] + blockIdx.x;
  if (r >= offsets[e_hi]) return;
  const int64_t t = tok[r];
  if (threadIdx.x == 0) rw[r] = wts[por[r]];
  const i32x4_t* src = reinterpret_cast<const i32x4_t*>(dout + t * row_bytes);
  i32x4_t* dst = reinterpret_cast<i32x4_t*>(dO + r * row_bytes);
  for (int64_t c = threadIdx.x; c < row_bytes / 16; c += blockDim.x) dst[c] = src[c];
}

// Transpose of the window's rows into the padded column layout: dst[c][poff[e] + i] = s_r src[r][c] for
// r = offsets[e] + i (i < count of e), zero in the padding; s_r = rowscale[r] (rounded once to the element
// type) or 1 without a scale.  64 x 64 tiles through LDS with 16-byte accesses on both sides (a source row
// segment in, a run of 16 / element-size consecutive destination columns out); blocks past poff[E_local] exit.
template <int DT>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint8_t* __restrict__ src, int C, int64_t Rpad,
                                                            const int32_t* __restrict__ offsets, int e_lo, int E_local,
                                                            const int32_t* __restrict__ poff,
                                                            const float* __restrict__ rowscale,
                                                            uint8_t* __restrict__ dst) {
  using T = typename std::conditional<DT == 0, uint32_t, uint16_t>::type;
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  constexpr int VPR = 64 / EPV;             // vectors per 64-element tile row
  constexpr int P = 64 + 4 / (int)sizeof(T); // row pitch (elements): one extra dword against bank conflicts
  __shared__ T tile[64 * P];
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (j0 >= poff[E_local]) return;
  int lo = 0, hi = E_local - 1;  // the expert whose padded range holds j0 (ranges are multiples of 64)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= j0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int64_t rbeg = offsets[e_lo + e], rend = offsets[e_lo + e + 1];
  const int64_t r0 = rbeg + (j0 - poff[e]);
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int i = v / VPR, q = v % VPR;  // tile row (source row r0 + i), vector q of its 64 columns
    const int64_t r = r0 + i;
    union {
      i32x4_t v4;
      T el[EPV];
    } u;
    u.v4 = (i32x4_t){0, 0, 0, 0};
    if (r < rend) {
      u.v4 = *reinterpret_cast<const i32x4_t*>(src + (r * C + c0 + q * EPV) * (int64_t)sizeof(T));
      if (rowscale != nullptr) {
        const float sr = rowscale[r];
#pragma unroll
        for (int x = 0; x < EPV; ++x) {
          const float f = DT == 0 ? __uint_as_float((uint32_t)u.el[x]) : __uint_as_float((uint32_t)u.el[x] << 16);
          u.el[x] = DT == 0 ? (T)__float_as_uint(sr * f) : (T)f32_to_bf16_bits(sr * f);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < EPV; ++x) tile[i * P + q * EPV + x] = u.el[x];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int c = v / VPR, q = v % VPR;  // destination row c0 + c, columns j0 + q * EPV ...
    union {
      i32x4_t v4;
      T el[EPV];
    } u;
#pragma unroll
    for (int x = 0; x < EPV; ++x) u.el[x] = tile[(q * EPV + x) * P + c];
    *reinterpret_cast<i32x4_t*>(dst + ((int64_t)(c0 + c) * Rpad + j0 + q * EPV) * (int64_t)sizeof(T)) = u.v4;
  }
}

// dx[t] = sum over the token's local kept picks (slot order) of dX[row], fp32 sums, one rounding
template <int DT>
__global__ __launch_bounds__(256) void unpermute_kernel(const float* __restrict__ dX, const int32_t* __restrict__ rop,
                                                        const int32_t* __restrict__ idx, int k, int H, int e_lo,
                                                        int E_local, uint8_t* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int ex = idx[t * k + j] - e_lo;
      const int r = rop[t * k + j];
      if (ex < 0 || ex >= E_local || r < 0) continue;
      s += *reinterpret_cast<const f32x4_t*>(dX + (int64_t)r * H + c);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) store_val<DT>(dx, t * H + c + q, s[q]);
  }
}

// Routing-weight gradients: dw[t][j] = <dout[t], y[row]> for local kept picks (0 otherwise), then, if requested,
// dlogits[t][idx_m] = w_m (dw_m - sum_i w_i dw_i) on the picks and 0 elsewhere.  One workgroup per token; each
// thread sums its columns in order, then a fixed LDS tree.
template <int DT>
__global__ __launch_bounds__(256) void dw_kernel(const uint8_t* __restrict__ dout, const float* __restrict__ y,
                                                 const int32_t* __restrict__ rop, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ wts, int k, int E, int H, int e_lo,
                                                 int E_local, float* __restrict__ dtw, float* __restrict__ dlogits) {
  __shared__ float red[256];
  __shared__ float s_dw[32];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  for (int j = 0; j < k; ++j) {
    const int ex = idx[t * k + j] - e_lo;
    const int r = rop[t * k + j];
    const bool on = ex >= 0 && ex < E_local && r >= 0;  // uniform over the workgroup
    float s = 0.0f;
    if (on)
      for (int c = tid; c < H; c += 256) s = __builtin_fmaf(load_val<DT>(dout, t * H + c), y[(int64_t)r * H + c], s);
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o >= 1; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) s_dw[j] = on ? red[0] : 0.0f;
    __syncthreads();
  }
  if (tid < k) dtw[t * k + tid] = s_dw[tid];
  if (dlogits != nullptr) {
    for (int e2 = tid; e2 < E; e2 += 256) dlogits[t * E + e2] = 0.0f;
    __syncthreads();
    if (tid == 0) {
      float sw = 0.0f;
      for (int j = 0; j < k; ++j) sw = __builtin_fmaf(wts[t * k + j], s_dw[j], sw);
      for (int j = 0; j < k; ++j) dlogits[t * E + idx[t * k + j]] = wts[t * k + j] * (s_dw[j] - sw);
    }
  }
}

template <int DT, int MODE, int BIG>
static void launch_gemm_cfg(GemmArgs a, int64_t R, hipStream_t s) {
  using C_ = Cfg<DT, BIG>;
  a.n_tiles = a.N / C_::BN;
  int64_t grid;
  if (MODE == MODE_WG) {
    a.m_tiles = a.M / C_::BM;
    grid = (int64_t)a.E_local * a.m_tiles * a.n_tiles;
  } else {
    a.m_tiles = (int)((R + C_::BM - 1) / C_::BM + a.E_local);  // worst case over the ragged experts
    grid = (int64_t)a.m_tiles * a.n_tiles;
  }
  hipLaunchKernelGGL((bwd_gemm_kernel<DT, MODE, BIG>), dim3((unsigned)grid), dim3(64 * C_::WM * C_::WN), 0, s, a);
}

// Tile choice: bf16 products whose output shape divides 256 take the 8-wavefront tiles (320 rows for the
// ragged row blocks when experts average >= 256 rows); everything else 128 x 128.
template <int DT, int MODE>
static void launch_gemm(const GemmArgs& a, int64_t R, hipStream_t s) {
  if constexpr (DT == 1) {
    if (MODE == MODE_WG && a.M % 256 == 0 && a.N % 256 == 0) return launch_gemm_cfg<DT, MODE, 1>(a, R, s);
    if (MODE != MODE_WG && a.N % 256 == 0 && R / a.E_local >= 256) return launch_gemm_cfg<DT, MODE, 2>(a, R, s);
  }
  launch_gemm_cfg<DT, MODE, 0>(a, R, s);
}

template <int DT>
static void launch_dt(const BwdLaunch& p, hipStream_t s) {
  constexpr int ESZ = Cfg<DT, 0>::ESZ;
  const int e_hi = p.e_lo + p.E_local;
  const int64_t R = p.R_max;
  const int64_t Rpad = (R + PADC - 1) / PADC * PADC + (int64_t)p.E_local * PADC;
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(64), 0, s, p.offsets, p.e_lo, p.E_local, p.poff);
  if (R > 0) {
    hipLaunchKernelGGL(pair_of_row_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s, p.token_of_row,
                       p.row_of_pair, p.k, p.offsets, p.e_lo, e_hi, p.por);
    hipLaunchKernelGGL(dout_gather_kernel, dim3((unsigned)R), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t*>(p.dout), (int64_t)p.H * ESZ, p.token_of_row, p.por, p.topk_w,
                       p.offsets, p.e_lo, e_hi, reinterpret_cast<uint8_t*>(p.dO), p.rw);
    // dh -> dg, du
    GemmArgs g{};
    g.A = reinterpret_cast<const uint8_t*>(p.dO);
    g.B0 = reinterpret_cast<const uint8_t*>(p.w_down);
    g.offsets = p.offsets;
    g.e_lo = p.e_lo;
    g.E_local = p.E_local;
    g.N = p.F;
    g.K = p.H;
    g.F = p.F;
    g.GU = p.gu;
    g.rw = p.rw;
    g.DGU = reinterpret_cast<uint8_t*>(p.dgu);
    launch_gemm<DT, MODE_DH>(g, R, s);
    // dX = [dg | du] [Wg | Wu]^T
    GemmArgs d{};
    d.A = reinterpret_cast<const uint8_t*>(p.dgu);
    d.B0 = reinterpret_cast<const uint8_t*>(p.w_gate);
    d.B1 = reinterpret_cast<const uint8_t*>(p.w_up);
    d.offsets = p.offsets;
    d.e_lo = p.e_lo;
    d.E_local = p.E_local;
    d.N = p.H;
    d.K = 2 * p.F;
    d.F = p.F;
    d.C = p.dX;
    launch_gemm<DT, MODE_DX>(d, R, s);
  }
  if (p.T > 0) {
    hipLaunchKernelGGL((unpermute_kernel<DT>), dim3((unsigned)p.T), dim3(256), 0, s, p.dX, p.row_of_pair, p.topk_idx,
                       p.k, p.H, p.e_lo, p.E_local, reinterpret_cast<uint8_t*>(p.dx));
    hipLaunchKernelGGL((dw_kernel<DT>), dim3((unsigned)p.T), dim3(256), 0, s, reinterpret_cast<const uint8_t*>(p.dout),
                       p.y_perm, p.row_of_pair, p.topk_idx, p.topk_w, p.k, p.E, p.H, p.e_lo, p.E_local, p.d_topk_w,
                       p.d_logits);
  }
  // transposed operands of the weight products, then the products themselves
  const unsigned jt = (unsigned)(Rpad / 64);
  auto tp = [&](const void* src, int C, const float* scale, void* dst) {
    hipLaunchKernelGGL((transpose_pad_kernel<DT>), dim3(jt, (unsigned)(C / 64)), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t*>(src), C, Rpad, p.offsets, p.e_lo, p.E_local, p.poff, scale,
                       reinterpret_cast<uint8_t*>(dst));
  };
  if (R > 0) {
    tp(p.h, p.F, p.rw, p.whT);
    tp(p.dO, p.H, nullptr, p.dOT);
    tp(p.x_perm, p.H, nullptr, p.xT);
    tp(p.dgu, 2 * p.F, nullptr, p.dguT);
  }
  auto wg = [&](const void* AT, const void* BT, int M, int N, float* out) {
    GemmArgs w{};
    w.A = reinterpret_cast<const uint8_t*>(AT);
    w.B0 = reinterpret_cast<const uint8_t*>(BT);
    w.poff = p.poff;
    w.E_local = p.E_local;
    w.M = M;
    w.N = N;
    w.K = (int)Rpad;
    w.C = out;
    launch_gemm<DT, MODE_WG>(w, R, s);
  };
  const uint8_t* dgT = reinterpret_cast<const uint8_t*>(p.dguT);
  const uint8_t* duT = dgT + (int64_t)p.F * Rpad * ESZ;
  wg(p.whT, p.dOT, p.F, p.H, p.dw_down);  // dWd_e [F][H] = (w h)^T dO
  wg(p.xT, dgT, p.H, p.F, p.dw_gate);    // dWg_e [H][F] = X^T dg
  wg(p.xT, duT, p.H, p.F, p.dw_up);      // dWu_e [H][F] = X^T du
}

}  // namespace bwd

void launch_ffn_backward(const BwdLaunch& p, hipStream_t s) {
  if (p.dtype == MOE_DTYPE_BF16)
    bwd::launch_dt<1>(p, s);
  else
    bwd::launch_dt<0>(p, s);
}

}  // namespace moe
