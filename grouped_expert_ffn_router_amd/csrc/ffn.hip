// Grouped SwiGLU expert FFN on MFMA: one launch per expert matrix product over the ragged per-expert slabs.
//
// Method: page "Expert parallelism and all-to-all", section "Walking through one MoE layer", step 3: each
// GPU runs its local experts on the tokens it received as one grouped matrix multiply.  The expert is a
// SwiGLU block: h = silu(x Wg) * (x Wu), y = h Wd.
//
//   GEMM1  [rows of expert e] x [Wg_e | Wu_e]  -> h = silu(G) * U, stored in the layer dtype
//   GEMM2  h x Wd_e                            -> y_perm, fp32
//
// Design (gfx950):
//  * Tiles of BM rows x BN weight rows.  Both operands are stored with the reduction dimension contiguous
//    (x_perm / h rows, and the packed weights), so one 128-byte slice of the reduction dimension per row is a
//    pipeline stage: 64 bf16, 128 fp8 or 32 fp32 values.
//  * global -> LDS with direct 16-byte loads (global_load_lds_dwordx4): each wavefront instruction fills 1 KiB
//    = 8 rows x 128 B.  The 16-byte chunk c of row r lives at chunk position c ^ (r & 7) so that the MFMA
//    fragment reads (32 rows, same chunk) hit distinct banks.  Two stages, double-buffered.
//  * v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x64_f8f6f4 (OCP e4m3, unit scales), v_mfma_f32_32x32x2f32.
//    The contraction pairs A's and B's register slots one-to-one, so any assignment of reduction indices to
//    (lane half, slot) works as long as both operands use it; lane half h of a 32x32 block reads chunks of
//    its own row (bf16: chunk 2s+h at step s; fp8: chunks 4s+2h and 4s+2h+1; fp32: element s%4 of chunk
//    2(s/4)+h).
//  * fp8: activation scales (per row per 128 columns) and weight scales (per 128 x 128 block) both change
//    along the reduction dimension, so each 128-wide stage is accumulated separately by the MFMA and then
//    added into the fp32 accumulators with the product of the two scales.
//  * Ragged M without a host sync: every workgroup finds its (expert, row range) from the device-resident
//    offsets with one wavefront scan over the experts' tile counts; the grid is sized for the worst case
//    (ceil(R/BM) + E_local M-tiles) and surplus workgroups exit at once.  Empty experts cost nothing.
//  * Workgroup ids are remapped so consecutive tiles (which share a row block or a weight block) land on the
//    same XCD and its L2.
//  * GEMM1 epilogue: silu(G) * U in fp32 is staged through LDS, then each row's 128 columns are written with
//    16-byte stores; for fp8 the 16 lanes holding a row reduce its amax and quantise with scale = amax / 448.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm {

template <int DT>
struct Tr;
template <>
struct Tr<0> {
  static constexpr int ESZ = 4;
};
template <>
struct Tr<1> {
  static constexpr int ESZ = 2;
};
template <>
struct Tr<2> {
  static constexpr int ESZ = 1;
};

struct Args {
  const uint8_t* A;         // [R_max][K] x_perm (GEMM1) or h (GEMM2)
  const float* A_scales;    // fp8: [R_max][K/128]
  const uint8_t* B0;        // packed weights [E_local][N_rows][K]: gate (GEMM1) or down (GEMM2)
  const uint8_t* B1;        // packed up weights (GEMM1)
  const float* B0_scales;   // fp8: [E_local][K/128][N_rows/128]
  const float* B1_scales;
  const int32_t* offsets;   // global expert offsets
  int e_lo, E_local;
  int K;                    // reduction length (elements)
  int N_rows;               // weight rows per expert (= output columns)
  int n_tiles;              // output-column tiles
  uint8_t* H_out;           // GEMM1: h [R_max][N_rows] in the layer dtype
  float* H_scales;          // GEMM1 fp8: [R_max][N_rows/128]
  float* Y;                 // GEMM2: [R_max][N_rows] fp32
};

MOE_DEV i32x4_t lds_chunk(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const i32x4_t*>(base + row * 128 + ((chunk ^ (row & 7)) << 4));
}

MOE_DEV int wave_incl_scan_i(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

template <int DT, int BM, int BN, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const Args a) {
  constexpr int ESZ = Tr<DT>::ESZ;
  static_assert(WM * WN == 4, "four wavefronts");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  static_assert(MB >= 1 && NB >= 1 && (!SWIGLU || NB % 2 == 0), "tile shape");
  constexpr int BNF = SWIGLU ? BN / 2 : BN;  // output columns per tile
  static_assert(!SWIGLU || BNF == 128, "the SwiGLU epilogue writes 128-column groups");
  constexpr int SA = DT == 2 ? (BM < 64 ? 64 : BM) * 4 : 0;  // whole wavefronts load scales
  constexpr int STAGE = (BM + BN) * 128 + SA;
  constexpr int LOOP_LDS = 2 * STAGE;
  constexpr int SP = BNF + 4;  // epilogue row pitch (floats)
  constexpr int EPI_LDS = SWIGLU ? BM * SP * 4 : 0;
  constexpr int LDS = LOOP_LDS > EPI_LDS ? LOOP_LDS : EPI_LDS;
  constexpr int A_INS = BM / 32;  // direct-load instructions per wavefront per stage
  constexpr int B_INS = BN / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  __shared__ int s_tile[3];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int lr = lane & 31, lh = lane >> 5;

  // consecutive logical tiles on one XCD (workgroups are dealt to the 8 XCDs round-robin)
  const int G = gridDim.x, per = G >> 3, bid = blockIdx.x;
  const int L = (bid < per * 8) ? (bid & 7) * per + (bid >> 3) : bid;
  const int qm = L / a.n_tiles, qn = L - qm * a.n_tiles;

  if (wid == 0) {
    int cum = 0, fe = -1, fm0 = 0, fend = 0;
    for (int base = 0; base < a.E_local; base += 64) {
      const int i = base + lane;
      int beg = 0, end = 0;
      if (i < a.E_local) {
        beg = a.offsets[a.e_lo + i];
        end = a.offsets[a.e_lo + i + 1];
      }
      const int tiles = (end - beg + BM - 1) / BM;
      const int incl = wave_incl_scan_i(tiles);
      const int excl = incl - tiles;
      const int rel = qm - cum;
      const uint64_t hm = __ballot(rel >= excl && rel < incl);
      if (hm) {
        const int src = __ffsll((unsigned long long)hm) - 1;
        fe = __shfl(i, src, 64);
        fm0 = __shfl(beg + (rel - excl) * BM, src, 64);
        fend = __shfl(end, src, 64);
        break;
      }
      cum += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      s_tile[0] = fe;
      s_tile[1] = fm0;
      s_tile[2] = fend;
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;
  const int m0 = s_tile[1], m_end = s_tile[2];
  const int n0 = qn * BNF;

  const int64_t Kb = (int64_t)a.K * ESZ;  // bytes per row
  const int nk = (int)(Kb >> 7);          // 128-byte stages
  const int nkb = a.K >> 7;               // fp8 scale blocks along K (== nk for fp8)

  // per-lane source rows of the direct loads
  const uint8_t* a_src[A_INS];
  const uint8_t* b_src[B_INS];
#pragma unroll
  for (int q = 0; q < A_INS; ++q) {
    const int r = (wid * A_INS + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int gr = min(m0 + r, m_end - 1);
    a_src[q] = a.A + (int64_t)gr * Kb + c * 16;
  }
  const uint8_t* Bb0 = a.B0 + (int64_t)e * a.N_rows * Kb;
  const uint8_t* Bb1 = SWIGLU ? a.B1 + (int64_t)e * a.N_rows * Kb : nullptr;
#pragma unroll
  for (int q = 0; q < B_INS; ++q) {
    const int r = (wid * B_INS + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const uint8_t* rowp;
    if (SWIGLU)
      rowp = r < BNF ? Bb0 + (int64_t)(n0 + r) * Kb : Bb1 + (int64_t)(n0 + r - BNF) * Kb;
    else
      rowp = Bb0 + (int64_t)(n0 + r) * Kb;
    b_src[q] = rowp + c * 16;
  }
  const float* sa_src = nullptr;
  if (DT == 2 && wid * 64 < BM) {
    const int gr = min(m0 + wid * 64 + lane, m_end - 1);
    sa_src = a.A_scales + (int64_t)gr * nkb;
  }

  auto issue_stage = [&](int kt, int buf) {
    uint8_t* st = smem + buf * STAGE;
#pragma unroll
    for (int q = 0; q < A_INS; ++q)
      load_lds16(a_src[q] + kt * 128, st + (wid * A_INS + q) * 1024);
#pragma unroll
    for (int q = 0; q < B_INS; ++q)
      load_lds16(b_src[q] + kt * 128, st + BM * 128 + (wid * B_INS + q) * 1024);
    if (DT == 2 && wid * 64 < BM)
      load_lds4(sa_src + kt, st + (BM + BN) * 128 + wid * 256);
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
  for (int j = 0; j < NB; ++j) {
    if (SWIGLU)
      brow[j] = (j < NB / 2 ? wn * (BNF / WN) + j * 32 : BNF + wn * (BNF / WN) + (j - NB / 2) * 32) + lr;
    else
      brow[j] = wn * WTN + j * 32 + lr;
  }

  issue_stage(0, 0);
  wait_vmcnt0();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue_stage(kt + 1, buf ^ 1);
    const uint8_t* As = smem + buf * STAGE;
    const uint8_t* Bs = As + BM * 128;
    if constexpr (DT == 1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) af[i] = __builtin_bit_cast(bf16x8_t, lds_chunk(As, arow[i], 2 * s + lh));
#pragma unroll
        for (int j = 0; j < NB; ++j) bfr[j] = __builtin_bit_cast(bf16x8_t, lds_chunk(Bs, brow[j], 2 * s + lh));
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_32x32x16_bf16(af[i], bfr[j], acc[i][j]);
      }
    } else if constexpr (DT == 0) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        f32x4_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) af[i] = __builtin_bit_cast(f32x4_t, lds_chunk(As, arow[i], 2 * s4 + lh));
#pragma unroll
        for (int j = 0; j < NB; ++j) bfr[j] = __builtin_bit_cast(f32x4_t, lds_chunk(Bs, brow[j], 2 * s4 + lh));
#pragma unroll
        for (int ss = 0; ss < 4; ++ss)
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = mfma_32x32x2_f32(af[i][ss], bfr[j][ss], acc[i][j]);
      }
    } else {
      // fp8: one 128-wide scale block per stage
      const float* sa = reinterpret_cast<const float*>(As + (BM + BN) * 128);
      i32x8_t af[MB][2];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x4_t lo = lds_chunk(As, arow[i], 4 * s + 2 * lh);
          const i32x4_t hi = lds_chunk(As, arow[i], 4 * s + 2 * lh + 1);
          af[i][s] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      f32x4_t sav[MB][4];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sav[i][q] = *reinterpret_cast<const f32x4_t*>(sa + wm * WTM + i * 32 + q * 8 + 4 * lh);
      const int nnb = a.N_rows >> 7;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        i32x8_t bfr[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x4_t lo = lds_chunk(Bs, brow[j], 4 * s + 2 * lh);
          const i32x4_t hi = lds_chunk(Bs, brow[j], 4 * s + 2 * lh + 1);
          bfr[s] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const bool up = SWIGLU && j >= NB / 2;
        const int col = SWIGLU ? n0 : n0 + wn * WTN + j * 32;
        const float* sbase = up ? a.B1_scales : a.B0_scales;
        const float sw = sbase[((int64_t)e * nkb + kt) * nnb + (col >> 7)];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          f32x16_t p;
#pragma unroll
          for (int v = 0; v < 16; ++v) p[v] = 0.0f;
          p = mfma_32x32x64_e4m3(af[i][0], bfr[0], p);
          p = mfma_32x32x64_e4m3(af[i][1], bfr[1], p);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(p[v], sav[i][v >> 2][v & 3] * sw, acc[i][j][v]);
        }
      }
    }
    wait_vmcnt0();
    __syncthreads();
  }

  if constexpr (SWIGLU) {
    // silu(G) * U -> LDS (fp32), then per-row stores in the layer dtype
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WTM + i * 32 + (v >> 2) * 8 + 4 * lh + (v & 3);
          const int col = wn * (BNF / WN) + j * 32 + lr;
          const float g = acc[i][j][v], u = acc[i][j + NB / 2][v];
          st[row * SP + col] = g / (1.0f + __expf(-g)) * u;
        }
    __syncthreads();
    const int F = a.N_rows;
    const int c8 = tid & 15;
    for (int r = tid >> 4; r < BM; r += 16) {
      const int gm = m0 + r;
      if (gm >= m_end) continue;  // uniform across the 16 lanes of a row
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(st + r * SP + c8 * 8);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(st + r * SP + c8 * 8 + 4);
      const int64_t off = (int64_t)gm * F + n0 + c8 * 8;
      if constexpr (DT == 1) {
        i32x4_t o;
        o[0] = (int)f32_to_bf16_bits(v0[0]) | ((int)f32_to_bf16_bits(v0[1]) << 16);
        o[1] = (int)f32_to_bf16_bits(v0[2]) | ((int)f32_to_bf16_bits(v0[3]) << 16);
        o[2] = (int)f32_to_bf16_bits(v1[0]) | ((int)f32_to_bf16_bits(v1[1]) << 16);
        o[3] = (int)f32_to_bf16_bits(v1[2]) | ((int)f32_to_bf16_bits(v1[3]) << 16);
        *reinterpret_cast<i32x4_t*>(a.H_out + off * 2) = o;
      } else if constexpr (DT == 0) {
        f32x4_t* d = reinterpret_cast<f32x4_t*>(a.H_out + off * 4);
        d[0] = v0;
        d[1] = v1;
      } else {
        float m = fmaxf(fmaxf(fmaxf(fabsf(v0[0]), fabsf(v0[1])), fmaxf(fabsf(v0[2]), fabsf(v0[3]))),
                        fmaxf(fmaxf(fabsf(v1[0]), fabsf(v1[1])), fmaxf(fabsf(v1[2]), fabsf(v1[3]))));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const float scale = m > 0.0f ? m / 448.0f : 1.0f;
        const uint32_t lo = f32x2_to_e4m3x2(v0[0] / scale, v0[1] / scale) |
                            (f32x2_to_e4m3x2(v0[2] / scale, v0[3] / scale) << 16);
        const uint32_t hi = f32x2_to_e4m3x2(v1[0] / scale, v1[1] / scale) |
                            (f32x2_to_e4m3x2(v1[2] / scale, v1[3] / scale) << 16);
        *reinterpret_cast<uint2*>(a.H_out + off) = make_uint2(lo, hi);
        if (c8 == 0) a.H_scales[(int64_t)gm * (F >> 7) + (n0 >> 7)] = scale;
      }
    }
  } else {
    const int N = a.N_rows;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * WTM + i * 32 + (v >> 2) * 8 + 4 * lh + (v & 3);
        if (gm < m_end) {
#pragma unroll
          for (int j = 0; j < NB; ++j) a.Y[(int64_t)gm * N + n0 + wn * WTN + j * 32 + lr] = acc[i][j][v];
        }
      }
  }
}

template <int DT, int BM, int BN, int WM, int WN, bool SWIGLU>
static void launch_one(const Args& a, int64_t R_max, hipStream_t s) {
  const int64_t mt = (R_max + BM - 1) / BM + a.E_local;
  const int64_t grid = mt * a.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_kernel<DT, BM, BN, WM, WN, SWIGLU>), dim3((unsigned)grid), dim3(256), 0, s, a);
}

// Row-block size from the mean rows per expert (the counts themselves stay on the device).
static int pick_bm(int64_t R_max, int E_local, int dt) {
  const int64_t avg = R_max / (E_local > 0 ? E_local : 1);
  if (dt == 1 && avg >= 256) return 256;
  if (avg >= 96) return 128;
  if (avg >= 48) return 64;
  return 32;
}

template <int DT, bool SWIGLU, int BN>
static void launch_bm(int bm, const Args& a, int64_t R_max, hipStream_t s) {
  switch (bm) {
    case 256:
      if constexpr (DT == 1) launch_one<DT, 256, BN, 2, 2, SWIGLU>(a, R_max, s);
      break;
    case 128:
      launch_one<DT, 128, BN, 2, 2, SWIGLU>(a, R_max, s);
      break;
    case 64:
      launch_one<DT, 64, BN, 2, 2, SWIGLU>(a, R_max, s);
      break;
    default:
      launch_one<DT, 32, BN, 1, 4, SWIGLU>(a, R_max, s);
      break;
  }
}

template <int DT>
static void launch_gemm1_dt(const FfnLaunch& p, hipStream_t s) {
  Args a{};  // rows x [Wg | Wu] -> h
  a.A = reinterpret_cast<const uint8_t*>(p.x_perm);
  a.A_scales = p.x_perm_scales;
  a.B0 = reinterpret_cast<const uint8_t*>(p.w_gate);
  a.B1 = reinterpret_cast<const uint8_t*>(p.w_up);
  a.B0_scales = p.s_gate;
  a.B1_scales = p.s_up;
  a.offsets = p.offsets;
  a.e_lo = p.e_lo;
  a.E_local = p.E_local;
  a.K = p.H;
  a.N_rows = p.F;
  a.n_tiles = p.F / 128;
  a.H_out = reinterpret_cast<uint8_t*>(p.h);
  a.H_scales = p.h_scales;
  launch_bm<DT, true, 256>(pick_bm(p.R_max, p.E_local, DT), a, p.R_max, s);
}

template <int DT>
static void launch_gemm2_dt(const FfnLaunch& p, hipStream_t s) {
  Args b{};  // h x Wd -> y_perm
  b.A = reinterpret_cast<const uint8_t*>(p.h);
  b.A_scales = p.h_scales;
  b.B0 = reinterpret_cast<const uint8_t*>(p.w_down);
  b.B0_scales = p.s_down;
  b.offsets = p.offsets;
  b.e_lo = p.e_lo;
  b.E_local = p.E_local;
  b.K = p.F;
  b.N_rows = p.H;
  b.Y = p.y_perm;
  const int bm = pick_bm(p.R_max, p.E_local, DT);
  if (p.H % 256 == 0) {
    b.n_tiles = p.H / 256;
    launch_bm<DT, false, 256>(bm, b, p.R_max, s);
  } else {
    b.n_tiles = p.H / 128;
    launch_bm<DT, false, 128>(bm, b, p.R_max, s);
  }
}

}  // namespace gemm

void launch_ffn_gemm1(const FfnLaunch& p, hipStream_t s) {
  if (p.dtype == MOE_DTYPE_BF16)
    gemm::launch_gemm1_dt<1>(p, s);
  else if (p.dtype == MOE_DTYPE_FP8_E4M3)
    gemm::launch_gemm1_dt<2>(p, s);
  else
    gemm::launch_gemm1_dt<0>(p, s);
}

void launch_ffn_gemm2(const FfnLaunch& p, hipStream_t s) {
  if (p.dtype == MOE_DTYPE_BF16)
    gemm::launch_gemm2_dt<1>(p, s);
  else if (p.dtype == MOE_DTYPE_FP8_E4M3)
    gemm::launch_gemm2_dt<2>(p, s);
  else
    gemm::launch_gemm2_dt<0>(p, s);
}

// ---------------------------------------------------------------------------------------------------------
// Weight packing: per-expert transpose [K][N] -> [N][K] through a 64 x 64 LDS tile.
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int K, int N) {
  __shared__ T tile[64][65];
  const int64_t ex = blockIdx.z;
  src += ex * (int64_t)K * N;
  dst += ex * (int64_t)K * N;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) tile[i][tx] = src[(int64_t)(k0 + i) * N + n0 + tx];
  __syncthreads();
  for (int i = ty; i < 64; i += 4) dst[(int64_t)(n0 + i) * K + k0 + tx] = tile[tx][i];
}

void launch_transpose(const void* src, void* dst, int esize, int E, int K, int N, hipStream_t s) {
  const dim3 grid(N / 64, K / 64, E);
  if (esize == 4)
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)src, (uint32_t*)dst, K, N);
  else if (esize == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst, K, N);
  else
    hipLaunchKernelGGL(transpose_kernel<uint8_t>, grid, dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, K, N);
}

}  // namespace moe
