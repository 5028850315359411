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
//  * Tiles of BM rows x BN weight rows.  BM from the mean rows per expert: 320 (bf16) or 256 (fp8) rows over 8
//    wavefronts for large slabs, then 128, 64, 32 rows over 4.  GEMM1's BN = 256 weight rows are 128 gate rows
//    and the matching 128 up rows, so each SwiGLU pair meets inside one tile.
//  * Both operands are stored with the reduction dimension contiguous (x_perm / h rows, and the packed weights),
//    so a pipeline stage is one slice of the reduction dimension per row: 128 bytes (64 bf16, 128 fp8, 32 fp32
//    values; whole cache lines) or 64 bytes for the smaller bf16 tiles.  Two stages for the large tiles, three
//    or four for the small ones.
//  * global -> LDS with direct 16-byte loads (global_load_lds_dwordx4, one wavefront instruction fills 1 KiB)
//    and counted vmcnt waits.  The 16-byte chunk c of row r lives at c ^ ((r >> 1) & 7) (128-byte rows) or
//    c ^ ((r >> 2) & 3) (64-byte rows), so the fragment reads (32 rows, one chunk) hit distinct banks.
//  * v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x2f32, and for fp8 v_mfma_scale_f32_16x16x128_f8f6f4 (OCP e4m3,
//    unit scales).  The contraction pairs A's and B's register slots one-to-one, so any assignment of reduction
//    indices to (lane, slot) works as long as both operands use it: lane half h of a 32x32 block reads chunk
//    2s+h of its own row at bf16 step s (fp32: element s%4 of chunk 2(s/4)+h); for fp8, lane group g = lane/16
//    of a 16x16 block reads chunks 2g and 2g+1.
//  * fp8: activation scales (per row per 128 columns) and weight scales (per 128 x 128 block) both change
//    along the reduction dimension, so each 128-wide stage is accumulated separately by the MFMA and then
//    added into the fp32 accumulators times the product of the two scales.  The products are formed once per
//    row and stage (one lane per row, into a per-wavefront LDS table) rather than once per lane and row
//    (vector instructions per stage 174 -> 144 on the gate/up product; measured +0.7% on the fp8 layer).
//  * Ragged M without a host sync: every workgroup finds its (expert, row range) from the device-resident
//    offsets with one wavefront scan over the experts' tile counts; the grid is sized for the worst case
//    (ceil(R/BM) + E_local M-tiles) and surplus workgroups exit at once.  Empty experts cost nothing.
//  * Tile order: expert by expert.  GEMM1 inside an expert: row tiles fastest (the row blocks sharing a weight
//    tile are consecutive), or weight tiles fastest when the expert has more rows than the product has weight
//    rows (its row blocks, the larger operand, then stream once while the weight tiles are re-read).  GEMM2:
//    weight (output column) tiles fastest, so the tiles in flight write whole fp32 output rows together and
//    share one row block (measured on the DeepSeek-V3 shape: 1350 -> 1250 us; neutral on the others).  Workgroup
//    ids are remapped so each XCD (and its L2) takes one contiguous range of tiles.
//  * GEMM2 splits its reduction dimension in two when its output tiles fill at most half of the CUs; the
//    second part's fp32 partial sums are added by a small kernel in a fixed order.
//  * GEMM1 epilogue: silu(G) * U in fp32 is staged through LDS, then each row's 128 columns are written with
//    16-byte stores; for fp8 the 16 lanes holding a row reduce its amax and quantise with scale = amax / 448.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace moe {
namespace gemm {

using tile::swz;

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
  float* Ypart;             // GEMM2 split over K: partial sums of parts 1.. [ksplit-1][R_max][N_rows]
  int ksplit;               // GEMM2: number of parts the reduction dimension is split into (1: none)
  int64_t R_max;
  // GEMM1 gather form: A row r is row rows[r] of the unpermuted activations (rows = token_of_row), so the
  // permuted copy is never written; null: A is already permuted.
  const int32_t* rows;
  // GEMM2 scatter form (Yslot != null): output row r times its routing weight goes to the pair slot p with
  // row_of_pair[p] == r, in a pair-major [T*k][N_rows] buffer; parts 1.. of a split reduction still write
  // permuted partials, which a reduction adds into the slots.
  float* Yslot;
  const int32_t* tok;       // token_of_row
  const int32_t* rop;       // row_of_pair
  const float* wts;         // routing weights [T*k]
  int k;
  // GEMM1 training form (fp32, bf16 layers): the pre-activations g and u too, [R_max][2 N_rows] fp32
  float* GU_out;
};

// LDS pipeline stages: the layout of gemm_tile.h (RB bytes of each tile row per stage, 16-byte chunk c of row r
// at chunk position c ^ tile::swz(r) against bank conflicts).
template <int DT, int BM, int BN, int RB, int NW>
struct Geo {
  static constexpr int RPI = 1024 / RB;               // rows one wavefront direct-load instruction fills
  static constexpr int A_INS = BM / (NW * RPI);       // direct-load instructions per wavefront per stage
  static constexpr int B_INS = BN / (NW * RPI);
  static constexpr int SA = DT == 2 ? NW * 256 : 0;    // fp8: every wavefront loads 64 row scales
  static constexpr int STAGE = (BM + BN) * RB + SA;
  static constexpr int NL = A_INS + B_INS + (DT == 2 ? 1 : 0);  // loads per wavefront per stage
  static_assert(A_INS >= 1 && B_INS >= 1, "every wavefront loads part of each operand");
};

template <int A_INS, int B_INS>
struct StageCtx {
  const uint8_t* a_base;          // uniform: first row of the tile's row block (slice 0)
  const uint8_t* b_base[B_INS];   // uniform: first weight row of each load's operand (gate or up), slice 0
  const uint8_t* sa_base;         // fp8: uniform row-scale base of the tile's row block
  uint32_t a_off[A_INS];          // this lane's byte offset of its 16-byte chunk of each direct load
  uint32_t b_off[B_INS];
  uint32_t sa_off;                // fp8: this lane's row-scale row
  const float* wsc;             // fp8: LDS copy of the tile's weight scales, [group][stage - k0]
  int k0, nk;                   // first stage and stage count of this tile's reduction range
  int wid, lane, lh, e, n0, wn, wm, nkb, nnb;
  // per-lane LDS offsets of the fragment reads (tile::frag_offsets of the first A and B row): bf16 / fp32
  // chunks lh + 2 s; fp8 chunks 2 lg and 2 lg + 1 of the row lane % 16
  tile::FragOff ao, bo;
  float* scp;                   // fp8: per-wavefront LDS table of scale products, [wavefront][group][64 rows]
};

// Direct global -> LDS loads of reduction slice kt into one stage buffer.
template <int DT, int BM, int BN, int RB, int A_INS, int B_INS>
MOE_DEV void load_stage(uint8_t* __restrict__ dst, int kt, const StageCtx<A_INS, B_INS>& cx) {
#pragma unroll
  for (int q = 0; q < A_INS; ++q) load_lds16(cx.a_base + kt * RB, cx.a_off[q], dst + (cx.wid * A_INS + q) * 1024);
#pragma unroll
  for (int q = 0; q < B_INS; ++q)
    load_lds16(cx.b_base[q] + kt * RB, cx.b_off[q], dst + BM * RB + (cx.wid * B_INS + q) * 1024);
  if (DT == 2) load_lds4(cx.sa_base + kt * 4, cx.sa_off, dst + (BM + BN) * RB + cx.wid * 256);
}

// One pipeline stage: start loading slice kn into `nxt`, multiply-accumulate the slice held in `cur`.
// FULL: all MB row blocks of this wavefront hold valid rows; otherwise only the first `act` do (the last tile of
// an expert slab), and the others skip their LDS reads and MFMAs.
template <int DT, int BM, int BN, int WM, int WN, bool SWIGLU, int RB, int A_INS, int B_INS, int MB, int NB, bool FULL>
MOE_DEV void gemm_stage(const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt, int kn, int kt,
                        const StageCtx<A_INS, B_INS>& cx, const int (&arow)[MB], const int (&brow)[NB],
                        f32x16_t (&acc)[MB][NB], int act) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  load_stage<DT, BM, BN, RB, A_INS, B_INS>(nxt, kn, cx);
  const uint8_t* As = cur;
  const uint8_t* Bs = cur + BM * RB;
  const int lh = cx.lh;
  if constexpr (DT == 1 && !FULL) {
    tile::mma_stage_bf16_partial<RB, MB, NB>(As, Bs, arow, brow, cx.ao, cx.bo, acc, act);
  } else if constexpr (DT == 1) {
    tile::mma_stage_bf16<RB, MB, NB>(As, Bs, arow, brow, cx.ao, cx.bo, acc);
  } else if constexpr (DT == 0) {
    static_assert(RB == 128, "fp32 stages hold 32 values per row");
    tile::mma_stage_f32<MB, NB>(As, Bs, arow, brow, cx.ao, cx.bo, acc, FULL ? MB : act);
  } else {
    // fp8: a stage is one 128-wide scale block, so one v_mfma_scale 16x16x128 per 16 x 16 sub-block gives that
    // block's partial sum directly; it is scaled (row scale x weight scale) into the fp32 accumulators.  Each
    // 32 x 32 accumulator block holds four 16 x 16 sub-blocks: element 4q + u is sub-block q = 2 si + sj,
    // row 16 si + 4 (lane / 16) + u, column 16 sj + lane % 16.
    static_assert(RB == 128, "fp8 stages hold one 128-wide scale block");
    const float* sa = reinterpret_cast<const float*>(As + (BM + BN) * RB);
    const int lg = cx.lane >> 4;      // reduction-byte group of this lane (32 bytes each)
    // fragment rows: arow[i] - lane % 32 + lane % 16 + 16 si (cx.ao / cx.bo: chunks 2 lg and 2 lg + 1 of the
    // first of them)
    tile::lds_u8_t* alo = tile::to_lds(As) + cx.ao.o[0];
    tile::lds_u8_t* ahi = tile::to_lds(As) + cx.ao.o[1];
    tile::lds_u8_t* blo = tile::to_lds(Bs) + cx.bo.o[0];
    tile::lds_u8_t* bhi = tile::to_lds(Bs) + cx.bo.o[1];
    i32x8_t af[MB][2];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int si = 0; si < 2; ++si) {
        const int d = (arow[i] - arow[0] + 16 * si) * RB;
        const i32x4_t lo = tile::lds_at(alo, d);
        const i32x4_t hi = tile::lds_at(ahi, d);
        af[i][si] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    // The weight scale is constant over a 128-column group.  A wavefront's N blocks fall in at most two groups:
    // gate and up (SwiGLU), or one group of the output columns (WTN <= 128, aligned).
    static_assert(SWIGLU || (WTN <= 128 && 128 % WTN == 0), "a wavefront's output columns share one scale group");
    constexpr int NG = SWIGLU ? 2 : 1;
    constexpr int JPG = NB / NG;  // N blocks per scale group
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // lane r (< WTM) forms the products of row r of this wavefront's rows with the groups' weight scales, once, in
    // the wavefront's own LDS table; every lane then reads the four products of its rows per sub-block
    float* tbl = cx.scp + cx.wid * (NG * 64);
    {
      const float sa_l = cx.lane < WTM ? sa[cx.wm * WTM + cx.lane] : 0.0f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int grp = SWIGLU ? g : (cx.wn * WTN) >> 7;
        tbl[g * 64 + cx.lane] = sa_l * cx.wsc[grp * cx.nk + (kt - cx.k0)];
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float* srow = tbl + g * 64 + 4 * lg;
      f32x4_t sc[MB][2];  // row scale x weight scale for this lane's rows of each 16-row sub-block
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int si = 0; si < 2; ++si) sc[i][si] = *reinterpret_cast<const f32x4_t*>(srow + i * 32 + 16 * si);
#pragma unroll
      for (int jj = 0; jj < JPG; ++jj) {
        const int j = g * JPG + jj;
        i32x8_t bfr[2];
#pragma unroll
        for (int sj = 0; sj < 2; ++sj) {
          const int d = (brow[j] - brow[0] + 16 * sj) * RB;
          const i32x4_t lo = tile::lds_at(blo, d);
          const i32x4_t hi = tile::lds_at(bhi, d);
          bfr[sj] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          if (!FULL && i >= act) continue;
          f32x4_t p[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) p[q] = mfma_16x16x128_e4m3(af[i][q >> 1], bfr[q & 1], zero);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u)
              acc[i][j][4 * q + u] = __builtin_fmaf(p[q][u], sc[i][q >> 1][u], acc[i][j][4 * q + u]);
        }
      }
    }
  }
}

// Position of accumulator element v of a lane inside its 32 x 32 block: the 32x32 MFMA layout (bf16, fp32) or
// four 16 x 16 sub-blocks (fp8).
template <int DT>
MOE_DEV int acc_row(int v, int lane) {
  if constexpr (DT == 2) return 16 * (v >> 3) + 4 * ((lane >> 4) & 3) + (v & 3);
  return (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
}
template <int DT>
MOE_DEV int acc_col(int v, int lane) {
  if constexpr (DT == 2) return 16 * ((v >> 2) & 1) + (lane & 15);
  return lane & 31;
}

// BM x BN tile (BN weight rows; for SwiGLU the first BN/2 are gate rows, the rest the matching up rows),
// 4 wavefronts in a WM x WN grid, NS pipeline stages of RB bytes per row.
template <int DT, int BM, int BN, int WM, int WN, bool SWIGLU, int RB, int NS>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm_kernel(const Args a) {
  constexpr int ESZ = Tr<DT>::ESZ;
  constexpr int NW = WM * WN;  // wavefronts per workgroup
  static_assert(NW == 4 || NW == 8, "four or eight wavefronts");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  static_assert(MB >= 1 && NB >= 1 && (!SWIGLU || NB % 2 == 0), "tile shape");
  constexpr int BNF = SWIGLU ? BN / 2 : BN;  // output columns per tile
  static_assert(!SWIGLU || BNF == 128, "the SwiGLU epilogue writes 128-column groups");
  using GG = Geo<DT, BM, BN, RB, NW>;
  constexpr int STAGE = GG::STAGE;
  constexpr int LOOP_LDS = NS * STAGE;
  constexpr int SP = BNF + 4;  // epilogue row pitch (floats)
  // The SwiGLU epilogue stages silu(G)*U in LDS; a tile too tall for that (320 rows) is staged one wavefront row
  // (WTM rows) at a time.
  constexpr int EPI_ROWS = BM * SP * 4 > 150 * 1024 ? WTM : BM;
  constexpr int EPI_PASSES = BM / EPI_ROWS;
  constexpr int EPI_LDS = SWIGLU ? EPI_ROWS * SP * 4 : 0;
  constexpr int LDS = LOOP_LDS > EPI_LDS ? LOOP_LDS : EPI_LDS;
  constexpr int A_INS = GG::A_INS, B_INS = GG::B_INS;
  static_assert(NS >= 2 && (NS - 2) * GG::NL < 64, "pipeline depth");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  __shared__ int s_tile[5];
  // fp8: the weight scales of the tile's reduction range (two 128-column groups: gate and up, or the tile's
  // two output column groups), read once per tile so no pipeline stage waits on a global load of its own
  constexpr int WSC_MAX = 512;  // K / 128 for K <= 65536
  __shared__ float s_wsc[DT == 2 ? 2 * WSC_MAX : 1];
  __shared__ __attribute__((aligned(16))) float s_scp[DT == 2 ? NW * 2 * 64 : 1];
  static_assert(DT != 2 || BM / WM <= 64, "one lane per wavefront row for the scale products");
  // down product, scatter form: the tile's row -> (pair slot, routing weight) map
  __shared__ int s_pair[SWIGLU ? 1 : BM];
  __shared__ float s_pw[SWIGLU ? 1 : BM];
  static_assert(DT != 2 || BM < NW * 64 + 1, "row scales: one per lane of the wavefronts");

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform_int(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const int lr = lane & 31, lh = lane >> 5;

  // Tile: the expert-major ragged schedule of tile::expert_tile (GEMM1: row blocks fastest, or weight tiles
  // fastest for an expert with more rows than the product has weight rows; GEMM2: weight tiles fastest), each
  // XCD taking one contiguous range of the valid tiles (their count comes from the device-resident offsets), so
  // a weight tile and its row blocks stay inside one L2.
  if (wid == 0) {
    const tile::ExpertTile t = tile::workgroup_tile<BM>(a.offsets, a.e_lo, a.E_local, a.n_tiles, a.ksplit,
                                                         SWIGLU ? 2 * a.N_rows : 0, blockIdx.x);
    if (lane == 0) {
      s_tile[0] = t.e;
      s_tile[1] = t.m0;
      s_tile[2] = t.m_end;
      s_tile[3] = t.ni * BNF;
      s_tile[4] = t.part;
    }
  }
  __syncthreads();
  // uniform: scalar registers for everything derived from the tile (addresses, loop bounds)
  const int e = uniform_int(s_tile[0]);
  if (e < 0) return;
  const int m0 = uniform_int(s_tile[1]), m_end = uniform_int(s_tile[2]);
  const int n0 = uniform_int(s_tile[3]);
  const int ks = uniform_int(s_tile[4]);

  const int64_t Kb = (int64_t)a.K * ESZ;  // bytes per row
  const int nk_all = (int)(Kb / RB);      // pipeline stages over the whole reduction dimension
  const int nk = nk_all / a.ksplit;       // this part's stages (the host picks ksplit dividing nk_all)
  const int k0 = ks * nk;                 // first stage of this part
  const int nkb = a.K >> 7;               // fp8 scale blocks along K (== nk for fp8)

  StageCtx<A_INS, B_INS> cx;
  constexpr int CPR = RB / 16;  // 16-byte chunks per row and stage
  // Offsets stay below 2^32: a tile spans at most 256 rows of at most 2^16 fp32 values.
  const int uwid = uniform_int(wid);
  static_assert(!SWIGLU || BNF % GG::RPI == 0, "a direct load never straddles the gate/up boundary");
  // permuted rows: offsets from the tile's first row; gathered rows: from the start of the activations (the host
  // checks T * row bytes < 2^32)
  cx.a_base = uniform_ptr(a.rows ? a.A : a.A + (int64_t)m0 * Kb);
#pragma unroll
  for (int q = 0; q < A_INS; ++q) {
    const int r = (uwid * A_INS + q) * GG::RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<RB>(r);
    const int gr = min(m0 + r, m_end - 1);
    const int64_t src = a.rows ? (int64_t)a.rows[gr] : (int64_t)(gr - m0);
    cx.a_off[q] = (uint32_t)(src * Kb + c * 16);
  }
#pragma unroll
  for (int q = 0; q < B_INS; ++q) {
    // every load covers RPI consecutive rows that are all gate rows or all up rows (RPI divides BNF)
    const int r0 = (uwid * B_INS + q) * GG::RPI;
    const int r = r0 + lane / CPR;
    const int c = (lane % CPR) ^ swz<RB>(r);
    const bool up = SWIGLU && r0 >= BNF;
    const uint8_t* mat = up ? a.B1 : a.B0;
    cx.b_base[q] = uniform_ptr(mat + ((int64_t)e * a.N_rows + n0) * Kb);
    cx.b_off[q] = (uint32_t)((up ? r - BNF : r) * Kb + c * 16);
  }
  cx.sa_base = nullptr;
  cx.sa_off = 0;
  if (DT == 2) {
    const int gr = min(m0 + uwid * 64 + lane, m_end - 1);
    cx.sa_base = uniform_ptr(a.rows ? a.A_scales : a.A_scales + (int64_t)m0 * nkb);
    cx.sa_off = (uint32_t)((a.rows ? (int64_t)a.rows[gr] : (int64_t)(gr - m0)) * nkb * 4);
  }
  cx.wid = uwid;
  cx.lane = lane;
  cx.lh = lh;
  cx.e = e;
  cx.n0 = n0;
  cx.wn = wn;
  cx.wm = wm;
  cx.nkb = nkb;
  cx.nnb = a.N_rows >> 7;
  cx.wsc = s_wsc;
  cx.scp = s_scp;
  cx.k0 = k0;
  cx.nk = nk;
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
  if constexpr (DT == 2) {
    // the 16 x 16 form: rows lane % 16 (+ 16), chunks 2 lg and 2 lg + 1
    const int rsh = lane & 16;
    cx.ao = tile::frag_offsets<RB, 2>(arow[0] - rsh, 2 * (lane >> 4), 1);
    cx.bo = tile::frag_offsets<RB, 2>(brow[0] - rsh, 2 * (lane >> 4), 1);
  } else {
    cx.ao = tile::frag_offsets<RB, RB / 32>(arow[0], lh, 2);
    cx.bo = tile::frag_offsets<RB, RB / 32>(brow[0], lh, 2);
  }

  // Prologue: slices 0 .. NS-2 in flight.  Each iteration then waits for its own slice (the NS-2 newer slices
  // may stay outstanding), meets the other wavefronts at the barrier (after which the buffer read in the
  // previous iteration is free), refills that buffer with slice kt + NS - 1 and computes slice kt.  Slices past
  // the end are clamped to the last one (loaded, never consumed), so every wavefront issues the same number of
  // loads per stage and the counted wait stays exact.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    load_stage<DT, BM, BN, RB, A_INS, B_INS>(smem + s * STAGE, k0 + min(s, nk - 1), cx);
  if constexpr (DT == 2) {
    // the tile's weight scales, read after the prologue's loads are issued so the two latencies overlap (the
    // main loop's first barrier orders these LDS writes before any stage reads them)
    const int nnb = a.N_rows >> 7;
    for (int idx = tid; idx < 2 * nk; idx += NW * 64) {
      const int g = idx >= nk, k = idx - g * nk;
      const float* table = SWIGLU && g ? a.B1_scales : a.B0_scales;
      const int nb = (n0 >> 7) + (SWIGLU ? 0 : g);
      s_wsc[idx] = nb < nnb ? table[((int64_t)e * nkb + k0 + k) * nnb + nb] : 0.0f;
    }
  }
  if constexpr (!SWIGLU) {
    // scatter form: find each row's pair slot right after the prologue's loads are issued, so the lookups'
    // first wait overlaps those loads (the table is read after the main loop's barriers)
    if (a.Yslot != nullptr && ks == 0) {
      for (int r = tid; r < BM; r += NW * 64) {
        const int gm = m0 + r;
        int pr = -1;
        if (gm < m_end) {
          const int t = a.tok[gm];
          for (int j = 0; j < a.k; ++j)
            if (a.rop[(int64_t)t * a.k + j] == gm) pr = t * a.k + j;
        }
        s_pair[r] = pr;
        s_pw[r] = pr >= 0 ? a.wts[pr] : 0.0f;
      }
    }
  }
  // row blocks of this wavefront holding valid rows (fewer than MB only in an expert's last tile)
  const int act = max(0, min(MB, (m_end - m0 - wm * WTM + 31) >> 5));
  int cb = 0;            // buffer holding slice kt
  int fb = NS - 1;       // buffer to refill
  if (act == MB) {
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NS - 2) * GG::NL>();
      __syncthreads();
      gemm_stage<DT, BM, BN, WM, WN, SWIGLU, RB, A_INS, B_INS, MB, NB, true>(
          smem + cb * STAGE, smem + fb * STAGE, k0 + min(kt + NS - 1, nk - 1), k0 + kt, cx, arow, brow, acc, act);
      cb = cb + 1 == NS ? 0 : cb + 1;
      fb = fb + 1 == NS ? 0 : fb + 1;
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<(NS - 2) * GG::NL>();
      __syncthreads();
      gemm_stage<DT, BM, BN, WM, WN, SWIGLU, RB, A_INS, B_INS, MB, NB, false>(
          smem + cb * STAGE, smem + fb * STAGE, k0 + min(kt + NS - 1, nk - 1), k0 + kt, cx, arow, brow, acc, act);
      cb = cb + 1 == NS ? 0 : cb + 1;
      fb = fb + 1 == NS ? 0 : fb + 1;
    }
  }
  wait_vmcnt0();
  __syncthreads();

  if constexpr (SWIGLU) {
    if constexpr (DT != 2) {
      if (a.GU_out != nullptr) {  // training form: keep g and u for the backward pass
        const int F2 = 2 * a.N_rows;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int gm = m0 + wm * WTM + i * 32 + acc_row<DT>(v, lane);
            if (gm >= m_end) continue;
#pragma unroll
            for (int j = 0; j < NB / 2; ++j) {
              const int64_t o = (int64_t)gm * F2 + n0 + wn * (BNF / WN) + j * 32 + acc_col<DT>(v, lane);
              a.GU_out[o] = acc[i][j][v];
              a.GU_out[o + a.N_rows] = acc[i][j + NB / 2][v];
            }
          }
      }
    }
    // silu(G) * U -> LDS (fp32), then per-row stores in the layer dtype
    float* st = reinterpret_cast<float*>(smem);
    const int F = a.N_rows;
    const int c8 = tid & 15;
    for (int pass = 0; pass < EPI_PASSES; ++pass) {
    if (EPI_PASSES == 1 || wm == pass) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB / 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wm * WTM + i * 32 + acc_row<DT>(v, lane) - pass * EPI_ROWS;
            const int col = wn * (BNF / WN) + j * 32 + acc_col<DT>(v, lane);
            const float g = acc[i][j][v], u = acc[i][j + NB / 2][v];
            st[row * SP + col] = g / (1.0f + __expf(-g)) * u;
          }
    }
    __syncthreads();
    for (int r = tid >> 4; r < EPI_ROWS; r += NW * 4) {
      const int gm = m0 + pass * EPI_ROWS + r;
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
    if (pass + 1 < EPI_PASSES) __syncthreads();
    }
  } else {
    const int N = a.N_rows;
    if (a.Yslot != nullptr && ks == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = wm * WTM + i * 32 + acc_row<DT>(v, lane);
          const int pr = m0 + lr < m_end ? s_pair[lr] : -1;
          if (pr >= 0) {
            const float wv = s_pw[lr];
#pragma unroll
            for (int j = 0; j < NB; ++j)
              a.Yslot[(int64_t)pr * N + n0 + wn * WTN + j * 32 + acc_col<DT>(v, lane)] = wv * acc[i][j][v];
          }
        }
    } else {
    float* Yout = ks == 0 ? a.Y : a.Ypart + (int64_t)(ks - 1) * a.R_max * N;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gm = m0 + wm * WTM + i * 32 + acc_row<DT>(v, lane);
        if (gm < m_end) {
#pragma unroll
          for (int j = 0; j < NB; ++j) Yout[(int64_t)gm * N + n0 + wn * WTN + j * 32 + acc_col<DT>(v, lane)] = acc[i][j][v];
        }
      }
    }
  }
}

template <int DT, int BM, int BN, int WM, int WN, bool SWIGLU, int RB, int NS>
static void launch_one(const Args& a, int64_t R_max, hipStream_t s) {
  const int64_t mt = (R_max + BM - 1) / BM + a.E_local;
  const int64_t grid = mt * a.n_tiles * a.ksplit;
  hipLaunchKernelGGL((grouped_gemm_kernel<DT, BM, BN, WM, WN, SWIGLU, RB, NS>), dim3((unsigned)grid),
                     dim3(64 * WM * WN), 0, s, a);
}

// Row-block size from the mean rows per expert (the counts themselves stay on the device).
static int pick_bm(int64_t R_max, int E_local, int dt) {
  const int64_t avg = R_max / (E_local > 0 ? E_local : 1);
  // bf16: 320-row tiles; experts a little over a multiple of 256 rows (the usual case for near-uniform
  // routing) then need no nearly empty last tile, which would stream a full weight slice for a few rows
  if (dt == 1 && avg >= 256) return 320;
  if (dt == 2 && avg >= 256) return 256;
  if (avg >= 96) return 128;
  if (avg >= 48) return 64;
  return 32;
}

// Output columns per down-product tile.  256 when H allows; with small row blocks (the weight-streaming regime
// of decode-sized batches) 128 when 256-column tiles would fill fewer than four rounds of the 256 CUs, so the
// last round's idle share is smaller.
static int down_bn(int64_t R_max, int E_local, int H, int dt) {
  if (H % 256) return 128;
  const int bm = pick_bm(R_max, E_local, dt);
  const int64_t tiles = ((R_max + bm - 1) / bm + E_local / 2) * (H / 256);
  return (bm <= 64 && tiles < 4 * 256) ? 128 : 256;
}

// Tile configurations: bf16 streams 64-byte row slices through 4 stages (3 in flight); fp8 needs a 128-wide
// scale block per stage (128-byte slices, 3 stages); fp32 keeps 2 stages; the 32-row decode tile 3 stages.
template <int DT, bool SWIGLU, int BN>
static void launch_bm(int bm, const Args& a, int64_t R_max, hipStream_t s) {
  switch (bm) {
    case 320:
      if constexpr (DT == 1) launch_one<DT, 320, BN, 2, 4, SWIGLU, 128, 2>(a, R_max, s);
      break;
    case 256:
      if constexpr (DT == 2) launch_one<DT, 256, BN, 4, 2, SWIGLU, 128, 2>(a, R_max, s);
      break;
    case 128:
      if constexpr (DT == 1)
        launch_one<DT, 128, BN, 2, 2, SWIGLU, 64, 4>(a, R_max, s);
      else if constexpr (DT == 2)
        launch_one<DT, 128, BN, 2, 2, SWIGLU, 128, 3>(a, R_max, s);
      else
        launch_one<DT, 128, BN, 2, 2, SWIGLU, 128, 2>(a, R_max, s);
      break;
    case 64:
      if constexpr (DT == 1)
        launch_one<DT, 64, BN, 2, 2, SWIGLU, 64, 4>(a, R_max, s);
      else if constexpr (DT == 2)
        launch_one<DT, 64, BN, 2, 2, SWIGLU, 128, 3>(a, R_max, s);
      else
        launch_one<DT, 64, BN, 2, 2, SWIGLU, 128, 2>(a, R_max, s);
      break;
    default:
      if constexpr (DT == 0)
        launch_one<DT, 32, BN, 1, 4, SWIGLU, 128, 2>(a, R_max, s);
      else
        launch_one<DT, 32, BN, 1, 4, SWIGLU, 128, 3>(a, R_max, s);
      break;
  }
}

template <int DT>
static void launch_gemm1_dt(const FfnLaunch& p, hipStream_t s) {
  Args a{};  // rows x [Wg | Wu] -> h
  a.A = reinterpret_cast<const uint8_t*>(p.x_perm);
  a.A_scales = p.x_perm_scales;
  a.rows = p.gather_rows;
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
  a.GU_out = p.gu;
  a.ksplit = 1;
  a.R_max = p.R_max;
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
  b.Ypart = p.y_part;
  b.Yslot = p.y_slot;
  b.tok = p.token_of_row;
  b.rop = p.row_of_pair;
  b.wts = p.topk_w;
  b.k = p.k;
  b.ksplit = p.ksplit;
  b.R_max = p.R_max;
  const int bm = pick_bm(p.R_max, p.E_local, DT);
  if (down_bn(p.R_max, p.E_local, p.H, DT) == 256) {
    b.n_tiles = p.H / 256;
    launch_bm<DT, false, 256>(bm, b, p.R_max, s);
  } else {
    b.n_tiles = p.H / 128;
    launch_bm<DT, false, 128>(bm, b, p.R_max, s);
  }
}

// y_perm[r] += part[0][r] + part[1][r] + ... (fixed order) for the window rows [offsets[e_lo], offsets[e_hi]).
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(float* __restrict__ y, const float* __restrict__ part,
                                                            int parts, int64_t R_max, int N, const int32_t* offsets,
                                                            int e_lo, int e_hi) {
  const int64_t r0 = offsets[e_lo], r1 = offsets[e_hi];
  const int64_t n4 = N >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one float4 per thread
  const int64_t r = i / n4;
  if (r < r0 || r >= r1) return;
  f32x4_t v = reinterpret_cast<const f32x4_t*>(y)[i];
  for (int s = 0; s < parts; ++s) {
    const f32x4_t p = reinterpret_cast<const f32x4_t*>(part + (int64_t)s * R_max * N)[i];
    v += p;
  }
  reinterpret_cast<f32x4_t*>(y)[i] = v;
}

// Scatter form of the split-reduction sum: one workgroup per permuted row r of the window; slot[p(r)] +=
// w(r) * part[s][r] for s = 0, 1, ... in order (part 0 of the sum was written, already weighted, by the GEMM).
__global__ __launch_bounds__(256) void ksplit_scatter_reduce_kernel(float* __restrict__ yslot,
                                                                    const float* __restrict__ part, int parts,
                                                                    int64_t R_max, int N, const int32_t* offsets,
                                                                    int e_lo, int e_hi, const int32_t* tok,
                                                                    const int32_t* rop, const float* wts, int k) {
  __shared__ int s_p;
  const int64_t r = blockIdx.x;
  const int64_t r0 = offsets[e_lo], r1 = offsets[e_hi];
  if (r < r0 || r >= r1) return;
  if (threadIdx.x == 0) {
    const int t = tok[r];
    int pr = -1;
    for (int j = 0; j < k; ++j)
      if (rop[(int64_t)t * k + j] == r) pr = t * k + j;
    s_p = pr;
  }
  __syncthreads();
  const int pr = s_p;
  if (pr < 0) return;
  const float wv = wts[pr];
  f32x4_t* dst = reinterpret_cast<f32x4_t*>(yslot + (int64_t)pr * N);
  for (int c = threadIdx.x; c < (N >> 2); c += blockDim.x) {
    f32x4_t v = dst[c];
    for (int s = 0; s < parts; ++s) {
      const f32x4_t q = reinterpret_cast<const f32x4_t*>(part + ((int64_t)s * R_max + r) * N)[c];
      v += wv * q;
    }
    dst[c] = v;
  }
}

}  // namespace gemm

// Parts the down GEMM's reduction dimension is split into.  A workgroup fills a CU, so t output tiles run in
// ceil(t / 256) rounds; two parts of half the work finish in ceil(2t / 256) half-length rounds, which is
// shorter only when the tiles fill at most half of the CUs (for t between 129 and 256 both take one full
// round, and the split adds the partial sums' write, read and reduction).  The counts stay on the device, so
// the tile count is estimated as R_max / BM + E_local / 2 (half a ragged tile per expert); the parts are
// summed afterwards in a fixed order.
int ffn_down_ksplit(int64_t R_max, int E_local, int H, int F, moe_dtype dtype) {
  const int dt = dtype == MOE_DTYPE_BF16 ? 1 : dtype == MOE_DTYPE_FP8_E4M3 ? 2 : 0;
  const int bm = gemm::pick_bm(R_max, E_local, dt);
  const int bn = gemm::down_bn(R_max, E_local, H, dt);
  const int64_t tiles = ((R_max + bm - 1) / bm + E_local / 2) * (H / bn);
  const int esz = dt == 0 ? 4 : dt == 1 ? 2 : 1;
  const int64_t nk = (int64_t)F * esz / 128;
  if (2 * tiles <= 256 && nk % 2 == 0 && nk >= 16) return 2;
  return 1;
}

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
  if (p.ksplit > 1 && p.y_slot != nullptr) {
    hipLaunchKernelGGL(gemm::ksplit_scatter_reduce_kernel, dim3((unsigned)p.R_max), dim3(256), 0, s, p.y_slot,
                       p.y_part, p.ksplit - 1, p.R_max, p.H, p.offsets, p.e_lo, p.e_lo + p.E_local, p.token_of_row,
                       p.row_of_pair, p.topk_w, p.k);
  } else if (p.ksplit > 1) {
    const int64_t n4 = p.R_max * (p.H / 4);
    hipLaunchKernelGGL(gemm::ksplit_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p.y_perm,
                       p.y_part, p.ksplit - 1, p.R_max, p.H, p.offsets, p.e_lo, p.e_lo + p.E_local);
  }
}

// ---------------------------------------------------------------------------------------------------------
// Weight packing: per-expert transpose [K][N] -> [N][K] through a 64 x 64 LDS tile, 16-byte accesses on both
// sides (a 64-element source row segment in, a run of 16 / element-size consecutive destination elements out).
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int K, int N) {
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int VPR = 64 / EPV;
  constexpr int P = 64 + 4 / (int)sizeof(T);  // row pitch (elements): one extra dword against bank conflicts
  __shared__ T tile[64 * P];
  const int64_t ex = blockIdx.z;
  src += ex * (int64_t)K * N;
  dst += ex * (int64_t)K * N;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  union V {
    i32x4_t v4;
    T el[EPV];
  };
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int i = v / VPR, q = v % VPR;  // source row k0 + i, columns n0 + q * EPV ...
    V u;
    u.v4 = *reinterpret_cast<const i32x4_t*>(src + (int64_t)(k0 + i) * N + n0 + q * EPV);
#pragma unroll
    for (int x = 0; x < EPV; ++x) tile[i * P + q * EPV + x] = u.el[x];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 64 * VPR; v += 256) {
    const int c = v / VPR, q = v % VPR;  // destination row n0 + c, columns k0 + q * EPV ...
    V u;
#pragma unroll
    for (int x = 0; x < EPV; ++x) u.el[x] = tile[(q * EPV + x) * P + c];
    *reinterpret_cast<i32x4_t*>(dst + (int64_t)(n0 + c) * K + k0 + q * EPV) = u.v4;
  }
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
