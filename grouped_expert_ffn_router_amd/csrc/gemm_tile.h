// Pieces shared by the grouped matrix products of the forward (ffn.hip) and the backward (bwd.hip): the LDS stage
// layout, the ragged per-expert tile schedule, and the bf16 / fp32 MFMA work of one pipeline stage.
#pragma once
#include "common.h"

namespace moe {
namespace tile {

// ---------------------------------------------------------------------------------------------------------
// LDS pipeline stages.  A stage holds RB bytes of the reduction dimension (RB = 64 or 128) for every tile row:
// row r occupies RB contiguous bytes and its 16-byte chunk c sits at chunk position c ^ swz(r).  An MFMA
// fragment read takes one chunk from 32 consecutive rows; gfx950 serves a 16-byte-per-lane LDS read 16 lanes
// at a time across 64 four-byte banks (256 bytes), so 16 consecutive rows must fall on 16 distinct 16-byte
// bank groups: two 128-byte rows share a 256-byte bank line (swizzle (r >> 1) & 7), four 64-byte rows do
// (swizzle (r >> 2) & 3).  Measured: the plain layout conflicts 8-way, (r & 7) 2-way, these not at all.
// ---------------------------------------------------------------------------------------------------------
template <int RB>
MOE_DEV int swz(int row) {
  return RB == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// ---------------------------------------------------------------------------------------------------------
// Ragged tiles without a host sync.  Local expert i owns rows [offsets[e_lo + i], offsets[e_lo + i + 1]); its
// row blocks of BM rows times nt column tiles times `parts` reduction parts are its tiles, enumerated expert by
// expert.  Inside an expert: row blocks fastest, so the row blocks sharing a weight tile are consecutive; for an
// expert with more rows than `nfast_rows` (callers pass its weight rows) column tiles fastest instead, so its
// row blocks, the larger operand, stream once while the smaller weight tiles are re-read from cache
// (nfast_rows = 0: column tiles fastest for every expert).  Reduction parts are outermost.  Called by one whole
// wavefront; every lane gets the same result.
// ---------------------------------------------------------------------------------------------------------
struct ExpertTile {
  int e;      // local expert, -1 for a surplus tile index
  int m0;     // first row of the row block
  int m_end;  // end of the expert's rows
  int ni;     // column tile
  int part;   // reduction part
};

template <int BM>
MOE_DEV int expert_tiles_total(const int32_t* offsets, int e_lo, int E_local, int nt, int parts) {
  const int lane = lane_id();
  int total = 0;
  for (int base = 0; base < E_local; base += 64) {
    const int i = base + lane;
    const int cnt = i < E_local ? offsets[e_lo + i + 1] - offsets[e_lo + i] : 0;
    int u = ((cnt + BM - 1) / BM) * nt * parts;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) u += __shfl_xor(u, o, 64);
    total += u;
  }
  return total;
}

// The tile of the lane holding it: lane `src` of the wavefront owns local expert i (rows [beg, end), `tiles` row
// blocks) and loc is the tile's index inside that expert (valid in lane src); every lane gets the fields.
template <int BM>
MOE_DEV ExpertTile tile_in_expert(uint64_t hm, int i, int beg, int end, int tiles, int loc, int nt,
                                  int nfast_rows) {
  ExpertTile t;
  const int src = __ffsll((unsigned long long)hm) - 1;
  const int tl = tiles > 0 ? tiles : 1;
  const bool nfast = end - beg > nfast_rows;
  const int mi = nfast ? (loc / nt) % tl : loc % tl;
  const int ni = nfast ? loc % nt : (loc / tl) % nt;
  t.e = __shfl(i, src, 64);
  t.m0 = __shfl(beg + mi * BM, src, 64);
  t.m_end = __shfl(end, src, 64);
  t.ni = __shfl(ni, src, 64);
  t.part = __shfl(loc / (tl * nt), src, 64);
  return t;
}

template <int BM>
MOE_DEV ExpertTile expert_tile(const int32_t* offsets, int e_lo, int E_local, int nt, int parts, int nfast_rows,
                               int L) {
  const int lane = lane_id();
  ExpertTile t{-1, 0, 0, 0, 0};
  int cum = 0;
  for (int base = 0; base < E_local; base += 64) {
    const int i = base + lane;
    int beg = 0, end = 0;
    if (i < E_local) {
      beg = offsets[e_lo + i];
      end = offsets[e_lo + i + 1];
    }
    const int tiles = (end - beg + BM - 1) / BM;
    const int units = tiles * nt * parts;
    const int incl = wave_incl_scan(units);
    const int excl = incl - units;
    const int rel = L - cum;
    const uint64_t hm = __ballot(rel >= excl && rel < incl);
    if (hm) {
      t = tile_in_expert<BM>(hm, i, beg, end, tiles, rel - excl, nt, nfast_rows);
      break;
    }
    cum += __shfl(incl, 63, 64);
  }
  return t;
}

// Workgroup ids are dealt to the 8 XCDs round-robin; this maps workgroup bid to the tile index L so that each
// XCD (and its L2) receives one contiguous range of the `total` valid tiles.  -1 for surplus workgroups.
MOE_DEV int xcd_tile_index(int total, int bid) {
  if (bid >= total) return -1;
  const int q = total >> 3, r = total & 7, x = bid & 7;
  return x * q + min(x, r) + (bid >> 3);
}

// The tile of workgroup bid: expert_tiles_total, xcd_tile_index and expert_tile in one pass over the offsets
// (one load per lane) when the window holds at most 64 experts, the three calls otherwise; e = -1 for a surplus
// workgroup.  Called by one whole wavefront.
template <int BM>
MOE_DEV ExpertTile workgroup_tile(const int32_t* offsets, int e_lo, int E_local, int nt, int parts, int nfast_rows,
                                  int bid) {
  ExpertTile t{-1, 0, 0, 0, 0};
  if (E_local > 64) {
    const int L = xcd_tile_index(expert_tiles_total<BM>(offsets, e_lo, E_local, nt, parts), bid);
    return L >= 0 ? expert_tile<BM>(offsets, e_lo, E_local, nt, parts, nfast_rows, L) : t;
  }
  const int lane = lane_id();
  int beg = 0, end = 0;
  if (lane < E_local) {
    beg = offsets[e_lo + lane];
    end = offsets[e_lo + lane + 1];
  }
  const int tiles = (end - beg + BM - 1) / BM;
  const int units = tiles * nt * parts;
  const int incl = wave_incl_scan(units);
  const int L = xcd_tile_index(__shfl(incl, 63, 64), bid);
  if (L < 0) return t;
  const int excl = incl - units;
  const uint64_t hm = __ballot(L >= excl && L < incl);
  return hm ? tile_in_expert<BM>(hm, lane, beg, end, tiles, L - excl, nt, nfast_rows) : t;
}

// ---------------------------------------------------------------------------------------------------------
// Fragment addresses.  A lane reads the rows row0 + d of an operand (d a multiple of 16, fixed at compile time
// for each fragment) and, at step s, chunk 2s + lh of each (the 16x16 fp8 form: chunks 2 lg and 2 lg + 1).  The
// swizzle depends on row bits 1..3 (128-byte rows) or 2..3 (64-byte rows) only, so rows 16 apart share chunk
// positions: every fragment address is one per-lane offset per step plus a compile-time byte offset.  The
// offsets are computed once per tile; a stage adds its buffer base once per offset, so its LDS reads cost no
// other address arithmetic.
// ---------------------------------------------------------------------------------------------------------
struct FragOff {
  uint32_t o[4];
};

// Offsets of chunks c0 + cstep * s (s < N <= 4) of row `row0`: byte row0 * RB + swizzled chunk position.
template <int RB, int N>
MOE_DEV FragOff frag_offsets(int row0, int c0, int cstep) {
  static_assert(N <= 4, "at most four chunks per lane and stage");
  FragOff f{};
#pragma unroll
  for (int s = 0; s < N; ++s) f.o[s] = (uint32_t)(row0 * RB + (((c0 + cstep * s) ^ swz<RB>(row0)) << 4));
  return f;
}

// LDS-typed byte pointers, so a base plus a compile-time offset becomes one ds_read with an immediate offset.
typedef __attribute__((address_space(3))) const uint8_t lds_u8_t;
typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;
MOE_DEV lds_u8_t* to_lds(const uint8_t* p) { return (lds_u8_t*)p; }
// 16-byte LDS read at a per-lane address plus a compile-time byte offset.
MOE_DEV i32x4_t lds_at(lds_u8_t* p, int imm) { return *(lds_i32x4_t*)(p + imm); }

// ---------------------------------------------------------------------------------------------------------
// One stage of MFMA work over LDS operands: acc[i][j] += A rows arow[i] (32 each) x B rows brow[j] over the
// stage's reduction slice.  A and B register slots pair one-to-one along the reduction, so lane half h of a
// 32 x 32 block reads chunk 2s + h of its own row at bf16 step s (fp32: element s % 4 of chunk 2 (s / 4) + h).
// ao / bo: frag_offsets of arow[0] / brow[0] (chunks lh, lh + 2, ...); arow[i] - arow[0] and brow[j] - brow[0]
// are compile-time multiples of 16 after inlining.
// ---------------------------------------------------------------------------------------------------------

// bf16: k-steps of 16 (one 16-byte chunk per lane half); fragments double-buffered in registers so step s+1's LDS
// reads overlap step s's MFMAs, interleaved one LDS read per group of MFMAs.
template <int RB, int MB, int NB>
MOE_DEV void mma_stage_bf16(const uint8_t* As, const uint8_t* Bs, const int (&arow)[MB], const int (&brow)[NB],
                            const FragOff& ao, const FragOff& bo,
                            f32x16_t (&acc)[MB][NB]) {
  constexpr int NSTEP = RB / 32;
  lds_u8_t* av[NSTEP];
  lds_u8_t* bv[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    av[s] = to_lds(As) + ao.o[s];
    bv[s] = to_lds(Bs) + bo.o[s];
  }
  bf16x8_t fa[2][MB], fb[2][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) fa[0][i] = __builtin_bit_cast(bf16x8_t, lds_at(av[0], (arow[i] - arow[0]) * RB));
#pragma unroll
  for (int j = 0; j < NB; ++j) fb[0][j] = __builtin_bit_cast(bf16x8_t, lds_at(bv[0], (brow[j] - brow[0]) * RB));
  sched_fence();
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int c = s & 1;
    if (s + 1 < NSTEP) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
        fa[c ^ 1][i] = __builtin_bit_cast(bf16x8_t, lds_at(av[s + 1], (arow[i] - arow[0]) * RB));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[c ^ 1][j] = __builtin_bit_cast(bf16x8_t, lds_at(bv[s + 1], (brow[j] - brow[0]) * RB));
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mfma_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j]);
    if (s + 1 < NSTEP) {
      constexpr int PER = (MB * NB) / (MB + NB) > 0 ? (MB * NB) / (MB + NB) : 1;
#pragma unroll
      for (int q = 0; q < MB + NB; ++q) {
        if constexpr (PER >= 4)
          sched_ds1_mfma4();
        else if constexpr (PER >= 2)
          sched_ds1_mfma2();
        else
          sched_ds1_mfma1();
      }
    }
    sched_fence();
  }
}

// bf16, a partial row block: only the first `act` row blocks of this wavefront hold rows; the others skip their
// LDS reads and MFMAs.
template <int RB, int MB, int NB>
MOE_DEV void mma_stage_bf16_partial(const uint8_t* As, const uint8_t* Bs, const int (&arow)[MB], const int (&brow)[NB],
                                    const FragOff& ao, const FragOff& bo,
                                    f32x16_t (&acc)[MB][NB], int act) {
  constexpr int NSTEP = RB / 32;
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    lds_u8_t* avs = to_lds(As) + ao.o[s];
    lds_u8_t* bvs = to_lds(Bs) + bo.o[s];
    bf16x8_t fb[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[j] = __builtin_bit_cast(bf16x8_t, lds_at(bvs, (brow[j] - brow[0]) * RB));
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i < act) {
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, lds_at(avs, (arow[i] - arow[0]) * RB));
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma_32x32x16_bf16(fa, fb[j], acc[i][j]);
      }
    }
  }
}

// fp32: 128-byte stages of 32 values, four chunks of four k-steps each; rows past `act` row blocks skipped.
template <int MB, int NB>
MOE_DEV void mma_stage_f32(const uint8_t* As, const uint8_t* Bs, const int (&arow)[MB], const int (&brow)[NB],
                           const FragOff& ao, const FragOff& bo, f32x16_t (&acc)[MB][NB],
                           int act) {
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    lds_u8_t* avs = to_lds(As) + ao.o[s4];
    lds_u8_t* bvs = to_lds(Bs) + bo.o[s4];
    f32x4_t af[MB], bf[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) af[i] = __builtin_bit_cast(f32x4_t, lds_at(avs, (arow[i] - arow[0]) * 128));
#pragma unroll
    for (int j = 0; j < NB; ++j) bf[j] = __builtin_bit_cast(f32x4_t, lds_at(bvs, (brow[j] - brow[0]) * 128));
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < act)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_32x32x2_f32(af[i][ss], bf[j][ss], acc[i][j]);
  }
}

}  // namespace tile
}  // namespace moe
