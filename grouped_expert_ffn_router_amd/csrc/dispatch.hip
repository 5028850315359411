// Dispatch: counts, offsets, the stable permutation of (token, pick) pairs by expert, and the row gather.
//
// Method: page "Expert Parallelism" (aiwiki), section "Implementation": sort the tokens by destination so
// each destination's rows form one contiguous slab, and count the rows per destination before the exchange.
// The sort here is stable (inside an expert slab the rows keep ascending pair order, which is ascending
// token order), so the permutation is unique and bit-exact.
//
// Three launches (small batches: two, see disp_small_kernel), all deterministic (no order-dependent atomics):
//   hist         one workgroup per count tile of DISP_HTPT tokens (their pairs): LDS histogram ->
//                tile_counts[e][count tile]
//   scan         one workgroup: a flat exclusive scan of tile_counts in (expert, count tile) order gives, for
//                every (e, count tile), the first row of that tile's pairs of expert e; offsets[e] is the (e, 0)
//                entry
//   rank+gather  one workgroup per rank tile of DISP_TPT tokens (DISP_SUB rank tiles per count tile): the
//                workgroup counts the pairs of the earlier rank tiles of its count tile per expert (LDS), then
//                wavefront 0 finds the stable rank of each of its own pairs among same-expert pairs (ballots over
//                the expert id bits: peers are lanes with the same id; the per-expert LDS count runs on across
//                the tile's 64-pair chunks) -> row_of_pair, token_of_row; then one wavefront per token reads the
//                token's row once (16-byte lane accesses, coalesced) and writes it to each of its k destination
//                rows; fp8 scale rows are copied alongside.
// Count tiles larger than rank tiles keep the table (E x T / DISP_HTPT entries) small for the one-workgroup scan;
// rank tiles small enough for one wavefront per token keep the gather spread over many workgroups.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

// Fixed scratch for moe_dispatch_permute_noalloc (callers that cannot allocate): the (expert, tile) count table
// and the uncapped offsets of the multi-workgroup form live here instead of in a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, so kernels receive the device address that hipGetSymbolAddress returns for the stream's device.
static __device__ __align__(256) uint8_t scratch[DISPATCH_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

hipError_t dispatch_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// The multi-workgroup form ranks and gathers in rank tiles of DISP_TPT tokens, i.e. their DISP_TPT * k pairs (at
// most DISP_MAX_CHUNKS chunks of 64 pairs for k <= 32), so every token's pairs lie in one tile; it counts in count
// tiles of DISP_HTPT = DISP_SUB * DISP_TPT tokens.
constexpr int DISP_TPT = 16;
constexpr int DISP_SUB = 8;
constexpr int DISP_HTPT = DISP_TPT * DISP_SUB;
constexpr int DISP_MAX_CHUNKS = DISP_TPT * 32 / 64;

int64_t dispatch_tiles(int64_t T) { return (T + DISP_HTPT - 1) / DISP_HTPT; }

__global__ __launch_bounds__(256) void disp_hist_kernel(const int32_t* __restrict__ idx, int64_t R, int k, int E,
                                                        int64_t n_tiles, int32_t* __restrict__ tile_counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int tp = DISP_HTPT * k;  // pairs per count tile
  const int64_t base = (int64_t)blockIdx.x * tp;
  for (int i = threadIdx.x; i < tp; i += blockDim.x) {
    const int64_t p = base + i;
    if (p < R) {
      const int e = idx[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) tile_counts[(int64_t)e * n_tiles + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(1024) void disp_scan_kernel(int32_t* __restrict__ tc, int E, int64_t n_tiles,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int capacity, int32_t* __restrict__ full_off) {
  __shared__ int wsum[16];
  __shared__ int s_carry;
  __shared__ int s_off[1025];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t N = (int64_t)E * n_tiles;
  if (tid == 0) s_carry = 0;
  for (int e = tid; e <= E; e += blockDim.x) s_off[e] = 0;
  __syncthreads();
  // 16 consecutive entries per thread, 16384 per pass (one pass up to 512 tiles of 32 experts)
  constexpr int VPT = 16;
  for (int64_t base = 0; base < N; base += 1024 * VPT) {
    int v[VPT];
    int tsum = 0;
    const int64_t p0 = base + tid * VPT;
    if (p0 + VPT <= N) {
#pragma unroll
      for (int q = 0; q < VPT / 4; ++q) {
        const i32x4_t u = *reinterpret_cast<const i32x4_t*>(tc + p0 + 4 * q);
        v[4 * q] = u[0];
        v[4 * q + 1] = u[1];
        v[4 * q + 2] = u[2];
        v[4 * q + 3] = u[3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) v[i] = p0 + i < N ? tc[p0 + i] : 0;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) tsum += v[i];
    const int incl = wave_incl_scan(tsum);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    if (wid == 0) {
      const int ws = lane < 16 ? wsum[lane] : 0;
      const int wi = wave_incl_scan(ws);
      if (lane < 16) wsum[lane] = wi - ws;  // exclusive prefix of wave totals
    }
    __syncthreads();
    int run = s_carry + wsum[wid] + incl - tsum;
    int64_t ex = p0 / n_tiles, tl = p0 - ex * n_tiles;  // (expert, tile) of entry p0
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = v[i];
      v[i] = run;  // exclusive prefix of entry p0 + i
      if (p0 + i < N && tl == 0) s_off[ex] = run;
      run += c;
      if (++tl == n_tiles) {
        tl = 0;
        ++ex;
      }
    }
    if (p0 + VPT <= N) {
#pragma unroll
      for (int q = 0; q < VPT / 4; ++q)
        *reinterpret_cast<i32x4_t*>(tc + p0 + 4 * q) = i32x4_t{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (p0 + i < N) tc[p0 + i] = v[i];
    }
    __syncthreads();
    if (tid == 1023) s_carry = run;  // the last thread's running value is the new carry
    __syncthreads();
  }
  if (tid == 0) s_off[E] = s_carry;
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) full_off[e] = s_off[e];
  if (capacity <= 0) {
    for (int e = tid; e <= E; e += blockDim.x) {
      offsets[e] = s_off[e];
      if (e < E) counts[e] = s_off[e + 1] - s_off[e];
    }
    return;
  }
  // fixed capacity: kept counts min(count, capacity) and their exclusive prefix, one thread per expert (E <= 1024)
  const int e = tid;
  const int v = e < E ? min(s_off[e + 1] - s_off[e], capacity) : 0;
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int ws = lane < 16 ? wsum[lane] : 0;
    const int wi = wave_incl_scan(ws);
    if (lane < 16) wsum[lane] = wi - ws;
  }
  __syncthreads();
  const int excl = wsum[wid] + incl - v;
  if (e < E) {
    offsets[e] = excl;
    counts[e] = v;
  }
  if (e == E - 1) offsets[E] = excl + v;
}

// Rank and gather, one workgroup per rank tile of DISP_TPT tokens.  The workgroup first counts, per expert in
// LDS, the pairs of the rank tiles before its own in its count tile (the table entry covers the whole count
// tile).  Wavefront 0 then ranks the tile's pairs chunk by chunk in pair order (peers = lanes with the same
// expert id, from ballots over its bits; the per-expert LDS count runs on across the chunks) and writes
// row_of_pair and token_of_row; then (GATHER) wavefront w copies token w of the tile: its row is read once
// (16-byte lanes) and written to each of its k rows, fp8 scale rows alongside.  CPL 16-byte chunks per lane per
// segment of the row.  n_htiles: count tiles (the table's columns).
template <int CPL, bool GATHER>
__global__ __launch_bounds__(GATHER ? 64 * DISP_TPT : 64) void disp_rank_gather_kernel(
    const int32_t* __restrict__ idx, int64_t R, int64_t T, int k, int E, int nbits, int64_t n_htiles,
    const int32_t* __restrict__ tbase, int32_t* __restrict__ row_of_pair, int32_t* __restrict__ token_of_row,
    int capacity, const int32_t* __restrict__ full_off, const int32_t* __restrict__ offsets,
    const uint8_t* __restrict__ x, const float* __restrict__ xs, int64_t row_bytes, int nsc,
    uint8_t* __restrict__ xp, float* __restrict__ xps) {
  extern __shared__ int cnt[];
  __shared__ int s_rows[DISP_TPT * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  const int64_t tile = blockIdx.x;
  const int64_t htile = tile / DISP_SUB;
  const int tp = DISP_TPT * k;
  const int64_t base = tile * tp;
  const int64_t hbase = htile * (int64_t)(DISP_HTPT * k);
  const int before = (int)(base - hbase);  // pairs of the earlier rank tiles of this count tile, all < R
  __syncthreads();
  for (int i = tid; i < before; i += blockDim.x) {
    const int e = idx[hbase + i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (w == 0) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int ev[DISP_MAX_CHUNKS];
    int rank[DISP_MAX_CHUNKS];
    int npeer[DISP_MAX_CHUNKS];
#pragma unroll
    for (int c = 0; c < DISP_MAX_CHUNKS; ++c) {
      const int64_t p = base + c * 64 + lane;
      int e = (c * 64 + lane < tp && p < R) ? idx[p] : -1;
      ev[c] = ((unsigned)e < (unsigned)E) ? e : -1;
    }
#pragma unroll
    for (int c = 0; c < DISP_MAX_CHUNKS; ++c) {
      const bool valid = ev[c] >= 0;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (ev[c] >> b) & 1;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
      }
      rank[c] = __popcll(m & lt_mask);
      npeer[c] = __popcll(m);
    }
    // Chunks in order: every lane reads the running count of its expert, then the first lane of each peer
    // group advances it.  Within one wavefront the LDS read of a chunk precedes that chunk's write.
#pragma unroll
    for (int c = 0; c < DISP_MAX_CHUNKS; ++c) {
      if (ev[c] >= 0) {
        const int before = cnt[ev[c]];
        __builtin_amdgcn_wave_barrier();
        if (rank[c] == 0) cnt[ev[c]] = before + npeer[c];
        rank[c] += before;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int c = 0; c < DISP_MAX_CHUNKS; ++c) {
      const int64_t p = base + c * 64 + lane;
      if (c * 64 + lane < tp && p < R) {
        int row = -1;
        if (ev[c] >= 0) {
          row = tbase[(int64_t)ev[c] * n_htiles + htile] + rank[c];
          if (capacity > 0) {  // rank among the expert's pairs: kept (packed) if below the capacity, else dropped
            const int re = row - full_off[ev[c]];
            row = re < capacity ? offsets[ev[c]] + re : -1;
          }
        }
        row_of_pair[p] = row;
        if (row >= 0) token_of_row[row] = (int)(p / k);
        s_rows[c * 64 + lane] = row;
      }
    }
  }
  if constexpr (GATHER) {
    __syncthreads();
    const int64_t t = tile * DISP_TPT + w;
    if (t >= T) return;
    const int myrow = lane < k ? s_rows[w * k + lane] : -1;
    const int64_t n16 = row_bytes >> 4;
    const i32x4_t* src = reinterpret_cast<const i32x4_t*>(x + t * row_bytes);
    for (int64_t seg = 0; seg < n16; seg += CPL * 64) {
      i32x4_t buf[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t c = seg + i * 64 + lane;
        if (c < n16) buf[i] = __builtin_nontemporal_load(src + c);
      }
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(myrow, j, 64);
        if (r < 0) continue;
        i32x4_t* dst = reinterpret_cast<i32x4_t*>(xp + (int64_t)r * row_bytes);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int64_t c = seg + i * 64 + lane;
          if (c < n16) dst[c] = buf[i];
        }
      }
    }
    if (nsc > 0) {
      for (int c0 = 0; c0 < nsc; c0 += 64) {
        const int c = c0 + lane;
        const float sv = c < nsc ? xs[t * nsc + c] : 0.0f;
        for (int j = 0; j < k; ++j) {
          const int r = __shfl(myrow, j, 64);
          if (r >= 0 && c < nsc) xps[(int64_t)r * nsc + c] = sv;
        }
      }
    }
  }
}

// Small batches (R <= DISP_SMALL_R pairs): counts, offsets and the permutation in one workgroup of 16 waves, the
// same definition as hist -> scan -> rank.  Wave w owns the contiguous pair range [w P, (w+1) P): it counts its
// pairs per expert in its own LDS row; each expert's counts are turned into an exclusive prefix over the waves;
// the experts' totals into offsets (kept counts min(count, C) when a capacity is set); then every wave ranks its
// pairs chunk by chunk in pair order exactly as the rank kernel does.  Saves two launches and their gaps.
constexpr int64_t DISP_SMALL_R = 16384;
__global__ __launch_bounds__(1024) void disp_small_kernel(const int32_t* __restrict__ idx, int64_t R, int k, int E,
                                                          int nbits, int capacity, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_of_pair,
                                                          int32_t* __restrict__ token_of_row) {
  extern __shared__ int sm[];
  int* cnt = sm;                   // [16][E]: per-wave counts, then running per-wave, per-expert row counters
  int* full = sm + 16 * E;         // [E + 1]: uncapped expert offsets
  int* kept = full + E + 1;        // [E + 1]: offsets of the kept rows
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t P = ((R + 15) / 16 + 63) / 64 * 64;  // pairs per wave, whole 64-pair chunks
  const int64_t p0 = w * P, p1 = min(R, p0 + P);
  for (int i = tid; i < 16 * E; i += 1024) cnt[i] = 0;
  __syncthreads();
  for (int64_t p = p0 + lane; p < p1; p += 64) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[w * E + e], 1);
  }
  __syncthreads();
  // per expert: exclusive prefix over the waves (each expert's rows in wave order), total in full[e]
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int v = 0; v < 16; ++v) {
      const int c = cnt[v * E + e];
      cnt[v * E + e] = run;
      run += c;
    }
    full[e] = run;
  }
  __syncthreads();
  // exclusive scans over the experts (E <= 1024: one expert per thread): totals, and kept counts
  {
    const int tot = tid < E ? full[tid] : 0;
    const int kp = tid < E ? (capacity > 0 ? min(tot, capacity) : tot) : 0;
    int it = tot, ik = kp;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int ut = __shfl_up(it, o, 64), uk = __shfl_up(ik, o, 64);
      if (lane >= o) {
        it += ut;
        ik += uk;
      }
    }
    if (lane == 63) wsum[w] = it;
    __syncthreads();
    int bt = 0;
    for (int v = 0; v < w; ++v) bt += wsum[v];
    __syncthreads();
    if (lane == 63) wsum[w] = ik;
    __syncthreads();
    int bk = 0;
    for (int v = 0; v < w; ++v) bk += wsum[v];
    __syncthreads();
    if (tid < E) {
      full[tid] = bt + it - tot;
      kept[tid] = bk + ik - kp;
      counts[tid] = kp;
      offsets[tid] = bk + ik - kp;
    }
    if (tid == E - 1) offsets[E] = bk + ik;
  }
  __syncthreads();
  // ranks: chunks of 64 pairs in order; peers = lanes with the same expert id (ballots over its bits)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = p0; c0 < p1; c0 += 64) {  // uniform over the wave
    const int64_t p = c0 + lane;
    int e = p < p1 ? idx[p] : -1;
    if ((unsigned)e >= (unsigned)E) e = -1;
    uint64_t m = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      m &= bit ? bal : ~bal;
    }
    const int rank = __popcll(m & lt_mask), npeer = __popcll(m);
    int re = 0;
    if (e >= 0) {
      const int before = cnt[w * E + e];
      __builtin_amdgcn_wave_barrier();
      if (rank == 0) cnt[w * E + e] = before + npeer;
      re = before + rank;  // rank among all of the expert's pairs
    }
    __builtin_amdgcn_wave_barrier();
    if (p < p1) {
      int row = -1;
      if (e >= 0) row = capacity > 0 ? (re < capacity ? kept[e] + re : -1) : full[e] + re;
      row_of_pair[p] = row;
      if (row >= 0) token_of_row[row] = (int)(p / k);
    }
  }
}

// One wavefront per token; CPL 16-byte chunks per lane per segment of the row.
template <int CPL>
__global__ __launch_bounds__(256) void disp_gather_kernel(const uint8_t* __restrict__ x, const float* __restrict__ xs,
                                                          int64_t T, int64_t row_bytes, int nsc, int k,
                                                          const int32_t* __restrict__ row_of_pair,
                                                          uint8_t* __restrict__ xp, float* __restrict__ xps) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int myrow = lane < k ? row_of_pair[t * k + lane] : -1;
  const int64_t n16 = row_bytes >> 4;
  const i32x4_t* src = reinterpret_cast<const i32x4_t*>(x + t * row_bytes);
  for (int64_t seg = 0; seg < n16; seg += CPL * 64) {
    i32x4_t buf[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t c = seg + i * 64 + lane;
      if (c < n16) buf[i] = __builtin_nontemporal_load(src + c);
    }
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(myrow, j, 64);
      if (r < 0) continue;
      i32x4_t* dst = reinterpret_cast<i32x4_t*>(xp + (int64_t)r * row_bytes);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t c = seg + i * 64 + lane;
        if (c < n16) dst[c] = buf[i];
      }
    }
  }
  if (nsc > 0) {
    for (int c0 = 0; c0 < nsc; c0 += 64) {
      const int c = c0 + lane;
      const float sv = c < nsc ? xs[t * nsc + c] : 0.0f;
      for (int j = 0; j < k; ++j) {
        const int r = __shfl(myrow, j, 64);
        if (r >= 0 && c < nsc) xps[(int64_t)r * nsc + c] = sv;
      }
    }
  }
}

void launch_dispatch(const void* x, const float* x_scales, int esize, int64_t T, int H, const int32_t* topk_idx, int k,
                     int E, int32_t* counts, int32_t* offsets, int32_t* row_of_pair, int32_t* token_of_row,
                     void* x_perm, float* x_perm_scales, void* workspace, int capacity, hipStream_t s) {
  const int64_t R = T * k;
  const int64_t n_tiles = dispatch_tiles(T);
  int32_t* tc = reinterpret_cast<int32_t*>(workspace);
  // uncapped expert offsets, after the (expert, tile) counts, 256-byte aligned
  int32_t* full_off = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(workspace) +
                                                 (((size_t)E * (size_t)n_tiles * 4 + 255) & ~(size_t)255));
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int64_t row_bytes = (int64_t)H * esize;
  const int nsc = x_scales ? H / 128 : 0;
  const int64_t chunks_per_lane = (row_bytes / 16 + 63) / 64;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  uint8_t* xpb = reinterpret_cast<uint8_t*>(x_perm);
  if (R == 0 || R > DISP_SMALL_R) {
    // counts per count tile, their scan, then ranks and (with x_perm) the gather in one launch per rank tile
    if (n_tiles > 0)
      hipLaunchKernelGGL(disp_hist_kernel, dim3((unsigned)n_tiles), dim3(256), E * sizeof(int), s, topk_idx, R, k,
                         E, n_tiles, tc);
    hipLaunchKernelGGL(disp_scan_kernel, dim3(1), dim3(1024), 0, s, tc, E, n_tiles, counts, offsets, capacity,
                       full_off);
    if (n_tiles == 0) return;
    const dim3 grid((unsigned)((T + DISP_TPT - 1) / DISP_TPT));
    const size_t lds = E * sizeof(int);
#define MOE_RG(CPL, G)                                                                                            \
  hipLaunchKernelGGL((disp_rank_gather_kernel<CPL, G>), grid, dim3(G ? 64 * DISP_TPT : 64), lds, s, topk_idx, R, \
                     T, k, E, nbits, n_tiles, tc, row_of_pair, token_of_row, capacity, full_off, offsets, xb,      \
                     x_scales, row_bytes, nsc, xpb, x_perm_scales)
    if (x_perm == nullptr)
      MOE_RG(1, false);
    else if (chunks_per_lane <= 1)
      MOE_RG(1, true);
    else if (chunks_per_lane <= 2)
      MOE_RG(2, true);
    else if (chunks_per_lane <= 4)
      MOE_RG(4, true);
    else if (chunks_per_lane <= 8)
      MOE_RG(8, true);
    else
      MOE_RG(16, true);
#undef MOE_RG
    return;
  }
  hipLaunchKernelGGL(disp_small_kernel, dim3(1), dim3(1024), (size_t)(18 * E + 2) * sizeof(int), s, topk_idx, R, k,
                     E, nbits, capacity, counts, offsets, row_of_pair, token_of_row);
  if (x_perm == nullptr) return;  // index only: the grouped FFN reads x through token_of_row
  const unsigned blocks = (unsigned)((T + 3) / 4);
  if (chunks_per_lane <= 1)
    hipLaunchKernelGGL((disp_gather_kernel<1>), dim3(blocks), dim3(256), 0, s, xb, x_scales, T, row_bytes, nsc, k,
                       row_of_pair, xpb, x_perm_scales);
  else if (chunks_per_lane <= 2)
    hipLaunchKernelGGL((disp_gather_kernel<2>), dim3(blocks), dim3(256), 0, s, xb, x_scales, T, row_bytes, nsc, k,
                       row_of_pair, xpb, x_perm_scales);
  else if (chunks_per_lane <= 4)
    hipLaunchKernelGGL((disp_gather_kernel<4>), dim3(blocks), dim3(256), 0, s, xb, x_scales, T, row_bytes, nsc, k,
                       row_of_pair, xpb, x_perm_scales);
  else if (chunks_per_lane <= 8)
    hipLaunchKernelGGL((disp_gather_kernel<8>), dim3(blocks), dim3(256), 0, s, xb, x_scales, T, row_bytes, nsc, k,
                       row_of_pair, xpb, x_perm_scales);
  else
    hipLaunchKernelGGL((disp_gather_kernel<16>), dim3(blocks), dim3(256), 0, s, xb, x_scales, T, row_bytes, nsc, k,
                       row_of_pair, xpb, x_perm_scales);
}

}  // namespace moe
