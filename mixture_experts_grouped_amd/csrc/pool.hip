// pool.hip -- dispatch pool builder, the grouped-GEMM tile map and the saved
// copy of the layer input.
//
// The pool is expert-contiguous and padded per expert to BLOCK_M rows, each
// expert starting at its true offset (DeepGEMM PR #9, "2026-09-21: restore
// wide-K wgrad safely" -> Implementation); padding rows of the gathered input
// are zero (PR #9, "Historical implementation" -> Summary).  Rows inside an
// expert follow ascending route index t*k + j, so the pool is a deterministic
// function of the routing (the pages' atomic dispatch order is not).
//
// With several adapters (OpenPipe/ART PR #1139, Behavior: dispatched rows
// carry adapter IDs) the pool's groups are (expert e, adapter q) pairs,
// group e * na + q, q the root of the route's token: each group's rows then
// share one adapter's expert-local factors, and the groups of one expert
// stay adjacent (its base weights serve them back to back).
#include "layer.hpp"
#include "trace.hpp"

namespace moelora {

constexpr int POOL_THREADS = 1024;
constexpr int POOL_WAVES = POOL_THREADS / 64;
constexpr int POOL_V = 16;                            // routes per thread per chunk
constexpr int POOL_CHUNK = POOL_THREADS * POOL_V;     // routes per chunk

__device__ __forceinline__ int pool_pad(int n, int bm) { return ((n + bm - 1) / bm) * bm; }

// Sum of v over the workgroup (every thread gets it).  `red` holds
// POOL_WAVES ints; the call ends with a barrier, so `red` can be reused.
__device__ __forceinline__ int pool_block_sum(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < POOL_WAVES; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Pool group of route f with expert id `id` (valid or not): -1 for a dropped
// or invalid id, else id * na + the root of token f / k.
__device__ __forceinline__ int route_group(int id, int f, int E, const PoolRoots& pr) {
  if (!(id >= 0 && id < E)) return -1;
  if (pr.na == 1) return id;
  const int t = f / pr.k;
  int q = 0;
  for (int i = 1; i < pr.na; ++i) q += t >= pr.roots[i];  // roots nondecreasing
  return id * pr.na + q;
}

// Workgroup e counts the routes of group e (workgroup 0 also the invalid
// ids): compares and a workgroup sum, no atomics.
__global__ __launch_bounds__(POOL_THREADS) void k_pool_count(const int32_t* __restrict__ idx, int nroutes,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ err, PoolRoots pr) {
  __shared__ int red[POOL_WAVES];
  const int tid = threadIdx.x, e = blockIdx.x;
  int m = 0, bad = 0;
  for (int c0 = 0; c0 < nroutes; c0 += POOL_CHUNK) {
    int ids[POOL_V];  // all of a chunk's loads in flight at once
#pragma unroll
    for (int v = 0; v < POOL_V; ++v) {
      const int f = c0 + v * POOL_THREADS + tid;
      ids[v] = (f < nroutes) ? idx[f] : -1;
    }
#pragma unroll
    for (int v = 0; v < POOL_V; ++v) {
      m += route_group(ids[v], c0 + v * POOL_THREADS + tid, E, pr) == e;
      bad += !(ids[v] >= -1 && ids[v] < E);
    }
  }
  const int n = pool_block_sum(m, red);
  if (tid == 0) counts[e] = n;
  if (e == 0) {
    const int nbad = pool_block_sum(bad, red);
    if (tid == 0 && err != nullptr) *err = nbad;
  }
}

// Workgroup e places the routes of group e (EV = E na groups): its padded
// offset is the sum of the padded counts before it; then it walks the routes in chunks of
// POOL_CHUNK (thread tid reads routes c0 + v * POOL_THREADS + tid, coalesced)
// and gives the routes of expert e consecutive rows in ascending route order:
// a route's row is the matches before it, counted with one ballot per (v,
// wave) and an exclusive scan of those counts in (v, wave) order, which is
// route order.  Workgroup 0 also marks dropped routes; the last workgroup
// clears the unused suffix of the pool.
__global__ __launch_bounds__(POOL_THREADS) void k_build_pool(
    const int32_t* __restrict__ idx, int nroutes, int E, int bm, long cap,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ r2row,
    int32_t* __restrict__ row2r, PoolRoots pr) {
  const int EV = E * pr.na;
  constexpr int NC = POOL_V * POOL_WAVES;  // (v, wave) counts per chunk
  static_assert(NC <= POOL_THREADS && NC % 64 == 0 && POOL_V <= 64, "scan layout");
  __shared__ int red[POOL_WAVES];
  __shared__ int cnt[NC];   // [v][wave] matches
  __shared__ int pre[NC];   // exclusive prefix of cnt
  __shared__ int wsum[NC / 64];
  __shared__ int total;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  int before = 0;
  for (int i = tid; i < e; i += POOL_THREADS) before += pool_pad(counts[i], bm);
  const int off = pool_block_sum(before, red);
  const int n = counts[e], padded = pool_pad(n, bm);
  if (tid == 0) {
    offsets[e] = off;
    if (e == EV - 1) offsets[EV] = off + padded;
  }
  for (int p = off + n + tid; p < off + padded; p += POOL_THREADS) row2r[p] = -1;  // padding rows
  if (e == EV - 1)
    for (long p = off + padded + tid; p < cap; p += POOL_THREADS) row2r[p] = -1;  // unused suffix
  const unsigned long long below = (1ull << lane) - 1ull;
  int run = off;  // next row of expert e (uniform)
  for (int c0 = 0; c0 < nroutes; c0 += POOL_CHUNK) {
    int ids[POOL_V];
    unsigned long long bal[POOL_V];
#pragma unroll
    for (int v = 0; v < POOL_V; ++v) {
      const int f = c0 + v * POOL_THREADS + tid;
      ids[v] = (f < nroutes) ? route_group(idx[f], f, E, pr) : -1;  // -1: dropped or invalid
    }
    int mine = 0;
#pragma unroll
    for (int v = 0; v < POOL_V; ++v) {
      bal[v] = __ballot(ids[v] == e);
      if (lane == v) mine = __popcll(bal[v]);
    }
    if (lane < POOL_V) cnt[lane * POOL_WAVES + wv] = mine;
    __syncthreads();
    int x = 0, c = 0;
    if (tid < NC) {
      c = cnt[tid];
      x = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[wv] = x;
    }
    __syncthreads();
    if (tid < NC) {
      int carry = 0;
      for (int w = 0; w < wv; ++w) carry += wsum[w];
      pre[tid] = carry + x - c;
      if (tid == NC - 1) total = carry + x;
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < POOL_V; ++v) {
      const int f = c0 + v * POOL_THREADS + tid;
      if (ids[v] == e) {
        const int pos = run + pre[v * POOL_WAVES + wv] + __popcll(bal[v] & below);
        r2row[f] = pos;
        row2r[pos] = f;
      } else if (e == 0 && f < nroutes && ids[v] < 0) {
        r2row[f] = -1;  // dropped or invalid route
      }
    }
    run += total;
    __syncthreads();  // cnt / pre / total are rewritten by the next chunk
  }
}

hipError_t launch_build_pool(const int32_t* idx, int nroutes, int E, int bm, long cap,
                             int32_t* counts, int32_t* offsets, int32_t* r2row, int32_t* row2r,
                             int32_t* err, const PoolRoots& pr, hipStream_t st) {
  const unsigned EV = (unsigned)(E * pr.na);
  MOE_LAUNCH(k_pool_count, dim3(EV), dim3(POOL_THREADS), 0, st, idx, nroutes, E, counts, err, pr);
  MOE_LAUNCH(k_build_pool, dim3(EV), dim3(POOL_THREADS), 0, st, idx, nroutes, E, bm, cap, counts,
             offsets, r2row, row2r, pr);
  return hipGetLastError();
}

// Grouped-GEMM M tiles: TMG rows of one pool group each, never crossing
// groups; and the same for TML-row tiles, whose `pad` is the accumulator-
// blocked row block index (acc_blk) of their first row: 8 x the TMG tile
// holding it plus its 32-row block inside that tile.
__global__ __launch_bounds__(64) void k_tile_map(LayerArgs a) {
  const int lane = threadIdx.x;
  int carry = 0, carry3 = 0;
  for (int b0 = 0; b0 < a.EV; b0 += 64) {
    const int e = b0 + lane;
    const int n = (e < a.EV) ? a.counts[e] : 0;
    const int nt = (n + TMG - 1) / TMG, nt3 = (n + TML - 1) / TML;
    int x = nt, x3 = nt3;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64), y3 = __shfl_up(x3, o, 64);
      if (lane >= o) {
        x += y;
        x3 += y3;
      }
    }
    const int start = carry + x - nt, start3 = carry3 + x3 - nt3;
    if (e < a.EV) {
      const int off = a.offsets[e];
      for (int t = 0; t < nt; ++t) a.tiles[start + t] = TileInfo{e, off + t * TMG, off + n, 8 * (start + t)};
      for (int t = 0; t < nt3; ++t)
        a.tiles3[start3 + t] = TileInfo{e, off + t * TML, off + n, 8 * start + t * (TML / 32)};
    }
    carry += __shfl(x, 63, 64);
    carry3 += __shfl(x3, 63, 64);
  }
  if (lane == 0) {
    a.ntiles[0] = carry;
    a.ntiles[1] = carry3;
    *a.status = 0;  // raised again by this forward's kernels only
  }
}

// Saved copy of the layer input for the backward (which is not given x):
// a plain 16-byte-per-lane copy, T x H bf16.
__global__ __launch_bounds__(256) void k_save_x(LayerArgs a) {
  const long n = (long)a.T * a.H / 8;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) ((u32x4*)a.Xs)[i] = ((const u32x4*)a.x)[i];
}

hipError_t launch_tile_map(const LayerArgs& a, hipStream_t st) {
  MOE_LAUNCH(k_tile_map, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_save_x(const LayerArgs& a, hipStream_t st) {
  const long n = (long)a.T * a.H / 8;  // H % 256 == 0
  MOE_LAUNCH(k_save_x, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moelora
