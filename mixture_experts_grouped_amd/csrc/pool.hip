// pool.hip -- dispatch pool builder, the grouped-GEMM tile map and the saved
// copy of the layer input.
//
// The pool is expert-contiguous and padded per expert to BLOCK_M rows, each
// expert starting at its true offset (DeepGEMM PR #9, "2026-09-21: restore
// wide-K wgrad safely" -> Implementation); padding rows of the gathered input
// are zero (PR #9, "Historical implementation" -> Summary).  Rows inside an
// expert follow ascending route index t*k + j, so the pool is a deterministic
// function of the routing (the pages' atomic dispatch order is not).
#include "layer.hpp"
#include "trace.hpp"

namespace moelora {

constexpr int POOL_THREADS = 1024;
constexpr int POOL_WAVES = POOL_THREADS / 64;

// One workgroup builds the whole pool: an LDS histogram, a wave scan of the
// padded counts, then the routes in chunks of 1024.  Inside a chunk every wave
// ranks its lanes among equal expert ids with ballots over the id bits; the
// per-wave counts are scanned per expert, giving each route its row in
// ascending route order.  Integer-only and deterministic.
__global__ __launch_bounds__(POOL_THREADS) void k_build_pool(
    const int32_t* __restrict__ idx, int nroutes, int E, int bm, long cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ r2row,
    int32_t* __restrict__ row2r, int32_t* __restrict__ err) {
  extern __shared__ int sm[];
  int* cnt = sm;                   // [E]   counts, later the running row of each expert
  int* base = sm + E;              // [E+1] padded offsets
  int* wcnt = sm + 2 * E + 1;      // [POOL_WAVES][E]
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += POOL_THREADS) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int f = tid; f < nroutes; f += POOL_THREADS) {
    const int e = idx[f];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else if (e != -1)
      atomicAdd(&bad, 1);
  }
  __syncthreads();
  if (wv == 0) {
    int carry = 0;
    for (int b0 = 0; b0 < E; b0 += 64) {
      const int e = b0 + lane;
      const int v = (e < E) ? ((cnt[e] + bm - 1) / bm) * bm : 0;
      int x = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (e < E) base[e] = carry + x - v;
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) base[E] = carry;
  }
  __syncthreads();
  for (int e = tid; e < E; e += POOL_THREADS) {
    counts[e] = cnt[e];
    offsets[e] = base[e];
    for (int p = base[e] + cnt[e]; p < base[e + 1]; ++p) row2r[p] = -1;  // padding rows
  }
  if (tid == 0) {
    offsets[E] = base[E];
    if (err != nullptr) *err = bad;
  }
  for (long p = base[E] + tid; p < cap; p += POOL_THREADS) row2r[p] = -1;  // unused suffix
  __syncthreads();
  for (int e = tid; e < E; e += POOL_THREADS) cnt[e] = base[e];
  int nbits = 1;
  while ((1 << nbits) <= E) ++nbits;  // ids 0..E (E = "no expert") fit in nbits
  for (int c0 = 0; c0 < nroutes; c0 += POOL_THREADS) {
    for (int i = tid; i < POOL_WAVES * E; i += POOL_THREADS) wcnt[i] = 0;
    __syncthreads();
    const int f = c0 + tid;
    const int e = (f < nroutes) ? idx[f] : -1;
    const bool ok = (e >= 0 && e < E);
    const int key = ok ? e : E;
    unsigned long long same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const unsigned long long m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    const int nsame = __popcll(same);
    if (ok && rank == nsame - 1) wcnt[wv * E + e] = nsame;
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += POOL_THREADS) {
      int run = cnt[e2];
      for (int w2 = 0; w2 < POOL_WAVES; ++w2) {
        const int c = wcnt[w2 * E + e2];
        wcnt[w2 * E + e2] = run;
        run += c;
      }
      cnt[e2] = run;
    }
    __syncthreads();
    if (ok) {
      const int row = wcnt[wv * E + e] + rank;
      r2row[f] = row;
      row2r[row] = f;
    } else if (f < nroutes) {
      r2row[f] = -1;
    }
    __syncthreads();
  }
}

hipError_t launch_build_pool(const int32_t* idx, int nroutes, int E, int bm, long cap,
                             int32_t* counts, int32_t* offsets, int32_t* r2row, int32_t* row2r,
                             int32_t* err, hipStream_t st) {
  const size_t lds = sizeof(int) * (size_t)(2 * E + 1 + POOL_WAVES * E);
  MOE_LAUNCH(k_build_pool, dim3(1), dim3(POOL_THREADS), lds, st, idx, nroutes, E, bm, cap,
                     counts, offsets, r2row, row2r, err);
  return hipGetLastError();
}

// Grouped-GEMM M tiles: TMG rows of one expert each, never crossing experts.
__global__ __launch_bounds__(64) void k_tile_map(LayerArgs a) {
  const int lane = threadIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < a.E; b0 += 64) {
    const int e = b0 + lane;
    const int n = (e < a.E) ? a.counts[e] : 0;
    const int nt = (n + TMG - 1) / TMG;
    int x = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const int start = carry + x - nt;
    if (e < a.E) {
      const int off = a.offsets[e];
      for (int t = 0; t < nt; ++t) a.tiles[start + t] = TileInfo{e, off + t * TMG, off + n, 0};
    }
    carry += __shfl(x, 63, 64);
  }
  if (lane == 0) *a.ntiles = carry;
}

// Saved copy of the layer input for the backward (which is not given x):
// a plain 16-byte-per-lane copy, T x H bf16.
__global__ __launch_bounds__(256) void k_save_x(LayerArgs a) {
  const long n = (long)a.T * a.H / 8;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) ((u32x4*)a.Xs)[i] = ((const u32x4*)a.x)[i];
}

hipError_t launch_pool_prologue(const LayerArgs& a, hipStream_t st) {
  MOE_LAUNCH(k_tile_map, dim3(1), dim3(64), 0, st, a);
  const long n = (long)a.T * a.H / 8;  // H % 256 == 0
  MOE_LAUNCH(k_save_x, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moelora
