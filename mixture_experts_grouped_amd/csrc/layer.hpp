// layer.hpp -- arguments shared by every kernel of one layer call, and the
// launchers the C ABI calls.  Internal to libmoelora.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "engine.hpp"

namespace moelora {

constexpr int TMG = 256;  // M tile of the grouped GEMMs (rows of one expert)
// M tile of the large W13 tile (384 x 256: the whole 160 KB of LDS for two
// stages, a third fewer operand bytes per product than 256 x 256)
constexpr int TML = 384;
// The XCD-aware tile order of the base GEMMs (group_tile): each pool group's
// M tiles, in chunks of at most TILE_GM, with all N tiles of a chunk, the
// M index running fastest.  Concurrent workgroups on one XCD then share one
// expert's weight panel in its L2.  Same box at the production share (an
// expert = six 256-row tiles): chunks of one whole expert against fixed
// groups of four M tiles, k_w13dgrad 2.91 -> 2.72 ms, k_w2 1.47 -> 1.41 ms;
// fixed groups of twelve (two experts) 3.00 ms for k_w13dgrad.
constexpr int TILE_GM = 8;
constexpr int MAX_ADAPTERS = 64;  // adapters of one multi-adapter pass
constexpr int KSPLIT = 4;  // fixed K split of the long-K token GEMMs (ZA = A x, q = B2^T go)
// Kernels whose output tile spans the rank (ZA, Z2, q, P and the adapter
// gradients) cover it in blocks of RBLK columns, one block per workgroup.
constexpr int RBLK = 128;
__host__ __device__ inline int rank_blocks(int r) { return (r + RBLK - 1) / RBLK; }

// Accumulator-blocked layout of a [tiles x 256, I] tensor (fp16 here) that is
// written and read only by kernels holding it in 32 x 32 MFMA accumulator
// blocks: block (M tile mt, row block rb of 8, column block cb of I/32) is
// 1024 elements, ordered [g (4)][lane (64)][q (4)] so that the lane's
// accumulator values 4g .. 4g + 3 are one access (8 bytes in fp16) and a
// wave's access is contiguous (512 bytes).  Row block index rbi = 8 mt + rb.
__device__ __forceinline__ long acc_blk(int rbi, int cb, int I) { return ((long)rbi * (I / 32) + cb) * 1024; }
__device__ __forceinline__ long acc_block(int mt, int rb, int cb, int I) { return acc_blk(mt * 8 + rb, cb, I); }

// Everything a kernel may touch, passed by value as the kernel argument.
// Pool-shaped tensors have `cap` rows; token-shaped tensors have T rows.
// bf16 tensors are uint16 bit patterns.  "_hl" tensors hold an fp32 quantity
// as two bf16 terms: [hi (r) | lo (r)] per rank-r factor.
struct LayerArgs {
  int T, H, I, E, k, r;
  float s;
  long cap;
  int maxtiles, maxtiles3;
  // adapters (multi-adapter pass, OpenPipe/ART PR #1139, Behavior): na roots
  // of tokens, root q = tokens roots[q] .. roots[q+1]-1, each with its own
  // factors.  The pool groups rows by (expert e, adapter q) as group
  // g = e * na + q (EV = E * na groups; na = 1: g = e).  Shared factors are
  // stacked [na, ...], expert-local ones [na, E, ...].
  int na, EV;
  int roots[MAX_ADAPTERS + 1];
  // few rows per pool group (bf16 base): the base GEMMs take 64-row parts of
  // each pool tile (bitwise the same results as full tiles)
  int small_tiles;
  // many rows per pool group (bf16 base): the W13 GEMM takes TML-row tiles
  int large_tiles;
  // at most half as many routes as pool groups: the P product takes k_p13s
  int few_routes;
  // pool
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* r2row;  // route -> pool row
  const int32_t* row2r;  // pool row -> route
  // inputs
  const uint16_t* x;
  const float* w;
  const uint16_t* go;
  // parameters
  const uint16_t *W13, *W2, *A1, *A3, *B1, *B3, *A2, *B2;
  // MXFP4 base (mx != 0): packed e2m1 W13 [E, 2I, H/2], W2 [E, H, I/2] and
  // their e8m0 scales [E, 2I, H/32], [E, H, I/32]
  int mx;
  int act;          // MOE_ACT_SWIGLU or MOE_ACT_GEGLU
  float clamp;      // activation clamp c > 0 (pre-activations clipped to [-c, c]); 0 = off
  const uint8_t *W13q, *W13s, *W2q, *W2s;
  // transformed bf16 base weights (optional, nullptr = read W13 / W2
  // directly), packed stage tiles (pack.hip): W13T = W13_e^T and W2T = W2_e^T
  // for the data gradients; W13P, W2P = W13_e, W2_e for the forward (bf16 base)
  const uint16_t *W13T, *W2T, *W13P, *W2P;
  // saved by the forward
  int* status;       // [1] status word at offset 0 of saved (MOE_SAVED_* bits)
  TileInfo* tiles;   // [maxtiles]   M tiles of TMG rows (pad: 8 x the tile's index)
  int* ntiles;       // [2]          live tiles of `tiles`, then of `tiles3`
  TileInfo* tiles3;  // [maxtiles3]  M tiles of TML rows (pad: the row block index of row0)
  uint16_t* Xs;      // [T, H]    copy of x for the backward (the W13 GEMM gathers x rows itself)
  uint16_t* ZA;      // [T, 4r]   s*A1 x, s*A3 x as hi/lo
  _Float16* G;       // gate pre-activation, fp16, accumulator-blocked (acc_block)
  _Float16* V;       // up pre-activation, same layout
  uint16_t* Hh;      // [cap, I]  silu(G) * V
  float* Z2;         // [cap, r]  s * A2_e h (scratch, forward only)
  // MXFP4 base, forward scratch: the two-term E2M3 split of the base GEMMs'
  // activations (engine_mx.hpp): codes [rows, 2K bytes], scale words [rows, K/64]
  uint8_t* XQ;       // x:  [T, 2H bytes]
  uint32_t* XS;      //     [T, H/64]
  uint8_t* HQ;       // h:  [cap, 2I bytes]
  uint32_t* HS;      //     [cap, I/64]
  uint16_t* Yb;      // [cap, H]  W2_e h, unweighted base output (scratch, forward only)
  uint16_t* zc;      // [T, 2r]   sum_j w Z2 as hi/lo
  float* zsp;        // [KSPLIT, T, 2r] partials of A1 x | A3 x (forward scratch)
  // forward output
  uint16_t* out;     // [T, H]
  // backward scratch
  float* q;          // [T, r]    B2^T grad_out
  float* qp;         // [KSPLIT, T, r] its partials over the quarters of H
  uint16_t* sq;      // [T, 2r]   s*q as hi/lo
  uint16_t* wsq;     // [cap, 2r] s*w*q per route as hi/lo
  uint16_t* dGV;     // [cap, 2I] dgate | dup
  uint16_t* dU;      // [cap, H]  W13_e^T [dg; dv]
  float* P;          // [cap, 2r] B1_e^T dg | B3_e^T dv
  uint16_t* pc;      // [T, 4r]   s * sum_j P as hi/lo (pc1 | pc3)
  float* part;       // [3, nsplit, H*r] split-K partials of the shared-factor gradients
                     // (chunks of kspl tokens, per root: token_tile(.., kspl, ..))
  uint16_t* ZAp;     // [cap, 4r] ZA gathered to pool rows (real rows only)
  float* dwp;        // [I/256, cap] router-gradient partials of the W2 dgrad's column tiles
  uint16_t* A2T;     // [na, E, I, r]  A2_e^T (backward scratch, with W2T only)
  uint16_t *A1T, *A3T;  // [na, H, r]  A1^T, A3^T (backward scratch)
  uint16_t *B1T, *B3T;  // [na, E, r, I]  B1_e^T, B3_e^T of the groups with rows (few_routes only)
  int nsplit, kspl;
  // backward outputs
  uint16_t* gx;
  float* gw;
  uint16_t *dA1, *dA3, *dB1, *dB3, *dA2, *dB2, *dW13, *dW2;
};

// Workgroup b of a grid over (at most) maxtiles x nn tiles of the tile list
// `tiles` (M tiles of TM rows, ordered by pool group), of which the first ntm
// are live: false for a dead workgroup; else its tile (mt, nt).  The live
// tiles are dealt so that each XCD owns a contiguous range of a logical
// order (xcd_remap) in which each group's M tiles come in chunks of at most
// gm, all N tiles of a chunk together, M fastest.  A chunk [cs, cs + sz)
// occupies logical indices [cs nn, (cs + sz) nn), so logical index L lies in
// the chunk of M tile L / nn.  (Wave-uniform: b is a block index.)
__device__ __forceinline__ bool group_tile(const LayerArgs& a, const TileInfo* tiles, int TM, int b, int ntm,
                                           int nn, int gm, int& mt, int& nt) {
  const int n = ntm * nn;
  if (b >= n) return false;
  const int L = xcd_remap(b, n);
  const int v = L / nn;
  const TileInfo tv = tiles[v];
  const int s = v - (tv.row0 - a.offsets[tv.e]) / TM;  // the group's first M tile
  const int cnt = (a.counts[tv.e] + TM - 1) / TM;      // and its number of M tiles
  const int cs = s + gm * ((v - s) / gm);
  const int sz = s + cnt - cs < gm ? s + cnt - cs : gm;
  const int r = L - cs * nn;
  mt = cs + r % sz;
  nt = r / sz;
  return true;
}

// Grids of nsub sub-tiles per M tile along x (at most maxtiles M tiles) and
// column blocks along y, whose workgroups of one pool group all read that
// group's rank-r factor slice: the live workgroups (the first ntiles x nsub
// x gridDim.y in dispatch order, x fastest) are dealt so that each XCD owns a
// contiguous range of the order (y, M tile, sub-tile), so one group's slice
// is fetched from HBM by about one XCD instead of by all eight.  False for a
// dead workgroup.  (Wave-uniform.)
__device__ __forceinline__ bool sub_tile(const LayerArgs& a, int nsub, int& mt, int& sub, int& y) {
  const int nx = *a.ntiles * nsub, n = nx * (int)gridDim.y;
  const int b = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  if (b >= n) return false;
  const int L = xcd_remap(b, n);
  y = L / nx;
  const int x = L - y * nx;
  mt = x / nsub;
  sub = x - mt * nsub;
  return true;
}

// Pool group g -> its expert (base weights), its adapter, and the index
// q * E + e of its expert-local factors in their [na, E, ...] stacks.
__device__ __forceinline__ int grp_expert(const LayerArgs& a, int g) { return a.na == 1 ? g : g / a.na; }
__device__ __forceinline__ int grp_adapter(const LayerArgs& a, int g) { return a.na == 1 ? 0 : g % a.na; }
__device__ __forceinline__ long grp_local(const LayerArgs& a, int g) {
  return a.na == 1 ? g : (long)(g % a.na) * a.E + g / a.na;
}

// Token tile b of TM tokens: tiles never cross roots, so every tile has one
// adapter.  Tiles of root q follow those of roots < q.  Returns false past
// the last tile.  (Wave-uniform: b is a block index.)
__device__ __forceinline__ bool token_tile(const LayerArgs& a, int b, int TM, int& t0, int& nt, int& ad) {
  if (a.na == 1) {
    t0 = b * TM;
    nt = a.T - t0 < TM ? a.T - t0 : TM;
    ad = 0;
    return nt > 0;
  }
  for (int q = 0; q < a.na; ++q) {
    const int r0 = a.roots[q], r1 = a.roots[q + 1];
    const int n = (r1 - r0 + TM - 1) / TM;
    if (b < n) {
      t0 = r0 + b * TM;
      nt = r1 - t0 < TM ? r1 - t0 : TM;
      ad = q;
      return true;
    }
    b -= n;
  }
  return false;
}
// Host side: the number of such tiles.
inline int token_tiles(const LayerArgs& a, int TM) {
  int n = 0;
  for (int q = 0; q < a.na; ++q) n += (a.roots[q + 1] - a.roots[q] + TM - 1) / TM;
  return n;
}

// The first error of a run of kernel-attribute calls.
struct AttrInit {
  hipError_t err = hipSuccess;
  void lds(const void* fn, int bytes) {
    if (err == hipSuccess) err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  }
};

// Kernel attributes are per device: run `init` (returning hipError_t) once
// on each device the library is called on; concurrent first calls wait for
// it.  A failed init is retried on the next call.
class PerDeviceOnce {
 public:
  template <class F>
  hipError_t run(F&& init) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu_);
    const bool tracked = dev >= 0 && dev < 64;
    if (tracked && ((done_ >> dev) & 1u)) return hipSuccess;
    e = init();
    if (e == hipSuccess && tracked) done_ |= 1ull << dev;
    return e;
  }

 private:
  std::mutex mu_;
  uint64_t done_ = 0;  // bit d: device d initialised
};

// The independent branches of one layer call run on a second stream of the
// device (non-blocking, default priority), ordered against the caller's
// stream by events: open() makes the branch wait for the caller's stream so
// far, signal / await order the two at the call's branch points (events
// 1 .. NEV-1), close() makes the caller's stream wait for all of the branch,
// so the call's work is complete in the caller's stream order as before.
// One call at a time holds a device's branch (a host lock from open to
// close; the destructor closes an open branch).  While the caller's stream
// is being captured into a graph, when `allow` is false, or if the stream
// cannot be made, the branch is the caller's stream itself and signal /
// await do nothing.
class Branch {
 public:
  static constexpr int NEV = 4;
  hipError_t open(hipStream_t st, bool allow);
  hipStream_t side() const { return side_; }
  hipError_t signal(hipStream_t from, int i);
  hipError_t await(hipStream_t to, int i);
  hipError_t close();
  ~Branch() { (void)close(); }

 private:
  hipStream_t main_ = nullptr, side_ = nullptr;
  hipEvent_t* ev_ = nullptr;  // the device's events; nullptr: one stream
  std::unique_lock<std::mutex> lk_;
};

// Roots of a multi-adapter pool build (na = 1: every route's group is its expert).
struct PoolRoots {
  int na, k;
  int roots[MAX_ADAPTERS + 1];
};
hipError_t launch_build_pool(const int32_t* idx, int nroutes, int E, int bm, long cap,
                             int32_t* counts, int32_t* offsets, int32_t* r2row, int32_t* row2r,
                             int32_t* err, const PoolRoots& pr, hipStream_t st);
// branch = false: every kernel on st (the allocation-free entry)
hipError_t launch_forward(const LayerArgs& a, hipStream_t st, bool branch = true);
// two-term E2M3 split of bf16 rows [rows, K] (engine_mx.hpp storage)
hipError_t launch_split_rows(const uint16_t* src, long rows, int K, uint8_t* codes, uint32_t* scales,
                             hipStream_t st);
// [B, R, C] -> [B, C, R] bf16 bits
hipError_t launch_transpose(const uint16_t* src, uint16_t* dst, int B, int R, int C, hipStream_t st,
                            const int32_t* counts = nullptr, int na = 1, int E = 0,
                            const uint16_t* src2 = nullptr, uint16_t* dst2 = nullptr);
hipError_t launch_backward(const LayerArgs& a, hipStream_t st);
// [nb, rs, cs] -> [nb, rd, cd] bf16, zero outside the source (pack.hip)
hipError_t launch_pad(const uint16_t* src, uint16_t* dst, long nb, int rs, int cs, int rd, int cd, hipStream_t st);
// bytes of one stage tile of an MXFP4 packed copy (kinds 4, 5 in pack.hip):
// 256 rows x 32 code bytes, then 256 scale words
constexpr int MX_TILE = 256 * 32 + 256 * 4;
// packed stage tiles of the base (kinds in pack.hip)
hipError_t launch_pack(int kind, const uint16_t* src, const uint8_t* q4, const uint8_t* sc, uint16_t* dst, int E,
                       int H, int I, hipStream_t st);

}  // namespace moelora
