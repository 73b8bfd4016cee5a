// engine2.hpp -- bf16 MFMA tile engine for gfx950 with direct-to-LDS loads.
//
// Same tile geometry and accumulator layout as engine.hpp (256 threads, four
// wave64s, v_mfma_f32_32x32x16_bf16, lanes own output rows, four consecutive
// output columns per register group), but the operands travel from global
// memory straight into LDS with `buffer_load_dwordx4 ... lds`: no staging
// registers, no LDS write instructions.  A stage is KT = 32 or 64 k deep;
// NBUF = 4 or 2 stages live in LDS (NBUF - 1 stages of loads in flight while
// one is multiplied).  The barrier between stages carries no memory fence:
// each wave first waits (vmcnt) for its own loads of the stage it is about to
// read, so prefetched stages stay in flight across the barrier.
//
// A wave's direct load writes 64 lanes x 16 bytes = 1 KB contiguous at a
// wave-uniform LDS address (lane L at +16 L); an out-of-range buffer offset
// writes zeros.  Tiles are therefore laid out so that every 1 KB is a run of
// whole rows, and each lane picks the global chunk that its slot must hold.
//
// Two tile layouts:
//   K tile  [rows][KT k], 2 KT bytes per row, 16-byte chunk c of row r stored
//           in slot c ^ f(r): for KT = 32, f(r) = ((r>>1 ^ r>>3) & 1) |
//           ((r>>2 & 1) << 1); for KT = 64, f(r) = (r ^ r>>3) & 7.  Fragment
//           reads (ds_read_b128, 32 rows x 8 k per lane group) hit distinct
//           banks under both 8-lane and 16-lane service.
//   T tile  [KT k][cols] (K-outer source), pitch 2*cols bytes, chunk j of
//           row k in slot j ^ 2(k & 3); fragments come from two
//           ds_read_b64_tr_b16 per lane: inside every 16-lane group lane i
//           receives element (i & 3) of the 8-byte reads of lanes
//           4q + (i >> 2), q = 0..3 (probed on the device), which turns four
//           k-rows of 16 columns into four consecutive k of one column.
#pragma once
#include <type_traits>

#include "engine.hpp"

namespace moelora {
namespace v2 {

template <int KT>
struct Depth {
  static_assert(KT == 32 || KT == 64, "stage depth");
  static constexpr int NBUF = (KT == 32) ? 4 : 2;
  static constexpr int KROW = 2 * KT;     // bytes per K-tile row
  static constexpr int CPR = KT / 8;      // 16-byte chunks per K-tile row
  static constexpr int RPI = 64 / CPR;    // K-tile rows per 1 KB wave instruction
  static constexpr int KSTEPS = KT / 16;  // MFMA k16 steps per stage
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int KT>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (KT == 32)
    return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
  else
    return (r ^ (r >> 3)) & 7;
}
template <int KT>
__device__ __forceinline__ int koff(int r, int c) {
  return r * Depth<KT>::KROW + ((c ^ kswz<KT>(r)) << 4);
}
// T tiles: 16-byte chunk j of k-row k sits in slot j ^ tswz(k).  A transposed
// fragment read touches chunks c .. c + 3 of k-rows k0 .. k0 + 3 and
// k0 + 8 .. k0 + 11; shifting by 4 chunks per k-row spreads the four rows of
// each half over all sixteen 16-byte bank groups (rows at least 16 chunks wide).
__device__ __forceinline__ int tswz(int k) { return (k & 3) << 2; }
__device__ __forceinline__ int toff(int k, int j, int pitch) {
  return k * pitch + ((j ^ tswz(k)) << 4);
}

__device__ __forceinline__ void lds_load16(rsrc_t rs, char* lds_wave_base, uint32_t off,
                                           uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_wave_base, 16, off, soff, 0, 0);
}

// ---------------------------------------------------------------------------
// geometry
// ---------------------------------------------------------------------------
// NBUF_: stage buffers (0 = the depth's default); NBUF - 1 stages are queued
// ahead of the one being multiplied.
template <int MB_, int NB_, int WM_, int WN_, bool MTR_ = false, bool NTR_ = false, int KT_ = 64, int NBUF_ = 0>
struct Geo2 {
  static constexpr int MB = MB_, NB = NB_, WM = WM_, WN = WN_, KT = KT_;
  static constexpr int NW = WM * WN, NT = 64 * NW;  // waves and threads per workgroup
  static constexpr int NBUF = NBUF_ > 0 ? NBUF_ : Depth<KT>::NBUF;
  static_assert(NBUF >= 2 && NBUF <= 4, "stage buffers");
  static constexpr bool MTR = MTR_, NTR = NTR_;  // operand tile stored K-outer (T tile)
  static constexpr int TM = WM * MB * 32, TN = WN * NB * 32;
  static constexpr int SM_BYTES = TM * 2 * KT, SN_BYTES = TN * 2 * KT;  // same for both layouts
  static constexpr int STAGE = SM_BYTES + SN_BYTES;
  static constexpr int LDS_BYTES = NBUF * STAGE;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NB % 2 == 0, "N blocks come in pairs");
  __device__ static constexpr int m_local(int wm, int mb) { return (wm * MB + mb) * 32; }
  __device__ static constexpr int n_local(int wn, int nb) {
    return (nb < NB / 2 ? 0 : TN / 2) + (wn * (NB / 2) + (nb % (NB / 2))) * 32;
  }
};

// MFMA operand for 32 rows/columns starting at `base` and k16 step kk.
template <bool TR, int COLS, int KT>
__device__ __forceinline__ bf16x8 frag(const char* tile, int base, int kk, int lane) {
  if constexpr (!TR) {
    const int r = base + (lane & 31);
    return *(const bf16x8*)(tile + koff<KT>(r, 2 * kk + (lane >> 5)));
  } else {
    constexpr int P = COLS * 2;
    const int g = lane >> 4, i = lane & 15;
    const int n = base + 16 * (g & 1) + 4 * (i & 3);
    const int kb = 16 * kk + 8 * (g >> 1) + (i >> 2);
    s16x4 v0, v1;
    {
      const int k = kb;
      v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + toff(k, n >> 3, P) + (n & 7) * 2));
    }
    {
      const int k = kb + 4;
      v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tile + toff(k, n >> 3, P) + (n & 7) * 2));
    }
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 w = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    return __builtin_bit_cast(bf16x8, w);
  }
}

template <class G, bool SPLIT>
__device__ __forceinline__ void load_frags2(const char* sM, const char* sN, bf16x8 (&a)[G::NB],
                                            bf16x8 (&b)[G::MB], int kk, int wm, int wn, int lane) {
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
    b[mb] = frag<G::MTR, G::TM, G::KT>(sM, G::m_local(wm, mb), kk, lane);
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    if (SPLIT && ((nb < G::NB / 2) != (kk < G::KT / 32))) continue;
    a[nb] = frag<G::NTR, G::TN, G::KT>(sN, G::n_local(wn, nb), kk, lane);
  }
}

// KT/16 k16 steps; fragments of step kk + 1 are read while step kk
// multiplies.  SPLIT: the first half of the N tile contracts only the first
// half of the stage's k, the second half only the second (two K ranges in one
// stage).
template <class G, bool SPLIT>
__device__ __forceinline__ void mma_stage2(const char* sM, const char* sN,
                                           f32x16 (&acc)[G::NB][G::MB], int wm, int wn, int lane) {
  constexpr int KS = G::KT / 16;
  bf16x8 a[2][G::NB], b[2][G::MB];
  load_frags2<G, SPLIT>(sM, sN, a[0], b[0], 0, wm, wn, lane);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < KS) load_frags2<G, SPLIT>(sM, sN, a[cur ^ 1], b[cur ^ 1], kk + 1, wm, wn, lane);
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
      if (SPLIT && ((nb < G::NB / 2) != (kk < KS / 2))) continue;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
        acc[nb][mb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][nb], b[cur][mb], acc[nb][mb], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// loaders.  `issue(stage, tile)` queues this thread's direct loads of one
// stage into `tile` (the operand's LDS tile of that stage).
// ---------------------------------------------------------------------------

// K tile of R rows (K-contiguous source).  Wave w's instruction j covers tile
// rows RPI (w + 4j) .. +RPI-1; lane L holds row RPI (w + 4j) + L/CPR, slot
// L % CPR.  Row window and folding as in RowsK.  SPLIT stages are KT/2 k per
// half: chunks c < CPR/2 read k = k0 + 8c, the others khalf + k0 + 8(c - CPR/2).
template <int R, int KT = 64, int NW = 4, bool TWO = false>
struct KLoad {
  static constexpr int CPR = Depth<KT>::CPR, RPI = Depth<KT>::RPI;
  static constexpr int NJ = R / (NW * RPI);
  static_assert(NJ >= 1 && NJ * NW * RPI == R, "tile rows per stage");
  static_assert(!TWO || NJ % 2 == 0, "two descriptors split the tile rows in halves");
  rsrc_t rs, rs2;  // with TWO, rs2 serves tile rows >= R/2 (a second source tensor)
  uint32_t roff[NJ];
  int span, period, lo_split, lo_b;

  __device__ static __forceinline__ int row_of(int j) {
    return RPI * ((threadIdx.x >> 6) + NW * j) + (threadIdx.x & 63) / CPR;
  }
  __device__ __forceinline__ void window(int span_, int period_ = 0, int lo_split_ = 1 << 30,
                                         int lo_b_ = 0) {
    span = span_;
    period = period_;
    lo_split = lo_split_;
    lo_b = lo_b_;
  }
  __device__ __forceinline__ void contig(const uint16_t* base, long row0, long nvalid, long ld) {
    rs = make_rsrc(base + row0 * ld, (uint64_t)(nvalid > 0 ? nvalid : 0) * ld * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      roff[j] = (row_of(j) < nvalid) ? (uint32_t)(row_of(j) * ld * 2) : OFF_NONE;
  }
  __device__ static __forceinline__ void tokens(int (&tk)[NJ], const int32_t* row2r, int topk,
                                                long row0, long nvalid) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) tk[j] = (row_of(j) < nvalid) ? row2r[row0 + row_of(j)] / topk : -1;
  }
  __device__ __forceinline__ void from_tokens(const uint16_t* base, long ntok, long ld,
                                              const int (&tk)[NJ]) {
    rs = make_rsrc(base, (uint64_t)ntok * ld * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) roff[j] = (tk[j] >= 0) ? (uint32_t)((long)tk[j] * ld * 2) : OFF_NONE;
  }
  __device__ __forceinline__ void issue(int k0, int khalf, bool split, char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases in SGPRs
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = row_of(j);
      const int c = (threadIdx.x % CPR) ^ kswz<KT>(r);
      const int kc = split ? ((c < CPR / 2) ? k0 + 8 * c : khalf + k0 + 8 * (c - CPR / 2))
                           : k0 + 8 * c;
      const int k = kc - (r >= lo_split ? lo_b : 0);
      const int kk = (period != 0 && k >= period) ? k - period : k;
      const bool ok = (k >= 0) && (k < span) && (roff[j] != OFF_NONE);
      lds_load16((TWO && 2 * j >= NJ) ? rs2 : rs, tile + 1024 * (w + NW * j),
                 ok ? roff[j] + 2u * (uint32_t)kk : OFF_NONE);
    }
  }
};

// K tile loader for a K range made of whole stages (every stage reads k0 ..
// k0 + KT - 1 of each row, all in range): each lane's byte offset is fixed
// at set-up and the stage's k0 travels in the scalar offset, so an issue
// costs no vector arithmetic.  A row outside the range has offset OFF_NONE,
// which stays beyond the descriptor's size whatever the scalar offset adds.
template <int R, int KT = 64, int NW = 4>
struct KLoadA {
  static constexpr int CPR = Depth<KT>::CPR, RPI = Depth<KT>::RPI;
  static constexpr int NJ = R / (NW * RPI);
  static_assert(NJ >= 1 && NJ * NW * RPI == R, "tile rows per stage");
  rsrc_t rs;
  uint32_t voff[NJ];

  __device__ static __forceinline__ int row_of(int j) { return KLoad<R, KT, NW>::row_of(j); }
  __device__ static __forceinline__ uint32_t chunk(int j) {
    return 16u * (uint32_t)((threadIdx.x % CPR) ^ kswz<KT>(row_of(j)));
  }
  // rows row0 .. row0 + nvalid - 1 of a row-major matrix with ld elements a row
  __device__ __forceinline__ void contig(const uint16_t* base, long row0, long nvalid, long ld) {
    rs = make_rsrc(base + row0 * ld, (uint64_t)(nvalid > 0 ? nvalid : 0) * ld * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      voff[j] = (row_of(j) < nvalid) ? (uint32_t)(row_of(j) * ld * 2) + chunk(j) : OFF_NONE;
  }
  // tile row j of this lane reads the row at byte offset roff (OFF_NONE: zeros)
  __device__ __forceinline__ void set_row(int j, uint32_t roff) {
    voff[j] = (roff != OFF_NONE) ? roff + chunk(j) : OFF_NONE;
  }
  // tile row j reads token tk[j]'s row of a [ntok, ld] matrix (tk < 0: zeros)
  __device__ __forceinline__ void from_tokens(const uint16_t* base, long ntok, long ld,
                                              const int (&tk)[NJ]) {
    rs = make_rsrc(base, (uint64_t)ntok * ld * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j) set_row(j, (tk[j] >= 0) ? (uint32_t)((long)tk[j] * ld * 2) : OFF_NONE);
  }
  __device__ __forceinline__ void issue(int k0, char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases in SGPRs
#pragma unroll
    for (int j = 0; j < NJ; ++j) lds_load16(rs, tile + 1024 * (w + NW * j), voff[j], 2u * (uint32_t)k0);
  }
};

// T tile of R columns x KT k (K-outer source).  1 KB holds 512/R k-rows;
// wave w's instruction j covers k-rows RPI (w + 4j) .. +RPI-1 with
// RPI = 512 / R; lane L holds k-row RPI (w + 4j) + L / (R/8), slot L % (R/8).
// Column mapping as in TransK (window, hi/lo halves).
template <int R, class KP, int KT = 64, int NW = 4>
struct TLoad {
  static constexpr int CPR = R / 8;           // 16-byte chunks per k-row
  static_assert(CPR >= 16, "the chunk swizzle needs 16 chunks per k-row");
  static constexpr int RPI = 64 / CPR;        // k-rows per wave instruction
  static constexpr int NJ = KT / (NW * RPI);  // instructions per wave per stage
  static_assert(NJ >= 1 && NJ * NW * RPI == KT, "k-rows per stage");
  KP kp;
  int n0, nvalid, hilo_half, lo_off;

  __device__ __forceinline__ void cols(int n0_, int nvalid_, int hilo_half_ = 0, int lo_off_ = 0) {
    n0 = n0_;
    nvalid = nvalid_;
    hilo_half = hilo_half_;
    lo_off = lo_off_;
  }
  __device__ __forceinline__ uint32_t col_off(int nl) const {
    int n = nl, extra = 0;
    if (hilo_half > 0 && nl >= hilo_half) {
      n = nl - hilo_half;
      extra = lo_off;
    }
    return (n < nvalid) ? 2u * (uint32_t)(n0 + extra + n) : OFF_NONE;
  }
  __device__ __forceinline__ void issue(int k0, char* tile) const {
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kr = RPI * (w + NW * j) + L / CPR;
      const int jc = (L % CPR) ^ tswz(kr);
      kp.issue_lds(k0 + kr, col_off(8 * jc), tile + 1024 * (w + NW * j));
    }
  }
};

// KLoadA for R consecutive rows of a row-major matrix: tile row j of a lane
// is its row 0 plus j * RPI * NW rows, so the lane keeps two byte offsets (the
// chunk swizzle alternates with j when NW = 4) and each instruction adds its
// row step in the scalar offset.  Rows past nvalid fall outside the
// descriptor (sized to nvalid rows) and read zero: the range check covers
// the scalar offset too.
template <int R, int KT = 64, int NW = 4>
struct KLoadS {
  static constexpr int CPR = Depth<KT>::CPR, RPI = Depth<KT>::RPI;
  static constexpr int NJ = R / (NW * RPI);
  static_assert(NJ >= 1 && NJ * NW * RPI == R, "tile rows per stage");
  rsrc_t rs;
  uint32_t v0, v1;   // lane offsets for even / odd j
  uint32_t jstep;    // bytes between consecutive j (RPI * NW rows)
  __device__ __forceinline__ void contig(const uint16_t* base, long row0, long nvalid, long ld) {
    rs = make_rsrc(base + row0 * ld, (uint64_t)(nvalid > 0 ? nvalid : 0) * ld * 2);
    const uint32_t ldb = (uint32_t)(ld * 2);
    jstep = (uint32_t)(RPI * NW) * ldb;
    const int r0 = KLoad<R, KT, NW>::row_of(0);
    v0 = (uint32_t)r0 * ldb + KLoadA<R, KT, NW>::chunk(0);
    v1 = (uint32_t)r0 * ldb + (NJ > 1 ? KLoadA<R, KT, NW>::chunk(1) : KLoadA<R, KT, NW>::chunk(0));
  }
  __device__ __forceinline__ void issue(int k0, char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases in SGPRs
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      lds_load16(rs, tile + 1024 * (w + NW * j), (j & 1) ? v1 : v0, 2u * (uint32_t)k0 + (uint32_t)j * jstep);
  }
};

// K tile of R rows x KT k from a packed copy of the matrix (pack.hip): each
// stage tile stored as its LDS image, tiles consecutive per N tile, so a
// stage is R * 2 * KT contiguous bytes and wave instruction j of wave w reads
// the 1 KB that lands at tile + 1024 (w + NW j).  The LDS contents equal
// those of KLoad / KLoadA / KLoadS on the plain matrix.
template <int R, int KT, int NW>
struct KLoadP {
  static constexpr int TILE = R * 2 * KT;  // bytes per stage tile
  static constexpr int NJ = TILE / (1024 * NW);
  static_assert(NJ >= 1 && NJ * NW * 1024 == TILE, "whole wave instructions per stage");
  rsrc_t rs;
  uint32_t lane_off;  // 1024 w + 16 lane
  uint32_t tile0;     // byte offset of the N tile's first stage tile
  // base: the expert's packed matrix (`bytes` long); the N tile `nt` of a
  // matrix with `nst` stages
  __device__ __forceinline__ void set(const void* base, uint64_t bytes, int nt, int nst) {
    rs = make_rsrc(base, bytes);
    lane_off = 1024u * (uint32_t)(threadIdx.x >> 6) + 16u * (uint32_t)(threadIdx.x & 63);
    tile0 = (uint32_t)nt * (uint32_t)nst * (uint32_t)TILE;
  }
  __device__ __forceinline__ void issue(int k0, char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases in SGPRs
    // the stage's offset is workgroup-uniform: keep it in an SGPR (the scalar
    // offset operand), whatever the compiler can prove about tile0
    const uint32_t st = __builtin_amdgcn_readfirstlane(tile0 + (uint32_t)(k0 / KT) * (uint32_t)TILE);
#pragma unroll
    for (int j = 0; j < NJ; ++j) lds_load16(rs, tile + 1024 * (w + NW * j), lane_off, st + 1024u * NW * j);
  }
};

// T tile loader for a K range made of whole stages of a row-major [K, ld]
// matrix, columns n0 .. n0 + R - 1 (all in range): offsets fixed at set-up,
// the stage's first k-row in the scalar offset (as KLoadA).
template <int R, int KT = 64, int NW = 4>
struct TLoadA {
  static constexpr int CPR = R / 8, RPI = 64 / CPR, NJ = KT / (NW * RPI);
  static_assert(NJ >= 1 && NJ * NW * RPI == KT, "k-rows per stage");
  static_assert(CPR >= 16, "the chunk swizzle needs 16 chunks per k-row");
  rsrc_t rs;
  uint32_t ldb;    // bytes per k-row
  uint32_t voff;   // this lane's offset for instruction 0; instruction j adds j RPI NW k-rows
  // (the chunk swizzle depends on k-row mod 4, which j does not change)
  __device__ __forceinline__ void set(const uint16_t* base, long nk, long ld, int n0) {
    rs = make_rsrc(base, (uint64_t)nk * ld * 2);
    ldb = (uint32_t)(ld * 2);
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int kr = RPI * w + L / CPR;
    const int jc = (L % CPR) ^ tswz(kr);
    voff = (uint32_t)kr * ldb + 2u * (uint32_t)(n0 + 8 * jc);
  }
  __device__ __forceinline__ void issue(int k0, char* tile) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: LDS bases in SGPRs
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      lds_load16(rs, tile + 1024 * (w + NW * j), voff, ((uint32_t)k0 + (uint32_t)(j * RPI * NW)) * ldb);
  }
};

// ---------------------------------------------------------------------------
// MXFP4 weights (OCP MX v1.0): e2m1 elements, two per byte with element 2i in
// the low nibble of byte i, and one e8m0 scale per 32 elements along the
// weight's own K axis (the forward contraction axis).  The data-gradient
// GEMMs contract the other axis, so the backward reads the packed bytes into
// registers when a stage is queued and, after the stage before it has been
// multiplied, expands them to bf16 into the T-tile layout the bf16 loaders
// produce (e2m1 x 2^(e-127) is exact in bf16).  The forward runs on the
// scaled matrix cores instead (engine_mx.hpp).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e8m0_value(uint32_t e) {
  // 2^(e-127); e = 0 is the denormal 2^-127
  return __builtin_bit_cast(float, e ? (e << 23) : 0x00400000u);
}
// 8 e2m1 values (one 32-bit word) times sc -> 8 bf16 (one 16-byte chunk)
__device__ __forceinline__ u32x4 fp4x8_bf16(uint32_t w, float sc) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return o;
}
__device__ __forceinline__ uint32_t bload_u8(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0), others untouched
}

// T tile of 256 columns x 64 k-rows from an MXFP4 matrix stored [K rows][N]
// with N the packed axis: thread t takes k-row t/8 and columns 32 (t%8) ..
// +31 (16 bytes and one scale).
template <int NT>
struct TLoadMX {
  static_assert(NT == 512, "eight threads per k-row, 64 k-rows");
  rsrc_t rq, rs;
  uint32_t qoff, soff;   // at stage k-row 0
  uint32_t qld, sld;     // bytes per k-row
  u32x4 q[2];            // two stages (buffer = stage parity)
  uint32_t e[2];
  // columns n0 .. n0 + 255 of a [nk, N] MXFP4 matrix
  __device__ __forceinline__ void set(const uint8_t* q_base, const uint8_t* s_base, long nk, long N, int n0) {
    rq = make_rsrc(q_base, (uint64_t)nk * (N / 2));
    rs = make_rsrc(s_base, (uint64_t)nk * (N / 32));
    qld = (uint32_t)(N / 2);
    sld = (uint32_t)(N / 32);
    const int kr = threadIdx.x >> 3, cg = threadIdx.x & 7;
    qoff = kr * qld + (uint32_t)(n0 / 2) + 16u * cg;
    soff = kr * sld + (uint32_t)(n0 / 32) + cg;
  }
  template <int B = 0>
  __device__ __forceinline__ void issue(int k0) {
    q[B] = bload(rq, qoff + (uint32_t)k0 * qld);
    e[B] = bload_u8(rs, soff + (uint32_t)k0 * sld);
  }
  template <int B = 0>
  __device__ __forceinline__ void finish(char* tile) const {
    const float sc = e8m0_value(e[B]);
    const int kr = threadIdx.x >> 3, cg = threadIdx.x & 7;
#pragma unroll
    for (int c = 0; c < 4; ++c) *(u32x4*)(tile + toff(kr, 4 * cg + c, 512)) = fp4x8_bf16(q[B][c], sc);
  }
};

// k-row policies of TLoad (the K-outer source's row for k)
struct TStrided {  // rows of a matrix: k in [lo, lo + span) -> row (k - lo) folded by period
  rsrc_t rs;
  uint32_t ldb;
  int lo, span, period;
  __device__ __forceinline__ void issue_lds(int k, uint32_t co, char* lds) const {
    int kk = k - lo;
    const bool ok = kk >= 0 && kk < span && co != OFF_NONE;
    if (period != 0 && kk >= period) kk -= period;
    lds_load16(rs, lds, ok ? (uint32_t)kk * ldb + co : OFF_NONE);
  }
};
// ---------------------------------------------------------------------------
// main loop: `L` provides issue(stage, sM, sN) and the compile-time count
// INSTS of direct-load instructions one wave issues per stage.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (whose fence
// waits for every outstanding load, including stages prefetched ahead).  The
// caller has already waited for the loads the next stage needs.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// Loaders with a register-staged operand provide finish(stage, sN) and run
// one stage ahead by step2.
template <class T, class = void>
struct HasFinish {
  static constexpr bool value = false;
};
template <class T>
struct HasFinish<T, decltype((void)&T::finish)> {
  static constexpr bool value = true;
};
// One pipeline step: wait for stage s, release the buffer stage s - 1 used,
// queue stage s + NBUF - 1 into it, multiply stage s.
template <class G, bool SPLIT, class L>
__device__ __forceinline__ void step2(L& ld, int s, int nst, f32x16 (&acc)[G::NB][G::MB],
                                      char* smem, int wm, int wn, int lane) {
  constexpr int IN = L::INSTS, NBUF = G::NBUF;
  const int left = nst - 1 - s;  // stages issued after s that may stay in flight
  if (NBUF >= 4 && left >= 2)
    wait_vm<2 * IN>();
  else if (NBUF >= 3 && left >= 1)
    wait_vm<IN>();
  else
    wait_vm<0>();
  bar();
  if (s + NBUF - 1 < nst) {
    const int b = (s + NBUF - 1) % NBUF;
    ld.issue(s + NBUF - 1, smem + b * G::STAGE, smem + b * G::STAGE + G::SM_BYTES);
  }
  const char* sM = smem + (s % NBUF) * G::STAGE;
  mma_stage2<G, SPLIT>(sM, sM + G::SM_BYTES, acc, wm, wn, lane);
  if constexpr (HasFinish<L>::value) {
    static_assert(NBUF == 2, "register-staged operands expand one stage ahead");
    if (s + 1 < nst) {
      wait_vm<0>();
      ld.finish(s + 1, smem + ((s + 1) % NBUF) * G::STAGE + G::SM_BYTES);
      wait_lgkm0();  // the next step's barrier publishes the expanded tile
    }
  }
}

// ---------------------------------------------------------------------------
// Ping-pong stage loop (eight waves, WM = 2): waves 0-3 (group A, rows
// 0..TM/2-1) and 4-7 (group B, the other rows) alternate between a memory
// phase -- group A queues the next stage's direct loads, each group reads all
// of the current stage's fragments into registers -- and a compute phase of
// back-to-back MFMAs, one barrier between phases.  Each SIMD then has one wave
// issuing MFMAs while its other wave issues memory instructions.  Group B
// runs one phase behind A:
//   A: mem(0) | comp(0) | mem(1) | comp(1) | ...          | (tail)
//   B:        | mem(0)  | comp(0)| mem(1)  | ... comp(n-1) |
// The loader's issue(s, sM, sN) is called by group A only (it maps the stage
// over four waves).  Both groups pass the same number of barriers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pbar() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// All four k-steps' fragments are read in the memory phase: the group that
// runs one phase behind (B) must be done with a buffer before the barrier at
// which group A starts refilling it, so no LDS read may move into the
// compute phase with two buffers.
template <class G, class L>
__device__ __forceinline__ void run_pingpong(L& ld, int nst, f32x16 (&acc)[G::NB][G::MB], char* smem) {
  static_assert(G::NW == 8 && G::WM == 2 && G::NBUF == 2, "two groups of four waves, two buffers");
  constexpr int KS = G::KT / 16;
  if (nst <= 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = w / G::WN, wn = w % G::WN;
  const bool ga = wm == 0;
  if (ga) ld.issue(0, smem, smem + G::SM_BYTES);
  wait_vm<0>();
  pbar();                 // stage 0 visible to both groups
  if (!ga) pbar();        // group B starts one phase behind
  bf16x8 fa[KS][G::NB], fb[KS][G::MB];
  for (int s = 0; s < nst; ++s) {
    char* cur = smem + (s & 1) * G::STAGE;
    if (ga && s + 1 < nst) {
      char* nxt = smem + ((s + 1) & 1) * G::STAGE;
      ld.issue(s + 1, nxt, nxt + G::SM_BYTES);
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) load_frags2<G, false>(cur, cur + G::SM_BYTES, fa[kk], fb[kk], kk, wm, wn, lane);
    wait_lgkm0();
    pbar();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][nb], fb[kk][mb], acc[nb][mb], 0, 0, 0);
    if (ga) wait_vm<0>();   // stage s+1 has landed before the phase that reads it
    pbar();
  }
  if (ga) pbar();         // match group B's last barrier
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Epilogue through LDS.  A lane's accumulators are four consecutive columns
// of one row, so a direct store instruction touches 32 rows.  Instead the
// waves park their values in an LDS image of the tile (rows padded by 16
// bytes) and the workgroup then writes whole rows, 16 bytes a lane.  Use
// after run_stages2, whose closing barrier frees LDS.
// ---------------------------------------------------------------------------
template <class G, int COLS, typename OUT>
struct TileImage {
  static constexpr int ES = sizeof(OUT);
  static_assert(ES == 2 || ES == 4, "bf16 bits or fp32");
  static constexpr int PITCH = COLS * ES + 16;  // bytes per image row
  static constexpr int BYTES = G::TM * PITCH;
  static constexpr int CPRW = COLS * ES / 16;   // 16-byte chunks per row
  // values of (row, col .. col + 3), tile coordinates
  __device__ static __forceinline__ void put(char* smem, int row, int col, f32x4 v) {
    char* p = smem + row * PITCH + col * ES;
    if constexpr (ES == 4)
      *(f32x4*)p = v;
    else
      *(u32x2*)p = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
  }
  // rows [0, nrows) of the image -> out (ld elements per row); call between
  // two barriers (after the puts, before LDS is reused)
  __device__ static __forceinline__ void flush(const char* smem, OUT* out, long ld, int nrows) {
    const int lim = (nrows < G::TM ? nrows : G::TM) * CPRW;
    for (int idx = threadIdx.x; idx < lim; idx += G::NT) {
      const int r = idx / CPRW, c = idx - r * CPRW;
      *(u32x4*)((char*)(out + (long)r * ld) + 16 * c) = *(const u32x4*)(smem + r * PITCH + 16 * c);
    }
  }
};

// SPLIT: 0 = no stage is split, 1 = every stage, 2 = the last ld.nsplit
// stages (a low-rank extension run after the base K range, in the same
// pipeline; the two kinds of stage run in loops of their own so that each
// loop body holds one fragment schedule).
template <class G, int SPLIT, class L>
__device__ __forceinline__ void run_stages2(L& ld, int nst, f32x16 (&acc)[G::NB][G::MB],
                                            char* smem) {
  if (nst <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / G::WN, wn = w % G::WN;
  constexpr int NBUF = G::NBUF;
  {
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p)
      if (p < nst) ld.issue(p, smem + p * G::STAGE, smem + p * G::STAGE + G::SM_BYTES);
    if constexpr (HasFinish<L>::value) {
      wait_vm<0>();
      ld.finish(0, smem + G::SM_BYTES);
      wait_lgkm0();
    }
    int s = 0;
    if constexpr (SPLIT == 2) {
      const int nb = nst - ld.nsplit > 0 ? nst - ld.nsplit : 0;
      for (; s < nb; ++s) step2<G, false>(ld, s, nst, acc, smem, wm, wn, lane);
      for (; s < nst; ++s) step2<G, true>(ld, s, nst, acc, smem, wm, wn, lane);
    } else {
      for (; s < nst; ++s) step2<G, SPLIT == 1>(ld, s, nst, acc, smem, wm, wn, lane);
    }
  }
  __syncthreads();
}


// ---------------------------------------------------------------------------
// Large wave tiles: twelve accumulator blocks (192 of the 256 registers a
// wave has at two waves per SIMD), both operands K tiles of 64 k, two stage
// buffers.  Fragment addresses: the chunk swizzle of tile row 32 j + l is
// (l & 7) ^ (l >> 3) ^ 4 (j & 1), so the fragment of row block j at k-step kk
// lies at 4096 j + o[kk ^ 2 (j & 1)]: four lane offsets serve every fragment
// of both tiles (the general frag() leaves the compiler one address per
// fragment and k-step, which does not fit beside the accumulators).  Each
// fragment is read once per k-step; a fragment of the next step is read
// right after the last product of this step that uses its register.
// ---------------------------------------------------------------------------
template <class G>
struct FragLT {
  static_assert(!G::MTR && !G::NTR && G::KT == 64 && G::NBUF == 2, "K tiles of 64 k, two buffers");
  static_assert((G::NB / 2) % 2 == 0 && (G::TN / 64) % 2 == 0, "N row block parity fixed by nb");
  uint32_t om[4], on[4];  // M tile (this wave's row block parity folded in), N tile
  __device__ __forceinline__ void init(int wm, int lane) {
    const int l = lane & 31;
    const uint32_t u = (uint32_t)((lane >> 5) ^ (l & 7) ^ (l >> 3));
    const bool odd = ((wm * G::MB) & 1) != 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) on[v] = 128u * (uint32_t)l + ((((uint32_t)(2 * v)) ^ u) << 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) om[v] = odd ? on[v ^ 2] : on[v];
  }
  // M row block mb of this wave (sM: the wave's first row block)
  __device__ __forceinline__ bf16x8 m(const char* sM, int mb, int kk) const {
    return *(const bf16x8*)(sM + om[kk ^ (2 * (mb & 1))] + 4096 * mb);
  }
  // N block nb of this wave (sN: the tile plus the wave's column offset)
  __device__ __forceinline__ bf16x8 n(const char* sN, int nb, int kk) const {
    constexpr int H2 = G::NB / 2;
    const int j = (nb < H2 ? 0 : G::TN / 64) + nb % H2;
    return *(const bf16x8*)(sN + on[kk ^ (2 * ((nb % H2) & 1))] + 4096 * j);
  }
};

template <class G, bool SPLIT>
__device__ __forceinline__ void mma_stage_lt(const char* sM, const char* sN, const FragLT<G>& fo,
                                             f32x16 (&acc)[G::NB][G::MB]) {
  constexpr int KS = 4;
  auto active = [](int nb, int kk) { return !SPLIT || ((nb < G::NB / 2) == (kk < KS / 2)); };
  bf16x8 a[G::NB], b[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) b[mb] = fo.m(sM, mb, 0);
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb)
    if (active(nb, 0)) a[nb] = fo.n(sN, nb, 0);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        if (active(nb, kk))
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[nb], b[mb], acc[nb][mb], 0, 0, 0);
        if (mb == G::MB - 1 && kk + 1 < KS && active(nb, kk + 1)) a[nb] = fo.n(sN, nb, kk + 1);
      }
      if (kk + 1 < KS) b[mb] = fo.m(sM, mb, kk + 1);
    }
  }
}

// Stages [0, nbase) plain, then next SPLIT stages; `ld.base(s, sM, sN)` and
// `ld.ext(s, sM, sN)` queue base stage s and extension stage s.  One barrier
// per stage; a stage is queued into the buffer the previous one used once
// every wave has passed that barrier.  The stage that queues the first
// extension stage is peeled, so that each loop issues one kind of stage
// (the loaders of the other kind hold no registers meanwhile).
template <class G, class L>
__device__ __forceinline__ void run_stages_lt(L& ld, int nbase, int next, f32x16 (&acc)[G::NB][G::MB],
                                              char* smem) {
  const int nst = nbase + next;
  if (nst <= 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = w / G::WN, wn = w % G::WN;
  FragLT<G> fo;
  fo.init(wm, lane);
  const int om = 4096 * G::MB * wm, on = G::SM_BYTES + 4096 * (G::NB / 2) * wn;
  auto buf = [&](int s) { return smem + (s & 1) * G::STAGE; };
  if (nbase > 0)
    ld.base(0, smem, smem + G::SM_BYTES);
  else
    ld.ext(0, smem, smem + G::SM_BYTES);
  int s = 0;
  for (; s + 1 < nbase; ++s) {
    wait_vm<0>();
    bar();
    ld.base(s + 1, buf(s + 1), buf(s + 1) + G::SM_BYTES);
    mma_stage_lt<G, false>(buf(s) + om, buf(s) + on, fo, acc);
  }
  if (s < nbase) {  // the last base stage
    wait_vm<0>();
    bar();
    if (next > 0) ld.ext(0, buf(s + 1), buf(s + 1) + G::SM_BYTES);
    mma_stage_lt<G, false>(buf(s) + om, buf(s) + on, fo, acc);
    ++s;
  }
  for (; s < nst; ++s) {
    wait_vm<0>();
    bar();
    if (s + 1 < nst) ld.ext(s + 1 - nbase, buf(s + 1), buf(s + 1) + G::SM_BYTES);
    mma_stage_lt<G, true>(buf(s) + om, buf(s) + on, fo, acc);
  }
  __syncthreads();
}

// K tile of R rows gathered by token, offsets formed at issue from the
// token ids (one register a tile row; the byte offsets would need one each
// for every source).  issue(): whole stages of a [*, ldb / 2] bf16 matrix;
// issue_split(): SPLIT stages (chunks c < CPR/2 read k = k0 + 8c, the others
// khalf + k0 + 8 (c - CPR/2); k past span reads zero).
template <int R, int KT, int NW>
struct KLoadTk {
  static constexpr int CPR = Depth<KT>::CPR, RPI = Depth<KT>::RPI;
  static constexpr int NJ = R / (NW * RPI);
  static_assert(NJ >= 1 && NJ * NW * RPI == R, "tile rows per stage");
  int tk[NJ];  // token of tile row j of this lane, -1: zeros
  __device__ static __forceinline__ int row_of(int j) { return KLoad<R, KT, NW>::row_of(j); }
  __device__ static __forceinline__ int slot(int j) { return (int)(threadIdx.x % CPR) ^ kswz<KT>(row_of(j)); }
  __device__ __forceinline__ void tokens(const int32_t* row2r, int topk, long row0, long nvalid) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) tk[j] = (row_of(j) < nvalid) ? row2r[row0 + row_of(j)] / topk : -1;
  }
  __device__ __forceinline__ void issue(rsrc_t rs, uint32_t ldb, int k0, char* tile) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      asm volatile("" : "+v"(tk[j]));  // form the offset here, not once for the loop in another register
      const uint32_t off = tk[j] >= 0 ? (uint32_t)tk[j] * ldb + 16u * (uint32_t)slot(j) : OFF_NONE;
      lds_load16(rs, tile + 1024 * (w + NW * j), off, 2u * (uint32_t)k0);
    }
  }
  __device__ __forceinline__ void issue_split(rsrc_t rs, uint32_t ldb, int k0, int khalf, int span,
                                              char* tile) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      asm volatile("" : "+v"(tk[j]));
      const int c = slot(j);
      const int k = (c < CPR / 2) ? k0 + 8 * c : khalf + k0 + 8 * (c - CPR / 2);
      const bool ok = tk[j] >= 0 && k < span;
      lds_load16(rs, tile + 1024 * (w + NW * j), ok ? (uint32_t)tk[j] * ldb + 2u * (uint32_t)k : OFF_NONE);
    }
  }
};

}  // namespace v2
}  // namespace moelora
