// forward.hip -- forward of the MoE side-LoRA expert layer.
//
// Steps (DeepGEMM PR #9, "Historical implementation" -> Summary: shrink and
// expand phases around the expert GEMMs, A1/A3/B2 shared, B1/B3/A2 local):
//   k_shrink    ZA_t = s [A1; A3] x_t, once per token (A1/A3 are shared, so
//               A u is the same for all k routes of a token)
//   k_w13       g = W1_e u + B1_e ZA1_t, v = W3_e u + B3_e ZA3_t; the B terms
//               ride as extra K on the W13 GEMM; SwiGLU in the epilogue;
//               saves G, V (fp16, accumulator-blocked) and h (bf16)
//   k_a2        Z2 = s A2_e h
//   k_w2        Ybase = W2_e h
//   k_zc        zc_t = sum_j w_tj Z2_(t,j)          (slot order, fp32)
//   k_rank_combine               out_t = B2 zc_t + sum_j w_tj Ybase_(t,j)
// The per-token evaluation of the shared factors is exact algebra:
// sum_j w_j B2 z_j = B2 sum_j w_j z_j.
#include <type_traits>

#include "../../include/moelora.h"
#include "engine2.hpp"
#include "engine_mx.hpp"
#include "gather_sum.hpp"
#include "layer.hpp"
#include "trace.hpp"

namespace moelora {

hipError_t launch_tile_map(const LayerArgs& a, hipStream_t st);
hipError_t launch_save_x(const LayerArgs& a, hipStream_t st);

// thin GEMMs (N = r): smaller M tiles so the grid fills the 256 CUs
using GS64 = Geo<1, 2, 2, 2>;   // 64 x 128 tile, wave 32 x 64
using GS128 = Geo<2, 2, 2, 2>;  // 128 x 128 tile, wave 64 x 64
constexpr int A2_SUB = TMG / GS128::TM;  // sub-tiles per pool M tile

// ----------------------------------------------------------------------------
// a3: ZA = s [A1; A3] x  (dense over tokens; N = 2r)
// ----------------------------------------------------------------------------
template <int R>
struct LdPlain {
  RowsK<R> m;
  RowsK<128> n;
  int k0 = 0;  // first k (a split's quarter of K)
  __device__ void load(int s) { m.load(k0 + s * KT, 0, false); n.load(k0 + s * KT, 0, false); }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

// One token tile (one root: the root's adapter's factor), one factor and
// one of KSPLIT quarters of H per workgroup: partial products to zsp, summed
// in split order by k_shrink_sum.  The split is fixed, so a token's ZA does
// not depend on the batch.
__global__ __launch_bounds__(256) void k_shrink(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int fac = blockIdx.y & 1, c0 = RBLK * (blockIdx.y >> 1);  // fac 0: A1, 1: A3; rank block c0..
  int t0, nt, ad;
  if (!token_tile(a, blockIdx.x, GS64::TM, t0, nt, ad)) return;
  const int r = a.r, ks = blockIdx.z, kh = a.H / KSPLIT;
  LdPlain<GS64::TM> L;
  L.k0 = ks * kh;
  L.m.contig(a.x, t0, nt, a.H);
  L.m.window(a.H);
  L.n.contig((fac ? a.A3 : a.A1) + ((long)ad * r + c0) * a.H, 0, r - c0, a.H);
  L.n.window(a.H);
  f32x16 acc[GS64::NB][GS64::MB];
  mainloop<GS64>(L, kh / KT, acc, smem);
  Epi<GS64> ep;
  float* part = a.zsp + (long)ks * a.T * 2 * r;
#pragma unroll
  for (int nb = 0; nb < GS64::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < GS64::MB; ++mb) {
      const int t = t0 + ep.row(mb);
      if (t >= t0 + nt) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = c0 + ep.col(nb, g);
        if (c >= r) continue;
        *(f32x4*)(part + (long)t * 2 * r + fac * r + c) =
            f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
      }
    }
}

// ZA = s x the splits' partials in order, as hi/lo.  One thread per 4 columns.
__global__ __launch_bounds__(256) void k_shrink_sum(LayerArgs a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int g4 = 2 * a.r / 4;
  if (i >= (long)a.T * g4) return;
  const long t = i / g4;
  const int c2 = (int)(i % g4) * 4, fac = c2 / a.r, c = c2 % a.r;  // r % 8 == 0: 4 columns of one factor
  f32x4 v = *(const f32x4*)(a.zsp + t * 2 * a.r + c2);
#pragma unroll
  for (int ks = 1; ks < KSPLIT; ++ks) {
    const f32x4 p = *(const f32x4*)(a.zsp + ((long)ks * a.T + t) * 2 * a.r + c2);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += p[q];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_hl(a.s * v[q], hi[q], lo[q]);
  uint16_t* dst = a.ZA + t * 4 * a.r + fac * 2 * a.r + c;
  *(u32x2*)dst = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
  *(u32x2*)(dst + a.r) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
}

// ----------------------------------------------------------------------------
// a4: W13 grouped GEMM (+ B1/B3 via K-extension) + SwiGLU
// N tile = 128 gate columns i0.. and the 128 up columns with the same i.
// ----------------------------------------------------------------------------
// N tile = TN/2 gate columns i0.. and the TN/2 up columns with the same i;
// each wave holds a gate block and its up partner, so SwiGLU runs in registers.
using GW13 = v2::Geo2<4, 2, 2, 4, false, false, 64>;  // 256 x 256 tile, eight waves
// Few rows per expert (small T): 64-row parts of a pool tile, with the LDS
// the smaller M tile frees spent on a third stage buffer (two weight stages
// in flight instead of one).  Each element still sums the same products in
// the same order, so the results are those of the full tile.
using GW13S = v2::Geo2<1, 2, 2, 4, false, false, 64, 3>;  // 64 x 256, eight waves
// Large tile (bf16 base, enough rows per expert): 384 x 256, eight waves of
// 96 x 128 (three row blocks by two gate/up block pairs).  Two stages fill
// the 160 KB of LDS; per product it reads 22 % fewer LDS fragment bytes and
// 17 % fewer operand bytes from L2 than the 256 x 256 tile, and each stage
// multiplies half as long again while the next one loads.
using GW13L = v2::Geo2<3, 4, 4, 2, false, false, 64>;
template <class G>
constexpr int w13_lds() { return cmax(G::LDS_BYTES, v2::TileImage<G, G::TN / 2, uint16_t>::BYTES); }
constexpr int W13_LDS = w13_lds<GW13>(), W13S_LDS = w13_lds<GW13S>(), W13L_LDS = w13_lds<GW13L>();
static_assert(W13L_LDS <= 160 * 1024, "the large tile fits the LDS of a CU");

// Stages [0, H/KT): the base K = H; the last nsplit stages: the B1/B3
// extension, SPLIT (KT/2 k of each half per stage).  M loaders: G::TM rows
// by token; N loaders: the 256 weight rows of the tile.
template <class G>
struct LdW13Base {
  using KL = v2::KLoad<G::TM, G::KT, G::NW>;          // ZA rows (M)
  using KL2 = v2::KLoad<256, G::KT, G::NW, true>;     // B1 | B3 rows (N)
  using KA = v2::KLoadA<G::TM, G::KT, G::NW>;         // x rows (M)
  using KN = v2::KLoadA<256, G::KT, G::NW>;           // W13 rows (N)
  KL me;
  KL2 ne;
  int r, nsplit;
};
// NL: the weight tile loader (KLoadA on W13, or KLoadP on its packed copy)
template <class G, class NL>
struct LdW13 : LdW13Base<G> {
  using B = LdW13Base<G>;
  static constexpr int INSTS = B::KL::NJ + B::KL2::NJ;
  static_assert(NL::NJ == B::KL2::NJ && B::KA::NJ == B::KL::NJ, "one instruction count per stage");
  typename B::KA mm;
  NL nm;
  int nbase;
  __device__ void issue(int s, char* sM, char* sN) {
    if (s >= nbase) {
      const int se = s - nbase;
      this->me.issue(se * (G::KT / 2), 2 * this->r, true, sM);
      this->ne.issue(se * (G::KT / 2), 2 * this->r, true, sN);
    } else {
      mm.issue(s * G::KT, sM);
      nm.issue(s * G::KT, sN);
    }
  }
};
// The large tile (GW13L): x rows and ZA rows by token through one token
// list, B1 | B3 rows, the weight tile loader NL.
template <class G, class NL>
struct LdW13L {
  using KT = v2::KLoadTk<G::TM, G::KT, G::NW>;
  using KL2 = typename LdW13Base<G>::KL2;
  KT m;
  KL2 ne;
  NL nm;
  rsrc_t rx, rza;
  uint32_t ldx, ldza;
  int r, nbase;
  __device__ void base(int s, char* sM, char* sN) {
    m.issue(rx, ldx, s * G::KT, sM);
    nm.issue(s * G::KT, sN);
  }
  __device__ void ext(int s, char* sM, char* sN) {
    m.issue_split(rza, ldza, s * (G::KT / 2), 2 * r, 4 * r, sM);
    ne.issue(s * (G::KT / 2), 2 * r, true, sN);
  }
};
// MXFP4 base (engine_mx.hpp): the split activation rows (x by token, or h
// by pool row), the weight tile and the scale words of each k64 stage (PK:
// from the packed copy); with an extension (W13), its 32-k bf16 stages run
// after the base range.
template <bool PK>
struct LdMX {
  mx::KA xa;
  mx::WLoad<PK> wl;
  __device__ void issue(int s, char* st) const {
    xa.issue(64 * s, st);
    wl.issue(s, st);
  }
  __device__ void issue_ext(int, char*) const {}  // no extension stages (next = 0)
};
template <bool PK>
struct LdW13MX : LdMX<PK> {
  mx::KE me;   // s A1 x, s A3 x (hi/lo) by token
  mx::KE2 ne;  // B1 rows (gate half of the tile), B3 rows (up half)
  int r;
  __device__ void issue_ext(int s, char* st) const {
    me.issue(s * 32, 2 * r, true, st);
    ne.issue(s * 32, 2 * r, true, st + mx::GE::SM_BYTES);
  }
};
static_assert(mx::LDS_BYTES <= GW13::LDS_BYTES, "the MX stages fit the bf16 pipeline's LDS");

// ACT: 0 SwiGLU (h = silu(g) v), 1 GeGLU (h = gelu(g) v, exact GELU).
// CL: activation clamp, h = f(clip(g)) clip(v) with clip to [-a.clamp, a.clamp]
// (PR #9 "Correctness coverage" names the clamp; the reading is the plainest
// one: both pre-activations are clipped).  Whether a value is clipped is
// decided on its fp16 rounding, the value saved for the backward, so that
// both passes take the same decision.
// PK: the base read from its packed copy W13P (pack.hip, kind 0; MXFP4:
// kind 4).
// SK: 64-row parts of the pool tiles (GW13S; bf16 base): the grid is SUB
// times larger and part `sub` takes rows row0 + 64 sub ..; parts past the
// tile's rows return at once.
// LT: the large tile (GW13L; bf16 base) over the TML-row tile list.
template <bool MX, int ACT, bool CL, bool PK, bool SK, bool LT>
__global__ __launch_bounds__(GW13::NT) void k_w13(LayerArgs a) {
  static_assert(!(MX && SK), "the small tiles are of a bf16 base");
  static_assert(!(LT && (MX || SK)), "the large tile is of a bf16 base with full tiles");
  extern __shared__ __align__(16) char smem[];
  using G = typename std::conditional<
      MX, mx::GMX, typename std::conditional<SK, GW13S, typename std::conditional<LT, GW13L, GW13>::type>::type>::type;
  static_assert(G::NT == GW13::NT && G::TN == GW13::TN, "same workgroup and N tile");
  using KL = typename LdW13Base<G>::KL;
  constexpr int TN = G::TN, HALF = TN / 2, SUB = LT ? 1 : TMG / G::TM;
  const int ntn = a.I / HALF;
  // part `sub` of pool tile work item b (SUB == 1: the block index itself)
  const int nb = SUB == 1 ? (int)gridDim.x : __builtin_amdgcn_readfirstlane(gridDim.x / SUB);
  const int b = SUB == 1 ? (int)blockIdx.x : __builtin_amdgcn_readfirstlane(blockIdx.x % nb);
  const int sub = SUB == 1 ? 0 : __builtin_amdgcn_readfirstlane(blockIdx.x / nb);
  int mt, nt;
  const TileInfo* tl = LT ? a.tiles3 : a.tiles;
  if (!group_tile(a, tl, LT ? TML : TMG, b, a.ntiles[LT ? 1 : 0], ntn, TILE_GM, mt, nt)) return;
  const TileInfo ti = tl[mt];
  const int row0 = ti.row0 + sub * G::TM;
  if (row0 >= ti.row_end) return;
  const int nrows = ti.row_end - row0 < G::TM ? ti.row_end - row0 : G::TM;
  const int e = grp_expert(a, ti.e), i0 = nt * HALF;
  const long le = grp_local(a, ti.e);  // the tile's adapter's B1/B3 of expert e
  const int r = a.r;
  const int nsplit = (2 * r + G::KT / 2 - 1) / (G::KT / 2);
  int tk[KL::NJ];  // the tile's rows are gathered by token: rows past the expert's count read zero
  KL::tokens(tk, a.row2r, a.k, row0, nrows);
  auto wrow = [&](int nl) { return (nl < HALF) ? i0 + nl : a.I + i0 + (nl - HALF); };
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  if constexpr (LT) {
    using KN = typename LdW13Base<G>::KN;
    using KL2 = typename LdW13Base<G>::KL2;
    using NL = typename std::conditional<PK, v2::KLoadP<256, G::KT, G::NW>, KN>::type;
    LdW13L<G, NL> L;
    L.r = r;
    L.nbase = a.H / G::KT;
    L.m.tokens(a.row2r, a.k, row0, nrows);
    L.rx = make_rsrc(a.x, (uint64_t)a.T * a.H * 2);
    L.ldx = (uint32_t)a.H * 2u;
    L.rza = make_rsrc(a.ZA, (uint64_t)a.T * 4 * r * 2);
    L.ldza = (uint32_t)(4 * r) * 2u;
    L.ne.rs = make_rsrc(a.B1 + le * a.I * r, (uint64_t)2 * r * a.I);
    L.ne.rs2 = make_rsrc(a.B3 + le * a.I * r, (uint64_t)2 * r * a.I);
#pragma unroll
    for (int j = 0; j < KL2::NJ; ++j) L.ne.roff[j] = (uint32_t)((i0 + (KL2::row_of(j) % HALF)) * r * 2);
    L.ne.window(2 * r, r, HALF, 2 * r);  // gate rows read k in [0, 2r), up rows [2r, 4r)
    if constexpr (PK) {
      L.nm.set(a.W13P + (long)e * 2 * a.I * a.H, (uint64_t)2 * a.I * a.H * 2, nt, a.H / G::KT);
    } else {
      L.nm.rs = make_rsrc(a.W13 + (long)e * 2 * a.I * a.H, (uint64_t)2 * a.I * a.H * 2);
#pragma unroll
      for (int j = 0; j < KN::NJ; ++j) L.nm.set_row(j, (uint32_t)((long)wrow(KN::row_of(j)) * a.H * 2));
    }
    v2::run_stages_lt<G>(L, L.nbase, nsplit, acc, smem);
  } else if constexpr (!MX) {
    using KN = typename LdW13Base<G>::KN;
    using KL2 = typename LdW13Base<G>::KL2;
    using NL = typename std::conditional<PK, v2::KLoadP<256, G::KT, G::NW>, KN>::type;
    LdW13<G, NL> L;
    L.r = r;
    L.nsplit = nsplit;
    L.nbase = a.H / G::KT;
    L.me.from_tokens(a.ZA, a.T, 4 * r, tk);
    L.me.window(4 * r);
    L.ne.rs = make_rsrc(a.B1 + le * a.I * r, (uint64_t)2 * r * a.I);
    L.ne.rs2 = make_rsrc(a.B3 + le * a.I * r, (uint64_t)2 * r * a.I);
#pragma unroll
    for (int j = 0; j < KL2::NJ; ++j) L.ne.roff[j] = (uint32_t)((i0 + (KL2::row_of(j) % HALF)) * r * 2);
    L.ne.window(2 * r, r, HALF, 2 * r);  // gate rows read k in [0, 2r), up rows [2r, 4r)
    L.mm.from_tokens(a.x, a.T, a.H, tk);
    if constexpr (PK) {
      L.nm.set(a.W13P + (long)e * 2 * a.I * a.H, (uint64_t)2 * a.I * a.H * 2, nt, a.H / G::KT);
    } else {
      L.nm.rs = make_rsrc(a.W13 + (long)e * 2 * a.I * a.H, (uint64_t)2 * a.I * a.H * 2);
#pragma unroll
      for (int j = 0; j < KN::NJ; ++j) L.nm.set_row(j, (uint32_t)((long)wrow(KN::row_of(j)) * a.H * 2));
    }
    v2::run_stages2<G, 2>(L, nsplit + a.H / G::KT, acc, smem);
  } else {
    // the base K range as k64 stages on the scaled matrix cores, then the
    // extension stages of 64 k (32 of the gate's 2r, 32 of the up's)
    using KE = mx::KE;
    LdW13MX<PK> L;
    L.r = r;
    {
      int tke[KE::NJ];
      KE::tokens(tke, a.row2r, a.k, row0, nrows);
      L.me.from_tokens(a.ZA, a.T, 4 * r, tke);
    }
    L.me.window(4 * r);
    L.ne.rs = make_rsrc(a.B1 + le * a.I * r, (uint64_t)2 * r * a.I);
    L.ne.rs2 = make_rsrc(a.B3 + le * a.I * r, (uint64_t)2 * r * a.I);
#pragma unroll
    for (int j = 0; j < KE::NJ; ++j) L.ne.roff[j] = (uint32_t)((i0 + (KE::row_of(j) % HALF)) * r * 2);
    L.ne.window(2 * r, r, HALF, 2 * r);
    L.xa.from_tokens((const uint16_t*)a.XQ, a.T, a.H, tk);  // 2H bytes a row, like a bf16 row
    // the scale words of x are stage-major [H/64][T]: token t's at 4 t
    auto xsw = [&](int row) { return row < nrows ? (uint32_t)(a.row2r[row0 + row] / a.k) * 4u : OFF_NONE; };
    if constexpr (PK) {
      const uint64_t bytes = (uint64_t)(2 * a.I / 256) * (a.H / 64) * MX_TILE;  // one expert's copy
      L.wl.set_packed((const uint8_t*)a.W13P + e * bytes, bytes, nt, a.H / 64, a.H, a.XS, a.T, xsw);
    } else {
      L.wl.set(a.W13q + (long)e * 2 * a.I * (a.H / 2), a.W13s + (long)e * 2 * a.I * (a.H / 32), 2L * a.I, a.H, wrow,
               a.XS, a.T, xsw);
    }
    mx::run_mx<G>(L, (2 * r + 31) / 32, a.H / 64, acc, smem);
  }
  // G and V go out as fp16 in the accumulator-blocked layout (512 bytes per
  // wave access);
  // h (bf16, row-major for the next GEMM) through an LDS image of the tile
  using ImgH = v2::TileImage<G, HALF, uint16_t>;
  Epi<G> ep;
  constexpr int NH = G::NB / 2;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform block offsets
  const int wm = wv / G::WN, wn = wv % G::WN, lane = threadIdx.x & 63;
  // Without a clamp a saved pre-activation must fit fp16: a finite value at
  // or beyond 65520 rounds to infinity, which would turn the backward's
  // gradients non-finite.  Such a forward raises MOE_SAVED_FP16_RANGE in the
  // status word (h and the forward output are computed from the fp32 values
  // and stay right).  With a clamp every such value is clipped anyway.
  bool wide = false;
  // G, V are blocked by TMG-row tiles: a large tile writes the 32-row blocks
  // inside the group's TMG tiles (rows past its count hold zeros, as a TMG
  // tile writes them; blocks past its last TMG tile belong to the next
  // group); a TMG tile writes all of its blocks
  int rlim = G::TM;
  if constexpr (LT) {
    const int off = a.offsets[ti.e];
    rlim = off + (ti.row_end - off + TMG - 1) / TMG * TMG - row0;
  }
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NH; ++nb) {
      if (LT && G::m_local(wm, mb) >= rlim) continue;
      const int cb = (i0 + G::n_local(wn, nb)) / 32;
      const long ob = acc_blk(ti.pad + G::m_local(wm, mb) / 32 + sub * (G::TM / 32), cb, a.I) + 4 * lane;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 gv, vv, hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gv[q] = acc[nb][mb][4 * g + q];
          vv[q] = acc[nb + NH][mb][4 * g + q];
        }
        const f16x4 g16 = __builtin_convertvector(gv, f16x4);  // round to nearest even
        const f16x4 v16 = __builtin_convertvector(vv, f16x4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float gq = gv[q], vq = vv[q];
          if constexpr (!CL) wide |= fabsf(gq) >= 65520.0f || fabsf(vq) >= 65520.0f;
          if constexpr (CL) {
            if (fabsf((float)g16[q]) > a.clamp) gq = copysignf(a.clamp, gq);
            if (fabsf((float)v16[q]) > a.clamp) vq = copysignf(a.clamp, vq);
          }
          if constexpr (ACT == 0)
            hv[q] = gq * sigmoidf_(gq) * vq;
          else
            hv[q] = gq * norm_cdf(gq) * vq;
        }
        *(f16x4*)(a.G + ob + 256 * g) = g16;
        *(f16x4*)(a.V + ob + 256 * g) = v16;
        ImgH::put(smem, ep.row(mb), ep.col(nb, g), hv);
      }
    }
  if (wide) *a.status = MOE_SAVED_FP16_RANGE;  // only ever 0 -> this bit: racing stores agree
  __syncthreads();
  ImgH::flush(smem, a.Hh + row0 * (long)a.I + i0, a.I, nrows);
  if constexpr (MX)  // the W2 GEMM's operand: the split of these bf16 rows of h
    mx::split_image_rows<HALF, G::NT>(smem, ImgH::PITCH, nrows, a.HQ + row0 * (long)(2 * a.I), a.HS + row0,
                                      a.cap, a.I, i0);
}

// ----------------------------------------------------------------------------
// a5: Z2 = s A2_e h  (grouped, N = r)
// a6: Ybase = W2_e h (grouped)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_a2(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  int mt, sub, y;
  if (!sub_tile(a, A2_SUB, mt, sub, y)) return;
  const TileInfo ti = a.tiles[mt];
  const long row0 = ti.row0 + (long)sub * GS128::TM;  // this sub-tile's rows
  if (row0 >= ti.row_end) return;
  const int c0 = RBLK * y;  // rank block
  const uint16_t* A2e = a.A2 + (grp_local(a, ti.e) * a.r + c0) * a.I;
  LdPlain<GS128::TM> L;
  L.m.contig(a.Hh, row0, ti.row_end - row0, a.I);
  L.m.window(a.I);
  L.n.contig(A2e, 0, a.r - c0, a.I);
  L.n.window(a.I);
  f32x16 acc[GS128::NB][GS128::MB];
  mainloop<GS128>(L, a.I / KT, acc, smem);
  Epi<GS128> ep;
#pragma unroll
  for (int mb = 0; mb < GS128::MB; ++mb) {
    const long row = row0 + ep.row(mb);
    if (row >= ti.row_end) continue;
#pragma unroll
    for (int nb = 0; nb < GS128::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = c0 + ep.col(nb, g);
        if (c >= a.r) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = a.s * acc[nb][mb][4 * g + q];
        *(f32x4*)(a.Z2 + row * a.r + c) = v;
      }
  }
}

// Few rows per expert: 64-row parts on the direct-load engine with four
// stage buffers (three stages queued), so the long K = I contraction is not
// bound by one load latency per stage.  Each element sums the same products
// in the same order as k_a2.
using GA2S = v2::Geo2<1, 2, 2, 2, false, false, 64, 4>;  // 64 x 128, four waves
struct LdA2S {
  using KM = v2::KLoad<GA2S::TM, GA2S::KT, GA2S::NW>;  // h rows
  using KN = v2::KLoad<128, GA2S::KT, GA2S::NW>;       // A2_e rows
  static constexpr int INSTS = KM::NJ + KN::NJ;
  KM m;
  KN n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GA2S::KT, 0, false, sM);
    n.issue(s * GA2S::KT, 0, false, sN);
  }
};

__global__ __launch_bounds__(GA2S::NT) void k_a2s(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  using G = GA2S;
  constexpr int SUB = TMG / G::TM;
  int mt, sub, y;
  if (!sub_tile(a, SUB, mt, sub, y)) return;
  const TileInfo ti = a.tiles[mt];
  const long row0 = ti.row0 + (long)sub * G::TM;  // this part's rows
  if (row0 >= ti.row_end) return;
  const int c0 = RBLK * y;  // rank block
  LdA2S L;
  L.m.contig(a.Hh, row0, ti.row_end - row0, a.I);
  L.m.window(a.I);
  L.n.contig(a.A2 + (grp_local(a, ti.e) * a.r + c0) * a.I, 0, a.r - c0, a.I);
  L.n.window(a.I);
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  v2::run_stages2<G, 0>(L, a.I / G::KT, acc, smem);
  Epi<G> ep;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const long row = row0 + ep.row(mb);
    if (row >= ti.row_end) continue;
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = c0 + ep.col(nb, g);
        if (c >= a.r) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = a.s * acc[nb][mb][4 * g + q];
        *(f32x4*)(a.Z2 + row * a.r + c) = v;
      }
  }
}

using GW2 = v2::Geo2<4, 2, 2, 4, false, false, 64>;  // 256 x 256 tile, eight waves
// few rows per expert: 64-row parts of each pool tile, a third stage buffer
using GW2S = v2::Geo2<1, 2, 2, 4, false, false, 64, 3>;
constexpr int W2_LDS = cmax(GW2::LDS_BYTES, v2::TileImage<GW2, GW2::TN, uint16_t>::BYTES);
constexpr int W2S_LDS = cmax(GW2S::LDS_BYTES, v2::TileImage<GW2S, GW2S::TN, uint16_t>::BYTES);
// the small-part pipeline: all eight waves queue a stage
template <class NL>
struct LdW2S {
  using KL = v2::KLoadS<GW2S::TM, GW2S::KT, GW2S::NW>;
  static constexpr int INSTS = KL::NJ + NL::NJ;
  KL m;
  NL n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW2S::KT, sM);
    n.issue(s * GW2S::KT, sN);
  }
};
template <class NL>  // the weight tile loader: KLoadS on W2, or KLoadP on its packed copy
struct LdW2 {
  // the ping-pong loop: the four waves of group A queue a whole stage
  using KL = v2::KLoadS<256, GW2::KT, 4>;
  static constexpr int INSTS = 2 * KL::NJ;
  static_assert(NL::NJ == KL::NJ, "one instruction count per stage");
  KL m;
  NL n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW2::KT, sM);
    n.issue(s * GW2::KT, sN);
  }
};

// PK: the base read from its packed copy W2P (pack.hip, kind 1; MXFP4: kind 5)
template <bool MX, bool PK, bool SK>
// SK: 64-row parts of the pool tiles (GW2S, bf16 base): the grid is SUB
// times larger and part `sub` takes rows row0 + 64 sub ..; parts past the
// tile's rows return at once (bitwise the same as the full tile).
__global__ __launch_bounds__(GW2::NT) void k_w2(LayerArgs a) {
  static_assert(!(MX && SK), "the small parts are of a bf16 base");
  extern __shared__ __align__(16) char smem[];
  using G = typename std::conditional<MX, mx::GMX, typename std::conditional<SK, GW2S, GW2>::type>::type;
  static_assert(G::NT == GW2::NT, "one workgroup size");
  constexpr int SUB = TMG / G::TM;
  const int ntn = a.H / G::TN;
  // part `sub` of pool tile work item b (SUB == 1: the block index itself)
  const int nb = SUB == 1 ? (int)gridDim.x : __builtin_amdgcn_readfirstlane(gridDim.x / SUB);
  const int b = SUB == 1 ? (int)blockIdx.x : __builtin_amdgcn_readfirstlane(blockIdx.x % nb);
  const int sub = SUB == 1 ? 0 : __builtin_amdgcn_readfirstlane(blockIdx.x / nb);
  int mt, nt;
  if (!group_tile(a, a.tiles, TMG, b, *a.ntiles, ntn, TILE_GM, mt, nt)) return;
  const TileInfo ti = a.tiles[mt];
  const int row0 = ti.row0 + sub * G::TM;
  if (row0 >= ti.row_end) return;
  const int h0 = nt * G::TN;
  const int nrows = ti.row_end - row0;  // rows to the expert's end (the tile holds at most TM of them)
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  if constexpr (SK) {
    using NL = typename std::conditional<PK, v2::KLoadP<256, G::KT, G::NW>, v2::KLoadS<256, G::KT, G::NW>>::type;
    LdW2S<NL> L;
    L.m.contig(a.Hh, row0, nrows, a.I);
    const long e = grp_expert(a, ti.e);
    if constexpr (PK)
      L.n.set(a.W2P + e * a.H * a.I, (uint64_t)a.H * a.I * 2, nt, a.I / G::KT);
    else
      L.n.contig(a.W2 + e * a.H * a.I, h0, G::TN, a.I);
    v2::run_stages2<G, 0>(L, a.I / G::KT, acc, smem);
  } else if constexpr (!MX) {
    using NL = typename std::conditional<PK, v2::KLoadP<256, GW2::KT, 4>, v2::KLoadS<256, GW2::KT, 4>>::type;
    LdW2<NL> L;
    L.m.contig(a.Hh, ti.row0, nrows, a.I);
    const long e = grp_expert(a, ti.e);
    if constexpr (PK)
      L.n.set(a.W2P + e * a.H * a.I, (uint64_t)a.H * a.I * 2, nt, a.I / G::KT);
    else
      L.n.contig(a.W2 + e * a.H * a.I, h0, G::TN, a.I);
    v2::run_pingpong<G>(L, a.I / G::KT, acc, smem);
  } else {
    // MXFP4 base: h as its two-term split, W2 packed, on the scaled matrix cores
    LdMX<PK> N;
    N.xa.contig((const uint16_t*)a.HQ, ti.row0, nrows, a.I);  // 2I bytes a row, like a bf16 row
    const long e = grp_expert(a, ti.e);
    // the scale words of h are stage-major [I/64][cap]: pool row p's at 4 p
    auto hsw = [&](int row) { return row < nrows ? (uint32_t)(ti.row0 + row) * 4u : OFF_NONE; };
    if constexpr (PK) {
      const uint64_t bytes = (uint64_t)(a.H / 256) * (a.I / 64) * MX_TILE;  // one expert's copy
      N.wl.set_packed((const uint8_t*)a.W2P + e * bytes, bytes, nt, a.I / 64, a.I, a.HS, a.cap, hsw);
    } else {
      N.wl.set(a.W2q + e * a.H * (a.I / 2), a.W2s + e * a.H * (a.I / 32), (long)a.H, a.I,
               [&](int n) { return h0 + n; }, a.HS, a.cap, hsw);
    }
    mx::run_mx<G>(N, 0, a.I / 64, acc, smem);
  }
  using Img = v2::TileImage<G, G::TN, uint16_t>;
  Epi<G> ep;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        Img::put(smem, ep.row(mb), ep.col(nb, g),
                 f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                       acc[nb][mb][4 * g + 3]});
  __syncthreads();
  Img::flush(smem, a.Yb + row0 * (long)a.H + h0, a.H, nrows);
}

// ----------------------------------------------------------------------------
// a7: zc_t = sum_j w_tj Z2_(t,j);  out_t = B2 zc_t + sum_j w_tj Ybase_(t,j)
// ----------------------------------------------------------------------------
// One thread per token and 4 columns: all of the token's route indices are
// loaded first, then one 16-byte Z2 load per live route (routes added in
// route order); hi and lo go out as 8-byte stores.
__global__ __launch_bounds__(256) void k_zc(LayerArgs a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int g4 = a.r / 4;  // r % 8 == 0
  if (i >= (long)a.T * g4) return;
  const int t = (int)(i / g4), c = (int)(i % g4) * 4;
  int rows[16];  // topk <= 16
#pragma unroll
  for (int j = 0; j < 16; ++j) rows[j] = j < a.k ? a.r2row[t * a.k + j] : -1;
  f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (rows[j] < 0) continue;  // a dropped route's weight is not read
    const float wj = a.w[t * a.k + j];
    const f32x4 p = *(const f32x4*)(a.Z2 + (long)rows[j] * a.r + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) z[q] += wj * p[q];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_hl(z[q], hi[q], lo[q]);
  uint16_t* d = a.zc + (long)t * 2 * a.r + c;
  *(u32x2*)d = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
  *(u32x2*)(d + a.r) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
}

struct LdRankC {
  using KM = v2::KLoad<GRK::TM, GRK::KT, GRK::NW>;
  using KN = v2::KLoad<GRK::TN, GRK::KT, GRK::NW>;
  static constexpr int INSTS = KM::NJ + KN::NJ;
  KM m;
  KN n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GRK::KT, 0, false, sM);
    n.issue(s * GRK::KT, 0, false, sN);
  }
};

// out = B2 zc_t + sum_j w_tj Ybase_(t,j) for 128 tokens (of one root) x 256
// columns (zc carries s and the routing weights; hi/lo halves fold onto B2's
// r columns; B2 of the root's adapter)
__global__ __launch_bounds__(GRK::NT, 2) void k_rank_combine(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  int t0, nt, ad;
  if (!token_tile(a, blockIdx.y, GRK::TM, t0, nt, ad)) return;
  const int h0 = blockIdx.x * GRK::TN;  // the column tiles of a token tile run side by side
  const int r = a.r;
  RouteVec rv;
  load_routes<true>(a, t0, t0 + nt, rv);
  LdRankC L;
  L.m.contig(a.zc, t0, nt, 2 * r);
  L.m.window(2 * r);
  L.n.contig(a.B2 + (long)ad * a.H * r, h0, GRK::TN, r);
  L.n.window(2 * r, r);
  f32x16 acc[GRK::NB][GRK::MB];
  zero_acc<GRK>(acc);
  v2::run_stages2<GRK, 0>(L, (2 * r + GRK::KT - 1) / GRK::KT, acc, smem);
  rank_route_sum<true>(acc, smem, a, rv, a.Yb, a.out, t0, t0 + nt, h0);
}

// ----------------------------------------------------------------------------

template <bool MX, int ACT, bool CL, bool PK, bool SK, bool LT>
static void launch_w13(const LayerArgs& a, hipStream_t st) {
  constexpr int SUB = SK ? TMG / GW13S::TM : 1;
  const dim3 grid((LT ? a.maxtiles3 : a.maxtiles) * (a.I / (GW13::TN / 2)) * SUB);
  MOE_LAUNCH_AS("k_w13", (k_w13<MX, ACT, CL, PK, SK, LT>), grid, dim3(GW13::NT),
                SK ? W13S_LDS : (LT ? W13L_LDS : W13_LDS), st, a);
}
template <bool MX, int ACT, bool PK, bool SK, bool LT>
static void launch_w13_cl(const LayerArgs& a, hipStream_t st) {
  if (a.clamp > 0.0f)
    launch_w13<MX, ACT, true, PK, SK, LT>(a, st);
  else
    launch_w13<MX, ACT, false, PK, SK, LT>(a, st);
}
template <bool MX, int ACT, bool PK>
static void launch_w13_sk(const LayerArgs& a, hipStream_t st) {
  if (!MX && a.small_tiles)
    launch_w13_cl<MX, ACT, PK, !MX, false>(a, st);
  else if (!MX && a.large_tiles)
    launch_w13_cl<MX, ACT, PK, false, !MX>(a, st);
  else
    launch_w13_cl<MX, ACT, PK, false, false>(a, st);
}
template <bool MX, bool PK, bool SK, bool LT>
static void set_w13_lds(AttrInit& ai) {
  const int lds = SK ? W13S_LDS : (LT ? W13L_LDS : W13_LDS);
  ai.lds((const void*)k_w13<MX, 0, false, PK, SK, LT>, lds);
  ai.lds((const void*)k_w13<MX, 1, false, PK, SK, LT>, lds);
  ai.lds((const void*)k_w13<MX, 0, true, PK, SK, LT>, lds);
  ai.lds((const void*)k_w13<MX, 1, true, PK, SK, LT>, lds);
}

hipError_t launch_split_rows(const uint16_t* src, long rows, int K, uint8_t* codes, uint32_t* scales,
                             hipStream_t st) {
  const long n = rows * (K / 32);
  MOE_LAUNCH_AS("k_quant_rows", mx::k_quant_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                codes, scales, rows, K);
  return hipGetLastError();
}

hipError_t launch_forward(const LayerArgs& a, hipStream_t st, bool branch) {
  static PerDeviceOnce attrs;
  hipError_t err = attrs.run([] {
    AttrInit ai;
    ai.lds((const void*)k_shrink, GS64::LDS_BYTES);
    set_w13_lds<false, false, false, false>(ai);
    set_w13_lds<false, true, false, false>(ai);
    set_w13_lds<false, false, true, false>(ai);
    set_w13_lds<false, true, true, false>(ai);
    set_w13_lds<false, false, false, true>(ai);
    set_w13_lds<false, true, false, true>(ai);
    set_w13_lds<true, false, false, false>(ai);
    set_w13_lds<true, true, false, false>(ai);
    ai.lds((const void*)k_a2, GS128::LDS_BYTES);
    ai.lds((const void*)k_a2s, GA2S::LDS_BYTES);
    ai.lds((const void*)k_w2<false, false, false>, W2_LDS);
    ai.lds((const void*)k_w2<false, true, false>, W2_LDS);
    ai.lds((const void*)k_w2<false, false, true>, W2S_LDS);
    ai.lds((const void*)k_w2<false, true, true>, W2S_LDS);
    ai.lds((const void*)k_w2<true, false, false>, W2_LDS);
    ai.lds((const void*)k_w2<true, true, false>, W2_LDS);
    ai.lds((const void*)k_rank_combine, RK_LDS);
    return ai.err;
  });
  if (err != hipSuccess) return err;
  // Two streams: the branch computes ZA (and an MXFP4 base's split of x)
  // and the saved copy of x while the caller's stream builds the tile map;
  // after the W13 GEMM the branch computes Z2 = s A2_e h and zc while the
  // caller's stream runs the W2 GEMM; the combine follows the join.
  Branch br;
  if ((err = br.open(st, branch)) != hipSuccess) return err;
  const hipStream_t sd = br.side();
  MOE_LAUNCH(k_shrink, dim3(token_tiles(a, GS64::TM), 2 * rank_blocks(a.r), KSPLIT), dim3(256), GS64::LDS_BYTES,
             sd, a);
  MOE_LAUNCH(k_shrink_sum, dim3((unsigned)(((long)a.T * (2 * a.r / 4) + 255) / 256)), dim3(256), 0, sd, a);
  if (a.mx) {  // x as its two-term E2M3 split for the scaled W13 GEMM
    const long n = (long)a.T * (a.H / 32);
    MOE_LAUNCH_AS("k_quant_x", mx::k_quant_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, sd, a.x,
                  a.XQ, a.XS, (long)a.T, a.H);
  }
  if ((err = br.signal(sd, 1)) != hipSuccess) return err;  // ZA (and the split of x) written
  if ((err = launch_save_x(a, sd)) != hipSuccess) return err;
  if ((err = launch_tile_map(a, st)) != hipSuccess) return err;
  if ((err = br.await(st, 1)) != hipSuccess) return err;
  {
    const bool pk = a.W13P != nullptr;
    if (a.mx && a.act == 1)
      pk ? launch_w13_sk<true, 1, true>(a, st) : launch_w13_sk<true, 1, false>(a, st);
    else if (a.mx)
      pk ? launch_w13_sk<true, 0, true>(a, st) : launch_w13_sk<true, 0, false>(a, st);
    else if (a.act == 1)
      pk ? launch_w13_sk<false, 1, true>(a, st) : launch_w13_sk<false, 1, false>(a, st);
    else
      pk ? launch_w13_sk<false, 0, true>(a, st) : launch_w13_sk<false, 0, false>(a, st);
  }
  if ((err = br.signal(st, 2)) != hipSuccess) return err;  // h (and its split) written
  if ((err = br.await(sd, 2)) != hipSuccess) return err;
  if (a.small_tiles)
    MOE_LAUNCH(k_a2s, dim3(a.maxtiles * (TMG / GA2S::TM), rank_blocks(a.r)), dim3(GA2S::NT), GA2S::LDS_BYTES, sd,
               a);
  else
    MOE_LAUNCH(k_a2, dim3(a.maxtiles * A2_SUB, rank_blocks(a.r)), dim3(256), GS128::LDS_BYTES, sd, a);
  const long nzc = (long)a.T * (a.r / 4);
  MOE_LAUNCH(k_zc, dim3((unsigned)((nzc + 255) / 256)), dim3(256), 0, sd, a);
  {
    const dim3 g(a.maxtiles * (a.H / GW2::TN)), gs(g.x * (TMG / GW2S::TM));
    if (a.mx && a.W2P != nullptr)
      MOE_LAUNCH_AS("k_w2", (k_w2<true, true, false>), g, dim3(GW2::NT), W2_LDS, st, a);
    else if (a.mx)
      MOE_LAUNCH_AS("k_w2", (k_w2<true, false, false>), g, dim3(GW2::NT), W2_LDS, st, a);
    else if (a.small_tiles && a.W2P != nullptr)
      MOE_LAUNCH_AS("k_w2", (k_w2<false, true, true>), gs, dim3(GW2::NT), W2S_LDS, st, a);
    else if (a.small_tiles)
      MOE_LAUNCH_AS("k_w2", (k_w2<false, false, true>), gs, dim3(GW2::NT), W2S_LDS, st, a);
    else if (a.W2P != nullptr)
      MOE_LAUNCH_AS("k_w2", (k_w2<false, true, false>), g, dim3(GW2::NT), W2_LDS, st, a);
    else
      MOE_LAUNCH_AS("k_w2", (k_w2<false, false, false>), g, dim3(GW2::NT), W2_LDS, st, a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = br.close()) != hipSuccess) return err;
  MOE_LAUNCH(k_rank_combine, dim3(a.H / GRK::TN, token_tiles(a, GRK::TM)), dim3(GRK::NT), RK_LDS, st, a);
  return hipGetLastError();
}

}  // namespace moelora
