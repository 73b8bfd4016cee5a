// backward.hip -- backward of the MoE side-LoRA expert layer.
//
// DeepGEMM PR #9, "Historical implementation" -> Summary: the backward
// returns grad-x, router gradients and the six adapter gradients (no frozen
// weight gradients, no full-width side-delta scratch); padding never enters
// the shared reductions.  Steps:
//   k_q             q_t = B2^T go_t, once per token (B2 is shared)
//   k_transpose     A2T = A2_e^T, when the caller passes the transformed base
//                   (W13T, W2T: PR #9 Summary, reusable transformed weights)
//   k_w2dgrad       dh = w (W2_e^T go_t + A2_e^T s q_t) (K-extended), then
//                   the SwiGLU backward from the saved fp16 G, V; per column
//                   tile, the partial router gradient <W2_e^T go + A2_e^T s q, h>
//   k_dw            grad_w[t,j] = sum of those partials (= <go_t, y_tj>), and
//                   s w q_t per route for dA2
//   k_w13dgrad      dU = W1_e^T dg + W3_e^T dv
//   (with the transformed base both dgrads read the weights as K tiles)
//   k_p13           P = [B1_e^T dg ; B3_e^T dv] (at most half as many routes
//                   as pool groups: k_p13s on B1_e^T, B3_e^T copied by k_transpose)
//   k_pc            pc_t = s sum_j P_(t,j)
//   k_rank_dx       grad_x_t = [A1; A3]^T pc_t + sum_j dU_(t,j)
//   k_wgrad_local   dB1_e, dB3_e, dA2_e: K-grouped over the expert's rows
//   k_wgrad_shared  dA1, dA3, dB2: over tokens, deterministic split-K
//   k_reduce_shared fixed-order sum of the split-K partials
#include <type_traits>

#include "engine2.hpp"
#include "gather_sum.hpp"
#include "layer.hpp"
#include "trace.hpp"

namespace moelora {

// thin GEMMs (N = r): smaller M tiles so the grid fills the 256 CUs
using GS64 = Geo<1, 2, 2, 2>;   // 64 x 128 tile, wave 32 x 64
using GS128 = Geo<2, 2, 2, 2>;  // 128 x 128 tile, wave 64 x 64
constexpr int P13_SUB = TMG / GS128::TM;  // sub-tiles per pool M tile

// ----------------------------------------------------------------------------
// a8: q = B2^T go per token, router gradients
// ----------------------------------------------------------------------------
struct LdQ {
  RowsK<GS64::TM> m;
  TransK<128, KStrided> n;
  int k0;  // this split's first k
  __device__ void load(int s) { m.load(k0 + s * KT, 0, false); n.load(k0 + s * KT); }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

// One token tile (one root) and one of KSPLIT quarters of H per workgroup
// (B2 of the root's adapter): the partial products go to qp, summed in
// split order by k_q_sum.  The split is fixed, so a token's q does not
// depend on the batch.
__global__ __launch_bounds__(256) void k_q(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  int t0, nt, ad;
  if (!token_tile(a, blockIdx.x, GS64::TM, t0, nt, ad)) return;
  const int r = a.r, ks = blockIdx.y, kh = a.H / KSPLIT, c0 = RBLK * blockIdx.z;  // rank block c0..
  LdQ L;
  L.k0 = ks * kh;
  L.m.contig(a.go, t0, nt, a.H);
  L.m.window(a.H);
  L.n.kp = KStrided{make_rsrc(a.B2 + (long)ad * a.H * r, (uint64_t)a.H * r * 2), (uint32_t)(2 * r), 0, a.H, 0};
  L.n.cols(c0, r - c0);
  f32x16 acc[GS64::NB][GS64::MB];
  mainloop<GS64>(L, kh / KT, acc, smem);
  Epi<GS64> ep;
  float* part = a.qp + (long)ks * a.T * r;
#pragma unroll
  for (int mb = 0; mb < GS64::MB; ++mb) {
    const int t = t0 + ep.row(mb);
    if (t >= t0 + nt) continue;
#pragma unroll
    for (int nb = 0; nb < GS64::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = c0 + ep.col(nb, g);
        if (c >= r) continue;
        *(f32x4*)(part + (long)t * r + c) =
            f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
      }
  }
}

// q = the splits' partials in order; s q as hi/lo.  One thread per 4 columns.
__global__ __launch_bounds__(256) void k_q_sum(LayerArgs a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int g4 = a.r / 4;
  if (i >= (long)a.T * g4) return;
  const long t = i / g4;
  const int c = (int)(i % g4) * 4;
  f32x4 v = *(const f32x4*)(a.qp + t * a.r + c);
#pragma unroll
  for (int ks = 1; ks < KSPLIT; ++ks) {
    const f32x4 p = *(const f32x4*)(a.qp + ((long)ks * a.T + t) * a.r + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += p[q];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_hl(a.s * v[q], hi[q], lo[q]);
  *(f32x4*)(a.q + t * a.r + c) = v;
  uint16_t* d = a.sq + t * 2 * a.r + c;
  *(u32x2*)d = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
  *(u32x2*)(d + a.r) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
}

// one wave per route (t, j)
// ----------------------------------------------------------------------------
// a9: dh = w (W2_e^T go + A2_e^T s q), SwiGLU backward -> dG, dV
// ----------------------------------------------------------------------------
using GW2D = v2::Geo2<4, 2, 2, 4, false, true, 64>;  // 256 x 256, weights K-outer
// epilogue: two LDS images (dg, dv) and the router-gradient row sums of the
// WN column-wave groups
constexpr int W2D_IMG = v2::TileImage<GW2D, GW2D::TN / 2, uint16_t>::BYTES;
constexpr int W2D_LDS = cmax(GW2D::LDS_BYTES, 2 * W2D_IMG + GW2D::WN * GW2D::TM * 4);
// Stages [0, next): the A2^T (s q) extension (rank-r K); then the base K = H.
constexpr int PPW = 4;  // waves that queue a stage in the ping-pong loops (group A)

template <int NWL>
struct LdW2dBase {
  using KL = v2::KLoad<256, GW2D::KT, NWL>;
  using TL = v2::TLoad<256, v2::TStrided, GW2D::KT, NWL>;
  using KA = v2::KLoadA<256, GW2D::KT, NWL>;
  static constexpr int INSTS = KL::NJ + TL::NJ;
  KL me;
  KA mm;
  TL ne;
  int next;
};
// ping-pong form: the rank-space extension (K = 2r) runs first through the
// plain pipeline (LdW2dExt), then the base K = H through the ping-pong loop
// (LdW2dMain, queued by four waves)
struct LdW2dExt {
  using KL = v2::KLoad<256, GW2D::KT, GW2D::NW>;
  using TL = v2::TLoad<256, v2::TStrided, GW2D::KT, GW2D::NW>;
  static constexpr int INSTS = KL::NJ + TL::NJ;
  KL me;
  TL ne;
  __device__ void issue(int s, char* sM, char* sN) {
    me.issue(s * GW2D::KT, 0, false, sM);
    ne.issue(s * GW2D::KT, sN);
  }
};
struct LdW2dMain {
  using KA = v2::KLoadA<256, GW2D::KT, 4>;
  static constexpr int INSTS = 2 * KA::NJ;
  KA mm;
  v2::TLoadA<256, GW2D::KT, 4> nm;
  __device__ void issue(int s, char* sM, char* sN) {
    mm.issue(s * GW2D::KT, sM);
    nm.issue(s * GW2D::KT, sN);
  }
};
struct LdW2dMX : LdW2dBase<GW2D::NW> {
  v2::TLoadMX<GW2D::NT> nq;
  __device__ void issue(int s, char* sM, char* sN) {
    if (s < next) {
      me.issue(s * GW2D::KT, 0, false, sM);
      ne.issue(s * GW2D::KT, sN);
    } else {
      mm.issue((s - next) * GW2D::KT, sM);
      nq.issue((s - next) * GW2D::KT);
    }
  }
  __device__ void finish(int s, char* sN) const {
    if (s >= next) nq.finish(sN);
  }
};

// With the transformed base weights (W2T = W2_e^T per expert, [E, I, H]) both
// operands are K tiles read with ds_read_b128 instead of transposing reads:
// stages [0, next) contract s q with A2T = A2_e^T (rows i0.., K = r folded
// twice for the hi and lo halves), then go with W2T rows i0.. (K = H); one
// plain pipeline (the ping-pong form spills here).
using GW2DK = v2::Geo2<4, 2, 2, 4, false, false, 64>;
static_assert(GW2DK::TM == GW2D::TM && GW2DK::TN == GW2D::TN && GW2DK::STAGE == GW2D::STAGE,
              "same tile and stage as the transposing form");
// Few rows per expert (small T), with the transformed weights: 64-row parts
// of each pool tile and a third stage buffer (bitwise the same products and
// order as the full tile).
using GW2DS = v2::Geo2<1, 2, 2, 4, false, false, 64, 3>;
constexpr int W2DS_LDS = cmax(GW2DS::LDS_BYTES, 2 * v2::TileImage<GW2DS, GW2DS::TN / 2, uint16_t>::BYTES +
                                                    GW2DS::WN * GW2DS::TM * 4);
// The small parts' rank-space extension reads A2 itself (a T tile over its
// rows, as the transposing form does), so no A2^T copy is made for them.
using GW2DST = v2::Geo2<1, 2, 2, 4, false, true, 64, 3>;
static_assert(GW2DST::STAGE == GW2DS::STAGE && GW2DST::NBUF == GW2DS::NBUF, "one LDS plan for both loops");
struct LdW2dExtS {
  using KL = v2::KLoad<GW2DST::TM, GW2DST::KT, GW2DST::NW>;
  using TL = v2::TLoad<256, v2::TStrided, GW2DST::KT, GW2DST::NW>;
  static constexpr int INSTS = KL::NJ + TL::NJ;
  KL me;
  TL ne;
  __device__ void issue(int s, char* sM, char* sN) {
    me.issue(s * GW2DST::KT, 0, false, sM);
    ne.issue(s * GW2DST::KT, sN);
  }
};
template <class G>
struct LdW2dK {
  using KL = v2::KLoad<G::TM, G::KT, G::NW>;   // s q by token (M)
  using KN = v2::KLoad<256, G::KT, G::NW>;     // A2T rows (N)
  using KA = v2::KLoadA<G::TM, G::KT, G::NW>;  // go by token (M)
  using KP = v2::KLoadP<256, G::KT, G::NW>;    // W2T rows, packed (pack.hip, kind 3) (N)
  static_assert(KA::NJ == KL::NJ && KP::NJ == KN::NJ, "one instruction count per stage");
  static constexpr int INSTS = KL::NJ + KN::NJ;
  KL me;
  KN ne;
  KA mm;
  KP nm;
  int next;
  __device__ void issue(int s, char* sM, char* sN) {
    if (s < next) {
      me.issue(s * G::KT, 0, false, sM);
      ne.issue(s * G::KT, 0, false, sN);
    } else {
      mm.issue((s - next) * G::KT, sM);
      nm.issue((s - next) * G::KT, sN);
    }
  }
};

// ACT: 0 SwiGLU, 1 GeGLU (exact GELU): f'(g) = Phi(g) + g phi(g).
// TW: read the transformed weights (bf16 base only).
// CL: activation clamp (as in the forward): g, v clipped to [-a.clamp,
// a.clamp] before the activation; the clip passes gradient only where
// |x| <= a.clamp, decided on the saved fp16 values as the forward decided.
// SK (with TW): 64-row parts of the pool tiles (GW2DS); the grid is SUB
// times larger and part `sub` takes rows row0 + 64 sub ..; parts past the
// tile's rows return at once.
template <bool MX, int ACT, bool TW, bool CL, bool SK>
__global__ __launch_bounds__(GW2D::NT) void k_w2dgrad(LayerArgs a) {
  static_assert(!(MX && TW) && (TW || !SK), "transformed weights are bf16; small parts read them");
  extern __shared__ __align__(16) char smem[];
  using G = typename std::conditional<SK, GW2DS, typename std::conditional<TW, GW2DK, GW2D>::type>::type;
  constexpr int SUB = TMG / G::TM;
  const int ntn = a.I / G::TN;
  // part `sub` of pool tile work item b (SUB == 1: the block index itself)
  const int nb = SUB == 1 ? (int)gridDim.x : __builtin_amdgcn_readfirstlane(gridDim.x / SUB);
  const int b = SUB == 1 ? (int)blockIdx.x : __builtin_amdgcn_readfirstlane(blockIdx.x % nb);
  const int sub = SUB == 1 ? 0 : __builtin_amdgcn_readfirstlane(blockIdx.x / nb);
  int mt, nt;
  if (!group_tile(a, a.tiles, TMG, b, *a.ntiles, ntn, TILE_GM, mt, nt)) return;
  const TileInfo ti = a.tiles[mt];
  const int row0 = ti.row0 + sub * G::TM;
  if (row0 >= ti.row_end) return;
  const int i0 = nt * G::TN;
  const int nrows = ti.row_end - row0;  // rows to the expert's end (the tile holds at most TM of them)
  const int r = a.r;
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  const int next = (2 * r + G::KT - 1) / G::KT;
  const long e = grp_expert(a, ti.e), le = grp_local(a, ti.e);  // base expert; A2 of its adapter
  if constexpr (SK) {
    // the extension through A2 (T tile), then the base through W2T (packed K tile)
    {
      LdW2dExtS X;
      int tk[LdW2dExtS::KL::NJ];
      LdW2dExtS::KL::tokens(tk, a.row2r, a.k, row0, nrows);
      X.me.from_tokens(a.sq, a.T, 2 * r, tk);
      X.me.window(2 * r);
      X.ne.kp = v2::TStrided{make_rsrc(a.A2 + le * r * a.I, (uint64_t)r * a.I * 2), (uint32_t)(2 * a.I), 0, 2 * r, r};
      X.ne.cols(i0, G::TN);
      v2::run_stages2<GW2DST, 0>(X, next, acc, smem);
    }
    using LT = LdW2dK<G>;
    LT L;
    L.next = 0;
    {
      int tk[LT::KA::NJ];
      LT::KL::tokens(tk, a.row2r, a.k, row0, nrows);
      L.mm.from_tokens(a.go, a.T, a.H, tk);
    }
    L.nm.set(a.W2T + e * a.I * a.H, (uint64_t)a.I * a.H * 2, nt, a.H / G::KT);
    v2::run_stages2<G, 0>(L, a.H / G::KT, acc, smem);
  } else if constexpr (TW) {
    using LT = LdW2dK<G>;
    LT L;
    L.next = next;
    {
      int tk[LT::KL::NJ];
      LT::KL::tokens(tk, a.row2r, a.k, row0, nrows);
      L.me.from_tokens(a.sq, a.T, 2 * r, tk);
      L.mm.from_tokens(a.go, a.T, a.H, tk);
    }
    L.me.window(2 * r);
    L.ne.contig(a.A2T + le * a.I * r, i0, G::TN, r);
    L.ne.window(2 * r, r);  // k in [r, 2r) reads A2T column k - r again (lo half)
    L.nm.set(a.W2T + e * a.I * a.H, (uint64_t)a.I * a.H * 2, nt, a.H / G::KT);
    v2::run_stages2<G, 0>(L, next + a.H / G::KT, acc, smem);
  } else if constexpr (!MX) {
    {
      LdW2dExt X;
      int tk[LdW2dExt::KL::NJ];
      LdW2dExt::KL::tokens(tk, a.row2r, a.k, ti.row0, nrows);
      X.me.from_tokens(a.sq, a.T, 2 * r, tk);
      X.me.window(2 * r);
      X.ne.kp = v2::TStrided{make_rsrc(a.A2 + le * r * a.I, (uint64_t)r * a.I * 2),
                             (uint32_t)(2 * a.I), 0, 2 * r, r};
      X.ne.cols(i0, G::TN);
      v2::run_stages2<G, 0>(X, next, acc, smem);
    }
    LdW2dMain Mn;
    {
      int tk[LdW2dMain::KA::NJ];
      v2::KLoad<256, G::KT, 4>::tokens(tk, a.row2r, a.k, ti.row0, nrows);
      Mn.mm.from_tokens(a.go, a.T, a.H, tk);
    }
    Mn.nm.set(a.W2 + e * a.H * a.I, a.H, a.I, i0);
    v2::run_pingpong<G>(Mn, a.H / G::KT, acc, smem);
  } else {
    // MXFP4 base: the W2 tile is register-staged and expanded to bf16 in LDS
    LdW2dMX L;
    using KL = LdW2dMX::KL;
    L.next = next;
    {
      int tk[KL::NJ];
      KL::tokens(tk, a.row2r, a.k, ti.row0, nrows);
      L.me.from_tokens(a.sq, a.T, 2 * r, tk);
      L.mm.from_tokens(a.go, a.T, a.H, tk);
    }
    L.me.window(2 * r);
    L.ne.kp = v2::TStrided{make_rsrc(a.A2 + le * r * a.I, (uint64_t)r * a.I * 2),
                           (uint32_t)(2 * a.I), 0, 2 * r, r};
    L.ne.cols(i0, G::TN);
    L.nq.set(a.W2q + e * a.H * (a.I / 2), a.W2s + e * a.H * (a.I / 32), a.H, a.I, i0);
    v2::run_stages2<G, 0>(L, L.next + a.H / G::KT, acc, smem);
  }
  // G and V come in accumulator-blocked (as the forward wrote them); dg and
  // dv leave row-major through LDS images, one half of the tile's columns
  // (one accumulator block column per wave) at a time
  using Img = v2::TileImage<G, G::TN / 2, uint16_t>;
  static_assert(G::NB == 2, "one block column per half");
  Epi<G> ep;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform block offsets
  const int wm = wv / G::WN, wn = wv % G::WN, lane = threadIdx.x & 63;
  // router weights of the lane's rows; the row index is clamped to the
  // tile's last real row (nrows >= 1) so that all loads issue together
  int rr[G::MB];
  float wr[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) rr[mb] = a.row2r[row0 + min(ep.row(mb), nrows - 1)];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const float wt = a.w[rr[mb]];
    wr[mb] = ep.row(mb) < nrows ? wt : 0.0f;
  }
  char* img_g = smem;
  char* img_v = smem + Img::BYTES;
  uint16_t* out = a.dGV + row0 * 2 * (long)a.I + i0;
  // router gradient: grad_w = <go, W2 h + s B2 A2 h> = <W2^T go + A2^T s q, h>,
  // i.e. the row dot product of the (unweighted) accumulator with h, which
  // the SwiGLU below recomputes in fp32 from G and V
  float dw[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) dw[mb] = 0.0f;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    // all of this half's G and V loads first: one memory round trip per half
    // (the asm statement below orders memory operations, so loads issued
    // inside the loop would each wait for the previous step)
    f16x4 gq[G::MB][4], vq[G::MB][4];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const long ob =
          acc_block(mt, G::m_local(wm, mb) / 32 + sub * (G::TM / 32), (i0 + G::n_local(wn, nb)) / 32, a.I) + 4 * lane;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        gq[mb][g] = *(const f16x4*)(a.G + ob + 256 * g);
        vq[mb][g] = *(const f16x4*)(a.V + ob + 256 * g);
      }
    }
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 gg = __builtin_convertvector(gq[mb][g], f32x4);
        const f32x4 vv = __builtin_convertvector(vq[mb][g], f32x4);
        f32x4 dg, dv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float av = acc[nb][mb][4 * g + q];
          float gq = gg[q], vq = vv[q];
          bool pass_g = true, pass_v = true;
          if constexpr (CL) {
            pass_g = fabsf(gq) <= a.clamp;
            pass_v = fabsf(vq) <= a.clamp;
            if (!pass_g) gq = copysignf(a.clamp, gq);
            if (!pass_v) vq = copysignf(a.clamp, vq);
          }
          if constexpr (ACT == 0) {
            // silu'(g) = sg (1 + g (1 - sg)), so av silu'(g) = t + u - u sg
            const float sg = sigmoidf_(gq);
            const float t = av * sg;
            const float u = t * gq;  // unweighted dv = av silu(g)
            dw[mb] += u * vq;
            dv[q] = wr[mb] * u;
            dg[q] = wr[mb] * vq * (t + fmaf(-u, sg, u));
          } else {
            float cdf, pdf;
            norm_cdf_pdf(gq, cdf, pdf);
            const float u = av * gq * cdf;  // unweighted dv
            dw[mb] += u * vq;
            dv[q] = wr[mb] * u;
            dg[q] = wr[mb] * av * vq * fmaf(gq, pdf, cdf);
          }
          if constexpr (CL) {
            if (!pass_v) dv[q] = 0.0f;
            if (!pass_g) dg[q] = 0.0f;
          }
        }
        // keep the running sum in place: otherwise the compiler sinks the
        // whole dot product past the loop and holds its operands meanwhile
        asm volatile("" : "+v"(dw[mb]));
        const int col = ep.col(nb, g) - nb * (G::TN / 2);
        Img::put(img_g, ep.row(mb), col, dg);
        Img::put(img_v, ep.row(mb), col, dv);
      }
    }
    __syncthreads();
    Img::flush(img_g, out + nb * (G::TN / 2), 2 * a.I, nrows);
    Img::flush(img_v, out + a.I + nb * (G::TN / 2), 2 * a.I, nrows);
    __syncthreads();
  }
  // a row's 256 columns: two lanes (lane, lane ^ 32) in each of the WN waves
  // of its row group; summed in a fixed order
  float* red = (float*)(smem + 2 * Img::BYTES);  // [WN][TM]
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const float v = dw[mb] + __shfl_xor(dw[mb], 32, 64);
    if (lane < 32) red[wn * G::TM + ep.row(mb)] = v;
  }
  __syncthreads();
  // (nrows counts to the expert's end; this tile holds at most TM of them)
  for (int lr = threadIdx.x; lr < nrows && lr < G::TM; lr += G::NT) {
    float t = 0.0f;
#pragma unroll
    for (int c = 0; c < G::WN; ++c) t += red[c * G::TM + lr];
    a.dwp[(long)nt * a.cap + row0 + lr] = t;
  }
}

// Sixteen lanes per route: grad_w = the column tiles' partials summed in
// tile order; s w q (hi/lo) for the rank-space gradients, 8 columns a lane.
constexpr int DW_LANES = 16;
__global__ __launch_bounds__(256) void k_dw(LayerArgs a) {
  const long f = (long)blockIdx.x * (256 / DW_LANES) + (threadIdx.x / DW_LANES);
  const int sl = threadIdx.x % DW_LANES;
  if (f >= (long)a.T * a.k) return;
  const int t = (int)(f / a.k);
  const int row = a.r2row[f];
  if (row < 0) {
    if (sl == 0) a.gw[f] = 0.0f;
    return;
  }
  if (sl == 0) {
    const int ntn = a.I / GW2D::TN;
    const float* p = a.dwp + row;
    float acc = 0.0f;
    int n = 0;
    for (; n + 8 <= ntn; n += 8) {  // eight loads in flight, added in order
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = p[(long)(n + j) * a.cap];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j];
    }
    for (; n < ntn; ++n) acc += p[(long)n * a.cap];
    a.gw[f] = acc;
  }
  const float sw = a.s * a.w[f];
  for (int c = 8 * sl; c < a.r; c += 8 * DW_LANES) {  // r % 8 == 0
    const f32x4* qp = (const f32x4*)(a.q + (long)t * a.r + c);
    const f32x4 q0 = qp[0], q1 = qp[1];
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      split_hl(sw * q0[j], hi[j], lo[j]);
      split_hl(sw * q1[j], hi[4 + j], lo[4 + j]);
    }
    uint16_t* d = a.wsq + (long)row * 2 * a.r + c;
    *(u32x4*)d = u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
    *(u32x4*)(d + a.r) =
        u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
  }
}

// ----------------------------------------------------------------------------
// a10: dU = W13_e^T [dg; dv]   (K = 2I, weights read K-outer)
// ----------------------------------------------------------------------------
using GW13D = v2::Geo2<4, 2, 2, 4, false, true, 64>;  // 256 x 256, weights K-outer
constexpr int W13D_LDS = cmax(GW13D::LDS_BYTES, v2::TileImage<GW13D, GW13D::TN, uint16_t>::BYTES);
struct LdW13d {
  using KA = v2::KLoadS<256, GW13D::KT, PPW>;
  using TA = v2::TLoadA<256, GW13D::KT, PPW>;
  static constexpr int INSTS = KA::NJ + TA::NJ;
  KA m;
  TA n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW13D::KT, sM);
    n.issue(s * GW13D::KT, sN);
  }
};
struct LdW13dMX {
  using KA = v2::KLoadS<256, GW13D::KT, GW13D::NW>;
  static constexpr int INSTS = KA::NJ;
  KA m;
  v2::TLoadMX<GW13D::NT> nq;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW13D::KT, sM);
    nq.issue(s * GW13D::KT);
  }
  __device__ void finish(int, char* sN) const { nq.finish(sN); }
};

// With the transformed base weights (W13T = W13_e^T per expert, [E, H, 2I])
// the weight operand is a K tile: W13T rows h0.. (K = 2I contiguous).
using GW13DK = v2::Geo2<4, 2, 2, 4, false, false, 64>;
static_assert(GW13DK::TM == GW13D::TM && GW13DK::TN == GW13D::TN && GW13DK::STAGE == GW13D::STAGE,
              "same tile and stage as the transposing form");
struct LdW13dK {
  using KA = v2::KLoadS<256, GW13DK::KT, PPW>;
  using KP = v2::KLoadP<256, GW13DK::KT, PPW>;
  static_assert(KP::NJ == KA::NJ, "one instruction count per stage");
  static constexpr int INSTS = 2 * KA::NJ;
  KA m;   // dGV rows
  KP n;   // W13T rows, packed (pack.hip, kind 2)
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW13DK::KT, sM);
    n.issue(s * GW13DK::KT, sN);
  }
};

// Few rows per expert (small T), with the transformed weights: 64-row parts
// of each pool tile and a third stage buffer, one plain pipeline over all
// eight waves (bitwise the same products and order as the full tile).
using GW13DS = v2::Geo2<1, 2, 2, 4, false, false, 64, 3>;
constexpr int W13DS_LDS = cmax(GW13DS::LDS_BYTES, v2::TileImage<GW13DS, GW13DS::TN, uint16_t>::BYTES);
struct LdW13dS {
  using KA = v2::KLoadS<GW13DS::TM, GW13DS::KT, GW13DS::NW>;
  using KP = v2::KLoadP<256, GW13DS::KT, GW13DS::NW>;
  static constexpr int INSTS = KA::NJ + KP::NJ;
  KA m;   // dGV rows
  KP n;   // W13T rows, packed
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GW13DS::KT, sM);
    n.issue(s * GW13DS::KT, sN);
  }
};

// TW: read the transformed weights (bf16 base only).  SK (with TW): 64-row
// parts of the pool tiles; the grid is SUB times larger and part `sub` takes
// rows row0 + 64 sub ..; parts past the tile's rows return at once.
template <bool MX, bool TW, bool SK>
__global__ __launch_bounds__(GW13D::NT) void k_w13dgrad(LayerArgs a) {
  static_assert(!(MX && TW) && (TW || !SK), "transformed weights are bf16; small parts read them");
  extern __shared__ __align__(16) char smem[];
  using G = typename std::conditional<SK, GW13DS, typename std::conditional<TW, GW13DK, GW13D>::type>::type;
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
  const int nrows = ti.row_end - row0 < G::TM ? ti.row_end - row0 : G::TM;
  const int h0 = nt * G::TN;
  const long e = grp_expert(a, ti.e);
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  if constexpr (SK) {
    LdW13dS L;
    L.m.contig(a.dGV, row0, nrows, 2 * a.I);
    L.n.set(a.W13T + e * a.H * 2 * a.I, (uint64_t)a.H * 2 * a.I * 2, nt, 2 * a.I / G::KT);
    v2::run_stages2<G, 0>(L, 2 * a.I / G::KT, acc, smem);
  } else if constexpr (TW) {
    LdW13dK L;
    L.m.contig(a.dGV, ti.row0, ti.row_end - ti.row0, 2 * a.I);
    L.n.set(a.W13T + e * a.H * 2 * a.I, (uint64_t)a.H * 2 * a.I * 2, nt, 2 * a.I / G::KT);
    v2::run_pingpong<G>(L, 2 * a.I / G::KT, acc, smem);
  } else {
    typename std::conditional<MX, LdW13dMX, LdW13d>::type L;
    L.m.contig(a.dGV, ti.row0, ti.row_end - ti.row0, 2 * a.I);
    if constexpr (MX)
      L.nq.set(a.W13q + e * 2 * a.I * (a.H / 2), a.W13s + e * 2 * a.I * (a.H / 32), 2 * a.I, a.H, h0);
    else
      L.n.set(a.W13 + e * 2 * a.I * a.H, 2 * a.I, a.H, h0);
    if constexpr (!MX)
      v2::run_pingpong<G>(L, 2 * a.I / G::KT, acc, smem);
    else
      v2::run_stages2<G, 0>(L, 2 * a.I / G::KT, acc, smem);
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
  Img::flush(smem, a.dU + row0 * (long)a.H + h0, a.H, nrows);
}

// ----------------------------------------------------------------------------
// a11: P1 = B1_e^T dg, P3 = B3_e^T dv   (blockIdx.y selects)
// ----------------------------------------------------------------------------
struct LdP {
  RowsK<GS128::TM> m;
  TransK<128, KStrided> n;
  __device__ void load(int s) { m.load(s * KT, 0, false); n.load(s * KT); }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

__global__ __launch_bounds__(256) void k_p13(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  int mt, sub, y;
  if (!sub_tile(a, P13_SUB, mt, sub, y)) return;
  const int which = y & 1, c0 = RBLK * (y >> 1);  // rank block c0..
  const TileInfo ti = a.tiles[mt];
  const long row0 = ti.row0 + (long)sub * GS128::TM;  // this sub-tile's rows
  if (row0 >= ti.row_end) return;
  const int r = a.r;
  LdP L;
  L.m.contig(a.dGV + which * a.I, row0, ti.row_end - row0, 2 * a.I);
  L.m.window(a.I);
  const uint16_t* Be = (which ? a.B3 : a.B1) + grp_local(a, ti.e) * a.I * r;
  L.n.kp = KStrided{make_rsrc(Be, (uint64_t)a.I * r * 2), (uint32_t)(2 * r), 0, a.I, 0};
  L.n.cols(c0, r - c0);
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
        if (c >= r) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * g + q];
        *(f32x4*)(a.P + row * 2 * r + which * r + c) = v;
      }
  }
}

// At most half as many routes as pool groups (a few tokens): 64-row parts on
// the direct-load engine with four stage buffers (three stages queued), as
// k_a2s does for Z2, so the long K = I contraction is not bound by one load
// latency per stage.  The weight operand is B1_e^T / B3_e^T (K = I
// contiguous), transposed per call for the groups that hold rows (a cost that
// grows with them: at T = 90 on 64 experts the copies took longer than the
// faster product saved); the LDS tiles then hold what k_p13's transposing
// loads produce, and each element sums the same products in the same order.
using GP13S = v2::Geo2<1, 2, 2, 2, false, false, 64, 4>;  // 64 x 128, four waves
struct LdP13S {
  using KM = v2::KLoad<GP13S::TM, GP13S::KT, GP13S::NW>;  // dg or dv rows
  using KN = v2::KLoad<128, GP13S::KT, GP13S::NW>;        // B1_e^T or B3_e^T rows
  static constexpr int INSTS = KM::NJ + KN::NJ;
  KM m;
  KN n;
  __device__ void issue(int s, char* sM, char* sN) {
    m.issue(s * GP13S::KT, 0, false, sM);
    n.issue(s * GP13S::KT, 0, false, sN);
  }
};

__global__ __launch_bounds__(GP13S::NT) void k_p13s(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  using G = GP13S;
  constexpr int SUB = TMG / G::TM;
  int mt, sub, y;
  if (!sub_tile(a, SUB, mt, sub, y)) return;
  const int which = y & 1, c0 = RBLK * (y >> 1);  // rank block c0..
  const TileInfo ti = a.tiles[mt];
  const long row0 = ti.row0 + (long)sub * G::TM;  // this part's rows
  if (row0 >= ti.row_end) return;
  const int r = a.r;
  LdP13S L;
  L.m.contig(a.dGV + which * a.I, row0, ti.row_end - row0, 2 * a.I);
  L.m.window(a.I);
  L.n.contig((which ? a.B3T : a.B1T) + (grp_local(a, ti.e) * r + c0) * a.I, 0, r - c0, a.I);
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
        if (c >= r) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * g + q];
        *(f32x4*)(a.P + row * 2 * r + which * r + c) = v;
      }
  }
}

// pc_t = s * sum_j P_(t,j), written as hi/lo [pc1 hi | pc1 lo | pc3 hi | pc3 lo].
// One thread per token and 4 columns (never straddling pc1 / pc3, r % 8 ==
// 0): the token's route indices first, then one 16-byte P load per live
// route, added in route order.
__global__ __launch_bounds__(256) void k_pc(LayerArgs a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int r2 = 2 * a.r, g4 = r2 / 4;
  if (i >= (long)a.T * g4) return;
  const int t = (int)(i / g4), c = (int)(i % g4) * 4;
  int rows[16];  // topk <= 16
#pragma unroll
  for (int j = 0; j < 16; ++j) rows[j] = j < a.k ? a.r2row[t * a.k + j] : -1;
  f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (rows[j] < 0) continue;
    const f32x4 p = *(const f32x4*)(a.P + (long)rows[j] * r2 + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) z[q] += p[q];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_hl(a.s * z[q], hi[q], lo[q]);
  const int fac = c / a.r, cc = c - fac * a.r;
  uint16_t* d = a.pc + (long)t * 4 * a.r + fac * 2 * a.r + cc;
  *(u32x2*)d = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
  *(u32x2*)(d + a.r) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
}

// ----------------------------------------------------------------------------
// a12: grad_x = [A1; A3]^T pc + sum_j dU
// ----------------------------------------------------------------------------
// P = [A1; A3]^T pc_t for 128 tokens x 256 columns.  Stages [0, nst): pc
// columns [0, 2r) against A1 (hi/lo halves fold onto the same r columns);
// stages [nst, 2 nst): pc columns [2r, 4r) against A3.  The A factors come in
// transposed per call (A1T, A3T = A1^T, A3^T, [H, r], by k_transpose), so the
// N operand is a K tile of rows h0..; past 2r in a pass the A columns read
// zero.
struct LdRankDxK {
  using KM = v2::KLoad<GRK::TM, GRK::KT, GRK::NW>;
  using KN = v2::KLoad<GRK::TN, GRK::KT, GRK::NW>;
  static constexpr int INSTS = KM::NJ + KN::NJ;
  KM m;
  KN n1, n3;
  int nst, r;
  __device__ void issue(int s, char* sM, char* sN) {
    const bool second = s >= nst;
    const int k0 = (second ? s - nst : s) * GRK::KT;
    m.issue((second ? 2 * r : 0) + k0, 0, false, sM);
    if (second)
      n3.issue(k0, 0, false, sN);
    else
      n1.issue(k0, 0, false, sN);
  }
};

// grad_x = [A1; A3]^T pc_t + sum_j dU_(t,j) for 128 tokens x 256 columns
__global__ __launch_bounds__(GRK::NT, 2) void k_rank_dx(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  int t0, nt, ad;
  if (!token_tile(a, blockIdx.y, GRK::TM, t0, nt, ad)) return;
  const int h0 = blockIdx.x * GRK::TN;  // the column tiles of a token tile run side by side
  const int r = a.r;
  RouteVec rv;
  load_routes<false>(a, t0, t0 + nt, rv);
  LdRankDxK L;
  L.r = r;
  L.nst = (2 * r + GRK::KT - 1) / GRK::KT;
  L.m.contig(a.pc, t0, nt, 4 * r);
  L.m.window(4 * r);
  L.n1.contig(a.A1T + (long)ad * a.H * r, h0, GRK::TN, r);  // the root's adapter's factors
  L.n1.window(2 * r, r);
  L.n3.contig(a.A3T + (long)ad * a.H * r, h0, GRK::TN, r);
  L.n3.window(2 * r, r);
  f32x16 acc[GRK::NB][GRK::MB];
  zero_acc<GRK>(acc);
  v2::run_stages2<GRK, 0>(L, 2 * L.nst, acc, smem);
  rank_route_sum<false>(acc, smem, a, rv, a.dU, a.gx, t0, t0 + nt, h0);
}

// ----------------------------------------------------------------------------
// a13: expert-local adapter gradients, contracted over each expert's rows.
//   which 0: dB1_e[i][c] = sum_rows dg[row][i] * (s A1 u)[c]
//   which 1: dB3_e[i][c] = sum_rows dv[row][i] * (s A3 u)[c]
//   which 2: dA2_e[c][i] = sum_rows (s w q)[c] * h[row][i]
// K tiles start at the expert's first row and rows past its count read zero,
// so the sum never touches another expert and does not depend on BLOCK_M.
// Each workgroup takes one block of RBLK rank columns c0 .. (blockIdx.y / 3);
// that block's rank operand is hi/lo split along N (tile columns c and
// c + 128), the two halves added in the epilogue.  An expert with no rows
// writes zeros.
// ----------------------------------------------------------------------------
// ZA rows in pool order, so the weight-gradient kernel reads its rank
// operand as contiguous rows of each expert.  One wave per pool row.
__global__ __launch_bounds__(256) void k_gather_za(LayerArgs a) {
  const long p = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= a.offsets[a.EV]) return;
  const int f = a.row2r[p];
  if (f < 0) return;  // padding rows are never read
  const u32x4* src = (const u32x4*)(a.ZA + (long)(f / a.k) * 4 * a.r);
  u32x4* dst = (u32x4*)(a.ZAp + p * 4 * a.r);
  for (int c = lane; c < a.r / 2; c += 64) dst[c] = src[c];  // 4r bf16 = r/2 chunks of 16 bytes
}

// Both operands K-outer (K = the expert's rows): T tiles with a k window of
// the expert's row count (rows past it read zero).  Each stage re-bases the
// two descriptors at its first row, so the byte offsets stay small whatever
// the expert's row count.
using GWG = v2::Geo2<4, 2, 2, 4, true, true, 64>;
struct LdWg2 {
  using TL = v2::TLoad<256, v2::TStrided, GWG::KT, GWG::NW>;
  static constexpr int INSTS = 2 * TL::NJ;
  TL m, n;
  const char *mbase, *nbase;  // the expert's first row of each operand
  int ne;                     // the expert's row count
  // row-major sources with mld / nld bytes a row
  __device__ void set(const void* mrow0, uint32_t mld, const void* nrow0, uint32_t nld, int ne_) {
    mbase = (const char*)mrow0;
    nbase = (const char*)nrow0;
    ne = ne_;
    m.kp = v2::TStrided{make_rsrc(mbase, 0), mld, 0, 0, 0};  // per stage in issue
    n.kp = v2::TStrided{make_rsrc(nbase, 0), nld, 0, 0, 0};
  }
  __device__ void issue(int s, char* sM, char* sN) {
    const int k0 = s * GWG::KT, left = ne - k0;
    m.kp.rs = make_rsrc(mbase + (long)k0 * m.kp.ldb, (uint64_t)left * m.kp.ldb);
    n.kp.rs = make_rsrc(nbase + (long)k0 * n.kp.ldb, (uint64_t)left * n.kp.ldb);
    m.kp.span = left;
    n.kp.span = left;
    m.issue(0, sM);
    n.issue(0, sN);
  }
};
constexpr int WG_LDS = cmax(GWG::LDS_BYTES, 128 * (256 * 2 + 16));

__global__ __launch_bounds__(GWG::NT) void k_wgrad_local(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  using G = GWG;
  const int nti = a.I / 256;
  // an expert's column tiles share its rank operand rows: keep them on one
  // XCD (each XCD walks a contiguous range of tiles), so its L2 serves them
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int e = b / nti, i0 = (b % nti) * 256, which = blockIdx.y % 3;  // e: pool group
  const int c0 = RBLK * (blockIdx.y / 3), rc = min(RBLK, a.r - c0);    // rank block c0 .. c0 + rc - 1
  const long le = grp_local(a, e);  // output slot of the group's expert-local factors
  const int r = a.r;
  const int ne = a.counts[e], off = a.offsets[e];
  LdWg2 L;
  if (which < 2) {
    L.set(a.dGV + (long)off * 2 * a.I, (uint32_t)(4 * a.I), a.ZAp + (long)off * 4 * r, (uint32_t)(8 * r), ne);
    L.m.cols(which * a.I + i0, 256);
    L.n.cols(which * 2 * r + c0, rc, 128, r);
  } else {
    L.set(a.Hh + (long)off * a.I, (uint32_t)(2 * a.I), a.wsq + (long)off * 2 * r, (uint32_t)(4 * r), ne);
    L.m.cols(i0, 256);
    L.n.cols(c0, rc, 128, r);
  }
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  v2::run_stages2<G, 0>(L, (ne + G::KT - 1) / G::KT, acc, smem);
  // hi + lo halves of the rank operand (tile columns c and c + 128) add up
  Epi<G> ep;
  static_assert(G::NB == 2, "one hi and one lo block per wave");
  const int cpr = rc / 8;  // 16-byte chunks of the block's columns in an output row (r % 8 == 0)
  if (which < 2) {
    // dB[e][i][c]: image rows i, columns c (pitch 128 + 8 bf16)
    constexpr int P = 128 * 2 + 16;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ep.col(0, g);
        u32x2 v;
        v[0] = pack2(acc[0][mb][4 * g] + acc[1][mb][4 * g], acc[0][mb][4 * g + 1] + acc[1][mb][4 * g + 1]);
        v[1] = pack2(acc[0][mb][4 * g + 2] + acc[1][mb][4 * g + 2], acc[0][mb][4 * g + 3] + acc[1][mb][4 * g + 3]);
        *(u32x2*)(smem + ep.row(mb) * P + c * 2) = v;
      }
    __syncthreads();
    uint16_t* d = (which ? a.dB3 : a.dB1) + (le * a.I + i0) * r + c0;
    for (int idx = threadIdx.x; idx < 256 * cpr; idx += G::NT) {
      const int row = idx / cpr, ch = idx - row * cpr;
      *(u32x4*)(d + (long)row * r + 8 * ch) = *(const u32x4*)(smem + row * P + 16 * ch);
    }
  } else {
    // dA2[e][c][i]: image rows c, columns i (pitch 256 + 8 bf16)
    constexpr int P = 256 * 2 + 16;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ep.col(0, g), i = ep.row(mb);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(uint16_t*)(smem + (c + q) * P + i * 2) = (uint16_t)f2bf(acc[0][mb][4 * g + q] + acc[1][mb][4 * g + q]);
      }
    __syncthreads();
    uint16_t* d = a.dA2 + (le * r + c0) * a.I + i0;
    for (int idx = threadIdx.x; idx < rc * 32; idx += G::NT) {
      const int c = idx / 32, ch = idx - c * 32;
      *(u32x4*)(d + (long)c * a.I + 8 * ch) = *(const u32x4*)(smem + c * P + 16 * ch);
    }
  }
}

// ----------------------------------------------------------------------------
// a14: shared-factor gradients over tokens (no pool rows involved):
//   which 0: dA1[c][h] = sum_t (s pc1)[t][c] x[t][h]   (x_t from the saved copy)
//   which 1: dA3[c][h] = sum_t (s pc3)[t][c] x[t][h]
//   which 2: dB2[h][c] = sum_t go[t][h] zc[t][c]
// Each root's token range split in fixed chunks of kspl tokens (the chunks
// of all roots numbered in root order); a root's partials are summed in
// chunk order into its adapter's gradients.
// ----------------------------------------------------------------------------
// Both operands K-outer (K = the split's tokens), as in k_wgrad_local.
__global__ __launch_bounds__(GWG::NT) void k_wgrad_shared(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  using G = GWG;
  const int ntm = a.H / 256;
  const int h0 = (blockIdx.x % ntm) * 256, sp = blockIdx.x / ntm, which = blockIdx.y % 3;
  const int r = a.r, c0 = RBLK * (blockIdx.y / 3), rc = min(RBLK, r - c0);  // rank block c0 ..
  int tb, nt, ad;
  if (!token_tile(a, sp, a.kspl, tb, nt, ad)) return;
  LdWg2 L;
  const uint16_t* mrow0 = (which < 2 ? a.Xs : a.go) + (long)tb * a.H;  // x_t from the forward's saved copy
  if (which < 2) {
    L.set(mrow0, (uint32_t)(2 * a.H), a.pc + (long)tb * 4 * r, (uint32_t)(8 * r), nt);
    L.n.cols(which * 2 * r + c0, rc, 128, r);
  } else {
    L.set(mrow0, (uint32_t)(2 * a.H), a.zc + (long)tb * 2 * r, (uint32_t)(4 * r), nt);
    L.n.cols(c0, rc, 128, r);
  }
  L.m.cols(h0, 256);
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  v2::run_stages2<G, 0>(L, (nt + G::KT - 1) / G::KT, acc, smem);
  // hi + lo halves of the rank operand (tile columns c and c + 128) add up
  Epi<G> ep;
  static_assert(G::NB == 2, "one hi and one lo block per wave");
  float* part = a.part + ((long)which * a.nsplit + sp) * (long)a.H * r;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    const int h = h0 + ep.row(mb);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = c0 + ep.col(0, g);
      if (c >= r) continue;
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = acc[0][mb][4 * g + q] + acc[1][mb][4 * g + q];
      if (which < 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) part[(long)(c + q) * a.H + h] = v[q];  // [c][h]
      } else {
        *(f32x4*)(part + (long)h * r + c) = v;  // [h][c]
      }
    }
  }
}

// Adapter blockIdx.z: the partials of its root's chunks, in chunk order (an
// empty root writes zeros).
__global__ __launch_bounds__(256) void k_reduce_shared(LayerArgs a) {
  const long n = (long)a.H * a.r;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int which = blockIdx.y, ad = blockIdx.z;
  if (i >= n) return;
  int c0 = 0;
  for (int q = 0; q < ad; ++q) c0 += (a.roots[q + 1] - a.roots[q] + a.kspl - 1) / a.kspl;
  const int nc = (a.roots[ad + 1] - a.roots[ad] + a.kspl - 1) / a.kspl;
  const float* p = a.part + ((long)which * a.nsplit + c0) * n + i;
  float s = 0.0f;
  for (int sp = 0; sp < nc; ++sp) s += p[(long)sp * n];
  uint16_t* d = which == 0 ? a.dA1 : (which == 1 ? a.dA3 : a.dB2);
  d[(long)ad * n + i] = (uint16_t)f2bf(s);
}

// ----------------------------------------------------------------------------
// a13, optional (the frozen-weight gradients of the ordinary path):
//   dW13_e = sum over e's rows of [dg; dv] u^T     ([2I, H])
//   dW2_e  = sum over e's rows of (w go) h^T       ([H, I])
// K-grouped over the expert's rows like the adapter gradients.  The token
// operand is first laid out in pool order -- x rows, or w * go rounded to
// bf16 -- in the dU space, which nothing reads after the grad-x sum.
// ----------------------------------------------------------------------------
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void k_pool_rows(LayerArgs a, const uint16_t* src, uint16_t* dst) {
  const long p = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= a.offsets[a.EV]) return;
  const int f = a.row2r[p];
  if (f < 0) return;  // padding rows are never read
  const u32x4* s = (const u32x4*)(src + (long)(f / a.k) * a.H);
  u32x4* d = (u32x4*)(dst + p * a.H);
  const float wr = WEIGHTED ? a.w[f] : 1.0f;
  for (int c = lane; c < a.H / 8; c += 64) {
    u32x4 v = s[c];
    if (WEIGHTED) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pack2(wr * bf2f(v[q] & 0xffffu), wr * bf2f(v[q] >> 16));
    }
    d[c] = v;
  }
}

using BaseImg = v2::TileImage<GWG, GWG::TN / 2, uint16_t>;
static_assert(BaseImg::BYTES <= WG_LDS, "epilogue image fits the pipeline's LDS");

// which 0: dW13 (M = 2I columns of dG|dV, N = H columns of x in pool order);
// which 1: dW2 (M = H columns of w go in pool order, N = I columns of h).
// Tiles of one expert are consecutive, N fastest, and each XCD walks a
// contiguous range of them.
__global__ __launch_bounds__(GWG::NT) void k_wgrad_base(LayerArgs a, int which) {
  extern __shared__ __align__(16) char smem[];
  using G = GWG;
  const int M = which == 0 ? 2 * a.I : a.H, N = which == 0 ? a.H : a.I;
  const int ntn = N / G::TN, per = (M / G::TM) * ntn;
  const int b = xcd_remap(blockIdx.x, a.E * per);
  const int e = b / per, mt = (b % per) / ntn, nt = b % ntn;
  const int ne = a.counts[e], off = a.offsets[e];
  const uint16_t* ms = which == 0 ? a.dGV : a.dU;  // pool-ordered [rows, M]
  const uint16_t* ns = which == 0 ? a.dU : a.Hh;   // pool-ordered [rows, N]
  LdWg2 L;
  L.set(ms + (long)off * M, (uint32_t)(2 * M), ns + (long)off * N, (uint32_t)(2 * N), ne);
  L.m.cols(mt * G::TM, G::TM);
  L.n.cols(nt * G::TN, G::TN);
  f32x16 acc[G::NB][G::MB];
  zero_acc<G>(acc);
  v2::run_stages2<G, 0>(L, (ne + G::KT - 1) / G::KT, acc, smem);  // an empty expert writes zeros
  uint16_t* out = (which == 0 ? a.dW13 : a.dW2) + (long)e * M * N + (long)mt * G::TM * N + nt * G::TN;
  Epi<G> ep;
  static_assert(G::NB == 2, "one block column per half");
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        BaseImg::put(smem, ep.row(mb), ep.col(nb, g) - nb * (G::TN / 2),
                     f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                           acc[nb][mb][4 * g + 3]});
    __syncthreads();
    BaseImg::flush(smem, out + nb * (G::TN / 2), N, G::TM);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// [B, R, C] -> [B, C, R] (bf16 bits) through a 64 x 64 LDS tile: the
// transformed base weights (PR #9 Summary: reusable transformed weights) and
// A2T = A2_e^T for the transformed-weight W2 dgrad.  16-byte row accesses
// where the row is whole, element accesses at ragged edges.
// ----------------------------------------------------------------------------
// A second pair (src2, dst2) of the same shape is done by the same launch
// (grid z 2B).  With counts, matrix b = q E + e of an [na, E, ...] stack is
// skipped when its pool group e na + q holds no rows (nothing reads its copy).
__global__ __launch_bounds__(256) void k_transpose(const uint16_t* src, uint16_t* dst, const uint16_t* src2,
                                                   uint16_t* dst2, int B, int R, int C, const int32_t* counts,
                                                   int na, int E) {
  __shared__ uint16_t t[64][72];  // padded rows: 144 bytes, keeps the 16-byte writes aligned
  long b = blockIdx.z;
  if (b >= B) {
    b -= B;
    src = src2;
    dst = dst2;
  }
  if (counts != nullptr && counts[(b % E) * na + b / E] == 0) return;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  src += b * (long)R * C;
  dst += b * (long)R * C;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rr = threadIdx.x / 8 + 32 * p, cc = (threadIdx.x % 8) * 8;
    const int r = r0 + rr, c = c0 + cc;
    if (r < R && c + 8 <= C && C % 8 == 0) {
      *(u32x4*)&t[rr][cc] = *(const u32x4*)(src + (long)r * C + c);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) t[rr][cc + q] = (r < R && c + q < C) ? src[(long)r * C + c + q] : 0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int cr = threadIdx.x / 8 + 32 * p, rc = (threadIdx.x % 8) * 8;
    const int c = c0 + cr, r = r0 + rc;
    if (c >= C) continue;
    if (r + 8 <= R && R % 8 == 0) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = (uint32_t)t[rc + 2 * q][cr] | ((uint32_t)t[rc + 2 * q + 1][cr] << 16);
      *(u32x4*)(dst + (long)c * R + r) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (r + q < R) dst[(long)c * R + r + q] = t[rc + q][cr];
    }
  }
}


hipError_t launch_transpose(const uint16_t* src, uint16_t* dst, int B, int R, int C, hipStream_t st,
                            const int32_t* counts, int na, int E, const uint16_t* src2, uint16_t* dst2) {
  if (B <= 0 || R <= 0 || C <= 0) return hipSuccess;
  if (counts != nullptr && (E <= 0 || B != na * E)) return hipErrorInvalidValue;
  const unsigned nz = (unsigned)B * (src2 != nullptr ? 2u : 1u);
  MOE_LAUNCH(k_transpose, dim3((C + 63) / 64, (R + 63) / 64, nz), dim3(256), 0, st, src, dst, src2, dst2, B, R, C,
             counts, na, E);
  return hipGetLastError();
}


template <bool MX, int ACT, bool TW, bool CL, bool SK>
static void launch_w2d(const LayerArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (SK)
    MOE_LAUNCH_AS("k_w2dgrad", (k_w2dgrad<MX, ACT, TW, CL, SK>), dim3(grid.x * (TMG / GW2DS::TM)), dim3(GW2D::NT),
                  W2DS_LDS, st, a);
  else
    MOE_LAUNCH_AS("k_w2dgrad", (k_w2dgrad<MX, ACT, TW, CL, SK>), grid, dim3(GW2D::NT), W2D_LDS, st, a);
}
template <bool MX, bool TW, bool SK>
static void launch_w2d_var(const LayerArgs& a, dim3 grid, hipStream_t st) {
  const bool cl = a.clamp > 0.0f;
  if (a.act == 1 && cl)
    launch_w2d<MX, 1, TW, true, SK>(a, grid, st);
  else if (a.act == 1)
    launch_w2d<MX, 1, TW, false, SK>(a, grid, st);
  else if (cl)
    launch_w2d<MX, 0, TW, true, SK>(a, grid, st);
  else
    launch_w2d<MX, 0, TW, false, SK>(a, grid, st);
}
template <bool MX, bool TW, bool SK>
static void set_w2d_lds(AttrInit& ai) {
  const int lds = SK ? W2DS_LDS : W2D_LDS;
  ai.lds((const void*)k_w2dgrad<MX, 0, TW, false, SK>, lds);
  ai.lds((const void*)k_w2dgrad<MX, 1, TW, false, SK>, lds);
  ai.lds((const void*)k_w2dgrad<MX, 0, TW, true, SK>, lds);
  ai.lds((const void*)k_w2dgrad<MX, 1, TW, true, SK>, lds);
}

hipError_t launch_backward(const LayerArgs& a, hipStream_t st) {
  static PerDeviceOnce attrs;
  const hipError_t ierr = attrs.run([] {
    AttrInit ai;
    ai.lds((const void*)k_q, GS64::LDS_BYTES);
    set_w2d_lds<false, false, false>(ai);
    set_w2d_lds<true, false, false>(ai);
    set_w2d_lds<false, true, false>(ai);
    set_w2d_lds<false, true, true>(ai);
    ai.lds((const void*)k_w13dgrad<false, false, false>, W13D_LDS);
    ai.lds((const void*)k_w13dgrad<true, false, false>, W13D_LDS);
    ai.lds((const void*)k_w13dgrad<false, true, false>, W13D_LDS);
    ai.lds((const void*)k_w13dgrad<false, true, true>, W13DS_LDS);
    ai.lds((const void*)k_p13, GS128::LDS_BYTES);
    ai.lds((const void*)k_p13s, GP13S::LDS_BYTES);
    ai.lds((const void*)k_rank_dx, RK_LDS);
    ai.lds((const void*)k_wgrad_local, WG_LDS);
    ai.lds((const void*)k_wgrad_base, WG_LDS);
    ai.lds((const void*)k_wgrad_shared, GWG::LDS_BYTES);
    return ai.err;
  });
  if (ierr != hipSuccess) return ierr;
  // Two streams: the branch gathers ZA to pool order and copies the rank
  // factors' transposes while the caller's stream runs q and the W2 dgrad;
  // once dG, dV and s w q exist the branch computes P, pc and the adapter
  // gradients while the caller's stream runs the W13 dgrad, then grad-x
  // (after pc); the optional frozen-weight gradients follow the join.  With
  // 768 or more routes per pool group the W13 dgrad fills the device alone
  // (the concurrent branch slowed the backward at the production share,
  // 5.81 -> 5.88 ms, same box), so that second part stays on the caller's
  // stream.
  Branch br;
  hipError_t e = br.open(st, true);
  if (e != hipSuccess) return e;
  const hipStream_t sd = br.side();
  const bool deep = (long)a.T * a.k >= 768L * a.EV;
  const hipStream_t sp = deep ? st : sd;  // stream of P, pc and the adapter gradients
  const long used_rows = a.cap;  // grid bound; rows past the pool's end return at once
  MOE_LAUNCH(k_gather_za, dim3((unsigned)((used_rows + 3) / 4)), dim3(256), 0, sd, a);
  if ((e = launch_transpose(a.A1, a.A1T, a.na, a.r, a.H, sd, nullptr, 1, 0, a.A3, a.A3T)) != hipSuccess) return e;
  if (a.few_routes &&
      (e = launch_transpose(a.B1, a.B1T, a.na * a.E, a.I, a.r, sd, a.counts, a.na, a.E, a.B3, a.B3T)) != hipSuccess)
    return e;
  if ((e = br.signal(sd, 3)) != hipSuccess) return e;  // ZA rows and the transposes written
  MOE_LAUNCH(k_q, dim3(token_tiles(a, GS64::TM), KSPLIT, rank_blocks(a.r)), dim3(256), GS64::LDS_BYTES, st, a);
  MOE_LAUNCH(k_q_sum, dim3((unsigned)(((long)a.T * (a.r / 4) + 255) / 256)), dim3(256), 0, st, a);
  {
    const dim3 grid(a.maxtiles * (a.I / GW2D::TN));
    const bool tw = a.W2T != nullptr;  // bf16 base, or the dequantised copy of an MXFP4 base
    if (tw && !a.small_tiles) {  // the small parts read A2 directly
      // A2T = A2_e^T per expert and adapter ([na, E, I, r]), the K-tile rank operand
      if ((e = launch_transpose(a.A2, a.A2T, a.na * a.E, a.r, a.I, st)) != hipSuccess) return e;
    }
    if (tw)
      a.small_tiles ? launch_w2d_var<false, true, true>(a, grid, st) : launch_w2d_var<false, true, false>(a, grid, st);
    else if (a.mx)
      launch_w2d_var<true, false, false>(a, grid, st);
    else
      launch_w2d_var<false, false, false>(a, grid, st);
  }
  const long nr = (long)a.T * a.k, dw_per_block = 256 / DW_LANES;
  MOE_LAUNCH(k_dw, dim3((unsigned)((nr + dw_per_block - 1) / dw_per_block)), dim3(256), 0, st, a);
  if ((e = br.signal(st, 1)) != hipSuccess) return e;  // dG, dV, s w q written
  {
    const dim3 grid(a.maxtiles * (a.H / GW13D::TN));
    if (a.W13T != nullptr && a.small_tiles)
      MOE_LAUNCH_AS("k_w13dgrad", (k_w13dgrad<false, true, true>), dim3(grid.x * (TMG / GW13DS::TM)),
                    dim3(GW13D::NT), W13DS_LDS, st, a);
    else if (a.W13T != nullptr)
      MOE_LAUNCH_AS("k_w13dgrad", (k_w13dgrad<false, true, false>), grid, dim3(GW13D::NT), W13D_LDS, st, a);
    else if (a.mx)
      MOE_LAUNCH_AS("k_w13dgrad", (k_w13dgrad<true, false, false>), grid, dim3(GW13D::NT), W13D_LDS, st, a);
    else
      MOE_LAUNCH_AS("k_w13dgrad", (k_w13dgrad<false, false, false>), grid, dim3(GW13D::NT), W13D_LDS, st, a);
  }
  // P, pc and the adapter gradients: on the branch once the W2 dgrad's
  // outputs exist (event 1); deep, on the caller's stream once the branch's
  // first part (ZA rows, transposes: event 3) is done
  if ((e = br.await(sp, deep ? 3 : 1)) != hipSuccess) return e;
  if (a.few_routes)
    MOE_LAUNCH(k_p13s, dim3(a.maxtiles * (TMG / GP13S::TM), 2 * rank_blocks(a.r)), dim3(GP13S::NT),
               GP13S::LDS_BYTES, sp, a);
  else
    MOE_LAUNCH(k_p13, dim3(a.maxtiles * P13_SUB, 2 * rank_blocks(a.r)), dim3(256), GS128::LDS_BYTES, sp, a);
  const long npc = (long)a.T * (2 * a.r / 4);
  MOE_LAUNCH(k_pc, dim3((unsigned)((npc + 255) / 256)), dim3(256), 0, sp, a);
  if ((e = br.signal(sp, 2)) != hipSuccess) return e;  // pc written (and A1^T, A3^T before it)
  MOE_LAUNCH(k_wgrad_local, dim3(a.EV * (a.I / 256), 3 * rank_blocks(a.r)), dim3(GWG::NT), WG_LDS, sp, a);
  MOE_LAUNCH(k_wgrad_shared, dim3((a.H / 256) * a.nsplit, 3 * rank_blocks(a.r)), dim3(GWG::NT), GWG::LDS_BYTES,
             sp, a);
  const long nsh = (long)a.H * a.r;
  MOE_LAUNCH(k_reduce_shared, dim3((unsigned)((nsh + 255) / 256), 3, a.na), dim3(256), 0, sp, a);
  if (!deep && (e = br.await(st, 2)) != hipSuccess) return e;
  MOE_LAUNCH(k_rank_dx, dim3(a.H / GRK::TN, token_tiles(a, GRK::TM)), dim3(GRK::NT), RK_LDS, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = br.close()) != hipSuccess) return e;
  if (a.dW13 != nullptr || a.dW2 != nullptr) {  // one adapter only (pool groups = experts)
    const unsigned prow = (unsigned)((a.cap + 3) / 4);  // rows past the pool's end return at once
    if (a.dW13 != nullptr) {
      MOE_LAUNCH(k_pool_rows<false>, dim3(prow), dim3(256), 0, st, a, a.Xs, a.dU);
      MOE_LAUNCH_AS("k_wgrad_w13", k_wgrad_base, dim3(a.E * (2 * a.I / GWG::TM) * (a.H / GWG::TN)), dim3(GWG::NT),
                    WG_LDS, st, a, 0);
    }
    if (a.dW2 != nullptr) {
      MOE_LAUNCH(k_pool_rows<true>, dim3(prow), dim3(256), 0, st, a, a.go, a.dU);
      MOE_LAUNCH_AS("k_wgrad_w2", k_wgrad_base, dim3(a.E * (a.H / GWG::TM) * (a.I / GWG::TN)), dim3(GWG::NT),
                    WG_LDS, st, a, 1);
    }
  }
  return hipGetLastError();
}

}  // namespace moelora
