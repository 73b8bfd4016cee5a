// gather_sum.hpp -- per-token sums over a token's routes:
//
//   out[t, h] = P[t, h] + sum_j c_tj R[route_tj row, h]
//
// The forward combine (mixture output, c = routing weight, R = the routes'
// base outputs, P = B2 zc_t with zc_t = s sum_j w_tj z_tj) and the input
// gradient (c = 1, R = the routes' W13^T [dg; dv], P = [A1; A3]^T pc_t) have
// this form.  P is a rank-r product per token: a 128-token x 256-column tile
// of it is one MFMA GEMM (k_rank_combine, k_rank_dx), and the route sum is
// that GEMM's epilogue (rank_route_sum below), so P never leaves the chip:
// one column half of the tile at a time is parked in LDS as fp32, then each
// 16-lane group takes one token, 8 columns a lane, loads the token's route
// rows (two tokens and up to eight routes a lane in flight) and writes the
// bf16 result.  The route rows add in route order j = 0, 1, ... after P, so
// the result does not depend on the pool layout.  A workgroup holds under
// half of a CU's LDS and registers, so two run on each CU and one's GEMM
// overlaps the other's route stream.
#pragma once
#include "engine2.hpp"
#include "layer.hpp"

namespace moelora {

// 128-token x 256-column tiles of P; four waves of 64 x 128, 32-k stages,
// three stage buffers.
using GRK = v2::Geo2<2, 4, 2, 2, false, false, 32, 3>;
using RankImg = v2::TileImage<GRK, GRK::TN / 2, float>;
constexpr int RK_LDS = cmax(GRK::LDS_BYTES, RankImg::BYTES);

constexpr int RS_TPT = 2;   // tokens a thread carries per step
constexpr int RS_JC = 8;    // route rows loaded per token before any is added
constexpr int RS_TOK = GRK::TM / (GRK::NT / 16);  // tokens per thread over the tile (8)
static_assert(GRK::TN / 2 == 16 * 8, "a 16-lane group covers one half row");
static_assert(2 * RK_LDS <= 160 * 1024, "two workgroups a CU");
static_assert(RS_TOK % RS_TPT == 0, "whole steps");

// Lane-distributed routes of the thread's tokens: for token slot i, lane g*16
// + j of each 16-lane group g holds route j's pool row (-1: dead route, or a
// token past the tile) and its coefficient (0 for a dead route, whose weight is not
// read).  topk <= 16.
struct RouteVec {
  int row[RS_TOK];
  float c[RS_TOK];
};

// Token slot i of thread (wave w, lane): tile row i * NT / 16 + 4 w + lane / 16.
__device__ __forceinline__ int rs_token(int i) {
  return i * (GRK::NT / 16) + 4 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 4);
}

// Issued before the GEMM, so the index loads are long done when the sum runs.
// The tile's tokens are t0 .. tend - 1.
template <bool WEIGHTED>
__device__ __forceinline__ void load_routes(const LayerArgs& a, int t0, int tend, RouteVec& rv) {
  const int j = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < RS_TOK; ++i) {
    const int t = t0 + rs_token(i);
    int row = -1;
    float c = 0.0f;
    if (t < tend && j < a.k) {
      row = a.r2row[(long)t * a.k + j];
      if (row >= 0) c = WEIGHTED ? a.w[(long)t * a.k + j] : 1.0f;
    }
    rv.row[i] = row;
    rv.c[i] = c;
  }
}

// acc holds the tile's P (tokens t0.., columns h0..); out rows t0 .. tend-1.
template <bool WEIGHTED>
__device__ __forceinline__ void rank_route_sum(const f32x16 (&acc)[GRK::NB][GRK::MB], char* smem,
                                               const LayerArgs& a, const RouteVec& rv,
                                               const uint16_t* __restrict__ R,
                                               uint16_t* __restrict__ out, int t0, int tend, int h0) {
  constexpr int NH = GRK::NB / 2;  // block columns per half (n_local: blocks [0, NH) in the first half)
  Epi<GRK> ep;
  const int lane = threadIdx.x & 63, gbase = lane & 48, li = lane & 15;
  const long H = a.H;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int nn = 0; nn < NH; ++nn)
#pragma unroll
      for (int mb = 0; mb < GRK::MB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nb = hf * NH + nn;
          RankImg::put(smem, ep.row(mb), ep.col(nb, g) - hf * (GRK::TN / 2),
                       f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                             acc[nb][mb][4 * g + 3]});
        }
    __syncthreads();
    const int hc = h0 + hf * (GRK::TN / 2) + 8 * li;
#pragma unroll
    for (int i0 = 0; i0 < RS_TOK; i0 += RS_TPT) {
      float o[RS_TPT][8];
#pragma unroll
      for (int u = 0; u < RS_TPT; ++u) {
        const char* pp = smem + rs_token(i0 + u) * RankImg::PITCH + 32 * li;
        const f32x4 p0 = *(const f32x4*)pp, p1 = *(const f32x4*)(pp + 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[u][q] = p0[q];
          o[u][4 + q] = p1[q];
        }
      }
      for (int j0 = 0; j0 < a.k; j0 += RS_JC) {
        u32x4 y[RS_TPT][RS_JC];
        float c[RS_TPT][RS_JC];
#pragma unroll
        for (int u = 0; u < RS_TPT; ++u)
#pragma unroll
          for (int jj = 0; jj < RS_JC; ++jj) {
            // j < 16: lanes past topk hold row -1 and weight 0
            const int src = gbase | (j0 + jj);
            const int row = __shfl(rv.row[i0 + u], src, 64);
            c[u][jj] = __shfl(rv.c[i0 + u], src, 64);
            y[u][jj] = row >= 0 ? *(const u32x4*)(R + (long)row * H + hc) : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
        for (int u = 0; u < RS_TPT; ++u)
#pragma unroll
          for (int jj = 0; jj < RS_JC; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              o[u][2 * q] += c[u][jj] * bf2f(y[u][jj][q] & 0xffffu);
              o[u][2 * q + 1] += c[u][jj] * bf2f(y[u][jj][q] >> 16);
            }
      }
#pragma unroll
      for (int u = 0; u < RS_TPT; ++u) {
        const int t = t0 + rs_token(i0 + u);
        if (t < tend)
          *(u32x4*)(out + (long)t * H + hc) = u32x4{pack2(o[u][0], o[u][1]), pack2(o[u][2], o[u][3]),
                                                    pack2(o[u][4], o[u][5]), pack2(o[u][6], o[u][7])};
      }
    }
    __syncthreads();
  }
}

}  // namespace moelora
