// gather_sum.hpp -- per-token sums over a token's routes:
//
//   out[t, h] = P[t, h] + sum_j c_tj R[route_tj row, h]
//
// The forward combine (mixture output, c = routing weight, R = the routes'
// base outputs, P = B2 zc_t with zc_t = s sum_j w_tj z_tj) and the input
// gradient (c = 1, R = the routes' W13^T [dg; dv], P = [A1; A3]^T pc_t) have
// this form.  P is a rank-r product per token, computed by a grouped-GEMM
// style kernel into an fp32 [T, H] scratch (RankImage below); the sum then
// runs as a pure streaming kernel (k_token_sum): one wave per token and
// 512-column chunk, 16 bytes a lane from every route row, all of a token's
// route rows in flight at once.  The route rows add in route order j = 0,
// 1, ... after P, so the result does not depend on the pool layout.
#pragma once
#include "engine2.hpp"
#include "layer.hpp"

namespace moelora {

// 256-token x 256-column tiles of P; eight waves of 128 x 64.
using GRK = v2::Geo2<4, 2, 2, 4, false, false, 64>;
using RankImg = v2::TileImage<GRK, GRK::TN / 2, float>;
constexpr int RK_LDS = cmax(GRK::LDS_BYTES, RankImg::BYTES);

// acc (a 256 x 256 tile of P, tokens t0.., columns h0..) -> P rows, through
// LDS images of one column half at a time.
template <class G>
__device__ __forceinline__ void store_rank_tile(const f32x16 (&acc)[G::NB][G::MB], char* smem,
                                                float* P, long H, int t0, int h0, int ntok) {
  static_assert(G::NB == 2, "one block column per half");
  Epi<G> ep;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        RankImg::put(smem, ep.row(mb), ep.col(nb, g) - nb * (G::TN / 2),
                     f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2],
                           acc[nb][mb][4 * g + 3]});
    __syncthreads();
    RankImg::flush(smem, P + (long)t0 * H + h0 + nb * (G::TN / 2), H, ntok);
    __syncthreads();
  }
}

constexpr int TS_COLS = 512;  // columns per wave of k_token_sum (8 per lane)
constexpr int TS_JC = 8;      // route rows loaded before any is added

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) { return bload(r, off); }

// out[t, h .. h + 7] for the wave's token t; lanes past H are idle.
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void k_token_sum(LayerArgs a, const uint16_t* R, const float* P,
                                                   uint16_t* out) {
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int h = blockIdx.y * TS_COLS + 8 * (threadIdx.x & 63);
  const bool live = h < a.H;
  const uint32_t voff = 2u * (uint32_t)h;
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
    const f32x4* pp = (const f32x4*)(P + (long)t * a.H + h);
    const f32x4 p0 = pp[0], p1 = pp[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = p0[q];
      o[4 + q] = p1[q];
    }
  }
  // lane j holds route j's pool row and weight: one vector load for all
  // routes, so the row loads below do not wait on each other's index
  const int lane = threadIdx.x & 63;
  int myrow = -1;
  float myc = 0.0f;
  if (lane < a.k) {
    myrow = a.r2row[(long)t * a.k + lane];
    myc = WEIGHTED ? a.w[(long)t * a.k + lane] : 1.0f;
    if (myrow < 0) myc = 0.0f;  // a dead route's weight is not read
  }
  for (int j0 = 0; j0 < a.k; j0 += TS_JC) {
    u32x4 y[TS_JC];
    float c[TS_JC];
#pragma unroll
    for (int jj = 0; jj < TS_JC; ++jj) {
      const int j = j0 + jj;  // < 64: lanes past k hold row -1, weight 0
      const int row = __builtin_amdgcn_readlane(myrow, j);
      c[jj] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myc), j));
      // a dead route gets an empty descriptor and reads zeros
      const rsrc_t rs = make_rsrc(R + (long)(row < 0 ? 0 : row) * a.H, row < 0 ? 0 : (uint64_t)a.H * 2);
      y[jj] = bload16(rs, voff);
    }
    // routes past k read zeros with weight 0 and add nothing
#pragma unroll
    for (int jj = 0; jj < TS_JC; ++jj) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[2 * q] += c[jj] * bf2f(y[jj][q] & 0xffffu);
        o[2 * q + 1] += c[jj] * bf2f(y[jj][q] >> 16);
      }
    }
  }
  if (live)
    *(u32x4*)(out + (long)t * a.H + h) =
        u32x4{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
}

}  // namespace moelora
