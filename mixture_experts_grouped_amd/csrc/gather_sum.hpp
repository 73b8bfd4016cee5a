// gather_sum.hpp -- per-token sums over a token's routes, fused with a small
// rank-space product computed on the matrix cores.
//
//   out[t, h] = P[t, h] + sum_j c_tj R[route_tj row, h]
//
// The forward combine (mixture output, c = routing weight, R = the routes'
// base outputs, P = s B2 (sum_j w_tj z_tj)) and the input gradient
// (c = 1, R = the routes' W13^T [dg; dv], P = the adapter terms through A1
// and A3) have this form; both are bound by HBM reads of R.
//
// The workgroup first computes its 64-token x 256-column tile of P with the
// MFMA pipeline, parks it in LDS as fp32, and then walks the tile row by row:
// one wave takes one token, its 64 lanes cover the 256 columns with 8-byte
// loads, so every gathered route row is read as 512 contiguous bytes.  The
// route rows sum in route order j = 0, 1, ... after P, so the result does not
// depend on the pool layout.
#pragma once
#include "engine2.hpp"
#include "layer.hpp"

namespace moelora {

// 64 tokens x 256 columns, eight waves of 32 x 64; GGS_T takes the N operand
// K-outer (columns contiguous in memory), same tile and register layout
using GGS = v2::Geo2<1, 2, 2, 4, false, false, 64>;
using GGS_T = v2::Geo2<1, 2, 2, 4, false, true, 64>;
static_assert(GGS::TM == 64 && GGS::TN == 256, "gather-sum tile");
static_assert(GGS_T::LDS_BYTES == GGS::LDS_BYTES, "same LDS footprint");

constexpr int GS_PITCH = GGS::TN + 4;  // floats per parked row (4 pad words)
constexpr int GS_LDS = (GGS::LDS_BYTES > GGS::TM * GS_PITCH * 4) ? GGS::LDS_BYTES
                                                                 : GGS::TM * GS_PITCH * 4;

__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// acc (the tile of P) -> LDS rows of GS_PITCH floats.  Call after the MFMA
// pipeline has released LDS.
__device__ __forceinline__ void park_tile(const f32x16 (&acc)[GGS::NB][GGS::MB], char* smem) {
  float* st = (float*)smem;
  Epi<GGS> ep;
#pragma unroll
  for (int mb = 0; mb < GGS::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < GGS::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[nb][mb][4 * g + q];
        *(f32x4*)(st + ep.row(mb) * GS_PITCH + ep.col(nb, g)) = v;
      }
  __syncthreads();
}

// Second half: tokens t0 .. t0 + 63 (those < T), columns h0 .. h0 + 255.
// R is [rows, H] bf16 (one row per pool row), out is [T, H] bf16.  With
// WEIGHTED, route j of token t is scaled by w[t k + j], else by one.
template <bool WEIGHTED>
__device__ __forceinline__ void gather_rows(const char* smem, const LayerArgs& a,
                                            const uint16_t* R, uint16_t* out, int t0, int h0) {
  constexpr int JC = 8;  // routes loaded before any is added
  const float* st = (const float*)smem;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t voff = 8u * lane;
  for (int tl = w; tl < GGS::TM; tl += GGS::NW) {
    const int t = t0 + tl;
    if (t >= a.T) break;  // uniform: the wave's token
    f32x4 o = *(const f32x4*)(st + tl * GS_PITCH + 4 * lane);
    for (int j0 = 0; j0 < a.k; j0 += JC) {
      u32x2 y[JC];
      float c[JC];
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        const int j = j0 + jj;
        int row = -1;
        float cj = 0.0f;
        if (j < a.k) {
          row = a.r2row[(long)t * a.k + j];
          cj = WEIGHTED ? a.w[(long)t * a.k + j] : 1.0f;
        }
        row = __builtin_amdgcn_readfirstlane(row);
        if (row < 0) cj = 0.0f;  // a dead route's weight is not read
        c[jj] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cj)));
        // a dead route (row < 0) gets an empty descriptor and reads zeros
        const rsrc_t rs = make_rsrc(R + (long)(row < 0 ? 0 : row) * a.H + h0, row < 0 ? 0 : 512);
        y[jj] = bload8(rs, voff);
      }
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        if (j0 + jj >= a.k) break;
        o[0] += c[jj] * bf2f(y[jj][0] & 0xffffu);
        o[1] += c[jj] * bf2f(y[jj][0] >> 16);
        o[2] += c[jj] * bf2f(y[jj][1] & 0xffffu);
        o[3] += c[jj] * bf2f(y[jj][1] >> 16);
      }
    }
    *(u32x2*)(out + (long)t * a.H + h0 + 4 * lane) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
  }
}

}  // namespace moelora
