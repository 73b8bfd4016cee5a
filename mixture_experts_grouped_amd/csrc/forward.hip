// forward.hip -- forward of the MoE side-LoRA expert layer.
//
// Steps (DeepGEMM PR #9, "Historical implementation" -> Summary: shrink and
// expand phases around the expert GEMMs, A1/A3/B2 shared, B1/B3/A2 local):
//   k_shrink    ZA_t = s [A1; A3] x_t, once per token (A1/A3 are shared, so
//               A u is the same for all k routes of a token)
//   k_w13       g = W1_e u + B1_e ZA1_t, v = W3_e u + B3_e ZA3_t; the B terms
//               ride as extra K on the W13 GEMM; SwiGLU in the epilogue;
//               saves G, V (fp32) and h (bf16)
//   k_a2        Z2 = s A2_e h
//   k_w2        Ybase = W2_e h
//   k_zc        zc_t = sum_j w_tj Z2_(t,j)          (slot order, fp32)
//   k_combine   out_t = B2 zc_t + sum_j w_tj Ybase_(t,j)
// The per-token evaluation of the shared factors is exact algebra:
// sum_j w_j B2 z_j = B2 sum_j w_j z_j.
#include "layer.hpp"

namespace moelora {

hipError_t launch_pool_prologue(const LayerArgs& a, hipStream_t st);

using G256 = Geo<4, 4, 2, 2>;  // 256 x 256 tile, wave 128 x 128
using G128 = Geo<4, 2, 2, 2>;  // 256 x 128 tile, wave 128 x 64

__device__ __forceinline__ int tok_of_row(const LayerArgs& a, long row) { return a.row2r[row] / a.k; }

// ----------------------------------------------------------------------------
// a3: ZA = s [A1; A3] x  (dense over tokens; N = 2r)
// ----------------------------------------------------------------------------
struct LdPlain {
  RowsK<256> m;
  RowsK<128> n;
  __device__ void load(int s) { m.load(s * KT, 0, false); n.load(s * KT, 0, false); }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

__global__ __launch_bounds__(256) void k_shrink(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int t0 = blockIdx.x * G128::TM, n0 = blockIdx.y * G128::TN;
  const int r = a.r;
  LdPlain L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + RowsK<256>::row_of(i);
    L.m.rp[i] = (t < a.T) ? a.x + (long)t * a.H : nullptr;
    L.m.lo[i] = 0;
  }
  L.m.span = a.H;
  L.m.period = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = n0 + RowsK<128>::row_of(i);
    L.n.rp[i] = (c < r) ? a.A1 + (long)c * a.H : (c < 2 * r ? a.A3 + (long)(c - r) * a.H : nullptr);
    L.n.lo[i] = 0;
  }
  L.n.span = a.H;
  L.n.period = 0;
  f32x16 acc[G128::NB][G128::MB];
  mainloop<G128>(L, a.H / KT, 1 << 30, acc, smem);
  Epi<G128> ep;
#pragma unroll
  for (int nb = 0; nb < G128::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < G128::MB; ++mb) {
      const int t = t0 + ep.row(mb);
      if (t >= a.T) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = n0 + ep.col(nb, g) + q;
          if (c >= 2 * r) continue;
          uint32_t hi, lo;
          split_hl(a.s * acc[nb][mb][4 * g + q], hi, lo);
          const int fac = c / r, cc = c - fac * r;  // 0: A1, 1: A3
          uint16_t* dst = a.ZA + (long)t * 4 * r + fac * 2 * r + cc;
          dst[0] = (uint16_t)hi;
          dst[r] = (uint16_t)lo;
        }
    }
}

// ----------------------------------------------------------------------------
// a4: W13 grouped GEMM (+ B1/B3 via K-extension) + SwiGLU
// N tile = 128 gate columns i0.. and the 128 up columns with the same i.
// ----------------------------------------------------------------------------
struct LdW13 {
  RowsK<256> m, n;
  int nmain, r, topk, row0, row_end, i0;
  const int32_t* row2r;
  const uint16_t *ZA, *B1e, *B3e;
  __device__ void to_ext() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const long row = row0 + RowsK<256>::row_of(i);
      m.rp[i] = (row < row_end) ? ZA + (long)(row2r[row] / topk) * 4 * r : nullptr;
      m.lo[i] = 0;
      const int nl = RowsK<256>::row_of(i);
      const bool gate = nl < 128;
      n.rp[i] = (gate ? B1e : B3e) + (long)(i0 + (nl & 127)) * r;
      n.lo[i] = gate ? 0 : 2 * r;
    }
    m.span = 4 * r;
    m.period = 0;
    n.span = 2 * r;
    n.period = r;
  }
  __device__ void load(int s) {
    if (s < nmain) {
      m.load(s * KT, 0, false);
      n.load(s * KT, 0, false);
      return;
    }
    if (s == nmain) to_ext();
    const int se = s - nmain;
    m.load(se * 32, 2 * r, true);
    n.load(se * 32, 2 * r, true);
  }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

__global__ __launch_bounds__(256) void k_w13(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int ntn = a.I / 128;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (mt >= *a.ntiles) return;
  const TileInfo ti = a.tiles[mt];
  const int e = ti.e, i0 = nt * 128;
  LdW13 L;
  L.r = a.r;
  L.topk = a.k;
  L.row0 = ti.row0;
  L.row_end = ti.row_end;
  L.i0 = i0;
  L.row2r = a.row2r;
  L.ZA = a.ZA;
  L.B1e = a.B1 + (long)e * a.I * a.r;
  L.B3e = a.B3 + (long)e * a.I * a.r;
  const uint16_t* W = a.W13 + (long)e * 2 * a.I * a.H;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long row = ti.row0 + RowsK<256>::row_of(i);
    L.m.rp[i] = (row < ti.row_end) ? a.Xp + row * a.H : nullptr;
    L.m.lo[i] = 0;
    const int nl = RowsK<256>::row_of(i);
    const int wrow = (nl < 128) ? i0 + nl : a.I + i0 + (nl - 128);
    L.n.rp[i] = W + (long)wrow * a.H;
    L.n.lo[i] = 0;
  }
  L.m.span = L.n.span = a.H;
  L.m.period = L.n.period = 0;
  L.nmain = a.H / KT;
  const int next = (2 * a.r + 31) / 32;
  f32x16 acc[G256::NB][G256::MB];
  mainloop<G256>(L, L.nmain + next, L.nmain, acc, smem);
  Epi<G256> ep;
#pragma unroll
  for (int mb = 0; mb < G256::MB; ++mb) {
    const long row = ti.row0 + ep.row(mb);
    if (row >= ti.row_end) continue;
#pragma unroll
    for (int nb = 0; nb < G256::NB / 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = i0 + ep.col(nb, g);
        f32x4 gv, vv;
        uint32_t hb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gg = acc[nb][mb][4 * g + q];
          const float v = acc[nb + G256::NB / 2][mb][4 * g + q];
          gv[q] = gg;
          vv[q] = v;
          hb[q] = f2bf(gg * sigmoidf_(gg) * v);
        }
        *(f32x4*)(a.G + row * a.I + i) = gv;
        *(f32x4*)(a.V + row * a.I + i) = vv;
        u32x2 hp = {hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        *(u32x2*)(a.Hh + row * a.I + i) = hp;
      }
  }
}

// ----------------------------------------------------------------------------
// a5: Z2 = s A2_e h  (grouped, N = r)
// a6: Ybase = W2_e h (grouped)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_a2(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int mt = blockIdx.x;
  if (mt >= *a.ntiles) return;
  const TileInfo ti = a.tiles[mt];
  const uint16_t* A2e = a.A2 + (long)ti.e * a.r * a.I;
  LdPlain L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long row = ti.row0 + RowsK<256>::row_of(i);
    L.m.rp[i] = (row < ti.row_end) ? a.Hh + row * a.I : nullptr;
    L.m.lo[i] = 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = RowsK<128>::row_of(i);
    L.n.rp[i] = (c < a.r) ? A2e + (long)c * a.I : nullptr;
    L.n.lo[i] = 0;
  }
  L.m.span = L.n.span = a.I;
  L.m.period = L.n.period = 0;
  f32x16 acc[G128::NB][G128::MB];
  mainloop<G128>(L, a.I / KT, 1 << 30, acc, smem);
  Epi<G128> ep;
#pragma unroll
  for (int mb = 0; mb < G128::MB; ++mb) {
    const long row = ti.row0 + ep.row(mb);
    if (row >= ti.row_end) continue;
#pragma unroll
    for (int nb = 0; nb < G128::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = ep.col(nb, g);
        if (c >= a.r) continue;
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = a.s * acc[nb][mb][4 * g + q];
        *(f32x4*)(a.Z2 + row * a.r + c) = v;
      }
  }
}

struct LdSq {
  RowsK<256> m, n;
  __device__ void load(int s) { m.load(s * KT, 0, false); n.load(s * KT, 0, false); }
  __device__ void store(char* sM, char* sN) { m.store(sM); n.store(sN); }
};

__global__ __launch_bounds__(256) void k_w2(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int ntn = a.H / 256;
  const int mt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
  if (mt >= *a.ntiles) return;
  const TileInfo ti = a.tiles[mt];
  const int h0 = nt * 256;
  const uint16_t* W = a.W2 + (long)ti.e * a.H * a.I;
  LdSq L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long row = ti.row0 + RowsK<256>::row_of(i);
    L.m.rp[i] = (row < ti.row_end) ? a.Hh + row * a.I : nullptr;
    L.m.lo[i] = 0;
    L.n.rp[i] = W + (long)(h0 + RowsK<256>::row_of(i)) * a.I;
    L.n.lo[i] = 0;
  }
  L.m.span = L.n.span = a.I;
  L.m.period = L.n.period = 0;
  f32x16 acc[G256::NB][G256::MB];
  mainloop<G256>(L, a.I / KT, 1 << 30, acc, smem);
  Epi<G256> ep;
#pragma unroll
  for (int mb = 0; mb < G256::MB; ++mb) {
    const long row = ti.row0 + ep.row(mb);
    if (row >= ti.row_end) continue;
#pragma unroll
    for (int nb = 0; nb < G256::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int h = h0 + ep.col(nb, g);
        u32x2 o = {pack2(acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1]),
                   pack2(acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3])};
        *(u32x2*)(a.Yb + row * a.H + h) = o;
      }
  }
}

// ----------------------------------------------------------------------------
// a7: zc_t = sum_j w_tj Z2_(t,j);  out_t = B2 zc_t + sum_j w_tj Ybase_(t,j)
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_zc(LayerArgs a) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)a.T * a.r) return;
  const int t = (int)(i / a.r), c = (int)(i % a.r);
  float z = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    const int row = a.r2row[t * a.k + j];
    if (row >= 0) z += a.w[t * a.k + j] * a.Z2[(long)row * a.r + c];
  }
  uint32_t hi, lo;
  split_hl(z, hi, lo);
  a.zc[(long)t * 2 * a.r + c] = (uint16_t)hi;
  a.zc[(long)t * 2 * a.r + a.r + c] = (uint16_t)lo;
}

__global__ __launch_bounds__(256) void k_combine(LayerArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int t0 = blockIdx.x * 256, h0 = blockIdx.y * 256;
  const int r = a.r;
  LdSq L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + RowsK<256>::row_of(i);
    L.m.rp[i] = (t < a.T) ? a.zc + (long)t * 2 * r : nullptr;
    L.m.lo[i] = 0;
    L.n.rp[i] = a.B2 + (long)(h0 + RowsK<256>::row_of(i)) * r;
    L.n.lo[i] = 0;
  }
  L.m.span = 2 * r;
  L.m.period = 0;
  L.n.span = 2 * r;
  L.n.period = r;
  f32x16 acc[G256::NB][G256::MB];
  mainloop<G256>(L, (2 * r + KT - 1) / KT, 1 << 30, acc, smem);
  Epi<G256> ep;
#pragma unroll
  for (int mb = 0; mb < G256::MB; ++mb) {
    const int t = t0 + ep.row(mb);
    if (t >= a.T) continue;
    int rows[16];
    float ws[16];
    for (int j = 0; j < a.k; ++j) {
      rows[j] = a.r2row[t * a.k + j];
      ws[j] = a.w[t * a.k + j];
    }
#pragma unroll
    for (int nb = 0; nb < G256::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int h = h0 + ep.col(nb, g);
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = acc[nb][mb][4 * g + q];
        for (int j = 0; j < a.k; ++j) {
          if (rows[j] < 0) continue;
          const u32x2 y = *(const u32x2*)(a.Yb + (long)rows[j] * a.H + h);
          o[0] += ws[j] * bf2f(y[0] & 0xffffu);
          o[1] += ws[j] * bf2f(y[0] >> 16);
          o[2] += ws[j] * bf2f(y[1] & 0xffffu);
          o[3] += ws[j] * bf2f(y[1] >> 16);
        }
        u32x2 ov = {pack2(o[0], o[1]), pack2(o[2], o[3])};
        *(u32x2*)(a.out + (long)t * a.H + h) = ov;
      }
  }
}

// ----------------------------------------------------------------------------
static void set_lds(const void* fn, int bytes) {
  hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_forward(const LayerArgs& a, hipStream_t st) {
  static bool init = false;
  if (!init) {
    set_lds((const void*)k_shrink, G128::LDS_BYTES);
    set_lds((const void*)k_w13, G256::LDS_BYTES);
    set_lds((const void*)k_a2, G128::LDS_BYTES);
    set_lds((const void*)k_w2, G256::LDS_BYTES);
    set_lds((const void*)k_combine, G256::LDS_BYTES);
    init = true;
  }
  hipError_t err = launch_pool_prologue(a, st);
  if (err != hipSuccess) return err;
  const int tm = (a.T + 255) / 256;
  hipLaunchKernelGGL(k_shrink, dim3(tm, (2 * a.r + 127) / 128), dim3(256), G128::LDS_BYTES, st, a);
  hipLaunchKernelGGL(k_w13, dim3(a.maxtiles * (a.I / 128)), dim3(256), G256::LDS_BYTES, st, a);
  hipLaunchKernelGGL(k_a2, dim3(a.maxtiles), dim3(256), G128::LDS_BYTES, st, a);
  hipLaunchKernelGGL(k_w2, dim3(a.maxtiles * (a.H / 256)), dim3(256), G256::LDS_BYTES, st, a);
  const long nzc = (long)a.T * a.r;
  hipLaunchKernelGGL(k_zc, dim3((unsigned)((nzc + 255) / 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_combine, dim3(tm, a.H / 256), dim3(256), G256::LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace moelora
