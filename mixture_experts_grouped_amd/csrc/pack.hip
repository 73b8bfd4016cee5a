// pack.hip -- packed copies of the frozen base weights, and the zero padding
// of adapter factors whose rank is not a multiple of 8.
//
// Each of the four base GEMMs reads its weights as the N operand: a K tile of
// 256 weight rows x 64 k per pipeline stage (32 KB), which the direct loads
// place in LDS with the chunk swizzle of engine2.hpp (row r's 16-byte chunk
// c in slot c ^ kswz(r)).  Read from the plain matrix, a stage takes a
// 128-byte run from each of 256 rows that lie K*2 bytes apart.  A packed
// copy stores every stage tile as its LDS image -- rows consecutive, chunks
// in their slots -- one tile after another (N tile major, K stage minor), so
// a stage is 32 KB of consecutive bytes and each 1 KB wave load reads 1 KB in
// order (v2::KLoadP).  The tile's bytes in LDS are the same either way, so
// results do not change.  Written once per set of base weights by
// moe_lora_transform_base (the pages' reusable transformed weights, DeepGEMM
// PR #9 Summary), like the transposed copies of the backward.
//
//   kind 0  W13 for the forward: N tile t = gate rows 128t .. 128t+127 and
//           up rows I + 128t .., K = H           ([E][I/128][H/64] tiles)
//   kind 1  W2 for the forward: rows h, K = I     ([E][H/256][I/64])
//   kind 2  W13^T for the W13 data gradient: rows h, K = 2I ([E][H/256][2I/64])
//   kind 3  W2^T for the W2 data gradient: rows i, K = H    ([E][I/256][H/64])
// Kinds 2 and 3 transpose through LDS; from an MXFP4 base they are the
// dequantised values (e2m1 x 2^(e-127), exact in bf16).
//   kind 4  an MXFP4 W13 for the forward's scaled GEMM (rows as kind 0,
//           K = H), kind 5 an MXFP4 W2 (rows h, K = I): each stage tile of
//           256 rows x 64 k is MX_TILE = 9 KB, [codes | scale words]: row n's
//           32 code bytes of the stage at 32 n, its two 16-byte halves
//           swapped when (n >> 3) & 1 (the LDS slots of mx::WLoad), then one
//           32-bit word per row, the row's scale bytes 4 (s / 2) .. + 3 (the
//           stage pair's four 32-blocks).  A stage is then 9 KB in order
//           instead of 32 bytes and 4 bytes from each of 256 rows.
#include "engine2.hpp"
#include "layer.hpp"
#include "trace.hpp"

namespace moelora {

constexpr int PK_ROWS = 256, PK_KT = 64;
constexpr int PK_TILE = PK_ROWS * PK_KT;  // elements per stage tile (32 KB)

// 8 bf16 values -> the tile chunk (row r, slot p) at byte 16 (8 r + p)
__device__ __forceinline__ void pk_store(uint16_t* tile, int r, int p, u32x4 v) {
  *(u32x4*)(tile + 8 * (8 * r + p)) = v;
}

// kinds 0, 1: row-major source [N rows, K] (bf16); row map for kind 0
__global__ __launch_bounds__(256) void k_pack_rows(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int kind, int N, int K, int I) {
  const int nst = K / PK_KT, ntile = kind == 0 ? 2 * I / PK_ROWS : N / PK_ROWS;
  const long b = blockIdx.x;
  const int s = (int)(b % nst), t = (int)((b / nst) % ntile);
  const long e = b / ((long)nst * ntile);
  uint16_t* tile = dst + b * PK_TILE;
  const uint16_t* m = src + e * (long)N * K;
#pragma unroll
  for (int u = 0; u < PK_TILE / 8 / 256; ++u) {
    const int q = threadIdx.x + 256 * u;  // tile chunk
    const int r = q / 8, p = q % 8;
    const int c = p ^ v2::kswz<PK_KT>(r);
    const int row = kind == 0 ? (r < 128 ? 128 * t + r : I + 128 * t + (r - 128)) : PK_ROWS * t + r;
    pk_store(tile, r, p, *(const u32x4*)(m + (long)row * K + PK_KT * s + 8 * c));
  }
}

// kinds 2, 3: the transpose of a source S [K, N] (bf16, or MXFP4 with scales
// per 32 along N): tile rows n0 .. n0 + 255, k0 .. k0 + 63
template <bool MX>
__global__ __launch_bounds__(256) void k_pack_cols(const uint16_t* __restrict__ src, const uint8_t* __restrict__ q4,
                                                   const uint8_t* __restrict__ sc, uint16_t* __restrict__ dst, int N,
                                                   int K) {
  __shared__ uint16_t t[PK_KT][PK_ROWS + 8];  // [k][n], rows padded by 16 bytes
  const int nst = K / PK_KT, ntile = N / PK_ROWS;
  const long b = blockIdx.x;
  const int s = (int)(b % nst), nt = (int)((b / nst) % ntile);
  const long e = b / ((long)nst * ntile);
  const int k0 = PK_KT * s, n0 = PK_ROWS * nt;
#pragma unroll
  for (int u = 0; u < PK_TILE / 8 / 256; ++u) {
    const int q = threadIdx.x + 256 * u;  // 8 consecutive n of one k-row
    const int kr = q / 32, cc = q % 32;
    const long row = e * (long)K + k0 + kr;
    u32x4 v;
    if constexpr (MX) {
      const uint32_t w = *(const uint32_t*)(q4 + row * (N / 2) + (n0 + 8 * cc) / 2);
      v = v2::fp4x8_bf16(w, v2::e8m0_value(sc[row * (N / 32) + (n0 + 8 * cc) / 32]));
    } else {
      v = *(const u32x4*)(src + row * N + n0 + 8 * cc);
    }
    *(u32x4*)&t[kr][8 * cc] = v;
  }
  __syncthreads();
  uint16_t* tile = dst + b * PK_TILE;
#pragma unroll
  for (int u = 0; u < PK_TILE / 8 / 256; ++u) {
    const int q = threadIdx.x + 256 * u;
    const int r = q / 8, p = q % 8;
    const int c = p ^ v2::kswz<PK_KT>(r);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)t[8 * c + 2 * i][r] | ((uint32_t)t[8 * c + 2 * i + 1][r] << 16);
    pk_store(tile, r, p, u32x4{w[0], w[1], w[2], w[3]});
  }
}

// kinds 4, 5: [E][N/256][K/64] tiles of MX_TILE bytes from packed e2m1 rows
// q4 [N, K/2] and scale rows sc [N, K/32] of each expert (N = 2I or H)
__global__ __launch_bounds__(256) void k_pack_mx(const uint8_t* __restrict__ q4, const uint8_t* __restrict__ sc,
                                                 uint8_t* __restrict__ dst, int kind, int N, int K, int I) {
  const int nst = K / PK_KT, ntile = N / PK_ROWS;
  const long b = blockIdx.x;
  const int s = (int)(b % nst), t = (int)((b / nst) % ntile);
  const long e = b / ((long)nst * ntile);
  uint8_t* tile = dst + b * MX_TILE;
  const uint8_t* q = q4 + e * (long)N * (K / 2);
  const uint8_t* scl = sc + e * (long)N * (K / 32);
  auto row_of = [&](int n) { return kind == 4 ? (n < 128 ? 128 * t + n : I + 128 * t + (n - 128)) : PK_ROWS * t + n; };
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qi = threadIdx.x + 256 * u;  // 16-byte slot p of row n
    const int n = qi / 2, p = qi % 2;
    const int c = p ^ ((n >> 3) & 1);
    *(u32x4*)(tile + 32 * n + 16 * p) = *(const u32x4*)(q + (long)row_of(n) * (K / 2) + 32 * s + 16 * c);
  }
  const int n = threadIdx.x;
  const uint8_t* sb = scl + (long)row_of(n) * (K / 32) + 4 * (s / 2);  // scale rows need no alignment
  *(uint32_t*)(tile + 32 * PK_ROWS + 4 * n) =
      (uint32_t)sb[0] | ((uint32_t)sb[1] << 8) | ((uint32_t)sb[2] << 16) | ((uint32_t)sb[3] << 24);
}

// kind 0 / 1 from a bf16 base; kind 2 / 3 from a bf16 (q4 == nullptr) or an
// MXFP4 base; kind 4 / 5 from an MXFP4 base (dst: bytes).  E experts of the
// kind's matrix.
hipError_t launch_pack(int kind, const uint16_t* src, const uint8_t* q4, const uint8_t* sc, uint16_t* dst, int E,
                       int H, int I, hipStream_t st) {
  if (kind == 4 || kind == 5) {
    const int N = kind == 4 ? 2 * I : H, K = kind == 4 ? H : I;
    const long tiles = (long)E * (N / PK_ROWS) * (K / PK_KT);
    MOE_LAUNCH(k_pack_mx, dim3((unsigned)tiles), dim3(256), 0, st, q4, sc, (uint8_t*)dst, kind, N, K, I);
  } else if (kind == 0 || kind == 1) {
    const int N = kind == 0 ? 2 * I : H, K = kind == 0 ? H : I;
    const long tiles = (long)E * (N / PK_ROWS) * (K / PK_KT);
    MOE_LAUNCH(k_pack_rows, dim3((unsigned)tiles), dim3(256), 0, st, src, dst, kind, N, K, I);
  } else {
    // S = W13 [2I, H] -> rows h, K = 2I;  S = W2 [H, I] -> rows i, K = H
    const int N = kind == 2 ? H : I, K = kind == 2 ? 2 * I : H;
    const long tiles = (long)E * (N / PK_ROWS) * (K / PK_KT);
    if (q4 != nullptr)
      MOE_LAUNCH(k_pack_cols<true>, dim3((unsigned)tiles), dim3(256), 0, st, nullptr, q4, sc, dst, N, K);
    else
      MOE_LAUNCH(k_pack_cols<false>, dim3((unsigned)tiles), dim3(256), 0, st, src, nullptr, nullptr, dst, N, K);
  }
  return hipGetLastError();
}

// Rank padding: dst [nb, rd, cd] from src [nb, rs, cs] (bf16), zero where
// the source has no element -- the adapter factors of a rank that is not a
// multiple of 8 widened with zero rows or columns, and (rd <= rs, cd <= cs)
// their gradients cut back to the caller's rank.
__global__ __launch_bounds__(256) void k_pad(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, long n,
                                             int rs, int cs, int rd, int cd) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % cd);
  const long br = i / cd;
  const int r = (int)(br % rd);
  const long b = br / rd;
  dst[i] = (r < rs && c < cs) ? src[(b * rs + r) * cs + c] : (uint16_t)0;
}

hipError_t launch_pad(const uint16_t* src, uint16_t* dst, long nb, int rs, int cs, int rd, int cd, hipStream_t st) {
  const long n = nb * rd * cd;
  if (n <= 0) return hipSuccess;
  MOE_LAUNCH(k_pad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst, n, rs, cs, rd, cd);
  return hipGetLastError();
}

}  // namespace moelora
