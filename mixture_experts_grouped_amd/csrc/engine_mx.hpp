// engine_mx.hpp -- MXFP4-base GEMM stages on gfx950's scaled matrix cores.
//
// The base weights are OCP MX v1.0 FP4 (E2M1, two per byte, element 2i in
// the low nibble of byte i) with one E8M0 scale per 32 along K; the
// activations are held as a two-term FP6 (E2M3) split with one E8M0 scale
// per term and 32-block: x ~ s1 q1 + s2 q2 (quant_term below).  Each k64
// step is two v_mfma_scale_f32_32x32x64_f8f6f4 per output block (one per
// term, weights as the fp4 first operand, activations as the fp6 second
// operand: with both operands of six bits or fewer the instruction runs at
// twice its fp8 rate), accumulating into the same fp32 32 x 32 accumulators
// as the bf16 engine, with the same lane layout: lanes own output rows,
// registers four consecutive output columns.
//
// Operand lane layouts of the scaled instruction (probed on the device):
//   fp4 operand: lane l holds row l % 32, k = 32 (l / 32) .. + 31 (16 bytes,
//                low nibble first); its scale is that 32-block's;
//   fp6 operand: lane l holds row l % 32, k = 32 (l / 32) .. + 31: element
//                e in bits 6e .. 6e + 5 of six dwords (little-endian across
//                them); its scale is that 32-block's;
//   the op_sel field picks the scale byte of the 32-bit scale register.
//
// Storage (per row, per 64-k chunk c of the contraction):
//   activation codes   128 bytes: term t (0: s1 q1, 1: s2 q2) at 64 t, its
//                      32-block h (k 64c + 32h ..) as dwords 0-3 at 16 h and
//                      dwords 4-5 at 32 + 8 h (bytes 48-63 unused): the row
//                      pitch of a bf16 row, so the bf16 K-tile loader
//                      (KLoadA / KLoadS) and its swizzle carry it, and each
//                      lane's six dwords are one 16-byte and one 8-byte read;
//   activation scales  one 32-bit word: bytes {s1 b0, s1 b1, s2 b0, s2 b1}
//                      for the chunk's two 32-blocks, stored stage-major
//                      ([K/64][rows]: the words of one chunk for all rows
//                      are consecutive);
//   weight codes       32 bytes at 32c of the packed row;
//   weight scales      byte 2c + b of the row's scale bytes;
//   or, from a packed copy of the weights (pack.hip kinds 4 and 5), each
//   stage's 256 rows of codes and scale words as one 9 KB block.
//
// One stage = one k64 step: LDS [A 256 x 128 B | W 256 x 32 B | A scales
// 256 x 4 B | W scales 256 x 4 B] = 42 KB, three stages in LDS (two in
// flight while one is multiplied).  Each wave issues the same number of
// direct-to-LDS loads per stage (INSTS), so one vmcnt wait per stage covers
// the stage it is about to read.
#pragma once
#include "engine2.hpp"
#include "layer.hpp"

namespace moelora {
namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int TM = 256, TN = 256, NT = 512, NW = 8;
constexpr int A_BYTES = TM * 128, W_BYTES = TN * 32, AS_BYTES = TM * 4, WS_BYTES = TN * 4;
constexpr int STAGE = A_BYTES + W_BYTES + AS_BYTES + WS_BYTES;  // 43008
constexpr int NBUF = 3;
constexpr int LDS_BYTES = NBUF * STAGE;
using KA = v2::KLoadA<TM, 64, NW>;  // activation rows: 128 bytes per stage, bf16-shaped
using KS = v2::KLoadS<TM, 64, NW>;
static_assert(KA::NJ == 4 && KS::NJ == 4, "four 1 KB activation loads per wave and stage");
constexpr int INSTS = KA::NJ + 1 + 1;  // activation rows, weight rows, one scale word row

// ---------------------------------------------------------------------------
// Two-term E2M3 split of one aligned 32-block (values exactly bf16, in fp32).
// s = 2^E with E the smallest integer such that amax <= 7.5 2^E (no element
// saturates; amax = 0 or below 2^-126 gives E = -127), q = E2M3(x / s) to
// nearest, ties to even, r = x - s q exactly, and the same again on r.
// Scale bytes are E + 127.  E2M3 (OCP MX v1.0 FP6): bias 1, subnormals m/8,
// normals (1 + m/8) 2^(e-1), largest 7.5; code 8 e + m, sign in bit 5.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int e2m3_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int field = (int)(b >> 23);  // amax >= 0
  if (field == 0) return -127;       // zero or subnormal
  const int p = field - 127;
  const int e = ((b & 0x7FFFFFu) <= 0x700000u) ? p - 2 : p - 1;  // mantissa 1.875 or less: p - 2
  return e < -127 ? -127 : e;
}
__device__ __forceinline__ float pow2f(int e) {  // 2^e for e in [-127, 127]
  return e > -127 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// 32 values -> six dwords of codes (element i in bits 6i .. 6i + 5) and the
// scale byte; also returns the residual x - s q in place of x.
__device__ __forceinline__ uint32_t quant_term(float (&v)[32], uint32_t (&q)[6]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int E = e2m3_scale_exp(amax);
  const float inv = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E, -E <= 127
  const float s = pow2f(E);
#pragma unroll
  for (int w = 0; w < 6; ++w) q[w] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float y = v[i] * inv;  // exact, |y| <= 7.5
    const uint32_t ab = __float_as_uint(y) & 0x7FFFFFFFu;
    // binade e of |y| from its exponent field, 0 below 2 (the step 1/8 of the
    // subnormals and of [1, 2)); integer arithmetic, no per-element masks
    const int e = min(max((int)(ab >> 23) - 127, 0), 2);
    const float mul = __uint_as_float((uint32_t)(130 - e) << 23);   // 2^(3-e)
    const float step = __uint_as_float((uint32_t)(124 + e) << 23);  // 2^(e-3)
    const float n = __builtin_rintf(__uint_as_float(ab) * mul);     // multiples of the step, half to even
    const uint32_t c = (8u * (uint32_t)e + (uint32_t)n) | ((__float_as_uint(y) >> 31) << 5);
    v[i] = fmaf(-copysignf(n * step, y), s, v[i]);  // exact residual
    const int b = 6 * i, wd = b >> 5, sh = b & 31;
    q[wd] |= c << sh;
    if (sh > 26) q[wd + 1] |= c >> (32 - sh);
  }
  return (uint32_t)(E + 127);
}

// One term's codes of 32-block h of a 64-k chunk at `chunk` (128 bytes).
__device__ __forceinline__ void store_term(uint8_t* chunk, int t, int h, const uint32_t (&q)[6]) {
  *(u32x4*)(chunk + 64 * t + 16 * h) = u32x4{q[0], q[1], q[2], q[3]};
  *(u32x2*)(chunk + 64 * t + 32 + 8 * h) = u32x2{q[4], q[5]};
}

// Rows of a bf16 [nrows, K] matrix -> codes [nrows, 2K bytes] and scale
// words [K/64, nrows]; one thread per (row, 32-block), the threads of a row
// adjacent (K % 64 == 0).
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ src, uint8_t* __restrict__ codes,
                                                    uint32_t* __restrict__ scales, long nrows, int K) {
  const int bpr = K / 32;  // blocks per row (even)
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = i / bpr;
  const int j = (int)(i - row * bpr);
  const bool live = row < nrows;
  float v[32];
  if (live) {
    const u32x4* p = (const u32x4*)(src + row * (long)K + 32 * j);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = p[c];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * c + 2 * q] = bf2f(w[q] & 0xffffu);
        v[8 * c + 2 * q + 1] = bf2f(w[q] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] = 0.0f;
  }
  uint32_t hi[6], lo[6];
  const uint32_t s1 = quant_term(v, hi);
  const uint32_t s2 = quant_term(v, lo);
  // partner block of the same 64-chunk (j ^ 1) sits in the neighbouring lane
  const uint32_t o1 = __shfl_xor(s1, 1, 64), o2 = __shfl_xor(s2, 1, 64);
  if (!live) return;
  uint8_t* chunk = codes + row * (long)(2 * K) + 128 * (j >> 1);
  store_term(chunk, 0, j & 1, hi);
  store_term(chunk, 1, j & 1, lo);
  if ((j & 1) == 0) scales[(long)(j >> 1) * nrows + row] = s1 | (o1 << 8) | (s2 << 16) | (o2 << 24);
}

// The split of a tile of bf16 rows parked in LDS (an epilogue image: rows of
// `pitch` bytes, COLS values from global column c0, a multiple of 64): the
// codes and scale words of rows [0, nrows) go to codes / scales (those rows'
// first elements; the global rows have 2K bytes, the scale words of chunk c
// sit sld words after those of chunk c - 1).  The same result as
// k_quant_rows on the stored rows.  All NT threads call it.
template <int COLS, int NTH>
__device__ __forceinline__ void split_image_rows(const char* img, int pitch, int nrows, uint8_t* codes,
                                                 uint32_t* scales, long sld, int K, int c0) {
  constexpr int BPR = COLS / 32;  // 32-blocks per image row (even)
  static_assert(BPR % 2 == 0 && (TM * BPR) % NTH == 0, "blocks of a chunk in neighbouring lanes");
#pragma unroll
  for (int q = 0; q < TM * BPR / NTH; ++q) {
    const int b = threadIdx.x + NTH * q;
    const int row = b / BPR, jb = b % BPR;
    const bool live = row < nrows;
    float v[32];
    const u32x4* p = (const u32x4*)(img + row * pitch + jb * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = p[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * c + 2 * e] = bf2f(w[e] & 0xffffu);
        v[8 * c + 2 * e + 1] = bf2f(w[e] >> 16);
      }
    }
    uint32_t hi[6], lo[6];
    const uint32_t s1 = quant_term(v, hi);
    const uint32_t s2 = quant_term(v, lo);
    const uint32_t o1 = __shfl_xor(s1, 1, 64), o2 = __shfl_xor(s2, 1, 64);
    if (live) {
      const int j = c0 / 32 + jb;  // global 32-block
      uint8_t* chunk = codes + (long)row * (2 * K) + 128 * (j >> 1);
      store_term(chunk, 0, j & 1, hi);
      store_term(chunk, 1, j & 1, lo);
      if ((j & 1) == 0) scales[(long)(j >> 1) * sld + row] = s1 | (o1 << 8) | (s2 << 16) | (o2 << 24);
    }
  }
}

// ---------------------------------------------------------------------------
// Stage loader.  Activation rows through KA/KS (set by the caller: 256 tile
// rows, 128 bytes a stage), the weight tile and the two scale rows here.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_load4(rsrc_t rs, char* lds_wave_base, uint32_t off, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (v2::lds_void*)lds_wave_base, 4, off, soff, 0, 0);
}

// PK: the weight codes and scale words from a packed copy (pack.hip kinds 4,
// 5: 9 KB stage tiles in order), else gathered from the packed rows and the
// scale rows.  The activation scale words are stage-major in both.
template <bool PK>
struct WLoad {
  rsrc_t rq, rs;     // packed rows (row pitch K/2 bytes) and scale bytes (K/32); PK: rq = the copy
  uint32_t qoff;     // this lane's weight-tile slot: row 32 w + L/2, logical 16-byte chunk (PK: 1024 w + 16 L)
  uint32_t tile0;    // PK: byte offset of the N tile's first stage tile in the copy
  rsrc_t ra;         // activation scale words, [K/64][arows]
  uint32_t astage;   // bytes between two chunks' words of ra
  uint32_t soff;     // this lane's scale word (waves 0-3: activation rows, 4-7: weight rows)
  // tile row n of the weight tile reads packed row wrow(n); tile rows of the
  // activation side read scale-word row aoff(row) (byte offset of the row's
  // word of chunk 0, OFF_NONE for no row)
  template <class WROW, class AOFF>
  __device__ __forceinline__ void set(const uint8_t* wq, const uint8_t* ws, long wrows, int K, WROW wrow,
                                      const uint32_t* as, long arows, AOFF aoff) {
    static_assert(!PK, "rows of the plain layout");
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    rq = make_rsrc(wq, (uint64_t)wrows * (K / 2));
    rs = make_rsrc(ws, (uint64_t)wrows * (K / 32));
    set_act(as, arows, K);
    const int n = 32 * w + (L >> 1);
    const int lc = (L & 1) ^ ((n >> 3) & 1);
    qoff = (uint32_t)wrow(n) * (uint32_t)(K / 2) + 16u * (uint32_t)lc;
    if (w < 4)
      soff = aoff(64 * w + L);
    else
      soff = (uint32_t)wrow(64 * (w - 4) + L) * (uint32_t)(K / 32);
  }
  // PK: the expert's copy (`bytes` long), N tile nt of a matrix with nst
  // stages
  template <class AOFF>
  __device__ __forceinline__ void set_packed(const uint8_t* copy, uint64_t bytes, int nt, int nst, int K,
                                             const uint32_t* as, long arows, AOFF aoff) {
    static_assert(PK, "the packed copy");
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    rq = make_rsrc(copy, bytes);
    set_act(as, arows, K);
    tile0 = (uint32_t)nt * (uint32_t)nst * (uint32_t)MX_TILE;
    qoff = 1024u * (uint32_t)w + 16u * (uint32_t)L;
    soff = (w < 4) ? aoff(64 * w + L) : W_BYTES + 256u * (uint32_t)(w - 4) + 4u * (uint32_t)L;
  }
  __device__ __forceinline__ void set_act(const uint32_t* as, long arows, int K) {
    ra = make_rsrc(as, (uint64_t)arows * (K / 64) * 4);
    astage = (uint32_t)arows * 4u;
  }
  // queue stage s (k = 64 s) into the stage buffer `st`
  __device__ __forceinline__ void issue(int s, char* st) const {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (PK) {
      const uint32_t t = __builtin_amdgcn_readfirstlane(tile0 + (uint32_t)s * (uint32_t)MX_TILE);
      v2::lds_load16(rq, st + A_BYTES + 1024 * w, qoff, t);
      if (w < 4)
        lds_load4(ra, st + A_BYTES + W_BYTES + 256 * w, soff, astage * (uint32_t)s);
      else
        lds_load4(rq, st + A_BYTES + W_BYTES + AS_BYTES + 256 * (w - 4), soff, t);
    } else {
      v2::lds_load16(rq, st + A_BYTES + 1024 * w, qoff, 32u * (uint32_t)s);
      if (w < 4)
        lds_load4(ra, st + A_BYTES + W_BYTES + 256 * w, soff, astage * (uint32_t)s);
      else
        lds_load4(rs, st + A_BYTES + W_BYTES + AS_BYTES + 256 * (w - 4), soff, 4u * (uint32_t)(s >> 1));
    }
  }
};
static_assert(MX_TILE == W_BYTES + WS_BYTES, "a packed stage tile is the weight part of an LDS stage");

// One k64 step from stage buffer `st` (stage index s: which half of the
// weight scale word).  G: the bf16 geometry whose accumulator layout the
// caller keeps (eight waves, 4 x 2 blocks of 32 x 32 per wave).
template <class G>
__device__ __forceinline__ void mma_mx(const char* st, int s, f32x16 (&acc)[G::NB][G::MB], int wm, int wn,
                                       int lane) {
  static_assert(G::TM == TM && G::TN == TN && G::NW == NW, "256 x 256 tile, eight waves");
  const int h = lane >> 5, r = lane & 31;
  const char* sA = st;
  const char* sW = st + A_BYTES;
  const uint32_t* sAs = (const uint32_t*)(st + A_BYTES + W_BYTES);
  const uint32_t* sWs = (const uint32_t*)(st + A_BYTES + W_BYTES + AS_BYTES);
  i32x8 wf[G::NB];
  int ws[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int n = G::n_local(wn, nb) + r;
    const u32x4 q = *(const u32x4*)(sW + n * 32 + 16 * (h ^ ((n >> 3) & 1)));
    wf[nb] = i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
    ws[nb] = (int)(sWs[n] >> (8 * (2 * (s & 1) + h)));
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int row = G::m_local(wm, mb) + r;
      const u32x4 a0 = *(const u32x4*)(sA + v2::koff<64>(row, 4 * t + h));
      const u32x2 a1 = *(const u32x2*)(sA + v2::koff<64>(row, 4 * t + 2) + 8 * h);
      const i32x8 xf = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], 0, 0};
      const int xs = (int)(sAs[row] >> (8 * (2 * t + h)));
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
        acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[nb], xf, acc[nb][mb], 4 /* first: fp4 */,
                                                                      2 /* second: fp6 E2M3 */, 0, ws[nb], 0, xs);
    }
}

// Geometry of the MXFP4 base GEMMs: the 256 x 256 tile as eight waves of
// 64 x 128 (two activation row blocks by four weight blocks).  Per k64 step
// a wave reads 48 bytes a lane of activation codes per row block and 16 of
// weight codes per weight block: the wider weight side reads 29 % fewer LDS
// bytes per product than 128 x 64 waves (k_w13 2.68 -> 2.60 ms, k_w2 1.054
// -> 1.031 ms at 98,304 rows with the packed weights).
using GMX = v2::Geo2<2, 4, 4, 2, false, false, 64>;
// Geometry of the low-rank extension stages that follow the base K range
// (bf16, the same accumulators: 64 k a stage, the two halves of the N tile
// contracting the two halves of the stage's k -- the SPLIT stages of the
// bf16 engine; two 64 KB buffers).
using GE = GMX;
static_assert(GE::NBUF * GE::STAGE <= LDS_BYTES + 2048, "the extension stages reuse the MX stage buffers");
using KE = v2::KLoad<TM, 64, NW>;
using KE2 = v2::KLoad<TM, 64, NW, true>;
constexpr int EXT_INSTS = 2 * KE::NJ;

// One extension stage (GE: 64 k, four k16 steps; the gate blocks contract
// the first two, the up blocks the last two), fragments read just before
// their MFMAs so that few are live next to the accumulators.
template <class G>
__device__ __forceinline__ void mma_ext(const char* st, f32x16 (&acc)[G::NB][G::MB], int wm, int wn, int lane) {
  const char* sM = st;
  const char* sN = st + GE::SM_BYTES;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8 b[G::MB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) b[mb] = v2::frag<false, GE::TM, 64>(sM, G::m_local(wm, mb), kk, lane);
#pragma unroll
    for (int nb = (kk / 2) * (G::NB / 2); nb < (kk / 2 + 1) * (G::NB / 2); ++nb) {
      const bf16x8 a = v2::frag<false, GE::TN, 64>(sN, G::n_local(wn, nb), kk, lane);
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[mb], acc[nb][mb], 0, 0, 0);
    }
  }
}

// The base K range, nst k64 stages (ld.issue(s, buffer); three buffers, two
// stages in flight), then -- in a loop of its own, so that each loop keeps
// one fragment schedule and the accumulators one register assignment --
// next extension stages (ld.issue_ext(s, buffer), bf16, two buffers).  Ends
// with a workgroup barrier (LDS free for the epilogue).
template <class G, class L>
__device__ __forceinline__ void run_mx(const L& ld, int next, int nst, f32x16 (&acc)[G::NB][G::MB], char* smem) {
  static_assert(GE::MB == G::MB && GE::NB == G::NB && GE::WM == G::WM && GE::WN == G::WN, "same accumulators");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = w / G::WN, wn = w % G::WN;
  if (nst > 0) {
    ld.issue(0, smem);
    if (nst > 1) ld.issue(1, smem + STAGE);
    for (int s = 0; s < nst; ++s) {
      if (s + 1 < nst)
        v2::wait_vm<INSTS>();
      else
        v2::wait_vm<0>();
      v2::bar();
      if (s + 2 < nst) ld.issue(s + 2, smem + ((s + 2) % NBUF) * STAGE);
      mma_mx<G>(smem + (s % NBUF) * STAGE, s, acc, wm, wn, lane);
    }
    __syncthreads();
  }
  if (next > 0) {  // two 64 KB buffers, one stage in flight
    ld.issue_ext(0, smem);
    for (int s = 0; s < next; ++s) {
      v2::wait_vm<0>();
      v2::bar();
      if (s + 1 < next) ld.issue_ext(s + 1, smem + ((s + 1) & 1) * GE::STAGE);
      mma_ext<G>(smem + (s & 1) * GE::STAGE, acc, wm, wn, lane);
    }
    __syncthreads();
  }
}

}  // namespace mx
}  // namespace moelora
