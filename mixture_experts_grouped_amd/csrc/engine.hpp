// engine.hpp -- bf16 MFMA tile engine for gfx950 (CDNA4).
//
// One workgroup = 256 threads = 4 wave64s.  A block computes a TM x TN tile of
//   C[m][n] = sum_k M[m][k] * N[n][k]
// where the "M side" supplies output rows (pool rows, tokens) and the "N side"
// supplies output columns (weight rows, adapter columns).  Both operands are
// staged into LDS as K-contiguous bf16 tiles (64 k per stage, 128 bytes per
// row, 16-byte chunks XOR-swizzled so that both the staging writes and the
// MFMA fragment reads are free of bank conflicts), double-buffered with one
// barrier per stage; global loads of stage s+1 are in flight while the MFMAs
// of stage s run.
//
// v_mfma_f32_32x32x16_bf16 is fed with the N-side fragment as its first
// operand and the M-side fragment as its second, so every lane owns one output
// row (m = lane % 32) and each group of four accumulator registers holds four
// consecutive output columns: epilogues store 16-byte (fp32) or 8-byte (bf16)
// runs per lane.  Lane layout (probed on the device): operand lane l carries
// row l % 32, k = 8 * (l / 32) .. +7; accumulator v of lane l is
// D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].
//
// Two staging patterns:
//   RowsK  -- the source is K-contiguous (x, weights in [out, in] layout used
//             as the N side of a forward GEMM); a thread moves 16-byte chunks.
//   TransK -- the source is K-outer ([k][n], n contiguous: weights in dgrad,
//             token rows in weight gradients); a thread loads an 8 x 8 block
//             (8 rows of 16 bytes), transposes it in registers and writes 8
//             K-contiguous chunks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NTHREADS = 256;
constexpr int KT = 64;     // k per stage
constexpr int LROW = 128;  // bytes per LDS tile row (KT bf16)

__device__ __forceinline__ int lds_off(int row, int c) {
  return row * LROW + ((c ^ (row & 7) ^ ((row >> 3) & 7)) << 4);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): v_cvt_pk_bf16_f32
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack2(f, 0.0f) & 0xffffu; }
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// two-term bf16 split of an fp32 value: v ~= hi + lo to about 16 significant bits
__device__ __forceinline__ void split_hl(float v, uint32_t& hi, uint32_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

// logistic sigmoid; the reciprocal is v_rcp_f32 (1 ulp) rather than an IEEE
// division (about ten instructions), which dominated the activation epilogues
__device__ __forceinline__ float sigmoidf_(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// erfc(x) for x >= 0 given ex2 = exp(-x^2): Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (erf to within 1.5e-7 absolute):
// erfc(x) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1/(1 + p x).
__device__ __forceinline__ float erfc_as7126(float x, float ex2) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = 1.061405429f;
  q = fmaf(q, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  return q * t * ex2;
}
// Phi(g) and phi(g) of the standard normal distribution (exact GELU = g Phi(g),
// gelu' = Phi + g phi) with one exponential:
// Phi(g) = erfc(-g / sqrt2) / 2, the tail taken directly (no 1 - erf
// cancellation for g < 0); exp(-x^2) at x = |g| / sqrt2 is exp(-g^2 / 2).
__device__ __forceinline__ void norm_cdf_pdf(float g, float& cdf, float& pdf) {
  const float e2 = __expf(-0.5f * g * g);
  const float half_tail = 0.5f * erfc_as7126(fabsf(g) * 0.70710678118654752f, e2);
  cdf = g < 0.0f ? half_tail : 1.0f - half_tail;
  pdf = 0.39894228040143268f * e2;
}
__device__ __forceinline__ float norm_cdf(float g) {
  float c, p;
  norm_cdf_pdf(g, c, p);
  return c;
}

// ---------------------------------------------------------------------------
// tile geometry: WM x WN waves, each wave MB x NB blocks of 32 x 32
// ---------------------------------------------------------------------------
template <int MB_, int NB_, int WM_, int WN_>
struct Geo {
  static constexpr int MB = MB_, NB = NB_, WM = WM_, WN = WN_;
  static constexpr int TM = WM * MB * 32, TN = WN * NB * 32;
  static constexpr int LDS_STAGE = (TM + TN) * LROW;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
  static_assert(WM * WN == 4, "four waves");
  static_assert(NB % 2 == 0, "N blocks come in pairs");
  // rows of the M tile owned by (wave row wm, block mb)
  __device__ static constexpr int m_local(int wm, int mb) { return (wm * MB + mb) * 32; }
  // columns of the N tile owned by (wave column wn, block nb): the first NB/2
  // blocks lie in the first half of the tile, the rest at the same offset in
  // the second half, so a wave holds column n and its partner n + TN/2.
  __device__ static constexpr int n_local(int wn, int nb) {
    return (nb < NB / 2 ? 0 : TN / 2) + (wn * (NB / 2) + (nb % (NB / 2))) * 32;
  }
};

// One stage of MFMAs.  SPLIT: the first half of the N tile contracts only the
// first 32 k of the stage, the second half only the last 32 k (two independent
// K ranges packed into one stage).
template <class G, bool SPLIT>
__device__ __forceinline__ void load_frags(const char* sM, const char* sN, bf16x8 (&a)[G::NB],
                                           bf16x8 (&b)[G::MB], int kk, int wm, int wn, int lane) {
  const int r = lane & 31, c = kk * 2 + (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
    b[mb] = *(const bf16x8*)(sM + lds_off(G::m_local(wm, mb) + r, c));
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    if (SPLIT && ((nb < G::NB / 2) != (kk < 2))) continue;
    a[nb] = *(const bf16x8*)(sN + lds_off(G::n_local(wn, nb) + r, c));
  }
}

// One stage of MFMAs.  SPLIT: the first half of the N tile contracts only the
// first 32 k of the stage, the second half only the last 32 k (two independent
// K ranges packed into one stage).  Fragments of step kk + 1 are read from LDS
// while the MFMAs of step kk run.
template <class G, bool SPLIT>
__device__ __forceinline__ void mma_stage(const char* sM, const char* sN,
                                          f32x16 (&acc)[G::NB][G::MB], int wm, int wn,
                                          int lane) {
  bf16x8 a[2][G::NB], b[2][G::MB];
  load_frags<G, SPLIT>(sM, sN, a[0], b[0], 0, wm, wn, lane);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < 4) load_frags<G, SPLIT>(sM, sN, a[cur ^ 1], b[cur ^ 1], kk + 1, wm, wn, lane);
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
      if (SPLIT && ((nb < G::NB / 2) != (kk < 2))) continue;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
        acc[nb][mb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][nb], b[cur][mb], acc[nb][mb], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Global loads go through buffer resource descriptors: the base address and
// the byte extent live in scalar registers, every lane supplies a 32-bit byte
// offset, and an offset past the extent reads zero in hardware.  Masked rows
// and k outside a window therefore cost a select, not a branch.  One
// descriptor covers at most 2 GB; callers base it at the expert, tile or
// tensor they read.
// ---------------------------------------------------------------------------
constexpr int cmax(int a, int b) { return a > b ? a : b; }

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OFF_NONE = 0x80000000u;
constexpr uint64_t RSRC_MAX = 0x7FFFFFF0ull;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = (uint32_t)(bytes < RSRC_MAX ? bytes : RSRC_MAX);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// ---------------------------------------------------------------------------
// RowsK: K-contiguous bf16 rows.  Thread t moves chunk c = t % 8 of tile rows
// t / 8 + 32 i.  roff[i] is the byte offset of that row in `rs` (OFF_NONE:
// the row reads zero).  The stage's k coordinate is read through a window
// [lo, lo + span) where lo = (row >= lo_split ? lo_b : 0); inside it the
// source column is k - lo, folded by `period` when non-zero (a rank-r row
// repeated for the hi and lo halves of a split operand).
// In SPLIT stages chunk c < 4 reads k = k0 + 8c and chunk c >= 4 reads
// k = khalf + k0 + 8(c - 4).
// ---------------------------------------------------------------------------
template <int R>
struct RowsK {
  static constexpr int NI = R / 32;
  rsrc_t rs, rs2;  // rs2 serves tile rows >= R/2 when two_rs (two source tensors)
  bool two_rs;
  uint32_t roff[NI];
  int span, period, lo_split, lo_b;
  u32x4 v[NI];

  __device__ __forceinline__ void window(int span_, int period_ = 0, int lo_split_ = 1 << 30,
                                         int lo_b_ = 0) {
    span = span_;
    period = period_;
    lo_split = lo_split_;
    lo_b = lo_b_;
  }
  __device__ __forceinline__ void load(int k0, int khalf, bool split) {
    const int c = threadIdx.x & 7;
    const int kc = split ? ((c < 4) ? k0 + 8 * c : khalf + k0 + 8 * (c - 4)) : k0 + 8 * c;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = kc - (row_of(i) >= lo_split ? lo_b : 0);
      const int kk = (period != 0 && k >= period) ? k - period : k;
      const bool ok = (k >= 0) && (k < span) && (roff[i] != OFF_NONE);
      v[i] = bload((two_rs && i >= NI / 2) ? rs2 : rs, ok ? roff[i] + 2u * (uint32_t)kk : OFF_NONE);
    }
  }
  __device__ __forceinline__ void store(char* s) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NI; ++i) *(u32x4*)(s + lds_off((t >> 3) + 32 * i, t & 7)) = v[i];
  }
  // tile row owned by slot i of this thread
  __device__ static __forceinline__ int row_of(int i) { return (threadIdx.x >> 3) + 32 * i; }

  // rows row0 + j (j < nvalid) of a row-major tensor with `ld` elements per row
  __device__ __forceinline__ void contig(const uint16_t* base, long row0, long nvalid, long ld) {
    rs = make_rsrc(base + row0 * ld, (uint64_t)(nvalid > 0 ? nvalid : 0) * ld * 2);
    two_rs = false;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      roff[i] = (row_of(i) < nvalid) ? (uint32_t)(row_of(i) * ld * 2) : OFF_NONE;
  }
  // token of each owned pool row row0 + j (-1 past nvalid), loaded once
  __device__ static __forceinline__ void tokens(int (&tk)[NI], const int32_t* row2r, int topk,
                                                long row0, long nvalid) {
#pragma unroll
    for (int i = 0; i < NI; ++i) tk[i] = (row_of(i) < nvalid) ? row2r[row0 + row_of(i)] / topk : -1;
  }
  // rows tk[i] of a token-major tensor (no memory access)
  __device__ __forceinline__ void from_tokens(const uint16_t* base, long ntok, long ld,
                                              const int (&tk)[NI]) {
    rs = make_rsrc(base, (uint64_t)ntok * ld * 2);
    two_rs = false;
#pragma unroll
    for (int i = 0; i < NI; ++i) roff[i] = (tk[i] >= 0) ? (uint32_t)((long)tk[i] * ld * 2) : OFF_NONE;
  }
  // pool rows row0 + j (j < nvalid) -> rows (token of the route) of `base`
  __device__ __forceinline__ void gather(const uint16_t* base, long ntok, long ld,
                                         const int32_t* row2r, int topk, long row0, long nvalid) {
    rs = make_rsrc(base, (uint64_t)ntok * ld * 2);
    two_rs = false;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      roff[i] = (row_of(i) < nvalid) ? (uint32_t)((long)(row2r[row0 + row_of(i)] / topk) * ld * 2)
                                     : OFF_NONE;
  }
};

// ---------------------------------------------------------------------------
// TransK: K-outer source rows ([k][n], n contiguous).  Tile = R columns x 64 k,
// made of 8 x 8 blocks; thread t < R handles block (nb = t % (R/8),
// kb = t / (R/8)).  The policy KP fetches 16 bytes of k-row k at a column
// byte offset (zero for rows or columns outside the source).  Tile column n reads source column n0 + n for
// n < nvalid.  With hilo_half > 0 the tile holds two halves: columns
// [0, half) read source column n0 + n and columns [half, 2 half) read source
// column n0 + lo_off + (n - half), each valid for n % half < nvalid.
// ---------------------------------------------------------------------------
template <int R, class KP>
struct TransK {
  KP kp;
  int n0, nvalid, hilo_half, lo_off;
  u32x4 v[8];

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
  __device__ __forceinline__ void load(int k0) {
    const int t = threadIdx.x;
    if (t >= R) return;
    const int nb = t % (R / 8), kb = t / (R / 8);
    const uint32_t co = col_off(nb * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = kp.fetch(k0 + kb * 8 + i, co);
  }
  __device__ __forceinline__ void store(char* s) const {
    const int t = threadIdx.x;
    if (t >= R) return;
    const int nb = t % (R / 8), kb = t / (R / 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = v[2 * d][j >> 1], b = v[2 * d + 1][j >> 1];
        o[d] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *(u32x4*)(s + lds_off(nb * 8 + j, kb)) = o;
    }
  }
};

// k-row policies for TransK
__device__ __forceinline__ u32x4 fetch_at(rsrc_t rs, uint32_t ro, uint32_t co) {
  return bload(rs, (ro != OFF_NONE && co != OFF_NONE) ? ro + co : OFF_NONE);
}
struct KStrided {  // rows of a matrix: k in [lo, lo + span) -> row (k - lo) folded by period
  rsrc_t rs;
  uint32_t ldb;  // row pitch in bytes
  int lo, span, period;
  __device__ __forceinline__ u32x4 fetch(int k, uint32_t co) const {
    int kk = k - lo;
    const bool ok = kk >= 0 && kk < span;
    if (period != 0 && kk >= period) kk -= period;
    return fetch_at(rs, ok ? (uint32_t)kk * ldb : OFF_NONE, co);
  }
};
struct KRows {  // k-th row of a contiguous range of pool rows or tokens
  // mode 0: row k of the range (rs based at the range's first row)
  // mode 1: pool row (row0 + k) -> its token's row (rs based at the tensor;
  //         map = row -> route)
  // mode 2: token (row0 + k) -> pool row of its first live route, read from
  //         `base` with a plain load (the whole pool may exceed one
  //         descriptor); map = route -> row; no live route reads zero
  rsrc_t rs;
  uint32_t ldb;
  const int32_t* map;
  const uint16_t* base;
  int topk;
  int row0, nrows, mode;
  __device__ __forceinline__ u32x4 fetch(int k, uint32_t co) const {
    if (mode == 2) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k < nrows && co != OFF_NONE) {
        const long t = row0 + k;
        long pr = -1;
        for (int j = 0; j < topk && pr < 0; ++j) pr = map[t * topk + j];
        if (pr >= 0) v = *(const u32x4*)((const char*)base + pr * (long)ldb + co);
      }
      return v;
    }
    uint32_t ro = OFF_NONE;
    if (k < nrows) ro = (uint32_t)((mode == 1) ? (long)(map[row0 + k] / topk) : (long)k) * ldb;
    return fetch_at(rs, ro, co);
  }
};

// ---------------------------------------------------------------------------
// main loop: `L` provides load(stage) (global -> registers) and
// store(sM, sN) (registers -> LDS).  run_stages accumulates `nst` stages into
// acc; consecutive runs (e.g. the base K range, then a low-rank extension with
// its own loader) share the accumulators.  Each run ends with a barrier so
// the next run may overwrite the LDS buffers.
// ---------------------------------------------------------------------------
template <class G>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[G::NB][G::MB]) {
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[nb][mb][q] = 0.0f;
}

template <class G, bool SPLIT, class L>
__device__ __forceinline__ void run_stages(L& ld, int nst, f32x16 (&acc)[G::NB][G::MB],
                                           char* smem) {
  if (nst <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / G::WN, wn = w % G::WN;
  ld.load(0);
  for (int s = 0; s < nst; ++s) {
    char* sM = smem + (s & 1) * G::LDS_STAGE;
    char* sN = sM + G::TM * LROW;
    ld.store(sM, sN);
    __syncthreads();
    if (s + 1 < nst) ld.load(s + 1);
    mma_stage<G, SPLIT>(sM, sN, acc, wm, wn, lane);
  }
  __syncthreads();
}

template <class G, class L>
__device__ __forceinline__ void mainloop(L& ld, int nst, f32x16 (&acc)[G::NB][G::MB], char* smem) {
  zero_acc<G>(acc);
  run_stages<G, false>(ld, nst, acc, smem);
}

// Epilogue coordinates of accumulator (nb, mb, group g) for this lane:
// output row m_local + (lane & 31), columns n .. n + 3.
template <class G>
struct Epi {
  int wm, wn, lane;
  __device__ Epi() {
    const int w = threadIdx.x >> 6;
    wm = w / G::WN;
    wn = w % G::WN;
    lane = threadIdx.x & 63;
  }
  __device__ __forceinline__ int row(int mb) const { return G::m_local(wm, mb) + (lane & 31); }
  __device__ __forceinline__ int col(int nb, int g) const {
    return G::n_local(wn, nb) + 8 * g + 4 * (lane >> 5);
  }
};

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8) and each XCD has its own L2.  xcd_remap turns the hardware id into a
// logical id such that every XCD walks a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int x = b & 7, j = b >> 3;
  const int q = nblocks >> 3, rem = nblocks & 7;
  return x * q + (x < rem ? x : rem) + j;
}
// Grouped-GEMM M tile: rows [row0, row_end) of expert e in the pool.
struct TileInfo {
  int e, row0, row_end, pad;  // e: the tile's pool group (its expert, with several adapters its adapter too)
};

}  // namespace moelora
