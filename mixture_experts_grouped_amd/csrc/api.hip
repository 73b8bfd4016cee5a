// api.hip -- the C ABI of libmoelora: host-side validation, workspace plan and
// launch order.  All checks run before any device work; on error nothing is
// launched and nothing is written.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moelora.h"
#include "layer.hpp"

using namespace moelora;

namespace {

constexpr int kVersion = 100;
constexpr int kBlockMs[] = {16, 32, 64, 96, 128, 192, 240};
constexpr int kSharedSplit = 1024;  // tokens per split of the shared-factor reductions
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

static_assert(MOE_ACT_SWIGLU == 0 && MOE_ACT_GEGLU == 1, "kernels take the activation as template 0 / 1");
static_assert(MOE_SAVED_STATUS_OFFSET == 0, "the status word is the first field of the saved plan");
static_assert(MOE_MAX_ADAPTERS == MAX_ADAPTERS, "one adapter limit");

moe_status check_desc(const moe_lora_desc* d) {
  if (d == nullptr) return MOE_ERR_INVALID;
  if (d->T < 1 || d->H < 1 || d->I < 1 || d->E < 1 || d->topk < 1 || d->rank < 1)
    return MOE_ERR_INVALID;
  if (!std::isfinite(d->scale)) return MOE_ERR_INVALID;
  if (d->block_m != 0) {
    bool ok = false;
    for (int b : kBlockMs) ok |= (b == d->block_m);
    if (!ok) return MOE_ERR_INVALID;
  }
  if (d->H % 256 != 0 || d->I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->E > 512 || d->topk > 16 || d->rank > 256) return MOE_ERR_UNSUPPORTED;
  if (d->activation != MOE_ACT_SWIGLU && d->activation != MOE_ACT_GEGLU) return MOE_ERR_UNSUPPORTED;
  if (std::isnan(d->clamp)) return MOE_ERR_INVALID;
  if (d->base_format != MOE_BASE_BF16 && d->base_format != MOE_BASE_MXFP4) return MOE_ERR_UNSUPPORTED;
  const int64_t routes = (int64_t)d->T * d->topk;
  const int64_t cap = routes + std::min<int64_t>(d->E, routes) * 239;
  if (cap >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  // token-indexed rows (x, grad_out) and one expert's weights are each read
  // through one 32-bit-offset buffer descriptor
  if ((int64_t)d->T * d->H * 2 > 0x7FFFFFF0LL || (int64_t)4 * d->I * d->H > 0x7FFFFFF0LL)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The roots of a call: one adapter holding every token, or the caller's.
struct Roots {
  int na = 1;
  int r[MAX_ADAPTERS + 1] = {};
  int tiles(int tm) const {  // token tiles of tm tokens that never cross roots
    int n = 0;
    for (int q = 0; q < na; ++q) n += (r[q + 1] - r[q] + tm - 1) / tm;
    return n;
  }
};

// ad == nullptr: a single adapter.  Otherwise count in [1, MAX_ADAPTERS] and
// host offsets 0 = o[0] <= o[1] <= ... <= o[count] = T.
moe_status read_roots(const moe_lora_desc* d, const moe_adapters* ad, Roots& out) {
  out = Roots{};
  if (ad == nullptr) {
    out.r[1] = d->T;
    return MOE_OK;
  }
  if (ad->offsets == nullptr || ad->count < 1) return MOE_ERR_INVALID;
  if (ad->count > MAX_ADAPTERS) return MOE_ERR_UNSUPPORTED;
  if (ad->offsets[0] != 0 || ad->offsets[ad->count] != d->T) return MOE_ERR_INVALID;
  for (int q = 0; q < ad->count; ++q)
    if (ad->offsets[q + 1] < ad->offsets[q]) return MOE_ERR_INVALID;
  out.na = ad->count;
  for (int q = 0; q <= ad->count; ++q) out.r[q] = ad->offsets[q];
  // the pool's row indices are int32 at any BLOCK_M
  const int64_t routes = (int64_t)d->T * d->topk;
  if (routes + std::min<int64_t>((int64_t)d->E * out.na, routes) * 239 >= (int64_t)1 << 31)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// check_desc, then the roots
moe_status check_call(const moe_lora_desc* d, const moe_adapters* ad, Roots& R) {
  const moe_status st = check_desc(d);
  return st != MOE_OK ? st : read_roots(d, ad, R);
}

// The kernels' rank: a multiple of 8.  A caller's rank below it runs on
// copies of the factors widened with zero rows or columns (the extra rank
// terms are exactly zero), whose gradients are cut back afterwards.
int rank_p(const moe_lora_desc* d) { return (d->rank + 7) & ~7; }
bool padded(const moe_lora_desc* d) { return rank_p(d) != d->rank; }

// Element offsets of the six factors of na adapters at rank rp in one
// contiguous block: A1, A3 [na, rp, H]; B1, B3 [na, E, I, rp];
// A2 [na, E, rp, I]; B2 [na, H, rp] (the gradients use the same layout).
struct FacBlock {
  size_t A1, A3, B1, B3, A2, B2, total;
  FacBlock(const moe_lora_desc* d, int na) {
    const size_t rp = rank_p(d), H = d->H, I = d->I, E = d->E;
    size_t o = 0;
    auto take = [&](size_t n) { const size_t at = o; o += (n + 127) & ~(size_t)127; return at; };  // 256-byte aligned
    A1 = take(na * rp * H);
    A3 = take(na * rp * H);
    B1 = take(na * E * I * rp);
    B3 = take(na * E * I * rp);
    A2 = take(na * E * rp * I);
    B2 = take(na * H * rp);
    total = o;
  }
};

int resolve_bm(const moe_lora_desc* d) {
  // The grouped-GEMM tiles start at each expert's first row and mask at its
  // count, so BLOCK_M changes only the padding; the smallest value wastes least.
  return d->block_m != 0 ? d->block_m : 16;
}

// Pool rows: every route plus the padding of each (expert, adapter) group.
int64_t capacity_of(const moe_lora_desc* d, int bm, int na = 1) {
  const int64_t routes = (int64_t)d->T * d->topk;
  return routes + std::min<int64_t>((int64_t)d->E * na, routes) * (bm - 1);
}

// At most 48 routes per (expert, adapter) group on average (bf16 base): most
// groups then fit one 64-row part, so the base GEMMs take 64-row parts (a
// larger group re-reads its weights per part).
bool small_tiles_of(const moe_lora_desc* d, int na) {
  return d->base_format == MOE_BASE_BF16 && (int64_t)d->T * d->topk <= (int64_t)48 * d->E * na;
}

// At most half as many routes as (expert, adapter) groups: the P product
// reads B1_e^T, B3_e^T copied for the groups that hold rows.
bool few_routes_of(const moe_lora_desc* d, int na) {
  return 2 * (int64_t)d->T * d->topk <= (int64_t)d->E * na;
}

struct Plan {
  int64_t cap;
  int maxtiles, maxtiles3, nsplit;
  size_t saved, scratch, fwd_scratch;
  // byte offsets
  size_t o_status, o_tiles, o_tiles3, o_ntiles, o_Xs, o_ZA, o_G, o_V, o_Hh, o_Z2, o_Yb, o_zc;
  size_t o_XQ, o_XS, o_HQ, o_HS;
  size_t o_fac, o_gfac, o_zsp, o_qp, o_q, o_sq, o_wsq, o_dGV, o_dU, o_P, o_pc, o_part, o_ZAp, o_dwp, o_A2T, o_A1T, o_A3T, o_B1T, o_B3T;
};

Plan make_plan(const moe_lora_desc* d, const Roots& R) {
  Plan p{};
  const int bm = resolve_bm(d);
  p.cap = capacity_of(d, bm, R.na);
  const int64_t routes = (int64_t)d->T * d->topk;
  p.maxtiles = (int)((routes + TMG - 1) / TMG + std::min<int64_t>((int64_t)d->E * R.na, routes));
  p.maxtiles3 = (int)((routes + TML - 1) / TML + std::min<int64_t>((int64_t)d->E * R.na, routes));
  p.nsplit = R.tiles(kSharedSplit);  // chunks of the shared-factor reductions, per root
  const size_t T = d->T, H = d->H, I = d->I, r = rank_p(d), cap = (size_t)p.cap;
  const size_t facb = padded(d) ? FacBlock(d, R.na).total * 2 : 0;  // the zero-padded factor copies
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = up(o + bytes); return at; };
  p.o_status = take(sizeof(int32_t));  // MOE_SAVED_STATUS_OFFSET
  p.o_tiles = take(sizeof(TileInfo) * p.maxtiles);
  p.o_tiles3 = take(sizeof(TileInfo) * p.maxtiles3);
  p.o_ntiles = take(2 * sizeof(int));
  p.o_Xs = take(T * H * 2);
  p.o_ZA = take(T * 4 * r * 2);
  p.o_G = take((size_t)p.maxtiles * TMG * I * 2);  // fp16, accumulator-blocked per M tile
  p.o_V = take((size_t)p.maxtiles * TMG * I * 2);
  p.o_Hh = take(cap * I * 2);
  p.o_zc = take(T * 2 * r * 2);
  p.saved = o;
  o = 0;
  // the forward's scratch first (Yb in dU's space, the shrink's split
  // partials, Z2 in P's), so that it is one prefix of the plan: fwd_scratch
  // bytes
  p.o_fac = take(facb);
  p.o_dU = take(cap * H * 2);
  p.o_zsp = take(KSPLIT * T * 2 * r * 4);
  p.o_P = take(cap * 2 * r * 4);
  p.fwd_scratch = p.o_P + up(cap * r * 4);  // Z2 = the first cap * r floats of P
  if (d->base_format == MOE_BASE_MXFP4) {
    // the split activations of the two base GEMMs (forward only)
    p.o_XQ = take(T * 2 * H);
    p.o_XS = take(T * (H / 64) * 4);
    p.o_HQ = take(cap * 2 * I);
    p.o_HS = take(cap * (I / 64) * 4);
    p.fwd_scratch = o;
  }
  p.o_gfac = take(facb);  // the padded rank's gradients, before they are cut back
  p.o_q = take(T * r * 4);
  p.o_qp = take(KSPLIT * T * r * 4);
  p.o_sq = take(T * 2 * r * 2);
  p.o_wsq = take(cap * 2 * r * 2);
  p.o_dGV = take(cap * 2 * I * 2);
  p.o_pc = take(T * 4 * r * 2);
  p.o_part = take((size_t)3 * p.nsplit * H * r * 4);
  p.o_ZAp = take(cap * 4 * r * 2);
  p.o_dwp = take((size_t)(I / 256) * cap * 4);
  const size_t na = R.na;
  p.o_A2T = take(na * d->E * I * r * 2);  // A2_e^T per adapter, with transformed base weights
  p.o_A1T = take(na * H * r * 2);         // A1^T, A3^T per adapter for the grad-x rank product
  p.o_A3T = take(na * H * r * 2);
  const size_t nbt = few_routes_of(d, R.na) ? na * d->E * I * r * 2 : 0;
  p.o_B1T = take(nbt);  // B1_e^T, B3_e^T for the few-route P product
  p.o_B3T = take(nbt);
  // forward-only tensors share space with backward-only ones: the base
  // outputs and Z2 are read only by the forward's combine
  p.o_Yb = p.o_dU;  // [cap, H] bf16, same size
  p.o_Z2 = p.o_P;   // [cap, r] fp32 inside [cap, 2r] fp32
  p.scratch = o;
  return p;
}

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

moe_status check_pool(const moe_lora_desc* d, const moe_pool* pool, const Plan& p) {
  if (pool == nullptr || pool->counts == nullptr || pool->offsets == nullptr ||
      pool->route_to_row == nullptr || pool->row_to_route == nullptr)
    return MOE_ERR_INVALID;
  if (pool->block_m != resolve_bm(d) || pool->capacity != p.cap) return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status check_params(const moe_lora_desc* d, const moe_lora_params* w) {
  if (w == nullptr) return MOE_ERR_INVALID;
  const void* ps[] = {w->W13, w->W2, w->A1, w->A3, w->B1, w->B3, w->A2, w->B2};
  for (const void* q : ps)
    if (!aligned16(q)) return MOE_ERR_INVALID;
  // scales: present exactly for an MXFP4 base (byte arrays, no alignment needed)
  const bool mx = d->base_format == MOE_BASE_MXFP4;
  if (mx != (w->W13_scale != nullptr) || mx != (w->W2_scale != nullptr)) return MOE_ERR_INVALID;
  // transformed base weights: optional bf16 copies (for an MXFP4 base, of
  // the dequantised weights)
  if ((w->W13T != nullptr && !aligned16(w->W13T)) || (w->W2T != nullptr && !aligned16(w->W2T)))
    return MOE_ERR_INVALID;
  // packed forward copies (bf16 stage tiles, or MXFP4 codes + scale words)
  if ((w->W13P != nullptr && !aligned16(w->W13P)) || (w->W2P != nullptr && !aligned16(w->W2P)))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

void fill_common(LayerArgs& a, const moe_lora_desc* d, const moe_pool* pool, const Plan& p,
                 const moe_lora_params* w, const Roots& R) {
  std::memset(&a, 0, sizeof(a));
  a.T = d->T;
  a.H = d->H;
  a.I = d->I;
  a.E = d->E;
  a.na = R.na;
  a.EV = d->E * R.na;
  a.small_tiles = small_tiles_of(d, R.na);
  a.few_routes = few_routes_of(d, R.na);
  // at least 768 routes per group on average: the TML-row tiles then pad
  // little more than TMG-row ones
  a.large_tiles = d->base_format == MOE_BASE_BF16 && (int64_t)d->T * d->topk >= (int64_t)768 * a.EV;
  for (int q = 0; q <= R.na; ++q) a.roots[q] = R.r[q];
  a.k = d->topk;
  a.r = rank_p(d);
  a.s = d->scale;
  a.cap = p.cap;
  a.maxtiles = p.maxtiles;
  a.maxtiles3 = p.maxtiles3;
  a.nsplit = p.nsplit;
  a.kspl = kSharedSplit;
  a.counts = pool->counts;
  a.offsets = pool->offsets;
  a.r2row = pool->route_to_row;
  a.row2r = pool->row_to_route;
  a.W13 = (const uint16_t*)w->W13;
  a.W2 = (const uint16_t*)w->W2;
  a.W13T = (const uint16_t*)w->W13T;
  a.W13P = (const uint16_t*)w->W13P;
  a.W2P = (const uint16_t*)w->W2P;
  a.W2T = (const uint16_t*)w->W2T;
  a.mx = d->base_format == MOE_BASE_MXFP4;
  a.act = d->activation;
  a.clamp = (d->clamp > 0.0f && std::isfinite(d->clamp)) ? d->clamp : 0.0f;
  if (a.mx) {
    a.W13q = (const uint8_t*)w->W13;
    a.W2q = (const uint8_t*)w->W2;
    a.W13s = w->W13_scale;
    a.W2s = w->W2_scale;
  }
  a.A1 = (const uint16_t*)w->A1;
  a.A3 = (const uint16_t*)w->A3;
  a.B1 = (const uint16_t*)w->B1;
  a.B3 = (const uint16_t*)w->B3;
  a.A2 = (const uint16_t*)w->A2;
  a.B2 = (const uint16_t*)w->B2;
}

void fill_saved(LayerArgs& a, const Plan& p, void* saved) {
  char* b = (char*)saved;
  a.status = (int*)(b + p.o_status);
  a.tiles = (TileInfo*)(b + p.o_tiles);
  a.tiles3 = (TileInfo*)(b + p.o_tiles3);
  a.ntiles = (int*)(b + p.o_ntiles);
  a.Xs = (uint16_t*)(b + p.o_Xs);
  a.ZA = (uint16_t*)(b + p.o_ZA);
  a.G = (_Float16*)(b + p.o_G);
  a.V = (_Float16*)(b + p.o_V);
  a.Hh = (uint16_t*)(b + p.o_Hh);
  a.zc = (uint16_t*)(b + p.o_zc);
}

void fill_scratch(LayerArgs& a, const Plan& p, void* base) {
  char* b = (char*)base;
  a.q = (float*)(b + p.o_q);
  a.qp = (float*)(b + p.o_qp);
  a.zsp = (float*)(b + p.o_zsp);
  a.sq = (uint16_t*)(b + p.o_sq);
  a.wsq = (uint16_t*)(b + p.o_wsq);
  a.dGV = (uint16_t*)(b + p.o_dGV);
  a.dU = (uint16_t*)(b + p.o_dU);
  a.P = (float*)(b + p.o_P);
  a.pc = (uint16_t*)(b + p.o_pc);
  a.part = (float*)(b + p.o_part);
  a.ZAp = (uint16_t*)(b + p.o_ZAp);
  a.Z2 = (float*)(b + p.o_Z2);
  a.Yb = (uint16_t*)(b + p.o_Yb);
  a.dwp = (float*)(b + p.o_dwp);
  a.A2T = (uint16_t*)(b + p.o_A2T);
  a.B1T = (uint16_t*)(b + p.o_B1T);
  a.B3T = (uint16_t*)(b + p.o_B3T);
  a.A1T = (uint16_t*)(b + p.o_A1T);
  if (a.mx) {
    a.XQ = (uint8_t*)(b + p.o_XQ);
    a.XS = (uint32_t*)(b + p.o_XS);
    a.HQ = (uint8_t*)(b + p.o_HQ);
    a.HS = (uint32_t*)(b + p.o_HS);
  }
  a.A3T = (uint16_t*)(b + p.o_A3T);
}

// ---------------------------------------------------------------------------
// The allocation-free forward (moe_lora_forward_noalloc) keeps its scratch in
// this file-scope device array.  Each device holds its own copy for the life
// of the process; its address on a device comes from hipGetSymbolAddress,
// taken once per device with that device current (in host code the array's
// name is not a device address).  Calls on one device share the array, so
// calls that overlap on one device race; nothing in it needs to start at
// zero (the forward writes every scratch element it later reads).
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up on its first use).
hipError_t scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// A rank that is not a multiple of 8 (rank_p): the six factors copied into
// the plan's zero-padded block, the layer pointed at the copies; after the
// backward its gradients are cut back into the caller's tensors.
struct PadJob {
  size_t off;     // in the factor block (elements)
  long nb;        // [nb, rows, cols] caller view
  int rows, cols, rows_p, cols_p;
};
void pad_jobs(const moe_lora_desc* d, int na, PadJob (&j)[6]) {
  const FacBlock f(d, na);
  const int r = d->rank, rp = rank_p(d), H = d->H, I = d->I;
  const long nE = (long)na * d->E;
  j[0] = PadJob{f.A1, na, r, H, rp, H};               // A1 [na, r, H]
  j[1] = PadJob{f.A3, na, r, H, rp, H};               // A3
  j[2] = PadJob{f.B1, nE * I, 1, r, 1, rp};           // B1 [na, E, I, r]
  j[3] = PadJob{f.B3, nE * I, 1, r, 1, rp};           // B3
  j[4] = PadJob{f.A2, nE, r, I, rp, I};               // A2 [na, E, r, I]
  j[5] = PadJob{f.B2, (long)na * H, 1, r, 1, rp};     // B2 [na, H, r]
}
hipError_t pad_factors(LayerArgs& a, const moe_lora_desc* d, const Plan& p, int na, void* scratch,
                       hipStream_t st) {
  if (!padded(d)) return hipSuccess;
  PadJob j[6];
  pad_jobs(d, na, j);
  uint16_t* b = (uint16_t*)((char*)scratch + p.o_fac);
  const uint16_t** fac[6] = {&a.A1, &a.A3, &a.B1, &a.B3, &a.A2, &a.B2};
  for (int i = 0; i < 6; ++i) {
    const hipError_t e = launch_pad(*fac[i], b + j[i].off, j[i].nb, j[i].rows, j[i].cols, j[i].rows_p, j[i].cols_p, st);
    if (e != hipSuccess) return e;
    *fac[i] = b + j[i].off;
  }
  return hipSuccess;
}
// the backward's gradient outputs: the padded block while the kernels run
void pad_grads(LayerArgs& a, const moe_lora_desc* d, const Plan& p, int na, void* scratch, uint16_t* (&user)[6]) {
  uint16_t** g[6] = {&a.dA1, &a.dA3, &a.dB1, &a.dB3, &a.dA2, &a.dB2};
  for (int i = 0; i < 6; ++i) user[i] = *g[i];
  if (!padded(d)) return;
  PadJob j[6];
  pad_jobs(d, na, j);
  uint16_t* b = (uint16_t*)((char*)scratch + p.o_gfac);
  for (int i = 0; i < 6; ++i) *g[i] = b + j[i].off;
}
hipError_t crop_grads(const LayerArgs& a, const moe_lora_desc* d, int na, uint16_t* const (&user)[6],
                      hipStream_t st) {
  if (!padded(d)) return hipSuccess;
  PadJob j[6];
  pad_jobs(d, na, j);
  const uint16_t* g[6] = {a.dA1, a.dA3, a.dB1, a.dB3, a.dA2, a.dB2};
  for (int i = 0; i < 6; ++i) {
    const hipError_t e = launch_pad(g[i], user[i], j[i].nb, j[i].rows_p, j[i].cols_p, j[i].rows, j[i].cols, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The forward behind both entry points.  noalloc: the scratch is the static
// array above (scratch / scratch_bytes are ignored); only the forward's part
// of the plan is used there.
moe_status forward_checked(const moe_lora_desc* d, const moe_adapters* ad, const moe_pool* pool, const void* x,
                           const float* topk_w, const moe_lora_params* params, void* out, void* saved,
                           size_t saved_bytes, void* scratch_arg, size_t scratch_bytes, bool noalloc,
                           void* stream) {
  Roots R;
  moe_status st = check_call(d, ad, R);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(d, R);
  if ((st = check_pool(d, pool, p)) != MOE_OK) return st;
  if ((st = check_params(d, params)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(out) || !aligned16(saved) || topk_w == nullptr)
    return MOE_ERR_INVALID;
  if (saved_bytes < p.saved) return MOE_ERR_WORKSPACE;
  const size_t act = (size_t)d->T * d->H * 2;
  const Range rx = rng(x, act), ro = rng(out, act), rs = rng(saved, p.saved);
  if (overlap(rx, ro) || overlap(ro, rs) || overlap(rx, rs)) return MOE_ERR_INVALID;
  void* sc = scratch_arg;
  if (noalloc) {
    if (p.fwd_scratch > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
    const hipError_t e = scratch_address(&sc);
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else {
    if (!aligned16(scratch_arg) || scratch_bytes < p.scratch) return MOE_ERR_WORKSPACE;
    const Range rsc = rng(scratch_arg, p.scratch);
    if (overlap(rsc, rx) || overlap(rsc, ro) || overlap(rsc, rs)) return MOE_ERR_INVALID;
  }
  LayerArgs a;
  fill_common(a, d, pool, p, params, R);
  fill_saved(a, p, saved);
  fill_scratch(a, p, sc);
  a.x = (const uint16_t*)x;
  a.w = topk_w;
  a.out = (uint16_t*)out;
  hipError_t e = pad_factors(a, d, p, R.na, sc, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_forward(a, (hipStream_t)stream, !noalloc);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status backward_checked(const moe_lora_desc* d, const moe_adapters* ad, const moe_pool* pool,
                            const void* grad_out, const float* topk_w, const moe_lora_params* params,
                            const void* saved, size_t saved_bytes, void* grad_x, float* grad_topk_w,
                            const moe_lora_grads* grads, void* scratch, size_t scratch_bytes, void* stream) {
  Roots R;
  moe_status st = check_call(d, ad, R);
  if (st != MOE_OK) return st;
  const Plan p = make_plan(d, R);
  if ((st = check_pool(d, pool, p)) != MOE_OK) return st;
  if ((st = check_params(d, params)) != MOE_OK) return st;
  if (!aligned16(grad_out) || !aligned16(grad_x) || !aligned16(saved) || !aligned16(scratch) ||
      topk_w == nullptr || grad_topk_w == nullptr || grads == nullptr)
    return MOE_ERR_INVALID;
  const void* gs[] = {grads->dA1, grads->dA3, grads->dB1, grads->dB3, grads->dA2, grads->dB2};
  for (const void* g : gs)
    if (!aligned16(g)) return MOE_ERR_INVALID;
  // the frozen-weight gradients are optional (NULL: not computed)
  if ((grads->dW13 != nullptr && !aligned16(grads->dW13)) || (grads->dW2 != nullptr && !aligned16(grads->dW2)))
    return MOE_ERR_INVALID;
  // frozen-weight gradients sum an expert's rows of every adapter: one adapter only
  if (R.na > 1 && (grads->dW13 != nullptr || grads->dW2 != nullptr)) return MOE_ERR_UNSUPPORTED;
  if (saved_bytes < p.saved || scratch_bytes < p.scratch) return MOE_ERR_WORKSPACE;
  const size_t act = (size_t)d->T * d->H * 2;
  const Range rgo = rng(grad_out, act), rgx = rng(grad_x, act), rs = rng(saved, p.saved),
              rsc = rng(scratch, p.scratch);
  if (overlap(rgo, rgx) || overlap(rgx, rs) || overlap(rgx, rsc) || overlap(rs, rsc) ||
      overlap(rgo, rsc))
    return MOE_ERR_INVALID;
  LayerArgs a;
  fill_common(a, d, pool, p, params, R);
  fill_saved(a, p, const_cast<void*>(saved));
  fill_scratch(a, p, scratch);
  a.go = (const uint16_t*)grad_out;
  a.w = topk_w;
  a.gx = (uint16_t*)grad_x;
  a.gw = grad_topk_w;
  a.dA1 = (uint16_t*)grads->dA1;
  a.dA3 = (uint16_t*)grads->dA3;
  a.dB1 = (uint16_t*)grads->dB1;
  a.dB3 = (uint16_t*)grads->dB3;
  a.dA2 = (uint16_t*)grads->dA2;
  a.dB2 = (uint16_t*)grads->dB2;
  a.dW13 = (uint16_t*)grads->dW13;
  a.dW2 = (uint16_t*)grads->dW2;
  uint16_t* user[6];
  pad_grads(a, d, p, R.na, scratch, user);
  hipError_t e = pad_factors(a, d, p, R.na, scratch, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_backward(a, (hipStream_t)stream);
  if (e == hipSuccess) e = crop_grads(a, d, R.na, user, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" {

const char* moe_lora_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int32_t moe_lora_version(void) { return kVersion; }

moe_status moe_lora_block_m(const moe_lora_desc* d, int32_t* block_m) {
  const moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (block_m == nullptr) return MOE_ERR_INVALID;
  *block_m = resolve_bm(d);
  return MOE_OK;
}

moe_status moe_lora_multi_pool_capacity(const moe_lora_desc* d, const moe_adapters* ad, int64_t* rows) {
  Roots R;
  const moe_status st = check_call(d, ad, R);
  if (st != MOE_OK) return st;
  if (rows == nullptr) return MOE_ERR_INVALID;
  *rows = capacity_of(d, resolve_bm(d), R.na);
  return MOE_OK;
}

moe_status moe_lora_pool_capacity(const moe_lora_desc* d, int64_t* rows) {
  return moe_lora_multi_pool_capacity(d, nullptr, rows);
}

moe_status moe_lora_multi_workspace_size(const moe_lora_desc* d, const moe_adapters* ad, size_t* saved_bytes,
                                         size_t* scratch_bytes) {
  Roots R;
  const moe_status st = check_call(d, ad, R);
  if (st != MOE_OK) return st;
  if (saved_bytes == nullptr || scratch_bytes == nullptr) return MOE_ERR_INVALID;
  const Plan p = make_plan(d, R);
  *saved_bytes = p.saved;
  *scratch_bytes = p.scratch;
  return MOE_OK;
}

moe_status moe_lora_workspace_size(const moe_lora_desc* d, size_t* saved_bytes, size_t* scratch_bytes) {
  return moe_lora_multi_workspace_size(d, nullptr, saved_bytes, scratch_bytes);
}

moe_status build_pool_multi(const moe_lora_desc* d, const moe_adapters* ad, const int32_t* topk_idx,
                            int32_t* counts, int32_t* offsets, int32_t* route_to_row, int32_t* row_to_route,
                            int64_t capacity, int32_t* device_error, void* stream) {
  Roots R;
  const moe_status st = check_call(d, ad, R);
  if (st != MOE_OK) return st;
  if (topk_idx == nullptr || counts == nullptr || offsets == nullptr || route_to_row == nullptr ||
      row_to_route == nullptr)
    return MOE_ERR_INVALID;
  const int bm = resolve_bm(d);
  if (capacity != capacity_of(d, bm, R.na)) return MOE_ERR_INVALID;
  PoolRoots pr;
  pr.na = R.na;
  pr.k = d->topk;
  for (int q = 0; q <= MAX_ADAPTERS; ++q) pr.roots[q] = q <= R.na ? R.r[q] : d->T;
  const hipError_t e = launch_build_pool(topk_idx, d->T * d->topk, d->E, bm, capacity, counts, offsets,
                                         route_to_row, row_to_route, device_error, pr, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status build_pool(const moe_lora_desc* d, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                      int32_t* route_to_row, int32_t* row_to_route, int64_t capacity, int32_t* device_error,
                      void* stream) {
  return build_pool_multi(d, nullptr, topk_idx, counts, offsets, route_to_row, row_to_route, capacity,
                          device_error, stream);
}

moe_status moe_lora_forward(const moe_lora_desc* d, const moe_pool* pool, const void* x,
                            const float* topk_w, const moe_lora_params* params, void* out,
                            void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                            void* stream) {
  return forward_checked(d, nullptr, pool, x, topk_w, params, out, saved, saved_bytes, scratch, scratch_bytes,
                         false, stream);
}

moe_status moe_lora_forward_multi(const moe_lora_desc* d, const moe_adapters* ad, const moe_pool* pool,
                                  const void* x, const float* topk_w, const moe_lora_params* params, void* out,
                                  void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                                  void* stream) {
  if (ad == nullptr) return MOE_ERR_INVALID;
  return forward_checked(d, ad, pool, x, topk_w, params, out, saved, saved_bytes, scratch, scratch_bytes, false,
                         stream);
}

moe_status moe_lora_forward_noalloc(const moe_lora_desc* d, const moe_pool* pool, const void* x,
                                    const float* topk_w, const moe_lora_params* params, void* out,
                                    void* saved, size_t saved_bytes, void* stream) {
  return forward_checked(d, nullptr, pool, x, topk_w, params, out, saved, saved_bytes, nullptr, 0, true, stream);
}

moe_status moe_lora_backward(const moe_lora_desc* d, const moe_pool* pool, const void* grad_out,
                             const float* topk_w, const moe_lora_params* params, const void* saved,
                             size_t saved_bytes, void* grad_x, float* grad_topk_w, const moe_lora_grads* grads,
                             void* scratch, size_t scratch_bytes, void* stream) {
  return backward_checked(d, nullptr, pool, grad_out, topk_w, params, saved, saved_bytes, grad_x, grad_topk_w,
                          grads, scratch, scratch_bytes, stream);
}

moe_status moe_lora_backward_multi(const moe_lora_desc* d, const moe_adapters* ad, const moe_pool* pool,
                                   const void* grad_out, const float* topk_w, const moe_lora_params* params,
                                   const void* saved, size_t saved_bytes, void* grad_x, float* grad_topk_w,
                                   const moe_lora_grads* grads, void* scratch, size_t scratch_bytes,
                                   void* stream) {
  if (ad == nullptr) return MOE_ERR_INVALID;
  return backward_checked(d, ad, pool, grad_out, topk_w, params, saved, saved_bytes, grad_x, grad_topk_w, grads,
                          scratch, scratch_bytes, stream);
}

moe_status moe_lora_split_e2m3x2(const void* src, int64_t rows, int32_t K, void* codes, void* scale_words,
                                 void* stream) {
  if (rows < 1 || K < 1) return MOE_ERR_INVALID;
  if (K % 64 != 0 || rows * (int64_t)(K / 32) >= ((int64_t)1 << 31) * 256) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(codes) || scale_words == nullptr || ((uintptr_t)scale_words & 3u) != 0)
    return MOE_ERR_INVALID;
  const size_t nsrc = (size_t)rows * K * 2, nscale = (size_t)rows * (K / 64) * 4;
  const Range rs = rng(src, nsrc), rc = rng(codes, nsrc), rw = rng(scale_words, nscale);
  if (overlap(rs, rc) || overlap(rs, rw) || overlap(rc, rw)) return MOE_ERR_INVALID;
  const hipError_t e = launch_split_rows((const uint16_t*)src, (long)rows, K, (uint8_t*)codes,
                                         (uint32_t*)scale_words, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_lora_transform_base(const moe_lora_desc* d, const moe_lora_params* params, void* W13T,
                                   void* W2T, void* W13P, void* W2P, void* stream) {
  const moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (params == nullptr) return MOE_ERR_INVALID;
  const bool mx = d->base_format == MOE_BASE_MXFP4;
  const size_t n13 = (size_t)d->E * 2 * d->I * d->H, n2 = (size_t)d->E * d->H * d->I;  // elements
  const size_t b13 = n13 * 2, b2 = n2 * 2;                                              // bf16 outputs
  const size_t in13 = mx ? n13 / 2 : b13, in2 = mx ? n2 / 2 : b2;                      // inputs
  if (mx && (params->W13_scale == nullptr || params->W2_scale == nullptr)) return MOE_ERR_INVALID;
  if (!aligned16(params->W13) || !aligned16(params->W2)) return MOE_ERR_INVALID;
  // every output: aligned, and disjoint from the inputs and the other outputs
  const Range ins[] = {rng(params->W13, in13), rng(params->W2, in2),
                       rng(mx ? params->W13_scale : nullptr, mx ? n13 / 32 : 0),
                       rng(mx ? params->W2_scale : nullptr, mx ? n2 / 32 : 0)};
  void* outs[] = {W13T, W2T, W13P, W2P};
  // the forward's copies of an MXFP4 base: 9 bytes per 16 weights (codes and scale words)
  const size_t sizes[] = {b13, b2, mx ? n13 / 16 * 9 : b13, mx ? n2 / 16 * 9 : b2};
  for (int i = 0; i < 4; ++i) {
    if (outs[i] == nullptr) continue;
    if (!aligned16(outs[i])) return MOE_ERR_INVALID;
    for (const Range& r : ins)
      if (overlap(rng(outs[i], sizes[i]), r)) return MOE_ERR_INVALID;
    for (int j = 0; j < i; ++j)
      if (outs[j] != nullptr && overlap(rng(outs[i], sizes[i]), rng(outs[j], sizes[j]))) return MOE_ERR_INVALID;
  }
  const hipStream_t s = (hipStream_t)stream;
  const uint16_t* w13 = mx ? nullptr : (const uint16_t*)params->W13;
  const uint16_t* w2 = mx ? nullptr : (const uint16_t*)params->W2;
  const uint8_t* q13 = mx ? (const uint8_t*)params->W13 : nullptr;
  const uint8_t* q2 = mx ? (const uint8_t*)params->W2 : nullptr;
  hipError_t e = hipSuccess;
  if (W13T != nullptr)
    e = launch_pack(2, w13, q13, params->W13_scale, (uint16_t*)W13T, d->E, d->H, d->I, s);
  if (e == hipSuccess && W2T != nullptr)
    e = launch_pack(3, w2, q2, params->W2_scale, (uint16_t*)W2T, d->E, d->H, d->I, s);
  if (e == hipSuccess && W13P != nullptr)
    e = launch_pack(mx ? 4 : 0, w13, q13, mx ? params->W13_scale : nullptr, (uint16_t*)W13P, d->E, d->H, d->I, s);
  if (e == hipSuccess && W2P != nullptr)
    e = launch_pack(mx ? 5 : 1, w2, q2, mx ? params->W2_scale : nullptr, (uint16_t*)W2P, d->E, d->H, d->I, s);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
