// api.cpp -- the C ABI: description checks (the pages' can_implement), plan
// creation (device query, tile configuration, persistent grid size) and the
// run entry points.  See include/migemm.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "../../include/migemm.h"
#include "kernel/params.hpp"
#include "launch.h"

using migemm::KernelArgs;
using migemm::KernelSelect;

struct migemm_plan {
  migemm_desc desc;
  KernelSelect sel;
  KernelArgs base;   // shape/stride part of the kernel arguments
  int64_t M, N, K;   // problem after any swap (D row-major)
  bool swapped;
  int grid;
  int cu_count;
  int device;
  // Stream-K workspace: arrival counters, then the partial tiles.
  int64_t sk_counters;        // 32-bit counters
  size_t sk_counter_bytes;    // rounded up to 256 bytes
  size_t workspace_bytes;
  // Hand-off debug area (MIGEMM_F_HANDOFF_DEBUG): header, then trace records.
  bool debug;
  int trace_tiles;
};

namespace {

// Orientation of one operand: K-contiguous ("row" for A, "col" for B) or not,
// and its leading (non-unit) stride.
struct Orient {
  bool row_major;  // column stride is 1
  int64_t ld;      // the non-unit stride
};

// rows x cols matrix with strides (rs, cs): exactly one unit stride, and the
// other at least the contiguous extent.  Row-major wins when both are 1.
bool orient(int64_t rows, int64_t cols, int64_t rs, int64_t cs, Orient* o) {
  if (cs == 1 && rs >= (cols > 1 ? cols : 1)) {
    *o = {true, rs};
    return true;
  }
  if (rs == 1 && cs >= (rows > 1 ? rows : 1)) {
    *o = {false, cs};
    return true;
  }
  return false;
}

int64_t extent_bytes(int64_t rows, int64_t cols, int64_t rs, int64_t cs, int es) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * rs + (cols - 1) * cs + 1) * es;
}

int elem_size(int32_t t) { return t == MIGEMM_BF16 ? 2 : (t == MIGEMM_FP8_E4M3 ? 1 : 0); }

// The bytes one operand may span -- its first batch matrix, and its last
// batch matrix from the first -- computed exactly (128-bit), must stay
// within 2^47 (128 TiB, beyond any device's memory).  Every later product of
// sizes and strides, here and in the kernels' 64-bit address arithmetic,
// then stays far from overflow; without this bound a huge stride could wrap
// a product past the other checks and put a buffer base outside any
// allocation.
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 47;
bool span_in_range(int64_t rows, int64_t cols, int64_t rs, int64_t cs, int es, int64_t L,
                   int64_t bs) {
  if (rows <= 0 || cols <= 0) return true;
  // (Called after the orientation check: the strides of a dimension longer
  // than 1 are at least 1.)  A factor beyond 2^47 alone puts the span past
  // the bound, so the products below only ever see factors up to 2^47.
  constexpr int64_t lim = kMaxOperandBytes;
  if ((rows > 1 && (rows - 1 > lim || rs > lim)) || (cols > 1 && (cols - 1 > lim || cs > lim)))
    return false;
  __int128 bytes = ((__int128)(rows - 1) * (rows > 1 ? rs : 0) +
                    (__int128)(cols - 1) * (cols > 1 ? cs : 0) + 1) * es;
  if (L > 1 && bs > 0) {  // (a negative batch stride is refused later)
    if (L - 1 > lim || bs > lim) return false;
    bytes += (__int128)(L - 1) * bs * es;
  }
  return bytes <= kMaxOperandBytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxRsrcSpan = 0x7FFFFFF0 - 1024;

// Everything after any swap: the canonical problem the kernel sees.
struct Canon {
  int64_t M, N, K;
  int64_t a_rs, a_cs, b_rs, b_cs, c_rs, c_cs, d_rs, d_cs;
  bool swapped;
  int64_t L;                       // batches (>= 1)
  int64_t a_bs, b_bs, c_bs, d_bs;  // batch strides in elements (0 when L == 1)
};

int validate(const migemm_desc* d, Canon* out) {
  if (!d) return MIGEMM_ERR_INVALID_ARG;
  if (d->M < 0 || d->N < 0 || d->K < 0 || d->reserved != 0 || d->max_workgroups < 0 ||
      d->reserved2 != 0 || d->debug_wait_ticks < 0 || d->debug_force_wait < 0)
    return MIGEMM_ERR_INVALID_ARG;
  // No dimension beyond 2^47 (even of an empty product): keeps tile counts
  // and every size product below from overflowing.
  if (d->M > kMaxOperandBytes || d->N > kMaxOperandBytes || d->K > kMaxOperandBytes)
    return MIGEMM_ERR_UNSUPPORTED;
  constexpr uint32_t kStreamK = MIGEMM_F_STREAM_K | MIGEMM_F_STREAM_K_FORCE;
  if ((d->flags & ~(MIGEMM_F_TILE_CONSUMER | MIGEMM_F_CONSUMER_OVERLAP | MIGEMM_F_HANDOFF_DEBUG |
                    MIGEMM_F_C_IN_EPILOGUE | kStreamK | MIGEMM_F_TILE_M256 |
                    MIGEMM_F_TILE_M192)) != 0)
    return MIGEMM_ERR_INVALID_ARG;
  if ((d->flags & MIGEMM_F_TILE_M192) &&
      (d->flags & (MIGEMM_F_TILE_M256 | MIGEMM_F_TILE_CONSUMER | kStreamK)))
    return MIGEMM_ERR_INVALID_ARG;  // 192-row tiles: whole tiles, no consumer
  if ((d->flags & MIGEMM_F_HANDOFF_DEBUG) && !(d->flags & MIGEMM_F_TILE_CONSUMER))
    return MIGEMM_ERR_INVALID_ARG;
  if (!(d->flags & MIGEMM_F_HANDOFF_DEBUG) && (d->debug_wait_ticks != 0 || d->debug_force_wait != 0))
    return MIGEMM_ERR_INVALID_ARG;
  if ((d->flags & MIGEMM_F_CONSUMER_OVERLAP) && !(d->flags & MIGEMM_F_TILE_CONSUMER))
    return MIGEMM_ERR_INVALID_ARG;
  if ((d->flags & MIGEMM_F_TILE_CONSUMER) && (d->flags & kStreamK))
    return MIGEMM_ERR_UNSUPPORTED;  // the consumer works on whole tiles
  const int es = elem_size(d->a_type);
  if (es == 0 || elem_size(d->b_type) == 0 || elem_size(d->c_type) == 0 ||
      elem_size(d->d_type) == 0)
    return MIGEMM_ERR_INVALID_ARG;
  if (d->a_type != d->b_type || d->c_type != MIGEMM_BF16 || d->d_type != MIGEMM_BF16)
    return MIGEMM_ERR_UNSUPPORTED;
  if ((d->flags & MIGEMM_F_TILE_M192) && es != 2) return MIGEMM_ERR_UNSUPPORTED;
  Orient oa, ob, oc, od;
  if (!orient(d->M, d->K, d->a_rs, d->a_cs, &oa) || !orient(d->K, d->N, d->b_rs, d->b_cs, &ob) ||
      !orient(d->M, d->N, d->c_rs, d->c_cs, &oc) || !orient(d->M, d->N, d->d_rs, d->d_cs, &od))
    return MIGEMM_ERR_INVALID_ARG;
  {
    const int64_t Lc = d->L > 1 ? d->L : 1;
    const bool b = Lc > 1;
    if (!span_in_range(d->M, d->K, d->a_rs, d->a_cs, es, Lc, b ? d->a_bs : 0) ||
        !span_in_range(d->K, d->N, d->b_rs, d->b_cs, es, Lc, b ? d->b_bs : 0) ||
        !span_in_range(d->M, d->N, d->c_rs, d->c_cs, 2, Lc, b ? d->c_bs : 0) ||
        !span_in_range(d->M, d->N, d->d_rs, d->d_cs, 2, Lc, b ? d->d_bs : 0))
      return MIGEMM_ERR_UNSUPPORTED;
  }
  if (oc.row_major != od.row_major) return MIGEMM_ERR_UNSUPPORTED;
  if ((d->flags & MIGEMM_F_TILE_CONSUMER) && !od.row_major) return MIGEMM_ERR_UNSUPPORTED;
  // 16-byte rows for every operand.
  // (Written without products: a leading stride may be huge where the other
  // dimension is 1.)
  const int64_t per16 = 16 / es;  // elements per 16 bytes
  if (oa.ld % per16 || ob.ld % per16 || oc.ld % 8 || od.ld % 8) return MIGEMM_ERR_MISALIGNED;
  // Batches: non-negative strides keeping every matrix 16-byte aligned; the
  // batches of D must not overlap (A, B and C may be shared).
  if (d->L < 0) return MIGEMM_ERR_INVALID_ARG;
  const int64_t L = d->L > 1 ? d->L : 1;
  int64_t a_bs = 0, b_bs = 0, c_bs = 0, d_bs = 0;
  if (L > 1) {
    a_bs = d->a_bs, b_bs = d->b_bs, c_bs = d->c_bs, d_bs = d->d_bs;
    if (a_bs < 0 || b_bs < 0 || c_bs < 0 || d_bs < 0) return MIGEMM_ERR_INVALID_ARG;
    if (d->M > 0 && d->N > 0 && d_bs * 2 < extent_bytes(d->M, d->N, d->d_rs, d->d_cs, 2))
      return MIGEMM_ERR_INVALID_ARG;
    if (a_bs % per16 || b_bs % per16 || c_bs % 8 || d_bs % 8) return MIGEMM_ERR_MISALIGNED;
  }

  Canon c;
  if (od.row_major) {
    c = {d->M, d->N, d->K, d->a_rs, d->a_cs, d->b_rs, d->b_cs,
         d->c_rs, d->c_cs, d->d_rs, d->d_cs, false, L, a_bs, b_bs, c_bs, d_bs};
  } else {
    // D^T = B^T A^T: swap the roles of A and B and transpose every operand.
    c = {d->N, d->M, d->K, d->b_cs, d->b_rs, d->a_cs, d->a_rs,
         d->c_cs, d->c_rs, d->d_cs, d->d_rs, true, L, b_bs, a_bs, c_bs, d_bs};
  }
  // 32-bit buffer offsets: 256 rows of a K-contiguous operand, or one stage
  // of K rows of an MN-contiguous one (128 bytes of K: 64 bf16 or 128 e4m3
  // rows), must span less than 2^31 bytes.
  const int64_t bk = migemm::kStageKBytes / es;
  Orient ca, cb;
  orient(c.M, c.K, c.a_rs, c.a_cs, &ca);
  orient(c.K, c.N, c.b_rs, c.b_cs, &cb);
  const bool ca_k = ca.row_major, cb_k = !cb.row_major;
  // (128-bit products: a leading stride may be anything where the other
  // dimension is 1, and must not wrap past the bound.)
  const __int128 span_a = (__int128)(ca_k ? migemm::kTileM : bk) * ca.ld * es;
  const __int128 span_b = (__int128)(cb_k ? migemm::kTileN : bk) * cb.ld * es;
  if (span_a > kMaxRsrcSpan || span_b > kMaxRsrcSpan) return MIGEMM_ERR_UNSUPPORTED;
  // The epilogue addresses a 256-row band of C and D with 32-bit offsets too.
  if ((__int128)migemm::kTileM * c.c_rs * 2 > kMaxRsrcSpan ||
      (__int128)migemm::kTileM * c.d_rs * 2 > kMaxRsrcSpan)
    return MIGEMM_ERR_UNSUPPORTED;
  if (c.M / migemm::kTileM >= (1 << 20) || c.N / migemm::kTileN >= (1 << 20))
    return MIGEMM_ERR_UNSUPPORTED;
  // Tile indices are 32-bit.
  const int64_t tiles = ((c.M + migemm::kTileM - 1) / migemm::kTileM) *
                        ((c.N + migemm::kTileN - 1) / migemm::kTileN);
  if (tiles > 0 && L > (int64_t)0x7FFFFFFF / tiles) return MIGEMM_ERR_UNSUPPORTED;
  if (out) *out = c;
  return MIGEMM_OK;
}

// Stream-K pays when the stages one workgroup runs, plus the fixup, come
// below those of whole tiles.  Whole tiles take ceil(T / G) rounds of KT
// stages; stream-K takes sk_first / G whole rounds, then ceil(units / G)
// stages, plus the fixup: two 256 KiB fp32 partials written and one read per
// split tile, which costs about as much as 24 stages on MI355X (fitted to
// 4000x3000x5000, 8192x1024x8192 and 2048x2048x8192 bf16).  When the units
// fall on tile boundaries nothing is split and whole tiles are the same.
constexpr int64_t kSkFixupStages = 24;

// Default budget of a bounded hand-off wait: 10^8 ticks of the 100 MHz
// real-time clock, one second.
constexpr int64_t kDefaultWaitTicks = 100000000;

bool stream_k_pays(int64_t T, int64_t G, int64_t kt, int64_t sk_first) {
  const int64_t units = (T - sk_first) * kt;
  if (units % G == 0 && (units / G) % kt == 0) return false;
  const int64_t whole = (T + G - 1) / G * kt;
  const int64_t split = sk_first / G * kt + (units + G - 1) / G + kSkFixupStages;
  return split < whole;
}

// The stages one workgroup runs under stream-K (see stream_k_pays).
int64_t stream_k_stages(int64_t T, int64_t G, int64_t kt, int64_t sk_first) {
  const int64_t units = (T - sk_first) * kt;
  return sk_first / G * kt + (units + G - 1) / G + kSkFixupStages;
}

// Tile height (bf16 whole tiles without the consumer).  A 192-row tile is
// 3/4 of a 256-row one, so where ceil(T192 / G) * 3/4 < ceil(T256 / G)
// rounds -- the 256-row tiles fill the last round poorly -- each workgroup
// has less work with 192.  kShortTileWork is a 192-row tile's time in
// thousandths of a 256-row one's: 3/4 of the flops at a 6% lower rate per
// flop (its K loop reads 7 operand fragments from LDS per 12 MFMAs against 8
// per 16; on MI355X 6144 x 8192 x 8192 in 192-row tiles ran at 1303 TFLOP/s,
// 8192^3 in 256-row ones at 1384, both four full rounds).
constexpr int64_t kShortTileWork = 800;

// The plans alive in this process.  Every entry point that takes a plan
// looks it up here first, so a destroyed plan (or any other pointer that is
// not a live plan) gives MIGEMM_ERR_INVALID_ARG instead of kernel arguments
// read from freed memory.  (A new plan created at the address of a destroyed
// one is that new plan: the check is exact for pointers that were never
// plans and for destroyed plans whose address has not been reused.)
// (The set is never freed, so a plan destroyed while the process exits --
// after static destructors have run -- still finds it.)
std::mutex g_plans_mu;
std::unordered_set<const migemm_plan*>& live_plans() {
  static std::unordered_set<const migemm_plan*>* s = new std::unordered_set<const migemm_plan*>();
  return *s;
}
bool plan_is_live(const migemm_plan* p) {
  if (!p) return false;
  std::lock_guard<std::mutex> lock(g_plans_mu);
  return live_plans().count(p) != 0;
}

bool trace_enabled() {
  const char* e = std::getenv("MIGEMM_TRACE");
  return e && e[0] && e[0] != '0';
}

}  // namespace

extern "C" {

int gemm_desc_validate(const migemm_desc* desc) { return validate(desc, nullptr); }

int gemm_plan_create(const migemm_desc* desc, migemm_plan** out) {
  if (!out) return MIGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  Canon c;
  int st = validate(desc, &c);
  if (st != MIGEMM_OK) return st;

  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return MIGEMM_ERR_DEVICE;
  if (desc->device < 0 || desc->device >= count) return MIGEMM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, desc->device) != hipSuccess) return MIGEMM_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MIGEMM_ERR_DEVICE;
  if (prop.sharedMemPerBlock < (size_t)migemm::kLdsLimit) return MIGEMM_ERR_DEVICE;

  migemm_plan* p = new (std::nothrow) migemm_plan;
  if (!p) return MIGEMM_ERR_INVALID_ARG;
  std::memset(p, 0, sizeof(*p));
  p->desc = *desc;
  p->device = desc->device;
  p->cu_count = prop.multiProcessorCount;
  p->M = c.M;
  p->N = c.N;
  p->K = c.K;
  p->swapped = c.swapped;

  const int es = elem_size(desc->a_type);
  Orient oa, ob;
  orient(c.M, c.K, c.a_rs, c.a_cs, &oa);
  orient(c.K, c.N, c.b_rs, c.b_cs, &ob);
  p->sel.elem_bytes = es;
  p->sel.a_kmajor = oa.row_major;   // A row-major = K-contiguous
  p->sel.b_kmajor = !ob.row_major;  // B column-major = K-contiguous
  p->sel.consumer = false;
  p->sel.consumer_overlap = (desc->flags & MIGEMM_F_CONSUMER_OVERLAP) != 0;
  p->sel.tile_m = migemm::kTileM;

  int grid = p->cu_count;
  if (desc->max_workgroups > 0 && desc->max_workgroups < grid) grid = desc->max_workgroups;
  const int64_t kt = (c.K + migemm::kStageKBytes / es - 1) / (migemm::kStageKBytes / es);
  {
    // 192-row tiles: forced, or chosen where they leave each workgroup less
    // work than 256-row tiles (whole, or stream-K where the plan may split).
    const int64_t tn = (c.N + migemm::kTileN - 1) / migemm::kTileN;
    const int64_t tm_short = (c.M + migemm::kTileMShort - 1) / migemm::kTileMShort;
    const bool fits = tm_short < (1 << 20) && (tm_short * tn == 0 ||
                                               c.L <= (int64_t)0x7FFFFFFF / (tm_short * tn));
    const uint32_t no_short = MIGEMM_F_TILE_CONSUMER | MIGEMM_F_STREAM_K_FORCE | MIGEMM_F_TILE_M256;
    if (desc->flags & MIGEMM_F_TILE_M192) {
      if (!fits) {
        delete p;
        return MIGEMM_ERR_UNSUPPORTED;
      }
      p->sel.tile_m = migemm::kTileMShort;
    } else if (es == 2 && !(desc->flags & no_short) && fits && kt > 0 && tm_short * tn > 0) {
      const int64_t G = grid;
      const int64_t T = c.L * ((c.M + migemm::kTileM - 1) / migemm::kTileM) * tn;
      const int64_t T_short = c.L * tm_short * tn;
      int64_t cost = (T + G - 1) / G * kt * 1000;
      if (desc->flags & MIGEMM_F_STREAM_K) {
        const int64_t sk_first = T >= 2 * G ? (T / G - 1) * G : 0;
        if (stream_k_pays(T, G, kt, sk_first)) cost = stream_k_stages(T, G, kt, sk_first) * 1000;
      }
      if ((T_short + G - 1) / G * kt * kShortTileWork < cost) p->sel.tile_m = migemm::kTileMShort;
    }
  }
  const int tile_m = p->sel.tile_m;

  KernelArgs& a = p->base;
  a.M = c.M;
  a.N = c.N;
  a.K = c.K;
  a.lda = oa.ld;
  a.ldb = ob.ld;
  a.ldc = c.c_rs;
  a.ldd = c.d_rs;
  a.a_bytes = extent_bytes(c.M, c.K, c.a_rs, c.a_cs, es);
  a.b_bytes = extent_bytes(c.K, c.N, c.b_rs, c.b_cs, es);
  a.tiles_m = (int32_t)((c.M + tile_m - 1) / tile_m);
  a.tiles_n = (int32_t)((c.N + migemm::kTileN - 1) / migemm::kTileN);
  a.tiles_per_batch = a.tiles_m * a.tiles_n;
  a.num_tiles = (int32_t)(c.L * a.tiles_per_batch);
  a.a_bs_bytes = c.a_bs * es;
  a.b_bs_bytes = c.b_bs * es;
  a.c_bs_bytes = c.c_bs * 2;
  a.d_bs_bytes = c.d_bs * 2;
  a.group_m = a.tiles_m < 8 ? (a.tiles_m > 0 ? a.tiles_m : 1) : 8;
  a.c_preload = 0;
  a.stat_ld = a.tiles_n;

  a.sk_kt = (int32_t)kt;
  a.sk_first = a.num_tiles;
  // Whole tiles for all but the last round (when there are at least two),
  // then the remaining tiles as K-stage units over the whole grid.
  const int T = a.num_tiles;
  const int sk_first = T >= 2 * grid ? (T / grid - 1) * grid : 0;
  const bool sk = kt > 0 && T > 0 && tile_m == migemm::kTileM &&
                  ((desc->flags & MIGEMM_F_STREAM_K_FORCE) ||
                   ((desc->flags & MIGEMM_F_STREAM_K) && stream_k_pays(T, grid, kt, sk_first)));
  if (sk) {
    a.sk_first = sk_first;
    const int64_t units = (int64_t)(T - a.sk_first) * kt;
    if (units < grid) grid = (int)units;  // every workgroup gets a unit
    p->sel.stream_k = true;
    p->sk_counters = (int64_t)(T - a.sk_first) * migemm::kWaves;
    p->sk_counter_bytes = (size_t)((p->sk_counters * 4 + 255) / 256 * 256);
    p->workspace_bytes = p->sk_counter_bytes + (size_t)grid * migemm::kSkPartialSlots *
                                                   (size_t)migemm::kSkPartialBytes;
  } else if (a.num_tiles < grid) {
    grid = a.num_tiles;
  }
  p->grid = grid;
  // The source C in the K loop's last two iterations pays where every
  // workgroup takes one round of whole tiles: C's read is then the kernel's
  // tail on every compute unit at once, and half of it moves under the last
  // stages' MFMAs (4096^3 with beta != 0: 6.2% over beta = 0 instead of
  // 7.9%).  With more rounds the extra loads in iteration KT-2 cost more than
  // they hide (8192^3: 4.8% instead of 2.8%).
  a.c_preload = !(desc->flags & MIGEMM_F_C_IN_EPILOGUE) && !p->sel.stream_k &&
                tile_m == migemm::kTileM && a.num_tiles <= grid && kt >= 2;
  if (desc->flags & MIGEMM_F_HANDOFF_DEBUG) {
    p->debug = true;
    p->trace_tiles = grid > 0 ? (a.num_tiles + grid - 1) / grid : 0;
    p->workspace_bytes = (size_t)migemm::kDebugHeaderBytes +
                         (size_t)grid * migemm::kWaves * (size_t)p->trace_tiles *
                             migemm::kTraceWords * sizeof(uint64_t);
  }

  hipError_t e = migemm::prepare_kernel(p->sel);
  if (e == hipSuccess && (desc->flags & MIGEMM_F_TILE_CONSUMER)) {
    KernelSelect s = p->sel;
    s.consumer = true;
    e = migemm::prepare_kernel(s);
  }
  if (e != hipSuccess) {
    delete p;
    return MIGEMM_ERR_DEVICE;
  }
  if (trace_enabled()) {
    std::fprintf(stderr,
                 "[migemm] plan M=%lld N=%lld K=%lld es=%d A:%s B:%s swapped=%d tile=%dx%d "
                 "tiles=%dx%d grid=%d group_m=%d lds=%d stages=%d cus=%d stream_k_tiles=%d "
                 "workspace=%zu\n",
                 (long long)c.M, (long long)c.N, (long long)c.K, es,
                 p->sel.a_kmajor ? "K-contig" : "M-contig", p->sel.b_kmajor ? "K-contig" : "N-contig",
                 (int)c.swapped, tile_m, migemm::kTileN, a.tiles_m, a.tiles_n, grid, a.group_m,
                 migemm::kernel_lds_bytes(p->sel), migemm::kStages, p->cu_count,
                 p->sel.stream_k ? a.num_tiles - a.sk_first : 0, p->workspace_bytes);
  }
  {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    live_plans().insert(p);
  }
  *out = p;
  return MIGEMM_OK;
}

int gemm_plan_destroy(migemm_plan* plan) {
  if (!plan) return MIGEMM_OK;
  {
    std::lock_guard<std::mutex> lock(g_plans_mu);
    if (live_plans().erase(plan) == 0) return MIGEMM_ERR_INVALID_ARG;  // not a live plan
  }
  delete plan;
  return MIGEMM_OK;
}

int gemm_plan_get_info(const migemm_plan* p, migemm_plan_info* out) {
  if (!plan_is_live(p) || !out) return MIGEMM_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  out->tiles_m = p->base.tiles_m;
  out->tiles_n = p->base.tiles_n;
  out->num_tiles = p->base.num_tiles;
  out->grid = p->grid;
  out->block_threads = migemm::kThreads;
  out->lds_bytes = migemm::kernel_lds_bytes(p->sel);
  out->stages = migemm::kStages;
  out->tile_m = p->sel.tile_m;
  out->tile_n = migemm::kTileN;
  out->tile_k = migemm::kStageKBytes / p->sel.elem_bytes;
  out->swapped = p->swapped ? 1 : 0;
  out->a_kmajor = p->sel.a_kmajor ? 1 : 0;
  out->b_kmajor = p->sel.b_kmajor ? 1 : 0;
  out->cu_count = p->cu_count;
  out->handoff_slots = migemm::kHandoffSlots;
  out->stream_k_tiles = p->sel.stream_k ? p->base.num_tiles - p->base.sk_first : 0;
  out->stream_k_units_per_tile = p->sel.stream_k ? p->base.sk_kt : 0;
  out->c_in_k_loop = p->base.c_preload;
  out->batches = p->base.tiles_per_batch > 0 ? p->base.num_tiles / p->base.tiles_per_batch
                                             : (p->desc.L > 1 ? p->desc.L : 1);
  return MIGEMM_OK;
}

size_t gemm_plan_workspace_size(const migemm_plan* plan) {
  return plan_is_live(plan) ? plan->workspace_bytes : 0;
}

int gemm_workspace_init(const migemm_plan* p, void* workspace, void* stream) {
  if (!plan_is_live(p)) return MIGEMM_ERR_INVALID_ARG;
  if (p->workspace_bytes == 0) return MIGEMM_OK;
  if (!workspace) return MIGEMM_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MIGEMM_ERR_MISALIGNED;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != p->device) return MIGEMM_ERR_DEVICE;
  // Stream-K: the arrival counters; debug: the header and every record.
  const int64_t words = p->debug ? (int64_t)(p->workspace_bytes / 4) : p->sk_counters;
  hipError_t e = migemm::launch_zero_words(static_cast<uint32_t*>(workspace), words,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIGEMM_OK : MIGEMM_ERR_LAUNCH;
}

// Argument checks of a run, before anything is launched (the workspace is
// checked by the caller: it is the caller's or the fixed scratch).
static int check_run(const migemm_plan* p, const void* A, const void* B, const void* C,
                     const void* D, float beta, bool consumer, const float* row_sum,
                     const float* row_max, const void* D_copy) {
  if (!plan_is_live(p)) return MIGEMM_ERR_INVALID_ARG;
  if (consumer && !(p->desc.flags & MIGEMM_F_TILE_CONSUMER)) return MIGEMM_ERR_INVALID_ARG;
  if (p->M == 0 || p->N == 0) return MIGEMM_OK;
  if (!D || (p->K > 0 && (!A || !B))) return MIGEMM_ERR_INVALID_ARG;
  if (beta != 0.0f && !C) return MIGEMM_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(D) || (beta != 0.0f && !aligned16(C)))
    return MIGEMM_ERR_MISALIGNED;
  if (consumer) {
    if (!row_sum || !row_max || !D_copy) return MIGEMM_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(row_sum) & 3u) || (reinterpret_cast<uintptr_t>(row_max) & 3u) ||
        !aligned16(D_copy))
      return MIGEMM_ERR_MISALIGNED;
    if (!(p->base.tiles_n > 0)) return MIGEMM_ERR_INVALID_ARG;
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != p->device) return MIGEMM_ERR_DEVICE;
  return MIGEMM_OK;
}

static int launch_run(const migemm_plan* p, const void* A, const void* B, const void* C, void* D,
                      float alpha, float beta, bool consumer, float* row_sum, float* row_max,
                      void* D_copy, void* workspace, hipStream_t stream) {
  KernelArgs a = p->base;
  // After a swap (column-major D) A and B trade places.
  a.A = p->swapped ? B : A;
  a.B = p->swapped ? A : B;
  a.C = beta != 0.0f ? C : nullptr;
  a.D = D;
  a.row_sum = row_sum;
  a.row_max = row_max;
  a.D_copy = D_copy;
  a.alpha = alpha;
  a.beta = beta;
  if (p->sel.stream_k) {
    a.sk_arrivals = static_cast<uint32_t*>(workspace);
    a.sk_partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + p->sk_counter_bytes);
  }
  if (p->debug && consumer) {
    a.dbg = static_cast<uint32_t*>(workspace);
    a.trace = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) +
                                          migemm::kDebugHeaderBytes);
    a.spin_budget = p->desc.debug_wait_ticks > 0 ? p->desc.debug_wait_ticks : kDefaultWaitTicks;
    a.force_wait = p->desc.debug_force_wait;
    a.trace_tiles = p->trace_tiles;
  }
  KernelSelect s = p->sel;
  s.consumer = consumer;
  hipError_t e = migemm::launch_gemm(s, a, p->grid, stream);
  return e == hipSuccess ? MIGEMM_OK : MIGEMM_ERR_LAUNCH;
}

static int run_common(const migemm_plan* p, const void* A, const void* B, const void* C, void* D,
                      float alpha, float beta, bool consumer, float* row_sum, float* row_max,
                      void* D_copy, void* workspace, void* stream) {
  int st = check_run(p, A, B, C, D, beta, consumer, row_sum, row_max, D_copy);
  if (st != MIGEMM_OK || p->M == 0 || p->N == 0) return st;
  if (p->workspace_bytes > 0) {
    if (!workspace) return MIGEMM_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return MIGEMM_ERR_MISALIGNED;
  }
  return launch_run(p, A, B, C, D, alpha, beta, consumer, row_sum, row_max, D_copy, workspace,
                    static_cast<hipStream_t>(stream));
}

int gemm_run(const migemm_plan* plan, const void* A, const void* B, const void* C, void* D,
             float alpha, float beta, void* workspace, void* stream) {
  return run_common(plan, A, B, C, D, alpha, beta, false, nullptr, nullptr, nullptr, workspace,
                    stream);
}

int gemm_run_with_tile_consumer(const migemm_plan* plan, const void* A, const void* B,
                                const void* C, void* D, float alpha, float beta, float* row_sum,
                                float* row_max, void* D_copy, void* workspace, void* stream) {
  return run_common(plan, A, B, C, D, alpha, beta, true, row_sum, row_max, D_copy, workspace,
                    stream);
}

int gemm_debug_read(const migemm_plan* p, const void* workspace, void* stream,
                    migemm_debug_info* out) {
  if (!plan_is_live(p) || !out || !workspace || !p->debug) return MIGEMM_ERR_INVALID_ARG;
  std::memset(out, 0, sizeof(*out));
  uint32_t head[2] = {0, 0};
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess ||
      hipMemcpy(head, workspace, sizeof(head), hipMemcpyDeviceToHost) != hipSuccess)
    return MIGEMM_ERR_DEVICE;
  out->waits_given_up = head[0];
  out->max_occupancy = head[1];
  out->trace_offset = migemm::kDebugHeaderBytes;
  out->grid = p->grid;
  out->waves = migemm::kWaves;
  out->trace_tiles = p->trace_tiles;
  out->trace_words = migemm::kTraceWords;
  return head[0] > 0 ? MIGEMM_ERR_TIMEOUT : MIGEMM_OK;
}

static_assert(migemm::kNoAllocScratchBytes == MIGEMM_NO_ALLOC_SCRATCH_BYTES,
              "the header states the fixed scratch size");

int gemm_run_no_alloc(const migemm_plan* plan, const void* A, const void* B, const void* C,
                      void* D, float alpha, float beta, void* stream) {
  int st = check_run(plan, A, B, C, D, beta, false, nullptr, nullptr, nullptr);
  if (st != MIGEMM_OK || plan->M == 0 || plan->N == 0) return st;
  void* ws = nullptr;
  if (plan->workspace_bytes > 0) {
    if (plan->workspace_bytes > (size_t)MIGEMM_NO_ALLOC_SCRATCH_BYTES) return MIGEMM_ERR_SCRATCH;
    if (migemm::no_alloc_scratch(plan->device, &ws) != hipSuccess) return MIGEMM_ERR_DEVICE;
    // The arrival counters must start at zero; the array keeps whatever the
    // last call on this device left, so they are cleared here every time
    // (with a fill kernel, which a graph capture can record).
    if (migemm::launch_zero_words(static_cast<uint32_t*>(ws), plan->sk_counters,
                                  static_cast<hipStream_t>(stream)) != hipSuccess)
      return MIGEMM_ERR_LAUNCH;
  }
  return launch_run(plan, A, B, C, D, alpha, beta, false, nullptr, nullptr, nullptr, ws,
                    static_cast<hipStream_t>(stream));
}

const char* gemm_status_string(int status) {
  switch (status) {
    case MIGEMM_OK: return "MIGEMM_OK";
    case MIGEMM_ERR_INVALID_ARG: return "MIGEMM_ERR_INVALID_ARG: invalid argument";
    case MIGEMM_ERR_UNSUPPORTED: return "MIGEMM_ERR_UNSUPPORTED: valid request not implemented";
    case MIGEMM_ERR_MISALIGNED: return "MIGEMM_ERR_MISALIGNED: pointer or stride not 16-byte aligned";
    case MIGEMM_ERR_DEVICE: return "MIGEMM_ERR_DEVICE: no usable gfx950 device";
    case MIGEMM_ERR_LAUNCH: return "MIGEMM_ERR_LAUNCH: kernel launch failed";
    case MIGEMM_ERR_TIMEOUT: return "MIGEMM_ERR_TIMEOUT: device wait timed out";
    case MIGEMM_ERR_SCRATCH:
      return "MIGEMM_ERR_SCRATCH: the plan's workspace exceeds the fixed scratch of "
             "gemm_run_no_alloc (MIGEMM_NO_ALLOC_SCRATCH_BYTES)";
    default: return "unknown migemm status";
  }
}

}  // extern "C"
