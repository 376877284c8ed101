// gemm_kernels.hip -- the persistent GEMM kernels and their instantiations.
//
// One workgroup of 4 waves per compute unit.  For every tile the scheduler
// hands it, the workgroup runs the pipelined K loop into a 256 x 256 fp32
// accumulator tile (128 x 128 per wave) and then the epilogue.  Stream-K
// kernels then take their range of K-stage units of the remaining tiles
// (streamk.hpp); tile-consumer kernels pass each finished tile through the
// hand-off ring to the consumer stage (handoff.hpp).  A second bf16 kernel
// takes 192 x 256 tiles, for shapes where 256-row tiles leave compute units
// idle in the last round.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernel/epilogue.hpp"
#include "kernel/gfx950.hpp"
#include "kernel/handoff.hpp"
#include "kernel/mainloop.hpp"
#include "kernel/params.hpp"
#include "kernel/scheduler.hpp"
#include "kernel/streamk.hpp"
#include "launch.h"

namespace migemm {

// The lane and wave index as values the compiler cannot see through.  Every
// per-lane offset of the K loop and the epilogue derives from them; taking
// them afresh for each tile keeps those offsets from being computed once
// before the tile loop and held (or spilled) across the whole of it -- a
// spilled offset comes back with a vmcnt(0) that would drain the ring.
struct LaneIds {
  int lane, wave;
  __device__ __forceinline__ LaneIds(int l, int w) : lane(l), wave(w) {
    asm volatile("" : "+v"(lane));
    asm volatile("" : "+s"(wave));
  }
};

template <int ES, bool AK, bool BK, int CONS, bool SK>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(KernelArgs a) {
  static_assert(!(CONS != kConsNone && SK), "the tile consumer runs on whole tiles only");
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int first = persistent_slot(blockIdx.x, gridDim.x);
  Accum acc;
  if constexpr (CONS == kConsNone) {
    NoSideWork none;
    const int whole = SK ? a.sk_first : a.num_tiles;  // tiles taken whole
    if (!SK && a.C != nullptr && a.c_preload) {
      // beta != 0: the last two K iterations load the tile's C into LDS
      // (CPreload), when the K loop has at least two stages.
      const bool preload = (a.K + StageGeom<ES>::kK - 1) / StageGeom<ES>::kK >= 2;
      for (int L = first; L < whole; L += gridDim.x) {
        const TileCoord t = tile_of(L, a);
        const KernelArgs ab = batch_args(a, t.l);
        const LaneIds id(lane, wave);
        CPreload pre;
        mainloop<ES, AK, BK>(acc, ab, t.tm, t.tn, id.wave, id.lane, pre);
        const LaneIds ie(lane, wave);
        epilogue_store(acc, ab, t.tm, t.tn, ie.wave, ie.lane, preload);
        wait_lgkmcnt<0>();
        barrier();
      }
    } else {
      for (int L = first; L < whole; L += gridDim.x) {
        const TileCoord t = tile_of(L, a);
        const KernelArgs ab = batch_args(a, t.l);
        const LaneIds id(lane, wave);
        mainloop<ES, AK, BK>(acc, ab, t.tm, t.tn, id.wave, id.lane, none);
        const LaneIds ie(lane, wave);
        epilogue_store(acc, ab, t.tm, t.tn, ie.wave, ie.lane);
        wait_lgkmcnt<0>();  // staging reads done ...
        barrier();          // ... in every wave before the ring is refilled
      }
    }
    if constexpr (SK) {
      // When every tile is split (no whole-tile rounds before), the slot is
      // the dispatch index itself.  The hardware deals consecutive
      // workgroups round-robin over the XCDs, so the contributors of one
      // tile land on different XCDs, and each XCD runs the same K range of
      // many tiles that share operand panels in its L2 (the remap would give
      // an XCD all K ranges of a few tiles instead).  Which workgroup holds
      // which slot does not change the result: the fixup adds the partials
      // in the order of their K ranges.
      const int w = a.sk_first == 0 ? (int)blockIdx.x : first;
      stream_k_tiles<ES, AK, BK>(acc, a, w, gridDim.x, lane, wave);
    }
  } else if constexpr (CONS == kConsStaged) {
    // Tile n of this workgroup goes through hand-off slot n % S (use n / S).
    // Once all four waves have committed it, each wave runs the consumer
    // stage on its 64 rows of the tile as the epilogue left it staged in
    // LDS, and releases the slot before the next K loop refills the ring
    // over the staging area.
    HandoffRing::init(a);
    __syncthreads();
    TileConsumer cons;
    cons.idle();
    NoSideWork none;
    int n = 0;
    for (int L = first; L < a.num_tiles; L += gridDim.x, ++n) {
      const TileCoord t = tile_of(L, a);
      const KernelArgs ab = batch_args(a, t.l);
      trace_event(n, wave, kEvLoopBegin, lane);
      const LaneIds id(lane, wave);
      mainloop<ES, AK, BK>(acc, ab, t.tm, t.tn, id.wave, id.lane, none);
      trace_event(n, wave, kEvLoopEnd, lane);
      const int s = handoff_slot(n);
      HandoffRing::acquire(s, handoff_use(n), lane);
      trace_event(n, wave, kEvAcquired, lane);
      const LaneIds ie(lane, wave);
      epilogue_store(acc, ab, t.tm, t.tn, ie.wave, ie.lane);
      const uint32_t occ = HandoffRing::commit(s, L, wave, lane);
      uint64_t* rec = trace_record(n, wave);
      trace_put(rec, kEvCommitted, now_ticks(), lane);
      trace_put(rec, kTrOccupancy, occ, lane);
      trace_put(rec, kTrTileId, (uint64_t)L, lane);
      cons.begin(a, s, handoff_use(n), n, wave, lane);
      cons.fold_staged(wave, lane);
      cons.copy_staged(wave, lane);
      wait_lgkmcnt<0>();  // staging reads done ...
      barrier();          // ... in every wave before the ring is refilled
    }
  } else {
    // Overlapped schedule.  Tile n of this workgroup goes through hand-off
    // slot n % S (use n / S).  Its row statistics are folded right after its
    // commit, from the staged tile; its copy runs inside tile n+1's K loop,
    // fetching the tile back from D, and whatever the loop leaves, plus the
    // release of its slot, comes after tile n+1's commit: the ring then
    // holds two committed tiles.  The last tile is copied from its staging
    // area after the loop.
    HandoffRing::init(a);
    __syncthreads();
    TileConsumer cons;
    cons.idle();
    int n = 0;
    for (int L = first; L < a.num_tiles; L += gridDim.x, ++n) {
      const TileCoord t = tile_of(L, a);
      const KernelArgs ab = batch_args(a, t.l);
      trace_event(n, wave, kEvLoopBegin, lane);
      const LaneIds id(lane, wave);
      mainloop<ES, AK, BK>(acc, ab, t.tm, t.tn, id.wave, id.lane, cons);
      trace_event(n, wave, kEvLoopEnd, lane);
      const int s = handoff_slot(n);
      HandoffRing::acquire(s, handoff_use(n), lane);
      trace_event(n, wave, kEvAcquired, lane);
      const LaneIds ie(lane, wave);
      epilogue_store(acc, ab, t.tm, t.tn, ie.wave, ie.lane);
      const uint32_t occ = HandoffRing::commit(s, L, wave, lane);
      uint64_t* rec = trace_record(n, wave);
      trace_put(rec, kEvCommitted, now_ticks(), lane);
      trace_put(rec, kTrOccupancy, occ, lane);
      trace_put(rec, kTrTileId, (uint64_t)L, lane);
      cons.drain(wave, lane);  // tile n-1: steps the K loop left, and its release
      cons.begin(a, s, handoff_use(n), n, wave, lane);
      cons.fold_staged(wave, lane);
      wait_lgkmcnt<0>();
      barrier();
    }
    cons.copy_staged(wave, lane);  // the last tile (no-op without tiles)
  }
}

// 192 x 256 tiles (wave tiles of 96 x 128), bf16, whole tiles, no tile
// consumer.  A problem whose 256 x 256 tiles number a little over a multiple
// of the grid (192 of them on 256 compute units: a quarter of the units idle)
// gets 4/3 as many tiles of 3/4 the work; the plan chooses the height that
// gives each workgroup the least work.  C (beta != 0) is read in the epilogue.
template <bool AK, bool BK>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel_m192(KernelArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int first = persistent_slot(blockIdx.x, gridDim.x);
  Accum acc;
  NoSideWork none;
  for (int L = first; L < a.num_tiles; L += gridDim.x) {
    const TileCoord t = tile_of(L, a);
    const KernelArgs ab = batch_args(a, t.l);
    const LaneIds id(lane, wave);
    mainloop<2, AK, BK, 3>(acc, ab, t.tm, t.tn, id.wave, id.lane, none);
    const LaneIds ie(lane, wave);
    epilogue_store<3>(acc, ab, t.tm, t.tn, ie.wave, ie.lane);
    wait_lgkmcnt<0>();  // staging reads done ...
    barrier();          // ... in every wave before the ring is refilled
  }
}

typedef void (*kernel_fn)(KernelArgs);

template <int ES, int CONS, bool SK>
static kernel_fn pick(bool ak, bool bk) {
  if (ak) return bk ? gemm_kernel<ES, true, true, CONS, SK> : gemm_kernel<ES, true, false, CONS, SK>;
  return bk ? gemm_kernel<ES, false, true, CONS, SK> : gemm_kernel<ES, false, false, CONS, SK>;
}

template <int ES>
static kernel_fn pick_mode(const KernelSelect& s) {
  if (s.consumer && s.consumer_overlap) return pick<ES, kConsOverlap, false>(s.a_kmajor, s.b_kmajor);
  if (s.consumer) return pick<ES, kConsStaged, false>(s.a_kmajor, s.b_kmajor);
  if (s.stream_k) return pick<ES, kConsNone, true>(s.a_kmajor, s.b_kmajor);
  return pick<ES, kConsNone, false>(s.a_kmajor, s.b_kmajor);
}

static kernel_fn select(const KernelSelect& s) {
  if (s.tile_m == 192) {
    if (s.a_kmajor) return s.b_kmajor ? gemm_kernel_m192<true, true> : gemm_kernel_m192<true, false>;
    return s.b_kmajor ? gemm_kernel_m192<false, true> : gemm_kernel_m192<false, false>;
  }
  return s.elem_bytes == 2 ? pick_mode<2>(s) : pick_mode<1>(s);
}

int kernel_lds_bytes(const KernelSelect& sel) {
  return sel.consumer ? kConsumerLdsBytes : kPlainLdsBytes;
}


hipError_t prepare_kernel(const KernelSelect& sel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(select(sel)),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kernel_lds_bytes(sel));
}

hipError_t launch_gemm(const KernelSelect& sel, const KernelArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(select(sel), dim3(grid), dim3(kThreads), kernel_lds_bytes(sel), stream, args);
  return hipGetLastError();
}

// Zero the stream-K arrival counters (a fill kernel rather than a memset,
// so that the call may be captured in a HIP graph).
__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  blocks = blocks > 1024 ? 1024 : blocks;
  hipLaunchKernelGGL(zero_words, dim3(blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// The device scratch of gemm_run_no_alloc: a stream-K workspace for callers
// that cannot allocate device memory.  Each device holds its own copy from
// the moment the code object is loaded there until the process ends.  In
// host code the name is only a stand-in: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t no_alloc_scratch(int device, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[device] = ptr;
  }
  *out = addr[device];
  return hipSuccess;
}

}  // namespace migemm
