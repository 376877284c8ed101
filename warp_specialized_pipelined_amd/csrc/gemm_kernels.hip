// gemm_kernels.hip -- the persistent GEMM kernel and its instantiations.
//
// One workgroup of 4 waves per compute unit.  For every tile the scheduler
// hands it, the workgroup runs the pipelined K loop into a 256 x 256 fp32
// accumulator tile (128 x 128 per wave) and then the epilogue.
#include <hip/hip_runtime.h>

#include "kernel/epilogue.hpp"
#include "kernel/gfx950.hpp"
#include "kernel/handoff.hpp"
#include "kernel/mainloop.hpp"
#include "kernel/params.hpp"
#include "kernel/scheduler.hpp"
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

template <int ES, bool AK, bool BK, bool CONS>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(KernelArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int first = persistent_slot(blockIdx.x, gridDim.x);
  Accum acc;
  if constexpr (!CONS) {
    NoSideWork none;
    for (int L = first; L < a.num_tiles; L += gridDim.x) {
      const TileCoord t = tile_of(L, a);
      const LaneIds id(lane, wave);
      mainloop<ES, AK, BK>(acc, a, t.tm, t.tn, id.wave, id.lane, none);
      const LaneIds ie(lane, wave);
      epilogue_store(acc, a, t.tm, t.tn, ie.wave, ie.lane);
      wait_lgkmcnt<0>();  // staging reads done ...
      barrier();          // ... in every wave before the ring is refilled
    }
  } else {
    // Tile n of this workgroup goes through hand-off slot n % S (use n / S).
    // The consumer stage of tile n runs inside tile n+1's K loop; the last
    // tile's runs after the loop.
    HandoffRing::init();
    __syncthreads();
    TileConsumer cons;
    cons.idle();
    int n = 0;
    for (int L = first; L < a.num_tiles; L += gridDim.x, ++n) {
      const TileCoord t = tile_of(L, a);
      if (n > 0) cons.begin(a, (n - 1) % kHandoffSlots, (n - 1) / kHandoffSlots, wave, lane);
      const LaneIds id(lane, wave);
      mainloop<ES, AK, BK>(acc, a, t.tm, t.tn, id.wave, id.lane, cons);
      cons.drain(a, wave, lane);
      const int s = n % kHandoffSlots;
      HandoffRing::acquire(s, n / kHandoffSlots);
      const LaneIds ie(lane, wave);
      epilogue_store(acc, a, t.tm, t.tn, ie.wave, ie.lane);
      HandoffRing::commit(s, L, wave, lane);
      wait_lgkmcnt<0>();
      barrier();
    }
    if (n > 0) {
      cons.begin(a, (n - 1) % kHandoffSlots, (n - 1) / kHandoffSlots, wave, lane);
      cons.drain(a, wave, lane);
    }
  }
}

typedef void (*kernel_fn)(KernelArgs);

template <int ES>
static kernel_fn pick(bool ak, bool bk, bool cons) {
  if (cons) {
    if (ak) return bk ? gemm_kernel<ES, true, true, true> : gemm_kernel<ES, true, false, true>;
    return bk ? gemm_kernel<ES, false, true, true> : gemm_kernel<ES, false, false, true>;
  }
  if (ak) return bk ? gemm_kernel<ES, true, true, false> : gemm_kernel<ES, true, false, false>;
  return bk ? gemm_kernel<ES, false, true, false> : gemm_kernel<ES, false, false, false>;
}

static kernel_fn select(const KernelSelect& s) {
  return s.elem_bytes == 2 ? pick<2>(s.a_kmajor, s.b_kmajor, s.consumer)
                           : pick<1>(s.a_kmajor, s.b_kmajor, s.consumer);
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

}  // namespace migemm
