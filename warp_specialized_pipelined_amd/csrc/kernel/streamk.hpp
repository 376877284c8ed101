// streamk.hpp -- stream-K tiles: K-range segments of output tiles, and the
// fixup that adds their partial accumulators.
//
// The CUTLASS SM90 cooperative kernel lets its tile scheduler hand a CTA a
// K range of a tile instead of a whole one (stream-K): the CTA then keeps a
// partial accumulator, the scheduler's fixup reduces the partials of a tile
// through a workspace the host sizes and initializes, and only the unit that
// finishes a tile runs the epilogue (kernel page: the scheduler's fixup and
// compute_epilogue calls, get_workspace_size and initialize_workspace, and
// the separate-reduction epilogue subtiles).
//
// Here (scheduler.hpp) every workgroup takes one contiguous range of K-stage
// units.  A segment that covers a whole tile runs the usual epilogue.  For a
// partial one, each wave stores its 128 x 128 fp32 partial in the
// workgroup's own workspace slot and counts itself in at the tile's arrival
// counter for that wave; the wave that arrives last adds the partials of all
// contributors, in the order of their K ranges (so the result does not depend
// on which one arrives last), runs the epilogue for its quarter of the tile
// and sets the counter back to zero for the next run.  No wave ever waits
// for another workgroup, so the scheme cannot deadlock whatever the order in
// which workgroups run.
//
// The L2 of each XCD is private.  Agent-scope fences would write back (on
// release) or invalidate (on acquire) the whole L2 of the XCD, throwing out
// operand lines its other compute units are still reading; with them the
// fixup cost more than the split saved.  The partials are instead written and
// read as agent-scope relaxed atomic data (the sc1 bit: coherent across the
// XCDs), and ordered by completion: every store has completed (vmcnt 0)
// before the arrival is counted, and the last arrival's loads are issued
// only after the count they depend on has returned.
#pragma once

#include "epilogue.hpp"
#include "gfx950.hpp"
#include "mainloop.hpp"
#include "params.hpp"
#include "scheduler.hpp"

namespace migemm {

// This wave's share of partial slot `which` of workgroup slot w: its 128 x 128
// accumulators in register order -- lane l's 16 values of block b as four
// 16-byte pieces at (4 b + q) * 64 + l -- so every store and load instruction
// moves 1 KiB of consecutive bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_slot(const KernelArgs& a, int w, int which,
                                                        int wave) {
  constexpr int64_t kWaveBytes = (int64_t)kWaveTile * kWaveTile * 4;  // 64 KiB
  return make_rsrc(reinterpret_cast<unsigned char*>(a.sk_partials) +
                       (((int64_t)w * kSkPartialSlots + which) * kWaves + wave) * kWaveBytes,
                   (uint32_t)kWaveBytes);
}
__device__ __forceinline__ uint32_t sk_piece(int b, int q, int lane) {
  return (uint32_t)(((4 * b + q) * 64 + lane) * 16);
}

// Partial slot that workgroup slot c uses for tile units [tu0, ...): 0 for the
// tile its range starts in, 1 for the tile it ends in.
__device__ __forceinline__ int sk_which(int64_t U, int c, int G, int64_t tu0) {
  return sk_begin(U, c, G) >= tu0 ? 0 : 1;
}


// A partial segment of stream-K tile s is done.  If this wave finishes the
// tile's quarter, add all partials into acc and return true (the caller then
// stores the quarter); otherwise publish the partial and return false.
//
// The contributor holding the tile's K stage 0 (the head, w_lo) often gets
// here last: when its range started in an earlier tile, this segment ends
// its range while the others run theirs first in theirs.  So the head looks
// at the counter once; if all the others have counted in, it takes their
// partials without storing its own.  Otherwise it publishes its partial like
// every other contributor and the last arrival finishes the tile.  Either
// way exactly one wave finishes, and nobody waits.
__device__ __forceinline__ bool stream_k_fixup(Accum& acc, const KernelArgs& a, int s, int w,
                                               int G, int64_t U, int wave, int lane) {
  const int64_t tu0 = (int64_t)s * a.sk_kt;
  const int w_lo = sk_owner(U, tu0, G);
  const int w_hi = sk_owner(U, tu0 + a.sk_kt - 1, G);
  const uint32_t others = (uint32_t)(w_hi - w_lo);
  uint32_t* counter = a.sk_arrivals + (int64_t)s * kWaves + wave;

  bool head_done = false;
  if (w == w_lo) {
    uint32_t seen = 0;
    if (lane == 0) seen = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    head_done = __builtin_amdgcn_readfirstlane(seen) == others;
  }
  if (!head_done) {
    const __amdgpu_buffer_rsrc_t mine = sk_slot(a, w, sk_which(U, w, G, tu0), wave);
#pragma unroll
    for (int b = 0; b < 16; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& v = acc.v[b >> 2][b & 3];
        const f32x4 piece = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, piece), mine,
                                               sk_piece(b, q, lane), 0, kCpolDevice);
      }
    // Release: every partial store has completed before the arrival counts.
    compiler_fence();
    wait_vmcnt<0>();
    compiler_fence();
    uint32_t before = 0;
    if (lane == 0) before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The last of all contributors finishes.  (When the head finished
    // without counting in, the others' counts stop one short of this.)
    if (__builtin_amdgcn_readfirstlane(before) != others) return false;
  }

  // Acquire: the loads below come after the count they depend on.
  compiler_fence();
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Sum in K order: ((p_lo + p_lo+1) + ...) + p_hi, this wave's own partial
  // taken from its registers.
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    f32x16 sum = acc.v[b >> 2][b & 3];
    for (int c = w_lo; c <= w_hi; ++c) {
      f32x16 x = acc.v[b >> 2][b & 3];
      if (c != w) {
        const __amdgpu_buffer_rsrc_t p = sk_slot(a, c, sk_which(U, c, G, tu0), wave);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 y = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(p, sk_piece(b, q, lane), 0, kCpolDevice));
          x[4 * q] = y[0];
          x[4 * q + 1] = y[1];
          x[4 * q + 2] = y[2];
          x[4 * q + 3] = y[3];
        }
      }
      sum = c == w_lo ? x : sum + x;
    }
    acc.v[b >> 2][b & 3] = sum;
  }
  return true;
}

// The lane and wave index as values the compiler cannot see through (as in
// the kernel's tile loop): per-lane offsets are recomputed per segment.
struct SkIds {
  int lane, wave;
  __device__ __forceinline__ SkIds(int l, int w) : lane(l), wave(w) {
    asm volatile("" : "+v"(lane));
    asm volatile("" : "+s"(wave));
  }
};

// Workgroup slot w's range of stream-K units, segment by segment.
template <int ES, bool AK, bool BK>
__device__ __forceinline__ void stream_k_tiles(Accum& acc, const KernelArgs& a, int w, int G,
                                               int lane, int wave) {
  const int64_t U = sk_units(a);
  const int64_t u1 = sk_begin(U, w + 1, G);
  const int kt = a.sk_kt;
  NoSideWork none;
  for (int64_t u = sk_begin(U, w, G); u < u1;) {
    const int s = (int)(u / kt);
    const int kb = (int)(u - (int64_t)s * kt);
    const int n = (int)((int64_t)(kt - kb) < u1 - u ? (int64_t)(kt - kb) : u1 - u);
    const TileCoord t = tile_of(a.sk_first + s, a);
    const KernelArgs ab = batch_args(a, t.l);
    // A segment that ends before the tile's last stage ends the K range
    // there: its loads past it fall out of range.
    const int64_t kend_stage = (int64_t)(kb + n) * StageGeom<ES>::kK;
    const int64_t kend = kend_stage < a.K ? kend_stage : a.K;
    int k0 = kb, nk = n;
    asm volatile("" : "+s"(k0), "+s"(nk));
    const SkIds id(lane, wave);
    mainloop_range<ES, AK, BK>(acc, ab, t.tm, t.tn, id.wave, id.lane, none, k0, nk, kend);
    const SkIds ie(lane, wave);
    bool finish = n == kt;
    if (!finish) finish = stream_k_fixup(acc, a, s, w, G, U, ie.wave, ie.lane);
    if (finish) epilogue_store(acc, ab, t.tm, t.tn, ie.wave, ie.lane);
    wait_lgkmcnt<0>();  // staging reads done ...
    barrier();          // ... in every wave before the ring is refilled
    u += n;
  }
}

}  // namespace migemm
