// handoff.hpp -- the tile hand-off ring and the consumer stage it feeds.
//
// CUTLASS issue #2900 asks for a pipeline between the epilogue (producer) and
// a consumer warp group: the producer acquires an empty slot, stores the
// finished tile to global memory and commits it; the consumer waits until the
// tile is ready, works on it, and releases the slot -- so that the consumer
// can run while the MMA warps start the next tile, which a store pipeline
// drained only at the very end cannot give.  The CUTLASS kernel page starts
// producers "at the opposite phase" so their first waits pass, and the CuTe
// DSL pipeline docs name the verbs (producer_acquire / producer_commit /
// consumer_release).
//
// Here the ring lives in LDS: kHandoffSlots slots of
//     { tile id, full count, empty count }.
// The payload is the tile itself, already stored in D.  The counters only
// grow, so no phase bit is needed: the u-th use of a slot (u = 0, 1, ...)
//   acquire  waits for  empty >= u * kWaves      (passes at once for u = 0)
//   commit   adds 1 to  full    (each producer wave, after its stores landed)
//   wait     waits for  full  >= (u + 1) * kWaves
//   release  adds 1 to  empty   (each consumer wave, after its reads landed)
// Every wave is both a producer (its quarter of the tile) and a consumer (64
// rows of the tile), because on gfx950 all waves of a kernel get the same
// register allocation and the 256 accumulator registers of a 128 x 128 wave
// tile leave no room for extra waves.  The consumer work on tile n is spread
// over the first iterations of tile n+1's K loop, one 16-byte chunk per lane
// per iteration, so it runs in the shadow of the MFMAs.
//
// Consumer work for a 256 x 256 tile at tile column t: for each of its rows r
// (one lane per row),
//   row_sum[r][t] = fp32 sum, in ascending column order from +0.0f, of the
//                   bf16 values of D in that row of the tile,
//   row_max[r][t] = maxNum of the same values, from -inf,
// and the row is copied bit for bit to D_copy.
#pragma once

#include "gfx950.hpp"
#include "params.hpp"
#include "scheduler.hpp"

namespace migemm {

typedef MIGEMM_LDS uint32_t lds_u32;

struct HandoffRing {
  enum { kTileId = 0, kFull = 1, kEmpty = 2 };
  __device__ __forceinline__ static lds_u32* word(int slot, int field) {
    return (lds_u32*)lds_at(kHandoffOffset + slot * 16 + field * 4);
  }
  // All slots empty and unused; call before the kernel's first barrier.
  __device__ __forceinline__ static void init() {
    if (threadIdx.x < kHandoffSlots * 4) *word(threadIdx.x >> 2, threadIdx.x & 3) = 0;
  }
  __device__ __forceinline__ static void spin_until(lds_u32* p, uint32_t target) {
    while (__atomic_load_n(p, __ATOMIC_RELAXED) < target) __builtin_amdgcn_s_sleep(1);
  }
  // Producer side.
  __device__ __forceinline__ static void acquire(int slot, uint32_t use) {
    spin_until(word(slot, kEmpty), use * kWaves);
  }
  // Publishes the caller's stores of the tile: the workgroup-scope release
  // fence waits for them to complete before the count goes up.
  __device__ __forceinline__ static void commit(int slot, int tile_id, int wave, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) {
      if (wave == 0) __atomic_store_n(word(slot, kTileId), (uint32_t)tile_id, __ATOMIC_RELAXED);
      __atomic_fetch_add(word(slot, kFull), 1u, __ATOMIC_RELAXED);
    }
  }
  // Consumer side.  Returns the committed tile's id; the acquire fence keeps
  // the consumer's reads of the tile after the observed commit.
  __device__ __forceinline__ static int wait(int slot, uint32_t use) {
    spin_until(word(slot, kFull), (use + 1) * kWaves);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return (int)__atomic_load_n(word(slot, kTileId), __ATOMIC_RELAXED);
  }
  // The slot (its tile id) is free again.  The consumer's reads of the tile
  // have completed by then: its last fetched chunk was folded in just before,
  // and vector loads complete in order.  The payload in D is never
  // overwritten inside one kernel, so no memory fence is needed.
  __device__ __forceinline__ static void release(int slot, int lane) {
    compiler_fence();
    if (lane == 0) __atomic_fetch_add(word(slot, kEmpty), 1u, __ATOMIC_RELAXED);
  }
};

// One lane's share of the consumer work on one tile: one row.
struct TileConsumer {
  static constexpr int kChunks = kTileN / 8;  // 16-byte chunks per tile row
  const unsigned short* src;   // D row, first column of the tile (NULL: no row)
  unsigned short* dst;         // D_copy row, same place
  float* sum_out;
  float* max_out;
  int ncols;                   // valid columns of the tile
  int step;                    // next step, 0 .. chunks()
  int slot;
  bool active;
  float sum, mx;
  u32x4 data;                  // chunk fetched by the previous step

  __device__ __forceinline__ int chunks() const { return (ncols + 7) >> 3; }

  __device__ __forceinline__ void idle() { active = false; }

  // Wait for the use-th commit of `slot`, then set up this lane's row.
  __device__ __forceinline__ void begin(const KernelArgs& a, int slot_, uint32_t use, int wave,
                                        int lane) {
    slot = slot_;
    const int tile_id = HandoffRing::wait(slot, use);
    const TileCoord t = tile_of(tile_id, a);
    const int64_t row = (int64_t)t.tm * kTileM + wave * 64 + lane;
    const int64_t col0 = (int64_t)t.tn * kTileN;
    const int64_t left = a.N - col0;
    ncols = (int)(left < kTileN ? left : kTileN);
    if (row < a.M) {
      src = static_cast<const unsigned short*>(a.D) + row * a.ldd + col0;
      dst = static_cast<unsigned short*>(a.D_copy) + row * a.ldd + col0;
      sum_out = a.row_sum + row * a.stat_ld + t.tn;
      max_out = a.row_max + row * a.stat_ld + t.tn;
    } else {
      src = nullptr;
    }
    step = 0;
    sum = 0.0f;
    mx = -__builtin_inff();
    active = true;
  }

  // Fetch chunk c of the row.  A whole chunk is one 16-byte load issued as
  // inline assembly, so that the compiler does not answer its result with a
  // vmcnt(0) that would also drain the K loop's LDS-DMA loads; advance()
  // waits for it explicitly.  The partial last chunk of a ragged tile uses
  // element loads the compiler tracks itself.
  __device__ __forceinline__ u32x4 fetch(int c) const {
    const int col = 8 * c;
    u32x4 v;
    if (col + 8 <= ncols) {
      asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(src + col) : "memory");
      return v;
    }
    v = u32x4{0, 0, 0, 0};
    for (int e = 0; col + e < ncols; ++e) v[e >> 1] |= (uint32_t)src[col + e] << (16 * (e & 1));
    return v;
  }

  // Wait until the chunk fetched by the previous step has arrived.  The
  // vector memory operations issued since then are the stage loads of this
  // K iteration (8, or none), and they complete after it (in order).
  __device__ __forceinline__ void wait_fetched(bool stage_loads_since) {
    if (stage_loads_since) {
      asm volatile("s_waitcnt vmcnt(8)" : "+v"(data) : : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(data) : : "memory");
    }
  }

  __device__ __forceinline__ void absorb(int c, u32x4 v) {
    const int col = 8 * c;
    const int n = ncols - col;
    if (n >= 8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
        sum = sum + x;
        mx = fmaxf(mx, x);
      }
      *reinterpret_cast<u32x4*>(dst + col) = v;
    } else {
      for (int e = 0; e < n; ++e) {
        const uint32_t h = v[e >> 1] >> (16 * (e & 1));
        const float x = __uint_as_float(h << 16);
        sum = sum + x;
        mx = fmaxf(mx, x);
        dst[col + e] = (unsigned short)h;
      }
    }
  }

  // One step: fold in the chunk fetched last time and fetch the next one.
  // stage_loads_since: the K loop issued stage loads since the last step.
  __device__ __forceinline__ void advance(int lane, bool stage_loads_since) {
    if (!active) return;
    const int nc = chunks();
    if (src) {
      if (step > 0) {
        wait_fetched(stage_loads_since);
        absorb(step - 1, data);
      }
      if (step < nc) data = fetch(step);
    }
    ++step;
    if (step > nc) {
      if (src) {
        *sum_out = sum;
        *max_out = mx;
      }
      active = false;
      HandoffRing::release(slot, lane);
    }
  }

  __device__ __forceinline__ void drain(int lane) {
    while (active) advance(lane, false);
  }
};

}  // namespace migemm
