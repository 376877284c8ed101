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
#include "mainloop.hpp"
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
  // have completed by then (its last fetch was waited for and read back just
  // before), and the payload in D is never overwritten inside one kernel, so
  // no memory fence is needed.
  __device__ __forceinline__ static void release(int slot, int lane) {
    compiler_fence();
    if (lane == 0) __atomic_fetch_add(word(slot, kEmpty), 1u, __ATOMIC_RELAXED);
  }
};

// One lane's share of the consumer work on one tile: one row.
//
// The row is read in 16-byte chunks.  Each chunk is fetched with an LDS-DMA
// load into the lane's 16 bytes of one of its wave's landing slots, then
// waited for, read back, and folded in.  Going through LDS (like the K-loop
// ring) keeps every wait explicit: the compiler never sees an outstanding
// load, so it never answers one with a vmcnt(0) that would also drain the
// ring.  Inside the K loop one chunk is fetched per iteration, just before
// the iteration's stage loads, and folded in one iteration later, when only
// those 8 stage loads are younger than it; after the loop the rest of the
// row is drained with kConsumerDepth fetches in flight.
struct TileConsumer {
  __amdgpu_buffer_rsrc_t rsrc;  // D from the tile's first row and column
  uint32_t row_off;            // byte offset of this lane's row in rsrc (kOobOffset: no row)
  unsigned short* dst;         // D_copy row, first column of the tile
  int64_t stat;                // index of this row's entry in row_sum / row_max
  int ncols;                   // valid columns of the tile
  int fetched;                 // chunks fetched so far
  int done;                    // chunks folded in so far
  int slot;
  bool active;
  bool has_row;
  float sum, mx;

  __device__ __forceinline__ int chunks() const { return (ncols + 7) >> 3; }
  __device__ __forceinline__ void idle() { active = false; }

  __device__ __forceinline__ static uint32_t landing(int wave, int c) {
    return kConsumerSlotOffset + (wave * kConsumerDepth + (c % kConsumerDepth)) * kConsumerSlotBytes;
  }

  // Wait for the use-th commit of `slot`, then set up this lane's row.
  __device__ __forceinline__ void begin(const KernelArgs& a, int slot_, uint32_t use, int wave,
                                        int lane) {
    slot = slot_;
    const int tile_id = HandoffRing::wait(slot, use);
    const TileCoord t = tile_of(tile_id, a);
    const int64_t r0 = (int64_t)t.tm * kTileM;
    const int64_t c0 = (int64_t)t.tn * kTileN;
    const int r = wave * 64 + lane;
    const int64_t left = a.N - c0;
    ncols = (int)(left < kTileN ? left : kTileN);
    const unsigned short* base = static_cast<const unsigned short*>(a.D) + r0 * a.ldd + c0;
    int64_t bytes = ((a.M - 1 - r0) * a.ldd + (a.N - c0)) * 2;
    bytes = (bytes + 15) & ~(int64_t)15;  // per-dword range checks: see OperandLoader::issue
    rsrc = make_rsrc(base, (uint32_t)(bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes));
    has_row = r0 + r < a.M;
    row_off = has_row ? (uint32_t)(r * a.ldd * 2) : kOobOffset;
    dst = static_cast<unsigned short*>(a.D_copy) + (r0 + r) * a.ldd + c0;
    stat = (r0 + r) * a.stat_ld + t.tn;
    fetched = 0;
    done = 0;
    sum = 0.0f;
    mx = -__builtin_inff();
    active = true;
  }

  __device__ __forceinline__ void fetch(int wave) {
    const int c = fetched++;
    dma16(rsrc, lds_at(landing(wave, c)), row_off == kOobOffset ? kOobOffset : row_off + 16 * c);
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

  // Fold in the oldest fetched chunk (its fetch must have completed).
  __device__ __forceinline__ void fold(const KernelArgs& a, int wave, int lane) {
    compiler_fence();
    const int c = done++;
    const u32x4 v = *(const MIGEMM_LDS u32x4*)lds_at(landing(wave, c) + 16 * lane);
    if (has_row) absorb(c, v);
    wait_lgkmcnt<0>();  // the read is done before the landing slot is refilled
    if (done == chunks()) {
      if (has_row) {
        a.row_sum[stat] = sum;
        a.row_max[stat] = mx;
      }
      active = false;
      HandoffRing::release(slot, lane);
    }
  }

  // K-loop hook, once per iteration: fold in the chunk fetched one iteration
  // earlier, then fetch the next.  Since that fetch the wave has issued the
  // `since` (8) stage loads of one iteration, all younger than it; vector
  // memory operations complete in order, so vmcnt(8) covers the fetch
  // without forcing those stage loads to land.
  __device__ __forceinline__ void step(const KernelArgs& a, int wave, int lane, int since) {
    if (!active) return;
    if (fetched > done) {
      if (since >= 8) {
        wait_vmcnt<8>();
      } else {
        wait_vmcnt<0>();
      }
      fold(a, wave, lane);
    }
    if (active && fetched < chunks()) fetch(wave);
  }

  // After the K loop: finish the row with up to kConsumerDepth fetches in
  // flight.  newer = fetches issued after the one being waited for.
  __device__ __forceinline__ void drain(const KernelArgs& a, int wave, int lane) {
    while (active) {
      while (fetched < chunks() && fetched - done < kConsumerDepth) fetch(wave);
      const int newer = fetched - done - 1;
      static_assert(kConsumerDepth <= 4, "drain waits are written for up to 4 fetches in flight");
      if (newer >= 3) {
        wait_vmcnt<3>();
      } else if (newer == 2) {
        wait_vmcnt<2>();
      } else if (newer == 1) {
        wait_vmcnt<1>();
      } else {
        wait_vmcnt<0>();
      }
      fold(a, wave, lane);
    }
  }
};

}  // namespace migemm
