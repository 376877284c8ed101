// handoff.hpp -- the tile hand-off ring and the consumer stage it feeds.
//
// CUTLASS issue #2900 asks for a pipeline between the epilogue (producer) and
// a consumer warp group: the producer acquires an empty slot, stores the
// finished tile to global memory and commits it; the consumer waits until the
// tile is ready, works on it, and releases the slot -- so that the consumer
// can run while the MMA warps start the next tile, which a store pipeline
// drained only at the very end cannot give.  The CUTLASS kernel page starts
// its producers with the phase inverted, so that their first waits pass, and
// the CuTe DSL pipeline docs name the verbs (producer_acquire /
// producer_commit / consumer_release).
//
// Here the ring lives in LDS: kHandoffSlots slots of
//     { tile id, full count, empty count }.
// The payload is the tile itself, already stored in D.  The counters only
// grow, so no phase bit is needed: the u-th use of a slot (u = 0, 1, ...)
//   acquire  waits for  empty >= u * kWaves      (passes at once for u = 0)
//   commit   adds 1 to  full    (each producer wave, its stores ordered before)
//   wait     waits for  full  >= (u + 1) * kWaves
//   release  adds 1 to  empty   (each consumer wave, after its reads landed)
// Every wave is both a producer (its quarter of the tile) and a consumer (64
// rows of the tile), because on gfx950 all waves of a kernel get the same
// register allocation and the 256 accumulator registers of a 128 x 128 wave
// tile leave no room for extra waves.  Right after the tile's commit each
// wave folds the row statistics from the tile as the epilogue left it
// staged in LDS (fold_staged), before the next K loop refills the ring over
// the staging area.  The copy runs on one of two schedules:
//   staged (default): at once, from the staged tile (copy_staged), and the
//     slot is released right after;
//   overlapped: inside tile n+1's K loop, one step per iteration fetched
//     back from D (after_barrier); steps the loop did not reach are finished
//     after tile n+1's commit (drain), and tile n's slot is released there
//     too -- so when tile n+1 is committed the ring holds two committed
//     tiles, n and n+1, and the producer never waits for the consumer's last
//     steps of tile n.  The last tile is copied from its staging area.
// The overlap is what the hand-off ring is for when consumer work waits on
// memory or links; for this consumer stage the staged schedule costs less:
// the K loop's side work holds the MFMA waves longer than the work takes on
// its own.
//
// Debugging (kernel arguments dbg/trace, set by the plan's hand-off debug
// flag): every ring wait is bounded by a budget of s_memrealtime ticks and
// counts a wait that gave up in the workspace header (the kernel then goes
// on, so it always ends), and each wave writes one trace record per tile of
// its workgroup: the real-time clock at the events below, the ring's
// occupancy right after its commit, and the tile id.
// Consumer work for a 256 x 256 tile at tile column t: for each of its rows r,
// over the tile's columns below N, with x_j the bf16 value of D[r][256t + j]
// widened to fp32:
//   row_sum[r][t] = s, where s = +0.0f and then s = s + x_j for j = 0, 1, ...
//                   in column order (one fp32 rounding per addition),
//   row_max[r][t] = the largest x_j that is not a NaN, with -0 < +0; -inf if
//                   there is none (IEEE 754-2019 maximumNumber),
// and the row is copied bit for bit to D_copy.  Both statistics have exactly
// one correct value given D.  One lane folds one whole row, so the sequential
// order costs no more additions than any other.
#pragma once

#include "gfx950.hpp"
#include "handoff_rules.hpp"
#include "params.hpp"
#include "mainloop.hpp"
#include "scheduler.hpp"

namespace migemm {

typedef MIGEMM_LDS uint32_t lds_u32;

// Trace record of one wave and tile (kTraceWords 64-bit words): the
// real-time clock (100 MHz) when the wave began the tile's K loop, ended it,
// acquired the tile's slot, committed the tile, saw the tile committed by
// all waves (its consumer's wait), stored the tile's first and last copy
// step, and released the slot; then the ring occupancy right after this
// wave's commit (tiles committed by every wave minus tiles released by every
// wave, over both slots) and the tile id.
enum TraceWord {
  kEvLoopBegin = 0, kEvLoopEnd, kEvAcquired, kEvCommitted, kEvWaitDone, kEvCopyFirst, kEvCopyLast,
  kEvReleased, kTrOccupancy, kTrTileId
};

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// The debug settings, copied into LDS once per kernel (HandoffRing::init)
// and read back where they are used, so that none of them occupies a
// register across the K loops.
struct HandoffDebug {
  uint32_t* dbg;         // debug header, or NULL: unbounded waits, no trace
  uint64_t* trace;       // trace records, or NULL
  int64_t budget;        // ticks a bounded wait may spin
  uint32_t force;        // added to every acquire's target (a wait that cannot pass)
  int32_t trace_tiles;   // records per wave
};
static_assert(sizeof(HandoffDebug) <= kHandoffRecOffset - kHandoffDebugOffset, "debug block");

// The block is kept as 64-bit words: [0] dbg, [1] trace, [2] budget,
// [3] force | trace_tiles << 32; then one record pointer per wave.
__device__ __forceinline__ MIGEMM_LDS uint64_t* debug_words() {
  return (MIGEMM_LDS uint64_t*)lds_at(kHandoffDebugOffset);
}
__device__ __forceinline__ HandoffDebug handoff_debug() {
  const MIGEMM_LDS uint64_t* q = debug_words();
  HandoffDebug d;
  d.dbg = reinterpret_cast<uint32_t*>(q[0]);
  d.trace = reinterpret_cast<uint64_t*>(q[1]);
  d.budget = (int64_t)q[2];
  d.force = (uint32_t)q[3];
  d.trace_tiles = (int32_t)(q[3] >> 32);
  return d;
}
__device__ __forceinline__ MIGEMM_LDS uint64_t* rec_slot(int wave) {
  return (MIGEMM_LDS uint64_t*)lds_at(kHandoffRecOffset + 8 * wave);
}
__device__ __forceinline__ uint64_t* rec_of(int wave) {
  return reinterpret_cast<uint64_t*>(*rec_slot(wave));
}

// The trace record of this wave for the workgroup's seq-th tile, or NULL.
__device__ __forceinline__ uint64_t* trace_record(int seq, int wave) {
  const HandoffDebug d = handoff_debug();
  if (d.trace == nullptr) return nullptr;
  return d.trace + ((int64_t)(blockIdx.x * kWaves + wave) * d.trace_tiles + seq) * kTraceWords;
}
// One word of a record, written by lane 0 with a vector store.
__device__ __forceinline__ void trace_put(uint64_t* rec, int word, uint64_t v, int lane) {
  if (rec != nullptr && lane == 0) rec[word] = v;
}
// The real-time clock into a word of this wave's record of the workgroup's
// seq-th tile (looked up here).
__device__ __forceinline__ void trace_event(int seq, int wave, int word, int lane) {
  trace_put(trace_record(seq, wave), word, now_ticks(), lane);
}

struct HandoffRing {
  enum { kTileId = 0, kFull = 1, kEmpty = 2 };
  __device__ __forceinline__ static lds_u32* word(int slot, int field) {
    return (lds_u32*)lds_at(kHandoffOffset + slot * 16 + field * 4);
  }
  // All slots empty and unused, and the debug settings in place; call
  // before the kernel's first barrier.
  __device__ __forceinline__ static void init(const KernelArgs& a) {
    if (threadIdx.x < kHandoffSlots * 4) *word(threadIdx.x >> 2, threadIdx.x & 3) = 0;
    if (threadIdx.x == 0) {
      MIGEMM_LDS uint64_t* q = debug_words();
      q[0] = reinterpret_cast<uint64_t>(a.dbg);
      q[1] = reinterpret_cast<uint64_t>(a.trace);
      q[2] = (uint64_t)a.spin_budget;
      q[3] = (uint64_t)(uint32_t)a.force_wait | ((uint64_t)(uint32_t)a.trace_tiles << 32);
    }
    if (threadIdx.x < kWaves) *rec_slot(threadIdx.x) = 0;
  }
  __device__ __forceinline__ static uint32_t load(lds_u32* p) {
    return __atomic_load_n(p, __ATOMIC_RELAXED);
  }
  // Spin until *p >= target.  With a debug header the spin is bounded: after
  // the budget's ticks the wait gives up, is counted in the header, and the
  // caller goes on (so the kernel always ends).
  __device__ __forceinline__ static void spin_until(lds_u32* p, uint32_t target, int lane) {
    if (load(p) >= target) return;
    const HandoffDebug d = handoff_debug();
    if (d.dbg == nullptr) {
      while (load(p) < target) __builtin_amdgcn_s_sleep(1);
      return;
    }
    const uint64_t t0 = now_ticks();
    while (load(p) < target) {
      if ((int64_t)(now_ticks() - t0) > d.budget) {
        if (lane == 0) __hip_atomic_fetch_add(d.dbg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // Producer side.
  __device__ __forceinline__ static void acquire(int slot, uint32_t use, int lane) {
    spin_until(word(slot, kEmpty), handoff_acquire_target(use) + handoff_debug().force, lane);
  }
  // Publishes the caller's stores of the tile: the workgroup-scope release
  // fence orders them before the count.  (The waves of a workgroup share
  // the compute unit's path to memory, so outside tgsplit mode this fence
  // compiles to no wait at all: the stores may still be in flight.)
  // With a debug header, returns the ring's occupancy right after this
  // commit -- the tiles all waves have committed minus the tiles all waves
  // have released, over both slots -- and keeps the largest in the header;
  // else 0.
  __device__ __forceinline__ static uint32_t commit(int slot, int tile_id, int wave, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) {
      if (wave == 0) __atomic_store_n(word(slot, kTileId), (uint32_t)tile_id, __ATOMIC_RELAXED);
      __atomic_fetch_add(word(slot, kFull), 1u, __ATOMIC_RELAXED);
    }
    uint32_t* dbg = handoff_debug().dbg;
    if (dbg == nullptr) return 0;
    uint32_t occ = 0;
#pragma unroll
    for (int s = 0; s < kHandoffSlots; ++s)
      occ += handoff_slot_occupancy(load(word(s, kFull)), load(word(s, kEmpty)));
    if (lane == 0) __hip_atomic_fetch_max(dbg + 1, occ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return occ;
  }
  // Consumer side.  Returns the committed tile's id; the acquire fence keeps
  // the consumer's reads of the tile after the observed commit.
  __device__ __forceinline__ static int wait(int slot, uint32_t use, int lane) {
    spin_until(word(slot, kFull), handoff_wait_target(use), lane);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return (int)load(word(slot, kTileId));
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

// Row maxima are tracked as keys of the bf16 codes: the 16-bit order key
// (a negative value's magnitude bits flipped, so that signed comparison
// orders the values with -0 < +0), plus 0x7F with 16-bit wrap-around.  The
// shift moves the NaN codes, whose keys sit just above +inf and just below
// -inf, below the key of -inf, so a plain signed maximum skips them; every
// other key keeps its order.  kNoKey lies below every key (columns past N).
constexpr int32_t kNoKey = -32768;
constexpr int32_t kKeyNegInf = -32514;  // key of -inf (code 0xFF80)

__device__ __forceinline__ int32_t max_key(uint32_t code) {
  const uint32_t k = code ^ ((0u - (code >> 15)) & 0x7FFFu);
  return (int32_t)(int16_t)(uint16_t)(k + 0x7Fu);
}
// The keys of the two bf16 codes in a 32-bit word, one per 16-bit half.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 max_keys2(uint32_t w) {
  const s16x2 x = __builtin_bit_cast(s16x2, w);
  const s16x2 neg = x >> 15;  // 0 or -1 per half
  const s16x2 flip = {0x7FFF, 0x7FFF};
  const s16x2 shift = {0x7F, 0x7F};
  return (x ^ (neg & flip)) + shift;
}
// The value a key stands for; -inf when no value was a number.
__device__ __forceinline__ float max_key_value(int32_t key) {
  if (key < kKeyNegInf) return -__builtin_inff();
  const uint32_t k = (uint32_t)(key - 0x7F) & 0xFFFFu;
  return __uint_as_float((k ^ ((0u - (k >> 15)) & 0x7FFFu)) << 16);
}

// The value of lane 0 as a wave-uniform one.  The consumer's counters and
// flags are the same in every lane; saying so keeps them in SGPRs and their
// branches scalar (the compiler cannot prove it through the hand-off ring's
// LDS loads and the K loop's phis, and otherwise keeps them in VGPRs with
// EXEC-masked branches).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// One wave's share of the consumer work on one tile: rows 64w .. 64w+63.
//
// The row statistics are folded right after the tile's commit, from the
// tile as the epilogue left it staged in LDS, one row per lane: lane L folds
// row 64 w + L alone, column after column.  The 16 rows that one read touches at the staging area's
// 272-byte pitch hit every bank once.  The statistics leave with one store
// per array (64 lanes, one entry each).
//
// The copy goes by steps of two rows: step j covers rows 64w + 2j (lanes
// 0-31) and 64w + 2j + 1 (lanes 32-63); lane l takes the 16 bytes (8
// columns) 8 (l % 32) .. + 7 of its row, so every store writes two whole
// 512-byte rows -- the memory pipeline sees 2 long segments per instruction
// instead of 64 short ones.  The staged schedule copies all 32 steps at
// once from the staged tile.  The overlapped one copies inside the next
// tile's K loop, one step per iteration, fetching the tile back from D:
//   iteration i:   fetch step j with an LDS-DMA load into one of the wave's
//                  landing slots (after the barrier, before the stage loads);
//   iteration i+1: after its barrier -- whose wait covered the fetch -- read
//                  the landing slot back;
//   iteration i+2: after its barrier, store the copy.
// Going through LDS keeps every wait explicit: the compiler never sees an
// outstanding load, so it never answers one with a vmcnt(0) that would also
// drain the ring.  Steps the K loop did not reach are finished after the
// next tile's commit (drain), kConsumerDepth at a time through the landing
// slots (the staging area then holds the next tile, which its row
// statistics still need); the drain also releases the slot.  The
// workgroup's last tile has no K loop after it and is copied from its
// staging area.
struct TileConsumer {
  static constexpr bool kLoadsC = false;        // the epilogue loads C itself
  __device__ __forceinline__ void c_load(const KernelArgs&, int, int, uint32_t, int) {}
  static constexpr int kSteps = kWaveTile / 4;  // 64 rows per wave, 2 per step: 32
  // Buffer resources from the tile's origin: D (fetch) and D_copy (store)
  // share their layout, so one offset serves both; the statistics have one
  // 4-byte entry per row.  Out-of-range offsets read zeros and drop stores,
  // which is how rows and columns outside the matrix are masked.
  __amdgpu_buffer_rsrc_t src, cpy, rsum, rmax;
  uint32_t lane_off;            // byte offset of this lane's 16 bytes in step 0
  uint32_t step_bytes;          // two rows of D
  uint32_t stat_lane_off;       // byte offset of the statistics entry of row 64 w + lane
  int row0;                     // this lane's row within the tile in step 0
  int rows;                     // valid rows of the tile
  int ncols;                    // valid columns of the tile
  int fetched;                  // copy steps fetched so far
  int read;                     // copy steps read back so far
  int slot;
  bool active;                  // copy steps of this tile remain to be stored
  bool finished;                // all steps stored; the slot waits for its release (overlapped)
  bool pending;                 // step pend_j is read back and waits for its store
  int pend_j;
  u32x4 v;                      // the pending step's 16 bytes

  __device__ __forceinline__ void idle() {
    active = false;
    finished = false;
    pending = false;
  }

  __device__ __forceinline__ static uint32_t landing(int wave, int c) {
    static_assert((kConsumerDepth & (kConsumerDepth - 1)) == 0, "landing slots are indexed with a mask");
    return kConsumerSlotOffset + (wave * kConsumerDepth + (c & (kConsumerDepth - 1))) * kConsumerSlotBytes;
  }
  // Wait for the use-th commit of `slot` (the workgroup's seq-th tile), then
  // set up this lane's share.
  __device__ __forceinline__ void begin(const KernelArgs& a, int slot_, uint32_t use, int seq,
                                        int wave, int lane) {
    // The lane id as a value the compiler cannot see through: the per-lane
    // offsets below are then computed here, per tile, instead of once at the
    // kernel's start and kept across the K loops in scratch (each reload a
    // round trip to memory that waits behind every load in flight).
    asm volatile("" : "+v"(lane));
    slot = slot_;
    const int tile_id = uni(HandoffRing::wait(slot, use, lane));
    uint64_t* rec = trace_record(seq, wave);
    trace_put(rec, kEvWaitDone, now_ticks(), lane);
    if (lane == 0) *rec_slot(wave) = reinterpret_cast<uint64_t>(rec);
    const TileCoord t = tile_of(tile_id, a);
    const KernelArgs ab = batch_args(a, t.l);
    const int64_t r0 = (int64_t)t.tm * kTileM;
    const int64_t c0 = (int64_t)t.tn * kTileN;
    const int64_t rleft = a.M - r0, cleft = a.N - c0;
    rows = uni((int)(rleft < kTileM ? rleft : kTileM));
    ncols = uni((int)(cleft < kTileN ? cleft : kTileN));
    row0 = wave * 64 + (lane >> 5);
    const int col = 8 * (lane & 31);
    int64_t bytes = ((a.M - 1 - r0) * a.ldd + (a.N - c0)) * 2;
    bytes = (bytes + 15) & ~(int64_t)15;  // per-dword range checks: see StageLoader::stage_rsrc
    const uint32_t nb = (uint32_t)(bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
    src = make_rsrc(static_cast<const unsigned short*>(ab.D) + r0 * a.ldd + c0, nb);
    cpy = make_rsrc(static_cast<const unsigned short*>(ab.D_copy) + r0 * a.ldd + c0, nb);
    // Statistics of batch l: rows l*M .. l*M + M-1 of an (L*M) x stat_ld array.
    const int64_t srow0 = (int64_t)t.l * a.M + r0;
    const int64_t s0 = srow0 * a.stat_ld + t.tn;
    int64_t sbytes = ((int64_t)t.l * a.M + a.M) * a.stat_ld * 4 - s0 * 4;
    sbytes = sbytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : sbytes;
    rsum = make_rsrc(a.row_sum + s0, (uint32_t)sbytes);
    rmax = make_rsrc(a.row_max + s0, (uint32_t)sbytes);
    lane_off = col < ncols ? (uint32_t)((row0 * a.ldd + col) * 2) : kOobOffset;
    step_bytes = (uint32_t)(2 * a.ldd * 2);
    const int srow = wave * 64 + lane;
    stat_lane_off = srow < rows ? (uint32_t)(srow * a.stat_ld * 4) : kOobOffset;
    // Opaque from here on: otherwise the compiler folds `lane_off + j *
    // step_bytes` back into the 64-bit formula they came from and keeps its
    // 64-bit parts live across the K loop (spilled, and a scratch reload in
    // the loop waits for every stage load in flight).
    asm volatile("" : "+v"(lane_off), "+v"(stat_lane_off));
    asm volatile("" : "+s"(step_bytes));
    fetched = 0;
    read = 0;
    active = true;
    pending = false;
  }

  // This lane's offset (from `base`, per step `step`) for step j, or an
  // out-of-range one when the step's row is past the tile's last.
  // (A select, not a branch: `&` rather than `&&`.)
  __device__ __forceinline__ uint32_t at(uint32_t base, uint32_t step, int j) const {
    const bool ok = (base != kOobOffset) & (row0 + 2 * j < rows);
    return ok ? base + (uint32_t)j * step : kOobOffset;
  }

  // Where the epilogue left this lane's 16 bytes of copy step j: wave q
  // staged the quarter of rows 128 (q / 2) .. + 127 and columns 128 (q % 2)
  // .. + 127, row by row at kStagingRowBytes.
  __device__ __forceinline__ static uint32_t staged_at(int wave, int lane, int j) {
    const int row = wave * 64 + 2 * j + (lane >> 5);
    const int col = 8 * (lane & 31);
    const int q = 2 * (row >> 7) + (col >> 7);
    return q * kStagingWaveBytes + (row & 127) * kStagingRowBytes + (col & 127) * 2;
  }

  // Adds a chunk of 8 columns to a row's running sum, one column at a time in
  // column order, and to its running maximum key.  n = the chunk's valid
  // columns from its first (n >= 8 whenever the tile is whole); columns past
  // N are left out of both.
  __device__ __forceinline__ void fold_chunk(const u32x4& x, int n, float& s, int32_t& mk) const {
    if (__builtin_expect(ncols == kTileN, 1)) {
      // A whole row slice: no column checks; the maximum on both halves
      // of each word at once.
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s = s + bf16_lo(x[w]);
        s = s + bf16_hi(x[w]);
      }
      s16x2 m2 = max_keys2(x[0]);
#pragma unroll
      for (int w = 1; w < 4; ++w) m2 = __builtin_elementwise_max(m2, max_keys2(x[w]));
      mk = max(mk, max((int32_t)m2.x, (int32_t)m2.y));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
        if (e < n) {
          s = s + __uint_as_float(h << 16);
          mk = max(mk, max_key(h));
        }
      }
    }
  }

  // The row statistics of the tile the epilogue has just staged (every wave
  // staged its quarter, and the ring is refilled only after the caller's
  // next barrier; the wait in begin() saw all four waves commit, which
  // orders their staging writes before these reads).  Lane L folds row
  // 64 w + L: s = +0.0f, then s = s + x_j for j = 0, 1, ..., in column order.
  __device__ __forceinline__ void fold_staged(int wave, int lane) {
    asm volatile("" : "+v"(lane));  // (as in begin)
    const int row = wave * 64 + lane;
    const uint32_t base = 2 * (row >> 7) * kStagingWaveBytes + (row & 127) * kStagingRowBytes;
    constexpr int kChunks = kTileN / 8;
    float s = 0.0f;
    int32_t mk = kNoKey;
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const u32x4 x = *(const MIGEMM_LDS u32x4*)lds_at(
          base + (k / (kChunks / 2)) * kStagingWaveBytes + (k % (kChunks / 2)) * 16);
      fold_chunk(x, ncols - 8 * k, s, mk);
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), rsum, stat_lane_off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(max_key_value(mk)), rmax,
                                          stat_lane_off, 0, 0);
  }

  // The copy of step j (16 bytes per lane).
  __device__ __forceinline__ void store_copy(const u32x4& x, int j, int lane) const {
    const uint32_t o = at(lane_off, step_bytes, j);
    if (__builtin_expect(ncols == kTileN, 1)) {
      __builtin_amdgcn_raw_buffer_store_b128(x, cpy, o, 0, kCpolNt);
    } else {
      // A tile cut short by N: column by column, past-N ones out of range.
      const int n = ncols - 8 * (lane & 31);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(x[e >> 1] >> (16 * (e & 1))), cpy,
                                              e < n ? o + 2 * e : kOobOffset, 0, 0);
    }
  }

  // A trace event of the tile this wave's consumer works on.
  __device__ __forceinline__ static void cons_trace(int word, int wave, int lane) {
    trace_put(rec_of(wave), word, now_ticks(), lane);
  }

  // Releases the tile's slot.  The tile's reads all completed before their
  // values were stored.
  __device__ __forceinline__ void release(int wave, int lane) {
    finished = false;
    cons_trace(kEvReleased, wave, lane);
    HandoffRing::release(slot, lane);
  }

  // Staged schedule (and the overlapped one's last tile): the copy steps
  // kCopyBatch at a time from the staged tile, then the release.
  static constexpr int kCopyBatch = 8;
  __device__ __forceinline__ void copy_staged(int wave, int lane) {
    static_assert(kSteps % kCopyBatch == 0, "whole batches of steps");
    asm volatile("" : "+v"(lane));  // (as in begin)
    if (!uni(active)) return;
    for (int j0 = 0; j0 < kSteps; j0 += kCopyBatch) {
      u32x4 x[kCopyBatch];
#pragma unroll
      for (int q = 0; q < kCopyBatch; ++q)
        x[q] = *(const MIGEMM_LDS u32x4*)lds_at(staged_at(wave, lane, j0 + q));
#pragma unroll
      for (int q = 0; q < kCopyBatch; ++q) store_copy(x[q], j0 + q, lane);
      if (j0 == 0) cons_trace(kEvCopyFirst, wave, lane);
    }
    cons_trace(kEvCopyLast, wave, lane);
    fetched = read = kSteps;
    active = false;
    release(wave, lane);
  }

  // Overlapped schedule.
  __device__ __forceinline__ void fetch(int wave) {
    const int j = uni(fetched);
    fetched = j + 1;
    dma16_w5_nt(src, lds_at(landing(wave, j)), at(lane_off, step_bytes, j));
  }
  // Read step `read` back from LDS at `slot` (its fetch must have completed).
  __device__ __forceinline__ void read_back_at(uint32_t slot_at, int lane) {
    compiler_fence();
    pend_j = uni(read);
    read = pend_j + 1;
    v = *(const MIGEMM_LDS u32x4*)lds_at(slot_at + 16 * lane);
    pending = true;
  }
  // Store the pending step's copy.  After the tile's last step the tile is
  // finished; its slot is released by the drain that follows the next
  // tile's commit.
  __device__ __forceinline__ void store_pending(int wave, int lane) {
    if (!uni(pending)) return;
    pending = false;
    const int j = uni(pend_j);
    store_copy(v, j, lane);
    if (j == 0) cons_trace(kEvCopyFirst, wave, lane);
    if (j == kSteps - 1) {
      cons_trace(kEvCopyLast, wave, lane);
      active = false;
      finished = true;
    }
  }

  // K-loop hook, right after the barrier.
  __device__ __forceinline__ void after_barrier(const KernelArgs& a, int wave, int lane) {
    (void)a;
    store_pending(wave, lane);
    if (!uni(active)) return;
    if (uni(fetched) > uni(read)) read_back_at(landing(wave, uni(read)), lane);
    if (uni(fetched) < kSteps) fetch(wave);
  }
  // After the next tile's commit: the copy steps the K loop did not finish,
  // then the release.  A step fetched by the loop but not yet read back is
  // still in its landing slot (landed: the loop ended with vmcnt(0) and a
  // barrier).  The rest go kConsumerDepth at a time through the landing
  // slots: the staging area now holds the next tile, whose row statistics
  // every wave still reads from it.
  __device__ __forceinline__ void drain(int wave, int lane) {
    asm volatile("" : "+v"(lane));  // (as in begin: lane offsets computed here, not spilled)
    store_pending(wave, lane);
    if (uni(active)) {
      while (uni(read) < uni(fetched)) {
        read_back_at(landing(wave, uni(read)), lane);
        store_pending(wave, lane);
      }
      while (uni(active)) {
        wait_lgkmcnt<0>();  // the landing slots' earlier read-backs have returned
        const int f0 = uni(fetched);
        const int n = kSteps - f0 < kConsumerDepth ? kSteps - f0 : kConsumerDepth;
        for (int i = 0; i < n; ++i) fetch(wave);
        wait_vmcnt<0>();
        for (int i = 0; i < n; ++i) {
          read_back_at(landing(wave, uni(read)), lane);
          store_pending(wave, lane);
        }
      }
    }
    if (uni(finished)) release(wave, lane);
  }
};

}  // namespace migemm
