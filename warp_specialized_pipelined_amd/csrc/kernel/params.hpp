// params.hpp -- the argument block every GEMM kernel receives, and the
// compile-time tile geometry.  Shared by host and device code.
#pragma once

#include <stdint.h>

namespace migemm {

// Output tile 256 x 256, 4 waves per workgroup as a 2 x 2 grid of 128 x 128
// wave tiles, one persistent workgroup per compute unit.
constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveTile = 128;
// The other tile height, for bf16 whole tiles without the tile consumer:
// 192 x 256, wave tiles of 96 x 128 (the plan chooses; gemm_kernel_m192).
constexpr int kTileMShort = 192;
// Each stage of the K-loop ring holds 128 bytes of K (64 bf16 or 128 e4m3
// values) for every row of the A and B tiles: 32 KiB of A + 32 KiB of B.
// Stage s lives in slot s % kStages of the LDS ring.
constexpr int kStageKBytes = 128;
constexpr int kOperandStageBytes = kTileM * kStageKBytes;  // 32 KiB
constexpr int kStageBytes = 2 * kOperandStageBytes;        // 64 KiB
constexpr int kStages = 2;                                 // LDS ring depth
constexpr int kRingBytes = kStages * kStageBytes;          // 128 KiB
constexpr int kLdsLimit = 160 * 1024;                      // LDS per workgroup on gfx950
// Epilogue staging: each wave's 128 x 128 bf16 quarter of the tile, rows
// padded from 256 to 272 bytes so that consecutive rows start 4 banks apart.
// It overlays the (then idle) ring and runs a little past it.
constexpr int kStagingRowBytes = kWaveTile * 2 + 16;                 // 272
constexpr int kStagingWaveBytes = kWaveTile * kStagingRowBytes;      // 34816
constexpr int kStagingBytes = kWaves * kStagingWaveBytes;            // 139264
constexpr int kPlainLdsBytes = kStagingBytes > kRingBytes ? kStagingBytes : kRingBytes;
// Consumer-stage landing slots (overlapped consumer): per wave
// kConsumerDepth slots of 1 KiB (16 bytes per lane), past both the ring and
// the staging area.  The consumer
// fetches while the K loop runs (so the slots must not overlap the ring),
// and one wave may still be draining its consumer work while another
// already stages its epilogue (so they must not overlap the staging either).
constexpr int kConsumerDepth = 4;
constexpr int kConsumerSlotOffset = kPlainLdsBytes;
constexpr int kConsumerSlotBytes = 64 * 16;
constexpr int kConsumerEnd = kConsumerSlotOffset + kWaves * kConsumerDepth * kConsumerSlotBytes;
// How a kernel runs the tile consumer stage: not at all; right after the
// tile's commit, on the tile as the epilogue staged it in LDS; or inside the
// next tile's K loop, fetching the tile back from D.
enum ConsumerMode { kConsNone = 0, kConsStaged = 1, kConsOverlap = 2 };
// Tile hand-off ring: two slots of {tile id, full count, empty count}.
// After the slots: the hand-off debug block (debug header and trace
// pointers, wait budget, forced wait, trace records per wave) and each
// wave's trace record pointer for the tile its consumer works on, kept in
// LDS rather than in registers across the K loop.
constexpr int kHandoffSlots = 2;
constexpr int kHandoffOffset = kConsumerEnd;
constexpr int kHandoffDebugOffset = kHandoffOffset + 32;
constexpr int kHandoffRecOffset = kHandoffOffset + 64;
constexpr int kHandoffBytes = 128;
constexpr int kConsumerLdsBytes = kHandoffOffset + kHandoffBytes;     // 155776
static_assert(kConsumerLdsBytes <= kLdsLimit, "consumer kernel LDS exceeds 160 KiB");

struct KernelArgs {
  const void* A;       // operand storage (after any swap of A and B)
  const void* B;
  const void* C;       // NULL when beta == 0
  void* D;
  float* row_sum;      // consumer outputs (tile-consumer kernels only)
  float* row_max;
  void* D_copy;
  int64_t M, N, K;
  int64_t lda, ldb;    // the non-unit stride of A and B, in elements
  int64_t ldc, ldd;    // row strides of C and D (row-major after any swap)
  int64_t a_bytes;     // byte extent of A and B as described by the strides
  int64_t b_bytes;
  float alpha, beta;
  int32_t tiles_m, tiles_n, num_tiles;
  int32_t group_m;     // tile rows per raster group
  int32_t stat_ld;     // ceil(N / 256): leading dimension of row_sum/row_max
  // Stream-K (stream-K kernels only; scheduler.hpp): tiles [sk_first,
  // num_tiles) are cut into K-stage units shared out over the grid.
  int32_t sk_first;    // first stream-K tile
  int32_t sk_kt;       // K stages (units) per tile
  float* sk_partials;  // workspace: kSkPartialSlots fp32 partial tiles per workgroup
  uint32_t* sk_arrivals;  // workspace: per stream-K tile and wave, zero between runs
  // Batches: tiles are numbered batch after batch (tiles_per_batch each);
  // matrix l of an operand starts l * stride bytes after its pointer.
  int32_t tiles_per_batch;
  int32_t c_preload;   // beta != 0: load C in the K loop's last two iterations (CPreload)
  int64_t a_bs_bytes, b_bs_bytes, c_bs_bytes, d_bs_bytes;
  // Hand-off debugging (tile-consumer kernels; all zero when off): a header
  // in the workspace ([0] ring waits that gave up, [1] the largest ring
  // occupancy seen, in tiles), then kTraceWords 64-bit words per wave
  // and tile of each workgroup (handoff.hpp), and the budget of a ring wait.
  uint32_t* dbg;
  uint64_t* trace;
  int64_t spin_budget;     // s_memrealtime ticks (100 MHz) a ring wait may spin
  int32_t trace_tiles;     // trace records per wave: ceil(tiles / grid)
  int32_t force_wait;      // added to every acquire's target: a wait that cannot pass
};

// Hand-off debugging: the workspace's header, and the trace record of one
// wave and tile (64-bit words; which word holds what: handoff.hpp).
constexpr int kDebugHeaderBytes = 256;
constexpr int kTraceWords = 16;

// Stream-K workspace: per workgroup, one partial tile for the segment its
// unit range starts in and one for the segment it ends in.
constexpr int kSkPartialSlots = 2;
constexpr int64_t kSkPartialBytes = (int64_t)kTileM * kTileN * 4;  // fp32 tile: 256 KiB

// The fixed device scratch of the entry point that allocates nothing: room
// for the stream-K workspace of a plan with up to about 120 workgroups.
constexpr int64_t kNoAllocScratchBytes = 64ll << 20;

}  // namespace migemm
