/*
 * migemm.h -- C ABI of a persistent, tile-scheduled, pipelined GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 *   D = alpha * A * B + beta * C          (fp32 accumulation, bf16 D)
 *
 * A is M x K, B is K x N, C and D are M x N.  A and B are both bf16, or both
 * OCP fp8 e4m3 ("fn": largest finite 448, no infinities); C and D are bf16.
 *
 * The operation and its interface shape follow the CUTLASS SM90 "TMA warp-
 * specialized cooperative" GEMM kernel page: an MNK problem shape, separate
 * element types and strides for A, B, C and D, an epilogue that forms
 * alpha * accumulator + beta * C (the source C is loaded only when it is
 * needed), a feasibility check before launch (can_implement), a caller-owned
 * workspace with a size query, and a persistent grid sized from the device's
 * compute-unit count.  The tile hand-off of gemm_run_with_tile_consumer is the
 * producer acquire/commit and consumer wait/release protocol that CUTLASS
 * issue #2900 ("How to build a pipeline between epilogue and communication
 * warp groups?") asks for, so that a consumer stage can work on each finished
 * output tile; with MIGEMM_F_CONSUMER_OVERLAP it does so while the next
 * tile's main loop runs.
 *
 * Conventions shared by every entry point:
 *   - all sizes and strides are int64_t; strides are in ELEMENTS;
 *   - element (r, c) of an operand X is at X + r * x_rs + c * x_cs;
 *   - every device pointer is owned by the caller; the library never
 *     allocates device memory, never frees, and never synchronizes a stream;
 *   - a plan owns host memory only and is immutable after creation; one plan
 *     may be run concurrently on several streams; every entry point taking a
 *     plan first checks that it is live (created and not yet destroyed) and
 *     gives MIGEMM_ERR_INVALID_ARG otherwise, without reading it;
 *   - every call returns a migemm_status (0 = OK, negative = error) and never
 *     throws.  Argument, device and alignment errors are found before
 *     anything is launched; a launch failure reported by the HIP runtime gives
 *     MIGEMM_ERR_LAUNCH; a fault inside a kernel surfaces at the caller's next
 *     synchronization, as for any HIP kernel.
 */
#ifndef MIGEMM_H
#define MIGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (the pages keep ElementA/B/C/D separate). */
typedef enum migemm_dtype {
  MIGEMM_BF16 = 1,
  MIGEMM_FP8_E4M3 = 2
} migemm_dtype;

typedef enum migemm_status {
  MIGEMM_OK = 0,
  MIGEMM_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, bad stride, C NULL with beta != 0 */
  MIGEMM_ERR_UNSUPPORTED = -2, /* valid request this library does not implement (see below) */
  MIGEMM_ERR_MISALIGNED = -3,  /* a base pointer or leading stride is not 16-byte aligned */
  MIGEMM_ERR_DEVICE = -4,      /* no HIP device, wrong ordinal, or not gfx950 */
  MIGEMM_ERR_LAUNCH = -5,      /* the HIP runtime rejected the kernel launch */
  MIGEMM_ERR_TIMEOUT = -6,     /* a bounded hand-off wait expired (MIGEMM_F_HANDOFF_DEBUG) */
  MIGEMM_ERR_SCRATCH = -7      /* gemm_run_no_alloc: the plan needs more workspace than
                                  MIGEMM_NO_ALLOC_SCRATCH_BYTES */
} migemm_status;

/* Plan flags. */
#define MIGEMM_F_TILE_CONSUMER 0x1u /* plan may run gemm_run_with_tile_consumer */
/* Stream-K (the kernel page's stream-K scheduler and fixup): the tiles of the
 * last round are cut into K ranges shared by every workgroup, so that no
 * compute unit idles while others finish whole tiles; the partial sums of a
 * split tile are added through the workspace.  gemm_run only (UNSUPPORTED
 * with MIGEMM_F_TILE_CONSUMER).  MIGEMM_F_STREAM_K lets the plan choose it
 * where its cost model predicts a gain (moving the partials costs about as
 * much as 24 K stages of MFMA work); MIGEMM_F_STREAM_K_FORCE uses it whenever
 * K > 0.  gemm_plan_get_info reports the choice (stream_k_tiles). */
#define MIGEMM_F_STREAM_K 0x2u
#define MIGEMM_F_STREAM_K_FORCE 0x4u
/* With MIGEMM_F_TILE_CONSUMER (else INVALID_ARG): copy each tile to D_copy
 * inside the next tile's main loop, fetching it back from D, instead of right
 * after the tile's commit from the tile still staged in LDS (the row
 * statistics are folded right after the commit either way).  Same results
 * bit for bit.  The overlap is CUTLASS issue #2900's goal -- consumer work
 * running while the MMA waves start the next tile -- but here the consumer
 * work shares the MMA waves, and in the K loop it costs more than it does
 * on its own (about 2.5% of the 8192^3 bf16 kernel's time).  It is the form
 * for consumer work that waits on long transfers rather than computing. */
#define MIGEMM_F_CONSUMER_OVERLAP 0x8u
/* With MIGEMM_F_TILE_CONSUMER (else INVALID_ARG): debugging of the hand-off
 * ring.  gemm_plan_workspace_size then includes a debug area, which every
 * run (gemm_run too) needs and gemm_workspace_init zeroes:
 *   - each ring wait (acquire, wait) is bounded: after debug_wait_ticks of
 *     the device's 100 MHz real-time clock (0: 10^8, one second) it gives
 *     up, is counted, and the kernel goes on, so it always ends;
 *     gemm_debug_read then reports MIGEMM_ERR_TIMEOUT (results may be wrong);
 *   - every wave writes a trace record per tile of its workgroup: the clock
 *     at each step of the protocol and the ring's occupancy at its commit
 *     (migemm_debug_info describes the layout).
 * debug_force_wait > 0 adds that much to every acquire's target: a wait
 * that cannot pass, for testing the bounded wait itself. */
#define MIGEMM_F_HANDOFF_DEBUG 0x10u
/* Where gemm_run reads C (beta != 0).  With this flag: in the epilogue, after
 * the tile's K loop.  Without it, a plan whose workgroups each take one round
 * of whole tiles (tiles <= grid, not stream-K, K at least two stages) reads C
 * into LDS during the K loop's last two iterations, as the ring's slots fall
 * free -- the kernel page's separate C-load role, here taken by the MMA
 * waves -- so that half the read overlaps the last stages' MFMAs instead of
 * waiting in the epilogue; other plans read it in the epilogue.  The tile
 * consumer always reads C in the epilogue.  gemm_plan_get_info reports the
 * choice (c_in_k_loop).  Same results bit for bit either way. */
#define MIGEMM_F_C_IN_EPILOGUE 0x20u
/* Output tile height (the kernel page's tile shape, a compile-time choice
 * there; here two kernels).  Plans take 256 x 256 tiles, except that a
 * bf16 plan without MIGEMM_F_TILE_CONSUMER may take 192 x 256 tiles where
 * that gives each persistent workgroup less work: with T tiles on G
 * workgroups the work is ceil(T / G) tiles, and a 192-row tile takes about
 * 0.8 of a 256-row one's time (3/4 of the flops at a slightly lower rate),
 * so a problem whose 256-row tiles leave a poorly filled last round (8192 x
 * 1024: 128 tiles on 256 compute units) runs 4/3 as many smaller tiles in
 * one round.  With MIGEMM_F_STREAM_K the plan compares against stream-K too.  MIGEMM_F_TILE_M256 keeps 256 rows;
 * MIGEMM_F_TILE_M192 forces 192 (bf16 only, else UNSUPPORTED; INVALID_ARG
 * with MIGEMM_F_TILE_M256, MIGEMM_F_TILE_CONSUMER or a stream-K flag).  A
 * 192-row plan reads C (beta != 0) in the epilogue.  gemm_plan_get_info
 * reports the choice (tile_m, tiles_m).  Same results bit for bit either
 * way: each output's sum runs over K in the same order. */
#define MIGEMM_F_TILE_M256 0x40u
#define MIGEMM_F_TILE_M192 0x80u

/* Output tile of the persistent scheduler (and the hand-off unit); a plan
 * may report tile_m 192 instead (MIGEMM_F_TILE_M192). */
#define MIGEMM_TILE_M 256
#define MIGEMM_TILE_N 256

/*
 * Problem description (the pages' Arguments: problem shape, element types,
 * strides, hardware info).
 *
 * Layout rules checked by gemm_desc_validate:
 *   - M, N, K >= 0;
 *   - type pairs: (A, B, C, D) = (BF16, BF16, BF16, BF16) or
 *     (FP8_E4M3, FP8_E4M3, BF16, BF16);
 *   - each of A, B, C, D has exactly one unit stride, and its other stride
 *     is at least the extent of the contiguous dimension;
 *   - the non-unit stride times the element size is a multiple of 16 bytes
 *     (K itself may be anything, in every layout); a multiple of 128 bytes
 *     (64 bf16, 128 e4m3) runs faster: the kernels read 128-byte row
 *     segments, which then each fall in one cache line (4000 x 3000 x 5000
 *     bf16 with rows of 10000 and 6000 bytes: 9% slower than with 10112
 *     and 6144);
 *   - C and D have the same orientation (both row-major or both column-
 *     major); a column-major D is computed as D^T = B^T A^T;
 *   - the tile-consumer flag requires a row-major D;
 *   - the byte span of 256 rows (or K rows) of an operand fits in 2^31;
 *   - each operand, with all its batches, spans at most 2^47 bytes (else
 *     UNSUPPORTED; this also rejects strides whose products would wrap);
 *   - batches (the pages' rank-4 problem shape, L appended to MNK): L = 0 or
 *     1 is one product; for L > 1 matrix l of X starts x_bs * l elements
 *     after X, every x_bs >= 0 and x_bs times the element size a multiple of
 *     16 bytes; A, B and C may share a matrix between batches (x_bs = 0), D
 *     may not (d_bs is at least the extent of one D, so batches of D do not
 *     overlap).  The tile consumer's outputs are per batch too: row_sum and
 *     row_max are L x M x ceil(N/256), D_copy uses d_bs.
 * c_* fields are ignored when the caller will always pass beta == 0, but
 * must still describe a valid layout (use the same values as D).
 */
typedef struct migemm_desc {
  int64_t M, N, K;
  int32_t a_type, b_type, c_type, d_type; /* migemm_dtype */
  int64_t a_rs, a_cs;                     /* A: M x K */
  int64_t b_rs, b_cs;                     /* B: K x N */
  int64_t c_rs, c_cs;                     /* C: M x N */
  int64_t d_rs, d_cs;                     /* D: M x N */
  int32_t device;                         /* HIP device ordinal; must be gfx950 */
  uint32_t flags;                         /* MIGEMM_F_* */
  int32_t max_workgroups;                 /* 0: one persistent workgroup per CU;
                                             >0: cap on the persistent grid */
  int32_t reserved;                       /* must be 0 */
  int64_t L;                              /* batch count (0 or 1: one product) */
  int64_t a_bs, b_bs, c_bs, d_bs;         /* batch strides in elements (L > 1) */
  int64_t debug_wait_ticks;               /* MIGEMM_F_HANDOFF_DEBUG: wait budget (0: default) */
  int32_t debug_force_wait;               /* MIGEMM_F_HANDOFF_DEBUG: see there; else 0 */
  int32_t reserved2;                      /* must be 0 */
} migemm_desc;

/* What a plan chose (for tracing and tests). */
typedef struct migemm_plan_info {
  int64_t tiles_m, tiles_n, num_tiles;
  int32_t grid;            /* persistent workgroups launched */
  int32_t block_threads;   /* threads per workgroup (4 waves of 64) */
  int32_t lds_bytes;       /* LDS per workgroup (of the kernel gemm_run launches) */
  int32_t stages;          /* depth of the main-loop LDS ring */
  int32_t tile_m, tile_n, tile_k; /* output tile (tile_m 256, or 192: MIGEMM_F_TILE_M192) and
                                      K per pipeline stage (64 bf16, 128 e4m3) */
  int32_t swapped;         /* 1: column-major D, computed as D^T = B^T A^T */
  int32_t a_kmajor;        /* 1: A (after any swap) is K-contiguous */
  int32_t b_kmajor;        /* 1: B (after any swap) is K-contiguous */
  int32_t cu_count;        /* compute units of the device */
  int32_t handoff_slots;   /* depth of the tile hand-off ring */
  int64_t stream_k_tiles;  /* tiles cut into K ranges (0: every tile is taken whole) */
  int32_t stream_k_units_per_tile; /* K stages (tile_k each) per such tile */
  int32_t c_in_k_loop;     /* 1: with beta != 0, gemm_run reads C in the K loop's last two
                              iterations (else in the epilogue); see MIGEMM_F_C_IN_EPILOGUE */
  int64_t batches;         /* L (1 for one product) */
} migemm_plan_info;

typedef struct migemm_plan migemm_plan; /* opaque, host memory only */

/* Pure host check of a description; needs no device.  Returns MIGEMM_OK or
 * the error code gemm_plan_create would give before its device query.
 * Defined by: the kernel page (sm90_gemm_tma_warpspecialized_cooperative.hpp),
 * can_implement -- may this kernel run these arguments (problem rank,
 * tile-size and alignment rules), answered before any launch. */
int gemm_desc_validate(const migemm_desc* desc);

/* Validate, query the device (must be gfx950), choose the tile configuration
 * and the persistent grid, and return a plan in *out (set to NULL on error).
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED (strides), DEVICE.
 * Defined by: the kernel page (sm90_gemm_tma_warpspecialized_cooperative.hpp),
 * to_underlying_arguments (arguments -> kernel parameters, the persistent
 * grid's size from the device's SM count in hw_info) and get_grid_shape;
 * its device-side guard against the wrong architecture. */
int gemm_plan_create(const migemm_desc* desc, migemm_plan** out);

/* Free a plan (NULL is accepted and does nothing).  A pointer that is not a
 * live plan (destroyed already, or never created) gives INVALID_ARG and
 * frees nothing.  Destroying a plan while another thread is inside a call
 * on it is the caller's error (the liveness check catches stale handles,
 * not such races); runs already enqueued do not need the plan.  Host
 * memory only; the pages have no counterpart (their Params live in the
 * caller's object). */
int gemm_plan_destroy(migemm_plan* plan);

/* Copy the plan's choices into *out (grid, block, tiles, ring depths).
 * Defined by: the kernel page (sm90_gemm_tma_warpspecialized_cooperative.hpp),
 * get_grid_shape and get_block_shape, the launch geometry a caller queries. */
int gemm_plan_get_info(const migemm_plan* plan, migemm_plan_info* out);

/* Bytes of device workspace gemm_run needs.  Defined by: the kernel page
 * (sm90_gemm_tma_warpspecialized_cooperative.hpp), get_workspace_size -- the
 * epilogue's and the tile scheduler's workspace (stream-K partials) summed.
 * Plans without stream-K tiles need none: 0, and `workspace` arguments below
 * may then be NULL.  A stream-K plan needs grid x 512 KiB of fp32 partial
 * tiles (two per workgroup) plus one 32-bit arrival counter per stream-K tile
 * and wave (rounded up to 256 bytes). */
size_t gemm_plan_workspace_size(const migemm_plan* plan);

/* Make `workspace` (gemm_plan_workspace_size(plan) bytes of device memory,
 * 256-byte aligned, owned by the caller) ready for the plan's runs.  Defined
 * by: the kernel page (sm90_gemm_tma_warpspecialized_cooperative.hpp),
 * initialize_workspace on a stream.  Zeroes the arrival counters (and a
 * MIGEMM_F_HANDOFF_DEBUG plan's whole debug area), with a kernel
 * enqueued on `stream` (so it may be captured in a HIP graph).  Every run
 * that completes leaves the counters at zero again; call this before the
 * first run, after a run that did not complete, and before a workspace is
 * used with another plan.  A no-op returning OK when the size is 0.
 * Errors: INVALID_ARG (NULL plan, or NULL workspace with a nonzero size),
 * MISALIGNED, DEVICE (current device is not the plan's), LAUNCH. */
int gemm_workspace_init(const migemm_plan* plan, void* workspace, void* stream);

/* D = alpha*A*B + beta*C, enqueued on `stream` (a hipStream_t; NULL = the
 * null stream).  Defined by: the kernel page
 * (sm90_gemm_tma_warpspecialized_cooperative.hpp), the persistent kernel's
 * body -- each CTA takes output tiles from the tile scheduler, its producer
 * loads K stages into a multi-stage ring that its consumers drain into
 * accumulators, and the epilogue forms alpha * accumulator + beta * C (C
 * loaded only when needed) and stores D.  A, B, D must be non-NULL and 16-byte aligned; C may be NULL
 * only when beta == 0, in which case C is never read (it may hold NaN).
 * With K == 0, D = beta*C.  M == 0 or N == 0 is a no-op.  C may alias D only
 * with identical strides.  Asynchronous: returns once the kernel is queued.
 * `workspace`: NULL when gemm_plan_workspace_size(plan) is 0; otherwise that
 * many bytes, 256-byte aligned, prepared by gemm_workspace_init (else
 * INVALID_ARG / MISALIGNED).  Runs that share a workspace must not overlap
 * in time.  With stream-K the fp32 partial sums of a tile are added in the
 * order of their K ranges, so a plan gives the same D on every run; plans
 * with another grid size can round differently in the last bit. */
int gemm_run(const migemm_plan* plan, const void* A, const void* B, const void* C, void* D,
             float alpha, float beta, void* workspace, void* stream);

/* gemm_run, and in the same kernel a consumer stage fed through a 2-slot
 * tile hand-off ring.  Defined by: CUTLASS issue #2900 ("How to build a
 * pipeline between epilogue and communication warp groups?"), the requested
 * protocol -- producer acquire, store the tile, commit; consumer wait, work
 * on the tile, release -- with the producer's first acquires passing at once
 * (the kernel page starts producer pipeline states at the opposite phase;
 * the CuTe DSL task_scheduling.pipeline page names producer_acquire,
 * producer_commit and consumer_release): every finished 256 x 256 tile of D is committed by the
 * waves that stored it; the consumer work waits for the commit, reads the
 * tile as the epilogue staged it in LDS (with MIGEMM_F_CONSUMER_OVERLAP the
 * copy instead reads it back from D while the next tile's main loop runs),
 * and then releases the slot.  For
 * the tile at tile column t = n / 256 it writes, for each row r of the tile,
 * over the bf16 values x_j = D[r][256t + j] of the columns below N, widened
 * exactly to fp32:
 *   row_sum[r * ceil(N/256) + t] = s, the plain sequential fp32 sum in
 *       ascending column order: s = +0.0f, then s = s + x_j for j = 0, 1, ...
 *       (one rounding per addition),
 *   row_max[r * ceil(N/256) + t] = the largest x_j that is not a NaN, with
 *       -0 < +0 (IEEE 754-2019 maximumNumber); -inf if there is none,
 * and copies the tile bit for bit into D_copy (same strides as D).  Both
 * statistics therefore have exactly one correct value given D.  (The hand-off
 * issue leaves the consumer's work open -- "do something with the tile";
 * these are the statistics this library's consumer stage computes.)
 * row_sum and row_max are M x ceil(N/256) fp32, row-major, 4-byte aligned;
 * D_copy is 16-byte aligned and must not overlap D.  Requires a plan created
 * with MIGEMM_F_TILE_CONSUMER and a row-major D. */
int gemm_run_with_tile_consumer(const migemm_plan* plan, const void* A, const void* B,
                                const void* C, void* D, float alpha, float beta,
                                float* row_sum, float* row_max, void* D_copy,
                                void* workspace, void* stream);

/* What the hand-off debug area of a MIGEMM_F_HANDOFF_DEBUG plan holds.  The
 * trace starts trace_offset bytes into the workspace: for workgroup g
 * (0 .. grid-1), wave w (0 .. waves-1) and the workgroup's n-th tile (0 ..
 * trace_tiles-1), a record of trace_words uint64 at index
 * ((g * waves + w) * trace_tiles + n) * trace_words, holding the device
 * real-time clock (100 MHz) when the wave
 *   [0] began the tile's K loop, [1] ended it, [2] acquired the tile's ring
 *   slot, [3] committed the tile, [4] saw it committed by every wave (its
 *   consumer's wait), [5] stored the tile's first and [6] its last copy
 *   step, [7] released the slot,
 * then [8] the ring's occupancy right after this wave's commit (tiles
 * committed by every wave minus tiles released by every wave, over both
 * slots) and [9] the tile id (records of tiles a workgroup does not have
 * stay zero). */
typedef struct migemm_debug_info {
  uint32_t waits_given_up;     /* bounded waits that expired since the last init */
  uint32_t max_occupancy;      /* largest ring occupancy seen, in tiles */
  int64_t trace_offset;        /* bytes from the workspace to the first record */
  int32_t grid, waves, trace_tiles, trace_words;
} migemm_debug_info;

/* Synchronizes `stream`, then reads the debug header of a
 * MIGEMM_F_HANDOFF_DEBUG plan's workspace into *out.  The waits it reports
 * on are those of the hand-off protocol of CUTLASS issue #2900 (producer
 * acquire, consumer wait), bounded here so that a protocol fault ends as a
 * status rather than a hang.  Returns
 * MIGEMM_ERR_TIMEOUT if a bounded ring wait has given up since the last
 * gemm_workspace_init, else MIGEMM_OK (or INVALID_ARG for a plan without
 * the flag, a NULL argument; DEVICE if the copy fails). */
int gemm_debug_read(const migemm_plan* plan, const void* workspace, void* stream,
                    migemm_debug_info* out);

/* Size of the fixed device scratch of gemm_run_no_alloc: 64 MiB per device. */
#define MIGEMM_NO_ALLOC_SCRATCH_BYTES (64ll << 20)

/* gemm_run for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation with the same plan, but a plan that needs a workspace
 * (stream-K) gets it from a fixed array inside the library instead of from
 * the caller.  The array is MIGEMM_NO_ALLOC_SCRATCH_BYTES of device memory
 * on every device the library runs on, held until the process ends; this
 * call allocates and frees nothing.  A plan whose gemm_plan_workspace_size
 * exceeds it gets MIGEMM_ERR_SCRATCH, with nothing launched (a stream-K plan
 * fits with up to about 120 workgroups; cap it with max_workgroups).  Each
 * call that uses the array first clears its arrival counters with a fill
 * kernel on `stream`.  Every call on one device shares that device's array:
 * calls whose executions overlap in time on one device race (use one stream,
 * or order them), and the array keeps the last call's contents.  Arguments,
 * results and the other errors are those of gemm_run. */
int gemm_run_no_alloc(const migemm_plan* plan, const void* A, const void* B, const void* C,
                      void* D, float alpha, float beta, void* stream);

/* Static text for a status code (never NULL).  No counterpart on the pages. */
const char* gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MIGEMM_H */
