// epilogue.hpp -- D = alpha * acc + beta * C in fp32, rounded to bf16
// (nearest even), staged through LDS and stored to a row-major D with
// 16-byte stores.
//
// The pages' epilogue copies accumulators to registers, converts them to the
// output type, writes them to a shared-memory staging buffer, synchronizes,
// and then copies whole rows of the staged tile out to global memory; it
// reads the source C only when the epilogue needs it (CuTe DSL persistent GEMM
// epilogue quoted in CUTLASS issue #2900; kernel page: is_producer_load_needed
// and collective_epilogue.store).
//
// Here each wave stages its own 128 x 128 quarter of the tile as bf16 in a
// slice of the (now idle) main-loop ring:
//   - with the (B^T A^T) block orientation of the main loop a lane holds four
//     consecutive columns of one row per group of four accumulators, so the
//     staging writes are 8-byte ds_write_b64 (lanes l and l+32 fill one
//     16-byte chunk of a row);
//   - staged rows are padded to 272 bytes, which puts consecutive rows 4 banks
//     apart: the 32 rows one write touches and the 4 rows one read touches
//     spread over all banks, and every address is a per-lane base plus a
//     constant, so it folds into the instruction's offset field;
//   - read back, one ds_read_b128 per lane covers 4 full 256-byte rows, which
//     leave as coalesced 16-byte buffer stores.
// C (when beta != 0) first lands in the wave's staging area, in the staging
// layout, through LDS-DMA loads of whole row segments; each lane then reads
// its 8 bytes of C at the place its result goes, so alpha*acc + beta*C is
// formed in fp32, rounded once, and written over that C.
#pragma once

#include "gfx950.hpp"
#include "mainloop.hpp"
#include "params.hpp"

namespace migemm {

// A buffer resource over a row-major bf16 matrix, starting at (r0, c0).
// round16: extend the range to the end of the last 16-byte block (for reads;
// range checks work per dword, see StageLoader::stage_rsrc).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t matrix_rsrc(const void* base, int64_t ld,
                                                              int64_t rows, int64_t cols,
                                                              int64_t r0, int64_t c0, bool round16) {
  const unsigned short* p = static_cast<const unsigned short*>(base) + r0 * ld + c0;
  int64_t bytes = (r0 < rows && c0 < cols) ? ((rows - 1 - r0) * ld + (cols - c0)) * 2 : 0;
  if (round16) bytes = (bytes + 15) & ~(int64_t)15;
  bytes = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes;
  return make_rsrc(p, (uint32_t)bytes);
}

// The source C, read inside the K loop (beta != 0; whole-tile kernels
// without the tile consumer).  The kernel page gives the epilogue's source
// its own load role -- a producer warp with its own pipeline, started after
// the mainloop load warp's first stage by a load-order barrier -- so that
// C's read overlaps the mainloop instead of stalling the epilogue.  Every
// wave here is an MMA wave and LDS holds no C tile beside the ring, so the
// C-load role takes the ring's two slots as they fall free in the tile's
// last two K iterations (mainloop_range) and loads C straight into the
// epilogue's staging layout: the epilogue then finds it in place.  Ordered
// after the mainloop's loads by the same barriers that order the ring.
// Measured without it: reading C in the epilogue added 8.5% to a 4096^3
// GEMM and 20% to 4096 x 4096 x 1024, every compute unit reading its C at
// the same moment.
struct CPreload {
  static constexpr bool kLoadsC = true;
  static_assert(kRingBytes + kWaves * 2 * 1024 <= kStagingBytes,
                "the staging tail past the ring takes 2 loads per wave");
  static_assert(kStagingWaveBytes % 1024 == 0 && kStageBytes % 1024 == 0,
                "every 1 KiB load lies in one wave's staging area");
  __device__ __forceinline__ void after_barrier(const KernelArgs&, int, int) {}
  // C for LDS bytes [x, x + 1024) of the staging layout (wave q's quarter
  // at q * kStagingWaveBytes, rows of kStagingRowBytes whose last 16 bytes
  // are padding), lane i taking bytes x + 16 i.  Rows past M read zeros;
  // columns past N land in outputs that are never stored.
  __device__ __forceinline__ void c_load(const KernelArgs& a, int tm, int tn, uint32_t x,
                                         int lane) {
    const uint32_t q = x / kStagingWaveBytes;  // wave-uniform
    const __amdgpu_buffer_rsrc_t rc =
        matrix_rsrc(a.C, a.ldc, a.M, a.N, (int64_t)tm * kTileM + (q >> 1) * kWaveTile,
                    (int64_t)tn * kTileN + (q & 1) * kWaveTile, true);
    const uint32_t o = x - q * kStagingWaveBytes + 16 * lane;
    const uint32_t row = o / kStagingRowBytes;
    const uint32_t c = o - row * kStagingRowBytes;
    dma16_w5(rc, lds_at(x),
             c < kWaveTile * 2 ? (uint32_t)(row * a.ldc * 2) + c : kOobOffset);
  }
};

// Stage, then store.  The ring must be idle (all waves past the main loop's
// closing barrier).  Returns with this wave's global stores issued.
// c_in_lds: C is already in the staging area (CPreload).  BM: the wave's
// 32-row blocks (4: 256-row tiles; 3: 192-row tiles, whose wave tiles are 96
// x 128 and use the first 96 rows of the same staging areas).
template <int BM = 4>
__device__ __forceinline__ void epilogue_store(const Accum& acc, const KernelArgs& a, int tm, int tn,
                                               int wave, int lane, bool c_in_lds = false) {
  constexpr int kRows = 32 * BM;                               // rows of the wave tile
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)tm * (2 * kRows) + wm * kRows;   // first row of the wave tile
  const int64_t n0 = (int64_t)tn * kTileN + wn * kWaveTile;   // first column
  const int lr = lane & 31;            // row within a 32 x 32 block
  const int half = lane >> 5;          // which 4 of the 8 columns of a chunk
  const uint32_t st_base = wave * kStagingWaveBytes + lr * kStagingRowBytes + 8 * half;

  if (a.beta != 0.0f) {
    // C of the wave's quarter lands in the wave's staging area, already in
    // the staging layout (rows of kStagingRowBytes, the last 16 bytes of
    // each unused), through LDS-DMA: lane i of load j fills bytes
    // 1024 j + 16 i, so it fetches the 16 bytes of C that belong there.
    // Whole row segments per instruction, instead of 8-byte pieces of 32
    // rows.  Out-of-range C reads return 0 or land in columns >= N; either
    // way they only feed outputs that are never stored.
    if (!c_in_lds) {
      const __amdgpu_buffer_rsrc_t rc = matrix_rsrc(a.C, a.ldc, a.M, a.N, m0, n0, true);
      const uint32_t wave_base = wave * kStagingWaveBytes;
      wait_lgkmcnt<0>();  // earlier reads of this area (the consumer's drain) are done
      static_assert(kStagingWaveBytes % 1024 == 0, "whole LDS-DMA loads per wave");
      // (96-row wave tiles: the last load also fills 2 staged rows past the
      // tile's, from C rows that are never stored.)
      constexpr int kLoads = (kRows * kStagingRowBytes + 1023) / 1024;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int b = 1024 * j + 16 * lane;
        const int row = b / kStagingRowBytes;
        const int off = b - row * kStagingRowBytes;
        dma16_w5_nt(rc, lds_at(wave_base + 1024 * j),
                    off < kWaveTile * 2 ? (uint32_t)(row * a.ldc * 2 + off) : kOobOffset);
      }
      wait_vmcnt<0>();
    }
    // One block row at a time: its 16 reads of C first, then the results
    // over them.  (Written read-compute-write per chunk, the compiler keeps
    // each read behind the previous chunk's write -- it cannot prove they do
    // not alias -- and every chunk then waits a full LDS round trip.)
#pragma unroll
    for (int bi = 0; bi < BM; ++bi) {
      u32x2 cw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        cw[i] = *(const MIGEMM_LDS u32x2*)lds_at(st_base + 32 * bi * kStagingRowBytes + i * 16);
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t at = st_base + 32 * bi * kStagingRowBytes + (4 * bj + q) * 16;
          const u32x2 c2 = cw[4 * bj + q];
          const f32x16& r = acc.v[bi][bj];
          const float v0 = a.alpha * r[4 * q + 0] + a.beta * bf16_lo(c2[0]);
          const float v1 = a.alpha * r[4 * q + 1] + a.beta * bf16_hi(c2[0]);
          const float v2 = a.alpha * r[4 * q + 2] + a.beta * bf16_lo(c2[1]);
          const float v3 = a.alpha * r[4 * q + 3] + a.beta * bf16_hi(c2[1]);
          const u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *(MIGEMM_LDS u32x2*)lds_at(at) = w;  // over the C it was formed from
        }
      }
    }
  } else {
#pragma unroll
    for (int bi = 0; bi < BM; ++bi)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& r = acc.v[bi][bj];
          const u32x2 w = {pack_bf16x2(a.alpha * r[4 * q + 0], a.alpha * r[4 * q + 1]),
                           pack_bf16x2(a.alpha * r[4 * q + 2], a.alpha * r[4 * q + 3])};
          *(MIGEMM_LDS u32x2*)lds_at(st_base + 32 * bi * kStagingRowBytes + (4 * bj + q) * 16) = w;
        }
  }

  // The wave reads back only what it wrote itself: LDS accesses of one wave
  // complete in order, so no barrier is needed here.
  const __amdgpu_buffer_rsrc_t rd = matrix_rsrc(a.D, a.ldd, a.M, a.N, m0, n0, false);
  const int rsub = lane >> 4;          // 4 rows per read
  const int chunk = lane & 15;
  const int64_t rows_left = a.M - m0;
  const int64_t cols_left = a.N - n0 - 8 * chunk;   // valid columns from this lane's chunk on
  const uint32_t rd_base = wave * kStagingWaveBytes + rsub * kStagingRowBytes + chunk * 16;
  const uint32_t d_lane = (uint32_t)((rsub * a.ldd + 8 * chunk) * 2);
#pragma unroll 8
  for (int i = 0; i < kRows / 4; ++i) {
    const u32x4 v = *(const MIGEMM_LDS u32x4*)lds_at(rd_base + 4 * i * kStagingRowBytes);
    const int row = 4 * i + rsub;
    if (row < rows_left && cols_left > 0) {
      const uint32_t off = d_lane + (uint32_t)(4 * i * a.ldd * 2);
      if (cols_left >= 8) {
        __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kCpolNt);
      } else {
        for (int e = 0; e < cols_left; ++e)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[e >> 1] >> (16 * (e & 1))), rd,
                                                off + 2 * e, 0, 0);
      }
    }
  }
}

}  // namespace migemm
