// mainloop.hpp -- the K loop: a 2-slot LDS ring filled by direct
// global->LDS buffer loads, drained by the MFMA core.
//
// The CUTLASS pages split this loop between a producer warp that waits for an
// empty stage, issues the TMA copies for it and lets the transaction barrier
// mark it full, and consumer warp groups that wait for a full stage, run
// WGMMA on it and release it (kernel page: mainloop producer warp and
// consumer warp-group loops; discussion #2761 on polling the next stage
// before issuing the current one).  gfx950 has no TMA, no transaction-count
// barriers and no per-role register reallocation, and a 128 x 128 fp32 wave
// tile needs 256 of a lane's 512 registers, so every one of the 4 waves is
// both producer and consumer:
//   - producer: each wave issues 1/4 of a stage's 16-byte LDS-DMA loads
//     (buffer_load_dwordx4 ... lds), one or two stages ahead of the stage
//     being consumed;
//   - full: a wave's own loads have landed when its vmcnt has dropped past
//     them; all waves' loads have landed after each waited and met at the
//     workgroup barrier;
//   - empty: the same barrier also certifies that every wave has finished
//     reading the stage the new loads overwrite.
// So the ring needs one s_waitcnt + one s_barrier per stage.
//
// A stage holds 128 bytes of K (64 bf16 or 128 e4m3) per row of each operand
// tile; the ring has 2 slots of 64 KiB:
//   - a K-contiguous operand is read in 128-byte row segments (8 lanes per
//     row), so both 64-byte halves of every line leave in one instruction and
//     the L1 turns them into one L2 request; with 64-byte segments every
//     line costs two (measured: L1 misses and L2 requests drop by a third, and
//     the address path stops stalling on the L1).  MN-contiguous operands are
//     read in whole 128-byte panel rows.  The memory pipeline serves
//     requests, not bytes: loads made of 64-byte segments reach only about
//     half the L2 and HBM throughput of 128-byte ones (~18 vs ~36 TB/s from
//     L2 over the chip);
//   - one barrier per 2048 MFMA cycles.
// With 2 slots, stage d+2 can only be loaded once every wave is done reading
// stage d.  The last k-step's fragments are read under the k-step before it,
// so the barrier sits after all but the last k-step's MFMAs, once those reads
// have returned; the first k-step of stage d+1 (certified by the same
// barrier) is read under the last k-step's MFMAs.
//   bf16 (4 k-steps of 16 MFMAs of 32 cycles): the barrier comes after 48 of
//     the stage's 64 MFMAs; stage d+2's 16 loads are spread over the 32 MFMAs
//     from that barrier to the end of stage d+1's first k-step (A in stage
//     d's last k-step, B in stage d+1's first), one behind every other MFMA,
//     and get at least 32 MFMAs to land.  How tightly the loads are packed
//     decides much of the speed (8192^3, pairs timed on one device): packed
//     into 16 MFMAs, one behind each, is 4% faster than into 8 MFMAs with two
//     behind each, and spreading them over 32 MFMAs gains another 2-2.5%.
//   e4m3 (2 k-steps of 16 MFMAs of 64 cycles): the barrier comes after the
//     first k-step; the 16 loads of stage d+2 sit one behind each MFMA of the
//     second (64 cycles apart, as in bf16), and get at least 16 MFMAs (1024
//     cycles) to land.  Loads in stage d+1's first k-step would have to land
//     by the barrier at its end.  (The previous e4m3 loop, 64-byte stages in
//     a 4-slot ring, was 5.5% slower.)
//
// LDS layout of one stage (64 KiB):  [A: 32 KiB][B: 32 KiB].
//   K-contiguous operand: 256 rows x 128 bytes of K; chunk c of row r is
//     stored at chunk c ^ ((r >> 1) & 7).
//   MN-contiguous operand: panels of 128 bytes of M or N (64 bf16 or 128
//     e4m3 columns), each holding the stage's K rows (64 or 128) of 128 bytes
//     back to back; chunk c of K row k stored at c ^ swz_mn(k).
// The swizzles make the fragment reads of one instruction hit every LDS bank
// equally often (measured on gfx950: a K-major 16-byte read takes ~4.5 cycles
// per instruction with a conflict-free pattern instead of 8, a transposing
// read ~3.8 instead of 4.5-8), and keep every fragment read of a wave at a
// per-lane base plus an immediate offset.  They are applied on the global
// side: LDS-DMA writes lane i's 16 bytes to a fixed LDS slot, so each lane
// fetches the chunk that belongs in its slot.
#pragma once

#include <type_traits>

#include "gfx950.hpp"
#include "params.hpp"

namespace migemm {

// Calls f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// MN-contiguous: a panel row is 128 bytes of M or N; chunk c of K row k is
// stored at chunk c ^ swz_mn(k).  bf16 swaps the 64-byte halves of every
// other pair of rows; e4m3 permutes the four 32-byte pieces.
template <int ES>
__device__ __forceinline__ int swz_mn(int k) {
  return ES == 2 ? ((k >> 1) & 1) << 2 : ((k >> 1) & 3) << 1;
}
constexpr int kPanelRowBytes = 128;

// The fragment type of one MFMA operand: 8 bf16 or 32 e4m3 per lane.
template <int ES>
struct FragType;
template <>
struct FragType<2> {
  typedef bf16x8 type;
};
template <>
struct FragType<1> {
  typedef i32x8 type;
};

template <int ES>
__device__ __forceinline__ f32x16 mfma(typename FragType<ES>::type a, typename FragType<ES>::type b,
                                       f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma<2>(bf16x8 a, bf16x8 b, f32x16 c) {
  return mfma_bf16_32x32x16(a, b, c);
}
template <>
__device__ __forceinline__ f32x16 mfma<1>(i32x8 a, i32x8 b, f32x16 c) {
  return mfma_fp8_32x32x64(a, b, c);
}

// The wave's 128 x 128 fp32 accumulator tile: 4 x 4 blocks of 32 x 32.
// Each block is computed as (B^T A^T) so that a lane ends up holding four
// consecutive columns of one row of D per group of 4 registers:
//   acc[bi][bj][4q + c] = D[m0 + 32 bi + l%32][n0 + 32 bj + 8q + 4(l/32) + c].
struct Accum {
  f32x16 v[4][4];
};

// Scheduling hint for one region: alternate one MFMA with a share of the LDS
// reads, so that reads are issued under the MFMAs instead of in one burst.
template <int kMfmas, int kReads>
__device__ __forceinline__ void interleave_mfma_reads() {
  constexpr int per = (kReads + kMfmas - 1) / kMfmas;
#pragma unroll
  for (int m = 0; m < kMfmas; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, per, 0);  // DS read
  }
}

// Keeps the compiler from moving any instruction across this point, so the
// phases of the K loop stay in the order written.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Work that rides along in the K loop: once per iteration, right after the
// barrier (before the iteration's stage loads), after_barrier() issues its
// memory operations.  A side work with kLoadsC also takes over the last two
// iterations' loads (see mainloop_range): c_load(x) loads the epilogue's
// source C into LDS byte x of the staging layout.
struct NoSideWork {
  static constexpr bool kLoadsC = false;
  __device__ __forceinline__ void after_barrier(const KernelArgs&, int, int) {}
  __device__ __forceinline__ void c_load(const KernelArgs&, int, int, uint32_t, int) {}
};

// Stage geometry for element size ES.
template <int ES>
struct StageGeom {
  static constexpr int kK = kStageKBytes / ES;               // K per stage: 64 bf16, 128 e4m3
  static constexpr int kKSteps = ES == 2 ? 4 : 2;            // MFMA k-steps per stage (16 / 64 K)
  static constexpr int kPanelCols = kPanelRowBytes / ES;     // 64 or 128
  static constexpr int kPanelBytes = kK * kPanelRowBytes;    // 8 or 16 KiB
  static constexpr int kLoadsPerPanel = kK / 8;              // 8 K rows per load
  static constexpr int kElemsPerChunk = 16 / ES;
};

// K-contiguous: chunk c of row r is stored at chunk c ^ swz_k8(r).  Rows of
// a fragment block start 32 rows apart, so the value depends on the lane
// alone.
__device__ __forceinline__ int swz_k8(int row) { return (row >> 1) & 7; }

// One operand's share of a wide stage: this wave's NL LDS-DMA loads of 1 KiB
// (8: a 256-row operand tile; 6: a 192-row one).  Load idx = NL wave + j of
// the stage goes to the stage's LDS kilobyte idx.
template <int ES, bool KMAJ, int NL = 8>
struct StageLoader {
  typedef StageGeom<ES> G;
  static_assert(NL == 8 || (NL == 6 && ES == 2), "192-row operand tiles are bf16 only");
  const unsigned char* tile_base;  // operand address of the tile's (row 0, k 0)
  int64_t kstep_bytes;             // address step from one stage of K to the next
  int64_t bytes_left;              // operand bytes from tile_base to its end
  uint32_t off[NL];                // this lane's byte offset for load j
  // The K index (within the stage) that this lane's load j starts at, kept
  // as the two values it takes (K-contiguous: by the parity of j) or as the
  // value for j = 0 (MN-contiguous: + 8 j), not as NL registers.  With 6
  // loads per wave an MN-contiguous operand's panels (8 loads each) start
  // inside a wave's share: kq[1] is then the wave's first load's position in
  // its panel.
  int32_t kq[2];
  __device__ __forceinline__ int32_t kpos(int j) const {
    if constexpr (KMAJ) return kq[j & 1];
    if constexpr (NL == 8) return kq[0] + 8 * j;
    return kq[0] + 8 * ((kq[1] + j) & 7);
  }

  __device__ __forceinline__ void init(const void* ptr, int64_t bytes, int64_t ld, int64_t origin,
                                       int wave, int lane) {
    const unsigned char* p = static_cast<const unsigned char*>(ptr);
    if constexpr (KMAJ) {
      // Load idx = NL wave + j covers rows 8 idx .. 8 idx + 7, 8 lanes a row.
      tile_base = p + origin * ld * ES;
      kstep_bytes = kStageKBytes;
      bytes_left = bytes - origin * ld * ES;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int row = (wave * NL + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz_k8(row);
        off[j] = (uint32_t)(row * ld * ES) + (uint32_t)(c * 16);
      }
      // chunk * elements per chunk for load j: swz_k8 of its row is
      // 4 (j & 1) + (lane >> 4) (NL is even).
      kq[0] = ((lane & 7) ^ (lane >> 4)) * G::kElemsPerChunk;
      kq[1] = ((lane & 7) ^ (4 + (lane >> 4))) * G::kElemsPerChunk;
    } else {
      // Load idx = NL wave + j fills K rows 8 (idx % L) .. + 7 of panel
      // idx / L (L loads per panel).
      tile_base = p + origin * ES;
      kstep_bytes = (int64_t)G::kK * ld * ES;
      bytes_left = bytes - origin * ES;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int idx = wave * NL + j;
        const int krow = (idx % G::kLoadsPerPanel) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_mn<ES>(krow);
        const int col = (idx / G::kLoadsPerPanel) * G::kPanelCols + chunk * G::kElemsPerChunk;
        off[j] = (uint32_t)(krow * ld * ES) + (uint32_t)(col * ES);
      }
      // krow of load j is 8 j + (lane >> 3), plus 64 for odd waves when a
      // panel takes 16 loads (e4m3).
      kq[0] = (G::kLoadsPerPanel == 16 ? 64 * (wave & 1) : 0) + (lane >> 3);
      kq[1] = NL == 8 ? 0 : (wave * NL) & 7;
    }
  }

  // Resource over the operand from K stage `kt` on, and the stage's valid K
  // (clamped: only "less than a stage or not" matters).  Buffer range checks
  // work per dword, so an operand whose last row ends inside a dword would
  // lose its last element: the range is rounded up to 16 bytes.  The base is
  // 16-byte aligned, so the extra bytes share the last element's 16-byte
  // block (and page) and only feed discarded columns.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(int kt, int64_t K, int* krem) const {
    const int64_t step = (int64_t)kt * kstep_bytes;
    int64_t left = (bytes_left - step + 15) & ~(int64_t)15;
    left = left < 0 ? 0 : (left > 0x7FFFFFF0 ? 0x7FFFFFF0 : left);
    const int64_t krem64 = K - (int64_t)kt * G::kK;
    *krem = krem64 > G::kK ? G::kK : (int)krem64;
    return make_rsrc(tile_base + step, (uint32_t)left);
  }

  // Load j (0..7) into the stage slot at LDS offset `slot`.  Stages past K
  // load out of range and only zero a free slot, which keeps every
  // iteration's count of loads fixed.  With
  // MASK false the stage is known to be complete (krem == kK), and the
  // per-lane K check -- two VALU instructions in front of every load -- is
  // left out.
  template <bool MASK = true>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int krem, uint32_t slot, int wave,
                                       int j) const {
    dma16(r, lds_at(slot + (wave * NL + j) * 1024),
          (!MASK || kpos(j) < krem) ? off[j] : kOobOffset);
  }
  // K-contiguous operands whose K is not a whole number of 16-byte chunks:
  // the chunk that holds the last K elements of a row also holds whatever
  // the row's storage has after K (padding, or anything else), which must
  // not reach the MFMAs -- a NaN or infinity there times the other operand's
  // zero is a NaN.  Once this wave's loads of the stage have landed (its own
  // vmcnt), it clears the bytes at K index krem and beyond in the chunks it
  // loaded; the barrier that follows publishes them.  Chunks wholly past K
  // were loaded out of range (zeros) and whole ones are left as they are.
  __device__ __forceinline__ void clear_k_tail(uint32_t slot, int krem, int wave, int lane) const {
    if constexpr (KMAJ) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int nb = (krem - kpos(j)) * ES;  // valid bytes of this lane's chunk
        if (nb > 0 && nb < 16) {
          MIGEMM_LDS u32x4* p = (MIGEMM_LDS u32x4*)lds_at(slot + (wave * NL + j) * 1024 + 16 * lane);
          u32x4 x = *p;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int vb = nb - 4 * w;  // valid bytes of word w
            x[w] &= vb >= 4 ? 0xFFFFFFFFu : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
          }
          *p = x;
        }
      }
    } else {
      (void)slot, (void)krem, (void)wave, (void)lane;
    }
  }
  __device__ __forceinline__ void load_all(int kt, uint32_t slot, int64_t K, int wave) const {
    int krem;
    const __amdgpu_buffer_rsrc_t r = stage_rsrc(kt, K, &krem);
#pragma unroll
    for (int j = 0; j < NL; ++j) load(r, krem, slot, wave, j);
  }
};

// Fragment reads from a wide stage: read<BLK, KS> returns the fragment of the
// wave's 32-row (or -column) block BLK (of NB) for k-step KS.
template <int ES, bool KMAJ, int NB = 4>
struct FragReader;

// K-contiguous bf16: one ds_read_b128; k-step ks is chunk 2 ks + (lane / 32).
template <int NB>
struct FragReader<2, true, NB> {
  static constexpr int kReads = 1;
  uint32_t off[4];  // per k-step
  __device__ __forceinline__ void init(int row0, int lane) {
    const int l = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      off[ks] = (row0 + l) * kStageKBytes + (((2 * ks + (lane >> 5)) ^ swz_k8(l)) << 4);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ bf16x8 read(uint32_t opnd_base) const {
    return *reinterpret_cast<const MIGEMM_LDS bf16x8*>(
        lds_at(opnd_base + off[KS] + BLK * 32 * kStageKBytes));
  }
};

// K-contiguous e4m3: two ds_read_b128 per fragment, the two 16-byte halves
// of the lane's 32 bytes of K: k-step ks, half h is chunk 4 ks + 2 (lane /
// 32) + h.
template <>
struct FragReader<1, true> {
  static constexpr int kReads = 2;
  uint32_t off[2][2];  // per k-step and half
  __device__ __forceinline__ void init(int row0, int lane) {
    const int l = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        off[ks][h] =
            (row0 + l) * kStageKBytes + (((4 * ks + 2 * (lane >> 5) + h) ^ swz_k8(l)) << 4);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ i32x8 read(uint32_t opnd_base) const {
    const i32x4 lo = *reinterpret_cast<const MIGEMM_LDS i32x4*>(
        lds_at(opnd_base + off[KS][0] + BLK * 32 * kStageKBytes));
    const i32x4 hi = *reinterpret_cast<const MIGEMM_LDS i32x4*>(
        lds_at(opnd_base + off[KS][1] + BLK * 32 * kStageKBytes));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// MN-contiguous bf16: two ds_read_b64_tr_b16 per fragment.  Within each group
// of 16 lanes the instruction reads a 4 x 16 block of bf16 (lanes 4r..4r+3
// each fetch 4 consecutive elements of row r) and hands lane i column i of
// the block.  Rows are K and columns are M or N here, so each lane receives 4
// consecutive k of its own column: lane l gets column l % 32 of the block and
// k = 8 (l / 32) + 0..3 (first read) and + 4..7 (second).  A 32-column block
// is one half of a 64-column panel; the swizzle flips which half depending on
// k, so even and odd blocks need one lane offset each.  k-step ks covers K
// rows 16 ks .. 16 ks + 15 of the panel (k + 16 ks and k + 4 keep swz_mn, so
// both are constant offsets).
template <>
struct FragReader<2, false> {
  typedef StageGeom<2> G;
  static constexpr int kReads = 2;
  uint32_t off[2];  // for even and odd blocks
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 8 * (g >> 1) + (t >> 2);
    const int chunk = 2 * (g & 1) + ((t & 3) >> 1);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      off[b] = (col0 / G::kPanelCols) * G::kPanelBytes + k * kPanelRowBytes +
               (((4 * b + chunk) ^ swz_mn<2>(k)) << 4) + 8 * (t & 1);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ bf16x8 read(uint32_t opnd_base) const {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    constexpr uint32_t c = (BLK >> 1) * G::kPanelBytes + 16 * KS * kPanelRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK & 1] + c));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK & 1] + c + 4 * kPanelRowBytes));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// MN-contiguous bf16, the 3 blocks of a wave's 96 rows of a 192-row tile:
// the same reads, but the second wave's blocks start in the second half of a
// 64-column panel (rows 96..191 of the tile), so each block has its own lane
// offset: block b is 32-column half-panel h = col0 / 32 + b, in panel h / 2,
// on the side h % 2 that the swizzle then flips with k.
template <>
struct FragReader<2, false, 3> {
  typedef StageGeom<2> G;
  static constexpr int kReads = 2;
  uint32_t off[3];  // per block
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 8 * (g >> 1) + (t >> 2);
    const int chunk = 2 * (g & 1) + ((t & 3) >> 1);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int h = col0 / 32 + b;
      off[b] = (h >> 1) * G::kPanelBytes + k * kPanelRowBytes +
               (((4 * (h & 1) + chunk) ^ swz_mn<2>(k)) << 4) + 8 * (t & 1);
    }
  }
  template <int BLK, int KS>
  __device__ __forceinline__ bf16x8 read(uint32_t opnd_base) const {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    constexpr uint32_t c = 16 * KS * kPanelRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK] + c));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK] + c + 4 * kPanelRowBytes));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// MN-contiguous e4m3: four ds_read_b64_tr_b8 per fragment.  Within each
// group of 16 lanes the instruction reads an 8 x 16 block of bytes (lanes 2r
// and 2r+1 fetch the two halves of row r) and hands lane i column i, i.e. 8
// consecutive k of its own column: lane l gets column l % 32 of the block and
// k = 32 (l / 32) + 8 h + 0..7 from read h.  The wave's 128 columns are one
// panel; a 32-column block is one 32-byte piece of it, placed by the
// swizzle, so each block has its own lane offset.  k-step ks covers K rows
// 64 ks .. 64 ks + 63 (k + 64 ks and k + 8 h keep swz_mn, so all reads are
// constant offsets apart).
template <>
struct FragReader<1, false> {
  typedef StageGeom<1> G;
  static constexpr int kReads = 4;
  uint32_t off[4];  // per block
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 32 * (g >> 1) + (t >> 1);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      off[b] = (col0 / G::kPanelCols) * G::kPanelBytes + k * kPanelRowBytes +
               (((2 * b + (g & 1)) ^ swz_mn<1>(k)) << 4) + 8 * (t & 1);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ i32x8 read(uint32_t opnd_base) const {
    i32x8 v;
    static_for<0, 4>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MIGEMM_LDS i32x2*)lds_at(
          opnd_base + off[BLK] + (64 * KS + 8 * h) * kPanelRowBytes));
      v[2 * h] = w[0];
      v[2 * h + 1] = w[1];
    });
    return v;
  }
};

// The fragments of two k-steps (buffer kb holds k-steps of parity kb): BM A
// and 4 B fragments each (64 VGPRs for bf16 with BM = 4, 128 for e4m3).
// BM is the wave's count of 32-row blocks: 4 (256-row tiles) or 3 (192).
template <int ES, bool AK, bool BK, int BM = 4>
struct Frags {
  typedef FragReader<ES, AK, BM> RA;
  typedef FragReader<ES, BK> RB;
  typedef typename FragType<ES>::type frag_t;
  static constexpr int kReadInsts = BM * RA::kReads + 4 * RB::kReads;  // per k-step
  frag_t a[2][BM];
  frag_t b[2][4];
  RA ra;
  RB rb;

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    ra.init(wm * 32 * BM, lane);
    rb.init(wn * kWaveTile, lane);
  }

  // Blocks [Q * 4 / NQ, (Q + 1) * 4 / NQ) of k-step KS into buffer KS & 1
  // (of A, those below BM).
  template <int KS, int Q, int NQ>
  __device__ __forceinline__ void read_part(uint32_t a_base, uint32_t b_base) {
    static_for<Q * 4 / NQ, (Q + 1) * 4 / NQ>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      if constexpr (x < BM) a[KS & 1][x] = ra.template read<x, KS>(a_base);
      b[KS & 1][x] = rb.template read<x, KS>(b_base);
    });
  }

  // MFMAs [FIRST, FIRST + COUNT) of the 4 BM of buffer KB: MFMA m is block
  // (m / 4) of A with block (m % 4) of B.
  template <int KB, int FIRST, int COUNT>
  __device__ __forceinline__ void mma(Accum& acc) const {
    static_for<FIRST, FIRST + COUNT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int i = m >> 2, j = m & 3;
      acc.v[i][j] = mfma<ES>(b[KB][j], a[KB][i], acc.v[i][j]);
    });
  }
};

// The K loop of one output tile.  Stage d lives in slot d % 2.
// bf16, per stage:
//   k-step 0: 16 MFMAs; k-step 1 read under the first 8, one A and one B
//             block at a time; B of stage d+1 loaded behind every other MFMA
//             (into stage d+1's slot, free since stage d-1's barrier);
//   k-steps 1, 2: 16 MFMAs each, under which the next k-step is read;
//   sync: wait until none of this wave's loads (only stage d+1's were in
//         flight) and none of its LDS reads is outstanding; barrier: stage
//         d+1 is in LDS for every wave, and every wave is done reading stage d;
//   the side work steps; k-step 3: 16 MFMAs; k-step 0 of stage d+1 read
//             under them; A of stage d+2 loaded behind every other MFMA (into
//             stage d's slot).
// e4m3, per stage:
//   k-step 0: 16 MFMAs; k-step 1 read under the first 8;
//   sync and barrier as above;
//   the side work steps; k-step 1: 16 MFMAs; k-step 0 of stage d+1 read
//             under them; the 16 loads of stage d+2 behind them, one each.
// One load blocks the issuing wave for a few dozen cycles, and the address
// path serves the four waves in turn, so loads packed closer than about 64
// cycles stall the MFMA stream.
//
// 192-row tiles (BM = 3, bf16 only): 12 MFMAs per k-step and 6 A loads per
// wave and stage.  The stage's 8 B loads no longer fit behind every other
// MFMA of the first k-step: 6 go there, and the last 2 (kBEarly) are issued
// one stage ahead, in the last k-step of the iteration before (into the
// slot its barrier frees), behind the MFMAs the A loads leave free.
//
// mainloop_range runs K stages [k0, k0 + KT) of the tile (a stream-K
// segment); K is the problem's K or, for a segment that ends before it, the
// segment's end: loads past it fall out of range like loads past the
// problem's K.  Only the first BM rows of blocks of acc are used.
template <int ES, bool AK, bool BK, int BM = 4, class SideWork>
__device__ __forceinline__ void mainloop_range(Accum& acc, const KernelArgs& a, int tm, int tn,
                                               int wave, int lane, SideWork& side, int k0, int KT,
                                               int64_t K) {
  typedef StageGeom<ES> G;
  typedef Frags<ES, AK, BK, BM> FW;
  static_assert(BM == 4 || (BM == 3 && ES == 2), "192-row tiles are bf16 only");
  static_assert(BM == 4 || !SideWork::kLoadsC, "C is read in the K loop of 256-row tiles only");
  constexpr bool kBf16 = ES == 2;
  constexpr int kLast = G::kKSteps - 1;
  constexpr int kM = 4 * BM;                  // MFMAs per k-step
  constexpr int kBEarly = BM == 4 ? 0 : 2;    // B loads issued one iteration early
  constexpr int kBLate = 8 - kBEarly;         // B loads in the first k-step
  constexpr uint32_t kB = kOperandStageBytes;
  StageLoader<ES, AK, 2 * BM> la;
  StageLoader<ES, BK> lb;
  la.init(a.A, a.a_bytes, a.lda, (int64_t)tm * (64 * BM), wave, lane);
  lb.init(a.B, a.b_bytes, a.ldb, (int64_t)tn * kTileN, wave, lane);
  const int wm = wave >> 1, wn = wave & 1;

#pragma unroll
  for (int i = 0; i < BM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][j] = f32x16{};

  FW f;
  f.init(wm, wn, lane);
  // The stage that the next barrier certifies (relative index rs, in the
  // ring slot at `slot`) ends inside a 16-byte chunk of a K-contiguous
  // operand: clear what lies past K (clear_k_tail).  Only the K tail can.
  constexpr bool kAnyKMajor = AK || BK;
  auto clear_tail = [&](int rs, uint32_t slot) {
    if constexpr (kAnyKMajor) {
      const int64_t krem = K - (int64_t)(k0 + rs) * G::kK;
      if (krem > 0 && krem < G::kK && ((krem * ES) & 15) != 0) {
        la.clear_k_tail(slot, (int)krem, wave, lane);
        lb.clear_k_tail(slot + kB, (int)krem, wave, lane);
        wait_lgkmcnt<0>();
      }
    }
  };
  if (KT > 0) {
    // Prologue: stage 0 and stage 1 in flight (bf16: stage 1's B is loaded in
    // the first iteration), stage 0 certified, its k-step 0 read.
    la.load_all(k0, 0, K, wave);
    lb.load_all(k0, kB, K, wave);
    la.load_all(k0 + 1, kStageBytes, K, wave);
    if constexpr (kBf16) {
      if constexpr (kBEarly > 0) {
        int krem;
        const __amdgpu_buffer_rsrc_t r = lb.stage_rsrc(k0 + 1, K, &krem);
        static_for<kBLate, 8>([&](auto jc) {
          lb.load(r, krem, kStageBytes + kB, wave, decltype(jc)::value);
        });
      }
      wait_vmcnt<2 * BM + kBEarly>();  // stage 0 has landed
    } else {
      lb.load_all(k0 + 1, kStageBytes + kB, K, wave);
      wait_vmcnt<16>();
    }
    clear_tail(0, 0);
    barrier();
    f.template read_part<0, 0, 1>(0, kB);
  }
  // The epilogue's source C (side work with kLoadsC): the two ring slots
  // fall free in the last two iterations, and the epilogue stages its tile
  // over them.  So the loads of stages past K that those iterations would
  // issue (they only zero a free slot) give way to loads of C, straight into
  // the staging layout: iteration KT-2 fills the slot it frees (and the
  // staging area's tail past the ring), iteration KT-1 the other one, and
  // the loop's closing wait covers both.  bf16's first k-step of iteration
  // KT-1 would load B of stage KT into the slot C already holds: skipped.
  constexpr bool kLoadsC = SideWork::kLoadsC;
  constexpr int kCLoads = 18;  // C loads per wave in iteration KT-2: 16 into the slot, 2 into the tail
  auto iteration = [&](const int d, auto mask_c) {
    constexpr bool kMask = decltype(mask_c)::value;
    const uint32_t cur = (d & 1) * kStageBytes;
    const uint32_t nxt = ((d + 1) & 1) * kStageBytes;
    bool c_here = false, skip_b = false;
    if constexpr (kMask && kLoadsC) {
      c_here = KT >= 2 && d >= KT - 2;
      skip_b = KT >= 2 && d == KT - 1;
    }
    int krem_a, krem_b;
    const __amdgpu_buffer_rsrc_t ra = la.stage_rsrc(k0 + d + 2, K, &krem_a);
    const __amdgpu_buffer_rsrc_t rb = lb.stage_rsrc(k0 + (kBf16 ? d + 1 : d + 2), K, &krem_b);
    static_for<0, kM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sched_fence();
      // k-step 1 read one A and one B block at a time, behind every other
      // MFMA (in two bursts of six reads it was 1% slower).
      if constexpr (m % 2 == 0 && m < 8) f.template read_part<1, m / 2, 4>(cur, cur + kB);
      f.template mma<0, m, 1>(acc);
      if constexpr (kBf16 && (m & 1) && (m >> 1) < kBLate) {
        if (!skip_b) lb.template load<kMask>(rb, krem_b, nxt + kB, wave, m >> 1);
      }
    });
    static_for<1, kLast>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      static_for<0, 2>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        f.template read_part<ks + 1, q, 2>(cur, cur + kB);
        f.template mma<ks & 1, 4 * q, 4>(acc);
        interleave_mfma_reads<4, FW::kReadInsts / 2>();
      });
      sched_fence();
      f.template mma<ks & 1, 8, kM - 8>(acc);
    });
    sched_fence();
    // The last k-step's fragments are in registers: this wave is done
    // reading stage d once its reads have returned.  (In iteration KT-1 of a
    // C-loading side work the only loads in flight are the kCLoads of C from
    // iteration KT-2, and stage KT is past K: they may stay in flight until
    // the loop's closing wait.)
    if (skip_b) {
      wait_vmcnt<kCLoads>();
    } else {
      wait_vmcnt<0>();
    }
    wait_lgkmcnt<0>();
    if constexpr (kMask) clear_tail(d + 1, nxt);
    barrier();
    // Anything the side work fetched after the previous barrier has landed.
    side.after_barrier(a, wave, lane);
    static_for<0, kM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sched_fence();
      if constexpr (m % 2 == 0 && m >= 2 && m < 10)
        f.template read_part<0, (m - 2) / 2, 4>(nxt, nxt + kB);
      f.template mma<kLast & 1, m, 1>(acc);
      if (c_here) {
        // 64 loads of 1 KiB fill the freed slot, 16 per wave, one behind
        // each MFMA; in iteration KT-2 two more per wave fill the tail.
        side.c_load(a, tm, tn, cur + 1024 * (16 * wave + m), lane);
        if constexpr (m < 2) {
          if (d == KT - 2) side.c_load(a, tm, tn, kRingBytes + 1024 * (2 * wave + m), lane);
        }
      } else if constexpr (kBf16) {
        if constexpr (m & 1) la.template load<kMask>(ra, krem_a, cur, wave, m >> 1);
        // 192-row tiles: B of stage d+2's last kBEarly loads, into the slot
        // this iteration's barrier freed; early load e behind MFMA e kM /
        // kBEarly (0 and 6).
        static_for<0, kBEarly>([&](auto ec) {
          constexpr int e = decltype(ec)::value;
          if constexpr (e * kM / kBEarly == m) {
            int krem_b2;
            const __amdgpu_buffer_rsrc_t rb2 = lb.stage_rsrc(k0 + d + 2, K, &krem_b2);
            lb.template load<kMask>(rb2, krem_b2, cur + kB, wave, kBLate + e);
          }
        });
      } else {
        if constexpr (m < 8) la.template load<kMask>(ra, krem_a, cur, wave, m);
        else lb.template load<kMask>(rb, krem_b, cur + kB, wave, m - 8);
      }
    });
  };
  // Iteration d loads stage d+2 (bf16: and B of stage d+1).  While those
  // stages are complete, the loads need no K check; the last iterations (the
  // K tail and the stages past K, which only zero a free slot) keep it.
  // (The two copies of the body must not push anything to scratch: a scratch
  // reload inside the loop waits for every stage load in flight.)
  int clean = (int)(K / G::kK) - k0 - 2;
  clean = clean < 0 ? 0 : (clean > KT ? KT : clean);
  int d = 0;
  for (; d < clean; ++d) iteration(d, std::integral_constant<bool, false>{});
  for (; d < KT; ++d) iteration(d, std::integral_constant<bool, true>{});
  // Every wave is done with the ring, and every load into it has landed,
  // before anyone reuses it.
  sched_fence();
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();
  barrier();
}

// The whole K loop of one output tile (BM: the wave's 32-row blocks).
template <int ES, bool AK, bool BK, int BM = 4, class SideWork>
__device__ __forceinline__ void mainloop(Accum& acc, const KernelArgs& a, int tm, int tn,
                                         int wave, int lane, SideWork& side) {
  int KT = (int)((a.K + StageGeom<ES>::kK - 1) / StageGeom<ES>::kK);
  // Opaque per tile, like the lane ids: tests on KT are then made where they
  // are used, not once before the tile loop and held (or spilled, and
  // reloaded with a vmcnt(0)) across it.
  asm volatile("" : "+s"(KT));
  mainloop_range<ES, AK, BK, BM>(acc, a, tm, tn, wave, lane, side, 0, KT, a.K);
}

}  // namespace migemm
