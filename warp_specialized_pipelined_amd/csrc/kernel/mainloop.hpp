// mainloop.hpp -- the K loop: an N-stage LDS ring filled by direct
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
//     (buffer_load_dwordx4 ... lds), S-1 stages ahead of the stage being
//     consumed;
//   - full: a wave's own loads have landed when its vmcnt has dropped past
//     them; all waves' loads have landed after each waited and met at the
//     workgroup barrier;
//   - empty: the same barrier also certifies that every wave has finished
//     reading the stage consumed one step earlier, which is the stage the
//     new loads overwrite.
// So the ring needs one s_waitcnt + one s_barrier per stage.
//
// LDS layout of one stage (32 KiB):  [A: 16 KiB][B: 16 KiB].
//   K-contiguous operand: 256 rows x 64 bytes of K, the four 16-byte chunks
//     of row r stored in the order c ^ swz_k(r), so that the eight rows read
//     by one group of lanes fall on distinct banks.
//   MN-contiguous operand: 8 panels of 32 columns (of M or N), each panel
//     holding the stage's (64 / elem_size) K rows back to back, 32 elements
//     per row (2 KiB per panel).  The transposing reads of one half-wave
//     then cover 256 consecutive bytes -- every bank once -- and every
//     fragment of a wave sits at a constant offset from its first one.
// The K-contiguous swizzle is applied on the global side: LDS-DMA writes
// lane i's 16 bytes to a fixed LDS slot, so each lane fetches the chunk that
// belongs in its slot.
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

__device__ __forceinline__ int swz_k(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Bytes of one MN-contiguous panel: 32 columns by a stage's K rows.
constexpr int kPanelBytes = 32 * kStageKBytes;  // 2 KiB

// One operand's share of the ring: where this wave's 4 loads per stage come
// from and go to.  ES = element size in bytes, KMAJ = K is the contiguous
// dimension of the operand.
template <int ES, bool KMAJ>
struct OperandLoader {
  static constexpr int kBK = kStageKBytes / ES;     // K per stage, elements
  static constexpr int kElemsPerChunk = 16 / ES;
  const unsigned char* tile_base;  // operand address of the tile's (row 0, k 0)
  int64_t kstep_bytes;             // address step from one stage of K to the next
  int64_t bytes_left;              // operand bytes from tile_base to its end
  uint32_t off[4];                 // this lane's byte offset for load j
  int32_t kpos[4];                 // K index (within the stage) that load j starts at

  // ptr/bytes: the operand; ld: its non-unit stride; origin: first row (M or
  // N index) of the tile.
  __device__ __forceinline__ void init(const void* ptr, int64_t bytes, int64_t ld, int64_t origin,
                                       int wave, int lane) {
    const unsigned char* p = static_cast<const unsigned char*>(ptr);
    if constexpr (KMAJ) {
      tile_base = p + origin * ld * ES;
      kstep_bytes = kStageKBytes;
      bytes_left = bytes - origin * ld * ES;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = (wave * 4 + j) * 16 + (lane >> 2);  // 16 rows of 64 B per KiB
        const int c = (lane & 3) ^ swz_k(row);
        off[j] = (uint32_t)(row * ld * ES) + (uint32_t)(c * 16);
        kpos[j] = c * kElemsPerChunk;
      }
    } else {
      // Load idx = 4 * wave + j fills half (idx & 1) of panel (idx >> 1):
      // kRowsPerLoad K rows of the panel's 32 columns, each row read by
      // kLanesPerRow lanes.
      constexpr int kLanesPerRow = 32 * ES / 16;         // 4 (bf16) or 2 (e4m3)
      constexpr int kRowsPerLoad = 64 / kLanesPerRow;    // 16 or 32
      tile_base = p + origin * ES;
      kstep_bytes = (int64_t)kBK * ld * ES;
      bytes_left = bytes - origin * ES;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = wave * 4 + j;
        const int krow = (idx & 1) * kRowsPerLoad + lane / kLanesPerRow;
        const int col = (idx >> 1) * 32 + (lane % kLanesPerRow) * kElemsPerChunk;
        off[j] = (uint32_t)(krow * ld * ES) + (uint32_t)(col * ES);
        kpos[j] = krow;
      }
    }
  }

  // Issue load j (0..3) of this wave's 4 loads of K stage `kt` into ring
  // slot `slot`.  `half` is 0 for A and kOperandStageBytes for B.
  __device__ __forceinline__ void issue_one(int kt, int slot, int half, int64_t K, int wave,
                                            int j) const {
    const int64_t step = (int64_t)kt * kstep_bytes;
    int64_t left = (bytes_left - step + 15) & ~(int64_t)15;
    left = left < 0 ? 0 : (left > 0x7FFFFFF0 ? 0x7FFFFFF0 : left);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(tile_base + step, (uint32_t)left);
    const int64_t krem64 = K - (int64_t)kt * kBK;
    const int krem = krem64 > kBK ? kBK : (int)krem64;
    const uint32_t v = (kpos[j] < krem) ? off[j] : kOobOffset;
    dma16(r, lds_at(slot * kStageBytes + half + (wave * 4 + j) * 1024), v);
  }

  // Issue this wave's 4 loads of K stage `kt` into ring slot `slot`.
  __device__ __forceinline__ void issue(int kt, int slot, int half, int64_t K, int wave) const {
    const int64_t step = (int64_t)kt * kstep_bytes;
    // Buffer range checks work per dword, so an operand whose last row ends
    // inside a dword would lose its last element: round the range up to 16
    // bytes.  The base is 16-byte aligned, so the extra bytes share the last
    // element's 16-byte block (and page) and only feed discarded columns.
    int64_t left = (bytes_left - step + 15) & ~(int64_t)15;
    left = left < 0 ? 0 : (left > 0x7FFFFFF0 ? 0x7FFFFFF0 : left);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(tile_base + step, (uint32_t)left);
    // Valid K in this stage (clamped: only "less than kBK or not" matters).
    const int64_t krem64 = K - (int64_t)kt * kBK;
    const int krem = krem64 > kBK ? kBK : (int)krem64;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = (kpos[j] < krem) ? off[j] : kOobOffset;
      dma16(r, lds_at(slot * kStageBytes + half + (wave * 4 + j) * 1024), v);
    }
  }
};

// Fragment reads.  A "fragment" is what one lane feeds one 32 x 32 MFMA: 32
// bytes of K (fp8) or 16 bytes (bf16, one of two k-steps per stage) of one
// row of A or one column of B.  Each reader keeps the lane's byte offsets of
// its wave's first 32-row (or -column) block; block BLK and k-step KS sit at
// a compile-time distance from them, which the LDS instructions take as an
// immediate offset, so a stage costs one address add per offset.
template <int ES, bool KMAJ>
struct FragReader;

// K-contiguous bf16: one ds_read_b128 per fragment.  Rows of a 32-row block
// start 32 rows apart, so the swizzle depends on the lane alone.
template <>
struct FragReader<2, true> {
  typedef bf16x8 frag_t;
  static constexpr int kSteps = 2;  // 32 k per stage, 16 per MFMA
  static constexpr int kReads = 1;  // LDS instructions per fragment
  uint32_t off[2];                  // per k-step
  __device__ __forceinline__ void init(int row0, int lane) {
    const int l = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      off[ks] = (row0 + l) * kStageKBytes + (((2 * ks + (lane >> 5)) ^ swz_k(l)) << 4);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ frag_t read(uint32_t opnd_base) const {
    return *reinterpret_cast<const MIGEMM_LDS frag_t*>(
        lds_at(opnd_base + off[KS] + BLK * 32 * kStageKBytes));
  }
};

// K-contiguous e4m3: two ds_read_b128 per fragment (the two 16-byte halves
// of the lane's 32 bytes of K).
template <>
struct FragReader<1, true> {
  typedef i32x8 frag_t;
  static constexpr int kSteps = 1;  // 64 k per stage, 64 per MFMA
  static constexpr int kReads = 2;
  uint32_t off[2];                  // per half
  __device__ __forceinline__ void init(int row0, int lane) {
    const int l = lane & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      off[h] = (row0 + l) * kStageKBytes + (((2 * (lane >> 5) + h) ^ swz_k(l)) << 4);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ frag_t read(uint32_t opnd_base) const {
    const i32x4 lo = *reinterpret_cast<const MIGEMM_LDS i32x4*>(
        lds_at(opnd_base + off[0] + BLK * 32 * kStageKBytes));
    const i32x4 hi = *reinterpret_cast<const MIGEMM_LDS i32x4*>(
        lds_at(opnd_base + off[1] + BLK * 32 * kStageKBytes));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// MN-contiguous bf16: two ds_read_b64_tr_b16 per fragment.  Within each
// group of 16 lanes the instruction reads a 4 x 16 block of bf16 (lanes
// 4r..4r+3 each fetch 4 consecutive elements of row r) and hands lane i
// column i of the block.  Rows are K and columns are M or N here, so each
// lane receives 4 consecutive k of its own column: lane l gets column l % 32
// of the block and k = 8 (l / 32) + 0..3 (first read) and + 4..7 (second).
template <>
struct FragReader<2, false> {
  typedef bf16x8 frag_t;
  static constexpr int kSteps = 2;
  static constexpr int kReads = 2;
  static constexpr int kRowBytes = 64;  // one K row of a panel
  uint32_t off;
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int n = 16 * (g & 1) + 4 * (t & 3);  // column within the panel
    const int k = 8 * (g >> 1) + (t >> 2);
    off = (col0 / 32) * kPanelBytes + k * kRowBytes + n * 2;
  }
  template <int BLK, int KS>
  __device__ __forceinline__ frag_t read(uint32_t opnd_base) const {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    constexpr uint32_t c = BLK * kPanelBytes + 16 * KS * kRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off + c));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off + c + 4 * kRowBytes));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(frag_t, v);
  }
};

// MN-contiguous e4m3: four ds_read_b64_tr_b8 per fragment.  Within each
// group of 16 lanes the instruction reads an 8 x 16 block of bytes (lanes 2r
// and 2r+1 fetch the two halves of row r) and hands lane i column i, i.e. 8
// consecutive k of its own column: lane l gets column l % 32 of the block and
// k = 32 (l / 32) + 8 h + 0..7 from read h.
template <>
struct FragReader<1, false> {
  typedef i32x8 frag_t;
  static constexpr int kSteps = 1;
  static constexpr int kReads = 4;
  static constexpr int kRowBytes = 32;
  uint32_t off;
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int n = 16 * (g & 1) + 8 * (t & 1);
    const int k = 32 * (g >> 1) + (t >> 1);
    off = (col0 / 32) * kPanelBytes + k * kRowBytes + n;
  }
  template <int BLK, int KS>
  __device__ __forceinline__ frag_t read(uint32_t opnd_base) const {
    i32x8 v;
    static_for<0, 4>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (MIGEMM_LDS i32x2*)lds_at(opnd_base + off + BLK * kPanelBytes + 8 * h * kRowBytes));
      v[2 * h] = w[0];
      v[2 * h + 1] = w[1];
    });
    return v;
  }
};

template <int ES>
__device__ __forceinline__ f32x16 mfma(typename FragReader<ES, true>::frag_t a,
                                       typename FragReader<ES, true>::frag_t b, f32x16 c);
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

// The fragments one wave needs from one stage, in two halves of 32 VGPRs so
// that one half can be refilled while the MFMAs of the other run.
//   bf16:  half h = the 4 A and 4 B fragments of k-step h (16 bytes each);
//   e4m3:  half h = A fragments {2h, 2h+1} and B fragments {2h, 2h+1}
//          (32 bytes each; the stage is a single k-step).
// MFMA (i, j) -- 32-row block i of A with 32-column block j of B -- runs in
//   phase 0: it needs half 0 only       (bf16: k-step 0; e4m3: i<2, j<2)
//   phase 1: it needs both halves       (bf16: none;     e4m3: the mixed ones)
//   phase 2: it needs half 1 only       (bf16: k-step 1; e4m3: i>=2, j>=2)
template <int ES, bool AK, bool BK>
struct FragHalves {
  typedef FragReader<ES, AK> RA;
  typedef FragReader<ES, BK> RB;
  static constexpr bool kBf16 = RA::kSteps == 2;
  static constexpr int kPerHalf = kBf16 ? 4 : 2;   // A (and B) fragments per half
  typename RA::frag_t a[2][kPerHalf];
  typename RB::frag_t b[2][kPerHalf];
  RA ra;
  RB rb;

  // LDS read instructions of one half, and MFMAs of each phase.
  static constexpr int kReadInsts = kPerHalf * (RA::kReads + RB::kReads);
  static constexpr int kPhase0 = kBf16 ? 16 : 4;
  static constexpr int kPhase1 = kBf16 ? 0 : 8;
  static constexpr int kPhase2 = kBf16 ? 16 : 4;

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    ra.init(wm * kWaveTile, lane);
    rb.init(wn * kWaveTile, lane);
  }

  // Fragments [Q * kPerHalf / NQ, (Q + 1) * kPerHalf / NQ) of half H from
  // ring slot `slot`.
  template <int H, int Q, int NQ>
  __device__ __forceinline__ void read_part(int slot) {
    const uint32_t a_base = slot * kStageBytes;
    const uint32_t b_base = a_base + kOperandStageBytes;
    static_for<Q * kPerHalf / NQ, (Q + 1) * kPerHalf / NQ>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      // bf16: block x of k-step H; e4m3: block 2H + x of the single k-step
      constexpr int blk = kBf16 ? x : 2 * H + x;
      constexpr int ks = kBf16 ? H : 0;
      a[H][x] = ra.template read<blk, ks>(a_base);
      b[H][x] = rb.template read<blk, ks>(b_base);
    });
  }

  // MFMAs [FIRST, FIRST + COUNT) of phase P (all indices compile-time, so
  // every fragment and accumulator stays in registers).
  template <int P, int FIRST, int COUNT>
  __device__ __forceinline__ void mma(Accum& acc) const {
    static_for<FIRST, FIRST + COUNT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (kBf16) {
        constexpr int h = P == 0 ? 0 : 1;  // phase 1 is empty for bf16
        constexpr int i = m >> 2, j = m & 3;
        acc.v[i][j] = mfma<ES>(b[h][j], a[h][i], acc.v[i][j]);
      } else {
        constexpr int i = P == 0 ? (m >> 1) : P == 2 ? 2 + (m >> 1)
                                            : (m < 4 ? (m >> 1) : 2 + ((m - 4) >> 1));
        constexpr int j = P == 0 ? (m & 1) : P == 2 ? 2 + (m & 1) : (m < 4 ? 2 + (m & 1) : (m & 1));
        acc.v[i][j] = mfma<ES>(b[j >> 1][j & 1], a[i >> 1][i & 1], acc.v[i][j]);
      }
    });
  }
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

// Wait until no more than `pending` stages of this wave's loads are in
// flight (each stage is 8 vector-memory ops per wave: 4 for A, 4 for B).
__device__ __forceinline__ void wait_stages_in_flight(int pending) {
  if (pending >= 2) {
    wait_vmcnt<16>();
  } else if (pending == 1) {  // (pending <= 0: wait for everything)
    wait_vmcnt<8>();
  } else {
    wait_vmcnt<0>();
  }
}

// Keeps the compiler from moving any instruction across this point, so the
// phases of the K loop stay in the order written.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Work that rides along in the K loop: step() is called once per iteration,
// right after the barrier.
struct NoSideWork {
  __device__ __forceinline__ void step(const KernelArgs&, int, int, bool) {}
};

// The whole K loop of one output tile.
//
// Iteration kt works on stage kt, whose half-0 fragments were read during the
// previous iteration.  The workgroup barrier certifies stage kt+1 (one ahead):
//   phase 0: MFMAs on half 0, under which half 1 of stage kt is read; the B
//            loads of stage kt+2 go out one per 4 MFMAs (bf16);
//   phase 1: MFMAs needing both halves (e4m3 only), with those B loads;
//   sync:    wait for this wave's loads of stage kt+1, barrier -- now stage
//            kt+1 is in LDS for every wave, and every wave is done reading
//            stage kt-1;
//   phase 2: the side work steps once; MFMAs on half 1, with the A loads of
//            stage kt+3 one per 4 MFMAs (e4m3: one per MFMA) and half 0 of
//            stage kt+1 read under them.
// Each stage's loads are thus spread over two iterations instead of leaving
// in one burst after the barrier, when all four waves would queue 32 of them
// on the CU's address unit at once and starve the MFMA pipe.  Stage s's A
// half leaves in iteration s-3 (after barrier s-3 freed stage s-4's slot) and
// its B half in iteration s-2; both are certified in iteration s-1.
template <int ES, bool AK, bool BK, class SideWork>
__device__ __forceinline__ void mainloop(Accum& acc, const KernelArgs& a, int tm, int tn, int wave,
                                         int lane, SideWork& side) {
  static_assert(kStages == 4, "the certify-ahead ring is written for 4 stages");
  typedef FragHalves<ES, AK, BK> FH;
  constexpr int kBK = kStageKBytes / ES;
  OperandLoader<ES, AK> la;
  OperandLoader<ES, BK> lb;
  la.init(a.A, a.a_bytes, a.lda, (int64_t)tm * kTileM, wave, lane);
  lb.init(a.B, a.b_bytes, a.ldb, (int64_t)tn * kTileN, wave, lane);
  const int wm = wave >> 1, wn = wave & 1;
  const int KT = (int)((a.K + kBK - 1) / kBK);
  constexpr int kB = kOperandStageBytes;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][j] = f32x16{};

  FH f;
  f.init(wm, wn, lane);
  if (KT > 0) {
    // Prologue: stages 0..2 in flight, stage 0 certified, its half 0 read.
    for (int s = 0; s < kStages - 1 && s < KT; ++s) {
      la.issue(s, s, 0, a.K, wave);
      lb.issue(s, s, kB, a.K, wave);
    }
    wait_stages_in_flight(min(kStages - 2, KT - 1));
    barrier();
    f.template read_part<0, 0, 1>(0);
  }
  for (int kt = 0; kt < KT; ++kt) {
    // Every iteration has the same shape (no branch around MFMAs, so the
    // accumulators never meet at a join): in the last ones the barrier is
    // redundant and the half-0 read fetches bytes nobody uses.
    const int slot = kt % kStages;
    const int sb = kt + 2;                       // stage whose B half leaves now
    const bool b_due = kt >= 1 && sb < KT;       // (stage 2's left in the prologue)
    const int sa = kt + 3;                       // stage whose A half leaves now
    const bool a_due = sa < KT;
    const int nslot = (kt + 1) % kStages;
    if constexpr (FH::kBf16) {
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        if (b_due) lb.issue_one(sb, sb % kStages, kB, a.K, wave, q);
        f.template read_part<1, q, 4>(slot);
        f.template mma<0, 4 * q, 4>(acc);
        interleave_mfma_reads<4, FH::kReadInsts / 4>();
      });
    } else {
      sched_fence();
      f.template read_part<1, 0, 1>(slot);
      f.template mma<0, 0, FH::kPhase0>(acc);
      interleave_mfma_reads<FH::kPhase0, FH::kReadInsts>();
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        if (b_due) lb.issue_one(sb, sb % kStages, kB, a.K, wave, q);
        f.template mma<1, 2 * q, 2>(acc);
      });
    }
    sched_fence();
    // Stage kt+1's last loads (its B half) left in iteration kt-1, or in the
    // prologue; younger than them are at most the 8 loads of stage kt+2, which
    // may stay in flight.  Any other vector memory operation issued after
    // them only makes this wait stricter: vector memory operations complete
    // in order.
    wait_stages_in_flight(min(KT - 2 - kt, 1));
    barrier();
    // Since the side work's previous step, this wave has issued exactly the
    // 8 stage loads of stage kt+2 (if that stage exists).
    side.step(a, wave, lane, kt + 2 < KT);
    if constexpr (FH::kBf16) {
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        if (a_due) la.issue_one(sa, sa % kStages, 0, a.K, wave, q);
        f.template read_part<0, q, 4>(nslot);
        f.template mma<2, 4 * q, 4>(acc);
        interleave_mfma_reads<4, FH::kReadInsts / 4>();
      });
    } else {
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        if (a_due) la.issue_one(sa, sa % kStages, 0, a.K, wave, q);
        f.template read_part<0, q, 4>(nslot);
        f.template mma<2, q, 1>(acc);
        interleave_mfma_reads<1, FH::kReadInsts / 2>();
      });
    }
  }
  // Every wave is done with the ring before anyone reuses it.
  sched_fence();
  wait_lgkmcnt<0>();
  barrier();
}

}  // namespace migemm
