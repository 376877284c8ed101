// mainloop.hpp -- the e4m3 K loop: an N-stage LDS ring filled by direct
// global->LDS buffer loads, drained by the MFMA core; and the pieces every K
// loop shares (swizzles, panels, MFMA wrappers, accumulator tile, scheduling
// helpers).  bf16 runs the 64-deep-stage loop of mainloop_wide.hpp.
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
//     of row r stored in the order c ^ swz_k(r).
//   MN-contiguous operand: panels of 128 bytes of M or N (128 e4m3
//     columns), each panel holding the stage's 64 K rows back to back, with
//     the 16-byte chunks of row k permuted by swz_mn(k).
// Both swizzles make the fragment reads of one instruction hit every LDS
// bank equally often (measured on gfx950: a K-major 16-byte read then takes
// ~4.5 cycles per instruction instead of 8, and a transposing read ~3.8
// instead of 4.5-8).  They are applied on the global side: LDS-DMA writes
// lane i's 16 bytes to a fixed LDS slot, so each lane fetches the chunk that
// belongs in its slot.
//
// Global side: every LDS-DMA instruction reads whole 128-byte segments (8
// lanes) for MN-contiguous operands.  The memory pipeline serves requests,
// not bytes: loads made of 64-byte segments reach only about half the L2 and
// HBM throughput of 128-byte ones (measured: ~18 vs ~36 TB/s from L2 over
// the chip).  K-contiguous operands read 64-byte segments (one stage holds
// 64 bytes of K per row).
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

// K-contiguous: chunk c of row r is stored at chunk c ^ swz_k(r).  Rows of
// a fragment block start 32 rows apart, so the value depends on the lane
// alone.
__device__ __forceinline__ int swz_k(int row) { return (row >> 2) & 3; }

// MN-contiguous: a panel row is 128 bytes of M or N; chunk c of K row k is
// stored at chunk c ^ swz_mn(k).  bf16 swaps the 64-byte halves of every
// other pair of rows; e4m3 permutes the four 32-byte pieces.
template <int ES>
__device__ __forceinline__ int swz_mn(int k) {
  return ES == 2 ? ((k >> 1) & 1) << 2 : ((k >> 1) & 3) << 1;
}
constexpr int kPanelRowBytes = 128;
template <int ES>
struct Panel {
  static constexpr int kCols = kPanelRowBytes / ES;             // 64 or 128
  static constexpr int kRows = kStageKBytes / ES;               // K rows: 32 or 64
  static constexpr int kBytes = kRows * kPanelRowBytes;         // 4 or 8 KiB
  static constexpr int kLoadsPerPanel = kBytes / 1024;          // 4 or 8
};

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
      // Load idx = 4 * wave + j fills K rows 8 (idx % L) .. + 7 of panel
      // idx / L (L loads per panel): 8 lanes per 128-byte row.
      typedef Panel<ES> P;
      tile_base = p + origin * ES;
      kstep_bytes = (int64_t)kBK * ld * ES;
      bytes_left = bytes - origin * ES;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = wave * 4 + j;
        const int krow = (idx % P::kLoadsPerPanel) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_mn<ES>(krow);
        const int col = (idx / P::kLoadsPerPanel) * P::kCols + chunk * kElemsPerChunk;
        off[j] = (uint32_t)(krow * ld * ES) + (uint32_t)(col * ES);
        kpos[j] = krow;
      }
    }
  }

  // A buffer resource over the operand from K stage `kt` on, and the K
  // elements left in that stage (clamped: only "less than kBK or not"
  // matters).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(int kt, int64_t K, int* krem) const {
    const int64_t step = (int64_t)kt * kstep_bytes;
    // Buffer range checks work per dword, so an operand whose last row ends
    // inside a dword would lose its last element: round the range up to 16
    // bytes.  The base is 16-byte aligned, so the extra bytes share the last
    // element's 16-byte block (and page) and only feed discarded columns.
    int64_t left = (bytes_left - step + 15) & ~(int64_t)15;
    left = left < 0 ? 0 : (left > 0x7FFFFFF0 ? 0x7FFFFFF0 : left);
    const int64_t krem64 = K - (int64_t)kt * kBK;
    *krem = krem64 > kBK ? kBK : (int)krem64;
    return make_rsrc(tile_base + step, (uint32_t)left);
  }

  // Load j (0..3) of this wave's 4 loads of a stage, from the stage's
  // resource `r` into the stage slot at LDS offset `slot`.  A stage past
  // the end of K (empty resource) still issues its loads: they fall out of
  // range and write zeros, which keeps the count of loads per iteration
  // fixed; the slot they fill holds no live stage.
  // With MASK false the stage is known to be complete and the per-lane K
  // check (two VALU instructions) is left out.
  template <bool MASK = true>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int krem, uint32_t slot, int wave,
                                       int j) const {
    dma16(r, lds_at(slot + (wave * 4 + j) * 1024),
          (!MASK || kpos[j] < krem) ? off[j] : kOobOffset);
  }
  __device__ __forceinline__ void load_all(int kt, uint32_t slot, int64_t K, int wave) const {
    int krem;
    const __amdgpu_buffer_rsrc_t r = stage_rsrc(kt, K, &krem);
#pragma unroll
    for (int j = 0; j < 4; ++j) load(r, krem, slot, wave, j);
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

// MN-contiguous e4m3: four ds_read_b64_tr_b8 per fragment.  Within each
// group of 16 lanes the instruction reads an 8 x 16 block of bytes (lanes 2r
// and 2r+1 fetch the two halves of row r) and hands lane i column i, i.e. 8
// consecutive k of its own column: lane l gets column l % 32 of the block and
// k = 32 (l / 32) + 8 h + 0..7 from read h.  A 32-column block is one 32-byte
// piece of a 128-column panel, placed by the swizzle, so each of a wave's
// four blocks has its own lane offset.
template <>
struct FragReader<1, false> {
  typedef i32x8 frag_t;
  static constexpr int kSteps = 1;
  static constexpr int kReads = 4;
  uint32_t off[4];  // per block
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 32 * (g >> 1) + (t >> 1);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      off[b] = (col0 / 128) * Panel<1>::kBytes + k * kPanelRowBytes +
               (((2 * b + (g & 1)) ^ swz_mn<1>(k)) << 4) + 8 * (t & 1);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ frag_t read(uint32_t opnd_base) const {
    i32x8 v;
    // k + 8 h keeps swz_mn, so the four reads are constant offsets apart.
    static_for<0, 4>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (MIGEMM_LDS i32x2*)lds_at(opnd_base + off[BLK] + 8 * h * kPanelRowBytes));
      v[2 * h] = w[0];
      v[2 * h + 1] = w[1];
    });
    return v;
  }
};

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

// The e4m3 fragments one wave needs from one stage, in two halves of 32
// VGPRs so that one half can be refilled while the MFMAs of the other run:
// half h = A fragments {2h, 2h+1} and B fragments {2h, 2h+1} (32 bytes each;
// the stage is a single k-step).  MFMA (i, j) needs A half i/2 and B half
// j/2, and the four phases are
//   phase 0: A0 B0,  phase 1: A1 B0,  phase 2: A0 B1,  phase 3: A1 B1,
// so B half 0 is free after phase 1 and A half 0 after phase 2.
template <int ES, bool AK, bool BK>
struct FragHalves {
  static_assert(ES == 1, "bf16 runs mainloop_wide.hpp");
  typedef FragReader<ES, AK> RA;
  typedef FragReader<ES, BK> RB;
  static constexpr int kPerHalf = 2;   // A (and B) fragments per half
  typename RA::frag_t a[2][kPerHalf];
  typename RB::frag_t b[2][kPerHalf];
  RA ra;
  RB rb;

  // LDS read instructions of one half.
  static constexpr int kReadInsts = kPerHalf * (RA::kReads + RB::kReads);

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    ra.init(wm * kWaveTile, lane);
    rb.init(wn * kWaveTile, lane);
  }

  // Fragments [Q * kPerHalf / NQ, (Q + 1) * kPerHalf / NQ) of half H from
  // the stage slots at LDS offsets a_base (A) and b_base (B).
  // OPS: 1 = A only, 2 = B only, 3 = both.
  template <int H, int Q, int NQ, int OPS = 3>
  __device__ __forceinline__ void read_part(uint32_t a_base, uint32_t b_base) {
    static_for<Q * kPerHalf / NQ, (Q + 1) * kPerHalf / NQ>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      constexpr int blk = 2 * H + x;  // of the stage's single k-step
      if constexpr ((OPS & 1) != 0) a[H][x] = ra.template read<blk, 0>(a_base);
      if constexpr ((OPS & 2) != 0) b[H][x] = rb.template read<blk, 0>(b_base);
    });
  }

  // MFMAs [FIRST, FIRST + COUNT) of phase P (all indices compile-time, so
  // every fragment and accumulator stays in registers).
  template <int P, int FIRST, int COUNT>
  __device__ __forceinline__ void mma(Accum& acc) const {
    static_for<FIRST, FIRST + COUNT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int ha = P & 1, hb = P >> 1;  // A and B half of this phase
      constexpr int i = 2 * ha + (m >> 1), j = 2 * hb + (m & 1);
      acc.v[i][j] = mfma<ES>(b[hb][m & 1], a[ha][m >> 1], acc.v[i][j]);
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

// Keeps the compiler from moving any instruction across this point, so the
// phases of the K loop stay in the order written.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Work that rides along in the K loop.  Once per iteration, right after the
// barrier (before the iteration's stage loads), after_barrier() issues what
// the work needs from memory; its arithmetic comes in pieces,
// compute<P>() for P = 0 .. 2, placed between the MFMAs that follow, so that
// it fills issue slots instead of holding the MFMA pipe.
struct NoSideWork {
  __device__ __forceinline__ void after_barrier(const KernelArgs&, int, int) {}
  template <int P>
  __device__ __forceinline__ void compute(int) {}
};

// The whole e4m3 K loop of one output tile.
//
// Iteration kt works on stage kt, whose half-0 fragments were read during the
// previous iteration.  The workgroup barrier in the middle certifies stage
// kt+1 (one ahead):
//   before:  MFMAs on what is already in registers, under which the rest of
//            stage kt is read: A0B0 with the half-1 reads, then A1B0;
//   sync:    wait until only the previous iteration's 8 loads are in flight
//            -- those of stage kt+2 -- so this wave's loads of stage kt+1 have
//            landed; barrier: now stage kt+1 is in LDS for every wave, and
//            every wave is done reading stage kt-1;
//   after:   the side work steps once; A0B1 and A1B1, each MFMA followed by
//            one of the 8 loads of stage kt+3 (into stage kt-1's slot), with
//            stage kt+1's half-0 reads between the two phases.
// Fragment reads are issued early in their phase so that they have landed
// before anything waits for them (the compiler waits for every LDS read at
// the top of the loop).  Each stage gets two iterations to land.  Loads of
// stages past K fall out of range and only zero a free slot, so every
// iteration issues exactly 8 loads per wave.  (Spreading a stage's loads
// over two iterations was measured to be slower: it costs more in latency
// budget than it gains in issue smoothness.)
template <int ES, bool AK, bool BK, class SideWork>
__device__ __forceinline__ void mainloop(Accum& acc, const KernelArgs& a, int tm, int tn, int wave,
                                         int lane, SideWork& side) {
  static_assert(kStages == 4, "the certify-ahead ring is written for 4 stages");
  static_assert(ES == 1, "bf16 runs mainloop_wide");
  typedef FragHalves<ES, AK, BK> FH;
  constexpr int kBK = kStageKBytes / ES;
  constexpr uint32_t kB = kOperandStageBytes;
  OperandLoader<ES, AK> la;
  OperandLoader<ES, BK> lb;
  la.init(a.A, a.a_bytes, a.lda, (int64_t)tm * kTileM, wave, lane);
  lb.init(a.B, a.b_bytes, a.ldb, (int64_t)tn * kTileN, wave, lane);
  const int wm = wave >> 1, wn = wave & 1;
  int KT = (int)((a.K + kBK - 1) / kBK);
  // Opaque per tile, like the lane ids: tests on KT are then made where they
  // are used, not once before the tile loop and held (or spilled, and
  // reloaded with a vmcnt(0)) across it.
  asm volatile("" : "+s"(KT));

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][j] = f32x16{};

  FH f;
  f.init(wm, wn, lane);
  if (KT > 0) {
    // Prologue: stages 0..2 in flight, stage 0 certified, its half 0 read.
    for (int s = 0; s < kStages - 1; ++s) {
      la.load_all(s, s * kStageBytes, a.K, wave);
      lb.load_all(s, s * kStageBytes + kB, a.K, wave);
    }
    wait_vmcnt<16>();
    barrier();
    f.template read_part<0, 0, 1>(0, kB);
  }
  // Every iteration has the same shape (no branch around MFMAs, so the
  // accumulators never meet at a join): in the last ones the barrier is
  // redundant and the half-0 read fetches bytes nobody uses.  Iterations
  // whose loaded stage (kt+3) lies inside K run a copy of the body without
  // the loads' per-lane K check.
  auto iteration = [&](const int kt, auto mask_c) {
    constexpr bool kMask = decltype(mask_c)::value;
    const uint32_t cur = (kt % kStages) * kStageBytes;
    const uint32_t nxt = ((kt + 1) % kStages) * kStageBytes;
    const uint32_t s3 = ((kt + 3) % kStages) * kStageBytes;
    int krem_a, krem_b;
    const __amdgpu_buffer_rsrc_t ra = la.stage_rsrc(kt + 3, a.K, &krem_a);
    const __amdgpu_buffer_rsrc_t rb = lb.stage_rsrc(kt + 3, a.K, &krem_b);
    sched_fence();
    f.template read_part<1, 0, 1, 1>(cur, cur + kB);  // A half 1 first: phase 1 needs it
    f.template read_part<1, 0, 1, 2>(cur, cur + kB);
    f.template mma<0, 0, 4>(acc);
    interleave_mfma_reads<4, FH::kReadInsts>();
    sched_fence();
    f.template mma<1, 0, 4>(acc);
    sched_fence();
    wait_vmcnt<8>();
    barrier();
    // Anything the side work fetched in the previous iteration left just
    // before that iteration's 8 loads, so the wait above covered it.
    side.after_barrier(a, wave, lane);
    // A0B1 (B half 0 is free now), one A load behind each MFMA, then B
    // half 0 of stage kt+1.
    static_for<0, 4>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      sched_fence();
      f.template mma<2, q, 1>(acc);
      la.template load<kMask>(ra, krem_a, s3, wave, q);
    });
    sched_fence();
    f.template read_part<0, 0, 1, 2>(nxt, nxt + kB);
    side.template compute<0>(lane);
    // A1B1 (A half 0 is free now), with A half 0 of stage kt+1 read first,
    // one B load behind each MFMA.
    sched_fence();
    f.template read_part<0, 0, 1, 1>(nxt, nxt + kB);
    static_for<0, 4>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      sched_fence();
      f.template mma<3, q, 1>(acc);
      lb.template load<kMask>(rb, krem_b, s3 + kB, wave, q);
      if constexpr (q == 1) side.template compute<1>(lane);
      if constexpr (q == 3) side.template compute<2>(lane);
    });
  };
  int clean = (int)(a.K / kBK) - 3;
  clean = clean < 0 ? 0 : (clean > KT ? KT : clean);
  int kt = 0;
  for (; kt < clean; ++kt) iteration(kt, std::integral_constant<bool, false>{});
  for (; kt < KT; ++kt) iteration(kt, std::integral_constant<bool, true>{});
  // Every wave is done with the ring, and every load into it (including the
  // zero-filling ones past K) has landed, before anyone reuses it.
  sched_fence();
  wait_vmcnt<0>();
  wait_lgkmcnt<0>();
  barrier();
}

}  // namespace migemm
