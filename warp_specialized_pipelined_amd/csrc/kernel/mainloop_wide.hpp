// mainloop_wide.hpp -- the bf16 K loop with 64-deep stages: a 2-slot LDS
// ring of 64 KiB stages, 64 k (128 bytes) per row of each operand tile.
//
// The same producer/consumer ring as mainloop.hpp (LDS-DMA loads, own vmcnt
// plus one workgroup barrier per stage; see the comment there for how the
// pages' TMA/mbarrier ring maps onto gfx950), with twice the K per stage:
//   - a K-contiguous operand is read in 128-byte row segments (8 lanes per
//     row), so both 64-byte halves of every line leave in one instruction and
//     the L1 turns them into one L2 request; with 64-byte segments every
//     line costs two (measured on this path: L1 misses and L2 requests drop
//     by a third, and the address path stops stalling on the L1);
//   - one barrier per 64 k instead of per 32.
// With 2 slots, stage d+2 can only be loaded once every wave is done reading
// stage d.  The last k-step's fragments are read under the third k-step's
// MFMAs, so the barrier can sit after 48 of the stage's 64 MFMAs, once those
// reads have returned; the first k-step of stage d+1 (certified by the same
// barrier) is read under the last k-step's 16 MFMAs.  Stage d+2's 16 loads
// are spread over the 32 MFMAs from that barrier to the end of stage d+1's
// first k-step, and get at least 32 MFMAs to land.  How tightly the loads
// are packed decides much of the speed (8192^3, pairs timed on one device):
// packed into 16 MFMAs, one behind each, is 4% faster than into 8 MFMAs with
// two behind each, and spreading them over 32 MFMAs gains another 2-2.5%.
//
// LDS layout of one stage (64 KiB):  [A: 32 KiB][B: 32 KiB].
//   K-contiguous operand: 256 rows x 128 bytes of K; chunk c of row r is
//     stored at chunk c ^ ((r >> 1) & 7).
//   MN-contiguous operand: 4 panels of 64 columns, each holding the stage's
//     64 K rows of 128 bytes back to back; chunk c of K row k stored at
//     c ^ swz_mn(k), as in mainloop.hpp.
// Both keep every fragment read of a wave at a per-lane base plus an
// immediate offset, and the reads of one instruction on distinct banks.
#pragma once

#include "gfx950.hpp"
#include "mainloop.hpp"
#include "params.hpp"

namespace migemm {

constexpr int kWideRowBytes = 128;                        // K bytes per row per stage
constexpr int kWideK = kWideRowBytes / 2;                 // 64 bf16
constexpr int kWideOpBytes = kTileM * kWideRowBytes;      // 32 KiB
constexpr int kWideStageBytes = 2 * kWideOpBytes;         // 64 KiB
constexpr int kWideSlots = 2;
constexpr int kWidePanelBytes = kWideK * kPanelRowBytes;  // 8 KiB: 64 columns x 64 K rows
static_assert(kWideSlots * kWideStageBytes <= kStagingBytes, "ring must fit under the staging overlay");

__device__ __forceinline__ int swz_k8(int row) { return (row >> 1) & 7; }

// One operand's share of a wide stage: this wave's 8 LDS-DMA loads of 1 KiB.
template <bool KMAJ>
struct WideLoader {
  const unsigned char* tile_base;  // operand address of the tile's (row 0, k 0)
  int64_t kstep_bytes;             // address step from one stage of K to the next
  int64_t bytes_left;              // operand bytes from tile_base to its end
  uint32_t off[8];                 // this lane's byte offset for load j
  // The K index (within the stage) that this lane's load j starts at, kept
  // as the two values it takes (K-contiguous: by the parity of j) or as the
  // value for j = 0 (MN-contiguous: + 8 j), not as 8 registers.
  int32_t kq[2];
  __device__ __forceinline__ int32_t kpos(int j) const {
    if constexpr (KMAJ) return kq[j & 1];
    return kq[0] + 8 * j;
  }

  __device__ __forceinline__ void init(const void* ptr, int64_t bytes, int64_t ld, int64_t origin,
                                       int wave, int lane) {
    const unsigned char* p = static_cast<const unsigned char*>(ptr);
    if constexpr (KMAJ) {
      // Load idx = 8 wave + j covers rows 8 idx .. 8 idx + 7, 8 lanes a row.
      tile_base = p + origin * ld * 2;
      kstep_bytes = kWideRowBytes;
      bytes_left = bytes - origin * ld * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = (wave * 8 + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz_k8(row);
        off[j] = (uint32_t)(row * ld * 2) + (uint32_t)(c * 16);
      }
      // c * 8 for load j: swz_k8 of its row is 4 (j & 1) + (lane >> 4).
      kq[0] = ((lane & 7) ^ (lane >> 4)) * 8;
      kq[1] = ((lane & 7) ^ (4 + (lane >> 4))) * 8;
    } else {
      // Load idx = 8 wave + j fills K rows 8 (idx % 8) .. + 7 of panel idx / 8.
      tile_base = p + origin * 2;
      kstep_bytes = (int64_t)kWideK * ld * 2;
      bytes_left = bytes - origin * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = wave * 8 + j;
        const int krow = (idx % 8) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz_mn<2>(krow);
        const int col = (idx / 8) * 64 + chunk * 8;
        off[j] = (uint32_t)(krow * ld * 2) + (uint32_t)(col * 2);
      }
      kq[0] = lane >> 3;  // krow of load j is 8 j + (lane >> 3)
      kq[1] = 0;
    }
  }

  // Resource over the operand from K stage `kt` on, and the stage's valid K
  // (clamped: only "less than kWideK or not" matters).  Range rounded up to
  // 16 bytes, as in OperandLoader::stage_rsrc.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(int kt, int64_t K, int* krem) const {
    const int64_t step = (int64_t)kt * kstep_bytes;
    int64_t left = (bytes_left - step + 15) & ~(int64_t)15;
    left = left < 0 ? 0 : (left > 0x7FFFFFF0 ? 0x7FFFFFF0 : left);
    const int64_t krem64 = K - (int64_t)kt * kWideK;
    *krem = krem64 > kWideK ? kWideK : (int)krem64;
    return make_rsrc(tile_base + step, (uint32_t)left);
  }

  // Load j (0..7) into the stage slot at LDS offset `slot`.  Stages past K
  // load out of range (zeros into a free slot), like mainloop.hpp's.  With
  // MASK false the stage is known to be complete (krem == kWideK), and the
  // per-lane K check -- two VALU instructions in front of every load -- is
  // left out.
  template <bool MASK = true>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int krem, uint32_t slot, int wave,
                                       int j) const {
    dma16(r, lds_at(slot + (wave * 8 + j) * 1024),
          (!MASK || kpos(j) < krem) ? off[j] : kOobOffset);
  }
  __device__ __forceinline__ void load_all(int kt, uint32_t slot, int64_t K, int wave) const {
    int krem;
    const __amdgpu_buffer_rsrc_t r = stage_rsrc(kt, K, &krem);
#pragma unroll
    for (int j = 0; j < 8; ++j) load(r, krem, slot, wave, j);
  }
};

// Fragment reads from a wide stage (bf16; 4 k-steps of 16 per stage).
template <bool KMAJ>
struct WideReader;

// K-contiguous: one ds_read_b128; k-step ks is chunk 2 ks + (lane / 32).
template <>
struct WideReader<true> {
  static constexpr int kReads = 1;
  uint32_t off[4];  // per k-step
  __device__ __forceinline__ void init(int row0, int lane) {
    const int l = lane & 31;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      off[ks] = (row0 + l) * kWideRowBytes + (((2 * ks + (lane >> 5)) ^ swz_k8(l)) << 4);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ bf16x8 read(uint32_t opnd_base) const {
    return *reinterpret_cast<const MIGEMM_LDS bf16x8*>(
        lds_at(opnd_base + off[KS] + BLK * 32 * kWideRowBytes));
  }
};

// MN-contiguous: two ds_read_b64_tr_b16 per fragment.  Within each group of
// 16 lanes the instruction reads a 4 x 16 block of bf16 (lanes 4r..4r+3 each
// fetch 4 consecutive elements of row r) and hands lane i column i of the
// block.  Rows are K and columns are M or N here, so each lane receives 4
// consecutive k of its own column: lane l gets column l % 32 of the block and
// k = 8 (l / 32) + 0..3 (first read) and + 4..7 (second).  A 32-column block
// is one half of a 64-column panel; the swizzle flips which half depending on
// k, so even and odd blocks need one lane offset each.  k-step ks covers K
// rows 16 ks .. 16 ks + 15 of the panel (k + 16 ks and k + 4 keep swz_mn, so
// both are constant offsets).
template <>
struct WideReader<false> {
  static constexpr int kReads = 2;
  uint32_t off[2];  // for even and odd blocks
  __device__ __forceinline__ void init(int col0, int lane) {
    const int g = lane >> 4, t = lane & 15;
    const int k = 8 * (g >> 1) + (t >> 2);
    const int chunk = 2 * (g & 1) + ((t & 3) >> 1);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      off[b] = (col0 / 64) * kWidePanelBytes + k * kPanelRowBytes +
               (((4 * b + chunk) ^ swz_mn<2>(k)) << 4) + 8 * (t & 1);
  }
  template <int BLK, int KS>
  __device__ __forceinline__ bf16x8 read(uint32_t opnd_base) const {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    constexpr uint32_t c = (BLK >> 1) * kWidePanelBytes + 16 * KS * kPanelRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK & 1] + c));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MIGEMM_LDS i16x4*)lds_at(opnd_base + off[BLK & 1] + c + 4 * kPanelRowBytes));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// The fragments of two k-steps (buffer kb holds k-steps of parity kb): 4 A
// and 4 B fragments each, 64 VGPRs in all.
template <bool AK, bool BK>
struct WideFrags {
  typedef WideReader<AK> RA;
  typedef WideReader<BK> RB;
  static constexpr int kReadInsts = 4 * (RA::kReads + RB::kReads);  // per k-step
  bf16x8 a[2][4];
  bf16x8 b[2][4];
  RA ra;
  RB rb;

  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    ra.init(wm * kWaveTile, lane);
    rb.init(wn * kWaveTile, lane);
  }

  // Blocks [Q * 4 / NQ, (Q + 1) * 4 / NQ) of k-step KS into buffer KS & 1.
  template <int KS, int Q, int NQ>
  __device__ __forceinline__ void read_part(uint32_t a_base, uint32_t b_base) {
    static_for<Q * 4 / NQ, (Q + 1) * 4 / NQ>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      a[KS & 1][x] = ra.template read<x, KS>(a_base);
      b[KS & 1][x] = rb.template read<x, KS>(b_base);
    });
  }

  // MFMAs [FIRST, FIRST + COUNT) of the 16 of buffer KB: MFMA m is block
  // (m / 4) of A with block (m % 4) of B.
  template <int KB, int FIRST, int COUNT>
  __device__ __forceinline__ void mma(Accum& acc) const {
    static_for<FIRST, FIRST + COUNT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int i = m >> 2, j = m & 3;
      acc.v[i][j] = mfma<2>(b[KB][j], a[KB][i], acc.v[i][j]);
    });
  }
};

// The whole K loop of one output tile (bf16).  Stage d lives in slot d % 2.
// Stage d+2's loads go into stage d's slot, which is free from stage d's
// barrier on, and must have landed by stage d+1's barrier: 32 MFMAs of that
// window carry them, one load behind every other MFMA (A in stage d's last
// k-step, B in stage d+1's first).  One load blocks the issuing wave for a
// few dozen cycles, and the address path serves the four waves in turn, so
// loads packed closer than that stall the MFMA stream.
//   k-step 0: 16 MFMAs; k-step 1 read under the first 8, one A and one B
//             block at a time; B of stage d+1 loaded behind every other MFMA
//             (into stage d+1's slot);
//   k-steps 1, 2: 16 MFMAs each, under which the next k-step is read;
//   sync: wait until none of this wave's loads (only stage d+1's were in
//         flight) and none of its LDS reads is outstanding; barrier: stage
//         d+1 is in LDS for every wave, and every wave is done reading stage d;
//   the side work steps; k-step 3: 16 MFMAs; k-step 0 of stage d+1 read
//             under them; A of stage d+2 loaded behind every other MFMA (into
//             stage d's slot).
template <bool AK, bool BK, class SideWork>
__device__ __forceinline__ void mainloop_wide(Accum& acc, const KernelArgs& a, int tm, int tn,
                                              int wave, int lane, SideWork& side) {
  typedef WideFrags<AK, BK> FW;
  constexpr uint32_t kB = kWideOpBytes;
  WideLoader<AK> la;
  WideLoader<BK> lb;
  la.init(a.A, a.a_bytes, a.lda, (int64_t)tm * kTileM, wave, lane);
  lb.init(a.B, a.b_bytes, a.ldb, (int64_t)tn * kTileN, wave, lane);
  const int wm = wave >> 1, wn = wave & 1;
  int KT = (int)((a.K + kWideK - 1) / kWideK);
  asm volatile("" : "+s"(KT));  // opaque per tile (see mainloop)

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc.v[i][j] = f32x16{};

  FW f;
  f.init(wm, wn, lane);
  if (KT > 0) {
    // Prologue: stage 0 and stage 1's A in flight (stage 1's B is loaded in
    // the first iteration), stage 0 certified, its k-step 0 read.
    la.load_all(0, 0, a.K, wave);
    lb.load_all(0, kB, a.K, wave);
    la.load_all(1, kWideStageBytes, a.K, wave);
    wait_vmcnt<8>();
    barrier();
    f.template read_part<0, 0, 1>(0, kB);
  }
  auto iteration = [&](const int d, auto mask_c) {
    constexpr bool kMask = decltype(mask_c)::value;
    const uint32_t cur = (d & 1) * kWideStageBytes;
    const uint32_t nxt = ((d + 1) & 1) * kWideStageBytes;
    int krem_a, krem_b;
    const __amdgpu_buffer_rsrc_t ra = la.stage_rsrc(d + 2, a.K, &krem_a);
    const __amdgpu_buffer_rsrc_t rb = lb.stage_rsrc(d + 1, a.K, &krem_b);
    static_for<0, 16>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sched_fence();
      // k-step 1 read one A and one B block at a time, behind every other
      // MFMA (in two bursts of six reads it was 1% slower).
      if constexpr (m % 2 == 0 && m < 8) f.template read_part<1, m / 2, 4>(cur, cur + kB);
      f.template mma<0, m, 1>(acc);
      if constexpr (m & 1) lb.template load<kMask>(rb, krem_b, nxt + kB, wave, m >> 1);
    });
    static_for<1, 3>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      static_for<0, 2>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        sched_fence();
        f.template read_part<ks + 1, q, 2>(cur, cur + kB);
        f.template mma<ks & 1, 4 * q, 4>(acc);
        interleave_mfma_reads<4, FW::kReadInsts / 2>();
      });
      sched_fence();
      f.template mma<ks & 1, 8, 8>(acc);
    });
    sched_fence();
    // k-step 3's fragments are in registers: this wave is done reading stage
    // d once its reads have returned.
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier();
    // Anything the side work fetched after the previous barrier has landed.
    side.after_barrier(a, wave, lane);
    static_for<0, 16>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sched_fence();
      if constexpr (m % 2 == 0 && m >= 2 && m < 10)
        f.template read_part<0, (m - 2) / 2, 4>(nxt, nxt + kB);
      f.template mma<1, m, 1>(acc);
      if constexpr (m & 1) la.template load<kMask>(ra, krem_a, cur, wave, m >> 1);
      if constexpr (m == 9) side.template compute<0>(lane);
      if constexpr (m == 11) side.template compute<1>(lane);
      if constexpr (m == 13) side.template compute<2>(lane);
    });
  };
  // Iteration d loads B of stage d+1 and A of stage d+2.  While both stages
  // are complete, the loads need no K check; the last iterations (the K
  // tail and the stages past K, which only zero a free slot) keep it.  (The
  // two copies of the body must not push anything to scratch: a scratch
  // reload inside the loop waits for every stage load in flight.)
  int clean = (int)(a.K / kWideK) - 2;
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

}  // namespace migemm
