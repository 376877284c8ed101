// ring_model.cpp -- a host model of the tile hand-off ring, with threads for
// waves, random delays, and the kernel's own counting rules
// (csrc/kernel/handoff_rules.hpp).  Built plain and under ThreadSanitizer by
// tests/test_ring_model.py.
//
// The protocol is CUTLASS issue #2900's producer acquire / store / commit
// and consumer wait / work / release around each finished tile, through
// kHandoffSlots slots that start free.  Each slot's payload here is a plain,
// non-atomic buffer that producers write (their quarter of the tile) and
// consumers read (all of it): it stands for the tile the slot carries, and
// the acquire/release order of the counters is all that separates those
// accesses -- a missing order is a data race ThreadSanitizer reports.
//
// Modes:
//   staged      the kernel's default schedule: each of the 4 waves, per tile,
//               runs its K loop (a barrier of all waves), acquires, stores its
//               quarter, commits, waits for all commits, reads the whole
//               tile, releases, and meets the others at the tile's closing
//               barrier;
//   overlapped  the kernel's MIGEMM_F_CONSUMER_OVERLAP schedule: tile n-1 is
//               read during tile n's K loop and released after tile n's
//               commit, so two committed tiles are in the ring at once;
//   split       the protocol alone, in the warp-specialized form the issue
//               describes: 4 producer threads and 4 consumer threads, no
//               shared barrier -- producers run ahead and must block at
//               depth kHandoffSlots.
// Checked: every payload read sees the tile it should; the tile id a
// consumer reads after its wait is that tile's; the ring never holds more
// than kHandoffSlots committed, unreleased tiles (overlapped reaches 2,
// staged stays at 1); the final counts; in split mode, that producers did
// block on a full ring.  Prints one line and exits 0, or names the first
// violation and exits 1.
//
//   ring_model MODE TILES SEED
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "handoff_rules.hpp"  // -I the kernel directory (or a copy, to plant a mistake)

using namespace migemm;

namespace {

constexpr int W = kWaves;
constexpr int S = kHandoffSlots;

struct Ring {
  std::atomic<uint32_t> full[S];
  std::atomic<uint32_t> empty[S];
  std::atomic<int> tile_id[S];
  int payload[S][W];  // plain: ordered only by the counters
};

Ring ring;
std::atomic<int> failures{0};
std::atomic<uint32_t> max_occupancy{0};
std::atomic<long> blocked_full{0};  // acquires that found the ring full

void fail(const char* what, int n, int w) {
  if (failures.fetch_add(1) == 0) std::printf("VIOLATION: %s (tile %d, thread %d)\n", what, n, w);
}

// A sense-reversing barrier of W threads (the kernel's s_barrier).
struct Barrier {
  std::atomic<int> count{0};
  std::atomic<int> phase{0};
  void wait() {
    const int ph = phase.load(std::memory_order_acquire);
    if (count.fetch_add(1, std::memory_order_acq_rel) == W - 1) {
      count.store(0, std::memory_order_relaxed);
      phase.store(ph + 1, std::memory_order_release);
    } else {
      while (phase.load(std::memory_order_acquire) == ph) std::this_thread::yield();
    }
  }
};
Barrier bar;

struct Rng {
  std::mt19937 g;
  void delay() {
    const unsigned r = g() % 64;
    if (r < 8) std::this_thread::yield();
    else
      for (volatile unsigned i = 0; i < r * 16; i = i + 1) {
      }
  }
};

void spin_until(std::atomic<uint32_t>& c, uint32_t target) {
  while (c.load(std::memory_order_acquire) < target) std::this_thread::yield();
}

uint32_t occupancy() {
  uint32_t occ = 0;
  for (int s = 0; s < S; ++s)
    occ += handoff_slot_occupancy(ring.full[s].load(std::memory_order_acquire),
                                  ring.empty[s].load(std::memory_order_acquire));
  return occ;
}

// Producer steps of tile n by wave (or producer thread) w.
void acquire(int n) {
  const int s = handoff_slot(n);
  const uint32_t target = handoff_acquire_target(handoff_use(n));
  if (ring.empty[s].load(std::memory_order_acquire) < target) {
    if (occupancy() >= (uint32_t)S) blocked_full.fetch_add(1);
    spin_until(ring.empty[s], target);
  }
}
void store_and_commit(int n, int w) {
  const int s = handoff_slot(n);
  ring.payload[s][w] = n;
  if (w == 0) ring.tile_id[s].store(n, std::memory_order_relaxed);
  ring.full[s].fetch_add(1, std::memory_order_release);
  const uint32_t occ = occupancy();
  if (occ > (uint32_t)S) fail("more committed, unreleased tiles than slots", n, w);
  uint32_t m = max_occupancy.load();
  while (occ > m && !max_occupancy.compare_exchange_weak(m, occ)) {
  }
}
// Consumer steps.
void wait_tile(int n, int w) {
  const int s = handoff_slot(n);
  spin_until(ring.full[s], handoff_wait_target(handoff_use(n)));
  if (ring.tile_id[s].load(std::memory_order_relaxed) != n) fail("tile id after wait", n, w);
}
void read_tile(int n, int w) {
  const int s = handoff_slot(n);
  for (int q = 0; q < W; ++q)
    if (ring.payload[s][q] != n) fail("payload overwritten or not yet stored", n, w);
}
void release(int n) {
  ring.empty[handoff_slot(n)].fetch_add(1, std::memory_order_release);
}

void staged(int w, int tiles, unsigned seed) {
  Rng r{std::mt19937(seed * 131 + w)};
  for (int n = 0; n < tiles; ++n) {
    r.delay();
    bar.wait();  // the K loop
    r.delay();
    acquire(n);
    r.delay();
    store_and_commit(n, w);
    wait_tile(n, w);
    r.delay();
    read_tile(n, w);
    release(n);
    bar.wait();  // the tile loop's closing barrier
  }
}

void overlapped(int w, int tiles, unsigned seed) {
  Rng r{std::mt19937(seed * 131 + w)};
  int pending = -1;
  for (int n = 0; n < tiles; ++n) {
    r.delay();
    if (pending >= 0) read_tile(pending, w);  // the copy inside the K loop
    bar.wait();
    r.delay();
    acquire(n);
    r.delay();
    store_and_commit(n, w);
    if (pending >= 0) {  // the drain: what the loop left, and the release
      read_tile(pending, w);
      release(pending);
    }
    wait_tile(n, w);
    r.delay();
    read_tile(n, w);  // the fold
    pending = n;
    bar.wait();
  }
  if (pending >= 0) {  // the last tile
    read_tile(pending, w);
    release(pending);
  }
}

void split_producer(int w, int tiles, unsigned seed) {
  Rng r{std::mt19937(seed * 131 + w)};
  for (int n = 0; n < tiles; ++n) {
    r.delay();
    acquire(n);
    store_and_commit(n, w);
  }
}
void split_consumer(int w, int tiles, unsigned seed) {
  Rng r{std::mt19937(seed * 977 + w)};
  for (int n = 0; n < tiles; ++n) {
    wait_tile(n, w);
    r.delay();
    r.delay();
    read_tile(n, w);
    release(n);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    std::printf("usage: ring_model staged|overlapped|split TILES SEED\n");
    return 2;
  }
  const char* mode = argv[1];
  const int tiles = std::atoi(argv[2]);
  const unsigned seed = (unsigned)std::atoi(argv[3]);
  for (int s = 0; s < S; ++s) {
    ring.full[s] = 0;
    ring.empty[s] = 0;
    ring.tile_id[s] = -1;
    for (int w = 0; w < W; ++w) ring.payload[s][w] = -1;
  }
  std::vector<std::thread> th;
  if (!std::strcmp(mode, "staged")) {
    for (int w = 0; w < W; ++w) th.emplace_back(staged, w, tiles, seed);
  } else if (!std::strcmp(mode, "overlapped")) {
    for (int w = 0; w < W; ++w) th.emplace_back(overlapped, w, tiles, seed);
  } else if (!std::strcmp(mode, "split")) {
    for (int w = 0; w < W; ++w) th.emplace_back(split_producer, w, tiles, seed);
    for (int w = 0; w < W; ++w) th.emplace_back(split_consumer, w, tiles, seed);
  } else {
    std::printf("unknown mode %s\n", mode);
    return 2;
  }
  for (auto& t : th) t.join();
  // Every slot committed and released by every wave, once per use.
  for (int s = 0; s < S; ++s) {
    const uint32_t uses = (uint32_t)((tiles - s + S - 1) / S);
    if (ring.full[s].load() != uses * W || ring.empty[s].load() != uses * W)
      fail("final counts", s, -1);
  }
  const uint32_t occ = max_occupancy.load();
  if (!std::strcmp(mode, "staged") && occ > 1) fail("staged ring held 2 tiles", -1, -1);
  if (!std::strcmp(mode, "overlapped") && tiles > 1 && occ != 2)
    fail("overlapped ring never held 2 tiles", -1, -1);
  if (!std::strcmp(mode, "split") && tiles > 8 && blocked_full.load() == 0)
    fail("no producer ever blocked on a full ring", -1, -1);
  if (failures.load()) return 1;
  std::printf("ring_model OK mode=%s tiles=%d max_occupancy=%u blocked_on_full=%ld\n", mode, tiles,
              occ, blocked_full.load());
  return 0;
}
