// handoff_rules.hpp -- the counting rules of the tile hand-off ring, as plain
// constexpr arithmetic: the kernel's HandoffRing (handoff.hpp) and the host
// model of the ring in the tests (tests/ring_model.cpp) both use these.
//
// CUTLASS issue #2900 ("How to build a pipeline between epilogue and
// communication warp groups?") asks for a producer acquire / store / commit
// and a consumer wait / work / release around every finished tile, through
// a ring of slots; the kernel page starts the producer's pipeline state at
// the opposite phase, so that the first use of each slot passes at once.
// Here each slot keeps two monotone counters, full and empty, each counted
// once per wave:
//   - tile n of a workgroup goes through slot n % kHandoffSlots, for the
//     (n / kHandoffSlots)-th time: its use u;
//   - acquire(u) passes once empty >= u * waves, i.e. every wave has
//     released the slot's previous u uses (use 0 passes at once);
//   - commit adds one to full per wave; wait(u) passes once full >=
//     (u + 1) * waves, i.e. every wave has committed use u;
//   - release adds one to empty per wave.
#pragma once

#include <stdint.h>

#include "params.hpp"

namespace migemm {

constexpr int handoff_slot(int n) { return n % kHandoffSlots; }
constexpr uint32_t handoff_use(int n) { return (uint32_t)(n / kHandoffSlots); }
constexpr uint32_t handoff_acquire_target(uint32_t use) { return use * (uint32_t)kWaves; }
constexpr uint32_t handoff_wait_target(uint32_t use) { return (use + 1) * (uint32_t)kWaves; }
// Tiles of one slot committed by every wave and not yet released by every
// wave.
constexpr uint32_t handoff_slot_occupancy(uint32_t full, uint32_t empty) {
  return full / (uint32_t)kWaves - empty / (uint32_t)kWaves;
}

}  // namespace migemm
