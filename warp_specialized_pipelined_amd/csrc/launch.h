// launch.h -- internal interface between the host plan layer (api.cpp) and
// the kernel translation unit (gemm_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel/params.hpp"

namespace migemm {

struct KernelSelect {
  int elem_bytes;   // 2: bf16 operands, 1: e4m3 operands
  bool a_kmajor;    // A is K-contiguous
  bool b_kmajor;    // B is K-contiguous
  bool consumer;    // tile hand-off + consumer stage
  bool consumer_overlap;  // the consumer stage inside the next tile's K loop
  bool stream_k;    // stream-K units after the whole tiles (not with consumer)
  int tile_m;       // 256, or 192 (bf16 whole tiles without consumer only)
};

// Dynamic LDS the selected kernel uses.
int kernel_lds_bytes(const KernelSelect& sel);

// Raise the kernel's dynamic-LDS limit to what it uses (once per process).
hipError_t prepare_kernel(const KernelSelect& sel);

// Enqueue one persistent GEMM kernel on `stream` with `grid` workgroups.
hipError_t launch_gemm(const KernelSelect& sel, const KernelArgs& args, int grid, hipStream_t stream);

// Enqueue a kernel that sets n 32-bit words at p to zero.
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream);

// The device address of the fixed scratch array (kNoAllocScratchBytes) on
// `device`, which must be the current device.  Looked up once per device.
hipError_t no_alloc_scratch(int device, void** out);

}  // namespace migemm
