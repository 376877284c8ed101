// gfx950.hpp -- the CDNA4 primitives the GEMM is built from: vector types,
// buffer resources, direct global->LDS loads, wait counters, the workgroup
// barrier and the bf16 / fp8 MFMA instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace migemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MIGEMM_LDS __attribute__((address_space(3)))
typedef MIGEMM_LDS unsigned char lds_u8;

// Byte offset -> LDS pointer of the dynamic shared segment.
__device__ __forceinline__ lds_u8* lds_at(uint32_t byte_offset) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char migemm_smem[];
  return (lds_u8*)(migemm_smem) + byte_offset;  // generic -> LDS address space
}

// A raw buffer resource over [base, base + bytes).  Loads at offsets >= bytes
// return zero and stores there are dropped, which is how tile edges and the
// K tail are masked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// An offset no buffer resource here covers (resources are capped below 2^31).
constexpr uint32_t kOobOffset = 0x80000000u;

// 16 bytes per lane from global memory straight into LDS (buffer_load_dwordx4
// ... lds).  Lane i of the wave writes LDS bytes [lds + 16 i, lds + 16 i + 16);
// `lds` must be wave-uniform (it goes to M0).  Lanes whose offset is out of
// the resource's range write zeros.
//
// Issued as inline assembly on purpose: the compiler cannot prove that the
// transposing LDS reads of a stage do not alias the DMA writes still in
// flight into other stages, and would otherwise drain every outstanding load
// (vmcnt(0)) before each stage.  The ring orders these writes itself with
// explicit vmcnt waits and barriers.  Hidden loads only make the compiler's
// own vmcnt waits stricter, never looser, because vector memory operations
// complete in order.
//
// The compiler's hazard pass does not look inside inline assembly, so the
// wait states the gfx9 family requires before this instruction are part of
// it: 1 after the SALU write of M0 that the "{m0}" operand puts right in
// front of it, and 5 after a VALU write of an SGPR the load reads.  The
// latter happens when SGPRs run short and the resource comes back from a
// spill lane with v_readlane right before the load; without the wait the
// load can take a half-updated descriptor.  dma16 carries 2 wait states,
// for the K-loop stage loads, whose resources SALU code builds at the top of
// every iteration; dma16_w5_nt carries 5, for loads whose resource lives
// across the K loop (the tile consumer's).  tests/test_asm_hazards.py checks both
// rules on every LDS-DMA load of every kernel.  Each wait state costs the
// MFMA stream a cycle: 2 instead of 5 on the 16 stage loads of a stage is
// worth 2% on 8192^3 bf16.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 1\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
               "{m0}"(m0)
               : "memory");
}
// 5 wait states (see above) and the non-temporal hint (nt): for data read
// once, which should not displace the operand lines that other compute
// units still need from the L2.
__device__ __forceinline__ void dma16_w5_nt(__amdgpu_buffer_rsrc_t r, lds_u8* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voffset), "s"(r),
               "{m0}"(m0)
               : "memory");
}

// 5 wait states, default cache policy.
__device__ __forceinline__ void dma16_w5(__amdgpu_buffer_rsrc_t r, lds_u8* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
               "{m0}"(m0)
               : "memory");
}

// Cache-policy operand of the buffer load/store builtins: the non-temporal
// hint (nt) for data this kernel writes and does not read back soon; device
// scope (sc1) for data other XCDs read during the kernel -- the encoding of
// an agent-scope relaxed atomic load or store, which misses any stale copy
// in the XCD's private L2 and writes through it.
constexpr int kCpolNt = 2;
constexpr int kCpolDevice = 16;

// s_waitcnt encodings (gfx9 family): vmcnt in [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8].  A field at its maximum means "do not wait".
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 15));
}
template <int LGKM>
__device__ __forceinline__ void wait_lgkmcnt() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, LGKM));
}

// Compiler-level memory fence: no memory access is moved across it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// The workgroup barrier alone (no implied s_waitcnt; callers wait first).
__device__ __forceinline__ void barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l holds row l%32 of
// A and column l%32 of B, 8 consecutive k each; result lane l holds column
// l%32, rows 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32 fp32) += A(32x64 e4m3) * B(64x32 e4m3), no block scales.  Lane l
// holds 32 bytes (k values) of row l%32 of A and column l%32 of B.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace migemm
