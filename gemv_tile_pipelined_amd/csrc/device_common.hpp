// device_common.hpp -- small gfx950 device primitives shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace gt {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// The kernels move 16-bit patterns and carry them in _Float16 containers
// whatever the element format (kF16 / kBF16, kernels.hpp); only the
// arithmetic (MFMA, dot) and the final rounding depend on it.

// FP32 -> the 16-bit output format, round to nearest even (v_cvt_f16_f32 /
// v_cvt_pk_bf16_f32), returned as a 16-bit pattern in a _Float16 container.
template <int DT>
__device__ inline _Float16 round_out(float x) {
  if constexpr (DT == kF16) return static_cast<_Float16>(x);
  else return __builtin_bit_cast(_Float16, static_cast<__bf16>(x));
}

// A 16-bit pattern of the element format, widened to FP32 (exact).
template <int DT>
__device__ inline float widen_in(uint16_t bits) {
  if constexpr (DT == kF16) return static_cast<float>(__builtin_bit_cast(_Float16, bits));
  else return __builtin_bit_cast(float, static_cast<uint32_t>(bits) << 16);
}

// The fused epilogue's activation: +0 for v < 0, else v (a NaN stays NaN).
__device__ inline float relu_act(float v) { return v < 0.0f ? 0.0f : v; }

#define GT_LDS __attribute__((address_space(3)))

// Byte offset of a __shared__ object inside the workgroup's LDS allocation.
__device__ inline uint32_t lds_addr(const void *p) {
  // A C-style cast from a generic pointer to address space 3 is an
  // address-space cast; the result is the 32-bit LDS byte address.
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const GT_LDS char *)p));
}

// Buffer resource descriptor for raw, byte-addressed loads from
// [base, base + bytes).  Stride 0, no swizzle; dword 3 = 0x00020000 is the
// gfx9-family setting (32-bit data format).  A load whose offset is at or
// beyond `bytes` returns zeros: this is how edge tiles are zero-filled.
// The descriptor must be wave-uniform, so every field goes through
// readfirstlane and lives in scalar registers.
__device__ inline int4_t make_buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  int4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r.w = 0x00020000;
  return r;
}

// An offset no valid buffer in this library reaches (all are < 2^31 bytes):
// a load from it returns zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

// One wave-wide direct-to-LDS load: lane i fetches 16 bytes from
// rsrc.base + voffset(i) and the hardware writes them to LDS at
// lds_base + 16*i (M0 holds lds_base), so one instruction fills 1 KiB of LDS
// without passing through VGPRs.  Completion is tracked by the wave's vmcnt.
//
// Issued as inline asm on purpose: the compiler treats its own LDS-DMA
// builtins as possibly aliasing every later LDS read and then waits for
// vmcnt(0) before each one, which would serialise the multi-stage ring.  The
// ring does its own vmcnt accounting instead.  The s_nop covers the one wait
// state required between writing M0 and an LDS-DMA instruction.
//
// M0 is written and used inside one asm statement, so no value of M0 lives
// across statements.  The compiler reserves M0 and warns that clobbering it
// may be unsafe: it would be if compiler-generated code kept a value in M0
// across one of these statements.  build.py checks the generated code of
// every kernel that uses this load and fails the build if any instruction
// outside these statements reads or writes M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// POLICY selects the cache-policy modifier of the load: 0 none, 2 nt
// (streamed: data read once).
template <int POLICY = 0>
__device__ inline void lds_dma_b128(int4_t rsrc, uint32_t voffset, uint32_t lds_base) {
  static_assert(POLICY == 0 || POLICY == 2, "cache policy");
  if constexpr (POLICY == 0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 : : "v"(voffset), "s"(lds_base), "s"(rsrc) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
                 : : "v"(voffset), "s"(lds_base), "s"(rsrc) : "memory", "m0");
  }
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `younger` K tiles of PER loads each are still pending
// (loads complete in issue order); `younger` is in [0, MAXY].  vmcnt takes
// an immediate, hence the unrolled choice.
template <int PER, int MAXY>
__device__ inline void wait_younger(int younger) {
  if constexpr (MAXY > 0) {
    if (younger >= MAXY) {
      wait_vmcnt<MAXY * PER>();
      return;
    }
    wait_younger<PER, MAXY - 1>(younger);
  } else {
    wait_vmcnt<0>();
  }
}

// Wait until all LDS reads and writes of this wave have completed.
__device__ inline void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier with no implied memory waits (the callers place the
// vmcnt / lgkmcnt waits they need right before it).  The "memory" clobber
// keeps the compiler from moving LDS accesses across it.
__device__ inline void workgroup_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace gt
