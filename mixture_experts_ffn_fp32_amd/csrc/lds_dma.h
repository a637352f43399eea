// Direct-to-LDS loading and synchronisation helpers shared by the pipelined
// MFMA kernels (gfx950).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n)&0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))
#define MOE_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14))

// One direct-to-LDS load: 16 bytes per lane from `base` + `off` (base
// wavefront-uniform) to LDS `wr` + 16 * lane.  It is issued as a buffer load
// (MUBUF) rather than a global one: the compiler counts a global (FLAT)
// direct-to-LDS load as a possible LDS access of unknown order and then
// waits for every outstanding LDS read (lgkmcnt(0)) before each MFMA that
// needs one; buffer loads keep its partial lgkmcnt waits exact.
// `nrec` bounds the offsets (bytes): 0 makes the load return zeros.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint8_t* __restrict__ wr,
                                      int nrec = 0x7fffffff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)wr, 16, off,
                                           0, 0, 0);
}

// Keeps a wavefront-uniform value in a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const uint8_t* uni(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(0) lgkmcnt(0), then a barrier without memory fences (the
// direct-to-LDS loads are ordered by the explicit wait instead).
__device__ __forceinline__ void pipe_sync() {
  MOE_WAIT_VMCNT(0);
  MOE_WAIT_LGKMCNT0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// LDS-only synchronisation: this wavefront's LDS operations are done, then a
// barrier.  Direct-to-LDS loads still in flight (into the other ring slot)
// are not waited for.
__device__ __forceinline__ void lds_sync() {
  MOE_WAIT_LGKMCNT0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Two float32 -> one word of two bfloat16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace
}  // namespace moe
