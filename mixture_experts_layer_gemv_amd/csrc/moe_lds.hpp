// Device helpers for streaming fragments from global memory into LDS with the
// gfx950 LDS-DMA load, shared by the grouped GEMM and the decode kernels.
//
// A 1 KiB fragment (64 lanes x 16 bytes) moves with one
// global_load_lds_dwordx4: lane l's 16 bytes land at LDS byte lds + 16 l, so
// the fragment is read back with one conflict-free ds_read_b128 per lane.
// The copies are inline assembly, so the compiler neither counts them in its
// own s_waitcnt bookkeeping nor adds conservative waits for them; the kernels
// order them with explicit vmcnt waits (vmcnt_imm) and ring_barrier().
// Vector-memory loads, copies into LDS included, complete in issue order for
// vmcnt, so "at most n operations outstanding" means every operation issued
// before the last n has landed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding copy (vmcnt(0)) and collapse the
// ring; the stage being consumed is waited for explicitly with vmcnt_imm.
// The wave's own LDS reads finish first (lgkmcnt(0)), so a stage it read is
// free once every wave has passed; the memory clobber keeps LDS accesses on
// their side of the barrier.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// global -> LDS copy of one fragment: lane l moves the 16 bytes at
// sbase + voff (a uniform base and its own 32-bit offset) into LDS byte
// address lds + 16 l.  The copy takes its LDS address from m0, a register the
// compiler reserves (and may hold a value of its own in), so m0 is saved in a
// scratch register first and restored right after the copy is issued (the
// copy reads m0 at issue).
__device__ __forceinline__ void copy_frag(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)p;
}

}  // namespace moe
