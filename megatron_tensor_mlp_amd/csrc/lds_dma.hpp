// Direct HBM -> LDS loads and the explicit waits and barriers that go with
// them (gfx950).
//
// Hazard: on this GPU family a vector memory instruction that reads an SGPR
// written by a VALU instruction (the descriptor bases below come from
// v_readfirstlane) needs 5 wait states in between, and an LDS DMA that reads
// M0 right after an SALU write of M0 needs 1.  The compiler inserts those
// wait states for the memory instructions it emits, but it cannot see into
// the asm statements below, and it may schedule the descriptor's
// v_readfirstlane one or two instructions before them; so every load here
// begins with s_nop 4 (5 wait states) of its own.
//
// A buffer load with the `lds` modifier writes the data of lane i straight to
// LDS at m0 + size * i, without passing through registers.  The loads are
// issued as inline asm so that the compiler adds no waits of its own for them:
// a kernel that uses them waits with explicit s_waitcnt immediates before the
// barrier that publishes a stage, and the compiler, which does not see the
// loads, neither delays nor reorders around them beyond the asm's memory
// clobber.  Lanes whose data lies outside the matrix get an offset at or past
// OOB, which the buffer range check turns into zeros without touching memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpmlp {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer range: reads as zero
constexpr int RSRC_WORD3 = 0x00020000;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= v only.
constexpr int wait_vm(int v) { return (v & 15) | (7 << 4) | (15 << 8) | ((v >> 4) << 14); }
// ... and for lgkmcnt == 0 as well.
constexpr int wait_vm_lgkm0(int v) { return (v & 15) | (7 << 4) | ((v >> 4) << 14); }

// Buffer descriptor of a raw (stride 0) buffer starting at `base` whose range
// covers every offset below 2^31; offsets at or past OOB read as zero.
__device__ __forceinline__ i32x4 rsrc(const void *base) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = 0x7fffffff;
  r[3] = RSRC_WORD3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_dst + 16 * lane.
__device__ __forceinline__ void dma16(const i32x4 &rs, const void *lds_dst, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst)))
               : "memory");
}

// The same with the nontemporal hint, for data read exactly once (streamed
// weights): the lines are not kept in the caches, so they do not displace data
// that is reused.
__device__ __forceinline__ void dma16_nt(const i32x4 &rs, const void *lds_dst, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst)))
               : "memory");
}

// 4 bytes per lane from buffer offset `voff` into LDS at lds_dst + 4 * lane.
__device__ __forceinline__ void dma4(const i32x4 &rs, const void *lds_dst, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst)))
               : "memory");
}

// Barrier between the waves of the workgroup with no memory fence: the waits
// it needs are issued explicitly before it.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace tpmlp
