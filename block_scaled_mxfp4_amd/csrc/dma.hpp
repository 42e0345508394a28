// Global -> LDS DMA on gfx950 and the waits around it, shared by the
// LDS-staged GEMM kernels (prefill.hip).
//
// A DMA (buffer_load ... lds) moves each lane's `size` bytes from a buffer
// straight to LDS address m0 + size * lane, without passing through
// registers; a lane whose offset lies past the buffer's size writes zeros.
// The instructions are issued as inline assembly so that the compiler, which
// cannot tell which LDS stage a DMA fills, adds no waits of its own to the
// stage reads; every stage read is preceded by a wait on this wave's
// vector-memory counter (loads return in issue order, so "at most N
// outstanding" means every DMA older than the last N has landed) and a
// workgroup barrier, which covers the other waves' DMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace situ {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// Tables written by earlier kernels and only read here: through the constant
// address space, uniform indices become scalar loads, whose waits (lgkmcnt)
// never drain the DMA ring.
typedef const __attribute__((address_space(4))) int32_t* cptr;

constexpr uint32_t kOobOff = 0x80000000u;   // an offset past every buffer: reads 0, drops writes

// Buffer resource as four SGPR words: base, stride 0, size in bytes, the
// gfx950 raw-buffer flags.
__device__ __forceinline__ v4i rsrc4(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) { return (uint32_t)(uintptr_t)(lds_u8*)p; }

// m0 is written one wait state before the DMA that reads it.
__device__ __forceinline__ void dma16(const v4i& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const v4i& r, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r) : "memory", "m0");
}

// The same with a wave-uniform byte offset added in the instruction's scalar
// offset field, so that a lane's vector offset can be shared by requests
// that differ only by uniform amounts.  A vector offset of kOobOff keeps the
// request past its buffer (it reads zeros) whether or not the range check
// counts the scalar offset: the scalar offsets used are below 2^31, so the
// sum cannot wrap.
__device__ __forceinline__ void dma16s(const v4i& r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const v4i& r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

// Workgroup barrier once this wave's DMAs up to the one N instructions back
// have landed and its LDS reads are done.
template <int N>
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same without the LDS/scalar wait, for loops whose stage reads are all
// consumed (so complete) before the barrier in program order: outstanding
// scalar loads of the next work item then stay in flight across it.
template <int N>
__device__ __forceinline__ void dma_barrier_vm() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace situ
