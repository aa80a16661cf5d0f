// lds_dma.h - direct-to-LDS loads written as inline asm, and the wait + barrier
// that completes them, shared by the FP8 forward and the backward kernels.
//
// gfx950's buffer loads can write their 16 (or 4) bytes per lane straight into
// LDS (lane l at byte 16 l, or 4 l, of a run whose base is in m0). The
// compiler's own wait insertion tracks such loads through the LDS object they
// write; once the kernel's LDS buffers are laid out as one block it can no
// longer tell them apart and makes every LDS read wait for every load in
// flight, which removes the overlap of the next tiles' loads with the current
// tile's work. Written as inline asm the loads are invisible to it, and the
// kernels place every wait on them themselves (wait_barrier). The asm has no
// register outputs; its address operands are read when it issues.
#ifndef ATTN_LDS_DMA_H
#define ATTN_LDS_DMA_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_dma {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor words for `bytes` bytes at `base`, as __builtin_amdgcn_make_buffer_rsrc
// builds them (stride 0; third word the record count; fourth word DATA_FORMAT = 32-bit).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFF), (int)bytes, 0x00020000};
}

// One direct-to-LDS load: 16 bytes per lane from byte offset voff of the buffer,
// lane l's bytes at LDS byte 16 l of the 1 KiB run at `lds`.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is clobbered on purpose: the kernel keeps nothing in it
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, const char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// The same with the run's LDS byte address given as a (wave-uniform) integer.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// The same with 4 bytes per lane (lane l at LDS byte 4 l of the 256-byte run at `lds`).
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voff, const void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop


// Wait until at most n of this wavefront's vector-memory loads are outstanding
// (and its LDS reads are done), then the workgroup barrier. Loads complete in
// issue order, so n = the loads issued after the ones needed.
template <int N_OUT>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N_OUT >= 0 && N_OUT < 16, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | N_OUT);  // vmcnt(N_OUT), expcnt any, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace attn_dma

#endif
