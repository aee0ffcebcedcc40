// Direct-to-LDS buffer loads for gfx950 (shared by the matrix-core kernels).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cpattn {
namespace {

typedef unsigned int dma_u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor (raw, stride 0: offsets >= bytes read as zero) as four
// scalar words, for the inline-assembly loads below.
__device__ __forceinline__ dma_u32x4 buffer_desc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  dma_u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane(uint32_t(a));
  d[1] = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS at
// lds + 16 lane (buffer_load_dwordx4 ... lds).  Issued as inline assembly so
// the compiler neither tracks nor waits for it: the caller orders it with
// explicit vmcnt waits and LDS barriers.  The memory clobber keeps the
// compiler from caching LDS contents across it.  The compiler's hazard
// checks do not look inside the assembly, so it carries its own wait states:
// a vector-memory instruction must not read an SGPR a VALU instruction wrote
// (v_readfirstlane, or v_readlane reloading a spilled SGPR) fewer than five
// wait states earlier, nor M0 right after its write; s_nop 4 covers both.
__device__ __forceinline__ void dma_lds16(dma_u32x4 desc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const __attribute__((address_space(3))) void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>(p));
}

}  // namespace
}  // namespace cpattn
