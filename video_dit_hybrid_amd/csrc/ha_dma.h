// Global -> LDS copies written as inline asm, for kernels that track their
// completion themselves (gfx950).
#pragma once

#include "ha_device.h"

namespace ha {

// Global -> LDS copies issued from inline asm. With the builtin form the
// compiler cannot tell which LDS bytes a copy writes and waits for every copy
// in flight before each later LDS read; with these the caller tracks
// completion by explicit vmcnt waits. m0 holds the wave-uniform LDS
// destination; lane l writes its bytes at m0 + l * size.
// s_nop 4: the compiler cannot see into the asm, and an SGPR operand it has
// just written with a VALU instruction (v_readlane of a spilled SGPR) needs
// five wait states before a VMEM read; m0 needs one.
__device__ __forceinline__ void dma16_asm(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4_asm(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr) : "memory");
}
// Four consecutive 1 KB copies (16 bytes per lane each) at instruction
// offsets 0, 1024, 2048, 3072. The instruction offset moves both the global
// address and the LDS destination (m0 + offset + 16 * lane), so one m0 /
// soffset pair and one s_nop serve all four; they count as four vmcnt events.
__device__ __forceinline__ void dma16x4_asm(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\t"
               "buffer_load_dwordx4 %0, %1, %2 offen lds\n\t"
               "buffer_load_dwordx4 %0, %1, %2 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %0, %1, %2 offen offset:2048 lds\n\t"
               "buffer_load_dwordx4 %0, %1, %2 offen offset:3072 lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr) : "memory");
}

// Wait for the asm copies of the oldest slice in flight, when min(later, MAXL)
// slices of PER copies each were issued after it and may stay in flight.
// Loads retire in order, so vmcnt <= later * PER leaves exactly those.
template <int MAXL, int PER>
__device__ __forceinline__ void wait_later_copies(int later) {
  static_assert(MAXL <= 4 && MAXL * PER <= 15, "vmcnt immediate");
  const int l = later < MAXL ? later : MAXL;
  if constexpr (MAXL >= 4) if (l == 4) { __builtin_amdgcn_s_waitcnt(0x0F70 | (4 * PER)); return; }
  if constexpr (MAXL >= 3) if (l == 3) { __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * PER)); return; }
  if constexpr (MAXL >= 2) if (l == 2) { __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * PER)); return; }
  if constexpr (MAXL >= 1) if (l == 1) { __builtin_amdgcn_s_waitcnt(0x0F70 | PER); return; }
  __builtin_amdgcn_s_waitcnt(0x0F70);
}
// Buffer descriptor words for the asm copies: base, range in bytes.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bytes), (uint32_t)kRsrcWord3};
}

}  // namespace ha
