// Direct global -> LDS copies and typed LDS reads for the LDS-tiled GEMMs.
#pragma once
#include "common.h"

namespace moe {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane, global (base + 32-bit lane offset) -> LDS at
// lds_wave_base + 16 * lane. Issued as inline assembly so that the compiler
// does not track it as an LDS write: it would otherwise drain every
// outstanding copy (vmcnt(0)) before each barrier and LDS read, serialising
// the ring. Completion is ordered by hand with MOE_WAIT_VMCNT before the
// barrier that publishes a stage. M0 holds the wave-uniform LDS destination;
// nothing else in these kernels uses M0. The base is a wave-uniform 64-bit
// SGPR pair, so advancing a step costs scalar adds only.
MOE_DEV void g2lds(const void* base, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_wave_base)
      : "memory");
}

// The same copy with the nontemporal hint, for weights that no other tile
// reads (an expert with a single tile): a stream that will not be reused.
MOE_DEV void g2lds_nt(const void* base, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(base), "s"(lds_wave_base)
      : "memory");
}

// Weight copy: nontemporal when nt (a wave-uniform flag), else plain.
MOE_DEV void g2lds_w(const void* base, uint32_t voff, uint32_t lds_wave_base,
                     bool nt) {
  if (nt)
    g2lds_nt(base, voff, lds_wave_base);
  else
    g2lds(base, voff, lds_wave_base);
}

MOE_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

MOE_DEV u32x4_t lds_read_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)a;
}

}  // namespace moe

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
// The compiler folds it into its own wait bookkeeping, so loads it tracks
// that are older than the waited-for copies are known complete afterwards.
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)
