// lds_dma.h -- direct-to-LDS DMA and transposing LDS reads on gfx950, shared
// by the forward kernels (HIP path only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

typedef short v4s __attribute__((ext_vector_type(4)));

// Direct-to-LDS DMA: 16 bytes per lane into LDS at M0 + 16 lane, either
// from a 64-bit lane address (global_load_lds_dwordx4) or from a buffer
// resource plus a 32-bit lane offset (buffer_load_dwordx4 ... lds).  The
// buffer form, with one resource per key/value head, measured 2.5% faster on
// the ring share; it is used when a head's rows span less than 4 GB.
// Each asm block begins with 5 wait states: the compiler does not look
// inside inline asm for hazards, and on gfx950 a VMEM instruction that reads
// an SGPR (M0, the resource, the scalar offset) written by a VALU instruction
// (v_readfirstlane, or v_readlane when the compiler restores a spilled SGPR)
// must follow it by at least 5 wait states.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
typedef int v4i __attribute__((ext_vector_type(4)));
// raw buffer resource: base address, stride 0, num_records 2^32 - 1, 32-bit data format
__device__ __forceinline__ v4i head_rsrc(const char* base) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
  r[2] = -1;
  r[3] = 0x00020000;
  return r;
}
// soff: the tile's byte offset (wave-uniform, scalar), voff: the lane's part
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t soff, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ v4s read_tr(const char* lds, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(
          (__attribute__((address_space(3))) char*)(lds + off)));
}

}  // namespace rattn
