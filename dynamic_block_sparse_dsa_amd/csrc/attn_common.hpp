// Pieces shared by the attention forward and backward kernels: vector types,
// address spaces, the XOR swizzles of K/V tiles in LDS, vmcnt waits and the
// global -> LDS DMA.
#pragma once

#include "dsa_internal.hpp"

namespace dsa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

// XOR swizzles of the 16-byte chunk index within a row of a tile in LDS.
// kswz spreads the row reads of an MFMA operand (32 rows, same chunk) over all
// banks; vswz does the same for the transposed reads (4 consecutive rows, 32
// bytes each).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}
// qswz serves tiles read both ways (the backward's Q, dO and K tiles): with
// 64 four-byte banks, 16 consecutive rows at one chunk land in 16 distinct
// chunk slots (a bijection of the row's low bits), and 4 consecutive rows x
// 4 aligned chunks (one transposed read of 32 lanes) do as well, since the
// swizzle's upper two bits follow the row within its group of 4.
template <int D>
__device__ __forceinline__ int qswz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// wait until at most n vector-memory operations of this wave are in flight
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte-per-lane DMA from global memory into LDS (lane l lands at
// lds_addr + 16 * l).  Written as a small asm block because the compiler
// cannot tell LDS DMA into one tile from reads of the other tile: with the
// builtin it drains every outstanding load before each LDS read, which would
// serialise the prefetch.  The block has no register outputs (the data goes
// to LDS); M0 is saved and restored so the compiler's view of it holds; the
// waits for the data are the explicit vmcnt waits + barriers in the loop.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

}  // namespace dsa
