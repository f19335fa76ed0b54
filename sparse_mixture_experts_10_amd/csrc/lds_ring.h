// Pieces of the global-to-LDS stage ring shared by the MFMA kernels (the
// grouped GEMM and the router's MFMA path).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Stage rows are 64 SUB bytes (32 SUB bf16 of K) with their 16-byte chunks
// permuted: logical chunk c of row r sits at chunk c ^ swz(r).  The LDS serves
// a ds_read_b128 eight lanes at a time from 128 bytes of banks, so the eight
// consecutive rows an MFMA operand read touches at one logical chunk must land
// on eight different 16-byte bank groups.  For 64-byte rows (SUB = 1) two rows
// share a 128-byte bank row and swz(r) = (r >> 1) & 3 separates them (4 LDS
// cycles per ds_read_b128; unpermuted, r & 3 or (r >> 2) & 3 take 8, measured
// on MI355X with bank-conflict counters); for 128-byte rows (SUB = 2) every
// row spans all bank groups and swz(r) = r & 7 does.
template <int SUB>
__device__ __forceinline__ int swz(int r) { return SUB == 1 ? (r >> 1) & 3 : r & 7; }

// The same for the 32 x 32 x 16 MFMA's operand reads, where lane l reads row
// l % 32 at logical chunk c + l / 32.  Placements measured on MI355X with one
// block of four waves issuing ds_read_b128 back to back (LDS cycles per wave
// read; about 7.3 is conflict-free, 128 bytes a cycle): 64-byte rows,
// (r >> 1) & 3 takes 8.2, (r >> 3) & 3 takes 7.5; 128-byte rows, r & 7 takes
// 8.2, (r >> 1) & 7 takes 7.5.
template <int SUB, int MF>
__device__ __forceinline__ int swz_mf(int r) {
  if constexpr (MF == 16) return swz<SUB>(r);
  else return SUB == 1 ? (r >> 3) & 3 : (r >> 1) & 7;
}

// Workgroup barrier for the slab ring.  It first waits for this wave's LDS
// reads: the compiler may leave the reads of one slab in flight across the
// next barrier (it places its own lgkmcnt wait at their first use), and a wave
// that passes the barrier then refills that slab's stage, racing those reads.
// Built from builtins, not inline asm: inline asm makes the compiler assume
// the kernel may use AGPRs and reserve registers for them, which cuts the
// number of blocks a CU holds.  The signal fences keep the compiler from
// moving LDS accesses across; lgkmcnt(0) (vmcnt and expcnt left at their
// maxima) waits for this wave's LDS reads before the barrier.
__device__ __forceinline__ void slab_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace moe
