// lds_dma.h -- helpers of the LDS-staged GEMM kernels (gemm.hip, mx.hip): explicit load-counter
// waits, a block barrier, direct global->LDS loads issued from inline asm (each LDS slot is its
// own LDS object so that the compiler can tell the slots apart; waits on the load counter are
// explicit), and the swizzled slot of a 16-byte chunk in a 64-byte LDS row.
#pragma once

#include "device.h"

namespace moe {
namespace {

// s_waitcnt operand: vmcnt <= n, lgkmcnt = 0 (expcnt left at its maximum).
constexpr int vm_wait_lgkm0(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    __builtin_amdgcn_s_waitcnt(vm_wait_lgkm0(N));
}

// 16 bytes per lane from global memory straight into LDS: lane l writes lds_base + 16*l.
// Issued through inline asm (setting M0 itself) so that the compiler does not treat the
// write as pending LDS data and wait for it before unrelated LDS reads; the caller owns the
// load counter.  M0 has no other use in the kernels that call this.
__device__ __forceinline__ void dma16(const void* src, const void* lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory");
}

// 4 bytes per lane from global memory straight into LDS: lane l writes lds_base + 4*l.
__device__ __forceinline__ void dma4(const void* src, const void* lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory");
}

// The same two loads with a scalar base address and a 32-bit per-lane byte offset (the global
// instruction's saddr form): the per-stage address step is a scalar add, with no 64-bit vector
// address arithmetic per load.  The caller guarantees that every offset fits 32 bits.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, const void* lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, const void* lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_base)));
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "memory");
}

// Work order of the prefill GEMMs.  Item i of the tile-major order (row tile i / ncols, column
// panel i % ncols) is re-mapped inside its expert: the expert's panels in groups of G (about
// kGroupBlocks blocks per group: G = kGroupBlocks / the expert's row tiles), and for each group
// all of the expert's row tiles before the next group, so that the blocks that read one weight
// panel are dispatched together.  An expert's tiles are adjacent in the tile list, so the
// re-mapping stays inside its range of items.  Returns the row tile; *panel gets the panel.
// Measured on the bf16 prefill workload (one process): kGroupBlocks 8 / 16 / 32 / 64 give
// forward 1.717 / 1.716 / 1.741 / 1.764 ms against 1.759-1.770 in tile-major order, weight
// fetches 4.91 against 5.11 GB per gate/up launch at 32; re-measured at 16 in the bf16 kernel:
// forward 1.754 -> 1.707 ms, gate/up 1.111 -> 1.090 ms, down 0.583 -> 0.560 ms.
constexpr int kGroupBlocks = 16;
__device__ __forceinline__ int grouped_item(const Tile* tiles, int tile_count, int item, int ncols,
                                            int* panel) {
    const int t0 = item / ncols;
    const int ex = tiles[t0].expert;
    int f = t0;
    while (f > 0 && tiles[f - 1].expert == ex) --f;
    int l = t0 + 1;
    while (l < tile_count && tiles[l].expert == ex) ++l;
    const int c = l - f;                                  // row tiles of the expert
    const int G = max(1, min(ncols, kGroupBlocks / c));   // panels per group
    const int idx = item - f * ncols;
    const int pg = idx / (c * G);
    const int gsz = min(G, ncols - pg * G);               // the last group may be narrower
    const int rem = idx - pg * c * G;
    *panel = pg * G + rem % gsz;
    return f + rem / gsz;
}

// 64-byte LDS rows of four 16-byte chunks: chunk ch of row r sits in slot ch ^ ((r >> 1) & 3),
// so that the fragment reads of 8 consecutive rows at one chunk hit distinct banks.
__device__ __forceinline__ int lds_slot32(int row, int ch) { return row * 4 + (ch ^ ((row >> 1) & 3)); }

}  // namespace
}  // namespace moe
