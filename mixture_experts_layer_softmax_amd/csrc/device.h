// device.h -- small device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kChunkTokens = 64;    // tokens per dispatch chunk (histogram / scatter block)
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

struct Tile {       // one row tile of one expert in a grouped GEMM
    int32_t expert;
    int32_t row0;   // first dispatched row
    int32_t row1;   // one past the last row
    int32_t pad;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// 16 bytes with the non-temporal hint (the load allocates no cache line for reuse): for data a
// kernel reads exactly once, such as weights streamed at decode, so that it does not evict the
// lines of data that is read again.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

__device__ __forceinline__ int clamp_expert(int e, int E) {
    return e < 0 ? 0 : (e >= E ? E - 1 : e);
}

// Inclusive prefix sum over the 64 lanes of a wavefront on the DPP lane network: shifts by 1, 2,
// 4 and 8 within rows of 16 (lanes shifted in from outside the row add 0), then the last lane of
// row 0 into row 1 and of row 2 into row 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan_i32(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum over v for threads 0..n-1 of a block of NT threads (n <= NT <= 1024).
// Returns the exclusive prefix; *total receives the sum.  All threads must call it.
template <int NT>
__device__ int block_exclusive_scan(int v, int* total) {
    __shared__ int s_wave[NT / kWave];
    __shared__ int s_total;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int x = wave_inclusive_scan_i32(v);
    if (lane == kWave - 1) s_wave[w] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < NT / kWave; ++i) {
            int t = s_wave[i];
            s_wave[i] = run;
            run += t;
        }
        s_total = run;
    }
    __syncthreads();
    int r = x - v + s_wave[w];
    *total = s_total;
    __syncthreads();
    return r;
}

// SwiGLU of one (gate, up) pair: silu(g) * u with silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

}  // namespace moe
