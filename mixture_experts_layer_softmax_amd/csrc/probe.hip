// probe.hip -- measurement microkernels (moe_probe.h): achievable bf16 MFMA rate and HBM read
// bandwidth of the device, for stating roofline fractions against measured peaks.
#include <hip/hip_runtime.h>

#include "device.h"
#include "grid_sync.h"
#include "launch.h"
#include "moe_probe.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
    const int tid = threadIdx.x;
    // operands depend on the thread so that nothing folds; values stay small and finite
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_bit_cast(__bf16, uint16_t(0x3c00 + ((tid + i) & 7)));
        b[i] = __builtin_bit_cast(__bf16, uint16_t(0x3c00 + ((tid * 3 + i) & 7)));
    }
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
    }
    const f32x4_t s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    const float v = s[0] + s[1] + s[2] + s[3];
    if (tid == 0) out[blockIdx.x] = v;
}

// Each block step reads one contiguous 32 KiB chunk, eight 16-byte loads per thread issued
// before any is used; the words past the last whole chunk are read grid-stride.  NT: the
// whole-chunk loads carry the non-temporal hint, like the decode GEMMs' weight streams (the
// stream then measured about 7.1 TB/s against 6.44 with default loads, which the decode GEMMs
// exceed); without it the loads allocate cache lines, so a read of a large buffer evicts
// whatever the caches held.
template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, long n16,
                                                         uint32_t* __restrict__ out) {
    constexpr int U = 8;
    constexpr long kChunk = 256L * U;
    const long nch = n16 / kChunk;
    uint32_t acc = 0;
    for (long c = blockIdx.x; c < nch; c += gridDim.x) {
        const uint4* q = p + c * kChunk + threadIdx.x;
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? load_nt16(q + u * 256) : q[u * 256];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].w;
    }
    for (long i = nch * kChunk + long(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += long(gridDim.x) * blockDim.x)
        acc ^= p[i].x;
    if (acc == 0x9e3779b9u) out[0] = acc;
}

// `barriers` grid barriers in a row (grid_sync.h), nothing else: the cost of one barrier of the
// single-launch decode kernel at this grid size.  Barrier values continue from the sequence
// word of `gs` like the decode kernel's (v = 65536 S + i), so any initial contents work.
__global__ __launch_bounds__(256) void barrier_probe_kernel(GridSync* gs, int barriers, unsigned spin_limit) {
    __shared__ uint64_t s_seq;
    if (threadIdx.x == 0) s_seq = load_agent(&gs->seq);
    __syncthreads();
    const uint64_t base = s_seq << 16;
    for (int i = 1; i <= barriers; ++i) grid_barrier(gs, base + uint64_t(i), spin_limit);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        __hip_atomic_store(&gs->seq, s_seq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_probe_grid_barrier(int32_t blocks, int32_t barriers, void* sync, uint32_t spin_limit,
                                             void* stream) {
    if (blocks < 1 || blocks > moe::kFusedMaxBlocks || barriers < 1 || barriers >= 65536 || !sync ||
        (reinterpret_cast<uintptr_t>(sync) & 15u))
        return MOE_ERR_INVALID_ARGUMENT;
    moe::GridSync* gs = static_cast<moe::GridSync*>(sync);
    void* params[] = {&gs, &barriers, &spin_limit};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(moe::barrier_probe_kernel),
                                                    dim3(blocks), dim3(256), params, 0,
                                                    static_cast<hipStream_t>(stream));
    return (e == hipSuccess && hipGetLastError() == hipSuccess) ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24) || !out ||
        (reinterpret_cast<uintptr_t>(out) & 3u))
        return MOE_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(moe::mfma_probe_kernel, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

template <bool NT>
static moe_status probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    if (!buf || !out || bytes == 0 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u) ||
        (reinterpret_cast<uintptr_t>(out) & 3u))
        return MOE_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(moe::read_probe_kernel<NT>, dim3(16384), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                       long(bytes / 16), out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

extern "C" moe_status moe_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    return probe_read<false>(buf, bytes, out, stream);
}

extern "C" moe_status moe_probe_read_nt(const void* buf, size_t bytes, uint32_t* out, void* stream) {
    return probe_read<true>(buf, bytes, out, stream);
}
