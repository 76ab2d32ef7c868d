// combine.hip -- weighted accumulation of each token's expert outputs back in token order.
//
// "CuTeDSL at Perplexity", section Mixture-of-Experts Dispatch/Combine, Local: the combine
// kernel uses the positions dispatch assigned to gather a token's expert rows and accumulates
// them in registers with vectorised accesses, then writes the final token.  Here: one block
// per token, 16-byte loads of y_perm rows (all rows of a vector issued before the first FMA),
// fp32 accumulation in ascending slot order, one rounding to the output type.  In bf16 the
// y_perm loads are non-temporal: every y_perm element is read once, and caching it only evicts
// other lines (kernel trace, median us, 8192 tokens x 8 slots x 4096: 113.5 -> 95.5; 4096 x 8
// x 4096: 54.7 -> 49.4; bit-identical).  The output keeps default stores: the next operation
// reads it (non-temporal stores measured 2.6 and 1.6 us less here).  Slots with a
// negative row were not dispatched here (their expert is held by another rank under expert
// parallelism) and are skipped, so the result is the local part of the combine that the pages
// follow with an all-reduce.
#include "device.h"
#include "launch.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(512) void combine_kernel(const void* __restrict__ y_perm,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      void* __restrict__ y, int k, int H, int A) {
    const int t = blockIdx.x;
    // slot j of the token at index j (compile-time indices keep everything in registers);
    // slots with a negative row are skipped, which keeps the ascending order of the others
    int rows[kMaxTopK];
    float ws[kMaxTopK];
    bool ok[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        rows[j] = 0;
        ws[j] = 0.0f;
        ok[j] = false;
        if (j < k) {
            const int r = inv_perm[size_t(t) * k + j];
            ok[j] = r >= 0;
            rows[j] = r < 0 ? 0 : (r >= A ? A - 1 : r);
            ws[j] = w[size_t(t) * k + j];
        }
    }
    if (BF16) {
        const uint4* src = static_cast<const uint4*>(y_perm);
        uint4* dst = static_cast<uint4*>(y);
        const int nv = H / 8;
        for (int v = threadIdx.x; v < nv; v += blockDim.x) {
            uint4 q[kMaxTopK];  // all of this vector's row loads in flight before the first FMA
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (ok[j]) q[j] = load_nt16(src + size_t(rows[j]) * nv + v);
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (!ok[j]) continue;
                const uint32_t u[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    acc[2 * p] = __builtin_fmaf(ws[j], bf16_lo(u[p]), acc[2 * p]);
                    acc[2 * p + 1] = __builtin_fmaf(ws[j], bf16_hi(u[p]), acc[2 * p + 1]);
                }
            }
            dst[size_t(t) * nv + v] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        }
    } else {
        const float4* src = static_cast<const float4*>(y_perm);
        float4* dst = static_cast<float4*>(y);
        const int nv = H / 4;
        for (int v = threadIdx.x; v < nv; v += blockDim.x) {
            float4 q[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (ok[j]) q[j] = src[size_t(rows[j]) * nv + v];
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (!ok[j]) continue;
                acc.x = __builtin_fmaf(ws[j], q[j].x, acc.x);
                acc.y = __builtin_fmaf(ws[j], q[j].y, acc.y);
                acc.z = __builtin_fmaf(ws[j], q[j].z, acc.z);
                acc.w = __builtin_fmaf(ws[j], q[j].w, acc.w);
            }
            dst[size_t(t) * nv + v] = acc;
        }
    }
}

hipError_t launch_combine(const void* y_perm, const int32_t* inv_perm, const float* w, void* y,
                          int T, int k, int H, int A, bool bf16, hipStream_t s) {
    const int nv = bf16 ? H / 8 : H / 4;
    // one 16-byte vector per thread up to H = 4096 (bf16): kernel trace, median us, 256 -> 512
    // threads: 4096-token prefill 58.4 -> 55.7, 64-token decode 6.1 -> 5.0
    const int threads = nv >= 512 ? 512 : ((nv + 63) / 64) * 64;
    if (bf16)
        hipLaunchKernelGGL((combine_kernel<true>), dim3(T), dim3(threads), 0, s, y_perm, inv_perm, w,
                           y, k, H, A);
    else
        hipLaunchKernelGGL((combine_kernel<false>), dim3(T), dim3(threads), 0, s, y_perm, inv_perm,
                           w, y, k, H, A);
    return hipGetLastError();
}

}  // namespace moe
