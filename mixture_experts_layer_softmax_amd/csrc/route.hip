// route.hip -- router logits (canonical fp32 order) and top-k / softmax selection.
//
// The router picks the experts of every token before dispatch ("CuTeDSL at Perplexity",
// section Mixture-of-Experts Dispatch/Combine, Local: the local kernel starts from the
// routing table; the Muse Spark Open megakernel article, section Model and new tensor
// parallelism: the expert step is only known once the router has run).
//
// Logits are computed on the VALU in the canonical order of the routing contract (moe.h);
// route.h holds the wavefront's computation.
#include "device.h"
#include "launch.h"
#include "route.h"
#include "select.h"

namespace moe {

// One wavefront per TM x TN block of logits.
template <bool BF16, int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x,
                                                            const void* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T,
                                                            int H, int E) {
    // the wavefront index as a scalar, so that the row bases stay scalar too (8 x 8 form: 231
    // -> 149 registers, 35 -> 16 64-bit address additions per chunk; NVFP4 prefill routing
    // 305 -> 274 us, bit-identical)
    router_logits_wave<BF16, TM, TN>(x, wr, bias, logits, T, H, E,
                                     __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave));
}

// One wavefront per token.
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    topk_token<EPL>(logits + size_t(t) * E, E, k, renorm, ids + size_t(t) * k, w + size_t(t) * k,
                    nullptr);
}

// ---------------------------------------------------------------------------------------

hipError_t launch_router_logits(const RouteArgs& a, hipStream_t s) {
    const int T = a.T, E = a.E;
    // large batches: 8x8 (token, expert) blocks per wave for operand reuse, 4x4 below 384 tokens
    // (four times the wavefronts, each with a quarter of the serial FMA work; kernel trace,
    // median us, 8x8 -> 4x4 at E=128: T=64 17.5 -> 12.0, T=128 17.5 -> 12.4, T=256 18.0 -> 14.4,
    // but T=512 19.3 -> 20.8 and T=4096 85.7 -> 126.3); small batches: one token and 2 experts
    // per wave, or one expert per wave while that still leaves at most 512 blocks (every wave
    // waits for the same memory latency, so more of them finish sooner: decode T=1 with E=128
    // measured about 1 us less per forward).  All shapes give bit-identical logits.
    if (T >= 64 && T < 384 && E >= 8) {
        const long waves = long((T + 3) / 4) * ((E + 3) / 4);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 4, 4>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 4, 4>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else if (T >= 64 && E >= 8) {
        const long waves = long((T + 7) / 8) * ((E + 7) / 8);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 8, 8>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 8, 8>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else if (long(T) * E <= 2048) {
        const long waves = long(T) * E;
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 1, 1>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 1, 1>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else {
        const long waves = long(T) * ((E + 1) / 2);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 1, 2>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 1, 2>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                       float* w, hipStream_t s) {
    dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1)
        hipLaunchKernelGGL((topk_kernel<1>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (epl <= 2)
        hipLaunchKernelGGL((topk_kernel<2>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (epl <= 4)
        hipLaunchKernelGGL((topk_kernel<4>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else
        hipLaunchKernelGGL((topk_kernel<8>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

}  // namespace moe
