// route.hip -- router logits (canonical fp32 order) and top-k / softmax selection.
//
// The router picks the experts of every token before dispatch ("CuTeDSL at Perplexity",
// section Mixture-of-Experts Dispatch/Combine, Local: the local kernel starts from the
// routing table; the Muse Spark Open megakernel article, section Model and new tensor
// parallelism: the expert step is only known once the router has run).
//
// Logits are computed on the VALU in the canonical order of the routing contract (moe.h):
// each of the 64 lanes of a wavefront owns one partial sum p and walks the 8-element chunks
// c = p, p+64, p+128, ... of the hidden vector with one v_fma_f32 per element; the partials
// are folded pairwise across lanes (lane p with lane p+off, off = 32..1).  Every lane loads
// 16 contiguous bytes per bf16 chunk, so a wavefront reads 1 KiB contiguous per row and step.
#include "device.h"
#include "launch.h"
#include "select.h"

namespace moe {

// One wavefront computes a TM x TN block of (token, expert) logits.  The reduction across
// lanes is a reduce-scatter: at each fold step a lane keeps half of its outputs and receives
// the partner's partials of that half, so after log2(TM*TN) steps every lane holds the
// complete partial of one output; remaining steps are plain butterflies.  Addition being
// commutative, every lane's value equals the canonical a[p] + a[p+off].
template <bool BF16, int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x,
                                                            const void* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T,
                                                            int H, int E) {
    constexpr int NO = TM * TN;
    static_assert((NO & (NO - 1)) == 0 && NO <= 64, "outputs per wave must be a power of 2");
    const int lane = lane_id();
    const int wave = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int tiles_e = (E + TN - 1) / TN;
    const int t0 = (wave / tiles_e) * TM;
    const int e0 = (wave % tiles_e) * TN;
    if (t0 >= T) return;  // uniform per wave

    float acc[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[o] = 0.0f;

    const int nchunks = H / 8;
    if (BF16) {
        const uint4* xr[TM];
        const uint4* wrr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            xr[i] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) +
                                                   size_t(min(t0 + i, T - 1)) * H);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            wrr[j] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(wr) +
                                                    size_t(min(e0 + j, E - 1)) * H);
        // small blocks (decode batches): unroll so that several chunks' loads are in flight
#pragma unroll(NO <= 2 ? 8 : 1)
        for (int c = lane; c < nchunks; c += kWave) {
            uint4 xv[TM], wv[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) xv[i] = xr[i][c];
#pragma unroll
            for (int j = 0; j < TN; ++j) wv[j] = wrr[j][c];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    float xf[TM], wf[TN];
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        uint32_t u = q == 0 ? xv[i].x : q == 1 ? xv[i].y : q == 2 ? xv[i].z : xv[i].w;
                        xf[i] = half ? bf16_hi(u) : bf16_lo(u);
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        uint32_t u = q == 0 ? wv[j].x : q == 1 ? wv[j].y : q == 2 ? wv[j].z : wv[j].w;
                        wf[j] = half ? bf16_hi(u) : bf16_lo(u);
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i * TN + j] = __builtin_fmaf(xf[i], wf[j], acc[i * TN + j]);
                }
            }
        }
    } else {
        const float4* xr[TM];
        const float4* wrr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            xr[i] = reinterpret_cast<const float4*>(static_cast<const float*>(x) +
                                                    size_t(min(t0 + i, T - 1)) * H);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            wrr[j] = reinterpret_cast<const float4*>(static_cast<const float*>(wr) +
                                                     size_t(min(e0 + j, E - 1)) * H);
        for (int c = lane; c < nchunks; c += kWave) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float4 xv[TM], wv[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) xv[i] = xr[i][2 * c + h];
#pragma unroll
                for (int j = 0; j < TN; ++j) wv[j] = wrr[j][2 * c + h];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            float a = q == 0 ? xv[i].x : q == 1 ? xv[i].y : q == 2 ? xv[i].z : xv[i].w;
                            float b = q == 0 ? wv[j].x : q == 1 ? wv[j].y : q == 2 ? wv[j].z : wv[j].w;
                            acc[i * TN + j] = __builtin_fmaf(a, b, acc[i * TN + j]);
                        }
            }
        }
    }

    // canonical fold across the 64 partials
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        const int off = 32 >> s;
        const int cur = (NO >> s) > 0 ? (NO >> s) : 1;
        if (cur >= 2) {
            const bool upper = (lane & off) != 0;
#pragma unroll
            for (int o = 0; o < cur / 2; ++o) {
                float send = upper ? acc[o] : acc[o + cur / 2];
                float keep = upper ? acc[o + cur / 2] : acc[o];
                acc[o] = keep + __shfl_xor(send, off);
            }
        } else {
            acc[0] = acc[0] + __shfl_xor(acc[0], off);
        }
    }
    constexpr int LOG_NO = NO == 1 ? 0 : NO == 2 ? 1 : NO == 4 ? 2 : NO == 8 ? 3 : NO == 16 ? 4 : NO == 32 ? 5 : 6;
    const int o = lane >> (6 - LOG_NO);
    if ((lane & ((64 >> LOG_NO) - 1)) == 0) {
        const int t = t0 + o / TN, e = e0 + o % TN;
        if (t < T && e < E) {
            float v = acc[0];
            if (bias) v = v + bias[e];
            logits[size_t(t) * E + e] = v;
        }
    }
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
