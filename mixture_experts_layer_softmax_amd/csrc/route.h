// route.h -- router logits in the canonical fp32 order of the routing contract (moe.h), as a
// device function of one wavefront, shared by the router kernel (route.hip) and the
// single-launch decode kernel (decode_fused.hip).
//
// Logits are computed on the VALU: each of the 64 lanes of a wavefront owns one partial sum p
// and walks the 8-element chunks c = p, p+64, p+128, ... of the hidden vector with one
// v_fma_f32 per element; the partials are folded pairwise across lanes (lane p with lane
// p+off, off = 32..1).  Every lane loads 16 contiguous bytes per bf16 chunk, so a wavefront
// reads 1 KiB contiguous per row and step.
#pragma once

#include "device.h"

namespace moe {

// One wavefront computes the TM x TN block `wave` of (token, expert) logits (blocks run along
// the experts first).  Waves past the last block do nothing.  The reduction across
// lanes is a reduce-scatter: at each fold step a lane keeps half of its outputs and receives
// the partner's partials of that half, so after log2(TM*TN) steps every lane holds the
// complete partial of one output; remaining steps are plain butterflies.  Addition being
// commutative, every lane's value equals the canonical a[p] + a[p+off].
template <bool BF16, int TM, int TN>
__device__ __forceinline__ void router_logits_wave(const void* __restrict__ x, const void* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int T, int H, int E, int wave) {
    constexpr int NO = TM * TN;
    static_assert((NO & (NO - 1)) == 0 && NO <= 64, "outputs per wave must be a power of 2");
    const int lane = lane_id();
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

}  // namespace moe
