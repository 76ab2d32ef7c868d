// select.h -- device building blocks shared by the routing and dispatch kernels: per-token
// top-k selection by one wavefront, and the GEMM tile list of a dispatch.
#pragma once

#include "device.h"

namespace moe {

// Top-k of one token by one wavefront: k rounds of a wave-wide argmax over (logit desc,
// expert asc), then the softmax weights in fp32.  `row` is the token's E logits; ids and w
// receive k values each (and ids_lds too, when given).  NaN logits rank below every number, so
// the comparison is a total order and every lane agrees on each winner: always k distinct valid
// experts, also for non-finite logits (whose weights are then unspecified).
template <int EPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int renorm,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int* ids_lds) {
    const int lane = lane_id();
    constexpr int NONE = 0x7fffffff;
    float v[EPL];
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        live[i] = e < E;
        v[i] = live[i] ? row[e] : 0.0f;
        if (v[i] != v[i]) v[i] = -__builtin_inff();  // NaN ranks last: a total order for selection
    }
    float selv[kMaxTopK];
    int sele[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        selv[j] = 0.0f;
        sele[j] = 0;
    }
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int be = NONE;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (live[i] && (be == NONE || v[i] > bv)) {  // ascending e within a lane
                bv = v[i];
                be = lane + kWave * i;
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            const bool take = oe != NONE && (be == NONE || ov > bv || (ov == bv && oe < be));
            if (take) {
                bv = ov;
                be = oe;
            }
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (be == lane + kWave * i) live[i] = false;
#pragma unroll
        for (int jj = 0; jj < kMaxTopK; ++jj)
            if (jj == j) {
                selv[jj] = bv;
                sele[jj] = be;
            }
    }
    // weights: exp(l_j - l_0) / z
    float z = 0.0f;
    if (renorm) {
        for (int j = 0; j < k; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int jj = 0; jj < kMaxTopK; ++jj)
                if (jj == j) s = selv[jj];
            z += expf(s - selv[0]);
        }
    } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) part += expf(row[e] - selv[0]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        z = part;
    }
    if (lane < k) {
        float s = 0.0f;
        int e = 0;
#pragma unroll
        for (int jj = 0; jj < kMaxTopK; ++jj)
            if (jj == lane) {
                s = selv[jj];
                e = sele[jj];
            }
        ids[lane] = e;
        w[lane] = expf(s - selv[0]) / z;
        if (ids_lds) ids_lds[lane] = e;
    }
}

// Write the tile list of one grouped GEMM with row-tile height bm from per-expert counts
// (thread e handles expert e; `start` = exclusive row offset of expert e).  A tile names its
// expert by weight index e - ebase (the caller's first held expert; experts not held have no
// rows).  At most `cap` tiles are written (a bound that valid counts never reach).
__device__ __forceinline__ void emit_tiles(int e, int E, int count, int start, int bm, Tile* tiles,
                           int* tile_count, int cap, int ebase) {
    const int nt = (e < E) ? (count + bm - 1) / bm : 0;
    int total;
    const int first = block_exclusive_scan<kMaxExperts>(nt, &total);
    for (int i = 0; i < nt && first + i < cap; ++i) {
        Tile t;
        t.expert = e - ebase;
        t.row0 = start + i * bm;
        t.row1 = min(start + count, start + (i + 1) * bm);
        t.pad = 0;
        tiles[first + i] = t;
    }
    if (threadIdx.x == 0) *tile_count = min(total, cap);
}

}  // namespace moe
