// select.h -- device building blocks shared by the routing and dispatch kernels: per-token
// top-k selection by one wavefront, the GEMM tile list of a dispatch, and the selection and
// dispatch of a small batch by one block.
#pragma once

#include "device.h"

namespace moe {

// Wave-wide reductions on the DPP lane network (no LDS round trips): within rows of 16 by
// quad permutes and mirrors, then across rows by the row-15 / row-31 broadcasts, so that lane 63
// holds the result, which is read out as a wave-uniform value.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __int_as_float(dpp_i32<0xb1>(__float_as_int(v))));        // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(dpp_i32<0x4e>(__float_as_int(v))));        // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(dpp_i32<0x141>(__float_as_int(v))));       // row_half_mirror
    v = fmaxf(v, __int_as_float(dpp_i32<0x140>(__float_as_int(v))));       // row_mirror
    v = fmaxf(v, __int_as_float(dpp_i32<0x142, 0xa>(__float_as_int(v))));  // row_bcast:15
    v = fmaxf(v, __int_as_float(dpp_i32<0x143, 0xc>(__float_as_int(v))));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, dpp_i32<0xb1>(v));
    v = min(v, dpp_i32<0x4e>(v));
    v = min(v, dpp_i32<0x141>(v));
    v = min(v, dpp_i32<0x140>(v));
    v = min(v, dpp_i32<0x142, 0xa>(v));
    v = min(v, dpp_i32<0x143, 0xc>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// The k rounds of the selection over values v (lane l holds experts l, l + 64, ...; live marks
// the experts that exist and are still unpicked).  Lane j < k receives the j-th pick in *sv /
// *se; every lane receives the first (largest) value in *m0.
template <int EPL>
__device__ __forceinline__ void topk_rounds(const float (&v)[EPL], bool (&live)[EPL], int k,
                                            float* sv, int* se, float* m0) {
    const int lane = lane_id();
    constexpr int NONE = 0x7fffffff;
    float mysv = 0.0f;
    int myse = 0;
    float first = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int be = NONE;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (live[i] && (be == NONE || v[i] > bv)) {  // ascending e within a lane
                bv = v[i];
                be = lane + kWave * i;
            }
        // a lane without a candidate holds -inf and NONE, so it never takes the index round
        const float m = wave_max_f32(bv);
        be = wave_min_i32((be != NONE && bv == m) ? be : NONE);
        bv = m;
        if (j == 0) first = bv;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (be == lane + kWave * i) live[i] = false;
        if (lane == j) {
            mysv = bv;
            myse = be;
        }
    }
    *sv = mysv;
    *se = myse;
    *m0 = first;
}

// Renormalised weights of the k picks: exp(l_j - l_0) / z, z summing the k terms in selection
// order; lane j < k writes pick j.
__device__ __forceinline__ void topk_write_renormalised(float sv, int se, float m0, int k,
                                                        int32_t* __restrict__ ids, float* __restrict__ w,
                                                        int* ids_lds) {
    const int lane = lane_id();
    float z = 0.0f;
    for (int j = 0; j < k; ++j)
        z += expf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), j)) - m0);
    if (lane < k) {
        ids[lane] = se;
        w[lane] = expf(sv - m0) / z;
        if (ids_lds) ids_lds[lane] = se;
    }
}

// Top-k of one token by one wavefront: k rounds of a wave-wide argmax over (logit desc,
// expert asc), then the softmax weights in fp32.  A round takes the largest value (a DPP max;
// fmaxf is exact), then the smallest expert index among the lanes whose candidate equals it
// (+0 and -0 compare equal, as in a plain comparison).  `row` is the token's E logits; ids and w
// receive k values each (and ids_lds too, when given).  NaN logits rank below every number, so
// the comparison is a total order and every lane agrees on each winner: always k distinct valid
// experts, also for non-finite logits (whose weights are then unspecified).
template <int EPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int renorm,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           int* ids_lds) {
    const int lane = lane_id();
    float v[EPL];
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        live[i] = e < E;
        v[i] = live[i] ? row[e] : 0.0f;
        if (v[i] != v[i]) v[i] = -__builtin_inff();  // NaN ranks last: a total order for selection
    }
    // lane j < k keeps the j-th selection (value and expert); m0 is the first (largest) value
    float mysv, m0;
    int myse;
    topk_rounds<EPL>(v, live, k, &mysv, &myse, &m0);
    if (renorm) {
        topk_write_renormalised(mysv, myse, m0, k, ids, w, ids_lds);
        return;
    }
    // full softmax: z sums every logit's term
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) part += expf(row[e] - m0);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    const float z = part;
    if (lane < k) {
        ids[lane] = myse;
        w[lane] = expf(mysv - m0) / z;
        if (ids_lds) ids_lds[lane] = myse;
    }
}

// Write the tile list of one grouped GEMM with row-tile height bm from per-expert counts
// (thread e handles expert e; `start` = exclusive row offset of expert e).  A tile names its
// expert by weight index e - ebase (the caller's first held expert; experts not held have no
// rows).  At most `cap` tiles are written (a bound that valid counts never reach).
// NT is the block size (every thread calls this).
template <int NT = kMaxExperts>
__device__ __forceinline__ void emit_tiles(int e, int E, int count, int start, int bm, Tile* tiles,
                           int* tile_count, int cap, int ebase) {
    const int nt = (e < E) ? (count + bm - 1) / bm : 0;
    int total;
    const int first = block_exclusive_scan<NT>(nt, &total);
    for (int i = 0; i < nt && first + i < cap; ++i) {
        Tile t;
        t.expert = e - ebase;
        t.row0 = start + i * bm;
        t.row1 = min(start + count, start + (i + 1) * bm);
        t.pad = 0;
        tiles[first + i] = t;
    }
    const int ntiles = min(total, cap);
    if (threadIdx.x == 0) *tile_count = ntiles;
    if (bm >= 128) {
        // prefill tile lists: the 8 XCDs' tile ranges, tile_count[8 + x] .. tile_count[9 + x],
        // cut where the running cost of the list (bm / 16 + ceil(rows / 16) per tile: a fixed
        // part per tile plus its rows) crosses x / 8 of the total
        const int last_rows = nt ? count - (nt - 1) * bm : 0;
        const int cost = nt ? (nt - 1) * (2 * bm / 16) + bm / 16 + (last_rows + 15) / 16 : 0;
        int ctotal;
        const int cstart = block_exclusive_scan<NT>(cost, &ctotal);
        if (threadIdx.x == 0) {
            tile_count[8] = 0;
            tile_count[16] = ntiles;
            // no rows: every range empty (nothing else writes them, and the area keeps the
            // previous list's ranges)
            if (ctotal == 0)
                for (int x = 1; x < 8; ++x) tile_count[8 + x] = 0;
        }
        if (cost > 0) {
            for (int x = 1; x < 8; ++x) {
                const long long target = (long long)x * ctotal / 8;
                if (target < cstart || target >= cstart + cost) continue;
                int cum = cstart, b = first + nt;
                for (int i = 0; i < nt; ++i) {
                    const int rows = i + 1 < nt ? bm : last_rows;
                    const int tc = bm / 16 + (rows + 15) / 16;
                    if (target < cum + tc) {
                        b = first + i + ((target - cum) * 2 >= tc ? 1 : 0);
                        break;
                    }
                    cum += tc;
                }
                tile_count[8 + x] = min(b, ntiles);
            }
        }
    }
}

// Small decode batches (any T <= 64): top-k selection and the whole dispatch (histogram, scan,
// tile lists, stable scatter) by one block of NT >= E threads, so a decode step spends one
// launch on it instead of four, or the single-launch decode kernel none.  Wavefront w selects
// tokens w, w + NT/64, ... one after the other; thread e < E then owns expert e.  Same results
// as topk_kernel + hist/scan/scatter: ids of a token in selection order, rows of an expert in
// (t, j) order.  Output pointers may point to global memory or to the caller's LDS.  Every
// thread of the block must call it.
template <int EPL, int NT>
__device__ __forceinline__ void select_dispatch_block(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* ids, float* tw,
    int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, Tile* tiles1,
    int* tile_count1, int bm1, Tile* tiles2, int* tile_count2, int bm2, int cap, int eb, int ee) {
    static_assert(NT % kWave == 0 && NT <= kMaxExperts * 2, "whole wavefronts");
    constexpr int NW = NT / kWave;
    __shared__ int sids[kChunkTokens * kMaxTopK];
    __shared__ int cnt[kMaxExperts];
    __shared__ int wc[NW][kMaxExperts];
    const int tid = threadIdx.x, w = tid / kWave;
    for (int t = w; t < T; t += NW)
        topk_token<EPL>(logits + size_t(t) * E, E, k, renorm, ids + size_t(t) * k, tw + size_t(t) * k,
                        sids + t * k);
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    const int A = T * k;
    for (int a = tid; a < A; a += NT) {
        const int id = clamp_expert(sids[a], E);
        if (id >= eb && id < ee) atomicAdd(&cnt[id], 1);
    }
    __syncthreads();
    const int c = tid < E ? cnt[tid] : 0;
    int total;
    const int start = block_exclusive_scan<NT>(c, &total);
    if (tid < E) {
        if (counts) counts[tid] = c;
        offsets[tid] = start;
    }
    if (tid == 0) offsets[E] = total;
    if (tiles1) emit_tiles<NT>(tid, E, c, start, bm1, tiles1, tile_count1, cap, eb);
    if (tiles2) emit_tiles<NT>(tid, E, c, start, bm2, tiles2, tile_count2, cap, eb);
    __syncthreads();
    if (tid < E) cnt[tid] = start;  // next free row of each expert
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int r0 = 0; r0 < A; r0 += NT) {
        for (int i = tid; i < NW * kMaxExperts; i += NT) (&wc[0][0])[i] = 0;
        __syncthreads();
        const int a = r0 + tid;
        const int id0 = a < A ? clamp_expert(sids[a], E) : 0;
        const bool valid = a < A && id0 >= eb && id0 < ee;
        if (a < A && !valid) inv_perm[a] = -1;
        const int id = valid ? id0 : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (id >> b) & 1;
            const uint64_t m = __ballot(valid && bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lanemask_lt());
        if (valid && rank == 0) wc[w][id] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int prefix = 0;
            for (int ww = 0; ww < w; ++ww) prefix += wc[ww][id];
            const int pos = cnt[id] + prefix + rank;
            sorted_token[pos] = a / k;
            inv_perm[a] = pos;
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) add += wc[ww][tid];
            cnt[tid] += add;
        }
        __syncthreads();
    }
}

}  // namespace moe
