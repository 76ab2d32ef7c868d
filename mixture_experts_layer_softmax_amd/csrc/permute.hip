// permute.hip -- dispatch: per-expert counts, offsets and the stable permutation.
//
// Follows the local dispatch of "CuTeDSL at Perplexity" (section Mixture-of-Experts
// Dispatch/Combine, Local): count the tokens routed to every expert, give each (token, slot)
// a unique index inside its expert's list, and lay the rows out per expert for the MoE GEMMs.
// The pages assign those indices with shared-memory atomics, first locally per block and then
// aggregated across blocks in global memory; here the same two-level structure is kept
// (per-chunk histograms -> one scan -> per-chunk scatter) but each index is a deterministic
// rank, so rows of one expert appear in ascending (token, slot) order and the permutation is
// unique.  A chunk is 64 tokens (64*k assignments); a batch of up to 64 tokens is a single
// chunk, i.e. one block, which is the pages' decode case.
#include "device.h"
#include "launch.h"
#include "select.h"

namespace moe {

// hist[c, e] = number of assignments of chunk c routed to expert e (integer atomics on LDS:
// the counts do not depend on their order).
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int T, int k,
                                                   int E, int eb, int ee, int32_t* __restrict__ hist) {
    __shared__ int cnt[kMaxExperts];
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const int a0 = c * kChunkTokens * k;
    const int a1 = min(T, (c + 1) * kChunkTokens) * k;
    for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
        const int id = clamp_expert(ids[a], E);
        if (id >= eb && id < ee) atomicAdd(&cnt[id], 1);  // only held experts are dispatched
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[size_t(c) * E + e] = cnt[e];
}

// One block of kScanThreads threads: counts, offsets, per-chunk bases, GEMM tile lists.  The
// chunks are cut into P = kScanThreads / Ep parts (Ep: E rounded up to a power of two), and
// thread (p, e) = (tid / Ep, tid % Ep) walks expert e's column of the chunk histograms over
// part p, 32 chunks per batch of independent loads, holding the part's values in registers
// when it has at most 32 chunks (every dispatch of up to 8192 tokens over up to 256 experts),
// so that the walk costs one memory round trip instead of one per batch and pass.  Measured,
// kernel trace median, 8192 tokens over 256 experts: 18.6 -> 13.0 us.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ hist,
                                                            int nchunks, int E, int Ep,
                                                            int32_t* __restrict__ base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            Tile* tiles1, int* tile_count1, int bm1,
                                                            Tile* tiles2, int* tile_count2,
                                                            int bm2, int cap, int eb) {
    constexpr int kBatch = 32;
    __shared__ int part_sum[kScanThreads];  // [p][e]: column sum of part p
    const int P = kScanThreads / Ep;
    const int p = threadIdx.x / Ep, e = threadIdx.x % Ep;
    const int per = (nchunks + P - 1) / P;
    const int c_begin = min(p * per, nchunks), c_end = min(c_begin + per, nchunks);
    const bool col = e < E;
    int h[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) h[i] = 0;
    int run = 0;
    if (col) {
        for (int c0 = c_begin; c0 < c_end; c0 += kBatch) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i) h[i] = (c0 + i < c_end) ? hist[size_t(c0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) run += h[i];
        }
    }
    part_sum[threadIdx.x] = run;
    __syncthreads();
    // thread (0, e) owns expert e's total; the block scan runs over threads in expert order
    int total_e = 0, before = 0;  // expert e's count; rows of e in parts before p
    if (col) {
        for (int q = 0; q < P; ++q) {
            const int v = part_sum[q * Ep + e];
            if (q < p) before += v;
            total_e += v;
        }
    }
    int total;
    const int start = block_exclusive_scan<kScanThreads>(p == 0 && col ? total_e : 0, &total);
    __shared__ int start_of[kMaxExperts];
    if (p == 0 && col) {
        start_of[e] = start;
        if (counts) counts[e] = total_e;
        offsets[e] = start;
    }
    __syncthreads();
    if (col) {
        int acc = start_of[e] + before;
        if (c_end - c_begin <= kBatch) {  // the part's values are still in registers
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (c_begin + i < c_end) base[size_t(c_begin + i) * E + e] = acc;
                acc += h[i];
            }
        } else {
            for (int c0 = c_begin; c0 < c_end; c0 += kBatch) {
#pragma unroll
                for (int i = 0; i < kBatch; ++i) h[i] = (c0 + i < c_end) ? hist[size_t(c0 + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    if (c0 + i < c_end) base[size_t(c0 + i) * E + e] = acc;
                    acc += h[i];
                }
            }
        }
    }
    if (threadIdx.x == 0) offsets[E] = total;
    // tile lists: one thread per expert (thread (0, e)), in expert order
    const int te = (p == 0) ? e : E;
    const int tcount = (p == 0 && col) ? total_e : 0;
    const int tstart = (p == 0 && col) ? start : 0;
    if (tiles1) emit_tiles<kScanThreads>(te, E, tcount, tstart, bm1, tiles1, tile_count1, cap, eb);
    if (tiles2) emit_tiles<kScanThreads>(te, E, tcount, tstart, bm2, tiles2, tile_count2, cap, eb);
}

// Tile list straight from caller-supplied offsets (stand-alone grouped GEMM entry point).
// Offsets are clamped to [0, A] so that no tile reaches past the A dispatched rows.
__global__ __launch_bounds__(kMaxExperts) void tiles_from_offsets_kernel(
    const int32_t* __restrict__ offsets, int E, int eb, int ee, int A, int bm, Tile* tiles,
    int* tile_count, int cap) {
    const int e = threadIdx.x;
    int start = 0, count = 0;
    if (e >= eb && e < ee) {  // rows of experts that are not held are never computed
        start = min(max(offsets[e], 0), A);
        const int end = min(max(offsets[e + 1], start), A);
        count = end - start;
    }
    emit_tiles(e, E, count, start, bm, tiles, tile_count, cap, eb);
}

// Stable scatter of one chunk.  Assignments are taken 256 at a time in (t, j) order; within a
// wave, lanes holding the same expert find each other with one ballot per id bit, and wave
// totals are prefix-summed across the 4 waves through LDS.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids, int T, int k,
                                                      int E, int eb, int ee,
                                                      const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ sorted_token,
                                                      int32_t* __restrict__ inv_perm) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int wc[4][kMaxExperts];
    const int c = blockIdx.x;
    const int lane = lane_id(), w = threadIdx.x / kWave;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    const int a0 = c * kChunkTokens * k;
    const int a1 = min(T, (c + 1) * kChunkTokens) * k;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int r0 = a0; r0 < a1; r0 += 256) {
        for (int i = threadIdx.x; i < 4 * kMaxExperts; i += blockDim.x) (&wc[0][0])[i] = 0;
        __syncthreads();
        const int a = r0 + threadIdx.x;
        const int id0 = a < a1 ? clamp_expert(ids[a], E) : 0;
        const bool valid = a < a1 && id0 >= eb && id0 < ee;
        if (a < a1 && !valid) inv_perm[a] = -1;  // routed to an expert that is not held
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
            const int pos = base[size_t(c) * E + id] + cnt[id] + prefix + rank;
            sorted_token[pos] = a / k;
            inv_perm[a] = pos;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += blockDim.x)
            cnt[e] += wc[0][e] + wc[1][e] + wc[2][e] + wc[3][e];
        __syncthreads();
    }
}

// x_perm[r] = x[sorted_token[r]]; 16-byte copies.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_token,
                                                          uint4* __restrict__ x_perm, int A, int T,
                                                          int row_vec) {
    const long n = long(A) * row_vec;
    for (long i = long(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += long(gridDim.x) * blockDim.x) {
        const long r = i / row_vec, v = i % row_vec;
        int t = sorted_token[r];
        t = t < 0 ? 0 : (t >= T ? T - 1 : t);
        x_perm[i] = x[long(t) * row_vec + v];
    }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int value) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = value;
}

// ---------------------------------------------------------------------------------------

hipError_t launch_fill_i32(int32_t* p, int n, int value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256),
                       0, s, p, n, value);
    return hipGetLastError();
}

template <int EPL, int NT>
__global__ __launch_bounds__(NT) void select_dispatch_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ ids,
    float* __restrict__ tw, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_perm, Tile* tiles1,
    int* tile_count1, int bm1, Tile* tiles2, int* tile_count2, int bm2, int cap, int eb, int ee) {
    static_assert(NT >= kMaxExperts, "a thread per expert");
    select_dispatch_block<EPL, NT>(logits, T, E, k, renorm, ids, tw, counts, offsets, sorted_token,
                                   inv_perm, tiles1, tile_count1, bm1, tiles2, tile_count2, bm2, cap,
                                   eb, ee);
}

hipError_t launch_select_dispatch_small(const float* logits, int renorm, int32_t* tw_ids,
                                        float* tw, const DispatchArgs& d, hipStream_t s) {
    const int epl = (d.E + kWave - 1) / kWave;
#define MOE_SDS(N, NT)                                                                              \
    hipLaunchKernelGGL((select_dispatch_small_kernel<N, NT>), dim3(1), dim3(NT), 0, s, logits,      \
                       d.T, d.E, d.k, renorm, tw_ids, tw, d.counts, d.offsets, d.sorted_token,      \
                       d.inv_perm, d.tiles1, d.tile_count1, d.bm1, d.tiles2, d.tile_count2, d.bm2,  \
                       d.tile_cap, d.ebegin, d.eend)
    // 16 wavefronts once there are more than 8 tokens, so that each selects at most two of 32
    // (kernel trace, median us, 512 -> 1024 threads: T=16 over 256 experts 13.8 -> 12.5, T=32
    // over 128 16.4 -> 14.4; but T=1 6.0 -> 6.7 and T=8 7.4 -> 7.5, so 8 wavefronts there)
    if (d.T > 8) {
        if (epl <= 1) MOE_SDS(1, 1024);
        else if (epl <= 2) MOE_SDS(2, 1024);
        else if (epl <= 4) MOE_SDS(4, 1024);
        else MOE_SDS(8, 1024);
    } else {
        if (epl <= 1) MOE_SDS(1, 512);
        else if (epl <= 2) MOE_SDS(2, 512);
        else if (epl <= 4) MOE_SDS(4, 512);
        else MOE_SDS(8, 512);
    }
#undef MOE_SDS
    return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& d, hipStream_t s) {
    const int nch = (d.T + kChunkTokens - 1) / kChunkTokens;
    hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(256), 0, s, d.ids, d.T, d.k, d.E, d.ebegin, d.eend,
                       d.hist);
    int ep = 64;
    while (ep < d.E) ep *= 2;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, d.hist, nch, d.E, ep, d.base,
                       d.counts, d.offsets, d.tiles1, d.tile_count1, d.bm1, d.tiles2,
                       d.tile_count2, d.bm2, d.tile_cap, d.ebegin);
    hipLaunchKernelGGL(scatter_kernel, dim3(nch), dim3(256), 0, s, d.ids, d.T, d.k, d.E, d.ebegin,
                       d.eend, d.base, d.sorted_token, d.inv_perm);
    return hipGetLastError();
}

hipError_t launch_tiles_from_offsets(const int32_t* offsets, int E, int eb, int ee, int A, int bm,
                                     Tile* tiles, int* tile_count, int cap, hipStream_t s) {
    hipLaunchKernelGGL(tiles_from_offsets_kernel, dim3(1), dim3(kMaxExperts), 0, s, offsets, E, eb,
                       ee, A, bm, tiles, tile_count, cap);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* sorted_token, void* x_perm, int A,
                              int T, int row_bytes, hipStream_t s) {
    const int row_vec = row_bytes / 16;
    const long n = long(A) * row_vec;
    const int blocks = int(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(x), sorted_token, static_cast<uint4*>(x_perm), A, T,
                       row_vec);
    return hipGetLastError();
}

}  // namespace moe
