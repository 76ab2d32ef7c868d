// decode_fused.hip -- the whole decode-sized layer in one cooperative launch.
//
// "CuTeDSL at Perplexity" (section Grid synchronization) runs small decode batches as a single
// kernel whose blocks meet at grid barriers instead of ending and relaunching, and its decode
// dispatch is one fused kernel (section Mixture-of-Experts Dispatch/Combine); the Muse Spark
// Open megakernel article keeps a whole layer in one launch.  Here one persistent grid (at most
// the blocks that fit on the GPU at once, launched cooperatively so that they are co-resident)
// walks four phases:
//   1. router logits, one (token, expert) block per wavefront of the grid (route.h);
//   -- grid barrier --
//   2. every block selects the top-k of every token and builds the dispatch (counts, offsets,
//      permutation, tile list) in its own LDS: the batch is small, so repeating this per block
//      costs less than another barrier; block 0 also writes the routing outputs.  Then the
//      gate/up + SwiGLU work items (gemv.h) in a grid-stride loop -> hid;
//   -- grid barrier --
//   3. the down work items -> y_perm;
//   -- grid barrier --
//   4. combine, fp32 in ascending slot order as combine.hip.
// Every phase runs the same device code, in the same order, as the multi-launch decode path,
// so with the same K split both paths give bit-identical results.
//
// Grid barriers: grid_sync.h.
#include <mutex>

#include "device.h"
#include "gemv.h"
#include "grid_sync.h"
#include "launch.h"
#include "route.h"
#include "select.h"

namespace moe {

// EPL: logits per lane in the selection (E <= 64 EPL); NV4: packed NVFP4 weights (else bf16).
template <int EPL, bool NV4>
__global__ __launch_bounds__(256) void decode_fused_kernel(FusedArgs a) {
    constexpr int NT = 256;
    __shared__ int s_ids[kFusedMaxRows];
    __shared__ float s_tw[kFusedMaxRows];
    __shared__ int s_counts[kFusedMaxExperts];
    __shared__ int s_off[kFusedMaxExperts + 1];
    __shared__ int s_st[kFusedMaxRows];
    __shared__ int s_ip[kFusedMaxRows];
    __shared__ Tile s_tiles[kFusedTileCap];
    __shared__ int s_tc;
    __shared__ uint64_t s_seq;
    __shared__ f32x4_t red[4][2][64];
    const int tid = threadIdx.x;
    const int T = a.T, E = a.E, k = a.k, A = T * k;

    if (tid == 0) s_seq = load_agent(&a.sync->seq);
    __syncthreads();
    const uint64_t base = 4 * s_seq;

    // 1. router logits: one (token, expert) block per wavefront
    {
        const int wave = blockIdx.x * (NT / kWave) + tid / kWave, nw = gridDim.x * (NT / kWave);
        if (long(T) * E <= 2048) {
            for (int w = wave; w < T * E; w += nw)
                router_logits_wave<true, 1, 1>(a.x, a.wr, a.bias, a.logits, T, a.H, E, w);
        } else {
            for (int w = wave; w < T * ((E + 1) / 2); w += nw)
                router_logits_wave<true, 1, 2>(a.x, a.wr, a.bias, a.logits, T, a.H, E, w);
        }
    }
    grid_barrier(a.sync, base + 1, a.spin_limit);

    // 2. selection and dispatch of the whole batch in this block's LDS, then gate/up + SwiGLU
    select_dispatch_block<EPL, NT>(a.logits, T, E, k, a.renorm, s_ids, s_tw, s_counts, s_off, s_st, s_ip,
                                   s_tiles, &s_tc, 16, nullptr, nullptr, 0, kFusedTileCap, a.eb, a.ee);
    __syncthreads();
    if (blockIdx.x == 0) {  // the routing outputs, as the multi-launch path writes them
        for (int i = tid; i < A; i += NT) {
            if (a.ids) a.ids[i] = s_ids[i];
            if (a.tw) a.tw[i] = s_tw[i];
            if (a.inv_perm) a.inv_perm[i] = s_ip[i];
            if (a.sorted_token) a.sorted_token[i] = s_st[i];
        }
        for (int e = tid; e <= E; e += NT) {
            if (a.offsets) a.offsets[e] = s_off[e];
            if (a.counts && e < E) a.counts[e] = s_counts[e];
        }
    }
    GemmArgs g1 = a.g1;
    g1.a_rows = s_st;
    g1.tiles = s_tiles;
    g1.tile_count = &s_tc;
    GemmArgs g2 = a.g2;
    g2.tiles = s_tiles;
    g2.tile_count = &s_tc;
    const int ntiles = s_tc;
    if constexpr (NV4) {
        const int n1 = ntiles * (g1.F / 16), n2 = ntiles * (g2.N / 16 / 2);
        for (int item = blockIdx.x; item < n1; item += gridDim.x) {
            __syncthreads();  // the previous item's split-K partials have been read
            decode_nvfp4p_item<kGateUp, 4, 1>(g1, item, red);
        }
        grid_barrier(a.sync, base + 2, a.spin_limit);
        // 3. down projection
        for (int item = blockIdx.x; item < n2; item += gridDim.x) {
            __syncthreads();
            decode_nvfp4p_item<kDown, 4, 2>(g2, item, reinterpret_cast<f32x4_t(*)[2][64]>(red));
        }
    } else {
        const int n1 = ntiles * (g1.F / 16), n2 = ntiles * (g2.N / 16);
        for (int item = blockIdx.x; item < n1; item += gridDim.x) {
            __syncthreads();
            decode_gemm_item<kGateUp, kWBF16, 4>(g1, item, red);
        }
        grid_barrier(a.sync, base + 2, a.spin_limit);
        for (int item = blockIdx.x; item < n2; item += gridDim.x) {
            __syncthreads();
            decode_gemm_item<kDown, kWBF16, 4>(g2, item, reinterpret_cast<f32x4_t(*)[1][64]>(red));
        }
    }
    grid_barrier(a.sync, base + 3, a.spin_limit);

    // 4. combine: y[t] = sum_j w[t,j] y_perm[inv_perm[t,j]], fp32 in ascending j, one rounding
    {
        const uint4* src = static_cast<const uint4*>(a.y_perm);
        uint4* dst = static_cast<uint4*>(a.y);
        const int nv = a.H / 8;
        for (int i = blockIdx.x * NT + tid; i < T * nv; i += gridDim.x * NT) {
            const int t = i / nv, v = i % nv;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < k; ++j) {
                const int r = s_ip[t * k + j];
                if (r < 0) continue;
                const uint4 q = src[size_t(min(r, A - 1)) * nv + v];
                const float wj = s_tw[t * k + j];
                const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    acc[2 * p] = __builtin_fmaf(wj, bf16_lo(u[p]), acc[2 * p]);
                    acc[2 * p + 1] = __builtin_fmaf(wj, bf16_hi(u[p]), acc[2 * p + 1]);
                }
            }
            dst[size_t(t) * nv + v] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        }
    }
    // every block read the sequence number before the first barrier; the next call uses S + 1
    if (blockIdx.x == 0 && tid == 0)
        __hip_atomic_store(&a.sync->seq, s_seq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------

namespace {

template <int EPL, bool NV4>
hipError_t launch_fused_variant(const FusedArgs& a, int blocks_per_cu, hipStream_t s) {
    // blocks that fit at once on this device (cached per device: a device property)
    static std::once_flag once[64];
    static int fit[64];
    int d = 0;
    hipError_t err = hipGetDevice(&d);
    if (err != hipSuccess) return err;
    if (d < 0 || d >= 64) return hipErrorInvalidDevice;
    std::call_once(once[d], [d] {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_fused_kernel<EPL, NV4>, 256, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess)
            per_cu = cus = 0;
        fit[d] = per_cu * 1024 + (cus < 1023 ? cus : 1023);  // both in one word
    });
    const int per_cu = fit[d] / 1024, cus = fit[d] % 1024;
    if (per_cu <= 0 || cus <= 0) return hipErrorLaunchFailure;
    const int bpc = blocks_per_cu > 0 && blocks_per_cu < per_cu ? blocks_per_cu : per_cu;
    const int grid = bpc * cus < kFusedMaxBlocks ? bpc * cus : kFusedMaxBlocks;
    FusedArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(decode_fused_kernel<EPL, NV4>), dim3(grid),
                                      dim3(256), params, 0, s);
}

}  // namespace

hipError_t launch_decode_fused(const FusedArgs& a, bool nv4, int blocks_per_cu, hipStream_t s) {
    const int epl = (a.E + kWave - 1) / kWave;  // E <= kFusedMaxExperts: at most 4 per lane
    hipError_t e;
    if (nv4) {
        e = epl <= 1 ? launch_fused_variant<1, true>(a, blocks_per_cu, s)
          : epl <= 2 ? launch_fused_variant<2, true>(a, blocks_per_cu, s)
                     : launch_fused_variant<4, true>(a, blocks_per_cu, s);
    } else {
        e = epl <= 1 ? launch_fused_variant<1, false>(a, blocks_per_cu, s)
          : epl <= 2 ? launch_fused_variant<2, false>(a, blocks_per_cu, s)
                     : launch_fused_variant<4, false>(a, blocks_per_cu, s);
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace moe
