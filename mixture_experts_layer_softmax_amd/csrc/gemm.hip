// gemm.hip -- grouped expert GEMMs of the MoE layer on gfx950.
//
// The MoE GEMMs multiply each expert's dispatched rows by that expert's weights ("Hosting
// Qwen on Blackwell", section MoE GEMM; "CuTeDSL at Perplexity", section Mixture-of-Experts
// Dispatch/Combine: dispatch feeds per-expert buffers to the MoE GEMM kernel).  Two kinds:
//   gate/up  hid[r] = silu(x_r . Wg[e]^T) * (x_r . Wu[e]^T)   (SwiGLU fused in the epilogue,
//            as the megakernel of the Muse Spark Open article dedicates a stage to SwiGLU)
//   down     y_perm[r] = hid[r] . W2[e]^T
// Work is a list of (expert, row range) tiles written on the device by dispatch, so the host
// never reads the routing; blocks past the list's end exit at once.
//
// bf16 path: v_mfma_f32_16x16x32_bf16, fp32 accumulate.  A block stages 64-wide K slices of
// its activation rows (gathered through the dispatch map, no permuted copy of x) and of its
// weight rows in LDS, double buffered, with 16-byte chunks XOR-swizzled by row so that the
// MFMA operand reads are free of bank conflicts.  Gate and up rows that feed the same hid
// column sit in the same wavefront, so SwiGLU is applied to accumulators in registers.
//
// NVFP4 weights (E2M1 nibbles, E4M3 scale per 16 along K, fp32 per-expert scale) are decoded
// on the way into LDS: e2m1 * e4m3 has at most 6 significant bits, so it is exact in bf16 and
// the MFMA sees the exact weight; the per-expert scale multiplies the fp32 accumulator.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int BK = 64;  // K elements per LDS stage (8 chunks of 16 bytes in bf16)

__device__ __forceinline__ int lds_slot(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// E4M3 (FN) byte -> its value times 2^14, in fp32 (integer decode; subnormals included).
__device__ __forceinline__ float e4m3_times_2p14(uint32_t c) {
    const uint32_t e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 0)
        v = float(m) * 0x1p-9f;
    else
        v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    v = (c & 0x80) ? -v : v;
    return v * 0x1p14f;
}

// One E2M1 nibble -> fp32 value times 2^-14: the nibble's exponent/mantissa bits placed in an
// IEEE half (sign to bit 15) read 2^-14 * e2m1 exactly, including the subnormal code 0.5.
__device__ __forceinline__ float e2m1_times_2m14(uint32_t n) {
    const unsigned short h = (unsigned short)(((n & 7u) << 9) | ((n & 8u) << 12));
    return float(__builtin_bit_cast(_Float16, h));
}

// 8 nibbles (elements 0..7, even element in the low nibble) with their block scale -> 8 bf16.
__device__ __forceinline__ uint4 dequant8(uint32_t word, float s14) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float f0 = e2m1_times_2m14((word >> (8 * p)) & 15u) * s14;
        const float f1 = e2m1_times_2m14((word >> (8 * p + 4)) & 15u) * s14;
        o[p] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);  // exact
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

}  // namespace

// BM x BN block tile, WM x WN wavefronts.  For the gate/up kind the BN weight rows of a block
// are, per wavefront column, NI/2 16-row groups of gate rows followed by the matching up rows;
// the block writes BN/2 hid columns.
template <int BM, int BN, int WM, int WN, int KIND, int WFMT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int NT = WM * WN * 64;
    constexpr int MI = BM / WM / 16;
    constexpr int NI = BN / WN / 16;
    static_assert(MI >= 1 && NI >= 1, "tile too small for the wave grid");
    static_assert(KIND != kGateUp || NI % 2 == 0, "gate/up pairs need an even NI");
    constexpr int A_IT = BM * 8 / NT;
    constexpr int B_IT = BN * 8 / NT;
    constexpr int Q_IT = BN * 2 / NT;  // NVFP4: 32-element half rows per thread
    static_assert(A_IT >= 1 && A_IT * NT == BM * 8, "A tile / thread mismatch");
    static_assert(WFMT != kWBF16 || (B_IT >= 1 && B_IT * NT == BN * 8), "B tile / thread mismatch");
    static_assert(WFMT != kWNVFP4 || (Q_IT >= 1 && Q_IT * NT == BN * 2), "B tile / thread mismatch");

    __shared__ uint4 sA[2][BM * 8];
    __shared__ uint4 sB[2][BN * 8];

    if (int(blockIdx.x) >= *g.tile_count) return;
    const Tile tile = g.tiles[blockIdx.x];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nt = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;  // weight rows per expert

    auto brow = [&](int n) -> int {
        if (KIND == kGateUp) {
            const int q = n % (NI * 16), half = NI * 8;
            const int f = nt * (BN / 2) + (n / (NI * 16)) * half + (q % half);
            return q < half ? f : g.F + f;
        } else {
            return min(nt * BN + n, g.N - 1);
        }
    };

    // per-thread global pointers of the rows this thread stages
    const uint16_t* pa[A_IT];
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
        const int idx = tid + it * NT, row = idx >> 3, ch = idx & 7;
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[it] = static_cast<const uint16_t*>(g.a) + size_t(src) * K + ch * 8;
    }
    const uint16_t* pb[WFMT == kWBF16 ? B_IT : 1];
    const uint8_t* pq[WFMT == kWNVFP4 ? Q_IT : 1];
    const uint8_t* ps[WFMT == kWNVFP4 ? Q_IT : 1];
    if (WFMT == kWBF16) {
#pragma unroll
        for (int it = 0; it < B_IT; ++it) {
            const int idx = tid + it * NT, row = idx >> 3, ch = idx & 7;
            pb[it] = static_cast<const uint16_t*>(g.w) + (size_t(e) * Nw + brow(row)) * K + ch * 8;
        }
    } else {
#pragma unroll
        for (int it = 0; it < Q_IT; ++it) {
            const int idx = tid + it * NT, row = idx >> 1, hf = idx & 1;
            const size_t wr = size_t(e) * Nw + brow(row);
            pq[it] = static_cast<const uint8_t*>(g.w) + wr * (K / 2) + hf * 16;
            ps[it] = g.wscale + wr * (K / 16) + hf * 2;
        }
    }

    uint4 ra[A_IT];
    uint4 rb[WFMT == kWBF16 ? B_IT : Q_IT];
    uint32_t rs[WFMT == kWNVFP4 ? Q_IT : 1];

    auto gload = [&](int k0) {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) ra[it] = *reinterpret_cast<const uint4*>(pa[it] + k0);
        if (WFMT == kWBF16) {
#pragma unroll
            for (int it = 0; it < B_IT; ++it) rb[it] = *reinterpret_cast<const uint4*>(pb[it] + k0);
        } else {
#pragma unroll
            for (int it = 0; it < Q_IT; ++it) {
                rb[it] = *reinterpret_cast<const uint4*>(pq[it] + k0 / 2);
                rs[it] = *reinterpret_cast<const uint16_t*>(ps[it] + k0 / 16);
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_IT; ++it) {
            const int idx = tid + it * NT;
            sA[buf][lds_slot(idx >> 3, idx & 7)] = ra[it];
        }
        if (WFMT == kWBF16) {
#pragma unroll
            for (int it = 0; it < B_IT; ++it) {
                const int idx = tid + it * NT;
                sB[buf][lds_slot(idx >> 3, idx & 7)] = rb[it];
            }
        } else {
#pragma unroll
            for (int it = 0; it < Q_IT; ++it) {
                const int idx = tid + it * NT, row = idx >> 1, hf = idx & 1;
                const float s0 = e4m3_times_2p14(rs[it] & 0xffu);
                const float s1 = e4m3_times_2p14(rs[it] >> 8);
                sB[buf][lds_slot(row, hf * 4 + 0)] = dequant8(rb[it].x, s0);
                sB[buf][lds_slot(row, hf * 4 + 1)] = dequant8(rb[it].y, s0);
                sB[buf][lds_slot(row, hf * 4 + 2)] = dequant8(rb[it].z, s1);
                sB[buf][lds_slot(row, hf * 4 + 3)] = dequant8(rb[it].w, s1);
            }
        }
    };

    f32x4_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 4 + (lane >> 4);
            bf16x8_t af[MI], bf[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                af[mi] = __builtin_bit_cast(bf16x8_t, sA[cur][lds_slot(wm * MI * 16 + mi * 16 + (lane & 15), ch)]);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bf[ni] = __builtin_bit_cast(bf16x8_t, sB[cur][lds_slot(wn * NI * 16 + ni * 16 + (lane & 15), ch)]);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    const float gs = (WFMT == kWNVFP4 && g.gscale) ? g.gscale[e] : 1.0f;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + wm * MI * 16 + mi * 16 + 4 * (lane >> 4) + i;
            if (row >= r1) continue;
            if (KIND == kGateUp) {
#pragma unroll
                for (int ni = 0; ni < NI / 2; ++ni) {
                    const int col = nt * (BN / 2) + wn * NI * 8 + ni * 16 + (lane & 15);
                    const float h = silu_mul(acc[mi][ni][i] * gs, acc[mi][ni + NI / 2][i] * gs);
                    out[size_t(row) * g.F + col] = (uint16_t)bf16_rne(h);
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const int col = nt * BN + wn * NI * 16 + ni * 16 + (lane & 15);
                    if (col < g.N) out[size_t(row) * g.N + col] = (uint16_t)bf16_rne(acc[mi][ni][i] * gs);
                }
            }
        }
}

// fp32 activations and weights: a plain 64 x 64 SIMT tile, 4 x 4 outputs per thread.  For the
// gate/up kind, B columns 0..31 are gate rows and 32..63 the matching up rows (32 hid columns).
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
    constexpr int TB = 64, TK = 16;
    __shared__ float sA[TK][TB + 4];
    __shared__ float sB[TK][TB + 4];
    if (int(blockIdx.x) >= *g.tile_count) return;
    const Tile tile = g.tiles[blockIdx.x];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nt = blockIdx.y, tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;
    const float* A = static_cast<const float*>(g.a);
    const float* W = static_cast<const float*>(g.w);
    auto brow = [&](int n) -> int {
        if (KIND == kGateUp) return n < 32 ? nt * 32 + n : g.F + nt * 32 + (n - 32);
        return min(nt * TB + n, g.N - 1);
    };
    // columns of this thread
    int cols[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        cols[j] = (KIND == kGateUp) ? ((j < 2) ? tx * 2 + j : 32 + tx * 2 + (j - 2)) : tx * 4 + j;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + it * 256, row = idx / TK, kk = idx % TK;
            const int rr = min(r0 + row, r1 - 1);
            int src = g.a_rows ? g.a_rows[rr] : rr;
            src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
            sA[kk][row] = A[size_t(src) * K + k0 + kk];
            sB[kk][row] = W[(size_t(e) * Nw + brow(row)) * K + k0 + kk];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = sB[kk][cols[j]];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* out = static_cast<float*>(g.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + ty * 4 + i;
        if (row >= r1) continue;
        if (KIND == kGateUp) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                out[size_t(row) * g.F + nt * 32 + tx * 2 + j] = silu_mul(acc[i][j], acc[i][j + 2]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = nt * TB + tx * 4 + j;
                if (col < g.N) out[size_t(row) * g.N + col] = acc[i][j];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------

namespace {
// prefill: 128 x 128 tiles, 2 x 2 wavefronts of 64 x 64; decode: 16 x 64 tiles, 1 x 2
// wavefronts of 16 x 32 (weight streaming, many blocks for few rows).
constexpr int PF_BM = 128, PF_BN = 128, PF_WM = 2, PF_WN = 2;
constexpr int DC_BM = 16, DC_BN = 64, DC_WM = 1, DC_WN = 2;
}  // namespace

int gemm_tile_rows(int family) {
    return family == kFamSimtF32 ? 64 : family == kFamPrefill ? PF_BM : DC_BM;
}

template <int BM, int BN, int WM, int WN>
static void launch_mfma(const GemmArgs& g, int max_tiles, hipStream_t s) {
    const int ncols = g.kind == kGateUp ? g.F / (BN / 2) : (g.N + BN - 1) / BN;
    dim3 grid(max_tiles, ncols), block(WM * WN * 64);
    if (g.kind == kGateUp) {
        if (g.wfmt == kWBF16)
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kGateUp, kWBF16>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kGateUp, kWNVFP4>), grid, block, 0, s, g);
    } else {
        if (g.wfmt == kWBF16)
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kDown, kWBF16>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, kDown, kWNVFP4>), grid, block, 0, s, g);
    }
}

hipError_t launch_gemm(const GemmArgs& g, int family, int max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    if (family == kFamSimtF32) {
        const int ncols = g.kind == kGateUp ? g.F / 32 : (g.N + 63) / 64;
        dim3 grid(max_tiles, ncols), block(256);
        if (g.kind == kGateUp)
            hipLaunchKernelGGL((gemm_f32_kernel<kGateUp>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((gemm_f32_kernel<kDown>), grid, block, 0, s, g);
    } else if (family == kFamPrefill) {
        launch_mfma<PF_BM, PF_BN, PF_WM, PF_WN>(g, max_tiles, s);
    } else {
        launch_mfma<DC_BM, DC_BN, DC_WM, DC_WN>(g, max_tiles, s);
    }
    return hipGetLastError();
}

}  // namespace moe
