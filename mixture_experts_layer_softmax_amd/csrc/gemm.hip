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
// Kernels (all v_mfma_f32_16x16x32_bf16 with fp32 accumulation, except the fp32 one):
//   gemm_prefill_bf16_kernel   many rows per expert, bf16 weights in the packed stage layout
//                              of moe.h: 256 x 256 tiles, operands DMA'd into an LDS ring
//   gemm_prefill_nvfp4_kernel  the same for NVFP4 weights: raw nibbles and scales DMA'd and
//                              decoded to bf16 in LDS by the block
//   gemm_decode_kernel         few rows per expert: weights stream straight into MFMA
//                              operand registers (bf16 packed, or NVFP4 row-major)
//   gemm_fallback_kernel       NVFP4 shapes the two above do not tile (F % 128 or K % 128)
//   gemm_f32_kernel            fp32 layers (fp32 MFMA)
// Gate and up rows that feed the same hid column sit in the same wavefront, so SwiGLU is
// applied to accumulators in registers.  Activation rows are gathered through the dispatch
// map (no permuted copy of x).
//
// NVFP4 weights (E2M1 nibbles, E4M3 scale per 16 along K, fp32 per-expert scale) are decoded
// before the MFMA: e2m1 * e4m3 has at most 6 significant bits, so it is exact in bf16 and the
// MFMA sees the exact weight; the per-expert scale multiplies the fp32 accumulator.
#include "device.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

namespace {

constexpr int BK = 64;  // K elements per LDS stage (8 chunks of 16 bytes in bf16)

__device__ __forceinline__ int lds_slot(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// E4M3 (FN) byte -> its value in fp32 (integer decode; subnormals included).  Both cases are
// computed and selected, so the decode is straight-line code with no divergent branch.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15, m = c & 7;
    const float sub = float(m) * 0x1p-9f;
    const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float v = e ? nrm : sub;
    return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// 8 nibbles (elements 0..7, even element in the low nibble) times their block scale -> 8 bf16.
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 gives the two E2M1 values of one byte exactly in
// fp32 (the instruction applies only the exponent of its scale, so the E4M3 scale, which has
// a mantissa, is multiplied separately).  e2m1 * e4m3 has at most 6 significant bits, so the
// product is exact in fp32 and its upper half is the exact bf16; v_perm_b32 packs two of them.
__device__ __forceinline__ uint4 dequant8(uint32_t word, float s) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f32x2_t v;
        if (p == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
        else if (p == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
        else if (p == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
        else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
        o[p] = __builtin_amdgcn_perm(__float_as_uint(v.y * s), __float_as_uint(v.x * s), 0x07060302u);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

// Fallback grouped GEMM for the NVFP4 shapes the kernels below do not tile (F % 128 != 0 for
// prefill, K % 128 != 0 for decode): BM x BN block tile, WM x WN wavefronts, operands staged
// through registers into a double-buffered LDS tile (64-wide K slices, XOR-swizzled chunks).
// For the gate/up kind the BN weight rows of a block are, per wavefront column, NI/2 16-row
// groups of gate rows followed by the matching up rows; the block writes BN/2 hid columns.
template <int BM, int BN, int WM, int WN, int KIND, int WFMT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_fallback_kernel(GemmArgs g) {
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
                const float s0 = e4m3_value(rs[it] & 0xffu);
                const float s1 = e4m3_value(rs[it] >> 8);
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


// ---------------------------------------------------------------------------------------
// Prefill kernel, bf16 weights: 256 x 256 block tile, 8 wavefronts (2 x 4) of 128 x 64, two
// per SIMD (128 fp32 accumulators and about 250 registers per lane each), so that while one
// wavefront waits for LDS data the other issues MFMAs.  K in 32-wide stages; a 4-slot LDS ring
// (4 x 32 KiB) is filled by direct global->LDS loads (each wavefront moves two 1 KiB groups of
// activation rows and two of weight rows per stage) and the operand fragments of the next
// stage are read from LDS into registers while the MFMAs of the current stage run.  Rows are 64
// bytes in LDS; the 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 3), which keeps the
// fragment reads (8 consecutive rows, one chunk) on distinct banks.  Activation rows are
// gathered through the dispatch map; weights come in the packed layout, where every stage of a
// 256-row tile is already this LDS image (one contiguous 16 KiB read).  The 16 groups of 16
// rows alternate between the two wavefront rows and groups past the tile's last row skip their
// MFMAs.  For gate/up, wavefront column c holds weight row groups {0, 1, 4, 5} + 8 (c >> 1) +
// 2 (c & 1) of the tile's 16: 32 gate rows and the 32 up rows of the same hid columns.
// ---------------------------------------------------------------------------------------


template <int KIND>
__global__ __launch_bounds__(512, 1) void gemm_prefill_bf16_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BKS = 32;
    constexpr int HALF = (KIND == kGateUp) ? BN / 2 : BN;
    __shared__ uint4 sA0[BM * 4], sA1[BM * 4], sA2[BM * 4], sA3[BM * 4];
    __shared__ uint4 sB0[BN * 4], sB1[BN * 4], sB2[BN * 4], sB3[BN * 4];

    const int ncols = (KIND == kGateUp) ? g.F / HALF : (g.N + BN - 1) / BN;
    const int items = *g.tile_count * ncols;
    const int run = (items + 7) >> 3;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int item = xcd * run + j;
    if (j >= run || item >= items) return;
    const Tile tile = g.tiles[item / ncols];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nsub = (r1 - r0 + 15) / 16;
    const int nt = item % ncols;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
    const int wr = wave >> 2, wc = wave & 3;                      // 2 x 4 wavefronts
    const int K = g.K;

    const char* pa[2];
    // A operand: gathered rows (64 bytes per row and stage), or for the down GEMM of a forward
    // the packed hid image of this row tile (one contiguous 16 KiB per stage, like the weights)
    const bool apk = KIND == kDown && g.hid_packed;
    const int astep = apk ? 512 : 2;  // bytes per K element along the A stream
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (apk) {
            pa[i] = static_cast<const char*>(g.a) + size_t(item / ncols) * size_t(K / BKS) * 16384 +
                    (i * 8 + wave) * 1024 + lane * 16;
            continue;
        }
        const int row = (i * 8 + wave) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[i] = static_cast<const char*>(g.a) + (size_t(src) * K + ch * 8) * 2;
    }
    const char* const wblk = static_cast<const char*>(g.w) + (size_t(e) * ncols + nt) * size_t(K / BKS) * 16384;
    const char* pb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) pb[i] = wblk + (i * 8 + wave) * 1024 + lane * 16;
    // B row groups of this wavefront: gate/up -> two gate groups and the matching up groups
    int gb[4];
    if (KIND == kGateUp) {
        const int base = (wc >> 1) * 8 + (wc & 1) * 2;
        gb[0] = base; gb[1] = base + 1; gb[2] = base + 4; gb[3] = base + 5;
    } else {
        gb[0] = 4 * wc; gb[1] = 4 * wc + 1; gb[2] = 4 * wc + 2; gb[3] = 4 * wc + 3;
    }

#define MOE_ISSUE8(SA, SB, K0)                                                                  \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                           \
            dma16(pa[i] + k0_ * astep, &SA[(i * 8 + wave) * 64]);                               \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                           \
            dma16(pb[i] + k0_ * 512, &SB[(i * 8 + wave) * 64]);                                 \
    } while (0)
#define MOE_READ8(SA, SB, AF, BF)                                                               \
    do {                                                                                        \
        const int ch_ = lane >> 4;                                                              \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) BF[ni] =                               \
            __builtin_bit_cast(bf16x8_t, SB[lds_slot32(gb[ni] * 16 + (lane & 15), ch_)]);        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) AF[mi] =                               \
            __builtin_bit_cast(bf16x8_t, SA[lds_slot32((mi * 2 + wr) * 16 + (lane & 15), ch_)]); \
    } while (0)
#define MOE_MFMA8(AF, BF)                                                                       \
    do {                                                                                        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) {                                      \
            if (mi * 2 + wr < nsub) {                                                           \
                _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) acc[mi][ni] =                  \
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[mi], BF[ni], acc[mi][ni], 0, 0, 0); \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    f32x4_t acc[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t a0[8], b0[4], a1[8], b1[4];

    const int nk = K / BKS;
    const int last = (nk - 1) * BKS;
    MOE_ISSUE8(sA0, sB0, 0);
    MOE_ISSUE8(sA1, sB1, min(1 * BKS, last));
    MOE_ISSUE8(sA2, sB2, min(2 * BKS, last));
    wait_vm_lgkm0<8>();
    block_barrier();
    MOE_READ8(sA0, sB0, a0, b0);
    MOE_ISSUE8(sA3, sB3, min(3 * BKS, last));
    for (int s = 0;; s += 4) {
        wait_vm_lgkm0<8>();
        block_barrier();
        MOE_READ8(sA1, sB1, a1, b1);
        MOE_ISSUE8(sA0, sB0, min((s + 4) * BKS, last));
        MOE_MFMA8(a0, b0);
        if (s + 1 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        MOE_READ8(sA2, sB2, a0, b0);
        MOE_ISSUE8(sA1, sB1, min((s + 5) * BKS, last));
        MOE_MFMA8(a1, b1);
        if (s + 2 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        MOE_READ8(sA3, sB3, a1, b1);
        MOE_ISSUE8(sA2, sB2, min((s + 6) * BKS, last));
        MOE_MFMA8(a0, b0);
        if (s + 3 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        MOE_READ8(sA0, sB0, a0, b0);
        MOE_ISSUE8(sA3, sB3, min((s + 7) * BKS, last));
        MOE_MFMA8(a1, b1);
        if (s + 4 >= nk) break;
    }
    wait_vm_lgkm0<0>();
#undef MOE_ISSUE8
#undef MOE_READ8
#undef MOE_MFMA8

    // Epilogue through LDS: every wavefront is past its last fragment read once all have reached
    // the barrier, so each takes one 16 KiB ring array for its output tile (128 rows, 64 bf16
    // columns; 32 hid columns for gate/up), writes its results there in the MFMA layout and
    // reads them back as 16-byte row chunks for full-width global stores.  Chunk c8 of tile row
    // lr sits in slot c8 ^ ((lr >> 2) & (W / 8 - 1)), so the four row groups of one LDS write
    // (rows 4 apart) fall on different banks.
    block_barrier();
    constexpr int W = (KIND == kGateUp) ? 32 : 64;  // columns per wavefront
    constexpr int SM = W / 8 - 1;
    uint16_t* const stg = reinterpret_cast<uint16_t*>(
        wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sA2 : wave == 3 ? sA3 :
        wave == 4 ? sB0 : wave == 5 ? sB1 : wave == 6 ? sB2 : sB3);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        if (mi * 2 + wr >= nsub) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = mi * 16 + 4 * (lane >> 4) + i;
#pragma unroll
            for (int ni = 0; ni < W / 16; ++ni) {
                const int lc = ni * 16 + (lane & 15);
                const float v = (KIND == kGateUp) ? silu_mul(acc[mi][ni][i], acc[mi][ni + 2][i]) : acc[mi][ni][i];
                stg[lr * W + ((((lc >> 3) ^ (lr >> 2)) & SM) << 3) + (lc & 7)] = (uint16_t)bf16_rne(v);
            }
        }
    }
    // the LDS unit keeps one wavefront's accesses in order; this keeps the compiler from moving
    // the 16-byte reads (another type than the 2-byte writes) above them
    asm volatile("" ::: "memory");
    const int colbase = (KIND == kGateUp) ? nt * HALF + (wc >> 1) * 64 + (wc & 1) * 32 : nt * BN + wc * 64;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int it = 0; it < 128 * (W / 8) / 64; ++it) {
        const int q = it * 64 + lane, lr = q / (W / 8), c8 = q % (W / 8);
        const int tr = ((lr >> 4) * 2 + wr) * 16 + (lr & 15);  // row within the block tile
        const int row = r0 + tr;
        if ((tr >> 4) >= nsub || row >= r1) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(&stg[lr * W + (((c8 ^ (lr >> 2)) & SM) << 3)]);
        const int col = colbase + c8 * 8;
        if (KIND == kGateUp) {
            if (g.hid_packed) {  // tile row tr, stage col / 32, chunk (col / 8) % 4 in its slot
                const size_t blk = size_t(item / ncols) * (g.F / BKS) + (col >> 5);
                *reinterpret_cast<uint4*>(&out[blk * 8192 + tr * 32 + ((((col >> 3) & 3) ^ ((tr >> 1) & 3)) << 3)]) = v;
            } else {
                *reinterpret_cast<uint4*>(&out[size_t(row) * g.F + col]) = v;
            }
        } else if (col < g.N) {
            *reinterpret_cast<uint4*>(&out[size_t(row) * g.N + col]) = v;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Prefill kernel, NVFP4 weights: the bf16 kernel's 256 x 256 tile and activation DMA ring with
// NW = 4 wavefronts (2 x 2, 128 x 128 each) or NW = 8 (2 x 4, 128 x 64 each; measured: 8 for
// the down GEMM, 4 for gate/up); the weights are DMA'd raw (16 nibble bytes and one 4-byte
// scale word per weight row and stage, straight from the row-major NVFP4 arrays) and decoded
// by the block into a bf16 LDS slot (e2m1 * e4m3 is exact in bf16) after the MFMAs of the
// current stage are issued, so the decode overlaps the matrix core.  The per-expert fp32 scale
// multiplies the accumulators.
//
// Iteration i: activation stage i+1 and raw weight stage i+2 have landed (issued three
// iterations earlier); read the fragments of stage i+1 (activations from ring slot (i+1)%4,
// decoded weights from bf16 slot (i+1)%2); DMA activation stage i+4 (slot i%4) and raw weight
// stage i+5 (raw slot (i+1)%4); run the MFMAs of stage i; decode raw stage i+2 (raw slot
// (i+2)%4) into bf16 slot i%2.  Every wavefront issues the same number of DMA instructions
// per iteration (NW = 4: four activation, one nibble, one scale; NW = 8: two activation and
// one nibble or scale), so "landed" is a fixed load count; the barrier at the top of the
// iteration also publishes each raw row to the thread that decodes it.
// ---------------------------------------------------------------------------------------

template <int KIND, int NW, bool PK>
__global__ __launch_bounds__(NW * 64, 1) void gemm_prefill_nvfp4_kernel(GemmArgs g) {
    static_assert(NW == 4 || NW == 8, "4 or 8 wavefronts");
    constexpr int BM = 256, BN = 256, BKS = 32;
    constexpr int NC = NW / 2;        // wavefront columns
    constexpr int NB = 16 / NC;       // 16-row weight groups per wavefront
    constexpr int A_DMA = 16 / NW;    // activation DMA instructions per wavefront and stage
    constexpr int OPS = A_DMA + (NW == 4 ? 2 : 1);  // DMA instructions per wavefront and stage
    constexpr int HALF = (KIND == kGateUp) ? BN / 2 : BN;
    __shared__ uint4 sA0[BM * 4], sA1[BM * 4], sA2[BM * 4], sA3[BM * 4];
    __shared__ uint4 sN0[BN], sN1[BN], sN2[BN], sN3[BN];     // raw nibbles of weight row r
    __shared__ uint32_t sS0[BN], sS1[BN], sS2[BN], sS3[BN];  // raw scale word of weight row r
    __shared__ uint4 sB0[BN * 4], sB1[BN * 4];               // decoded bf16 stages

    const int ncols = (KIND == kGateUp) ? g.F / HALF : (g.N + BN - 1) / BN;
    const int items = *g.tile_count * ncols;
    const int run = (items + 7) >> 3;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int item = xcd * run + j;
    if (j >= run || item >= items) return;
    const Tile tile = g.tiles[item / ncols];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nsub = (r1 - r0 + 15) / 16;
    const int nt = item % ncols;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / NC, wc = wave % NC;
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;

    const char* pa[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int row = (i * NW + wave) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[i] = static_cast<const char*>(g.a) + (size_t(src) * K + ch * 8) * 2;
    }
    // raw weights: wavefront w moves the nibbles (NW = 4: and the scale words) of weight rows
    // 64 (w & 3) + lane, for NW = 8 wavefronts 4..7 the scale words; tile row r holds, per
    // 128-row half, 64 gate rows then the matching up rows (the packed bf16 order)
    const int mrow = (wave & 3) * 64 + lane;
    int wrow;
    if (KIND == kGateUp) {
        const int q = mrow & 127;
        const int f = nt * HALF + (mrow >> 7) * 64 + (q & 63);
        wrow = q < 64 ? f : g.F + f;
    } else {
        wrow = min(nt * BN + mrow, g.N - 1);
    }
    const size_t wrow_g = size_t(e) * Nw + wrow;
    // PK: tile nt of the PACKED layout holds exactly these rows in this order (row mrow at
    // 16 mrow of each 4 KiB stage block and at 4 mrow of each 1 KiB stage-pair scale block)
    const size_t tb = size_t(e) * ((KIND == kGateUp) ? g.F / 128 : g.N / 256) + nt;
    const char* const pq = PK ? static_cast<const char*>(g.w) + tb * (K / 32) * 4096 + mrow * 16
                              : static_cast<const char*>(g.w) + wrow_g * (K / 2);
    const char* const ps = PK ? reinterpret_cast<const char*>(g.wscale) + tb * (K / 64) * 1024 + mrow * 4
                              : reinterpret_cast<const char*>(g.wscale) + wrow_g * (K / 16);
    // weight row groups of this wavefront: gate/up, NB/2 gate groups then their up groups
    int gb[NB];
    int gcol;  // first hid column (gate/up) or output column (down) of this wavefront
#pragma unroll
    for (int ni = 0; ni < NB; ++ni) {
        if (KIND == kGateUp) {
            const int base = NW == 4 ? wc * 8 : (wc >> 1) * 8 + (wc & 1) * 2;
            gb[ni] = base + (ni < NB / 2 ? ni : 4 + ni - NB / 2);
        } else {
            gb[ni] = NB * wc + ni;
        }
    }
    if (KIND == kGateUp)
        gcol = nt * HALF + (NW == 4 ? wc * 64 : (wc >> 1) * 64 + (wc & 1) * 32);
    else
        gcol = nt * BN + wc * NB * 16;

#define MOE_ISSUE_A(SA, K0)                                                                     \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        _Pragma("unroll") for (int i = 0; i < A_DMA; ++i)                                       \
            dma16(pa[i] + k0_ * 2, &SA[(i * NW + wave) * 64]);                                  \
    } while (0)
    // nibbles of stage k0/32, and the scale word holding its two scales (stages 2m, 2m+1)
#define MOE_ISSUE_W(SN, SS, K0)                                                                 \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        if (NW == 4 || wave < 4)                                                                \
            dma16(pq + (PK ? (k0_ >> 5) * 4096 : k0_ / 2), &SN[(wave & 3) * 64]);               \
        if (NW == 4 || wave >= 4)                                                               \
            dma4(ps + (PK ? (k0_ >> 6) * 1024 : ((k0_ >> 4) & ~3)), &SS[(wave & 3) * 64]);      \
    } while (0)
    // NW = 4: thread t decodes weight row t; NW = 8: half h = t & 1 of row t >> 1 (chunks
    // 2h, 2h+1, scale h)
#define MOE_DECODE(SN, SS, SB, K0)                                                              \
    do {                                                                                        \
        if constexpr (NW == 4) {                                                                \
            const uint4 nib_ = SN[tid];                                                         \
            const uint32_t sw_ = SS[tid] >> ((((K0) >> 5) & 1) * 16);                           \
            const float s0_ = e4m3_value(sw_ & 0xffu), s1_ = e4m3_value((sw_ >> 8) & 0xffu);      \
            SB[lds_slot32(tid, 0)] = dequant8(nib_.x, s0_);                                     \
            SB[lds_slot32(tid, 1)] = dequant8(nib_.y, s0_);                                     \
            SB[lds_slot32(tid, 2)] = dequant8(nib_.z, s1_);                                     \
            SB[lds_slot32(tid, 3)] = dequant8(nib_.w, s1_);                                     \
        } else {                                                                                \
            const int row_ = tid >> 1, h_ = tid & 1;                                            \
            const uint2 nib_ = reinterpret_cast<const uint2*>(SN)[row_ * 2 + h_];               \
            const uint32_t sw_ = SS[row_] >> ((((K0) >> 5) & 1) * 16 + 8 * h_);                 \
            const float sc_ = e4m3_value(sw_ & 0xffu);                                          \
            SB[lds_slot32(row_, 2 * h_)] = dequant8(nib_.x, sc_);                               \
            SB[lds_slot32(row_, 2 * h_ + 1)] = dequant8(nib_.y, sc_);                           \
        }                                                                                       \
    } while (0)
#define MOE_READ(SA, SB, AF, BF)                                                                \
    do {                                                                                        \
        const int ch_ = lane >> 4;                                                              \
        _Pragma("unroll") for (int ni = 0; ni < NB; ++ni) BF[ni] =                              \
            __builtin_bit_cast(bf16x8_t, SB[lds_slot32(gb[ni] * 16 + (lane & 15), ch_)]);        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) AF[mi] =                               \
            __builtin_bit_cast(bf16x8_t, SA[lds_slot32((mi * 2 + wr) * 16 + (lane & 15), ch_)]); \
    } while (0)
#define MOE_MFMA(AF, BF)                                                                        \
    do {                                                                                        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) {                                      \
            if (mi * 2 + wr < nsub) {                                                           \
                _Pragma("unroll") for (int ni = 0; ni < NB; ++ni) acc[mi][ni] =                 \
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[mi], BF[ni], acc[mi][ni], 0, 0, 0); \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    f32x4_t acc[8][NB];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < NB; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t a0[8], b0[NB], a1[8], b1[NB];

    const int nk = K / BKS;
    const int last = (nk - 1) * BKS;
    // prologue: raw stages 0 and 1, activation stage 0; decode both; then activation stages
    // 1..3 and raw stages 2..4 in the steady-state issue order
    MOE_ISSUE_W(sN0, sS0, 0);
    MOE_ISSUE_W(sN1, sS1, min(1 * BKS, last));
    MOE_ISSUE_A(sA0, 0);
    wait_vm_lgkm0<0>();
    block_barrier();
    MOE_DECODE(sN0, sS0, sB0, 0);
    MOE_DECODE(sN1, sS1, sB1, min(1 * BKS, last));
    wait_vm_lgkm0<0>();
    block_barrier();
    MOE_READ(sA0, sB0, a0, b0);
    MOE_ISSUE_A(sA1, min(1 * BKS, last));
    MOE_ISSUE_W(sN2, sS2, min(2 * BKS, last));
    MOE_ISSUE_A(sA2, min(2 * BKS, last));
    MOE_ISSUE_W(sN3, sS3, min(3 * BKS, last));
    MOE_ISSUE_A(sA3, min(3 * BKS, last));
    MOE_ISSUE_W(sN0, sS0, min(4 * BKS, last));
    for (int s = 0;; s += 4) {
#define MOE_IT(S, FA, FB, GA, GB, SAr, SBr, SAw, SNw, SSw, SNd, SSd, SBd)      \
        wait_vm_lgkm0<2 * OPS>();                                            \
        block_barrier();                                                     \
        MOE_READ(SAr, SBr, GA, GB);                                          \
        MOE_ISSUE_A(SAw, min((s + S + 4) * BKS, last));                      \
        MOE_ISSUE_W(SNw, SSw, min((s + S + 5) * BKS, last));                 \
        MOE_MFMA(FA, FB);                                                    \
        if (s + S + 1 >= nk) break;                                          \
        MOE_DECODE(SNd, SSd, SBd, min((s + S + 2) * BKS, last));
        MOE_IT(0, a0, b0, a1, b1, sA1, sB1, sA0, sN1, sS1, sN2, sS2, sB0)
        MOE_IT(1, a1, b1, a0, b0, sA2, sB0, sA1, sN2, sS2, sN3, sS3, sB1)
        MOE_IT(2, a0, b0, a1, b1, sA3, sB1, sA2, sN3, sS3, sN0, sS0, sB0)
        MOE_IT(3, a1, b1, a0, b0, sA0, sB0, sA3, sN0, sS0, sN1, sS1, sB1)
#undef MOE_IT
    }
    wait_vm_lgkm0<0>();
#undef MOE_ISSUE_A
#undef MOE_ISSUE_W
#undef MOE_DECODE
#undef MOE_READ
#undef MOE_MFMA

    const float gs = g.gscale ? g.gscale[e] : 1.0f;
    // Epilogue through LDS, as in the bf16 kernel, in two rounds of 64 tile rows (the ring's
    // activation arrays hold a 64-row slice of every wavefront's output: W columns of bf16,
    // at most 16 KiB): write the slice in the MFMA layout, read it back as 16-byte row chunks.
    block_barrier();
    constexpr int W = (KIND == kGateUp ? NB / 2 : NB) * 16;  // columns per wavefront
    constexpr int SM = W / 8 - 1;
    static_assert(64 * W * 2 * (NW / 4) <= 16384, "a 64-row slice per wavefront fits its array");
    uint16_t* const stg = reinterpret_cast<uint16_t*>(
        (wave & 3) == 0 ? sA0 : (wave & 3) == 1 ? sA1 : (wave & 3) == 2 ? sA2 : sA3) + (wave >> 2) * 64 * W;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            const int mi = 4 * half + m4;
            if (mi * 2 + wr >= nsub) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lr = m4 * 16 + 4 * (lane >> 4) + i;
#pragma unroll
                for (int ni = 0; ni < W / 16; ++ni) {
                    const int lc = ni * 16 + (lane & 15);
                    const float v = (KIND == kGateUp) ? silu_mul(acc[mi][ni][i] * gs, acc[mi][ni + NB / 2][i] * gs)
                                                      : acc[mi][ni][i] * gs;
                    stg[lr * W + ((((lc >> 3) ^ (lr >> 2)) & SM) << 3) + (lc & 7)] = (uint16_t)bf16_rne(v);
                }
            }
        }
        asm volatile("" ::: "memory");  // reads of another type after the writes (one wavefront: in order)
#pragma unroll
        for (int it = 0; it < W / 8; ++it) {
            const int q = it * 64 + lane, lr = q / (W / 8), c8 = q % (W / 8);
            const int mi = 4 * half + (lr >> 4);
            const int row = r0 + (mi * 2 + wr) * 16 + (lr & 15);
            if (mi * 2 + wr >= nsub || row >= r1) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(&stg[lr * W + (((c8 ^ (lr >> 2)) & SM) << 3)]);
            const int col = gcol + c8 * 8;
            if (KIND == kGateUp)
                *reinterpret_cast<uint4*>(&out[size_t(row) * g.F + col]) = v;
            else if (col < g.N)
                *reinterpret_cast<uint4*>(&out[size_t(row) * g.N + col]) = v;
        }
        asm volatile("" ::: "memory");  // the next round's writes after these reads
    }
}

// ---------------------------------------------------------------------------------------
// Decode kernel: few rows per expert, so the layer streams the selected experts' weights once
// from HBM ("Hosting Qwen on Blackwell", section Decoders: decode matmuls are bound by weight
// loads).  One wavefront owns 16 weight rows (gate/up: 16 gate rows and the 16 matching up
// rows) and up to 16 dispatched rows of one expert; weights go from global memory straight
// into MFMA operand registers (no LDS), two 128-wide K blocks in flight per lane.
//
// bf16 weights come packed: MFMA i of K block j is stage 4 j + i, and lane (row n, k-group q)
// reads logical chunk q of its row in that stage (16 rows x 64 bytes of a stage are one
// contiguous KiB).  NVFP4 weights are row-major; there the reduction index is permuted inside
// each 128-wide block so that one lane's 32 nibbles are contiguous: MFMA i takes, in k-group
// q, elements 128 j + 32 q + 8 i .. +7 of both operands (a common permutation of K leaves the
// dot products unchanged).
//
// SPLITK wavefronts of a block share 16 columns and split K; their partial sums meet in LDS
// and are added in a fixed order (deterministic).
// ---------------------------------------------------------------------------------------

template <int KIND, int WFMT, int SPLITK, bool WIN4 = false>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g) {
    constexpr int CG = 4 / SPLITK;              // column groups per block
    constexpr int NB = (KIND == kGateUp) ? 2 : 1;  // weight row sets per column group
    __shared__ f32x4_t red[4][NB][64];

    const int ncg = (KIND == kGateUp) ? g.F / 16 : (g.N + 15) / 16;
    const int per_tile = (ncg + CG - 1) / CG;
    const int item = blockIdx.x;
    if (item >= *g.tile_count * per_tile) return;
    const Tile tile = g.tiles[item / per_tile];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cg = (item % per_tile) * CG + wave / SPLITK;
    const int kp = wave % SPLITK;
    const bool live = cg < ncg;                 // uniform per wavefront
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;
    const int n = lane & 15, q = lane >> 4;

    // this lane's activation row and weight rows
    const int rr = min(r0 + n, r1 - 1);
    int src = g.a_rows ? g.a_rows[rr] : rr;
    src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
    const uint16_t* pa = static_cast<const uint16_t*>(g.a) + size_t(src) * K + (WFMT == kWBF16 ? 8 : WIN4 ? 128 : 32) * q;
    const int col = min(cg, ncg - 1) * 16 + n;
    int wrow0, wrow1 = 0;
    if (KIND == kGateUp) {
        wrow0 = col;
        wrow1 = g.F + col;
    } else {
        wrow0 = min(col, g.N - 1);
    }

    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const int nblk = K / 128 / SPLITK;
    const int j0 = kp * nblk, jend = j0 + nblk;

    // One 128-wide K block of operands, in named registers.  Two blocks are kept in flight:
    // the loads of block j+1 are outstanding while the MFMAs of block j run.
    struct Blk {
        uint4 a0, a1, a2, a3;      // activations, MFMA i = 0..3
        uint4 g0, g1, g2, g3;      // bf16 weight rows (gate / down)
        uint4 u0, u1, u2, u3;      // bf16 up rows
        uint4 pg, pu;              // NVFP4 packed nibbles (gate / down, up)
        uint32_t sg, su;           // NVFP4 scale pairs
    };
    auto ld16 = [](const void* p) __attribute__((always_inline)) { return *reinterpret_cast<const uint4*>(p); };
    // bf16 (packed): lane's 16 bytes of stage st of its gate/down row and of its up row
    const uint16_t* pw0 = nullptr;
    const uint16_t* pw1 = nullptr;
    if constexpr (WFMT == kWBF16) {
        const int nst = K / 32;
        int t, r_a;
        if (KIND == kGateUp) {
            t = col >> 7;
            r_a = ((col >> 6) & 1) * 128 + (col & 63);  // gate tile row; the up row is 64 below
        } else {
            t = wrow0 >> 8;
            r_a = wrow0 & 255;
        }
        const int ntiles = (KIND == kGateUp) ? g.F / 128 : g.N / 256;
        const uint16_t* blk = static_cast<const uint16_t*>(g.w) + (size_t(e) * ntiles + t) * size_t(nst) * 8192;
        pw0 = blk + r_a * 32 + (q ^ ((r_a >> 1) & 3)) * 8;
        if (KIND == kGateUp) {
            const int r_u = r_a + 64;
            pw1 = blk + r_u * 32 + (q ^ ((r_u >> 1) & 3)) * 8;
        }
    }
    const size_t w0 = size_t(e) * Nw + wrow0, w1 = size_t(e) * Nw + wrow1;
    const uint8_t* pq0 = static_cast<const uint8_t*>(g.w) + w0 * (K / 2) + (WIN4 ? 64 : 16) * q;
    const uint8_t* pq1 = static_cast<const uint8_t*>(g.w) + w1 * (K / 2) + (WIN4 ? 64 : 16) * q;
    const uint8_t* ps0 = g.wscale + w0 * (K / 16) + (WIN4 ? 8 : 2) * q;
    const uint8_t* ps1 = g.wscale + w1 * (K / 16) + (WIN4 ? 8 : 2) * q;
    auto load = [&](Blk& b, int j) __attribute__((always_inline)) {
        const int k = 128 * j;
        if constexpr (WFMT == kWBF16) {
            b.a0 = ld16(pa + k);
            b.a1 = ld16(pa + k + 32);
            b.a2 = ld16(pa + k + 64);
            b.a3 = ld16(pa + k + 96);
            const size_t so = size_t(4 * j) * 8192;  // stage 4 j
            b.g0 = ld16(pw0 + so);
            b.g1 = ld16(pw0 + so + 8192);
            b.g2 = ld16(pw0 + so + 16384);
            b.g3 = ld16(pw0 + so + 24576);
            if constexpr (KIND == kGateUp) {
                b.u0 = ld16(pw1 + so);
                b.u1 = ld16(pw1 + so + 8192);
                b.u2 = ld16(pw1 + so + 16384);
                b.u3 = ld16(pw1 + so + 24576);
            }
        } else {
            b.a0 = ld16(pa + k);
            b.a1 = ld16(pa + k + 8);
            b.a2 = ld16(pa + k + 16);
            b.a3 = ld16(pa + k + 24);
            b.pg = ld16(pq0 + 64 * j);
            b.sg = *reinterpret_cast<const uint16_t*>(ps0 + 8 * j);
            if constexpr (KIND == kGateUp) {
                b.pu = ld16(pq1 + 64 * j);
                b.su = *reinterpret_cast<const uint16_t*>(ps1 + 8 * j);
            }
        }
    };
    auto mma = [&](f32x4_t& acc, const uint4& x, const uint4& w) __attribute__((always_inline)) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), __builtin_bit_cast(bf16x8_t, w), acc, 0, 0, 0);
    };
    auto compute = [&](const Blk& b) __attribute__((always_inline)) {
        if constexpr (WFMT == kWBF16) {
            mma(acc0, b.a0, b.g0);
            mma(acc0, b.a1, b.g1);
            mma(acc0, b.a2, b.g2);
            mma(acc0, b.a3, b.g3);
            if constexpr (KIND == kGateUp) {
                mma(acc1, b.a0, b.u0);
                mma(acc1, b.a1, b.u1);
                mma(acc1, b.a2, b.u2);
                mma(acc1, b.a3, b.u3);
            }
        } else {
            const float fa = e4m3_value(b.sg & 0xffu), fb = e4m3_value(b.sg >> 8);
            mma(acc0, b.a0, dequant8(b.pg.x, fa));
            mma(acc0, b.a1, dequant8(b.pg.y, fa));
            mma(acc0, b.a2, dequant8(b.pg.z, fb));
            mma(acc0, b.a3, dequant8(b.pg.w, fb));
            if constexpr (KIND == kGateUp) {
                const float ua = e4m3_value(b.su & 0xffu), ub = e4m3_value(b.su >> 8);
                mma(acc1, b.a0, dequant8(b.pu.x, ua));
                mma(acc1, b.a1, dequant8(b.pu.y, ua));
                mma(acc1, b.a2, dequant8(b.pu.z, ub));
                mma(acc1, b.a3, dequant8(b.pu.w, ub));
            }
        }
    };
    if constexpr (WFMT == kWNVFP4 && WIN4) {
        // NVFP4, 512-wide windows (nblk % 4 == 0): inside window w lane q owns the 128
        // contiguous elements 512 w + 128 q .. +127, so its 8 block scales are 8 contiguous
        // bytes (one 8-byte load per window and row instead of one 2-byte load per block);
        // 128-wide block jj of the window is that range's jj-th 32 elements, MFMA i of the
        // block its elements 32 jj + 8 i .. +7 (the same permutation of K on both operands).
        struct QBlk {
            uint4 a0, a1, a2, a3, pg, pu;
        };
        auto qload = [&](QBlk& b, int j) __attribute__((always_inline)) {
            const int w = j >> 2, jj = j & 3;
            const uint16_t* xa = pa + 512 * w + 32 * jj;
            b.a0 = ld16(xa);
            b.a1 = ld16(xa + 8);
            b.a2 = ld16(xa + 16);
            b.a3 = ld16(xa + 24);
            b.pg = ld16(pq0 + 256 * w + 16 * jj);
            if constexpr (KIND == kGateUp) b.pu = ld16(pq1 + 256 * w + 16 * jj);
        };
        auto sload = [&](uint2& sg, uint2& su, int w) __attribute__((always_inline)) {
            sg = *reinterpret_cast<const uint2*>(ps0 + 32 * w);
            if constexpr (KIND == kGateUp) su = *reinterpret_cast<const uint2*>(ps1 + 32 * w);
        };
        auto qmma = [&](f32x4_t& acc, const QBlk& b, const uint4& p, uint2 sc, int jj) __attribute__((always_inline)) {
            const uint32_t word = (jj < 2) ? sc.x : sc.y;
            const int sh = (jj & 1) * 16;
            const float fa = e4m3_value((word >> sh) & 0xffu), fb = e4m3_value((word >> (sh + 8)) & 0xffu);
            mma(acc, b.a0, dequant8(p.x, fa));
            mma(acc, b.a1, dequant8(p.y, fa));
            mma(acc, b.a2, dequant8(p.z, fb));
            mma(acc, b.a3, dequant8(p.w, fb));
        };
        auto qcompute = [&](const QBlk& b, uint2 sg, uint2 su, int jj) __attribute__((always_inline)) {
            qmma(acc0, b, b.pg, sg, jj);
            if constexpr (KIND == kGateUp) qmma(acc1, b, b.pu, su, jj);
        };
        if (live && nblk > 0) {
            const int wlast = (jend >> 2) - 1;
            QBlk x0{}, x1{};
            uint2 sg0{}, su0{}, sg1{}, su1{};
            sload(sg0, su0, j0 >> 2);
            qload(x0, j0);
            qload(x1, j0 + 1);
            for (int j = j0; j < jend; j += 4) {  // loads past the end re-read the last block
                qcompute(x0, sg0, su0, 0);
                qload(x0, min(j + 2, jend - 1));
                qcompute(x1, sg0, su0, 1);
                qload(x1, min(j + 3, jend - 1));
                sload(sg1, su1, min((j >> 2) + 1, wlast));
                qcompute(x0, sg0, su0, 2);
                qload(x0, min(j + 4, jend - 1));
                qcompute(x1, sg0, su0, 3);
                qload(x1, min(j + 5, jend - 1));
                sg0 = sg1;
                su0 = su1;
            }
        }
    } else if (live && nblk > 0) {
        Blk x0{}, x1{};
        load(x0, j0);
        load(x1, min(j0 + 1, jend - 1));  // past the end: a harmless re-read of the last block
        for (int j = j0;; j += 2) {
            compute(x0);
            if (j + 1 >= jend) break;
            load(x0, min(j + 2, jend - 1));
            compute(x1);
            if (j + 2 >= jend) break;
            load(x1, min(j + 3, jend - 1));
        }
    }

    if constexpr (SPLITK > 1) {
        red[wave][0][lane] = acc0;
        if (KIND == kGateUp) red[wave][NB - 1][lane] = acc1;
        __syncthreads();
        if (kp != 0) return;
        acc0 = red[wave][0][lane];
        if (KIND == kGateUp) acc1 = red[wave][NB - 1][lane];
#pragma unroll
        for (int p = 1; p < SPLITK; ++p) {
            acc0 += red[wave + p][0][lane];
            if (KIND == kGateUp) acc1 += red[wave + p][NB - 1][lane];
        }
    }
    if (!live) return;

    const float gs = (WFMT == kWNVFP4 && g.gscale) ? g.gscale[e] : 1.0f;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + 4 * q + i;
        if (row >= r1) continue;
        if (KIND == kGateUp) {
            out[size_t(row) * g.F + col] = (uint16_t)bf16_rne(silu_mul(acc0[i] * gs, acc1[i] * gs));
        } else if (col < g.N) {
            out[size_t(row) * g.N + col] = (uint16_t)bf16_rne(acc0[i] * gs);
        }
    }
}

// Decode kernel for PACKED NVFP4 weights.  Lane (n, q) of a wavefront owns weight row n of
// each of the wavefront's NCG consecutive 16-row groups (gate/up: the gate rows and the matching
// up rows) and K-group q: in 128-wide K block j it takes stage 4 j + q of those rows (16 bytes
// at 16 r of the stage's 4 KiB block of the tile) and the scale word at 4 r of stage pair
// 2 j + q / 2 (half q & 1).  A row group c lies 16 c rows below the first in the same tile, so
// one base address serves all of them.  The activation fragments of a block are loaded once
// and feed the MFMAs of every group: activation bytes per weight byte fall by NCG, which
// relieves the L1-to-register return path that the 4-bit weights otherwise share with
// activations four times their size.  Two K blocks in flight; SPLITK wavefronts split K and
// meet in LDS in a fixed order.
template <int KIND, int SPLITK, int NCG>
__global__ __launch_bounds__(256) void gemm_decode_nvfp4p_kernel(GemmArgs g) {
    static_assert(NCG == 1 || NCG == 2 || NCG == 4, "row groups must stay inside a 64-row half");
    constexpr int WPB = 4 / SPLITK;                 // group sets per block
    constexpr int NB = (KIND == kGateUp) ? 2 : 1;   // gate and up rows, or down rows
    __shared__ f32x4_t red[SPLITK > 1 ? 4 : 1][NB * NCG][64];

    const int ncg = (KIND == kGateUp) ? g.F / 16 : g.N / 16;  // F % 128 == 0, N % 256 == 0
    const int per_tile = (ncg + WPB * NCG - 1) / (WPB * NCG);
    const int item = blockIdx.x;
    if (item >= *g.tile_count * per_tile) return;
    const Tile tile = g.tiles[item / per_tile];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cgw = ((item % per_tile) * WPB + wave / SPLITK) * NCG;  // first group, NCG-aligned
    const int kp = wave % SPLITK;
    const bool live = cgw < ncg;  // uniform per wavefront; ncg % NCG == 0, so all NCG groups exist
    const int K = g.K, nst = K / 32;
    const int n = lane & 15, q = lane >> 4;

    const int rr = min(r0 + n, r1 - 1);
    int src = g.a_rows ? g.a_rows[rr] : rr;
    src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
    const uint16_t* pa = static_cast<const uint16_t*>(g.a) + size_t(src) * K + 32 * q;
    const int col = min(cgw, ncg - NCG) * 16 + n;  // column of group 0 (clamped for idle waves)
    int t, r_a;
    if (KIND == kGateUp) {
        t = col >> 7;
        r_a = ((col >> 6) & 1) * 128 + (col & 63);  // gate tile row; the up row is 64 below
    } else {
        t = col >> 8;
        r_a = col & 255;
    }
    const size_t tb = size_t(e) * ((KIND == kGateUp) ? g.F / 128 : g.N / 256) + t;
    const uint8_t* pq = static_cast<const uint8_t*>(g.w) + tb * nst * 4096 + (q * 256 + r_a) * 16;
    const uint8_t* ps = g.wscale + tb * (nst / 2) * 1024 + ((q >> 1) * 256 + r_a) * 4;
    const int ssh = (q & 1) * 16;

    f32x4_t acc[NB * NCG];
#pragma unroll
    for (int i = 0; i < NB * NCG; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nblk = K / 128 / SPLITK;
    const int j0 = kp * nblk, jend = j0 + nblk;

    struct Blk {
        uint4 a[4];             // activations, MFMA i = 0..3
        uint4 p[NB * NCG];      // bytes: group c gate (or down) at c, up at NCG + c
        uint32_t sc[NB * NCG];  // scale words shifted to this lane's stage
    };
    auto ld16 = [](const void* p) __attribute__((always_inline)) { return *reinterpret_cast<const uint4*>(p); };
    auto load = [&](Blk& b, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b.a[i] = ld16(pa + 128 * j + 8 * i);
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int c = 0; c < NCG; ++c) {
                b.p[h * NCG + c] = ld16(pq + 16384 * j + h * 1024 + c * 256);
                b.sc[h * NCG + c] = *reinterpret_cast<const uint32_t*>(ps + 2048 * j + h * 256 + c * 64) >> ssh;
            }
    };
    auto mma = [&](f32x4_t& a, const uint4& x, const uint4& w) __attribute__((always_inline)) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), __builtin_bit_cast(bf16x8_t, w), a, 0, 0, 0);
    };
    auto compute = [&](const Blk& b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NB * NCG; ++i) {  // e4m3_value reads only the low 8 bits
            const float fa = e4m3_value(b.sc[i]), fb = e4m3_value(b.sc[i] >> 8);
            mma(acc[i], b.a[0], dequant8(b.p[i].x, fa));
            mma(acc[i], b.a[1], dequant8(b.p[i].y, fa));
            mma(acc[i], b.a[2], dequant8(b.p[i].z, fb));
            mma(acc[i], b.a[3], dequant8(b.p[i].w, fb));
        }
    };
    if (live && nblk > 0) {
        Blk x0, x1;
        load(x0, j0);
        load(x1, min(j0 + 1, jend - 1));  // past the end: a harmless re-read of the last block
        for (int j = j0;; j += 2) {
            compute(x0);
            if (j + 1 >= jend) break;
            load(x0, min(j + 2, jend - 1));
            compute(x1);
            if (j + 2 >= jend) break;
            load(x1, min(j + 3, jend - 1));
        }
    }

    if constexpr (SPLITK > 1) {
#pragma unroll
        for (int i = 0; i < NB * NCG; ++i) red[wave][i][lane] = acc[i];
        __syncthreads();
        if (kp != 0) return;
#pragma unroll
        for (int i = 0; i < NB * NCG; ++i) {
            acc[i] = red[wave][i][lane];
#pragma unroll
            for (int p = 1; p < SPLITK; ++p) acc[i] += red[wave + p][i][lane];
        }
    }
    if (!live) return;

    const float gs = g.gscale ? g.gscale[e] : 1.0f;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + 4 * q + i;
        if (row >= r1) continue;
#pragma unroll
        for (int c = 0; c < NCG; ++c) {
            const int cc = col + 16 * c;
            if (KIND == kGateUp)
                out[size_t(row) * g.F + cc] = (uint16_t)bf16_rne(silu_mul(acc[c][i] * gs, acc[NCG + c][i] * gs));
            else
                out[size_t(row) * g.N + cc] = (uint16_t)bf16_rne(acc[c][i] * gs);
        }
    }
}

// fp32 activations and weights on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): a 64 x 64
// block tile (64 dispatched rows, 64 weight rows), 4 wavefronts (2 x 2) of 32 x 32, K
// in 16-wide stages through a two-slot LDS ring; the next stage's elements are loaded into
// registers while the current stage's MFMAs run.  An MFMA step takes 4 consecutive k: lane l
// supplies row l % 16 of A and column l % 16 of B at k = k0 + l / 16 and receives rows
// 4 (l / 16) + i, column l % 16, of the 16 x 16 result.  LDS rows are padded to 80 floats so
// that the four k rows one fragment read touches start 16 banks apart.  For the gate/up kind a
// wavefront holds 16 gate columns (B columns 16 wn ...) and the 16 matching up columns
// (32 + 16 wn ...), so SwiGLU pairs registers of one lane.
template <int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
    constexpr int TB = 64, TK = 16, LD = TB + 16;
    __shared__ float sA[2][TK][LD];
    __shared__ float sB[2][TK][LD];
    if (int(blockIdx.x) >= *g.tile_count) return;
    const Tile tile = g.tiles[blockIdx.x];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nt = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;
    const float* A = static_cast<const float*>(g.a);
    const float* W = static_cast<const float*>(g.w);
    auto brow = [&](int n) -> int {
        if (KIND == kGateUp) return n < 32 ? nt * 32 + n : g.F + nt * 32 + (n - 32);
        return min(nt * TB + n, g.N - 1);
    };
    // staged element it of this thread: tile row idx / 16, k offset idx % 16 within the stage
    const float* pa[4];
    const float* pb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = tid + it * 256, row = idx / TK, kk = idx % TK;
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[it] = A + size_t(src) * K + kk;
        pb[it] = W + (size_t(e) * Nw + brow(row)) * K + kk;
    }
    int bcol[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
        bcol[ni] = (KIND == kGateUp ? (ni == 0 ? 16 * wn : 32 + 16 * wn) : 32 * wn + 16 * ni) + (lane & 15);
    f32x4_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ra[4], rb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        ra[it] = pa[it][0];
        rb[it] = pb[it][0];
    }
    const int nk = K / TK;
    for (int st = 0; st < nk; ++st) {
        const int buf = st & 1;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + it * 256, row = idx / TK, kk = idx % TK;
            sA[buf][kk][row] = ra[it];
            sB[buf][kk][row] = rb[it];
        }
        // one barrier per stage: slot buf is written again only at stage st + 2, after every
        // thread has passed the barrier of stage st + 1 and so finished reading it
        __syncthreads();
        if (st + 1 < nk) {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                ra[it] = pa[it][(st + 1) * TK];
                rb[it] = pb[it][(st + 1) * TK];
            }
        }
#pragma unroll
        for (int k4 = 0; k4 < TK; k4 += 4) {
            const int kr = k4 + (lane >> 4);
            float af[2], bf[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) af[mi] = sA[buf][kr][wm * 32 + mi * 16 + (lane & 15)];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) bf[ni] = sB[buf][kr][bcol[ni]];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
        }
    }
    float* out = static_cast<float*>(g.out);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + wm * 32 + mi * 16 + 4 * (lane >> 4) + i;
            if (row >= r1) continue;
            if (KIND == kGateUp) {
                out[size_t(row) * g.F + nt * 32 + 16 * wn + (lane & 15)] = silu_mul(acc[mi][0][i], acc[mi][1][i]);
            } else {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int col = nt * TB + 32 * wn + 16 * ni + (lane & 15);
                    if (col < g.N) out[size_t(row) * g.N + col] = acc[mi][ni][i];
                }
            }
        }
}

// ---------------------------------------------------------------------------------------

namespace {
// prefill: 128 x 128 tiles, 2 x 2 wavefronts of 64 x 64; decode: 16 x 64 tiles, 1 x 2
// wavefronts of 16 x 32 (weight streaming, many blocks for few rows).
constexpr int PF_BM = 128, PF_BN = 128, PF_WM = 2, PF_WN = 2;   // NVFP4 prefill
constexpr int DC_BM = 16, DC_BN = 64, DC_WM = 1, DC_WN = 2;
// Decode GEMMs split K over up to 4 wavefronts of a block until the worst-case tile count gives
// this many wavefronts.  Measured on MI355X (forward, one process): 32768 against 4096 makes
// decode T=8 322.7 -> 305.5 us, T=24 641.7 -> 621.0 us, T=64 812.7 -> 792.1 us, and the NVFP4
// decode GEMMs (T=16) 183.5 / 103.9 -> 178.2 / 97.2 us; 16384 gains only at T=8.
constexpr long kDecodeWaves = 32768;
}  // namespace

int gemm_tile_rows(int family, int wfmt, int ffn) {
    if (family == kFamF32) return 64;
    if (family == kFamPrefill) return (wfmt == kWBF16 || ffn % 128 == 0) ? 256 : PF_BM;
    if (wfmt == kWMXFP8 || wfmt == kWMXFP4) return 32;  // the MX decode kernel's 32 x 32 MFMA tiles
    return DC_BM;
}

template <int BM, int BN, int WM, int WN>
static void launch_mfma(const GemmArgs& g, int max_tiles, hipStream_t s) {
    const int ncols = g.kind == kGateUp ? g.F / (BN / 2) : (g.N + BN - 1) / BN;
    dim3 grid(max_tiles, ncols), block(WM * WN * 64);
    if (g.kind == kGateUp)
        hipLaunchKernelGGL((gemm_fallback_kernel<BM, BN, WM, WN, kGateUp, kWNVFP4>), grid, block, 0, s, g);
    else
        hipLaunchKernelGGL((gemm_fallback_kernel<BM, BN, WM, WN, kDown, kWNVFP4>), grid, block, 0, s, g);
}

// Work items of the prefill kernels: (row tile, column tile) pairs, a multiple of 8 blocks so
// that every XCD walks the same number of slots.
static dim3 prefill_grid(const GemmArgs& g, int max_tiles, int bn) {
    const int ncols = g.kind == kGateUp ? g.F / (bn / 2) : (g.N + bn - 1) / bn;
    return dim3(((max_tiles * ncols + 7) / 8) * 8);
}

hipError_t launch_gemm(const GemmArgs& g, int family, int max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    if (g.wfmt == kWMXFP8 || g.wfmt == kWMXFP4) return launch_gemm_mxfp8(g, family, max_tiles, s);  // mx.hip
    const bool up = g.kind == kGateUp;
    if (family == kFamF32) {
        const int ncols = up ? g.F / 32 : (g.N + 63) / 64;
        dim3 grid(max_tiles, ncols), block(256);
        if (up)
            hipLaunchKernelGGL((gemm_f32_kernel<kGateUp>), grid, block, 0, s, g);
        else
            hipLaunchKernelGGL((gemm_f32_kernel<kDown>), grid, block, 0, s, g);
    } else if (family == kFamPrefill && g.wfmt == kWBF16) {  // packed weights: F % 128 == 0, H % 256 == 0
        const dim3 grid = prefill_grid(g, max_tiles, 256);
        if (up)
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kGateUp>), grid, dim3(512), 0, s, g);
        else
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kDown>), grid, dim3(512), 0, s, g);
    } else if (family == kFamPrefill && g.F % 128 == 0) {
        const dim3 grid = prefill_grid(g, max_tiles, 256);
        // packed weights: 8 wavefronts for both kinds (gate/up 2.97 -> 2.69 ms against 4 on
        // the NVFP4 prefill shape); row-major: 4 for gate/up, where 4 measured faster
        if (up && g.wpacked)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kGateUp, 8, true>), grid, dim3(512), 0, s, g);
        else if (up)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kGateUp, 4, false>), grid, dim3(256), 0, s, g);
        else if (g.wpacked)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kDown, 8, true>), grid, dim3(512), 0, s, g);
        else
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kDown, 8, false>), grid, dim3(512), 0, s, g);
    } else if (family == kFamPrefill) {
        if (g.wpacked) return hipErrorInvalidValue;  // PACKED NVFP4 needs F % 128 == 0
        launch_mfma<PF_BM, PF_BN, PF_WM, PF_WN>(g, max_tiles, s);
    } else if (g.wpacked) {  // PACKED NVFP4 decode: NCG row groups per wavefront
        // measured on the NVFP4 decode shape (T=16, H4096, F2048): the down GEMM (activations
        // four times the weight bytes at NCG = 1) is 20 % faster with NCG = 2 than with 1 and
        // faster than with 4; gate/up (activations twice the weight bytes) is fastest with 1
        constexpr int NCG_UP = 1, NCG_DOWN = 2;
        const int ncg = up ? g.F / 16 / NCG_UP : g.N / 16 / NCG_DOWN;  // wavefront group sets
        int split = 1;
        while (split < 4 && long(max_tiles) * ncg * split < kDecodeWaves && g.K % (128 * split * 2) == 0) split *= 2;
        const int wpb = 4 / split;
        dim3 grid(max_tiles * ((ncg + wpb - 1) / wpb)), block(256);
#define MOE_DECP(KD, SK, NC) hipLaunchKernelGGL((gemm_decode_nvfp4p_kernel<KD, SK, NC>), grid, block, 0, s, g)
        if (up) { if (split == 1) MOE_DECP(kGateUp, 1, NCG_UP); else if (split == 2) MOE_DECP(kGateUp, 2, NCG_UP); else MOE_DECP(kGateUp, 4, NCG_UP); }
        else    { if (split == 1) MOE_DECP(kDown, 1, NCG_DOWN);   else if (split == 2) MOE_DECP(kDown, 2, NCG_DOWN);   else MOE_DECP(kDown, 4, NCG_DOWN); }
#undef MOE_DECP
    } else if (g.K % 128 == 0) {
        // split K until the worst-case tile count gives kDecodeWaves wavefronts
        const int ncg = up ? g.F / 16 : (g.N + 15) / 16;
        int split = 1;
        while (split < 4 && long(max_tiles) * ncg * split < kDecodeWaves && g.K % (128 * split * 2) == 0) split *= 2;
        const int cgb = 4 / split;
        dim3 grid(max_tiles * ((ncg + cgb - 1) / cgb)), block(256);
#define MOE_DEC(KD, WF, SK) hipLaunchKernelGGL((gemm_decode_kernel<KD, WF, SK>), grid, block, 0, s, g)
        if (g.wfmt == kWBF16) {
            if (up) { if (split == 1) MOE_DEC(kGateUp, kWBF16, 1); else if (split == 2) MOE_DEC(kGateUp, kWBF16, 2); else MOE_DEC(kGateUp, kWBF16, 4); }
            else    { if (split == 1) MOE_DEC(kDown, kWBF16, 1);   else if (split == 2) MOE_DEC(kDown, kWBF16, 2);   else MOE_DEC(kDown, kWBF16, 4); }
        } else if ((g.K / 128 / split) % 4 == 0) {  // 512-wide scale windows
#define MOE_DEC4(KD, SK) hipLaunchKernelGGL((gemm_decode_kernel<KD, kWNVFP4, SK, true>), grid, block, 0, s, g)
            if (up) { if (split == 1) MOE_DEC4(kGateUp, 1); else if (split == 2) MOE_DEC4(kGateUp, 2); else MOE_DEC4(kGateUp, 4); }
            else    { if (split == 1) MOE_DEC4(kDown, 1);   else if (split == 2) MOE_DEC4(kDown, 2);   else MOE_DEC4(kDown, 4); }
#undef MOE_DEC4
        } else {
            if (up) { if (split == 1) MOE_DEC(kGateUp, kWNVFP4, 1); else if (split == 2) MOE_DEC(kGateUp, kWNVFP4, 2); else MOE_DEC(kGateUp, kWNVFP4, 4); }
            else    { if (split == 1) MOE_DEC(kDown, kWNVFP4, 1);   else if (split == 2) MOE_DEC(kDown, kWNVFP4, 2);   else MOE_DEC(kDown, kWNVFP4, 4); }
        }
#undef MOE_DEC
    } else {  // NVFP4 with K % 128 != 0
        if (g.wpacked) return hipErrorInvalidValue;  // PACKED NVFP4 needs H % 256, F % 128 == 0
        launch_mfma<DC_BM, DC_BN, DC_WM, DC_WN>(g, max_tiles, s);
    }
    return hipGetLastError();
}

}  // namespace moe
