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
#include "gemv.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

namespace {

constexpr int BK = 64;  // K elements per LDS stage (8 chunks of 16 bytes in bf16)

__device__ __forceinline__ int lds_slot(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

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
// stage are read from LDS into registers while the MFMAs of the current stage run: the weight
// fragments first, each row group's activation fragment right after that group's MFMAs, into
// the same registers (one activation set, 32 registers fewer; bf16 prefill gate/up 1.073 ->
// 1.064 ms, forward 1.685 -> 1.670 ms, one process, bit-identical).  The stage's four loads
// are issued between the MFMA groups (after groups 1, 3, 5 and 7) rather than before them
// (gate/up 1.066 -> 1.053 ms, down 0.550 -> 0.541 ms, one process, bit-identical).  Rows are 64
// bytes in LDS; the 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 3), which keeps the
// fragment reads (8 consecutive rows, one chunk) on distinct banks.  Activation rows are
// gathered through the dispatch map; weights come in the packed layout, where every stage of a
// 256-row tile is already this LDS image (one contiguous 16 KiB read), or row-major, where each
// lane fetches the chunk of its weight row that belongs in its slot (64 bytes per row and stage,
// like the activations; the same LDS image, so bit-identical results).  The 16 groups of 16
// rows alternate between the two wavefront rows and groups past the tile's last row skip their
// MFMAs.  For gate/up, wavefront column c holds weight row groups {0, 1, 4, 5} + 8 (c >> 1) +
// 2 (c & 1) of the tile's 16: 32 gate rows and the 32 up rows of the same hid columns.
// ---------------------------------------------------------------------------------------


template <int KIND, bool A32>
__global__ __launch_bounds__(512, 1) void gemm_prefill_bf16_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BKS = 32;
    constexpr int HALF = (KIND == kGateUp) ? BN / 2 : BN;
    __shared__ uint4 sA0[BM * 4], sA1[BM * 4], sA2[BM * 4], sA3[BM * 4];
    __shared__ uint4 sB0[BN * 4], sB1[BN * 4], sB2[BN * 4], sB3[BN * 4];

    const int ncols = (KIND == kGateUp) ? g.F / HALF : (g.N + BN - 1) / BN;
    // XCD x (blocks b with b % 8 == x) takes the items of row tiles tile_count[8 + x] ..
    // tile_count[9 + x], ranges the dispatch cut by cost (bf16 prefill gate/up 1.053-1.059 ->
    // 1.041-1.052 ms, down 0.542-0.545 -> 0.532-0.539 ms against equal item counts per XCD)
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int item = g.tile_count[8 + xcd] * ncols + j;
    if (item >= g.tile_count[9 + xcd] * ncols) return;
    int nt;
    const int tix = grouped_item(g.tiles, *g.tile_count, item, ncols, &nt);
    const Tile tile = g.tiles[tix];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nsub = (r1 - r0 + 15) / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
    const int wr = wave >> 2, wc = wave & 3;                      // 2 x 4 wavefronts
    // row groups mi * 2 + wr < nsub of this wavefront hold rows: mi < na (a scalar count, so
    // that each group's MFMAs sit behind one scalar compare and branch)
    const int na = __builtin_amdgcn_readfirstlane((nsub - wr + 1) >> 1);
    const int K = g.K;

    const char* pa[2];
    uint32_t va[2];  // the same as offsets from a_s (scalar-base loads: A32 or the packed hid)
    // A operand: gathered rows (64 bytes per row and stage), or for the down GEMM of a forward
    // the packed hid image of this row tile (one contiguous 16 KiB per stage, like the weights)
    const bool apk = KIND == kDown && g.hid_packed;
    const int astep = apk ? 512 : 2;  // bytes per K element along the A stream
    const char* const a_s = static_cast<const char*>(g.a) +
                            (apk ? size_t(tix) * size_t(K / BKS) * 16384 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (apk) {
            va[i] = (i * 8 + wave) * 1024 + lane * 16;
            pa[i] = a_s + va[i];
            continue;
        }
        const int row = (i * 8 + wave) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[i] = a_s + (size_t(src) * K + ch * 8) * 2;
        va[i] = static_cast<uint32_t>((size_t(src) * K + ch * 8) * 2);
    }
    const bool a_scalar = apk || A32;
    // B operand: packed weights (each stage of the 256-row tile is one contiguous 16 KiB, the LDS
    // image), or row-major weights read like the gathered activations (64 bytes per weight row
    // and stage, the lane's chunk taken from the slot it lands in)
    const char* pb[2];
    size_t wst;  // bytes from one 32-element stage of the lane's chunk to the next
    const char* const wblk = static_cast<const char*>(g.w) + (size_t(e) * ncols + nt) * size_t(K / BKS) * 16384;
    const uint32_t vb = wave * 1024 + lane * 16;  // packed: the lane's place in a stage block (+ 8 KiB i)
    if (g.wpacked) {
#pragma unroll
        for (int i = 0; i < 2; ++i) pb[i] = wblk + (i * 8 + wave) * 1024 + lane * 16;
        wst = 16384;
    } else {
        const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = (i * 8 + wave) * 16 + (lane >> 2);
            const int ch = (lane & 3) ^ ((row >> 1) & 3);
            int wrow;
            if (KIND == kGateUp) {
                const int q = row & 127, f = nt * HALF + 64 * (row >> 7) + (q & 63);
                wrow = q < 64 ? f : g.F + f;
            } else {
                wrow = min(nt * BN + row, g.N - 1);
            }
            pb[i] = static_cast<const char*>(g.w) + ((size_t(e) * Nw + wrow) * K + ch * 8) * 2;
        }
        wst = 64;
    }
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
        if (a_scalar) {                                                                         \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
                dma16s(a_s + size_t(k0_) * astep, va[i], &SA[(i * 8 + wave) * 64]);             \
        } else {                                                                                \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
                dma16(pa[i] + k0_ * astep, &SA[(i * 8 + wave) * 64]);                           \
        }                                                                                       \
        if (g.wpacked) {                                                                        \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
                dma16s(wblk + size_t(k0_ / BKS) * 16384, vb + i * 8192, &SB[(i * 8 + wave) * 64]); \
        } else {                                                                                \
            _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
                dma16(pb[i] + (k0_ / BKS) * wst, &SB[(i * 8 + wave) * 64]);                     \
        }                                                                                       \
    } while (0)
    // chunk I of a stage's loads: activation rows (i * 8 + wave) * 16.. and weight rows alike
#define MOE_ISSUE8_A(SA, K0, I)                                                                 \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        if (a_scalar) dma16s(a_s + size_t(k0_) * astep, va[I], &SA[((I) * 8 + wave) * 64]);     \
        else dma16(pa[I] + k0_ * astep, &SA[((I) * 8 + wave) * 64]);                             \
    } while (0)
#define MOE_ISSUE8_W(SB, K0, I)                                                                 \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        if (g.wpacked) dma16s(wblk + size_t(k0_ / BKS) * 16384, vb + (I) * 8192, &SB[((I) * 8 + wave) * 64]); \
        else dma16(pb[I] + (k0_ / BKS) * wst, &SB[((I) * 8 + wave) * 64]);                       \
    } while (0)
#define MOE_READ8(SA, SB, AF, BF)                                                               \
    do {                                                                                        \
        const int ch_ = lane >> 4;                                                              \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) BF[ni] =                               \
            __builtin_bit_cast(bf16x8_t, SB[lds_slot32(gb[ni] * 16 + (lane & 15), ch_)]);        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) AF[mi] =                               \
            __builtin_bit_cast(bf16x8_t, SA[lds_slot32((mi * 2 + wr) * 16 + (lane & 15), ch_)]); \
    } while (0)
#define MOE_READB8(SB, BF)                                                                      \
    do {                                                                                        \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) BF[ni] =                               \
            __builtin_bit_cast(bf16x8_t, SB[lds_slot32(gb[ni] * 16 + (lane & 15), lane >> 4)]);  \
    } while (0)
    // the MFMAs of one stage; row group mi's activation fragment of the next stage (ring slot
    // SAN) is read into AF[mi] right after the group's MFMAs, under the same row test
#define MOE_MFMA8(AF, BF, SAN, SAW, SBW, KW)                                                     \
    do {                                                                                        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) {                                      \
            if (__builtin_expect(mi < na_, 1)) {                                                \
                _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) acc[mi][ni] =                  \
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[mi], BF[ni], acc[mi][ni], 0, 0, 0); \
                AF[mi] = __builtin_bit_cast(bf16x8_t, SAN[lds_slot32((mi * 2 + wr) * 16 + (lane & 15), lane >> 4)]); \
            }                                                                                   \
            if (mi == 1) MOE_ISSUE8_A(SAW, KW, 0);                                              \
            if (mi == 3) MOE_ISSUE8_A(SAW, KW, 1);                                              \
            if (mi == 5) MOE_ISSUE8_W(SBW, KW, 0);                                              \
            if (mi == 7) MOE_ISSUE8_W(SBW, KW, 1);                                              \
        }                                                                                       \
    } while (0)

    f32x4_t acc[8][4];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t af[8], b0[4], b1[4];
    int na_;  // na, re-read each stage so that the group tests stay scalar compares

    const int nk = K / BKS;
    const int last = (nk - 1) * BKS;
    MOE_ISSUE8(sA0, sB0, 0);
    MOE_ISSUE8(sA1, sB1, min(1 * BKS, last));
    MOE_ISSUE8(sA2, sB2, min(2 * BKS, last));
    wait_vm_lgkm0<8>();
    block_barrier();
    MOE_READ8(sA0, sB0, af, b0);
    MOE_ISSUE8(sA3, sB3, min(3 * BKS, last));
    for (int s = 0;; s += 4) {
        wait_vm_lgkm0<8>();
        block_barrier();
        na_ = na;
        asm volatile("" : "+s"(na_));
        MOE_READB8(sB1, b1);
        MOE_MFMA8(af, b0, sA1, sA0, sB0, min((s + 4) * BKS, last));
        if (s + 1 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        na_ = na;
        asm volatile("" : "+s"(na_));
        MOE_READB8(sB2, b0);
        MOE_MFMA8(af, b1, sA2, sA1, sB1, min((s + 5) * BKS, last));
        if (s + 2 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        na_ = na;
        asm volatile("" : "+s"(na_));
        MOE_READB8(sB3, b1);
        MOE_MFMA8(af, b0, sA3, sA2, sB2, min((s + 6) * BKS, last));
        if (s + 3 >= nk) break;
        wait_vm_lgkm0<8>();
        block_barrier();
        na_ = na;
        asm volatile("" : "+s"(na_));
        MOE_READB8(sB0, b0);
        MOE_MFMA8(af, b1, sA0, sA3, sB3, min((s + 7) * BKS, last));
        if (s + 4 >= nk) break;
    }
    wait_vm_lgkm0<0>();
#undef MOE_ISSUE8
#undef MOE_ISSUE8_A
#undef MOE_ISSUE8_W
#undef MOE_READ8
#undef MOE_READB8
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
                const size_t blk = size_t(tix) * (g.F / BKS) + (col >> 5);
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
// both kinds with packed weights, 4 for gate/up with row-major ones); the weights are DMA'd raw (16 nibble bytes and one 4-byte
// scale word per weight row and stage, straight from the row-major NVFP4 arrays) and decoded
// by the block into a bf16 LDS slot (e2m1 * e4m3 is exact in bf16) after the MFMAs of the
// current stage are issued, so the decode overlaps the matrix core.  The per-expert fp32 scale
// multiplies the accumulators.
//
// Iteration i: activation stage i+1 and raw weight stage i+2 have landed (issued three
// iterations earlier); read the raw words of stage i+2 this thread decodes (raw slot
// (i+2)%4) and the weight fragments of stage i+1 (bf16 slot (i+1)%2); DMA activation stage
// i+4 (slot i%4) and raw weight stage i+5 (raw slot (i+1)%4); run the MFMAs of stage i with
// the decode of raw stage i+2 into bf16 slot i%2 interleaved (NW = 8: one output word after
// each 16-row group's MFMAs, so that the VALU work runs beside the matrix core instead of
// after it; measured: NVFP4 prefill gate/up 2.79 -> 2.67 ms, down 1.40 -> 1.38 ms, forward
// 4.52 -> 4.35 ms, bit-identical).  Each row group's activation fragment of stage i+1 (ring
// slot (i+1)%4) is read right after that group's MFMAs of stage i, into the same registers
// and under the same row test: groups past the tile's last row cost no LDS reads, and one
// fragment set instead of two frees 24 registers (measured, one process: gate/up 2.45 ->
// 2.39 ms with the real routing, 1.25 -> 1.07 ms with 32 rows per expert; down 1.226 ->
// 1.216 ms; bit-identical).  Every wavefront issues the same number of DMA instructions
// per iteration (NW = 4: four activation, one nibble, one scale; NW = 8: two activation and
// one nibble or scale), so "landed" is a fixed load count; the barrier at the top of the
// iteration also publishes each raw row to the thread that decodes it.
// ---------------------------------------------------------------------------------------

template <int KIND, int NW, bool PK, bool A32>
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
    // Work order: blocks b, b + 8, ... run on XCD b % 8, and XCD x takes the row tiles
    // tile_count[8 + x] .. tile_count[9 + x] of the list, ranges that the dispatch cut by cost
    // (a fixed part per tile plus its rows), tile-major, so that the blocks of one row tile
    // share its activations, and an expert's consecutive row tiles its weight panels, in that
    // XCD's L2.  Equal numbers of items per XCD left some XCDs with more of the costly full
    // tiles of the hot experts (NVFP4 prefill gate/up 2.41-2.44 ms; pairs of row tiles dealt
    // to the XCDs in turn 2.36-2.38 ms in the same process).  The cut by cost measured the same
    // as the pairs dealt in turn here (2.32-2.33 against 2.30-2.34 ms, down 1.18-1.20 against
    // 1.19 ms) and serves the bf16 kernel too, where it is 1% faster.  The grouped order of the
    // bf16 kernel measured no faster here.
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int item = g.tile_count[8 + xcd] * ncols + j;  // this XCD's range of row tiles
    if (item >= g.tile_count[9 + xcd] * ncols) return;
    const Tile tile = g.tiles[item / ncols];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nsub = (r1 - r0 + 15) / 16;
    const int nt = item % ncols;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / NC, wc = wave % NC;
    // row groups mi * 2 + wr < nsub of this wavefront hold rows: mi < na (a scalar count, so
    // that each group's MFMAs sit behind one scalar compare and branch)
    const int na = __builtin_amdgcn_readfirstlane((nsub - wr + 1) >> 1);
    const int K = g.K;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;

    // A32: every activation row offset fits 32 bits, so the loads take the scalar-base form
    const char* pa[A_DMA];
    uint32_t va[A_DMA];
    const char* const a_s = static_cast<const char*>(g.a);
    constexpr bool a_scalar_ = A32;  // activation loads in the scalar-base form
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int row = (i * NW + wave) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        const int rr = min(r0 + row, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
        pa[i] = a_s + (size_t(src) * K + ch * 8) * 2;
        va[i] = static_cast<uint32_t>((size_t(src) * K + ch * 8) * 2);
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
    // NW = 8: a wavefront moves either nibbles (waves 0-3) or scale words (4-7): one pointer
    const char* const pw = (NW == 8 && wave >= 4) ? ps : pq;
    // PK: the tile's stage blocks as scalar bases, the row's place in a block as the offset
    const char* const wq_s = static_cast<const char*>(g.w) + tb * (K / 32) * 4096;
    const char* const ws_s = reinterpret_cast<const char*>(g.wscale) + tb * (K / 64) * 1024;
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
            if constexpr (A32) dma16s(a_s + k0_ * 2, va[i], &SA[(i * NW + wave) * 64]);       \
            else dma16(pa[i] + k0_ * 2, &SA[(i * NW + wave) * 64]);                             \
    } while (0)
    // nibbles of stage k0/32, and the scale word holding its two scales (stages 2m, 2m+1); with
    // NW = 8 the word is loaded with the pair's first stage only (SC: the stage is a pair's
    // first), and the thread that decodes a row keeps it in a register for the second
#define MOE_ISSUE_W(SN, SS, K0, SC)                                                             \
    do {                                                                                        \
        const int k0_ = (K0);                                                                   \
        if constexpr (PK) {                                                                     \
            if (NW == 4 || wave < 4)                                                            \
                dma16s(wq_s + (k0_ >> 5) * 4096, mrow * 16, &SN[(wave & 3) * 64]);              \
            if (NW == 4 || (wave >= 4 && (SC)))                                                 \
                dma4s(ws_s + (k0_ >> 6) * 1024, mrow * 4, &SS[(wave & 3) * 64]);                \
        } else {                                                                                \
            if (NW == 4 || wave < 4)                                                            \
                dma16((NW == 8 ? pw : pq) + k0_ / 2, &SN[(wave & 3) * 64]);                     \
            if (NW == 4 || (wave >= 4 && (SC)))                                                 \
                dma4((NW == 8 ? pw : ps) + ((k0_ >> 4) & ~3), &SS[(wave & 3) * 64]);            \
        }                                                                                       \
    } while (0)
    // NW = 4: thread t decodes weight row t; NW = 8: half h = t & 1 of row t >> 1 (chunks
    // 2h, 2h+1, scale h)
#define MOE_DECODE(SN, SS, SB, K0)                                                              \
    do {                                                                                        \
        if constexpr (NW == 4) {                                                                \
            const uint4 nib_ = SN[tid];                                                         \
            const uint32_t sw_ = SS[tid] >> ((((K0) >> 5) & 1) * 16);                           \
            const float s0_ = e4m3_value(sw_);                                                  \
            const float s1_ = e4m3_value(sw_ >> 8);                                             \
            SB[lds_slot32(tid, 0)] = dequant8(nib_.x, s0_);                                     \
            SB[lds_slot32(tid, 1)] = dequant8(nib_.y, s0_);                                     \
            SB[lds_slot32(tid, 2)] = dequant8(nib_.z, s1_);                                     \
            SB[lds_slot32(tid, 3)] = dequant8(nib_.w, s1_);                                     \
        } else {                                                                                \
            const int row_ = tid >> 1, h_ = tid & 1;                                            \
            const uint2 nib_ = reinterpret_cast<const uint2*>(SN)[row_ * 2 + h_];               \
            const uint32_t sw_ = SS[row_] >> ((((K0) >> 5) & 1) * 16 + 8 * h_);                 \
            const float sc_ = e4m3_value(sw_);                                                  \
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
#define MOE_READ_B(SB, BF)                                                                      \
    do {                                                                                        \
        _Pragma("unroll") for (int ni = 0; ni < NB; ++ni) BF[ni] =                              \
            __builtin_bit_cast(bf16x8_t, SB[lds_slot32(gb[ni] * 16 + (lane & 15), lane >> 4)]);  \
    } while (0)
    // row group mi's activation fragment of the next stage (ring slot SA) is read into AF[mi]
    // right after the group's MFMAs, under the same test, so that a group without rows is
    // neither multiplied nor read and one fragment set serves both stages
#define MOE_READ_A1(SA, AF, mi)                                                                 \
    AF[mi] = __builtin_bit_cast(bf16x8_t, SA[lds_slot32(((mi) * 2 + wr) * 16 + (lane & 15), lane >> 4)])
#define MOE_MFMA(AF, BF, FULLC, SAR)                                                            \
    do {                                                                                        \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) {                                      \
            if (FULLC || __builtin_expect(mi < na_, 1)) {                                       \
                _Pragma("unroll") for (int ni = 0; ni < NB; ++ni) acc[mi][ni] =                 \
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[mi], BF[ni], acc[mi][ni], 0, 0, 0); \
                MOE_READ_A1(SAR, AF, mi);                                                       \
            }                                                                                   \
        }                                                                                       \
    } while (0)
    // NW = 8: the MFMAs of one stage with the decode of raw stage K0 (into SB) interleaved: after
    // row group mi's MFMAs, output word mi of this thread's 8 (two chunks of four words); the
    // stage's loads (activation chunks after groups 1 and 3, raw weights after group 5) are
    // issued between the groups too, so that a load that waits for the address unit does not
    // hold back the MFMAs (NVFP4 prefill forward 4.02-4.04 -> 3.98 ms, one process)
#define MOE_MFMA_DEC(AF, BF, SB, NIB, SW, K0, FULLC, SAW, SNW, SSW, KA, KW, SCW, SAR)            \
    do {                                                                                        \
        typedef __attribute__((ext_vector_type(2))) float f2_;                                  \
        const int row_ = tid >> 1, h_ = tid & 1;                                                \
        const uint2 nib_ = NIB;                                                                 \
        const uint32_t sw_ = (SW) >> ((((K0) >> 5) & 1) * 16 + 8 * h_);                         \
        const float sc_ = e4m3_value(sw_);                                                      \
        uint32_t w_[8];                                                                         \
        _Pragma("unroll") for (int mi = 0; mi < 8; ++mi) {                                      \
            if (FULLC || __builtin_expect(mi < na_, 1)) {                                       \
                _Pragma("unroll") for (int ni = 0; ni < NB; ++ni) acc[mi][ni] =                 \
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[mi], BF[ni], acc[mi][ni], 0, 0, 0); \
                MOE_READ_A1(SAR, AF, mi);                                                       \
            }                                                                                   \
            {                                                                                   \
                const uint32_t src_ = (mi < 4) ? nib_.x : nib_.y;                               \
                f2_ v_;                                                                         \
                if ((mi & 3) == 0) v_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src_, 1.0f, 0); \
                else if ((mi & 3) == 1) v_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src_, 1.0f, 1); \
                else if ((mi & 3) == 2) v_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src_, 1.0f, 2); \
                else v_ = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src_, 1.0f, 3);              \
                w_[mi] = __builtin_amdgcn_perm(__float_as_uint(v_.y * sc_), __float_as_uint(v_.x * sc_), 0x07060302u); \
                /* keeps word mi after group mi's MFMAs; unpinned, the compiler moved the     \
                   words to the two LDS writes (gate/up 2.43 -> 2.40 ms, bit-identical) */    \
                asm volatile("" : "+v"(w_[mi]));                                                \
            }                                                                                   \
            if (mi == 3) SB[lds_slot32(row_, 2 * h_)] = make_uint4(w_[0], w_[1], w_[2], w_[3]);  \
            if (mi == 1 || mi == 3) {                                                           \
                const int i_ = mi >> 1;                                                         \
                if (a_scalar_) dma16s(a_s + size_t(KA) * 2, va[i_], &SAW[(i_ * NW + wave) * 64]); \
                else dma16(pa[i_] + size_t(KA) * 2, &SAW[(i_ * NW + wave) * 64]);               \
            }                                                                                   \
            if (mi == 5) MOE_ISSUE_W(SNW, SSW, KW, SCW);                                        \
        }                                                                                       \
        SB[lds_slot32(row_, 2 * h_ + 1)] = make_uint4(w_[4], w_[5], w_[6], w_[7]);               \
    } while (0)

    f32x4_t acc[8][NB];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < NB; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t af[8], b0[NB], b1[NB];

    const int nk = K / BKS;
    const int last = (nk - 1) * BKS;
    // prologue: raw stages 0 and 1, activation stage 0; decode both; then activation stages
    // 1..3 and raw stages 2..4 in the steady-state issue order
    MOE_ISSUE_W(sN0, sS0, 0, true);
    MOE_ISSUE_W(sN1, sS1, min(1 * BKS, last), false);
    MOE_ISSUE_A(sA0, 0);
    wait_vm_lgkm0<0>();
    block_barrier();
    MOE_DECODE(sN0, sS0, sB0, 0);
    MOE_DECODE(sN1, (NW == 8 ? sS0 : sS1), sB1, min(1 * BKS, last));  // NW = 8: stage 0's word
    wait_vm_lgkm0<0>();
    block_barrier();
    MOE_READ(sA0, sB0, af, b0);
    MOE_ISSUE_A(sA1, min(1 * BKS, last));
    MOE_ISSUE_W(sN2, sS2, min(2 * BKS, last), true);
    MOE_ISSUE_A(sA2, min(2 * BKS, last));
    MOE_ISSUE_W(sN3, sS3, min(3 * BKS, last), false);
    MOE_ISSUE_A(sA3, min(3 * BKS, last));
    MOE_ISSUE_W(sN0, sS0, min(4 * BKS, last), true);
    uint2 nibd_ = make_uint2(0, 0);  // raw weight words this thread decodes in the next MFMA block
    uint32_t swd_ = 0;
    int na_;  // na, re-read each stage so that the group tests stay scalar compares
#define MOE_IT(FULLC, S, FB, GB, SAr, SBr, SAw, SNw, SSw, SNd, SSd, SBd)      \
        /* NW = 8: wavefronts 4-7 issue one load fewer per stage pair */      \
        if (NW == 8 && wave >= 4) wait_vm_lgkm0<2 * OPS - 1>();              \
        else wait_vm_lgkm0<2 * OPS>();                                       \
        block_barrier();                                                     \
        na_ = na;                                                            \
        asm volatile("" : "+s"(na_));                                        \
        if constexpr (NW == 8) {                                             \
            nibd_ = reinterpret_cast<const uint2*>(SNd)[tid];                \
            if ((S & 1) == 0) swd_ = SSd[tid >> 1]; /* odd stages: kept */   \
        }                                                                    \
        MOE_READ_B(SBr, GB);                                                 \
        if constexpr (NW == 4) {                                             \
            MOE_ISSUE_A(SAw, min((s + S + 4) * BKS, last));                  \
            MOE_ISSUE_W(SNw, SSw, min((s + S + 5) * BKS, last), true);       \
        }                                                                    \
        if constexpr (NW == 8) {                                             \
            MOE_MFMA_DEC(af, FB, SBd, nibd_, swd_, min((s + S + 2) * BKS, last), FULLC, SAw, SNw, SSw, min((s + S + 4) * BKS, last), min((s + S + 5) * BKS, last), ((S) & 1) == 1, SAr); \
            if (s + S + 1 >= nk) break;                                      \
        } else {                                                             \
            MOE_MFMA(af, FB, FULLC, SAr);                                    \
            if (s + S + 1 >= nk) break;                                      \
            MOE_DECODE(SNd, SSd, SBd, min((s + S + 2) * BKS, last));         \
        }
#define MOE_LOOP(FULLC)                                                      \
    for (int s = 0;; s += 4) {                                           \
        MOE_IT(FULLC, 0, b0, b1, sA1, sB1, sA0, sN1, sS1, sN2, sS2, sB0) \
        MOE_IT(FULLC, 1, b1, b0, sA2, sB0, sA1, sN2, sS2, sN3, sS3, sB1) \
        MOE_IT(FULLC, 2, b0, b1, sA3, sB1, sA2, sN3, sS3, sN0, sS0, sB0) \
        MOE_IT(FULLC, 3, b1, b0, sA0, sB0, sA3, sN0, sS0, sN1, sS1, sB1) \
    }
    MOE_LOOP(false)
#undef MOE_LOOP
#undef MOE_IT
    wait_vm_lgkm0<0>();
#undef MOE_ISSUE_A
#undef MOE_ISSUE_W
#undef MOE_DECODE
#undef MOE_READ
#undef MOE_MFMA
#undef MOE_MFMA_DEC
#undef MOE_READ_B
#undef MOE_READ_A1

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

template <int KIND, int WFMT, int SPLITK, bool WIN4 = false>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g) {
    __shared__ f32x4_t red[4][(KIND == kGateUp) ? 2 : 1][64];
    decode_gemm_item<KIND, WFMT, SPLITK, WIN4>(g, blockIdx.x, red);
}

template <int KIND, int SPLITK, int NCG>
__global__ __launch_bounds__(256) void gemm_decode_nvfp4p_kernel(GemmArgs g) {
    __shared__ f32x4_t red[SPLITK > 1 ? 4 : 1][((KIND == kGateUp) ? 2 : 1) * NCG][64];
    decode_nvfp4p_item<KIND, SPLITK, NCG>(g, blockIdx.x, red);
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

// Blocks for the XCD ranges of a prefill tile list: a tile costs between half a full tile and a
// full one, so a range cut at an eighth of the cost, rounded to a tile, holds fewer than
// twice the mean number of tiles plus two
static dim3 xcd_grid(const GemmArgs& g, int max_tiles) {
    const int ncols = g.kind == kGateUp ? g.F / 128 : (g.N + 255) / 256;
    return dim3(8 * (2 * ((max_tiles + 7) / 8) + 2) * ncols);
}

hipError_t launch_gemm(const GemmArgs& g, int family, int max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    // every kernel below reads the scales its format has, and only those
    if ((g.wfmt == kWNVFP4 || g.wfmt == kWMXFP8 || g.wfmt == kWMXFP4) && !g.wscale) return hipErrorInvalidValue;
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
        const dim3 grid = xcd_grid(g, max_tiles);
        // the scalar-base activation loads need every row offset below 4 GiB
        const bool a32 = size_t(g.a_rows_limit) * size_t(g.K) * 2 <= 0xffffffffull;
        if (up && a32)
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kGateUp, true>), grid, dim3(512), 0, s, g);
        else if (up)
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kGateUp, false>), grid, dim3(512), 0, s, g);
        else if (a32)
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kDown, true>), grid, dim3(512), 0, s, g);
        else
            hipLaunchKernelGGL((gemm_prefill_bf16_kernel<kDown, false>), grid, dim3(512), 0, s, g);
    } else if (family == kFamPrefill && g.wfmt == kWNVFP4 && g.F % 128 == 0) {
        const dim3 grid = xcd_grid(g, max_tiles);
        // packed weights: 8 wavefronts for both kinds (gate/up 2.97 -> 2.69 ms against 4 on
        // the NVFP4 prefill shape); row-major: 4 for gate/up, where 4 measured faster
        // the scalar-base activation loads need every row offset below 4 GiB
        const bool a32 = size_t(g.a_rows_limit) * size_t(g.K) * 2 <= 0xffffffffull;
        if (up && g.wpacked && a32)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kGateUp, 8, true, true>), grid, dim3(512), 0, s, g);
        else if (up && g.wpacked)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kGateUp, 8, true, false>), grid, dim3(512), 0, s, g);
        else if (up)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kGateUp, 4, false, false>), grid, dim3(256), 0, s, g);
        else if (g.wpacked && a32)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kDown, 8, true, true>), grid, dim3(512), 0, s, g);
        else if (g.wpacked)
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kDown, 8, true, false>), grid, dim3(512), 0, s, g);
        else
            hipLaunchKernelGGL((gemm_prefill_nvfp4_kernel<kDown, 8, false, false>), grid, dim3(512), 0, s, g);
    } else if (family == kFamPrefill) {
        if (g.wfmt != kWNVFP4 || g.wpacked) return hipErrorInvalidValue;  // PACKED NVFP4 needs F % 128 == 0
        launch_mfma<PF_BM, PF_BN, PF_WM, PF_WN>(g, max_tiles, s);
    } else if (g.wfmt == kWNVFP4 && g.wpacked) {  // PACKED NVFP4 decode: NCG row groups per wavefront
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
        if (g.wfmt != kWNVFP4 || g.wpacked) return hipErrorInvalidValue;  // PACKED NVFP4 needs H % 256, F % 128 == 0
        launch_mfma<DC_BM, DC_BN, DC_WM, DC_WN>(g, max_tiles, s);
    }
    return hipGetLastError();
}

}  // namespace moe
