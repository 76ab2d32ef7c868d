// gemv.h -- the weight-streaming (decode) grouped GEMMs of the MoE layer as device functions:
// one call computes one block-sized work item, so the same code serves the stand-alone decode
// kernels (one item per block, gemm.hip) and the single-launch decode kernel (a persistent
// grid walking the items, decode_fused.hip).  Also the exact NVFP4 decode shared by every GEMM.
// Every call must be made by all 256 threads of a block (work items are block-uniform; the
// split-K reduction passes a block barrier).
#pragma once

#include "device.h"
#include "launch.h"

namespace moe {
namespace {

// E4M3 (FN) byte 0 of c -> its value in fp32, by the hardware conversion: exact for every code
// (subnormals included; S.1111.111 gives NaN, as the format defines).  The instruction applies
// only the exponent of its scale operand, so a scale of 1.0 leaves the value as it is.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    return __builtin_amdgcn_cvt_scalef32_f32_fp8(c, 1.0f, 0);
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

// ---------------------------------------------------------------------------------------
// Decode kernel: few rows per expert, so the layer streams the selected experts' weights once
// from HBM ("Hosting Qwen on Blackwell", section Decoders: decode matmuls are bound by weight
// loads).  One wavefront owns 16 weight rows (gate/up: 16 gate rows and the 16 matching up
// rows) and up to 16 dispatched rows of one expert; weights go from global memory straight
// into MFMA operand registers (no LDS), two 128-wide K blocks in flight per lane.  Weight
// loads carry the non-temporal hint (each weight byte is read once per call; activations keep
// the default, being read by every wavefront of their expert): forward medians, bit-identical,
// decode T=8 310.7 -> 288.3 us, T=64 799.6 -> 745.4 us, NVFP4 T=16 281.4 -> 271.1 us, T=1
// (caches flushed) unchanged at 75 us.
//
// bf16 weights: MFMA i of K block j is stage 4 j + i, and lane (row n, k-group q) reads
// logical chunk q of its row in that stage, from the packed layout (16 rows x 64 bytes of a
// stage are one contiguous KiB) or from the row-major matrix (the same elements, 64 bytes per
// row and stage; same arithmetic, so both layouts give bit-identical results).  NVFP4 weights are row-major; there the reduction index is permuted inside
// each 128-wide block so that one lane's 32 nibbles are contiguous: MFMA i takes, in k-group
// q, elements 128 j + 32 q + 8 i .. +7 of both operands (a common permutation of K leaves the
// dot products unchanged).
//
// SPLITK wavefronts of a block share 16 columns and split K; their partial sums meet in LDS
// and are added in a fixed order (deterministic).
// ---------------------------------------------------------------------------------------

template <int KIND, int WFMT, int SPLITK, bool WIN4 = false>
__device__ __forceinline__ void decode_gemm_item(const GemmArgs& g, int item,
                                                 f32x4_t (*red)[(KIND == kGateUp) ? 2 : 1][64]) {
    constexpr int CG = 4 / SPLITK;              // column groups per block
    constexpr int NB = (KIND == kGateUp) ? 2 : 1;  // weight row sets per column group

    const int ncg = (KIND == kGateUp) ? g.F / 16 : (g.N + 15) / 16;
    const int per_tile = (ncg + CG - 1) / CG;
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
    auto ldw = [](const void* p) __attribute__((always_inline)) { return load_nt16(p); };
    // bf16 (packed): lane's 16 bytes of stage st of its gate/down row and of its up row
    const uint16_t* pw0 = nullptr;
    const uint16_t* pw1 = nullptr;
    size_t sst = 32;  // elements from one 32-element stage of the lane's chunk to the next
    if (WFMT == kWBF16 && !g.wpacked) {  // row-major: the lane's chunk q of its own rows
        pw0 = static_cast<const uint16_t*>(g.w) + (size_t(e) * Nw + wrow0) * K + 8 * q;
        pw1 = static_cast<const uint16_t*>(g.w) + (size_t(e) * Nw + wrow1) * K + 8 * q;
    } else if constexpr (WFMT == kWBF16) {
        sst = 8192;
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
            const size_t so = size_t(4 * j) * sst;  // stage 4 j
            b.g0 = ldw(pw0 + so);
            b.g1 = ldw(pw0 + so + sst);
            b.g2 = ldw(pw0 + so + 2 * sst);
            b.g3 = ldw(pw0 + so + 3 * sst);
            if constexpr (KIND == kGateUp) {
                b.u0 = ldw(pw1 + so);
                b.u1 = ldw(pw1 + so + sst);
                b.u2 = ldw(pw1 + so + 2 * sst);
                b.u3 = ldw(pw1 + so + 3 * sst);
            }
        } else {
            b.a0 = ld16(pa + k);
            b.a1 = ld16(pa + k + 8);
            b.a2 = ld16(pa + k + 16);
            b.a3 = ld16(pa + k + 24);
            b.pg = ldw(pq0 + 64 * j);
            b.sg = *reinterpret_cast<const uint16_t*>(ps0 + 8 * j);
            if constexpr (KIND == kGateUp) {
                b.pu = ldw(pq1 + 64 * j);
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
            b.pg = ldw(pq0 + 256 * w + 16 * jj);
            if constexpr (KIND == kGateUp) b.pu = ldw(pq1 + 256 * w + 16 * jj);
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
__device__ __forceinline__ void decode_nvfp4p_item(const GemmArgs& g, int item,
                                                   f32x4_t (*red)[((KIND == kGateUp) ? 2 : 1) * NCG][64]) {
    static_assert(NCG == 1 || NCG == 2 || NCG == 4, "row groups must stay inside a 64-row half");
    constexpr int WPB = 4 / SPLITK;                 // group sets per block
    constexpr int NB = (KIND == kGateUp) ? 2 : 1;   // gate and up rows, or down rows

    const int ncg = (KIND == kGateUp) ? g.F / 16 : g.N / 16;  // F % 128 == 0, N % 256 == 0
    const int per_tile = (ncg + WPB * NCG - 1) / (WPB * NCG);
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
    auto ldw = [](const void* p) __attribute__((always_inline)) { return load_nt16(p); };
    auto load = [&](Blk& b, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b.a[i] = ld16(pa + 128 * j + 8 * i);
#pragma unroll
        for (int h = 0; h < NB; ++h)
#pragma unroll
            for (int c = 0; c < NCG; ++c) {
                b.p[h * NCG + c] = ldw(pq + 16384 * j + h * 1024 + c * 256);
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

}  // namespace moe
