// mx.hip -- the MXFP8 layer on gfx950's block-scaled fp8 matrix cores.
//
// MXFP8 (OCP microscaling formats v1.0): E4M3 elements with one E8M0 scale 2^(s-127) per 32
// consecutive elements along K; "Hosting Qwen on Blackwell" (section Quantization) deploys its
// MoE weights in it, and "CuTeDSL at Perplexity" (section Blackwell) notes the per-32-element
// absolute-maximum reductions its activation quantizers need.  Two kernels:
//   mx_quantize_kernel        bf16 rows -> E4M3 codes + E8M0 scales, one thread per block of 32
//                             (x before the gate/up GEMM, hid before the down GEMM)
//   gemm_prefill_mxfp8_kernel the grouped GEMM of gemm.hip's bf16 prefill kernel (256 x 256
//                             block tile, 8 wavefronts of 128 x 64, 4-slot LDS ring of 64-byte
//                             rows filled by direct global->LDS loads) on
//                             v_mfma_scale_f32_32x32x64_f8f6f4: one 64-wide K stage of the
//                             ring is one MFMA K step.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured on the hardware against exact
// CPU products): lane l feeds row l & 31 of its operand; lane group g = l >> 5 supplies the
// E8M0 scale of the 32-element block g (elements [32g, 32g + 32)) in its scale operand.  An fp8
// operand holds the K elements [16g, 16g + 16) in bytes 0..15 and [32 + 16g, 48 + 16g) in
// bytes 16..31: with 64-byte LDS rows of four 16-byte chunks, lane group g reads chunks g and
// g + 2.  An fp4 (E2M1, format 4) operand holds elements [32g, 32g + 32) in its first 16 bytes,
// the even element in the low nibble: with 32-byte rows, lane group g reads chunk g.  The
// result is the usual 32 x 32 accumulator layout: element i of lane l is row
// 8 (i / 4) + 4 (l >> 5) + (i % 4), column l & 31.
//
// MXFP4 weights (E2M1 + E8M0 per 32) run through the same GEMM with BF4 = 1: fp8 activations
// times fp4 weights, 32-byte weight rows per stage (8 KiB packed blocks, chunk c of row r in
// slot c ^ ((r >> 2) & 1)), one weight DMA per wavefront per stage.
#include "device.h"
#include "launch.h"
#include "lds_dma.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// ---------------------------------------------------------------------------------------
// Activation quantizer.  Per block of 32 bf16 values v: X = floor(log2 max|v|) - 8 (-127 for an
// all-zero block, at least -127), scale byte X + 127; element code = the E4M3 value nearest to
// min(|v| 2^-X, 448), ties to the even code, with the sign bit of v.  Every step is exact in
// fp32 (bf16 times a power of two), so the codes are a pure function of the bf16 input.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t e4m3_code(float q) {  // 0 <= q <= 448
    if (q < 0.015625f) return uint32_t(__builtin_rintf(q * 512.0f));  // subnormal grid m 2^-9
    const uint32_t u = __float_as_uint(q);
    const uint32_t e = (u >> 23) - 127u + 7u;           // biased E4M3 exponent, 1..15
    const uint32_t mant = u & 0x7fffffu;
    const uint32_t r = mant + 0x7ffffu + ((mant >> 20) & 1u);  // round 23 -> 3 bits, nearest even
    return (e << 3) + (r >> 20);                         // a carry moves into the exponent
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint4* __restrict__ in, long nblocks,
                                                          uint4* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    for (long b = long(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
         b += long(gridDim.x) * blockDim.x) {
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 q = in[b * 4 + i];
            w[4 * i] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            amax = fmaxf(amax, fabsf(bf16_lo(w[i])));
            amax = fmaxf(amax, fabsf(bf16_hi(w[i])));
        }
        const uint32_t amax_bits = __float_as_uint(amax);
        int X = -127;  // floor(log2 amax) - 8 from the exponent field; subnormal amax gives <= -127
        if (amax > 0.0f) X = max(int((amax_bits >> 23) & 0xffu) - 127 - 8, -127);
        const float inv = __uint_as_float(uint32_t(127 - X) << 23);  // 2^-X, normal for X in [-127, 119]
        uint32_t out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 4 * i + j;                       // element 0..31
                const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
                const float v = __uint_as_float(bits << 16);
                const float q = fminf(fabsf(v) * inv, 448.0f);
                const uint32_t c = e4m3_code(q) | ((bits >> 8) & 0x80u);
                word |= c << (8 * j);
            }
            out[i] = word;
        }
        codes[b * 2] = make_uint4(out[0], out[1], out[2], out[3]);
        codes[b * 2 + 1] = make_uint4(out[4], out[5], out[6], out[7]);
        scales[b] = uint8_t(X + 127);
    }
}

hipError_t launch_mx_quantize(const void* in, long rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
    const long nb = rows * (K / 32);
    if (nb <= 0) return hipSuccess;
    const long want = (nb + 255) / 256;
    const int blocks = int(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(mx_quantize_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(in),
                       nb, reinterpret_cast<uint4*>(codes), scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// MXFP8 grouped GEMM, prefill tiles.  a: E4M3 codes [rows, K] (gathered through a_rows for
// gate/up), ascale: E8M0 [rows, K/32]; w: E4M3 codes in the PACKED layout of moe.h (each stage
// of a 256-row weight tile is one contiguous 16 KiB block, exactly the LDS image; a stage is 64
// fp8 elements here), wscale: E8M0 [E, Nw, K/32] row-major.  Block tile 256 x 256; wavefronts
// 2 x 4 of 128 x 64: wavefront (wr, wc) holds the 32-row groups 2 mi + wr (mi = 0..3) and two
// 32-row weight groups.  In a gate/up tile, rows 128 h + (0..63) are gate rows
// f = 128 nt + 64 h + (0..63) and rows 128 h + 64 + (0..63) the matching up rows F + f, so
// wavefront column wc takes weight groups 4 (wc >> 1) + (wc & 1) (gate) and that + 2 (up): hid
// columns 128 nt + 64 (wc >> 1) + 32 (wc & 1) + (0..31), and SwiGLU applies in registers.
//
// Pipeline: K in 64-wide stages (64-byte rows), a 4-slot LDS ring filled by dma16 as in the
// bf16 kernel (each wavefront moves two 16-row groups of activations, gathered, and two 1 KiB
// pieces of the packed weight stage per stage).  E8M0 scales come in chunks of 8 stages: 16 scale bytes per row (one dma16 per
// wavefront per chunk: wavefronts 0-3 activation rows, 4-7 weight rows) into one of two scale
// slots, issued with the chunk's first stage; a slot is rewritten 16 stages after it was
// filled, long after its last read and behind a barrier.  Needs K % 512 == 0.
//
// Iteration s: issue the MFMAs of stage s from the fragment registers; wait until stage s+1 has
// landed (a wavefront issues 4 or 5 DMA instructions per stage, so at most 8 outstanding ones
// means stage s+1 and every earlier one are in LDS) and pass the barrier that publishes it and
// frees stage s's ring slot; read stage s+1's fragments into the same registers (the MFMAs have
// taken their operands by then; the other wavefront on the SIMD covers the wait); issue the
// loads of stage s+4.  Two fragment sets do not fit beside 128 accumulators in 256 registers.
// ---------------------------------------------------------------------------------------

template <int KIND, int BF4>
__global__ __launch_bounds__(512, 1) void gemm_prefill_mxfp8_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256;
    constexpr int HALF = (KIND == kGateUp) ? BN / 2 : BN;
    constexpr int BCH = BF4 ? 2 : 4;             // 16-byte chunks per weight row per stage
    constexpr int NDMA = 2 + (BF4 ? 1 : 2);      // DMA instructions per wavefront per stage (+ scales)
    __shared__ uint4 sA0[BM * 4], sA1[BM * 4], sA2[BM * 4], sA3[BM * 4];
    __shared__ uint4 sB0[BN * BCH], sB1[BN * BCH], sB2[BN * BCH], sB3[BN * BCH];
    __shared__ uint4 tS[2][BM + BN];  // per chunk of 8 stages: 16 scale bytes per activation row, then per weight row

    const int ncols = (KIND == kGateUp) ? g.F / HALF : (g.N + BN - 1) / BN;
    const int items = *g.tile_count * ncols;
    const int run = (items + 7) >> 3;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int item = xcd * run + j;
    if (j >= run || item >= items) return;
    const Tile tile = g.tiles[item / ncols];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int nsub = (r1 - r0 + 31) / 32;  // 32-row groups holding rows
    const int nt = item % ncols;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
    const int wr = wave >> 2, wc = wave & 3;
    const int K = g.K, KB = K / 32;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;

    auto weight_row = [&](int r) {  // weight row (of this expert) behind tile row r
        if (KIND == kGateUp) {
            const int q = r & 127, f = nt * 128 + 64 * (r >> 7) + (q & 63);
            return q < 64 ? f : g.F + f;
        }
        return nt * BN + r;
    };
    auto act_row = [&](int r) {  // row of `a` behind tile row r (padded rows repeat the last)
        const int rr = min(r0 + r, r1 - 1);
        int src = g.a_rows ? g.a_rows[rr] : rr;
        return src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
    };
    const int nk = K / 64;
    const char* const wblk = static_cast<const char*>(g.w) + (size_t(e) * ncols + nt) * size_t(nk) * (BN * BCH * 16);
    const char* pa[2];
    const char* pb[2];
    // weights: packed (one contiguous (tile, stage) block per stage, the LDS image), or row-major
    // (each lane fetches the chunk of its weight row that belongs in its LDS slot: 64 fp8 or 32
    // fp4 bytes per row and stage; the same LDS image, so bit-identical results)
    const size_t wst = g.wpacked ? size_t(BN) * BCH * 16 : BCH * 16;  // bytes per stage
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (i * 8 + wave) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 1) & 3);
        pa[i] = static_cast<const char*>(g.a) + size_t(act_row(row)) * K + ch * 16;
        if (g.wpacked) {
            pb[i] = wblk + (BF4 ? wave : i * 8 + wave) * 1024 + lane * 16;
        } else if (BF4) {  // 32 rows of 32 bytes per wavefront: lane l -> row 32 wave + l / 2, slot l & 1
            const int r4 = wave * 32 + (lane >> 1), c4 = (lane & 1) ^ ((r4 >> 2) & 1);
            pb[i] = static_cast<const char*>(g.w) + (size_t(e) * Nw + weight_row(r4)) * (K / 2) + c4 * 16;
        } else {
            pb[i] = static_cast<const char*>(g.w) + (size_t(e) * Nw + weight_row(row)) * K + ch * 16;
        }
    }
    const char* psc;  // this lane's row of scales: 16 bytes per chunk of 8 stages
    {
        const int row = (wave & 3) * 64 + lane;
        psc = wave < 4 ? reinterpret_cast<const char*>(g.ascale) + size_t(act_row(row)) * KB
                       : reinterpret_cast<const char*>(g.wscale) + (size_t(e) * Nw + weight_row(row)) * KB;
    }
    const int sc_off = (wave < 4 ? 0 : BM) + (wave & 3) * 64;  // this wavefront's scale rows in a slot

    const int last = nk - 1;
    const int gbn0 = (KIND == kGateUp) ? 4 * (wc >> 1) + (wc & 1) : 2 * wc;  // this wavefront's two
    const int gbn1 = (KIND == kGateUp) ? gbn0 + 2 : 2 * wc + 1;              // 32-row weight groups
    const int g2 = lane >> 5;  // lane group: chunks g2 and g2 + 2, scale block g2

#define MOE_MXISSUE(SA, SB, ST)                                                               \
    do {                                                                                      \
        const int st_ = min((ST), last);                                                      \
        _Pragma("unroll") for (int i = 0; i < 2; ++i)                                         \
            dma16(pa[i] + st_ * 64, &SA[(i * 8 + wave) * 64]);                                \
        _Pragma("unroll") for (int i = 0; i < (BF4 ? 1 : 2); ++i)                             \
            dma16(pb[i] + size_t(st_) * wst, &SB[(i * 8 + wave) * 64]);                       \
        if (((ST) & 7) == 0)                                                                  \
            dma16(psc + (st_ >> 3) * 16, &tS[((ST) >> 3) & 1][sc_off]);                      \
    } while (0)
#define MOE_MXFRAG(S, ROW, F)                                                                 \
    do {                                                                                      \
        typedef __attribute__((ext_vector_type(4))) int i32x4_t_;                             \
        const i32x4_t_ lo_ = __builtin_bit_cast(i32x4_t_, S[lds_slot32((ROW), g2)]);          \
        const i32x4_t_ hi_ = __builtin_bit_cast(i32x4_t_, S[lds_slot32((ROW), g2 + 2)]);      \
        F = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7);                        \
    } while (0)
#define MOE_MXSCALE(ST, ROW) \
    (int)reinterpret_cast<const uint8_t*>(&tS[((ST) >> 3) & 1][0])[(ROW) * 16 + ((ST) & 7) * 2 + g2]
#define MOE_MXFRAG4(S, ROW, F)                                                                \
    do {                                                                                      \
        const int r4_ = (ROW);                                                                \
        const uint4 c_ = S[r4_ * 2 + (g2 ^ ((r4_ >> 2) & 1))];                                \
        F = i32x8_t{int(c_.x), int(c_.y), int(c_.z), int(c_.w), 0, 0, 0, 0};                  \
    } while (0)
#define MOE_MXREAD(SA, SB, ST)                                                                \
    do {                                                                                      \
        if (BF4) {                                                                            \
            MOE_MXFRAG4(SB, gbn0 * 32 + (lane & 31), bf[0]);                                  \
            MOE_MXFRAG4(SB, gbn1 * 32 + (lane & 31), bf[1]);                                  \
        } else {                                                                              \
            MOE_MXFRAG(SB, gbn0 * 32 + (lane & 31), bf[0]);                                   \
            MOE_MXFRAG(SB, gbn1 * 32 + (lane & 31), bf[1]);                                   \
        }                                                                                     \
        bs[0] = MOE_MXSCALE((ST), BM + gbn0 * 32 + (lane & 31));                              \
        bs[1] = MOE_MXSCALE((ST), BM + gbn1 * 32 + (lane & 31));                              \
        _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                    \
            MOE_MXFRAG(SA, (mi * 2 + wr) * 32 + (lane & 31), af[mi]);                         \
            as[mi] = MOE_MXSCALE((ST), (mi * 2 + wr) * 32 + (lane & 31));                     \
        }                                                                                     \
    } while (0)
#define MOE_MXMFMA()                                                                          \
    do {                                                                                      \
        _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                    \
            if (mi * 2 + wr < nsub) {                                                         \
                _Pragma("unroll") for (int ni = 0; ni < 2; ++ni) acc[mi][ni] =                \
                    __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf[ni], acc[mi][ni], \
                                                                    0, BF4 ? 4 : 0, 0, as[mi], 0, bs[ni]); \
            }                                                                                 \
        }                                                                                     \
    } while (0)

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.0f;
    i32x8_t af[4], bf[2];
    int as[4], bs[2];

    MOE_MXISSUE(sA0, sB0, 0);
    MOE_MXISSUE(sA1, sB1, 1);
    MOE_MXISSUE(sA2, sB2, 2);
    wait_vm_lgkm0<2 * NDMA>();  // stage 0 (and the first scale chunk) landed
    block_barrier();
    MOE_MXREAD(sA0, sB0, 0);
    MOE_MXISSUE(sA3, sB3, 3);
    for (int s = 0;; s += 4) {
        MOE_MXMFMA();
        if (s + 1 >= nk) break;
        wait_vm_lgkm0<2 * NDMA>();
        block_barrier();
        MOE_MXREAD(sA1, sB1, s + 1);
        MOE_MXISSUE(sA0, sB0, s + 4);
        MOE_MXMFMA();
        if (s + 2 >= nk) break;
        wait_vm_lgkm0<2 * NDMA>();
        block_barrier();
        MOE_MXREAD(sA2, sB2, s + 2);
        MOE_MXISSUE(sA1, sB1, s + 5);
        MOE_MXMFMA();
        if (s + 3 >= nk) break;
        wait_vm_lgkm0<2 * NDMA>();
        block_barrier();
        MOE_MXREAD(sA3, sB3, s + 3);
        MOE_MXISSUE(sA2, sB2, s + 6);
        MOE_MXMFMA();
        if (s + 4 >= nk) break;
        wait_vm_lgkm0<2 * NDMA>();
        block_barrier();
        MOE_MXREAD(sA0, sB0, s + 4);
        MOE_MXISSUE(sA3, sB3, s + 7);
    }
    wait_vm_lgkm0<0>();
#undef MOE_MXISSUE
#undef MOE_MXFRAG
#undef MOE_MXSCALE
#undef MOE_MXFRAG4
#undef MOE_MXREAD
#undef MOE_MXMFMA

    // Epilogue through LDS (as in the bf16 kernel): once every wavefront is past its last
    // fragment read, each stages a 64-row slice of its output (W bf16 columns, chunk slots
    // XOR-swizzled by row) in half of one activation ring array, in two rounds, and stores the
    // slice as 16-byte row chunks.
    block_barrier();
    constexpr int W = (KIND == kGateUp) ? 32 : 64;  // columns per wavefront
    constexpr int SM = W / 8 - 1;
    uint16_t* const stg = reinterpret_cast<uint16_t*>(
        (wave & 3) == 0 ? sA0 : (wave & 3) == 1 ? sA1 : (wave & 3) == 2 ? sA2 : sA3) + (wave >> 2) * 64 * W;
    const int colbase = (KIND == kGateUp) ? nt * HALF + 64 * (wc >> 1) + 32 * (wc & 1) : nt * BN + wc * 64;
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int mi = 2 * half + m2;
            if (mi * 2 + wr >= nsub) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int lr = m2 * 32 + 8 * (i / 4) + 4 * g2 + (i % 4);
#pragma unroll
                for (int ni = 0; ni < W / 32; ++ni) {
                    const int lc = ni * 32 + (lane & 31);
                    const float v = (KIND == kGateUp) ? silu_mul(acc[mi][0][i], acc[mi][1][i]) : acc[mi][ni][i];
                    stg[lr * W + ((((lc >> 3) ^ (lr >> 2)) & SM) << 3) + (lc & 7)] = (uint16_t)bf16_rne(v);
                }
            }
        }
        asm volatile("" ::: "memory");  // reads of another type after the writes (one wavefront: in order)
#pragma unroll
        for (int it = 0; it < W / 8; ++it) {
            const int q = it * 64 + lane, lr = q / (W / 8), c8 = q % (W / 8);
            const int mi = 2 * half + (lr >> 5);
            const int row = r0 + (mi * 2 + wr) * 32 + (lr & 31);
            if (mi * 2 + wr >= nsub || row >= r1) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(&stg[lr * W + (((c8 ^ (lr >> 2)) & SM) << 3)]);
            const int col = colbase + c8 * 8;
            if (KIND == kGateUp)
                *reinterpret_cast<uint4*>(&out[size_t(row) * g.F + col]) = v;
            else if (col < g.N)
                *reinterpret_cast<uint4*>(&out[size_t(row) * g.N + col]) = v;
        }
        asm volatile("" ::: "memory");  // the next round's writes after these reads
    }
}

// ---------------------------------------------------------------------------------------
// MX decode kernel: few rows per expert (row tiles of 32), so the layer streams the selected
// experts' weights once, from the packed layout straight into MFMA operand registers (no
// LDS).  Lane l = 32 g + n of a wavefront feeds operand row n (token row n of the tile for the
// activations, weight row n of a 32-row group for the weights) and K half g of the
// v_mfma_scale_f32_32x32x64_f8f6f4 layout above: per 64-wide stage an fp8 operand takes chunks
// g and g + 2 of its row's four 16-byte chunks, an fp4 operand chunk g of its two, and the
// lane supplies the E8M0 scale of block 2 s + g.  Scales are loaded 16 bytes (8 stages) per
// row at a time, one chunk ahead.  A wavefront owns two 32-row weight groups that share the
// activation fragments: gate/up, the gate and up rows of 32 hid columns (SwiGLU in
// registers); down, 64 output columns.  Two stages in flight; SPLITK wavefronts of a block
// split the stages and meet in LDS in a fixed order.
// ---------------------------------------------------------------------------------------

template <int KIND, int BF4, int SPLITK>
__global__ __launch_bounds__(256) void gemm_decode_mx_kernel(GemmArgs g) {
    constexpr int NG = 2;                       // weight row groups per wavefront
    constexpr int WPB = 4 / SPLITK;             // group pairs per block
    constexpr int BCH = BF4 ? 2 : 4;            // 16-byte chunks per weight row and stage
    constexpr size_t SBLK = size_t(256) * BCH * 16;  // bytes of one (tile, stage) block
    __shared__ f32x16_t red[SPLITK > 1 ? 4 : 1][NG][64];

    const int nsets = (KIND == kGateUp) ? g.F / 32 : g.N / 64;
    const int per_tile = (nsets + WPB - 1) / WPB;
    const int item = blockIdx.x;
    if (item >= *g.tile_count * per_tile) return;
    const Tile tile = g.tiles[item / per_tile];
    const int e = tile.expert, r0 = tile.row0, r1 = tile.row1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int set = (item % per_tile) * WPB + wave / SPLITK;
    const int kp = wave % SPLITK;
    const bool live = set < nsets;  // uniform per wavefront
    const int K = g.K, nst = K / 64;
    const int n = lane & 31, g2 = lane >> 5;

    const int rr = min(r0 + n, r1 - 1);
    int src = g.a_rows ? g.a_rows[rr] : rr;
    src = src < 0 ? 0 : (src >= g.a_rows_limit ? g.a_rows_limit - 1 : src);
    const uint8_t* pa = static_cast<const uint8_t*>(g.a) + size_t(src) * K + 16 * g2;
    const uint8_t* psa = g.ascale + size_t(src) * (K / 32);

    // the wavefront's weight rows: tile t, tile rows trow[h], weight rows wrow[h]
    const int sc = min(set, nsets - 1);  // idle wavefronts stay in bounds
    const int c0 = sc * (KIND == kGateUp ? 32 : 64);
    int t, trow[NG], wrow[NG];
    if (KIND == kGateUp) {
        t = c0 >> 7;
        trow[0] = ((c0 >> 6) & 1) * 128 + (c0 & 63) + n;  // gate row; the up row is 64 below
        trow[1] = trow[0] + 64;
        wrow[0] = c0 + n;
        wrow[1] = g.F + c0 + n;
    } else {
        t = c0 >> 8;
        trow[0] = (c0 & 255) + n;
        trow[1] = trow[0] + 32;
        wrow[0] = c0 + n;
        wrow[1] = c0 + 32 + n;
    }
    const int ntiles = (KIND == kGateUp) ? g.F / 128 : g.N / 256;
    const int Nw = (KIND == kGateUp) ? 2 * g.F : g.N;
    const uint8_t* wt = static_cast<const uint8_t*>(g.w) + (size_t(e) * ntiles + t) * nst * SBLK;
    // packed: offsets of the lane's chunks inside a (tile, stage) block, SBLK bytes per stage;
    // row-major: the lane's chunks of its own weight rows, 64 (fp8) or 32 (fp4) bytes per stage
    size_t off0[NG], off1[NG];
    const uint8_t* psw[NG];
    const size_t wst = g.wpacked ? SBLK : BCH * 16;
    if (!g.wpacked) wt = static_cast<const uint8_t*>(g.w);
#pragma unroll
    for (int h = 0; h < NG; ++h) {
        const int r = trow[h];
        const size_t rm = (size_t(e) * Nw + wrow[h]) * (BF4 ? K / 2 : K);  // row-major row start
        if (BF4) {
            off0[h] = g.wpacked ? size_t(r * 32 + ((g2 ^ ((r >> 2) & 1)) * 16)) : rm + 16 * g2;
            off1[h] = 0;
        } else {
            off0[h] = g.wpacked ? size_t(r * 64 + ((g2 ^ ((r >> 1) & 3)) * 16)) : rm + 16 * g2;
            off1[h] = g.wpacked ? size_t(r * 64 + (((g2 + 2) ^ ((r >> 1) & 3)) * 16)) : rm + 16 * (g2 + 2);
        }
        psw[h] = g.wscale + (size_t(e) * Nw + wrow[h]) * (K / 32);
    }

    f32x16_t acc[NG];
#pragma unroll
    for (int h = 0; h < NG; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;
    const int per = nst / SPLITK;  // a multiple of 8 (launcher)
    const int s0 = kp * per, s1 = s0 + per;

    typedef __attribute__((ext_vector_type(4))) int i32x4_t;
    auto ld16 = [](const void* p) __attribute__((always_inline)) {
        return __builtin_bit_cast(i32x4_t, *reinterpret_cast<const uint4*>(p));
    };
    // weight loads: the non-temporal hint for fp4 codes only (forward medians, bit-identical,
    // MXFP4 decode T=64 267.3 -> 248.6 us; MXFP8 465.9 -> 512.5 us, so fp8 codes keep the
    // default)
    auto ldw = [](const void* p) __attribute__((always_inline)) {
        if constexpr (BF4)
            return __builtin_bit_cast(i32x4_t, load_nt16(p));
        else
            return __builtin_bit_cast(i32x4_t, *reinterpret_cast<const uint4*>(p));
    };
    struct Stg {
        i32x8_t a;
        i32x4_t b0[NG], b1[NG];
    };
    struct Scl {
        uint4 a, w[NG];
    };
    auto load = [&](Stg& x, int st) __attribute__((always_inline)) {
        const i32x4_t lo = ld16(pa + 64 * st), hi = ld16(pa + 64 * st + 32);
        x.a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const uint8_t* blk = wt + size_t(st) * wst;
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            x.b0[h] = ldw(blk + off0[h]);
            if (!BF4) x.b1[h] = ldw(blk + off1[h]);
        }
    };
    auto sload = [&](Scl& c, int chunk) __attribute__((always_inline)) {
        c.a = *reinterpret_cast<const uint4*>(psa + 16 * chunk);
#pragma unroll
        for (int h = 0; h < NG; ++h) c.w[h] = *reinterpret_cast<const uint4*>(psw[h] + 16 * chunk);
    };
    // stage 2 p + odd of a chunk: scale byte 4 p + 2 odd + g2 of the chunk's 16, i.e. word p,
    // bit offset (2 odd + g2) * 8 (p and odd are compile-time constants below)
    auto word = [](const uint4& v, int p) __attribute__((always_inline)) {
        return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
    };
    auto compute = [&](const Stg& x, const Scl& c, int p, int odd) __attribute__((always_inline)) {
        const int sh = (2 * odd + g2) * 8;
        const int as = int((word(c.a, p) >> sh) & 0xffu);
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            const i32x4_t z = {0, 0, 0, 0};
            const i32x8_t b = __builtin_shufflevector(x.b0[h], BF4 ? z : x.b1[h], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[h] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                x.a, b, acc[h], 0, BF4 ? 4 : 0, 0, as, 0, int((word(c.w[h], p) >> sh) & 0xffu));
        }
    };
    if (live && per > 0) {
        const int c0s = s0 >> 3, clast = (s1 - 1) >> 3;
        Stg x0, x1;
        Scl cur, nxt;
        sload(cur, c0s);
        sload(nxt, min(c0s + 1, clast));
        load(x0, s0);
        load(x1, s0 + 1);
        // whole chunks of 8 stages (per is a multiple of 8), two stages in flight; the last
        // pair's loads re-read the last stage (cache hits), which keeps one loop exit and one
        // set of accumulators
        for (int ch = c0s; ch <= clast; ++ch) {
            if (ch != c0s) {
                cur = nxt;
                sload(nxt, min(ch + 1, clast));
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int st = ch * 8 + 2 * p;
                compute(x0, cur, p, 0);
                load(x0, min(st + 2, s1 - 1));
                compute(x1, cur, p, 1);
                load(x1, min(st + 3, s1 - 1));
            }
        }
    }

    if constexpr (SPLITK > 1) {
#pragma unroll
        for (int h = 0; h < NG; ++h) red[wave][h][lane] = acc[h];
        __syncthreads();
        if (kp != 0) return;
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            acc[h] = red[wave][h][lane];
#pragma unroll
            for (int p = 1; p < SPLITK; ++p) acc[h] += red[wave + p][h][lane];
        }
    }
    if (!live) return;

    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = r0 + 8 * (i / 4) + 4 * g2 + (i % 4);
        if (row >= r1) continue;
        if (KIND == kGateUp) {
            out[size_t(row) * g.F + c0 + n] = (uint16_t)bf16_rne(silu_mul(acc[0][i], acc[1][i]));
        } else {
#pragma unroll
            for (int h = 0; h < NG; ++h) out[size_t(row) * g.N + c0 + 32 * h + n] = (uint16_t)bf16_rne(acc[h][i]);
        }
    }
}

// Prefill blocks: (row tile, column tile) pairs, a multiple of 8 so that every XCD walks the
// same number.  Decode blocks: (row tile, group pairs of four wavefronts), K split over up to
// four wavefronts for small grids.  MXFP8 weights (kWMXFP8) and MXFP4 weights (kWMXFP4), both
// with MXFP8 activations.
hipError_t launch_gemm_mxfp8(const GemmArgs& g, int family, int max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    if (family == kFamDecode) {
        const bool up = g.kind == kGateUp, f4 = g.wfmt == kWMXFP4;
        const int nsets = up ? g.F / 32 : g.N / 64, nst = g.K / 64;  // K % 512 == 0
        // K split until the worst-case tile count gives 32768 wavefronts (measured against 4096:
        // MXFP4 decode T=64 300.5 -> 273.5 us per forward, MXFP8 T=16 350.2 -> 326.0 us)
        int split = 1;
        while (split < 4 && long(max_tiles) * nsets * split < 32768 && nst % (8 * split * 2) == 0) split *= 2;
        const int wpb = 4 / split;
        const dim3 grid(max_tiles * ((nsets + wpb - 1) / wpb)), block(256);
#define MOE_MXD(KD, F4, SK) hipLaunchKernelGGL((gemm_decode_mx_kernel<KD, F4, SK>), grid, block, 0, s, g)
#define MOE_MXD_SPLIT(KD, F4) \
    do { if (split == 1) MOE_MXD(KD, F4, 1); else if (split == 2) MOE_MXD(KD, F4, 2); else MOE_MXD(KD, F4, 4); } while (0)
        if (up) { if (f4) MOE_MXD_SPLIT(kGateUp, 1); else MOE_MXD_SPLIT(kGateUp, 0); }
        else    { if (f4) MOE_MXD_SPLIT(kDown, 1);   else MOE_MXD_SPLIT(kDown, 0); }
#undef MOE_MXD_SPLIT
#undef MOE_MXD
        return hipGetLastError();
    }
    const int ncols = g.kind == kGateUp ? g.F / 128 : (g.N + 255) / 256;
    const dim3 grid(((max_tiles * ncols + 7) / 8) * 8);
    const bool f4 = g.wfmt == kWMXFP4;
    if (g.kind == kGateUp) {
        if (f4) hipLaunchKernelGGL((gemm_prefill_mxfp8_kernel<kGateUp, 1>), grid, dim3(512), 0, s, g);
        else hipLaunchKernelGGL((gemm_prefill_mxfp8_kernel<kGateUp, 0>), grid, dim3(512), 0, s, g);
    } else {
        if (f4) hipLaunchKernelGGL((gemm_prefill_mxfp8_kernel<kDown, 1>), grid, dim3(512), 0, s, g);
        else hipLaunchKernelGGL((gemm_prefill_mxfp8_kernel<kDown, 0>), grid, dim3(512), 0, s, g);
    }
    return hipGetLastError();
}

}  // namespace moe
