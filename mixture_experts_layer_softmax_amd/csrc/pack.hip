// pack.hip -- one-time rewrite of bf16, MXFP8 (E4M3 codes), MXFP4 (E2M1 codes) or NVFP4 (bytes
// and E4M3 scales) expert weights into the packed layouts of moe.h.  For bf16 and MXFP8 a stage
// is 64 bytes of a row (32 bf16 or 64 fp8 elements; pack_bf16_kernel moves 16-byte chunks and
// counts a row in 2-byte units); for MXFP4 a stage of 64 elements is 32 bytes
// (pack_fp4_kernel); for NVFP4 a stage of 32 elements is 16 bytes (pack_nvfp4_kernel).
//
// Each (expert, 256-row tile, 32-element stage) block becomes the byte image of an LDS slot of
// the grouped GEMMs (rows 64 bytes, chunk c of row r in slot c ^ ((r >> 1) & 3)), so that the
// kernels stream every stage of a weight tile as one contiguous 16 KiB read and 16 rows of a
// stage as one contiguous 1 KiB.  Row-strided reads of the same bytes (256 rows, 8 KiB apart,
// 64 bytes each) reach about three quarters of the HBM bandwidth of contiguous ones on MI355X.
#include "device.h"
#include "launch.h"

namespace moe {

// One thread per 16-byte destination chunk (grid-stride).  kind 0: w13 (gate/up tiles of 128
// hid columns), kind 1: w2 (tiles of 256 output rows); esize = bytes per element (2 or 1).
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int kind, int E,
                                                        int F, int H, int esize) {
    const int K = (kind == 0 ? H : F) * esize / 2;   // 2-byte units per weight row
    const int Nw = kind == 0 ? 2 * F : H;            // weight rows per expert
    const int ntiles = kind == 0 ? F / 128 : H / 256;
    const int nst = K / 32;
    const long total = long(E) * ntiles * nst * 1024;
    for (long d = long(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += long(gridDim.x) * blockDim.x) {
        const long blk = d >> 10;
        const int w = int(d & 1023), r = w >> 2, slot = w & 3;
        const int c = slot ^ ((r >> 1) & 3);
        const int st = int(blk % nst);
        const long et = blk / nst;
        const int t = int(et % ntiles), e = int(et / ntiles);
        int wrow;
        if (kind == 0) {
            const int q = r & 127;
            const int f = 128 * t + 64 * (r >> 7) + (q & 63);
            wrow = q < 64 ? f : F + f;
        } else {
            wrow = 256 * t + r;
        }
        dst[d] = src[((long(e) * Nw + wrow) * K + st * 32 + c * 8) / 8];
    }
}

// MXFP4 codes (two E2M1 per byte, K/2 bytes per row): one thread per 16-byte destination chunk
// of 8 KiB (expert, tile, stage) blocks: 256 rows x 2 chunks, chunk c of row r in slot
// c ^ ((r >> 2) & 1); tiles and row order as above.
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint4* __restrict__ src,
                                                       uint4* __restrict__ dst, int kind, int E,
                                                       int F, int H) {
    const int Kb = (kind == 0 ? H : F) / 2;          // bytes per weight row
    const int Nw = kind == 0 ? 2 * F : H;
    const int ntiles = kind == 0 ? F / 128 : H / 256;
    const int nst = Kb / 32;
    const long total = long(E) * ntiles * nst * 512;
    for (long d = long(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += long(gridDim.x) * blockDim.x) {
        const long blk = d >> 9;
        const int w = int(d & 511), r = w >> 1, slot = w & 1;
        const int c = slot ^ ((r >> 2) & 1);
        const int st = int(blk % nst);
        const long et = blk / nst;
        const int t = int(et % ntiles), e = int(et / ntiles);
        int wrow;
        if (kind == 0) {
            const int q = r & 127;
            const int f = 128 * t + 64 * (r >> 7) + (q & 63);
            wrow = q < 64 ? f : F + f;
        } else {
            wrow = 256 * t + r;
        }
        dst[d] = src[((long(e) * Nw + wrow) * Kb + st * 32 + c * 16) / 16];
    }
}

// NVFP4 bytes (U = 16-byte unit: one 32-element stage of a row) or E4M3 scales (U = 4-byte
// unit: the scales of one stage pair of a row): one thread per destination unit of
// [expert][tile][stage][256 rows] blocks; tiles and row order as above, no slots.  A row holds
// `upr` units in either case (K/32 stages of 16 bytes, K/64 stage pairs of 4 scale bytes).
template <typename U>
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(const U* __restrict__ src, U* __restrict__ dst,
                                                         int kind, int E, int F, int H, int upr) {
    const int Nw = kind == 0 ? 2 * F : H;
    const int ntiles = kind == 0 ? F / 128 : H / 256;
    const long total = long(E) * ntiles * upr * 256;
    for (long d = long(blockIdx.x) * blockDim.x + threadIdx.x; d < total; d += long(gridDim.x) * blockDim.x) {
        const long blk = d >> 8;
        const int r = int(d & 255);
        const int st = int(blk % upr);
        const long et = blk / upr;
        const int t = int(et % ntiles), e = int(et / ntiles);
        int wrow;
        if (kind == 0) {
            const int q = r & 127;
            const int f = 128 * t + 64 * (r >> 7) + (q & 63);
            wrow = q < 64 ? f : F + f;
        } else {
            wrow = 256 * t + r;
        }
        dst[d] = src[(long(e) * Nw + wrow) * upr + st];
    }
}

hipError_t launch_pack_nvfp4(const void* src, void* dst, int kind, int E, int F, int H, bool scales,
                             hipStream_t s) {
    const int K = kind == 0 ? H : F;
    if (scales)
        hipLaunchKernelGGL(pack_nvfp4_kernel<uint32_t>, dim3(8192), dim3(256), 0, s,
                           static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), kind, E, F, H, K / 64);
    else
        hipLaunchKernelGGL(pack_nvfp4_kernel<uint4>, dim3(8192), dim3(256), 0, s,
                           static_cast<const uint4*>(src), static_cast<uint4*>(dst), kind, E, F, H, K / 32);
    return hipGetLastError();
}

hipError_t launch_pack_fp4(const void* src, void* dst, int kind, int E, int F, int H, hipStream_t s) {
    hipLaunchKernelGGL(pack_fp4_kernel, dim3(8192), dim3(256), 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), kind, E, F, H);
    return hipGetLastError();
}

hipError_t launch_pack_bf16(const void* src, void* dst, int kind, int E, int F, int H, int esize,
                            hipStream_t s) {
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(8192), dim3(256), 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), kind, E, F, H, esize);
    return hipGetLastError();
}

}  // namespace moe
