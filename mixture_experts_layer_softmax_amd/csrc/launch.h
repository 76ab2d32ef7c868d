// launch.h -- internal launchers of the MoE kernels (host side, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace moe {

struct RouteArgs {
    const void* x;      // [T,H] fp32 or bf16
    const void* wr;     // [E,H]
    const float* bias;  // [E] or null
    float* logits;      // [T,E]
    int T, H, E;
    bool bf16;
};

struct DispatchArgs {
    const int32_t* ids;  // [T,k]
    int T, k, E;
    int32_t* hist;       // [nchunks,E]
    int32_t* base;       // [nchunks,E]
    int32_t* counts;     // [E] or null
    int32_t* offsets;    // [E+1]
    int32_t* sorted_token;
    int32_t* inv_perm;
    Tile* tiles1;        // tile list for GEMM1 (or null)
    int* tile_count1;
    int bm1;
    Tile* tiles2;
    int* tile_count2;
    int bm2;
    int tile_cap;        // capacity of each tile list
    int ebegin, eend;    // held experts [ebegin, eend): only their assignments are dispatched
};

enum GemmKind { kGateUp = 0, kDown = 1 };
enum WeightFmt { kWF32 = 0, kWBF16 = 1, kWNVFP4 = 2, kWMXFP8 = 3, kWMXFP4 = 4 };
enum GemmFamily { kFamF32 = 0, kFamPrefill = 1, kFamDecode = 2 };

struct GemmArgs {
    const void* a;          // activations: bf16 or fp32, row length K
    const int32_t* a_rows;  // gather map (dispatched row -> row of a) or null
    int a_rows_limit;       // rows in a (gathered indices are clamped below it)
    const Tile* tiles;
    const int* tile_count;
    const void* w;          // [E, Nw, K] values or [E, Nw, K/2] packed nibbles
    const uint8_t* wscale;  // [E, Nw, K/16] (NVFP4) or [E, Nw, K/32] (MXFP8)
    int wpacked;            // weights (NVFP4: bytes and scales) in the PACKED layout (tile/stage
                            // blocks); 0: row-major
    int hid_packed;         // bf16 prefill inside moe_forward: gate/up writes hid and down reads
                            // it as [tile][stage] blocks of 256 rows x 64 bytes (the weights' image)
    const uint8_t* ascale;  // MXFP8: E8M0 scales of `a` [rows, K/32] (a holds E4M3 codes)
    const float* gscale;    // [E] or null (NVFP4)
    void* out;              // [A, N]
    int K, N, F;            // reduction length, output columns, gate/up split
    int kind;               // GemmKind
    int wfmt;               // WeightFmt
};

// Single-launch decode (decode_fused.hip): batches of at most kFusedMaxTokens tokens over at
// most kFusedMaxExperts experts run as one cooperative launch of at most kFusedMaxBlocks
// blocks of 256 threads.
constexpr int kFusedMaxTokens = 16;
constexpr int kFusedMaxExperts = 256;
constexpr int kFusedMaxBlocks = 1024;
constexpr int kFusedMaxRows = kFusedMaxTokens * kMaxTopK;
constexpr int kFusedTileCap = kFusedMaxRows / 16 + kFusedMaxExperts + 1;  // 16-row decode tiles

// Grid-barrier words of the single-launch decode kernel (at the start of its workspace).
struct GridSync {
    uint64_t seq;         // calls made so far on this workspace (any initial value)
    uint32_t timeouts;    // barrier waits that gave up (cumulative; zero it to watch a call)
    uint32_t pad0;
    uint64_t go;          // last barrier value released by block 0
    uint64_t pad1[5];
    uint64_t arrive[kFusedMaxBlocks];  // last barrier value each block reached
};
static_assert(sizeof(GridSync) == 8256, "MOE_PROBE_SYNC_BYTES in moe_probe.h");

struct FusedArgs {
    const void* x;        // [T,H] bf16
    const void* wr;       // [E,H] bf16
    const float* bias;    // [E] or null
    float* logits;        // [T,E] (workspace)
    int T, H, E, k, renorm, eb, ee;
    int32_t* ids;         // routing outputs (each may be null)
    float* tw;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_token;
    int32_t* inv_perm;
    GemmArgs g1, g2;      // gate/up (a = x, out = hid) and down (a = hid, out = y_perm); their
                          // tile lists and gather maps are set inside the kernel
    void* y_perm;         // [A,H] bf16 (workspace)
    void* y;              // [T,H] bf16
    GridSync* sync;
    unsigned spin_limit;  // polls before a barrier wait gives up
};

int gemm_tile_rows(int family, int wfmt, int ffn);
// One cooperative launch of decode_fused_kernel for a bf16 (nv4 = 0) or packed NVFP4 (nv4 = 1)
// layer; `blocks_per_cu` caps the persistent grid (0: as many as fit).
hipError_t launch_decode_fused(const FusedArgs& a, bool nv4, int blocks_per_cu, hipStream_t s);
hipError_t launch_router_logits(const RouteArgs& a, hipStream_t s);
// Screened routing (bf16 activations, renormalised weights): approximate logits on the matrix
// cores, canonical logits only for the experts that can be selected, -inf for the rest (route.hip
// states why the selection equals the full canonical one), then the top-k selection into ids
// [T,k] and tw [T,k].  Scratch: logits [T,E], mpart [KS,T,E] (partial approximate logits over
// KS slices of K, KS = screen_k_split(T, H, E)) and wn2 [KS,E] (squared router-row norms).
struct ScreenConst {
    float gamma;     // relative bound of the two dot products, the slice sum and the bias addition
    float flush;     // 2^-126 H: terms flushed to zero
    float norm_abs;  // sqrt(H) 2^-63: norm lost to squares that underflow
};
ScreenConst screen_const(int H, int KS);
int screen_k_split(int T, int H, int E);
hipError_t launch_router_screened(const RouteArgs& a, float* mpart, float* wn2, int k, int32_t* ids,
                                  float* tw, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                       float* w, hipStream_t s);
hipError_t launch_dispatch(const DispatchArgs& d, hipStream_t s);
// T <= kChunkTokens: top-k of the logits (ids/weights into tw_ids/tw) and the dispatch of
// d in one single-block launch (d.ids, d.hist and d.base are not used).
hipError_t launch_select_dispatch_small(const float* logits, int renorm, int32_t* tw_ids, float* tw,
                                        const DispatchArgs& d, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int value, hipStream_t s);
hipError_t launch_tiles_from_offsets(const int32_t* offsets, int E, int eb, int ee, int A, int bm, Tile* tiles,
                                     int* tile_count, int cap, hipStream_t s);
// MXFP8 (mx.hip): bf16 rows [rows, K] -> E4M3 codes [rows, K] + E8M0 scales [rows, K/32];
// the grouped GEMM on block-scaled fp8 MFMA (prefill: 256-row tiles; decode: 32-row tiles).
hipError_t launch_mx_quantize(const void* in, long rows, int K, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_gemm_mxfp8(const GemmArgs& g, int family, int max_tiles, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* sorted_token, void* x_perm, int A,
                              int T, int row_bytes, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, int family, int max_tiles, hipStream_t s);
// esize: bytes per element (2: bf16, 1: MXFP8 codes)
hipError_t launch_pack_bf16(const void* src, void* dst, int kind, int E, int F, int H, int esize,
                            hipStream_t s);
// MXFP4 codes (two E2M1 per byte) into 8 KiB stage blocks
// NVFP4 PACKED layout: bytes (16 per row and 32-element stage) or E4M3 scales (4 per row and
// stage pair) of w13 (kind 0) or w2 (kind 1) into [expert][tile][stage] blocks of 256 rows.
hipError_t launch_pack_nvfp4(const void* src, void* dst, int kind, int E, int F, int H, bool scales,
                             hipStream_t s);
hipError_t launch_pack_fp4(const void* src, void* dst, int kind, int E, int F, int H, hipStream_t s);
hipError_t launch_combine(const void* y_perm, const int32_t* inv_perm, const float* w, void* y,
                          int T, int k, int H, int A, bool bf16, hipStream_t s);

}  // namespace moe
