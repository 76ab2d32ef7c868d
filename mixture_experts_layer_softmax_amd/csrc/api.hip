// api.hip -- the C ABI of include/moe.h: validation, workspace layout, kernel policy.
//
// Host-side launcher in the spirit of the pages' dispatch() host code ("CuTeDSL at
// Perplexity", sections Prefill and decode specialization and Grid synchronization): the
// problem size picks the kernel family (few rows per expert -> weight-streaming decode tiles,
// many -> large MFMA tiles), and every data-dependent decision after routing stays on the
// device (tile lists), so nothing is read back and no call synchronises.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "../../include/moe_probe.h"
#include "launch.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
    size_t sync, logits, mpart, wn2, ids, w, hist, base, counts, offsets, sorted, inv, tiles1, tiles2,
        tcount, hid, yperm, xq, xs, hq, hs, total;
    int family, bm, max_tiles;
};

int act_bytes(const moe_problem& p) { return p.act_dtype == MOE_F32 ? 4 : 2; }

// Held experts [ebegin, eend): all E unless local_experts is set (expert parallelism).
int ebegin(const moe_problem& p) { return p.local_experts ? p.expert_begin : 0; }
int eend(const moe_problem& p) { return p.local_experts ? p.expert_begin + p.local_experts : p.num_experts; }

int wfmt_of(const moe_problem& p) {
    switch (p.w_dtype) {
        case MOE_F32: return kWF32;
        case MOE_BF16: return kWBF16;
        case MOE_NVFP4: return kWNVFP4;
        case MOE_MXFP8: return kWMXFP8;
        default: return kWMXFP4;
    }
}

bool is_mx(const moe_problem& p) { return p.w_dtype == MOE_MXFP8 || p.w_dtype == MOE_MXFP4; }

int family_of(const moe_problem& p) {
    if (p.act_dtype == MOE_F32) return kFamF32;
    int path = p.path;
    if (path == MOE_PATH_AUTO) {
        const long A = long(p.num_tokens) * p.top_k;
        path = (A < 16L * p.num_experts) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
    }
    return (path == MOE_PATH_DECODE || path == MOE_PATH_DECODE_FUSED) ? kFamDecode : kFamPrefill;
}

moe_status check_problem(const moe_problem* p) {
    if (!p) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens < 0 || p->hidden <= 0 || p->ffn <= 0 || p->num_experts < 1 ||
        p->num_experts > kMaxExperts || p->top_k < 1 || p->top_k > kMaxTopK ||
        p->top_k > p->num_experts || (p->renormalize != 0 && p->renormalize != 1) ||
        p->path < MOE_PATH_AUTO || p->path > MOE_PATH_DECODE_FUSED)
        return MOE_ERR_INVALID_ARGUMENT;
    if (p->expert_begin < 0 || p->local_experts < 0 ||
        long(p->expert_begin) + p->local_experts > p->num_experts ||
        (p->local_experts == 0 && p->expert_begin != 0))
        return MOE_ERR_INVALID_ARGUMENT;
    if (p->act_dtype != MOE_F32 && p->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (p->w_dtype < MOE_F32 || p->w_dtype > MOE_MXFP4) return MOE_ERR_INVALID_ARGUMENT;
    if (p->hidden % 64 || p->ffn % 64) return MOE_ERR_UNSUPPORTED;
    if (p->w_dtype == MOE_BF16 && (p->hidden % 256 || p->ffn % 128)) return MOE_ERR_UNSUPPORTED;
    // MXFP8: 256-row tiles, and E8M0 scales loaded 16 per row (8 stages of 64) at a time
    if (is_mx(*p) && (p->hidden % 512 || p->ffn % 512)) return MOE_ERR_UNSUPPORTED;
    if (is_mx(*p) && p->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->act_dtype == MOE_F32 && p->w_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (p->act_dtype == MOE_BF16 && p->w_dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (long(p->num_tokens) * p->top_k > (1L << 30) || long(p->num_tokens) * p->hidden > (1L << 40))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// moe_forward on the bf16 prefill kernels hands hid from the gate/up GEMM to the down GEMM in
// the packed tile image, so that the down GEMM reads each stage of a row tile as one contiguous
// 16 KiB, like its weights, instead of 256 rows of 64 bytes each
bool hid_packed(const moe_problem& p) { return family_of(p) == kFamPrefill && p.w_dtype == MOE_BF16; }

// Screened routing (route.hip) for large bf16 batches with renormalised weights: the same ids
// and weights as the full canonical router.  Below 256 tokens the full router is as fast (it
// is latency-bound there), and the full softmax (renormalize = 0) needs every canonical logit.
bool screened_routing(const moe_problem& p) {
    return p.act_dtype == MOE_BF16 && p.renormalize && p.num_tokens >= 256 && p.num_experts >= 16;
}

Layout layout(const moe_problem& p) {
    Layout L{};
    const size_t T = p.num_tokens, E = p.num_experts, k = p.top_k, H = p.hidden, F = p.ffn;
    const size_t A = T * k;
    const size_t nch = (T + kChunkTokens - 1) / kChunkTokens;
    L.family = family_of(p);
    L.bm = gemm_tile_rows(L.family, wfmt_of(p), p.ffn);
    L.max_tiles = int((A + L.bm - 1) / L.bm + (A < E ? A : E) + 1);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += up(bytes > 0 ? bytes : 1); return r; };
    L.sync = take(sizeof(GridSync));  // grid-barrier words of the single-launch decode kernel
    L.logits = take(T * E * 4);
    // screened routing: partial approximate logits and squared router-row norms per K slice
    const size_t ks = screened_routing(p) ? size_t(screen_k_split(p.num_tokens, p.hidden, p.num_experts)) : 0;
    L.mpart = take(ks * T * E * 4);
    L.wn2 = take(ks * E * 4);
    L.ids = take(A * 4);
    L.w = take(A * 4);
    L.hist = take(nch * E * 4);
    L.base = take(nch * E * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.sorted = take(A * 4);
    L.inv = take(A * 4);
    L.tiles1 = take(size_t(L.max_tiles) * sizeof(Tile));
    L.tiles2 = take(size_t(L.max_tiles) * sizeof(Tile));
    L.tcount = take(32 * sizeof(int));  // tile counts; [8..16]: the prefill list's XCD ranges
    // bf16 prefill forward: hid in the packed tile image (every tile a full 256 rows)
    L.hid = take(hid_packed(p) ? size_t(L.max_tiles) * 256 * F * 2 : A * F * act_bytes(p));
    L.yperm = take(A * H * act_bytes(p));
    const bool mx = is_mx(p);  // MXFP8 copies of the GEMM inputs (codes + scales)
    L.xq = take(mx ? A * H : 0);
    L.xs = take(mx ? A * H / 32 : 0);
    L.hq = take(mx ? A * F : 0);
    L.hs = take(mx ? A * F / 32 : 0);
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(const moe_problem& p, void* ws, size_t bytes) {
    if (!ws || !aligned(ws)) return MOE_ERR_INVALID_ARGUMENT;
    if (bytes < layout(p).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return MOE_OK;
}

// NVFP4 PACKED: whole 256-row tiles of w13 (128 hid columns) and w2, whole stage pairs of K
bool nvfp4_packable(const moe_problem& p) { return p.hidden % 256 == 0 && p.ffn % 128 == 0; }

moe_status check_weights(const moe_problem& p, const moe_expert_weights* w) {
    if (!w || !w->w13 || !w->w2 || !aligned(w->w13) || !aligned(w->w2)) return MOE_ERR_INVALID_ARGUMENT;
    // every format is accepted row-major; bf16, MX and NVFP4 weights also in the PACKED layout
    // (fp32 weights are row-major only)
    if (w->layout != MOE_LAYOUT_ROW_MAJOR && w->layout != MOE_LAYOUT_PACKED) return MOE_ERR_INVALID_ARGUMENT;
    if (w->layout == MOE_LAYOUT_PACKED && p.w_dtype == MOE_F32) return MOE_ERR_INVALID_ARGUMENT;
    if (w->layout == MOE_LAYOUT_PACKED && p.w_dtype == MOE_NVFP4 && !nvfp4_packable(p)) return MOE_ERR_UNSUPPORTED;
    if (is_mx(p)) {
        if (!w->w13_scale || !w->w2_scale || !aligned(w->w13_scale) || !aligned(w->w2_scale))
            return MOE_ERR_INVALID_ARGUMENT;
    }
    if (p.w_dtype == MOE_NVFP4) {
        if (!w->w13_scale || !w->w2_scale) return MOE_ERR_INVALID_ARGUMENT;
        // the decode kernel reads scales in 2- and 8-byte pieces; like every pointer of the ABI
        // the scale arrays must be 16-byte aligned
        if (!aligned(w->w13_scale) || !aligned(w->w2_scale)) return MOE_ERR_INVALID_ARGUMENT;
        if ((reinterpret_cast<uintptr_t>(w->w13_gscale) & 3u) || (reinterpret_cast<uintptr_t>(w->w2_gscale) & 3u))
            return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// The single-launch decode kernel covers bf16 activations with bf16 weights (either layout) or
// packed NVFP4 weights, up to kFusedMaxTokens tokens over up to kFusedMaxExperts experts, and K
// a multiple of 512 in both GEMMs (its GEMVs split K over four wavefronts of 128-wide blocks).
bool fused_eligible(const moe_problem& p, const moe_expert_weights& w) {
    if (family_of(p) != kFamDecode || p.act_dtype != MOE_BF16) return false;
    if (p.num_tokens > kFusedMaxTokens || p.num_experts > kFusedMaxExperts) return false;
    if (p.hidden % 512 || p.ffn % 512) return false;
    return p.w_dtype == MOE_BF16 || (p.w_dtype == MOE_NVFP4 && w.layout == MOE_LAYOUT_PACKED);
}

// MOE_PATH_DECODE_FUSED asks for the single-launch decode kernel; MOE_PATH_AUTO takes it for
// eligible batches where it measured faster than the multi-launch decode path.
bool use_fused(const moe_problem& p, const moe_expert_weights& w) {
    if (!fused_eligible(p, w)) return false;
    return p.path == MOE_PATH_DECODE_FUSED;
}

// Test and measurement hooks of the single-launch decode kernel, read from the environment:
// MOE_FUSED_SPIN_LIMIT (polls before a barrier wait gives up, default 2^20) and
// MOE_FUSED_BLOCKS_PER_CU (cap on the persistent grid, default: as many as fit).
unsigned env_unsigned(const char* name, unsigned dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    char* end = nullptr;
    const unsigned long x = std::strtoul(v, &end, 10);
    return (end && *end == 0 && x <= 0xffffffffUL) ? unsigned(x) : dflt;
}

// Scratch of moe_forward_static: one array per GPU, in the library's device data, held until the
// process ends.  Host code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept per device.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

moe_status static_scratch(void** out) {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) return MOE_ERR_DEVICE;
    if (d < 0 || d >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[d], [d] {
        void* ptr = nullptr;
        g_scratch_err[d] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[d] = ptr;
    });
    if (g_scratch_err[d] != hipSuccess || !g_scratch_ptr[d]) return MOE_ERR_DEVICE;
    *out = g_scratch_ptr[d];
    return MOE_OK;
}

#define MOE_TRY(x)                           \
    do {                                     \
        moe_status _s = (x);                 \
        if (_s != MOE_OK) return _s;         \
    } while (0)

moe_status run_route(const moe_problem& p, const void* x, const void* wr, const float* bias,
                     int32_t* ids, float* w, const Layout& L, void* ws, hipStream_t s) {
    RouteArgs r{x, wr, bias, at<float>(ws, L.logits), p.num_tokens, p.hidden, p.num_experts,
                p.act_dtype == MOE_BF16};
    if (screened_routing(p))
        return dev(launch_router_screened(r, at<float>(ws, L.mpart), at<float>(ws, L.wn2), p.top_k, ids, w, s));
    MOE_TRY(dev(launch_router_logits(r, s)));
    return dev(launch_topk(r.logits, p.num_tokens, p.num_experts, p.top_k, p.renormalize, ids, w, s));
}

GemmArgs gemm_args(const moe_problem& p, int kind, const void* a, const int32_t* a_rows,
                   const Tile* tiles, const int* tcount, const moe_expert_weights& w, void* out) {
    GemmArgs g{};
    g.a = a;
    g.a_rows = a_rows;
    g.tiles = tiles;
    g.tile_count = tcount;
    g.out = out;
    g.F = p.ffn;
    g.kind = kind;
    g.wfmt = wfmt_of(p);
    g.wpacked = w.layout == MOE_LAYOUT_PACKED;
    const int A = p.num_tokens * p.top_k;
    if (kind == kGateUp) {
        g.K = p.hidden;
        g.N = p.ffn;
        g.w = w.w13;
        g.wscale = w.w13_scale;
        g.gscale = w.w13_gscale;
        g.a_rows_limit = a_rows ? p.num_tokens : A;
    } else {
        g.K = p.ffn;
        g.N = p.hidden;
        g.w = w.w2;
        g.wscale = w.w2_scale;
        g.gscale = w.w2_gscale;
        g.a_rows_limit = A;
    }
    return g;
}

// MXFP8: quantize the GEMM's bf16 input rows (g.a_rows_limit of them) to E4M3 codes + E8M0
// scales in the workspace and point the GEMM at them.  Other formats: nothing to do.
moe_status mx_input(const moe_problem& p, GemmArgs& g, void* ws, const Layout& L, hipStream_t s) {
    if (!is_mx(p)) return MOE_OK;
    const bool up = g.kind == kGateUp;
    uint8_t* codes = at<uint8_t>(ws, up ? L.xq : L.hq);
    uint8_t* scales = at<uint8_t>(ws, up ? L.xs : L.hs);
    MOE_TRY(dev(launch_mx_quantize(g.a, g.a_rows_limit, g.K, codes, scales, s)));
    g.a = codes;
    g.ascale = scales;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_DEVICE: return "device error";
        case MOE_ERR_SCRATCH_TOO_SMALL: return "problem needs more scratch than the static scratch buffer holds";
    }
    return "unknown status";
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
    MOE_TRY(check_problem(p));
    if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
    *bytes = layout(*p).total;
    return MOE_OK;
}

moe_status moe_packed_weights_size(const moe_problem* p, size_t* w13_bytes, size_t* w2_bytes) {
    MOE_TRY(check_problem(p));
    if ((p->w_dtype != MOE_BF16 && p->w_dtype != MOE_NVFP4 && !is_mx(*p)) || !w13_bytes || !w2_bytes)
        return MOE_ERR_INVALID_ARGUMENT;
    if (p->w_dtype == MOE_NVFP4 && !nvfp4_packable(*p)) return MOE_ERR_UNSUPPORTED;
    const size_t E = eend(*p) - ebegin(*p), H = p->hidden, F = p->ffn;  // held experts
    const size_t num = p->w_dtype == MOE_BF16 ? 2 : 1;
    const size_t den = (p->w_dtype == MOE_MXFP4 || p->w_dtype == MOE_NVFP4) ? 2 : 1;
    *w13_bytes = E * 2 * F * H * num / den;
    *w2_bytes = E * H * F * num / den;
    return MOE_OK;
}

moe_status moe_pack_weights(const moe_problem* p, const void* w13, const void* w2, void* w13_packed,
                            void* w2_packed, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->w_dtype != MOE_BF16 && p->w_dtype != MOE_NVFP4 && !is_mx(*p)) return MOE_ERR_INVALID_ARGUMENT;
    if ((w13 == nullptr) != (w13_packed == nullptr) || (w2 == nullptr) != (w2_packed == nullptr))
        return MOE_ERR_INVALID_ARGUMENT;
    for (const void* q : {w13, w2, (const void*)w13_packed, (const void*)w2_packed})
        if (q && !aligned(q)) return MOE_ERR_INVALID_ARGUMENT;
    if ((w13 && w13 == w13_packed) || (w2 && w2 == w2_packed)) return MOE_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int held = eend(*p) - ebegin(*p);
    if (p->w_dtype == MOE_NVFP4) {
        if (!nvfp4_packable(*p)) return MOE_ERR_UNSUPPORTED;
        if (w13) MOE_TRY(dev(launch_pack_nvfp4(w13, w13_packed, 0, held, p->ffn, p->hidden, false, s)));
        if (w2) MOE_TRY(dev(launch_pack_nvfp4(w2, w2_packed, 1, held, p->ffn, p->hidden, false, s)));
        return MOE_OK;
    }
    if (p->w_dtype == MOE_MXFP4) {
        if (p->hidden % 512 || p->ffn % 512) return MOE_ERR_UNSUPPORTED;  // whole 32-byte stages
        if (w13) MOE_TRY(dev(launch_pack_fp4(w13, w13_packed, 0, held, p->ffn, p->hidden, s)));
        if (w2) MOE_TRY(dev(launch_pack_fp4(w2, w2_packed, 1, held, p->ffn, p->hidden, s)));
        return MOE_OK;
    }
    const int es = p->w_dtype == MOE_BF16 ? 2 : 1;
    if (w13) MOE_TRY(dev(launch_pack_bf16(w13, w13_packed, 0, held, p->ffn, p->hidden, es, s)));
    if (w2) MOE_TRY(dev(launch_pack_bf16(w2, w2_packed, 1, held, p->ffn, p->hidden, es, s)));
    return MOE_OK;
}

moe_status moe_pack_scales(const moe_problem* p, const uint8_t* w13_scale, const uint8_t* w2_scale,
                           uint8_t* w13_scale_packed, uint8_t* w2_scale_packed, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->w_dtype != MOE_NVFP4) return MOE_ERR_INVALID_ARGUMENT;
    if ((w13_scale == nullptr) != (w13_scale_packed == nullptr) ||
        (w2_scale == nullptr) != (w2_scale_packed == nullptr))
        return MOE_ERR_INVALID_ARGUMENT;
    for (const void* q : {(const void*)w13_scale, (const void*)w2_scale, (const void*)w13_scale_packed,
                          (const void*)w2_scale_packed})
        if (q && !aligned(q)) return MOE_ERR_INVALID_ARGUMENT;
    if ((w13_scale && w13_scale == w13_scale_packed) || (w2_scale && w2_scale == w2_scale_packed))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!nvfp4_packable(*p)) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int held = eend(*p) - ebegin(*p);
    if (w13_scale)
        MOE_TRY(dev(launch_pack_nvfp4(w13_scale, w13_scale_packed, 0, held, p->ffn, p->hidden, true, s)));
    if (w2_scale)
        MOE_TRY(dev(launch_pack_nvfp4(w2_scale, w2_scale_packed, 1, held, p->ffn, p->hidden, true, s)));
    return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* router_bias, int32_t* topk_ids, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->num_tokens == 0) return MOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w || !aligned(x) || !aligned(w_router) ||
        !aligned(topk_ids) || !aligned(topk_w) || (router_bias && !aligned(router_bias)))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_ws(*p, workspace, workspace_bytes));
    const Layout L = layout(*p);
    return run_route(*p, x, w_router, router_bias, topk_ids, topk_w, L, workspace,
                     static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, const void* x,
                       void* x_perm, void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    if (!counts || !offsets || !aligned(counts) || !aligned(offsets)) return MOE_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->num_tokens == 0) {  // counts and offsets are still defined: all zero
        MOE_TRY(dev(launch_fill_i32(counts, p->num_experts, 0, s)));
        return dev(launch_fill_i32(offsets, p->num_experts + 1, 0, s));
    }
    if (!topk_ids || !sorted_token || !inv_perm || !aligned(topk_ids) || !aligned(sorted_token) ||
        !aligned(inv_perm))
        return MOE_ERR_INVALID_ARGUMENT;
    if ((x == nullptr) != (x_perm == nullptr) || (x && (!aligned(x) || !aligned(x_perm))))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_ws(*p, workspace, workspace_bytes));
    const Layout L = layout(*p);
    DispatchArgs d{topk_ids, p->num_tokens, p->top_k, p->num_experts, at<int32_t>(workspace, L.hist),
                   at<int32_t>(workspace, L.base), counts, offsets, sorted_token, inv_perm,
                   nullptr, nullptr, 0, nullptr, nullptr, 0, L.max_tiles, ebegin(*p), eend(*p)};
    MOE_TRY(dev(launch_dispatch(d, s)));
    if (x)
        MOE_TRY(dev(launch_gather_rows(x, sorted_token, x_perm, p->num_tokens * p->top_k,
                                       p->num_tokens, p->hidden * act_bytes(*p), s)));
    return MOE_OK;
}

moe_status moe_grouped_gemm(const moe_problem* p, moe_gemm_kind kind, const void* a,
                            const int32_t* a_rows, const int32_t* offsets,
                            const moe_expert_weights* w, void* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    if (kind != MOE_GEMM_GATE_UP_SWIGLU && kind != MOE_GEMM_DOWN) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens == 0) return MOE_OK;
    if (!a || !offsets || !out || !aligned(a) || !aligned(offsets) || !aligned(out) ||
        (a_rows && !aligned(a_rows)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (kind == MOE_GEMM_DOWN && a_rows) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_weights(*p, w));
    MOE_TRY(check_ws(*p, workspace, workspace_bytes));
    const Layout L = layout(*p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Tile* tiles = at<Tile>(workspace, L.tiles1);
    int* tcount = at<int>(workspace, L.tcount);
    MOE_TRY(dev(launch_tiles_from_offsets(offsets, p->num_experts, ebegin(*p), eend(*p),
                                          p->num_tokens * p->top_k, L.bm, tiles, tcount,
                                          L.max_tiles, s)));
    GemmArgs g = gemm_args(*p, kind == MOE_GEMM_GATE_UP_SWIGLU ? kGateUp : kDown, a, a_rows, tiles,
                           tcount, *w, out);
    MOE_TRY(mx_input(*p, g, workspace, L, s));
    return dev(launch_gemm(g, L.family, L.max_tiles, s));
}

moe_status moe_probe_grouped_gemm_times(const moe_problem* p, moe_gemm_kind kind, const void* a,
                                        const int32_t* a_rows, const int32_t* offsets,
                                        const moe_expert_weights* w, void* out, void* workspace,
                                        size_t workspace_bytes, const void* flush_buf,
                                        size_t flush_bytes, uint32_t* flush_out, int32_t launches,
                                        float* ms, void* stream) {
    MOE_TRY(check_problem(p));
    if (kind != MOE_GEMM_GATE_UP_SWIGLU && kind != MOE_GEMM_DOWN) return MOE_ERR_INVALID_ARGUMENT;
    if (launches < 1 || launches > 100000 || !ms) return MOE_ERR_INVALID_ARGUMENT;
    if (flush_bytes && (!flush_buf || !flush_out || flush_bytes % 16 || !aligned(flush_buf)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens == 0) {
        for (int i = 0; i < launches; ++i) ms[i] = 0.0f;
        return MOE_OK;
    }
    if (!a || !offsets || !out || !aligned(a) || !aligned(offsets) || !aligned(out) ||
        (a_rows && !aligned(a_rows)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (kind == MOE_GEMM_DOWN && a_rows) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_weights(*p, w));
    MOE_TRY(check_ws(*p, workspace, workspace_bytes));
    const Layout L = layout(*p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Tile* tiles = at<Tile>(workspace, L.tiles1);
    int* tcount = at<int>(workspace, L.tcount);
    MOE_TRY(dev(launch_tiles_from_offsets(offsets, p->num_experts, ebegin(*p), eend(*p),
                                          p->num_tokens * p->top_k, L.bm, tiles, tcount,
                                          L.max_tiles, s)));
    GemmArgs g = gemm_args(*p, kind == MOE_GEMM_GATE_UP_SWIGLU ? kGateUp : kDown, a, a_rows, tiles,
                           tcount, *w, out);
    std::vector<hipEvent_t> ev(2 * size_t(launches), nullptr);
    moe_status st = MOE_OK;
    for (auto& e : ev)
        if (st == MOE_OK && hipEventCreate(&e) != hipSuccess) st = MOE_ERR_DEVICE;
    for (int i = 0; st == MOE_OK && i < launches; ++i) {
        if (flush_bytes) st = moe_probe_read(flush_buf, flush_bytes, flush_out, stream);
        if (st == MOE_OK) st = dev(hipEventRecord(ev[2 * i], s));
        if (st == MOE_OK) st = mx_input(*p, g, workspace, L, s);
        if (st == MOE_OK) st = dev(launch_gemm(g, L.family, L.max_tiles, s));
        if (st == MOE_OK) st = dev(hipEventRecord(ev[2 * i + 1], s));
    }
    if (st == MOE_OK) st = dev(hipStreamSynchronize(s));
    for (int i = 0; st == MOE_OK && i < launches; ++i)
        st = dev(hipEventElapsedTime(&ms[i], ev[2 * i], ev[2 * i + 1]));
    for (auto& e : ev)
        if (e) (void)hipEventDestroy(e);
    return st;
}

moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* inv_perm,
                       const float* topk_w, void* y, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->num_tokens == 0) return MOE_OK;
    if (!y_perm || !inv_perm || !topk_w || !y || !aligned(y_perm) || !aligned(inv_perm) ||
        !aligned(topk_w) || !aligned(y))
        return MOE_ERR_INVALID_ARGUMENT;
    return dev(launch_combine(y_perm, inv_perm, topk_w, y, p->num_tokens, p->top_k, p->hidden,
                              p->num_tokens * p->top_k, p->act_dtype == MOE_BF16,
                              static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              void* stream) {
    if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARGUMENT;
    if (rows == 0) return MOE_OK;
    if (!x || !codes || !scales || !aligned(x) || !aligned(codes)) return MOE_ERR_INVALID_ARGUMENT;
    if (rows > (1L << 40) / K) return MOE_ERR_UNSUPPORTED;
    return dev(launch_mx_quantize(x, rows, K, codes, scales, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router,
                       const float* router_bias, const moe_expert_weights* w, void* y,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_token, int32_t* inv_perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    for (const void* q : {(const void*)topk_ids, (const void*)topk_w, (const void*)counts,
                          (const void*)offsets, (const void*)sorted_token, (const void*)inv_perm})
        if (q && !aligned(q)) return MOE_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->num_tokens == 0) {  // no rows: x, y and the workspace may be empty (NULL)
        if (counts) MOE_TRY(dev(launch_fill_i32(counts, p->num_experts, 0, s)));
        if (offsets) MOE_TRY(dev(launch_fill_i32(offsets, p->num_experts + 1, 0, s)));
        return MOE_OK;
    }
    if (!x || !w_router || !y || !aligned(x) || !aligned(w_router) || !aligned(y) ||
        (router_bias && !aligned(router_bias)))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_weights(*p, w));
    MOE_TRY(check_ws(*p, workspace, workspace_bytes));
    const Layout L = layout(*p);
    int32_t* ids = topk_ids ? topk_ids : at<int32_t>(workspace, L.ids);
    float* tw = topk_w ? topk_w : at<float>(workspace, L.w);
    int32_t* off = offsets ? offsets : at<int32_t>(workspace, L.offsets);
    int32_t* st = sorted_token ? sorted_token : at<int32_t>(workspace, L.sorted);
    int32_t* ip = inv_perm ? inv_perm : at<int32_t>(workspace, L.inv);
    int* tcount = at<int>(workspace, L.tcount);
    Tile* tiles = at<Tile>(workspace, L.tiles1);

    DispatchArgs d{ids, p->num_tokens, p->top_k, p->num_experts, at<int32_t>(workspace, L.hist),
                   at<int32_t>(workspace, L.base), counts, off, st, ip, tiles, tcount, L.bm,
                   nullptr, nullptr, 0, L.max_tiles, ebegin(*p), eend(*p)};
    // up to 32 tokens (four per wavefront of the dispatch block): logits, then selection and
    // dispatch in one single-block launch; larger batches select with one wavefront per token
    // (measured on MI355X: one launch instead of four saves about 5 us at 16 tokens and 4 us for
    // 32 tokens over 8 experts, is neutral at 24-32 tokens over 128 experts, and at 48 and 64
    // tokens the serial selection in one block costs 3-12 us more than it saves)
    if (p->num_tokens <= 4 * (kMaxExperts / kWave)) {
        RouteArgs r{x, w_router, router_bias, at<float>(workspace, L.logits), p->num_tokens, p->hidden,
                    p->num_experts, p->act_dtype == MOE_BF16};
        MOE_TRY(dev(launch_router_logits(r, s)));
        MOE_TRY(dev(launch_select_dispatch_small(r.logits, p->renormalize, ids, tw, d, s)));
    } else {
        MOE_TRY(run_route(*p, x, w_router, router_bias, ids, tw, L, workspace, s));
        MOE_TRY(dev(launch_dispatch(d, s)));
    }
    void* hid = at<void>(workspace, L.hid);
    void* yperm = at<void>(workspace, L.yperm);
    if (p->path == MOE_PATH_DECODE_FUSED && !fused_eligible(*p, *w)) return MOE_ERR_UNSUPPORTED;
    if (use_fused(*p, *w)) {
        // the whole layer in one cooperative launch; routing outputs only where the caller asks
        FusedArgs f{};
        f.x = x;
        f.wr = w_router;
        f.bias = router_bias;
        f.logits = at<float>(workspace, L.logits);
        f.T = p->num_tokens;
        f.H = p->hidden;
        f.E = p->num_experts;
        f.k = p->top_k;
        f.renorm = p->renormalize;
        f.eb = ebegin(*p);
        f.ee = eend(*p);
        f.ids = topk_ids;
        f.tw = topk_w;
        f.counts = counts;
        f.offsets = offsets;
        f.sorted_token = sorted_token;
        f.inv_perm = inv_perm;
        f.g1 = gemm_args(*p, kGateUp, x, nullptr, nullptr, nullptr, *w, hid);
        f.g1.a_rows_limit = p->num_tokens;  // the kernel gathers token rows through its dispatch
        f.g2 = gemm_args(*p, kDown, hid, nullptr, nullptr, nullptr, *w, yperm);
        f.y_perm = yperm;
        f.y = y;
        f.sync = at<GridSync>(workspace, L.sync);
        f.spin_limit = env_unsigned("MOE_FUSED_SPIN_LIMIT", 1u << 20);
        return dev(launch_decode_fused(f, p->w_dtype == MOE_NVFP4, int(env_unsigned("MOE_FUSED_BLOCKS_PER_CU", 0)), s));
    }
    GemmArgs g1 = gemm_args(*p, kGateUp, x, st, tiles, tcount, *w, hid);
    g1.hid_packed = hid_packed(*p);
    MOE_TRY(mx_input(*p, g1, workspace, L, s));
    MOE_TRY(dev(launch_gemm(g1, L.family, L.max_tiles, s)));
    GemmArgs g2 = gemm_args(*p, kDown, hid, nullptr, tiles, tcount, *w, yperm);
    g2.hid_packed = hid_packed(*p);  // both GEMMs walk the same tile list
    MOE_TRY(mx_input(*p, g2, workspace, L, s));
    MOE_TRY(dev(launch_gemm(g2, L.family, L.max_tiles, s)));
    return dev(launch_combine(yperm, ip, tw, y, p->num_tokens, p->top_k, p->hidden,
                              p->num_tokens * p->top_k, p->act_dtype == MOE_BF16, s));
}

moe_status moe_forward_static(const moe_problem* p, const void* x, const void* w_router,
                              const float* router_bias, const moe_expert_weights* w, void* y,
                              int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_token, int32_t* inv_perm, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->num_tokens == 0)  // no scratch needed
        return moe_forward(p, x, w_router, router_bias, w, y, topk_ids, topk_w, counts, offsets,
                           sorted_token, inv_perm, nullptr, 0, stream);
    if (layout(*p).total > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
    void* ws = nullptr;
    MOE_TRY(static_scratch(&ws));
    return moe_forward(p, x, w_router, router_bias, w, y, topk_ids, topk_w, counts, offsets,
                       sorted_token, inv_perm, ws, MOE_STATIC_SCRATCH_BYTES, stream);
}

}  // extern "C"
