/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts FFN layer, forward pass, one GPU.
 *
 * The layer is the single-GPU ("TP=1, local") MoE path described in "CuTeDSL at Perplexity"
 * (Perplexity blog), section "Mixture-of-Experts Dispatch/Combine", subsection "Local":
 *   route    router logits, top-k expert selection per token and its weights;
 *   dispatch count the tokens of each expert and give every (token, slot) a unique index in
 *            its expert's list, so the expert GEMMs see contiguous rows;
 *   GEMMs    per expert: gate/up projection with SwiGLU, then the down projection ("MoE GEMM",
 *            "Hosting Qwen on Blackwell", section MoE GEMM; SwiGLU as a stage of the layer in
 *            the Muse Spark Open megakernel article, section Megakernel implementation);
 *   combine  the weighted sum of each token's expert outputs, back in token order.
 *
 * Notation: T tokens, H hidden, E experts, k experts per token, F expert FFN width,
 * A = T*k assignments.  All matrices are dense row-major.  Expert weights are stored
 * [out, in] (y = x W^T): w13 is [E, 2F, H] with gate rows 0..F-1 and up rows F..2F-1;
 * w2 is [E, H, F].
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE memory owned by the caller, 16-byte aligned.  The library never
 *    allocates, frees or retains device memory; scratch comes from the caller's workspace
 *    (size from moe_workspace_size).  No global mutable state: calls on different streams
 *    with different workspaces may run concurrently.  (The one exception is
 *    moe_forward_static, at the end of this header, whose scratch is a static per-GPU array.)
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work
 *    on it; nothing synchronises and no device data is read on the host.  Results are valid
 *    once the caller has synchronised the stream.
 *  - What is enqueued is kernel launches only (no memset, no copy), so a call may be
 *    captured into a HIP graph and replayed.  Grids are sized from the host-side problem
 *    fields alone, so a replay is valid for new contents of the same buffers (other tokens,
 *    other routings), not for another moe_problem.
 *  - Errors are return codes; nothing is thrown and nothing aborts.  All arguments are
 *    validated on the host before any HIP call: MOE_ERR_INVALID_ARGUMENT for a null required
 *    pointer, a misaligned pointer, negative sizes, k < 1, k > E, k > 16, E > 512 or an
 *    expert range outside [0, E);
 *    MOE_ERR_UNSUPPORTED for shapes with no compiled kernel (H % 64, F % 64 != 0; bf16
 *    weights with H % 256 or F % 128 != 0; MXFP8 with H % 512 or F % 512 != 0; bf16
 *    activations with fp32 weights or the reverse; NVFP4 or MXFP8 with fp32 activations), and
 *    MOE_ERR_INVALID_ARGUMENT for an unknown weight layout or PACKED fp32 weights
 *    (moe_layout);
 *    MOE_ERR_WORKSPACE_TOO_SMALL; MOE_ERR_DEVICE when a launch reports an error.
 *  - T = 0 is a successful no-op (token-sized buffers and the workspace may then be NULL;
 *    moe_permute and moe_forward still set counts/offsets, when given, to zero).
 *  - Determinism: identical inputs give bitwise identical outputs (no floating-point atomics).
 *  - Non-finite inputs give unspecified (but memory-safe) values; the routing stays valid:
 *    every token still gets k distinct experts in [0, E) (a NaN logit ranks below every
 *    number) and the permutation stays a bijection.
 *
 * Routing contract (bit-exact):
 *  - logits l[t,e] are fp32 in a canonical order: H is cut into chunks of 8 consecutive
 *    elements, chunk c feeds partial sum p = c mod 64; each partial starts at +0 and takes its
 *    chunks in ascending order, one correctly rounded fused multiply-add per element; the 64
 *    partials fold as a[p] += a[p+off] for off = 32,16,8,4,2,1; the bias is added last.
 *  - selection: the k largest logits, ties to the lower expert index, stored in that order.
 *  - weights (fp32): softmax over the k selected logits (renormalize = 1), or the full
 *    softmax probability of each selected expert (renormalize = 0).
 *  - dispatch order: assignments a = t*k + j sorted stably by expert, so rows of one expert
 *    appear in ascending (t, j) order; offsets are the exclusive prefix sum of the counts.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_DEVICE = 4,
    MOE_ERR_SCRATCH_TOO_SMALL = 5  /* moe_forward_static: the problem needs more than its scratch */
} moe_status;

/* Storage formats.  MOE_NVFP4 (weights only): 4-bit E2M1 values, two per byte with the even
 * element in the low nibble, one E4M3 (FN) scale per 16 consecutive elements along the input
 * dimension, and an optional fp32 scale per expert and matrix: w = e2m1 * e4m3 * gscale.
 * MOE_MXFP8 (weights only; OCP microscaling formats v1.0, the scheme "Hosting Qwen on
 * Blackwell" deploys, section Quantization): one E4M3 (FN) byte per element and one E8M0 scale
 * byte s per 32 consecutive elements along the input dimension: w = e4m3 * 2^(s - 127).  An
 * MXFP8 layer also runs its activations in MXFP8: the bf16 x rows are quantized before the
 * gate/up GEMM and the hid rows before the down GEMM, per block of 32 along K, with the shared
 * exponent X = floor(log2(max |v|)) - 8 (X = -127 for an all-zero block, clamped to
 * [-127, 127]) and elements v / 2^X clamped to +-448 and rounded to the nearest E4M3 value,
 * ties to the even code (sign kept); the GEMMs multiply on the block-scaled fp8 matrix cores
 * with fp32 accumulation.  Outputs (hid, y_perm, y) stay bf16.  Needs H % 512 == 0 and
 * F % 512 == 0, bf16 activations; the E4M3 codes row-major or PACKED (moe_layout), the E8M0
 * scales row-major.
 * MOE_MXFP4 (weights only; OCP MX v1.0 with E2M1 elements, which "Hosting Qwen on Blackwell"
 * evaluates beside MXFP8): two E2M1 values per byte, even element in the low nibble, one E8M0
 * scale per 32 along the input dimension: w = e2m1 * 2^(s - 127).  Activations run in MXFP8
 * exactly as for MOE_MXFP8; the GEMMs multiply fp8 activations by fp4 weights on the
 * block-scaled matrix cores.  Same shape rules; codes row-major or PACKED (the 4-bit variant
 * below), scales row-major. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_NVFP4 = 2, MOE_MXFP8 = 3, MOE_MXFP4 = 4 } moe_dtype;

typedef enum { MOE_GEMM_GATE_UP_SWIGLU = 0, MOE_GEMM_DOWN = 1 } moe_gemm_kind;

/* Kernel family.  AUTO picks DECODE when there are fewer than 16 assignments per expert on
 * average (weight streaming with small row tiles) and PREFILL otherwise (large MFMA tiles).
 * Both families give bit-identical routing and dispatch.
 * DECODE_FUSED runs moe_forward's decode family as ONE cooperative launch ("CuTeDSL at
 * Perplexity", section Grid synchronization: small decode batches as one kernel whose blocks
 * meet at grid barriers): router logits, grid barrier, selection and dispatch repeated in
 * every block, gate/up + SwiGLU, grid barrier, down, grid barrier, combine.  Same device code
 * and order as DECODE, so the same routing and, with the same K split, the same outputs.  It
 * covers bf16 activations with bf16 weights or PACKED NVFP4 weights, T <= 16, E <= 256,
 * H % 512 == 0 and F % 512 == 0 (moe_forward returns MOE_ERR_UNSUPPORTED otherwise); the stage
 * entry points treat it as DECODE.  Its barrier words live at the start of the workspace: a
 * 64-bit sequence number that the kernel advances (any initial value works), and a 32-bit
 * count of barrier waits that gave up (byte offset 8; every wait is bounded, so a grid that
 * could not be co-resident ends with unspecified outputs and a non-zero count instead of
 * hanging; the launch itself fails with MOE_ERR_DEVICE when the grid cannot be co-resident).
 * The workspace must not be shared by calls that overlap in time. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_PREFILL = 1, MOE_PATH_DECODE = 2, MOE_PATH_DECODE_FUSED = 3 } moe_path;

typedef struct {
    int32_t num_tokens;   /* T >= 0 */
    int32_t hidden;       /* H, multiple of 64 */
    int32_t num_experts;  /* E, 1..512 */
    int32_t top_k;        /* k, 1..min(E,16) */
    int32_t ffn;          /* F, multiple of 64 */
    int32_t act_dtype;    /* MOE_F32 | MOE_BF16: x, router weight, hid, y_perm, y */
    int32_t w_dtype;      /* MOE_F32 (with F32 acts) | MOE_BF16 | MOE_NVFP4 | MOE_MXFP8 | MOE_MXFP4 (BF16 acts) */
    int32_t renormalize;  /* 1: softmax over the selected k (default); 0: full softmax */
    int32_t path;         /* moe_path */
    int32_t expert_begin;  /* expert parallelism: the caller holds the experts           */
    int32_t local_experts; /* [expert_begin, expert_begin + local_experts); 0 = all E    */
} moe_problem;

/* Expert parallelism with replicated inputs ("CuTeDSL at Perplexity", section
 * Mixture-of-Experts Dispatch/Combine: with tensor parallelism every rank sees every token,
 * its dispatch keeps only the tokens routed to the experts it holds, and a local combine is
 * followed by an all-reduce across ranks; "Hosting Qwen on Blackwell", section Expert Parallel,
 * for prefill).  With local_experts = n > 0 the caller holds experts [b, b + n), b =
 * expert_begin:
 *  - routing is unchanged: logits, selection and weights always cover all E experts;
 *  - dispatch keeps only the assignments whose expert is held: counts[e] = 0 for the others,
 *    offsets[E] = the number of dispatched rows A_local, inv_perm = -1 for every assignment
 *    that is not dispatched; rows of held experts keep the stable (t, j) order, so they are
 *    exactly the rows [offsets[b], offsets[b+n]) of the dispatch over all experts;
 *  - the expert weights (and NVFP4 scales) hold the n experts only: expert e is at index e - b;
 *  - combine skips assignments with inv_perm < 0, so y is this caller's partial output (zero
 *    for a token with no held expert).  Summing the partial outputs of a partition of the
 *    experts (the all-reduce, which is the caller's) gives the layer's output.
 * Rows of hid, y_perm and x_perm past A_local are unspecified.  expert_begin = local_experts =
 * 0 (a zero-initialised struct) is the single-GPU layer. */

/* Weight layouts.  Every weight format is accepted ROW_MAJOR, the dense [E,2F,H] / [E,H,F]
 * layouts described in moe_expert_weights (MX and NVFP4: bytes [E,2F,H/2] ... for 4-bit
 * codes, scales always row-major unless noted).  bf16, MXFP8 and MXFP4 weights are also
 * accepted PACKED (written once by moe_pack_weights), and NVFP4 weights PACKED (bytes by
 * moe_pack_weights and scales by moe_pack_scales, both packed; needs H % 256 == 0 and
 * F % 128 == 0).  fp32 weights are ROW_MAJOR only.  Both layouts give bit-identical layers on
 * the bf16 and MX kernels (the same values reach the same LDS image or operand registers in
 * the same order) and on the NVFP4 prefill kernels; the NVFP4 decode kernels take K in another
 * order for each layout (results within the tolerance of each other).  PACKED is the fast
 * path: a stage of a 256-row tile is one contiguous block, where ROW_MAJOR reads 16 to 64
 * bytes per weight row and stage, one cache line of each of many rows per load instruction.
 *
 * PACKED (bf16 and MXFP8 codes; needs H % 256 == 0 and F % 128 == 0; same byte size as
 * row-major): weights are cut into tiles of 256 weight rows and stages of 64 bytes of a row
 * (32 bf16 or 64 E4M3 elements); each (expert, tile, stage) block is 16 KiB = 256 rows x 4
 * chunks of 16 bytes, and chunk c of tile row r is stored in slot c ^ ((r >> 1) & 3) of that
 * row.  Blocks are ordered [expert][tile][stage].
 *   w13: F/128 tiles of H/32 (bf16) or H/64 (MXFP8) stages; tile row r of tile t is the gate row
 *        f = 128 t + 64 (r / 128) + (r % 64) when r % 128 < 64, else the up row F + f.
 *   w2:  H/256 tiles of F/32 or F/64 stages; tile row r of tile t is weight row 256 t + r.
 * PACKED for MXFP4 codes: the same tiles and row order, stages of 64 elements = 32 bytes of a
 * row; each (expert, tile, stage) block is 8 KiB = 256 rows x 2 chunks of 16 bytes, chunk c of
 * tile row r in slot c ^ ((r >> 2) & 1).
 * PACKED for NVFP4: the same tiles and row order, stages of 32 elements; each (expert, tile,
 * stage) block of the bytes is 4 KiB = 256 rows x 16 bytes (tile row r at byte 16 r, no
 * slots), and each (expert, tile, stage pair) block of the scales is 1 KiB = 256 rows x the 4
 * scale bytes of stages 2m and 2m+1 of that row (tile row r at byte 4 r).  Blocks are ordered
 * [expert][tile][stage] and [expert][tile][stage pair].
 * One stage of one tile is then one contiguous 16 KiB read that lands in LDS unchanged, and
 * 16 consecutive rows of one stage are one contiguous 1 KiB. */
typedef enum { MOE_LAYOUT_ROW_MAJOR = 0, MOE_LAYOUT_PACKED = 1 } moe_layout;

typedef struct {
    const void* w13;              /* [E,2F,H] fp32 / bf16 / MXFP8 codes; NVFP4, MXFP4 bytes [E,2F,H/2]; or PACKED */
    const void* w2;               /* [E,H,F] fp32 / bf16 / MXFP8 codes; NVFP4, MXFP4 bytes [E,H,F/2]; or PACKED */
    const uint8_t* w13_scale;     /* NVFP4: E4M3 [E,2F,H/16]; MXFP8, MXFP4: E8M0 [E,2F,H/32] */
    const uint8_t* w2_scale;      /* NVFP4: E4M3 [E,H,F/16]; MXFP8, MXFP4: E8M0 [E,H,F/32] */
    const float* w13_gscale;      /* NVFP4 only, nullable (=> 1.0): fp32 [E] */
    const float* w2_gscale;       /* NVFP4 only, nullable (=> 1.0): fp32 [E] */
    int32_t layout;               /* moe_layout: ROW_MAJOR (any format) or PACKED (bf16, MX, NVFP4) */
} moe_expert_weights;

/* Text of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* Bytes of workspace every entry point below needs for problem `p` (an upper bound valid
 * for all of them).  Host only; touches no device.  Returns MOE_ERR_INVALID_ARGUMENT /
 * MOE_ERR_UNSUPPORTED for problems the entry points would reject. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/* Bytes of the packed w13 and w2 of problem `p` (bf16, MXFP8, MXFP4 or NVFP4 weights; for
 * NVFP4 the bytes, not the scales, whose packed size equals their row-major size).  Host only. */
moe_status moe_packed_weights_size(const moe_problem* p, size_t* w13_bytes, size_t* w2_bytes);
/* (both sizes and moe_pack_weights below cover the held experts only: local_experts of them
 * when it is non-zero, else all E) */

/* Rewrite row-major bf16 expert weights (or MXFP8 / MXFP4 codes, or NVFP4 bytes) w13 [E,2F,H]
 * and w2 [E,H,F] (MXFP4 and NVFP4: bytes [E,2F,H/2], [E,H,F/2]) into the PACKED layout (see
 * moe_layout).  A one-time transform of static weights; the outputs must not alias the
 * inputs.  Either pair (w13 -> w13_packed, w2 -> w2_packed) may be NULL to skip it.
 * MOE_ERR_UNSUPPORTED for shapes the PACKED layout does not cover. */
moe_status moe_pack_weights(const moe_problem* p, const void* w13, const void* w2,
                            void* w13_packed, void* w2_packed, void* stream);

/* NVFP4 only: rewrite the row-major E4M3 scales w13_scale [E,2F,H/16] and w2_scale [E,H,F/16]
 * into the PACKED layout of NVFP4 scales (see moe_layout); same byte sizes.  The outputs must
 * not alias the inputs; either pair may be NULL to skip it.
 * MOE_ERR_INVALID_ARGUMENT for other weight formats, MOE_ERR_UNSUPPORTED unless H % 256 == 0
 * and F % 128 == 0. */
moe_status moe_pack_scales(const moe_problem* p, const uint8_t* w13_scale, const uint8_t* w2_scale,
                           uint8_t* w13_scale_packed, uint8_t* w2_scale_packed, void* stream);

/* Route.  x [T,H] and w_router [E,H] in act_dtype; router_bias fp32 [E] or NULL.
 * Writes topk_ids int32 [T,k] and topk_w fp32 [T,k] (routing contract above).  From 256 bf16
 * tokens with renormalize = 1 the router screens first: approximate logits on the matrix cores
 * and a bound on their distance to the canonical ones that holds for any summation order
 * decide which experts can still be selected, and only those get canonical logits; the ids and
 * weights are the ones the contract defines, bit for bit (tokens with non-finite or huge values
 * get the canonical logits of every expert). */
moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* router_bias, int32_t* topk_ids, float* topk_w,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch.  From topk_ids [T,k] (values in [0,E)) writes counts int32 [E], offsets int32
 * [E+1], sorted_token int32 [A] (token of each dispatched row) and inv_perm int32 [A]
 * (dispatched row of assignment t*k+j).  If x and x_perm are both non-NULL it also copies
 * the token rows into x_perm [A,H] (act_dtype) in dispatch order. */
moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                       const void* x, void* x_perm, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Grouped expert GEMM over dispatched rows; expert e owns rows offsets[e]..offsets[e+1]-1.
 *  GATE_UP_SWIGLU: row r of the input is a[a_rows[r]] ([T,H], a_rows = sorted_token) or
 *                  a[r] ([A,H], a_rows = NULL); out[r] = silu(g) * u with g / u the gate / up
 *                  projections by w13[e]: out is hid [A,F] in act_dtype.
 *  DOWN:           input a = hid [A,F] (a_rows must be NULL); out = y_perm [A,H] =
 *                  hid W2[e]^T, in act_dtype.
 * fp32 accumulation; NVFP4 weights are decoded exactly to bf16 inside the kernel; for MXFP8
 * the bf16 input rows are first quantized to MXFP8 (into the workspace) and the product runs
 * on the block-scaled fp8 matrix cores.
 * `offsets` [E+1] is read on the device; values are clamped to [0, A] so that a malformed
 * table cannot make the kernel reach past the A rows of `a`/`out`.  Only the rows of held
 * experts are computed (all experts unless local_experts is set); other rows are untouched. */
moe_status moe_grouped_gemm(const moe_problem* p, moe_gemm_kind kind, const void* a,
                            const int32_t* a_rows, const int32_t* offsets,
                            const moe_expert_weights* w, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Combine.  y[t] = sum_j topk_w[t,j] * y_perm[inv_perm[t*k+j]] accumulated in fp32 in
 * ascending j and rounded once to act_dtype; assignments with inv_perm < 0 (not dispatched
 * to this caller's experts) are skipped.  y_perm [A,H], y [T,H] in act_dtype. */
moe_status moe_combine(const moe_problem* p, const void* y_perm, const int32_t* inv_perm,
                       const float* topk_w, void* y, void* stream);

/* MXFP8 quantization of bf16 rows, the layer's own activation step (rule under moe_dtype):
 * x [rows, K] bf16 -> codes [rows, K] E4M3 and scales [rows, K/32] E8M0, all row-major.
 * For callers that keep activations in MXFP8.  K % 32 == 0; x and codes 16-byte aligned. */
moe_status moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* The whole layer: route -> dispatch -> gate/up GEMM + SwiGLU -> down GEMM -> combine.
 * y [T,H] in act_dtype.  The routing/dispatch outputs are optional (NULL = keep them in the
 * workspace); when given they receive the same values the stage entry points produce. */
moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router,
                       const float* router_bias, const moe_expert_weights* w, void* y,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_token, int32_t* inv_perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward without a workspace argument.  Every
 * argument means what it means for moe_forward; the scratch comes from a static device array
 * of MOE_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends (its device address is looked up once per device, with that device current; the call
 * uses the current device, which must be the stream's).  Nothing is allocated or freed.
 *  - MOE_ERR_SCRATCH_TOO_SMALL, before any device work, when moe_workspace_size(p) exceeds
 *    MOE_STATIC_SCRATCH_BYTES (decode-sized problems fit: for H 4096, F 1536, k 8 up to about
 *    700 tokens; prefill-sized ones do not and take moe_forward with a workspace).
 *  - Every call on a GPU uses that GPU's one array, which keeps the last call's contents;
 *    nothing in it needs to start at zero (each call writes every byte it reads first).
 *    Calls that overlap in time on one GPU (other streams, other host threads) race on it and
 *    must be serialised by the caller.
 *  - Otherwise as moe_forward (enqueues kernel launches only; capturable). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_static(const moe_problem* p, const void* x, const void* w_router,
                              const float* router_bias, const moe_expert_weights* w, void* y,
                              int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_token, int32_t* inv_perm, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
