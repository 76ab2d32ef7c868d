/*
 * moe_probe.h -- measurement aids for the MoE layer library on MI355X (gfx950).
 *
 * Microkernels that measure what the device actually sustains, so that a benchmark can state its
 * kernels' roofline fractions against measured peaks beside the data-sheet ones (bf16 dense
 * MFMA 2.5 PFLOP/s, HBM3E 8 TB/s), what one grid barrier of the single-launch decode kernel
 * costs, and how long the grouped GEMM kernel alone takes.  Apart from the last (which runs
 * moe_grouped_gemm's own computation) they compute nothing of the layer.
 * Same conventions as moe.h: device pointers owned by the caller, work enqueued on `stream`
 * (a hipStream_t, NULL = default stream), return codes only, arguments validated on the host
 * before any HIP call.
 */
#ifndef MOE_MI355X_PROBE_H
#define MOE_MI355X_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA issue rate: `blocks` blocks of 256 threads; every wavefront runs `iters`
 * rounds of 8 independent v_mfma_f32_16x16x32_bf16 (16x16x32 multiply-adds each) on register
 * operands.  Work = blocks * 4 * iters * 8 * 16384 FLOP.  out: device float[blocks], written
 * (one value per block) so the chains stay live.  blocks in [1, 1<<20], iters in [1, 1<<24],
 * else MOE_ERR_INVALID_ARGUMENT. */
moe_status moe_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

/* HBM read stream: every 16-byte word of buf[0, bytes) is read once by 16-byte loads; 16384
 * blocks of 256 threads take contiguous 32 KiB chunks in turn, eight loads in flight per
 * thread.  out: device uint32_t[1], written only for one particular XOR of the data (so the
 * loads cannot be elided).  bytes must be a positive multiple of 16 and buf 16-byte aligned,
 * else MOE_ERR_INVALID_ARGUMENT. */
moe_status moe_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* The same read stream with non-temporal loads (no cache lines allocated for reuse): the rate
 * of a stream like the decode GEMMs' weight loads.  Unlike moe_probe_read it does not evict
 * the caches.  Arguments and errors as moe_probe_read. */
moe_status moe_probe_read_nt(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Grid barriers alone: one cooperative launch of `blocks` blocks of 256 threads (they must fit
 * on the device at once, else MOE_ERR_DEVICE) that pass `barriers` grid barriers of the
 * single-launch decode kernel (MOE_PATH_DECODE_FUSED) in a row and do nothing else.  sync:
 * device memory of MOE_PROBE_SYNC_BYTES, 16-byte aligned, any contents (it keeps a sequence
 * number; at byte offset 8 a 32-bit count of barrier waits that gave up after `spin_limit`
 * polls).  blocks in [1, 1024], barriers in [1, 65535], else MOE_ERR_INVALID_ARGUMENT. */
#define MOE_PROBE_SYNC_BYTES 8256
moe_status moe_probe_grid_barrier(int32_t blocks, int32_t barriers, void* sync, uint32_t spin_limit,
                                  void* stream);

/* moe_grouped_gemm's GEMM timed on its own: the arguments of moe_grouped_gemm (same checks,
 * same results in `out`) plus timing.  The tile list is built from `offsets` once; then the GEMM
 * (for MX weights with its input quantization, which is part of every moe_grouped_gemm call) is
 * launched `launches` times on `stream`, each launch bracketed by two HIP events, so the tile-list
 * kernel stays outside the brackets.  With flush_bytes > 0, every launch is preceded (outside its
 * bracket) by a moe_probe_read of flush_buf[0, flush_bytes) into flush_out, which evicts the
 * layer's operands from the caches.  ms: host float[launches], receives each launch's duration in
 * milliseconds; the call synchronizes `stream`.  launches in [1, 100000], ms not NULL, and a flush
 * buffer as moe_probe_read requires when flush_bytes > 0, else MOE_ERR_INVALID_ARGUMENT.  With
 * num_tokens == 0 nothing is launched and ms is filled with 0. */
moe_status moe_probe_grouped_gemm_times(const moe_problem* p, moe_gemm_kind kind, const void* a,
                                        const int32_t* a_rows, const int32_t* offsets,
                                        const moe_expert_weights* w, void* out, void* workspace,
                                        size_t workspace_bytes, const void* flush_buf,
                                        size_t flush_bytes, uint32_t* flush_out, int32_t launches,
                                        float* ms, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_PROBE_H */
