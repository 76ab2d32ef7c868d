// route.hip -- router logits (canonical fp32 order) and top-k / softmax selection.
//
// The router picks the experts of every token before dispatch ("CuTeDSL at Perplexity",
// section Mixture-of-Experts Dispatch/Combine, Local: the local kernel starts from the
// routing table; the Muse Spark Open megakernel article, section Model and new tensor
// parallelism: the expert step is only known once the router has run).
//
// Logits are computed on the VALU in the canonical order of the routing contract (moe.h);
// route.h holds the wavefront's computation.
#include "device.h"
#include "launch.h"
#include "route.h"
#include "select.h"

#include <cmath>

namespace moe {

// One wavefront per TM x TN block of logits.
template <bool BF16, int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x,
                                                            const void* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T,
                                                            int H, int E) {
    // the wavefront index as a scalar, so that the row bases stay scalar too (8 x 8 form: 231
    // -> 149 registers, 35 -> 16 64-bit address additions per chunk; NVFP4 prefill routing
    // 305 -> 274 us, bit-identical)
    router_logits_wave<BF16, TM, TN>(x, wr, bias, logits, T, H, E,
                                     __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave));
}

// One wavefront per token.
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    topk_token<EPL>(logits + size_t(t) * E, E, k, renorm, ids + size_t(t) * k, w + size_t(t) * k,
                    nullptr);
}

// ---------------------------------------------------------------------------------------
// Screened routing (large bf16 batches).  The canonical logits cost one VALU FMA per element of
// T x E x H; selection needs the canonical value only of the experts that can still be among a
// token's k largest.  So:
//  1. router_mfma_kernel: approximate logits m[t,e] = x_t . w_e + b_e on the bf16 matrix cores
//     (fp32 accumulation, in whatever order the matrix core adds, as partial sums over slices of
//     K), and the squared norms |w_e|^2;
//  2. router_screen_kernel, one wavefront per token: |x_t|^2, a bound beta_e >= |l[t,e] - m[t,e]|
//     that holds for any summation order (below); tau = the k-th largest m_e - beta_e; experts with
//     m_e + beta_e >= tau get their canonical logit (router_logits_wave, the code of the full
//     router), the others -inf;
//  3. the selection of topk_kernel on those values (in the same kernel).
// An expert with m_e + beta_e < tau has l_e < tau <= l_f for at least k experts f (those whose
// m_f - beta_f >= tau, themselves candidates), so it is not selected whatever the ties.  The k
// selected experts are candidates, with their canonical logits, so ids and weights are those of
// the full canonical router bit for bit.
//
// The bound: both dot products sum H exact bf16 x bf16 products (16 significant bits fit
// fp32).  A sum whose additions are each accurate to a relative u is within
// ((1 + u)^n - 1) sum |x_i w_i| of the exact sum when no term passes through more than n
// additions (the forward error bound of summation, Higham, Accuracy and Stability of
// Numerical Algorithms, section 4.2).  The canonical order is IEEE fused multiply-adds
// (u = 2^-24): at most H / 64 + 8 per partial, a fold of 6 and the bias, n <= H / 64 + 16.
// For the matrix cores nothing is assumed about the order or the rounding inside an
// instruction beyond each addition being accurate to u = 2^-23 (round to nearest, or
// truncation): an instruction adds
// 32 products and the accumulator, so a term passes through at most 32 additions per
// instruction of its K slice, H / KS in all, then the KS - 1 additions of the slices and the
// bias: n = H / KS + KS + 1.  sum |x_i w_i| <= |x| |w| (Cauchy-Schwarz).  Inputs, products or
// partial sums flushed to zero below 2^-126 add at most 2^-126 (max|x| + max|w| + 2) per term,
// a term in 2^-126 H (|x| + |w| + 2).  The norms are computed in fp32 from squares, which can
// underflow: |x| <= (1 + 2^-10) sqrt(sum x^2) + sqrt(H) 2^-63.  |m| 2^-21 absorbs the
// rounding of m +- beta.  A token whose m or norms are not finite, or exceed 2^100 (|m|, |b|)
// or 2^50 (norms, so that the bound stays finite), gets the canonical logits of all E experts.

constexpr int kRT = 64, kRE = 128, kRK = 64;  // screening MFMA block tile: tokens, experts, K

__device__ __forceinline__ float sumsq_bf16x8(uint4 v, float acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = bf16_lo(w[q]), hi = bf16_hi(w[q]);
        acc = __builtin_fmaf(lo, lo, acc);
        acc = __builtin_fmaf(hi, hi, acc);
    }
    return acc;
}

// Block tile: 64 tokens x 128 experts x one of KS slices of K, 8 wavefronts (2 x 4) of 32 x 32,
// K in stages of 64 through a two-buffer LDS ring; each thread's share of a stage (three 16-byte
// chunks) is loaded into registers four stages ahead.  The K split multiplies the blocks, and so
// the loads in flight, by KS (the kernel waits on memory latency, not on its MFMAs): slice ks
// writes its partial sums to m + ks T E (the bias in slice 0) and the screen adds the KS
// partials, an order the bound covers.  Blocks b, b + 8, ... run on one XCD, and the blocks of a
// token tile are dealt to one XCD, so that they read its x rows from that XCD's L2.  The blocks
// of token tile 0 also sum the squared router rows over their slice (wn2 + ks E).
__global__ __launch_bounds__(512) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ m, float* __restrict__ wn2,
                                                          int T, int H, int E, int KS) {
    __shared__ uint4 sX[2][kRT * 8];  // row r, 16-byte chunk c at r * 8 + (c ^ ((r >> 1) & 7))
    __shared__ uint4 sW[2][kRE * 8];
    const int tilesT = (T + kRT - 1) / kRT, tilesE = (E + kRE - 1) / kRE;
    const int b = blockIdx.x, q = b >> 3;
    const int ks = q % KS;
    const int et = (q / KS) % tilesE;
    const int tt = (b & 7) + 8 * (q / (KS * tilesE));
    if (tt >= tilesT) return;
    const int t0 = tt * kRT, e0 = et * kRE;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wt = wave >> 2, we = wave & 3;
    const int c = tid & 7, r = tid >> 3;  // chunk c of x row r and of router rows r, r + 64
    const bool wnorm = tt == 0;
    const int nst = H / kRK / KS;       // stages of this slice
    const size_t k0 = size_t(ks) * nst * kRK;

    const uint4* const px = reinterpret_cast<const uint4*>(x + size_t(min(t0 + r, T - 1)) * H + k0) + c;
    const uint4* const pw0 = reinterpret_cast<const uint4*>(wr + size_t(min(e0 + r, E - 1)) * H + k0) + c;
    const uint4* const pw1 = reinterpret_cast<const uint4*>(wr + size_t(min(e0 + r + 64, E - 1)) * H + k0) + c;

    uint4 r0[3], r1[3], r2[3], r3[3];  // stages s with s % 4 = 0, 1, 2, 3 in flight
    float sw0 = 0.f, sw1 = 0.f;
    f32x4_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#define MOE_RLOAD(R, S)            \
    do {                           \
        R[0] = px[(S) * 8];        \
        R[1] = pw0[(S) * 8];       \
        R[2] = pw1[(S) * 8];       \
    } while (0)
#define MOE_RSTORE(R, BUF)                                                   \
    do {                                                                     \
        if (wnorm) {                                                         \
            sw0 = sumsq_bf16x8(R[1], sw0);                                   \
            sw1 = sumsq_bf16x8(R[2], sw1);                                   \
        }                                                                    \
        sX[BUF][r * 8 + (c ^ ((r >> 1) & 7))] = R[0];                               \
        sW[BUF][r * 8 + (c ^ ((r >> 1) & 7))] = R[1];                               \
        sW[BUF][(r + 64) * 8 + (c ^ ((r >> 1) & 7))] = R[2];                        \
    } while (0)
#define MOE_RMFMA(BUF)                                                                        \
    do {                                                                                      \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                    \
            const int ch = ks * 4 + (lane >> 4);                                              \
            bf16x8_t af[2], bfr[2];                                                           \
            _Pragma("unroll") for (int mi = 0; mi < 2; ++mi) {                                \
                const int row = wt * 32 + mi * 16 + (lane & 15);                              \
                af[mi] = __builtin_bit_cast(bf16x8_t, sX[BUF][row * 8 + (ch ^ ((row >> 1) & 7))]);   \
            }                                                                                 \
            _Pragma("unroll") for (int ni = 0; ni < 2; ++ni) {                                \
                const int row = we * 32 + ni * 16 + (lane & 15);                              \
                bfr[ni] = __builtin_bit_cast(bf16x8_t, sW[BUF][row * 8 + (ch ^ ((row >> 1) & 7))]);  \
            }                                                                                 \
            _Pragma("unroll") for (int mi = 0; mi < 2; ++mi)                                  \
                _Pragma("unroll") for (int ni = 0; ni < 2; ++ni)                              \
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0); \
        }                                                                                     \
    } while (0)
    // stage s: registers r(s % 4), then LDS buffer s % 2; loaded four stages ahead of its MFMAs
    MOE_RLOAD(r0, 0);
    if (1 < nst) MOE_RLOAD(r1, 1);
    if (2 < nst) MOE_RLOAD(r2, 2);
    if (3 < nst) MOE_RLOAD(r3, 3);
    MOE_RSTORE(r0, 0);
    __syncthreads();
#define MOE_RPHASE(J, RL, RS)                                  \
    {                                                          \
        const int cs = s + (J);                                \
        if (cs >= nst) break;                                  \
        if (cs + 4 < nst) MOE_RLOAD(RL, cs + 4);               \
        MOE_RMFMA((J) & 1);                                    \
        if (cs + 1 < nst) MOE_RSTORE(RS, ((J) + 1) & 1);       \
        __syncthreads();                                       \
    }
    for (int s = 0; s < nst; s += 4) {
        MOE_RPHASE(0, r0, r1)
        MOE_RPHASE(1, r1, r2)
        MOE_RPHASE(2, r2, r3)
        MOE_RPHASE(3, r3, r0)
    }
#undef MOE_RPHASE
#undef MOE_RLOAD
#undef MOE_RSTORE
#undef MOE_RMFMA
    // 16 x 16 output block (mi, ni): lane holds column lane % 16, rows 4 (lane / 16) + i
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const int e = e0 + we * 32 + ni * 16 + (lane & 15);
            if (e >= E) continue;
            const float be = (bias && ks == 0) ? bias[e] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + wt * 32 + mi * 16 + 4 * (lane >> 4) + i;
                if (t < T) m[(size_t(ks) * T + t) * E + e] = acc[mi][ni][i] + be;
            }
        }
    if (wnorm) {  // the 8 threads of a row (consecutive lanes) hold its 8 chunk partials
        sw0 += __shfl_xor(sw0, 1);
        sw0 += __shfl_xor(sw0, 2);
        sw0 += __shfl_xor(sw0, 4);
        sw1 += __shfl_xor(sw1, 1);
        sw1 += __shfl_xor(sw1, 2);
        sw1 += __shfl_xor(sw1, 4);
        if (c == 0 && e0 + r < E) wn2[ks * E + e0 + r] = sw0;
        if (c == 0 && e0 + r + 64 < E) wn2[ks * E + e0 + r + 64] = sw1;
    }
}

// Canonical logits of two experts of one token whose hidden row a wavefront holds in registers
// (CPL chunks of 8 per lane, lane p holding chunks p, p + 64, ..., as fp32): the order of
// router_logits_wave for one (token, expert), computed for both experts side by side.
template <int CPL>
__device__ __forceinline__ void canonical_pair(const float (&xf)[CPL * 8], const uint16_t* __restrict__ wr,
                                               int H, int e0, int e1, float* v0, float* v1) {
    const int lane = lane_id();
    const uint4* const w0 = reinterpret_cast<const uint4*>(wr + size_t(e0) * H);
    const uint4* const w1 = reinterpret_cast<const uint4*>(wr + size_t(e1) * H);
    uint4 a[CPL], b[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        a[i] = w0[lane + kWave * i];
        b[i] = w1[lane + kWave * i];
    }
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint32_t ua[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
        const uint32_t ub[4] = {b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s0 = __builtin_fmaf(xf[i * 8 + 2 * q], bf16_lo(ua[q]), s0);
            s1 = __builtin_fmaf(xf[i * 8 + 2 * q], bf16_lo(ub[q]), s1);
            s0 = __builtin_fmaf(xf[i * 8 + 2 * q + 1], bf16_hi(ua[q]), s0);
            s1 = __builtin_fmaf(xf[i * 8 + 2 * q + 1], bf16_hi(ub[q]), s1);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        s0 = s0 + __shfl_xor(s0, off);
        s1 = s1 + __shfl_xor(s1, off);
    }
    *v0 = s0;
    *v1 = s1;
}

// One wavefront per token: m is the sum of the KS partials mpart + ks T E, the squared router
// norms the sum of wn2 + ks E; the selection (ids, weights) follows from the screened canonical
// logits.  CPL > 0: H = 512 CPL, the token row is held in registers (as fp32), candidates are
// taken two at a time and their logits stay in registers for the selection; CPL = 0: any H,
// each candidate through router_logits_wave into the token's logits row (the others -inf), from
// which the selection reads.  Either way the selection runs the code of topk_kernel on the same
// values.
template <int EPL, int CPL>
__global__ __launch_bounds__(256) void router_screen_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            const float* __restrict__ mpart,
                                                            float* __restrict__ logits,
                                                            const float* __restrict__ wn2, int T,
                                                            int H, int E, int k, int KS, ScreenConst sc,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ tw) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;  // uniform per wave
    const int lane = lane_id();
    float* const row = logits + size_t(t) * E;
    const uint4* const xr = reinterpret_cast<const uint4*>(x + size_t(t) * H);
    constexpr int XF = CPL > 0 ? CPL * 8 : 1;
    float xf[XF];
    float ss = 0.0f;  // this lane's share of |x_t|^2
    if constexpr (CPL > 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint4 v = xr[lane + kWave * i];
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xf[i * 8 + 2 * q] = bf16_lo(u[q]);
                xf[i * 8 + 2 * q + 1] = bf16_hi(u[q]);
            }
        }
#pragma unroll
        for (int i = 0; i < XF; ++i) ss = __builtin_fmaf(xf[i], xf[i], ss);
    } else {
        xf[0] = 0.0f;
        for (int cidx = lane; cidx < H / 8; cidx += kWave) ss = sumsq_bf16x8(xr[cidx], ss);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float xs = __builtin_sqrtf(ss) * (1.0f + 0x1p-10f) + sc.norm_abs;
    float mv[EPL], bnd[EPL];
    bool live[EPL];
    bool ok = xs <= 0x1p50f;  // false for NaN and infinities too
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        live[i] = e < E;
        mv[i] = 0.0f;
        bnd[i] = 0.0f;
        if (live[i]) {
            // all slices' loads in flight before the first sum (KS <= 4), summed in slice order
            float mp[4], wp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < KS) {
                    mp[q] = mpart[(size_t(q) * T + t) * E + e];
                    wp[q] = wn2[q * E + e];
                }
            float w2 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < KS) {
                    mv[i] += mp[q];
                    w2 += wp[q];
                }
            const float ws = __builtin_sqrtf(w2) * (1.0f + 0x1p-10f) + sc.norm_abs;
            const float ab = bias ? __builtin_fabsf(bias[e]) : 0.0f;
            ok = ok && ws <= 0x1p50f && ab <= 0x1p100f && __builtin_fabsf(mv[i]) <= 0x1p100f;
            bnd[i] = sc.gamma * (xs * ws + ab) + sc.flush * (xs + ws + 2.0f) +
                     __builtin_fabsf(mv[i]) * 0x1p-21f + 0x1p-120f;
        }
    }
    if (__builtin_amdgcn_ballot_w64(!ok) != 0) {  // non-finite or huge: the full canonical row
        for (int e = 0; e < E; ++e) router_logits_wave<true, 1, 1>(x, wr, bias, logits, T, H, E, t * E + e);
        __threadfence_block();  // the row's stores (lane 0) before its loads (every lane)
        topk_token<EPL>(row, E, k, 1, ids + size_t(t) * k, tw + size_t(t) * k, nullptr);
        return;
    }
    // tau: the k-th largest lower bound (k rounds, each removing one occurrence of the maximum)
    float lo[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) lo[i] = live[i] ? mv[i] - bnd[i] : -__builtin_inff();
    float tau = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = -1;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lo[i] > bv) {
                bv = lo[i];
                bi = i;
            }
        const float mx = wave_max_f32(bv);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(bi >= 0 && bv == mx);
        if (lane == int(__builtin_ctzll(hit))) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == bi) lo[i] = -__builtin_inff();
        }
        tau = mx;
    }
    int pend = -1;  // CPL > 0: a candidate waiting for its pair
    float cv[EPL];  // CPL > 0: canonical logits of the candidates, -inf elsewhere
#pragma unroll
    for (int i = 0; i < EPL; ++i) cv[i] = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const bool cand = live[i] && mv[i] + bnd[i] >= tau;
        if (CPL == 0 && live[i] && !cand) row[lane + kWave * i] = -__builtin_inff();
        uint64_t cm = __builtin_amdgcn_ballot_w64(cand);
        while (cm) {
            const int e = kWave * i + int(__builtin_ctzll(cm));
            cm &= cm - 1;
            if constexpr (CPL > 0) {
                if (pend < 0) {
                    pend = e;
                    continue;
                }
                float v0, v1;
                canonical_pair<CPL>(xf, wr, H, pend, e, &v0, &v1);
                if (bias) {
                    v0 = v0 + bias[pend];
                    v1 = v1 + bias[e];
                }
#pragma unroll
                for (int q = 0; q < EPL; ++q) {
                    if (pend == lane + kWave * q) cv[q] = v0;
                    if (e == lane + kWave * q) cv[q] = v1;
                }
                pend = -1;
            } else {
                router_logits_wave<true, 1, 1>(x, wr, bias, logits, T, H, E, t * E + e);
            }
        }
    }
    if constexpr (CPL > 0) {
        if (pend >= 0) {  // an odd candidate: pair it with itself
            float v0, v1;
            canonical_pair<CPL>(xf, wr, H, pend, pend, &v0, &v1);
            if (bias) v0 = v0 + bias[pend];
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (pend == lane + kWave * q) cv[q] = v0;
        }
        float sv, m0;
        int se;
        topk_rounds<EPL>(cv, live, k, &sv, &se, &m0);
        topk_write_renormalised(sv, se, m0, k, ids + size_t(t) * k, tw + size_t(t) * k, nullptr);
    } else {
        __threadfence_block();  // the row's stores before its loads
        topk_token<EPL>(row, E, k, 1, ids + size_t(t) * k, tw + size_t(t) * k, nullptr);
    }
}

// ---------------------------------------------------------------------------------------

ScreenConst screen_const(int H, int KS) {
    ScreenConst c;
    const double n_mfma = double(H) / KS + KS + 1, n_can = double(H) / 64 + 16;
    const double g = std::expm1(n_mfma * std::log1p(std::ldexp(1.0, -23))) +
                     std::expm1(n_can * std::log1p(std::ldexp(1.0, -24)));
    c.gamma = float(g * 1.001);
    c.flush = float(std::ldexp(1.0, -126) * double(H) * 1.001);
    c.norm_abs = float(std::sqrt(double(H)) * std::ldexp(1.0, -63) * 1.001);
    return c;
}

template <int EPL>
static void launch_screen(int cpl, dim3 g, const uint16_t* x, const uint16_t* wr, const float* bias,
                          const float* mpart, float* logits, const float* wn2, int T, int H, int E,
                          int k, int KS, ScreenConst sc, int32_t* ids, float* tw, hipStream_t s) {
    if (cpl == 8)
        hipLaunchKernelGGL((router_screen_kernel<EPL, 8>), g, dim3(256), 0, s, x, wr, bias, mpart, logits, wn2, T, H, E, k, KS, sc, ids, tw);
    else if (cpl == 4)
        hipLaunchKernelGGL((router_screen_kernel<EPL, 4>), g, dim3(256), 0, s, x, wr, bias, mpart, logits, wn2, T, H, E, k, KS, sc, ids, tw);
    else if (cpl == 2)
        hipLaunchKernelGGL((router_screen_kernel<EPL, 2>), g, dim3(256), 0, s, x, wr, bias, mpart, logits, wn2, T, H, E, k, KS, sc, ids, tw);
    else
        hipLaunchKernelGGL((router_screen_kernel<EPL, 0>), g, dim3(256), 0, s, x, wr, bias, mpart, logits, wn2, T, H, E, k, KS, sc, ids, tw);
}

// K slices of the screening GEMM: enough blocks for the loads in flight (measured, routing
// alone, median us: 8192 tokens x 256 experts, slices 1 / 2 / 4 / 8: 119 / 107 / 117 / 135;
// 4096 x 128: 86 / 68 / 61 / 63), so four slices below 256 blocks, two below 512, else one.
// At most four: the screen kernel sums up to four slices.
int screen_k_split(int T, int H, int E) {
    const int nst = H / kRK;
    const long blocks = long((T + kRT - 1) / kRT + 7) / 8 * 8 * ((E + kRE - 1) / kRE);
    int ks = blocks < 256 ? 4 : (blocks < 512 ? 2 : 1);
    while (nst % ks) ks >>= 1;
    return ks;
}

hipError_t launch_router_screened(const RouteArgs& a, float* mpart, float* wn2, int k, int32_t* ids,
                                  float* tw, hipStream_t s) {
    const int T = a.T, E = a.E, H = a.H;
    const int tilesT = (T + kRT - 1) / kRT, tilesE = (E + kRE - 1) / kRE;
    const int KS = screen_k_split(T, H, E);
    dim3 grid(((tilesT + 7) / 8) * 8 * tilesE * KS);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    const uint16_t* wr = static_cast<const uint16_t*>(a.wr);
    hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(512), 0, s, x, wr, a.bias, mpart, wn2, T, H, E, KS);
    const ScreenConst sc = screen_const(H, KS);
    const dim3 g2((T + 3) / 4);
    // token row in registers for H = 1024, 2048, 4096
    const int cpl = (H == 4096) ? 8 : (H == 2048) ? 4 : (H == 1024) ? 2 : 0;
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1)
        launch_screen<1>(cpl, g2, x, wr, a.bias, mpart, a.logits, wn2, T, H, E, k, KS, sc, ids, tw, s);
    else if (epl <= 2)
        launch_screen<2>(cpl, g2, x, wr, a.bias, mpart, a.logits, wn2, T, H, E, k, KS, sc, ids, tw, s);
    else if (epl <= 4)
        launch_screen<4>(cpl, g2, x, wr, a.bias, mpart, a.logits, wn2, T, H, E, k, KS, sc, ids, tw, s);
    else
        launch_screen<8>(cpl, g2, x, wr, a.bias, mpart, a.logits, wn2, T, H, E, k, KS, sc, ids, tw, s);
    return hipGetLastError();
}

hipError_t launch_router_logits(const RouteArgs& a, hipStream_t s) {
    const int T = a.T, E = a.E;
    // large batches: 8x8 (token, expert) blocks per wave for operand reuse, 4x4 below 384 tokens
    // (four times the wavefronts, each with a quarter of the serial FMA work; kernel trace,
    // median us, 8x8 -> 4x4 at E=128: T=64 17.5 -> 12.0, T=128 17.5 -> 12.4, T=256 18.0 -> 14.4,
    // but T=512 19.3 -> 20.8 and T=4096 85.7 -> 126.3); small batches: one token and 2 experts
    // per wave, or one expert per wave while that still leaves at most 1024 blocks (every wave
    // waits for the same memory latency, so more of them finish sooner: decode T=1 with E=128
    // measured about 1 us less per forward, 16 tokens over 256 experts 0.8 us).  All shapes
    // give bit-identical logits.
    if (T >= 64 && T < 384 && E >= 8) {
        const long waves = long((T + 3) / 4) * ((E + 3) / 4);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 4, 4>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 4, 4>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else if (T >= 64 && E >= 8) {
        const long waves = long((T + 7) / 8) * ((E + 7) / 8);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 8, 8>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 8, 8>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else if (long(T) * E <= 4096) {
        const long waves = long(T) * E;
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 1, 1>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 1, 1>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    } else {
        const long waves = long(T) * ((E + 1) / 2);
        dim3 grid((waves + 3) / 4), block(256);
        if (a.bf16)
            hipLaunchKernelGGL((router_logits_kernel<true, 1, 2>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
        else
            hipLaunchKernelGGL((router_logits_kernel<false, 1, 2>), grid, block, 0, s, a.x, a.wr,
                               a.bias, a.logits, T, a.H, E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                       float* w, hipStream_t s) {
    dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + kWave - 1) / kWave;
    if (epl <= 1)
        hipLaunchKernelGGL((topk_kernel<1>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (epl <= 2)
        hipLaunchKernelGGL((topk_kernel<2>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else if (epl <= 4)
        hipLaunchKernelGGL((topk_kernel<4>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    else
        hipLaunchKernelGGL((topk_kernel<8>), grid, block, 0, s, logits, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

}  // namespace moe
