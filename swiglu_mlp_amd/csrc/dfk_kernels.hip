// dfk_kernels.hip -- hand-written CDNA4 (gfx950) kernels of the decode-stage SwiGLU MLP.
//
// Two operations ("Deep Kernel Fusion for Transformer Decoding", podcast episode
// page, episode summary):
//   gate-up  h[b,n] = SiLU(sum_k x[b,k] Wg[n,k]) * (sum_k x[b,k] Wu[n,k])
//            -- the up projection, the gate projection, SiLU and the product in
//               ONE kernel; g and u live only in registers.
//   down     y[b,m] = RNE_bf16(sum_n h[b,n] Wd[m,n])   -- a separate kernel.
// Decode is memory-bound ("Deep Kernel Fusion for Transformers", hgpu.org post,
// abstract: the SwiGLU weights exceed cache capacity), so every kernel is a
// weight stream: each weight byte is loaded from HBM exactly once per call, in
// 16-byte vectors, and everything else (x, h, reductions) stays on chip.
//
// Engines
//   VALU (B <= 8): 64 lanes of a wave span 512 consecutive K elements of a
//     weight row (one 16-byte load per lane = 1 KB per row per instruction).
//     gate-up multiplies bf16 pairs with v_dot2c_f32_bf16 against x resident in
//     LDS; down widens bf16 weights and uses fp32 FMAs against fp32 h.  Lane
//     partials are summed with a fixed DPP butterfly (lane 63 gets the total).
//   MFMA (B >= 16, or where VALU does not fit): v_mfma_f32_16x16x32_bf16 with
//     the weight tile as the A operand (16 rows x 32 K, one 16-byte load per
//     lane) and x^T (or h^T) as the B operand, batch padded to 16.  The fp32 h
//     of the down projection is split into bf16 hi + lo and fed as two MFMAs,
//     which keeps ~16 significant bits of h.
// Traversals (the row-major / column-major variants of the episode summary)
//   ROW  one wave owns each output row's whole dot product (VALU: lanes along
//        K and a DPP reduction; MFMA: a 16-row tile over all of K).
//   COL  a workgroup owns a group of rows and its waves split the columns (K)
//        of those rows into contiguous slices; the per-wave sums are added in
//        wave order through LDS.  The split stays inside one workgroup on
//        purpose: combining partial sums across workgroups needs agent-scope
//        release/acquire, which on a multi-XCD gfx950 means writing back and
//        invalidating an XCD's whole L2 per arrival (measured: it turns a
//        37 us kernel into 1.5 ms).  Both traversals are deterministic.
// Every kernel is persistent-style: the grid is sized to the machine and each
// wave / workgroup walks a strided list of work items.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>

#include "dfk_kernels.h"

namespace dfk {

// Matrix-core steady loops: keep the next block's loads ahead of the current
// block's work.  Without a scheduling fence the compiler sinks those loads
// into (or past) the current block's MFMAs, and each block's weights then
// arrive only after its predecessor is done: memory and matrix work
// alternate instead of overlapping.
#ifndef DFK_FENCE_LOADS
#define DFK_FENCE_LOADS 1
#endif
#if DFK_FENCE_LOADS
#define DFK_ISSUE_FENCE() __builtin_amdgcn_sched_barrier(0)
#else
#define DFK_ISSUE_FENCE() ((void)0)
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
#ifndef DFK_VALU_BLOCK
#define DFK_VALU_BLOCK 512
#endif
constexpr int kValuBlock = DFK_VALU_BLOCK;  // 8 waves
constexpr int kMfmaRowBlock = 256;  // 4 waves, one tile group each

// ---------------------------------------------------------------- helpers --

// Weights are read exactly once per call: stream them with the non-temporal
// hint so they do not evict x / h / scratch from the caches.
__device__ __forceinline__ u32x4_t load_stream(const u32x4_t *p) {
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// c + sum of the 8 bf16 products of two 16-byte vectors, in element order.
__device__ __forceinline__ float dot8_bf16(u32x4_t w, u32x4_t x, float c) {
    c = dot2_bf16(w.x, x.x, c);
    c = dot2_bf16(w.y, x.y, c);
    c = dot2_bf16(w.z, x.z, c);
    c = dot2_bf16(w.w, x.w, c);
    return c;
}

__device__ __forceinline__ float bf16_lo(unsigned v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned v) {
    return __builtin_bit_cast(float, v & 0xffff0000u);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v) {
    // Lanes a row mask disables read 0, the identity of the sum.
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes of a wave with a fixed DPP pattern; the total lands in
// lane 63 (other lanes hold partial sums).  quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror, row_bcast:15 (rows 1,3), row_bcast:31 (rows 2,3).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += dpp_f32<0xb1>(v);
    v += dpp_f32<0x4e>(v);
    v += dpp_f32<0x141>(v);
    v += dpp_f32<0x140>(v);
    v += dpp_f32<0x142, 0xa>(v);
    v += dpp_f32<0x143, 0xc>(v);
    return v;
}

// SiLU(g) * u with SiLU(z) = z / (1 + e^-z).  For very negative z, e^-z
// overflows to +inf and the quotient is -0 (the limit), never NaN.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t to_bf16_rne(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Split 8 fp32 values into bf16 hi = RNE(v) and lo = RNE(v - hi).
__device__ __forceinline__ void split_hi_lo(f32x4_t a, f32x4_t b, bf16x8_t &hi, bf16x8_t &lo) {
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __bf16 h = (__bf16)v[i];
        hi[i] = h;
        lo[i] = (__bf16)(v[i] - (float)h);
    }
}


// ------------------------------------------------------------- arguments --

struct GateUpArgs {
    const uint16_t *x;
    const uint16_t *wg;
    const uint16_t *wu;
    float *h;
    int B, K, N;  // batch, d_model, d_ff
    int C;        // 16-byte chunks per weight row (K / 8)
    int groups;   // work items: row groups (ROW: per wave, COL: per workgroup)
    int ldw;      // elements from one row of W_gate (and of W_up) to the next: K, or 2K row-interleaved
    const uint8_t *qg, *qu;  // FP8-weight matrix-core kernels: E4M3 codes [N][K]
    const float *sg, *su;    //   and row scales [N]
    const uint16_t *gain;  // RMS normalization (NORM kernels only): gain [d_model]
    double eps;            //   and epsilon
};

struct DownArgs {
    const float *h;
    const uint16_t *wd;
    uint16_t *y;
    int B, K, M;  // batch, d_ff, d_model
    int C, groups;
    const uint8_t *qd;  // FP8-weight matrix-core kernels: E4M3 codes [M][K]
    const float *sd;    //   and row scales [M]
};

// ================================================== VALU building blocks ==
//
// Lane l of a wave takes chunks c_beg + l, c_beg + l + 64, ... of each weight
// row it streams: every load instruction moves 64 x 16 B = 1 KB of one row.
// U groups of loads are in flight per lane; a group past the end of the range
// is skipped by a wave-uniform branch, and the last partial group clamps its
// addresses (in bounds) while the lanes past the end skip the arithmetic.

// gate-up: R gate rows and the same R up rows; x from LDS ([B][C] chunks).
template <int B, int R, int U>
__device__ __forceinline__ void gu_valu_accumulate(const u32x4_t *const (&rg)[R], const u32x4_t *const (&ru)[R],
                                                   const u32x4_t *xs, int C, int c_beg, int c_end, int lane,
                                                   float (&ag)[R][B], float (&au)[R][B]) {
    for (int c0 = c_beg; c0 < c_end; c0 += kWave * U) {
        u32x4_t wgv[U][R], wuv[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u == 0 || c0 + kWave * u < c_end) {
                const int c = min(c0 + kWave * u + lane, c_end - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    wgv[u][r] = load_stream(rg[r] + c);
                    wuv[u][r] = load_stream(ru[r] + c);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + kWave * u + lane;
            if (c < c_end) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const u32x4_t xv = xs[b * C + c];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        ag[r][b] = dot8_bf16(wgv[u][r], xv, ag[r][b]);
                        au[r][b] = dot8_bf16(wuv[u][r], xv, au[r][b]);
                    }
                }
            }
        }
    }
}

// down: R rows of W_down; h from LDS (HLDS: all of h, [B][2C] f32x4) or
// straight from global memory through the caches.
template <int B, int R, int U, bool HLDS>
__device__ __forceinline__ void dn_valu_accumulate(const u32x4_t *const (&rd)[R], const f32x4_t *hg,
                                                   const f32x4_t *hl, int C, int c_beg, int c_end, int lane,
                                                   float (&acc)[R][B]) {
    for (int c0 = c_beg; c0 < c_end; c0 += kWave * U) {
        u32x4_t wv[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u == 0 || c0 + kWave * u < c_end) {
                const int c = min(c0 + kWave * u + lane, c_end - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) wv[u][r] = load_stream(rd[r] + c);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + kWave * u + lane;
            if (c < c_end) {
                f32x4_t hv[B][2];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const size_t o = (size_t)b * 2 * C + 2 * c;
                    hv[b][0] = HLDS ? hl[o] : hg[o];
                    hv[b][1] = HLDS ? hl[o + 1] : hg[o + 1];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4_t w = wv[u][r];
                    const float w0 = bf16_lo(w.x), w1 = bf16_hi(w.x), w2 = bf16_lo(w.y), w3 = bf16_hi(w.y),
                                w4 = bf16_lo(w.z), w5 = bf16_hi(w.z), w6 = bf16_lo(w.w), w7 = bf16_hi(w.w);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const f32x4_t h0 = hv[b][0], h1 = hv[b][1];
                        float t = acc[r][b];
                        t = fmaf(w0, h0.x, t);
                        t = fmaf(w1, h0.y, t);
                        t = fmaf(w2, h0.z, t);
                        t = fmaf(w3, h0.w, t);
                        t = fmaf(w4, h1.x, t);
                        t = fmaf(w5, h1.y, t);
                        t = fmaf(w6, h1.z, t);
                        t = fmaf(w7, h1.w, t);
                        acc[r][b] = t;
                    }
                }
            }
        }
    }
}

// Stage `n` 16-byte vectors from global memory into LDS (whole workgroup).
// Up to 8 loads per thread are issued before their stores, so the staging
// costs about one memory latency per 8 x blockDim vectors, not one per
// blockDim.
template <typename T>
__device__ __forceinline__ void stage_lds(T *dst, const T *src, int n) {
    constexpr int kBatch = 8;
    const int step = blockDim.x;
    for (int base = threadIdx.x; base < n; base += kBatch * step) {
        T v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (base + q * step < n) v[q] = src[base + q * step];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (base + q * step < n) dst[base + q * step] = v[q];
    }
    __syncthreads();
}

// stage_lds for data other workgroups of the same launch wrote with
// device-coherent stores: device-coherent 8-byte loads (they bypass the
// caches that are not coherent across the chip's dies), kValuBlock threads.
__device__ __forceinline__ void stage_lds_coherent(f32x4_t *dst, const f32x4_t *src, int n) {
    constexpr int kBatch = 8;
    constexpr int step = kValuBlock;
    unsigned long long *s = reinterpret_cast<unsigned long long *>(const_cast<f32x4_t *>(src));
    unsigned long long *d = reinterpret_cast<unsigned long long *>(dst);
    const int n2 = 2 * n;
    for (int base = threadIdx.x; base < n2; base += kBatch * step) {
        unsigned long long v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (base + q * step < n2)
                v[q] = __hip_atomic_load(s + base + q * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (base + q * step < n2) d[base + q * step] = v[q];
    }
    __syncthreads();
}

// ---------------------------------------------------- RMS normalization ----
//
// xn[b,k] = bf16_RNE((x[b,k] * inv_b) * gain[k]), inv_b = 1 / sqrt(mean_k
// x[b,k]^2 + eps): Llama-style RMSNorm ahead of the gate and up projections
// (the GPULlama3.java pull-request page fuses RMS normalization with them).
// Rounding xn to bf16 decides the projections' inputs, so it is taken from
// fp64 values, rounded once (no detour through binary32, which would round
// twice).

__device__ __forceinline__ double widen_bf16_f64(uint32_t bits16) { return (double)__uint_as_float(bits16 << 16); }

// Nearest bf16 of a double, ties to even, rounded once: 8 significant bits,
// the binary32 exponent range, subnormals down to 2^-133, overflow to
// infinity, NaN to the quiet NaN 0x7FC0.  With |d| in [2^e, 2^(e+1)) (e
// clamped to [-126, 128]), C = 1.5 * 2^(e+45) has an fp64 ulp of 2^(e-7), the
// bf16 spacing at that binade (2^-133 for the subnormals), and |d| + C stays in
// C's binade: the fp64 addition rounds |d| to that spacing, ties to even, and
// subtracting C again is exact.  The result is then exact in binary32
// (2^128 and above become infinity there).
__device__ __forceinline__ uint32_t bf16_rne_from_f64(double d) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(d);
    const uint32_t hi = (uint32_t)(u >> 32);
    uint32_t e = hi & 0x7FF00000u;
    e = min(max(e, (1023u - 126u) << 20), (1023u + 128u) << 20);
    const double c = __longlong_as_double((long long)((unsigned long long)(e + (45u << 20) + 0x00080000u) << 32));
    const double r = (fabs(d) + c) - c;
    const uint32_t bits = (__float_as_uint((float)r) >> 16) | ((hi >> 16) & 0x8000u);
    return d != d ? 0x7FC0u : bits;
}

// Sum of squares of one 16-byte chunk (8 values, in column order) added to ss.
__device__ __forceinline__ double rms_sumsq_chunk(u32x4_t v, double ss) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double lo = widen_bf16_f64(w[e] & 0xFFFFu), hi = widen_bf16_f64(w[e] >> 16);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
    }
    return ss;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
    // both halves moved with the same pattern; disabled lanes read +0.0
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// The fp64 sum over the 64 lanes in the DPP pattern of wave_sum_to_lane63;
// the total lands in lane 63.
__device__ __forceinline__ double wave_sum_f64_to_lane63(double v) {
    v += dpp_f64<0xb1>(v);
    v += dpp_f64<0x4e>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    v += dpp_f64<0x142, 0xa>(v);
    v += dpp_f64<0x143, 0xc>(v);
    return v;
}

// The normalization code runs in workgroups of kValuBlock threads (the VALU
// gate-up kernels and the standalone kernel); the size is a constant so that
// it never has to be read from the dispatch packet, a memory load whose wait
// would also wait for the weight loads in flight.
constexpr int kNormThreads = kValuBlock;

// inv_b = 1 / sqrt(ss_b / K + eps) for b < B from every thread's partial sum
// ss[b]: the wave sums, then the waves' in wave order through LDS (part:
// B * kNormThreads / 64 doubles).  Every thread returns the same values.
template <int MAXB>
__device__ void rms_inv_from_partials(double (&ss)[MAXB], int B, int K, double eps, double *part,
                                      double (&inv)[MAXB]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    constexpr int waves = kNormThreads / kWave;
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
        const double t = wave_sum_f64_to_lane63(ss[b]);
        if (b < B && lane == kWave - 1) part[b * waves + wave] = t;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
        double s = 0.0;
        if (b < B)
            for (int w = 0; w < waves; ++w) s += part[b * waves + w];
        inv[b] = 1.0 / sqrt(s / (double)K + eps);
    }
}

// One 16-byte chunk (8 columns) of a row, normalized: (x * inv) * gain in
// fp64, rounded to bf16.
__device__ __forceinline__ u32x4_t rms_apply_chunk(u32x4_t v, u32x4_t g, double inv) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = bf16_rne_from_f64((widen_bf16_f64(w[e] & 0xFFFFu) * inv) * widen_bf16_f64(gw[e] & 0xFFFFu));
        const uint32_t hi = bf16_rne_from_f64((widen_bf16_f64(w[e] >> 16) * inv) * widen_bf16_f64(gw[e] >> 16));
        o[e] = lo | (hi << 16);
    }
    return u32x4_t{o[0], o[1], o[2], o[3]};
}

// A thread's first kGainRegs gain chunks (c = tid + i * kNormThreads), loaded
// ahead of x so that they arrive with it (indices clamped into the row).
constexpr int kGainRegs = 2;
__device__ __forceinline__ void rms_gain_prefetch(const uint16_t *gain, int C, u32x4_t (&g)[kGainRegs]) {
    const u32x4_t *gg = reinterpret_cast<const u32x4_t *>(gain);
#pragma unroll
    for (int i = 0; i < kGainRegs; ++i) g[i] = gg[min((int)threadIdx.x + i * kNormThreads, C - 1)];
}

// Normalize x staged in LDS ([B][C] chunks) in place (whole workgroup).  Each
// thread sums and rewrites its chunks c = tid, tid + kNormThreads, ... of
// every row, in that order.
template <int B>
__device__ void rms_normalize_lds(u32x4_t *xs, const GateUpArgs &a, double *part, const u32x4_t (&greg)[kGainRegs]) {
    double ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = 0.0;
    for (int c = threadIdx.x; c < a.C; c += kNormThreads)
#pragma unroll
        for (int b = 0; b < B; ++b) ss[b] = rms_sumsq_chunk(xs[(size_t)b * a.C + c], ss[b]);
    double inv[B];
    rms_inv_from_partials<B>(ss, B, a.K, a.eps, part, inv);
    auto apply = [&](int c, u32x4_t g) {
#pragma unroll
        for (int b = 0; b < B; ++b) xs[(size_t)b * a.C + c] = rms_apply_chunk(xs[(size_t)b * a.C + c], g, inv[b]);
    };
#pragma unroll
    for (int i = 0; i < kGainRegs; ++i) {
        const int c = threadIdx.x + i * kNormThreads;
        if (c < a.C) apply(c, greg[i]);
    }
    const u32x4_t *gg = reinterpret_cast<const u32x4_t *>(a.gain);
    for (int c = threadIdx.x + kGainRegs * kNormThreads; c < a.C; c += kNormThreads) apply(c, gg[c]);
    __syncthreads();
}

// Standalone: one workgroup per batch row, of the VALU gate-up kernels' size
// and with their order of summation, so that it gives the x they normalize
// in LDS bit for bit.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t *x, const uint16_t *gain, double eps,
                                                               uint16_t *xn, int K) {
    __shared__ double part[kNormThreads / kWave];
    const int C = K / 8;
    const int tid = threadIdx.x;
    constexpr int nt = kNormThreads;
    const u32x4_t *row = reinterpret_cast<const u32x4_t *>(x + (size_t)blockIdx.x * K);
    const u32x4_t *gg = reinterpret_cast<const u32x4_t *>(gain);
    u32x4_t *out = reinterpret_cast<u32x4_t *>(xn + (size_t)blockIdx.x * K);
    u32x4_t greg[kGainRegs], xr[kGainRegs];
    rms_gain_prefetch(gain, C, greg);
#pragma unroll
    for (int i = 0; i < kGainRegs; ++i) xr[i] = row[min(tid + i * nt, C - 1)];
    double ss[1] = {0.0};
#pragma unroll
    for (int i = 0; i < kGainRegs; ++i)
        if (tid + i * nt < C) ss[0] = rms_sumsq_chunk(xr[i], ss[0]);
    for (int c = tid + kGainRegs * nt; c < C; c += nt) ss[0] = rms_sumsq_chunk(row[c], ss[0]);
    double inv[1];
    rms_inv_from_partials<1>(ss, 1, K, eps, part, inv);
#pragma unroll
    for (int i = 0; i < kGainRegs; ++i)
        if (tid + i * nt < C) out[tid + i * nt] = rms_apply_chunk(xr[i], greg[i], inv[0]);
    for (int c = tid + kGainRegs * nt; c < C; c += nt) out[c] = rms_apply_chunk(row[c], gg[c], inv[0]);
}

// ==================================================== VALU row kernels =====
//
// ROW: a wave owns R rows (gate-up: R neurons, i.e. R rows of W_gate and the
// same R rows of W_up) for the whole of K; lane partials are summed with the
// DPP butterfly and lane 63 runs the epilogue.  Persistent: wave w takes row
// groups w, w + total_waves, ...

// The row kernels walk a wave's (row group, load group) sequence flattened,
// with two register buffers: the next load group (possibly the next row
// group's first) is issued before the current one is multiplied, so loads
// stay in flight across row boundaries and under the reductions.  Loads are
// unconditional (addresses clamped into the row, the lanes past its end
// masked at use) and the last one or two groups are peeled, so every wait in
// the loop is for the oldest loads only.
// The body, shared with the persistent MLP kernel: xs is the workgroup's LDS,
// [B][C] chunks (NORM: then B * 8 doubles); wave_id (wave-uniform) and
// total_waves place the wave in the persistent walk.
// COH: h is stored device-coherent, for readers in other workgroups of the
// same launch.
template <int B, int R, int U, bool NORM, bool COH = false>
__device__ __forceinline__ void gate_up_row_body(const GateUpArgs &a, u32x4_t *xs, int wave_id, int total_waves) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int G = kWave * U;                     // chunks per load group
    const int gpr = (a.C + G - 1) / G;               // load groups per row group
    const int rows = max(0, (a.groups - wave_id + total_waves - 1) / total_waves);
    const int total = rows * gpr;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    float ag[R][B], au[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;
    auto load = [&](u32x4_t (&wg)[U][R], u32x4_t (&wu)[U][R], int k, int j) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(gi * R + r, a.N - 1);
            const u32x4_t *pg = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)n * a.ldw);
            const u32x4_t *pu = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)n * a.ldw);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(j * G + kWave * u + lane, a.C - 1);
                wg[u][r] = load_stream(pg + c);
                wu[u][r] = load_stream(pu + c);
            }
        }
    };
    auto compute = [&](const u32x4_t (&wg)[U][R], const u32x4_t (&wu)[U][R], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = j * G + kWave * u + lane;
            const bool ok = c < a.C;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const u32x4_t xv = ok ? xs[b * a.C + c] : zero;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    ag[r][b] = dot8_bf16(wg[u][r], xv, ag[r][b]);
                    au[r][b] = dot8_bf16(wu[u][r], xv, au[r][b]);
                }
            }
        }
    };
    auto finish = [&](int k) {  // a row group's last load group is done: reduce, SiLU * u, store
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                ag[r][b] = wave_sum_to_lane63(ag[r][b]);
                au[r][b] = wave_sum_to_lane63(au[r][b]);
            }
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = gi * R + r;
                if (n < a.N)
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float v = silu_mul(ag[r][b], au[r][b]);
                        if constexpr (COH)
                            __hip_atomic_store(a.h + (size_t)b * a.N + n, v, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        else
                            a.h[(size_t)b * a.N + n] = v;
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;
    };
    auto step = [&](const u32x4_t (&wg)[U][R], const u32x4_t (&wu)[U][R], int k, int j) {
        compute(wg, wu, j);
        if (j == gpr - 1) finish(k);
    };
    auto next = [&](int &k, int &j) {
        if (++j == gpr) {
            j = 0;
            ++k;
        }
    };
    // the walk from item t on; buffer A holds item t (its loads issued)
    auto walk = [&](auto &ga, auto &ua, auto &gb, auto &ub, int t, int ka, int ja) {
        for (; t + 2 < total; t += 2) {
            int kb = ka, jb = ja;
            next(kb, jb);
            load(gb, ub, kb, jb);
            __builtin_amdgcn_sched_barrier(0);
            step(ga, ua, ka, ja);
            int kc = kb, jc = jb;
            next(kc, jc);
            load(ga, ua, kc, jc);
            __builtin_amdgcn_sched_barrier(0);
            step(gb, ub, kb, jb);
            ka = kc;
            ja = jc;
        }
        if (t + 1 < total) {
            int kb = ka, jb = ja;
            next(kb, jb);
            load(gb, ub, kb, jb);
            __builtin_amdgcn_sched_barrier(0);
            step(ga, ua, ka, ja);
            step(gb, ub, kb, jb);
        } else {
            step(ga, ua, ka, ja);
        }
    };
    u32x4_t g0[U][R], u0[U][R], g1[U][R], u1[U][R];
    int k0 = 0, j0 = 0;
    // the first weight loads go out before x is staged (they do not need it;
    // a wave without work loads a clamped row and leaves after the barrier)
    load(g0, u0, k0, j0);
    u32x4_t greg[kGainRegs];
    if constexpr (NORM) rms_gain_prefetch(a.gain, a.C, greg);
    __builtin_amdgcn_sched_barrier(0);
    stage_lds(xs, reinterpret_cast<const u32x4_t *>(a.x), B * a.C);
    if constexpr (NORM) {
        // the second load group goes out before the normalization, so that
        // HBM keeps streaming under its arithmetic
        int k1 = k0, j1 = j0;
        next(k1, j1);
        const bool more = total > 1;
        if (more) load(g1, u1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        rms_normalize_lds<B>(xs, a, reinterpret_cast<double *>(xs + (size_t)B * a.C), greg);
        if (wave_id >= a.groups) return;
        step(g0, u0, k0, j0);
        if (more) walk(g1, u1, g0, u0, 1, k1, j1);
    } else {
        if (wave_id >= a.groups) return;
        walk(g0, u0, g1, u1, 0, k0, j0);
    }
}

template <int B, int R, int U, bool NORM>
__global__ __launch_bounds__(kValuBlock) void gate_up_valu_row_kernel(GateUpArgs a) {
    extern __shared__ u32x4_t xs[];
    constexpr int waves = kValuBlock / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    gate_up_row_body<B, R, U, NORM>(a, xs, wave_id, gridDim.x * waves);
}

// (same flattened, double-buffered walk as the gate-up row kernel; without h
// in LDS a load group also carries its h values, issued before its weights)
//
// The body, shared with the persistent MLP kernel: hs is the workgroup's LDS
// (HLDS: [B][2C]).  before_stage() runs after the first weight loads are
// issued and before h is read (the persistent kernel's grid barrier); with
// poison set every output is NaN (a barrier that timed out).
// COH (with HLDS): h, written in this launch, is staged with device-coherent
// loads.
template <int B, int R, int U, bool HLDS, bool COH, class Hook>
__device__ __forceinline__ void down_row_body(const DownArgs &a, f32x4_t *hs, int wave_id, int total_waves,
                                              Hook before_stage) {
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    constexpr int G = kWave * U;
    constexpr int HU = HLDS ? 1 : U;  // h registers per group (none used with h in LDS)
    const int gpr = (a.C + G - 1) / G;
    const int rows = max(0, (a.groups - wave_id + total_waves - 1) / total_waves);
    const int total = rows * gpr;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    bool poison = false;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    auto load = [&](u32x4_t (&wv)[U][R], f32x4_t (&hv)[HU][B][2], int k, int j) {
        if constexpr (!HLDS) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(j * G + kWave * u + lane, a.C - 1);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    hv[u][b][0] = hg[(size_t)b * 2 * a.C + 2 * c];
                    hv[u][b][1] = hg[(size_t)b * 2 * a.C + 2 * c + 1];
                }
            }
        }
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = min(gi * R + r, a.M - 1);
            const u32x4_t *pw = reinterpret_cast<const u32x4_t *>(a.wd + (size_t)m * a.K);
#pragma unroll
            for (int u = 0; u < U; ++u) wv[u][r] = load_stream(pw + min(j * G + kWave * u + lane, a.C - 1));
        }
    };
    auto compute = [&](const u32x4_t (&wv)[U][R], const f32x4_t (&hv)[HU][B][2], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = j * G + kWave * u + lane;
            const bool ok = c < a.C;
            f32x4_t h2[B][2];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if constexpr (HLDS) {
                    const int cc = min(c, a.C - 1);
                    h2[b][0] = hs[(size_t)b * 2 * a.C + 2 * cc];
                    h2[b][1] = hs[(size_t)b * 2 * a.C + 2 * cc + 1];
                } else {
                    h2[b][0] = hv[u][b][0];
                    h2[b][1] = hv[u][b][1];
                }
                if (!ok) h2[b][0] = h2[b][1] = fzero;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4_t w = wv[u][r];
                const float w0 = bf16_lo(w.x), w1 = bf16_hi(w.x), w2 = bf16_lo(w.y), w3 = bf16_hi(w.y),
                            w4 = bf16_lo(w.z), w5 = bf16_hi(w.z), w6 = bf16_lo(w.w), w7 = bf16_hi(w.w);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const f32x4_t h0 = h2[b][0], h1 = h2[b][1];
                    float t = acc[r][b];
                    t = fmaf(w0, h0.x, t);
                    t = fmaf(w1, h0.y, t);
                    t = fmaf(w2, h0.z, t);
                    t = fmaf(w3, h0.w, t);
                    t = fmaf(w4, h1.x, t);
                    t = fmaf(w5, h1.y, t);
                    t = fmaf(w6, h1.z, t);
                    t = fmaf(w7, h1.w, t);
                    acc[r][b] = t;
                }
            }
        }
    };
    auto finish = [&](int k) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int m = gi * R + r;
                if (m < a.M)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        a.y[(size_t)b * a.M + m] = to_bf16_rne(poison ? __builtin_nanf("") : acc[r][b]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    };
    auto step = [&](const u32x4_t (&wv)[U][R], const f32x4_t (&hv)[HU][B][2], int k, int j) {
        compute(wv, hv, j);
        if (j == gpr - 1) finish(k);
    };
    auto next = [&](int &k, int &j) {
        if (++j == gpr) {
            j = 0;
            ++k;
        }
    };
    u32x4_t w0[U][R], w1[U][R];
    f32x4_t h0[HU][B][2], h1[HU][B][2];
    int k0 = 0, j0 = 0;
    // the first loads go out before h is staged (a wave without work loads a
    // clamped row and leaves after the barrier); h must not be read before
    // before_stage() (h registers come with the weights only without HLDS)
    load(w0, h0, k0, j0);
    __builtin_amdgcn_sched_barrier(0);
    poison = before_stage();
    if constexpr (HLDS && COH) stage_lds_coherent(hs, hg, B * 2 * a.C);
    else if constexpr (HLDS) stage_lds(hs, hg, B * 2 * a.C);
    if (wave_id >= a.groups) return;
    int t = 0;
    for (; t + 2 < total; t += 2) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(w1, h1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(w0, h0, k0, j0);
        int k2 = k1, j2 = j1;
        next(k2, j2);
        load(w0, h0, k2, j2);
        __builtin_amdgcn_sched_barrier(0);
        step(w1, h1, k1, j1);
        k0 = k2;
        j0 = j2;
    }
    if (t + 1 < total) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(w1, h1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(w0, h0, k0, j0);
        step(w1, h1, k1, j1);
    } else {
        step(w0, h0, k0, j0);
    }
}

template <int B, int R, int U, bool HLDS>
__global__ __launch_bounds__(kValuBlock) void down_valu_row_kernel(DownArgs a) {
    extern __shared__ f32x4_t hs[];
    constexpr int waves = kValuBlock / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    down_row_body<B, R, U, HLDS, false>(a, hs, wave_id, gridDim.x * waves, [] { return false; });
}

// ============================================= FP8 weights (row, VALU) =====
//
// Weight-only FP8 (the GPULlama3.java pull request fuses dequantization into
// the matrix-vector product): weights are OCP FP8 E4M3 codes with one fp32
// scale per row, W[r, c] = s[r] * e4m3(q[r, c]).  The codes stream from HBM
// (half the bytes of bf16) and are widened in registers; the row scale
// multiplies the row's fp32 sum once.  Same flattened, double-buffered row
// walk as the bf16 row kernels, one 16-byte load now carrying 16 weights.
// Each load group also loads its rows' scales (all lanes the same address),
// so the epilogue never waits on a load issued after the weights.

struct GateUpF8Args {
    const uint16_t *x;
    const uint8_t *qg, *qu;  // [N][K] E4M3 codes
    const float *sg, *su;    // [N] row scales
    float *h;
    int B, K, N;  // batch, d_model, d_ff
    int C;        // 16-byte x chunks per row (K / 8)
    int C16;      // 16-byte weight chunks per row (K / 16)
    int groups;
};

struct DownF8Args {
    const float *h;
    const uint8_t *qd;  // [M][K] E4M3 codes
    const float *sd;    // [M] row scales
    uint16_t *y;
    int B, K, M;  // batch, d_ff, d_model
    int C16;      // 16-byte weight chunks per row (K / 16)
    int groups;
};

// Two E4M3 codes (the low or high half of a word) as a bf16 pair; exact, every
// E4M3 value being a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 16 codes (k .. k+15) as two chunks of 8 bf16 (k .. k+7, k+8 .. k+15).
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t q, u32x4_t &lo, u32x4_t &hi) {
    lo = u32x4_t{e4m3x2_to_bf16x2<false>(q.x), e4m3x2_to_bf16x2<true>(q.x), e4m3x2_to_bf16x2<false>(q.y),
                 e4m3x2_to_bf16x2<true>(q.y)};
    hi = u32x4_t{e4m3x2_to_bf16x2<false>(q.z), e4m3x2_to_bf16x2<true>(q.z), e4m3x2_to_bf16x2<false>(q.w),
                 e4m3x2_to_bf16x2<true>(q.w)};
}

template <int B, int R, int U>
__global__ __launch_bounds__(kValuBlock) void gate_up_fp8_row_kernel(GateUpF8Args a) {
    extern __shared__ u32x4_t xs[];  // [B][C]
    constexpr int waves = kValuBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    const int total_waves = gridDim.x * waves;
    constexpr int G = kWave * U;  // weight chunks per load group
    const int gpr = (a.C16 + G - 1) / G;
    const int rows = max(0, (a.groups - wave_id + total_waves - 1) / total_waves);
    const int total = rows * gpr;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    float ag[R][B], au[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;
    struct Buf {
        u32x4_t g[U][R], u[U][R];
        float sg[R], su[R];
    };
    auto load = [&](Buf &f, int k, int j) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(gi * R + r, a.N - 1);
            const u32x4_t *pg = reinterpret_cast<const u32x4_t *>(a.qg + (size_t)n * a.K);
            const u32x4_t *pu = reinterpret_cast<const u32x4_t *>(a.qu + (size_t)n * a.K);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(j * G + kWave * u + lane, a.C16 - 1);
                f.g[u][r] = load_stream(pg + c);
                f.u[u][r] = load_stream(pu + c);
            }
            f.sg[r] = a.sg[n];
            f.su[r] = a.su[n];
        }
    };
    auto compute = [&](const Buf &f, int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = j * G + kWave * u + lane;
            const bool ok = c < a.C16;
            const int cc = min(c, a.C16 - 1);  // unconditional reads, masked after
            u32x4_t x0[B], x1[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                x0[b] = xs[b * a.C + 2 * cc];
                x1[b] = xs[b * a.C + 2 * cc + 1];
                if (!ok) x0[b] = x1[b] = zero;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                u32x4_t lo, hi;
                e4m3x16_to_bf16(f.g[u][r], lo, hi);
#pragma unroll
                for (int b = 0; b < B; ++b) ag[r][b] = dot8_bf16(hi, x1[b], dot8_bf16(lo, x0[b], ag[r][b]));
                e4m3x16_to_bf16(f.u[u][r], lo, hi);
#pragma unroll
                for (int b = 0; b < B; ++b) au[r][b] = dot8_bf16(hi, x1[b], dot8_bf16(lo, x0[b], au[r][b]));
            }
        }
    };
    auto finish = [&](const Buf &f, int k) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                ag[r][b] = wave_sum_to_lane63(ag[r][b]);
                au[r][b] = wave_sum_to_lane63(au[r][b]);
            }
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = gi * R + r;
                if (n < a.N)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        a.h[(size_t)b * a.N + n] = silu_mul(f.sg[r] * ag[r][b], f.su[r] * au[r][b]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;
    };
    auto step = [&](const Buf &f, int k, int j) {
        compute(f, j);
        if (j == gpr - 1) finish(f, k);
    };
    auto next = [&](int &k, int &j) {
        if (++j == gpr) {
            j = 0;
            ++k;
        }
    };
    Buf f0, f1;
    int k0 = 0, j0 = 0;
    load(f0, k0, j0);
    __builtin_amdgcn_sched_barrier(0);
    stage_lds(xs, reinterpret_cast<const u32x4_t *>(a.x), B * a.C);
    if (wave_id >= a.groups) return;
    int t = 0;
    for (; t + 2 < total; t += 2) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(f1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(f0, k0, j0);
        int k2 = k1, j2 = j1;
        next(k2, j2);
        load(f0, k2, j2);
        __builtin_amdgcn_sched_barrier(0);
        step(f1, k1, j1);
        k0 = k2;
        j0 = j2;
    }
    if (t + 1 < total) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(f1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(f0, k0, j0);
        step(f1, k1, j1);
    } else {
        step(f0, k0, j0);
    }
}

// Two E4M3 codes (the low or high half of a word) as two floats, exact.
template <bool HI>
__device__ __forceinline__ void e4m3x2_to_f32(uint32_t w, float &a, float &b) {
    const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
    a = v[0];
    b = v[1];
}

// K is cut into gridDim.y panels of CS weight chunks, each small enough that
// its slice of h (16 CS fp32 per batch row) sits in LDS; one panel writes y
// directly, several write scaled fp32 partial sums that panel_reduce_kernel
// adds.  In LDS each batch row's slice is four planes: plane q holds the
// q-th 16-byte quarter of every chunk (pitch CS + 1), so the 64 lanes of a
// wave, which take consecutive chunks, read consecutive 16-byte words of a
// plane (without the planes, lanes 4 chunks apart would share LDS banks).
template <int B, int R, int U>
__global__ __launch_bounds__(kValuBlock) void down_fp8_row_kernel(DownF8Args a, float *partial, int CS) {
    extern __shared__ f32x4_t hs[];  // [B][4][CS + 1]: this panel's h
    constexpr int waves = kValuBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    const int total_waves = gridDim.x * waves;
    const int panel = blockIdx.y, panels = gridDim.y;
    const int c_lo = panel * CS;
    const int cn = min(CS, a.C16 - c_lo);  // weight chunks in this panel
    const int HC = a.K / 4;                // f32x4 chunks of a whole h row
    const int P = CS + 1;                  // LDS pitch of a quarter plane
    const int HP = 4 * P;                  // LDS pitch of a panel's h row
    constexpr int G = kWave * U;
    const int gpr = (cn + G - 1) / G;
    const int rows = max(0, (a.groups - wave_id + total_waves - 1) / total_waves);
    const int total = rows * gpr;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    struct Buf {
        u32x4_t w[U][R];
        float s[R];
    };
    auto load = [&](Buf &f, int k, int j) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = min(gi * R + r, a.M - 1);
            const u32x4_t *pw = reinterpret_cast<const u32x4_t *>(a.qd + (size_t)m * a.K) + c_lo;
#pragma unroll
            for (int u = 0; u < U; ++u) f.w[u][r] = load_stream(pw + min(j * G + kWave * u + lane, cn - 1));
            f.s[r] = a.sd[m];
        }
    };
    auto compute = [&](const Buf &f, int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = j * G + kWave * u + lane;
            const bool ok = c < cn;
            const int cc = min(c, cn - 1);
            // 16 weights k = 16c .. 16c+15, in four quarters of four
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4_t hv[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    hv[b] = hs[(size_t)b * HP + q * P + cc];  // unconditional read, masked after
                    if (!ok) hv[b] = fzero;
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t word = q == 0 ? f.w[u][r].x : q == 1 ? f.w[u][r].y : q == 2 ? f.w[u][r].z
                                                                                                  : f.w[u][r].w;
                    float w0, w1, w2, w3;
                    e4m3x2_to_f32<false>(word, w0, w1);
                    e4m3x2_to_f32<true>(word, w2, w3);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        float t = acc[r][b];
                        t = fmaf(w0, hv[b].x, t);
                        t = fmaf(w1, hv[b].y, t);
                        t = fmaf(w2, hv[b].z, t);
                        t = fmaf(w3, hv[b].w, t);
                        acc[r][b] = t;
                    }
                }
            }
        }
    };
    auto finish = [&](const Buf &f, int k) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int m = gi * R + r;
                if (m < a.M)
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float v = f.s[r] * acc[r][b];
                        if (panels == 1) a.y[(size_t)b * a.M + m] = to_bf16_rne(v);
                        else partial[((size_t)panel * B + b) * a.M + m] = v;
                    }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    };
    auto step = [&](const Buf &f, int k, int j) {
        compute(f, j);
        if (j == gpr - 1) finish(f, k);
    };
    auto next = [&](int &k, int &j) {
        if (++j == gpr) {
            j = 0;
            ++k;
        }
    };
    Buf f0, f1;
    int k0 = 0, j0 = 0;
    load(f0, k0, j0);
    __builtin_amdgcn_sched_barrier(0);
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    {
        // this panel's slice of each of the B rows of h (4 cn quarters, the
        // whole row with one panel), quarter g of the slice to plane g % 4
        const int rc = 4 * cn;
        constexpr int kBatch = 8;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const f32x4_t *src = hg + (size_t)b * HC + 4 * c_lo;
            f32x4_t *dst = hs + (size_t)b * HP;
            for (int base = threadIdx.x; base < rc; base += kBatch * kValuBlock) {
                f32x4_t v[kBatch];
#pragma unroll
                for (int s = 0; s < kBatch; ++s)
                    if (base + s * kValuBlock < rc) v[s] = src[base + s * kValuBlock];
#pragma unroll
                for (int s = 0; s < kBatch; ++s) {
                    const int g = base + s * kValuBlock;
                    if (g < rc) dst[(g & 3) * P + (g >> 2)] = v[s];
                }
            }
        }
        __syncthreads();
    }
    if (wave_id >= a.groups) return;
    int t = 0;
    for (; t + 2 < total; t += 2) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(f1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(f0, k0, j0);
        int k2 = k1, j2 = j1;
        next(k2, j2);
        load(f0, k2, j2);
        __builtin_amdgcn_sched_barrier(0);
        step(f1, k1, j1);
        k0 = k2;
        j0 = j2;
    }
    if (t + 1 < total) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(f1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(f0, k0, j0);
        step(f1, k1, j1);
    } else {
        step(f0, k0, j0);
    }
}

// ================================================ down, VALU row K panels ====
//
// The down row walk for batches whose fp32 h does not fit in LDS whole: K is
// cut into gridDim.y panels of CS 16-byte weight chunks whose h slice
// ([B][8 CS] fp32) does; each panel's waves walk their rows over the panel
// only and write fp32 partial sums that panel_reduce_kernel adds (fixed
// order).  h is read from LDS, never through the caches.
template <int B, int R, int U>
__global__ __launch_bounds__(kValuBlock) void down_valu_panel_kernel(DownArgs a, float *partial, int CS) {
    extern __shared__ f32x4_t hs[];  // [B][2 CS]: this panel's h
    constexpr int waves = kValuBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    const int total_waves = gridDim.x * waves;
    const int panel = blockIdx.y;
    const int c_lo = panel * CS;
    const int cn = min(CS, a.C - c_lo);  // weight chunks in this panel
    const int HC = 2 * a.C;              // f32x4 chunks of a whole h row
    const int HP = 2 * CS;               // LDS pitch of a panel's h row
    constexpr int G = kWave * U;
    const int gpr = (cn + G - 1) / G;
    const int rows = max(0, (a.groups - wave_id + total_waves - 1) / total_waves);
    const int total = rows * gpr;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    auto load = [&](u32x4_t (&wv)[U][R], int k, int j) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = min(gi * R + r, a.M - 1);
            const u32x4_t *pw = reinterpret_cast<const u32x4_t *>(a.wd + (size_t)m * a.K) + c_lo;
#pragma unroll
            for (int u = 0; u < U; ++u) wv[u][r] = load_stream(pw + min(j * G + kWave * u + lane, cn - 1));
        }
    };
    auto compute = [&](const u32x4_t (&wv)[U][R], int j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = j * G + kWave * u + lane;
            const bool ok = c < cn;
            const int cc = min(c, cn - 1);
            f32x4_t h2[B][2];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                h2[b][0] = hs[(size_t)b * HP + 2 * cc];  // unconditional reads, masked after
                h2[b][1] = hs[(size_t)b * HP + 2 * cc + 1];
                if (!ok) h2[b][0] = h2[b][1] = fzero;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4_t w = wv[u][r];
                const float w0 = bf16_lo(w.x), w1 = bf16_hi(w.x), w2 = bf16_lo(w.y), w3 = bf16_hi(w.y),
                            w4 = bf16_lo(w.z), w5 = bf16_hi(w.z), w6 = bf16_lo(w.w), w7 = bf16_hi(w.w);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const f32x4_t h0 = h2[b][0], h1 = h2[b][1];
                    float t = acc[r][b];
                    t = fmaf(w0, h0.x, t);
                    t = fmaf(w1, h0.y, t);
                    t = fmaf(w2, h0.z, t);
                    t = fmaf(w3, h0.w, t);
                    t = fmaf(w4, h1.x, t);
                    t = fmaf(w5, h1.y, t);
                    t = fmaf(w6, h1.z, t);
                    t = fmaf(w7, h1.w, t);
                    acc[r][b] = t;
                }
            }
        }
    };
    auto finish = [&](int k) {
        const int gi = wave_id + k * total_waves;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int m = gi * R + r;
                if (m < a.M)
#pragma unroll
                    for (int b = 0; b < B; ++b) partial[((size_t)panel * B + b) * a.M + m] = acc[r][b];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
    };
    auto step = [&](const u32x4_t (&wv)[U][R], int k, int j) {
        compute(wv, j);
        if (j == gpr - 1) finish(k);
    };
    auto next = [&](int &k, int &j) {
        if (++j == gpr) {
            j = 0;
            ++k;
        }
    };
    u32x4_t w0[U][R], w1[U][R];
    int k0 = 0, j0 = 0;
    load(w0, k0, j0);
    __builtin_amdgcn_sched_barrier(0);
    {
        // this panel's slice of each of the B rows of h (2 cn chunks)
        const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
        const int rc = 2 * cn;
        constexpr int kBatch = 8;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const f32x4_t *src = hg + (size_t)b * HC + 2 * c_lo;
            f32x4_t *dst = hs + (size_t)b * HP;
            for (int base = threadIdx.x; base < rc; base += kBatch * kValuBlock) {
                f32x4_t v[kBatch];
#pragma unroll
                for (int s = 0; s < kBatch; ++s)
                    if (base + s * kValuBlock < rc) v[s] = src[base + s * kValuBlock];
#pragma unroll
                for (int s = 0; s < kBatch; ++s)
                    if (base + s * kValuBlock < rc) dst[base + s * kValuBlock] = v[s];
            }
        }
        __syncthreads();
    }
    if (wave_id >= a.groups) return;
    int t = 0;
    for (; t + 2 < total; t += 2) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(w1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(w0, k0, j0);
        int k2 = k1, j2 = j1;
        next(k2, j2);
        load(w0, k2, j2);
        __builtin_amdgcn_sched_barrier(0);
        step(w1, k1, j1);
        k0 = k2;
        j0 = j2;
    }
    if (t + 1 < total) {
        int k1 = k0, j1 = j0;
        next(k1, j1);
        load(w1, k1, j1);
        __builtin_amdgcn_sched_barrier(0);
        step(w0, k0, j0);
        step(w1, k1, j1);
    } else {
        step(w0, k0, j0);
    }
}

// ============================================ persistent MLP (row, VALU) =====
//
// Both kernels of the MLP in one cooperative launch (every workgroup
// resident): the gate-up row walk, then a grid-wide barrier, then the down row
// walk, so that no launch gap separates them and W_down starts streaming
// while the slowest gate-up waves finish.  Each wave issues its first W_down
// load group before the barrier (the weights do not depend on h); h is staged
// into LDS (where x was) after it.  Barrier state: two words, zero before the
// first launch and left zero-count after each (the last workgroup to arrive
// resets the count and advances the generation the others wait on).

// Barrier state (kBarrierWords words, zero before the first launch): 16 group
// counters, a top counter and 16 copies of the generation, each in its own
// 128-byte line.  Workgroup w arrives on group counter w % 16; the last of a
// group to arrive bumps the top counter; the last group resets the counters
// and advances every copy of the generation; workgroup w waits on copy w % 16.
// Spreading the arrivals keeps the same-address atomics, which the memory
// system serializes, to a few dozen per address.
struct GridBarrier {
    unsigned *words;
};
constexpr int kBarrierGroups = 16;
constexpr int kBarrierLine = 32;  // words per 128-byte line
__device__ __forceinline__ unsigned *bar_group(const GridBarrier &g, int i) { return g.words + i * kBarrierLine; }
__device__ __forceinline__ unsigned *bar_top(const GridBarrier &g) { return g.words + kBarrierGroups * kBarrierLine; }
__device__ __forceinline__ unsigned *bar_gen(const GridBarrier &g, int i) {
    return g.words + (kBarrierGroups + 1 + i) * kBarrierLine;
}

// Upper bound on the spin of a waiting workgroup (each turn sleeps ~128
// cycles plus a memory round trip): far beyond any launch's skew, it only
// keeps a launch whose workgroups are not all resident from hanging.
constexpr unsigned kBarrierSpins = 1u << 20;

// The protocol uses no cache-maintenance fences: a device-scope release or
// acquire writes back or invalidates a whole L2 per die, far too slow here.
// Instead h travels device-coherent: written with coherent stores that each
// wave waits to complete before its workgroup arrives, and read (after the
// generation moves) with coherent loads.

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): this wave's stores are
// complete.
__device__ __forceinline__ void wait_stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The launch's generation as workgroup w sees it, read at the kernel's start:
// it moves only when every workgroup of this launch has arrived.
__device__ __forceinline__ unsigned grid_generation(const GridBarrier &g) {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(bar_gen(g, blockIdx.x % kBarrierGroups), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Arrive and wait (whole workgroup, after every wave's coherent h stores
// completed).  Returns true (every thread) when the wait gave up.
__device__ bool grid_sync(const GridBarrier &g, unsigned gen) {
    __shared__ int timed_out;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nb = gridDim.x, grp = blockIdx.x % kBarrierGroups;
        const int groups = min(nb, kBarrierGroups);
        const unsigned in_group = (unsigned)((nb - grp + kBarrierGroups - 1) / kBarrierGroups);
        const unsigned a = __hip_atomic_fetch_add(bar_group(g, grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (a == in_group - 1) {
            __hip_atomic_store(bar_group(g, grp), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned b = __hip_atomic_fetch_add(bar_top(g), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (b == (unsigned)groups - 1) {
                __hip_atomic_store(bar_top(g), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                wait_stores_done();
                for (int i = 0; i < kBarrierGroups; ++i)
                    __hip_atomic_fetch_add(bar_gen(g, i), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        int bad = 0;
        unsigned spins = 0;
        while (__hip_atomic_load(bar_gen(g, grp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins == kBarrierSpins) {
                bad = 1;
                break;
            }
        }
        timed_out = bad;
    }
    __syncthreads();
    return timed_out != 0;
}

template <int B, int RG, int UG, int RD, int UD>
__global__ __launch_bounds__(kValuBlock) void mlp_valu_row_persistent_kernel(GateUpArgs ga, DownArgs da,
                                                                              GridBarrier bar) {
    extern __shared__ u32x4_t smem[];  // x [B][d_model / 8], later h [B][2 d_ff / 8]
    constexpr int waves = kValuBlock / kWave;
    const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * waves + threadIdx.x / kWave);
    const int total_waves = gridDim.x * waves;
    const unsigned gen = grid_generation(bar);
    gate_up_row_body<B, RG, UG, false, true>(ga, smem, wave_id, total_waves);
    wait_stores_done();  // this wave's coherent h stores are complete before its workgroup arrives
    down_row_body<B, RD, UD, true, true>(da, reinterpret_cast<f32x4_t *>(smem), wave_id, total_waves,
                                         [&] { return grid_sync(bar, gen); });
}

// ==================================================== VALU col kernels =====
//
// COL: a workgroup owns R rows; its waves split the columns (K) of those rows
// into contiguous slices, each wave streams its slice of every row with lanes
// along K, and the waves' DPP-reduced sums are added in wave order through
// LDS before wave 0 runs the epilogue.  More waves per row than ROW: the
// choice when rows are few or long.  Persistent over row groups.

template <int B, int R, int U, bool NORM>
__global__ __launch_bounds__(kValuBlock) void gate_up_valu_col_kernel(GateUpArgs a) {
    constexpr int NV = 2 * R * B;
    // x [B][C], then red [waves][NV] floats (NORM: then B * waves doubles)
    extern __shared__ u32x4_t smem[];
    u32x4_t *xs = smem;
    float *red = reinterpret_cast<float *>(smem + (size_t)B * a.C);
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    u32x4_t greg[kGainRegs];
    if constexpr (NORM) rms_gain_prefetch(a.gain, a.C, greg);
    stage_lds(xs, reinterpret_cast<const u32x4_t *>(a.x), B * a.C);
    if constexpr (NORM) rms_normalize_lds<B>(xs, a, reinterpret_cast<double *>(red + waves * NV), greg);
    const int cw = (a.C + waves - 1) / waves;
    const int c_beg = min(wave * cw, a.C);
    const int c_end = min(c_beg + cw, a.C);

    for (int gi = blockIdx.x; gi < a.groups; gi += gridDim.x) {
        const u32x4_t *rg[R];
        const u32x4_t *ru[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(gi * R + r, a.N - 1);
            rg[r] = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)n * a.ldw);
            ru[r] = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)n * a.ldw);
        }
        float ag[R][B], au[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;
        gu_valu_accumulate<B, R, U>(rg, ru, xs, a.C, c_beg, c_end, lane, ag, au);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                ag[r][b] = wave_sum_to_lane63(ag[r][b]);
                au[r][b] = wave_sum_to_lane63(au[r][b]);
            }
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    red[wave * NV + r * B + b] = ag[r][b];
                    red[wave * NV + R * B + r * B + b] = au[r][b];
                }
        }
        __syncthreads();
        if (wave == 0 && lane < R * B) {
            const int r = lane / B, b = lane - (lane / B) * B;
            float g = 0.0f, u = 0.0f;
            for (int w = 0; w < waves; ++w) {
                g += red[w * NV + lane];
                u += red[w * NV + R * B + lane];
            }
            const int n = gi * R + r;
            if (n < a.N) a.h[(size_t)b * a.N + n] = silu_mul(g, u);
        }
        __syncthreads();
    }
}

template <int B, int R, int U, bool HLDS>
__global__ __launch_bounds__(kValuBlock) void down_valu_col_kernel(DownArgs a) {
    constexpr int NV = R * B;
    extern __shared__ f32x4_t smem4[];  // HLDS: h [B][2C]; then red [waves][NV] floats
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    float *red = reinterpret_cast<float *>(smem4 + (HLDS ? (size_t)B * 2 * a.C : 0));
    if (HLDS) stage_lds(smem4, hg, B * 2 * a.C);
    const int cw = (a.C + waves - 1) / waves;
    const int c_beg = min(wave * cw, a.C);
    const int c_end = min(c_beg + cw, a.C);

    for (int gi = blockIdx.x; gi < a.groups; gi += gridDim.x) {
        const u32x4_t *rd[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = min(gi * R + r, a.M - 1);
            rd[r] = reinterpret_cast<const u32x4_t *>(a.wd + (size_t)m * a.K);
        }
        float acc[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
        dn_valu_accumulate<B, R, U, HLDS>(rd, hg, smem4, a.C, c_beg, c_end, lane, acc);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) red[wave * NV + r * B + b] = acc[r][b];
        }
        __syncthreads();
        if (wave == 0 && lane < R * B) {
            const int r = lane / B, b = lane - (lane / B) * B;
            float v = 0.0f;
            for (int w = 0; w < waves; ++w) v += red[w * NV + lane];
            const int m = gi * R + r;
            if (m < a.M) a.y[(size_t)b * a.M + m] = to_bf16_rne(v);
        }
        __syncthreads();
    }
}

// ================================== VALU down, h held in registers =====
//
// The down projection at small batch with h kept in registers for the whole
// launch.  A workgroup's waves cut K (d_ff) into contiguous slices, one per
// wave; lane l of wave w holds h[b][8c .. 8c+7] for the chunks
// c = c_w + l + 64 j (j < J) of its slice, for every batch row b.  The
// workgroup then walks groups of R rows of W_down (groups blockIdx.x,
// blockIdx.x + gridDim.x, ...): each wave streams its slice of every row of
// the group (one load instruction = 1 KB contiguous of one row), the loads of
// the next group are in flight while the current group is multiplied, and the
// waves' sums are added in wave order through LDS (two buffers, one barrier
// per group; the barrier waits for LDS traffic only, so the prefetched
// weights stay in flight across it).  No K split crosses workgroups, so no
// second kernel adds partial sums, and h is read from memory once per
// workgroup.
constexpr int kHregMaxWaves = 16;

// LDS-only workgroup barrier: this wave's LDS writes are done and every wave
// has arrived; outstanding global loads are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest workgroup an instance is compiled for: 16 waves hold at most 128
// VGPRs each, so the instances with more than four chunks per lane (used with
// at most eight waves) get 256.
constexpr int hreg_max_waves(int J) { return J <= 4 ? kHregMaxWaves : 8; }

// F8: W_down as FP8 E4M3 codes with a scale per row (16 codes per 16-byte
// chunk, widened exactly to fp32; y = bf16(scale * sum)); a.C counts the
// 16-byte chunks of a row either way.  Each lane's scale for a group rides
// with the group's weight loads, issued before them.
template <int B, int J, int R, bool F8 = false>
__global__ __launch_bounds__(hreg_max_waves(J) * kWave) void down_valu_hreg_kernel(DownArgs a) {
    constexpr int H4 = F8 ? 4 : 2;  // f32x4 of h per chunk and batch row
    __shared__ float red[2][kHregMaxWaves][R * B];
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int cw = (a.C + waves - 1) / waves;
    const int c_beg = min(wave * cw, a.C);
    const int c_end = min(c_beg + cw, a.C);
    // this lane's chunks; one past the slice loads a chunk in bounds (the
    // slice's last, or chunk 0 for an empty slice) and multiplies it by zero
    int cj[J];
    bool okj[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = c_beg + lane + kWave * j;
        okj[j] = c < c_end;
        cj[j] = okj[j] ? c : (c_end > c_beg ? c_end - 1 : 0);
    }
    const u32x4_t *wd = reinterpret_cast<const u32x4_t *>(F8 ? static_cast<const void *>(a.qd)
                                                              : static_cast<const void *>(a.wd));
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    // row groups of this workgroup: blockIdx.x + t * gridDim.x, t < n
    if ((int)blockIdx.x >= a.groups) return;  // the whole workgroup, before any barrier
    const int n = (a.groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    // F8: the lanes that write y (lane < R * B, row lane / B) load their row's
    // scale; the others load row 0's
    const int srow = lane < R * B ? lane / B : 0;
    auto load = [&](u32x4_t (&w)[J][R], float &sc, int t) {
        const int gi = (int)blockIdx.x + t * (int)gridDim.x;
        if constexpr (F8) sc = a.sd[min(gi * R + srow, a.M - 1)];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int m = min(gi * R + r, a.M - 1);
            const u32x4_t *p = wd + (size_t)m * a.C;
#pragma unroll
            for (int j = 0; j < J; ++j) w[j][r] = load_stream(p + cj[j]);
        }
    };
    u32x4_t w0[J][R], w1[J][R];
    float s0 = 1.0f, s1 = 1.0f;
    load(w0, s0, 0);
    DFK_ISSUE_FENCE();
    f32x4_t hv[J][B][H4];
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int q = 0; q < H4; ++q) {
                const f32x4_t v = hg[((size_t)b * a.C + cj[j]) * H4 + q];
                hv[j][b][q] = okj[j] ? v : fzero;
            }
    float acc[R][B];
    auto compute = [&](const u32x4_t (&w)[J][R]) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4_t v = w[j][r];
                if constexpr (F8) {
                    // chunk element 4q + i is code i of word q
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t word = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
                        float e0, e1, e2, e3;
                        e4m3x2_to_f32<false>(word, e0, e1);
                        e4m3x2_to_f32<true>(word, e2, e3);
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const f32x4_t hq = hv[j][b][q];
                            float t = acc[r][b];
                            t = fmaf(e0, hq.x, t);
                            t = fmaf(e1, hq.y, t);
                            t = fmaf(e2, hq.z, t);
                            t = fmaf(e3, hq.w, t);
                            acc[r][b] = t;
                        }
                    }
                } else {
                    const float e0 = bf16_lo(v.x), e1 = bf16_hi(v.x), e2 = bf16_lo(v.y), e3 = bf16_hi(v.y),
                                e4 = bf16_lo(v.z), e5 = bf16_hi(v.z), e6 = bf16_lo(v.w), e7 = bf16_hi(v.w);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const f32x4_t h0 = hv[j][b][0], h1 = hv[j][b][1];
                        float t = acc[r][b];
                        t = fmaf(e0, h0.x, t);
                        t = fmaf(e1, h0.y, t);
                        t = fmaf(e2, h0.z, t);
                        t = fmaf(e3, h0.w, t);
                        t = fmaf(e4, h1.x, t);
                        t = fmaf(e5, h1.y, t);
                        t = fmaf(e6, h1.z, t);
                        t = fmaf(e7, h1.w, t);
                        acc[r][b] = t;
                    }
                }
            }
    };
    // group t's sums go through LDS buffer t & 1: a buffer is written again
    // two groups later, after a barrier that wave 0 reaches only when it has
    // read the buffer
    auto finish = [&](int t, float sc) {
        const int buf = t & 1;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) red[buf][wave][r * B + b] = acc[r][b];
        }
        lds_barrier();
        if (wave == 0 && lane < R * B) {
            float v = 0.0f;
            for (int w = 0; w < waves; ++w) v += red[buf][w][lane];
            if constexpr (F8) v = sc * v;
            const int r = lane / B, b = lane - (lane / B) * B;
            const int m = ((int)blockIdx.x + t * (int)gridDim.x) * R + r;
            if (m < a.M) a.y[(size_t)b * a.M + m] = to_bf16_rne(v);
        }
    };
    // group t is in w0 at the top of each turn; the loads in the loop are
    // unconditional, so the compiler's load counting waits only for the
    // buffer about to be multiplied
    int t = 0;
    for (; t + 2 < n; t += 2) {
        load(w1, s1, t + 1);
        DFK_ISSUE_FENCE();
        compute(w0);
        finish(t, s0);
        load(w0, s0, t + 2);
        DFK_ISSUE_FENCE();
        compute(w1);
        finish(t + 1, s1);
    }
    if (t + 1 < n) {
        load(w1, s1, t + 1);
        DFK_ISSUE_FENCE();
        compute(w0);
        finish(t, s0);
        compute(w1);
        finish(t + 1, s1);
    } else {
        compute(w0);
        finish(t, s0);
    }
}

// ================================================================ MFMA =====
//
// v_mfma_f32_16x16x32_bf16, lane l: r = l & 15, q = l >> 4.
//   A[i][k]  = W[row0 + i][k]      lane (i, q) holds k = k0 + 8q .. 8q+7
//   B[k][j]  = operand[b0 + j][k]  lane (j, q) holds the same 8 k
//   D[i][j]  -> lane (j, i / 4), element i % 4
// A 32-wide K step is 4 consecutive 16-byte chunks of a row: chunk c of the
// row goes to lanes with q = c mod 4.  Any fixed assignment of k to
// (q, element) works as long as A and B agree; this one keeps each weight
// load instruction at 16 rows x 64 contiguous bytes.  The B operand is read
// from global memory by the lanes whose batch column exists (x bf16, or fp32
// h split into bf16 hi + lo on the fly); padded columns are zero.

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// One tile group (TR tiles of 16 neurons, gate and up) over K steps
// [st_beg, st_end).
template <int BT, int TR, int U>
__device__ __forceinline__ void gu_mfma_accumulate(const GateUpArgs &a, int row0, int st_beg, int st_end, int lr,
                                                   int lq, f32x4_t (&accg)[TR][BT], f32x4_t (&accu)[TR][BT]) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t *pg[TR];
    const u32x4_t *pu[TR];
#pragma unroll
    for (int t = 0; t < TR; ++t) {
        const int n = min(row0 + t * 16 + lr, a.N - 1);
        pg[t] = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)n * a.ldw);
        pu[t] = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)n * a.ldw);
    }
    const u32x4_t *px[BT];
    bool bvalid[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) {
        const int b = bt * 16 + lr;
        bvalid[bt] = b < a.B;
        px[bt] = reinterpret_cast<const u32x4_t *>(a.x + (size_t)min(b, a.B - 1) * a.K);
    }
    for (int st = st_beg; st < st_end; st += U) {
        u32x4_t ag[U][TR], au[U][TR], bx[U][BT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = min((st + u) * 4 + lq, a.C - 1);
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                ag[u][t] = load_stream(pg[t] + cc);
                au[u][t] = load_stream(pu[t] + cc);
            }
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) bx[u][bt] = bvalid[bt] ? px[bt][cc] : zero;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kv = ((st + u) * 4 + lq < a.C) && (st + u < st_end);
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                const bf16x8_t wa = as_bf16x8(kv ? ag[u][t] : zero);
                const bf16x8_t wb = as_bf16x8(kv ? au[u][t] : zero);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const bf16x8_t xb = as_bf16x8(kv ? bx[u][bt] : zero);
                    accg[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb, accg[t][bt], 0, 0, 0);
                    accu[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, accu[t][bt], 0, 0, 0);
                }
            }
        }
    }
}

template <int BT, int TR, int U>
__device__ __forceinline__ void dn_mfma_accumulate(const DownArgs &a, int row0, int st_beg, int st_end, int lr,
                                                   int lq, f32x4_t (&acc)[TR][BT]) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    const u32x4_t *pw[TR];
#pragma unroll
    for (int t = 0; t < TR; ++t) {
        const int m = min(row0 + t * 16 + lr, a.M - 1);
        pw[t] = reinterpret_cast<const u32x4_t *>(a.wd + (size_t)m * a.K);
    }
    const f32x4_t *ph[BT];
    bool bvalid[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) {
        const int b = bt * 16 + lr;
        bvalid[bt] = b < a.B;
        ph[bt] = reinterpret_cast<const f32x4_t *>(a.h + (size_t)min(b, a.B - 1) * a.K);
    }
    for (int st = st_beg; st < st_end; st += U) {
        u32x4_t aw[U][TR];
        f32x4_t hb[U][BT][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = min((st + u) * 4 + lq, a.C - 1);
#pragma unroll
            for (int t = 0; t < TR; ++t) aw[u][t] = load_stream(pw[t] + cc);
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                hb[u][bt][0] = bvalid[bt] ? ph[bt][2 * cc] : fzero;
                hb[u][bt][1] = bvalid[bt] ? ph[bt][2 * cc + 1] : fzero;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool kv = ((st + u) * 4 + lq < a.C) && (st + u < st_end);
            bf16x8_t hhi[BT], hlo[BT];
#pragma unroll
            for (int bt = 0; bt < BT; ++bt)
                split_hi_lo(kv ? hb[u][bt][0] : fzero, kv ? hb[u][bt][1] : fzero, hhi[bt], hlo[bt]);
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                const bf16x8_t wa = as_bf16x8(kv ? aw[u][t] : zero);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, hhi[bt], acc[t][bt], 0, 0, 0);
                    acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, hlo[bt], acc[t][bt], 0, 0, 0);
                }
            }
        }
    }
}

// h[b][n..n+3] = SiLU(g) * u for one lane's four accumulator rows.
template <int BT, int TR>
__device__ __forceinline__ void gu_mfma_epilogue(const GateUpArgs &a, int row0, int lr, int lq,
                                                 const f32x4_t (&accg)[TR][BT], const f32x4_t (&accu)[TR][BT]) {
#pragma unroll
    for (int t = 0; t < TR; ++t) {
        const int n = row0 + t * 16 + 4 * lq;  // 4 consecutive neurons
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
            const int b = bt * 16 + lr;
            if (b < a.B && n < a.N) {
                f32x4_t o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = silu_mul(accg[t][bt][e], accu[t][bt][e]);
                *reinterpret_cast<f32x4_t *>(a.h + (size_t)b * a.N + n) = o;
            }
        }
    }
}

template <int BT, int TR>
__device__ __forceinline__ void dn_mfma_epilogue(const DownArgs &a, int row0, int lr, int lq,
                                                 const f32x4_t (&acc)[TR][BT]) {
#pragma unroll
    for (int t = 0; t < TR; ++t) {
        const int m = row0 + t * 16 + 4 * lq;
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
            const int b = bt * 16 + lr;
            if (b < a.B && m < a.M) {
                const unsigned lo = to_bf16_rne(acc[t][bt][0]) | ((unsigned)to_bf16_rne(acc[t][bt][1]) << 16);
                const unsigned hi = to_bf16_rne(acc[t][bt][2]) | ((unsigned)to_bf16_rne(acc[t][bt][3]) << 16);
                *reinterpret_cast<uint2 *>(a.y + (size_t)b * a.M + m) = make_uint2(lo, hi);
            }
        }
    }
}

// ------------------------------------------------- MFMA, LDS-transposed -----
//
// Streaming weights at full HBM rate needs few rows per load instruction: on
// MI355X a 16-row x 64-byte load (the MFMA A-fragment shape) streams ~20 %
// slower than 2 rows x 512 bytes.  These kernels load each block of a 16-row
// weight tile (16 rows x 256 elements) as 8 instructions of 2 rows x 512 B,
// park it in a wave-private, bank-padded LDS tile, and read it back in MFMA
// A-fragment order while the next block's loads are in flight.  A workgroup
// owns WAVES / KSPLIT tiles; the KSPLIT waves of a tile take contiguous runs
// of its blocks and are combined through LDS (KSPLIT = 1: the row traversal).

// A block is 16 rows x KBC chunks of 16 B (KBC = 32: 256 elements, loaded as
// 8 instructions of 2 rows x 512 B; KBC = 64: 512 elements, 16 instructions
// of 1 row x 1 KB).  The LDS tile pitch is KBC + 1 chunks (bank padding).
template <int KBC> struct Lt {
    static constexpr int kRowsPerInst = 64 / KBC;
    static constexpr int kInsts = 16 / kRowsPerInst;
    static constexpr int kPitch = KBC + 1;
    static constexpr int kTile = 16 * kPitch;  // 16-byte chunks of LDS per matrix per wave
    static constexpr int kSteps = KBC / 4;     // MFMA K steps per block

    // Issue the loads of block kb (rows and chunks clamped into the matrix).
    static __device__ __forceinline__ void load(u32x4_t (&v)[kInsts], const uint16_t *w, int K, int C, int row0,
                                                int rows, int kb, int lane) {
        const int c = min(kb * KBC + lane % KBC, C - 1);
#pragma unroll
        for (int i = 0; i < kInsts; ++i) {
            const int row = min(row0 + i * kRowsPerInst + lane / KBC, rows - 1);
            v[i] = load_stream(reinterpret_cast<const u32x4_t *>(w + (size_t)row * K) + c);
        }
    }
    // Park block kb in the wave's LDS tile, zeroing chunks past the row end.
    static __device__ __forceinline__ void store(u32x4_t *lt, const u32x4_t (&v)[kInsts], int kb, int C, int lane) {
        const bool ok = kb * KBC + lane % KBC < C;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kInsts; ++i) lt[(i * kRowsPerInst + lane / KBC) * kPitch + lane % KBC] = ok ? v[i] : zero;
    }
    // A fragment of step j (chunks 4j..4j+3 of the block): lane (r, q) -> row r, chunk 4j + q.
    static __device__ __forceinline__ bf16x8_t frag(const u32x4_t *lt, int j, int lr, int lq) {
        return as_bf16x8(lt[lr * kPitch + 4 * j + lq]);
    }
    // The block's chunk at tile position p (the B operand's K index for it).
    static __device__ __forceinline__ int kpos(int p) { return p; }
};

// The same LDS tile filled from FP8 E4M3 codes: one 16-byte load carries 16
// codes (two bf16 chunks), so a row of a block takes KBC / 2 lanes and an
// instruction covers 64 / (KBC / 2) rows; the codes are widened to bf16
// (exactly) on the way into LDS.  C counts bf16 chunks (K / 8) as for Lt.
// A lane parks its two bf16 chunks (2p, 2p + 1) side by side, so the lanes'
// 16-byte words in one store are 32 bytes apart and pairs of lanes share an
// LDS bank.  SPLIT parks the low chunk at tile position p and the high one at
// KBC / 2 + p instead (consecutive positions per store, no shared bank) and
// permutes the block's K order in the tile accordingly: kpos maps a tile
// position to its chunk, and the B operand is read at that chunk (any order
// of K within a block gives the same sum terms, paired alike on both
// operands).  Taken where the B operand comes from LDS planes that are read
// once per block anyway (the staged-h down kernel); where it is loaded from
// memory per fragment, the permuted order splits each fragment's 64
// contiguous bytes and costs more than the conflicts.
// SWZ (natural K order): the lanes with p mod 8 < 4 park their low chunk
// first and the others their high chunk, so each store of a group of eight
// lanes covers eight different banks.  Taken by the gate-up kernel with x
// staged in LDS (FP8 MLP at B = 64: 76.1 -> 71.3 us); the column gate-up with
// x fragments from memory measured 5 us slower with it at B = 4-16.
template <int KBC, bool SPLIT = false, bool SWZ = false> struct Lt8 {
    static constexpr int kC8 = KBC / 2;
    static constexpr int kRowsPerInst = 64 / kC8;
    static constexpr int kInsts = 16 / kRowsPerInst;
    static constexpr int kPitch = KBC + 1;
    static constexpr int kTile = 16 * kPitch;
    static constexpr int kSteps = KBC / 4;

    static __device__ __forceinline__ void load(u32x4_t (&v)[kInsts], const uint8_t *q, int K, int C, int row0,
                                                int rows, int kb, int lane) {
        const int c = min(kb * kC8 + lane % kC8, C / 2 - 1);
#pragma unroll
        for (int i = 0; i < kInsts; ++i) {
            const int row = min(row0 + i * kRowsPerInst + lane / kC8, rows - 1);
            v[i] = load_stream(reinterpret_cast<const u32x4_t *>(q + (size_t)row * K) + c);
        }
    }
    static __device__ __forceinline__ void store(u32x4_t *lt, const u32x4_t (&v)[kInsts], int kb, int C, int lane) {
        const bool ok = kb * kC8 + lane % kC8 < C / 2;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kInsts; ++i) {
            u32x4_t lo, hi;
            e4m3x16_to_bf16(v[i], lo, hi);
            u32x4_t *dst = lt + (i * kRowsPerInst + lane / kC8) * kPitch + (SPLIT ? 1 : 2) * (lane % kC8);
            if constexpr (SWZ && !SPLIT) {
                const bool lo_first = ((lane % kC8) & 4) == 0;
                dst[lo_first ? 0 : 1] = ok ? (lo_first ? lo : hi) : zero;
                dst[lo_first ? 1 : 0] = ok ? (lo_first ? hi : lo) : zero;
            } else {
                dst[0] = ok ? lo : zero;
                dst[SPLIT ? kC8 : 1] = ok ? hi : zero;
            }
        }
    }
    static __device__ __forceinline__ bf16x8_t frag(const u32x4_t *lt, int j, int lr, int lq) {
        return as_bf16x8(lt[lr * kPitch + 4 * j + lq]);
    }
    static __device__ __forceinline__ int kpos(int p) {
        return !SPLIT ? p : p < kC8 ? 2 * p : 2 * (p - kC8) + 1;
    }
};

template <bool C, class A, class B> struct Pick { using T = A; };
template <class A, class B> struct Pick<false, A, B> { using T = B; };

// The B operand (x, or h as bf16 hi + lo) is read as MFMA B fragments straight
// from global memory (it is small and L2-resident).  Loads return in issue
// order, so a fragment load issued after the next weight block would make the
// wave wait for that whole block: for BT <= kPreBT the fragments of a whole
// block are issued before the next block's weights (one register buffer),
// otherwise one step ahead.  Fragment reads are never predicated: rows past B
// read row B - 1 (their output columns are dropped) and chunks past the row
// end read the last chunk, masked to zero in the tail block only.
// F8: the weights are FP8 codes (a.qg, a.qu) with row scales (a.sg, a.su).
template <int BT, int KSPLIT, int WAVES, bool F8 = false>
__global__ __launch_bounds__(WAVES * kWave) void gate_up_mfma_lt_kernel(GateUpArgs a) {
    using L = typename Pick<F8, Lt8<32>, Lt<32>>::T;
    constexpr int KBC = 32;
    constexpr bool kPre = BT <= 2;
    constexpr int XS = kPre ? L::kSteps : 2;
    constexpr int TPW = WAVES / KSPLIT;  // tiles per workgroup
    constexpr int NV = 2 * BT * 4;
    extern __shared__ u32x4_t smem[];    // [WAVES][2][L::kTile], then red [WAVES][NV][64] floats
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    const int slot = wave / KSPLIT, ks = wave - slot * KSPLIT;
    u32x4_t *ltg = smem + (size_t)wave * 2 * L::kTile;
    u32x4_t *ltu = ltg + L::kTile;
    float *red = reinterpret_cast<float *>(smem + (size_t)WAVES * 2 * L::kTile);
    const int nb = (a.C + KBC - 1) / KBC;
    const int per = (nb + KSPLIT - 1) / KSPLIT;
    const int kb_beg = min(ks * per, nb), kb_end = min(kb_beg + per, nb);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t *px[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
        px[bt] = reinterpret_cast<const u32x4_t *>(a.x + (size_t)min(bt * 16 + lr, a.B - 1) * a.K);
    const int wg_items = (a.groups + TPW - 1) / TPW;

    for (int g = blockIdx.x; g < wg_items; g += gridDim.x) {
        const int tile = g * TPW + slot;
        const bool active = tile < a.groups;
        const int row0 = tile * 16;
        f32x4_t accg[BT], accu[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) accg[bt] = accu[bt] = f32x4_t{0, 0, 0, 0};
        float scg[4], scu[4];  // F8: the scales of this lane's output rows, loaded ahead of the weights
        if constexpr (F8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = min(row0 + 4 * lq + e, a.N - 1);
                scg[e] = a.sg[n];
                scu[e] = a.su[n];
            }
        }

        u32x4_t xf[XS][BT];
        auto load_x = [&](int kb, int j, u32x4_t (&xb)[BT]) {
            const int c = min(kb * KBC + L::kpos(4 * j + lq), a.C - 1);
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) xb[bt] = px[bt][c];
        };
        auto load_block = [&](int kb) {
            if constexpr (kPre) {
#pragma unroll
                for (int j = 0; j < L::kSteps; ++j) load_x(kb, j, xf[j]);
            } else {
                load_x(kb, 0, xf[0]);
            }
        };
        auto compute = [&](int kb) {
            const bool tail = (kb + 1) * KBC > a.C;
#pragma unroll
            for (int j = 0; j < L::kSteps; ++j) {
                const int slotj = kPre ? j : (j & 1);
                if constexpr (!kPre) {
                    if (j + 1 < L::kSteps) load_x(kb, j + 1, xf[(j + 1) & 1]);
                }
                const bool cok = !tail || kb * KBC + L::kpos(4 * j + lq) < a.C;
                const bf16x8_t ag = L::frag(ltg, j, lr, lq);
                const bf16x8_t au = L::frag(ltu, j, lr, lq);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const bf16x8_t xb = as_bf16x8(cok ? xf[slotj][bt] : zero);
                    accg[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, xb, accg[bt], 0, 0, 0);
                    accu[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, xb, accu[bt], 0, 0, 0);
                }
            }
        };
        if (active && kb_beg < kb_end) {
            u32x4_t vg0[L::kInsts], vu0[L::kInsts], vg1[L::kInsts], vu1[L::kInsts];
            auto load_w = [&](u32x4_t (&vg)[L::kInsts], u32x4_t (&vu)[L::kInsts], int kb) {
                if constexpr (F8) {
                    L::load(vg, a.qg, a.K, a.C, row0, a.N, kb, lane);
                    L::load(vu, a.qu, a.K, a.C, row0, a.N, kb, lane);
                } else {
                    L::load(vg, a.wg, a.ldw, a.C, row0, a.N, kb, lane);
                    L::load(vu, a.wu, a.ldw, a.C, row0, a.N, kb, lane);
                }
            };
            auto step = [&](u32x4_t (&vg)[L::kInsts], u32x4_t (&vu)[L::kInsts], int kb) {
                L::store(ltg, vg, kb, a.C, lane);
                L::store(ltu, vu, kb, a.C, lane);
                if constexpr (!kPre) load_block(kb);
                compute(kb);
            };
            // Software pipeline, one weight block ahead.  The steady loop has
            // no conditional loads, so every wait is for the oldest block only.
            if constexpr (kPre) load_block(kb_beg);
            load_w(vg0, vu0, kb_beg);
            int kb = kb_beg;
            for (; kb + 2 < kb_end; kb += 2) {
                load_w(vg1, vu1, kb + 1);
                DFK_ISSUE_FENCE();
                step(vg0, vu0, kb);
                if constexpr (kPre) load_block(kb + 1);
                load_w(vg0, vu0, kb + 2);
                DFK_ISSUE_FENCE();
                step(vg1, vu1, kb + 1);
                if constexpr (kPre) load_block(kb + 2);
            }
            if (kb + 1 < kb_end) {
                load_w(vg1, vu1, kb + 1);
                DFK_ISSUE_FENCE();
                step(vg0, vu0, kb);
                if constexpr (kPre) load_block(kb + 1);
                step(vg1, vu1, kb + 1);
            } else {
                step(vg0, vu0, kb);
            }
        }
        if (KSPLIT > 1) {
            if (ks > 0) {
                float *dst = red + (size_t)wave * NV * kWave;
#pragma unroll
                for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dst[((bt * 4 + e) * 2) * kWave + lane] = accg[bt][e];
                        dst[((bt * 4 + e) * 2 + 1) * kWave + lane] = accu[bt][e];
                    }
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int w = 1; w < KSPLIT; ++w) {
                    const float *src = red + (size_t)(wave + w) * NV * kWave;
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            accg[bt][e] += src[((bt * 4 + e) * 2) * kWave + lane];
                            accu[bt][e] += src[((bt * 4 + e) * 2 + 1) * kWave + lane];
                        }
                }
            }
            __syncthreads();
        }
        if (ks == 0 && active) {
            const int n = row0 + 4 * lq;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (b < a.B && n < a.N) {
                    f32x4_t o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (F8) o[e] = silu_mul(scg[e] * accg[bt][e], scu[e] * accu[bt][e]);
                        else o[e] = silu_mul(accg[bt][e], accu[bt][e]);
                    }
                    *reinterpret_cast<f32x4_t *>(a.h + (size_t)b * a.N + n) = o;
                }
            }
        }
    }
}

// F8: W_down is FP8 codes (a.qd) with row scales (a.sd).
template <int BT, int KSPLIT, int WAVES, int KBC, bool F8 = false>
__global__ __launch_bounds__(WAVES * kWave) void down_mfma_lt_kernel(DownArgs a) {
    using L = typename Pick<F8, Lt8<KBC>, Lt<KBC>>::T;
    constexpr bool kPre = BT <= 1;
    constexpr int HS = kPre ? L::kSteps : 2;
    constexpr int TPW = WAVES / KSPLIT;
    constexpr int NV = BT * 4;
    extern __shared__ u32x4_t smem[];    // [WAVES][L::kTile], then red [WAVES][NV][64] floats
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    const int slot = wave / KSPLIT, ks = wave - slot * KSPLIT;
    u32x4_t *ltw = smem + (size_t)wave * L::kTile;
    float *red = reinterpret_cast<float *>(smem + (size_t)WAVES * L::kTile);
    const int nb = (a.C + KBC - 1) / KBC;
    const int per = (nb + KSPLIT - 1) / KSPLIT;
    const int kb_beg = min(ks * per, nb), kb_end = min(kb_beg + per, nb);
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t *ph[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
        ph[bt] = reinterpret_cast<const f32x4_t *>(a.h + (size_t)min(bt * 16 + lr, a.B - 1) * a.K);
    const int wg_items = (a.groups + TPW - 1) / TPW;

    for (int g = blockIdx.x; g < wg_items; g += gridDim.x) {
        const int tile = g * TPW + slot;
        const bool active = tile < a.groups;
        const int row0 = tile * 16;
        f32x4_t acc[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) acc[bt] = f32x4_t{0, 0, 0, 0};
        float scd[4];  // F8: the scales of this lane's output rows, loaded ahead of the weights
        if constexpr (F8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) scd[e] = a.sd[min(row0 + 4 * lq + e, a.M - 1)];
        }

        f32x4_t hf[HS][BT][2];
        auto load_h = [&](int kb, int j, f32x4_t (&hb)[BT][2]) {
            const int c = min(kb * KBC + L::kpos(4 * j + lq), a.C - 1);
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                hb[bt][0] = ph[bt][2 * c];
                hb[bt][1] = ph[bt][2 * c + 1];
            }
        };
        auto load_block = [&](int kb) {
            if constexpr (kPre) {
#pragma unroll
                for (int j = 0; j < L::kSteps; ++j) load_h(kb, j, hf[j]);
            } else {
                load_h(kb, 0, hf[0]);
            }
        };
        auto compute = [&](int kb) {
            const bool tail = (kb + 1) * KBC > a.C;
#pragma unroll
            for (int j = 0; j < L::kSteps; ++j) {
                const int slotj = kPre ? j : (j & 1);
                if constexpr (!kPre) {
                    if (j + 1 < L::kSteps) load_h(kb, j + 1, hf[(j + 1) & 1]);
                }
                const bool cok = !tail || kb * KBC + L::kpos(4 * j + lq) < a.C;
                const bf16x8_t aw = L::frag(ltw, j, lr, lq);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    bf16x8_t hi, lo;
                    split_hi_lo(cok ? hf[slotj][bt][0] : fzero, cok ? hf[slotj][bt][1] : fzero, hi, lo);
                    acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, hi, acc[bt], 0, 0, 0);
                    acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, lo, acc[bt], 0, 0, 0);
                }
            }
        };
        if (active && kb_beg < kb_end) {
            u32x4_t v0[L::kInsts], v1[L::kInsts];
            auto step = [&](u32x4_t (&v)[L::kInsts], int kb) {
                L::store(ltw, v, kb, a.C, lane);
                if constexpr (!kPre) load_block(kb);
                compute(kb);
            };
            // software pipeline, one weight block ahead, no conditional loads
            // in the steady loop
            auto load_w = [&](u32x4_t (&v)[L::kInsts], int kb) {
                if constexpr (F8) L::load(v, a.qd, a.K, a.C, row0, a.M, kb, lane);
                else L::load(v, a.wd, a.K, a.C, row0, a.M, kb, lane);
            };
            if constexpr (kPre) load_block(kb_beg);
            load_w(v0, kb_beg);
            int kb = kb_beg;
            for (; kb + 2 < kb_end; kb += 2) {
                load_w(v1, kb + 1);
                DFK_ISSUE_FENCE();
                step(v0, kb);
                if constexpr (kPre) load_block(kb + 1);
                load_w(v0, kb + 2);
                DFK_ISSUE_FENCE();
                step(v1, kb + 1);
                if constexpr (kPre) load_block(kb + 2);
            }
            if (kb + 1 < kb_end) {
                load_w(v1, kb + 1);
                DFK_ISSUE_FENCE();
                step(v0, kb);
                if constexpr (kPre) load_block(kb + 1);
                step(v1, kb + 1);
            } else {
                step(v0, kb);
            }
        }
        if (KSPLIT > 1) {
            if (ks > 0) {
                float *dst = red + (size_t)wave * NV * kWave;
#pragma unroll
                for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(bt * 4 + e) * kWave + lane] = acc[bt][e];
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int w = 1; w < KSPLIT; ++w) {
                    const float *src = red + (size_t)(wave + w) * NV * kWave;
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[bt][e] += src[(bt * 4 + e) * kWave + lane];
                }
            }
            __syncthreads();
        }
        if (ks == 0 && active) {
            const int m = row0 + 4 * lq;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (b < a.B && m < a.M) {
                    f32x4_t v = acc[bt];
                    if constexpr (F8) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= scd[e];
                    }
                    const unsigned lo = to_bf16_rne(v[0]) | ((unsigned)to_bf16_rne(v[1]) << 16);
                    const unsigned hi = to_bf16_rne(v[2]) | ((unsigned)to_bf16_rne(v[3]) << 16);
                    *reinterpret_cast<uint2 *>(a.y + (size_t)b * a.M + m) = make_uint2(lo, hi);
                }
            }
        }
    }
}

// ---------------------------------------------------------- MFMA row ------
// A wave owns a tile group of 16*TR rows for the whole of K; no LDS.

template <int BT, int TR, int U>
__global__ __launch_bounds__(kMfmaRowBlock) void gate_up_mfma_row_kernel(GateUpArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int lr = lane & 15, lq = lane >> 4;
    const int steps = (a.C + 3) / 4;
    for (int tg = blockIdx.x * waves + threadIdx.x / kWave; tg < a.groups; tg += gridDim.x * waves) {
        f32x4_t accg[TR][BT], accu[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) accg[t][bt] = accu[t][bt] = f32x4_t{0, 0, 0, 0};
        gu_mfma_accumulate<BT, TR, U>(a, tg * 16 * TR, 0, steps, lr, lq, accg, accu);
        gu_mfma_epilogue<BT, TR>(a, tg * 16 * TR, lr, lq, accg, accu);
    }
}

template <int BT, int TR, int U>
__global__ __launch_bounds__(kMfmaRowBlock) void down_mfma_row_kernel(DownArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int lr = lane & 15, lq = lane >> 4;
    const int steps = (a.C + 3) / 4;
    for (int tg = blockIdx.x * waves + threadIdx.x / kWave; tg < a.groups; tg += gridDim.x * waves) {
        f32x4_t acc[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[t][bt] = f32x4_t{0, 0, 0, 0};
        dn_mfma_accumulate<BT, TR, U>(a, tg * 16 * TR, 0, steps, lr, lq, acc);
        dn_mfma_epilogue<BT, TR>(a, tg * 16 * TR, lr, lq, acc);
    }
}

// ---------------------------------------------------------- MFMA col ------
// A workgroup owns a tile group; its WAVES waves split the K steps into
// contiguous slices and their accumulators are added in wave order through
// LDS; wave 0 runs the epilogue.

template <int BT, int TR, int U, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void gate_up_mfma_col_kernel(GateUpArgs a) {
    constexpr int NV = 2 * TR * BT * 4;
    extern __shared__ float red[];  // [WAVES-1][NV][64]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & 15, lq = lane >> 4;
    const int steps = (a.C + 3) / 4;
    const int per_wave = (steps + WAVES - 1) / WAVES;
    const int st_beg = min(wave * per_wave, steps);
    const int st_end = min(st_beg + per_wave, steps);
    for (int tg = blockIdx.x; tg < a.groups; tg += gridDim.x) {
        f32x4_t accg[TR][BT], accu[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) accg[t][bt] = accu[t][bt] = f32x4_t{0, 0, 0, 0};
        gu_mfma_accumulate<BT, TR, U>(a, tg * 16 * TR, st_beg, st_end, lr, lq, accg, accu);
        if (wave > 0) {
            float *dst = red + (size_t)(wave - 1) * NV * kWave;
            int v = 0;
#pragma unroll
            for (int t = 0; t < TR; ++t)
#pragma unroll
                for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dst[(v++) * kWave + lane] = accg[t][bt][e];
                        dst[(v++) * kWave + lane] = accu[t][bt][e];
                    }
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < WAVES; ++w) {
                const float *src = red + (size_t)(w - 1) * NV * kWave;
                int v = 0;
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            accg[t][bt][e] += src[(v++) * kWave + lane];
                            accu[t][bt][e] += src[(v++) * kWave + lane];
                        }
            }
            gu_mfma_epilogue<BT, TR>(a, tg * 16 * TR, lr, lq, accg, accu);
        }
        __syncthreads();  // LDS reuse by the next tile group
    }
}

template <int BT, int TR, int U, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void down_mfma_col_kernel(DownArgs a) {
    constexpr int NV = TR * BT * 4;
    extern __shared__ float red[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & 15, lq = lane >> 4;
    const int steps = (a.C + 3) / 4;
    const int per_wave = (steps + WAVES - 1) / WAVES;
    const int st_beg = min(wave * per_wave, steps);
    const int st_end = min(st_beg + per_wave, steps);
    for (int tg = blockIdx.x; tg < a.groups; tg += gridDim.x) {
        f32x4_t acc[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[t][bt] = f32x4_t{0, 0, 0, 0};
        dn_mfma_accumulate<BT, TR, U>(a, tg * 16 * TR, st_beg, st_end, lr, lq, acc);
        if (wave > 0) {
            float *dst = red + (size_t)(wave - 1) * NV * kWave;
            int v = 0;
#pragma unroll
            for (int t = 0; t < TR; ++t)
#pragma unroll
                for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(v++) * kWave + lane] = acc[t][bt][e];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < WAVES; ++w) {
                const float *src = red + (size_t)(w - 1) * NV * kWave;
                int v = 0;
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[t][bt][e] += src[(v++) * kWave + lane];
            }
            dn_mfma_epilogue<BT, TR>(a, tg * 16 * TR, lr, lq, acc);
        }
        __syncthreads();
    }
}

// ------------------------------------------ MFMA, B operand staged in LDS --
//
// Above 16 batch rows the B operand (x, or h) is the larger stream out of L2:
// every 16-row weight tile needs all of it.  In these kernels the WAVES tiles
// of a workgroup walk K together in blocks of 256 elements.  Each block of the
// B operand is loaded once per workgroup with wide, coalesced loads, zeroed
// past B and outside the K range, and parked in LDS with a padded pitch; the
// waves read their MFMA B fragments from there.  Weights arrive as A fragments
// straight from HBM, one block ahead in registers, and every load of the
// steady loop is unconditional.  The last block of a K range is shifted back
// to end at the range end (the chunks it repeats are zeroed in the staged
// block), so weight loads stay inside their row.  The down kernel may also
// split K across S workgroups: partial sums, then the panel reduce kernel.
// NBUF = 2 double-buffers the staged block (one barrier per block), NBUF = 1
// halves the LDS (two barriers).

constexpr int kStKbc = 32;            // 16-byte chunks per K block (256 elements)
constexpr int kStPitch = kStKbc + 1;  // LDS pitch of one staged row, in chunks

// First chunk of block kb of the K range [c0, c1)
__device__ __forceinline__ int st_block_start(int kb, int c0, int c1) {
    return c1 - c0 >= kStKbc ? min(c0 + kb * kStKbc, c1 - kStKbc) : c0;
}

template <int BT, int WAVES, int NBUF, int WPE>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void gate_up_mfma_staged_kernel(
    GateUpArgs a) {
    constexpr int NT = WAVES * kWave;
    constexpr int XR = 16 * BT;                   // staged rows: the padded batch
    constexpr int XPT = XR * kStKbc / NT;         // staged chunks per thread
    static_assert(XR * kStKbc % NT == 0, "staging split");
    constexpr int XBUF = XR * kStPitch;
    extern __shared__ u32x4_t smem[];             // [NBUF][XR][kStPitch]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    const int nb = (a.C + kStKbc - 1) / kStKbc;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t *xg = reinterpret_cast<const u32x4_t *>(a.x);
    const int wg_items = (a.groups + WAVES - 1) / WAVES;

    auto load_x = [&](u32x4_t (&xr)[XPT], int kb) {
        const int cs = st_block_start(kb, 0, a.C);
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int i = t * NT + tid;
            const int b = min(i / kStKbc, a.B - 1);
            const int c = min(cs + i % kStKbc, a.C - 1);
            xr[t] = xg[(size_t)b * a.C + c];
        }
    };
    auto store_x = [&](const u32x4_t (&xr)[XPT], int kb) {
        const int cs = st_block_start(kb, 0, a.C);
        u32x4_t *dst = smem + (NBUF == 2 ? (kb & 1) : 0) * XBUF;
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int i = t * NT + tid;
            const int b = i / kStKbc, cc = i % kStKbc;
            const int c = cs + cc;
            const bool ok = b < a.B && c >= kb * kStKbc && c < a.C;
            dst[b * kStPitch + cc] = ok ? xr[t] : zero;
        }
    };

    for (int g = blockIdx.x; g < wg_items; g += gridDim.x) {
        const int tile = g * WAVES + wave;
        const int row = min(tile * 16 + lr, a.N - 1);
        const u32x4_t *pg = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)row * a.ldw);
        const u32x4_t *pu = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)row * a.ldw);
        f32x4_t accg[BT], accu[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) accg[bt] = accu[bt] = f32x4_t{0, 0, 0, 0};

        auto load_w = [&](u32x4_t (&wgr)[8], u32x4_t (&wur)[8], int kb) {
            const int cs = st_block_start(kb, 0, a.C);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = min(cs + 4 * j + lq, a.C - 1);
                wgr[j] = load_stream(pg + c);
                wur[j] = load_stream(pu + c);
            }
        };
        auto compute = [&](const u32x4_t (&wgr)[8], const u32x4_t (&wur)[8], int kb) {
            const u32x4_t *xs = smem + (NBUF == 2 ? (kb & 1) : 0) * XBUF;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const bf16x8_t xb = as_bf16x8(xs[(bt * 16 + lr) * kStPitch + 4 * j + lq]);
                    accg[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wgr[j]), xb, accg[bt], 0, 0, 0);
                    accu[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wur[j]), xb, accu[bt], 0, 0, 0);
                }
        };
        u32x4_t xr[XPT];
        u32x4_t wg0[8], wu0[8], wg1[8], wu1[8];
        // prefetch block kb + 1 (x first, then the weights), multiply block kb,
        // then park x(kb + 1) in LDS
        auto step = [&](auto &cg, auto &cu, auto &ng, auto &nu, int kb) {
            load_x(xr, kb + 1);
            load_w(ng, nu, kb + 1);
            DFK_ISSUE_FENCE();
            compute(cg, cu, kb);
            if constexpr (NBUF == 1) __syncthreads();
            store_x(xr, kb + 1);
            __syncthreads();
        };
        auto last = [&](auto &cg, auto &cu, int kb) {
            compute(cg, cu, kb);
            __syncthreads();
        };
        load_x(xr, 0);
        load_w(wg0, wu0, 0);
        store_x(xr, 0);
        __syncthreads();
        int kb = 0;
        for (; kb + 2 < nb; kb += 2) {
            step(wg0, wu0, wg1, wu1, kb);
            step(wg1, wu1, wg0, wu0, kb + 1);
        }
        if (kb + 1 < nb) {
            step(wg0, wu0, wg1, wu1, kb);
            last(wg1, wu1, kb + 1);
        } else {
            last(wg0, wu0, kb);
        }
        if (tile < a.groups) {
            const int n = tile * 16 + 4 * lq;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (b < a.B && n < a.N) {
                    f32x4_t o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = silu_mul(accg[bt][e], accu[bt][e]);
                    *reinterpret_cast<f32x4_t *>(a.h + (size_t)b * a.N + n) = o;
                }
            }
        }
    }
}

// F8 staging: a 16-byte load of E4M3 codes carries the A fragments of two
// MFMA steps.  Lane (r, q) loads code chunk 4 i + q of its row (16 codes,
// 16 (4 i + q) .. + 15 of the block) and feeds the first 8 to step 2 i and the
// last 8 to step 2 i + 1, so the block's K order is permuted: bf16 chunk a of
// the block (8 elements) is consumed in step j = 2 (a / 8) + a % 2 by lanes
// q = (a / 2) % 4, i.e. from B-fragment slot 4 j + q.  The staged h takes the
// same permutation (the contraction does not depend on the order of K).
__device__ __forceinline__ int f8_step_slot(int a) { return 4 * (2 * (a / 8) + a % 2) + (a / 2) % 4; }

// down: h staged as bf16 hi + lo planes; work item = (row-tile group, K split);
// each wave owns TR consecutive 16-row tiles, so every B fragment it reads
// from LDS feeds TR tiles (LDS traffic per weight byte / TR).
// F8: W_down is FP8 codes (a.qd, loaded as above) with row scales (a.sd),
// applied to each split's sums.
template <int BT, int WAVES, int NBUF, int WPE, int TR, bool F8 = false>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void down_mfma_staged_kernel(
    DownArgs a, float *partial, int S, int CS) {
    constexpr int NT = WAVES * kWave;
    constexpr int XR = 16 * BT;
    constexpr int XPT = XR * kStKbc / NT;
    static_assert(XR * kStKbc % NT == 0, "staging split");
    constexpr int PLANE = XR * kStPitch;
    extern __shared__ u32x4_t smem[];  // [NBUF][hi, lo][XR][kStPitch]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    const int row_groups = (a.groups + WAVES * TR - 1) / (WAVES * TR);
    const int items = row_groups * S;

    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int sp = it % S, g = it / S;
        const int c0 = sp * CS, c1 = min(c0 + CS, a.C);
        const int nb = (c1 - c0 + kStKbc - 1) / kStKbc;
        const int tile0 = (g * WAVES + wave) * TR;
        const u32x4_t *pw[TR];
        float scd[TR][4];  // F8: the scales of this lane's output rows
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            const size_t row = (size_t)min((tile0 + t) * 16 + lr, a.M - 1);
            if constexpr (F8) {
                pw[t] = reinterpret_cast<const u32x4_t *>(a.qd + row * a.K);
#pragma unroll
                for (int e = 0; e < 4; ++e) scd[t][e] = a.sd[min((tile0 + t) * 16 + 4 * lq + e, a.M - 1)];
            } else {
                pw[t] = reinterpret_cast<const u32x4_t *>(a.wd + row * a.K);
            }
        }
        f32x4_t acc[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[t][bt] = f32x4_t{0, 0, 0, 0};

        auto load_h = [&](f32x4_t (&hr)[XPT][2], int kb) {
            const int cs = st_block_start(kb, c0, c1);
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = min(i / kStKbc, a.B - 1);
                const int c = min(cs + i % kStKbc, a.C - 1);
                hr[t][0] = hg[(size_t)b * 2 * a.C + 2 * c];
                hr[t][1] = hg[(size_t)b * 2 * a.C + 2 * c + 1];
            }
        };
        auto store_h = [&](const f32x4_t (&hr)[XPT][2], int kb) {
            const int cs = st_block_start(kb, c0, c1);
            u32x4_t *dhi = smem + (NBUF == 2 ? (kb & 1) : 0) * 2 * PLANE;
            u32x4_t *dlo = dhi + PLANE;
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = i / kStKbc, cc = i % kStKbc;
                const int c = cs + cc;
                const bool ok = b < a.B && c >= c0 + kb * kStKbc && c < c1;
                bf16x8_t hi, lo;
                split_hi_lo(ok ? hr[t][0] : fzero, ok ? hr[t][1] : fzero, hi, lo);
                const int v = F8 ? f8_step_slot(cc) : cc;
                dhi[b * kStPitch + v] = __builtin_bit_cast(u32x4_t, hi);
                dlo[b * kStPitch + v] = __builtin_bit_cast(u32x4_t, lo);
            }
        };
        auto load_w = [&](u32x4_t (&wr)[TR][8], int kb) {
            const int cs = st_block_start(kb, c0, c1);
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                if constexpr (F8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) wr[t][i] = load_stream(pw[t] + min(cs / 2 + 4 * i + lq, a.C / 2 - 1));
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) wr[t][j] = load_stream(pw[t] + min(cs + 4 * j + lq, a.C - 1));
                }
            }
        };
        // each B fragment read from LDS serves the wave's TR row tiles
        auto compute = [&](const u32x4_t (&wr)[TR][8], int kb) {
            const u32x4_t *shi = smem + (NBUF == 2 ? (kb & 1) : 0) * 2 * PLANE;
            const u32x4_t *slo = shi + PLANE;
            u32x4_t wf[TR][2];  // F8: the widened codes of steps j (even) and j + 1
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if constexpr (F8) {
                    if (j % 2 == 0) {
#pragma unroll
                        for (int t = 0; t < TR; ++t) e4m3x16_to_bf16(wr[t][j / 2], wf[t][0], wf[t][1]);
                    }
                }
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const int o = (bt * 16 + lr) * kStPitch + 4 * j + lq;
                    const bf16x8_t bhi = as_bf16x8(shi[o]), blo = as_bf16x8(slo[o]);
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        const bf16x8_t aw = as_bf16x8(F8 ? wf[t][j % 2] : wr[t][j]);
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bhi, acc[t][bt], 0, 0, 0);
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, blo, acc[t][bt], 0, 0, 0);
                    }
                }
            }
        };
        f32x4_t hr[XPT][2];
        u32x4_t w0[TR][8], w1[TR][8];
        auto step = [&](auto &cw, auto &nw, int kb) {
            load_h(hr, kb + 1);
            load_w(nw, kb + 1);
            DFK_ISSUE_FENCE();
            compute(cw, kb);
            if constexpr (NBUF == 1) __syncthreads();
            store_h(hr, kb + 1);
            __syncthreads();
        };
        auto last = [&](auto &cw, int kb) {
            compute(cw, kb);
            __syncthreads();
        };
        load_h(hr, 0);
        load_w(w0, 0);
        store_h(hr, 0);
        __syncthreads();
        int kb = 0;
        for (; kb + 2 < nb; kb += 2) {
            step(w0, w1, kb);
            step(w1, w0, kb + 1);
        }
        if (kb + 1 < nb) {
            step(w0, w1, kb);
            last(w1, kb + 1);
        } else {
            last(w0, kb);
        }
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            if (tile0 + t >= a.groups) break;
            const int m = (tile0 + t) * 16 + 4 * lq;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (b < a.B && m < a.M) {
                    f32x4_t v = acc[t][bt];
                    if constexpr (F8) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= scd[t][e];
                    }
                    if (S == 1) {
                        const unsigned lo = to_bf16_rne(v[0]) | ((unsigned)to_bf16_rne(v[1]) << 16);
                        const unsigned hi = to_bf16_rne(v[2]) | ((unsigned)to_bf16_rne(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(a.y + (size_t)b * a.M + m) = make_uint2(lo, hi);
                    } else {
                        *reinterpret_cast<f32x4_t *>(partial + ((size_t)sp * a.B + b) * a.M + m) = v;
                    }
                }
            }
        }
    }
}

// -------------------------- MFMA, LDS-transposed weights + x staged in LDS --
//
// Gate-up for a few batch tiles (BT >= 2): the LDS-transposed weight stream of
// the kernels above (2 rows x 512 B per load instruction, parked in a
// wave-private padded LDS tile, read back in A-fragment order, one block
// ahead in registers) with x staged in LDS per workgroup, block by block, as
// the B-operand-staged kernels do: the B fragments of every tile of the
// workgroup come from one staged copy instead of from L2 per wave.  One
// staged x buffer: a barrier before it is overwritten and one after.  A wave
// owns one 16-row tile (rows of W_gate and W_up); waves whose tile is past
// the end stream clamped rows and write nothing, so every wave reaches every
// barrier.
// F8: the weights are FP8 codes (a.qg, a.qu) with row scales (a.sg, a.su).
// NBUF = 2 double-buffers the staged x block (one barrier per block).
template <int BT, int WAVES, bool F8 = false, int NBUF = 1, int KBC = 32>
__global__ __launch_bounds__(WAVES * kWave) void gate_up_mfma_lts_kernel(GateUpArgs a) {
    using L = typename Pick<F8, Lt8<KBC, false, true>, Lt<KBC>>::T;
    constexpr int KP = KBC + 1;           // LDS pitch of a staged x row, chunks
    constexpr int NT = WAVES * kWave;
    constexpr int XR = 16 * BT;           // staged x rows: the padded batch
    constexpr int XPT = XR * KBC / NT;    // staged chunks per thread
    static_assert(XR * KBC % NT == 0, "staging split");
    static_assert(!(F8 && NBUF == 2), "FP8 instances keep one x buffer");
    constexpr int XBUF = XR * KP;
    extern __shared__ u32x4_t smem[];     // x blocks [NBUF][XR][KP], then [WAVES][2][L::kTile]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    // F8 (one x buffer) reaches its x block through xs, the bf16 kernels
    // through smem directly: the same addresses, but the two forms compile
    // to different schedules, and each is the faster one for its weights
    // (measured at the Llama-3-8B shape: FP8 at B = 64 49.9 us against
    // 56.8 us; bf16 at B = 17-32 with few row tiles 0.5-1.5 us faster)
    u32x4_t *xs = smem;
    u32x4_t *ltg = smem + NBUF * XBUF + (size_t)wave * 2 * L::kTile;
    u32x4_t *ltu = ltg + L::kTile;
    const int nb = (a.C + KBC - 1) / KBC;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t *xg = reinterpret_cast<const u32x4_t *>(a.x);
    const int wg_items = (a.groups + WAVES - 1) / WAVES;

    auto load_x = [&](u32x4_t (&xr)[XPT], int kb) {
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int i = t * NT + tid;
            const int b = min(i / KBC, a.B - 1);
            const int c = min(kb * KBC + i % KBC, a.C - 1);
            xr[t] = xg[(size_t)b * a.C + c];
        }
    };
    auto store_x = [&](const u32x4_t (&xr)[XPT], int kb) {
        u32x4_t *xd = F8 ? xs : smem + (NBUF == 2 ? (kb & 1) : 0) * XBUF;
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int i = t * NT + tid;
            const int b = i / KBC, cc = i % KBC;
            const bool ok = b < a.B && kb * KBC + cc < a.C;
            xd[b * KP + cc] = ok ? xr[t] : zero;
        }
    };

    for (int g = blockIdx.x; g < wg_items; g += gridDim.x) {
        const int tile = g * WAVES + wave;
        const int row0 = tile * 16;
        f32x4_t accg[BT], accu[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) accg[bt] = accu[bt] = f32x4_t{0, 0, 0, 0};
        float scg[4], scu[4];  // F8: the scales of this lane's output rows, loaded ahead of the weights
        if constexpr (F8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = min(row0 + 4 * lq + e, a.N - 1);
                scg[e] = a.sg[n];
                scu[e] = a.su[n];
            }
        }
        auto load_w = [&](u32x4_t (&vg)[L::kInsts], u32x4_t (&vu)[L::kInsts], int kb) {
            if constexpr (F8) {
                L::load(vg, a.qg, a.K, a.C, row0, a.N, kb, lane);
                L::load(vu, a.qu, a.K, a.C, row0, a.N, kb, lane);
            } else {
                L::load(vg, a.wg, a.ldw, a.C, row0, a.N, kb, lane);
                L::load(vu, a.wu, a.ldw, a.C, row0, a.N, kb, lane);
            }
        };
        auto compute = [&](u32x4_t (&vg)[L::kInsts], u32x4_t (&vu)[L::kInsts], int kb) {
            const u32x4_t *xd = F8 ? xs : smem + (NBUF == 2 ? (kb & 1) : 0) * XBUF;
            L::store(ltg, vg, kb, a.C, lane);
            L::store(ltu, vu, kb, a.C, lane);
#pragma unroll
            for (int j = 0; j < L::kSteps; ++j) {
                const bf16x8_t ag = L::frag(ltg, j, lr, lq);
                const bf16x8_t au = L::frag(ltu, j, lr, lq);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const bf16x8_t xb = as_bf16x8(xd[(bt * 16 + lr) * KP + L::kpos(4 * j + lq)]);
                    accg[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, xb, accg[bt], 0, 0, 0);
                    accu[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, xb, accu[bt], 0, 0, 0);
                }
            }
        };
        u32x4_t xr[XPT];
        u32x4_t vg0[L::kInsts], vu0[L::kInsts], vg1[L::kInsts], vu1[L::kInsts];
        // prefetch block kb + 1 (x first, then the weights), multiply block
        // kb, then park x(kb + 1) (with one buffer, once every wave is done
        // with x(kb); with two, the other buffer was released by the barrier
        // that ended block kb - 1)
        auto step = [&](auto &cg, auto &cu, auto &ng, auto &nu, int kb) {
            load_x(xr, kb + 1);
            load_w(ng, nu, kb + 1);
            DFK_ISSUE_FENCE();
            compute(cg, cu, kb);
            if constexpr (NBUF == 1) __syncthreads();
            store_x(xr, kb + 1);
            __syncthreads();
        };
        auto last = [&](auto &cg, auto &cu, int kb) {
            compute(cg, cu, kb);
            __syncthreads();
        };
        load_x(xr, 0);
        load_w(vg0, vu0, 0);
        store_x(xr, 0);
        __syncthreads();
        int kb = 0;
        for (; kb + 2 < nb; kb += 2) {
            step(vg0, vu0, vg1, vu1, kb);
            step(vg1, vu1, vg0, vu0, kb + 1);
        }
        if (kb + 1 < nb) {
            step(vg0, vu0, vg1, vu1, kb);
            last(vg1, vu1, kb + 1);
        } else {
            last(vg0, vu0, kb);
        }
        if (tile < a.groups) {
            const int n = row0 + 4 * lq;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (b < a.B && n < a.N) {
                    f32x4_t o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (F8) o[e] = silu_mul(scg[e] * accg[bt][e], scu[e] * accu[bt][e]);
                        else o[e] = silu_mul(accg[bt][e], accu[bt][e]);
                    }
                    *reinterpret_cast<f32x4_t *>(a.h + (size_t)b * a.N + n) = o;
                }
            }
        }
    }
}

// Down for a few batch tiles: LDS-transposed weight streaming (as the
// LT kernels) with h staged in LDS per workgroup, block by block, already
// split into bf16 hi + lo planes (as the B-operand-staged kernels), so the
// split and the h reads from L2 are shared by the workgroup's WAVES tiles.
// A work item is (WAVES row tiles, one of S K splits); S > 1 writes fp32
// partial sums that panel_reduce_kernel adds in split order.  Waves whose tile
// is past the end stream clamped rows and write nothing, so every wave
// reaches every barrier.
template <int BT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void down_mfma_lts_kernel(DownArgs a, float *partial, int S, int CS) {
    using L = Lt<32>;
    constexpr int KBC = 32;
    constexpr int NT = WAVES * kWave;
    constexpr int XR = 16 * BT;           // staged h rows: the padded batch
    constexpr int XPT = XR * KBC / NT;    // staged chunks per thread
    static_assert(XR * KBC % NT == 0, "staging split");
    constexpr int PLANE = XR * kStPitch;
    extern __shared__ u32x4_t smem[];     // h hi [XR][kStPitch], lo [XR][kStPitch], then [WAVES][L::kTile]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    u32x4_t *shi = smem, *slo = smem + PLANE;
    u32x4_t *ltw = smem + 2 * PLANE + (size_t)wave * L::kTile;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    const int row_groups = (a.groups + WAVES - 1) / WAVES;
    const int items = row_groups * S;

    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int sp = it % S, g = it / S;
        const int c0 = sp * CS, nch = min(CS, a.C - c0);
        const int nb = (nch + KBC - 1) / KBC;
        const int tile = g * WAVES + wave;
        const int row0 = tile * 16;
        f32x4_t acc[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) acc[bt] = fzero;
        auto load_h = [&](f32x4_t (&hr)[XPT][2], int kb) {
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = min(i / KBC, a.B - 1);
                const int c = min(c0 + kb * KBC + i % KBC, a.C - 1);
                hr[t][0] = hg[(size_t)b * 2 * a.C + 2 * c];
                hr[t][1] = hg[(size_t)b * 2 * a.C + 2 * c + 1];
            }
        };
        auto store_h = [&](const f32x4_t (&hr)[XPT][2], int kb) {
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = i / KBC, cc = i % KBC;
                const bool ok = b < a.B && kb * KBC + cc < nch;
                bf16x8_t hi, lo;
                split_hi_lo(ok ? hr[t][0] : fzero, ok ? hr[t][1] : fzero, hi, lo);
                shi[b * kStPitch + cc] = __builtin_bit_cast(u32x4_t, hi);
                slo[b * kStPitch + cc] = __builtin_bit_cast(u32x4_t, lo);
            }
        };
        auto load_w = [&](u32x4_t (&v)[L::kInsts], int kb) {
            L::load(v, a.wd + (size_t)c0 * 8, a.K, nch, row0, a.M, kb, lane);
        };
        auto compute = [&](u32x4_t (&v)[L::kInsts], int kb) {
            L::store(ltw, v, kb, nch, lane);
#pragma unroll
            for (int j = 0; j < L::kSteps; ++j) {
                const bf16x8_t aw = L::frag(ltw, j, lr, lq);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const int o = (bt * 16 + lr) * kStPitch + 4 * j + lq;
                    acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, as_bf16x8(shi[o]), acc[bt], 0, 0, 0);
                    acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, as_bf16x8(slo[o]), acc[bt], 0, 0, 0);
                }
            }
        };
        f32x4_t hr[XPT][2];
        u32x4_t v0[L::kInsts], v1[L::kInsts];
        // prefetch block kb + 1 (h first, then the weights), multiply block
        // kb, then park h(kb + 1) once every wave is done with h(kb)
        auto step = [&](auto &cv, auto &nv, int kb) {
            load_h(hr, kb + 1);
            load_w(nv, kb + 1);
            DFK_ISSUE_FENCE();
            compute(cv, kb);
            __syncthreads();
            store_h(hr, kb + 1);
            __syncthreads();
        };
        auto last = [&](auto &cv, int kb) {
            compute(cv, kb);
            __syncthreads();
        };
        load_h(hr, 0);
        load_w(v0, 0);
        store_h(hr, 0);
        __syncthreads();
        int kb = 0;
        for (; kb + 2 < nb; kb += 2) {
            step(v0, v1, kb);
            step(v1, v0, kb + 1);
        }
        if (kb + 1 < nb) {
            step(v0, v1, kb);
            last(v1, kb + 1);
        } else {
            last(v0, kb);
        }
        const int m = row0 + 4 * lq;
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
            const int b = bt * 16 + lr;
            if (tile < a.groups && b < a.B && m < a.M) {
                if (S == 1) {
                    const unsigned lo = to_bf16_rne(acc[bt][0]) | ((unsigned)to_bf16_rne(acc[bt][1]) << 16);
                    const unsigned hi = to_bf16_rne(acc[bt][2]) | ((unsigned)to_bf16_rne(acc[bt][3]) << 16);
                    *reinterpret_cast<uint2 *>(a.y + (size_t)b * a.M + m) = make_uint2(lo, hi);
                } else {
                    *reinterpret_cast<f32x4_t *>(partial + ((size_t)sp * a.B + b) * a.M + m) = acc[bt];
                }
            }
        }
    }
}

// Down for several batch tiles: the LDS-transposed weight stream with h
// staged per workgroup as bf16 hi + lo planes (as down_mfma_lts_kernel), but
// each wave owns TR consecutive 16-row tiles.  A wave parks its tiles one after
// the other in its single LDS tile and keeps their A fragments in registers,
// so every B fragment read from LDS feeds TR tiles while the LDS holds only
// one weight tile per wave next to the staged h (at four batch tiles, eight
// waves: 66 KiB of h planes + 66 KiB of tiles).  The LDS-transposed loads (2
// rows x 512 B per instruction) stream faster than A fragments loaded straight
// from HBM (16 rows x 64 B), the shape of down_mfma_staged_kernel.  A work
// item is (WAVES x TR row tiles, one of S K splits); S > 1 writes fp32 partial
// sums that panel_reduce_kernel adds in split order.  Waves whose tiles are
// past the end stream clamped rows and write nothing, so every wave reaches
// every barrier.  The next block's loads are issued before the current
// block's work (h first, then the weights); h(kb + 1) is parked once every
// wave is done with h(kb) (NBUF = 2: double-buffered h planes, one barrier
// per block).  F8: W_down is FP8 codes (a.qd), widened into the tile, with
// row scales (a.sd) applied to each split's sums.
template <int BT, int WAVES, int TR, int WPE, bool F8 = false, int NBUF = 1, int KBC = 32>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void down_mfma_ltsw_kernel(
    DownArgs a, float *partial, int S, int CS) {
    using L = typename Pick<F8, Lt8<KBC, true>, Lt<KBC>>::T;
    constexpr int KP = KBC + 1;           // LDS pitch of a staged h row, chunks
    constexpr int NT = WAVES * kWave;
    constexpr int XR = 16 * BT;           // staged h rows: the padded batch
    constexpr int XPT = XR * KBC / NT;    // staged chunks per thread
    static_assert(XR * KBC % NT == 0, "staging split");
    constexpr int PLANE = XR * KP;
    extern __shared__ u32x4_t smem[];     // [NBUF][h hi [XR][KP], lo [XR][KP]], then [WAVES][L::kTile]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    u32x4_t *ltw = smem + NBUF * 2 * PLANE + (size_t)wave * L::kTile;
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);
    const int row_groups = (a.groups + WAVES * TR - 1) / (WAVES * TR);
    const int items = row_groups * S;

    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int sp = it % S, g = it / S;
        const int c0 = sp * CS, nch = min(CS, a.C - c0);
        const int nb = (nch + KBC - 1) / KBC;
        const int tile0 = (g * WAVES + wave) * TR;
        f32x4_t acc[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[t][bt] = fzero;
        auto load_h = [&](f32x4_t (&hr)[XPT][2], int kb) {
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = min(i / KBC, a.B - 1);
                const int c = min(c0 + kb * KBC + i % KBC, a.C - 1);
                hr[t][0] = hg[(size_t)b * 2 * a.C + 2 * c];
                hr[t][1] = hg[(size_t)b * 2 * a.C + 2 * c + 1];
            }
        };
        auto store_h = [&](const f32x4_t (&hr)[XPT][2], int kb) {
            u32x4_t *shi = smem + (NBUF == 2 ? (kb & 1) : 0) * 2 * PLANE, *slo = shi + PLANE;
#pragma unroll
            for (int t = 0; t < XPT; ++t) {
                const int i = t * NT + tid;
                const int b = i / KBC, cc = i % KBC;
                const bool ok = b < a.B && kb * KBC + cc < nch;
                bf16x8_t hi, lo;
                split_hi_lo(ok ? hr[t][0] : fzero, ok ? hr[t][1] : fzero, hi, lo);
                shi[b * KP + cc] = __builtin_bit_cast(u32x4_t, hi);
                slo[b * KP + cc] = __builtin_bit_cast(u32x4_t, lo);
            }
        };
        auto load_w = [&](u32x4_t (&v)[TR][L::kInsts], int kb) {
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                if constexpr (F8) L::load(v[t], a.qd + (size_t)c0 * 8, a.K, nch, (tile0 + t) * 16, a.M, kb, lane);
                else L::load(v[t], a.wd + (size_t)c0 * 8, a.K, nch, (tile0 + t) * 16, a.M, kb, lane);
            }
        };
        // each B fragment read from LDS serves the wave's TR row tiles
        auto compute = [&](u32x4_t (&v)[TR][L::kInsts], int kb) {
            const u32x4_t *shi = smem + (NBUF == 2 ? (kb & 1) : 0) * 2 * PLANE, *slo = shi + PLANE;
            bf16x8_t af[TR][L::kSteps];
#pragma unroll
            for (int t = 0; t < TR; ++t) {
                L::store(ltw, v[t], kb, nch, lane);
#pragma unroll
                for (int j = 0; j < L::kSteps; ++j) af[t][j] = L::frag(ltw, j, lr, lq);
            }
#pragma unroll
            for (int j = 0; j < L::kSteps; ++j) {
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const int o = (bt * 16 + lr) * KP + L::kpos(4 * j + lq);
                    const bf16x8_t bhi = as_bf16x8(shi[o]), blo = as_bf16x8(slo[o]);
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][j], bhi, acc[t][bt], 0, 0, 0);
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t][j], blo, acc[t][bt], 0, 0, 0);
                    }
                }
            }
        };
        f32x4_t hr[XPT][2];
        u32x4_t v0[TR][L::kInsts], v1[TR][L::kInsts];
        auto step = [&](auto &cv, auto &nv, int kb) {
            load_h(hr, kb + 1);
            load_w(nv, kb + 1);
            DFK_ISSUE_FENCE();
            compute(cv, kb);
            // with two buffers, h(kb + 1) goes to the one that block kb - 1
            // used, released by the barrier that ended it
            if constexpr (NBUF == 1) __syncthreads();
            store_h(hr, kb + 1);
            __syncthreads();
        };
        auto last = [&](auto &cv, int kb) {
            compute(cv, kb);
            __syncthreads();
        };
        load_h(hr, 0);
        load_w(v0, 0);
        store_h(hr, 0);
        __syncthreads();
        int kb = 0;
        for (; kb + 2 < nb; kb += 2) {
            step(v0, v1, kb);
            step(v1, v0, kb + 1);
        }
        if (kb + 1 < nb) {
            step(v0, v1, kb);
            last(v1, kb + 1);
        } else {
            last(v0, kb);
        }
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            const int tile = tile0 + t;
            const int m = tile * 16 + 4 * lq;
            float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (F8) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sc[e] = a.sd[min(m + e, a.M - 1)];
            }
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const int b = bt * 16 + lr;
                if (tile < a.groups && b < a.B && m < a.M) {
                    f32x4_t v = acc[t][bt];
                    if constexpr (F8) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= sc[e];
                    }
                    if (S == 1) {
                        const unsigned lo = to_bf16_rne(v[0]) | ((unsigned)to_bf16_rne(v[1]) << 16);
                        const unsigned hi = to_bf16_rne(v[2]) | ((unsigned)to_bf16_rne(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(a.y + (size_t)b * a.M + m) = make_uint2(lo, hi);
                    } else {
                        *reinterpret_cast<f32x4_t *>(partial + ((size_t)sp * a.B + b) * a.M + m) = v;
                    }
                }
            }
        }
    }
}

// ----------------------- MFMA, workgroup-cooperative weight tile (down) -----
//
// The down projection's row traversal on the matrix cores, for batches up to
// 16.  A workgroup owns whole rows: a tile of 16 rows of W_down, walked over
// all of K in stages of KSC 16-byte chunks per row.  In a stage every wave
// loads whole runs of its RPW rows, one row x 1 KB per load instruction (the
// access shape that streams at full HBM rate), and parks them in a shared,
// double-buffered LDS tile (pitch KSC + 1).  After one barrier each wave
// multiplies its own K slice of the stage (KSC / WAVES chunks) over the 16 rows
// on the matrix cores, with B fragments (h split into bf16 hi + lo) from
// registers.  Two register buffers (weights and B fragments) alternate between
// the halves of a loop unrolled by two: a stage's B fragments and then its
// weights are issued before the previous stage's weights are waited for, and
// since loads complete in issue order every wait is for the oldest loads only
// (scheduling barriers keep that issue order).  At the end of a tile the
// waves' partial sums are added in wave order through the LDS tile just used.
// A workgroup takes tiles in sequence and the pipeline runs across tile
// boundaries; the last one or two stages are peeled, so no load in the loop is
// conditional.  K spans at least one stage (the plan guarantees it) and the
// last stage is shifted back to end at the row end, the chunks it repeats
// zeroed in the tile and in the B fragments: no load leaves its row and none
// needs a clamp.

template <int WAVES, int KSC> struct Coop {
    static constexpr int RPW = 16 / WAVES;     // tile rows loaded per wave
    static constexpr int NI = RPW * KSC / 64;  // load instructions per wave and stage
    static constexpr int PITCH = KSC + 1;      // LDS tile pitch, chunks
    static constexpr int SL = KSC / WAVES;     // chunks of a wave's K slice
    static constexpr int STEPS = SL / 4;       // MFMA K steps per wave and stage
    static constexpr int TILE = 16 * PITCH;    // one LDS tile, chunks
    static_assert(RPW * WAVES == 16 && NI * 64 == RPW * KSC && STEPS * 4 * WAVES == KSC && KSC % 64 == 0,
                  "cooperative tile shape");
    static_assert(WAVES * 4 * 64 * 4 <= TILE * 16, "the combine area fits a tile");
};

template <int WAVES, int KSC>
__global__ __launch_bounds__(WAVES * kWave) void down_mfma_coop_kernel(DownArgs a) {
    using T = Coop<WAVES, KSC>;
    extern __shared__ u32x4_t smem[];  // tiles [2][16][PITCH]; the tile-end combine reuses one
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lr = lane & 15, lq = lane >> 4;
    const int ns = (a.C + KSC - 1) / KSC;  // stages per tile
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
    // stage st of tile t: first chunk (the last stage ends at the row end) and
    // the first chunk not counted by an earlier stage
    auto start = [&](int st) { return min(st * KSC, a.C - KSC); };
    auto load_w = [&](u32x4_t (&wv)[T::NI], int t, int st) {
        const int cs = start(st);
        const int row0 = t * 16 + wave * T::RPW;
#pragma unroll
        for (int i = 0; i < T::NI; ++i) {
            const int row = min(row0 + i * kWave / KSC, a.M - 1);
            const u32x4_t *pw = reinterpret_cast<const u32x4_t *>(a.wd + (size_t)row * a.K) + cs + (i * kWave) % KSC;
            wv[i] = load_stream(pw + lane);
        }
    };
    // B fragments of this wave's K slice: h[b][8 floats] per lane and step
    const char *hlane = reinterpret_cast<const char *>(a.h) + ((size_t)min(lr, a.B - 1) * a.K + 8 * lq) * 4;
    auto load_h = [&](f32x4_t (&hb)[T::STEPS][2], int st) {
        const int cs = start(st);
#pragma unroll
        for (int j = 0; j < T::STEPS; ++j) {
            const f32x4_t *ph = reinterpret_cast<const f32x4_t *>(hlane + (size_t)(cs + wave * T::SL + 4 * j) * 32);
            hb[j][0] = ph[0];
            hb[j][1] = ph[1];
        }
    };
    f32x4_t acc = fzero;
    // park the stage's weights, then multiply this wave's slice; after the
    // tile's last stage combine the waves and write y
    auto half = [&](const u32x4_t (&wv)[T::NI], const f32x4_t (&hb)[T::STEPS][2], int t, int st, int buf) {
        const int cs = start(st), lo = st * KSC;  // chunks below lo belong to earlier stages
        u32x4_t *tile = smem + buf * T::TILE;
#pragma unroll
        for (int i = 0; i < T::NI; ++i) {
            const int cc = (i * kWave) % KSC + lane;
            tile[(wave * T::RPW + i * kWave / KSC) * T::PITCH + cc] = cs + cc >= lo ? wv[i] : zero;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < T::STEPS; ++j) {
            const int cc = wave * T::SL + 4 * j + lq;
            const bool ok = cs + cc >= lo;
            bf16x8_t hi, lo8;
            split_hi_lo(ok ? hb[j][0] : fzero, ok ? hb[j][1] : fzero, hi, lo8);
            const bf16x8_t aw = as_bf16x8(tile[lr * T::PITCH + cc]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, hi, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, lo8, acc, 0, 0, 0);
        }
        if (st + 1 == ns) {
            float *red = reinterpret_cast<float *>(tile);
            __syncthreads();  // every wave is done with the tile
            float *dst = red + (size_t)wave * 4 * kWave;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e * kWave + lane] = acc[e];
            __syncthreads();
            if (wave == 0) {
                f32x4_t sum = fzero;
                for (int w = 0; w < WAVES; ++w)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum[e] += red[((size_t)w * 4 + e) * kWave + lane];
                const int m = t * 16 + 4 * lq;
                if (lr < a.B && m < a.M) {
                    const unsigned l2 = to_bf16_rne(sum[0]) | ((unsigned)to_bf16_rne(sum[1]) << 16);
                    const unsigned h2 = to_bf16_rne(sum[2]) | ((unsigned)to_bf16_rne(sum[3]) << 16);
                    *reinterpret_cast<uint2 *>(a.y + (size_t)lr * a.M + m) = make_uint2(l2, h2);
                }
            }
            acc = fzero;
        }
    };
    if ((int)blockIdx.x >= a.groups) return;
    // the workgroup's stages: tiles blockIdx.x, blockIdx.x + gridDim.x, ...
    const int total = ((a.groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * ns;
    u32x4_t w0[T::NI], w1[T::NI];
    f32x4_t h0[T::STEPS][2], h1[T::STEPS][2];
    int t0 = blockIdx.x, s0 = 0;
    auto next = [&](int &t, int &st) {
        if (++st == ns) {
            st = 0;
            t += gridDim.x;
        }
    };
    load_h(h0, s0);
    load_w(w0, t0, s0);
    __builtin_amdgcn_sched_barrier(0);
    int g = 0;
    for (; g + 2 < total; g += 2) {
        int t1 = t0, s1 = s0;
        next(t1, s1);
        load_h(h1, s1);
        load_w(w1, t1, s1);
        __builtin_amdgcn_sched_barrier(0);
        half(w0, h0, t0, s0, 0);
        int t2 = t1, s2 = s1;
        next(t2, s2);
        load_h(h0, s2);
        load_w(w0, t2, s2);
        __builtin_amdgcn_sched_barrier(0);
        half(w1, h1, t1, s1, 1);
        t0 = t2;
        s0 = s2;
    }
    if (g + 1 < total) {
        int t1 = t0, s1 = s0;
        next(t1, s1);
        load_h(h1, s1);
        load_w(w1, t1, s1);
        __builtin_amdgcn_sched_barrier(0);
        half(w0, h0, t0, s0, 0);
        half(w1, h1, t1, s1, 1);
    } else {
        half(w0, h0, t0, s0, 0);
    }
}

// y[i] = RNE_bf16(sum_{s ascending} partial[s][i]) for i < n (n % 4 == 0),
// four outputs per thread.  The partial sums were written by workgroups on
// every die, so each load goes to the memory-side cache or HBM: a thread
// issues DFK_REDUCE_BATCH of its loads before it adds them (still in
// ascending s), and small workgroups spread the few threads over many CUs.
#ifndef DFK_REDUCE_BLOCK
#define DFK_REDUCE_BLOCK 64
#endif
#ifndef DFK_REDUCE_BATCH
#define DFK_REDUCE_BATCH 8
#endif
constexpr int kReduceBlock = DFK_REDUCE_BLOCK;

__global__ __launch_bounds__(kReduceBlock) void panel_reduce_kernel(const float *partial, uint16_t *y, int S, int n) {
    const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    const f32x4_t *p = reinterpret_cast<const f32x4_t *>(partial + i);
    const size_t stride = (size_t)n / 4;  // one split, in 16-byte vectors
    constexpr int kBatch = DFK_REDUCE_BATCH;
    f32x4_t v = p[0];
    for (int s0 = 1; s0 < S; s0 += kBatch) {
        f32x4_t t[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (s0 + q < S) t[q] = p[(size_t)(s0 + q) * stride];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (s0 + q < S) v += t[q];
    }
    const unsigned lo = to_bf16_rne(v[0]) | ((unsigned)to_bf16_rne(v[1]) << 16);
    const unsigned hi = to_bf16_rne(v[2]) | ((unsigned)to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<uint2 *>(y + i) = make_uint2(lo, hi);
}

static hipError_t launch_reduce(const float *partial, uint16_t *y, int S, int n, hipStream_t stream) {
    void *rargv[] = {&partial, &y, &S, &n};
    return hipLaunchKernel((const void *)panel_reduce_kernel, dim3((unsigned)((n / 4 + kReduceBlock - 1) / kReduceBlock)),
                           dim3(kReduceBlock), rargv, 0, stream);
}

// ======================================================== kernel tables ====
//
// Tile parameters, overridable at compile time (-D) for sweeps.
//   VALU: R rows (pairs) per item, U load groups in flight per lane.
//   MFMA: TR row tiles of 16 per item, U K steps per load group, WAVES per
//         workgroup of the col kernels (their LDS combine needs
//         (WAVES-1) x NV x 256 bytes).  BT = ceil(B / 16) batch tiles.
// (defaults from a sweep on the Llama-3-8B layer shape, MI355X)
#ifndef DFK_GU_VALU_R
#define DFK_GU_VALU_R(B) 1
#endif
#ifndef DFK_GU_VALU_U
#define DFK_GU_VALU_U(B) ((B) == 4 ? 3 : 4)
#endif
#ifndef DFK_DN_VALU_R
#define DFK_DN_VALU_R(B) ((B) <= 2 ? 2 : 4)
#endif
#ifndef DFK_DN_VALU_U
#define DFK_DN_VALU_U(B) ((B) <= 2 ? 4 : 1)
#endif
#ifndef DFK_GU_MFMA_TR
#define DFK_GU_MFMA_TR(BT) 1
#endif
#ifndef DFK_GU_MFMA_U
#define DFK_GU_MFMA_U(BT) ((BT) <= 2 ? 4 : ((BT) <= 8 ? 2 : 1))
#endif
#ifndef DFK_GU_MFMA_WAVES
#define DFK_GU_MFMA_WAVES(BT) ((BT) <= 4 ? 8 : 4)
#endif
#ifndef DFK_DN_MFMA_TR
#define DFK_DN_MFMA_TR(BT) 1
#endif
#ifndef DFK_DN_MFMA_U
#define DFK_DN_MFMA_U(BT) ((BT) <= 2 ? 4 : 2)
#endif
#ifndef DFK_DN_MFMA_WAVES
#define DFK_DN_MFMA_WAVES(BT) ((BT) <= 4 ? 8 : 4)
#endif
// all of h stays in LDS for the VALU down kernels up to this many bytes
#ifndef DFK_HLDS_LIMIT
#define DFK_HLDS_LIMIT kHLdsLimit
#endif
// 0: persistent grid (at most the blocks that fit the machine at once);
// 1: one block per group of work items (the hardware dispatcher balances)
#ifndef DFK_GRID_MODE
#define DFK_GRID_MODE 0
#endif
// 1: size persistent grids so every work item slot gets the same item count
#ifndef DFK_BALANCE
#define DFK_BALANCE 1
#endif
// the down projection's col traversal uses K panels across workgroups up to
// this batch (h panels in LDS), and the in-workgroup K split above it
// MFMA row/col kernels: the LDS-transposed weight stream (1) or the direct
// 16-row fragment loads (0); the transposed kernels cover B <= 128
// gate-up row traversal for BT in [2, DFK_GU_LTS_MAX_BT]: LDS-transposed
// weights with x staged in LDS (DFK_GU_LTS_WAVES waves per workgroup).  At
// the Llama-3-8B shape this took B = 32 from 49.8 to 44.1 us and B = 64 from
// 58.1 to 53.9 us against the B-operand-staged kernel; 2 waves per workgroup
// were ~1 us faster at BT = 2 there but 22 us slower at the 70B shape
#ifndef DFK_GU_LTS_MAX_BT
#define DFK_GU_LTS_MAX_BT 4
#endif
// the same kernel from this many batch tiles, bf16 and FP8 weights; bf16 at
// one batch tile only while the row tiles number fewer than
// DFK_GU_LTS_BT1_TILES_X10 / 10 per CU.  Event-timed gate-up row traversal,
// us at B = 4 / 8 / 16, the LT kernel against this one: 3072 x 8192 20.0 /
// 19.9 / 20.4 against 17.6 / 17.5 / 17.5; 5120 x 13824 48.3 / 49.4 / 53.6
// against 47.0 / 47.0 / 47.2; but Llama-3-8B (3.5 tiles per CU) 39.7 / 40.2 /
// 42.0 against 40.7 / 40.8 / 40.9 and Llama-3-70B 153 against 171.  FP8 codes
// at one batch tile too: event-timed FP8 row traversal, us at B = 4 / 8 / 16,
// the LT kernel against this one: Llama-3-8B 31.9 / 29.9 / 29.9 against 29.8 /
// 26.4 / 26.1, 5120 x 13824 34.2 / 34.5 / 36.4 against 30.5 / 30.5 / 30.7, but
// Llama-3-70B (7 row tiles per CU) 82.3 / 83.4 / 90.2 against 94.9 / 96.5 /
// 96.0; there (at least DFK_GU_LTS_F8_BT1_TILES_X10 / 10 row tiles per CU)
// one batch tile takes 128-element blocks, 79.3 / 79.6 / 79.3 (below it they
// lost: 8B 28.2 / 27.8 / 27.9, 5120 x 13824 32.8 / 32.9 / 33.0)
#ifndef DFK_GU_LTS_NBUF_BT2
#define DFK_GU_LTS_NBUF_BT2 1
#endif
// x buffers at four batch tiles (regular width): two measured 51.5 / 188.3 /
// 64.2 us against 52.1 / 190.5 / 65.2 us at B = 64 (8B / 70B / 5120 x 13824)
#ifndef DFK_GU_LTS_NBUF_BT4
#define DFK_GU_LTS_NBUF_BT4 2
#endif
#ifndef DFK_GU_LTS_MIN_BT
#define DFK_GU_LTS_MIN_BT 1
#endif
// K block of the bf16 staged-x gate-up kernel: 16 chunks (128 elements, a
// double-buffered x block, a third of the LDS) from DFK_GU_LTS_K16_MIN_BT
// batch tiles, with four-wave workgroups from DFK_GU_LTS_K16_W4_X row tiles
// per CU and two-wave ones below (more workgroups per CU).  Event-timed
// gate-up at B = 64, us, 32 chunks against 16: 8B 51.8 against 48.8 (four
// waves); 70B 188.5 against 185.0 (four); 5120 x 13824 64.4 against 56.2
// (four); 3072 x 8192 31.1 against 27.7 (two); 2048 x 5632 21.9 against 19.7
// (two).  At three batch tiles (B = 40 / 48) 8B 46.1 / 46.2 against 44.7 /
// 44.9, 5120 x 13824 56.8 / 57.0 against 49.8 / 50.4, 3072 x 8192 and 2048 x
// 5632 1.1-1.8 us faster, but 70B 168.9 / 170.1 against 178.5 / 176.7: there
// (at least DFK_GU_LTS_K16_BT3_MAX_X row tiles per CU) 32 chunks stay.  At two
// batch tiles it was shape-dependent (70B B = 32: 159 against 166-175 us), so
// 32 chunks stay there.
#ifndef DFK_GU_LTS_K16_MIN_BT
#define DFK_GU_LTS_K16_MIN_BT 3
#endif
#ifndef DFK_GU_LTS_K16_BT3_MAX_X
#define DFK_GU_LTS_K16_BT3_MAX_X 4
#endif
// FP8 codes in the staged-x gate-up kernel from this many batch tiles (and at
// one batch tile from DFK_GU_LTS_F8_BT1_TILES_X10 / 10 row tiles per CU):
// 128-element blocks (one x buffer), workgroup width as for bf16.  Event-timed
// FP8 gate-up, us at B = 40 / 64, 256-element blocks against 128: 70B 141.8 /
// 168.4 against 107.7 / 124.7; 3072 x 8192 28.9 / 34.0 against 22.0 / 25.5;
// 2048 x 5632 20.4 / 23.7 against 15.9 / 18.2; 5120 x 13824 46.5 / 54.8
// against 46.5 / 51.3; 8B 38.2 / 44.9 against 38.3 / 42.6; at B = 24 / 32 70B
// 121.3 / 121.1 against 95.6 / 98.6, 3072 x 8192 24.6 / 24.8 against 21.7 /
// 21.7, 2048 x 5632 17.3 / 17.4 against 15.3 / 15.3, 8B and 5120 x 13824
// within 0.3 us.
#ifndef DFK_GU_LTS_F8_K16_MIN_BT
#define DFK_GU_LTS_F8_K16_MIN_BT 2
#endif
#ifndef DFK_GU_LTS_K16_W4_X
#define DFK_GU_LTS_K16_W4_X 3
#endif
#ifndef DFK_GU_LTS_BT1_TILES_X10
#define DFK_GU_LTS_BT1_TILES_X10 35
#endif
#ifndef DFK_GU_LTS_F8_MIN_BT
#define DFK_GU_LTS_F8_MIN_BT 1
#endif
#ifndef DFK_GU_LTS_F8_BT1_TILES_X10
#define DFK_GU_LTS_F8_BT1_TILES_X10 50
#endif
#ifndef DFK_GU_LTS_WAVES
#define DFK_GU_LTS_WAVES 4
#endif
// fewer waves per workgroup (more workgroups) when the 16-row tiles number
// fewer than DFK_GU_LTS_NARROW_X2 / 2 per CU (DFK_GU_LTS_NARROW_X2_BT2 / 2 at
// BT = 2).  Swept over the scheduler's shapes at B = 32 / 48 / 64: d_model
// 2048 (352 tiles) 21.5 / 23.9 / 26.3 -> 16.7 / 22.4 / 24.0 us; d_model 3072
// (512 tiles, where 4-wave workgroups would fill half of the CUs) 33.5 /
// 34.9 / 38.4 -> 25.8 / 34.2 / 34.4 us; 2 waves at BT = 3-4 with 864-896
// tiles were 9-11 us slower, at the 70B shape (1792 tiles) slower too
#ifndef DFK_GU_LTS_NARROW_WAVES
#define DFK_GU_LTS_NARROW_WAVES 2
#endif
#ifndef DFK_GU_LTS_NARROW_X2
#define DFK_GU_LTS_NARROW_X2 5
#endif
#ifndef DFK_GU_LTS_NARROW_X2_BT2
#define DFK_GU_LTS_NARROW_X2_BT2 8
#endif
// staged x buffers of the regular-width kernel at BT = 3 (two: one barrier
// per block; measured at B = 48, 8B / 5120 x 13824 / 70B shapes: 48.7 /
// 62.6 / 178.3 us against 50.5 / 64.2 / 186.0 with one; at BT = 4 two were
// slower)
#ifndef DFK_GU_LTS_NBUF_BT3
#define DFK_GU_LTS_NBUF_BT3 2
#endif
#ifndef DFK_MFMA_LT
#define DFK_MFMA_LT 1
#endif
// waves per workgroup and K split of the transposed kernels (LDS: 8.25 KB
// per wave and weight matrix, plus the K-split combine)
#ifndef DFK_LT_GU_WAVES
#define DFK_LT_GU_WAVES(BT) 4
#endif
// the row traversal (no K split) runs one tile per workgroup: more, smaller
// workgroups spread the 16-neuron tiles over every CU
#ifndef DFK_LT_GU_ROW_WAVES
#define DFK_LT_GU_ROW_WAVES(BT) 1
#endif
#ifndef DFK_LT_GU_KSPLIT
#define DFK_LT_GU_KSPLIT(BT) 4
#endif
#ifndef DFK_LT_DN_WAVES
#define DFK_LT_DN_WAVES(BT) 4
#endif
#ifndef DFK_LT_DN_KBC
#define DFK_LT_DN_KBC 32
#endif
#ifndef DFK_LT_DN_KSPLIT
#define DFK_LT_DN_KSPLIT(BT) 4
#endif
// down column traversal at one batch tile (B <= 16): the LDS-transposed
// kernel with staged h, DFK_DN_LTS_WAVES tiles per workgroup
// (DFK_DN_LTS_WIDE_WAVES above B = 8 when the row tiles number two per CU or
// more), K splits of at least DFK_DN_LTS_MIN_CHUNKS chunks.  Event-timed down,
// us, Llama-3-8B shape B = 8 / 16: 25.6 / 26.6 against 27.5 / 32.4 for the LT
// column kernel and the K-panel kernel it replaced; Llama-3-70B shape B = 8 /
// 16: 78.7 / 84.0 against 95.6 / 104.9.  Two batch tiles (B = 17-32) gained
// about 1 us at the 8B shape and nothing at 70B: the staged kernel stays.
#ifndef DFK_DN_LTS_WAVES
#define DFK_DN_LTS_WAVES 2
#endif
#ifndef DFK_DN_LTS_WIDE_WAVES
#define DFK_DN_LTS_WIDE_WAVES 4
#endif
#ifndef DFK_DN_LTS_MIN_CHUNKS
#define DFK_DN_LTS_MIN_CHUNKS 128
#endif
// down column traversal from DFK_DN_LTSW_MIN_BT to DFK_DN_LTSW_MAX_BT batch
// tiles (0: never): LDS-transposed weights, h staged per workgroup; workgroups
// of DFK_DN_LTSW_WAVES waves, of four when at most two batch tiles meet fewer
// row tiles than DFK_DN_LTSW_NARROW_PCT % of the CUs; DFK_DN_LTSW_TR row tiles
// per wave at one or two batch tiles when the row tiles number at least
// DFK_DN_LTSW_TR2_X per CU, one otherwise; K splits of at least
// DFK_DN_LTSW_MIN_CHUNKS chunks.  FP8 codes take the same kernel from
// DFK_DN_LTSW_F8_MIN_BT to DFK_DN_LTSW_F8_MAX_BT batch tiles (event-timed
// FP8 down, us at B = 4 / 8 / 16: 17.3 / 17.8 / 17.9 against 18.9 / 19.8 /
// 22.2 on the staged kernel at the Llama-3-8B shape, 45.7 / 46.2 / 47.8
// against 52.2 / 53.2 / 55.2 at Llama-3-70B; at three and four batch tiles it
// lost, 94 / 115 against 76 / 87 us at 70B, B = 48 / 64).  With
// DFK_DN_LTSW_MIN_BT above 1, bf16 weights at one batch tile take
// down_mfma_lts_kernel instead (event-timed down, us at B = 1 / 8 / 16, that
// kernel against this one: 8B shape 23.1 / 23.9 / 25.7 against 22.4 / 22.7 /
// 23.2; 70B 76.2 / 79.5 / 80.3 against 73.2 / 73.7 / 74.5; 5120 x 13824
// 31.3 / 32.1 / 34.4 against 25.7 / 26.3 / 27.0; 2048 x 5632 12.3 / 12.5 /
// 12.7 against 9.3 / 9.7 / 10.1; 3072 x 8192 0.1-0.2 us faster).
#ifndef DFK_DN_LTSW_MIN_BT
#define DFK_DN_LTSW_MIN_BT 1
#endif
#ifndef DFK_DN_LTSW_MAX_BT
#define DFK_DN_LTSW_MAX_BT 4
#endif
#ifndef DFK_DN_LTSW_WAVES
#define DFK_DN_LTSW_WAVES 8
#endif
#ifndef DFK_DN_LTSW_TR
#define DFK_DN_LTSW_TR 2
#endif
#ifndef DFK_DN_LTSW_TR2_X
#define DFK_DN_LTSW_TR2_X 2
#endif
// h buffers of the bf16 instances at one or two batch tiles (two fit next to
// the tiles there: one barrier per block instead of two).  Event-timed down,
// us, one buffer against two: 8B B = 8 / 16 / 24 / 32 22.8 / 23.3 / 27.3 /
// 28.7 against 22.6 / 23.1 / 26.8 / 27.6; 70B B = 32 84.0 against 81.9; FP8
// codes within +-0.3 us either way, so they keep one.
// bf16 K block at four batch tiles: 32 chunks (256 elements) or 16.  With 16,
// two row tiles per wave fit in registers (239 VGPRs, no spill), taken when
// the row tiles number at least DFK_DN_LTSW_BT4_TR2_Q quarters per CU, and
// three batch tiles run the four-tile instance (one zero tile; 48 rows x 16
// chunks do not split evenly over 512 threads) when DFK_DN_LTSW_BT3_AS_BT4
// and the row tiles number at least one per CU (B = 33 / 40 / 48, us: 70B
// 100.6 / 102.3 / 105.3 -> 87.2 / 89.2 / 91.0; 5120 x 13824 39.2 / 40.2 ->
// 36.0 / 36.1 at B = 40 / 48; 8B 31.4 / 32.4 / 33.1 -> 30.4 / 31.5 / 32.9; on
// the two smaller shapes 0.4-1 us slower).
// Event-timed down at B = 64, us, 32 chunks and one tile per wave against 16
// chunks and two: 8B 39.4 against 35.8; 70B 123.8 against 95.8; 5120 x 13824
// 45.6 against 39.3; 3072 x 8192 24.7 against 23.1; 2048 x 5632 (half a row
// tile per CU) 16.9 against 19.4, and 16.4 with 16 chunks and one tile.
#ifndef DFK_DN_LTSW_KBC_BT4
#define DFK_DN_LTSW_KBC_BT4 16
#endif
// the same at two batch tiles (B = 17 / 24 / 32, us, 32 chunks against 16:
// 70B 78.2 / 79.1 / 81.3 against 74.6 / 75.4 / 77.4; 8B 26.1 / 26.5 / 27.4
// against 25.0 / 26.1 / 27.3; 5120 x 13824 31.3 / 32.3 against 29.9 / 31.2 at
// B = 24 / 32; 3072 x 8192 within 0.3 us).  One batch tile keeps 32 chunks:
// 16 rows x 16 chunks do not split over eight waves.
#ifndef DFK_DN_LTSW_KBC_BT2
#define DFK_DN_LTSW_KBC_BT2 16
#endif
// one batch tile with 16 chunks needs four-wave workgroups; measured mixed
// against eight waves and 32 chunks (us at B = 1 / 4 / 16: 8B 23.3 / 23.4 /
// 25.3 against 22.8 / 22.8 / 23.1; 3072 x 8192 12.4 / 12.8 / 14.1 against 13.2
// / 13.4 / 14.0; 70B 72.3 / 72.4 / 76.6 against 73.4 / 73.6 / 74.6), so 32
#ifndef DFK_DN_LTSW_KBC_BT1
#define DFK_DN_LTSW_KBC_BT1 32
#endif
#ifndef DFK_DN_LTSW_BT4_TR2_Q
#define DFK_DN_LTSW_BT4_TR2_Q 3
#endif
#ifndef DFK_DN_LTSW_BT3_AS_BT4
#define DFK_DN_LTSW_BT3_AS_BT4 1
#endif
#ifndef DFK_DN_LTSW_NBUF_BT12
#define DFK_DN_LTSW_NBUF_BT12 2
#endif
#ifndef DFK_DN_LTSW_F8_MIN_BT
#define DFK_DN_LTSW_F8_MIN_BT 1
#endif
#ifndef DFK_DN_LTSW_F8_MAX_BT
#define DFK_DN_LTSW_F8_MAX_BT 1
#endif
#ifndef DFK_DN_LTSW_MIN_CHUNKS
#define DFK_DN_LTSW_MIN_CHUNKS 64
#endif
#ifndef DFK_DN_LTSW_NARROW_PCT
#define DFK_DN_LTSW_NARROW_PCT 50
#endif
// B-operand-staged MFMA kernels: used from this many batch tiles up to
// kStMaxBT (gate-up ROW traversal, down COL traversal); waves per workgroup
// and LDS buffers per staged block
#ifndef DFK_ST_GU_MIN_BT
#define DFK_ST_GU_MIN_BT 3
#endif
#ifndef DFK_ST_DN_MIN_BT
#define DFK_ST_DN_MIN_BT 2
#endif
#ifndef DFK_ST_GU_NBUF
#define DFK_ST_GU_NBUF(BT) ((BT) <= 4 ? 2 : 1)
#endif
// FP8 down column traversal on the staged kernel from this many batch tiles
// (B = 6-16 at the Llama-3-8B shape: 23-25 us, against 28-32 us for the
// LDS-transposed kernel)
// wide (8-wave) staged down kernels from BT = 3 only when the row tiles
// number more than DFK_ST_DN_WIDE_X2 / 2 per CU; splits down to this many
// chunks when the row groups times the regular splits do not reach one work
// item per CU.  At d_model 2048 (d_ff 5632), B = 48 / 64: 17.4 / 20.8 us
// instead of 42.2 / 46.3 us (40 work items on 256 CUs before); no change at
// the larger shapes of the sweep
#ifndef DFK_ST_DN_WIDE_X2
#define DFK_ST_DN_WIDE_X2 1
#endif
#ifndef DFK_ST_DN_SMALL_MIN_CHUNKS
#define DFK_ST_DN_SMALL_MIN_CHUNKS 64
#endif
#ifndef DFK_ST_DN_F8_MIN_BT
#define DFK_ST_DN_F8_MIN_BT 1
#endif
#ifndef DFK_ST_DN_NBUF
#define DFK_ST_DN_NBUF(BT) ((BT) <= 2 ? 2 : 1)
#endif
// Workgroups of 8 waves share each staged block among more tiles; they are
// used when they still give (almost) every CU a workgroup, i.e. when
// ceil(tiles / 8) >= 7/8 of the CUs (gate-up), and for down when the row
// tiles number at least two per CU, or BT >= 3 with more than
// DFK_ST_DN_WIDE_X2 / 2 tiles per CU (its K split fills the machine).
// The staged down kernel splits K so that (row groups x splits) fills every
// CU's resident workgroups, with no split shorter than this many chunks
#ifndef DFK_ST_DN_MIN_CHUNKS
#define DFK_ST_DN_MIN_CHUNKS 128
#endif
// 16-row tiles per wave in the staged down kernel: two in the 8-wave
// kernels (many row tiles or BT >= 3) up to BT = 4, where they fit in
// registers without spilling (at the Llama-3-70B shape, B = 64: 136 us
// instead of 160 us); one otherwise
#ifndef DFK_ST_DN_TR
#define DFK_ST_DN_TR(W, BT) ((W) >= 8 && (BT) <= 4 ? 2 : 1)
#endif
// Workgroup-cooperative down kernel (ROW traversal, B <= 16): waves per
// workgroup and K chunks per stage
#ifndef DFK_COOP
#define DFK_COOP 1
#endif
#ifndef DFK_COOP_DN_WAVES
#define DFK_COOP_DN_WAVES 8
#endif
#ifndef DFK_COOP_DN_KSC
#define DFK_COOP_DN_KSC 128
#endif

struct KernelInfo {
    const void *fn;
    int rows_per_group;
    int block;
    int waves_per_item;  // 1: wave items (ROW); block/64: workgroup items (COL)
    int nv;              // COL combine floats per lane
};

template <int B, bool NORM> KernelInfo gu_valu_row_t() {
    constexpr int R = DFK_GU_VALU_R(B), U = DFK_GU_VALU_U(B);
    return {(const void *)gate_up_valu_row_kernel<B, R, U, NORM>, R, kValuBlock, 1, 0};
}
template <int B, bool NORM> KernelInfo gu_valu_col_t() {
    constexpr int R = DFK_GU_VALU_R(B), U = DFK_GU_VALU_U(B);
    return {(const void *)gate_up_valu_col_kernel<B, R, U, NORM>, R, kValuBlock, kValuBlock / kWave, 2 * R * B};
}
template <int B> KernelInfo gu_valu_row() { return gu_valu_row_t<B, false>(); }
template <int B> KernelInfo gu_valu_col() { return gu_valu_col_t<B, false>(); }
template <int B> KernelInfo gu_valu_row_norm() { return gu_valu_row_t<B, true>(); }
template <int B> KernelInfo gu_valu_col_norm() { return gu_valu_col_t<B, true>(); }
template <int B, bool HLDS> KernelInfo dn_valu_row_t() {
    constexpr int R = DFK_DN_VALU_R(B), U = DFK_DN_VALU_U(B);
    return {(const void *)down_valu_row_kernel<B, R, U, HLDS>, R, kValuBlock, 1, 0};
}
// rows per workgroup and load groups in flight of the down column walk: one
// row at B = 1, else those of the row walk.  Event-timed down column walk,
// us at B = 1, two rows against one: 8B 21.2 against 19.6 (the row walk:
// 19.7-20.1), 5120 x 13824 24.7 against 22.7, 3072 x 8192 and 2048 x 5632
// within 0.1 us; at B = 2 one row was 1-4 us slower.
#ifndef DFK_DN_VALU_COL_R
#define DFK_DN_VALU_COL_R(B) ((B) == 1 ? 1 : DFK_DN_VALU_R(B))
#endif
#ifndef DFK_DN_VALU_COL_U
#define DFK_DN_VALU_COL_U(B) DFK_DN_VALU_U(B)
#endif
template <int B, bool HLDS> KernelInfo dn_valu_col_t() {
    constexpr int R = DFK_DN_VALU_COL_R(B), U = DFK_DN_VALU_COL_U(B);
    return {(const void *)down_valu_col_kernel<B, R, U, HLDS>, R, kValuBlock, kValuBlock / kWave, R * B};
}
// load groups in flight per lane in the K-panel down walk (B = 4: one, which
// took the 70B shape from 79.0 to 76.3 us and the 8B shape from 24.8 to 24.0 us)
#ifndef DFK_DN_PANEL_VALU_U
#define DFK_DN_PANEL_VALU_U(B) ((B) == 4 ? 1 : 2)
#endif
template <int B> KernelInfo dn_valu_panel() {
    constexpr int R = DFK_DN_VALU_R(B), U = DFK_DN_PANEL_VALU_U(B);
    return {(const void *)down_valu_panel_kernel<B, R, U>, R, kValuBlock, 1, 0};
}
template <int B> KernelInfo dn_valu_row() { return dn_valu_row_t<B, false>(); }
template <int B> KernelInfo dn_valu_row_lds() { return dn_valu_row_t<B, true>(); }
template <int B> KernelInfo dn_valu_col() { return dn_valu_col_t<B, false>(); }
template <int B> KernelInfo dn_valu_col_lds() { return dn_valu_col_t<B, true>(); }

template <int BT> KernelInfo gu_mfma_row() {
    constexpr int TR = DFK_GU_MFMA_TR(BT), U = DFK_GU_MFMA_U(BT);
    return {(const void *)gate_up_mfma_row_kernel<BT, TR, U>, 16 * TR, kMfmaRowBlock, 1, 0};
}
template <int BT> KernelInfo dn_mfma_row() {
    constexpr int TR = DFK_DN_MFMA_TR(BT), U = DFK_DN_MFMA_U(BT);
    return {(const void *)down_mfma_row_kernel<BT, TR, U>, 16 * TR, kMfmaRowBlock, 1, 0};
}
template <int BT> KernelInfo gu_mfma_col() {
    constexpr int TR = DFK_GU_MFMA_TR(BT), U = DFK_GU_MFMA_U(BT), W = DFK_GU_MFMA_WAVES(BT);
    return {(const void *)gate_up_mfma_col_kernel<BT, TR, U, W>, 16 * TR, W * kWave, W, 2 * TR * BT * 4};
}
template <int BT> KernelInfo dn_mfma_col() {
    constexpr int TR = DFK_DN_MFMA_TR(BT), U = DFK_DN_MFMA_U(BT), W = DFK_DN_MFMA_WAVES(BT);
    return {(const void *)down_mfma_col_kernel<BT, TR, U, W>, 16 * TR, W * kWave, W, TR * BT * 4};
}

static long ceil_div(long a, long b) { return (a + b - 1) / b; }


template <int BT> KernelInfo gu_lt_row() {
    constexpr int W = DFK_LT_GU_ROW_WAVES(BT);
    return {(const void *)gate_up_mfma_lt_kernel<BT, 1, W>, 16, W * kWave, 1, 2 * BT * 4};
}
template <int BT> KernelInfo gu_lt_col() {
    constexpr int W = DFK_LT_GU_WAVES(BT), KS = DFK_LT_GU_KSPLIT(BT);
    return {(const void *)gate_up_mfma_lt_kernel<BT, KS, W>, 16, W * kWave, KS, 2 * BT * 4};
}
template <int BT> KernelInfo dn_lt_row() {
    constexpr int W = DFK_LT_DN_WAVES(BT);
    return {(const void *)down_mfma_lt_kernel<BT, 1, W, DFK_LT_DN_KBC>, 16, W * kWave, 1, BT * 4};
}
template <int BT> KernelInfo dn_lt_col() {
    constexpr int W = DFK_LT_DN_WAVES(BT), KS = DFK_LT_DN_KSPLIT(BT);
    return {(const void *)down_mfma_lt_kernel<BT, KS, W, DFK_LT_DN_KBC>, 16, W * kWave, KS, BT * 4};
}

template <int W, int BT> KernelInfo gu_staged_w() {
    constexpr int NB = DFK_ST_GU_NBUF(BT);
    return {(const void *)gate_up_mfma_staged_kernel<BT, W, NB, (W >= 8 ? 2 : 1)>, 16, W * kWave, NB, 0};
}
// rows_per_group: the 16 TR rows one wave owns
template <int W, int BT> KernelInfo dn_staged_w() {
    constexpr int NB = DFK_ST_DN_NBUF(BT), TR = DFK_ST_DN_TR(W, BT);
    return {(const void *)down_mfma_staged_kernel<BT, W, NB, (W >= 8 ? 2 : 1), TR>, 16 * TR, W * kWave, NB, 0};
}
template <int W, int BT> KernelInfo dn_staged_w_f8() {
    constexpr int NB = DFK_ST_DN_NBUF(BT), TR = DFK_ST_DN_TR(W, BT);
    return {(const void *)down_mfma_staged_kernel<BT, W, NB, (W >= 8 ? 2 : 1), TR, true>, 16 * TR, W * kWave, NB, 0};
}
template <int BT> KernelInfo dn_staged4_f8() { return dn_staged_w_f8<4, BT>(); }
template <int BT> KernelInfo dn_staged8_f8() { return dn_staged_w_f8<8, BT>(); }
template <int BT> KernelInfo gu_staged4() { return gu_staged_w<4, BT>(); }
template <int BT> KernelInfo gu_staged8() { return gu_staged_w<8, BT>(); }
template <int BT> KernelInfo dn_staged4() { return dn_staged_w<4, BT>(); }
template <int BT> KernelInfo dn_staged8() { return dn_staged_w<8, BT>(); }

#define DFK_B_TABLE(F) {F<1>(), F<2>(), F<3>(), F<4>(), F<5>(), F<6>(), F<7>(), F<8>()}
#define DFK_BT_TABLE(F)                                                                                 \
    {F<1>(), F<2>(), F<3>(), F<4>(), F<5>(), F<6>(), F<7>(), F<8>(), F<9>(), F<10>(), F<11>(), F<12>(), \
     F<13>(), F<14>(), F<15>(), F<16>()}

constexpr int kMaxBT = 16;  // B <= 256

static const KernelInfo kGuValuRow[kValuMaxBatch] = DFK_B_TABLE(gu_valu_row);
static const KernelInfo kGuValuCol[kValuMaxBatch] = DFK_B_TABLE(gu_valu_col);
static const KernelInfo kGuValuRowNorm[kValuMaxBatch] = DFK_B_TABLE(gu_valu_row_norm);
static const KernelInfo kGuValuColNorm[kValuMaxBatch] = DFK_B_TABLE(gu_valu_col_norm);
static const KernelInfo kDnValuRow[kValuMaxBatch] = DFK_B_TABLE(dn_valu_row);
static const KernelInfo kDnValuRowLds[kValuMaxBatch] = DFK_B_TABLE(dn_valu_row_lds);
static const KernelInfo kDnValuCol[kValuMaxBatch] = DFK_B_TABLE(dn_valu_col);
static const KernelInfo kDnValuColLds[kValuMaxBatch] = DFK_B_TABLE(dn_valu_col_lds);
static const KernelInfo kDnValuPanel[kValuMaxBatch] = DFK_B_TABLE(dn_valu_panel);
static const KernelInfo kGuMfmaRow[kMaxBT] = DFK_BT_TABLE(gu_mfma_row);
static const KernelInfo kDnMfmaRow[kMaxBT] = DFK_BT_TABLE(dn_mfma_row);
static const KernelInfo kGuMfmaCol[kMaxBT] = DFK_BT_TABLE(gu_mfma_col);
static const KernelInfo kDnMfmaCol[kMaxBT] = DFK_BT_TABLE(dn_mfma_col);
constexpr int kLtMaxBT = 8;
static const KernelInfo kGuLtRow[kLtMaxBT] = DFK_B_TABLE(gu_lt_row);
static const KernelInfo kGuLtCol[kLtMaxBT] = DFK_B_TABLE(gu_lt_col);
static const KernelInfo kDnLtRow[kLtMaxBT] = DFK_B_TABLE(dn_lt_row);
static const KernelInfo kDnLtCol[kLtMaxBT] = DFK_B_TABLE(dn_lt_col);

// The LDS-transposed kernels over FP8 weights (codes widened on the way into LDS).
template <int BT> KernelInfo gu_lt_row_f8() {
    constexpr int W = DFK_LT_GU_ROW_WAVES(BT);
    return {(const void *)gate_up_mfma_lt_kernel<BT, 1, W, true>, 16, W * kWave, 1, 2 * BT * 4};
}
template <int BT> KernelInfo gu_lt_col_f8() {
    constexpr int W = DFK_LT_GU_WAVES(BT), KS = DFK_LT_GU_KSPLIT(BT);
    return {(const void *)gate_up_mfma_lt_kernel<BT, KS, W, true>, 16, W * kWave, KS, 2 * BT * 4};
}
// FP8 gate-up column traversal on shapes with fewer than
// DFK_LT_GU_F8_KS2_TILES row tiles per CU: K split two ways, two tiles per
// workgroup.  Event-timed FP8 gate-up, us at B = 4 / 8 / 16, four-way against
// two-way: 8B 25.3 / 26.1 / 29.6 against 24.2 / 24.4 / 27.9; 5120 x 13824 31.4 /
// 38.3 against 29.4 / 36.3 at B = 4 / 16; but 70B (7 tiles per CU) 76.5 / 90.8
// against 94.4 / 104.9 at B = 4 / 16.
#ifndef DFK_LT_GU_F8_KS2_TILES
#define DFK_LT_GU_F8_KS2_TILES 4
#endif
template <int BT> KernelInfo gu_lt_col_f8_k2() {
    constexpr int W = DFK_LT_GU_WAVES(BT);
    return {(const void *)gate_up_mfma_lt_kernel<BT, 2, W, true>, 16, W * kWave, 2, 2 * BT * 4};
}
template <int BT> KernelInfo dn_lt_row_f8() {
    constexpr int W = DFK_LT_DN_WAVES(BT);
    return {(const void *)down_mfma_lt_kernel<BT, 1, W, DFK_LT_DN_KBC, true>, 16, W * kWave, 1, BT * 4};
}
template <int BT> KernelInfo dn_lt_col_f8() {
    constexpr int W = DFK_LT_DN_WAVES(BT), KS = DFK_LT_DN_KSPLIT(BT);
    return {(const void *)down_mfma_lt_kernel<BT, KS, W, DFK_LT_DN_KBC, true>, 16, W * kWave, KS, BT * 4};
}
static const KernelInfo kGuLtRowF8[kLtMaxBT] = DFK_B_TABLE(gu_lt_row_f8);
static const KernelInfo kGuLtColF8[kLtMaxBT] = DFK_B_TABLE(gu_lt_col_f8);
static const KernelInfo kGuLtColF8K2[kLtMaxBT] = DFK_B_TABLE(gu_lt_col_f8_k2);
static const KernelInfo kDnLtRowF8[kLtMaxBT] = DFK_B_TABLE(dn_lt_row_f8);
static const KernelInfo kDnLtColF8[kLtMaxBT] = DFK_B_TABLE(dn_lt_col_f8);
constexpr int kStMaxBT = 8;
// (waves_per_item holds the staged kernels' LDS buffer count)
static const KernelInfo kGuStaged4[kStMaxBT] = DFK_B_TABLE(gu_staged4);
static const KernelInfo kGuStaged8[kStMaxBT] = DFK_B_TABLE(gu_staged8);
static const KernelInfo kDnStaged4[kStMaxBT] = DFK_B_TABLE(dn_staged4);
static const KernelInfo kDnStaged8[kStMaxBT] = DFK_B_TABLE(dn_staged8);
static const KernelInfo kDnStaged4F8[kStMaxBT] = DFK_B_TABLE(dn_staged4_f8);
static const KernelInfo kDnStaged8F8[kStMaxBT] = DFK_B_TABLE(dn_staged8_f8);

// FP8 row kernels: rows per work item (R) and 16-byte weight loads per lane
// and row in one load group (U).
#ifndef DFK_F8_GU_R
#define DFK_F8_GU_R(B) 1
#endif
#ifndef DFK_F8_GU_U
#define DFK_F8_GU_U(B) ((B) <= 2 ? 4 : 2)
#endif
#ifndef DFK_F8_DN_R
#define DFK_F8_DN_R(B) ((B) <= 2 ? 2 : 4)
#endif
#ifndef DFK_F8_DN_U
#define DFK_F8_DN_U(B) ((B) <= 4 ? 2 : 1)
#endif
template <int B> KernelInfo gu_f8_row() {
    constexpr int R = DFK_F8_GU_R(B), U = DFK_F8_GU_U(B);
    return {(const void *)gate_up_fp8_row_kernel<B, R, U>, R, kValuBlock, 1, 0};
}
template <int B> KernelInfo dn_f8_row() {
    constexpr int R = DFK_F8_DN_R(B), U = DFK_F8_DN_U(B);
    return {(const void *)down_fp8_row_kernel<B, R, U>, R, kValuBlock, 1, 0};
}
static const KernelInfo kGuF8Row[kF8MaxBatch] = DFK_B_TABLE(gu_f8_row);
static const KernelInfo kDnF8Row[kF8MaxBatch] = DFK_B_TABLE(dn_f8_row);

// The persistent MLP kernel per batch: its gate-up and down row counts per
// work item.
#ifndef DFK_MLP_DN_R
#define DFK_MLP_DN_R(B) DFK_DN_VALU_R(B)
#endif
#ifndef DFK_MLP_DN_U
#define DFK_MLP_DN_U(B) DFK_DN_VALU_U(B)
#endif
struct MlpKernel {
    const void *fn;
    int rg, rd;
};
template <int B> MlpKernel mlp_persistent() {
    constexpr int RG = DFK_GU_VALU_R(B), UG = DFK_GU_VALU_U(B), RD = DFK_MLP_DN_R(B), UD = DFK_MLP_DN_U(B);
    return {(const void *)mlp_valu_row_persistent_kernel<B, RG, UG, RD, UD>, RG, RD};
}
static const MlpKernel kMlpPersistent[kMlpMaxBatch] = {mlp_persistent<1>(), mlp_persistent<2>(),
                                                       mlp_persistent<3>(), mlp_persistent<4>()};

// Blocks of a kernel that fit on one CU (cached per kernel, block and LDS).
static int blocks_per_cu(const void *fn, int block, size_t lds) {
    static std::mutex mu;
    struct Entry { const void *fn; int block; size_t lds; int n; };
    static Entry cache[512];
    static int ncache = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ncache; ++i)
        if (cache[i].fn == fn && cache[i].block == block && cache[i].lds == lds) return cache[i].n;
    // allow the kernel all the dynamic LDS a gfx950 CU has (the default cap is lower)
    if (lds > 0) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, block, lds) != hipSuccess || n < 1) n = 1;
    (void)hipGetLastError();
    if (ncache < 512) cache[ncache++] = Entry{fn, block, lds, n};
    return n;
}

// Workgroups of 8 waves for the B-operand-staged kernels (see the tile
// parameters above).
static bool staged_wide(bool gu, int BT, long tiles, int cus) {
    return gu ? ceil_div(tiles, 8L) * 8 >= 7L * cus
              : ((BT >= 3 && 2 * tiles > (long)DFK_ST_DN_WIDE_X2 * cus) || tiles >= 2L * cus);
}

// The LDS-transposed staged-h down kernel: instances for (BT, waves, tiles
// per wave); two tiles per wave up to two batch tiles only (beyond, the two
// tiles' weights and fragments do not fit in registers without spilling)
// K block (bf16 chunks) and h buffers: 128-element blocks at four batch tiles
// (bf16) when DFK_DN_LTSW_KBC_BT4 says so, two buffers where they fit next to
// the tiles
constexpr int ltsw_kbc(int BT, bool f8, int W) {
    return f8 ? 32 : BT == 4 ? DFK_DN_LTSW_KBC_BT4 : BT == 2 ? DFK_DN_LTSW_KBC_BT2
                   : (BT == 1 && W < 8) ? DFK_DN_LTSW_KBC_BT1 : 32;
}
constexpr int ltsw_nbuf(int BT, bool f8, int W) {
    return !f8 && (BT <= 2 || ltsw_kbc(BT, f8, W) == 16) ? DFK_DN_LTSW_NBUF_BT12 : 1;
}
template <int BT, int W, int TR, bool F8> const void *ltsw_fn() {
    return (const void *)down_mfma_ltsw_kernel<BT, W, TR, (W >= 8 ? 2 : 1), F8, ltsw_nbuf(BT, F8, W),
                                               ltsw_kbc(BT, F8, W)>;
}
template <bool F8> const void *ltsw_pick(int BT, int W, int TR) {
    static_assert(DFK_DN_LTSW_MAX_BT <= 4, "instantiated for BT <= 4");
    static const void *const w8[2][4] = {
        {ltsw_fn<1, 8, 1, F8>(), ltsw_fn<2, 8, 1, F8>(), ltsw_fn<3, 8, 1, F8>(), ltsw_fn<4, 8, 1, F8>()},
        {ltsw_fn<1, 8, 2, F8>(), ltsw_fn<2, 8, 2, F8>(), nullptr,
         ltsw_kbc(4, F8, 8) == 16 ? ltsw_fn<4, 8, 2, F8>() : nullptr}};
    static const void *const w4[4] = {ltsw_fn<1, 4, 1, F8>(), ltsw_fn<2, 4, 1, F8>(), ltsw_fn<3, 4, 1, F8>(),
                                      ltsw_fn<4, 4, 1, F8>()};
    static const void *const w4tr2 = ltsw_kbc(1, F8, 4) == 16 ? ltsw_fn<1, 4, 2, F8>() : nullptr;
    return W >= 8 ? w8[TR > 1 ? 1 : 0][BT - 1] : (TR > 1 && BT == 1) ? w4tr2 : w4[BT - 1];
}

// K split count for row_groups work-item rows over `slots` resident
// workgroups: the S that minimizes the modelled HBM time, bytes streamed by
// the busiest slots (rounds x slots x (split + a two-block ramp) of weights
// per item) plus the split sums written and read back by the reduce.
static long pick_splits(long row_groups, long rows_per_item, long C, long slots, long min_chunks, long B,
                        long M) {
    const long max_s = std::max(1L, C / min_chunks);
    long best = 1;
    double best_cost = 0.0;
    for (long s = 1; s <= max_s; ++s) {
        long cs = ceil_div(C, s);
        if (C >= 32) cs = ceil_div(cs, 32L) * 32;
        const long S = ceil_div(C, cs);
        const long rounds = ceil_div(row_groups * S, slots);
        const double cost = (double)rounds * slots * rows_per_item * (cs + 64) * 16.0 +
                            (S > 1 ? 8.0 * S * B * M : 0.0);
        if (s == 1 || cost < best_cost) {
            best_cost = cost;
            best = S;
        }
    }
    return best;
}

// Fill the launch shape of down_mfma_ltsw_kernel (q holds the op, B, rows and
// K): the waves and row tiles per wave of the DFK_DN_LTSW_* rules, one
// workgroup per resident slot, and the K split of pick_splits (a multiple of
// the 32-chunk block).
static bool plan_ltsw(bool f8, int BT, int C, int cus, Plan *q) {
    const long tiles = ceil_div((long)q->rows, 16L);
    if (BT == 3 && DFK_DN_LTSW_BT3_AS_BT4 && ltsw_kbc(4, f8, 8) == 16 && tiles >= cus) BT = 4;  // padded batch tile
    const int W = ((BT <= 2 && 100 * tiles < (long)DFK_DN_LTSW_NARROW_PCT * cus) || (BT == 1 && ltsw_kbc(1, f8, 4) == 16))
                      ? 4 : DFK_DN_LTSW_WAVES;
    const bool k16 = ltsw_kbc(BT, f8, W) == 16;
    const int tr = (W >= 8 && BT <= 2 && !k16 && tiles >= (long)DFK_DN_LTSW_TR2_X * cus) ? DFK_DN_LTSW_TR
                   : ((W >= 8 || BT == 1) && k16 && 4 * tiles >= (long)DFK_DN_LTSW_BT4_TR2_Q * cus) ? 2
                   : 1;
    const void *fn = f8 ? ltsw_pick<true>(BT, W, tr) : ltsw_pick<false>(BT, W, tr);
    if (!fn) return false;
    q->kind = KIND_DN_MFMA_STAGED;
    q->block = W * kWave;
    const int kbc = ltsw_kbc(BT, f8, W);
    q->lds_bytes = (size_t)ltsw_nbuf(BT, f8, W) * 2 * 16 * BT * (kbc + 1) * 16 +
                   (size_t)W * 16 * (kbc + 1) * 16;
    if (q->lds_bytes > kLdsLimit) return false;
    q->rows_per_group = 16;
    q->groups = (int)tiles;
    const long occ = blocks_per_cu(fn, q->block, q->lds_bytes);
    const long row_groups = ceil_div(tiles, (long)W * tr);
    const long target = (long)cus * occ;
    const long S = pick_splits(row_groups, 16L * W * tr, C, target, DFK_DN_LTSW_MIN_CHUNKS, q->B, q->rows);
    long cs = ceil_div((long)C, S);
    if (C >= 32) cs = ceil_div(cs, 32L) * 32;
    q->splits = (int)ceil_div((long)C, cs);
    q->chunks_per_split = (int)cs;
    q->partial_floats = q->splits > 1 ? (size_t)q->splits * q->B * q->rows : 0;
    q->grid = (int)std::max(1L, std::min(target, row_groups * q->splits));
    q->fn = fn;
    return true;
}

// Fill the launch shape of a B-operand-staged kernel (q holds the op, B,
// rows and K): LDS per workgroup, a grid that fills every CU's resident
// workgroups, and for down the K splits (none shorter than
// DFK_ST_DN_MIN_CHUNKS chunks, a multiple of the 32-chunk block).
static bool plan_staged(bool gu, int B, int BT, int C, int cus, const KernelInfo &ki, Plan *q) {
    const int waves = ki.block / kWave;
    q->lds_bytes = (size_t)ki.waves_per_item * (gu ? 1 : 2) * 16 * BT * kStPitch * 16;
    if (q->lds_bytes > kLdsLimit) return false;
    q->kind = gu ? KIND_GU_MFMA_STAGED : KIND_DN_MFMA_STAGED;
    q->block = ki.block;
    q->rows_per_group = 16;
    q->groups = (int)ceil_div(q->rows, 16);
    const long occ = blocks_per_cu(ki.fn, q->block, q->lds_bytes);
    const long row_groups = ceil_div((long)q->groups, (long)waves * (ki.rows_per_group / 16));
    const long target = (long)cus * occ;
    long S = 1;
    if (!gu) {
        long max_s = std::max(1L, (long)C / DFK_ST_DN_MIN_CHUNKS);
        if (row_groups * max_s < cus) max_s = std::max(1L, (long)C / DFK_ST_DN_SMALL_MIN_CHUNKS);
        S = std::min(max_s, std::max(1L, ceil_div(target, row_groups)));
        long cs = ceil_div((long)C, S);
        if (C >= kStKbc) cs = ceil_div(cs, (long)kStKbc) * kStKbc;
        S = ceil_div((long)C, cs);
        q->chunks_per_split = (int)cs;
    }
    q->splits = (int)S;
    q->partial_floats = S > 1 ? (size_t)S * B * q->rows : 0;
    q->grid = (int)std::max(1L, std::min(target, row_groups * S));
    q->fn = ki.fn;
    return true;
}



// Down with h held in registers (COL traversal, vector ALU): instances for
// J chunks per lane and batch B where the J * 8 * B h registers stay within
// DFK_DN_HREG_VGPRS; R rows per group.  The plan takes the first waves-per-
// workgroup count (DFK_DN_HREG_WAVES, then 16, 8, 4) whose slice gives an
// instantiated J.
#ifndef DFK_DN_HREG
#define DFK_DN_HREG 1
#endif
#ifndef DFK_DN_HREG_VGPRS
#define DFK_DN_HREG_VGPRS 64
#endif
// rows per group: two where a lane holds at most two chunks of h per batch
// row (Llama-3-8B down at B = 3 / 4, 16-wave workgroups: 22.9 / 24.1 ->
// 21.2 / 22.3 us), else one (two at four chunks: B = 1 20.2 -> 22.5 us)
#ifndef DFK_DN_HREG_R
#define DFK_DN_HREG_R(J) ((J) <= 2 ? 2 : 1)
#endif
#ifndef DFK_DN_HREG_WAVES
#define DFK_DN_HREG_WAVES 8
#endif
// from this batch up, and at B = 1 on W_down of at most DFK_DN_HREG_B1_MAX
// elements (at B = 1 the column walk with h in LDS is faster on the larger
// shapes, kernel durations at 4096 x 14336 19.7 against 20.4 us and at
// 5120 x 13824 22.8 against 23.8 us; slower on the smaller ones, 3072 x 8192
// 10.9 against 10.6 us and 2048 x 5632 6.9 against 6.6 us)
#ifndef DFK_DN_HREG_MIN_B
#define DFK_DN_HREG_MIN_B 2
#endif
#ifndef DFK_DN_HREG_B1_MAX
#define DFK_DN_HREG_B1_MAX (3072L * 8192L)
#endif
constexpr int kHregMaxJ = 8;
// FP8 codes: 16 h values per chunk and batch row, so J * 16 * B registers,
// and two rows per group at one chunk per lane
#ifndef DFK_DN_HREG_F8_R
#define DFK_DN_HREG_F8_R(J) ((J) <= 1 ? 2 : 1)
#endif
template <int B, int J> const void *hreg_inst() {
    if constexpr (J * 8 * B <= DFK_DN_HREG_VGPRS) return (const void *)down_valu_hreg_kernel<B, J, DFK_DN_HREG_R(J)>;
    else return nullptr;
}
template <int B, int J> const void *hreg_inst_f8() {
    if constexpr (J * 16 * B <= DFK_DN_HREG_VGPRS)
        return (const void *)down_valu_hreg_kernel<B, J, DFK_DN_HREG_F8_R(J), true>;
    else return nullptr;
}
#define DFK_HREG_ROW(F, B) \
    {F<B, 1>(), F<B, 2>(), F<B, 3>(), F<B, 4>(), F<B, 5>(), F<B, 6>(), F<B, 7>(), F<B, 8>()}
static const void *const kDnHreg[kValuMaxBatch][kHregMaxJ] = {
    DFK_HREG_ROW(hreg_inst, 1), DFK_HREG_ROW(hreg_inst, 2), DFK_HREG_ROW(hreg_inst, 3), DFK_HREG_ROW(hreg_inst, 4),
    DFK_HREG_ROW(hreg_inst, 5), DFK_HREG_ROW(hreg_inst, 6), DFK_HREG_ROW(hreg_inst, 7), DFK_HREG_ROW(hreg_inst, 8)};
static const void *const kDnHregF8[4][kHregMaxJ] = {
    DFK_HREG_ROW(hreg_inst_f8, 1), DFK_HREG_ROW(hreg_inst_f8, 2), DFK_HREG_ROW(hreg_inst_f8, 3),
    DFK_HREG_ROW(hreg_inst_f8, 4)};
#undef DFK_HREG_ROW

// C: 16-byte chunks per W_down row (K / 8 bf16, K / 16 FP8 codes)
static bool plan_hreg(int B, int C, int M, int cus, Plan *q, bool f8 = false) {
    if (!DFK_DN_HREG || B < 1 || B > (f8 ? 4 : kValuMaxBatch) || C < 1) return false;
    if (!f8 && B < DFK_DN_HREG_MIN_B && (long)M * C * 8 > DFK_DN_HREG_B1_MAX) return false;
    const int order[4] = {DFK_DN_HREG_WAVES, 16, 8, 4};
    for (int w : order) {
        if (w < 1 || w > kHregMaxWaves) continue;
        const long J = ceil_div(ceil_div((long)C, (long)w), (long)kWave);
        if (J > kHregMaxJ) continue;
        const void *fn = (f8 ? kDnHregF8 : kDnHreg)[B - 1][J - 1];
        if (!fn || w > hreg_max_waves((int)J)) continue;
        q->kind = KIND_DN_VALU_HREG;
        q->block = w * kWave;
        q->lds_bytes = 0;
        q->rows_per_group = f8 ? DFK_DN_HREG_F8_R((int)J) : DFK_DN_HREG_R((int)J);
        q->groups = (int)ceil_div((long)M, (long)q->rows_per_group);
        const long slots = (long)cus * blocks_per_cu(fn, q->block, 0);
        // balanced: every workgroup walks the same number of row groups
        const long per_wg = ceil_div((long)q->groups, slots);
        q->grid = (int)std::max(1L, ceil_div((long)q->groups, per_wg));
        q->fn = fn;
        return true;
    }
    return false;
}

bool make_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus, Plan *out,
               bool norm) {
    if (B < 1 || d_model < 8 || d_ff < 8 || (d_model % 8) || (d_ff % 8) || cus < 1) return false;
    Plan q{};
    q.op = op;
    q.engine = engine;
    q.trav = trav;
    q.B = B;
    q.rows = (op == OP_GATE_UP) ? d_ff : d_model;
    q.K = (op == OP_GATE_UP) ? d_model : d_ff;
    const bool gu = (op == OP_GATE_UP);
    const bool row = (trav == TRAV_ROW);
    q.splits = 1;
    q.chunks_per_split = q.K / 8;
    KernelInfo ki{};
    if (engine == ENGINE_VALU) {
        if (B > kValuMaxBatch) return false;
        if (gu) {
            // x stays whole in LDS (+ the col combine buffer, + the norm's
            // per-wave sums of squares)
            if (norm) ki = row ? kGuValuRowNorm[B - 1] : kGuValuColNorm[B - 1];
            else ki = row ? kGuValuRow[B - 1] : kGuValuCol[B - 1];
            q.lds_bytes = (size_t)B * d_model * 2 + (size_t)(ki.block / kWave) * ki.nv * sizeof(float) +
                          (norm ? (size_t)B * (ki.block / kWave) * sizeof(double) : 0);
            if (q.lds_bytes > kLdsLimit) return false;
            q.fused_norm = norm;
            q.kind = row ? KIND_GU_VALU_ROW : KIND_GU_VALU_COL;
        } else if (!row && plan_hreg(B, q.K / 8, q.rows, cus, &q)) {
            // h in registers, row groups walked with the next group's loads in flight
            *out = q;
            return true;
        } else if (row && (size_t)B * q.K * 4 > DFK_HLDS_LIMIT) {
            // h does not fit in LDS whole: cut K into the fewest panels whose h
            // slice does (32 bytes per weight chunk and batch row), partial
            // sums added by the reduce kernel
            const long C = q.K / 8;
            const long max_cs = std::max(1L, (long)(DFK_HLDS_LIMIT / ((size_t)B * 32)));
            const long cs = ceil_div(C, ceil_div(C, max_cs));
            const KernelInfo pk = kDnValuPanel[B - 1];
            q.kind = KIND_DN_VALU_PANEL;
            q.splits = (int)ceil_div(C, cs);
            q.chunks_per_split = (int)cs;
            q.partial_floats = (size_t)q.splits * B * q.rows;
            q.h_in_lds = true;
            q.lds_bytes = (size_t)B * cs * 32;
            q.block = pk.block;
            q.rows_per_group = pk.rows_per_group;
            q.groups = (int)ceil_div(q.rows, pk.rows_per_group);
            const long waves = std::max(1L, (long)cus * blocks_per_cu(pk.fn, q.block, q.lds_bytes) *
                                                (q.block / kWave) / q.splits);
            const long per_wave = ceil_div((long)q.groups, waves);
            q.grid = (int)std::max(1L, ceil_div(ceil_div((long)q.groups, per_wave), q.block / kWave));
            q.fn = pk.fn;
            *out = q;
            return true;
        } else {
            // keep all of h in LDS when it is small, else read it through the caches
            const size_t whole = (size_t)B * q.K * 4;
            const bool hlds = whole <= DFK_HLDS_LIMIT;
            if (row) ki = hlds ? kDnValuRowLds[B - 1] : kDnValuRow[B - 1];
            else ki = hlds ? kDnValuColLds[B - 1] : kDnValuCol[B - 1];
            q.lds_bytes = (hlds ? whole : 0) + (size_t)(ki.block / kWave) * ki.nv * sizeof(float);
            q.kind = row ? KIND_DN_VALU_ROW : KIND_DN_VALU_COL;
            q.h_in_lds = hlds;
        }
    } else {
        const int BT = (int)ceil_div(B, 16);
        if (BT > kMaxBT) return false;
        const int C = q.K / 8;
        constexpr int dw = DFK_COOP_DN_WAVES, dk = DFK_COOP_DN_KSC;
        const size_t coop_lds = (size_t)2 * Coop<dw, dk>::TILE * 16;
        if (DFK_COOP && BT == 1 && !gu && row && C >= dk && coop_lds <= kLdsLimit) {
            // down ROW: workgroup-cooperative 16-row tile over all of K (K must
            // span at least one stage)
            const void *fn = (const void *)down_mfma_coop_kernel<dw, dk>;
            q.kind = KIND_DN_MFMA_COOP;
            q.block = dw * kWave;
            q.lds_bytes = coop_lds;
            q.rows_per_group = 16;
            q.groups = (int)ceil_div(q.rows, 16);
            const long slots = (long)cus * blocks_per_cu(fn, q.block, q.lds_bytes);
            const long per_wg = ceil_div((long)q.groups, slots);  // tiles per workgroup, balanced
            q.grid = (int)std::max(1L, ceil_div((long)q.groups, per_wg));
            q.fn = fn;
            *out = q;
            return true;
        }
        if (!gu && !row && BT == 1 && DFK_DN_LTSW_MIN_BT > 1) {
            // LDS-transposed weights with h staged in LDS per workgroup
            constexpr int W = DFK_DN_LTS_WAVES, WW = DFK_DN_LTS_WIDE_WAVES;
            q.groups = (int)ceil_div(q.rows, 16);
            const bool wide = B > 8 && q.groups >= 2L * cus;
            const int w = wide ? WW : W;
            const void *fn = wide ? (const void *)down_mfma_lts_kernel<1, WW> : (const void *)down_mfma_lts_kernel<1, W>;
            q.kind = KIND_DN_MFMA_STAGED;
            q.block = w * kWave;
            q.lds_bytes = (size_t)2 * 16 * BT * kStPitch * 16 + (size_t)w * Lt<32>::kTile * 16;
            if (q.lds_bytes > kLdsLimit) return false;
            q.rows_per_group = 16;
            const long occ = blocks_per_cu(fn, q.block, q.lds_bytes);
            const long row_groups = ceil_div((long)q.groups, (long)w);
            const long target = (long)cus * occ;
            const long max_s = std::max(1L, (long)C / DFK_DN_LTS_MIN_CHUNKS);
            long S = std::min(max_s, std::max(1L, ceil_div(target, row_groups)));
            long cs = ceil_div((long)C, S);
            if (C >= 32) cs = ceil_div(cs, 32L) * 32;
            S = ceil_div((long)C, cs);
            q.splits = (int)S;
            q.chunks_per_split = (int)cs;
            q.partial_floats = S > 1 ? (size_t)S * B * q.rows : 0;
            q.grid = (int)std::max(1L, std::min(target, row_groups * S));
            q.fn = fn;
            *out = q;
            return true;
        }
        if (gu && row && BT >= DFK_GU_LTS_MIN_BT && BT <= DFK_GU_LTS_MAX_BT &&
            (BT > 1 || 10 * ceil_div(q.rows, 16) < (long)DFK_GU_LTS_BT1_TILES_X10 * cus)) {
            // LDS-transposed weights, x staged in LDS per workgroup
            constexpr int W = DFK_GU_LTS_WAVES, WN = DFK_GU_LTS_NARROW_WAVES;
            constexpr int NB3 = DFK_GU_LTS_NBUF_BT3;
            static const void *const lts[2][4] = {
                {DFK_GU_LTS_MIN_BT <= 1 ? (const void *)gate_up_mfma_lts_kernel<1, W> : nullptr,
                 (const void *)gate_up_mfma_lts_kernel<2, W, false, DFK_GU_LTS_NBUF_BT2>,
                 (const void *)gate_up_mfma_lts_kernel<3, W, false, NB3>,
                 (const void *)gate_up_mfma_lts_kernel<4, W, false, DFK_GU_LTS_NBUF_BT4>},
                {DFK_GU_LTS_MIN_BT <= 1 ? (const void *)gate_up_mfma_lts_kernel<1, WN> : nullptr,
                 (const void *)gate_up_mfma_lts_kernel<2, WN>, (const void *)gate_up_mfma_lts_kernel<3, WN>,
                 (const void *)gate_up_mfma_lts_kernel<4, WN>}};
            static_assert(DFK_GU_LTS_MAX_BT <= 4, "instantiated for BT <= 4");
            q.groups = (int)ceil_div(q.rows, 16);
            if (BT >= DFK_GU_LTS_K16_MIN_BT && (BT > 3 || q.groups < (long)DFK_GU_LTS_K16_BT3_MAX_X * cus)) {
                // 128-element blocks, x double-buffered
                static const void *const lts16[2][2] = {
                    {(const void *)gate_up_mfma_lts_kernel<3, 2, false, 2, 16>,
                     (const void *)gate_up_mfma_lts_kernel<4, 2, false, 2, 16>},
                    {(const void *)gate_up_mfma_lts_kernel<3, 4, false, 2, 16>,
                     (const void *)gate_up_mfma_lts_kernel<4, 4, false, 2, 16>}};
                static_assert(DFK_GU_LTS_K16_MIN_BT >= 3, "instantiated for BT 3 and 4");
                const int w = q.groups >= (long)DFK_GU_LTS_K16_W4_X * cus ? 4 : 2;
                q.kind = KIND_GU_MFMA_LT;
                q.block = w * kWave;
                q.lds_bytes = (size_t)2 * 16 * BT * 17 * 16 + (size_t)w * 2 * Lt<16>::kTile * 16;
                q.rows_per_group = 16;
                q.fn = lts16[w == 4 ? 1 : 0][BT - 3];
                const long occ = blocks_per_cu(q.fn, q.block, q.lds_bytes);
                q.grid = (int)std::max(1L, std::min((long)cus * occ, ceil_div((long)q.groups, (long)w)));
                *out = q;
                return true;
            }
            const bool narrow = 2L * q.groups < (long)(BT == 2 ? DFK_GU_LTS_NARROW_X2_BT2 : DFK_GU_LTS_NARROW_X2) * cus;
            const int w = narrow ? WN : W;
            q.kind = KIND_GU_MFMA_LT;
            q.block = w * kWave;
            const int nbuf = narrow ? 1 : BT == 2 ? DFK_GU_LTS_NBUF_BT2 : BT == 3 ? NB3 : BT == 4 ? DFK_GU_LTS_NBUF_BT4 : 1;
            q.lds_bytes = (size_t)nbuf * 16 * BT * kStPitch * 16 + (size_t)w * 2 * Lt<32>::kTile * 16;
            if (q.lds_bytes > kLdsLimit) return false;
            q.rows_per_group = 16;
            q.fn = lts[narrow ? 1 : 0][BT - 1];
            const long occ = blocks_per_cu(q.fn, q.block, q.lds_bytes);
            q.grid = (int)std::max(1L, std::min((long)cus * occ, ceil_div((long)q.groups, (long)w)));
            *out = q;
            return true;
        }
        if (!gu && !row && BT >= DFK_DN_LTSW_MIN_BT && BT <= DFK_DN_LTSW_MAX_BT) {
            // LDS-transposed weights, h staged in LDS, several row tiles per wave
            if (!plan_ltsw(false, BT, C, cus, &q)) return false;
            *out = q;
            return true;
        }
        if (BT >= (gu ? DFK_ST_GU_MIN_BT : DFK_ST_DN_MIN_BT) && BT <= kStMaxBT && (gu ? row : !row)) {
            // B operand staged in LDS per workgroup: gate-up ROW, down COL
            const long tiles = ceil_div(q.rows, 16);
            ki = gu ? (staged_wide(true, BT, tiles, cus) ? kGuStaged8 : kGuStaged4)[BT - 1]
                    : (staged_wide(false, BT, tiles, cus) ? kDnStaged8 : kDnStaged4)[BT - 1];
            if (!plan_staged(gu, B, BT, C, cus, ki, &q)) return false;
            *out = q;
            return true;
        }
        if (DFK_MFMA_LT && BT <= kLtMaxBT) {
            // LDS-transposed weight stream; waves_per_item = the K split
            if (row) ki = gu ? kGuLtRow[BT - 1] : kDnLtRow[BT - 1];
            else ki = gu ? kGuLtCol[BT - 1] : kDnLtCol[BT - 1];
            const int waves = ki.block / kWave;
            q.lds_bytes = (size_t)waves * (gu ? 2 * Lt<32>::kTile : Lt<DFK_LT_DN_KBC>::kTile) * 16 +
                          (ki.waves_per_item > 1 ? (size_t)waves * ki.nv * kWave * sizeof(float) : 0);
            if (q.lds_bytes > kLdsLimit) return false;
            q.kind = gu ? KIND_GU_MFMA_LT : KIND_DN_MFMA_LT;
            q.block = ki.block;
            q.rows_per_group = 16;
            q.groups = (int)ceil_div(q.rows, 16);
            const int occ = blocks_per_cu(ki.fn, q.block, q.lds_bytes);
            const long tiles_per_wg = waves / ki.waves_per_item;
            const long wg_items = ceil_div(q.groups, tiles_per_wg);
            q.grid = (int)std::max(1L, DFK_GRID_MODE ? wg_items : std::min((long)cus * occ, wg_items));
            q.fn = ki.fn;
            *out = q;
            return true;
        }
        if (row) ki = gu ? kGuMfmaRow[BT - 1] : kDnMfmaRow[BT - 1];
        else ki = gu ? kGuMfmaCol[BT - 1] : kDnMfmaCol[BT - 1];
        q.lds_bytes = row ? 0 : (size_t)(ki.waves_per_item - 1) * ki.nv * kWave * sizeof(float);
        q.kind = gu ? (row ? KIND_GU_MFMA_ROW : KIND_GU_MFMA_COL) : (row ? KIND_DN_MFMA_ROW : KIND_DN_MFMA_COL);
    }
    q.block = ki.block;
    q.rows_per_group = ki.rows_per_group;
    q.groups = (int)ceil_div(q.rows, ki.rows_per_group);
    const int occ = blocks_per_cu(ki.fn, q.block, q.lds_bytes);
    const long items_per_block = (ki.block / kWave) / ki.waves_per_item;
    const long all_items = ceil_div(q.groups, items_per_block);
    q.grid = (int)std::max(1L, DFK_GRID_MODE ? all_items : std::min((long)cus * occ, all_items));
    if (DFK_BALANCE && !DFK_GRID_MODE) {
        // persistent grid sized so that every work item slot gets the same
        // number of items: no last round run by a fraction of the waves
        const long slots = (long)q.grid * items_per_block;
        const long per_slot = ceil_div((long)q.groups, slots);
        q.grid = (int)std::max(1L, ceil_div(ceil_div((long)q.groups, per_slot), items_per_block));
    }
    q.fn = ki.fn;
    *out = q;
    return true;
}

bool make_mlp_plan(int B, int d_model, int d_ff, int cus, MlpPlan *out) {
    if (B < 1 || B > kMlpMaxBatch || d_model < 8 || d_ff < 8 || (d_model % 8) || (d_ff % 8) || cus < 1) return false;
    const size_t x_bytes = (size_t)B * d_model * 2, h_bytes = (size_t)B * d_ff * 4;
    if (h_bytes > kHLdsLimit || x_bytes > kLdsLimit) return false;
    const MlpKernel &mk = kMlpPersistent[B - 1];
    MlpPlan q{};
    q.B = B;
    q.d_model = d_model;
    q.d_ff = d_ff;
    q.fn = mk.fn;
    q.block = kValuBlock;
    q.lds_bytes = std::max(x_bytes, h_bytes);
    q.gu_groups = (int)ceil_div(d_ff, mk.rg);
    q.dn_groups = (int)ceil_div(d_model, mk.rd);
    // every workgroup resident (a cooperative launch), no more than the work
    const long slots = (long)cus * blocks_per_cu(q.fn, q.block, q.lds_bytes);
    const long need = ceil_div(std::max(q.gu_groups, q.dn_groups), kValuBlock / kWave);
    q.grid = (int)std::max(1L, std::min(slots, need));
    *out = q;
    return true;
}

hipError_t launch_mlp(const MlpPlan &p, const uint16_t *x, const uint16_t *w_gate, const uint16_t *w_up,
                      const uint16_t *w_down, float *h, uint16_t *y, unsigned *barrier, hipStream_t stream) {
    if (!barrier) return hipErrorInvalidValue;
    GateUpArgs ga{};
    ga.x = x; ga.wg = w_gate; ga.wu = w_up; ga.h = h;
    ga.B = p.B; ga.K = p.d_model; ga.N = p.d_ff; ga.C = p.d_model / 8; ga.groups = p.gu_groups; ga.ldw = p.d_model;
    DownArgs da{};
    da.h = h; da.wd = w_down; da.y = y;
    da.B = p.B; da.K = p.d_ff; da.M = p.d_model; da.C = p.d_ff / 8; da.groups = p.dn_groups;
    GridBarrier bar{barrier};
    void *argv[] = {&ga, &da, &bar};
    return hipLaunchCooperativeKernel(p.fn, dim3(p.grid), dim3(p.block), argv, (unsigned)p.lds_bytes, stream);
}

bool make_fp8_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus, Plan *out) {
    if (B < 1 || d_model < 16 || d_ff < 16 || (d_model % 16) || (d_ff % 16) || cus < 1) return false;
    const bool gu = (op == OP_GATE_UP);
    if (engine == ENGINE_VALU && trav == TRAV_COL) {
        // down only: the column walk with h held in registers
        if (gu) return false;
        Plan q{};
        q.op = op;
        q.engine = engine;
        q.trav = trav;
        q.B = B;
        q.rows = d_model;
        q.K = d_ff;
        q.splits = 1;
        q.chunks_per_split = q.K / 16;
        if (!plan_hreg(B, d_ff / 16, d_model, cus, &q, true)) return false;
        *out = q;
        return true;
    }
    if (engine == ENGINE_MFMA) {
        // the LDS-transposed matrix-core kernels, FP8 codes widened into LDS
        const int BT = (int)ceil_div(B, 16);
        if (BT > kLtMaxBT) return false;
        const bool row = (trav == TRAV_ROW);
        if (!gu && !row && BT >= DFK_DN_LTSW_F8_MIN_BT && BT <= DFK_DN_LTSW_F8_MAX_BT) {
            Plan q{};
            q.op = op;
            q.engine = ENGINE_MFMA;
            q.trav = trav;
            q.B = B;
            q.rows = d_model;
            q.K = d_ff;
            q.chunks_per_split = q.K / 8;
            if (!plan_ltsw(true, BT, d_ff / 8, cus, &q)) return false;
            *out = q;
            return true;
        }
        if (!gu && !row && BT >= DFK_ST_DN_F8_MIN_BT && BT <= kStMaxBT) {
            // h staged in LDS per workgroup, codes loaded as A fragments (as
            // for bf16 weights)
            Plan q{};
            q.op = op;
            q.engine = ENGINE_MFMA;
            q.trav = trav;
            q.B = B;
            q.rows = d_model;
            q.K = d_ff;
            q.chunks_per_split = q.K / 8;
            const long tiles = ceil_div((long)d_model, 16L);
            const KernelInfo ki = (staged_wide(false, BT, tiles, cus) ? kDnStaged8F8 : kDnStaged4F8)[BT - 1];
            if (!plan_staged(false, B, BT, d_ff / 8, cus, ki, &q)) return false;
            *out = q;
            return true;
        }
        if (gu && row && BT >= DFK_GU_LTS_F8_MIN_BT && BT <= DFK_GU_LTS_MAX_BT) {
            // x staged in LDS per workgroup (as for bf16 weights)
            constexpr int W = DFK_GU_LTS_WAVES;
            static const void *const lts[4] = {DFK_GU_LTS_F8_MIN_BT <= 1 ? (const void *)gate_up_mfma_lts_kernel<1, W, true> : nullptr,
                                               (const void *)gate_up_mfma_lts_kernel<2, W, true>,
                                               (const void *)gate_up_mfma_lts_kernel<3, W, true>,
                                               (const void *)gate_up_mfma_lts_kernel<4, W, true>};
            Plan q{};
            q.op = op;
            q.engine = ENGINE_MFMA;
            q.trav = trav;
            q.B = B;
            q.rows = d_ff;
            q.K = d_model;
            q.splits = 1;
            q.chunks_per_split = q.K / 8;
            q.kind = KIND_GU_MFMA_LT;
            q.groups = (int)ceil_div(q.rows, 16);
            if (BT >= DFK_GU_LTS_F8_K16_MIN_BT ||
                10 * (long)q.groups >= (long)DFK_GU_LTS_F8_BT1_TILES_X10 * cus) {
                // 128-element blocks (as for bf16 weights; one x buffer)
                static const void *const lts16[2][4] = {
                    {(const void *)gate_up_mfma_lts_kernel<1, 2, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<2, 2, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<3, 2, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<4, 2, true, 1, 16>},
                    {(const void *)gate_up_mfma_lts_kernel<1, 4, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<2, 4, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<3, 4, true, 1, 16>,
                     (const void *)gate_up_mfma_lts_kernel<4, 4, true, 1, 16>}};
                const int w = q.groups >= (long)DFK_GU_LTS_K16_W4_X * cus ? 4 : 2;
                q.block = w * kWave;
                q.lds_bytes = (size_t)16 * BT * 17 * 16 + (size_t)w * 2 * Lt8<16>::kTile * 16;
                q.rows_per_group = 16;
                q.fn = lts16[w == 4 ? 1 : 0][BT - 1];
                const long occ = blocks_per_cu(q.fn, q.block, q.lds_bytes);
                q.grid = (int)std::max(1L, std::min((long)cus * occ, ceil_div((long)q.groups, (long)w)));
                *out = q;
                return true;
            }
            q.block = W * kWave;
            q.lds_bytes = (size_t)16 * BT * kStPitch * 16 + (size_t)W * 2 * Lt8<32>::kTile * 16;
            if (q.lds_bytes > kLdsLimit) return false;
            q.rows_per_group = 16;
            q.groups = (int)ceil_div(q.rows, 16);
            q.fn = lts[BT - 1];
            const long occ = blocks_per_cu(q.fn, q.block, q.lds_bytes);
            q.grid = (int)std::max(1L, std::min((long)cus * occ, ceil_div((long)q.groups, (long)W)));
            *out = q;
            return true;
        }
        const bool ks2 = gu && !row && ceil_div((long)d_ff, 16L) < (long)DFK_LT_GU_F8_KS2_TILES * cus;
        const KernelInfo ki = row ? (gu ? kGuLtRowF8 : kDnLtRowF8)[BT - 1]
                                  : (gu ? (ks2 ? kGuLtColF8K2 : kGuLtColF8) : kDnLtColF8)[BT - 1];
        Plan q{};
        q.op = op;
        q.engine = ENGINE_MFMA;
        q.trav = trav;
        q.B = B;
        q.rows = gu ? d_ff : d_model;
        q.K = gu ? d_model : d_ff;
        q.splits = 1;
        q.chunks_per_split = q.K / 8;
        const int waves = ki.block / kWave;
        q.lds_bytes = (size_t)waves * (gu ? 2 * Lt8<32>::kTile : Lt8<DFK_LT_DN_KBC>::kTile) * 16 +
                      (ki.waves_per_item > 1 ? (size_t)waves * ki.nv * kWave * sizeof(float) : 0);
        if (q.lds_bytes > kLdsLimit) return false;
        q.kind = gu ? KIND_GU_MFMA_LT : KIND_DN_MFMA_LT;
        q.block = ki.block;
        q.rows_per_group = 16;
        q.groups = (int)ceil_div(q.rows, 16);
        const int occ = blocks_per_cu(ki.fn, q.block, q.lds_bytes);
        const long wg_items = ceil_div(q.groups, waves / ki.waves_per_item);
        q.grid = (int)std::max(1L, std::min((long)cus * occ, wg_items));
        q.fn = ki.fn;
        *out = q;
        return true;
    }
    if (trav != TRAV_ROW || B > kF8MaxBatch) return false;
    Plan q{};
    q.op = op;
    q.engine = ENGINE_VALU;
    q.trav = TRAV_ROW;
    q.B = B;
    q.rows = gu ? d_ff : d_model;
    q.K = gu ? d_model : d_ff;
    q.splits = 1;
    q.chunks_per_split = q.K / 16;
    KernelInfo ki{};
    if (gu) {
        ki = kGuF8Row[B - 1];
        q.lds_bytes = (size_t)B * d_model * 2;  // x
        if (q.lds_bytes > kLdsLimit) return false;
        q.kind = KIND_GU_FP8_ROW;
    } else {
        // h in LDS, K cut into the fewest panels whose h slice fits
        const long c16 = q.K / 16;
        // (cs + 1) x 64 bytes per batch row: four quarter planes, each
        // padded by one 16-byte word
        const long max_cs = std::max(1L, (long)(kHLdsLimit / ((size_t)B * 64)) - 1);
        const long S = ceil_div(c16, max_cs);
        const long cs = ceil_div(c16, S);
        q.splits = (int)ceil_div(c16, cs);
        q.chunks_per_split = (int)cs;
        q.partial_floats = q.splits > 1 ? (size_t)q.splits * B * q.rows : 0;
        q.h_in_lds = true;
        ki = kDnF8Row[B - 1];
        q.lds_bytes = (size_t)B * (cs + 1) * 64;
        q.kind = KIND_DN_FP8_ROW;
    }
    q.block = ki.block;
    q.rows_per_group = ki.rows_per_group;
    q.groups = (int)ceil_div(q.rows, ki.rows_per_group);
    // persistent, balanced: every wave of a panel gets the same number of row
    // groups (the panels share the resident waves)
    const long waves = std::max(1L, (long)cus * blocks_per_cu(ki.fn, q.block, q.lds_bytes) * (q.block / kWave) /
                                        q.splits);
    const long per_wave = ceil_div((long)q.groups, waves);
    q.grid = (int)std::max(1L, ceil_div(ceil_div((long)q.groups, per_wave), q.block / kWave));
    q.fn = ki.fn;
    *out = q;
    return true;
}

hipError_t launch_gate_up_fp8(const Plan &p, const uint16_t *x, const uint8_t *q_gate, const float *s_gate,
                              const uint8_t *q_up, const float *s_up, float *h, hipStream_t stream) {
    if (p.kind == KIND_GU_MFMA_LT) {
        GateUpArgs a{};
        a.x = x; a.qg = q_gate; a.qu = q_up; a.sg = s_gate; a.su = s_up; a.h = h;
        a.B = p.B; a.K = p.K; a.N = p.rows; a.C = p.K / 8; a.groups = p.groups; a.ldw = p.K;
        void *argv[] = {&a};
        return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    }
    if (p.kind != KIND_GU_FP8_ROW) return hipErrorInvalidValue;
    GateUpF8Args a{};
    a.x = x; a.qg = q_gate; a.qu = q_up; a.sg = s_gate; a.su = s_up; a.h = h;
    a.B = p.B; a.K = p.K; a.N = p.rows; a.C = p.K / 8; a.C16 = p.K / 16; a.groups = p.groups;
    void *argv[] = {&a};
    return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
}

hipError_t launch_down_fp8(const Plan &p, const float *h, const uint8_t *q_down, const float *s_down, uint16_t *y,
                           float *partial, hipStream_t stream) {
    if (p.kind == KIND_DN_VALU_HREG) {
        DownArgs a{};
        a.h = h; a.qd = q_down; a.sd = s_down; a.y = y;
        a.B = p.B; a.K = p.K; a.M = p.rows; a.C = p.K / 16; a.groups = p.groups;
        void *argv[] = {&a};
        return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    }
    if (p.kind == KIND_DN_MFMA_LT) {
        DownArgs a{};
        a.h = h; a.qd = q_down; a.sd = s_down; a.y = y;
        a.B = p.B; a.K = p.K; a.M = p.rows; a.C = p.K / 8; a.groups = p.groups;
        void *argv[] = {&a};
        return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    }
    if (p.kind == KIND_DN_MFMA_STAGED) {
        DownArgs a{};
        a.h = h; a.qd = q_down; a.sd = s_down; a.y = y;
        a.B = p.B; a.K = p.K; a.M = p.rows; a.C = p.K / 8; a.groups = p.groups;
        int S = p.splits, CS = p.chunks_per_split;
        if (S > 1 && !partial) return hipErrorInvalidValue;
        float *part = S > 1 ? partial : nullptr;
        void *argv[] = {&a, &part, &S, &CS};
        hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
        if (e != hipSuccess || S == 1) return e;
        return launch_reduce(partial, y, S, p.B * p.rows, stream);
    }
    if (p.kind != KIND_DN_FP8_ROW) return hipErrorInvalidValue;
    if (p.splits > 1 && !partial) return hipErrorInvalidValue;
    DownF8Args a{};
    a.h = h; a.qd = q_down; a.sd = s_down; a.y = y;
    a.B = p.B; a.K = p.K; a.M = p.rows; a.C16 = p.K / 16; a.groups = p.groups;
    int cs = p.chunks_per_split;
    void *argv[] = {&a, &partial, &cs};
    hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid, p.splits), dim3(p.block), argv, p.lds_bytes, stream);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_reduce(partial, y, p.splits, p.B * p.rows, stream);
}

hipError_t launch_gate_up(const Plan &p, const uint16_t *x, const uint16_t *w_gate, const uint16_t *w_up,
                          float *h, float *partial, hipStream_t stream, const NormArgs *norm, int ldw) {
    GateUpArgs a;
    a.x = x; a.wg = w_gate; a.wu = w_up; a.h = h;
    a.B = p.B; a.K = p.K; a.N = p.rows; a.C = p.K / 8; a.groups = p.groups;
    a.ldw = ldw > 0 ? ldw : p.K;
    if (a.ldw < p.K) return hipErrorInvalidValue;
    a.gain = nullptr; a.eps = 0.0;
    if (p.fused_norm) {
        if (!norm || !norm->gain) return hipErrorInvalidValue;
        a.gain = norm->gain;
        a.eps = norm->eps;
    }
    (void)partial;
    void *argv[] = {&a};
    return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
}

hipError_t launch_rmsnorm(const uint16_t *x, const NormArgs &norm, uint16_t *xn, int B, int K, hipStream_t stream) {
    if (B < 1 || K < 8 || (K % 8) || !norm.gain) return hipErrorInvalidValue;
    const uint16_t *gain = norm.gain;
    double eps = norm.eps;
    void *argv[] = {&x, &gain, &eps, &xn, &K};
    return hipLaunchKernel((const void *)rmsnorm_kernel, dim3(B), dim3(kNormThreads), argv, 0, stream);
}

hipError_t launch_down(const Plan &p, const float *h, const uint16_t *w_down, uint16_t *y, float *partial,
                       hipStream_t stream) {
    DownArgs a;
    a.h = h; a.wd = w_down; a.y = y;
    a.B = p.B; a.K = p.K; a.M = p.rows; a.C = p.K / 8; a.groups = p.groups;
    if (p.kind == KIND_DN_VALU_PANEL) {
        if (!partial) return hipErrorInvalidValue;
        int cs = p.chunks_per_split;
        void *argv[] = {&a, &partial, &cs};
        hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid, p.splits), dim3(p.block), argv, p.lds_bytes, stream);
        if (e != hipSuccess) return e;
        return launch_reduce(partial, y, p.splits, p.B * p.rows, stream);
    }
    if (p.kind != KIND_DN_MFMA_STAGED) {
        void *argv[] = {&a};
        return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    }
    int S = p.splits, CS = p.chunks_per_split;
    if (p.kind == KIND_DN_MFMA_STAGED && S == 1) {
        float *none = nullptr;
        void *argv[] = {&a, &none, &S, &CS};
        return hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    }
    if (!partial) return hipErrorInvalidValue;
    void *argv[] = {&a, &partial, &S, &CS};
    hipError_t e = hipLaunchKernel(p.fn, dim3(p.grid), dim3(p.block), argv, p.lds_bytes, stream);
    if (e != hipSuccess) return e;
    return launch_reduce(partial, y, S, p.B * p.rows, stream);
}

// --------------------------------------------- static scratch (no alloc) --
//
// The whole-MLP entry point for callers that cannot allocate keeps h and the
// down projection's split sums here instead of in the library's growable
// workspace.  Host code must never pass `scratch` itself to a kernel: on the
// host the name stands for a host-side shadow, not a device address.  Kernels
// get the address that hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(int dev, void **ptr) {
    static std::mutex mu;
    static std::map<int, void *> addr;  // device -> address of its copy
    std::lock_guard<std::mutex> lock(mu);
    auto it = addr.find(dev);
    if (it != addr.end()) {
        *ptr = it->second;
        return hipSuccess;
    }
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return e != hipSuccess ? e : hipErrorInvalidSymbol;
    }
    addr[dev] = p;
    *ptr = p;
    return hipSuccess;
}

}  // namespace dfk
