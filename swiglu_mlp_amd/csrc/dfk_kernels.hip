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
//   ROW  each output row's whole dot product belongs to one wave (VALU) or one
//        workgroup (MFMA, its 4 waves split K and combine through LDS).
//   COL  the weight matrix is cut into K panels; a panel's partial sums go to
//        scratch and the last arrival for a row block (an atomic counter)
//        adds the panels in fixed order and runs the epilogue.  Deterministic.
// Every kernel is persistent-style: the grid is sized to the machine and each
// wave / workgroup walks a strided list of work items.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "dfk_kernels.h"

namespace dfk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kValuBlock = 512;  // 8 waves
constexpr int kMfmaBlock = 256;  // 4 waves
constexpr int kMfmaWaves = kMfmaBlock / kWave;

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

// Last-arrival protocol of the COL traversal.  Every wave that finished a
// panel of row group `group` calls this after storing its partials; exactly
// one caller (the last) gets true, sees every panel's partials, and must
// reset the counter.  Release/acquire fences at agent scope make the
// partials visible across XCDs (each XCD has its own L2).
__device__ __forceinline__ bool arrive_last(unsigned *counter, int panels) {
    __threadfence();
    unsigned prev = 0;
    if ((threadIdx.x & (kWave - 1)) == 0) prev = atomicAdd(counter, 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev == (unsigned)(panels - 1)) {
        __threadfence();
        return true;
    }
    return false;
}

// ------------------------------------------------------------- arguments --

struct GateUpArgs {
    const uint16_t *x;
    const uint16_t *wg;
    const uint16_t *wu;
    float *h;
    float *partial;
    unsigned *counters;
    int B, K, N;   // batch, d_model, d_ff
    int C;         // 16-byte chunks per weight row (K / 8)
    int S;         // K panels
    int CS;        // chunks per panel
    int groups;    // row groups
    int items;     // groups * S
};

struct DownArgs {
    const float *h;
    const uint16_t *wd;
    uint16_t *y;
    float *partial;
    unsigned *counters;
    int B, K, M;   // batch, d_ff, d_model
    int C, S, CS, groups, items;
};

// ==================================================== VALU gate-up kernel ==
//
// Work item = (row group of R neurons, K panel).  The wave streams the R rows
// of W_gate and the same R rows of W_up over the panel; lane l owns chunks
// l, l+64, ... (8 elements each); x is resident in LDS for the whole kernel
// (loaded once per workgroup) and each x chunk read serves 2R weight rows.
template <int B, int R, int U>
__global__ __launch_bounds__(kValuBlock) void gate_up_valu_kernel(GateUpArgs a) {
    extern __shared__ u32x4_t xs[];  // [B][C]
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int gw = blockIdx.x * waves + threadIdx.x / kWave;
    const int total_waves = gridDim.x * waves;

    const u32x4_t *xg = reinterpret_cast<const u32x4_t *>(a.x);
    for (int i = threadIdx.x; i < B * a.C; i += blockDim.x) xs[i] = xg[i];
    __syncthreads();

    for (int item = gw; item < a.items; item += total_waves) {
        const int gi = item / a.S;
        const int s = item - gi * a.S;
        const int c_beg = s * a.CS;
        const int c_end = min(c_beg + a.CS, a.C);
        const u32x4_t *rg[R];
        const u32x4_t *ru[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(gi * R + r, a.N - 1);
            rg[r] = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)n * a.K);
            ru[r] = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)n * a.K);
        }
        float ag[R][B], au[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) ag[r][b] = au[r][b] = 0.0f;

        for (int c0 = c_beg; c0 < c_end; c0 += kWave * U) {
            u32x4_t wgv[U][R], wuv[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // clamped so every load is in bounds; out-of-panel lanes skip the math
                const int c = min(c0 + kWave * u + lane, c_end - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    wgv[u][r] = load_stream(rg[r] + c);
                    wuv[u][r] = load_stream(ru[r] + c);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + kWave * u + lane;
                if (c < c_end) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const u32x4_t xv = xs[b * a.C + c];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            ag[r][b] = dot8_bf16(wgv[u][r], xv, ag[r][b]);
                            au[r][b] = dot8_bf16(wuv[u][r], xv, au[r][b]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                ag[r][b] = wave_sum_to_lane63(ag[r][b]);
                au[r][b] = wave_sum_to_lane63(au[r][b]);
            }

        if (a.S == 1) {
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int n = gi * R + r;
                    if (n < a.N)
#pragma unroll
                        for (int b = 0; b < B; ++b) a.h[(size_t)b * a.N + n] = silu_mul(ag[r][b], au[r][b]);
                }
            }
        } else {
            constexpr int NV = 2 * R * B;
            float *p = a.partial + ((size_t)gi * a.S + s) * NV;
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        p[r * B + b] = ag[r][b];
                        p[R * B + r * B + b] = au[r][b];
                    }
            }
            if (arrive_last(a.counters + gi, a.S)) {
                if (lane < R * B) {
                    const int r = lane / B, b = lane - (lane / B) * B;
                    const int n = gi * R + r;
                    const float *q = a.partial + (size_t)gi * a.S * NV;
                    float g = 0.0f, u = 0.0f;
                    for (int t = 0; t < a.S; ++t) {
                        g += q[(size_t)t * NV + lane];
                        u += q[(size_t)t * NV + R * B + lane];
                    }
                    if (n < a.N) a.h[(size_t)b * a.N + n] = silu_mul(g, u);
                }
                if (lane == 0) a.counters[gi] = 0u;
            }
        }
    }
}

// ======================================================= VALU down kernel ==
//
// Work item = (group of R rows of W_down, K panel).  Lane l owns chunks l,
// l+64, ...; for each chunk it widens 8 bf16 weights per row and does fp32
// FMAs against 8 fp32 values of h per batch row (h read through the caches;
// one h read serves R rows).
template <int B, int R, int U>
__global__ __launch_bounds__(kValuBlock) void down_valu_kernel(DownArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const int gw = blockIdx.x * waves + threadIdx.x / kWave;
    const int total_waves = gridDim.x * waves;
    const f32x4_t *hg = reinterpret_cast<const f32x4_t *>(a.h);  // [B][2C]

    for (int item = gw; item < a.items; item += total_waves) {
        const int gi = item / a.S;
        const int s = item - gi * a.S;
        const int c_beg = s * a.CS;
        const int c_end = min(c_beg + a.CS, a.C);
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

        for (int c0 = c_beg; c0 < c_end; c0 += kWave * U) {
            u32x4_t wv[U][R];
            f32x4_t hv[U][B][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(c0 + kWave * u + lane, c_end - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) wv[u][r] = load_stream(rd[r] + c);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    hv[u][b][0] = hg[(size_t)b * 2 * a.C + 2 * c];
                    hv[u][b][1] = hg[(size_t)b * 2 * a.C + 2 * c + 1];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + kWave * u + lane;
                if (c < c_end) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const u32x4_t w = wv[u][r];
                        const float w0 = bf16_lo(w.x), w1 = bf16_hi(w.x), w2 = bf16_lo(w.y),
                                    w3 = bf16_hi(w.y), w4 = bf16_lo(w.z), w5 = bf16_hi(w.z),
                                    w6 = bf16_lo(w.w), w7 = bf16_hi(w.w);
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            const f32x4_t h0 = hv[u][b][0], h1 = hv[u][b][1];
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
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = wave_sum_to_lane63(acc[r][b]);

        if (a.S == 1) {
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int m = gi * R + r;
                    if (m < a.M)
#pragma unroll
                        for (int b = 0; b < B; ++b) a.y[(size_t)b * a.M + m] = to_bf16_rne(acc[r][b]);
                }
            }
        } else {
            constexpr int NV = R * B;
            float *p = a.partial + ((size_t)gi * a.S + s) * NV;
            if (lane == kWave - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int b = 0; b < B; ++b) p[r * B + b] = acc[r][b];
            }
            if (arrive_last(a.counters + gi, a.S)) {
                if (lane < R * B) {
                    const int r = lane / B, b = lane - (lane / B) * B;
                    const int m = gi * R + r;
                    const float *q = a.partial + (size_t)gi * a.S * NV;
                    float v = 0.0f;
                    for (int t = 0; t < a.S; ++t) v += q[(size_t)t * NV + lane];
                    if (m < a.M) a.y[(size_t)b * a.M + m] = to_bf16_rne(v);
                }
                if (lane == 0) a.counters[gi] = 0u;
            }
        }
    }
}

// ==================================================== MFMA gate-up kernel ==
//
// Work item = (tile of 16*TR neurons, K panel), owned by a workgroup of 4
// waves that split the panel's 32-wide K steps into 4 contiguous runs.
// Lane l: r = l & 15 (tile row for A, batch column for B), q = l >> 4 (which
// 8-element chunk of the 32-wide K step).  MFMA 16x16x32 bf16:
//   A[i][k] = W[n0+i][k]   (lane (i, q) holds 8 consecutive k)
//   B[k][j] = x[b0+j][k]   (same k assignment, so the sum pairs up correctly)
//   D[i][j] -> lane (j, i/4) element i%4.
// The 4 waves' accumulators are added in wave order through LDS; wave 0 runs
// the epilogue (ROW) or stores the panel partials (COL).
template <int BT, int TR, int U>
__global__ __launch_bounds__(kMfmaBlock) void gate_up_mfma_kernel(GateUpArgs a) {
    constexpr int NV = 2 * TR * BT * 4;  // accumulator floats per lane
    extern __shared__ float red[];       // [waves-1][NV][64]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & 15;
    const int lq = lane >> 4;

    for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
        const int gi = item / a.S;
        const int s = item - gi * a.S;
        // panel in chunks -> in 32-wide steps (4 chunks each)
        const int c_beg = s * a.CS;
        const int c_end = min(c_beg + a.CS, a.C);
        const int steps = (c_end - c_beg + 3) / 4;
        const int per_wave = (steps + kMfmaWaves - 1) / kMfmaWaves;
        const int st_beg = min(wave * per_wave, steps);
        const int st_end = min(st_beg + per_wave, steps);

        const u32x4_t *pg[TR];
        const u32x4_t *pu[TR];
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            const int n = min(gi * 16 * TR + t * 16 + lr, a.N - 1);
            pg[t] = reinterpret_cast<const u32x4_t *>(a.wg + (size_t)n * a.K);
            pu[t] = reinterpret_cast<const u32x4_t *>(a.wu + (size_t)n * a.K);
        }
        const u32x4_t *px[BT];
        bool bvalid[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
            const int b = bt * 16 + lr;
            bvalid[bt] = b < a.B;
            px[bt] = reinterpret_cast<const u32x4_t *>(a.x + (size_t)min(b, a.B - 1) * a.K);
        }
        f32x4_t accg[TR][BT], accu[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) accg[t][bt] = accu[t][bt] = f32x4_t{0, 0, 0, 0};

        for (int st = st_beg; st < st_end; st += U) {
            u32x4_t ag[U][TR], au[U][TR], bx[U][BT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c_beg + (st + u) * 4 + lq;
                const int cc = min(c, c_end - 1);
#pragma unroll
                for (int t = 0; t < TR; ++t) {
                    ag[u][t] = load_stream(pg[t] + cc);
                    au[u][t] = load_stream(pu[t] + cc);
                }
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) bx[u][bt] = px[bt][cc];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c_beg + (st + u) * 4 + lq;
                const bool kv = (c < c_end) && (st + u < st_end);
                const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int t = 0; t < TR; ++t) {
                    const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, kv ? ag[u][t] : zero);
                    const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, kv ? au[u][t] : zero);
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt) {
                        const bf16x8_t xb =
                            __builtin_bit_cast(bf16x8_t, (kv && bvalid[bt]) ? bx[u][bt] : zero);
                        accg[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, xb, accg[t][bt], 0, 0, 0);
                        accu[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, accu[t][bt], 0, 0, 0);
                    }
                }
            }
        }

        // combine the 4 waves in order 0 + 1 + 2 + 3 through LDS
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
            for (int w = 1; w < kMfmaWaves; ++w) {
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
            if (a.S == 1) {
#pragma unroll
                for (int t = 0; t < TR; ++t) {
                    const int n = gi * 16 * TR + t * 16 + 4 * lq;  // 4 consecutive neurons
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
            } else {
                float *p = a.partial + ((size_t)gi * a.S + s) * NV * kWave;
                int v = 0;
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            p[(v++) * kWave + lane] = accg[t][bt][e];
                            p[(v++) * kWave + lane] = accu[t][bt][e];
                        }
                if (arrive_last(a.counters + gi, a.S)) {
                    const float *q = a.partial + (size_t)gi * a.S * NV * kWave;
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        const int n = gi * 16 * TR + t * 16 + 4 * lq;
#pragma unroll
                        for (int bt = 0; bt < BT; ++bt) {
                            const int b = bt * 16 + lr;
                            const int v0 = ((t * BT + bt) * 4) * 2;
                            f32x4_t o;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float g = 0.0f, u = 0.0f;
                                for (int pn = 0; pn < a.S; ++pn) {
                                    const float *qq = q + (size_t)pn * NV * kWave;
                                    g += qq[(v0 + 2 * e) * kWave + lane];
                                    u += qq[(v0 + 2 * e + 1) * kWave + lane];
                                }
                                o[e] = silu_mul(g, u);
                            }
                            if (b < a.B && n < a.N)
                                *reinterpret_cast<f32x4_t *>(a.h + (size_t)b * a.N + n) = o;
                        }
                    }
                    if (lane == 0) a.counters[gi] = 0u;
                }
            }
        }
        __syncthreads();  // LDS reuse by the next item
    }
}

// ======================================================= MFMA down kernel ==
//
// Same tiling as the MFMA gate-up kernel with one weight matrix: A = W_down
// tile (16*TR rows of d_model), B = h^T.  Each lane widens 8 fp32 h values,
// splits them into bf16 hi + lo and issues two MFMAs per tile.
template <int BT, int TR, int U>
__global__ __launch_bounds__(kMfmaBlock) void down_mfma_kernel(DownArgs a) {
    constexpr int NV = TR * BT * 4;
    extern __shared__ float red[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & 15;
    const int lq = lane >> 4;

    for (int item = blockIdx.x; item < a.items; item += gridDim.x) {
        const int gi = item / a.S;
        const int s = item - gi * a.S;
        const int c_beg = s * a.CS;
        const int c_end = min(c_beg + a.CS, a.C);
        const int steps = (c_end - c_beg + 3) / 4;
        const int per_wave = (steps + kMfmaWaves - 1) / kMfmaWaves;
        const int st_beg = min(wave * per_wave, steps);
        const int st_end = min(st_beg + per_wave, steps);

        const u32x4_t *pw[TR];
#pragma unroll
        for (int t = 0; t < TR; ++t) {
            const int m = min(gi * 16 * TR + t * 16 + lr, a.M - 1);
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
        f32x4_t acc[TR][BT];
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) acc[t][bt] = f32x4_t{0, 0, 0, 0};

        for (int st = st_beg; st < st_end; st += U) {
            u32x4_t aw[U][TR];
            f32x4_t hb[U][BT][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c_beg + (st + u) * 4 + lq;
                const int cc = min(c, c_end - 1);
#pragma unroll
                for (int t = 0; t < TR; ++t) aw[u][t] = load_stream(pw[t] + cc);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    hb[u][bt][0] = ph[bt][2 * cc];
                    hb[u][bt][1] = ph[bt][2 * cc + 1];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c_beg + (st + u) * 4 + lq;
                const bool kv = (c < c_end) && (st + u < st_end);
                const u32x4_t zero = {0u, 0u, 0u, 0u};
                const f32x4_t fzero = {0.0f, 0.0f, 0.0f, 0.0f};
                bf16x8_t hhi[BT], hlo[BT];
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const bool ok = kv && bvalid[bt];
                    split_hi_lo(ok ? hb[u][bt][0] : fzero, ok ? hb[u][bt][1] : fzero, hhi[bt], hlo[bt]);
                }
#pragma unroll
                for (int t = 0; t < TR; ++t) {
                    const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, kv ? aw[u][t] : zero);
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt) {
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, hhi[bt], acc[t][bt], 0, 0, 0);
                        acc[t][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, hlo[bt], acc[t][bt], 0, 0, 0);
                    }
                }
            }
        }

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
            for (int w = 1; w < kMfmaWaves; ++w) {
                const float *src = red + (size_t)(w - 1) * NV * kWave;
                int v = 0;
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[t][bt][e] += src[(v++) * kWave + lane];
            }
            if (a.S == 1) {
#pragma unroll
                for (int t = 0; t < TR; ++t) {
                    const int m = gi * 16 * TR + t * 16 + 4 * lq;
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt) {
                        const int b = bt * 16 + lr;
                        if (b < a.B && m < a.M) {
                            uint16_t *o = a.y + (size_t)b * a.M + m;
                            const unsigned lo = to_bf16_rne(acc[t][bt][0]) | ((unsigned)to_bf16_rne(acc[t][bt][1]) << 16);
                            const unsigned hi = to_bf16_rne(acc[t][bt][2]) | ((unsigned)to_bf16_rne(acc[t][bt][3]) << 16);
                            *reinterpret_cast<uint2 *>(o) = make_uint2(lo, hi);
                        }
                    }
                }
            } else {
                float *p = a.partial + ((size_t)gi * a.S + s) * NV * kWave;
                int v = 0;
#pragma unroll
                for (int t = 0; t < TR; ++t)
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) p[(v++) * kWave + lane] = acc[t][bt][e];
                if (arrive_last(a.counters + gi, a.S)) {
                    const float *q = a.partial + (size_t)gi * a.S * NV * kWave;
#pragma unroll
                    for (int t = 0; t < TR; ++t) {
                        const int m = gi * 16 * TR + t * 16 + 4 * lq;
#pragma unroll
                        for (int bt = 0; bt < BT; ++bt) {
                            const int b = bt * 16 + lr;
                            const int v0 = (t * BT + bt) * 4;
                            float o[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float sum = 0.0f;
                                for (int pn = 0; pn < a.S; ++pn)
                                    sum += q[(size_t)pn * NV * kWave + (v0 + e) * kWave + lane];
                                o[e] = sum;
                            }
                            if (b < a.B && m < a.M) {
                                uint16_t *dst = a.y + (size_t)b * a.M + m;
                                const unsigned lo = to_bf16_rne(o[0]) | ((unsigned)to_bf16_rne(o[1]) << 16);
                                const unsigned hi = to_bf16_rne(o[2]) | ((unsigned)to_bf16_rne(o[3]) << 16);
                                *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
                            }
                        }
                    }
                    if (lane == 0) a.counters[gi] = 0u;
                }
            }
        }
        __syncthreads();
    }
}

// ======================================================== kernel tables ====
//
// Per-batch tile parameters.  VALU: R rows (pairs) per wave item, U
// load-groups in flight per lane.  MFMA: BT batch tiles of 16, TR row tiles
// of 16 per item, U K-steps per load group.

template <int B> struct ValuGU { static constexpr int R = (B <= 2) ? 1 : 2; static constexpr int U = (B <= 2) ? 4 : 2; };
template <int B> struct ValuDn { static constexpr int R = (B <= 2) ? 2 : 4; static constexpr int U = (B <= 4) ? 2 : 1; };
template <int BT> struct MfmaGU { static constexpr int TR = (BT <= 2) ? 2 : 1; static constexpr int U = (BT <= 2) ? 2 : 1; };
template <int BT> struct MfmaDn { static constexpr int TR = (BT <= 2) ? 4 : (BT <= 4 ? 2 : 1); static constexpr int U = (BT <= 2) ? 2 : 1; };

typedef void (*GateUpFn)(GateUpArgs);
typedef void (*DownFn)(DownArgs);

template <int B> constexpr GateUpFn gu_valu_fn() { return gate_up_valu_kernel<B, ValuGU<B>::R, ValuGU<B>::U>; }
template <int B> constexpr DownFn dn_valu_fn() { return down_valu_kernel<B, ValuDn<B>::R, ValuDn<B>::U>; }
template <int BT> constexpr GateUpFn gu_mfma_fn() { return gate_up_mfma_kernel<BT, MfmaGU<BT>::TR, MfmaGU<BT>::U>; }
template <int BT> constexpr DownFn dn_mfma_fn() { return down_mfma_kernel<BT, MfmaDn<BT>::TR, MfmaDn<BT>::U>; }

static const GateUpFn kGuValu[kValuMaxBatch] = {gu_valu_fn<1>(), gu_valu_fn<2>(), gu_valu_fn<3>(), gu_valu_fn<4>(),
                                                gu_valu_fn<5>(), gu_valu_fn<6>(), gu_valu_fn<7>(), gu_valu_fn<8>()};
static const int kGuValuR[kValuMaxBatch] = {ValuGU<1>::R, ValuGU<2>::R, ValuGU<3>::R, ValuGU<4>::R,
                                            ValuGU<5>::R, ValuGU<6>::R, ValuGU<7>::R, ValuGU<8>::R};
static const DownFn kDnValu[kValuMaxBatch] = {dn_valu_fn<1>(), dn_valu_fn<2>(), dn_valu_fn<3>(), dn_valu_fn<4>(),
                                              dn_valu_fn<5>(), dn_valu_fn<6>(), dn_valu_fn<7>(), dn_valu_fn<8>()};
static const int kDnValuR[kValuMaxBatch] = {ValuDn<1>::R, ValuDn<2>::R, ValuDn<3>::R, ValuDn<4>::R,
                                            ValuDn<5>::R, ValuDn<6>::R, ValuDn<7>::R, ValuDn<8>::R};

constexpr int kMaxBT = 16;  // B <= 256
static const GateUpFn kGuMfma[kMaxBT] = {
    gu_mfma_fn<1>(), gu_mfma_fn<2>(), gu_mfma_fn<3>(), gu_mfma_fn<4>(), gu_mfma_fn<5>(), gu_mfma_fn<6>(),
    gu_mfma_fn<7>(), gu_mfma_fn<8>(), gu_mfma_fn<9>(), gu_mfma_fn<10>(), gu_mfma_fn<11>(), gu_mfma_fn<12>(),
    gu_mfma_fn<13>(), gu_mfma_fn<14>(), gu_mfma_fn<15>(), gu_mfma_fn<16>()};
static const int kGuMfmaTR[kMaxBT] = {MfmaGU<1>::TR, MfmaGU<2>::TR, MfmaGU<3>::TR, MfmaGU<4>::TR,
                                      MfmaGU<5>::TR, MfmaGU<6>::TR, MfmaGU<7>::TR, MfmaGU<8>::TR,
                                      MfmaGU<9>::TR, MfmaGU<10>::TR, MfmaGU<11>::TR, MfmaGU<12>::TR,
                                      MfmaGU<13>::TR, MfmaGU<14>::TR, MfmaGU<15>::TR, MfmaGU<16>::TR};
static const DownFn kDnMfma[kMaxBT] = {
    dn_mfma_fn<1>(), dn_mfma_fn<2>(), dn_mfma_fn<3>(), dn_mfma_fn<4>(), dn_mfma_fn<5>(), dn_mfma_fn<6>(),
    dn_mfma_fn<7>(), dn_mfma_fn<8>(), dn_mfma_fn<9>(), dn_mfma_fn<10>(), dn_mfma_fn<11>(), dn_mfma_fn<12>(),
    dn_mfma_fn<13>(), dn_mfma_fn<14>(), dn_mfma_fn<15>(), dn_mfma_fn<16>()};
static const int kDnMfmaTR[kMaxBT] = {MfmaDn<1>::TR, MfmaDn<2>::TR, MfmaDn<3>::TR, MfmaDn<4>::TR,
                                      MfmaDn<5>::TR, MfmaDn<6>::TR, MfmaDn<7>::TR, MfmaDn<8>::TR,
                                      MfmaDn<9>::TR, MfmaDn<10>::TR, MfmaDn<11>::TR, MfmaDn<12>::TR,
                                      MfmaDn<13>::TR, MfmaDn<14>::TR, MfmaDn<15>::TR, MfmaDn<16>::TR};

// Blocks of a kernel that fit on one CU (cached; the answer depends only on
// the kernel, block size and LDS).
static int blocks_per_cu(const void *fn, int block, size_t lds) {
    static std::mutex mu;
    struct Entry { const void *fn; int block; size_t lds; int n; };
    static Entry cache[256];
    static int ncache = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ncache; ++i)
        if (cache[i].fn == fn && cache[i].block == block && cache[i].lds == lds) return cache[i].n;
    // allow the kernel the dynamic LDS it asks for (the default cap is below
    // the 160 KB a gfx950 CU has)
    if (lds > 0)
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kValuLdsLimit);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, block, lds) != hipSuccess || n < 1) n = 1;
    (void)hipGetLastError();
    if (ncache < 256) cache[ncache++] = Entry{fn, block, lds, n};
    return n;
}

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

bool make_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus, Plan *p) {
    if (B < 1 || d_model < 8 || d_ff < 8 || (d_model % 8) || (d_ff % 8) || cus < 1) return false;
    Plan q{};
    q.op = op;
    q.engine = engine;
    q.trav = trav;
    q.B = B;
    q.rows = (op == OP_GATE_UP) ? d_ff : d_model;
    q.K = (op == OP_GATE_UP) ? d_model : d_ff;
    const int C = q.K / 8;
    const void *fn = nullptr;
    int rows_per_group = 1;
    int waves_per_item_block = 1;  // items per block-wave unit
    int nv_per_item = 0;           // COL partial floats per item
    if (engine == ENGINE_VALU) {
        if (B > kValuMaxBatch) return false;
        q.block = kValuBlock;
        if (op == OP_GATE_UP) {
            q.lds_bytes = (size_t)B * d_model * 2;
            if (q.lds_bytes > kValuLdsLimit) return false;
            rows_per_group = kGuValuR[B - 1];
            fn = (const void *)kGuValu[B - 1];
            nv_per_item = 2 * rows_per_group * B;
        } else {
            q.lds_bytes = 0;
            rows_per_group = kDnValuR[B - 1];
            fn = (const void *)kDnValu[B - 1];
            nv_per_item = rows_per_group * B;
        }
        q.kernel_id = B - 1;
        waves_per_item_block = kValuBlock / kWave;  // one item per wave
    } else {
        const int BT = ceil_div(B, 16);
        if (BT > kMaxBT) return false;
        q.block = kMfmaBlock;
        const int TR = (op == OP_GATE_UP) ? kGuMfmaTR[BT - 1] : kDnMfmaTR[BT - 1];
        rows_per_group = 16 * TR;
        const int nv = (op == OP_GATE_UP ? 2 : 1) * TR * BT * 4;
        q.lds_bytes = (size_t)(kMfmaWaves - 1) * nv * kWave * sizeof(float);
        fn = (op == OP_GATE_UP) ? (const void *)kGuMfma[BT - 1] : (const void *)kDnMfma[BT - 1];
        nv_per_item = nv * kWave;
        q.kernel_id = BT - 1;
        waves_per_item_block = 1;  // one item per workgroup
    }
    q.groups = ceil_div(q.rows, rows_per_group);
    const int occ = blocks_per_cu(fn, q.block, q.lds_bytes);
    const long slots = (long)cus * occ * waves_per_item_block;  // concurrent items
    if (trav == TRAV_ROW) {
        q.splits = 1;
    } else {
        // Enough panels to give every item slot ~2 items, but keep each
        // panel at least 4 KB of a weight row (256 chunks) so loads stay long.
        int S = ceil_div(2 * slots, q.groups);
        S = std::max(2, std::min(S, std::max(1, C / 256)));
        S = std::min(S, C);
        q.splits = std::max(1, S);
    }
    q.chunks_per_split = ceil_div(C, q.splits);
    // make sure no panel is empty
    q.splits = ceil_div(C, q.chunks_per_split);
    const long items = (long)q.groups * q.splits;
    q.grid = (int)std::max(1L, std::min((long)cus * occ, (items + waves_per_item_block - 1) / waves_per_item_block));
    if (q.splits > 1) {
        q.partial_floats = (size_t)items * nv_per_item;
        q.counters = (size_t)q.groups;
    }
    *p = q;
    return true;
}

hipError_t launch_gate_up(const Plan &p, const uint16_t *x, const uint16_t *w_gate, const uint16_t *w_up,
                          float *h, float *partial, unsigned *counters, hipStream_t stream) {
    GateUpArgs a;
    a.x = x; a.wg = w_gate; a.wu = w_up; a.h = h; a.partial = partial; a.counters = counters;
    a.B = p.B; a.K = p.K; a.N = p.rows; a.C = p.K / 8; a.S = p.splits; a.CS = p.chunks_per_split;
    a.groups = p.groups; a.items = p.groups * p.splits;
    GateUpFn fn = (p.engine == ENGINE_VALU) ? kGuValu[p.kernel_id] : kGuMfma[p.kernel_id];
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(p.grid), dim3(p.block), args, p.lds_bytes,
                           stream);
}

hipError_t launch_down(const Plan &p, const float *h, const uint16_t *w_down, uint16_t *y, float *partial,
                       unsigned *counters, hipStream_t stream) {
    DownArgs a;
    a.h = h; a.wd = w_down; a.y = y; a.partial = partial; a.counters = counters;
    a.B = p.B; a.K = p.K; a.M = p.rows; a.C = p.K / 8; a.S = p.splits; a.CS = p.chunks_per_split;
    a.groups = p.groups; a.items = p.groups * p.splits;
    DownFn fn = (p.engine == ENGINE_VALU) ? kDnValu[p.kernel_id] : kDnMfma[p.kernel_id];
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(p.grid), dim3(p.block), args, p.lds_bytes,
                           stream);
}

}  // namespace dfk
