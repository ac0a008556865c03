// dfk_kernels.h -- internal interface between the C-ABI runtime and the HIP kernels.
// Not installed; the public interface is include/dfk.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfk {

enum Engine { ENGINE_VALU = 0, ENGINE_MFMA = 1 };
enum Traversal { TRAV_ROW = 0, TRAV_COL = 1 };
enum Op { OP_GATE_UP = 0, OP_DOWN = 1 };

// Largest batch the VALU kernels are instantiated for.  Above it (and where a
// VALU kernel's LDS staging would not fit) the MFMA kernels run.
constexpr int kValuMaxBatch = 8;
// LDS of one gfx950 CU: the most a workgroup may ask for (the VALU gate-up
// kernels keep all of x there).
constexpr size_t kLdsLimit = 160 * 1024;
// The VALU down kernels keep all of h in LDS up to this size (one workgroup
// per CU at the top; measured faster than reading h through the caches), else
// they read it through the caches.
constexpr size_t kHLdsLimit = 128 * 1024;

enum Kind {
    KIND_GU_VALU_ROW = 0,
    KIND_GU_VALU_COL = 1,
    KIND_DN_VALU_ROW = 2,
    KIND_DN_VALU_COL = 3,
    KIND_GU_MFMA_ROW = 4,
    KIND_GU_MFMA_COL = 5,
    KIND_DN_MFMA_ROW = 6,
    KIND_DN_MFMA_COL = 7,
    KIND_GU_MFMA_LT = 10,    // gate-up, weights streamed through a wave-private LDS transpose
    KIND_DN_MFMA_LT = 11,
    KIND_GU_MFMA_STAGED = 12,  // gate-up, B operand staged in LDS per workgroup (B > 16)
    KIND_DN_MFMA_STAGED = 13,  // down, the same, K split across workgroups + a reduce kernel
    KIND_DN_MFMA_COOP = 15,    // down ROW (B <= 16), workgroup-cooperative LDS weight tile
    KIND_GU_FP8_ROW = 16,      // gate-up over FP8 E4M3 weights + row scales, VALU row walk
    KIND_DN_FP8_ROW = 17,      // down, the same
    KIND_DN_VALU_PANEL = 18,   // down VALU row walk over K panels whose h fits in LDS + a reduce kernel
    KIND_DN_VALU_HREG = 19     // down VALU column walk, h held in registers, row groups pipelined
};

// A fully resolved launch: which kernel and how the weight matrix is cut.
struct Plan {
    Op op;
    Engine engine;
    Traversal trav;
    Kind kind;
    int B;
    int rows;            // output rows: d_ff (gate-up) or d_model (down)
    int K;               // reduction length: d_model (gate-up) or d_ff (down)
    int rows_per_group;  // rows of one work item
    int groups;          // work items
    int grid;            // workgroups
    int block;           // threads per workgroup
    size_t lds_bytes;    // dynamic LDS per workgroup
    bool h_in_lds;       // VALU down: all of h staged in LDS
    int splits;          // K panels (panel kinds), else 1
    int chunks_per_split;     // 16-byte chunks per panel
    size_t partial_floats;    // scratch the plan needs (panel partial sums), else 0
    bool fused_norm;     // gate-up: the kernel applies the RMS normalization itself
    const void *fn;      // the kernel
};

// RMS normalization ahead of gate-up: xn = bf16_RNE((x * inv) * gain),
// inv = 1 / sqrt(mean_k x^2 + eps) per batch row, all in fp64.
struct NormArgs {
    const uint16_t *gain;  // [d_model] bf16
    double eps;
};

// Fill a plan for the given shape, engine and traversal.  Returns false when
// the engine cannot run the shape (e.g. VALU with B above kValuMaxBatch, or x
// too large to keep in LDS).  `cus` is the device's compute-unit count.
// norm (gate-up only): fold the RMS normalization in where the kernel stages
// x in LDS (VALU: p.fused_norm is set); other kernels keep their plan and the
// caller normalizes x into a buffer first (launch_rmsnorm).
bool make_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus,
               Plan *plan, bool norm = false);

// Enqueue the kernel of a plan on `stream`.
// `partial` must hold p.partial_floats floats when that is non-zero.
// `ldw`: elements from one row of W_gate (and of W_up) to the next, >= the
// plan's K (0: K, dense); 2K for row-interleaved gate/up storage.
hipError_t launch_gate_up(const Plan &p, const uint16_t *x, const uint16_t *w_gate,
                          const uint16_t *w_up, float *h, float *partial, hipStream_t stream,
                          const NormArgs *norm = nullptr, int ldw = 0);
// xn [B][K] = the RMS normalization of x [B][K] (one workgroup per batch row).
hipError_t launch_rmsnorm(const uint16_t *x, const NormArgs &norm, uint16_t *xn, int B, int K,
                          hipStream_t stream);
// Weight-only FP8 (E4M3 codes, one fp32 scale per weight row), d_model and
// d_ff multiples of 16: VALU row kernels (ROW only, B <= kF8MaxBatch) or the
// LDS-transposed matrix-core kernels (ROW or COL, B <= 128).
constexpr int kF8MaxBatch = 8;
bool make_fp8_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus, Plan *plan);
hipError_t launch_gate_up_fp8(const Plan &p, const uint16_t *x, const uint8_t *q_gate, const float *s_gate,
                              const uint8_t *q_up, const float *s_up, float *h, hipStream_t stream);
// `partial` must hold p.partial_floats floats when that is non-zero (K cut
// into panels whose h fits in LDS, added by a second kernel).
hipError_t launch_down_fp8(const Plan &p, const float *h, const uint8_t *q_down, const float *s_down, uint16_t *y,
                           float *partial, hipStream_t stream);

// The persistent MLP: the VALU gate-up row walk, a grid barrier and the VALU
// down row walk (h in LDS) in one cooperative launch, every workgroup
// resident.  Batches up to kMlpMaxBatch, h up to kHLdsLimit bytes.
constexpr int kMlpMaxBatch = 4;
struct MlpPlan {
    int B, d_model, d_ff;
    int grid, block;
    size_t lds_bytes;
    int gu_groups, dn_groups;  // row groups of the two walks
    const void *fn;
};
bool make_mlp_plan(int B, int d_model, int d_ff, int cus, MlpPlan *plan);
// The barrier's state: kBarrierWords unsigned words, zero before the first
// launch; each launch leaves its counters at zero again.  One state per
// stream: launches that may run concurrently must not share it.
constexpr int kBarrierWords = (16 + 1 + 16) * 32;
hipError_t launch_mlp(const MlpPlan &p, const uint16_t *x, const uint16_t *w_gate, const uint16_t *w_up,
                      const uint16_t *w_down, float *h, uint16_t *y, unsigned *barrier, hipStream_t stream);
// Fixed-size scratch in static device memory for the entry point that
// allocates nothing (h and the split sums of one whole-MLP call).  Each
// device holds its own copy for the life of the process.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// The scratch's device address on device `dev`, which must be the current
// device: looked up with hipGetSymbolAddress on the first request for that
// device and cached; later requests only read the cache.
hipError_t static_scratch(int dev, void **ptr);
// The plain streaming read (dfk_stream.hip): `bytes` (a multiple of 16) of
// `buf` read once with 16-byte loads; `sink` (64 words) is written only when
// the folded words hit a fixed pattern.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, int cus, hipStream_t stream);
// `partial` must hold p.partial_floats floats when that is non-zero.
hipError_t launch_down(const Plan &p, const float *h, const uint16_t *w_down, uint16_t *y,
                       float *partial, hipStream_t stream);

}  // namespace dfk
