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
// Dynamic LDS the VALU gate-up kernel may use to keep x resident.
constexpr size_t kValuLdsLimit = 160 * 1024;

// A fully resolved launch: which kernel, how the weight matrix is cut, how
// much scratch the COL combine needs.
struct Plan {
    Op op;
    Engine engine;
    Traversal trav;
    int B;
    int rows;          // output rows: d_ff (gate-up) or d_model (down)
    int K;             // reduction length: d_model (gate-up) or d_ff (down)
    int groups;        // row groups (a wave's unit of rows)
    int splits;        // K panels (1 for ROW)
    int chunks_per_split;  // 8-element chunks per panel
    int grid;          // workgroups
    int block;         // threads per workgroup
    size_t lds_bytes;  // dynamic LDS per workgroup
    size_t partial_floats;  // COL scratch: per-panel partial sums
    size_t counters;        // COL scratch: arrival counters (one per row group)
    int kernel_id;     // index into the kernel table of the op/engine
};

// Fill a plan for the given shape, engine and traversal.  Returns false when
// the engine cannot run the shape (e.g. VALU with B above kValuMaxBatch, or x
// too large to keep in LDS).  `cus` is the device's compute-unit count.
bool make_plan(Op op, Engine engine, Traversal trav, int B, int d_model, int d_ff, int cus,
               Plan *plan);

// Enqueue the kernel of a plan.  `partial` and `counters` must hold the plan's
// scratch (counters zeroed before first use; the kernel leaves them zeroed).
hipError_t launch_gate_up(const Plan &p, const uint16_t *x, const uint16_t *w_gate,
                          const uint16_t *w_up, float *h, float *partial, unsigned *counters,
                          hipStream_t stream);
hipError_t launch_down(const Plan &p, const float *h, const uint16_t *w_down, uint16_t *y,
                       float *partial, unsigned *counters, hipStream_t stream);

}  // namespace dfk
