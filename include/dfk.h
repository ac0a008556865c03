/*
 * dfk.h -- C ABI of the fused decode-stage SwiGLU MLP library for MI355X (gfx950).
 *
 * The method ("Deep Kernel Fusion for Transformer Decoding", podcast episode
 * page, episode summary; "Deep Kernel Fusion for Transformers", hgpu.org post,
 * abstract): in the decode stage of a transformer, the SwiGLU MLP
 *     h = SiLU(x W_gate^T) * (x W_up^T),     y = h W_down^T
 * is memory-bandwidth bound.  The gate projection, the up projection, SiLU and
 * the elementwise product run as ONE kernel that streams both weight matrices
 * once; the down projection is a SEPARATE kernel; a profiler-driven scheduler
 * picks a row-major or a column-major traversal variant of each kernel.
 *
 * Conventions shared by every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Tensors are dense and row-major with no strides:
 *       x       [B, d_model]        bf16
 *       W_gate  [d_ff, d_model]     bf16   (nn.Linear layout: [out, in])
 *       W_up    [d_ff, d_model]     bf16
 *       W_down  [d_model, d_ff]     bf16
 *       h       [B, d_ff]           fp32   (SiLU(g) * u, unrounded fp32)
 *       out     [B, d_model]        bf16   (fp32 accumulation, round-to-nearest-even)
 *   - Every tensor pointer is a DEVICE pointer owned by the caller (e.g.
 *     allocated by PyTorch); the library never frees or retains it beyond the
 *     call's kernels.  Outputs must not alias inputs.  Pointers must be 16-byte
 *     aligned.
 *   - Calls are asynchronous on `stream` (0 = the null stream): they enqueue
 *     kernels and return without synchronising.  Faults inside kernels surface
 *     at the caller's next synchronisation.  The functions are thread-safe.
 *   - Arguments are validated before anything is enqueued; on any error status
 *     nothing has been launched.  No C++ exception crosses this ABI.
 *   - Limits: 1 <= B <= 256 (decode batch; larger B is prefill, not served
 *     here), d_model and d_ff positive multiples of 8 (rows are whole 16-byte
 *     vectors), d_model * d_ff < 2^31.
 *   - Inputs are assumed finite; NaN or Inf propagate through the arithmetic
 *     and are not checked.
 *   - Library-owned workspace (h between the two kernels, K-split partial
 *     sums): one buffer per (device, stream), allocated on the first call
 *     that needs it and grown (at least doubled) by a later call that needs
 *     more.  Growing never frees the earlier buffer, since work already queued
 *     or a HIP graph captured on the stream may still use it; all of a
 *     device's buffers are freed by dfk_release_workspace.  While `stream` is
 *     being captured into a graph nothing is allocated: a call that would
 *     have to grow the workspace returns DFK_ERR_UNSUPPORTED and enqueues
 *     nothing (make one eager call of the largest shape on the stream before
 *     capturing).  A graph uses the workspace of the stream it was captured
 *     on: its replays must not overlap other work of that stream.
 */
#ifndef DFK_H
#define DFK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Weight-traversal variant ("Deep Kernel Fusion for Transformer Decoding",
 * episode summary: the kernel comes in two variants, one walking the weights
 * by rows and one by columns).  Weights are
 * always stored row-major ([out, in], as nn.Linear keeps them); the layout
 * picks how a kernel walks them.  ROW: a wave or workgroup owns whole output
 * rows and walks all of K.  COL: K is split, among the waves of a workgroup or
 * across workgroups, and the partial sums are added in a fixed order.
 *   AUTO       the scheduler's choice for the shape (dfk_schedule_select)
 *   ROW, COL   that traversal; the engine is VALU below 16 batch rows, else
 *              the matrix cores (and the matrix cores when VALU cannot hold
 *              the shape).  Every variant computes the same mathematics over
 *              the same storage and differs only in fp32 summation order;
 *              all are run-to-run deterministic (no float atomics).
 *   *_VALU     that traversal on the vector ALUs (bf16 dot2 / fp32 FMA),
 *              B <= 8; DFK_ERR_UNSUPPORTED beyond what the engine holds
 *   *_MFMA     that traversal on the matrix cores (bf16 MFMA, fp32
 *              accumulation), any B <= 256
 *   ROW_PERSISTENT  dfk_swiglu_mlp only: both kernels' vector-ALU row walks
 *              in ONE cooperative launch with a grid-wide barrier between
 *              them (no launch gap; W_down starts streaming while the last
 *              gate-up rows finish; "FlashFormer: Whole-Model Kernels for
 *              Efficient Low-Batch Inference", abstract: launch overhead and
 *              bandwidth dominate at low batch).  B <= 4 and B * d_ff * 4 <= 128 KiB (h
 *              is staged in LDS), not on a stream being captured into a
 *              graph; DFK_ERR_UNSUPPORTED otherwise, and from the other entry
 *              points.  Launches on one stream share a small barrier state;
 *              a barrier that cannot complete (its workgroups not all
 *              resident) gives up after a bounded wait and writes NaN to out.
 */
typedef enum {
    DFK_LAYOUT_AUTO = 0,
    DFK_LAYOUT_ROW = 1,
    DFK_LAYOUT_COL = 2,
    DFK_LAYOUT_ROW_VALU = 3,
    DFK_LAYOUT_COL_VALU = 4,
    DFK_LAYOUT_ROW_MFMA = 5,
    DFK_LAYOUT_COL_MFMA = 6,
    DFK_LAYOUT_ROW_PERSISTENT = 7
} dfk_layout_t;

typedef enum {
    DFK_OK = 0,
    DFK_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum value */
    DFK_ERR_UNSUPPORTED = 2, /* B > 256, a dim not a multiple of 8, too large, or a forced
                                engine that cannot run the shape */
    DFK_ERR_MISALIGNED = 3,  /* a tensor pointer not 16-byte aligned */
    DFK_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
    DFK_ERR_OOM = 5          /* the library could not allocate its workspace */
} dfk_status_t;

/*
 * Fused gate + up projection + SiLU + elementwise product ("Deep Kernel Fusion
 * for Transformer Decoding", episode summary: one decode-stage kernel for the
 * up projection, the gate projection, the SiLU activation and the elementwise
 * multiply).  Computes, for b < B and n < d_ff,
 *     g = sum_k x[b,k] W_gate[n,k],  u = sum_k x[b,k] W_up[n,k],
 *     h[b,n] = g / (1 + exp(-g)) * u
 * with fp32 accumulation; h is written in fp32 (not rounded to bf16).
 * Each weight matrix is read from HBM once per call, and g and u never touch
 * HBM: they stay in registers (and LDS, where the waves of one workgroup split
 * K) until SiLU * u is written.  One launch per call; no scratch memory.
 */
dfk_status_t dfk_gate_up_silu_mul(const uint16_t *x, const uint16_t *W_gate,
                                  const uint16_t *W_up, float *h, int B, int d_model,
                                  int d_ff, dfk_layout_t layout, hipStream_t stream);

/*
 * Down projection, a separate kernel (same passage: the down projection stays
 * out of the fused kernel).  out[b,m] = RNE_bf16( sum_n h[b,n] W_down[m,n] ),
 * fp32 accumulation from the fp32 h.  Variants that split K across
 * workgroups (the vector-ALU row walk when h exceeds its LDS budget, and
 * the matrix-core column traversal) add the split sums with a second, small
 * kernel on the same stream, in split order; their scratch (splits * B *
 * d_model * 4 bytes) is the library-owned workspace (above).  The other
 * variants are one launch with no scratch memory.
 */
dfk_status_t dfk_down_proj(const float *h, const uint16_t *W_down, uint16_t *out, int B,
                           int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream);

/*
 * The whole MLP: dfk_gate_up_silu_mul then dfk_down_proj on the same stream,
 * with h in the library-owned workspace (B * d_ff * 4 bytes, plus the down
 * projection's split sums; see the conventions above).  Two launches per
 * call (three when down adds K splits).  The layout applies to both kernels; with
 * AUTO each kernel takes the scheduler's own choice.
 */
dfk_status_t dfk_swiglu_mlp(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up,
                            const uint16_t *W_down, uint16_t *out, int B, int d_model,
                            int d_ff, dfk_layout_t layout, hipStream_t stream);

/* Bytes of the static device buffer behind dfk_swiglu_mlp_noalloc (per device). */
#define DFK_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * dfk_swiglu_mlp for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results (bit for bit) as
 * dfk_swiglu_mlp with the same layout; h and the down projection's split sums
 * live in a buffer of DFK_NOALLOC_SCRATCH_BYTES that the library keeps in
 * static device memory (each device holds its own copy until the process
 * ends) instead of the growable per-stream workspace.  It never calls
 * hipMalloc, hipFree or any other allocating routine.  The first call on a
 * device looks the buffer's address up (hipGetSymbolAddress) and caches it;
 * make that first call outside a graph capture.
 *   - A call whose h (B * d_ff * 4 bytes, rounded up to 256) plus split sums
 *     exceed the buffer returns DFK_ERR_UNSUPPORTED with nothing enqueued
 *     (every Llama-3-8B and -70B layer shape fits up to B = 64).
 *   - Every call on a device shares that device's buffer, which keeps the
 *     last call's contents; nothing in it needs to start at zero.  Calls that
 *     can overlap on one device (other streams, graph replays beside eager
 *     calls) race on it: the caller must order them.
 *   - DFK_LAYOUT_ROW_PERSISTENT is DFK_ERR_UNSUPPORTED; other errors as for
 *     dfk_swiglu_mlp.
 */
dfk_status_t dfk_swiglu_mlp_noalloc(const uint16_t *x, const uint16_t *W_gate, const uint16_t *W_up,
                                    const uint16_t *W_down, uint16_t *out, int B, int d_model,
                                    int d_ff, dfk_layout_t layout, hipStream_t stream);

/*
 * How W_gate and W_up share one packed weight tensor W_gu [2 * d_ff, d_model]
 * ("Optimizing QKV Projection with Operator Fusion", "Implementing Fusion:
 * Packed Projections": projections packed into one weight read through one
 * base pointer, the same principle carried over to SwiGLU's gate and up).
 *   BLOCKED      rows [0, d_ff) are W_gate, rows [d_ff, 2 d_ff) are W_up
 *   INTERLEAVED  row 2n is W_gate's row n, row 2n + 1 is W_up's row n, so a
 *                neuron's gate and up weights are one contiguous 4 * d_model
 *                byte stream
 */
typedef enum { DFK_PACK_BLOCKED = 0, DFK_PACK_INTERLEAVED = 1 } dfk_packing_t;

/*
 * dfk_gate_up_silu_mul with W_gate and W_up packed in W_gu (device, bf16,
 * [2 * d_ff, d_model], layout per `packing`).  Same kernels, same results bit
 * for bit as passing the two halves separately; only the weights' addresses
 * differ.  A bad `packing` value is DFK_ERR_INVALID_ARG.
 */
dfk_status_t dfk_gate_up_silu_mul_packed(const uint16_t *x, const uint16_t *W_gu, float *h, int B,
                                         int d_model, int d_ff, dfk_packing_t packing,
                                         dfk_layout_t layout, hipStream_t stream);

/*
 * dfk_swiglu_mlp with W_gate and W_up packed in W_gu (as above); W_down is
 * separate.  DFK_LAYOUT_ROW_PERSISTENT takes the blocked packing only
 * (DFK_ERR_UNSUPPORTED for the interleaved one).
 */
dfk_status_t dfk_swiglu_mlp_packed(const uint16_t *x, const uint16_t *W_gu, const uint16_t *W_down,
                                   uint16_t *out, int B, int d_model, int d_ff,
                                   dfk_packing_t packing, dfk_layout_t layout, hipStream_t stream);

/*
 * Weight-only FP8 weights, dequantized inside the kernels (GPULlama3.java
 * pull request "[FP16] ... fusing dequantize with compute", PR summary:
 * quantized weights are dequantized inside the matrix-vector product and
 * never written back dequantized).  The page fixes no format; here a weight
 * matrix W [rows, cols] is stored as
 *     Wq  [rows, cols]  uint8  OCP FP8 E4M3 codes (bias 7, 3 fraction bits,
 *                              subnormals, no infinities, S.1111.111 = NaN)
 *     s   [rows]        fp32   one scale per row (output channel)
 * standing for W[r, c] = s[r] * e4m3(Wq[r, c]).  The codes stream from HBM at
 * half the bytes of bf16 and are widened in registers; each row's fp32 sum is
 * multiplied by its scale once.  The computed h and out are those of the bf16
 * entry points over the dequantized weights (to fp32 summation order).
 * Engines: the vector-ALU row walk (B <= 8; x kept in LDS, so
 * B * d_model * 2 <= 160 KiB), for the down projection also a vector-ALU
 * column walk with h held in registers (B <= 4, d_ff small enough that a
 * lane's share of h fits: 16 * B fp32 per 16-byte chunk, at most 64), and
 * the matrix-core kernels (B <= 128),
 * which widen the codes to bf16 exactly: on their way into LDS, or in
 * registers (the down projection's column traversal).  Layouts:
 * AUTO = the tuning table's FP8 entry for the shape (see
 * dfk_schedule_select), else the measured best at the Llama-3-8B layer shape
 * (gate-up: vector ALU to B = 3, matrix-core column traversal to B = 16, row
 * traversal above; down: vector ALU to B = 2, matrix-core column traversal
 * above); ROW = vector ALU up to B = 8, else matrix cores; COL = matrix
 * cores; ROW_VALU, ROW_MFMA, COL_MFMA force the engine; COL_VALU forces
 * the down column walk (DFK_ERR_UNSUPPORTED for gate-up, and where h does
 * not fit); ROW_PERSISTENT is DFK_ERR_UNSUPPORTED.  d_model and d_ff must be
 * multiples of 16.  Code and tensor pointers must be 16-byte aligned, scale
 * pointers 4-byte aligned.
 */
dfk_status_t dfk_gate_up_silu_mul_fp8(const uint16_t *x, const uint8_t *Wq_gate, const float *s_gate,
                                      const uint8_t *Wq_up, const float *s_up, float *h, int B,
                                      int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream);

/* The down projection over FP8 W_down ([d_model, d_ff] codes, [d_model]
 * scales); as dfk_down_proj otherwise. */
dfk_status_t dfk_down_proj_fp8(const float *h, const uint8_t *Wq_down, const float *s_down,
                               uint16_t *out, int B, int d_model, int d_ff, dfk_layout_t layout,
                               hipStream_t stream);

/* The whole MLP over FP8 weights: the two kernels above on one stream, h in
 * the library-owned workspace of dfk_swiglu_mlp. */
dfk_status_t dfk_swiglu_mlp_fp8(const uint16_t *x, const uint8_t *Wq_gate, const float *s_gate,
                                const uint8_t *Wq_up, const float *s_up, const uint8_t *Wq_down,
                                const float *s_down, uint16_t *out, int B, int d_model, int d_ff,
                                dfk_layout_t layout, hipStream_t stream);

/*
 * RMS normalization of the MLP input (GPULlama3.java pull request "[FP16] ...
 * fusing dequantize with compute", commit list: RMS normalization fused with
 * the gate and up projections; the page does not define the normalization,
 * so this is Llama's RMSNorm).  For each batch row b,
 *     inv_b = 1 / sqrt( (sum_k x[b,k]^2) / d_model + eps ),
 *     xn[b,k] = RNE_bf16( (x[b,k] * inv_b) * gain[k] ),
 * all in fp64 and rounded once, fp64 -> bf16, ties to even.
 *   x     [B, d_model]  bf16 device    gain [d_model] bf16 device
 *   xn    [B, d_model]  bf16 device output (must not alias x)
 *   eps   >= 0 and finite, else DFK_ERR_INVALID_ARG (eps = 0 with an all-zero
 *         row gives NaN, as the formula does)
 * One launch (one workgroup per batch row), no scratch memory.  B and d_model
 * follow the limits above.
 */
dfk_status_t dfk_rmsnorm(const uint16_t *x, const uint16_t *gain, double eps, uint16_t *xn, int B,
                         int d_model, hipStream_t stream);

/*
 * dfk_rmsnorm then dfk_gate_up_silu_mul, with the normalization fused into
 * gate-up where that kernel stages x in LDS (the vector-ALU variants: each
 * workgroup normalizes its copy of x there, one launch, no scratch).  The
 * matrix-core variants run dfk_rmsnorm into a library-owned bf16 buffer
 * (B * d_model * 2 bytes, per (device, stream)) and then their usual kernel.
 * Either way h is bit for bit what dfk_rmsnorm followed by
 * dfk_gate_up_silu_mul with the same plan gives.  The layout picks the
 * gate-up variant as for dfk_gate_up_silu_mul.
 */
dfk_status_t dfk_rmsnorm_gate_up_silu_mul(const uint16_t *x, const uint16_t *gain, double eps,
                                          const uint16_t *W_gate, const uint16_t *W_up, float *h, int B,
                                          int d_model, int d_ff, dfk_layout_t layout, hipStream_t stream);

/*
 * The whole MLP on RMS-normalized input: dfk_rmsnorm_gate_up_silu_mul then
 * dfk_down_proj on the same stream, h (and, for matrix-core gate-up plans,
 * the normalized x) in the library-owned workspace of dfk_swiglu_mlp.
 */
dfk_status_t dfk_rmsnorm_swiglu_mlp(const uint16_t *x, const uint16_t *gain, double eps,
                                    const uint16_t *W_gate, const uint16_t *W_up, const uint16_t *W_down,
                                    uint16_t *out, int B, int d_model, int d_ff, dfk_layout_t layout,
                                    hipStream_t stream);

/*
 * Profiler-driven variant choice ("Deep Kernel Fusion for Transformer
 * Decoding", episode summary: profiling decides, while serving, which of the
 * row- and column-walking kernel variants runs; "Deep Kernel Fusion for
 * Transformers", abstract: a kernel scheduler).  Host only; never touches the device.
 * Looks the shape up in the tuning table (the file named by the environment
 * variable DFK_TUNING_TABLE, else the table installed beside the library):
 * exact (B, d_model, d_ff) entry, else the entry for the same (d_model, d_ff)
 * with the nearest tuned batch at or above B (else the largest below), else
 * a built-in heuristic.  Writes explicit variants (never AUTO) to both
 * outputs.  DFK_FORCE_LAYOUT=row|col overrides the traversal.  The table
 * records the library and HIP versions it was tuned for; a table for other
 * versions (or a missing or malformed one) is not used: the heuristic serves
 * and dfk_tuning_table_source says why.  The same table holds the FP8 entry
 * points' choices (ops gate_up_fp8, down_fp8), which their AUTO layout reads.
 */
dfk_status_t dfk_schedule_select(int B, int d_model, int d_ff, dfk_layout_t *gate_up_layout,
                                 dfk_layout_t *down_layout);

/* Static, human-readable name of a status code (never NULL). */
const char *dfk_status_string(dfk_status_t s);

/* Static name of a layout value, e.g. "row_valu" (never NULL). */
const char *dfk_layout_name(dfk_layout_t layout);

/* Library version string, e.g. "dfk 0.2.0 gfx950 (HIP 7.2.26015)". */
const char *dfk_version(void);

/*
 * Reload the tuning table from `path` (NULL: the default location).  Returns
 * DFK_OK when a table was loaded, DFK_ERR_INVALID_ARG when the file is
 * missing, malformed or tuned for another library or HIP version (the
 * scheduler then uses its heuristic).  Host only.
 */
dfk_status_t dfk_load_tuning_table(const char *path);

/*
 * Where the scheduler's current table came from: the path of the loaded file,
 * "heuristic" when none is loaded, or "heuristic (table PATH tuned for ...)"
 * when the table was for other versions.  Static storage, valid until the next
 * dfk_load_tuning_table call.
 */
const char *dfk_tuning_table_source(void);

/*
 * Measurement helper, not part of the MLP: read `bytes` (a positive multiple
 * of 16) of the device buffer `buf` once, on `stream`, with the access shape
 * of the vector-ALU weight walk: 16-byte non-temporal loads, 1 KiB per wave
 * load, each wave walking two contiguous segments (in the two halves of the
 * buffer) with four loads in flight on each.  It gives the
 * practical HBM read ceiling the kernels are compared with.  `sink` is a
 * device array of 64 uint32_t that the kernel may write (only when the folded
 * words hit a fixed pattern).  Errors: null pointers or bytes = 0
 * DFK_ERR_INVALID_ARG, bytes not a multiple of 16 DFK_ERR_UNSUPPORTED, buf not
 * 16-byte or sink not 4-byte aligned DFK_ERR_MISALIGNED.
 */
dfk_status_t dfk_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/*
 * Free every workspace buffer the library holds for the current device (the
 * current ones and those retired by growth), after waiting for the device.
 * HIP graphs captured against them must not be replayed afterwards; later
 * calls allocate afresh.  Without this call the buffers are held until the
 * process ends.
 */
dfk_status_t dfk_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* DFK_H */
