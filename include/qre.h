/*
 * qre.h — C ABI of the MI355X (gfx950) routed-expert MoE feed-forward with
 * group-quantized expert weights.
 *
 * The operation is the routed-expert feed-forward of a block-diffusion LLM
 * server ("coder543/minnow" README, opening paragraphs and section
 * "Quantization"; "LLaDA2.2-flash for minnow" model card, section "Checkpoints
 * and precision" and its precision table):
 *
 *   for every token t and each of its K routed experts e = topk_ids[t][k]:
 *       g = W_gate[e] x_t,  u = W_up[e] x_t          (gate/up projections, I outputs)
 *       h = bf16( silu(g) * u )                      (fused gate/up/SiLU)
 *       y = bf16( W_down[e] h )                      (down projection, H outputs)
 *   out_t = bf16( sum_k topk_w[t][k] * y_{t,k} )     (FP32, k ascending, one FMA per term)
 *
 * Weights are signed INT4 or INT8 with one FP16 scale per 128 consecutive
 * weights along each projection's input (reduction) dimension; w = s * q.
 * Activations are BF16 (W4A16 / W8A16), or, with act_int8, the expert inputs x
 * and h are quantized per 128 values to signed INT8 with an FP32 scale
 * s = max|v| / 127, group dot products are exact INT32 sums and the scaled
 * groups are combined in FP32 (model card, paragraph on
 * --int8-expert-activations).  Expert outputs return to BF16.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller unless the
 *    comment says "host".  The library never allocates, frees or retains
 *    memory, keeps no mutable global state (only a per-thread copy of the
 *    last HIP error code, see qre_last_hip_error), and may be called from
 *    several threads on different streams.
 *  - Work is enqueued on `stream` and the call returns without synchronizing,
 *    except qre_read_device_error, which synchronizes `stream`.
 *  - Arguments are validated on the host before anything is enqueued.  On any
 *    error code nothing has been enqueued.  A problem with zero tokens is valid
 *    and enqueues nothing (qre_route still writes its per-expert outputs).
 *  - Device pointers must be 16-byte aligned (QRE_ERR_ALIGN otherwise).
 *  - A routed expert id outside [0, E) drops that slot: it contributes zero to
 *    the output and is counted (see qre_read_device_error).  Duplicate ids
 *    within a token are legal; each slot is computed and summed.
 *  - Non-finite inputs give unspecified (but memory-safe) results.
 *
 * Layouts (row-major, C order)
 *    x                 bf16  [T][H]
 *    topk_ids          int32 [T][K]     slot s = t*K + k
 *    topk_w            fp32  [T][K]
 *    out               bf16  [T][H]
 *    gate_q, up_q      bytes [E][I][H*bits/8]   INT8: one code per byte;
 *    down_q            bytes [E][H][I*bits/8]   INT4: element 2j in the low
 *                                               nibble of byte j, 2j+1 in the
 *                                               high nibble, two's complement
 *    gate_s, up_s      fp16  [E][I][H/128]
 *    down_s            fp16  [E][H][I/128]
 */
#ifndef QRE_H
#define QRE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t.  Declared through its underlying struct so that this header
 * needs no HIP include; pass NULL for the null stream. */
struct ihipStream_t;
typedef struct ihipStream_t* qre_stream_t;

/* Status codes.  Every entry point returns one. */
#define QRE_OK             0
#define QRE_ERR_NULL      -1  /* a required pointer is NULL */
#define QRE_ERR_SHAPE     -2  /* a size is negative, zero where it may not be, or not a multiple of 128 */
#define QRE_ERR_BITS      -3  /* weight_bits is not 4 or 8 */
#define QRE_ERR_GROUP     -4  /* group_size is not 128 */
#define QRE_ERR_ALIGN     -5  /* a device pointer is not 16-byte aligned */
#define QRE_ERR_WORKSPACE -6  /* workspace too small */
#define QRE_ERR_HIP       -7  /* a HIP launch or call failed (see qre_last_hip_error) */
#define QRE_ERR_MODE      -8  /* act_int8 is not 0 or 1, or an argument required by the mode is missing */
#define QRE_ERR_LIMIT     -9  /* a size exceeds a library limit (E > QRE_MAX_EXPERTS, T*K >= 2^31, ...) */

#define QRE_GROUP 128
#define QRE_MAX_EXPERTS 512

/* Problem descriptor (host memory). */
typedef struct qre_desc {
  int32_t T;            /* tokens, >= 0 */
  int32_t H;            /* hidden size, multiple of 128 */
  int32_t I;            /* expert intermediate size, multiple of 128 */
  int32_t E;            /* routed experts, 1..QRE_MAX_EXPERTS */
  int32_t K;            /* experts per token, 1..E */
  int32_t weight_bits;  /* 4 or 8: signed symmetric codes, no zero-point */
  int32_t group_size;   /* must be 128 */
  int32_t act_int8;     /* 0: BF16 activations; 1: INT8 activations, FP32 scale per 128 */
} qre_desc;

/* Packed expert weights (device pointers, layouts above). */
typedef struct qre_weights {
  const void* gate_q; const void* gate_s;
  const void* up_q;   const void* up_s;
  const void* down_q; const void* down_s;
} qre_weights;

/* Bytes of device workspace qre_moe_forward needs for `desc` (host out): the
 * routing permutation, the GEMM row-tile lists, the intermediate h (BF16
 * [T*K][I]) and y (BF16 [T*K][H]) in sorted-row order, and in INT8 mode the
 * INT8 codes and FP32 scales of x and h (model card, paragraph on
 * --int8-expert-activations).  QRE_ERR_* for an invalid descriptor. */
int qre_workspace_bytes(const qre_desc* desc, size_t* bytes);

/* The whole routed-expert feed-forward (minnow README, "Quantization": fused
 * gate/up/SiLU kernels, GPU routing of decode blocks; model card,
 * "Checkpoints and precision"): x, topk_ids, topk_w, weights -> out.
 * Runs the permutation, the INT8 activation quantizer (act_int8 only), the
 * fused gate/up/SiLU grouped GEMM, the down grouped GEMM and the combine.  For
 * up to 2048 slots with the usual expert shapes the permutation is computed
 * inside the gate/up kernel (each expert's workgroups find that expert's slots)
 * instead of by a separate launch; the results are the same.
 * `workspace` (>= qre_workspace_bytes) holds the permutation, h and y; after
 * the call it also holds what qre_read_device_error reads. */
int qre_moe_forward(const qre_desc* desc, const void* x, const int32_t* topk_ids,
                    const float* topk_w, const qre_weights* weights, void* out,
                    void* workspace, size_t workspace_bytes, qre_stream_t stream);

/* qre_moe_forward for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a device array of QRE_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, created when the library is loaded and held until
 * the process ends; this call allocates nothing.  Problems whose workspace
 * (qre_workspace_bytes) exceeds that size are rejected with QRE_ERR_LIMIT
 * (decode blocks and batched blocks at H = 2048 fit; prefill-sized ones do
 * not).  All calls on one GPU share its array: calls that overlap in time on
 * one GPU (different streams, different threads) race and give undefined
 * results; calls ordered on one stream are fine.  The workspace needs no
 * clearing (every call writes what it reads), and after the call it holds
 * what qre_read_device_error would read from a caller's workspace. */
#define QRE_NOALLOC_SCRATCH_BYTES (32u << 20)
int qre_moe_forward_noalloc(const qre_desc* desc, const void* x, const int32_t* topk_ids,
                            const float* topk_w, const qre_weights* weights, void* out,
                            qre_stream_t stream);

/* qre_moe_forward that also records events[i] (host array of eight, each a
 * hipEvent_t created by the caller, or NULL to skip it) on `stream` between
 * its steps: [0] before the permutation, [1] before the gate/up GEMM, [2]
 * after it, [3] before the down GEMM, [4] after it, [5] after the combine;
 * [6] and [7] are handed to the launch of the gate/up GEMM kernel itself
 * (hipExtLaunchKernelGGL), so they hold that dispatch's own begin and end,
 * the interval a kernel trace reports, without the cost of an event record
 * in between.  The kernels are the same as qre_moe_forward's; this is a
 * measurement aid. */
int qre_moe_forward_timed(const qre_desc* desc, const void* x, const int32_t* topk_ids,
                          const float* topk_w, const qre_weights* weights, void* out,
                          void* workspace, size_t workspace_bytes, void* const* events,
                          qre_stream_t stream);

/* Number of slots whose expert id was outside [0, E) (host out) in the last
 * routing that used `workspace`: a qre_moe_forward or qre_route workspace
 * (every workspace starts with this counter).  Such a slot is a precondition
 * violation of the caller; it is dropped (contributes zero) and counted.
 * Synchronizes `stream`, so the count is that of the last call enqueued. */
int qre_read_device_error(const void* workspace, int32_t* n_bad_ids, qre_stream_t stream);

/* Device addresses, inside a qre_moe_forward workspace, of the permutation the
 * last call computed (layouts of qre_route; host out).  Reading them after
 * the call has finished gives the same arrays qre_route would produce. */
int qre_workspace_permutation(const qre_desc* desc, void* workspace, int32_t** counts,
                              int32_t** offsets, int32_t** sorted_slot, int32_t** slot_row);

/* ---- Stage entry points (same conventions).  They compute exactly what the
 * corresponding step of qre_moe_forward computes, with the same kernels. ---- */

/* Token->expert permutation: a stable counting sort of the S = T*K slots by
 * expert id (minnow README, "Quantization": GPU routing of decode blocks).
 *   counts[E]        slots per expert
 *   offsets[E+1]     exclusive prefix sum of counts; offsets[E] = valid slots
 *   sorted_slot[S]   sorted_slot[offsets[e] + j] = j-th smallest slot with id e;
 *                    entries at and past offsets[E] are -1
 *   slot_row[S]      position of slot s in sorted_slot, or -1 if dropped
 * Bit-exact and deterministic (no atomics decide any order).  `workspace`
 * (>= qre_route_workspace_bytes, 16-byte aligned) holds the routing scratch
 * and the dropped-slot counter of qre_read_device_error.  counts and offsets
 * are written even when T == 0. */
int qre_route_workspace_bytes(int32_t T, int32_t K, int32_t E, size_t* bytes);
int qre_route(const int32_t* topk_ids, int32_t T, int32_t K, int32_t E, int32_t* counts,
              int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row, void* workspace,
              size_t workspace_bytes, qre_stream_t stream);

/* Per-row, per-128 INT8 quantizer (model card, --int8-expert-activations):
 * s = max|v| / 127 in FP32 (IEEE division), q = clamp(rint(v / s), -127, 127),
 * ties to even; an all-zero group gives s = 0, q = 0.
 *   v bf16 [rows][cols], q int8 [rows][cols], s fp32 [rows][cols/128]; cols % 128 == 0. */
int qre_quantize_act(const void* v, int32_t rows, int32_t cols, int8_t* q, float* s,
                     qre_stream_t stream);

/* Fused gate/up projection and SiLU*mul for every valid sorted row r
 * (expert e with offsets[e] <= r < offsets[e+1], token t = sorted_slot[r] / K)
 * (minnow README, "Quantization": fused gate/up/SiLU; model card, "Checkpoints
 * and precision": gate and up projections, weights dequantized to BF16 in
 * registers, INT32 group dot products combined in FP32 with INT8 activations):
 *   h[r][i] = bf16( silu(g) * u ),  g = sum_h x[t][h] Wg[e][i][h],  u likewise.
 * BF16 mode reads x (bf16 [T][H]); INT8 mode reads xq (int8 [T][H]) and xs
 * (fp32 [T][H/128]), combines INT32 group sums in FP32, and, when hq and hs
 * are given, also writes h quantized per 128 values (the input of the INT8
 * down projection): hq int8 [T*K][I], hs fp32 [T*K][I/128], exactly what
 * qre_quantize_act gives for h (with INT8 weights and 64 or more rows per
 * expert the gate/up kernel quantizes h in its epilogue; otherwise the
 * quantizer runs on h after it).  h: bf16 [T*K][I], optional in INT8 mode
 * when hq/hs are given.  Rows past offsets[E] are not written.  sorted_slot
 * and offsets are qre_route's outputs (or any stable permutation in the same
 * form).  `workspace` (>= qre_stage_workspace_bytes) receives the row-tile
 * list built from offsets.  QRE_ERR_MODE if an input of the mode is missing,
 * or hq/hs are given in BF16 mode. */
int qre_gate_up(const qre_desc* desc, const void* x, const int8_t* xq, const float* xs,
                const int32_t* sorted_slot, const int32_t* offsets, const qre_weights* weights,
                void* h, int8_t* hq, float* hs, void* workspace, size_t workspace_bytes,
                qre_stream_t stream);

/* Down projection for every valid sorted row r (model card, "Checkpoints and
 * precision": down projection of the routed experts; expert outputs return to
 * BF16): y[r][j] = bf16( sum_i h[r][i] Wd[e][j][i] ).  BF16 mode reads h
 * (bf16 [T*K][I]); INT8 mode reads hq (int8 [T*K][I]) and hs
 * (fp32 [T*K][I/128]).  y: bf16 [T*K][H].  offsets and `workspace` as for
 * qre_gate_up. */
int qre_down(const qre_desc* desc, const void* h, const int8_t* hq, const float* hs,
             const int32_t* offsets, const qre_weights* weights, void* y, void* workspace,
             size_t workspace_bytes, qre_stream_t stream);

/* Workspace bytes qre_gate_up and qre_down need for `desc` (the row-tile
 * lists, and in INT8 mode room for h when only hq/hs are asked for). */
int qre_stage_workspace_bytes(const qre_desc* desc, size_t* bytes);

/* Per-token combine (the top-k weighted sum of the routed experts' outputs;
 * the order, k ascending with one FMA per term, is this library's reading,
 * which makes the result deterministic): out[t][j] = bf16( fma chain over k ascending of
 * topk_w[t][k] * y[slot_row[t*K+k]][j] ) in FP32, starting from 0; a slot with
 * slot_row = -1 is skipped.  y bf16 [T*K][H] in sorted-row order. */
int qre_combine(const void* y, const int32_t* slot_row, const float* topk_w, int32_t T, int32_t K,
                int32_t H, void* out, qre_stream_t stream);

/* Router ahead of the permutation (minnow README, "Quantization": routing of
 * decode blocks runs on the GPU; LLaDA2.2-flash model card, "Checkpoints and
 * precision": routers keep floating-point weights).  The rule is the plain
 * top-K softmax: for each token t, topk_ids[t][0..K) are the K experts with
 * the largest logits[t][e], in descending order of logit, equal logits going
 * to the lower id; topk_w[t][k] = exp(l_k - l_0) / sum_j exp(l_j - l_0) over
 * the K selected logits, in FP32 (expf, a fixed-order sum, IEEE division).
 * logits fp32 [T][E], topk_ids int32 [T][K], topk_w fp32 [T][K], all device
 * memory owned by the caller; the outputs are exactly what qre_moe_forward
 * takes.  1 <= K <= E (QRE_ERR_SHAPE), E <= QRE_ROUTER_MAX_EXPERTS and
 * K <= QRE_ROUTER_MAX_K (QRE_ERR_LIMIT); T == 0 is a no-op.  -0 and +0 count
 * as equal; NaN or infinite logits give unspecified results (ids stay in
 * [0, E) and distinct). */
#define QRE_ROUTER_MAX_EXPERTS 1024
#define QRE_ROUTER_MAX_K 64
int qre_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t K, int32_t* topk_ids, float* topk_w,
                     qre_stream_t stream);

/* Weight conversion (minnow README, "Quantization": convert --experts
 * int4|int8): w fp32 [rows][cols] -> q [rows][cols*bits/8] bytes in the packed
 * layout above and s fp16 [rows][cols/128] with s = fp16(max|w| / qmax),
 * qmax = 7 (INT4) or 127 (INT8), q = clamp(rint(w / s), -8|-127, 7|127) using
 * the stored FP16 scale; an all-zero group (or one whose scale rounds to 0)
 * stores s = 0 and q = 0.  cols % 128 == 0. */
int qre_quantize_weights(const float* w, int64_t rows, int64_t cols, int32_t bits, void* q,
                         void* s, qre_stream_t stream);

/* Measurement aid: what qre_moe_forward launches for `desc` (host out, a bit
 * mask).  QRE_PLAN_ROUTE_IN_GATE_UP: the permutation is computed inside the
 * gate/up kernel (no routing launch).  QRE_PLAN_COMBINE_IN_DOWN: the combine
 * runs inside the down kernel (no combine launch).  QRE_PLAN_BIG_TILES:
 * the big-tile MFMA kernels for the gate/up GEMM (64 or more slots per expert
 * and a hidden size of at most 8192: 64-row tiles with BF16 activations,
 * 128-row tiles with INT8 activations). */
#define QRE_PLAN_ROUTE_IN_GATE_UP 1
#define QRE_PLAN_COMBINE_IN_DOWN 2
#define QRE_PLAN_BIG_TILES 4
int qre_forward_plan(const qre_desc* desc, int32_t* plan);

/* Measurement aid: a streaming read of `bytes` (a nonzero multiple of 16) of
 * device memory `buf`, folded into words stored to `sink` (device, at least
 * 4096 bytes).  Its duration gives the HBM read bandwidth the memory-bound
 * kernels are compared with, next to the published peak. */
int qre_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, qre_stream_t stream);

/* ------------------------------------------------------------------------
 * NVFP4 (W4A4) experts (model card "LLaDA2.2-flash for minnow", precision
 * table, NVFP4 row; README "Quantization": FP32 accumulation; model card,
 * paragraph after the table: without native FP4 tensor cores the already
 * quantized FP4 operands are rebuilt for 16-bit matrix cores and the input
 * quantization is kept).  The feed-forward is the one above with:
 *   - weights: E2M1 codes, an E4M3 scale per 16 consecutive weights along the
 *     reduction dimension and an FP32 outer scale per expert matrix;
 *     w = e2m1(c) * e4m3(b) * outer;
 *   - expert inputs x (gate/up) and h (down), BF16, quantized per row to E2M1
 *     with an E4M3 scale per 16 values and an FP32 outer scale per row;
 *   - dot products of the dequantized values accumulated in FP32; h and y
 *     materialized in BF16.
 * Quantizer (a reading; the pages give the format only): outer
 * S = max|v| / 2688 (FP32; 2688 = 6 * 448), block scale b = E4M3 of
 * max|block| / (S * 6), code = E2M1 of v / (e4m3(b) * S), every product and
 * quotient rounded to FP32 first, both roundings to nearest-even and
 * saturating (E4M3 at 448, E2M1 at 6), a zero magnitude stored as code 0,
 * S = 0 giving all-zero codes and scales.  Finite inputs only.
 *
 * Layouts (row-major; a row is one output feature or one input row)
 *    codes q           bytes [rows][cols/2]   element 2j in the low nibble of
 *                                             byte j, 2j+1 in the high nibble;
 *                                             E2M1: bit 3 sign, bits 2:1
 *                                             exponent (bias 1), bit 0 mantissa
 *    block scales s    bytes [rows][cols/16]  E4M3 (bias 7, max 448, no inf)
 *    weights           gate, up [E][I][H] and down [E][H][I] as above, one
 *                      FP32 outer scale per expert matrix: outer [E]
 *    quantized inputs  x: [T][H] codes/scales + fp32 [T];
 *                      h: [T*K][I] codes/scales + fp32 [T*K] (sorted rows)
 * A descriptor selects NVFP4 with weight_bits = 4, group_size =
 * QRE_NVFP4_BLOCK and act_int8 = 0 (QRE_ERR_BITS / QRE_ERR_GROUP /
 * QRE_ERR_MODE otherwise); H and I must be multiples of 128 (QRE_ERR_SHAPE);
 * the GEMMs stage up to 16 rows of x in LDS as FP16, which bounds H (4992
 * when T*K > 4E, 10112 otherwise; QRE_ERR_LIMIT beyond).  The shared
 * conventions above hold, except that the FP32 outer scales (read one value
 * at a time) need only 4-byte alignment.
 * ------------------------------------------------------------------------ */
#define QRE_NVFP4_BLOCK 16

typedef struct qre_nvfp4_matrix {
  const void* q;        /* codes [E][rows][cols/2] */
  const void* s;        /* E4M3 block scales [E][rows][cols/16] */
  const float* outer;   /* FP32 [E] */
} qre_nvfp4_matrix;

typedef struct qre_nvfp4_weights {
  qre_nvfp4_matrix gate, up, down;
} qre_nvfp4_weights;

/* Quantize `mats` float32 matrices w [mats][rows][cols] (cols % 16 == 0) to
 * codes q [mats][rows][cols/2], block scales s [mats][rows][cols/16] and one
 * outer scale per matrix, outer [mats] (which also serves as the kernels'
 * scratch for the matrices' maxima).  Load-time utility. */
int qre_nvfp4_quantize_weights(const float* w, int64_t mats, int64_t rows, int64_t cols, void* q, void* s,
                               float* outer, qre_stream_t stream);

/* Quantize BF16 rows v [rows][cols] (cols % 16 == 0) to codes q
 * [rows][cols/2], block scales s [rows][cols/16] and row_scale [rows]. */
int qre_nvfp4_quantize_act(const void* v, int32_t rows, int32_t cols, void* q, void* s, float* row_scale,
                           qre_stream_t stream);

/* Bytes of device workspace qre_nvfp4_moe_forward needs: the permutation,
 * the row-tile lists, the quantized x, h (BF16 [T*K][I]) and its quantized
 * form, y (BF16 [T*K][H]). */
int qre_nvfp4_workspace_bytes(const qre_desc* desc, size_t* bytes);

/* The whole NVFP4 feed-forward: routing permutation, quantization of x, fused
 * gate/up/SiLU GEMM, quantization of h, down GEMM, combine (same contract and
 * out layout as qre_moe_forward).  After the call the workspace also holds
 * what qre_read_device_error reads and what
 * qre_nvfp4_workspace_permutation points into. */
int qre_nvfp4_moe_forward(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                          const qre_nvfp4_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                          qre_stream_t stream);

/* Measurement aid: qre_nvfp4_moe_forward that also records caller-created
 * hipEvent_t (events[0..7], host array of eight; NULL entries skipped) on
 * `stream`: [0..5] before the routing, after the routing and the quantization
 * of x, after gate/up, after the quantization of h, after down, after the
 * combine; [6] and [7] the begin and end of the gate/up GEMM dispatch itself
 * (as for qre_moe_forward_timed). */
int qre_nvfp4_moe_forward_timed(const qre_desc* desc, const void* x, const int32_t* topk_ids, const float* topk_w,
                                const qre_nvfp4_weights* weights, void* out, void* workspace, size_t workspace_bytes,
                                void* const* events, qre_stream_t stream);

/* Device pointers into an NVFP4 forward workspace (host out): the
 * permutation of the last qre_nvfp4_moe_forward that used it. */
int qre_nvfp4_workspace_permutation(const qre_desc* desc, void* workspace, int32_t** counts, int32_t** offsets,
                                    int32_t** sorted_slot, int32_t** slot_row);

/* Workspace of the NVFP4 stage calls below (row-tile lists). */
int qre_nvfp4_stage_workspace_bytes(const qre_desc* desc, size_t* bytes);

/* NVFP4 gate/up stage: from x quantized by qre_nvfp4_quantize_act (xq codes,
 * xs block scales, xr row scales; [T] rows) and the permutation of qre_route
 * (sorted_slot, offsets), h [T*K][I] BF16 by sorted row; rows past
 * offsets[E] are not written. */
int qre_nvfp4_gate_up(const qre_desc* desc, const void* xq, const void* xs, const float* xr, const int32_t* sorted_slot,
                      const int32_t* offsets, const qre_nvfp4_weights* weights, void* h, void* workspace,
                      size_t workspace_bytes, qre_stream_t stream);

/* NVFP4 down stage: from h quantized per sorted row (hq, hs, hr; [T*K] rows),
 * y [T*K][H] BF16 by sorted row. */
int qre_nvfp4_down(const qre_desc* desc, const void* hq, const void* hs, const float* hr, const int32_t* offsets,
                   const qre_nvfp4_weights* weights, void* y, void* workspace, size_t workspace_bytes,
                   qre_stream_t stream);

/* Human-readable name of a status code (static string). */
const char* qre_status_string(int status);

/* The HIP error code behind the last QRE_ERR_HIP on this thread (0 if none). */
int qre_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QRE_H */
