/*
 * pc.h -- C ABI of the MI355X (gfx950) probabilistic-circuit sum-layer library.
 *
 * The library evaluates circuits made of categorical input layers, product
 * layers and log-space sum layers, and their backward pass (element flows and
 * parameter flows) and EM update, with hand-written HIP kernels.  The sum
 * layer is the one of the PyJuice pull request #62 ("precision option for the
 * sum layers"), Summary item 2: children are exponentiated against their
 * per-sample maximum, multiplied by the weights, and the log is taken:
 *
 *     v[i,b] = m[b] + log( sum_j theta[i,j] * exp(v[j,b] - m[b]) ),
 *     m[b]   = max over the group's children j of v[j,b]        (Tests section:
 *                                               "per-group column maximum").
 *
 * Conventions used by every call
 *  - All float buffers are IEEE float32.  Node values and node flows are
 *    node-major: entry (node n, sample b) lives at [n * batch + b].
 *  - "device pointer" = memory of the HIP device the handle was compiled for,
 *    owned by the caller (for example a torch tensor); the library never frees
 *    or keeps it beyond the call.
 *  - `stream` is a hipStream_t (0 = the null stream).  Device work is
 *    enqueued on it and the call returns without synchronising; the library
 *    allocates no device memory inside pc_forward / pc_backward / pc_em_step /
 *    pc_em_step_corrected: every scratch byte comes from the caller's
 *    workspace.  (With parameter-flow chunks, PC_OPT_PARAM_CHUNK, the first
 *    pc_backward of a handle creates the handle's second stream and events;
 *    pc_backward joins that stream into `stream` before it returns.)
 *  - Return value: PC_OK or a PC_ERR_* code; pc_last_error() gives a message
 *    for the calling thread.  A failed call enqueues no device work.
 *  - Calls on one handle must not overlap in time (they share the handle's
 *    state); different handles are independent.
 */
#ifndef PC_H_
#define PC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PC_OK               0
#define PC_ERR_INVALID_ARG  1   /* malformed descriptor, null pointer, bad size or mode */
#define PC_ERR_UNSUPPORTED  2   /* well formed but not provided (see each call) */
#define PC_ERR_WORKSPACE    3   /* workspace smaller than pc_workspace_bytes() */
#define PC_ERR_HIP          4   /* a HIP runtime call failed (message names it) */
#define PC_ERR_NO_DEVICE    5   /* handle compiled without a device (device < 0) */

/* ---- precision modes (PyJuice pull request #62, Summary item 1) ---------
 * PC_PREC_AUTO: sum-layer products from bfloat16 operands (round to nearest
 *   even) with float32 accumulation -- the counterpart of the page's "auto"
 *   mode, whose forward uses bf16 products; each product splits one of its
 *   operands into hi + lo planes (see pc_set_split).
 * PC_PREC_FP32: fp32-level products: each float32 operand is split into
 *   bfloat16 planes (hi, lo: x ~ hi + lo) and the cross products up to the
 *   second order are accumulated in float32 -- the counterpart of the page's
 *   three-pass "tf32x3" fp32 mode, built from bf16 matrix cores.
 * PC_PREC_TF32: the page's "tf32" mode.  gfx950 has no TF32/XF32 matrix
 *   instruction, so this mode returns PC_ERR_UNSUPPORTED.
 * As on the page, batches below 16 always run fp32-level products.  */
#define PC_PREC_AUTO 0
#define PC_PREC_FP32 1
#define PC_PREC_TF32 2

/* ---- circuit descriptor ------------------------------------------------ */
#define PC_LAYER_INPUT_CAT      0   /* categorical input nodes */
#define PC_LAYER_INPUT_EXTERNAL 1   /* values supplied by the caller in node_vals */
#define PC_LAYER_PRODUCT        2   /* v[p] = sum of children's values */
#define PC_LAYER_SUM            3   /* groups of log-space sum nodes */

/* One group of a sum layer: `num_nodes` (M) consecutive output nodes from
 * `out_start`, over N = num_ch_blocks * ch_block_size children listed as
 * blocks of consecutive node ids starting at ch_block_start[k] (child j of the
 * group is node ch_block_start[j / ch_block_size] + j % ch_block_size).  The
 * weights are a row-major [M, N] float32 matrix at params[param_offset].
 * Groups with equal param_offset share (tie) their weights and must have equal
 * M and N; their parameter flows are summed.  lowrank_slot >= 0 makes the
 * group a LowRank scaled group (pyjuice.parameterizations.LowRank): per
 * sample b its weights are theta * g_b normalised over the children, with the
 * scale g_b made from A_b, B_b (slot `lowrank_slot` of pc_lowrank_io) by the
 * circuit's lowrank_form: exp(A_b B_b) or sum_r exp(A_b[:, r]) exp(B_b[r, :]).
 * A group's children must be distinct nodes. */
typedef struct pc_sum_group {
  int32_t out_start;
  int32_t num_nodes;
  int32_t num_ch_blocks;
  int32_t ch_block_size;
  const int32_t* ch_block_start;   /* host pointer, [num_ch_blocks] */
  int64_t param_offset;
  int32_t lowrank_slot;            /* -1: plain sum group */
} pc_sum_group;

/* One layer.  Fields not used by the layer's kind are ignored.
 *  INPUT_CAT: nodes [node_start, node_start + num_nodes); node u reads
 *    category tokens[b * num_vars + var[u]] of row row[u] of a [num_rows,
 *    num_cats] float32 table at params[param_offset]: v[u,b] = log of that
 *    weight (-inf for a zero weight).  Nodes with the same row share it.
 *  INPUT_EXTERNAL: nodes [node_start, node_start + num_nodes) whose values the
 *    caller writes into node_vals before pc_forward (left untouched).
 *  PRODUCT: nodes [node_start, node_start + num_nodes); node p has children
 *    ch_ids[ch_ptr[p - node_start] .. ch_ptr[p - node_start + 1]) (>= 1 each).
 *  SUM: num_groups groups. */
typedef struct pc_layer_desc {
  int32_t kind;
  int32_t node_start;
  int32_t num_nodes;
  int32_t num_cats;
  int32_t num_rows;
  int64_t param_offset;
  const int32_t* var;              /* host, [num_nodes] */
  const int32_t* row;              /* host, [num_nodes] */
  const int32_t* ch_ptr;           /* host, [num_nodes + 1] */
  const int32_t* ch_ids;           /* host, [ch_ptr[num_nodes]] */
  int32_t num_groups;
  const pc_sum_group* groups;      /* host, [num_groups] */
} pc_layer_desc;

/* The circuit: layers in topological order (every child is defined by an
 * earlier layer), every node id in [0, num_nodes) defined exactly once.
 * root: node whose value pc_forward copies to `ll` (-1: none).
 * lowrank_rank: rank k of every LowRank slot (1..64: the fused kernels'
 *   limit, pyjuice.parameterizations.LowRank, Note), 0 if none.
 * lowrank_form: how every LowRank slot's factors make the scale
 *   (pyjuice.parameterizations.LowRank, definition): PC_LOWRANK_EXP_SUM
 *   g_b = exp(A_b B_b), PC_LOWRANK_SUM_EXP g_b[i,j] = sum_r exp(A_b[i,r])
 *   exp(B_b[r,j]); other values: PC_ERR_UNSUPPORTED. */
#define PC_LOWRANK_EXP_SUM 0
#define PC_LOWRANK_SUM_EXP 1
typedef struct pc_circuit_desc {
  int32_t num_nodes;
  int32_t num_vars;
  int64_t num_params;
  int32_t num_layers;
  const pc_layer_desc* layers;     /* host, [num_layers] */
  int32_t root;
  int32_t lowrank_rank;
  int32_t lowrank_form;
} pc_circuit_desc;

typedef struct pc_handle_s* pc_handle;

/* LowRank factors and gradients, one entry per slot (host arrays of device
 * pointers).  A[s]: [batch, M_s, k], B[s]: [batch, k, N_s] float32, in this
 * order (pyjuice.parameterizations.LowRank, "Tensor layout").  dA[s], dB[s]:
 * same shapes, written (overwritten) by pc_backward with dLL/dA and dLL/dB.
 * z_flows (nullable, device, [num_params] float32): the denominator statistic
 * of the conditional M-step (pyjuice.parameterizations.LowRank, Training,
 * apply_z_correction), W[i,j] = sum over samples and tied copies of
 * f_b[i] * exp(A_b B_b)[i,j] / Z_b[i] for every LowRank weight block, in the
 * parameter flows' layout; pc_backward ADDS it (like param_flows; only the
 * LowRank blocks' entries are touched; 0 where f = 0 or Z = 0).  NULL skips
 * it (the statistic costs one more pass over every (sample, node, child)).
 * Supported factor range: the kernels form theta * g in float32 with no
 * per-row shift, so every exp(h) (h = (A_b B_b)[i,j], or each exp(A) and
 * exp(B) of the "sum_exp" form) must be finite and each row's largest
 * theta * g a normal float32: h <= about 88 + |log theta| nats and the row's
 * largest h above about -87 + |log theta|.  Outside it a row's value is
 * non-finite or -inf where the exact one is finite. */
typedef struct pc_lowrank_io {
  int32_t num_slots;
  const float* const* A;
  const float* const* B;
  float* const* dA;
  float* const* dB;
  float* z_flows;
} pc_lowrank_io;

/* Read-only summary of a compiled layout (for inspection and tests). */
#define PC_CLASS_SHARED  0   /* all groups share one child list: exponentiated once */
#define PC_CLASS_STRIDED 1   /* equal-shape groups at even strides: one batched GEMM */
#define PC_CLASS_GENERAL 2   /* any other block-sparse layout */
#define PC_CLASS_LOWRANK 3   /* LowRank-scaled groups (fused exp_sum kernels) */
typedef struct pc_layout_summary {
  int32_t num_layers;
  int32_t num_sum_layers;
  int32_t num_param_blocks;      /* distinct (untied) sum weight matrices */
  int32_t num_row_segments;      /* parameter row runs normalised by EM */
  int64_t num_params;
  int32_t num_outputs;           /* nodes with no parent */
  int32_t device;                /* -1 if compiled host-only */
} pc_layout_summary;

/* ---- calls --------------------------------------------------------------- */

/* Validate and compile a circuit descriptor into a handle (host-side layout
 * compiler: checks, sum-layer classification SHARED / STRIDED / GENERAL after
 * PyJuice pull request #62 Summary item 2, tying, flow-write plan).  The
 * descriptor's host arrays are copied; the caller may free them afterwards.
 * device >= 0: also upload the handle's index tables to that HIP device (the
 * only device allocations the library makes; freed by pc_destroy).
 * device < 0: host-only handle for inspection (pc_forward etc. then return
 * PC_ERR_NO_DEVICE).
 * Errors: PC_ERR_INVALID_ARG (null pointers, ids out of range, a node defined
 * twice or used before it is defined, empty product, tied groups of different
 * shape, parameters out of range, overlapping parameter blocks),
 * PC_ERR_UNSUPPORTED (LowRank rank > 64 or < 1), PC_ERR_HIP. */
int pc_compile_layout(const pc_circuit_desc* desc, int device, pc_handle* out);

/* Free a handle and its device tables (null is accepted). */
int pc_destroy(pc_handle h);

/* Set the precision mode for subsequent calls (PyJuice pull request #62,
 * Summary item 1: the mode can be changed at any time).  Errors:
 * PC_ERR_INVALID_ARG (unknown mode), PC_ERR_UNSUPPORTED (PC_PREC_TF32). */
int pc_set_precision(pc_handle h, int mode);
int pc_get_precision(pc_handle h, int* mode);

/* Operand split used by a precision mode for one kind of product (advanced).
 * gemm_kind: 0 forward theta x E, 1 element flows theta^T x G, 2 parameter
 * flows G x E^T.  planes_a / planes_b: bfloat16 planes of the first / second
 * operand; the products of planes whose order is below the larger count are
 * accumulated: (1,1) one bf16 product; (2,1) or (1,2) one operand split,
 * two products; (2,2) hi/lo split, three products; (3,3) hi/mid/lo split,
 * six products.  Defaults: auto (2,2) for the forward and the element flows
 * (both operands split: a value dominated by one child, or a flow dominated
 * by one parent, then carries no bf16 rounding of e or of g = f / S, the
 * rounding -- up to 2^-8 -- that otherwise compounds from layer to layer past
 * 5e-3 end to end) and (2,1) for the parameter flows (g split, e rounded:
 * they are summed over samples); the weights, whose rounding would be the
 * same for every sample, are never rounded alone; fp32-level (3,3)
 * everywhere.  Errors: PC_ERR_INVALID_ARG for other counts or kinds. */
int pc_set_split(pc_handle h, int mode, int gemm_kind, int planes_a, int planes_b);

/* Product-kernel tuning (advanced; results change only by float32 summation
 * order).  PC_OPT_LAYER_TILE: output tile of the per-layer forward and
 * element-flow products, 0 automatic (64 x 128 when the first operand has
 * more bfloat16 planes than the second, else 128 x 64), 1 128 x 128,
 * 2 256 x 128, 3 128 x 256, 4 128 x 64, 5 64 x 128.
 * PC_OPT_PARAM_TILE: tile of the parameter-flow product, 0 automatic
 * (128 x 256 when the first operand has more bfloat16 planes than the
 * second, else 128 x 128), 1 128 x 128, 2 256 x 256 (when the operand split
 * allows), 3 128 x 256.
 * PC_OPT_SPLIT_MAX: largest K split of a per-layer product (1, 2, 4 or 8;
 * default 8).  PC_OPT_FUSE: 1 (default) evaluates a product layer inside the
 * adjacent sum layer's memory-bound kernels where the layout allows it (the
 * forward in the next sum layer's column maxima, the backward in the previous
 * sum layer's scaled-flow packing; identical results), 0 launches the
 * product kernels separately.  PC_OPT_PARAM_CHUNK: 0 computes the
 * parameter flows in one product after the layers; n > 0 computes them in
 * chunks of n tied copies per weight block on a second stream of the
 * handle, each as soon as its copies' scaled flows exist, overlapping the
 * element flows (deterministic; the float32 sum is grouped by chunk, so the
 * bits can differ from n = 0); -1 (default) chooses: one chunk of all the
 * copies of each block when the layout has at most 8 weight blocks and one of
 * them is tied (2 or more copies), else 0.  pc_backward joins that stream
 * into the caller's before it returns.  PC_OPT_LR_PACK: when the bfloat16 fragment records of
 * the LowRank factors are made: 0 (default) all at once at the start of
 * pc_forward, kept for pc_backward; 1 each group's just before its layer, in
 * both passes (identical results).  PC_OPT_SUMEXP_FUSED: how LowRank
 * groups of the "sum_exp" form run: 0 (default) as products with the shared
 * weights on a virtual batch of batch x rank columns
 * (pyjuice.parameterizations.LowRank, definition and Note: "sum_exp" is k
 * matmuls with the shared parameters), 1 through the fused LowRank kernels
 * (one visit per sample, node and child; results differ by rounding).
 * PC_OPT_FLOW_FP8 (pyjuice.parameterizations.LowRank, Parameters:
 * flow_precision "fp8"): 0 (default) bf16 operands, 1 the two products at the
 * end of a "sum_exp" backward on the virtual batch -- the parameter flows
 * theta * (Y1 X^T) and the denominator statistic W = Y2 C^T over every
 * (copy, sample, rank) -- from e4m3 operands with one power-of-two scale per
 * row and 32 consecutive (sample, rank) columns, fp32 accumulation.  Applies
 * in PC_PREC_AUTO only (the fp32-level mode, and batches below 16, keep their
 * split products) and to nothing else: values, element flows and dLL/dA,
 * dLL/dB are unchanged; the statistics are about 16x less accurate.
 * Changing an option can change pc_workspace_bytes.
 * Errors: PC_ERR_INVALID_ARG (unknown option or value). */
#define PC_OPT_LAYER_TILE 0
#define PC_OPT_PARAM_TILE 1
#define PC_OPT_SPLIT_MAX  2
#define PC_OPT_FUSE       3
#define PC_OPT_PARAM_CHUNK 4
#define PC_OPT_LR_PACK    5
#define PC_OPT_SUMEXP_FUSED 6
#define PC_OPT_FLOW_FP8   7
int pc_set_option(pc_handle h, int option, int value);

/* Bytes of workspace pc_forward / pc_backward need for `batch` samples in the
 * handle's current precision mode (batch < 16 counts as fp32-level).  The
 * workspace holds the bfloat16 operand planes (weights, exponentiated children
 * and scaled flows kept from the forward for the parameter flows), the
 * per-sample column maxima and small per-batch tables.  Errors:
 * PC_ERR_INVALID_ARG (batch < 1). */
int pc_workspace_bytes(pc_handle h, int batch, size_t* bytes);

/* Forward pass on `batch` samples.
 *  tokens    device int32 [batch, num_vars] (null if no categorical layer);
 *            values must lie in [0, num_cats) of the layer reading them.
 *  params    device float32 [num_params].
 *  node_vals device float32 [num_nodes, batch]: rows of INPUT_EXTERNAL layers
 *            are read, every other row is written.
 *  ll        device float32 [batch] (nullable): value of the root node.
 *  lowrank   factors (nullable unless the circuit has LowRank groups).
 *  ws        device workspace of ws_bytes >= pc_workspace_bytes(); its content
 *            is kept for the pc_backward call on the same batch.
 * Errors: PC_ERR_INVALID_ARG, PC_ERR_WORKSPACE, PC_ERR_NO_DEVICE, PC_ERR_HIP. */
int pc_forward(pc_handle h, int batch, const int32_t* tokens, const float* params,
               float* node_vals, float* ll, const pc_lowrank_io* lowrank,
               void* ws, size_t ws_bytes, void* stream);

/* Forward pass that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments and results
 * as pc_forward (node values and log-likelihoods; LowRank factors read),
 * minus the workspace: the scratch is a static device array of
 * PC_STATIC_SCRATCH_BYTES that each device the library runs on holds until
 * the process ends.  Forward only: nothing is kept for pc_backward (the
 * transposed weights, the operands of the parameter flows and the scaled sums
 * are not written), so a pc_backward needs its own pc_forward.
 * Every call on one device shares that device's array (and leaves its content
 * behind; the call clears what must start at zero), so calls that overlap in
 * time on one device -- other streams, other threads, other handles -- race
 * and give wrong results.  No timing events are recorded.
 * Errors: PC_ERR_WORKSPACE when the forward of `batch` samples needs more than
 * PC_STATIC_SCRATCH_BYTES of scratch (the message gives the size; use
 * pc_forward with a workspace); PC_ERR_HIP when the array's device address
 * could not be resolved; otherwise as pc_forward. */
#define PC_STATIC_SCRATCH_BYTES (128u * 1024u * 1024u)
int pc_forward_static(pc_handle h, int batch, const int32_t* tokens, const float* params,
                      float* node_vals, float* ll, const pc_lowrank_io* lowrank, void* stream);

/* Backward pass (element flows and parameter flows; PyJuice pull request #62,
 * Summary item 3) after pc_forward on the same batch, tokens, params, node_vals,
 * workspace and precision mode.
 *  node_flows  device float32 [num_nodes, batch], overwritten with
 *              dLL/dv (element flows).  Seeds: without PC_BWD_SEEDED the
 *              root's flow is 1 for every sample (other output nodes 0); with
 *              PC_BWD_SEEDED the caller has written the seeds into the rows of
 *              the output nodes (nodes with no parent), which are kept.
 *  param_flows device float32 [num_params], ACCUMULATED (+=): for every sum
 *              weight sum over samples and tied copies of
 *              f[i] * theta[i,j] * exp(v[j] - v[i]); for every input weight the
 *              summed flow of the samples showing that category.
 *  lowrank     with dA / dB outputs for LowRank groups (overwritten) and,
 *              if z_flows is set, the denominator statistic W (accumulated).
 * Errors: as pc_forward. */
#define PC_BWD_SEEDED 1
int pc_backward(pc_handle h, int batch, const int32_t* tokens, const float* params,
                const float* node_vals, float* node_flows, float* param_flows, int flags,
                const pc_lowrank_io* lowrank, void* ws, size_t ws_bytes, void* stream);

/* EM update of every parameter row (tied rows once), in place:
 *   theta <- (1 - step_size) * theta + step_size * (F + pseudocount / n) / (sum F + pseudocount)
 * with F the row's parameter flows and n its length; a row whose
 * (sum F + pseudocount) is 0 keeps its weights.  Plain EM (step_size 1,
 * pseudocount 0) is the "normalize(F+)" of pyjuice.parameterizations.LowRank,
 * Training.  Does not clear param_flows.
 * Errors: PC_ERR_INVALID_ARG (step_size outside [0, 1], pseudocount < 0). */
int pc_em_step(pc_handle h, float* params, const float* param_flows, float step_size,
               float pseudocount, void* stream);

/* The EM update with the LowRank conditional M-step
 * (pyjuice.parameterizations.LowRank, Training, compute_em_correction):
 * theta <- normalize(theta * F+ / F-) with F- = theta * W.  Every row of a
 * LowRank weight block takes R[j] = F+[j] / W[j] (entries with theta > 0 and
 * W > 0; 0 elsewhere) in place of F in pc_em_step's formula (same step size
 * and pseudocount); every other row is exactly pc_em_step.  z_flows: device
 * float32 [num_params], the W that pc_backward accumulated.  In place on
 * params; clears neither statistic.
 * Errors: as pc_em_step; PC_ERR_INVALID_ARG for a null z_flows. */
int pc_em_step_corrected(pc_handle h, float* params, const float* param_flows, const float* z_flows,
                         float step_size, float pseudocount, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* pc_last_error(void);

/* Layout summary, and the class (PC_CLASS_*) of layer `layer` (-1 for layers
 * that are not sum layers). */
int pc_layout_info(pc_handle h, pc_layout_summary* info);
int pc_layer_class(pc_handle h, int layer, int* cls);

/* Kernel timing: when enabled, every kernel that pc_forward / pc_backward
 * launch on `stream` is launched with a HIP event pair that its own dispatch
 * packet stamps at the kernel's start and end (hipExtLaunchKernelGGL), so a
 * pair measures one kernel's execution, the duration a kernel trace reports;
 * pc_kernel_times() then returns, per kernel kind, the number of launches and
 * the summed milliseconds of all launches recorded since the last reset (it
 * synchronises on those events).  Copies and fills through the HIP runtime
 * are not counted.
 * kinds: 0 sum forward GEMM, 1 element-flow GEMM, 2 parameter-flow GEMM,
 * 3 weight split, 4 column max, 5 exponentiate children, 6 scaled flows,
 * 7 input forward, 8 input backward, 9 product forward, 10 product backward,
 * 11 EM, 12 LowRank forward, 13 LowRank backward, 14 other,
 * 15 LowRank flow coefficients. */
#define PC_NUM_KERNEL_KINDS 16
int pc_set_timing(pc_handle h, int enable);
int pc_kernel_times(pc_handle h, int64_t* launches, double* ms);

#ifdef __cplusplus
}
#endif
#endif /* PC_H_ */
