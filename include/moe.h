/*
 * moe.h - C ABI of the MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * The layer (DeepSeek-V2 walkthrough page, DeepSeekMoE architecture section and
 * its MoEGate / MoE code; DeepSeek-V3 basics page, section 1.2):
 *
 *   h'_t = [u_t] + FFN_shared(u_t) + sum_{k<K} g_{t,k} * FFN_{idx_{t,k}}(u_t)
 *   FFN(u) = W_down (SiLU(W_gate u) * (W_up u)),   SiLU(z) = z / (1 + e^-z)
 *
 * Router: logits l = x * gate_w^T in fp32; scores s = softmax(l) or sigmoid(l);
 * selection scores z = s + sel_bias (bias used only to choose experts); groups
 * are contiguous runs of E/G experts scored by max z; the best topk_group groups
 * are kept (ties: lower group), the other experts are excluded; the K largest z
 * among the kept experts are chosen (ties: lower index). Gates g = s[idx]
 * (unbiased), renormalised over the K if norm_topk, then times
 * routed_scaling_factor.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *    except the moe_params / moe_weights structs, which are host memory read
 *    during the call only. A moe_cfg is owned by the library.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Work is
 *    enqueued asynchronously on it; no entry point synchronises the host.
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid call returns an error status and launches nothing.
 *  - A moe_cfg holds one workspace: calls on one cfg must be ordered (same
 *    stream, or externally synchronised). Use one cfg per concurrent stream.
 *  - Status: 0 = OK, negative = error (moe_status_string names it).
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
  MOE_ERR_INVALID_ARG = -1, /* bad pointer, size or parameter combination */
  MOE_ERR_UNSUPPORTED = -2, /* valid layer, but a shape/dtype the library does not run */
  MOE_ERR_OOM = -3,         /* workspace allocation failed */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_SCRATCH = -5      /* moe_layer_forward_noalloc: the call needs more
                               workspace than its fixed scratch array holds */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Which expert-GEMM kernels run. AUTO picks by token count. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GROUPED = 1, MOE_PATH_STREAM = 2 } moe_path;

/* Expert-GEMM inputs (architecture article, section 4.2: fp8 GEMM inputs with
 * fp32 accumulation and block-wise quantisation).
 * NONE: the expert GEMMs multiply bf16 token rows and bf16 h.
 * E4M3_1X128 (FP8_E4M3 weights and BF16 x only): the token rows and h are
 * quantised to e4m3 with one fp32 scale per 1 x 128 block of a row (largest
 * magnitude / 448, codes rounded to nearest even, see
 * moe_quantize_e4m3_1x128) and multiplied on the fp8 matrix cores with the
 * weights' 128 x 128 block scales; accumulation is fp32. The router still
 * reads x unquantised. Runs the grouped kernels at every token count
 * (path STREAM is rejected with MOE_ERR_UNSUPPORTED). */
typedef enum { MOE_ACT_QUANT_NONE = 0, MOE_ACT_QUANT_E4M3_1X128 = 1 } moe_act_quant;

typedef struct {
  int dim;            /* D: model dim (row length of x and out) */
  int n_routed;       /* E: routed experts, 1..512 */
  int hidden;         /* H: hidden size of each routed expert */
  int shared_hidden;  /* Hs: hidden of the fused shared expert (N_s shared experts
                         of hidden h fused as one of hidden N_s*h); 0 = none */
  int top_k;          /* K: routed experts per token, 1..16 */
  int n_group;        /* G: expert groups, E % G == 0; 1 = greedy */
  int topk_group;     /* groups kept per token, 1..G; K <= topk_group*E/G */
  int score_fn;       /* moe_score_fn */
  int norm_topk;      /* 1: g /= sum of the K chosen scores */
  float routed_scaling_factor;
  int act_dtype;      /* x dtype: MOE_F32 or MOE_BF16 */
  int weight_dtype;   /* expert weights: MOE_F32 (with F32 x), MOE_BF16 or
                         MOE_FP8_E4M3 (with BF16 x) */
  int out_dtype;      /* MOE_F32 or MOE_BF16 */
  int add_residual;   /* 1: out includes x (h'_t = u_t + ...) */
  int max_tokens;     /* largest T any call on this cfg may pass */
  int path;           /* moe_path */
  int act_quant;      /* moe_act_quant */
  int backward;       /* 1: also allocate the workspace of moe_layer_backward
                         (BF16 x and BF16 weights only) */
} moe_params;

/* Expert weights in nn.Linear layout [out, in], row-major, dtype weight_dtype.
 * Routed set (E experts):   gate_up [E][2H][D] (rows 0..H-1 = W_gate,
 *                           rows H..2H-1 = W_up), down [E][D][H].
 * Shared expert:            gate_up [2Hs][D], down [D][Hs].
 * FP8_E4M3 only: one fp32 scale per 128x128 block, w = e4m3(q) * scale:
 *   gate_up_scale [E][2H/128][D/128] (shared: [2Hs/128][D/128]),
 *   down_scale    [E][D/128][H/128]  (shared: [D/128][Hs/128]).
 * For F32 / BF16 weights the scale pointers are ignored. */
typedef struct {
  const void* gate_up;
  const void* down;
  const float* gate_up_scale;
  const float* down_scale;
} moe_weights;

typedef struct moe_cfg moe_cfg;

/* Validates *p and allocates the workspace for up to p->max_tokens tokens on
 * the current HIP device. Returns MOE_ERR_INVALID_ARG for an invalid layer
 * (E % G != 0, topk_group > G, K > topk_group*E/G, ...), MOE_ERR_UNSUPPORTED
 * for a dtype/shape the library does not run (bf16/fp8 weights need D, H, Hs
 * multiples of 128 and max_tokens*D*2, max_tokens*max(H,Hs)*2 and
 * 2*max(H,Hs)*D*2 below 2^32 bytes; f32 needs D % 32 == 0), MOE_ERR_OOM if
 * the workspace does not fit. On success *out owns the workspace until
 * moe_cfg_destroy. */
moe_status moe_cfg_create(const moe_params* p, moe_cfg** out);

/* Frees the workspace (synchronises the device first). NULL is a no-op. */
moe_status moe_cfg_destroy(moe_cfg* cfg);

/* Bytes of device workspace the cfg holds. */
size_t moe_cfg_workspace_bytes(const moe_cfg* cfg);

/* The layer forward (page-1 MoE forward with the V3 bias rule).
 *   x           [T][D]  act_dtype
 *   gate_w      [E][D]  fp32 router weight
 *   sel_bias    [E]     fp32 selection-only bias, or NULL (= 0)
 *   expert_w    routed weights (see moe_weights), required
 *   shared_w    shared expert weights; required iff shared_hidden > 0
 *               (pass NULL to skip the shared expert only when Hs == 0)
 *   out         [T][D]  out_dtype; written in full
 *   expert_counts [E] int32 tokens routed to each expert, or NULL; overwritten
 * 0 <= T <= max_tokens. T == 0 only zeroes expert_counts. */
moe_status moe_layer_forward(moe_cfg* cfg, const void* x, int T, const float* gate_w,
                             const float* sel_bias, const moe_weights* expert_w,
                             const moe_weights* shared_w, void* out, int32_t* expert_counts,
                             void* stream);

/* The layer forward without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, semantics and results (the same kernels)
 * as moe_layer_forward on a cfg created from *params, with two differences:
 *  - there is no cfg: *params (host memory, read during the call) describes
 *    the layer; its max_tokens and backward fields are ignored;
 *  - the workspace is a fixed array of 64 MiB in device memory, one per GPU,
 *    loaded with the library's code and held until the process ends. The
 *    call needs the workspace a cfg with max_tokens = T would allocate
 *    (moe_cfg_workspace_bytes); above 64 MiB it returns MOE_ERR_SCRATCH and
 *    launches nothing (the V3 decode shape, D = 7168, E = 256, H = 2048,
 *    K = 8, fits up to T = 256 tokens).
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind (nothing in it needs to start at zero: each call writes what it
 * reads): calls that overlap on one GPU race, so keep them on one stream or
 * synchronise them. The first call on each device looks up the array's
 * device address (hipGetSymbolAddress) and the device's CU count; later calls
 * make no runtime query beyond hipGetDevice. No hipMalloc, hipFree or other
 * allocating call is made. Score sums (moe_cfg_set_score_sums) and stage
 * timing belong to a cfg and are not available here. */
moe_status moe_layer_forward_noalloc(const moe_params* params, const void* x, int T, const float* gate_w,
                                     const float* sel_bias, const moe_weights* expert_w,
                                     const moe_weights* shared_w, void* out, int32_t* expert_counts,
                                     void* stream);

/* Gradients of a layer (the back-propagation step of the training data flow
 * in the "Transformer block" article, which updates experts and router):
 * for L = sum(d_out * out), with out = moe_layer_forward on the same inputs.
 * The expert choice (group limit and top-K) is piecewise constant, so it is
 * held fixed; the gradient reaches the router through the gate values
 * g_k = rsf * s_k (/ sum of the K chosen s when norm_topk), then through the
 * score function to the logits, x and gate_w. sel_bias only changes the
 * choice and gets no gradient (moe_bias_update adjusts it).
 *   d_out         [T][D] fp32 (input; 16-byte aligned)
 *   dx            [T][D] fp32 dL/dx (includes d_out itself when add_residual;
 *                 16-byte aligned)
 *   d_gate_w      [E][D] fp32 dL/dgate_w
 *   d_expert_w    fp32 dL/dW in the layout of moe_weights: gate_up
 *                 [E][2H][D], down [E][D][H]; every expert is written
 *                 (zeros for an expert that received no token)
 *   d_shared_w    the same for the shared expert ([2Hs][D], [D][Hs]);
 *                 required iff shared_hidden > 0
 * Other arguments as moe_layer_forward. The cfg must have been created with
 * backward = 1, BF16 x and BF16 weights (else MOE_ERR_UNSUPPORTED). The
 * routing is recomputed (same kernels as the forward, so the same choice),
 * and the gate/up pre-activations are recomputed rather than stored.
 * Products run on bf16 MFMA with fp32 accumulation: d_out and gate_w are
 * rounded to bf16 for them, the intermediates [a | u], g*h, [dA | dU] and
 * the per-slot dx rows are bf16. T == 0 zeroes every output. */
typedef struct {
  float* gate_up;
  float* down;
} moe_weight_grads;

moe_status moe_layer_backward(moe_cfg* cfg, const void* x, int T, const float* gate_w, const float* sel_bias,
                              const moe_weights* expert_w, const moe_weights* shared_w, const float* d_out,
                              float* dx, float* d_gate_w, const moe_weight_grads* d_expert_w,
                              const moe_weight_grads* d_shared_w, void* stream);

/* The forward of a training step (same arguments as moe_layer_forward): the
 * output of moe_layer_forward on the grouped path, bit for bit (the expert
 * GEMMs take that path whatever T is), and, left in the cfg's workspace, what the
 * backward pass needs from the gate/up products: the pre-activations
 * [a | u] and g * SiLU(a) * u of every routed row and of the shared expert,
 * from the same fp32 accumulators as h, so moe_layer_backward_saved can skip
 * their recompute. The cfg must have been created with backward = 1, BF16 x
 * and BF16 weights (else MOE_ERR_UNSUPPORTED). The saved values stay valid
 * until the next moe_layer_forward_train or moe_layer_backward on this cfg. */
moe_status moe_layer_forward_train(moe_cfg* cfg, const void* x, int T, const float* gate_w,
                                   const float* sel_bias, const moe_weights* expert_w,
                                   const moe_weights* shared_w, void* out, int32_t* expert_counts,
                                   void* stream);

/* moe_layer_backward (same arguments, outputs and results) that reads [a | u]
 * and g * h left by the last moe_layer_forward_train on this cfg instead of
 * recomputing them (the routing is still recomputed). That forward must have
 * had the same T (else MOE_ERR_INVALID_ARG, nothing launched) and the same x,
 * gate_w, sel_bias and weights, which is not checked: with other inputs the
 * gradients are those of a mixture of the two. On the stream order: the
 * forward must be ordered before this call (same stream, or synchronised). */
moe_status moe_layer_backward_saved(moe_cfg* cfg, const void* x, int T, const float* gate_w,
                                    const float* sel_bias, const moe_weights* expert_w,
                                    const moe_weights* shared_w, const float* d_out, float* dx,
                                    float* d_gate_w, const moe_weight_grads* d_expert_w,
                                    const moe_weight_grads* d_shared_w, void* stream);

/* The router alone (the MoEGate forward plus the selection bias):
 *   topk_idx [T][K] int32, listed by descending z then ascending index
 *   topk_gate [T][K] fp32 gate values in the same order
 *   expert_counts [E] int32 or NULL. */
moe_status moe_router_forward(moe_cfg* cfg, const void* x, int T, const float* gate_w,
                              const float* sel_bias, int32_t* topk_idx, float* topk_gate,
                              int32_t* expert_counts, void* stream);

/* Dispatch alone, from a given routing (the page-1 MoE code's
 * repeat_interleave + per-expert mask gather, done as histogram + prefix scan
 * + permutation):
 *   topk_idx    [T][K] int32 in [0, E)   (input; entries outside [0, E)
 *               are skipped and leave their slot_row entry unwritten)
 *   offsets     [E+1]  int32: rows of expert e are offsets[e] .. offsets[e+1]-1
 *   row_token   [T*K]  int32: token of each expert-contiguous row
 *   slot_row    [T*K]  int32: row that holds (t, k), at index t*K + k
 * The permutation is stable: the row of (t, k) with expert e is
 * offsets[e] + #{(t', k') before (t, k) in row-major order with expert e},
 * so an expert's rows hold its tokens in ascending order and every output is
 * unique. */
moe_status moe_dispatch_forward(moe_cfg* cfg, const int32_t* topk_idx, int T, int32_t* offsets,
                                int32_t* row_token, int32_t* slot_row, void* stream);

/* The activation quantiser of MOE_ACT_QUANT_E4M3_1X128 alone (architecture
 * article, section 4.2, block-wise fp8 quantisation):
 *   x      [rows][cols] bf16 (input; finite values)
 *   codes  [rows][cols] uint8 OCP e4m3 codes (output)
 *   scales [rows][cols/128] fp32 (output)
 * Each block b of 128 consecutive values of a row gets scale = amax / 448
 * (fp32, correctly rounded; 1 when the block is all zero) and each value v
 * the e4m3 code nearest to v / scale (fp32 division), ties to the even code;
 * the block maximum maps to +-448; the code's sign bit is v's sign bit.
 * cols must be a positive multiple of 128 and rows * cols at most 2^34;
 * rows == 0 launches nothing. MOE_ERR_INVALID_ARG (nothing launched) for a
 * null pointer with rows > 0 or a bad size. No cfg; stream-ordered. */
moe_status moe_quantize_e4m3_1x128(const void* x, int rows, int cols, uint8_t* codes, float* scales,
                                   void* stream);

/* Load balance between steps (no cfg; stream-ordered; one small launch).
 *
 * moe_bias_update: the auxiliary-loss-free update of the DeepSeek-V3 basics
 * page, section 1.2 -- after a step, an overloaded expert's selection bias is
 * lowered by gamma and an underloaded expert's raised by gamma. Overloaded
 * means expert_counts[e] * E > sum(expert_counts), underloaded < (decided in
 * integers); at exactly the mean load the bias stays. sel_bias [E] fp32 is
 * updated in place (each new value is the fp32 sum).
 *   expert_counts [E] int32 >= 0 (e.g. the counts a forward wrote)
 *   E in [1, 512]; gamma finite.
 *
 * moe_load_stats: the load statistics of the load-balance code in the
 * DeepSeekMoE + MLA notes (page 3): with load_e = counts_e / sum(counts),
 *   stats[0] = standard deviation of load over the experts (n-1 denominator)
 *   stats[1] = mean_e (load_e - 1/E)^2   (the load term of the expert-level
 *              balance loss, before its weight)
 *   stats[2] = max_e counts_e / (sum(counts)/E) - 1   (maximum violation)
 * all 0 when sum(counts) == 0. stats: 3 fp32 in device memory.
 *
 * Both return MOE_ERR_INVALID_ARG (and launch nothing) for a null pointer, E
 * outside [1, 512] or a non-finite gamma. */
moe_status moe_bias_update(const int32_t* expert_counts, int E, float gamma, float* sel_bias, void* stream);
moe_status moe_load_stats(const int32_t* expert_counts, int E, float* stats, void* stream);

/* Score column sums for the importance statistic (the load-balance code in the
 * DeepSeekMoE + MLA notes, page 3, sums every token's scores per expert).
 * With score_sum set (device memory, [E] fp32), every later
 * moe_layer_forward and moe_router_forward on this cfg also writes
 *   score_sum[e] = sum over the call's T tokens of s[t][e]
 * (s = the unbiased softmax or sigmoid scores of all E experts, fp32; summed
 * in token order over chunks of 256 tokens, the chunks added in order in
 * double, so repeated calls give identical bits; T == 0 writes zeros). It adds
 * a write of the T x E scores and two small launches to the router stage.
 * NULL turns it off (the default). The pointer is used by calls on the cfg's
 * stream until it is replaced. MOE_ERR_INVALID_ARG for a NULL cfg. */
moe_status moe_cfg_set_score_sums(moe_cfg* cfg, float* score_sum);

/* The balance statistics of that code, expert- and device-level, in one
 * small launch (no cfg; stream-ordered). Inputs in device memory:
 *   expert_counts [E] int32 >= 0, score_sum [E] fp32 >= 0 (as written above).
 * load_e = counts_e / sum(counts), importance_e = score_sum_e / sum(score_sum);
 * devices own contiguous runs of E / n_devices experts (the placement of one
 * expert group per device), device load and importance are the sums over their
 * experts, renormalised to sum 1. Written to stats [9] fp32 (device memory):
 *   [0] std of load (n-1 denominator)    [1] mean_e (load_e - 1/E)^2
 *   [2] max_e counts_e / (sum/E) - 1      [3] std of importance
 *   [4] mean_e (importance_e - 1/E)^2     [5] std of device load
 *   [6] mean_d (dev_load_d - 1/n_devices)^2
 *   [7] std of device importance          [8] mean_d (dev_imp_d - 1/n_devices)^2
 * The losses are the page's loss_load / loss_importance terms before their
 * weights alpha. Statistics of a quantity whose total is 0 are 0; a std over
 * one value is 0. MOE_ERR_INVALID_ARG (nothing launched) for a NULL pointer, E
 * outside [1, 512], or n_devices outside [1, E] or not dividing E. */
moe_status moe_balance_stats(const int32_t* expert_counts, const float* score_sum, int E, int n_devices,
                             float* stats, void* stream);

/* Stage timing (observability): when enabled, moe_layer_forward records HIP
 * events on its stream around each stage -- 0 router, 1 dispatch, 2 gate/up
 * GEMM, 3 down GEMM, 4 combine -- for up to MOE_TIMING_CALLS calls.
 * moe_cfg_stage_times waits for the last recorded call, writes the summed
 * milliseconds of each stage to ms[MOE_NUM_STAGES] and the number of timed
 * calls to *calls, and starts a new window. Enabling creates the events
 * (host-side HIP calls); timing does not synchronise the host inside
 * forward. */
#define MOE_NUM_STAGES 5
#define MOE_TIMING_CALLS 256
moe_status moe_cfg_set_stage_timing(moe_cfg* cfg, int enable);
moe_status moe_cfg_stage_times(moe_cfg* cfg, double* ms, int* calls);

/* Debug builds (the library compiled with MOE_DEBUG, built as
 * libmoe_mi355x_debug.so): every index a kernel reads from memory (gathered
 * token rows, slot -> row maps, expert indices, dispatch placements) is
 * checked against its buffer; a violation is recorded -- the first one's
 * check site and offending value -- and the index replaced by 0, so the
 * access stays inside the buffer instead of faulting. moe_debug_status
 * synchronises the device, writes that site (0 = no violation since the last
 * call) and value, and clears the record. Sites: 1 grouped-GEMM token row,
 * 2 grouped-GEMM tile row, 3 e4m3-GEMM token row, 4 streaming-GEMM token row,
 * 5 fp32-GEMM token row, 6 combine slot row, 7 backward expert index,
 * 8 backward slot row, 9 dispatch placement. Release builds return
 * MOE_ERR_UNSUPPORTED (site and value 0); MOE_ERR_INVALID_ARG for NULL. */
moe_status moe_debug_status(int* site, int* value);

/* HIP error code behind the last MOE_ERR_HIP on this cfg (0 if none). */
int moe_cfg_last_hip_error(const moe_cfg* cfg);

const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
