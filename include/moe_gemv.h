/*
 * moe_gemv.h -- C ABI of a mixture-of-experts layer forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * Problem statement.  An MoE layer replaces a transformer block's FFN with a
 * router and E experts; the router sends each of the T tokens (hidden size m)
 * to its top-k experts, each expert is a two-layer MLP with W1 of m x p and
 * W2 of p x m, and the experts' outputs are gathered back to their tokens
 * (HARMOEny article, yejing.asia/?p=12: section 1 for the router + expert
 * structure, section 3.2 "expert prefetch" for the expert x*W1*W2 with W1
 * m x p and W2 p x m, section 3.3 for route -> dispatch -> expert compute ->
 * gather).  The expert comes in two forms: the ReLU MLP relu(x W1) W2 and the
 * SwiGLU form (SiLU(x W1) * (x W3)) W2, whose W3 is a second m x p matrix.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    16-byte aligned.  bf16 tensors hold raw bfloat16 bit patterns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call except
 *    moe_weights_create/moe_weights_destroy/moe_profile_end only enqueues work
 *    on that stream and returns without synchronising.
 *  - Every call returns a moe_status.  Arguments are validated before
 *    anything is enqueued: a non-OK status means nothing was launched.
 *    moe_last_error() gives a message for the calling thread's last failure.
 *  - The library keeps no caller pointer after a call returns.  The only
 *    memory it owns is the packed weight store inside a moe_weights.
 *  - Calls are reentrant.  One moe_weights may serve several streams at once
 *    if every in-flight call has its own workspace.
 *  - Shape limits: 1 <= E <= 64, 1 <= k <= E, m and p positive multiples of
 *    64, T*k < 2^31.  T == 0 is a successful no-op.
 *  - Supported (activation / weight / expert) combinations: F32/F32 and
 *    BF16/BF16 with either expert kind; BF16 activations with I8, I4, FP8 or
 *    MXFP4 weights and either expert kind (I4 and MXFP4: m and p multiples
 *    of 128).  Anything else returns MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_GEMV_H
#define MOE_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, k > E, shape mismatch, misalignment */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside the limits above */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_OOM = 5          /* device allocation failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_I8 = 2,
  MOE_I4 = 3,
  MOE_FP8 = 4,
  MOE_MXFP4 = 5,
  MOE_FP8A8 = 6, /* fp8 weights and fp8 activations (moe_weights_create) */
  MOE_I8A8 = 7   /* int8 weights and int8 activations (moe_weights_create) */
} moe_dtype;
typedef enum { MOE_MLP_RELU = 0, MOE_SWIGLU = 1 } moe_ffn_kind;

#define MOE_MAX_EXPERTS 64
/* moe_route_topk flag: skip the router product and read fp32 logits from `logits`. */
#define MOE_ROUTE_LOGITS_IN 1u

/* Opaque, library-owned expert weights in the packed device layout. */
typedef struct moe_weights moe_weights;

/* Message describing the calling thread's most recent failure ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int moe_abi_version(void);

/*
 * moe_weights_create -- take a layer's expert weights and re-lay them out
 * once, at initialisation, so that the forward pass streams every weight
 * byte in full 128-byte lines (the DeepSpeed-Inference summary,
 * datalearner.com, section 3 "SBI-GeMM", part 3: weights transposed at
 * initialisation so each thread reads consecutive input-dimension
 * elements of one output column).
 *
 *  m, p, E       hidden size, expert inner size, number of experts.
 *  kind          MOE_MLP_RELU (w1 = W1, w2 = W2, w_up must be NULL) or
 *                MOE_SWIGLU (w1 = gate W1, w_up = up W3, w2 = down W2).
 *  w_dtype       MOE_F32, MOE_BF16, MOE_I8, MOE_I8A8, MOE_I4, MOE_FP8,
 *                MOE_FP8A8 or MOE_MXFP4.  MOE_FP8A8 takes the weights and scales of
 *                MOE_FP8 and also quantises each token's input to the experts
 *                to E4M3 with one power-of-two scale per token (2^X, X the
 *                smallest integer with max|x| <= 448 * 2^X), as the
 *                DeepSpeed-Inference summary's INT8 GeMM quantises its
 *                activations (section 4); routing reads x unquantised.  At
 *                prefill sizes its first projection then runs on the fp8
 *                matrix cores.  MOE_I8A8 likewise with the weights and scales
 *                of MOE_I8 and the input quantised to int8 (scale 2^X, X the
 *                smallest integer with max|x| <= 127 * 2^X, q = round-half-
 *                even(x / 2^X)): the INT8 GeMM with both operands quantised,
 *                its first projection on the int8 matrix cores at prefill
 *                sizes.
 *  w1, w_up      device [E][m][p] in w_dtype (MOE_I4: one int8 per weight,
 *                holding q in [-8, 7], stored packed two per byte; MOE_FP8:
 *                (and MOE_FP8A8) one OCP E4M3 code per byte; MOE_MXFP4: one E2M1 code per
 *                byte in its low nibble, stored packed two per byte).
 *  w2            device [E][p][m] in w_dtype (as above).
 *  s1, s_up      MOE_I8 / MOE_I8A8 / MOE_I4 / MOE_FP8 / MOE_FP8A8: device fp32 [E][p] per-output-
 *                channel scales of w1 and w_up (the weight is q * s, or
 *                e4m3(code) * s).  MOE_MXFP4: device uint8 [E][m/32][p] E8M0
 *                exponents, one per block of 32 consecutive rows k of a column
 *                (the weight is e2m1(code) * 2^(X - 127)); the kernels are
 *                exact for X in [27, 227].  NULL for bf16 and fp32.
 *  s2            the same for w2: fp32 [E][m], or uint8 [E][p/32][m].
 *  stream        packing runs on this stream; the call synchronises it
 *                before returning, so the inputs may be freed afterwards.
 *  out           receives the handle; release it with moe_weights_destroy.
 * Errors: INVALID_ARG, UNSUPPORTED, OOM, HIP.  On error *out is NULL.
 */
moe_status moe_weights_create(int m, int p, int E, int kind, int w_dtype, const void* w1, const void* w_up,
                              const void* w2, const void* s1, const void* s_up, const void* s2, void* stream,
                              moe_weights** out);

/* Free a handle from moe_weights_create (NULL is accepted).  Synchronises the device. */
moe_status moe_weights_destroy(moe_weights* w);

/*
 * moe_weights_offload -- keep a layer's experts in host memory and stream
 * them to the GPU as forwards need them: the expert prefetch of the HARMOEny
 * article (yejing.asia, section 3.2: one expert computes while the next is
 * fetched; experts may then live in CPU memory) with the device expert cache
 * and second copy stream of the GPU-cache article (coreui.cn, sections 2.2
 * and 3.2).
 *  The packed weights of every expert move to pinned host memory and their
 *  device copy is freed; `slots` (1 <= slots <= E) device slots of one
 *  expert each cache experts between forwards (least recently used first
 *  out).  Scales stay on the device.  Afterwards moe_layer_forward,
 *  moe_layer_forward_fused and moe_expert_ffn on this handle: route and
 *  dispatch, copy the per-expert row counts to the host (the one host
 *  synchronisation of such a forward), then run the touched experts one at a
 *  time -- cached ones first, then the others by decreasing rows -- each
 *  missing expert copied into a slot on the handle's copy stream (default
 *  priority) while the experts before it compute.  Results equal those of the
 *  device-resident handle.  Calls on one offloaded handle serialise on the
 *  host.  Graph capture and moe_layer_forward_noalloc refuse such a handle
 *  (MOE_ERR_UNSUPPORTED).  An expert's transfer hides behind the previous
 *  expert's compute when that one holds more than about phi * dtype / (2 *
 *  beta) rows (phi the compute rate, beta the host link's bytes per second;
 *  the article's threshold q).
 *  stream   the copies to host memory run on it; the call synchronises it.
 * Errors: INVALID_ARG (NULL, slots out of range, already offloaded),
 * UNSUPPORTED (fp32 weights), OOM, HIP.
 */
moe_status moe_weights_offload(moe_weights* w, int slots, void* stream);

/* Counters of an offloaded handle since moe_weights_offload: experts found
 * in a slot, experts copied in, and the bytes copied host -> device. */
moe_status moe_weights_offload_stats(const moe_weights* w, long long* hits, long long* misses, long long* bytes);

/* Bytes of device workspace moe_layer_forward / moe_expert_ffn need for T
 * tokens at top-k.  A pure function of the handle (its shape, dtype and
 * tuning), T, k and the device's compute-unit count: the process
 * environment plays no part. */
moe_status moe_workspace_size(const moe_weights* w, int T, int k, size_t* bytes);

/*
 * Launch tuning.  Which kernels serve the expert FFN and their launch shapes
 * are chosen on the host from (m, p, E, expert kind, weight dtype, T, k); a
 * moe_tuning attached to a handle overrides single choices.  Every field is
 * 0 for "automatic"; a tri-state switch is 1 (on) or -1 (off).  The
 * automatic choices are the measured defaults, so callers normally never set
 * one; the fields exist so that every launch form can be tested and timed.
 */
typedef struct moe_tuning {
  int ffn_path;         /* MOE_PATH_AUTO, MOE_PATH_SKINNY (decode kernels) or MOE_PATH_GEMM (grouped GEMM) */
  int skinny_mt;        /* decode kernels: 16-row M tiles per work item (1, 2 or 4) */
  int skinny_pack;      /* decode kernels: activations as packed fragments (1) or gathered rows (-1) */
  int skinny_splitk;    /* decode kernels: a workgroup's waves split the reduction (1) or the columns (-1) */
  int skinny_shared;    /* decode kernels, columns split: one LDS copy of the activations per workgroup (1/-1) */
  int skinny_wide;      /* decode kernels: hot experts on twelve-tile items in both projections (1/-1) */
  int skinny_wide_down; /* the same for the down projection alone (1/-1) */
  int up_ct;            /* decode kernels: column tiles per wave of the up projection (1, 2 or 4) */
  int down_ct;          /* the same for the down projection */
  int down_ksplit;      /* decode down projection: reduction slices (1 .. p/64) */
  int down_rows;        /* decode down projection: unweighted rows + combine kernel (1) or weighted fp32
                           atomics into an accumulator (-1) */
  int gemm_cg;          /* grouped GEMM: column blocks per group of its work order (>= 1) */
  int gemm_skip;        /* grouped GEMM: skip the products of empty row fragments (1/-1) */
  int route_quant;      /* 8-bit-activation layers: quantise the experts' input rows in the routing pass
                           (1) or in a kernel of their own (-1) */
} moe_tuning;
#define MOE_PATH_AUTO 0
#define MOE_PATH_SKINNY 1
#define MOE_PATH_GEMM 2

/*
 * moe_weights_set_tuning -- attach tuning to a handle (NULL: all automatic).
 * It applies to every later call with the handle, moe_workspace_size
 * included, so a workspace must be sized after the tuning is set.  Not to be
 * called while a forward pass with the handle is being enqueued on another
 * thread.  A forced path the weights cannot take (the grouped GEMM needs
 * bf16, int8, int4 or fp8 weights) falls back to the decode kernels.
 * Errors: INVALID_ARG (NULL handle, a value out of range).
 */
moe_status moe_weights_set_tuning(moe_weights* w, const moe_tuning* t);
moe_status moe_weights_get_tuning(const moe_weights* w, moe_tuning* t);

/*
 * moe_workspace_size_for -- moe_workspace_size for a layer that has no
 * handle yet: the same result as moe_workspace_size on a handle created with
 * (m, p, E, kind, w_dtype) and tuning t (NULL: automatic).  Host only; it
 * touches no device memory.
 * Errors: INVALID_ARG, UNSUPPORTED.
 */
moe_status moe_workspace_size_for(int m, int p, int E, int kind, int w_dtype, const moe_tuning* t, int T, int k,
                                  size_t* bytes);

/*
 * moe_route_topk -- router product, top-k and gate weights for T tokens.
 * The gating network runs on the GPU and maps every token to its experts
 * (GPU-cache article, coreui.cn, section 3.1; HARMOEny article, section 3.3
 * step one).
 *   logits[t][e] = sum_i x[t][i] * w_router[i][e] (+ b_router[e]), fp32.
 *   Experts are ranked by (logit descending, expert index ascending); NaN
 *   ranks below every number and +0 equals -0.  topk_idx[t][j] is the j-th
 *   ranked expert, and topk_w[t][j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *   (softmax over the selected k).
 *
 *  x          device [T][m], x_dtype MOE_F32 or MOE_BF16 (ignored with LOGITS_IN).
 *  w_router   device fp32 [m][E] (ignored with LOGITS_IN).
 *  b_router   device fp32 [E] or NULL.
 *  flags      0 or MOE_ROUTE_LOGITS_IN (read logits instead of computing them).
 *  logits     device fp32 [T][E]: output (may be NULL) or, with LOGITS_IN, input.
 *  topk_idx   device int32 [T][k] output.   topk_w  device fp32 [T][k] output.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
moe_status moe_route_topk(const void* x, int x_dtype, const float* w_router, const float* b_router, int T, int m, int E,
                          int k, unsigned flags, float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * moe_dispatch -- group the T*k assignments (a = t*k + j) by expert: the
 * single-GPU form of sending tokens to their experts (HARMOEny article,
 * section 3.3 step four).
 *   counts[e]  = number of assignments to expert e;
 *   offsets    = exclusive prefix sum of counts, offsets[E] = T*k;
 *   perm[r]    = assignment id at permuted row r: expert-major, and within
 *                an expert in increasing assignment id (stable);
 *   inv_perm[a]= the row r with perm[r] = a.
 *  topk_idx   device int32 [T*k] input; an id outside [0, E) is clamped into
 *             range (the result stays a valid permutation, its grouping is
 *             then meaningless).
 *  counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]: device int32 outputs.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, void* stream);

/*
 * moe_expert_ffn -- every expert on its rows: for each permuted row r of
 * expert e (offsets[e] <= r < offsets[e+1]) with token t = perm[r] / k,
 *   y_perm[r] = relu(x_t W1_e) W2_e              (MOE_MLP_RELU)
 *   y_perm[r] = (SiLU(x_t W1_e) * (x_t W3_e)) W2_e  (MOE_SWIGLU)
 * unweighted, fp32 (HARMOEny article, section 3.2: the expert is x*W1*W2).
 * For bf16/int8 weights the hidden activation is rounded to bf16 between the
 * two projections; accumulation is fp32.
 *  w          handle from moe_weights_create (m, p, E must match).
 *  x          device [T][m] in x_dtype.
 *  perm, offsets   from moe_dispatch (device int32).
 *  y_perm     device fp32 [T*k][m] output.
 *  workspace  device, >= moe_workspace_size(w, T, k) bytes, 256-byte aligned.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
moe_status moe_expert_ffn(const moe_weights* w, const void* x, int x_dtype, int T, int m, int p, int E, int k,
                          const int32_t* perm, const int32_t* offsets, float* y_perm, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * moe_combine -- gather the expert outputs back to their tokens, weighted
 * (HARMOEny article, section 3.3 step six; GPU-cache article, section 3.1):
 *   y[t] = sum_{j<k} topk_w[t][j] * y_perm[inv_perm[t*k + j]]   (fp32 sum)
 *  y_perm     device fp32 [T*k][m];  inv_perm  device int32 [T*k];
 *  topk_w     device fp32 [T][k];    y  device [T][m] in y_dtype (F32 or BF16).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w, int T, int m, int k, void* y,
                       int y_dtype, void* stream);

/*
 * moe_quantize_rows_e4m3 -- the first step of an fp8-activation layer's
 * experts (MOE_FP8A8): each row of x quantised to OCP E4M3 with one
 * power-of-two scale, the INT8 GeMM's activation quantisation of the
 * DeepSpeed-Inference summary (datalearner.com, section 4) in 8-bit float
 * form.  moe_expert_ffn and the layer forwards of an MOE_FP8A8 handle run it
 * themselves; it is exposed for callers that quantise once and for checks.
 *   scale[t] = 2^X, X the smallest integer with max_i |x[t][i]| <= 448 * 2^X
 *   xq[t][i] = e4m3(round-to-nearest-even(x[t][i] / scale[t])) * scale[t]
 *  x      device bf16 [T][m] (finite values);  m a multiple of 64.
 *  xq     device bf16 [T][m]: the quantised values (exactly representable).
 *  scale  device fp32 [T].
 *  16-byte aligned x and xq.  Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
moe_status moe_quantize_rows_e4m3(const void* x, int T, int m, void* xq, float* scale, void* stream);
/* The int8 form for MOE_I8A8 layers: scale[t] = 2^X, X the smallest integer
 * with max_i |x[t][i]| <= 127 * 2^X; xq[t][i] = round-half-even(x[t][i] /
 * scale[t]) * scale[t] (bf16, exact).  Arguments and errors as above. */
moe_status moe_quantize_rows_i8(const void* x, int T, int m, void* xq, float* scale, void* stream);

/*
 * moe_layer_forward -- the whole layer: route + top-k, dispatch, experts and
 * the weighted combine, fused where possible and all on `stream`, with no
 * host synchronisation.
 *  w_router, b_router, x, x_dtype   as in moe_route_topk.
 *  y          device [T][m] output in y_dtype (F32 or BF16).
 *  workspace  device, >= moe_workspace_size(w, T, k) bytes, 256-byte aligned.
 *  dbg_*      optional device outputs of the intermediate stages (each may be
 *             NULL): topk_idx [T][k], topk_w [T][k], logits [T][E],
 *             counts [E], offsets [E+1], perm [T*k].
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
moe_status moe_layer_forward(const moe_weights* w, const float* w_router, const float* b_router, const void* x, int x_dtype,
                             int T, int m, int p, int E, int k, void* y, int y_dtype, void* workspace, size_t ws_bytes,
                             int32_t* dbg_topk_idx, float* dbg_topk_w, float* dbg_logits, int32_t* dbg_counts,
                             int32_t* dbg_offsets, int32_t* dbg_perm, void* stream);

/*
 * moe_layer_forward_fused -- moe_layer_forward with the layer's neighbouring
 * ops done inside it (DeepSpeed-Inference summary, section 4, fusion regions
 * "post-attention layer norm + intermediate GeMM" and "bias and residual
 * add"; section 2: a norm's reductions run along the row within one tile):
 *   x' = norm(x);  y = residual + MoE(x')
 *  norm      MOE_NORM_NONE, MOE_NORM_LAYER (per row: mean and biased
 *            variance over the m columns, (x - mean) / sqrt(var + eps) *
 *            gamma + beta) or MOE_NORM_RMS (x / sqrt(mean(x^2) + eps) *
 *            gamma).  The norm is computed in fp32 inside the routing pass
 *            and rounded to x's dtype; routing and experts use x'.
 *  gamma     device fp32 [m] (required with a norm); beta device fp32 [m] or
 *            NULL (layer norm only); both 16-byte aligned.  eps in [0, 1].
 *  residual  device [T][m] in y_dtype, or NULL; added to the fp32 sum before
 *            y is rounded.
 *  x_norm    optional device [T][m] in x_dtype, 16-byte aligned: receives x'
 *            (else it stays in the workspace).  Needs a norm.
 *  dbg_*     as in moe_layer_forward (may be NULL).
 * Other arguments and errors as moe_layer_forward.
 */
#define MOE_NORM_NONE 0
#define MOE_NORM_LAYER 1
#define MOE_NORM_RMS 2
moe_status moe_layer_forward_fused(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                                   int x_dtype, int norm, const float* gamma, const float* beta, float eps,
                                   const void* residual, int T, int m, int p, int E, int k, void* y, int y_dtype,
                                   void* workspace, size_t ws_bytes, void* x_norm, int32_t* dbg_topk_idx,
                                   float* dbg_topk_w, float* dbg_logits, void* stream);

/*
 * moe_layer_graph_create / moe_graph_launch / moe_graph_destroy -- the layer
 * forward captured once into a HIP graph and replayed with one launch (the
 * CUDA-Graph capture of the DeepSpeed-Inference summary, section 4, as HIP
 * graphs).  moe_layer_graph_create records exactly the launches
 * moe_layer_forward makes for these arguments (same meaning as there; no
 * dbg outputs) on a capture stream of its own; nothing runs until a launch.
 * The graph holds the pointers, sizes and launch shapes: each
 * moe_graph_launch recomputes y from whatever x, router and expert weights
 * then hold, on `stream` (NULL: the default stream), with no host
 * synchronisation.  The caller keeps x, y, the workspace and the weights
 * alive and unmoved while the graph exists, and must not run two launches of
 * one graph (or a launch and moe_layer_forward on the same workspace) at the
 * same time.  Shapes, dtypes or T need a new graph.  *out receives the handle
 * (NULL on error); destroy frees it.  Capture is refused while
 * moe_profile_begin is active.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP (as moe_layer_forward),
 * OOM.
 */
typedef struct moe_graph moe_graph;
moe_status moe_layer_graph_create(const moe_weights* w, const float* w_router, const float* b_router, const void* x,
                                  int x_dtype, int T, int m, int p, int E, int k, void* y, int y_dtype, void* workspace,
                                  size_t ws_bytes, moe_graph** out);
moe_status moe_graph_launch(const moe_graph* g, void* stream);
moe_status moe_graph_destroy(moe_graph* g);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: its workspace is a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  Arguments, results and
 * errors as moe_layer_forward without the workspace and dbg outputs, plus
 * UNSUPPORTED when T tokens need more workspace than the array holds (the
 * Mixtral-shaped decode layers fit up to a few hundred tokens; prefill
 * batches need moe_layer_forward).  Every call on one GPU uses that GPU's one
 * array: calls that overlap on a GPU (on different streams, or threads)
 * race, so the caller serialises them.  Nothing in the array needs clearing
 * between calls.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_weights* w, const float* w_router, const float* b_router,
                                     const void* x, int x_dtype, int T, int m, int p, int E, int k, void* y,
                                     int y_dtype, void* stream);

/*
 * Measurement aid (not part of the layer).  Between moe_profile_begin and
 * moe_profile_end every kernel the library launches is bracketed by HIP
 * events on its own stream.  moe_profile_end waits for the last event and
 * folds the durations into per-kernel totals readable with
 * moe_profile_query(name, &total_ms, &launches).  Process-global, not
 * thread-safe; max_launches bounds the events recorded (later launches are
 * not timed).  Kernel names: "route_topk", "dispatch", "ffn_up", "ffn_down",
 * "ffn_f32_up", "ffn_f32_down", "combine", "finalize", "fill".
 */
moe_status moe_profile_begin(int max_launches);
moe_status moe_profile_end(void);
moe_status moe_profile_query(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GEMV_H */
