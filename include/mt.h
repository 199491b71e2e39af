/*
 * mt.h - C ABI of the layer-streamed transformer training step.
 *
 * Method ("MegaTrain: Full Precision Training of 100B+ Parameter LLMs on a
 * Single GPU", abstract): parameters and optimizer state live in host memory
 * and the GPU is a transient compute engine; per layer, parameters stream in
 * and gradients stream out; a double-buffered pipeline overlaps prefetch,
 * compute and gradient offload on several streams; stateless layer templates
 * are bound to whichever weights are resident. Activations are recomputed in
 * backward and the optimizer step runs on the CPU over fp32 master weights and
 * moments ("Technical Brief: MegaTrain's Single-GPU 120B-Parameter Training
 * Breakthrough", section "Checkpointing, Manual Gradients, and CPU-Side
 * Optimizer Steps").
 *
 * The model is a Llama-style decoder: RMSNorm, half-split rotary embeddings,
 * causal grouped-query attention, SwiGLU MLP, final RMSNorm, untied LM head,
 * mean next-token cross-entropy, AdamW with decoupled weight decay.
 *
 * Conventions for every entry point:
 *  - Return 0 (MT_OK) on success, a negative MT_E* code on failure; no C++
 *    exception crosses the ABI. After an error, mt_last_error() describes it
 *    and the context can still be destroyed.
 *  - Pointers are plain host pointers unless stated otherwise.
 *  - Calls on one context are not thread-safe: the caller serialises them.
 *
 * Canonical tensor order (ids used by mt_set_param / mt_params / mt_grads /
 * mt_opt_state), all fp32, row-major, Linear weights [out, in] (y = x W^T):
 *   0                 tok_emb   [vocab, d]
 *   1 + 9*l + 0..8    layer l:  attn_norm [d], wq [H*hd, d], wk [Hkv*hd, d],
 *                               wv [Hkv*hd, d], wo [d, H*hd], mlp_norm [d],
 *                               w_gate [F, d], w_up [F, d], w_down [d, F]
 *   1 + 9*L           final_norm [d]
 *   2 + 9*L           lm_head   [vocab, d]
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ---- */
#define MT_OK 0
#define MT_EINVAL -1      /* bad config, id, shape, pointer, or token id outside [0, vocab) */
#define MT_EHOSTOOM -2    /* host (pinned or pageable) allocation failed */
#define MT_EDEVOOM -3     /* device allocation failed */
#define MT_EHIP -4        /* a HIP runtime call failed; mt_last_error() has its text */
#define MT_ENONFINITE -5  /* the step's loss was not finite: no update was applied */
#define MT_ETIMEOUT -6    /* a host-side wait exceeded its limit */
#define MT_ENOGRADS -7    /* gradients were not kept (MT_KEEP_GRADS off) */
#define MT_ESTATE -8      /* call not valid in the context's current state */

/* ---- compute dtypes ---- */
#define MT_FP32 0   /* fp32 weights streamed, fp32 matrix-core products */
#define MT_BF16 1   /* bf16 shadow streamed, bf16 operands, fp32 accumulation */

/* ---- flags ---- */
#define MT_KEEP_GRADS 1u     /* keep every tensor's gradient in host memory (mt_grads) */
#define MT_KERNEL_TIMING 2u  /* time every kernel launch with HIP events (mt_kernel_stats) */
#define MT_TRACE 4u          /* record the per-unit schedule log (mt_schedule, mt_trace_dump) */
/* Let the host AdamW of a step finish during the next step: mt_train_step
 * returns once every gradient has landed in host memory, the remaining
 * updates run in the order the next forward needs them (embedding, layers
 * 0..L-1, head), and the next step loads a unit only after its update has
 * landed. Results are identical to the synchronous mode. Accessors that read
 * or write the host state (mt_params, mt_grads, mt_opt_state, mt_set_param)
 * and mt_destroy wait for pending updates first; mt_sync waits explicitly. */
#define MT_OVERLAP_OPT 8u
/* Print one line to stderr as each forward, head and backward item of a step
 * finishes on the device (for steps that take minutes). */
#define MT_PROGRESS 16u
/* With a device cache (n_layer_buffers > 2): do not refresh cached units in
 * the backward; their next image is fetched by the next forward instead, so
 * the backward's link carries only gradients. */
#define MT_CACHE_NO_REFRESH 32u
/* Gradients cross the host link as bf16 (round to nearest even) instead of
 * fp32, halving the gradient copy bytes; the host AdamW widens them exactly
 * (mt_grads then returns the widened values). A measured variant: the
 * default keeps the gradients at full precision ("MegaTrain: Full Precision
 * Training of 100B+ Parameter Large Language Models on a Single GPU"); the
 * technical brief's "Limitations of Current Throughput Metrics and Empirical
 * Validation" leaves batch and transfer configurations open. */
#define MT_BF16_GRADS 64u

typedef struct mt_model_cfg {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;   /* must divide n_heads; query head h reads kv head h / (H/Hkv) */
  int32_t head_dim;     /* fp32: 16, 32, 64 or 128; bf16: 64 or 128 */
  int32_t ffn_dim;
  int32_t vocab;
  int32_t max_batch;    /* largest B accepted by mt_train_step */
  int32_t max_seq;      /* largest T accepted by mt_train_step */
  int32_t compute_dtype;     /* MT_FP32 or MT_BF16 */
  /* Device layer buffers. 2 = every unit (layer or head) streams through two
   * buffers. k in [3, n_layers]: a device cache -- the head and the top k - 3
   * layers keep a buffer each, the other layers stream through two. k >=
   * n_layers + 1: every unit keeps a buffer of its own. A unit with its own
   * buffer is not fetched again for its backward, and its updated image is
   * copied into that buffer as soon as its AdamW has landed (during the
   * backward, or in the next step's forward), so the next forward does not
   * fetch it either. Results do not depend on k. */
  int32_t n_layer_buffers;
  int32_t host_threads;      /* AdamW / gather pool size; 0 = online CPUs (at most 64) */
  uint32_t flags;            /* MT_KEEP_GRADS | MT_KERNEL_TIMING | MT_TRACE | MT_OVERLAP_OPT | MT_PROGRESS |
                                MT_CACHE_NO_REFRESH | MT_BF16_GRADS */
  float rms_eps;
  float rope_base;
  double lr, beta1, beta2, adam_eps, weight_decay;   /* AdamW hyperparameters */
  /* Token rows per chunk of the QKV projection and the MLP (forward,
   * recompute and backward): their intermediates are sized by the chunk, not
   * the batch. 0 = automatic (the whole batch unless the MLP intermediates of
   * max_batch * max_seq rows would exceed 4 GiB). Weight gradients sum the
   * chunks in order, so a different chunk size changes their rounding. */
  int32_t chunk_rows;
  /* Residual checkpoints x_1..x_k (layer inputs) parked in host memory
   * between the forward and the backward instead of device memory: each in
   * a pageable slab of its own, crossing the host link once each way through
   * one of two pinned bounce slabs (the worker pool copies between a bounce
   * slab and the parked slab). 0 = automatic (none
   * unless the device cannot hold all L + 1 of them next to the workspace);
   * k in [1, n_layers - 2] = exactly k. Parking k of them frees k + 1
   * device slots (x_0 is re-sent from the gathered embedding rows). Results
   * do not depend on k. */
  int32_t ckpt_host;
  /* Pinned gradient staging slots when MT_KEEP_GRADS is off (each holds one
   * unit's gradients from their D2H until that unit's AdamW has read them).
   * 0 = automatic (synchronous: 3 slots of the largest unit; MT_OVERLAP_OPT:
   * as many layer-sized slots as fit in 16 GiB, 3 to 16, plus one for the
   * head). k in [1, 64] = exactly k slots (plus the head's with
   * MT_OVERLAP_OPT). Fewer slots make a gradient copy wait for an earlier
   * unit's update to release its slot; results do not depend on k. */
  int32_t grad_ring_slots;
  /* Limit, in milliseconds, on any host-side wait inside a step (the
   * dispatcher waiting for a copy, a kernel sequence, a staging slot or an
   * AdamW update to make progress; the final wait for the updates). 0 = no
   * limit. When a wait exceeds it, mt_train_step stops issuing work, waits
   * for what it already issued, and returns MT_ETIMEOUT with mt_last_error()
   * naming the item it was waiting for; the host state may then hold part of
   * the step's updates, and the context accepts no further steps (MT_ESTATE)
   * but can still be read and destroyed. */
  int32_t wait_timeout_ms;
  /* Gradient accumulation over micro-batches inside each streamed unit. 0 or
   * 1: the step's B sequences run through each layer together. k >= 2: each
   * unit runs them as k micro-batches of ceil(B / k) sequences (the last may
   * be smaller), and its weight gradients sum over the micro-batches on the
   * device before they leave it; the weights still cross the link once per
   * step. The activation workspace is sized for one micro-batch (the
   * residual checkpoints and the residual gradient still hold the whole
   * batch). Results equal the whole-batch step up to the order in which the
   * weight gradients add up. Must be at most max_batch. */
  int32_t micro_batches;
} mt_model_cfg;

/* Optional streams for the three pipeline stages (hipStream_t values passed as
 * void*) and device memory. NULL env, or a NULL member, makes the library
 * create its own streams and take its device memory with hipMalloc.
 * workspace: a caller-owned block of workspace_bytes device bytes (256-byte
 * aligned; from a framework's allocator, for example) from which the
 * context carves every device buffer instead (layer and gradient buffers,
 * the activation workspace, residual checkpoint slots). It must hold at
 * least mt_device_plan's fixed_bytes plus two checkpoint slots (or all
 * n_layers + 1 slots when n_layers < 3); checkpoints that do not fit in the
 * rest are parked in host memory (cfg.ckpt_host = 0). It must stay
 * allocated, and untouched by the caller, until mt_destroy. The library
 * takes no device memory during a step either way. */
typedef struct mt_device_env {
  void* copy_in;
  void* compute;
  void* copy_out;
  void* workspace;
  int64_t workspace_bytes;
} mt_device_env;

typedef struct mt_ctx mt_ctx;

/* Number of tensors in the canonical order: 9 * n_layers + 3. */
int32_t mt_tensor_count(const mt_model_cfg* cfg);

/* Name (NUL-terminated, truncated to name_cap) and shape of tensor id.
 * ndim is 1 or 2; shape[1] is 1 for vectors. */
int mt_tensor_info(const mt_model_cfg* cfg, int32_t id, char* name, int32_t name_cap,
                   int64_t shape[2], int32_t* ndim);

/* Host memory that mt_create(cfg) allocates, without allocating it (no GPU
 * needed): for sizing a model to a machine's RAM. state_bytes: the fp32
 * master p and the AdamW moments m and v, 12 bytes per parameter ("MegaTrain
 * fits 120B LLM training on one GPU using CPU RAM", section "Who this is
 * actually for": about 12 GB of host RAM per billion parameters).
 * pinned_bytes: page-locked memory (the bf16
 * images, the gradient slots or kept gradients, staging; the fp32 master in
 * fp32 mode). pageable_bytes: the rest (m, v, the embedding). Parked residual
 * checkpoints, chosen at create time from free device memory, add
 * parked_ckpt_bytes of pageable memory each, plus two pinned bounce slabs of
 * that size when any is parked. Any output may be NULL. MT_EINVAL on a bad
 * cfg. */
int mt_host_bytes(const mt_model_cfg* cfg, int64_t* state_bytes, int64_t* pinned_bytes,
                  int64_t* pageable_bytes, int64_t* parked_ckpt_bytes);

/* Device memory a context of cfg takes, without a device: fixed_bytes for
 * the layer buffers, gradient buffers and activation workspace, and
 * ckpt_slot_bytes for each residual checkpoint slot it keeps on the device
 * (n_layers + 1 slots when none is parked; with k parked, n_layers - k).
 * Any output may be NULL. MT_EINVAL on a bad cfg. */
int mt_device_plan(const mt_model_cfg* cfg, int64_t* fixed_bytes, int64_t* ckpt_slot_bytes);

/* Create a context ("MegaTrain: Full Precision Training of 100B+ Parameter
 * Large Language Models on a Single GPU", abstract: parameters and optimizer
 * states live in host memory, the GPU is a transient compute engine; the
 * double-buffered engine needs device buffers for layers in flight).
 * Validates cfg, allocates the host store (fp32 master p,
 * AdamW m and v zeroed, step count 0, the bf16 device-format shadow in bf16
 * mode, gradient buffers), the device layer buffers, gradient buffers,
 * checkpoints and activation workspace, the three streams and the events.
 * host_param_ptrs: NULL (parameters start at zero; fill them with mt_set_param)
 * or an array of mt_tensor_count(cfg) caller-owned fp32 tensors in canonical
 * order, copied during the call. On failure *out is NULL and
 * mt_last_error(NULL) describes the error. */
int mt_create(const mt_model_cfg* cfg, const float* const* host_param_ptrs,
              const mt_device_env* env, mt_ctx** out);

/* Copy one tensor's fp32 values into the master store and refresh its
 * device-format shadow (the host store is the parameters' home, abstract
 * above). Valid between steps; waits for updates still in flight. */
int mt_set_param(mt_ctx* ctx, int32_t id, const float* src);

/* One training step on tokens / targets, each [B, T] int32 row-major
 * (read during the call; every id must lie in [0, vocab)): the layer-wise
 * streamed forward, the head, recompute + backward in reverse layer order,
 * gradients streamed out and the CPU AdamW (abstract above; "Technical
 * Brief: MegaTrain's Single-GPU 120B-Parameter Training Breakthrough",
 * section "Checkpointing, Manual Gradients, and CPU-Side Optimizer Steps").
 * It returns after every AdamW update has landed in host memory, or, with
 * MT_OVERLAP_OPT, once every gradient has (the updates then finish during
 * the next step). *loss_out is the mean cross-entropy over the B*T
 * positions. On MT_ENONFINITE the state is unchanged and the step count is
 * not advanced; on MT_ETIMEOUT see cfg.wait_timeout_ms; MT_ESTATE after an
 * earlier MT_ETIMEOUT. */
int mt_train_step(mt_ctx* ctx, const int32_t* tokens, const int32_t* targets, int32_t B,
                  int32_t T, float* loss_out);

/* Wait until every AdamW update submitted so far has landed in host memory
 * (a no-op unless MT_OVERLAP_OPT left some running). */
int mt_sync(mt_ctx* ctx);

/* Per-token losses of the last step in (b, t) order: *n = B*T. Library-owned,
 * valid until the next mt_train_step or mt_destroy. */
int mt_token_losses(mt_ctx* ctx, const float** ptr, int64_t* n);

/* Read-only, library-owned views of the fp32 master parameters, the raw
 * gradients dL/dp of the last step (MT_ENOGRADS unless MT_KEEP_GRADS), and
 * the AdamW moments with the step count: the host-resident state the
 * technical brief's CPU-side optimizer keeps in full precision (section
 * "Checkpointing, Manual Gradients, and CPU-Side Optimizer Steps"). Each
 * waits for updates still in flight. Valid until the next mt_train_step /
 * mt_set_param / mt_destroy. */
int mt_params(mt_ctx* ctx, int32_t id, const float** ptr, int64_t* numel);
int mt_grads(mt_ctx* ctx, int32_t id, const float** ptr, int64_t* numel);
int mt_opt_state(mt_ctx* ctx, int32_t id, const float** m, const float** v, int64_t* t);

typedef struct mt_step_stats {
  double step_ms;          /* wall time of the last mt_train_step */
  double forward_ms;       /* start of step to the loss being known on the host */
  double h2d_bytes, d2h_bytes;      /* bytes moved over the host link by the step */
  double h2d_busy_ms, d2h_busy_ms;  /* summed copy durations (MT_TRACE only, else 0) */
  double compute_busy_ms;           /* summed unit compute durations (MT_TRACE only, else 0) */
  double adamw_ms;         /* summed wall time of the host AdamW tasks */
  double adamw_bytes;      /* host DRAM bytes the AdamW pass reads and writes */
  double tail_ms;          /* from the last gradient landing to the step's return */
  double model_flops;      /* 6 * matmul params * tokens + causal attention (fwd + bwd) */
  double hw_flops;         /* model FLOPs plus the recompute */
  int64_t tokens;
  int64_t step;            /* AdamW step count after the step */
} mt_step_stats;

/* Measurement of the last step: link bytes and copy time, compute time, the
 * host AdamW's time and traffic (the technical brief, "Limitations of Current
 * Throughput Metrics and Empirical Validation", names link use, host memory
 * bandwidth and optimizer latency as what to measure). */
int mt_stats(mt_ctx* ctx, mt_step_stats* out);

/* Per-kernel-class totals of the last step (needs MT_KERNEL_TIMING), measured
 * with HIP events on the compute stream around each launch. */
#define MT_KCLASS_COUNT 12
typedef struct mt_kernel_stat {
  char name[32];           /* e.g. "gemm_nt_bf16" */
  int64_t launches;
  double ms;               /* summed launch durations */
  double flops;            /* summed algorithmic FLOPs (2*M*N*K for products) */
  double bytes;            /* summed algorithmic HBM bytes */
} mt_kernel_stat;

int mt_kernel_stats(mt_ctx* ctx, mt_kernel_stat* out, int32_t cap, int32_t* n);

/* Schedule log of the last step (needs MT_TRACE): one entry per unit stage. */
#define MT_PH_LOAD 0      /* H2D of a unit image into a layer buffer (stream 0) */
#define MT_PH_FWD 1       /* forward of a layer (stream 1) */
#define MT_PH_HEAD 2      /* head forward + backward (stream 1) */
#define MT_PH_BWD 3       /* recompute + backward of a layer (stream 1) */
#define MT_PH_GRAD 4      /* D2H of a unit's gradients (stream 2) */
#define MT_PH_ADAMW 5     /* host AdamW of a unit (stream 3 = host) */
#define MT_PH_CKPT_OUT 6  /* D2H of a parked residual checkpoint (stream 2; unit = its index) */
#define MT_PH_CKPT_IN 7   /* H2D of a parked residual checkpoint (stream 0; unit = its index) */
#define MT_PH_REFRESH 8   /* H2D of a cached unit's updated image into its own buffer (stream 0) */
#define MT_UNIT_EMB -1
#define MT_UNIT_HEAD -2
typedef struct mt_sched_entry {
  int32_t phase;
  int32_t unit;            /* layer index, MT_UNIT_HEAD or MT_UNIT_EMB */
  int32_t buffer;          /* layer buffer (LOAD/FWD/HEAD/BWD) or gradient buffer (GRAD) */
  int32_t stream;          /* 0 copy-in, 1 compute, 2 copy-out, 3 host AdamW,
                              4 host time spent submitting the stage's work */
  double t0_ms, t1_ms;     /* relative to the start of the step */
} mt_sched_entry;

int mt_schedule(mt_ctx* ctx, mt_sched_entry* out, int32_t cap, int32_t* n);

/* Write the schedule log as Chrome trace-event JSON: one timeline row per
 * stream (copy-in, compute, copy-out, host AdamW, host submission), showing
 * the overlap of prefetch, compute and gradient offload that the abstract's
 * double-buffered engine is built for. */
int mt_trace_dump(mt_ctx* ctx, const char* path);

/* Device bytes the context holds (buffers, checkpoints, workspace). */
int mt_device_bytes(mt_ctx* ctx, int64_t* bytes);

/* Placement chosen at creation: token rows per chunk, residual checkpoints
 * parked in host memory, and checkpoint slots held in device memory. */
int mt_layout_info(mt_ctx* ctx, int64_t* chunk_rows, int32_t* ckpt_host, int32_t* ckpt_device_slots);

/* Text of the last error on ctx (or, when ctx is NULL, of the last failed
 * mt_create or mt_op_* call on this thread that reports one). Never NULL. */
const char* mt_last_error(const mt_ctx* ctx);

void mt_destroy(mt_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MT_H */
