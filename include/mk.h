/*
 * mk.h — C ABI of the persistent decode megakernel for MI355X (gfx950).
 *
 * One call of mk_decode_step runs one autoregressive decode step of a
 * Llama-style decoder (optionally with a sparse mixture-of-experts FFN) for a
 * fixed batch of independent sequences, as ONE kernel launch.  Inside that
 * launch every CU runs an interpreter over a queue of tile tasks built ahead
 * of time on the host (the on-GPU interpreter and per-SM instruction queues of
 * the koas-w.github.io megakernel notes, "on-GPU interpreter / persistent
 * kernel" and "static and dynamic scheduling"; the Hazy Research megakernel
 * news page, section 4, "fusion big bang": instruction sequences built once in
 * Python and reused for hundreds of forward passes).  Tasks order themselves
 * through integer counters in global memory (same page, section 4,
 * "synchronisation"; MPK news page, part 2: a task increments its trigger
 * event, an event fires at a threshold) and prefetch the next tasks' weights
 * into paged LDS (same Hazy page, section 4, "shared memory to remove memory
 * bubbles").
 *
 * Conventions for every entry point:
 *   - (dev) marks device memory, (host) host memory.
 *   - No call prints, throws or exits; failures are reported by the status.
 *   - A handle is not thread-safe; steps on one handle must be issued in order
 *     on one stream.
 *   - All weights are bf16 bit patterns (uint16), row-major [out][in].
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_handle mk_handle;

typedef enum {
    MK_OK = 0,
    MK_E_INVALID = 1,      /* bad argument or unsupported shape (host-side check) */
    MK_E_UNSUPPORTED = 2,  /* valid request this build does not implement */
    MK_E_NOMEM = 3,        /* device or host allocation failed */
    MK_E_HIP = 4,          /* a HIP runtime call failed */
    MK_E_NOT_RESIDENT = 5, /* the persistent grid cannot be co-resident on the device */
    MK_E_DEVICE = 6,       /* the kernel recorded an error (see mk_check_device_error) */
    MK_E_NO_DEVICE = 7     /* no usable GPU */
} mk_status;

/* Per-layer weights (dev, bf16, [out][in]); the caller keeps ownership.
 * attn_norm, ffn_norm: [hidden].  wq [n_q*d][hidden], wk/wv [n_kv*d][hidden],
 * wo [hidden][n_q*d]; dense FFN: w_gate/w_up [ffn][hidden], w_down [hidden][ffn].
 * MoE FFN (n_experts > 0): router [n_experts][hidden], exp_gate/exp_up
 * [n_experts][expert_ffn][hidden], exp_down [n_experts][hidden][expert_ffn]. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
    const void *router, *exp_gate, *exp_up, *exp_down;
} mk_layer_weights;

/* Model description.  head_dim must be 64 or 128; n_q a multiple of n_kv.
 * RMSNorm: x * g / sqrt(mean(x^2) + rms_eps).  RoPE pairs (j, j + d/2) of each
 * head at angle position * rope_theta^(-2j/d).  tok_embed [vocab][hidden];
 * lm_head [vocab][hidden] or NULL when tied_lm_head (then tok_embed is used);
 * final_norm [hidden].  layers: (host) array of n_layers entries. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    int32_t n_experts, top_k, expert_ffn_dim; /* n_experts == 0: dense SwiGLU FFN */
    float rms_eps, rope_theta;
    int32_t tied_lm_head;
    const void *tok_embed, *lm_head, *final_norm;
    const mk_layer_weights *layers;
} mk_model_desc;

/* Build options; pass NULL for the defaults.  A zero-filled struct is the default
 * configuration: every field's 0 means "automatic" or "off". */
typedef struct {
    int32_t sched;             /* 0 static per-CU queues (default), 1 dynamic global queue (atomic pop),
                                * 2 event-driven: tasks taken from a global ready queue in the order their
                                * events activated them, the activating worker appending the dependents;
                                * 3 event-driven with scheduler waves: the activating worker posts the event
                                * to the activated-event queue of workgroup (event mod workgroups), whose
                                * second loader wave dispatches its dependents to the ready queue (MPK news
                                * page, part 2: scheduler units with activated-event queues); 2 and 3 keep
                                * one counter per event */
    int32_t n_workgroups;      /* persistent workgroups; 0 = one per CU of the device */
    int32_t policy;            /* static assignment: 0 round-robin, 1 least-loaded (bytes) first */
    int32_t attn_splits;       /* KV chunks per (sequence, KV head), at most 16; 0 = automatic */
    int32_t debug_timeout_ms;  /* bound on every in-kernel wait; 0 = 2000 ms */
    int32_t debug_drop_signal; /* n > 0: the task with index n - 1 skips its signal (tests of the timeout
                                  path); 0 or negative = off */
    int32_t trace;             /* 1: record per-task timestamps (mk_read_trace) */
    int32_t cooperative;       /* 1: cooperative launch (co-residency of every workgroup guaranteed by the
                                  runtime, about 20 us more per step); 0 (default): plain launch of one
                                  workgroup per CU, which needs the device to itself: if some workgroups
                                  could not start, the others' waits time out and the step reports
                                  MK_E_DEVICE instead of hanging */
    int32_t page_kib;          /* LDS page size in KiB: 0 or 16.  The ring is eight 16 KiB pages (128 KiB of
                                  the CU's 160 KiB LDS) and is not a run-time choice: the packed weight layout
                                  stores every GEMV tile as 1 KiB matrix-core blocks, sixteen to a page, so the
                                  page size is part of the layout built here.  Any other value: MK_E_INVALID */
    int32_t poison;            /* 1: before every step, fill the step's scratch that producers overwrite (query
                                  rows, attention partials, SiLU(gate)*up rows, matrix-core operand regions,
                                  router logits) and the logits and hidden outputs with NaN, so a task that
                                  read any of them before its producer wrote it would put NaN in the outputs
                                  (precision-regression testing of fused kernels: cloud.baidu.com
                                  explainer, section 8).  Costs one extra kernel launch per step. */
    int32_t reserved[6];
} mk_options;

/* Validates the description, copies the weights into a handle-owned packed
 * layout (the caller may free its copies afterwards), builds the task graph,
 * the event targets and the queues, and uploads them to the current device.
 * 1 <= batch <= 64 sequences (batch > 1 also needs hidden <= 2048; the
 * projections of up to 16 sequences share one pass over the weights, so
 * 17..32 sequences take two, 33..64 up to four); max_ctx >= 1 positions per sequence in the KV
 * cache.  Errors: MK_E_INVALID (NULL pointers, unsupported shapes, bad options),
 * MK_E_UNSUPPORTED (batch > 64; batch > 1, or a mixture of experts, with
 * hidden > 2048), MK_E_NO_DEVICE, MK_E_NOMEM, MK_E_HIP.  On success *out
 * receives the handle.  Defined by: the task graph built once on the host and
 * reused for every forward (Hazy Research megakernel news page, section 4,
 * "fusion big bang"; MPK news page, part 1: the model becomes a graph of tasks
 * and events; koas-w.github.io notes, "SM-level task graph"). */
mk_status mk_build_graph(const mk_model_desc *desc, int32_t batch, int32_t max_ctx, const mk_options *opt,
                         mk_handle **out);

/* Host-only planning: builds the task graph and queues exactly as
 * mk_build_graph would for `n_workgroups` workgroups (weight pointers in desc
 * are ignored and may be NULL) and writes the export image (format as
 * mk_export_graph) into buf (host) of capacity cap; *need receives the size.
 * Touches no GPU.  Returns MK_E_INVALID when cap is too small (need is set).
 * Defined by: static per-SM queues fixed before launch, or one global queue
 * claimed at run time (koas-w.github.io notes, "static and dynamic
 * scheduling"; MPK news page, part 1, the task graph). */
mk_status mk_plan_graph(const mk_model_desc *desc, int32_t batch, int32_t max_ctx, const mk_options *opt,
                        int32_t n_workgroups, void *buf, size_t cap, size_t *need);

/* ---- The prompt (prefill) megakernel ------------------------------------------
 * The pass that runs once per request over the whole prompt before decoding starts,
 * as its own persistent megakernel (knowledge-base digest "megakernel boundary
 * selection": prefill in its list of first-used concepts; its planner gives Llama-1B
 * a second megakernel, Figure 4, Table IV).  The same interpreter, queues and events
 * as the decode step; the tasks are RMSNorm tiles of 16 tokens, matrix-core GEMM tiles
 * (rows x 64 or 128 tokens) of the Q/K/V, O, gate/up and down projections, causal
 * attention tiles of 16 query tokens x one KV group, and LM-head tiles for the last
 * token.  Dense models with head_dim 64, hidden a multiple of 512 up to 2048, ffn_dim
 * and n_q*head_dim multiples of 128.
 *
 * Builds a prompt handle for prompts of exactly n_tokens tokens (>= 1) of one sequence
 * whose KV cache holds max_ctx >= n_tokens positions (the cache layout of a batch-1
 * decode handle with the same max_ctx, so a decode handle continues from it).
 * Options as mk_build_graph (attn_splits is ignored).  Errors: MK_E_INVALID (NULL
 * pointers, n_tokens < 1 or > max_ctx, bad options), MK_E_UNSUPPORTED (a mixture of
 * experts, head_dim other than 64, hidden above 2048 or not a multiple of 512, ffn_dim
 * or n_q*head_dim not a multiple of 128), MK_E_NO_DEVICE, MK_E_NOMEM, MK_E_HIP.
 * mk_decode_step and mk_decode_step_noalloc refuse the handle (MK_E_INVALID); the
 * other handle functions apply: mk_next_tokens gives 1 token, mk_hidden_out
 * [n_tokens rounded up to 16][hidden] (the first n_tokens rows: every prompt token's
 * final residual), mk_kv_cache_bytes the cache size, mk_export_graph the graph. */
mk_status mk_build_prefill(const mk_model_desc *desc, int32_t n_tokens, int32_t max_ctx, const mk_options *opt,
                           mk_handle **out);

/* Host-only planning of a prompt graph for `n_workgroups` workgroups, exported as
 * mk_plan_graph does (touches no GPU; weight pointers may be NULL). */
mk_status mk_plan_prefill(const mk_model_desc *desc, int32_t n_tokens, int32_t max_ctx, const mk_options *opt,
                          int32_t n_workgroups, void *buf, size_t cap, size_t *need);

/* One prompt, asynchronous on `stream`; enqueues exactly one kernel.  tokens (dev)
 * int32 [n_tokens]: the prompt, at positions pos0 .. pos0 + n_tokens - 1 (host int;
 * 0 <= pos0 <= max_ctx - n_tokens, else MK_E_INVALID); cache slots 0 .. pos0 - 1 of
 * kv_cache (dev) hold the earlier context (a longer prompt in chunks: pos0 advancing by
 * n_tokens).  Writes K/V slots pos0 .. pos0 + n_tokens - 1 of every layer, the final
 * residual of every prompt token (mk_hidden_out), the logits of the last token into
 * logits (dev, float [vocab]) unless NULL, and its greedy next token (mk_next_tokens).
 * A token outside [0, vocab) records a device error (mk_check_device_error).
 * Errors: MK_E_INVALID (NULL handle/tokens/kv_cache, a decode handle, pos0 out of
 * range), MK_E_HIP, MK_E_NOT_RESIDENT. */
mk_status mk_prefill(mk_handle *h, const int32_t *tokens, int32_t pos0, void *kv_cache, float *logits, void *stream);

/* Bytes of the KV cache the caller allocates for this handle: K then V, each
 * bf16 [n_layers][batch][n_kv][max_ctx][head_dim] (the model's attention cache;
 * the pages take the model as given). */
size_t mk_kv_cache_bytes(const mk_handle *h);

/* One decode step, asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream); enqueues exactly one kernel.  tokens (dev) int32 [batch]: the token
 * fed at this step; positions (dev) int32 [batch]: its position, i.e. the
 * number of tokens already in the cache; the step writes K/V slot
 * positions[b] of every layer of kv_cache (dev, layout of mk_kv_cache_bytes)
 * and reads slots 0..positions[b].  logits (dev) float [batch][vocab] or NULL.
 * tokens may be the pointer returned by mk_next_tokens (greedy chaining).
 * Device-side checks (token outside [0, vocab), position outside
 * [0, max_ctx), a wait exceeding debug_timeout_ms) record an error that
 * mk_check_device_error reports; outputs are then unspecified.
 * Errors: MK_E_INVALID (NULL handle/tokens/positions/kv_cache), MK_E_HIP,
 * MK_E_NOT_RESIDENT.  Defined by: one persistent kernel runs the whole forward,
 * every SM interpreting its instruction queue (Hazy Research megakernel news
 * page, section 4; koas-w.github.io notes, "on-GPU interpreter / persistent
 * kernel"); tasks wait on and increment counters in global memory (same Hazy
 * page, section 4, "synchronisation"; MPK news page, part 2). */
mk_status mk_decode_step(mk_handle *h, const int32_t *tokens, const int32_t *positions, void *kv_cache,
                         float *logits, void *stream);

/* The same step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): enqueues a small fill
 * kernel and the step kernel on `stream` and calls no hipMalloc, hipFree or allocating
 * library routine.  Arguments, outputs and errors as mk_decode_step.  The step's scratch
 * (event counters, control words, residual accumulators, query rows, attention partials,
 * m rows, operand regions, argmax keys and tickets) lives in one file-scope device array
 * of 32 MiB that each GPU running the library holds until the process ends, instead of
 * the handle's buffers; the fill kernel first clears what must start at zero (so every
 * call starts from step 1 of a fresh handle), since the array keeps whatever the last
 * call on that GPU left in it.  Calls that overlap on one GPU (on two streams, or from
 * two threads) share the array and race: the caller must order them.  The handle (built
 * by mk_build_graph) still owns the weights, task graph and outputs.  MK_E_UNSUPPORTED
 * when the handle's scratch exceeds the array (about 1.1 MiB at the 1B shape with one
 * sequence, 20 MiB with 16 sequences, 40 MiB with 32: refused).  mk_check_device_error
 * reports a device error of such a step while it is the handle's last step and no other
 * allocation-free step has run on that GPU since. */
mk_status mk_decode_step_noalloc(mk_handle *h, const int32_t *tokens, const int32_t *positions, void *kv_cache,
                                 float *logits, void *stream);

/* (dev) int32 [batch]: greedy next token of the last step (lowest index among
 * equal maximal logits), the argmax of the LM head that ends the forward (Hazy
 * Research megakernel news page, section 5: the LM head closes the forward).
 * Owned by the handle, valid until mk_destroy. */
const int32_t *mk_next_tokens(const mk_handle *h);

/* (dev) float [batch][hidden]: the final residual (before the final norm) of
 * the last step, for precision checks of the fused step against a plain
 * evaluation (cloud.baidu.com explainer, section 8).  Owned by the handle. */
const float *mk_hidden_out(const mk_handle *h);

/* (dev) int32 [n_layers][batch][top_k]: experts chosen in the last step (MoE
 * models only; NULL otherwise), the data-dependent routing decided inside the
 * step (MPK news page, outlook: dynamic routing as the open problem of static
 * task graphs; cloud.baidu.com explainer, section 2).  Owned by the handle. */
const int32_t *mk_expert_ids(const mk_handle *h);

/* Synchronises the device, then reports a device-side error of the last
 * steps: MK_OK if none, MK_E_DEVICE with a message in msg (host, cap bytes)
 * otherwise.  Clears the record and re-arms the counters so the handle can be
 * used again.  (A fused kernel is hard to debug from outside: cloud.baidu.com
 * explainer, section 8; the record names the workgroup, task and event.) */
mk_status mk_check_device_error(mk_handle *h, char *msg, size_t cap);

/* Writes the task graph of the handle (records, event targets, queues) into
 * buf (host, cap bytes) in the export format of mk_plan_graph; *need gets the
 * size.  MK_E_INVALID if cap is too small.  (The task graph: MPK news page,
 * part 1; koas-w.github.io notes, "SM-level task graph".) */
mk_status mk_export_graph(const mk_handle *h, void *buf, size_t cap, size_t *need);

/* Test hook: synchronises the device and copies the event counters (summed
 * over their sub-counters) into host (n entries) and the step epoch into
 * *epoch.  After k steps from a fresh handle, counter e equals k * target(e)
 * (counters that finishing tasks increment and waiting tasks compare with
 * their target: Hazy Research megakernel news page, section 4). */
mk_status mk_read_counters(mk_handle *h, uint32_t *host, size_t n, uint32_t *epoch);

/* Test hook: synchronises and copies per-task execution counts (n_tasks
 * entries, host) — each task runs exactly once per step (every instruction of
 * the queues executes once per forward: Hazy Research megakernel news page,
 * section 4). */
mk_status mk_read_task_counts(mk_handle *h, uint32_t *host, size_t n);

/* Trace (when built with trace=1): per task of the last step, sixteen uint64
 * values {workgroup, t_fetch, t_inputs_ready, t_staged, t_computed, t_end,
 * t_stored, t_last_page, first LDS page, t_epilogue_issued, t_epilogue_acked,
 * t_wave0_epilogue_issued, t_first_page_issued, t_last_page_issued,
 * t_last_page_published, page_wait}; times in ticks of the 100 MHz device
 * clock (the three loader stamps: 0 for a task without pages; "published":
 * loader wave 0 saw the page's loads land and handed it to the compute waves;
 * page_wait: ticks compute wave 0 spent waiting for pages, in the attention and
 * several-sequence GEMV tasks, else 0).
 * t_staged: inputs in LDS (attention: queries staged); t_computed:
 * arithmetic done (attention: all context pages folded in); t_epilogue_issued /
 * t_epilogue_acked: the last compute wave to issue its result stores / to have
 * them acknowledged by memory; t_stored: every wave done, just before the
 * signal; t_end: signal issued; t_last_page: compute wave 0 held the last of
 * its pages (0 if it had none).  n_tasks * 16 entries into host (the
 * per-phase time breakdown of the Hazy Research megakernel news page,
 * section 5). */
mk_status mk_read_trace(mk_handle *h, uint64_t *host, size_t n);

/* Frees every allocation of the handle (synchronises the device first).  NULL is a no-op. */
void mk_destroy(mk_handle *h);

/* Static text of a status code ("unknown status" for values outside mk_status). */
const char *mk_status_str(mk_status s);

/* ---- One-kernel-per-op baseline ----------------------------------------------
 * The same decode step run the conventional way, one kernel per operator
 * (embedding, RMSNorm, Q/K/V GEMVs, RoPE + KV append, attention partials and
 * merge, O-proj + residual, RMSNorm, gate/up + SiLU, down + residual, final
 * RMSNorm, LM head, argmax), for comparison: the execution model the Hazy
 * Research megakernel news page (section 3) contrasts the megakernel with.
 * Same inputs, layouts and arithmetic as the megakernel; reads the caller's
 * weights in place (no copy), so they must outlive the handle.  batch 1..64,
 * dense models only, n_q_heads / n_kv_heads <= 8.  batch 1: hidden,
 * n_q*head_dim and ffn_dim must be powers of two in [512, 8192] (vector-ALU
 * GEMVs).  batch > 1: the projections run on the matrix cores with each fp32
 * activation carried as two bf16 parts, K cut into slices whose partial sums the
 * consuming kernel adds; hidden, n_q*head_dim and ffn_dim must be multiples of
 * 256, every projection's row count a multiple of 16, and of 64 where a stacked
 * projection (Q/K/V, gate/up, LM head) has 8192 rows or more.  The KV cache,
 * tokens, positions and logits are laid out as for mk_decode_step. */
typedef struct mkb_handle mkb_handle;

/* Validates the description against the limits above and allocates the baseline's activation buffers
 * (the weights are read in place).  Errors: MK_E_INVALID (NULL pointers, batch outside 1..64, a mixture
 * of experts, head_dim other than 64 or 128), MK_E_UNSUPPORTED (projection shapes outside the limits
 * above), MK_E_NOMEM, MK_E_HIP.  (One kernel per
 * operator, a launch boundary as the only synchronisation: Hazy Research megakernel news page, section 3.) */
mk_status mkb_create(const mk_model_desc *desc, int32_t batch, int32_t max_ctx, mkb_handle **out);

/* Enqueues the step's kernels on `stream`.  tokens/positions (dev) int32 [batch]:
 * as for mk_decode_step.  When advance != 0 the last kernel also stores the
 * next tokens into tokens[] and increments every positions[b], so a graph
 * captured from one call can be replayed for consecutive greedy steps.  Errors: MK_E_INVALID (NULL
 * handle/tokens/positions/kv_cache), MK_E_HIP. */
mk_status mkb_decode_step(mkb_handle *h, int32_t *tokens, int32_t *positions, void *kv_cache, float *logits,
                          void *stream, int32_t advance);

const int32_t *mkb_next_tokens(const mkb_handle *h); /* (dev) int32 [batch] */
const float *mkb_hidden_out(const mkb_handle *h);    /* (dev) float [batch][hidden] */
int32_t mkb_launches_per_step(const mkb_handle *h);  /* kernels the last mkb_decode_step enqueued (0 before any) */
void mkb_destroy(mkb_handle *h);                     /* frees the handle; NULL is a no-op */

/* ---- Measurement microbenchmarks ----------------------------------------------
 * The costs the megakernel trades against each other, each measured on the current
 * device with its own allocations (freed before returning).  All are synchronous.
 * Errors: MK_E_INVALID for arguments outside the stated ranges, MK_E_HIP for a
 * failing HIP call, MK_E_DEVICE if a wait in the kernel gave up. */

/* Launch cost of an empty kernel: n (1..100000) launches on a new stream, then the
 * same n captured in one HIP graph and replayed; microseconds per kernel of each
 * (Hazy Research megakernel news page, section 3: per-kernel launch overhead). */
mk_status mkm_launch_latency(int32_t n, float *us_stream, float *us_graph);

/* One dependency hop between two workgroups: a counter passed back and forth
 * `rounds` times (1..10^6) through device memory with device-scope stores and
 * loads, as the megakernel's events are; nanoseconds per one-way hop.  same_xcd:
 * 0 = the workgroups sit on different XCDs, 1 = on the same one; the XCD ids
 * the two workgroups ran on are returned (Hazy Research megakernel news page,
 * section 4: the cost of one synchronisation through global memory). */
mk_status mkm_pingpong(int32_t rounds, int32_t same_xcd, float *ns_per_hop, int32_t *xcd_a, int32_t *xcd_b);

/* Nanoseconds per workgroup barrier of 384 threads, over n (1..10^7) barriers. */
mk_status mkm_barrier(int32_t n, float *ns_per_barrier);

/* LDS fill rate: n_wg (1..4096) workgroups each stream bytes_per_wg (a multiple of
 * 4096, at least 64 KiB) from device memory into LDS with direct 16-byte
 * global-to-LDS loads, depth (4, 8 or 16) loads in flight per wave; GB/s over all. */
mk_status mkm_lds_fill(uint64_t bytes_per_wg, int32_t n_wg, int32_t depth, float *gbps);

/* Plain streaming read of `bytes` (a multiple of 16, at least 1 MiB) of device
 * memory by the whole device; GB/s. */
mk_status mkm_stream_read(uint64_t bytes, float *gbps);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
