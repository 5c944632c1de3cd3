/*
 * pe.h — paged-expert MoE layer for one AMD Instinct MI355X (gfx950).
 *
 * What is computed (SGLang "Paged Experts" documentation page, sections "The
 * K-slot table and the host store", "A step: waves, page-in, merge", steps
 * 1-4, and "Captured decode"): every expert of every MoE layer lives in a
 * page-locked host store, and only K of a layer's E experts occupy its GPU
 * slot table at a time.  A forward step gathers the experts its tokens route
 * to, processes them in groups of at most K (those already in a slot go
 * first), and before each group runs, fills the group's missing experts into
 * slots whose occupants the group does not use, oldest use first.  The
 * SwiGLU FFN then runs per (token, expert) entry, scaled by the entry's
 * router weight; the entries are kept apart (per block of output rows in LDS
 * on a device-planned step, in a merged buffer on a host-planned one) until
 * one top-k sum in a fixed order makes each token's output.  That output is
 * the unpaged layer's.
 *
 * Conventions for every entry point:
 *   - Return 0 (PE_OK) on success or a negative PE_ERR_* code; no exception
 *     or abort crosses this boundary.  pe_last_error() gives a message for
 *     the calling thread's most recent failure.
 *   - "device" pointers are HIP device memory (hipMalloc, or a PyTorch CUDA
 *     tensor's data_ptr()); "host" pointers are ordinary host memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it asynchronously; the caller keeps every buffer it
 *     passes alive until that work has completed (for a captured graph: for
 *     the life of the graph).
 *   - A context is used from one stream at a time and is not re-entrant;
 *     pe_load_expert alone may be called concurrently from several host
 *     threads for distinct (layer, expert) pairs.
 */
#ifndef PE_H
#define PE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define PE_OK                   0
#define PE_ERR_INVALID_ARG     -1   /* a bad argument or configuration        */
#define PE_ERR_UNSUPPORTED     -2   /* valid request this build does not do   */
#define PE_ERR_OOM_HOST_PIN    -3   /* page-locked host allocation failed     */
#define PE_ERR_OOM_DEVICE      -4   /* device allocation failed               */
#define PE_ERR_HIP             -5   /* a HIP runtime call failed              */
#define PE_ERR_NOT_CAPTURABLE  -6   /* host-planned step under stream capture */

/* ---- expert weight formats (docs page, "Supported Configurations") ---- */
#define PE_W_BF16       0   /* unquantized bf16                                   */
#define PE_W_FP8_B128   1   /* OCP e4m3fn codes, one fp32 multiplier per 128x128  */
#define PE_W_INT4_G128  2   /* symmetric int4, one fp16 scale per 128 inputs/row  */
#define PE_W_INT8_G128  3   /* symmetric int8 (GPTQ int8), fp16 scale per 128     */
#define PE_W_MXFP4_B32  4   /* OCP MXFP4: E2M1 codes, one E8M0 scale per 32 inputs
                               of a row (the blog's added formats, gpt-oss-20b)   */

/* ---- configuration flags --------------------------------------------- */
#define PE_FLAG_PAGEIN_DMA      1u  /* host-planned steps copy with hipMemcpyAsync
                                       instead of the mapped-read page-in kernel  */
#define PE_FLAG_FORCE_HOST_PLAN 2u  /* plan every step on the host                */
#define PE_FLAG_UNPAGED         4u  /* reference mode: K = E, slot e holds expert e
                                       for good, no host store, no paging         */
#define PE_FLAG_PLAN_LOG        8u  /* keep a per-layer device ring of every step's
                                       plan (see pe_get_plan_log); needs
                                       plan_log_steps >= 1                        */

typedef struct pe_ctx pe_ctx;

typedef struct {
  int num_layers;     /* MoE layers L, each with its own slot table and LRU  */
  int num_experts;    /* routed experts per layer E (1..1024)                */
  int top_k;          /* routed experts per token k (1..E)                   */
  int num_resident;   /* slots per layer K, top_k <= K <= E (ignored, = E,
                         with PE_FLAG_UNPAGED)                               */
  int hidden;         /* H <= 4096, multiple of 128 (of 8 for bf16, of 64
                         for MXFP4)                                          */
  int inter;          /* expert SwiGLU intermediate I, same rule as H        */
  int max_tokens;     /* largest T passed to pe_forward                      */
  int device;         /* HIP device ordinal                                  */
  int wtype;          /* PE_W_*                                              */
  unsigned flags;     /* PE_FLAG_*                                           */
  int plan_log_steps; /* records per layer in the plan log (PE_FLAG_PLAN_LOG
                         only; ignored otherwise)                            */
} pe_config;

/* Counters since creation (or the last pe_reset_stats). */
typedef struct {
  uint64_t steps;            /* pe_forward calls with T > 0                        */
  uint64_t device_planned;   /* of which planned on the device (capturable path)   */
  uint64_t host_planned;     /* of which planned on the host                       */
  uint64_t waves;            /* waves run                                          */
  uint64_t page_ins;         /* experts copied host -> slot (M)                    */
  uint64_t page_in_bytes;    /* bytes those copies moved                           */
  uint64_t distinct;         /* distinct experts summed over steps (D)             */
  uint64_t entries;          /* routed (token, expert) entries                     */
  uint64_t bad_ids;          /* entries whose id was outside [0, E) (sticky error) */
} pe_stats;

/* Create a context: validates the configuration (K >= top_k as the docs'
 * "Usage" section requires, K <= E, format-dependent divisibility), allocates
 * the page-locked mapped host store (L*E expert blobs; hipHostMalloc with
 * hipHostMallocMapped; docs, "The K-slot table and the host store"), the
 * device slot tables (L*K blobs), the per-layer LRU state (reset to empty),
 * plan buffers, the plan log if asked for, and scratch sized by max_tokens.
 * On failure nothing is leaked and *out is NULL. */
int pe_create(const pe_config* cfg, pe_ctx** out);

/* Free everything pe_create allocated.  The caller must make sure no work
 * enqueued on the context is still running.  NULL is ignored. */
void pe_destroy(pe_ctx* ctx);

/* Write one expert's weights into its host-store row (docs page, "The K-slot
 * table and the host store": the weight loader writes a one-row view of the
 * host store, and host rows have the layout the GPU slots have).  All
 * pointers are host memory, row-major:
 *   PE_W_BF16:      w13 bf16 [2I, H] (gate rows 0..I-1, up rows I..2I-1),
 *                   w2 bf16 [H, I]; s13 = s2 = NULL.
 *   PE_W_FP8_B128:  w13 u8 e4m3fn [2I, H], w2 u8 [H, I], s13 fp32
 *                   [2I/128, H/128], s2 fp32 [H/128, I/128]; weight = code * s.
 *   PE_W_INT4_G128: w13 u8 [2I, H/2], w2 u8 [H, I/2] (element 2c is the low
 *                   nibble of byte c), s13 fp16 [2I, H/128], s2 fp16
 *                   [H, I/128]; weight = (nibble - 8) * s.
 *   PE_W_INT8_G128: w13 u8 [2I, H], w2 u8 [H, I], s13 fp16 [2I, H/128],
 *                   s2 fp16 [H, I/128]; weight = (byte - 128) * s.
 *   PE_W_MXFP4_B32: w13 u8 [2I, H/2], w2 u8 [H, I/2] (OCP E2M1 codes, element
 *                   2c the low nibble of byte c), s13 u8 [2I, H/32], s2 u8
 *                   [H, I/32] (OCP E8M0 scale bytes, one per row and 32
 *                   inputs); weight = e2m1(code) * 2^(scale - 127).
 * The blob holds W13 | W2 | S13 | S2 in this order, each part starting on a
 * 256-byte boundary; pe_expert_bytes gives its size.
 * The data is copied; the caller keeps ownership.  With PE_FLAG_UNPAGED the
 * blob goes straight to device slot `expert` (synchronous copy).  An expert
 * that is resident when it is reloaded keeps its old slot contents until it
 * is paged in again (call pe_reset_lru after reloading). */
int pe_load_expert(pe_ctx* ctx, int layer, int expert,
                   const void* w13, const void* w2, const void* s13, const void* s2);

/* One forward step of MoE layer `layer` over T tokens (0 <= T <= max_tokens;
 * T = 0 is a no-op):
 *   x        device bf16 [T, H]   hidden states
 *   topk_ids device int32 [T, k]  routed expert ids, E-wide (not slot ids)
 *   topk_w   device fp32 [T, k]   router weights
 *   out      device bf16 [T, H]   sum_j topk_w[t,j] * FFN_{ids[t,j]}(x[t]),
 *                                 summed in j order in fp32, rounded once
 * If T*k <= K (and PE_FLAG_FORCE_HOST_PLAN is off) the step is one wave
 * planned on the device with no host synchronisation ("Captured decode" on
 * the docs page), so the call may be captured into a hipGraph.  Otherwise
 * one launch writes the ids and the layer's LRU state into page-locked host
 * memory, the stream is synchronised once, the host plans the waves ("A
 * step: waves, page-in, merge", steps 1-2) and enqueues them; under stream
 * capture that path returns PE_ERR_NOT_CAPTURABLE without enqueuing
 * anything.  Both paths read and update one LRU state per layer, whatever
 * changed it last (an eager step, a replayed graph, a reset).
 * Entries whose id is outside [0, E) contribute 0 and are counted in
 * pe_stats.bad_ids. */
int pe_forward(pe_ctx* ctx, int layer, const void* x, const int32_t* topk_ids,
               const float* topk_w, int T, void* out, void* stream);

/* Empty the slot table of `layer` (-1: every layer): no expert resident,
 * every slot's last use 0, tick 1 -- the state of a fresh table, which the
 * pages leave unspecified (read here as empty, with no expert preloaded).
 * Used to start a measurement window cold and after reloading experts.
 * With PE_FLAG_UNPAGED the identity map is restored instead.  Enqueued on
 * `stream`; device-planned and host-planned steps both see the reset (they
 * share one LRU state per layer, docs "Captured decode").  The plan log is
 * not cleared. */
int pe_reset_lru(pe_ctx* ctx, int layer, void* stream);

/* ---- sizes and introspection (host calls) ------------------------------ */

/* Bytes of one expert blob: `algorithmic` = weights plus scales, `copied` =
 * what one page-in moves (sub-tensors 256-byte aligned).  No GPU needed. */
int pe_expert_bytes(int wtype, int hidden, int inter, size_t* algorithmic, size_t* copied);

/* Slots per layer that fit a device-memory budget: one resident expert per
 * layer costs its blob bytes times the MoE layers (docs page, "Choosing K"),
 * so K = floor(budget_bytes / (copied blob bytes x num_layers)), capped at
 * num_experts.  Returns K, or PE_ERR_INVALID_ARG if the budget holds fewer
 * than top_k slots (the method needs K >= top_k) or an argument is invalid.
 * No GPU needed. */
int pe_suggest_k(int wtype, int hidden, int inter, int num_layers, int num_experts, int top_k,
                 double budget_bytes);

/* Largest decode batch whose step is device-planned: floor(K / top_k)
 * (docs page, "Captured decode").  Returns the value, or < 0 on error. */
int pe_max_captured_batch(const pe_ctx* ctx);

/* Most waves one step can need: ceil(min(max_tokens*k, E) / K). */
int pe_max_waves(const pe_ctx* ctx);

/* Copy the LRU state of `layer` (docs, "A step: waves, page-in, merge", step
 * 2, read as: the expert in each slot, the tick of the wave that last used
 * each slot, and the layer's next tick) to host arrays (slot_expert [K]
 * int32, -1 = empty; last_use [K]; *tick).  Synchronises `stream`.  Any
 * pointer may be NULL. */
int pe_get_lru_state(pe_ctx* ctx, int layer, int32_t* slot_expert, uint32_t* last_use,
                     uint32_t* tick, void* stream);

/* The plan of wave `wave` of the most recent step of `layer` (the plan the
 * docs' "Captured decode" planner writes to device buffers: experts, slots,
 * count): *count page-ins, experts[r] copied into slots[r] evicting
 * evicted[r] (-1 = slot was empty), r < *count (arrays of K entries), and
 * *n_waves of that step.  Synchronises `stream`.  Pointers may be NULL. */
int pe_get_plan(pe_ctx* ctx, int layer, int wave, int32_t* count, int32_t* experts,
                int32_t* slots, int32_t* evicted, int32_t* n_waves, void* stream);

/* Slot each routed entry of the most recent step of `layer` ran in (the
 * slot remap of docs, "A step: waves, page-in, merge", step 3; slot_of
 * [T*k], -1 for an invalid id), T of that step.  Synchronises. */
int pe_get_slot_map(pe_ctx* ctx, int layer, int32_t* slot_of, int T, void* stream);

/* Plan log (PE_FLAG_PLAN_LOG): every step of a layer, device-planned or not,
 * captured in a graph or not, appends one record of int32 words to the
 * layer's ring of plan_log_steps records, written on the device after the
 * step's kernels (a replayed graph logs every replay).  Record layout, with
 * MW = pe_max_waves and N = max_tokens * top_k:
 *   [0] step number of the layer since pe_create (0, 1, ...), [1] T,
 *   [2] the layer's tick after the step, [3] 0,
 *   [4] n_waves, then count[MW], experts[MW*K], slots[MW*K], evicted[MW*K]
 *       (wave w's page-ins r < count[w] at [w*K + r]; entries past n_waves
 *       or count[w] are stale), then slot_of[N] (first T*k valid),
 *   then slot_expert[K] and last_use[K] after the step,
 *   padded to pe_plan_log_record_words words.
 * pe_plan_log_record_words returns that size (or < 0). */
int pe_plan_log_record_words(const pe_ctx* ctx);

/* Copy the most recent min(steps logged, plan_log_steps, max_records) records
 * of `layer`, oldest first, to `records` (max_records * record words int32,
 * host); *n_records gets the count.  Synchronises `stream`.  Returns
 * PE_ERR_INVALID_ARG without PE_FLAG_PLAN_LOG. */
int pe_get_plan_log(pe_ctx* ctx, int layer, int32_t* records, int max_records, int* n_records, void* stream);

/* Counters of the docs' "Captured decode" dispatch and of the pages'
 * byte accounting (page-ins times blob bytes; synchronises the device to read
 * the device-side ones). */
int pe_get_stats(pe_ctx* ctx, pe_stats* out);
int pe_reset_stats(pe_ctx* ctx);

/* Time `reps` host->device copies of `bytes` from page-locked host memory,
 * either with hipMemcpyAsync (use_kernel = 0) or with the mapped-read copy
 * routine the page-in kernel uses (use_kernel = 1); *gbps gets the best
 * rate in GB/s (1e9 bytes/s).  Allocates and frees its own buffers. */
int pe_link_probe(pe_ctx* ctx, size_t bytes, int use_kernel, int reps, double* gbps, void* stream);

/* The host wave planner pe_forward uses for steps that do not fit one wave,
 * run on a caller-held LRU state with no GPU (docs page, "A step: waves,
 * page-in, merge", steps 1-2).  In/out: slot_expert [K] (-1 = empty),
 * last_use [K], *tick.  Out: *n_waves, and per wave w < max_waves: counts[w]
 * page-ins, experts/slots/evicted [w*K + r] for r < counts[w]; slot_of [T*k]
 * (slot each entry ran in, -1 for an id outside [0, E)).  Returns
 * PE_ERR_INVALID_ARG if the step needs more than max_waves waves. */
int pe_plan_host(int num_experts, int num_resident, int top_k, int T, const int32_t* topk_ids,
                 int32_t* slot_expert, uint32_t* last_use, uint32_t* tick, int max_waves,
                 int32_t* n_waves, int32_t* counts, int32_t* experts, int32_t* slots,
                 int32_t* evicted, int32_t* slot_of);

/* ---- measurement ------------------------------------------------------ */
#define PE_STAGE_PLAN     0   /* (unused: planning runs inside PAGE_IN)             */
#define PE_STAGE_PAGE_IN  1   /* the launch that plans (device-planned) and pages in
                                 the missing experts with their gate/up projection
                                 while the resident ones run theirs; or a wave's
                                 page-in kernel / DMA copies                     */
#define PE_STAGE_GATE_UP  2   /* separate gate/up launches (MFMA and unpaged paths) */
#define PE_STAGE_DOWN     3   /* down projection x router weight (with the top-k
                                 sum on a device-planned step)                   */
#define PE_STAGE_TOPK_SUM 4   /* separate fixed-order top-k sum launch            */
#define PE_NUM_STAGES     5

/* While enabled, pe_forward brackets each stage's launches with a pair of
 * hipEvents on its stream (so it must not be captured).  pe_get_timing
 * synchronises, and returns per stage the number of bracketed launches and
 * their summed elapsed time in milliseconds since timing was enabled (arrays
 * of PE_NUM_STAGES; either may be NULL).  Enabling clears the sums. */
int pe_set_timing(pe_ctx* ctx, int enable);
int pe_get_timing(pe_ctx* ctx, uint64_t* launches, double* total_ms);

/* ---- a variant for callers that cannot allocate ---------------------------
 *
 * For code that must not call hipMalloc (under hipGraph capture, in tight
 * serving loops, in harnesses that forbid it): pe_forward with the step's
 * activations (the bf16 gate/up results and the fp32 merged entries) in a
 * fixed device scratch area the library holds from load time, of
 * PE_STATIC_SCRATCH_BYTES per GPU, instead of the context's buffers.  It
 * allocates nothing.  A step needs (T*top_k*inter*2 rounded up to 256) +
 * T*top_k*hidden*4 bytes; a larger step is rejected with PE_ERR_INVALID_ARG
 * and enqueues nothing.  Everything else (arguments, results, capture rules,
 * host-planned steps) is pe_forward's; stage timing is not recorded.  Every
 * call on one GPU shares that GPU's area, whatever the context: calls that
 * overlap in time on one GPU (two streams, two threads) race and give wrong
 * results.  Nothing in the area needs to start at zero. */
#define PE_STATIC_SCRATCH_BYTES (16u << 20)
int pe_forward_static(pe_ctx* ctx, int layer, const void* x, const int32_t* topk_ids,
                      const float* topk_w, int T, void* out, void* stream);

const char* pe_strerror(int status);
const char* pe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PE_H */
