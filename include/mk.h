/*
 * mk.h -- C ABI of libmk: one decode step of a mixture-of-experts transformer
 * on one MI355X (gfx950), run either as a single persistent megakernel or as a
 * per-op chain of kernel launches over the same tiles.
 *
 * What the library implements, and where the pages say it:
 *  - The whole decode step as one persistent kernel, with one resident
 *    workgroup set per compute unit for the whole step, each walking a list of
 *    small tasks prepared on the host, and counters in global memory recording
 *    when a task's inputs are ready ("Cohere Publishes One-Kernel Server for
 *    North Mini Code, Claims 1.58x vLLM Speedup", section "One resident
 *    program, many small tasks"; "Inside the Megakernel Serving Engine for
 *    North Mini Code", paragraph 4).
 *  - Tile-granular scheduling with backfill, no false dependencies, and weights
 *    loaded before a task's activation input is ready (first page, section
 *    "What the scheduling change is meant to avoid").
 *  - Tiles sharing one calling convention, built from plain tiled
 *    matrix-vector products and paged attention (first page, section "A
 *    hand-built approach to a specialized server"; second page, paragraph 5).
 *  - Continuous batching with ragged sequence lengths over a paged KV cache
 *    (first page, opening section; "Cohere fuses an entire decode step into
 *    one GPU program", paragraph 4).
 *  - The per-op chain is the conventional pipeline the pages contrast it with:
 *    one launch per operation, each waiting for the previous to drain (first
 *    page, section "The delay is between operations").
 *
 * Conventions for every entry point:
 *  - Device pointers point into memory of the device given to mk_create; the
 *    caller owns all of it (weights, KV pools, workspace, tokens, logits) and
 *    the stream. The library allocates no device memory; it owns only the
 *    handle and small pinned host staging buffers.
 *  - Host-detectable errors return synchronously and enqueue nothing.
 *    Device-detected errors (watchdog timeout, token out of range) are sticky
 *    and reported by mk_sync_check.
 *  - No C++ exception crosses this boundary. mk_last_error() returns a
 *    thread-local message for the last failing call on the calling thread.
 *  - A handle is used by one host thread at a time. Its steps may be enqueued
 *    on different streams: a step enqueued on another stream than the
 *    previous one first waits for the previous step (the workspace holds one
 *    step's inputs at a time). During a stream capture nothing is waited on:
 *    the caller orders graph replays against other steps of the handle.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MK_OK = 0,
    MK_ERR_INVALID = -1,     /* bad argument (NULL, negative size, ...) */
    MK_ERR_UNSUPPORTED = -2, /* model dims or options this build does not handle */
    MK_ERR_CAPACITY = -3,    /* batch, context, pages or workspace too small */
    MK_ERR_BAD_PAGE = -4,    /* a block-table entry the step needs is outside the pool */
    MK_ERR_HIP = -5,         /* a HIP runtime call failed (message has hipGetErrorString) */
    MK_ERR_TIMEOUT = -6,     /* device watchdog: a dependency wait exceeded its bound */
    MK_ERR_DEVICE = -7       /* device-detected bad input (token id out of range) */
} mk_status;

enum {
    MK_MODE_MEGAKERNEL = 0, /* one persistent cooperative launch per step */
    MK_MODE_PEROP = 1       /* one launch per operation level, stream-ordered */
};

/*
 * Model shape. Pre-norm decoder: RMSNorm, fused QKV projection (no bias),
 * rotate-half RoPE, grouped-query attention over a paged BF16 KV cache,
 * output projection, RMSNorm, router (optional fp32 bias) with top-k and a
 * softmax over the selected logits, SwiGLU experts, final RMSNorm and an
 * untied LM head. The pages give no architecture; this is the plainest model
 * that has every operation they name (first page, section "The delay is
 * between operations"; third page, paragraph 2).
 */
typedef struct mk_dims {
    int32_t n_layers;
    int32_t hidden;      /* H */
    int32_t n_q_heads;   /* Hq */
    int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0, Hq / Hkv <= 16 */
    int32_t head_dim;    /* D: 64 or 128 */
    int32_t n_experts;   /* E <= 256 */
    int32_t top_k;       /* k <= 8 */
    int32_t moe_inter;   /* I */
    int32_t vocab;       /* V */
    int32_t page_size;   /* P: 16 */
    float rms_eps;
    float rope_theta;
    int32_t max_batch;          /* largest B a step may use */
    int32_t max_pages_per_seq;  /* block-table row length */
    int64_t n_pages;            /* pages in each layer's pool */
} mk_dims;

/*
 * Weights: BF16 device pointers, row-major, rows = output features
 * ([out][in]). Per-layer entries are host arrays of n_layers device pointers
 * (copied at mk_create; the pointed-to memory must outlive the handle).
 *   embed [V][H], lm_head [V][H], final_norm [H]
 *   attn_norm[l] [H], wqkv[l] [(Hq + 2 Hkv) D][H] (q rows, then k, then v),
 *   wo[l] [H][Hq D], ffn_norm[l] [H], router[l] [E][H],
 *   w_gate[l], w_up[l] [E][I][H], w_down[l] [E][H][I],
 *   router_bias: NULL, or a host array of n_layers device pointers to fp32 [E].
 */
typedef struct mk_weights {
    const void* embed;
    const void* lm_head;
    const void* final_norm;
    const void* const* attn_norm;
    const void* const* wqkv;
    const void* const* wo;
    const void* const* ffn_norm;
    const void* const* router;
    const void* const* w_gate;
    const void* const* w_up;
    const void* const* w_down;
    const float* const* router_bias;
} mk_weights;

typedef struct mk_options {
    int32_t mode;            /* MK_MODE_MEGAKERNEL or MK_MODE_PEROP */
    int32_t trace;           /* nonzero: record per-task timestamps (mk_get_trace) */
    int64_t watchdog_ns;     /* bound on each dependency wait; 0 = 2 s */
    int32_t wg_per_cu;       /* persistent workgroups per compute unit; 0 = auto */
    int32_t split_kv_tokens; /* attention chunk length in tokens (multiple of 64); 0 = auto */
    int32_t n_cu_override;   /* 0 = the device's compute-unit count */
    int32_t time_kernels;    /* nonzero: bracket each step's kernels with HIP events (mk_kernel_time) */
    int32_t shared_levels;   /* batches of 3+, megakernel mode: levels whose tiles workgroups claim from a
                                pool (claim tasks, see mk_plan_build) instead of fixed per-workgroup
                                lists. 0 = the attention, merge, output-projection and expert levels when
                                the sequences need different numbers of attention chunks, else none;
                                1 = the attention level; 2 = those five levels always; -1 = none */
    int32_t validate_plans;  /* nonzero: check every plan mk_decode_step builds with the same checks as
                                mk_plan_build before using it (MK_ERR_INVALID if one fails) */
    int32_t mfma_min_batch;  /* smallest batch run by the matrix-core schedule (every weight product on
                                MFMA, a routing level and an expert-sum level); smaller batches run the
                                one- and two-token schedule (GEMV tiles on packed BF16 dot products).
                                0 = 3; 1..3 allowed: the one- and two-token kernels are compiled for
                                exactly one or two tokens, so the threshold can be lowered, not raised */
    int32_t poison_exchange; /* debug: nonzero fills the buffers that carry floating-point data between
                                tiles (activations, query/key/value rows, attention partials, router
                                logits, expert activations and outputs) with NaN before each step, with a
                                fill kernel on the step's stream. A tile that read such data before its
                                producer wrote it in this step would turn the step's outputs into NaN;
                                with every read covered by a wait, outputs are bit-identical to a step
                                without it (the pages' counters mark inputs ready: "Cohere Publishes
                                One-Kernel Server for North Mini Code, Claims 1.58x vLLM Speedup",
                                "One resident program, many small tasks"). Costs the fill (up to the
                                attention partials' size) per step. */
    int32_t mm_row_blocks;   /* batches of 3+: row blocks per expert tile (8-row blocks of the expert width
                                per gate/up tile, 16-row blocks of the hidden size per down tile), so that
                                a wave multiplies one load of its tokens' activations by that many blocks
                                of an expert's weights. 0 = choose per step (2 when the expected number of
                                distinct experts gives each wave of a tile about two slots, else 1); 1 or 2
                                force it. Results are bit-identical either way: each output row sums the
                                same products in the same order. */
    int32_t reserved0;       /* must be 0 */
} mk_options;

typedef struct mk_handle mk_handle;

/*
 * KV pool layout, one K pool and one V pool per model, each n_layers *
 * n_pages pages of Hkv heads:
 *   K: [L][n_pages][Hkv][P][D]  BF16 (token-major inside a page)
 *   V: [L][n_pages][Hkv][D][P]  BF16 (dimension-major inside a page)
 * Token t of a sequence with block table bt lives in page bt[t / P], slot
 * t % P: the paged KV cache of "Cohere Publishes One-Kernel Server for North Mini Code, Claims 1.58x vLLM Speedup",
 * opening section. Returns the bytes of one pool (K and V are the same size).
 */
size_t mk_kv_pool_bytes(const mk_dims* dims);

/* Bytes of device workspace mk_create needs for these dims and options: the
 * counters in global memory and the task lists of the resident program (same
 * page, section "One resident program, many small tasks"), the exchanged
 * activations and attention partials. 0 on bad input. */
size_t mk_workspace_bytes(const mk_dims* dims, const mk_options* opts);

/*
 * Create a handle on `device` (HIP ordinal): the state of the one resident
 * program that runs every step ("Cohere Publishes One-Kernel Server ...",
 * section "One resident program, many small tasks"). Validates the dims,
 * queries the device, carves `workspace` (device memory of at least mk_workspace_bytes,
 * 256-byte aligned, owned by the caller) and clears its counters with a
 * synchronous launch on the null stream. Returns MK_ERR_UNSUPPORTED for dims
 * outside the supported set and MK_ERR_CAPACITY for a short workspace.
 */
mk_status mk_create(const mk_dims* dims, const mk_weights* weights, void* k_pool, void* v_pool,
                    void* workspace, size_t workspace_bytes, const mk_options* opts, int device,
                    mk_handle** out);

/*
 * Enqueue one decode step for `batch` sequences on `stream` and return: the
 * whole step, embedding to logits, as one launch of the resident program
 * ("Cohere Publishes One-Kernel Server ...", section "One resident program,
 * many small tasks"; "Cohere fuses an entire decode step into one GPU
 * program", paragraphs 1-2), or as the per-op chain (mk_set_mode).
 *   seq_ids      host [B]: distinct ids (tracing only)
 *   positions    host [B]: tokens already cached; the new token's KV goes to
 *                that position and attention covers positions 0..positions[b]
 *   block_tables host [B][max_pages_per_seq]: page ids; entries past
 *                positions[b] / P are ignored
 *   tokens       device int32 [B]: input token ids
 *   logits       device fp32 [B][V]: output
 * Host errors (bad page, capacity, ...) return before anything is enqueued.
 * The step is idempotent given (KV pool, positions, block tables, tokens):
 * it writes its KV slot before reading it.
 */
mk_status mk_decode_step(mk_handle* h, int32_t batch, const int32_t* seq_ids,
                         const int32_t* positions, const int32_t* block_tables,
                         const int32_t* tokens, float* logits, void* stream);

/*
 * Enqueue one multi-token step: a batch whose rows may feed several new
 * tokens of one sequence at once (a prompt block being ingested, or a mix of
 * prompt blocks and decode rows). The pages' server admits new requests into
 * a running batch over a paged KV cache ("Cohere Publishes One-Kernel Server
 * for North Mini Code, Claims 1.58x vLLM Speedup", opening section; "Cohere
 * fuses an entire decode step into one GPU program", paragraph 4), so a
 * prompt's tokens have to reach the cache through the same kernel; they are
 * computed causally, which is exactly sequential decoding of those tokens.
 *   seq_ids      host [B], required: rows with equal ids must be adjacent, at
 *                consecutive positions, with equal block-table entries over
 *                the pages they share; distinct runs have distinct ids
 *   positions, block_tables, tokens, logits: as for mk_decode_step, per row
 * Row b writes the KV slot at positions[b] and attends over positions
 * 0..positions[b] of its sequence: the cached prefix plus the rows of its run
 * up to itself. Every row gets its logits. Runs of one row are decode rows,
 * so mk_decode_step is this call with distinct seq_ids. Errors as for
 * mk_decode_step, plus MK_ERR_INVALID for a malformed run.
 */
mk_status mk_forward_step(mk_handle* h, int32_t batch, const int32_t* seq_ids,
                          const int32_t* positions, const int32_t* block_tables,
                          const int32_t* tokens, float* logits, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): mk_decode_step with the
 * step's counters and exchange buffers (the residual stream, attention
 * partials, router logits, expert activations and the like) in the library's
 * static device scratch instead of the handle's workspace. Same arguments,
 * same results (the same kernels and plan), and like every step it calls no
 * hipMalloc, hipFree, hipHostMalloc or other device or pinned allocator; the
 * plan's host bookkeeping uses ordinary heap memory.
 *  - The scratch is 64 MiB per device, held from the library's first use on
 *    that device until the process ends. A handle whose step needs more
 *    (mk_workspace_bytes minus the task tables, about the per-layer
 *    attention partials for its max_batch and max_pages_per_seq) gets
 *    MK_ERR_CAPACITY, before anything is enqueued.
 *  - Every call on a device shares that device's scratch, which keeps the
 *    last call's contents; each call clears the counters it needs with a
 *    fill kernel on `stream`. Calls that overlap on one device (other
 *    streams, other handles) race: order them.
 *  - mk_get_debug_ptrs refers to the handle's workspace, not to the scratch.
 */
mk_status mk_decode_step_noalloc(mk_handle* h, int32_t batch, const int32_t* seq_ids,
                                 const int32_t* positions, const int32_t* block_tables,
                                 const int32_t* tokens, float* logits, void* stream);

/* Switch between MK_MODE_MEGAKERNEL and MK_MODE_PEROP for later steps. The
 * per-op mode is the conventional chain of one kernel per operation that the
 * pages measure against ("Cohere Publishes One-Kernel Server ...", section
 * "The delay is between operations"), running the same tiles. */
mk_status mk_set_mode(mk_handle* h, int32_t mode);

/* Synchronize `stream`, then report and clear the device error word:
 * MK_OK, MK_ERR_TIMEOUT or MK_ERR_DEVICE. Not an operation of the pages (they
 * describe no error handling): the boundary's report of a watchdog timeout on
 * a counter wait, a token out of range or a task the kernel cannot run. */
mk_status mk_sync_check(mk_handle* h, void* stream);

/*
 * Device addresses of per-step results kept in the workspace, for checking
 * and tracing (not an operation of the pages: parity and tracing access to
 * the exchange buffers the resident program's tiles pass between them).
 * Valid until mk_destroy; contents refer to the last step.
 * Slices are padded: pad64(n) is n rounded up to a multiple of 64 floats.
 *   x_layers: fp32 [2L + 1] slices of stride pad64(max_batch * H), each
 *             [max_batch][H]: the residual stream; slice 0 is the embedding,
 *             2l + 1 the residual after layer l's attention block, 2l + 2
 *             after its MoE block
 *   route_ids: int32 [L][max_batch][k], route_w: fp32 [L][max_batch][k]
 *   router_logits: fp32 [L] slices of stride pad64(max_batch * E)
 */
typedef struct mk_debug_ptrs {
    const float* x_layers;
    const int32_t* route_ids;
    const float* route_w;
    const float* router_logits;
    const uint64_t* trace;   /* see mk_get_trace */
    int64_t trace_capacity;  /* records */
} mk_debug_ptrs;
mk_status mk_get_debug_ptrs(mk_handle* h, mk_debug_ptrs* out);

/*
 * Task-graph plan of the last step, copied to host memory. Each task record
 * is 12 int32: {op, layer, a0, a1, a2, a3, pre_ctr, pre_target, ctr, target,
 * signal, level}; `wg_offsets` has n_wg + 1 entries (CSR: tasks of workgroup
 * w are [wg_offsets[w], wg_offsets[w + 1])). Pass NULL buffers to query sizes.
 * Batches of 3+: tasks of op 11 (claim) in a workgroup's list stand for the
 * tiles of one level held in a pool: tasks [a0, a0 + a1), which follow all
 * the lists (from wg_offsets[n_wg] on); the workgroups holding a claim task
 * for the level take the pool's tiles in order until none is left.
 */
typedef struct mk_plan_info {
    int32_t n_wg;
    int32_t n_tasks;
    int32_t n_counters;
    int32_t n_levels;
    int32_t chunk_tokens;
    int32_t cap_tasks; /* tasks a handle of these dims and options reserves for
                          any batch on at most n_wg workgroups (n_tasks <= it) */
    int32_t reserved[2];
} mk_plan_info;

/*
 * Build a plan on the host without a device or handle (CPU testing of the
 * task-graph builder): the per-workgroup task lists and counter targets the
 * host prepares for the resident program ("Cohere Publishes One-Kernel Server
 * for North Mini Code, Claims 1.58x vLLM Speedup", section "One resident
 * program, many small tasks"). `n_wg` workgroups; positions host [batch].
 * `tasks` (12 * n_tasks int32), `wg_offsets` (n_wg + 1 int32) and
 * `counter_targets` (n_counters int32: the value each counter reaches when
 * the step completes) may be NULL to query sizes; `cap_tasks` bounds tasks.
 */
mk_status mk_plan_build(const mk_dims* dims, const mk_options* opts, int32_t n_wg, int32_t batch,
                        const int32_t* positions, mk_plan_info* info, int32_t* tasks,
                        int64_t cap_tasks, int32_t* wg_offsets, int32_t* counter_targets);

/*
 * Check a task table against the plan builder's invariants without a
 * device: the table (12 int32 per task, as mk_plan_build writes it) and
 * per-workgroup offsets for n_wg workgroups, for this batch and these
 * positions. MK_OK, or MK_ERR_INVALID with the first violated rule in
 * mk_last_error: counter targets equal to their producer counts, every wait
 * on a lower level, workgroup lists in level order (deadlock freedom with
 * all workgroups resident), each operation's output covered exactly once,
 * and read coverage: every range a tile reads (residual stream, QKV rows of
 * its KV group, attention partials of its head, routing, expert
 * activations) is written by tiles whose completion its waits imply,
 * directly or through the waits of the tiles it waits on. This is the "no
 * missing dependency" property of tile-level scheduling ("Cohere Publishes
 * One-Kernel Server for North Mini Code, Claims 1.58x vLLM Speedup",
 * section "What the scheduling change is meant to avoid").
 */
mk_status mk_plan_check(const mk_dims* dims, const mk_options* opts, int32_t n_wg, int32_t batch,
                        const int32_t* positions, const int32_t* tasks, int64_t n_tasks,
                        const int32_t* wg_offsets);

/*
 * Per-task timestamps of the last step (when mk_options.trace was set), the
 * measure of the idle time between dependent tiles that the scheduling change
 * targets ("Cohere Publishes One-Kernel Server ...", section "What the
 * scheduling change is meant to avoid"): one
 * record of 8 uint64 per task, {task index | workgroup << 32, t_start,
 * t_after_wait, four phase stamps inside the tile (0 if unused), t_end}, in
 * the device's constant wall clock (100 MHz ticks).
 */
mk_status mk_get_trace(mk_handle* h, void* host_buf, size_t bytes, size_t* written);

/*
 * Task table of the plan the last step ran (the host-prepared task list of
 * "Cohere Publishes One-Kernel Server ...", section "One resident program,
 * many small tasks"): the records that the task
 * indices of mk_get_trace refer to, 12 int32 each as for mk_plan_build, in
 * the order the last step's kernels indexed them (grouped per workgroup in
 * the megakernel mode, per dependency level in the per-op mode). Host work
 * only. *n_tasks is always set; with tasks NULL nothing is copied.
 * Errors: MK_ERR_INVALID (null handle or n_tasks, no step run yet),
 * MK_ERR_CAPACITY (tasks non-NULL and cap_tasks < *n_tasks; nothing copied).
 */
mk_status mk_get_plan(mk_handle* h, int32_t* tasks, int64_t cap_tasks, int64_t* n_tasks);

/*
 * Device time of the last step's kernels in milliseconds (the step time
 * behind the pages' speed-of-light accounting, "Inside the Megakernel
 * Serving Engine for North Mini Code", paragraph 2), from HIP events
 * recorded on the step's stream immediately before the first and after the
 * last kernel of the step (per-step staging copies excluded). Needs
 * mk_options.time_kernels; waits for the step to finish.
 */
mk_status mk_kernel_time(mk_handle* h, float* ms);

/* Release the handle: its pinned staging, events and host plan. The caller's
 * device buffers are untouched. Not an operation of the pages (handle
 * lifetime). NULL is a no-op. */
void mk_destroy(mk_handle* h);

/* Thread-local message of the calling thread's last failing call (never
 * NULL). Not an operation of the pages (the boundary's error text). */
const char* mk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
