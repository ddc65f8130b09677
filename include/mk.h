/*
 * mk.h -- C ABI of the MI355X decode-step megakernel library (libmk.so).
 *
 * What it computes: one autoregressive decode step of a transformer LLM
 * (embedding row -> per layer: RMSNorm, QKV projection, rotary embedding,
 * attention over the paged KV cache, O projection + residual, RMSNorm,
 * SwiGLU MLP or softmax top-k MoE + residual -> final RMSNorm, LM head,
 * greedy argmax).  The Cohere megakernel article ("Egyetlen tartós kernelre
 * épül a kiszolgálás") describes running that whole forward pass as one
 * persistent kernel with one resident block per SM, working from a task list
 * prepared on the host, with data dependencies signalled through counters in
 * global memory; the Mirage MPK summary ("Part 1. Compiler", "Part 2.
 * Runtime") describes the same split into a compiler that lowers the graph
 * into fine-grained tasks and events, and a runtime whose workers run tasks
 * and bump event counters.  This library is that design for one MI355X:
 * mk_build_plan is the host-side lowering, mk_decode_step launches the
 * persistent kernel (one workgroup per CU).
 *
 * Conventions
 *  - Every pointer named *_dev or held in mk_weights / mk_kv is a device
 *    pointer (HIP device memory of the plan's device).  The caller owns all of
 *    them; the library never frees them and never writes weights.
 *  - bf16 = IEEE bfloat16 bit patterns (uint16).  Matrices are row-major
 *    [out_features][in_features]; a projection is y = W x.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls that take a stream are asynchronous and stream-ordered; they do
 *    not synchronise the host (mk_plan_status excepted).
 *  - Functions return MK_OK (0) or a negative MK_ERR_* code; the message of
 *    the last failure on the calling thread is returned by mk_last_error().
 *    No C++ exception crosses this boundary.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MK_OK = 0,
  MK_ERR_INVALID_CONFIG = -1, /* model shape the library cannot plan        */
  MK_ERR_INVALID_ARG = -2,    /* bad pointer / size / index argument          */
  MK_ERR_HIP = -3,            /* a HIP runtime call failed                    */
  MK_ERR_OOM = -4,            /* device allocation failed                     */
  MK_ERR_PLAN = -5,           /* planner produced an invalid task graph       */
  MK_ERR_TIMEOUT = -6,        /* a device-side dependency wait hit its budget */
  MK_ERR_UNSUPPORTED = -7     /* valid request outside what is implemented    */
};

/* Executors.  PERSISTENT: one launch per step, grid = one workgroup per CU,
 * each workgroup running its own planner-assigned queue of tasks in list
 * order, ordered across workgroups by HBM event counters.
 * KERNEL_PER_OP: the same task code, one launch per operation of each layer,
 * stream order standing in for the counters (the launch-overhead baseline).
 * SCHEDULED: the MPK runtime's other design (MPK summary, "Part 2. Runtime":
 * Worker, Scheduler, event-based execution): one launch per step; workgroup 0
 * holds four scheduler wavefronts, every other workgroup is a worker with a
 * task queue in HBM.  A worker runs the tasks dispatched to its queue in
 * arrival order and bumps their events' counters; the task that completes an
 * event activates it into a scheduler's queue; the scheduler counts the event
 * for each dependent task and dispatches the tasks whose events have all
 * fired.  Single-slot and vector multi-slot plans (no matrix-core tiles). */
enum { MK_EXEC_PERSISTENT = 0, MK_EXEC_KERNEL_PER_OP = 1, MK_EXEC_SCHEDULED = 2 };

/* Task operations (values of mk_task_info.op). */
enum {
  MK_OP_EMBED = 1, MK_OP_QKV = 2, MK_OP_ATTN = 3, MK_OP_MERGE = 4,
  MK_OP_OPROJ = 5, MK_OP_GATEUP = 6, MK_OP_DOWN = 7, MK_OP_ROUTER = 8,
  MK_OP_TOPK = 9, MK_OP_EGATEUP = 10, MK_OP_EDOWN = 11, MK_OP_COMBINE = 12,
  MK_OP_LMHEAD = 13, MK_OP_ARGMAX = 14, MK_OP_KVAPP = 15
};

/* Model shape and capacity.  n_experts == 0 selects the dense SwiGLU MLP
 * (ffn_dim used); n_experts > 0 selects the MoE MLP (top_k, expert_ffn_dim).
 * max_batch: decode slots per step.  page_size must be 16.
 * max_pages_per_seq: columns of the page table.  n_pages: pages in each pool. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps;
  double rope_theta;
  int32_t n_experts, top_k, expert_ffn_dim;
  int32_t max_batch, page_size, max_pages_per_seq, n_pages;
} mk_config;

/* Device pointers to the weights (bf16).  Per-layer tensors are given by a
 * host array of n_layers device pointers; expert tensors by a host array of
 * n_layers*n_experts pointers indexed [layer*n_experts + expert].  Shapes:
 *   embed, lm_head [vocab][hidden]; final_norm, attn_norm[l], ffn_norm[l]
 *   [hidden]; wq[l] [n_q_heads*head_dim][hidden]; wk[l], wv[l]
 *   [n_kv_heads*head_dim][hidden]; wo[l] [hidden][n_q_heads*head_dim];
 *   dense: w_gate[l], w_up[l] [ffn_dim][hidden], w_down[l] [hidden][ffn_dim];
 *   MoE: router[l] [n_experts][hidden]; e_gate, e_up [expert_ffn][hidden];
 *   e_down [hidden][expert_ffn].  Unused members may be NULL.
 * The host arrays are copied during mk_build_plan. */
typedef struct {
  const void *embed, *lm_head, *final_norm;
  const void *const *attn_norm, *const *ffn_norm;
  const void *const *wq, *const *wk, *const *wv, *const *wo;
  const void *const *w_gate, *const *w_up, *const *w_down;
  const void *const *router, *const *e_gate, *const *e_up, *const *e_down;
} mk_weights;

/* Paged KV cache (caller-owned), bf16.  k_pool:
 * [n_layers][n_pages][n_kv_heads][page_size][head_dim]; v_pool:
 * [n_layers][n_pages][n_kv_heads][head_dim][page_size] (values transposed
 * within a page: the 16 positions of one dimension are contiguous, the
 * operand layout of the matrix-core attention products).  page_table: device
 * int32 [max_batch][max_pages_per_seq]; entry [b][j] is the pool page holding
 * positions 16j..16j+15 of slot b.  The caller may edit page_table and the
 * pools between steps (sequences joining / retiring). */
typedef struct {
  void *k_pool, *v_pool;
  int32_t *page_table;
} mk_kv;

typedef struct {
  int32_t executor;      /* MK_EXEC_*                                        */
  int32_t n_workgroups;  /* persistent workers (grid size); 0 = number of CUs.
                            All must be resident at once (cooperative launch) */
  int32_t attn_splits;   /* KV splits per (sequence, KV head); 0 = auto       */
  int32_t planned_ctx;   /* context the auto split is sized for; 0 = capacity */
  int32_t debug_trace;   /* 1: per-task start/finish tickets (serialising) and
                            times; 2: per-task times only                    */
  int32_t device;        /* HIP device ordinal; -1 = current device            */
  int64_t spin_budget;   /* dependency-wait budget in 100 MHz ticks; 0 = 1 s   */
  int32_t n_cus;         /* override the CU count used for tile sizing; 0 = query */
  int32_t graph_replay;  /* 1: every step first clears the plan's counters with a
                            kernel and counts from zero, so a step captured in a
                            HIP graph can be replayed; 0: counters stay
                            monotonic across steps (no clearing launch)       */
  int32_t batched_mfma;  /* static-weight GEMVs as bf16 matrix-core tiles for
                            batches of up to 64 slots: 0 = auto (on when
                            max_batch >= 3 and every row count is a multiple
                            of 16), 1 = on from 2 slots, -1 = off (vector
                            path)                                            */
  int32_t attn_pool;     /* persistent executor: attention tasks of a layer are
                            claimed at run time from a shared counter by the
                            workers that reach them (balances sequences of
                            different lengths): 0 = auto (on when a layer has
                            more attention tasks than workers), 1 = on,
                            -1 = off (static placement)                       */
  int32_t weight_lds;    /* single-slot plans: stream part of every weight pass
                            through LDS (more weights in flight across each
                            dependency wait), possible when the staged
                            activations fit 72 KiB: 0 = auto (dense models),
                            1 = on, -1 = off                                 */
  int32_t debug_withhold; /* test hook: list index + 1 of one task whose counter
                            signals the persistent executor withholds, so the
                            waits on them end in MK_ERR_TIMEOUT after
                            spin_budget (every workgroup still exits); cleared
                            by the mk_plan_status call that reports the error.
                            0 = none                                         */
  int32_t shared_seqs;   /* 1: several slots of one step may hold one sequence
                            (a prompt chunk at consecutive positions, mixed
                            with other sequences' decode tokens: see
                            mk_batch_step); every slot's key and value are
                            stored before the layer's attention reads the
                            cache.  0: each slot holds its own sequence      */
  int32_t prefill_chunk; /* mk_prefill: prompt tokens per launch, run as the
                            slots of an internal shared-sequence plan of that
                            many slots (matrix-core tiles at 16..64): 0 = auto
                            (64 when the model's row counts allow matrix-core
                            tiles, else token by token), -1 = one token per
                            decode step, 16..64 = that many                  */
  int32_t attn_order;    /* claim order of pooled attention tasks (plans with
                            claimed attention, at most 64 slots): 0 = auto
                            (= 1); 1 = longest context first (throughput: the
                            layer's last claims are its shortest tasks);
                            2 = higher mk_batch_step priority first, then
                            longest context (latency targets of some
                            sequences ahead of others); -1 = slot order      */
} mk_plan_options;

typedef struct mk_plan mk_plan;

/* Fill *opts with defaults (persistent executor, auto sizes).  opts NULL is
 * ignored. */
void mk_plan_options_default(mk_plan_options *opts);

/* The host-side lowering (MPK summary, "Part 1. Compiler": the computation
 * graph becomes a task graph of per-tile tasks joined by events; Cohere,
 * "Egyetlen tartós kernelre épül a kiszolgálás": the blocks work from a task
 * list prepared on the host, dependencies signalled by counters in global
 * memory): lower the model into a task list, validate it, allocate the
 * plan's device state (task table, event counters, activation scratch, RoPE
 * table) on the device and upload it.  Synchronous.  *out receives the plan
 * (free with mk_free); the plan keeps pointers to the caller's weights, pools
 * and page table, which must outlive it.  opts may be NULL.  Errors:
 * MK_ERR_INVALID_ARG (NULL or unaligned pointers, bad options),
 * MK_ERR_INVALID_CONFIG / MK_ERR_UNSUPPORTED (shapes the kernels cannot run),
 * MK_ERR_OOM, MK_ERR_HIP; *out is NULL on failure. */
int mk_build_plan(const mk_config *cfg, const mk_weights *w, const mk_kv *kv,
                  const mk_plan_options *opts, mk_plan **out);

/* For callers that cannot allocate device memory (steps under HIP graph
 * capture, serving loops that forbid allocation): mk_build_plan without any
 * device allocation.  The plan's device state (task table, counters,
 * activation scratch, RoPE table) is placed in the library's static scratch
 * array of 32 MiB, which every device the library runs on holds until the
 * process ends; a plan that needs more is refused with MK_ERR_UNSUPPORTED.
 * Calls no hipMalloc / hipFree (host-side planning uses the C++ heap) and
 * synchronises the device first.  There is one such array per device, so
 * building another plan this way replaces the state of the previous one on
 * that device: steps of the older plan then fail with MK_ERR_INVALID_ARG, and
 * steps of two such plans that overlap on one device would race.
 * mk_free releases only the host side. */
int mk_build_plan_noalloc(const mk_config *cfg, const mk_weights *w, const mk_kv *kv,
                          const mk_plan_options *opts, mk_plan **out);

/* One decode step for all max_batch slots, as one launch of the persistent
 * kernel (Cohere, "Egyetlen tartós kernelre épül a kiszolgálás": one resident
 * block per SM runs the whole forward pass from the task list; MPK summary,
 * "Part 2. Runtime": workers run their task queues and bump event counters).
 * Asynchronous on `stream`; returns MK_ERR_INVALID_ARG for NULL required
 * pointers; device-side errors (a token outside the vocabulary, a position
 * beyond the page table, a page id outside the pool, a dependency wait past
 * its budget) are reported by mk_plan_status.
 *  tokens_dev[b]     input token of slot b (int32, device)
 *  positions_dev[b]  0-based position of that token (= number of tokens
 *                    already cached for the slot); < 0 marks an empty slot
 *  next_tokens_dev   out: greedy argmax per slot (-1 for empty slots)
 *  logits_dev        out, optional (NULL): fp32 [max_batch][vocab]
 * The step writes the slot's key/value at `position` into the page given by
 * page_table[b][position/16].  tokens_dev may alias next_tokens_dev.  */
int mk_decode_step(mk_plan *plan, const int32_t *tokens_dev,
                   const int32_t *positions_dev, void *stream,
                   int32_t *next_tokens_dev, float *logits_dev);

/* One step of a mixed batch (MPK summary, "भविष्य की दिशा", and Cohere,
 * "Folyamatos batchkezelés": chunked prefill beside decode in one launch):
 * slot b feeds tokens_dev[b] at position positions_dev[b] (< 0: empty) of the
 * sequence whose pages are page_table row seq_rows_dev[b] (device int32
 * [max_batch], each in [0, max_batch)).  Several slots may name one row --
 * the consecutive positions of a prompt chunk of that sequence, each attending
 * causally to everything before it including the chunk's earlier tokens --
 * only in plans built with shared_seqs = 1; otherwise the rows must be
 * distinct.  priorities_dev (optional, device int32 [max_batch], higher =
 * more urgent) orders the claimed attention tasks of plans built with
 * attn_order = 2 (MPK summary, "भविष्य की दिशा": priority-based task
 * scheduling); it changes no result.  Outputs as mk_decode_step (per slot). */
int mk_batch_step(mk_plan *plan, const int32_t *tokens_dev, const int32_t *positions_dev,
                  const int32_t *seq_rows_dev, const int32_t *priorities_dev, void *stream,
                  int32_t *next_tokens_dev, float *logits_dev);

/* Feed n prompt tokens tokens_dev[0..n) of one slot at positions
 * start_pos..start_pos+n-1, filling its KV pages (other slots are left
 * untouched): the full causal forward over the prompt (MPK summary, "MPK का
 * मुख्य मूल्य": the prompt before greedy decoding).  With prefill_chunk
 * enabled the prompt runs in chunks of up to that many tokens, each chunk one
 * launch of an internal shared-sequence plan whose projections are
 * matrix-core tiles with the chunk's tokens as the M dimension; otherwise one
 * decode step per token.  next_token_dev (optional) receives the greedy token
 * after the last prompt token, logits_dev (optional) its fp32 logits [vocab].
 * Device-side errors of the chunks are reported by mk_plan_status. */
int mk_prefill(mk_plan *plan, int32_t slot, const int32_t *tokens_dev,
               int32_t n, int32_t start_pos, void *stream,
               int32_t *next_token_dev, float *logits_dev);

/* Synchronise `stream` and report a device-side error of this plan's last
 * steps (MK_ERR_TIMEOUT when a dependency wait exceeded its budget, the
 * message naming the task and the event; MK_ERR_INVALID_ARG for a bad token,
 * position, page id or page-table row).  The error is cleared and the plan's
 * counters are reset, so the next step runs normally.  The event-counter
 * protocol it watches is the MPK summary's ("Part 2. Runtime", event-based
 * execution: a finished task bumps its event's counter, the event fires at
 * its threshold). */
int mk_plan_status(mk_plan *plan, void *stream);

/* Release everything the plan allocated (after synchronising its device).
 * The caller's weights, pools and page table are untouched.  NULL is
 * ignored. */
void mk_free(mk_plan *plan);

/* Message of the last failing call on this thread ("" if none). */
const char *mk_last_error(void);

/* Hash of the sources the library was built from (16 hex digits), so a
 * caller can refuse a library built from other sources. */
const char *mk_build_id(void);

/* ---- introspection (host only; no GPU needed) ----------------------------
 * The task graph of the MPK summary's "Part 1. Compiler" (tasks, events and
 * the edges between them) as the planner builds it.
 * mk_inspect_plan runs the planner for `cfg` with opts->n_cus CUs and
 * opts->n_workgroups workers (0: 256 each) without touching a device and
 * copies the task graph into caller arrays (cap = capacity in elements;
 * *n_tasks / *n_events receive the true counts even when they exceed the
 * capacity).  Event thresholds are per step. */
typedef struct {
  int32_t op, layer, a0, a1, a2, a3, a4;
  int32_t sig_count;         /* completions reported (0: reported by a later
                                task of the same worker's run)               */
  int32_t n_wait, wait_ev[3];
  int32_t n_sig, sig_ev[2];
  int32_t phase;             /* launch index under KERNEL_PER_OP            */
  int32_t worker;            /* persistent workgroup whose queue holds it   */
  int32_t rows_per_pass;     /* static-weight GEMVs: rows streamed per pass
                                (one register tile); 0 for other tasks       */
  int64_t bytes;             /* algorithmic HBM bytes this task reads       */
  int32_t data_edges;        /* bit k (k < 3): wait k is a data edge (the
                                inputs carry the step's tag; no counter is
                                polled); bit 3 + k: signal k is (the outputs
                                are tagged; no counter is incremented)       */
  int32_t pad_;
} mk_task_info;

int mk_inspect_plan(const mk_config *cfg, const mk_plan_options *opts,
                    mk_task_info *tasks, int32_t task_cap, int32_t *n_tasks,
                    int32_t *ev_thresholds, int32_t ev_cap, int32_t *n_events);

/* Persistent-executor trace of the last step run with debug_trace = 1:
 * per task {start ticket, finish ticket, run count, workgroup,
 * deps-ready time, finish time (100 MHz ticks, low 32 bits)}, 6 x uint32
 * each (debug_trace = 2: words 0 and 1 hold intermediate times instead of
 * tickets).  The check it serves: every task runs once, after every producer
 * of its inputs (MPK summary, "Part 2. Runtime").  Synchronises `stream`.
 * cap in tasks.  MK_ERR_INVALID_ARG for a plan built without debug_trace. */
int mk_read_trace(mk_plan *plan, void *stream, uint32_t *out, int32_t cap);

/* MoE plans (Cohere, "Honnan jön a gyorsulás?": the router, then each expert
 * down projection after its experts' up projections): the expert ids (int32)
 * and renormalised routing weights (fp32)
 * the last step chose, [n_layers][max_batch][top_k] each, ids ascending per
 * (layer, slot).  Synchronises `stream`; cap in entries; either output may be
 * NULL.  MK_ERR_INVALID_ARG for a dense model. */
int mk_read_routing(mk_plan *plan, void *stream, int32_t *ids, float *weights, int32_t cap);

/* Number of tasks and events of a built plan, the number of CUs it was
 * sized for (the wave-quantization target of Cohere, "Honnan jön a
 * gyorsulás?") and its launches per step under KERNEL_PER_OP.  Any output
 * may be NULL. */
int mk_plan_info(const mk_plan *plan, int32_t *n_tasks, int32_t *n_events,
                 int32_t *n_cus, int32_t *n_phases);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
