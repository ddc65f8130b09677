// mk_task.h -- task table, device-side plan state and sizing constants shared
// by the host planner (planner.cpp), the C ABI (capi.cpp) and the device code
// (kernels.hip).  Plain C++: no HIP types, so the planner builds without HIP.
//
// Design (Mirage MPK summary, "Part 1. Compiler" / "Part 2. Runtime"; Cohere
// megakernel article, "Egyetlen tartós kernelre épül a kiszolgálás"): the
// host lowers a decode step into tasks, each one tile of one operation; every
// task waits on up to three event counters and bumps up to two.  An event
// fires once its counter reaches its threshold (the number of producer tasks
// per step).  Counters are monotonic across steps: a waiter of step `epoch`
// needs counter >= (epoch + 1) * threshold, so no reset launch is needed.
#pragma once
#include <stdint.h>

namespace mk {

// ---- workgroup geometry ---------------------------------------------------
// One workgroup per CU: wave 0 is the control wave (dependency polls, task
// descriptors, output stores, signals); waves 1..7 stream weights and
// compute.  Small tasks (attention, merges, routing, argmax) use all eight.
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kCW = kWaves - 1;        // compute waves
// A GEMV tile is streamed as "wave-chunks": 64 lanes x one vector load each
// (16 B per lane; 8 B when a row is not a multiple of 1 KiB).  Each compute
// wave holds up to kMaxChunks 16-byte loads per lane.
constexpr int kMaxChunks = 16;
constexpr int kMaxTileUnits16 = kCW * kMaxChunks;           // 1 KiB units/tile
// Single-slot plans whose staged activations fit kLdsWbufOff bytes extend
// every pass by kLdsSlots chunks per compute wave held in LDS (filled by
// LDS-DMA at [kLdsWbufOff, kLdsXBytes) of the activation stage): a pass is
// then kMaxTileUnits 1 KiB units, and more weights stream ahead of each
// dependency wait.
constexpr int kLdsSlots = 8;
constexpr int kMaxTileUnits = kCW * (kMaxChunks + kLdsSlots);
constexpr int kPageSize = 16;
constexpr int kMaxGroup = 8;           // query heads per KV head
constexpr int kMaxBatchGemv = 4;       // slots a GEMV tile handles at once
// A GEMV task streams its rows in passes of at most one tile each; passes x
// slots per task are bounded by the LDS partial-sum buffers.
constexpr int kMaxPass = 6;
// Batched decode (16..64 slots) runs the static-weight GEMVs as bf16
// matrix-core tiles: 16-row groups, at most kMfmaGroups per task.
constexpr int kMfmaGroups = 14;
constexpr int kMfmaMaxBatch = 64;
constexpr int kMaxKSplit = 16;          // column ranges per split-K matrix-core row block
constexpr int kLdsBytes = 160 * 1024;  // LDS per CU on gfx950
constexpr int kLdsXBytes = 128 * 1024; // budget for staged activations
constexpr int kLdsWbufOff = kLdsXBytes - kCW * kLdsSlots * 1024;  // 72 KiB

enum Op : int16_t {
  OP_EMBED = 1, OP_QKV = 2, OP_ATTN = 3, OP_MERGE = 4, OP_OPROJ = 5,
  OP_GATEUP = 6, OP_DOWN = 7, OP_ROUTER = 8, OP_TOPK = 9, OP_EGATEUP = 10,
  OP_EDOWN = 11, OP_COMBINE = 12, OP_LMHEAD = 13, OP_ARGMAX = 14, OP_KVAPP = 15
};

// 128-byte task descriptor.  Field use per op:
//   EMBED   a0=slot
//   QKV     a0=matrix (0 q, 1 k, 2 v) a1=row0 a2=rows
//   ATTN    a0=slot a1=kv head a2=split; claimed plans also a3 = this
//           worker's consecutive entries of the layer (first entry only),
//           a4 = the layer's first ATTN task, rpp = count | claims per step << 16
//   MERGE   a0=slot a1=kv head
//   OPROJ/DOWN/ROUTER  a1=row0 a2=rows
//   GATEUP  a1=row0 a2=rows per matrix (gate rows then the same up rows)
//   (static-weight GEMVs: rpp = rows per pass; the task streams a2 rows as
//   ceil(a2 / rpp) passes of rpp rows, the last one shorter)
//   EGATEUP a0=slot a1=row0 a2=rows per matrix a3=expert slot (the j-th
//           smallest routed expert id); rpp as for static weights
//   EDOWN   a0=slot a1=row0 a2=rows of every routed expert (the task's tile
//           is top_k segments, one per expert, each whole 1 KiB chunks)
//   (TOPK, COMBINE: no longer emitted; routing runs inside EGATEUP, the
//   combine inside EDOWN)
//   LMHEAD  a1=row0 a2=rows a4=LM-head task index (argmax partial)
//   ARGMAX  a0=slot
//   KVAPP   a0=slot (shared-sequence plans: rotate the slot's new key, store
//           key and value of every KV head into its page before any
//           attention task of the layer runs)
// a5 (every op): how many completions this task reports to its events.  A
// worker that runs several consecutive tasks signalling the same events
// reports them once, from the last task of the run (a5 = run length); the
// others carry a5 = 0.
// The second half is resolved by the C ABI once the plan's buffers exist, so
// a task needs one scalar load and no chain of dependent table lookups:
//   w0, w1  first weight row of the tile in segment 0 / 1 (experts: the
//           layer's expert 0, the expert is chosen at run time)
//   src     activation input of slot 0 (slots are K apart)
//   dst     output of slot 0 at the tile's first row (slots `ostride` apart)
//   aux     residual input, indexed like dst (null when unused)
//   gain    RMSNorm gain applied to src, or null
struct alignas(16) Task {
  int16_t op, layer, n_wait, n_sig;
  int32_t a0, a1, a2, a3, a4, a5;
  int32_t wait_ev[3];
  int32_t wait_thr[3];
  int32_t sig_ev[2];
  const uint16_t *w0, *w1;
  const float *src;
  float *dst;
  const float *aux;
  const uint16_t *gain;
  int32_t K, ostride;
  int32_t gidx;             // the task's index in list order
  int32_t rpp;              // rows per pass (static-weight GEMVs), else 0
};
static_assert(sizeof(Task) == 128, "task descriptor is 128 bytes");

// Event counters, split-attention and split-K arrival counters and
// claimed-attention counters are polled or counted on by many workgroups at
// once: each sits alone in a 128-byte line
// (stride in u32 words), so polls and atomics on one counter do not queue
// behind those on its neighbours.
constexpr int kCtrStride = 32;
// An event counter is kEvReplicas such lines: each worker counts on one of
// them and waiters add them up, so the completions of an operation's tiles
// (one atomic each, all at about the same time) and the waiters' polls do
// not all queue on one line (8, 16 and 32 replicas measured alike).
constexpr int kEvReplicas = 8;

// control words (u32) at the head of the counter buffer
enum Ctrl {
  CTRL_TICKET = 0, CTRL_DONE = 1, CTRL_ERR = 2, CTRL_ERR_TASK = 3,
  CTRL_ERR_EV = 4, CTRL_ERR_SEEN = 5, CTRL_ERR_WANT = 6, CTRL_CLOCK = 7,
  CTRL_TAG = 8,    // data tag of graph-replayed steps (bumped by a kernel per step)
  CTRL_WORDS = 16
};
enum DevErr { DEVERR_NONE = 0, DEVERR_TIMEOUT = 1, DEVERR_BAD_INPUT = 2 };

// Static plan state; the plan keeps a copy in device memory.
struct DevPlan {
  // shape
  int32_t L, H, nq, nkv, hd, F, V, E, topk, Fe, B, maxp, npages, S, G;
  int32_t max_pos, n_lm_tiles;
  int32_t mfma;            // static GEMVs as matrix-core tiles (batch 16..64)
  int32_t lds_slots;       // kLdsSlots when passes extend into LDS, else 0
  int32_t mx_sc1;          // matrix-core tiles copy their activations with
                           // device-coherent (sc1) LDS-DMA and wait without
                           // the agent-scope acquire fence
  float eps;
  // weights (bf16 as uint16)
  const uint16_t *embed, *lm_head, *final_norm;
  const uint16_t *const *attn_norm, *const *ffn_norm;   // device tables [L]
  const uint16_t *const *wq, *const *wk, *const *wv, *const *wo;
  const uint16_t *const *w_gate, *const *w_up, *const *w_down;
  const uint16_t *const *router;                        // [L]
  const uint16_t *const *e_gate, *const *e_up, *const *e_down;  // [L*E]
  // elements between consecutive experts of a layer when every expert table
  // is evenly strided (expert e = expert 0 + e * e_stride), else 0 (the
  // tables are read)
  int64_t e_stride;
  // KV cache
  uint16_t *k_pool, *v_pool;
  const int32_t *page_table;
  // scratch (fp32 unless noted); layouts in planner.cpp
  float *x, *xmid, *q, *k, *v, *part, *attn, *h;   // all but part: tagged pairs
  float *rl;                                        // router logits: tagged pairs
  // matrix-core plans: an fp32 copy (values only) of every tagged vector
  // that matrix-core tiles read; element i of the pairs at p lives at
  // shadow[(p + 2i - pair0) / 2] (null in other plans)
  const float *pair0;
  float *shadow;
  float *tk_w, *he, *amax_v;
  int32_t *tk_ids, *amax_i;
  const float *rope_cos, *rope_sin;                     // [max_pos][hd/2]
  // control
  uint32_t *ev;            // event counters, after CTRL_WORDS control words
  int32_t ev_rep;          // replicas per event counter (1 in scheduled plans)
  uint32_t *att_cnt;       // split-attention arrivals per (layer, slot, KV head),
                           // after the event counters; monotonic like them
  uint32_t *kcnt;          // split-K arrivals per matrix-core row block, after att_cnt
  uint32_t *pool_cnt;      // claimed-attention counters per layer, after kcnt
  int32_t attn_pool;       // persistent workers claim attention tasks at run time
  int32_t attn_order;      // claim order of pooled attention: 0 slot order,
                           // 1 longest context first, 2 caller priority first
                           // (then longest context)
  float *kpart;            // split-K partial products, kpart_slot(B) floats per tile
  uint32_t *ctrl;
  const Task *tasks;           // worker-major: each worker's queue is contiguous
  int32_t n_tasks;
  const int32_t *worker_off;   // [n_workers + 1]: worker w runs tasks[off[w], off[w+1])
  const int32_t *task_pos;     // list index -> position in `tasks`
  int32_t n_workers;
  int64_t spin_budget;     // in s_memrealtime ticks (100 MHz)
  // scheduled executor (null otherwise): consumers of each event
  // [cons_off[e], cons_off[e+1]) in cons, counter waits per task, worker of
  // each task; per-worker queue sizes and offsets into wring, per-scheduler
  // activation counts and offsets into sring; the monotonic counters
  // pending[T], wtail[W], stail[NS] (after the arrival counters, reset with
  // them)
  const int32_t *cons_off, *cons, *n_deps, *t_worker;
  const int32_t *w_count, *w_off, *s_count, *s_off;
  const int32_t *roots, *ev_thr;  // tasks with no waits; per-step thresholds
  int32_t n_roots;
  uint32_t *pending, *wtail, *stail;
  uint64_t *wring, *sring;
  int32_t n_sched;
  uint32_t *trace;         // 6 u32 per task, or null
  int32_t trace_mode;      // 1: dependency tickets + times, 2: times only,
                           // 3: the scheduled executor records (tickets + times)
  int32_t withhold;        // test hook: list index of a task whose counter
                           // signals are withheld, or -1
  int32_t pt_rows;         // rows of the page table (the slots of the plan
                           // that owns it; an internal prefill plan maps its
                           // slots onto one of them)
  int32_t kv_first;        // shared-sequence plan: KVAPP tasks store every
                           // slot's key/value before the layer's attention,
                           // which reads all positions (its own included)
                           // from the cache
};

// Per-step arguments, passed by value next to a device copy of DevPlan.
struct CallArgs {
  const int32_t *tokens, *positions;
  const int32_t *rows;   // page-table row of each slot's sequence; null: row = slot
  const int32_t *prio;   // per-slot priority (higher first) for attn_order 2, or null
  int32_t *next_tokens;
  float *logits;
  uint32_t epoch;
  uint32_t tag;   // this step's data tag (nonzero); 0: read CTRL_TAG (graph replay)
};

// Tagged activations.  The vectors that one operation writes and the next
// reads in full (x, xmid, attn, h; q, k, v for attention) hold (value, tag)
// pairs: each element is
// one 8-byte store of its fp32 value and the step's tag, so a reader that
// sees the current tag has the value too.  An edge into a task that reads
// such a vector is a data edge: the reader loads until every tag is
// current instead of waiting for an event counter, and the writer signals
// nothing (no drain, no atomic).  Event ids with kDataEdge set are data
// edges; the task lists keep them so the graph can be checked.
constexpr int32_t kDataEdge = 1 << 30;

// scratch sizes (elements), shared by planner and device code
inline int64_t part_stride(int hd) { return hd + 4; }  // o[hd], m, l, pad
// floats per split-K partial slot: the products of one matrix-core tile (at
// most kMfmaGroups groups of 16 rows) for the padded batch, [row][slot],
// then the slots' partial sums of squares
constexpr int64_t kpart_slot(int B) { return (int64_t)(kMfmaGroups * 16 + 1) * ((B + 15) / 16 * 16); }

}  // namespace mk
