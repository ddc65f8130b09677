// capi.cpp -- the C ABI (include/mk.h): argument checks, plan lifetime,
// device allocations, step launches and device-error read-back.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <memory>
#include <cstdio>
#include <cstring>
#include <exception>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "launch.h"
#include "mk_task.h"
#include "planner.h"

using namespace mk;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &m) {
  g_err = m;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(e == hipErrorOutOfMemory ? MK_ERR_OOM : MK_ERR_HIP, m);
}

#define HIP_TRY(call, what)                         \
  do {                                              \
    hipError_t e_ = (call);                         \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) hipSetDevice(prev);
  }
};

}  // namespace

struct mk_plan {
  HostPlan hp;
  int device = 0;
  int grid = 0;
  int executor = MK_EXEC_PERSISTENT;
  bool trace = false;
  DevPlan d{};
  DevPlan *d_dev = nullptr;  // device copy of d
  std::vector<void *> allocs;
  uint32_t epoch = 0;
  uint32_t epoch_limit = 1;
  uint32_t tag = 0;          // data tag of the last step (never 0 once used)
  bool graph_replay = false;
  int32_t *stage_tok = nullptr, *stage_pos = nullptr, *stage_next = nullptr;
  int32_t *stage_rows = nullptr;
  mk_plan *prefill = nullptr;  // internal shared-sequence plan that runs mk_prefill
                               // in chunks, or null (token by token)
  float *stage_logits = nullptr;
  uint32_t *ctrl = nullptr;  // CTRL_WORDS control words, the event counters, then
                             // the split-attention and split-K arrival counters
  int ev_rep = 1;            // replicas per event counter
  int n_ev_words = 0;        // event counters, kCtrStride words per replica
  int n_att_cnt = 0;         // words of the arrival and claim counters after them
  int n_ctrl_words = 0;
  // Plans built by mk_build_plan_noalloc carve their device state out of the
  // device's static scratch array instead of allocating it.
  char *arena = nullptr;
  size_t arena_off = 0, arena_cap = 0;
  uint32_t arena_gen = 0;    // which of the device's static plans this is

  ~mk_plan() {
    delete prefill;
    for (void *p : allocs) hipFree(p);
  }
  template <class T>
  int alloc(T **p, size_t count, const char *what) {
    *p = nullptr;
    if (count == 0) return MK_OK;
    if (arena) {
      const size_t off = (arena_off + 255) & ~(size_t)255;
      if (off + count * sizeof(T) > arena_cap)
        return fail(MK_ERR_UNSUPPORTED,
                    std::string("the plan's device state (") + what + " and what precedes it, " +
                        std::to_string(off + count * sizeof(T)) +
                        " bytes) exceeds the static scratch of " + std::to_string(arena_cap) +
                        " bytes; use mk_build_plan");
      *p = (T *)(arena + off);
      arena_off = off + count * sizeof(T);
      return MK_OK;
    }
    void *v = nullptr;
    hipError_t e = hipMalloc(&v, count * sizeof(T));
    if (e != hipSuccess) return hip_fail(e, what);
    allocs.push_back(v);
    *p = (T *)v;
    return MK_OK;
  }
};

namespace {
// Generation of the newest static plan per device: building one replaces the
// device state of the one before, whose handle then refuses to run.
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_static_gen[kMaxDevices];
}  // namespace

extern "C" {

const char *mk_last_error(void) { return g_err.c_str(); }

#ifndef MK_SOURCE_HASH
#define MK_SOURCE_HASH "unknown"
#endif
const char *mk_build_id(void) { return MK_SOURCE_HASH; }

void mk_plan_options_default(mk_plan_options *o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->executor = MK_EXEC_PERSISTENT;
  o->device = -1;
}

int mk_inspect_plan(const mk_config *cfg, const mk_plan_options *opts, mk_task_info *tasks,
                    int32_t task_cap, int32_t *n_tasks, int32_t *ev_thresholds,
                    int32_t ev_cap, int32_t *n_events) {
  try {
    if (!cfg) return fail(MK_ERR_INVALID_ARG, "cfg is NULL");
    mk_plan_options o;
    mk_plan_options_default(&o);
    if (opts) o = *opts;
    int n_cus = o.n_cus > 0 ? o.n_cus : 256;
    int n_workers = o.n_workgroups > 0 ? o.n_workgroups : n_cus;
    if (o.executor == MK_EXEC_SCHEDULED) n_workers -= 1;  // workgroup 0 schedules
    HostPlan hp;
    std::string err;
    int rc = build_host_plan(*cfg, o, n_cus, n_workers, hp, err);
    if (rc != MK_OK) return fail(rc, err);
    const int T = (int)hp.tasks.size(), E = (int)hp.ev_thr.size();
    if (n_tasks) *n_tasks = T;
    if (n_events) *n_events = E;
    for (int i = 0; tasks && i < T && i < task_cap; ++i) {
      const Task &t = hp.tasks[i];
      mk_task_info &q = tasks[i];
      std::memset(&q, 0, sizeof q);
      q.op = t.op; q.layer = t.layer;
      q.a0 = t.a0; q.a1 = t.a1; q.a2 = t.a2; q.a3 = t.a3; q.a4 = t.a4; q.sig_count = t.a5;
      q.n_wait = t.n_wait;
      for (int k = 0; k < 3; ++k) {
        q.wait_ev[k] = k < t.n_wait ? t.wait_ev[k] & ~kDataEdge : -1;
        if (k < t.n_wait && (t.wait_ev[k] & kDataEdge)) q.data_edges |= 1 << k;
      }
      q.n_sig = t.n_sig;
      for (int k = 0; k < 2; ++k) {
        q.sig_ev[k] = k < t.n_sig ? t.sig_ev[k] & ~kDataEdge : -1;
        if (k < t.n_sig && (t.sig_ev[k] & kDataEdge)) q.data_edges |= 1 << (3 + k);
      }
      q.phase = hp.task_phase[i];
      q.worker = hp.task_worker[i];
      q.rows_per_pass = t.rpp;
      q.bytes = hp.task_bytes[i];
    }
    for (int e = 0; ev_thresholds && e < E && e < ev_cap; ++e) ev_thresholds[e] = hp.ev_thr[e];
    return MK_OK;
  } catch (const std::exception &ex) {
    return fail(MK_ERR_PLAN, ex.what());
  }
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Elements between consecutive experts when, in every layer and for each of
// gate, up and down, expert e starts e * Fe * H elements after expert 0 (the
// usual stacked [E, rows, cols] tensors); 0 otherwise.  Lets the device
// compute an expert's address instead of reading the table.
static int64_t expert_stride(const mk_config &c, const std::vector<const void *> &tab) {
  const int L = c.n_layers, E = c.n_experts;
  if (E == 0) return 0;
  const int64_t st = (int64_t)c.hidden * c.expert_ffn_dim;
  for (int m = 0; m < 3; ++m)
    for (int l = 0; l < L; ++l) {
      const size_t b = (size_t)10 * L + ((size_t)m * L + l) * E;
      const char *p0 = (const char *)tab[b];
      for (int e = 1; e < E; ++e)
        if ((const char *)tab[b + e] != p0 + (size_t)e * st * 2) return 0;
    }
  return st;
}

// Fill the device addresses of every GEMV task (weights of its tile, input
// activations, output and residual) once the plan's buffers exist.  `tab`
// holds the per-layer weight pointers in check_weights' order.
static void resolve_tasks(HostPlan &hp, const std::vector<const void *> &tab, const mk_weights &w,
                          const DevPlan &d) {
  const mk_config &c = hp.cfg;
  const int L = c.n_layers, B = c.max_batch, H = c.hidden;
  const int QD = c.n_q_heads * c.head_dim, KVD = c.n_kv_heads * c.head_dim;
  const int F = c.ffn_dim, E = c.n_experts, TK = c.top_k, Fe = c.expert_ffn_dim;
  auto W = [&](int kind, int l) { return (const uint16_t *)tab[(size_t)kind * L + l]; };
  // element e of a tagged (value, tag) vector buffer
  auto TG = [](float *base, size_t e) { return base + 2 * e; };
  // expert 0 of layer l of expert tensor m (0 gate, 1 up, 2 down)
  auto EX = [&](int m, int l) {
    return (const uint16_t *)tab[(size_t)10 * L + ((size_t)m * L + l) * E];
  };
  for (Task &t : hp.tasks) {
    const int l = t.layer;
    t.w0 = t.w1 = nullptr;
    t.src = t.aux = nullptr;
    t.dst = nullptr;
    t.gain = nullptr;
    t.K = 0;
    t.ostride = 0;
    switch (t.op) {
      case OP_QKV: {
        const int Nm = t.a0 == 0 ? QD : KVD;
        float *base = t.a0 == 0 ? d.q : (t.a0 == 1 ? d.k : d.v);
        t.w0 = W(2 + t.a0, l) + (size_t)t.a1 * H;
        t.src = TG(d.x, (size_t)l * B * H);
        t.gain = W(0, l);
        t.K = H;
        t.dst = TG(base, (size_t)l * B * Nm + t.a1);
        t.ostride = Nm;
        break;
      }
      case OP_OPROJ:
        t.w0 = W(5, l) + (size_t)t.a1 * QD;
        t.src = TG(d.attn, (size_t)l * B * QD);
        t.K = QD;
        t.dst = TG(d.xmid, (size_t)l * B * H + t.a1);
        t.aux = TG(d.x, (size_t)l * B * H + t.a1);
        t.ostride = H;
        break;
      case OP_GATEUP:
        t.w0 = W(6, l) + (size_t)t.a1 * H;
        t.w1 = W(7, l) + (size_t)t.a1 * H;
        t.src = TG(d.xmid, (size_t)l * B * H);
        t.gain = W(1, l);
        t.K = H;
        t.dst = TG(d.h, (size_t)l * B * F + t.a1);
        t.ostride = F;
        break;
      case OP_DOWN:
        t.w0 = W(8, l) + (size_t)t.a1 * F;
        t.src = TG(d.h, (size_t)l * B * F);
        t.K = F;
        t.dst = TG(d.x, (size_t)(l + 1) * B * H + t.a1);
        t.aux = TG(d.xmid, (size_t)l * B * H + t.a1);
        t.ostride = H;
        break;
      case OP_ROUTER:
        t.w0 = W(9, l) + (size_t)t.a1 * H;
        t.src = TG(d.xmid, (size_t)l * B * H);
        t.gain = W(1, l);
        t.K = H;
        t.dst = TG(d.rl, (size_t)l * B * E + t.a1);
        t.ostride = E;
        break;
      case OP_LMHEAD:
        t.w0 = (const uint16_t *)w.lm_head + (size_t)t.a1 * H;
        t.src = TG(d.x, (size_t)L * B * H);
        t.gain = (const uint16_t *)w.final_norm;
        t.K = H;
        break;
      case OP_EGATEUP: {
        const size_t bj = ((size_t)l * B + t.a0) * TK + t.a3;
        t.w0 = EX(0, l);
        t.w1 = EX(1, l);
        t.src = TG(d.xmid, ((size_t)l * B + t.a0) * H);
        t.gain = W(1, l);
        t.K = H;
        t.dst = d.he + bj * Fe + t.a1;
        break;
      }
      case OP_EDOWN: {  // all k routed experts of the slot, rows a1..a1+a2
        const size_t bx = (size_t)l * B + t.a0;
        t.w0 = EX(2, l);
        t.src = d.he + bx * TK * Fe;
        t.K = Fe;
        t.dst = TG(d.x, (bx + B) * H + t.a1);
        t.aux = TG(d.xmid, bx * H + t.a1);
        t.ostride = H;
        break;
      }
      default:
        break;
    }
  }
}

static int check_weights(const mk_config &c, const mk_weights &w, std::vector<const void *> &tab,
                         std::string &err) {
  const int L = c.n_layers, E = c.n_experts;
  auto need = [&](const void *p, const char *name, int i) {
    if (!p) {
      err = std::string("weight pointer ") + name + "[" + std::to_string(i) + "] is NULL";
      return false;
    }
    if (!aligned16(p)) {
      err = std::string("weight pointer ") + name + "[" + std::to_string(i) +
            "] is not 16-byte aligned";
      return false;
    }
    return true;
  };
  if (!need(w.embed, "embed", 0) || !need(w.lm_head, "lm_head", 0) ||
      !need(w.final_norm, "final_norm", 0))
    return MK_ERR_INVALID_ARG;
  // table order: attn_norm, ffn_norm, wq, wk, wv, wo, w_gate, w_up, w_down,
  // router [L each], then e_gate, e_up, e_down [L*E each]
  const void *const *per_layer[10] = {w.attn_norm, w.ffn_norm, w.wq, w.wk, w.wv,
                                      w.wo, w.w_gate, w.w_up, w.w_down, w.router};
  const char *names[10] = {"attn_norm", "ffn_norm", "wq", "wk", "wv",
                           "wo", "w_gate", "w_up", "w_down", "router"};
  tab.assign((size_t)10 * L + (size_t)3 * L * E, nullptr);
  for (int k = 0; k < 10; ++k) {
    const bool used = k < 6 || (E == 0 ? (k >= 6 && k <= 8) : k == 9);
    if (!used) continue;
    if (!per_layer[k]) {
      err = std::string("weight table ") + names[k] + " is NULL";
      return MK_ERR_INVALID_ARG;
    }
    for (int l = 0; l < L; ++l) {
      if (!need(per_layer[k][l], names[k], l)) return MK_ERR_INVALID_ARG;
      tab[(size_t)k * L + l] = per_layer[k][l];
    }
  }
  if (E > 0) {
    const void *const *ex[3] = {w.e_gate, w.e_up, w.e_down};
    const char *en[3] = {"e_gate", "e_up", "e_down"};
    for (int k = 0; k < 3; ++k) {
      if (!ex[k]) {
        err = std::string("weight table ") + en[k] + " is NULL";
        return MK_ERR_INVALID_ARG;
      }
      for (int i = 0; i < L * E; ++i) {
        if (!need(ex[k][i], en[k], i)) return MK_ERR_INVALID_ARG;
        tab[(size_t)10 * L + (size_t)k * L * E + i] = ex[k][i];
      }
    }
  }
  return MK_OK;
}

static int build_plan(const mk_config *cfg, const mk_weights *w, const mk_kv *kv,
                      const mk_plan_options *opts, mk_plan **out, bool noalloc,
                      int pt_rows = 0) {
  try {
    if (!out) return fail(MK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !w || !kv) return fail(MK_ERR_INVALID_ARG, "cfg, weights and kv are required");
    mk_plan_options o;
    mk_plan_options_default(&o);
    if (opts) o = *opts;
    if (o.executor != MK_EXEC_PERSISTENT && o.executor != MK_EXEC_KERNEL_PER_OP &&
        o.executor != MK_EXEC_SCHEDULED)
      return fail(MK_ERR_INVALID_ARG, "unknown executor");
    const bool sched = o.executor == MK_EXEC_SCHEDULED;
    if (o.prefill_chunk > 0 && (o.prefill_chunk < 16 || o.prefill_chunk > kMfmaMaxBatch))
      return fail(MK_ERR_INVALID_ARG, "prefill_chunk must be 0, -1 or 16..64");
    if (o.attn_order < -1 || o.attn_order > 2)
      return fail(MK_ERR_INVALID_ARG, "attn_order must be -1, 0, 1 or 2");
    if (o.attn_order > 0 && cfg->max_batch > kMfmaMaxBatch)
      return fail(MK_ERR_UNSUPPORTED, "attn_order needs max_batch <= 64");
    std::string err;
    int rc = check_config(*cfg, err);
    if (rc != MK_OK) return fail(rc, err);
    std::vector<const void *> tab;
    rc = check_weights(*cfg, *w, tab, err);
    if (rc != MK_OK) return fail(rc, err);
    if (!kv->k_pool || !kv->v_pool || !kv->page_table)
      return fail(MK_ERR_INVALID_ARG, "kv pools and page table are required");
    if (!aligned16(kv->k_pool) || !aligned16(kv->v_pool))
      return fail(MK_ERR_INVALID_ARG, "kv pools must be 16-byte aligned");

    int dev = o.device;
    if (dev < 0) HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    DeviceGuard guard(dev);
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
    if ((size_t)persistent_lds_bytes() > prop.sharedMemPerBlock)
      return fail(MK_ERR_UNSUPPORTED, "device has less LDS per workgroup than the kernels need");

    std::unique_ptr<mk_plan> p(new mk_plan());
    if (noalloc) {
      if (dev >= kMaxDevices) return fail(MK_ERR_UNSUPPORTED, "device ordinal too large");
      // every earlier static plan's work has finished before its state is
      // overwritten
      HIP_TRY(hipDeviceSynchronize(), "hipDeviceSynchronize");
      void *base = nullptr;
      HIP_TRY(static_scratch(dev, &base), "static scratch address");
      p->arena = (char *)base;
      p->arena_cap = kStaticScratchBytes;
      p->arena_gen = ++g_static_gen[dev];
    }
    p->device = dev;
    p->executor = o.executor;
    p->graph_replay = o.graph_replay != 0;
    p->trace = o.debug_trace != 0;
    const int hw_cus = prop.multiProcessorCount;
    const int n_cus = o.n_cus > 0 ? o.n_cus : hw_cus;
    p->grid = o.n_workgroups > 0 ? o.n_workgroups : hw_cus;
    if (p->grid > hw_cus)
      return fail(MK_ERR_INVALID_ARG, "more persistent workers than CUs (one resident workgroup per CU)");
    if (sched && p->grid < 2)
      return fail(MK_ERR_INVALID_ARG, "the scheduled executor needs at least 2 workgroups");
    // scheduled executor: workgroup 0 holds the schedulers, the rest are workers
    rc = build_host_plan(*cfg, o, n_cus, sched ? p->grid - 1 : p->grid, p->hp, err);
    if (rc != MK_OK) return fail(rc, err);
    HostPlan &hp = p->hp;
    const mk_config &c = hp.cfg;
    const int T = (int)hp.tasks.size(), E = (int)hp.ev_thr.size();
    const int L = c.n_layers, B = c.max_batch;

    // epoch limit: (epoch + 1) * max threshold must stay below 2^31
    int32_t max_thr = 1;
    for (int32_t v : hp.ev_thr) max_thr = std::max(max_thr, v);
    max_thr = std::max(max_thr, hp.S);  // split-attention arrival counters
    max_thr = std::max(max_thr, kMaxKSplit);  // split-K arrival counters
    for (const Task &t : hp.tasks)              // claimed-attention counters
      if (t.op == OP_ATTN && hp.attn_pool) max_thr = std::max(max_thr, t.rpp >> 16);
    // scheduled executor: per-task dependency counts, queue reservations
    std::vector<int32_t> s_cons_off, s_cons, s_deps, s_worker, s_wcount, s_woff, s_scount,
        s_soff, s_roots;
    const int NS = 4;
    if (sched) {
      const int W = hp.n_workers;
      s_cons_off.assign(E + 1, 0);
      s_deps.assign(T, 0);
      s_worker.assign(hp.task_worker.begin(), hp.task_worker.end());
      for (int i = 0; i < T; ++i) {
        s_deps[i] = hp.tasks[i].n_wait;
        for (int k = 0; k < hp.tasks[i].n_wait; ++k)
          s_cons_off[(hp.tasks[i].wait_ev[k] & ~kDataEdge) + 1]++;
        if (hp.tasks[i].n_wait == 0) s_roots.push_back(i);
      }
      for (int e = 0; e < E; ++e) s_cons_off[e + 1] += s_cons_off[e];
      s_cons.assign(s_cons_off[E], 0);
      std::vector<int32_t> fill(s_cons_off.begin(), s_cons_off.end() - 1);
      for (int i = 0; i < T; ++i)
        for (int k = 0; k < hp.tasks[i].n_wait; ++k)
          s_cons[fill[hp.tasks[i].wait_ev[k] & ~kDataEdge]++] = i;
      s_wcount.assign(W, 0);
      for (int i = 0; i < T; ++i) s_wcount[hp.task_worker[i]]++;
      s_woff.assign(W + 1, 0);
      for (int w = 0; w < W; ++w) s_woff[w + 1] = s_woff[w] + s_wcount[w];
      s_scount.assign(NS, 0);
      for (int e = 0; e < E; ++e) s_scount[e % NS]++;
      s_soff.assign(NS + 1, 0);
      for (int k = 0; k < NS; ++k) s_soff[k + 1] = s_soff[k] + s_scount[k];
      for (int v : s_wcount) max_thr = std::max(max_thr, v);
      for (int v : s_scount) max_thr = std::max(max_thr, v);
    }
    p->epoch_limit = (uint32_t)(((1u << 31) - 1u) / (uint32_t)max_thr) - 2u;

    // device allocations
    Task *d_tasks;
    if ((rc = p->alloc(&d_tasks, T, "task table"))) return rc;
    int32_t *d_wq;
    if ((rc = p->alloc(&d_wq, hp.worker_off.size() + hp.worker_list.size(), "worker queues")))
      return rc;
    p->ev_rep = sched ? 1 : kEvReplicas;
    p->n_ev_words = E * p->ev_rep * kCtrStride;
    p->n_att_cnt = (c.n_layers * c.max_batch * c.n_kv_heads + hp.n_kcnt + c.n_layers) * kCtrStride;
    const int n_sched_cnt = sched ? T + hp.n_workers + NS : 0;  // pending, wtail, stail
    p->n_att_cnt += n_sched_cnt;
    p->n_ctrl_words = CTRL_WORDS + p->n_ev_words + p->n_att_cnt;
    if ((rc = p->alloc(&p->ctrl, p->n_ctrl_words, "event counters"))) return rc;
    const int64_t n_kpart = hp.n_kpart * kpart_slot(B);
    // matrix-core plans: the values-only copy of the tagged vectors (x
    // through rl), half their span, placed first so every buffer after it
    // keeps the base's alignment
    const int64_t n_tagged =
        2 * (hp.n_x + hp.n_xmid + hp.n_q + 2 * hp.n_k + hp.n_attn + hp.n_h + hp.n_rl) + hp.n_part;
    const int64_t n_shadow = hp.mfma ? (n_tagged / 2 + 63) / 64 * 64 : 0;
    const int64_t nf = n_shadow + n_tagged + hp.n_tk + hp.n_he + hp.n_amax + n_kpart;
    float *fs;
    if ((rc = p->alloc(&fs, (size_t)nf, "activation scratch"))) return rc;
    int32_t *is;
    if ((rc = p->alloc(&is, (size_t)(hp.n_tk + hp.n_amax + 4 * B), "index scratch"))) return rc;
    const void **d_tab;
    if ((rc = p->alloc(&d_tab, tab.size(), "weight tables"))) return rc;
    const int half = c.head_dim / 2;
    float *rope;
    if ((rc = p->alloc(&rope, (size_t)2 * hp.max_pos * half, "rope tables"))) return rc;
    uint32_t *trace = nullptr;
    if (p->trace && (rc = p->alloc(&trace, (size_t)T * 6, "trace"))) return rc;
    int32_t *sched_ints = nullptr;
    uint64_t *sched_rings = nullptr;
    const size_t n_sched_ints = s_cons_off.size() + s_cons.size() + s_deps.size() +
                                s_worker.size() + s_wcount.size() + s_woff.size() +
                                s_scount.size() + s_soff.size() + s_roots.size() +
                                (sched ? (size_t)E : 0);
    if (sched) {
      if ((rc = p->alloc(&sched_ints, n_sched_ints, "scheduler tables"))) return rc;
      if ((rc = p->alloc(&sched_rings, (size_t)T + E, "scheduler queues"))) return rc;
      HIP_TRY(hipMemset(sched_rings, 0, ((size_t)T + E) * 8), "zero queues");
    }
    if ((rc = p->alloc(&p->stage_logits, (size_t)B * c.vocab, "prefill logits"))) return rc;

    // uploads
    HIP_TRY(hipMemcpy(d_tab, tab.data(), tab.size() * sizeof(void *), hipMemcpyHostToDevice),
            "upload weight tables");
    HIP_TRY(hipMemcpy(d_wq, hp.worker_off.data(), hp.worker_off.size() * 4, hipMemcpyHostToDevice),
            "upload worker queues");
    {
      // rotary tables: angle p * theta^(-2i/hd) and its cos/sin in double,
      // rounded once to float
      std::vector<float> cs((size_t)hp.max_pos * half), sn((size_t)hp.max_pos * half);
      for (int i = 0; i < half; ++i) {
        const double f = std::pow(c.rope_theta, -2.0 * i / c.head_dim);
        for (int ps = 0; ps < hp.max_pos; ++ps) {
          const double a = (double)ps * f;
          cs[(size_t)ps * half + i] = (float)std::cos(a);
          sn[(size_t)ps * half + i] = (float)std::sin(a);
        }
      }
      HIP_TRY(hipMemcpy(rope, cs.data(), cs.size() * 4, hipMemcpyHostToDevice), "upload rope");
      HIP_TRY(hipMemcpy(rope + cs.size(), sn.data(), sn.size() * 4, hipMemcpyHostToDevice),
              "upload rope");
    }
    HIP_TRY(hipMemset(p->ctrl, 0, (size_t)p->n_ctrl_words * 4), "zero counters");
    HIP_TRY(hipMemset(fs, 0, (size_t)nf * 4), "zero scratch");
    HIP_TRY(hipMemset(is, 0, (size_t)(hp.n_tk + hp.n_amax + 4 * B) * 4), "zero scratch");
    if (trace) HIP_TRY(hipMemset(trace, 0, (size_t)T * 24), "zero trace");

    DevPlan &d = p->d;
    d.L = L; d.H = c.hidden; d.nq = c.n_q_heads; d.nkv = c.n_kv_heads; d.hd = c.head_dim;
    d.F = c.ffn_dim; d.V = c.vocab; d.E = c.n_experts; d.topk = c.top_k;
    d.Fe = c.expert_ffn_dim; d.B = B; d.maxp = c.max_pages_per_seq; d.npages = c.n_pages;
    d.S = hp.S; d.G = hp.G; d.max_pos = hp.max_pos; d.n_lm_tiles = hp.n_lm_tiles;
    d.mfma = hp.mfma ? 1 : 0;
    d.kv_first = hp.kv_first ? 1 : 0;
    d.pt_rows = pt_rows > 0 ? pt_rows : B;
    d.lds_slots = hp.lds_slots;
    // Up to one 16-slot tile, matrix-core tiles copy their activations with
    // device-coherent loads and skip the acquire fence (measured on the 8B
    // shape, ragged contexts: 4 slots -4.0 %, 8 slots -3.8 %, 16 slots
    // -1.7 %); with more slots the slices the tiles of an XCD share are
    // larger, and reading them through the L2 after the fence is ahead
    // (64 slots: +0.8 % with coherent copies).
    d.mx_sc1 = hp.mfma && B <= 16 ? 1 : 0;
    d.eps = c.rms_eps;
    d.embed = (const uint16_t *)w->embed;
    d.lm_head = (const uint16_t *)w->lm_head;
    d.final_norm = (const uint16_t *)w->final_norm;
    const uint16_t *const *T16 = (const uint16_t *const *)d_tab;
    d.attn_norm = T16 + 0 * L; d.ffn_norm = T16 + 1 * L;
    d.wq = T16 + 2 * L; d.wk = T16 + 3 * L; d.wv = T16 + 4 * L; d.wo = T16 + 5 * L;
    d.w_gate = T16 + 6 * L; d.w_up = T16 + 7 * L; d.w_down = T16 + 8 * L;
    d.router = T16 + 9 * L;
    const size_t LE = (size_t)L * c.n_experts;
    d.e_gate = T16 + 10 * L; d.e_up = T16 + 10 * L + LE; d.e_down = T16 + 10 * L + 2 * LE;
    d.e_stride = expert_stride(c, tab);
    d.k_pool = (uint16_t *)kv->k_pool;
    d.v_pool = (uint16_t *)kv->v_pool;
    d.page_table = kv->page_table;
    float *f = fs;
    auto take = [&](int64_t n) { float *r = n ? f : nullptr; f += n; return r; };
    d.shadow = take(n_shadow);
    d.x = take(2 * hp.n_x); d.xmid = take(2 * hp.n_xmid); d.q = take(2 * hp.n_q);
    d.k = take(2 * hp.n_k); d.v = take(2 * hp.n_k); d.part = take(hp.n_part);
    d.attn = take(2 * hp.n_attn);
    d.h = take(2 * hp.n_h);
    d.rl = take(2 * hp.n_rl); d.tk_w = take(hp.n_tk); d.he = take(hp.n_he);
    d.amax_v = take(hp.n_amax);
    d.kpart = take(n_kpart);
    d.pair0 = d.shadow ? d.x : nullptr;
    d.tk_ids = hp.n_tk ? is : nullptr;
    d.amax_i = is + hp.n_tk;
    p->stage_tok = is + hp.n_tk + hp.n_amax;
    p->stage_pos = p->stage_tok + B;
    p->stage_next = p->stage_pos + B;
    p->stage_rows = p->stage_next + B;
    d.rope_cos = rope;
    d.rope_sin = rope + (size_t)hp.max_pos * half;
    d.ctrl = p->ctrl;
    d.ev = p->ctrl + CTRL_WORDS;
    d.ev_rep = p->ev_rep;
    d.att_cnt = d.ev + p->n_ev_words;
    d.kcnt = d.att_cnt + (size_t)c.n_layers * c.max_batch * c.n_kv_heads * kCtrStride;
    d.pool_cnt = d.kcnt + (size_t)hp.n_kcnt * kCtrStride;
    d.attn_pool = hp.attn_pool ? 1 : 0;
    // claim order: longest context first unless asked otherwise (measured on
    // the 8B shape with contexts U[128, 16384]: 16 slots -3.3 %, 64 -0.6 %)
    d.attn_order = !hp.attn_pool || o.attn_order < 0 || c.max_batch > kMfmaMaxBatch
                       ? 0
                       : (o.attn_order == 0 ? 1 : o.attn_order);
    d.tasks = d_tasks;
    d.n_tasks = T;
    d.worker_off = d_wq;
    d.task_pos = d_wq + hp.worker_off.size();
    d.n_workers = hp.n_workers;
    d.spin_budget = o.spin_budget > 0 ? o.spin_budget : 100000000LL;  // 1 s at 100 MHz
    d.trace = trace;
    d.trace_mode = sched && trace ? 3 : o.debug_trace;
    if (sched) {
      int32_t *q = sched_ints;
      auto put = [&](const std::vector<int32_t> &v) -> const int32_t * {
        int32_t *at = q;
        if (!v.empty())
          (void)hipMemcpy(at, v.data(), v.size() * 4, hipMemcpyHostToDevice);
        q += v.size();
        return at;
      };
      d.cons_off = put(s_cons_off);
      d.cons = put(s_cons);
      d.n_deps = put(s_deps);
      d.t_worker = put(s_worker);
      d.w_count = put(s_wcount);
      d.w_off = put(s_woff);
      d.s_count = put(s_scount);
      d.s_off = put(s_soff);
      d.roots = put(s_roots);
      d.ev_thr = put(hp.ev_thr);
      d.n_roots = (int32_t)s_roots.size();
      d.n_sched = NS;
      HIP_TRY(hipDeviceSynchronize(), "upload scheduler tables");
      d.wring = sched_rings;
      d.sring = sched_rings + T;
      // counters after the arrival counters: reset with them
      d.pending = p->ctrl + CTRL_WORDS + p->n_ev_words + (p->n_att_cnt - n_sched_cnt);
      d.wtail = d.pending + T;
      d.stail = d.wtail + hp.n_workers;
    }
    if (o.debug_withhold < 0 || o.debug_withhold > T)
      return fail(MK_ERR_INVALID_ARG, "debug_withhold names no task of the plan");
    d.withhold = o.debug_withhold - 1;
    resolve_tasks(hp, tab, *w, d);
    {
      // device table in worker-major order, plus list index -> position
      std::vector<Task> stream((size_t)T);
      std::vector<int32_t> pos((size_t)T);
      for (int k = 0; k < T; ++k) {
        const int g = hp.worker_list[k];
        stream[k] = hp.tasks[g];
        stream[k].gidx = g;
        pos[g] = k;
      }
      HIP_TRY(hipMemcpy(d_tasks, stream.data(), (size_t)T * sizeof(Task), hipMemcpyHostToDevice),
              "upload tasks");
      HIP_TRY(hipMemcpy(d_wq + hp.worker_off.size(), pos.data(), (size_t)T * 4,
                        hipMemcpyHostToDevice),
              "upload task positions");
    }
    if ((rc = p->alloc(&p->d_dev, 1, "plan copy"))) return rc;
    HIP_TRY(hipMemcpy(p->d_dev, &d, sizeof d, hipMemcpyHostToDevice), "upload plan");
    // Chunked prefill: a second plan over the same weights, pools and page
    // table whose slots are the tokens of one prompt chunk (one sequence at
    // consecutive positions), run on matrix-core tiles where the row counts
    // allow; token by token otherwise, and for plans that may not allocate.
    if (!noalloc && pt_rows == 0 && o.prefill_chunk >= 0 && o.debug_trace == 0) {
      const mk_config &cc = *cfg;
      const bool rows16 = cc.hidden % 16 == 0 && (cc.n_q_heads * cc.head_dim) % 16 == 0 &&
                          cc.vocab % 16 == 0 &&
                          (cc.n_experts ? cc.n_experts % 16 == 0 : cc.ffn_dim % 16 == 0);
      const int chunk = o.prefill_chunk > 0 ? o.prefill_chunk : (rows16 ? kMfmaMaxBatch : 0);
      if (chunk > 0) {
        mk_config pc = cc;
        pc.max_batch = chunk;
        mk_plan_options po = o;
        po.shared_seqs = 1;
        po.prefill_chunk = -1;
        po.graph_replay = 0;
        po.debug_withhold = 0;
        po.attn_splits = 0;
        po.attn_pool = 0;
        po.device = dev;
        rc = build_plan(&pc, w, kv, &po, &p->prefill, false, cc.max_batch);
        if (rc != MK_OK) return rc;
      }
    }
    *out = p.release();
    return MK_OK;
  } catch (const std::exception &ex) {
    return fail(MK_ERR_PLAN, ex.what());
  }
}

int mk_build_plan(const mk_config *cfg, const mk_weights *w, const mk_kv *kv,
                  const mk_plan_options *opts, mk_plan **out) {
  return build_plan(cfg, w, kv, opts, out, false);
}

int mk_build_plan_noalloc(const mk_config *cfg, const mk_weights *w, const mk_kv *kv,
                          const mk_plan_options *opts, mk_plan **out) {
  return build_plan(cfg, w, kv, opts, out, true);
}

// A static plan whose device state a newer static plan has replaced.
static bool stale_static(const mk_plan *plan) {
  return plan->arena && plan->arena_gen != g_static_gen[plan->device].load();
}

static int step_impl(mk_plan *plan, const int32_t *tokens, const int32_t *positions,
                     const int32_t *rows, hipStream_t s, int32_t *next, float *logits,
                     const int32_t *prio = nullptr) {
  const DevPlan &d = plan->d;
  CallArgs ca;
  ca.tokens = tokens;
  ca.positions = positions;
  ca.rows = rows;
  ca.prio = prio;
  ca.next_tokens = next;
  ca.logits = logits;
  if (plan->graph_replay) {
    // a replayable step: counters from zero and a data tag bumped on the
    // device, no state carried on the host
    HIP_TRY(launch_zero_u32(d.ev, plan->n_ev_words + plan->n_att_cnt, s),
            "counter clear");
    HIP_TRY(launch_bump_tag(plan->ctrl + CTRL_TAG, s), "tag bump");
    plan->epoch = 0;
    ca.tag = 0;
  } else {
    if (++plan->tag == 0) plan->tag = 1;
    ca.tag = plan->tag;
  }
  ca.epoch = plan->epoch;
  if (plan->executor == MK_EXEC_SCHEDULED) {
    if (plan->trace) {
      HIP_TRY(launch_zero_u32(d.trace, (int)plan->hp.tasks.size() * 6, s), "trace reset");
      HIP_TRY(launch_zero_u32(plan->ctrl + CTRL_CLOCK, 1, s), "trace reset");
    }
    HIP_TRY(launch_sched(plan->d_dev, ca, plan->grid, s), "scheduled launch");
  } else if (plan->executor == MK_EXEC_PERSISTENT) {
    if (plan->trace) {
      HIP_TRY(launch_zero_u32(d.trace, (int)plan->hp.tasks.size() * 6, s), "trace reset");
      HIP_TRY(launch_zero_u32(plan->ctrl + CTRL_CLOCK, 1, s), "trace reset");
    }
    const int mode = plan->hp.mfma ? 2 : (plan->hp.cfg.max_batch == 1 ? 1 : 0);
    HIP_TRY(launch_persistent(plan->d_dev, ca, plan->grid, mode, s),
            "persistent launch");
  } else {
    for (auto &ph : plan->hp.phases)
      HIP_TRY(launch_phase(plan->d_dev, ca, ph.first, ph.second - ph.first, s), "phase launch");
  }
  // counters are monotonic per step (both executors count split-attention
  // arrivals); reset them before they could wrap
  if (!plan->graph_replay && ++plan->epoch >= plan->epoch_limit) {
    HIP_TRY(launch_zero_u32(d.ev, plan->n_ev_words + plan->n_att_cnt, s),
            "counter reset");
    plan->epoch = 0;
  }
  return MK_OK;
}

int mk_decode_step(mk_plan *plan, const int32_t *tokens_dev, const int32_t *positions_dev,
                   void *stream, int32_t *next_tokens_dev, float *logits_dev) {
  try {
    if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
    if (!tokens_dev || !positions_dev || !next_tokens_dev)
      return fail(MK_ERR_INVALID_ARG, "tokens, positions and next_tokens are required");
    if (stale_static(plan))
      return fail(MK_ERR_INVALID_ARG, "a newer mk_build_plan_noalloc plan replaced this plan's state");
    DeviceGuard guard(plan->device);
    return step_impl(plan, tokens_dev, positions_dev, nullptr, (hipStream_t)stream,
                     next_tokens_dev, logits_dev);
  } catch (const std::exception &ex) {
    return fail(MK_ERR_PLAN, ex.what());
  }
}

int mk_batch_step(mk_plan *plan, const int32_t *tokens_dev, const int32_t *positions_dev,
                  const int32_t *seq_rows_dev, const int32_t *priorities_dev, void *stream,
                  int32_t *next_tokens_dev, float *logits_dev) {
  try {
    if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
    if (!tokens_dev || !positions_dev || !seq_rows_dev || !next_tokens_dev)
      return fail(MK_ERR_INVALID_ARG, "tokens, positions, seq_rows and next_tokens are required");
    if (stale_static(plan))
      return fail(MK_ERR_INVALID_ARG, "a newer mk_build_plan_noalloc plan replaced this plan's state");
    DeviceGuard guard(plan->device);
    return step_impl(plan, tokens_dev, positions_dev, seq_rows_dev, (hipStream_t)stream,
                     next_tokens_dev, logits_dev, priorities_dev);
  } catch (const std::exception &ex) {
    return fail(MK_ERR_PLAN, ex.what());
  }
}

int mk_prefill(mk_plan *plan, int32_t slot, const int32_t *tokens_dev, int32_t n,
               int32_t start_pos, void *stream, int32_t *next_token_dev, float *logits_dev) {
  try {
    if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
    const mk_config &c = plan->hp.cfg;
    if (slot < 0 || slot >= c.max_batch) return fail(MK_ERR_INVALID_ARG, "slot out of range");
    if (!tokens_dev || n < 1) return fail(MK_ERR_INVALID_ARG, "need n >= 1 prompt tokens");
    if (start_pos < 0 || (int64_t)start_pos + n > plan->hp.max_pos)
      return fail(MK_ERR_INVALID_ARG, "prompt positions exceed the page-table capacity");
    if (stale_static(plan))
      return fail(MK_ERR_INVALID_ARG, "a newer mk_build_plan_noalloc plan replaced this plan's state");
    DeviceGuard guard(plan->device);
    hipStream_t s = (hipStream_t)stream;
    if (mk_plan *q = plan->prefill) {
      // chunks of up to C tokens, each one step of the prefill plan; the
      // last token's slot gives the next token and the logits
      const int C = q->hp.cfg.max_batch;
      for (int i0 = 0; i0 < n; i0 += C) {
        const int cnt = std::min(C, n - i0);
        const bool last = i0 + cnt == n;
        HIP_TRY(launch_stage_chunk(q->stage_tok, q->stage_pos, q->stage_rows, C, tokens_dev + i0,
                                   cnt, start_pos + i0, slot, s),
                "prefill staging");
        int rc = step_impl(q, q->stage_tok, q->stage_pos, q->stage_rows, s, q->stage_next,
                           (last && logits_dev) ? q->stage_logits : nullptr);
        if (rc != MK_OK) return rc;
        if (last) {
          const int j = cnt - 1;
          if (next_token_dev)
            HIP_TRY(hipMemcpyAsync(next_token_dev, q->stage_next + j, 4, hipMemcpyDeviceToDevice,
                                   s),
                    "prefill token copy");
          if (logits_dev)
            HIP_TRY(hipMemcpyAsync(logits_dev, q->stage_logits + (size_t)j * c.vocab,
                                   (size_t)c.vocab * 4, hipMemcpyDeviceToDevice, s),
                    "prefill logits copy");
        }
      }
      return MK_OK;
    }
    for (int i = 0; i < n; ++i) {
      HIP_TRY(launch_stage(plan->stage_tok, plan->stage_pos, c.max_batch, slot, tokens_dev, i,
                           start_pos, s),
              "prefill staging");
      int rc = step_impl(plan, plan->stage_tok, plan->stage_pos, nullptr, s, plan->stage_next,
                         (i == n - 1 && logits_dev) ? plan->stage_logits : nullptr);
      if (rc != MK_OK) return rc;
    }
    if (next_token_dev)
      HIP_TRY(hipMemcpyAsync(next_token_dev, plan->stage_next + slot, 4, hipMemcpyDeviceToDevice, s),
              "prefill token copy");
    if (logits_dev)
      HIP_TRY(hipMemcpyAsync(logits_dev, plan->stage_logits + (size_t)slot * c.vocab,
                             (size_t)c.vocab * 4, hipMemcpyDeviceToDevice, s),
              "prefill logits copy");
    return MK_OK;
  } catch (const std::exception &ex) {
    return fail(MK_ERR_PLAN, ex.what());
  }
}

int mk_plan_status(mk_plan *plan, void *stream) {
  if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
  if (stale_static(plan))
    return fail(MK_ERR_INVALID_ARG, "a newer mk_build_plan_noalloc plan replaced this plan's state");
  if (plan->prefill) {  // errors of the prompt chunks land in the prefill plan
    const int rc = mk_plan_status(plan->prefill, stream);
    if (rc != MK_OK) {
      g_err = "prefill: " + g_err;
      return rc;
    }
  }
  DeviceGuard guard(plan->device);
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  uint32_t w[CTRL_WORDS];
  HIP_TRY(hipMemcpy(w, plan->ctrl, sizeof w, hipMemcpyDeviceToHost), "read error word");
  if (w[CTRL_ERR] == DEVERR_NONE) return MK_OK;
  char buf[256];
  int code;
  if (w[CTRL_ERR] == DEVERR_TIMEOUT) {
    snprintf(buf, sizeof buf,
             "dependency wait timed out: task %u waited on event %u (counter %u, needed %u)",
             w[CTRL_ERR_TASK], w[CTRL_ERR_EV], w[CTRL_ERR_SEEN], w[CTRL_ERR_WANT]);
    code = MK_ERR_TIMEOUT;
  } else {
    snprintf(buf, sizeof buf,
             "invalid device-side input in task %u (kind %d): value %d, limit %u",
             w[CTRL_ERR_TASK], (int)w[CTRL_ERR_EV], (int)w[CTRL_ERR_SEEN], w[CTRL_ERR_WANT]);
    code = MK_ERR_INVALID_ARG;
  }
  // Reset the error and the counters, keeping the data tag of graph-replayed
  // steps: the failed step's partial outputs carry that tag, so the next
  // step must count on from it, not restart where stale values would pass.
  HIP_TRY(hipMemset(plan->ctrl, 0, (size_t)CTRL_TAG * 4), "reset control words");
  HIP_TRY(hipMemset(plan->ctrl + CTRL_WORDS, 0, (size_t)(plan->n_ctrl_words - CTRL_WORDS) * 4),
          "reset counters");
  plan->epoch = 0;
  if (plan->d.withhold >= 0) {  // the test hook applies until its error is reported
    plan->d.withhold = -1;
    HIP_TRY(hipMemcpy(plan->d_dev, &plan->d, sizeof plan->d, hipMemcpyHostToDevice),
            "upload plan");
  }
  return fail(code, buf);
}

int mk_read_trace(mk_plan *plan, void *stream, uint32_t *out, int32_t cap) {
  if (!plan || !out) return fail(MK_ERR_INVALID_ARG, "plan and out are required");
  if (!plan->d.trace) return fail(MK_ERR_INVALID_ARG, "plan was built without debug_trace");
  DeviceGuard guard(plan->device);
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  const int T = (int)plan->hp.tasks.size();
  const int n = std::min(T, (int)cap);
  HIP_TRY(hipMemcpy(out, plan->d.trace, (size_t)n * 24, hipMemcpyDeviceToHost), "read trace");
  return MK_OK;
}

int mk_read_routing(mk_plan *plan, void *stream, int32_t *ids, float *weights, int32_t cap) {
  if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->d.tk_ids) return fail(MK_ERR_INVALID_ARG, "the plan's model has no experts");
  DeviceGuard guard(plan->device);
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  const int64_t n = std::min<int64_t>(plan->hp.n_tk, cap);
  if (n < 0) return fail(MK_ERR_INVALID_ARG, "negative capacity");
  if (ids) HIP_TRY(hipMemcpy(ids, plan->d.tk_ids, (size_t)n * 4, hipMemcpyDeviceToHost), "read ids");
  if (weights)
    HIP_TRY(hipMemcpy(weights, plan->d.tk_w, (size_t)n * 4, hipMemcpyDeviceToHost), "read weights");
  return MK_OK;
}

int mk_plan_info(const mk_plan *plan, int32_t *n_tasks, int32_t *n_events, int32_t *n_cus,
                 int32_t *n_phases) {
  if (!plan) return fail(MK_ERR_INVALID_ARG, "plan is NULL");
  if (n_tasks) *n_tasks = (int32_t)plan->hp.tasks.size();
  if (n_events) *n_events = (int32_t)plan->hp.ev_thr.size();
  if (n_cus) *n_cus = plan->hp.n_cus;
  if (n_phases) *n_phases = (int32_t)plan->hp.phases.size();
  return MK_OK;
}

void mk_free(mk_plan *plan) {
  if (!plan) return;
  DeviceGuard guard(plan->device);
  hipDeviceSynchronize();
  delete plan;
}

}  // extern "C"
