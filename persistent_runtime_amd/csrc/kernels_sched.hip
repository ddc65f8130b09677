// kernels_sched.hip -- the scheduled executor: the Mirage MPK runtime's
// division of the GPU into workers and schedulers (MPK summary, "Part 2.
// Runtime": Worker, Scheduler, event-based execution), over the same task
// code as the other executors.
//
// Workgroup 0 holds four scheduler wavefronts (the summary's "up to four
// schedulers, one warp each"); every other workgroup is a worker.  A worker
// takes the tasks dispatched into its queue in arrival order, runs each one
// (its inputs are complete when it is dispatched: no dependency polls), then
// adds its completion to each event it signals; the task whose addition
// brings an event to its threshold activates the event into the queue of
// scheduler (event mod 4).  A scheduler takes its activated events in
// order, counts each event for the tasks that wait on it, and dispatches a
// task into its worker's queue once all of its events have fired.  Every
// queue entry carries the step's tag, every counter is monotonic across steps
// (step e's thresholds are (e + 1) times the per-step ones), so no reset
// launch is needed; every wait has the plan's spin budget.
#include "kernels.h"

namespace mk {

constexpr int kSchedulers = 4;

DEV uint64_t ld64(const uint64_t *p) {
  return __hip_atomic_load((const AS1 uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st64(uint64_t *p, uint64_t v) {
  __hip_atomic_store((AS1 uint64_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint32_t add32(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int rd(const int32_t *p) { return __builtin_amdgcn_readfirstlane(ldg(p)); }

// The payload (id + 1) of queue entry p once it carries this step's tag, or
// 0 when the step is abandoned (an error elsewhere, or this wait's budget).
// One lane polls.
DEV int poll_entry(CP &d, const CallArgs &ca, const uint64_t *p, int who, int what) {
  uint64_t v = ld64(p);
  if ((uint32_t)(v >> 32) == ca.tag) return (int)(uint32_t)v;
  const uint64_t t0 = wall_clock64();
  for (int it = 1;; ++it) {  // (the error word and the clock every 16th retry)
    __builtin_amdgcn_s_sleep(1);
    v = ld64(p);
    if ((uint32_t)(v >> 32) == ca.tag) return (int)(uint32_t)v;
    if (it % 16) continue;
    if (error_set(d)) return 0;
    if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
      set_error(d, DEVERR_TIMEOUT, who, what, (uint32_t)(v >> 32), ca.tag);
      return 0;
    }
  }
}

// Put task c into its worker's queue (the next free entry of this step).
DEV void dispatch(CP &d, const CallArgs &ca, int c) {
  const int w = ldg(d.t_worker + c);
  const uint32_t n = (uint32_t)ldg(d.w_count + w);
  const uint32_t slot = add32(d.wtail + w, 1u) - ca.epoch * n;
  if (slot >= n) {  // a task dispatched twice: report, never write past the queue
    set_error(d, DEVERR_BAD_INPUT, c, -6, slot, n);
    return;
  }
  st64(d.wring + ldg(d.w_off + w) + slot, ((uint64_t)ca.tag << 32) | (uint32_t)(c + 1));
}

// Event e reached its threshold: hand it to its scheduler.
DEV void activate(CP &d, const CallArgs &ca, int e) {
  const int s = e % d.n_sched;
  const uint32_t n = (uint32_t)ldg(d.s_count + s);
  const uint32_t slot = add32(d.stail + s, 1u) - ca.epoch * n;
  if (slot >= n) {
    set_error(d, DEVERR_BAD_INPUT, -1, -7, slot, n);
    return;
  }
  st64(d.sring + ldg(d.s_off + s) + slot, ((uint64_t)ca.tag << 32) | (uint32_t)(e + 1));
}

DEV void sched_trace(CP &d, int task, int word_ticket, int word_time) {
  if (d.trace) {
    uint32_t *tr = d.trace + (size_t)task * 6;
    stg(tr + word_ticket, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
    stg(tr + word_time, (uint32_t)wall_clock64());
    if (word_ticket == 1) atomicAdd(&tr[2], 1u);
    else stg(tr + 3, (uint32_t)blockIdx.x);
  }
}

__global__ void __launch_bounds__(kThreads)
    mk_sched_kernel(const DevPlan *__restrict__ dplan, CallArgs ca_in) {
  __shared__ Smem sm;
  CP &d = *(CP *)dplan;
  const CallArgs ca = resolve_args(d, ca_in);
  const int lane = tidx() & 63, wave = __builtin_amdgcn_readfirstlane(tidx() >> 6);
  if (blockIdx.x == 0) {
    // ---- schedulers: one wavefront each; the workgroup's other waves idle
    if (wave >= d.n_sched) return;
    const int s = wave;
    for (int i = s; i < d.n_roots; i += d.n_sched)
      if (lane == 0) dispatch(d, ca, ldg(d.roots + i));
    const int n = rd(d.s_count + s), off = rd(d.s_off + s);
    for (int k = 0; k < n; ++k) {
      int e1 = 0;
      if (lane == 0) e1 = poll_entry(d, ca, d.sring + off + k, -2, s);
      e1 = __shfl(e1, 0, 64);
      if (e1 <= 0) return;
      const int e = e1 - 1;
      const int c0 = rd(d.cons_off + e), c1 = rd(d.cons_off + e + 1);
      for (int i = c0 + lane; i < c1; i += 64) {
        const int c = ldg(d.cons + i);
        const uint32_t old = add32(d.pending + c, 1u);
        if (old + 1u == (ca.epoch + 1u) * (uint32_t)ldg(d.n_deps + c)) dispatch(d, ca, c);
      }
    }
    return;
  }
  // ---- workers
  if (tidx() == 0) sm.imisc[2] = 0;
  const int w = (int)blockIdx.x - 1;
  const int n = rd(d.w_count + w), off = rd(d.w_off + w);
  for (int k = 0; k < n; ++k) {
    if (tidx() == 0) sm.imisc[4] = poll_entry(d, ca, d.wring + off + k, -3 - w, k);
    __syncthreads();
    const int id = __builtin_amdgcn_readfirstlane(sm.imisc[4]) - 1;
    if (id < 0 || id >= d.n_tasks) break;
    const TD t = td_from_table(d.tasks, ((const AS4 int *)d.task_pos)[id]);
    if (tidx() == 0) sched_trace(d, id, 0, 4);
    WState ws;
    init_ws(ws);
    run_task_once(sm, d, ca, t, ws);
    vm_drain();  // this task's outputs are complete before its events count it
    __syncthreads();
    if (tidx() == 0) {
      sched_trace(d, id, 1, 5);
      // split attention: only the split that arrived last (and merged)
      // reports its group's completion
      const uint32_t cnt = (t.op == OP_ATTN && d.S > 1) ? (uint32_t)(sm.imisc[1] != 0) : 1u;
      for (int i = 0; i < t.n_sig && i < 2; ++i) {
        const int e = t.sig_ev[i] & ~kDataEdge;
        if (cnt == 0) continue;
        const uint32_t want = (ca.epoch + 1u) * (uint32_t)ldg(d.ev_thr + e);
        if (add32(d.ev + (size_t)e * kCtrStride, cnt) + cnt == want) activate(d, ca, e);  // (ev_rep 1)
      }
      sm.imisc[4] = 0;
    }
    __syncthreads();
  }
  vm_drain();  // LDS-DMA loads the compiler does not track complete before the wave ends
}

hipError_t launch_sched(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s) {
  void *args[] = {(void *)&d, (void *)&ca};
  // workers and schedulers wait on each other: all must be resident
  return hipLaunchCooperativeKernel((const void *)mk_sched_kernel, dim3(grid), dim3(kThreads),
                                    args, 0, s);
}

}  // namespace mk
