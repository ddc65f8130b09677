// kernels.h -- device code of the decode-step megakernel for gfx950, included
// by the kernel sources (one per persistent-kernel mode, compiled in parallel).
//
// The persistent kernel follows the Cohere megakernel article ("Egyetlen
// tartós kernelre épül a kiszolgálás"): exactly one workgroup per CU stays
// resident for the whole step and works from a task list the host prepared;
// dependencies are counters in global memory.  Each workgroup is one worker of
// the Mirage MPK runtime ("Part 2. Runtime", Worker): it runs its own queue of
// tasks in order and bumps event counters as tasks finish.  Inside the
// workgroup the roles MPK gives to separate SMs are split between waves: wave
// 0 is the control wave (it polls dependency counters, keeps the next task
// descriptors in an LDS ring, writes a tile's outputs and signals), waves 1..7
// only stream weights and compute.  Keeping control traffic out of the
// compute waves matters on gfx950, where one counter (vmcnt) tracks all of a
// wave's outstanding loads and stores: a wave that polls or drains its stores
// would also wait for its weight prefetches.
//
// Weights never change, so the compute waves load the next tile's weights
// while the current tile is still being reduced and published, and before the
// next tile's inputs are ready: the Cohere article's weight prefetch ("Honnan
// jön a gyorsulás?").
//
// Activations a task writes and another reads go through HBM with
// agent-coherent (sc1) stores and loads; a producer's wave waits for its
// stores to complete and then bumps the counter with a relaxed atomic, so no
// L2 write-back or invalidate fence is needed on the multi-XCD MI355X.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "mk_task.h"

namespace mk {

#define DEV __device__ __forceinline__

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers --
// The plan and the task table are read through the constant address space
// (scalar loads, uniform values in SGPRs); activations, weights and the KV
// cache through the global address space (global_load / global_store rather
// than flat accesses, which would also count against LDS waits).
#define AS1 __attribute__((address_space(1)))
#define AS4 __attribute__((address_space(4)))
typedef const AS4 DevPlan CP;
typedef const AS4 Task CT;

template <class T> DEV T ldg(const T *p) { return *(const AS1 T *)p; }
template <class T> DEV void stg(T *p, T v) { *(AS1 T *)p = v; }
template <class T> DEV T ldnt(const T *p) { return __builtin_nontemporal_load((const AS1 T *)p); }
template <class T> DEV const T *tab(const T *const *t, size_t i) {
  return ((const T *const AS4 *)t)[i];
}

DEV float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
DEV float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
DEV float bf1(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
DEV uint16_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
// The work-item id, re-materialised at each use: the opaque copy keeps the
// compiler from hoisting lane-dependent offsets out of the worker loop and
// holding them in registers for the whole kernel.
DEV int tidx() {
  int v = (int)threadIdx.x;
  asm volatile("" : "+v"(v));
  return v;
}
DEV float unif(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
DEV float lanef(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// DPP lane permutations (all 64 lanes must be active)
enum : int {
  DPP_XOR1 = 0xB1,        // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,        // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141,  // lane i <- lane 7-i within 8
  DPP_MIRROR = 0x140,       // lane i <- lane 15-i within 16
  DPP_ROR8 = 0x128          // lane i <- lane i^8 within 16 (row rotate by 8)
};
template <int CTRL> DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL> DEV int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// sum of all 64 lanes, returned uniform
DEV float wave_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  v += dpp<DPP_MIRROR>(v);  // every lane holds its 16-lane row sum
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}
// maximum of all 64 lanes, returned uniform
DEV float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}
DEV float silu(float z) { return z / (1.0f + __expf(-z)); }
// (value, index) maximum; NaN never wins, equal values keep the lower index
DEV bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
// (value, index) maximum over the wave, uniform result
DEV void wave_argmax(float &v, int &i) {
#define MK_STEP(C)                                    \
  {                                                   \
    const float ov = dpp<C>(v);                       \
    const int oi = dppi<C>(i);                        \
    if (better(ov, oi, v, i)) { v = ov; i = oi; }     \
  }
  MK_STEP(DPP_XOR1)
  MK_STEP(DPP_XOR2)
  MK_STEP(DPP_HALF_MIRROR)
  MK_STEP(DPP_MIRROR)
#undef MK_STEP
  float bv = lanef(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
  for (int r = 16; r < 64; r += 16) {
    const float ov = lanef(v, r);
    const int oi = __builtin_amdgcn_readlane(i, r);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  v = bv;
  i = bi;
}

// Activations that one task writes and another reads: agent-coherent
// accesses (sc1: written through to memory, read past the per-XCD L2).
DEV float lda(const float *p) {
  return __hip_atomic_load((const AS1 float *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void sta(float *p, float v) {
  __hip_atomic_store((AS1 float *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void sta16(uint16_t *p, uint16_t v) {
  __hip_atomic_store((AS1 uint16_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int ldai(const int32_t *p) {
  return __hip_atomic_load((const AS1 int32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void stai(int32_t *p, int32_t v) {
  __hip_atomic_store((AS1 int32_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Element i of a tagged vector (value, tag pairs): one 8-byte store, so a
// reader that sees the tag sees the value; the value alone for readers whose
// ordering is already established.
DEV void stt(float *pairs, size_t i, float v, uint32_t tag) {
  __hip_atomic_store((AS1 uint64_t *)pairs + i, ((uint64_t)tag << 32) | __float_as_uint(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV float ldv(const float *pairs, size_t i) { return lda(pairs + 2 * i); }
// The values-only copy of a tagged vector (matrix-core plans; see DevPlan).
DEV const float *shadow_of(CP &d, const float *pairs) {
  return d.shadow + (pairs - d.pair0) / 2;
}
// stt, plus the value into the copy when the plan keeps one: for the
// vectors matrix-core tiles read (x, x_mid, attention output, h)
DEV void stv(CP &d, float *pairs, size_t i, float v, uint32_t tag) {
  stt(pairs, i, v, tag);
  if (d.shadow) sta(const_cast<float *>(shadow_of(d, pairs)) + i, v);
}
constexpr int kCpolSc1 = 16;  // cache-policy bit: device-scope coherent
DEV __amdgpu_buffer_rsrc_t rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}
// 16-byte coherent load at byte offset `off` from a uniform base
DEV f32x4 lda4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
}
// wait until this wave's vector memory operations (its stores) completed
DEV void vm_drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kPartSlot = kMaxTileUnits * 4;   // GEMV partials per slot of a tile
constexpr int kRowSlot = kMaxTileUnits * 2;    // rows per tile (rows hold >= 256 elements)
#ifndef MK_REFILL_PER_SLOT
#define MK_REFILL_PER_SLOT 0
#endif
constexpr bool kRefillPerSlot = MK_REFILL_PER_SLOT;
constexpr int kRing = 4;                          // task descriptors kept ahead
constexpr int kAttnScratchOff = kLdsWbufOff - kWaves * 1024;  // attention: a kilobyte per wave

struct Smem {
  float xs[kLdsXBytes / 4];                                 // staged activations
  float red[kMaxPass][kPartSlot];                           // GEMV partials [pass*n + slot]
  float rows[kMaxPass][kRowSlot];                           // GEMV row sums, same order
  uint32_t ring[kRing][32];                                 // task descriptors
  float misc[64];
  int imisc[64];
  int order[kMfmaMaxBatch];  // claimed attention: slot of each claim rank
};

// A task descriptor held in scalar registers.
struct TD {
  int op, layer, n_wait, n_sig, a0, a1, a2, a3, a4, a5;
  int wait_ev[3], wait_thr[3], sig_ev[2];
  const uint16_t *w0, *w1;
  const float *src;
  float *dst;
  const float *aux;
  const uint16_t *gain;
  int K, ostride, gidx, rpp;
};

DEV const void *ptr_of(uint32_t lo, uint32_t hi) {
  return (const void *)(((uint64_t)hi << 32) | lo);
}
// Decode the 32 words of a Task (layout in mk_task.h); `w` must be uniform.
DEV TD decode_td(const uint32_t *w) {
  TD t;
  t.op = (int)(int16_t)(w[0] & 0xffffu);
  t.layer = (int)(int16_t)(w[0] >> 16);
  t.n_wait = (int)(int16_t)(w[1] & 0xffffu);
  t.n_sig = (int)(int16_t)(w[1] >> 16);
  t.a0 = (int)w[2]; t.a1 = (int)w[3]; t.a2 = (int)w[4]; t.a3 = (int)w[5];
  t.a4 = (int)w[6]; t.a5 = (int)w[7];
  for (int i = 0; i < 3; ++i) { t.wait_ev[i] = (int)w[8 + i]; t.wait_thr[i] = (int)w[11 + i]; }
  t.sig_ev[0] = (int)w[14]; t.sig_ev[1] = (int)w[15];
  t.w0 = (const uint16_t *)ptr_of(w[16], w[17]);
  t.w1 = (const uint16_t *)ptr_of(w[18], w[19]);
  t.src = (const float *)ptr_of(w[20], w[21]);
  t.dst = (float *)ptr_of(w[22], w[23]);
  t.aux = (const float *)ptr_of(w[24], w[25]);
  t.gain = (const uint16_t *)ptr_of(w[26], w[27]);
  t.K = (int)w[28]; t.ostride = (int)w[29]; t.gidx = (int)w[30]; t.rpp = (int)w[31];
  return t;
}
// From the LDS ring (every lane reads the same words; made uniform).
DEV TD td_from_ring(const uint32_t *slot) {
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 v = ((const u32x4 *)slot)[i];
    w[4 * i + 0] = (uint32_t)uni((int)v.x);
    w[4 * i + 1] = (uint32_t)uni((int)v.y);
    w[4 * i + 2] = (uint32_t)uni((int)v.z);
    w[4 * i + 3] = (uint32_t)uni((int)v.w);
  }
  return decode_td(w);
}
// From global memory through the scalar cache (kernel-per-op launches).
DEV TD td_from_table(const Task *tab, int pos) {
  const AS4 uint32_t *p = (const AS4 uint32_t *)(tab + pos);
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = p[i];
  return decode_td(w);
}

// Per-worker uniform state carried from task to task (identical in every
// wave, so uniform decisions need no communication).
struct WState {
  const float *x_src;      // LDS activation cache key: source, gain, row length
  const uint16_t *x_gain;
  int x_K, x_nb;
  int sat_ev[2];           // recently satisfied waits (event, wanted count)
  uint32_t sat_want[2];
  int rt_layer, rt_slot;   // routing held in LDS (sm.imisc/misc[48..]) for this
                           // (layer, slot) of this step, or -1
};

DEV void init_ws(WState &ws) {
  ws.x_src = nullptr;
  ws.x_gain = nullptr;
  ws.x_K = 0;
  ws.x_nb = 0;
  ws.sat_ev[0] = ws.sat_ev[1] = -1;
  ws.sat_want[0] = ws.sat_want[1] = 0;
  ws.rt_layer = ws.rt_slot = -1;
}

DEV void set_error(CP &d, uint32_t code, int task, int ev, uint32_t seen, uint32_t want);

// The page-table row of slot b's sequence (a prompt chunk's slots share one);
// a row outside the table is reported (task tix) and row 0 read instead.
DEV const int32_t *page_row(CP &d, const CallArgs &ca, int b, int tix) {
  const int r = ca.rows ? uni(ldg(ca.rows + b)) : b;
  const bool ok = r >= 0 && r < d.pt_rows;
  if (!ok && tidx() == 0) set_error(d, DEVERR_BAD_INPUT, tix, -5, (uint32_t)r, (uint32_t)d.pt_rows);
  return d.page_table + (size_t)(ok ? r : 0) * d.maxp;
}

DEV void set_error(CP &d, uint32_t code, int task, int ev, uint32_t seen, uint32_t want) {
  if (atomicCAS(&d.ctrl[CTRL_ERR], 0u, code) == 0u) {
    __hip_atomic_store(&d.ctrl[CTRL_ERR_TASK], (uint32_t)task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_EV], (uint32_t)ev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_SEEN], seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_WANT], want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// Event counter e is ev_rep replicas, each in a line of its own: a worker
// counts its completions on replica (worker % ev_rep), a waiter adds them
// up, so the signals of an operation's tiles spread over ev_rep lines.
DEV uint32_t *ev_word(CP &d, int e, int r) {
  return d.ev + ((size_t)e * d.ev_rep + r) * kCtrStride;
}
// Control wave: the count of event e over its replicas (lane r loads r).
DEV uint32_t ev_count(CP &d, int e) {
  const int lane = tidx() & 63;
  uint32_t v = 0;
  if (lane < d.ev_rep) v = __hip_atomic_load(ev_word(d, e, lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t s = 0;
  for (int r = 0; r < d.ev_rep; ++r) s += (uint32_t)__builtin_amdgcn_readlane((int)v, r);
  return s;
}
DEV bool error_set(CP &d) {
  return __hip_atomic_load(&d.ctrl[CTRL_ERR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// ------------------------------------------------------- dependency waits --
// A task needs each of its events' counters to reach (epoch+1)*threshold.
// Waits this worker already saw satisfied in this step are skipped without a
// poll (tiles of one operation share their input event).  Otherwise thread 0
// (control wave) polls; a barrier hands the outcome to the workgroup.
// Only the task's waits i0 .. i1-1 are considered (a task may wait for its
// inputs in stages).  Returns false when the step is being drained after an
// error.
DEV bool static_weights(int op);
DEV bool wait_deps(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws, int i0 = 0,
                   int i1 = 3) {
  i1 = min(i1, t.n_wait);
  bool need = false;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i < i0) continue;
    if (i >= i1) break;
    const int e = t.wait_ev[i];
    if (e & kDataEdge) continue;  // the staged data carries its own readiness
    const uint32_t want = (ca.epoch + 1u) * (uint32_t)t.wait_thr[i];
    const bool seen = (ws.sat_ev[0] == e && ws.sat_want[0] == want) ||
                      (ws.sat_ev[1] == e && ws.sat_want[1] == want);
    need = need || !seen;
  }
  if (!need) return true;
  if (uni(tidx() >> 6) == 0) {  // the control wave polls (lane r: replica r)
    int ok = 1;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i < i0) continue;
      if (i >= i1 || !ok) break;
      if (t.wait_ev[i] & kDataEdge) continue;
      const int e = t.wait_ev[i];
      const uint32_t want = (ca.epoch + 1u) * (uint32_t)t.wait_thr[i];
      uint32_t seen = ev_count(d, e);
      if ((int32_t)(seen - want) < 0) {
        const uint64_t t0 = wall_clock64();
        // one memory round trip per retry: the error word and the clock are
        // looked at every 16th
        for (int it = 1;; ++it) {
          __builtin_amdgcn_s_sleep(1);
          seen = ev_count(d, e);
          if ((int32_t)(seen - want) >= 0) break;
          if (it % 16) continue;
          if (error_set(d)) { ok = 0; break; }
          if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
            set_error(d, DEVERR_TIMEOUT, t.gidx, t.wait_ev[i], seen, want);
            ok = 0;
            break;
          }
        }
      }
    }
    // Matrix-core plans read their inputs through the L2 (every CU of an
    // XCD stages the same activations): acquire at agent scope, which
    // drops lines the XCD's L2 may hold from before the producers wrote.
    // Plans whose tiles copy their activations device-coherently (mx_sc1)
    // skip it for those tiles: every other input of a tile (residuals,
    // split-K partials) is read with coherent loads as well.  Attention
    // skips it too, unless the layer's KVAPP tasks wrote cache pages in this
    // step: it reads the query, key and value with coherent loads, and the
    // pages and the page table were written before the launch (8B ragged:
    // 4 slots -1.2 %, 8 slots -1.7 %, 16 slots -0.8 %).
    if (ok && d.mfma && !(d.mx_sc1 && static_weights(t.op)) &&
        !(t.op == OP_ATTN && !d.kv_first))
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tidx() == 0) sm.imisc[0] = ok;
  }
  __syncthreads();
  const bool ok = sm.imisc[0] != 0;
  if (ok) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i < i0) continue;
      if (i >= i1) break;
      if (t.wait_ev[i] & kDataEdge) continue;
      ws.sat_ev[1] = ws.sat_ev[0];
      ws.sat_want[1] = ws.sat_want[0];
      ws.sat_ev[0] = t.wait_ev[i];
      ws.sat_want[0] = (ca.epoch + 1u) * (uint32_t)t.wait_thr[i];
    }
  }
  return ok;
}

// Debug trace, 6 words per task: start / finish tickets from one shared
// clock counter (trace mode 1 only: it serialises), run count, workgroup,
// start / finish time (100 MHz).  Trace mode 2 keeps times only and uses
// words 0 and 1 for intermediate time stamps.
DEV void trace_start(CP &d, const TD &t) {
  if (d.trace && d.trace_mode != 3 && tidx() == 0) {
    uint32_t *tr = d.trace + (size_t)t.gidx * 6;
    if (d.trace_mode == 1) stg(tr + 0, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
    atomicAdd(&tr[2], 1u);
    stg(tr + 3, (uint32_t)blockIdx.x);
    stg(tr + 4, (uint32_t)wall_clock64());
  }
}
DEV void trace_finish(CP &d, const TD &t) {
  if (d.trace && d.trace_mode != 3 && tidx() == 0) {
    uint32_t *tr = d.trace + (size_t)t.gidx * 6;
    if (d.trace_mode == 1) stg(tr + 1, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
    stg(tr + 5, (uint32_t)wall_clock64());
  }
}
DEV void trace_mark(CP &d, const TD &t, int word) {
  if (d.trace && d.trace_mode == 2 && tidx() == 0)
    stg(d.trace + (size_t)t.gidx * 6 + word, (uint32_t)wall_clock64());
}
// Report the task's completions (a5 of them; 0 when a later task of the same
// run reports them).  The caller (thread 0) has drained its wave's stores.
DEV void signal_count(CP &d, const TD &t, int count) {
  if (tidx() == 0 && count > 0 && t.gidx != d.withhold) {
    const int r = (int)(blockIdx.x % (uint32_t)d.ev_rep);  // this worker's replica
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (i < t.n_sig && !(t.sig_ev[i] & kDataEdge))
        __hip_atomic_fetch_add(ev_word(d, t.sig_ev[i], r), (uint32_t)count, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  }
}
DEV void signal_done(CP &d, const TD &t) { signal_count(d, t, t.a5); }
DEV bool signals_counter(const TD &t) {
  return (t.n_sig > 0 && !(t.sig_ev[0] & kDataEdge)) || (t.n_sig > 1 && !(t.sig_ev[1] & kDataEdge));
}

// ------------------------------------------------------------ GEMV tiles --
// A tile is `nseg` blocks of `seg_rows` consecutive rows (row length K bf16)
// cut at the same row offset (gate and up share a tile), read as one
// flattened sequence of elements.  It is streamed as 1 KiB chunks (64 lanes x
// 16 bytes); compute wave c owns chunks [c*cpw, (c+1)*cpw).  Every lane keeps
// its loads in registers and multiplies them with the activations staged in
// LDS; each 16-lane DPP row of a chunk (128 elements) is summed and stored as
// one partial, so the partials of the tile are in element order.  Rows are
// multiples of 256 elements, hence a row owns the contiguous partials
// [r*K/128, (r+1)*K/128), which the epilogue adds up in a fixed order
// (deterministic).  No lane-dependent branch is needed anywhere: a chunk's
// address is a select between the two segment bases, the lane's column
// advances by 512 mod K per chunk.
typedef u32x4 Buf[kMaxChunks];  // one tile's weights, per lane (16-byte slots)


struct Geo {
  const uint16_t *seg0, *seg1;
  uint32_t seg_bytes;  // bytes of the first segment
  int K, units, cpw, step;
};

DEV Geo make_geo(const uint16_t *s0, const uint16_t *s1, int seg_rows, int nseg, int K) {
  Geo g;
  g.seg0 = s0;
  g.seg1 = s1;
  g.seg_bytes = (uint32_t)seg_rows * (uint32_t)K * 2u;
  g.K = K;
  g.units = (nseg * seg_rows * K) >> 9;
  g.cpw = (g.units + kCW - 1) / kCW;
  g.step = 512 % K;
  return g;
}
DEV int cw_chunks(const Geo &g, int cw) { return min(g.cpw, g.units - cw * g.cpw); }

// Target of the refills that have no next tile: one 1 KiB line every CU
// reads (it stays in the L2), so a register slot is always written by a load
// without streaming anything from HBM.
static __device__ __attribute__((aligned(1024))) u32x4 kIdleLine[64];
DEV uint64_t idle_addr() { return (uint64_t)&kIdleLine[tidx() & 63]; }

// Address of lane's 16 bytes of chunk j of compute wave cw in tile g; slots
// beyond the wave's chunks read the idle line instead, so every slot is
// written by a load.  Unconditional loads
// keep each slot in one register across tiles: a slot that a branch might
// leave unchanged would be copied between registers, which forces a wait for
// every load in flight.
DEV uint64_t slot_addr(const Geo &g, int cw, int j) {
  const uint32_t lane16 = (uint32_t)(tidx() & 63) * 16u;
  const uint32_t o = (uint32_t)(cw * g.cpw + j) * 1024u + lane16;
  const uint64_t b0 = (uint64_t)g.seg0, b1 = (uint64_t)g.seg1 - g.seg_bytes;
  const uint64_t a = (o < g.seg_bytes ? b0 : b1) + o;
  return j < cw_chunks(g, cw) ? a : idle_addr();
}

// LDS slots (single-slot plans): compute wave cw's chunks kMaxChunks ..
// kMaxChunks+kLdsSlots-1 of every pass live in LDS at kLdsWbufOff of the
// activation stage, one 1 KiB slot each, and are filled by LDS-DMA (64 lanes
// x 16 bytes to consecutive addresses from the M0 base; the compiler does
// not track these loads, nothing else in this kernel uses M0).  Every pass
// issues the register refills first, then the slots' DMAs, always all of
// them (slots without a chunk load the idle line), so when the slots are
// consumed exactly kMaxChunks vector-memory operations were issued after the
// last DMA: waiting for that count completes them all.  The compiler's own
// waits for the register slots do not count the DMAs and wait for a few
// loads more than needed, which is safe.
DEV uint32_t wslot(const float *xs, int cw, int s) {
  return (uint32_t)(uintptr_t)xs + (uint32_t)kLdsWbufOff + (uint32_t)(cw * kLdsSlots + s) * 1024u;
}
DEV void dma16(uint64_t src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
               : "memory", "m0");
}
// The same, device-coherent (sc1): reads what other CUs wrote through to
// memory without an L2 invalidate.
DEV void dma16_sc1(uint64_t src, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src), "s"(m0)
               : "memory", "m0");
}
// All kLdsSlots slots of a pass at once: the last slot's DMA (and so every
// earlier one) is complete once only the kMaxChunks register reloads issued
// after it remain; then four reads at a time, each group waited for in its
// own statement.
DEV void take_slots(uint32_t a, u32x4 (&v)[kLdsSlots]) {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kMaxChunks) : "memory");
#pragma unroll
  for (int s = 0; s < kLdsSlots; s += 4)
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(v[s]), "=v"(v[s + 1]), "=v"(v[s + 2]), "=v"(v[s + 3])
        : "v"(a + (uint32_t)s * 1024u)
        : "memory");
}

// Issue the loads of compute wave cw's chunks of a tile into w (and its LDS
// slots when lds).
DEV void load_slots(const Geo &g, Buf &w, int cw, const float *xs, bool lds) {
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) w[j] = ldnt((const u32x4 *)slot_addr(g, cw, j));
  if (lds) {
#pragma unroll
    for (int s = 0; s < kLdsSlots; ++s) dma16(slot_addr(g, cw, kMaxChunks + s), wslot(xs, cw, s));
  }
}

DEV float dot8(u32x4 w, const float *x) {
  const f32x4 a = *(const f32x4 *)x, b = *(const f32x4 *)(x + 4);
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  s = fmaf(bf_lo(w.z), b.x, s);
  s = fmaf(bf_hi(w.z), b.y, s);
  s = fmaf(bf_lo(w.w), b.z, s);
  s = fmaf(bf_hi(w.w), b.w, s);
  return s;
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets it.
DEV float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Compute wave cw: the partials of its chunks with the staged activations xs
// of one slot into part[4*chunk + DPP row].  Each slot is reloaded with the
// same slot of `gn` as soon as it has been used (the idle line where gn has
// no such chunk), so the next pass streams in while this one is consumed.
// The body is straight-line code (uniform branches only), which lets the
// compiler wait for each slot with "all but the newest loads done" instead
// of draining the queue.
DEV void gemv_dot1(const Geo &g, Buf &w, const float *xs, float *part, int cw, const Geo &gn,
                   bool lds) {
  const int lane = tidx() & 63;
  const int cnt = cw_chunks(g, cw);
  const int q0 = cw * g.cpw;
  int col = (int)(((uint32_t)q0 * 512u + (uint32_t)lane * 8u) % (uint32_t)g.K);
  float *pp = part + q0 * 4 + (lane >> 4);
  const bool writer = (lane & 15) == 0;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    if (j < cnt) {
      const float v = row16_sum(dot8(w[j], xs + col));
      if (writer) pp[j * 4] = v;
      col += g.step;
      col = col >= g.K ? col - g.K : col;
    }
    w[j] = ldnt((const u32x4 *)slot_addr(gn, cw, j));
    __builtin_amdgcn_sched_barrier(0);  // keep each reload right after its use
  }
  if (lds) {
    u32x4 v[kLdsSlots];
    take_slots(wslot(xs, cw, 0) + (uint32_t)lane * 16u, v);
#pragma unroll
    for (int s = 0; s < kLdsSlots; ++s) {
      const int j = kMaxChunks + s;
      if (j < cnt) {
        const float r = row16_sum(dot8(v[s], xs + col));
        if (writer) pp[j * 4] = r;
        col += g.step;
        col = col >= g.K ? col - g.K : col;
      }
    }
#pragma unroll
    for (int s = 0; s < kLdsSlots; ++s) dma16(slot_addr(gn, cw, kMaxChunks + s), wslot(xs, cw, s));
  }
}

// The same for n > 1 staged slots (rows xs[b*K ..), partials at
// part[b*kPartSlot ..)); the next tile is loaded after the last slot.
DEV void gemv_dotn(const Geo &g, Buf &w, const float *xs, int n, float *part, int cw) {
  const int lane = tidx() & 63;
  const int cnt = cw_chunks(g, cw);
  const int q0 = cw * g.cpw;
  const bool writer = (lane & 15) == 0;
  for (int b = 0; b < n; ++b) {
    int col = (int)(((uint32_t)q0 * 512u + (uint32_t)lane * 8u) % (uint32_t)g.K);
    float *pp = part + b * kPartSlot + q0 * 4 + (lane >> 4);
    const float *xb = xs + b * g.K;
#pragma unroll
    for (int j = 0; j < kMaxChunks; ++j) {
      if (j < cnt) {
        const float v = row16_sum(dot8(w[j], xb + col));
        if (writer) pp[j * 4] = v;
        col += g.step;
        col = col >= g.K ? col - g.K : col;
      }
    }
  }
}

// Row sums of a task's rows for n slots, over the compute waves: row r of
// pass p is the sum of its K/128 partials part[(p*n + b)*kPartSlot + r*K/128
// ..].  Each 16-lane DPP row takes one output row: every lane adds up a
// strided share of the partials, then the 16 lanes reduce by DPP (fixed
// order: deterministic).  rows_p(p) gives the rows of pass p (both segments).
template <class RowsOf>
DEV void gemv_rows(int K, int P, RowsOf rows_p, const float *part, float *rows, int n, int cw) {
  const int lane = tidx() & 63, grp = lane >> 4, j = lane & 15;
  const int ne = K >> 7;
  for (int p = 0; p < P; ++p) {
    const int R = rows_p(p);
    for (int b = 0; b < n; ++b) {
      const float *pp = part + (p * n + b) * kPartSlot;
      float *rr = rows + (p * n + b) * kRowSlot;
      for (int r0 = cw * 4; r0 < R; r0 += kCW * 4) {
        const int r = r0 + grp;
        float v = 0.f;
        if (r < R)
          for (int e = j; e < ne; e += 16) v += pp[r * ne + e];
        v = row16_sum(v);
        if (j == 0 && r < R) rr[r] = v;
      }
    }
  }
}

// Stage nb activation rows src[b*K .. +K) (written by other tasks) into LDS;
// with a gain vector, RMS-normalise each row: x / sqrt(mean(x^2) + eps) * g.
// All waves take part.  Skipped when the same rows are already staged (the
// worker's previous tile of the same operation).  Ends with a barrier.
DEV void stage_x(Smem &sm, WState &ws, const float *src, int K, int nb, const uint16_t *gain,
                 float eps) {
  if (ws.x_src == src && ws.x_gain == gain && ws.x_K == K && ws.x_nb == nb) return;
  const int tid = tidx(), lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t r = rsrc(src);
  if (!gain) {
    // no normalisation: the nb rows are one flat copy, four 16-byte loads
    // in flight per lane (K is a multiple of 256: every range test below is
    // wave-uniform)
    const int n4 = nb * (K / 4);
    f32x4 *d4 = (f32x4 *)sm.xs;
    for (int i0 = uni(wave) * 64; i0 < n4; i0 += 4 * kThreads) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * kThreads < n4)
          v[u] = lda4(r, (uint32_t)((size_t)(i0 + u * kThreads + lane) * 16));
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * kThreads < n4) d4[i0 + u * kThreads + lane] = v[u];
    }
    __syncthreads();
    ws.x_src = src;
    ws.x_gain = gain;
    ws.x_K = K;
    ws.x_nb = nb;
    return;
  }
  const u32x2 *g2 = (const u32x2 *)gain;  // four bf16 gains per 16-byte vector
  for (int b = 0; b < nb; ++b) {
    f32x4 *d4 = (f32x4 *)(sm.xs + (size_t)b * K);
    float ss = 0.f;
    // Up to four 16-byte loads (and their gains) in flight per lane before
    // any is consumed.  K is a multiple of 256, so every range test below is
    // wave-uniform.  LDS receives x * gain; the row's 1/rms follows below.
    for (int i0 = uni(wave) * 64; i0 < K / 4; i0 += 4 * kThreads) {
      f32x4 v[4];
      u32x2 gv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        gv[u] = (u32x2){0x3f803f80u, 0x3f803f80u};  // bf16 ones
        if (i0 + u * kThreads < K / 4) {
          const int i = i0 + u * kThreads + lane;
          v[u] = lda4(r, (uint32_t)((size_t)b * K * 4 + (size_t)i * 16));
          if (gain) gv[u] = ldg(g2 + i);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ss = fmaf(v[u].x, v[u].x, ss);
        ss = fmaf(v[u].y, v[u].y, ss);
        ss = fmaf(v[u].z, v[u].z, ss);
        ss = fmaf(v[u].w, v[u].w, ss);
        if (i0 + u * kThreads < K / 4)
          d4[i0 + u * kThreads + lane] =
              (f32x4){v[u].x * bf_lo(gv[u].x), v[u].y * bf_hi(gv[u].x), v[u].z * bf_lo(gv[u].y),
                      v[u].w * bf_hi(gv[u].y)};
      }
    }
    if (gain) {
      ss = wave_sum(ss);
      if (lane == 0) sm.misc[b * kWaves + wave] = ss;
    }
  }
  __syncthreads();
  if (gain) {
    for (int b = 0; b < nb; ++b) {
      float tot = 0.f;
      for (int w = 0; w < kWaves; ++w) tot += sm.misc[b * kWaves + w];
      const float rs = 1.0f / sqrtf(tot / (float)K + eps);
      f32x4 *xb = (f32x4 *)(sm.xs + (size_t)b * K);
      for (int i = tid; i < K / 4; i += kThreads) xb[i] = xb[i] * rs;
    }
    __syncthreads();
  }
  ws.x_src = src;
  ws.x_gain = gain;
  ws.x_K = K;
  ws.x_nb = nb;
}

// A lane whose 16-byte load (two value/tag pairs of a tagged vector) shows
// an older tag loads it again until both tags are this step's, the spin
// budget runs out or another worker has failed; sm.imisc[2] = tag marks a
// failure for the workgroup.
DEV u32x4 wait_pairs(Smem &sm, CP &d, const CallArgs &ca, const TD &t,
                     __amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  const uint32_t tag = ca.tag;
  const uint64_t t0 = wall_clock64();
  // one memory round trip per retry: the error word and the clock are
  // looked at before every 16th
  for (int it = 0; v.y != tag || v.w != tag; ++it) {
    if (it % 16 == 15) {
      if (error_set(d)) {
        sm.imisc[2] = (int)tag;
        break;
      }
      if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
        set_error(d, DEVERR_TIMEOUT, t.gidx, -4, v.y != tag ? v.y : v.w, tag);
        sm.imisc[2] = (int)tag;
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
    v = __builtin_bit_cast(u32x4, lda4(r, off));
  }
  return v;
}

// Value of element i of a tagged vector, loaded until it carries this step's
// tag (or the step is abandoned: sm.imisc[2] = tag).
DEV uint64_t ldt_raw(const float *pairs, size_t i) {
  return __hip_atomic_load((const AS1 uint64_t *)pairs + i, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// ldt_wait, given the pair's first load v (issued earlier, beside others)
DEV float ldt_then(Smem &sm, CP &d, const CallArgs &ca, const TD &t, const float *pairs, size_t i,
                   uint64_t v) {
  const AS1 uint64_t *p = (const AS1 uint64_t *)pairs + i;
  if ((uint32_t)(v >> 32) != ca.tag) {
    const uint64_t t0 = wall_clock64();
    for (int it = 0; (uint32_t)(v >> 32) != ca.tag; ++it) {
      if (it % 16 == 15) {  // (as in wait_pairs)
        if (error_set(d)) {
          sm.imisc[2] = (int)ca.tag;
          break;
        }
        if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
          set_error(d, DEVERR_TIMEOUT, t.gidx, -4, (uint32_t)(v >> 32), ca.tag);
          sm.imisc[2] = (int)ca.tag;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
      v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return __uint_as_float((uint32_t)v);
}
DEV float ldt_wait(Smem &sm, CP &d, const CallArgs &ca, const TD &t, const float *pairs, size_t i) {
  return ldt_then(sm, d, ca, t, pairs, i, ldt_raw(pairs, i));
}

// Stage nb rows of a tagged vector into LDS exactly as stage_x does (x*g,
// then 1/rms).  The tags stand in for the dependency wait: the rows are
// complete once every element carries this step's tag.  Returns false (in
// every wave) when the step is abandoned.
DEV bool stage_xt(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws, const float *src,
                  int K, int nb, const uint16_t *gain) {
  if (ws.x_src == src && ws.x_gain == gain && ws.x_K == K && ws.x_nb == nb) return true;
  const int tid = tidx(), lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t r = rsrc(src);
  const int K2 = K / 2;                         // 16-byte loads per row
  const uint32_t *g1 = (const uint32_t *)gain;  // two bf16 gains per load
  for (int b = 0; b < nb; ++b) {
    float2 *d2 = (float2 *)(sm.xs + (size_t)b * K);
    float ss = 0.f;
    // K is a multiple of 256: every range test below is wave-uniform
    for (int i0 = uni(wave) * 64; i0 < K2; i0 += 4 * kThreads) {
      u32x4 v[4];
      uint32_t gv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gv[u] = 0x3f803f80u;  // bf16 ones
        if (i0 + u * kThreads < K2) {
          const int i = i0 + u * kThreads + lane;
          v[u] = __builtin_bit_cast(u32x4, lda4(r, (uint32_t)(((size_t)b * K2 + i) * 16)));
          if (gain) gv[u] = ldg(g1 + i);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u * kThreads < K2) {
          const int i = i0 + u * kThreads + lane;
          if (v[u].y != ca.tag || v[u].w != ca.tag)
            v[u] = wait_pairs(sm, d, ca, t, r, (uint32_t)(((size_t)b * K2 + i) * 16), v[u]);
          const float x0 = __uint_as_float(v[u].x), x1 = __uint_as_float(v[u].z);
          ss = fmaf(x0, x0, ss);
          ss = fmaf(x1, x1, ss);
          d2[i] = make_float2(x0 * bf_lo(gv[u]), x1 * bf_hi(gv[u]));
        }
      }
    }
    if (gain) {
      ss = wave_sum(ss);
      if (lane == 0) sm.misc[b * kWaves + wave] = ss;
    }
  }
  __syncthreads();
  if (sm.imisc[2] == (int)ca.tag) return false;
  if (gain) {
    for (int b = 0; b < nb; ++b) {
      float tot = 0.f;
      for (int w = 0; w < kWaves; ++w) tot += sm.misc[b * kWaves + w];
      const float rs = 1.0f / sqrtf(tot / (float)K + d.eps);
      f32x4 *xb = (f32x4 *)(sm.xs + (size_t)b * K);
      for (int i = tid; i < K / 4; i += kThreads) xb[i] = xb[i] * rs;
    }
    __syncthreads();
  }
  ws.x_src = src;
  ws.x_gain = gain;
  ws.x_K = K;
  ws.x_nb = nb;
  return true;
}

// single-segment-input GEMV tasks (the expert down projection has its own code)
DEV bool is_gemv(int op) {
  return op == OP_QKV || op == OP_OPROJ || op == OP_GATEUP || op == OP_DOWN ||
         op == OP_ROUTER || op == OP_LMHEAD || op == OP_EGATEUP;
}
// weights known before the task's inputs are (prefetchable)
DEV bool static_weights(int op) { return is_gemv(op) && op != OP_EGATEUP; }
// Passes of a static-weight task: rows [p*rpp, min((p+1)*rpp, a2)) of each
// segment.
DEV int task_rpp(int rpp, int rows) { return rpp > 0 && rpp < rows ? rpp : rows; }
DEV int n_passes(const TD &t) {
  const int r = task_rpp(t.rpp, t.a2);
  return (t.a2 + r - 1) / r;
}
DEV Geo pass_geo(const uint16_t *w0, const uint16_t *w1, int rows, int rpp, int K, int p) {
  const int r = task_rpp(rpp, rows);
  const size_t off = (size_t)p * r * K;
  return make_geo(w0 + off, w1 ? w1 + off : nullptr, min(r, rows - p * r), w1 ? 2 : 1, K);
}
DEV Geo static_geo(const TD &t) { return pass_geo(t.w0, t.w1, t.a2, t.rpp, t.K, 0); }

// ---- MoE routing -----------------------------------------------------------
// Order-preserving map of a float to a u32 key (a larger float has a larger
// key); NaN maps to 0, below every number.
DEV uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return f != f ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
}
DEV float unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// maximum / minimum of a u32 over the wave by DPP steps (rows, then across
// rows by row broadcasts), returned uniform
template <bool MAX> DEV uint32_t wave_ext_u32(uint32_t v) {
  auto f = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  v = f(v, (uint32_t)dppi<DPP_XOR1>((int)v));
  v = f(v, (uint32_t)dppi<DPP_XOR2>((int)v));
  v = f(v, (uint32_t)dppi<DPP_HALF_MIRROR>((int)v));
  v = f(v, (uint32_t)dppi<DPP_MIRROR>((int)v));
  // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = f(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of the router logits of (layer, slot) in one wave.  The k largest
// logits win (equal logits: the lower expert id; NaN only once no number is
// left); the chosen experts are put in ascending id order and lane j < k ends
// with the j-th one's id and its weight, the softmax over the k chosen
// logits.  Each lane keeps the best of its own untaken logits; a round takes
// the wave's best key, then the lowest id holding it, and only the lane that
// owned it rescans.  The logits are a tagged vector: the loads wait for
// this step's tag (a failure leaves sm.imisc[2] = tag for the caller).
DEV void route_wave(Smem &sm, CP &d, const CallArgs &ca, const TD &t, int &sid, float &sw) {
  const int lane = tidx() & 63, E = d.E, K = d.topk;
  const size_t r0 = ((size_t)t.layer * d.B + t.a0) * E;
  constexpr int kPer = 8;  // logits per lane: E <= 512
  uint32_t key[kPer];
  uint64_t raw[kPer];  // every logit load issued before any is waited for
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    raw[i] = 0u;
    if (i * 64 < E && i * 64 + lane < E) raw[i] = ldt_raw(d.rl, r0 + i * 64 + lane);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    key[i] = 0u;
    if (i * 64 < E && i * 64 + lane < E)
      key[i] = fkey(ldt_then(sm, d, ca, t, d.rl, r0 + i * 64 + lane, raw[i]));
  }
  uint32_t taken = 0;
  auto scan = [&](uint32_t &bk, uint32_t &bi) {  // best untaken (key, id) of this lane
    bk = 0u;
    bi = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (i * 64 >= E) break;
      const uint32_t e = (uint32_t)(i * 64 + lane);
      const bool ok = e < (uint32_t)E && !((taken >> i) & 1u) && (key[i] > bk || (key[i] == bk && e < bi));
      bk = ok ? key[i] : bk;
      bi = ok ? e : bi;
    }
  };
  uint32_t lk, li;
  scan(lk, li);
  int my_id = lane;
  uint32_t my_key = 0u;
  for (int j = 0; j < K; ++j) {
    const uint32_t kmax = wave_ext_u32<true>(lk);
    const uint32_t win = wave_ext_u32<false>(lk == kmax ? li : 0xffffffffu);
    if (lane == j) { my_id = (int)win; my_key = kmax; }
    if ((int)(win & 63u) == lane && win < (uint32_t)E) {
      taken |= 1u << (win >> 6);
      scan(lk, li);
    }
  }
  // ascending id order: each chosen lane's rank, then a push to that lane
  // (lanes >= k push to themselves)
  int rank = lane;
  if (lane < K) {
    rank = 0;
    for (int k2 = 0; k2 < K; ++k2) rank += __builtin_amdgcn_readlane(my_id, k2) < my_id ? 1 : 0;
  }
  const uint32_t okey = (uint32_t)__builtin_amdgcn_ds_permute(rank * 4, (int)my_key);
  const int oid = __builtin_amdgcn_ds_permute(rank * 4, my_id);
  const float slg = lane < K ? unkey(okey) : -INFINITY;
  const float mx = wave_max(slg);
  const float ex = lane < K ? expf(slg - mx) : 0.f;
  sw = ex / wave_sum(ex);
  sid = lane < K && oid >= 0 && oid < E ? oid : 0;
}

// Expert e of layer l of expert tensor m (0 gate, 1 up, 2 down); base0 is
// the layer's expert 0.  Uniform e (scalar table read) / per-lane e.
DEV const uint16_t *const *expert_tab(CP &d, int m) {
  return m == 0 ? d.e_gate : (m == 1 ? d.e_up : d.e_down);
}
DEV const uint16_t *expert_w_uni(CP &d, int m, int l, int e, const uint16_t *base0) {
  if (d.e_stride) return base0 + (size_t)e * (size_t)d.e_stride;
  return tab(expert_tab(d, m), (size_t)l * d.E + e);
}
DEV const uint16_t *expert_w_lane(CP &d, int m, int l, int e, const uint16_t *base0) {
  if (d.e_stride) return base0 + (size_t)e * (size_t)d.e_stride;
  return ldg((const uint16_t *const *)expert_tab(d, m) + (size_t)l * d.E + e);
}

// Control wave: write the outputs of rows [0, rows) for slots b0..b0+n-1.
DEV void gemv_epilogue(CP &d, const CallArgs &ca, const TD &t, const float *rsum, int bfirst,
                       int b0, int n, float aux0, int rpp) {
  const int lane = tidx() & 63;
  const int op = t.op, rows = t.a2;
  // output row i of slot bi: pass p = i / rpp, row r of the pass; the pass's
  // row sums (segment 0 rows, then segment 1) are at rsum[(p*n + bi)*kRowSlot]
  auto at = [&](int bi, int i, int seg) {
    const int p = i / rpp, r = i - p * rpp;
    const int rp = min(rpp, rows - p * rpp);
    return rsum[(p * n + bi) * kRowSlot + seg * rp + r];
  };
  if (op == OP_LMHEAD) {
    for (int bi = 0; bi < n; ++bi) {
      const int b = bfirst + b0 + bi;
      float bv = -INFINITY;
      int bix = 0x7fffffff;
      for (int i = lane; i < rows; i += 64) {
        const float y = at(bi, i, 0);
        if (ca.logits) stg(ca.logits + (size_t)b * d.V + t.a1 + i, y);
        if (better(y, t.a1 + i, bv, bix)) { bv = y; bix = t.a1 + i; }
      }
      wave_argmax(bv, bix);
      if (lane == 0) {
        const size_t o = (size_t)b * d.n_lm_tiles + t.a4;
        sta(d.amax_v + o, bv);
        stai(d.amax_i + o, bix);
      }
    }
    return;
  }
  const size_t os = (size_t)t.ostride;
  for (int idx = lane; idx < n * rows; idx += 64) {
    const int bi = idx / rows, i = idx - bi * rows;
    const float y = at(bi, i, 0);
    const size_t e = (size_t)(b0 + bi) * os + i;  // output element (slot b0+bi, row i)
    switch (op) {
      case OP_OPROJ: case OP_DOWN:  // residual add (first outputs: preloaded); tagged
        stv(d, t.dst, e, (idx < 64 ? aux0 : ldv(t.aux, e)) + y, ca.tag);
        break;
      case OP_GATEUP:  // SwiGLU of the gate and up rows; tagged
        stv(d, t.dst, e, silu(y) * at(bi, i, 1), ca.tag);
        break;
      case OP_EGATEUP:
        sta(t.dst + e, silu(y) * at(bi, i, 1));
        break;
      case OP_QKV:  // tagged
        stt(t.dst, e, y, ca.tag);
        break;
      default:  // ROUTER; tagged
        stt(t.dst, e, y, ca.tag);
        break;
    }
  }
}

// ---- GEMV tasks, split by wave role ------------------------------------
// Wave 0 (gemv_ctl) and waves 1-7 (gemv_cmp) run separate code for a GEMV
// task and meet at the same barriers; both take every decision from the same
// uniform data.  Keeping the two apart keeps the compute waves' code close to
// a plain streaming loop, so the compiler holds each tile slot in one
// register and waits for each slot's own load only.
struct GemvShape2 {
  Geo g;        // the first pass
  const uint16_t *w0, *w1;  // the task's first rows (experts: chosen here)
  int nb, bfirst, P, rpp, bb_max;
  int sid;      // expert tasks: lane j < k holds the j-th routed expert id
  float sw;     //   and its weight
  bool skip;    // expert task of an empty slot: no work
  bool fail;    // the routing's logits never arrived (step abandoned)
};

// B1: compiled for plans with one slot (no slot chunks).
template <bool B1>
DEV GemvShape2 gemv_shape(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws) {
  GemvShape2 q;
  q.skip = false;
  q.fail = false;
  q.sid = 0;
  q.sw = 0.f;
  q.w0 = t.w0;
  q.w1 = t.w1;
  if (t.op == OP_EGATEUP) {
    q.nb = 1;
    q.bfirst = t.a0;
    q.skip = ldg(ca.positions + t.a0) < 0;
    if (!q.skip) {
      // the control wave routes the slot; the ids reach the other waves
      // through LDS (sm.imisc[48..] ids, sm.misc[48..] weights)
      if (ws.rt_layer != t.layer || ws.rt_slot != t.a0) {
        if (uni(tidx() >> 6) == 0) {
          route_wave(sm, d, ca, t, q.sid, q.sw);
          if ((tidx() & 63) < d.topk) {
            sm.imisc[48 + (tidx() & 63)] = q.sid;
            sm.misc[48 + (tidx() & 63)] = q.sw;
          }
        }
        __syncthreads();
        q.fail = sm.imisc[2] == (int)ca.tag;
        ws.rt_layer = t.layer;
        ws.rt_slot = t.a0;
      }
      if ((tidx() & 63) < d.topk) {
        q.sid = sm.imisc[48 + (tidx() & 63)];
        q.sw = sm.misc[48 + (tidx() & 63)];
      }
      const int e = sm.imisc[48 + t.a3];
      q.w0 = expert_w_uni(d, 0, t.layer, e, t.w0) + (size_t)t.a1 * t.K;
      q.w1 = expert_w_uni(d, 1, t.layer, e, t.w1) + (size_t)t.a1 * t.K;
    }
  } else {
    q.nb = B1 ? 1 : d.B;
    q.bfirst = 0;
  }
  q.g = pass_geo(q.w0, q.w1, t.a2, t.rpp, t.K, 0);
  q.P = n_passes(t);
  q.rpp = task_rpp(t.rpp, t.a2);
  q.bb_max = B1 ? 1 : min(kMaxBatchGemv, kLdsXBytes / (q.g.K * 4));
  return q;
}
// An expert gate/up task stages its slot's activation row (ready since the
// output projection) before it routes the slot: the router logits come
// later, and the staging round trip then overlaps that wait instead of
// following the routing.  All waves; the staging call after the routing
// finds the row in place.  False when the step is abandoned.
DEV bool prestage(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws) {
  if (t.op != OP_EGATEUP || ldg(ca.positions + t.a0) < 0) return true;
  return stage_xt(sm, d, ca, t, ws, t.src, t.K, 1, t.gain);
}

// the planner never emits more passes x slots than the partial buffers hold
DEV bool gemv_fits(CP &d, const TD &t, const GemvShape2 &q) {
  if (q.P > 1 && q.P * min(q.nb, q.bb_max) > kMaxPass) {
    if (tidx() == 0) set_error(d, DEVERR_BAD_INPUT, t.gidx, -1, (uint32_t)q.P, (uint32_t)q.nb);
    return false;
  }
  return true;
}

// Control wave: dependencies, activation staging (shared), the residual
// preload, the outputs, the completion signal.
template <bool B1>
DEV bool gemv_ctl(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws) {
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  if (!prestage(sm, d, ca, t, ws)) return false;
  const GemvShape2 q = gemv_shape<B1>(sm, d, ca, t, ws);
  if (q.fail) return false;
  if (q.skip) {
    if (persistent) {
      trace_start(d, t);
      trace_finish(d, t);
      signal_done(d, t);
    }
    return true;
  }
  if (!gemv_fits(d, t, q)) return false;
  const int K = q.g.K, lane = tidx() & 63;
  for (int b0 = 0; b0 < q.nb; b0 += q.bb_max) {
    const int n = min(q.bb_max, q.nb - b0);
    if (n < q.nb) ws.x_src = nullptr;  // chunked batch: no reuse
    if (!stage_xt(sm, d, ca, t, ws, t.src + 2 * (size_t)b0 * K, K, n, t.gain)) return false;
    if (b0 == 0) trace_start(d, t);  // inputs complete
    trace_mark(d, t, 0);
    // the residual of the first outputs, loaded while the compute waves work
    float aux0 = 0.f;
    if ((t.op == OP_OPROJ || t.op == OP_DOWN) && lane < n * t.a2) {
      const int bi = lane / t.a2, i = lane - bi * t.a2;
      aux0 = ldv(t.aux, (size_t)(b0 + bi) * t.ostride + i);
    }
    __syncthreads();  // partials complete
    __syncthreads();  // row sums complete
    trace_mark(d, t, 1);
    if (persistent && b0 == 0) trace_finish(d, t);  // before the outputs: consumers start after
    gemv_epilogue(d, ca, t, &sm.rows[0][0], q.bfirst, b0, n, aux0, q.rpp);
    if (n < q.nb) {
      ws.x_src = nullptr;
      __syncthreads();  // the next slot chunk restages xs and reuses the buffers
    }
  }
  // the slot's routing, for the down projection and for read-back
  if (t.op == OP_EGATEUP && t.a1 == 0 && t.a3 == 0 && lane < d.topk) {
    const size_t o = ((size_t)t.layer * d.B + t.a0) * d.topk + lane;
    stai(d.tk_ids + o, q.sid);
    sta(d.tk_w + o, q.sw);
  }
  if (persistent) {
    // The epilogue's stores are all this wave's: drain them only where the
    // run's completions are reported to a counter (the wait covers the
    // earlier tasks too); tagged outputs need neither.
    if (t.a5 > 0 && signals_counter(t)) vm_drain();
    signal_done(d, t);
  }
  return true;
}

// Compute waves: stream the task's passes through `w` (holding the first
// pass when w_loaded), reloading each slot right after its use with the next
// pass; then the row sums.  When `pre`, the first pass of the next task `gn`
// follows: interleaved with the last pass when `inter` (the next task waits
// only for this task's operation), else, in single-slot plans, issued once
// the row sums are written, so that this task's outputs, and the chain of
// operations behind them that the next task waits for, are not held behind
// its loads.
template <bool B1>
DEV bool gemv_cmp(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws, Buf &w, bool w_loaded, bool pre, const Geo &gn, bool inter) {
  const int cw = uni(tidx() >> 6) - 1;
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  if (!prestage(sm, d, ca, t, ws)) return false;
  const GemvShape2 q = gemv_shape<B1>(sm, d, ca, t, ws);
  if (q.fail) return false;
  if (q.skip) return true;
  const bool lds = d.lds_slots != 0;  // (single-slot plans only)
  if (!w_loaded) load_slots(q.g, w, cw, sm.xs, lds);
  if (!gemv_fits(d, t, q)) return false;
  const int K = q.g.K;
  auto geo_of = [&](int p) { return p == 0 ? q.g : pass_geo(q.w0, q.w1, t.a2, t.rpp, K, p); };
  float *red = &sm.red[0][0];
  float *rsum = &sm.rows[0][0];
  for (int b0 = 0; b0 < q.nb; b0 += q.bb_max) {
    const int n = min(q.bb_max, q.nb - b0);
    const bool last = b0 + n >= q.nb;
    if (n < q.nb) ws.x_src = nullptr;
    if (!stage_xt(sm, d, ca, t, ws, t.src + 2 * (size_t)b0 * K, K, n, t.gain)) return false;
    // The first pass was loaded before the task; waiting for all of it here
    // lets the pass loop wait per slot for the loads it issues itself.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    // every pass reloads its slots with the next pass; the last one with the
    // next task only when interleaved, else with the idle line (a slot chunk
    // before the last keeps its single pass for the next chunk)
    const bool defer = B1 && !inter;  // (multi-slot tiles measured better without)
    const bool tail = pre && last && !defer;
    Geo idle = gn;
    idle.units = 0;
    idle.cpw = 0;
    for (int p = 0; p < q.P; ++p) {
      const bool lastp = p + 1 == q.P;
      const Geo gq = !lastp ? geo_of(p + 1) : tail ? gn : idle;
      if (B1 || n == 1) {
        gemv_dot1(geo_of(p), w, sm.xs, red + p * kPartSlot, cw, gq, lds);
      } else {
        gemv_dotn(geo_of(p), w, sm.xs, n, red + p * n * kPartSlot, cw);
        if (!lastp || tail) load_slots(gq, w, cw, sm.xs, false);
      }
    }
    __syncthreads();  // partials complete
    gemv_rows(K, q.P, [&](int p) { return geo_of(p).units * 512 / K; }, red, rsum, n, cw);
    __syncthreads();  // row sums complete
    if (pre && last && defer) load_slots(gn, w, cw, sm.xs, lds);  // (outputs being written)
    if (n < q.nb) {
      ws.x_src = nullptr;
      __syncthreads();
    }
  }
  return true;
}

// ---- MoE down projection + combine ------------------------------------------
// Output rows [a1, a1+a2) of slot a0 over all k routed experts.  The tile is
// k segments, segment j being rows [a1, a1+a2) of the j-th routed expert's
// down matrix (ascending expert id), each a whole number of 1 KiB chunks, so
// every chunk lies in one segment; segment j multiplies that expert's h,
// staged in LDS at j*Fe.  Row sums of segment j land at rows[j*a2 + r]; the
// control wave writes x_mid + sum_j w_j y_j (ascending expert order).
struct DownShape {
  int units, cpw, cps;  // 1 KiB chunks of the tile, per compute wave, per segment
  bool skip;            // empty slot
};
DEV DownShape down_shape(CP &d, const CallArgs &ca, const TD &t) {
  DownShape s;
  s.skip = ldg(ca.positions + t.a0) < 0;
  s.cps = (t.a2 * t.K * 2) >> 10;
  s.units = s.cps * d.topk;
  s.cpw = (s.units + kCW - 1) / kCW;
  return s;
}
// A down task waits in two stages: for the router logits (its first
// waits), from which it routes the slot itself -- the same top-k as the
// slot's gate/up tasks -- and issues its experts' weight loads; then for the
// experts' activations (its last wait), which the weights no longer have to
// wait behind.  The control wave routes; lane j < k of every wave gets the
// j-th expert id and weight through LDS.
DEV bool down_route(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                    WState &ws, int &id, float &w) {
  if (persistent && !wait_deps(sm, d, ca, t, ws, 0, t.n_wait - 1)) return false;
  const int lane = tidx() & 63;
  if (ws.rt_layer != t.layer || ws.rt_slot != t.a0) {  // not routed by this worker yet
    if (uni(tidx() >> 6) == 0) {
      int sid;
      float sw;
      route_wave(sm, d, ca, t, sid, sw);
      if (lane < d.topk) {
        sm.imisc[48 + lane] = sid;
        sm.misc[48 + lane] = sw;
      }
    }
    __syncthreads();
    if (sm.imisc[2] == (int)ca.tag) return false;  // the logits never arrived
    ws.rt_layer = t.layer;
    ws.rt_slot = t.a0;
  }
  id = lane < d.topk ? sm.imisc[48 + lane] : 0;
  w = lane < d.topk ? sm.misc[48 + lane] : 0.f;
  return true;
}

DEV bool down_ctl(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws) {
  const DownShape s = down_shape(d, ca, t);
  const int lane = tidx() & 63;
  if (s.skip) {
    if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
    trace_start(d, t);
    if (persistent) trace_finish(d, t);
    for (int i = lane; i < t.a2; i += 64) stv(d, t.dst, i, 0.f, ca.tag);
  } else {
    int id;
    float w;
    if (!down_route(sm, d, ca, t, persistent, ws, id, w)) return false;
    // (the compute waves issue the experts' weight loads here)
    if (persistent && !wait_deps(sm, d, ca, t, ws, t.n_wait - 1, t.n_wait)) return false;
    trace_start(d, t);
    stage_x(sm, ws, t.src, t.K, d.topk, nullptr, d.eps);
    trace_mark(d, t, 0);
    const float aux0 = lane < t.a2 ? ldv(t.aux, lane) : 0.f;
    __syncthreads();  // partials complete
    __syncthreads();  // row sums complete
    trace_mark(d, t, 1);
    if (persistent) trace_finish(d, t);  // before the outputs: consumers start after
    const float *rsum = &sm.rows[0][0];
    for (int i = lane; i < t.a2; i += 64) {
      float acc = 0.f;
      for (int j = 0; j < d.topk; ++j) acc = fmaf(lanef(w, j), rsum[j * t.a2 + i], acc);
      stv(d, t.dst, i, (i < 64 ? aux0 : ldv(t.aux, i)) + acc, ca.tag);
    }
  }
  if (persistent) {
    if (t.a5 > 0 && signals_counter(t)) vm_drain();
    signal_done(d, t);
  }
  return true;
}

DEV bool down_cmp(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws) {
  const int cw = uni(tidx() >> 6) - 1, lane = tidx() & 63;
  const DownShape s = down_shape(d, ca, t);
  if (s.skip) return !persistent || wait_deps(sm, d, ca, t, ws);
  int id;
  float wt;
  if (!down_route(sm, d, ca, t, persistent, ws, id, wt)) return false;
  // lane j: the first row of segment j
  const uint64_t base = (uint64_t)(expert_w_lane(d, 2, t.layer, id, t.w0) + (size_t)t.a1 * t.K);
  const int blo = (int)(uint32_t)base, bhi = (int)(uint32_t)(base >> 32);
  const int q0 = cw * s.cpw;
  const int cnt = min(s.cpw, s.units - q0);
  const uint32_t lane16 = (uint32_t)lane * 16u;
  Buf w;
  int sg = q0 / s.cps, rr = q0 - sg * s.cps;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int sj = j < cnt ? sg : 0, rj = j < cnt ? rr : 0;
    const uint64_t b = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(bhi, sj) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane(blo, sj);
    w[j] = ldnt((const u32x4 *)(b + (uint64_t)rj * 1024u + lane16));
    if (j < cnt && ++rr == s.cps) { rr = 0; ++sg; }
  }
  if (persistent && !wait_deps(sm, d, ca, t, ws, t.n_wait - 1, t.n_wait)) return false;
  stage_x(sm, ws, t.src, t.K, d.topk, nullptr, d.eps);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  const int Fe = t.K, step = 512 % Fe;
  float *red = &sm.red[0][0];
  int col = (int)(((uint32_t)q0 * 512u + (uint32_t)lane * 8u) % (uint32_t)Fe);
  sg = q0 / s.cps;
  rr = q0 - sg * s.cps;
  float *pp = red + q0 * 4 + (lane >> 4);
  const bool writer = (lane & 15) == 0;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    if (j < cnt) {
      const float v = row16_sum(dot8(w[j], sm.xs + sg * Fe + col));
      if (writer) pp[j * 4] = v;
      col += step;
      col = col >= Fe ? col - Fe : col;
      if (++rr == s.cps) { rr = 0; ++sg; }
    }
  }
  __syncthreads();  // partials complete
  const int R = d.topk * t.a2;
  gemv_rows(Fe, 1, [&](int) { return R; }, red, &sm.rows[0][0], 1, cw);
  __syncthreads();  // row sums complete
  return true;
}

// ------------------------------------------------- batched GEMV, matrix cores --
// For 16..64 slots the static-weight GEMVs run on v_mfma_f32_16x16x32_bf16.
// A task covers NGs 16-row groups of each of its nseg matrices (gate and up
// share a task) and all K.  Compute wave cw owns row slot cw of each matrix
// (and slot cw + 7 of a single matrix with more than 7 groups) and streams
// its groups along K in slices of Ks columns, one slice per pass.  A 1 KiB
// chunk is 16 rows x 32 columns, loaded as one 16-byte load per lane in the
// instruction's A layout (lane l: row l%16, columns 8(l/16)..+8), so loads
// feed the matrix cores without reshuffling.  The control wave stages each
// slice of activations (all slots) into LDS in the B layout (lane l: slot
// l%16 of a 16-slot tile, the same 8 columns), split into a bf16 value and
// a bf16 remainder: two products per tile keep about 16 bits of the fp32
// activation.  It copies the slice from the plan's values-only copy of the
// input with LDS-DMA (no registers, so a whole slice is in flight at once)
// and converts it in place.  Slices are double-buffered, one barrier per
// pass, each slice's copy issued a pass ahead.  With a gain the staged
// values are x*g and the outputs are scaled by 1/rms of their slot at the
// end; the sums of squares are accumulated while converting.
// The accumulators (16 rows x 16 slots per tile) go to LDS after the last
// pass and the control wave writes the outputs.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// A matrix-core tile: NGs 16-row groups per matrix (nseg matrices) times K
// columns starting at column k0 of rows ld elements long (split-K tiles
// cover part of the row; s0/s1 point at column k0 of the first row).
struct MGeo {
  const uint16_t *s0, *s1;
  int K, NGs, nseg, Ks, nkb, P, B16, ld, k0;
};
DEV MGeo mgeo(const uint16_t *w0, const uint16_t *w1, int rows, int K, int B, int ld, int k0) {
  MGeo g;
  g.s0 = w0 + k0;
  g.s1 = w1 ? w1 + k0 : nullptr;
  g.K = K;
  g.ld = ld;
  g.k0 = k0;
  g.NGs = rows >> 4;
  g.nseg = w1 ? 2 : 1;
  g.B16 = (B + 15) >> 4;
  const int maxg = (g.nseg == 2 || g.NGs > kCW) ? 2 : 1;
  int ks = (kMaxChunks / maxg) * 32;                       // register slots
  ks = min(ks, kLdsXBytes / (2 * g.B16 * 16 * 4));         // two slices of hi+lo bf16
  ks = ks / 64 * 64;                                       // whole 64-column pairs
  ks = min(ks, K);
  g.Ks = ks;
  g.nkb = ks >> 5;
  g.P = (K + ks - 1) / ks;
  return g;
}
// Split-K tiles carry rpp = kc | rb << 16 with kc < K; whole-row tiles rpp = K.
DEV int ksplit_kc(int rpp, int K) { return min(rpp & 0xffff, K); }
DEV MGeo mgeo_of(CP &d, const TD &t) {
  const int kc = ksplit_kc(t.rpp, t.K);
  return mgeo(t.w0, t.w1, t.a2, min(kc, t.K - t.a3), d.B, t.K, t.a3);
}

// matrix and row slot of wave cw's gi-th group; false when it has none
DEV bool mgroup(const MGeo &g, int cw, int gi, int &seg, int &slot) {
  if (g.nseg == 2) {
    seg = gi;
    slot = cw;
    return cw < g.NGs;
  }
  seg = 0;
  slot = cw + gi * kCW;
  return slot < g.NGs;
}

// Address of lane's 16 bytes of register slot j (group j / NKB, k-block
// j % NKB) of wave cw in pass p; slots without a chunk read the idle line.
// Slots are loaded in pairs (k-blocks 2i, 2i+1: 64 columns, one 128-byte
// line of each of the group's 16 rows), so every load covers 8 whole lines:
// the even slot P takes rows 0-7, the odd one Q rows 8-15.  Lane l = 16q + r
// of slot h loads row 8h + r%8, columns 8q..+8 of k-block 0 of the pair
// when r/8 == h (exactly its own A operand of that k-block), else of
// k-block 1 (the A operand lane l^8 needs for k-block 1).  mpair then
// builds both A operands with a select and a rotate within 16 lanes.
// Lanes whose columns lie beyond the tile read the idle line (tiles are
// whole pairs wide; this only guards memory).
template <int NKB>
DEV uint64_t maddr(const MGeo &g, int cw, int j, int p) {
  const int lane = tidx() & 63, r = lane & 15, q = lane >> 4;
  const int gi = j / NKB, kb = j % NKB, h = kb & 1;
  int seg = 0, slot = 0;
  const int k2 = p * g.Ks + (kb & ~1) * 32;  // the pair's first column
  const int col = k2 + 8 * (q + 4 * ((r >> 3) ^ h));
  const bool ok = gi < 2 && mgroup(g, cw, gi, seg, slot) && (kb & ~1) < g.nkb && col < g.K;
  const uint16_t *base = seg ? g.s1 : g.s0;
  const int row = slot * 16 + (r & 7) + 8 * h;
  const uint64_t a = (uint64_t)(base + (size_t)row * g.ld + col);
  return ok ? a : idle_addr();
}
// A loaded pair into the A operands of its two k-blocks, in place: lanes
// r < 8 hold their k-block-0 operand in P, lanes r >= 8 in Q; the
// k-block-1 operand of lane l sits in lane l^8 (of Q for r < 8, of P for
// r >= 8): a select, then a rotate by 8 within each row of 16 lanes.
DEV void mpair(u32x4 &P, u32x4 &Q) {
  const bool lo = (tidx() & 15) < 8;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = (int)P[e], qq = (int)Q[e];
    P[e] = (uint32_t)(lo ? p : qq);
    Q[e] = (uint32_t)dppi<DPP_ROR8>(lo ? qq : p);
  }
}
DEV uint64_t maddr_any(const MGeo &g, int cw, int j, int p) {
  return g.nkb >= 16 ? maddr<16>(g, cw, j, p) : maddr<8>(g, cw, j, p);
}
DEV void mload(const MGeo &g, Buf &w, int cw) {
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) w[j] = ldnt((const u32x4 *)maddr_any(g, cw, j, 0));
}

// One pass of wave cw: the products of its chunks with the staged slice
// `xb`; each register slot is refilled right after use with the same chunk
// of the next pass, or (after the last pass) of the next task's first pass.
template <int NKB, int B16>
DEV void mpass(const MGeo &g, Buf &w, f32x4 (&acc)[2][4], const char *xb, int cw, int p,
               bool pre, const MGeo &gn) {
  const int lane = tidx() & 63;
  const bool last = p + 1 == g.P;
#pragma unroll
  for (int j = 0; j < kMaxChunks; j += 2) {  // slot pairs: k-blocks kb, kb + 1
    const int gi = j / NKB, kb = j % NKB;
    int seg, slot;
    const bool has = gi < 2 && mgroup(g, cw, gi, seg, slot) && kb < g.nkb;
    const bool ok0 = has && p * g.Ks + kb * 32 < g.K;
    const bool ok1 = has && p * g.Ks + (kb + 1) * 32 < g.K;
    if (ok0) {
      mpair(w[j], w[j + 1]);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m == 1 && !ok1) break;
        const bf16x8 a = __builtin_bit_cast(bf16x8, w[j + m]);
        // value parts of every slot tile, then the remainders: consecutive
        // products accumulate into different tiles
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 xv[4];
#pragma unroll
          for (int st = 0; st < 4; ++st)
            if (st < B16)
              xv[st] = *(const bf16x8 *)(xb + ((kb + m) * B16 + st) * 2048 + half * 1024 + lane * 16);
#pragma unroll
          for (int st = 0; st < 4; ++st)
            if (st < B16)
              acc[gi][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xv[st], acc[gi][st], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint64_t na = !last ? maddr<NKB>(g, cw, j + m, p + 1)
                                : (pre ? maddr_any(gn, cw, j + m, 0) : idle_addr());
      w[j + m] = ldnt((const u32x4 *)na);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Staging of slice p of the activations (all slots) into LDS buffer pb.  A
// unit is one 16-slot tile (st) of one 32-column k-block (kb) in 2 KiB.  The
// copy puts the fp32 values there, lane l's 32 bytes at l*32: slot
// st*16 + l%16, columns 8(l/16)..+8 of the k-block; the conversion rewrites
// the unit as 64 x 16 bytes of bf16 values of x*gain (lane l at l*16, the B
// layout) followed by 64 x 16 bytes of their bf16 remainders.
DEV int mx_units(const MGeo &g, int p) { return (min(g.Ks, g.K - p * g.Ks) >> 5) * g.B16; }
DEV uint32_t mx_buf(const Smem &sm, const MGeo &g, int pb) {
  return (uint32_t)(uintptr_t)sm.xs + (uint32_t)(pb * (g.nkb * g.B16 * 2048));
}
// Control wave: the LDS-DMA copies of slice p, two 16-byte copies per lane
// and unit (copy i, lane j: bytes 16j.. of the unit's half i, i.e. half j%2
// of value lane 32i + j/2).  Lanes of slots beyond the batch copy nothing;
// the conversion zeroes those slots.  Nothing waits here: mx_convert does.
DEV void mx_dma(Smem &sm, CP &d, const MGeo &g, const TD &t, int p, int pb) {
  const int lane = tidx() & 63, B16 = g.B16;
  const int nu = mx_units(g, p);
  const float *src = shadow_of(d, t.src);
  const uint32_t xb = mx_buf(sm, g, pb);
  for (int u = 0; u < nu; ++u) {
    const int kb = u / B16, st = u - kb * B16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int L = 32 * i + (lane >> 1);
      const int b = st * 16 + (L & 15);
      const int col = g.k0 + p * g.Ks + kb * 32 + 8 * (L >> 4) + 4 * (lane & 1);
      if (b < d.B) {
        const uint64_t a = (uint64_t)(src + (size_t)b * g.ld + col);
        const uint32_t l = xb + (uint32_t)(u * 2048 + i * 1024);
        if (d.mx_sc1) dma16_sc1(a, l); else dma16(a, l);
      }
    }
  }
}
// One unit in place: lane's 32 bytes of fp32 values (zero for a slot
// beyond the batch when `live` is false), times the gains gv (8 bf16), into
// the unit's bf16 values and remainders; their sum of squares to ss.
template <bool GAIN, bool RAGGED>
DEV void mx_unit(char *ub, u32x4 gv, bool live, float &ss) {
  const int lane = tidx() & 63;
  const f32x4 a0 = *(const f32x4 *)(ub + lane * 32);
  const f32x4 a1 = *(const f32x4 *)(ub + lane * 32 + 16);
  f32x8 x = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  if (RAGGED) x = live ? x : (f32x8){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  f32x8 v = x;
  if (GAIN) {
    const f32x8 gf = {bf_lo(gv.x), bf_hi(gv.x), bf_lo(gv.y), bf_hi(gv.y),
                      bf_lo(gv.z), bf_hi(gv.z), bf_lo(gv.w), bf_hi(gv.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    v = x * gf;
  }
  // the bf16 values, widened back from their packed bits (low half of each
  // word: even element), and the bf16 remainders
  const bf16x8 h = __builtin_convertvector(v, bf16x8);
  const u32x4 hb = __builtin_bit_cast(u32x4, h);
  const f32x8 hf = {__uint_as_float(hb.x << 16), __uint_as_float(hb.x & 0xffff0000u),
                    __uint_as_float(hb.y << 16), __uint_as_float(hb.y & 0xffff0000u),
                    __uint_as_float(hb.z << 16), __uint_as_float(hb.z & 0xffff0000u),
                    __uint_as_float(hb.w << 16), __uint_as_float(hb.w & 0xffff0000u)};
  const bf16x8 lo = __builtin_convertvector(v - hf, bf16x8);
  *(bf16x8 *)(ub + lane * 16) = h;
  *(bf16x8 *)(ub + 1024 + lane * 16) = lo;
}
// Control wave, slices after the first: wait for this wave's copies (all of
// them: the next slice's are issued after this), then convert slice p in
// place, unit by unit: each lane reads its 32 bytes, and only then (the same
// wave, in order) writes its 16 + 16 bytes of the unit.  The gains of eight
// k-blocks are loaded together, ahead of the wait.
template <bool GAIN, bool RAGGED>
DEV void mx_convert_t(Smem &sm, CP &d, const MGeo &g, const TD &t, int p, int pb,
                      float (&ssl)[4]) {
  const int lane = tidx() & 63, B16 = g.B16;
  const int nkb = mx_units(g, p) / B16;
  char *xb = (char *)sm.xs + pb * (g.nkb * B16 * 2048);
  for (int k0 = 0; k0 < nkb; k0 += 8) {
    u32x4 gq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = g.k0 + p * g.Ks + (k0 + j) * 32 + 8 * (lane >> 4);
      gq[j] = (u32x4){0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
      if (GAIN && k0 + j < nkb) gq[j] = ldg((const u32x4 *)(t.gain + col));
    }
    if (k0 == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (k0 + j >= nkb) break;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st >= B16) break;
        mx_unit<GAIN, RAGGED>(xb + ((k0 + j) * B16 + st) * 2048, gq[j],
                              st * 16 + lane % 16 < d.B, ssl[st]);
      }
    }
  }
}
// with or without a gain, with or without slots beyond the batch in a tile
DEV void mx_convert(Smem &sm, CP &d, const MGeo &g, const TD &t, int p, int pb,
                    float (&ssl)[4]) {
  const bool ragged = g.B16 * 16 > d.B;
  if (t.gain) {
    if (ragged) mx_convert_t<true, true>(sm, d, g, t, p, pb, ssl);
    else mx_convert_t<true, false>(sm, d, g, t, p, pb, ssl);
  } else {
    if (ragged) mx_convert_t<false, true>(sm, d, g, t, p, pb, ssl);
    else mx_convert_t<false, false>(sm, d, g, t, p, pb, ssl);
  }
}
// The first slice is converted by every wave (the compute waves have nothing
// else to do before it): the control wave copies it and puts its gains in
// LDS (sm.red, bf16 pairs) before a barrier; then wave w converts units w,
// w+8, ... with gains from LDS, so no wave waits for a vector memory load.
DEV uint32_t *mx_gains(Smem &sm) { return (uint32_t *)&sm.red[0][0]; }
DEV void mx_copy0(Smem &sm, CP &d, const MGeo &g, const TD &t) {
  const int lane = tidx() & 63;
  mx_dma(sm, d, g, t, 0, 0);
  const int n16 = min(g.Ks, g.K) / 8;  // 16-byte chunks of gains (Ks <= 512: one per lane)
  if (t.gain && lane < n16)
    ((u32x4 *)mx_gains(sm))[lane] = ldg((const u32x4 *)(t.gain + g.k0) + lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
template <bool GAIN, bool RAGGED>
DEV void mx_convert0_t(Smem &sm, CP &d, const MGeo &g, float (&ssl)[4]) {
  const int lane = tidx() & 63, wave = uni(tidx() >> 6), B16 = g.B16;
  const int nu = mx_units(g, 0);
  const u32x4 *gl = (const u32x4 *)mx_gains(sm);
  for (int u = wave; u < nu; u += kWaves) {
    const int kb = u / B16, st = u - kb * B16;
    const u32x4 gv = GAIN ? gl[kb * 4 + (lane >> 4)]
                          : (u32x4){0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    float ss = 0.f;
    mx_unit<GAIN, RAGGED>((char *)sm.xs + u * 2048, gv, st * 16 + lane % 16 < d.B, ss);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2)
      if (s2 == st) ssl[s2] += ss;
  }
}
DEV void mx_convert0(Smem &sm, CP &d, const MGeo &g, const TD &t, float (&ssl)[4]) {
  const bool ragged = g.B16 * 16 > d.B;
  if (t.gain) {
    if (ragged) mx_convert0_t<true, true>(sm, d, g, ssl);
    else mx_convert0_t<true, false>(sm, d, g, ssl);
  } else {
    if (ragged) mx_convert0_t<false, true>(sm, d, g, ssl);
    else mx_convert0_t<false, false>(sm, d, g, ssl);
  }
}
// Every wave's sums of squares to LDS (sm.red as [wave][lane][tile]); after
// a barrier, 1/rms of slot b is reduced from the lanes holding its shares.
DEV void mss_publish(Smem &sm, const float (&ssl)[4]) {
  const int lane = tidx() & 63, wave = uni(tidx() >> 6);
  f32x4 *dst = (f32x4 *)&sm.red[0][0];
  dst[wave * 64 + lane] = (f32x4){ssl[0], ssl[1], ssl[2], ssl[3]};
}
DEV void mss_rms(Smem &sm, CP &d, const MGeo &g, float *rs) {
  const int lane = tidx() & 63;
  const f32x4 *src = (const f32x4 *)&sm.red[0][0];
  if (lane < g.B16 * 16) {
    const int st = lane >> 4, l16 = lane & 15;
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w)
      for (int m = 0; m < 4; ++m) s += src[w * 64 + m * 16 + l16][st];
    rs[lane] = 1.0f / sqrtf(s / (float)g.ld + d.eps);
  }
}

// Control wave: outputs of rows r0 .. r0+R of a matrix-core task from
// out[row][slot] (LDS, Bp slots per row; gate/up: the R gate rows, then the
// same up rows), scaled by the slots' 1/rms (rs) when the input was
// normalised.
DEV void mepilogue(CP &d, const CallArgs &ca, const TD &t, int R, int Bp, int r0,
                   const float *out, const float *rs) {
  const int lane = tidx() & 63;
  const int B = d.B, op = t.op;
  const size_t os = (size_t)t.ostride;
  auto y_at = [&](int row, int b) { return out[row * Bp + b] * (t.gain ? rs[b] : 1.f); };
  if (op == OP_LMHEAD) {
    for (int b = 0; b < B; ++b) {
      float bv = -INFINITY;
      int bix = 0x7fffffff;
      for (int i = lane; i < R; i += 64) {
        const float y = y_at(i, b);
        if (ca.logits) stg(ca.logits + (size_t)b * d.V + t.a1 + i, y);
        if (better(y, t.a1 + i, bv, bix)) { bv = y; bix = t.a1 + i; }
      }
      wave_argmax(bv, bix);
      if (lane == 0) {
        const size_t o = (size_t)b * d.n_lm_tiles + t.a4;
        sta(d.amax_v + o, bv);
        stai(d.amax_i + o, bix);
      }
    }
    return;
  }
  // eight outputs per lane in flight: residual loads first, then the stores
  const int n = B * R;
  for (int i0 = 0; i0 < n; i0 += 8 * 64) {
    float a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = i0 + u * 64 + lane;
      a[u] = 0.f;
      if ((op == OP_OPROJ || op == OP_DOWN) && idx < n) {
        const int b = idx / R, i = idx - b * R;
        a[u] = ldv(t.aux, (size_t)b * os + r0 + i);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = i0 + u * 64 + lane;
      if (idx >= n) break;
      const int b = idx / R, i = idx - b * R;
      const float y = y_at(i, b);
      const size_t e = (size_t)b * os + r0 + i;
      if (op == OP_GATEUP)
        stv(d, t.dst, e, silu(y) * y_at(R + i, b), ca.tag);
      else if (op == OP_OPROJ || op == OP_DOWN)
        stv(d, t.dst, e, a[u] + y, ca.tag);
      else
        stt(t.dst, e, y, ca.tag);  // QKV, ROUTER
    }
  }
}

// ---- split-K matrix-core tiles ---------------------------------------------
// The ns tiles of a row block (column ranges ks = 0..ns-1) each publish
// their products [row][slot] and the slots' sums of squares over their
// columns into the partial slot (rb, ks), then count themselves on the
// block's arrival counter.  Once all ns have arrived, tile ks adds up rows
// [ks*Rs, (ks+1)*Rs) of every matrix (Rs = ceil(rows / ns)) over the ns
// slots in split order (deterministic) and writes them as the operation's
// output; every tile reports its completion after its own rows.
struct KSplit {
  int ns, ks, rb, kc;
};
DEV KSplit ksplit_of(const TD &t) {
  KSplit k;
  k.kc = ksplit_kc(t.rpp, t.K);
  k.ns = (t.K + k.kc - 1) / k.kc;
  k.ks = t.a3 / k.kc;
  k.rb = (t.rpp >> 16) & 0x7fff;
  return k;
}
DEV float *kslot(CP &d, const KSplit &k, int ks) {
  return d.kpart + ((size_t)k.rb * k.ns + ks) * (size_t)kpart_slot(d.B);
}
DEV void ksplit_rows(const MGeo &g, const KSplit &k, int &lo, int &nr) {
  const int R = g.NGs * 16, rs = (R + k.ns - 1) / k.ns;
  lo = min(R, k.ks * rs);
  nr = min(R, lo + rs) - lo;
}
// sum of squares of slot `lane` over the tile's columns (lane < 16 * B16)
DEV float mss_sum(Smem &sm, const MGeo &g, int lane) {
  const f32x4 *src = (const f32x4 *)&sm.red[0][0];
  const int st = lane >> 4, l16 = lane & 15;
  float s = 0.f;
  for (int w = 0; w < kWaves; ++w)
    for (int m = 0; m < 4; ++m) s += src[w * 64 + m * 16 + l16][st];
  return s;
}
// Control wave: the tile's products (LDS out[row][slot]) and sums of squares
// to its partial slot, with coherent stores.
DEV void ksplit_publish(Smem &sm, CP &d, const MGeo &g, const KSplit &k) {
  const int lane = tidx() & 63, Bp = g.B16 * 16;
  float *slot = kslot(d, k, k.ks);
  const __amdgpu_buffer_rsrc_t r = rsrc(slot);
  const f32x4 *src = (const f32x4 *)sm.xs;
  const int n4 = g.nseg * g.NGs * 16 * Bp / 4;
  for (int u = lane; u < n4; u += 64)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, src[u]), r, (uint32_t)u * 16u,
                                           0, kCpolSc1);
  if (lane < Bp) sta(slot + (size_t)kMfmaGroups * 16 * Bp + lane, mss_sum(sm, g, lane));
}
// Every wave: count this tile (thread 0, after the control wave drained its
// stores) and wait until the block's ns tiles have arrived.  False when the
// step is abandoned.
DEV bool ksplit_arrive(Smem &sm, CP &d, const CallArgs &ca, const TD &t, const KSplit &k) {
  if (tidx() == 0) {
    uint32_t *c = d.kcnt + (size_t)t.a4 * kCtrStride;
    const uint32_t want = (ca.epoch + 1u) * (uint32_t)k.ns;
    uint32_t seen =
        __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    int ok = 1;
    if ((int32_t)(seen - want) < 0) {
      const uint64_t t0 = wall_clock64();
      for (int it = 1;; ++it) {  // (the error word and the clock every 16th retry)
        __builtin_amdgcn_s_sleep(1);
        seen = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(seen - want) >= 0) break;
        if (it % 16) continue;
        if (error_set(d)) { ok = 0; break; }
        if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
          set_error(d, DEVERR_TIMEOUT, t.gidx, -5, seen, want);
          ok = 0;
          break;
        }
      }
    }
    sm.imisc[0] = ok;
  }
  __syncthreads();
  return sm.imisc[0] != 0;
}
// Every wave: rows [lo, lo+nr) of each matrix of the block summed over the
// ns partial slots into out[(m*nr + r)][slot], the sums of squares into
// ss[slot]; 16 bytes (4 slots) per thread and slot, loads issued 8 at a time.
DEV void ksplit_reduce(CP &d, const MGeo &g, const KSplit &k, int lo, int nr, float *out,
                       float *ss) {
  const int Bp = g.B16 * 16, c4 = Bp / 4, R = g.NGs * 16;
  const int nrow = g.nseg * nr * c4;
  const int nu = nrow + c4;
  const uint32_t slot_b = (uint32_t)kpart_slot(d.B) * 4u;
  const __amdgpu_buffer_rsrc_t r = rsrc(kslot(d, k, 0));
  for (int u = tidx(); u < nu; u += kThreads) {
    uint32_t off;
    float *dst;
    if (u < nrow) {
      const int m = u / (nr * c4), rem = u - m * nr * c4, rr = rem / c4, c = rem - rr * c4;
      off = (uint32_t)(((m * R + lo + rr) * Bp + 4 * c) * 4);
      dst = out + (m * nr + rr) * Bp + 4 * c;
    } else {
      const int c = u - nrow;
      off = (uint32_t)((kMfmaGroups * 16 * Bp + 4 * c) * 4);
      dst = ss + 4 * c;
    }
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k.ns; j0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = j0 + j < k.ns ? j0 + j : 0;
        v[j] = lda4(r, off + (uint32_t)jj * slot_b);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j0 + j < k.ns) a = j0 + j == 0 ? v[j] : a + v[j];
    }
    *(f32x4 *)dst = a;
  }
}

DEV bool gemv_mfma_ctl(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                       WState &ws) {
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  trace_start(d, t);
  const MGeo g = mgeo_of(d, t);
  float ssl[4] = {0.f, 0.f, 0.f, 0.f};
  mx_copy0(sm, d, g, t);
  __syncthreads();  // slice 0 copied, its gains in LDS
  mx_convert0(sm, d, g, t, ssl);
  if (g.P > 1) mx_dma(sm, d, g, t, 1, 1);
  trace_mark(d, t, 0);
  __syncthreads();  // slice 0 staged
  for (int p = 0; p < g.P; ++p) {
    if (p + 1 < g.P) mx_convert(sm, d, g, t, p + 1, (p + 1) & 1, ssl);
    __syncthreads();  // pass p done, slice p + 1 staged
    if (p + 2 < g.P) mx_dma(sm, d, g, t, p + 2, p & 1);  // into the buffer pass p read
  }
  mss_publish(sm, ssl);
  __syncthreads();  // accumulators and sums of squares in LDS
  trace_mark(d, t, 1);
  float *rs = &sm.rows[0][0];
  const int Bp = g.B16 * 16;
  const KSplit k = ksplit_of(t);
  if (k.ns > 1) {
    ksplit_publish(sm, d, g, k);
    vm_drain();
    if (!ksplit_arrive(sm, d, ca, t, k)) return false;  // every tile's partial published
    int lo, nr;
    ksplit_rows(g, k, lo, nr);
    float *red = sm.xs + kMfmaGroups * 16 * 64, *ss = &sm.rows[1][0];
    ksplit_reduce(d, g, k, lo, nr, red, ss);
    __syncthreads();  // the slice's sums in LDS
    if (t.gain && (tidx() & 63) < Bp)
      rs[tidx() & 63] = 1.0f / sqrtf(ss[tidx() & 63] / (float)g.ld + d.eps);
    mepilogue(d, ca, t, nr, Bp, lo, red, rs);
  } else {
    if (t.gain) mss_rms(sm, d, g, rs);  // this wave's own LDS writes: no barrier needed
    mepilogue(d, ca, t, g.NGs * 16, Bp, 0, sm.xs, rs);
  }
  if (persistent) {
    if (t.a5 > 0) vm_drain();
    trace_finish(d, t);
    signal_done(d, t);
  }
  __syncthreads();  // LDS free for the next task
  ws.x_src = nullptr;
  return true;
}

DEV bool gemv_mfma_cmp(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                       WState &ws, Buf &w, bool w_loaded, bool pre, const MGeo &gn) {
  const int cw = uni(tidx() >> 6) - 1, lane = tidx() & 63;
  const MGeo g = mgeo_of(d, t);
  if (!w_loaded) mload(g, w, cw);  // weights do not wait for the inputs
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float ssl[4] = {0.f, 0.f, 0.f, 0.f};  // (the control wave stages the later slices)
  const KSplit k = ksplit_of(t);
  __syncthreads();  // slice 0 copied, its gains in LDS
  mx_convert0(sm, d, g, t, ssl);
  __syncthreads();  // slice 0 staged
  for (int p = 0; p < g.P; ++p) {
    const char *xb = (const char *)sm.xs + (p & 1) * (g.nkb * g.B16 * 2048);
    // the slot-tile count as a constant: no branch around any product
    if (g.nkb >= 16) {
      switch (g.B16) {
        case 1: mpass<16, 1>(g, w, acc, xb, cw, p, pre, gn); break;
        case 2: mpass<16, 2>(g, w, acc, xb, cw, p, pre, gn); break;
        case 3: mpass<16, 3>(g, w, acc, xb, cw, p, pre, gn); break;
        default: mpass<16, 4>(g, w, acc, xb, cw, p, pre, gn); break;
      }
    } else {
      switch (g.B16) {
        case 1: mpass<8, 1>(g, w, acc, xb, cw, p, pre, gn); break;
        case 2: mpass<8, 2>(g, w, acc, xb, cw, p, pre, gn); break;
        case 3: mpass<8, 3>(g, w, acc, xb, cw, p, pre, gn); break;
        default: mpass<8, 4>(g, w, acc, xb, cw, p, pre, gn); break;
      }
    }
    __syncthreads();  // pass p done, slice p + 1 staged (by the control wave)
  }
  mss_publish(sm, ssl);
  // accumulators to out[row][slot]: row = matrix*NGs*16 + slot*16 + 4(l/16) + e
  const int Bp = g.B16 * 16;
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    int seg, slot;
    if (!mgroup(g, cw, gi, seg, slot)) continue;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st >= g.B16) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = seg * g.NGs * 16 + slot * 16 + 4 * (lane >> 4) + e;
        sm.xs[row * Bp + st * 16 + (lane & 15)] = acc[gi][st][e];
      }
    }
  }
  __syncthreads();  // accumulators and sums of squares in LDS
  if (k.ns > 1) {
    if (!ksplit_arrive(sm, d, ca, t, k)) return false;
    int lo, nr;
    ksplit_rows(g, k, lo, nr);
    ksplit_reduce(d, g, k, lo, nr, sm.xs + kMfmaGroups * 16 * 64, &sm.rows[1][0]);
    __syncthreads();  // the slice's sums in LDS
  }
  __syncthreads();  // outputs written: LDS free for the next task
  ws.x_src = nullptr;
  return true;
}

// -------------------------------------------------------------- attention --
// One (slot, KV head, split) task: the query heads of the group attend to
// the cached keys of positions [lo, min(hi, pos)) of the split, read page by
// page (16 positions) from the paged pools; the split that contains the
// current position also rotates and stores the new key/value (bf16) and
// attends to it.  Softmax runs online in base 2 on log2(e)/sqrt(hd)-scaled
// scores; the task leaves (max, sum, weighted values) for the merge, or the
// normalised output when there is a single split.  Wave w takes the split's
// pages w, w+8, ...: their page ids are read 64 at a time (lane i holding the
// i-th) and two pages' keys and values are in flight while one is consumed.
// The cached pages do not depend on this step's projections: the ids and the
// first two pages are loaded before the task waits for the query/key/value
// tiles of its group.
// Returns false when the step is drained after an error.
template <int HD>
DEV bool run_attn(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws) {
  const int tix = t.gidx;
  const int l = t.layer, b = t.a0, g = t.a1, sp = t.a2;
  const int G = d.G, S = d.S, B = d.B, nkv = d.nkv, nq = d.nq;
  const int tid = tidx(), lane = tid & 63, wave = uni(tid >> 6);
  constexpr int PS = HD + 4;
  // Queries: each head's row is four quarters of HD/4, a lane reading the
  // quarter of its key dims; quarters are padded by 16 bytes so the four
  // quarters a wave reads at once lie in different LDS banks.
  constexpr int QQ = HD / 4 + 4, QROW = 4 * QQ;
  float *qs = sm.xs;                         // [G][4][QQ]
  float *kc = qs + kMaxGroup * QROW;         // [HD]
  float *vc = kc + HD;                       // [HD]
  float *wm = vc + HD;                       // [kWaves][kMaxGroup]
  float *wl = wm + kWaves * kMaxGroup;       // [kWaves][kMaxGroup]
  float *wo = wl + kWaves * kMaxGroup;       // [kWaves][kMaxGroup][HD]
  float *scur = wo + kWaves * kMaxGroup * HD;
  // below the waves' scratch kilobytes, which sit below the LDS weight
  // slots (those may hold loads in flight)
  static_assert((kMaxGroup * QROW + 2 * HD + 2 * kWaves * kMaxGroup + kWaves * kMaxGroup * HD +
                 kMaxGroup) * 4 <= kAttnScratchOff, "attention LDS overlaps its scratch");

  const int pos = uni(ldg(ca.positions + b));
  const size_t head0 = ((size_t)l * B + b) * nq + (size_t)g * G;  // first head row
  constexpr int KB = HD / 32;  // 32-dim blocks of a key row: score products per page
  constexpr int NB = HD / 16;  // 16-dim blocks of a value row: output products per pair
  const int r16 = lane & 15, grp = lane >> 4;
  const bool pos_ok = pos >= 0 && pos < d.max_pos;
  const int n = pos + 1;
  const int lo = pos_ok ? (int)((int64_t)sp * n / S) : 0;
  const int hi = pos_ok ? (int)((int64_t)(sp + 1) * n / S) : 0;
  // cached keys [lo, chi); in shared-sequence plans the current one is
  // cached too (stored by the layer's KVAPP tasks before this task runs)
  const bool kvf = d.kv_first != 0;
  const int chi = kvf || hi < pos ? hi : pos;
  const int blk0 = lo / kPageSize, blk1 = chi > lo ? (chi - 1) / kPageSize : -1;
  // this wave's pages: blk0 + wave + i * kWaves for i < npw
  const int npw = blk1 >= blk0 + wave ? (blk1 - blk0 - wave) / kWaves + 1 : 0;
  const int32_t *prow = pos_ok ? page_row(d, ca, b, tix) : d.page_table;
  const int32_t *ptab = prow + blk0 + wave;
  auto page_ids = [&](int c0) {  // lane i: the id of page c0 + i (or -1)
    const int i = c0 + lane;
    return i < npw ? ldg(ptab + (size_t)i * kWaves) : -1;
  };
  // The wave's pages are taken in pairs.  Keys of a page are the A operand
  // of the score products (lane: position r16, dims kb*32 + 8*grp .. +8, one
  // 16-byte load per k-block); the values of a pair are the B operand of the
  // output products (lane: dim nn*16 + r16 of the pair's first page for
  // lanes 0-31, of its second for 32-63, positions 8*(grp&1) .. +8: the
  // value pool is transposed within a page, so that is one 16-byte load).
  u32x4 kq[2][KB], vq[NB];
  auto page_base = [&](int pid, int i) -> size_t {
    int pg = __builtin_amdgcn_readlane(pid, i);
    pg = pg >= 0 && pg < d.npages ? pg : 0;  // a bad id is reported before use
    return (((size_t)l * d.npages + pg) * nkv + g) * kPageSize * HD;
  };
  auto load_keys = [&](int pid, int i, u32x4 (&kr)[KB]) {
    const size_t pb = page_base(pid, i);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      kr[kb] = ldg((const u32x4 *)(d.k_pool + pb + r16 * HD + kb * 32 + 8 * grp));
  };
  auto load_values = [&](int pid, int i0, int i1) {
    const size_t pa = page_base(pid, i0), pz = page_base(pid, i1);
    const size_t pb = lane < 32 ? pa : pz;
#pragma unroll
    for (int nn = 0; nn < NB; ++nn)
      vq[nn] = ldg((const u32x4 *)(d.v_pool + pb + (size_t)(nn * 16 + r16) * kPageSize +
                                   8 * (grp & 1)));
  };
  // (Everything loaded here has arrived before the page loop: the task's
  // own input loads after the wait are waited for in order.)
  int pid = -1;
  auto first_pair = [&]() {
    if (npw > 0) {
      pid = page_ids(0);
      load_keys(pid, 0, kq[0]);
      load_keys(pid, min(1, npw - 1), kq[1]);
      load_values(pid, 0, min(1, npw - 1));
    }
  };
  // (shared-sequence plans: this step writes into the pages, so they are
  // read only after the wait)
  if (!kvf) {
    first_pair();
    // A wave with a second (and last) pair brings it into the L2 as well
    // (LDS-DMA of each page's keys and values, 1 KiB at a time, into a
    // scratch kilobyte of the wave above the attention's LDS): the page
    // loop's own loads of it then come from the L2.  (Nothing reads the
    // scratch; the copies complete before the task's first wait for its
    // register loads, which counts them.)  Longer page walks skip it: the
    // copies would sit ahead of the polls for the task's inputs.
    const int nwarm = npw <= 4 ? npw : 0;
    if (nwarm > 2) {
      const uint32_t junk = (uint32_t)(uintptr_t)sm.xs + (uint32_t)(kAttnScratchOff + wave * 1024);
      constexpr int kChunks = kPageSize * HD * 2 / 1024;  // 1 KiB pieces of a page
      for (int i = 2; i < nwarm; ++i) {
        const size_t pb = page_base(pid, i);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          dma16((uint64_t)(d.k_pool + pb) + (uint64_t)(c * 1024 + lane * 16), junk);
          dma16((uint64_t)(d.v_pool + pb) + (uint64_t)(c * 1024 + lane * 16), junk);
        }
      }
    }
  }
  // The rotation of this position (a thread's query and key elements all
  // use element (tid mod HD) mod HD/2 of it) and the page of the current
  // position do not depend on this step's data either: loaded before the
  // wait as well.
  const bool has_cur = pos_ok && !kvf && hi == n;
  float cv = 0.f, sv = 0.f;
  int pg = 0;
  if (pos_ok) {
    const int i0 = (tid % HD) & (HD / 2 - 1);
    cv = ldg(d.rope_cos + (size_t)pos * (HD / 2) + i0);
    sv = ldg(d.rope_sin + (size_t)pos * (HD / 2) + i0);
    if (has_cur) pg = uni(ldg(prow + pos / kPageSize));
  }
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  if (kvf) first_pair();
  if (!pos_ok) {
    trace_start(d, t);
    if (pos >= d.max_pos && tid == 0)
      set_error(d, DEVERR_BAD_INPUT, tix, -1, (uint32_t)pos, (uint32_t)d.max_pos);
    if (S == 1 && persistent) trace_finish(d, t);  // before the (tagged) outputs
    for (int idx = tid; idx < G * HD; idx += kThreads) {
      const int h = idx / HD, dd = idx - h * HD;
      if (S == 1) {
        stv(d, d.attn, (head0 + h) * HD + dd, 0.f, ca.tag);
      } else {
        float *pp = d.part + ((head0 + h) * S + sp) * PS;
        sta(pp + dd, 0.f);
        if (dd == 0) { sta(pp + HD, -INFINITY); sta(pp + HD + 1, 0.f); }
      }
    }
    return true;
  }
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  // q, k, v are tagged: the loads double as the wait for the projections.
  // A thread's first loads of its key/value and query elements are issued
  // together; only stale ones are then polled, one after another.
  const size_t q0 = head0 * HD;
  const size_t kvo = (((size_t)l * B + b) * nkv + g) * HD;
  uint64_t kra = 0, krc = 0, vr = 0;
  if (has_cur && tid < HD) {
    const int i0 = tid & (HD / 2 - 1);
    kra = ldt_raw(d.k, kvo + i0);
    krc = ldt_raw(d.k, kvo + i0 + HD / 2);
    vr = ldt_raw(d.v, kvo + tid);
  }
  for (int idx = tid; idx < G * HD; idx += kThreads) {
    const int h = idx / HD, i = idx - h * HD, i0 = i & (HD / 2 - 1);
    const uint64_t ra = ldt_raw(d.q, q0 + h * HD + i0);
    const uint64_t rc = ldt_raw(d.q, q0 + h * HD + i0 + HD / 2);
    const float a = ldt_then(sm, d, ca, t, d.q, q0 + h * HD + i0, ra);
    const float c2 = ldt_then(sm, d, ca, t, d.q, q0 + h * HD + i0 + HD / 2, rc);
    const float r = (i < HD / 2) ? a * cv - c2 * sv : a * sv + c2 * cv;
    qs[h * QROW + (i / (HD / 4)) * QQ + (i & (HD / 4 - 1))] = r * scale;
  }
  if (has_cur) {
    const bool pg_ok = pg >= 0 && pg < d.npages;
    if (!pg_ok && tid == 0) set_error(d, DEVERR_BAD_INPUT, tix, -2, (uint32_t)pg, (uint32_t)d.npages);
    for (int i = tid; i < HD; i += kThreads) {  // (HD <= kThreads: i == tid)
      const int i0 = i & (HD / 2 - 1);
      const float a = ldt_then(sm, d, ca, t, d.k, kvo + i0, kra);
      const float c2 = ldt_then(sm, d, ca, t, d.k, kvo + i0 + HD / 2, krc);
      const float kr = (i < HD / 2) ? a * cv - c2 * sv : a * sv + c2 * cv;
      const uint16_t kb = f2bf(kr), vb = f2bf(ldt_then(sm, d, ca, t, d.v, kvo + i, vr));
      kc[i] = bf1(kb);
      vc[i] = bf1(vb);
      if (pg_ok) {
        const size_t page = ((size_t)l * d.npages + pg) * nkv + g;
        const int ps = pos & (kPageSize - 1);
        stg(d.k_pool + (page * kPageSize + ps) * HD + i, kb);
        stg(d.v_pool + (page * HD + i) * kPageSize + ps, vb);  // [dim][position]
      }
    }
  }
  __syncthreads();
  if (sm.imisc[2] == (int)ca.tag) return false;  // projections never arrived
  trace_start(d, t);  // inputs complete
  trace_mark(d, t, 0);

  // --- page loop (matrix cores)
  // Queries as the B operand of the score products: lane = head r16 (zero
  // past G), dims kb*32 + 8*grp .. +8, as a bf16 value and a bf16 remainder
  // (two products keep about 16 bits of the fp32 query).
  bf16x8 qh[KB], ql[KB];
  {
    const int hq = r16 < G ? r16 : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int d0 = kb * 32 + 8 * grp;
      const float *qp = qs + hq * QROW + (d0 / (HD / 4)) * QQ + (d0 & (HD / 4 - 1));
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = r16 < G ? qp[e] : 0.f;
      qh[kb] = __builtin_convertvector(x, bf16x8);
      ql[kb] = __builtin_convertvector(x - __builtin_convertvector(qh[kb], f32x8), bf16x8);
    }
  }
  // Online softmax in base 2 per head: lane r16's head; its running max and
  // sum are kept in the four lanes of the head (one per 16-lane group).  The
  // outputs o[nn] hold heads 4*grp + j, dims nn*16 + r16.
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NB];
#pragma unroll
  for (int nn = 0; nn < NB; ++nn) o[nn] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < npw; c0 += 64) {
    const int nc = min(64, npw - c0);
    if (c0 > 0) {
      pid = page_ids(c0);
      load_keys(pid, 0, kq[0]);
      load_keys(pid, min(1, nc - 1), kq[1]);
      load_values(pid, 0, min(1, nc - 1));
    }
    const uint64_t bad = __ballot(lane < nc && (pid < 0 || pid >= d.npages));
    if (bad) {
      if (lane == (int)__builtin_ctzll(bad))
        set_error(d, DEVERR_BAD_INPUT, tix, -2, (uint32_t)pid, (uint32_t)d.npages);
      break;
    }
    for (int i = 0;; i += 2) {
      // (the wave's last pair issues no loads: a load left in flight at the
      // end of the loop would be waited for before its registers are reused)
      const bool more = i + 2 < nc;
      // scores of pages i, i+1: lane = head r16, positions 4*grp + j
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, kq[0][kb]);
        const bf16x8 kz = __builtin_bit_cast(bf16x8, kq[1][kb]);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[kb], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kz, qh[kb], sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[kb], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kz, ql[kb], sb, 0, 0, 0);
      }
      // the next pair's keys (an odd count reads its last page twice)
      const int n0 = min(i + 2, nc - 1), n1 = min(i + 3, nc - 1);
      if (more) {
        load_keys(pid, n0, kq[0]);
        load_keys(pid, n1, kq[1]);
      }
      const int pa = (blk0 + wave + (c0 + i) * kWaves) * kPageSize + 4 * grp;
      const int pz = pa + kWaves * kPageSize;
      const bool has_z = i + 1 < nc;
      float sc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = pa + j >= lo && pa + j < chi ? sa[j] : -INFINITY;
        sc[4 + j] = has_z && pz + j >= lo && pz + j < chi ? sb[j] : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run, mx);
      const bool live = mn != -INFINITY;
      const float alpha = live ? exp2f(m_run - mn) : 1.f;
      float pe[8], rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = live ? exp2f(sc[e] - mn) : 0.f;
        rs += pe[e];
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run = l_run * alpha + rs;
      m_run = live ? mn : m_run;
      // rescale the outputs of heads 4*grp + j (their factors sit in lanes
      // 4*grp + j)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * grp + j, 64);
#pragma unroll
        for (int nn = 0; nn < NB; ++nn) o[nn][j] *= aj;
      }
      // the weights as the A operand of the output products: lane = head
      // r16, positions 8*grp .. +8 of the pair (grp 0-1: first page, 2-3:
      // second), gathered from the lanes holding them
      const int src0 = r16 + 32 * (grp & 1), src1 = src0 + 16;
      f32x8 pv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = __shfl(pe[j], src0, 64), z0 = __shfl(pe[4 + j], src0, 64);
        const float a1 = __shfl(pe[j], src1, 64), z1 = __shfl(pe[4 + j], src1, 64);
        pv[j] = grp < 2 ? a0 : z0;
        pv[4 + j] = grp < 2 ? a1 : z1;
      }
      const bf16x8 ph = __builtin_convertvector(pv, bf16x8);
      const bf16x8 pl = __builtin_convertvector(pv - __builtin_convertvector(ph, f32x8), bf16x8);
      // A masked position has weight exactly 0, but 0 times a non-finite
      // value is NaN: on a pair that reaches outside [lo, chi) (the split's
      // edges, the tail page read twice, slots after the current position
      // that hold whatever the caller's pool holds) the values of those
      // positions are cleared before the products.
      {
        const int pfirst = (blk0 + wave + (c0 + i) * kWaves) * kPageSize;
        const int plast = pfirst + (has_z ? kWaves * kPageSize : 0) + kPageSize;
        if (pfirst < lo || plast > chi || !has_z) {
          const int p0 = pfirst + (lane < 32 ? 0 : kWaves * kPageSize) + 8 * (grp & 1);
          const bool page_ok = lane < 32 || has_z;
          uint32_t vmask[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int pe0 = p0 + 2 * c, pe1 = pe0 + 1;
            vmask[c] = (page_ok && pe0 >= lo && pe0 < chi ? 0x0000ffffu : 0u) |
                    (page_ok && pe1 >= lo && pe1 < chi ? 0xffff0000u : 0u);
          }
#pragma unroll
          for (int nn = 0; nn < NB; ++nn) {
            vq[nn].x &= vmask[0];
            vq[nn].y &= vmask[1];
            vq[nn].z &= vmask[2];
            vq[nn].w &= vmask[3];
          }
        }
      }
#pragma unroll
      for (int nn = 0; nn < NB; ++nn) {
        const bf16x8 vv = __builtin_bit_cast(bf16x8, vq[nn]);
        o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vv, o[nn], 0, 0, 0);
        o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vv, o[nn], 0, 0, 0);
      }
      if (!more) break;
      load_values(pid, n0, n1);  // the next pair's values
    }
  }
  // per-wave state to LDS: lane h < G holds head h's max and sum
  if (lane < G) {
    wm[wave * kMaxGroup + lane] = m_run;
    wl[wave * kMaxGroup + lane] = l_run;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * grp + j;
    if (h < G) {
#pragma unroll
      for (int nn = 0; nn < NB; ++nn) wo[(wave * kMaxGroup + h) * HD + nn * 16 + r16] = o[nn][j];
    }
  }
  if (has_cur && wave < G) {  // score of the current key for head `wave`
    float a = 0.f;
    for (int i = lane; i < HD; i += 64)
      a = fmaf(qs[wave * QROW + (i / (HD / 4)) * QQ + (i & (HD / 4 - 1))], kc[i], a);
    a = wave_sum(a);
    if (lane == 0) scur[wave] = a;
  }
  __syncthreads();
  trace_mark(d, t, 1);
  if (S == 1 && persistent) trace_finish(d, t);  // before the (tagged) outputs
  // merge the waves (fixed order) and the current key: four consecutive
  // dims per thread, written 16 bytes at a time (fewer stores for the
  // arrival's drain and the consumers' polls to wait for)
  const __amdgpu_buffer_rsrc_t ro = rsrc(S == 1 ? (const void *)d.attn : (const void *)d.part);
  for (int idx = tid * 4; idx < G * HD; idx += kThreads * 4) {
    const int h = idx / HD, dd = idx - h * HD;
    float M = -INFINITY;
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, wm[w2 * kMaxGroup + h]);
    if (has_cur) M = fmaxf(M, scur[h]);
    float Ls = 0.f;
    f32x4 Os = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float mw = wm[w2 * kMaxGroup + h];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        Ls = fmaf(f, wl[w2 * kMaxGroup + h], Ls);
        const f32x4 o = *(const f32x4 *)&wo[(w2 * kMaxGroup + h) * HD + dd];
        Os.x = fmaf(f, o.x, Os.x);
        Os.y = fmaf(f, o.y, Os.y);
        Os.z = fmaf(f, o.z, Os.z);
        Os.w = fmaf(f, o.w, Os.w);
      }
      if (has_cur) {
        const float f = exp2f(scur[h] - M);
        Ls += f;
        const f32x4 v = *(const f32x4 *)&vc[dd];
        Os.x = fmaf(f, v.x, Os.x);
        Os.y = fmaf(f, v.y, Os.y);
        Os.z = fmaf(f, v.z, Os.z);
        Os.w = fmaf(f, v.w, Os.w);
      }
    }
    if (S == 1) {
      // (value, tag) pairs, two per 16-byte store: each pair is one 8-byte
      // half of it, so a reader that sees a pair's tag sees its value
      const f32x4 y = Ls > 0.f ? (f32x4){Os.x / Ls, Os.y / Ls, Os.z / Ls, Os.w / Ls}
                               : (f32x4){0.f, 0.f, 0.f, 0.f};
      const size_t e = (head0 + h) * HD + dd;
      const u32x4 p0 = {__float_as_uint(y.x), ca.tag, __float_as_uint(y.y), ca.tag};
      const u32x4 p1 = {__float_as_uint(y.z), ca.tag, __float_as_uint(y.w), ca.tag};
      __builtin_amdgcn_raw_buffer_store_b128(p0, ro, (uint32_t)(e * 8), 0, kCpolSc1);
      __builtin_amdgcn_raw_buffer_store_b128(p1, ro, (uint32_t)(e * 8 + 16), 0, kCpolSc1);
      if (d.shadow)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y),
                                               rsrc(shadow_of(d, d.attn)), (uint32_t)(e * 4), 0,
                                               kCpolSc1);
    } else {
      const size_t o = ((head0 + h) * S + sp) * PS;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Os), ro,
                                             (uint32_t)((o + dd) * 4), 0, kCpolSc1);
      if (dd == 0)  // (max, sum) in one 8-byte store
        __hip_atomic_store((AS1 uint64_t *)(d.part + o + HD),
                           ((uint64_t)__float_as_uint(Ls) << 32) | __float_as_uint(M),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return true;
}

// Shared-sequence plans: store slot b's rotated key and its value, every KV
// head, into the page of its position (the same rotation and bf16 rounding
// as the attention task's own store in the other plans).  The layer's
// attention tasks wait for all of these, so each slot of a prompt chunk sees
// the keys of the chunk's earlier positions.
DEV void run_kvapp(Smem &sm, CP &d, const CallArgs &ca, const TD &t) {
  const int l = t.layer, b = t.a0, HD = d.hd, half = HD / 2, nkv = d.nkv;
  const int pos = uni(ldg(ca.positions + b));
  if (pos < 0) return;
  if (pos >= d.max_pos) {
    if (tidx() == 0) set_error(d, DEVERR_BAD_INPUT, t.gidx, -1, (uint32_t)pos, (uint32_t)d.max_pos);
    return;
  }
  const int pg = uni(ldg(page_row(d, ca, b, t.gidx) + pos / kPageSize));
  if (pg < 0 || pg >= d.npages) {
    if (tidx() == 0) set_error(d, DEVERR_BAD_INPUT, t.gidx, -2, (uint32_t)pg, (uint32_t)d.npages);
    return;
  }
  const float *cs = d.rope_cos + (size_t)pos * half;
  const float *sn = d.rope_sin + (size_t)pos * half;
  const size_t kv0 = ((size_t)l * d.B + b) * nkv * HD;
  const int ps = pos & (kPageSize - 1);
  for (int idx = tidx(); idx < nkv * HD; idx += kThreads) {
    const int g = idx / HD, i = idx - g * HD, i0 = i & (half - 1);
    const float a = ldt_wait(sm, d, ca, t, d.k, kv0 + g * HD + i0);
    const float c2 = ldt_wait(sm, d, ca, t, d.k, kv0 + g * HD + i0 + half);
    const float cv = ldg(cs + i0), sv = ldg(sn + i0);
    const float kr = (i < half) ? a * cv - c2 * sv : a * sv + c2 * cv;
    const size_t page = ((size_t)l * d.npages + pg) * nkv + g;
    // agent-coherent stores: other CUs read these pages later in this step
    sta16(d.k_pool + (page * kPageSize + ps) * HD + i, f2bf(kr));
    sta16(d.v_pool + (page * HD + i) * kPageSize + ps,
          f2bf(ldt_wait(sm, d, ca, t, d.v, kv0 + g * HD + i)));
  }
}

// Log-sum-exp merge of the S split partials (o[HD], m, l) of one (slot, KV
// head): the group's G query heads.  Every thread takes one 16-byte output
// vector and a subset of the splits (split sp goes to subset sp mod nsub);
// its first 16 partial vectors are loaded together with every split's (m, l)
// before anything is consumed.  One wave per head turns (m, l) into the
// weights 2^(m_s - M) / L in LDS; each thread adds up its weighted vectors,
// and the subsets are added in a fixed order (deterministic).
DEV void run_merge(Smem &sm, CP &d, const CallArgs &ca, const TD &t) {
  const int l = t.layer, b = t.a0, g = t.a1, G = d.G, S = d.S, HD = d.hd;
  const int PS = HD + 4, hv = HD / 4, nvec = G * hv, npairs = G * S;
  const int nsub = kThreads / nvec;
  const int tid = tidx(), lane = tid & 63, wave = uni(tid >> 6);
  const size_t head0 = ((size_t)l * d.B + b) * d.nq + (size_t)g * G;
  const float *part0 = d.part + head0 * S * PS;
  const __amdgpu_buffer_rsrc_t r = rsrc(part0);
  const int v = tid % nvec, sub = tid / nvec;
  const bool act = sub < nsub;
  const int h = v / hv, dd = (v - h * hv) * 4;
  constexpr int kBatch = 16;
  f32x4 ov[kBatch];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sp = base + sub + k * nsub;
      ov[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (act && sp < S) ov[k] = lda4(r, (uint32_t)((((size_t)h * S + sp) * PS + dd) * 4));
    }
  };
  load_batch(0);
  float2 *ml = (float2 *)&sm.red[0][0];  // [G * S]: (m, l), then (weight, -)
  for (int i = tid; i < npairs; i += kThreads) {
    const float *pp = part0 + (size_t)i * PS + HD;  // pair i = head * S + split
    const uint64_t w = __hip_atomic_load((const AS1 uint64_t *)pp, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);  // (max, sum)
    ml[i] = make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
  }
  __syncthreads();
  for (int hh = wave; hh < G; hh += kWaves) {
    float mx = -INFINITY;
    for (int sp = lane; sp < S; sp += 64) mx = fmaxf(mx, ml[hh * S + sp].x);
    mx = wave_max(mx);
    float lsum = 0.f;
    for (int sp = lane; sp < S; sp += 64) {
      const float2 e = ml[hh * S + sp];
      lsum = fmaf(e.x == -INFINITY ? 0.f : exp2f(e.x - mx), e.y, lsum);
    }
    lsum = wave_sum(lsum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    for (int sp = lane; sp < S; sp += 64) {
      const float mv = ml[hh * S + sp].x;
      ml[hh * S + sp].x = mv == -INFINITY ? 0.f : exp2f(mv - mx) * inv;
    }
  }
  __syncthreads();
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < S; base += kBatch * nsub) {
    if (base > 0) load_batch(base);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int sp = base + sub + k * nsub;
      if (act && sp < S) o += ml[h * S + sp].x * ov[k];
    }
  }
  f32x4 *red = (f32x4 *)sm.xs;  // [nsub][nvec]
  const __amdgpu_buffer_rsrc_t ro = rsrc(d.attn);
  if (act) red[sub * nvec + v] = o;
  __syncthreads();
  for (int vv = tid; vv < nvec; vv += kThreads) {
    f32x4 sum = red[vv];
    for (int q = 1; q < nsub; ++q) sum += red[q * nvec + vv];
    const int hh = vv / hv, d0 = (vv - hh * hv) * 4;
    const size_t e = (head0 + hh) * HD + d0;
    // two (value, tag) pairs per 16-byte store, as the attention writes them
    const u32x4 p0 = {__float_as_uint(sum.x), ca.tag, __float_as_uint(sum.y), ca.tag};
    const u32x4 p1 = {__float_as_uint(sum.z), ca.tag, __float_as_uint(sum.w), ca.tag};
    __builtin_amdgcn_raw_buffer_store_b128(p0, ro, (uint32_t)(e * 8), 0, kCpolSc1);
    __builtin_amdgcn_raw_buffer_store_b128(p1, ro, (uint32_t)(e * 8 + 16), 0, kCpolSc1);
    if (d.shadow)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sum),
                                             rsrc(shadow_of(d, d.attn)), (uint32_t)(e * 4), 0,
                                             kCpolSc1);
  }
}

// ------------------------------------------------------------- small ops --
DEV void run_embed(CP &d, const CallArgs &ca, const TD &t) {
  const int tix = t.gidx;
  const int b = t.a0, H = d.H;
  const int pos = uni(ldg(ca.positions + b));
  const int tok = uni(ldg(ca.tokens + b));
  const bool ok = pos >= 0 && tok >= 0 && tok < d.V;
  if (pos >= 0 && !ok && tidx() == 0)
    set_error(d, DEVERR_BAD_INPUT, tix, -3, (uint32_t)tok, (uint32_t)d.V);
  const uint16_t *e = d.embed + (size_t)(ok ? tok : 0) * H;
  for (int i = tidx(); i < H; i += kThreads)
    stv(d, d.x, (size_t)b * H + i, ok ? bf1(ldg(e + i)) : 0.f, ca.tag);
}

// Softmax router top-k: k rounds of (max, lowest index) over the logits not
// yet taken; weights = softmax over the chosen logits; ids ascending.
DEV void run_argmax(Smem &sm, CP &d, const CallArgs &ca, const TD &t) {
  const int b = t.a0, nt = d.n_lm_tiles;
  const int tid = tidx(), lane = tid & 63, wave = tid >> 6;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < nt; i += kThreads) {
    const float v = lda(d.amax_v + (size_t)b * nt + i);
    const int ix = ldai(d.amax_i + (size_t)b * nt + i);
    if (better(v, ix, bv, bi)) { bv = v; bi = ix; }
  }
  wave_argmax(bv, bi);
  if (lane == 0) { sm.misc[wave] = bv; sm.imisc[32 + wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    float cv = sm.misc[0];
    int ci = sm.imisc[32];
    for (int w2 = 1; w2 < kWaves; ++w2)
      if (better(sm.misc[w2], sm.imisc[32 + w2], cv, ci)) { cv = sm.misc[w2]; ci = sm.imisc[32 + w2]; }
    if (ci < 0 || ci >= d.V) ci = 0;
    stg(ca.next_tokens + b, ldg(ca.positions + b) >= 0 ? ci : -1);
  }
}

// Non-GEMV task (all waves): wait, run, publish (every wave drains its
// stores, then thread 0 reports).
DEV bool run_small(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent, WState &ws) {
  if (t.op == OP_ATTN) {  // waits for its inputs itself, after a prefetch
    const bool ok = d.hd == 128 ? run_attn<128>(sm, d, ca, t, persistent, ws)
                                : run_attn<64>(sm, d, ca, t, persistent, ws);
    if (!ok) return false;
  } else {
    if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
    trace_start(d, t);
  }
  switch (t.op) {
    case OP_EMBED:
      if (persistent) trace_finish(d, t);  // before the (tagged) outputs
      run_embed(d, ca, t);
      break;
    case OP_ARGMAX: run_argmax(sm, d, ca, t); break;
    case OP_KVAPP: run_kvapp(sm, d, ca, t); break;
    default: break;
  }
  ws.x_src = nullptr;  // LDS reused: the activation cache is gone
  if (t.op == OP_ATTN && d.S > 1) {
    // Split attention: the partials are visible before this split's
    // arrival is counted; the split that arrives last for its (slot, KV
    // head) merges the group and reports its completion.
    vm_drain();
    __syncthreads();
    if (persistent) trace_finish(d, t);
    if (tidx() == 0) {
      const uint32_t old = __hip_atomic_fetch_add(
          d.att_cnt + (((size_t)t.layer * d.B + t.a0) * d.nkv + t.a1) * kCtrStride, 1u, __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT);
      sm.imisc[1] = old == (ca.epoch + 1u) * (uint32_t)d.S - 1u;
    }
    __syncthreads();
    const bool last = sm.imisc[1] != 0;
    if (last) {
      run_merge(sm, d, ca, t);
      if (signals_counter(t)) vm_drain();
    }
    __syncthreads();
    if (persistent) signal_count(d, t, last ? 1 : 0);
    return true;
  }
  if (persistent && signals_counter(t)) vm_drain();
  __syncthreads();
  if (persistent) {
    // (embeddings and single-split attention recorded theirs before the
    // outputs)
    if (t.op != OP_EMBED && !(t.op == OP_ATTN && d.S == 1)) trace_finish(d, t);
    signal_done(d, t);
  }
  return true;
}

// Claimed attention (persistent, batched plans): the workgroup takes the
// layer's ATTN tasks one at a time from a shared counter until none is left.
// The counter grows by every claim, the failed last claim of each worker that
// holds entries of the layer included, so step e's claims start at
// e * (claims per step).  Every task still runs exactly once; each reports
// its own completion as it would in a worker queue.
// Claim order of pooled attention for this step (the MPK summary's roadmap,
// "भविष्य की दिशा": priority-based and throughput-oriented task scheduling).
// Slot b's rank is the number of slots whose key is larger, ties going to the
// lower slot; the key is (priority, context length) for order 2 and the
// context length for order 1, so the longest attention tasks of the most
// urgent sequences are claimed first and the layer's last claims are the
// shortest (longest-processing-time-first).  Empty slots rank last.
DEV void claim_order(Smem &sm, CP &d, const CallArgs &ca) {
  const int b = tidx();
  if (b < d.B) {
    auto key = [&](int s) -> int64_t {
      const int p = ldg(ca.positions + s);
      if (p < 0) return INT64_MIN;
      const int64_t pr = (d.attn_order == 2 && ca.prio) ? (int64_t)ldg(ca.prio + s) : 0;
      return (pr << 32) + p;
    };
    const int64_t kb = key(b);
    int rank = 0;
    for (int s = 0; s < d.B; ++s) {
      const int64_t ks = key(s);
      rank += ks > kb || (ks == kb && s < b);
    }
    sm.order[rank] = b;
  }
}

DEV bool run_attn_pool(Smem &sm, CP &d, const CallArgs &ca, const TD &t0, WState &ws) {
  const int first = t0.a4, n = t0.rpp & 0xffff;
  const int per_slot = n / d.B;  // the layer's tasks are slot-major
  const uint32_t per_step = (uint32_t)t0.rpp >> 16;
  uint32_t *cnt = d.pool_cnt + (size_t)t0.layer * kCtrStride;
  for (;;) {
    if (tidx() == 0) {
      const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.imisc[3] = (int)(old - ca.epoch * per_step);
    }
    __syncthreads();
    const int idx = uni(sm.imisc[3]);
    __syncthreads();  // every wave has read the claim
    if (idx < 0 || idx >= n) return true;
    const int k = d.attn_order ? sm.order[idx / per_slot] * per_slot + idx % per_slot : idx;
    const TD t = td_from_table(d.tasks, ((const AS4 int *)d.task_pos)[first + k]);
    if (!run_small(sm, d, ca, t, true, ws)) return false;
  }
}

// Run task t; `w` holds its weights when w_loaded.  When the worker's next
// task has static weights (pre), their tile geometry is gn and this task
// leaves them loading into `w`.  Returns whether it did; `alive` turns false
// when the step is drained after an error.  Uniform across waves.
// One task of the kernel-per-op executor (all waves of one workgroup).
DEV void run_task_once(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws) {
  if (t.op == OP_EDOWN) {
    if (uni(tidx() >> 6) == 0)
      down_ctl(sm, d, ca, t, false, ws);
    else
      down_cmp(sm, d, ca, t, false, ws);
  } else if (d.mfma && static_weights(t.op)) {
    if (uni(tidx() >> 6) == 0) {
      gemv_mfma_ctl(sm, d, ca, t, false, ws);
    } else {
      Buf w;
      MGeo gn;
      gemv_mfma_cmp(sm, d, ca, t, false, ws, w, false, false, gn);
    }
  } else if (!is_gemv(t.op)) {
    run_small(sm, d, ca, t, false, ws);
  } else if (uni(tidx() >> 6) == 0) {
    gemv_ctl<false>(sm, d, ca, t, false, ws);
  } else {
    Buf w;
    Geo gn;
    gemv_cmp<false>(sm, d, ca, t, false, ws, w, false, false, gn, false);
  }
}

// Whether the task with descriptor words `nx` waits for nothing but what the
// task `cur` reports (another tile of the same operation, or a direct
// consumer): its first pass is then loaded while `cur` finishes.  A task
// that waits for a later operation (the output projection behind attention)
// gets its loads after `cur`'s outputs, which its wait leaves time for.
// Words: 0 op | layer << 16, 1 n_wait | n_sig << 16, 8-10 waited events,
// 14-15 signalled events.
DEV bool waits_on(const uint32_t *nx, const uint32_t *cur) {
  const int w0 = uni((int)nx[0]), c0 = uni((int)cur[0]);
  if (w0 == c0) return true;
  const int nw = uni((int)(nx[1] & 0xffffu)), ns = uni((int)(cur[1] >> 16));
  for (int i = 0; i < nw && i < 3; ++i) {
    const int e = uni((int)nx[8 + i]);
    bool found = false;
    for (int j = 0; j < ns && j < 2; ++j) found = found || e == uni((int)cur[14 + j]);
    if (!found) return false;
  }
  return nw > 0;
}

// Geometry of the next task's first pass from its descriptor words in the
// ring: op (word 0), rows (a2, word 4), w0 / w1 (words 16-19), K (word 28),
// rows per pass (word 31).
DEV bool next_geo(const uint32_t *slot, Geo &g) {
  const int op = (int)(int16_t)(uni((int)slot[0]) & 0xffff);
  if (!static_weights(op)) return false;
  const int rows = uni((int)slot[4]);
  const uint16_t *w0 = (const uint16_t *)ptr_of((uint32_t)uni((int)slot[16]), (uint32_t)uni((int)slot[17]));
  const uint16_t *w1 = (const uint16_t *)ptr_of((uint32_t)uni((int)slot[18]), (uint32_t)uni((int)slot[19]));
  const int K = uni((int)slot[28]);
  const int rpp = uni((int)slot[31]);
  g = pass_geo(w0, w1, rows, rpp, K, 0);
  return true;
}

// The persistent worker runs its queue in order.  An LDS ring holds the
// descriptors of the current and the next tasks (refilled by compute wave 1).
// Wave 0 and waves 1-7 run separate loops over the same queue, meeting at
// each task's barriers.  On the compute side consecutive static-weight GEMV
// tasks form a run: one register tile buffer, local to the run, carries the
// weights of each pass into the next, and of each task's last pass into the
// next task's first (loaded before that task's dependency wait).
// The step's data tag: the launch argument, or for graph-replayed steps the
// device word that a kernel bumped before this one.
DEV CallArgs resolve_args(CP &d, CallArgs ca) {
  if (ca.tag == 0u) ca.tag = (uint32_t)uni((int)ldg(d.ctrl + CTRL_TAG));
  return ca;
}

// MODE 0: any batch on the vector path; 1: one slot; 2: matrix-core GEMVs
// (batches of 16..64 slots).
template <int MODE>
__global__ void __launch_bounds__(kThreads)
    mk_persistent_kernel(const DevPlan *__restrict__ dplan, CallArgs ca_in) {
  constexpr bool B1 = MODE == 1;
  __shared__ Smem sm;
  CP &d = *(CP *)dplan;
  const CallArgs ca = resolve_args(d, ca_in);
  if (tidx() == 0) sm.imisc[2] = 0;  // no tagged-data failure (the tag is never 0)
  if (d.attn_pool && d.attn_order) claim_order(sm, d, ca);  // read after the barrier below
  const int wid = blockIdx.x;
  const int beg = ((const AS4 int *)d.worker_off)[wid];
  const int end = ((const AS4 int *)d.worker_off)[wid + 1];
  const int wave = uni(tidx() >> 6), lane = tidx() & 63, cw = wave - 1;
  const u32x4 *tabv = (const u32x4 *)d.tasks;  // 8 x 16 bytes per descriptor
  u32x4 pend = {0u, 0u, 0u, 0u};
  if (wave == 1 && lane < 8) {
    for (int i = 0; i < 3 && beg + i < end; ++i)
      ((u32x4 *)sm.ring[i])[lane] = ldg(tabv + (size_t)(beg + i) * 8 + lane);
    if (beg + 3 < end) pend = ldg(tabv + (size_t)(beg + 3) * 8 + lane);
  }
  __syncthreads();
  WState ws;
  init_ws(ws);
  if (wave == 0) {
    for (int k = beg; k < end; ++k) {
      const TD t = td_from_ring(sm.ring[(k - beg) % kRing]);
      if (t.op == OP_ATTN && d.attn_pool) {
        if (!run_attn_pool(sm, d, ca, t, ws)) return;
        k += t.a3 - 1;    // this worker's other entries of the pool
        __syncthreads();  // the ring reloaded for the next task
        continue;
      }
      const bool alive =
          t.op == OP_EDOWN                      ? down_ctl(sm, d, ca, t, true, ws)
          : (MODE == 2 && static_weights(t.op)) ? gemv_mfma_ctl(sm, d, ca, t, true, ws)
          : is_gemv(t.op)                       ? gemv_ctl<B1>(sm, d, ca, t, true, ws)
                                                : run_small(sm, d, ca, t, true, ws);
      if (!alive) return;
    }
    return;
  }
  // Ring refill after task k (read two tasks later, after the next task's
  // barriers).  Compute wave 1 does it: the descriptor load, issued behind
  // the next tile's weights, has completed by the next weight wait; the
  // control wave's queue holds epilogue stores instead.
  auto refill = [&](int k) {
    if (wave == 1 && lane < 8) {
      const int i = k - beg;
      if (k + 3 < end) ((u32x4 *)sm.ring[(i + 3) % kRing])[lane] = pend;
      if (k + 4 < end) pend = ldg(tabv + (size_t)(k + 4) * 8 + lane);
    }
  };
  int k = beg;
  while (k < end) {
    TD t = td_from_ring(sm.ring[(k - beg) % kRing]);
    if (MODE == 2 && static_weights(t.op)) {
      // Matrix-core tiles: each tile's last pass refills the idle line; the
      // next tile issues its first pass before it waits for its inputs, so
      // those weights stream during the wait.  (Refilling with the next
      // tile during the last pass would hold this tile's end behind the
      // issue of those loads.)
      Buf w;
      MGeo gn;
      if (!gemv_mfma_cmp(sm, d, ca, t, true, ws, w, false, false, gn)) goto done;
      refill(k);
      ++k;
    } else if (static_weights(t.op)) {
      Buf w;
      load_slots(static_geo(t), w, cw, sm.xs, d.lds_slots != 0);
      for (;;) {
        Geo gn;
        const uint32_t *nx = sm.ring[(k + 1 - beg) % kRing];
        const bool pre = k + 1 < end && next_geo(nx, gn);
        const bool inter = pre && waits_on(nx, sm.ring[(k - beg) % kRing]);
        if (!gemv_cmp<B1>(sm, d, ca, t, true, ws, w, true, pre, gn, inter)) goto done;
        refill(k);
        ++k;
        if (!pre) break;
        t = td_from_ring(sm.ring[(k - beg) % kRing]);
      }
    } else if (t.op == OP_ATTN && d.attn_pool) {
      if (!run_attn_pool(sm, d, ca, t, ws)) goto done;
      k += t.a3;  // past this worker's entries of the pool: reload the ring there
      if (wave == 1 && lane < 8) {
        for (int i = 0; i < 3 && k + i < end; ++i)
          ((u32x4 *)sm.ring[(k + i - beg) % kRing])[lane] = ldg(tabv + (size_t)(k + i) * 8 + lane);
        if (k + 3 < end) pend = ldg(tabv + (size_t)(k + 3) * 8 + lane);
      }
      __syncthreads();
    } else {
      bool alive;
      if (t.op == OP_EDOWN) {
        alive = down_cmp(sm, d, ca, t, true, ws);
      } else if (is_gemv(t.op)) {
        Buf w;
        Geo gn;
        alive = gemv_cmp<B1>(sm, d, ca, t, true, ws, w, false, false, gn, false);
      } else {
        alive = run_small(sm, d, ca, t, true, ws);
      }
      if (!alive) goto done;
      refill(k);
      ++k;
    }
  }
done:
  vm_drain();  // LDS-DMA loads the compiler does not track complete before the wave ends
}

}  // namespace mk
