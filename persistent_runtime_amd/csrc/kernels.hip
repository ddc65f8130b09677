// kernels.hip -- device code of the decode-step megakernel for gfx950.
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
  DPP_MIRROR = 0x140        // lane i <- lane 15-i within 16
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
// sum over the 4 lanes of each quad (result in all 4)
DEV float quad_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  return v;
}
// values replicated within quads: max / sum over the 16 quads, uniform
DEV float quads_max(float v) {
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}
DEV float quads_sum(float v) {
  v += dpp<DPP_HALF_MIRROR>(v);
  v += dpp<DPP_MIRROR>(v);
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
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
DEV int ldai(const int32_t *p) {
  return __hip_atomic_load((const AS1 int32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void stai(int32_t *p, int32_t v) {
  __hip_atomic_store((AS1 int32_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

constexpr int kPartSlot = kMaxTileUnits16 * 4;   // GEMV partials per slot of a tile
constexpr int kRowSlot = kMaxTileUnits16 * 2;    // rows per tile (rows hold >= 256 elements)
#ifndef MK_REFILL_PER_SLOT
#define MK_REFILL_PER_SLOT 0
#endif
constexpr bool kRefillPerSlot = MK_REFILL_PER_SLOT;
constexpr int kRing = 4;                          // task descriptors kept ahead

struct Smem {
  float xs[kLdsXBytes / 4];                                 // staged activations
  float red[kMaxPass][kPartSlot];                           // GEMV partials [pass*n + slot]
  float rows[kMaxPass][kRowSlot];                           // GEMV row sums, same order
  uint32_t ring[kRing][32];                                 // task descriptors
  float misc[64];
  int imisc[64];
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
};

DEV void init_ws(WState &ws) {
  ws.x_src = nullptr;
  ws.x_gain = nullptr;
  ws.x_K = 0;
  ws.x_nb = 0;
  ws.sat_ev[0] = ws.sat_ev[1] = -1;
  ws.sat_want[0] = ws.sat_want[1] = 0;
}

DEV void set_error(CP &d, uint32_t code, int task, int ev, uint32_t seen, uint32_t want) {
  if (atomicCAS(&d.ctrl[CTRL_ERR], 0u, code) == 0u) {
    __hip_atomic_store(&d.ctrl[CTRL_ERR_TASK], (uint32_t)task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_EV], (uint32_t)ev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_SEEN], seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&d.ctrl[CTRL_ERR_WANT], want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
DEV bool error_set(CP &d) {
  return __hip_atomic_load(&d.ctrl[CTRL_ERR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// ------------------------------------------------------- dependency waits --
// A task needs each of its events' counters to reach (epoch+1)*threshold.
// Waits this worker already saw satisfied in this step are skipped without a
// poll (tiles of one operation share their input event).  Otherwise thread 0
// (control wave) polls; a barrier hands the outcome to the workgroup.
// Returns false when the step is being drained after an error.
DEV bool wait_deps(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws) {
  bool need = false;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i >= t.n_wait) break;
    const int e = t.wait_ev[i];
    const uint32_t want = (ca.epoch + 1u) * (uint32_t)t.wait_thr[i];
    const bool seen = (ws.sat_ev[0] == e && ws.sat_want[0] == want) ||
                      (ws.sat_ev[1] == e && ws.sat_want[1] == want);
    need = need || !seen;
  }
  if (!need) return true;
  if (tidx() == 0) {
    int ok = 1;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= t.n_wait || !ok) break;
      uint32_t *c = d.ev + t.wait_ev[i];
      const uint32_t want = (ca.epoch + 1u) * (uint32_t)t.wait_thr[i];
      uint32_t seen = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int32_t)(seen - want) < 0) {
        const uint64_t t0 = wall_clock64();
        for (;;) {
          __builtin_amdgcn_s_sleep(1);
          seen = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int32_t)(seen - want) >= 0) break;
          if (error_set(d)) { ok = 0; break; }
          if ((int64_t)(wall_clock64() - t0) > d.spin_budget) {
            set_error(d, DEVERR_TIMEOUT, t.gidx, t.wait_ev[i], seen, want);
            ok = 0;
            break;
          }
        }
      }
    }
    sm.imisc[0] = ok;
  }
  __syncthreads();
  const bool ok = sm.imisc[0] != 0;
  if (ok) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= t.n_wait) break;
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
  if (d.trace && tidx() == 0) {
    uint32_t *tr = d.trace + (size_t)t.gidx * 6;
    if (d.trace_mode == 1) stg(tr + 0, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
    atomicAdd(&tr[2], 1u);
    stg(tr + 3, (uint32_t)blockIdx.x);
    stg(tr + 4, (uint32_t)wall_clock64());
  }
}
DEV void trace_finish(CP &d, const TD &t) {
  if (d.trace && tidx() == 0) {
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
  if (tidx() == 0 && count > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (i < t.n_sig)
        __hip_atomic_fetch_add(d.ev + t.sig_ev[i], (uint32_t)count, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  }
}
DEV void signal_done(CP &d, const TD &t) { signal_count(d, t, t.a5); }

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

// Address of lane's 16 bytes of chunk j of compute wave cw in tile g; slots
// beyond the wave's chunks read the tile's first chunk instead (always
// inside the tile), so every slot is written by a load.  Unconditional loads
// keep each slot in one register across tiles: a slot that a branch might
// leave unchanged would be copied between registers, which forces a wait for
// every load in flight.
DEV uint64_t slot_addr(const Geo &g, int cw, int j) {
  const uint32_t lane16 = (uint32_t)(tidx() & 63) * 16u;
  const uint32_t o = (uint32_t)(cw * g.cpw + j) * 1024u + lane16;
  const uint64_t b0 = (uint64_t)g.seg0, b1 = (uint64_t)g.seg1 - g.seg_bytes;
  const uint64_t a = (o < g.seg_bytes ? b0 : b1) + o;
  return j < cw_chunks(g, cw) ? a : b0 + lane16;
}

// Issue the loads of compute wave cw's chunks of a tile into w.
DEV void load_slots(const Geo &g, Buf &w, int cw) {
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) w[j] = ldnt((const u32x4 *)slot_addr(g, cw, j));
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
// of one slot into part[4*chunk + DPP row].  When `pre`, each slot is
// refilled with the next tile `gn` as soon as it has been used, so the next
// tile streams in while this one is consumed.  The body is straight-line
// code (uniform branches only), which lets the compiler wait for each slot
// with "all but the newest loads done" instead of draining the queue.
DEV void gemv_dot1(const Geo &g, Buf &w, const float *xs, float *part, int cw, bool pre,
                   const Geo &gn) {
  const int lane = tidx() & 63;
  const int cnt = cw_chunks(g, cw);
  const int q0 = cw * g.cpw;
  int col = (int)(((uint32_t)q0 * 512u + (uint32_t)lane * 8u) % (uint32_t)g.K);
  float *pp = part + q0 * 4 + (lane >> 4);
  const bool writer = (lane & 15) == 0;
  // without a next tile the slots re-read this tile's first chunk
  const Geo &gr = pre ? gn : g;
  const int crw = pre ? cw : 0;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    if (j < cnt) {
      const float v = row16_sum(dot8(w[j], xs + col));
      if (writer) pp[j * 4] = v;
      col += g.step;
      col = col >= g.K ? col - g.K : col;
    }
    w[j] = ldnt((const u32x4 *)(pre ? slot_addr(gr, crw, j) : slot_addr(g, 0, kMaxChunks)));
    __builtin_amdgcn_sched_barrier(0);  // keep each refill right after its use
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

DEV bool is_gemv(int op) {
  return op == OP_QKV || op == OP_OPROJ || op == OP_GATEUP || op == OP_DOWN ||
         op == OP_ROUTER || op == OP_LMHEAD || op == OP_EGATEUP || op == OP_EDOWN;
}
// weights known before the task's inputs are (prefetchable)
DEV bool static_weights(int op) { return is_gemv(op) && op != OP_EGATEUP && op != OP_EDOWN; }
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

// Expert tiles: the expert the router chose for (slot, expert slot).
// Returns false (and flags an error) for an out-of-range id.
DEV bool expert_geo(CP &d, const TD &t, Geo &g) {
  const int e = uni(ldai(d.tk_ids + ((size_t)t.layer * d.B + t.a0) * d.topk + t.a3));
  if (e < 0 || e >= d.E) {
    if (tidx() == 0) set_error(d, DEVERR_BAD_INPUT, t.gidx, -1, (uint32_t)e, (uint32_t)d.E);
    return false;
  }
  const size_t le = (size_t)t.layer * d.E + e;
  if (t.op == OP_EGATEUP)
    g = make_geo(tab(d.e_gate, le) + (size_t)t.a1 * d.H, tab(d.e_up, le) + (size_t)t.a1 * d.H,
                 t.a2, 2, d.H);
  else
    g = make_geo(tab(d.e_down, le) + (size_t)t.a1 * d.Fe, nullptr, t.a2, 1, d.Fe);
  return true;
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
    float *dst = t.dst + (size_t)(b0 + bi) * os + i;
    switch (op) {
      case OP_OPROJ: case OP_DOWN:  // residual add (first pass: preloaded)
        sta(dst, (idx < 64 ? aux0 : lda(t.aux + (size_t)(b0 + bi) * os + i)) + y);
        break;
      case OP_GATEUP: case OP_EGATEUP:  // SwiGLU of the gate and up rows
        sta(dst, silu(y) * at(bi, i, 1));
        break;
      default:  // QKV, ROUTER, EDOWN
        sta(dst, y);
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
  Geo g;        // the first pass (static weights) or the expert tile
  int nb, bfirst, P, rpp, bb_max;
  bool skip;    // expert task of an empty slot or rejected expert: no work
};

// B1: compiled for plans with one slot (no slot chunks).
template <bool B1>
DEV GemvShape2 gemv_shape(CP &d, const CallArgs &ca, const TD &t) {
  GemvShape2 q;
  q.skip = false;
  q.P = 1;
  q.rpp = t.a2;
  if (!static_weights(t.op)) {
    q.nb = 1;
    q.bfirst = t.a0;
    q.skip = ldg(ca.positions + t.a0) < 0 || !expert_geo(d, t, q.g);
  } else {
    q.nb = B1 ? 1 : d.B;
    q.bfirst = 0;
    q.g = static_geo(t);
    q.P = n_passes(t);
    q.rpp = task_rpp(t.rpp, t.a2);
  }
  q.bb_max = B1 ? 1 : min(kMaxBatchGemv, kLdsXBytes / (q.g.K * 4));
  return q;
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
  trace_start(d, t);
  const GemvShape2 q = gemv_shape<B1>(d, ca, t);
  if (q.skip) {
    if (persistent) {
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
    stage_x(sm, ws, t.src + (size_t)b0 * K, K, n, t.gain, d.eps);
    trace_mark(d, t, 0);
    // the residual of the first outputs, loaded while the compute waves work
    float aux0 = 0.f;
    if ((t.op == OP_OPROJ || t.op == OP_DOWN) && lane < n * t.a2) {
      const int bi = lane / t.a2, i = lane - bi * t.a2;
      aux0 = lda(t.aux + (size_t)(b0 + bi) * t.ostride + i);
    }
    __syncthreads();  // partials complete
    __syncthreads();  // row sums complete
    trace_mark(d, t, 1);
    gemv_epilogue(d, ca, t, &sm.rows[0][0], q.bfirst, b0, n, aux0, q.rpp);
    if (n < q.nb) {
      ws.x_src = nullptr;
      __syncthreads();  // the next slot chunk restages xs and reuses the buffers
    }
  }
  if (persistent) {
    // The epilogue's stores are all this wave's: drain them only where the
    // run's completions are reported (the wait covers the earlier tasks too).
    if (t.a5 > 0) vm_drain();
    trace_finish(d, t);  // before the signal: consumers start after it
    signal_done(d, t);
  }
  return true;
}

// Compute waves: stream the task's passes through `w` (holding the first
// pass when w_loaded), refilling each slot right after its use with the next
// pass, and after the last pass with the first pass of the next task `gn`
// when `pre`; then the row sums.
template <bool B1>
DEV bool gemv_cmp(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws, Buf &w, bool w_loaded, bool pre, const Geo &gn) {
  const int cw = uni(tidx() >> 6) - 1;
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  const GemvShape2 q = gemv_shape<B1>(d, ca, t);
  if (q.skip) return true;
  if (!w_loaded) load_slots(q.g, w, cw);
  if (!gemv_fits(d, t, q)) return false;
  const int K = q.g.K;
  auto geo_of = [&](int p) { return p == 0 ? q.g : pass_geo(t.w0, t.w1, t.a2, t.rpp, K, p); };
  float *red = &sm.red[0][0];
  float *rsum = &sm.rows[0][0];
  for (int b0 = 0; b0 < q.nb; b0 += q.bb_max) {
    const int n = min(q.bb_max, q.nb - b0);
    const bool last = b0 + n >= q.nb;
    if (n < q.nb) ws.x_src = nullptr;
    stage_x(sm, ws, t.src + (size_t)b0 * K, K, n, t.gain, d.eps);
    // The first pass was loaded before the task; waiting for all of it here
    // lets the pass loop wait per slot for the loads it issues itself.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int p = 0; p < q.P; ++p) {
      const Geo gp = geo_of(p);
      const bool lastp = p + 1 == q.P;
      const Geo gq = lastp ? gn : geo_of(p + 1);
      const bool pre_p = lastp ? (pre && last) : true;
      if (B1 || n == 1) {
        gemv_dot1(gp, w, sm.xs, red + p * kPartSlot, cw, pre_p, gq);
      } else {
        gemv_dotn(gp, w, sm.xs, n, red + p * n * kPartSlot, cw);
        if (pre_p) load_slots(gq, w, cw);
      }
    }
    __syncthreads();  // partials complete
    gemv_rows(K, q.P, [&](int p) { return geo_of(p).units * 512 / K; }, red, rsum, n, cw);
    __syncthreads();  // row sums complete
    if (n < q.nb) {
      ws.x_src = nullptr;
      __syncthreads();
    }
  }
  return true;
}

// -------------------------------------------------------------- attention --
// One (slot, KV head, split) task: the query heads of the group attend to
// the cached keys of positions [lo, min(hi, pos)) of the split, read page by
// page (16 positions) from the paged pools; the split that contains the
// current position also rotates and stores the new key/value (bf16) and
// attends to it.  Softmax runs online in base 2 on log2(e)/sqrt(hd)-scaled
// scores; the task leaves (max, sum, weighted values) for the merge, or the
// normalised output when there is a single split.  The cached pages do not
// depend on this step's projections: each wave loads its first page before
// the task waits for the query/key/value tiles of its group.
// Returns false when the step is drained after an error.
template <int HD>
DEV bool run_attn(Smem &sm, CP &d, const CallArgs &ca, const TD &t, bool persistent,
                  WState &ws) {
  const int tix = t.gidx;
  const int l = t.layer, b = t.a0, g = t.a1, sp = t.a2;
  const int G = d.G, S = d.S, B = d.B, nkv = d.nkv, nq = d.nq;
  const int tid = tidx(), lane = tid & 63, wave = uni(tid >> 6);
  constexpr int PS = HD + 4;
  float *qs = sm.xs;                         // [G][HD]
  float *kc = qs + kMaxGroup * HD;           // [HD]
  float *vc = kc + HD;                       // [HD]
  float *wm = vc + HD;                       // [kWaves][kMaxGroup]
  float *wl = wm + kWaves * kMaxGroup;       // [kWaves][kMaxGroup]
  float *wo = wl + kWaves * kMaxGroup;       // [kWaves][kMaxGroup][HD]
  float *scur = wo + kWaves * kMaxGroup * HD;

  const int pos = uni(ldg(ca.positions + b));
  const size_t head0 = ((size_t)l * B + b) * nq + (size_t)g * G;  // first head row
  constexpr int DQ = HD / 4;                  // key dims per lane
  constexpr int KV4 = DQ / 8;                 // 16-byte loads per lane
  constexpr int VPOS = HD == 128 ? 16 : 8;    // value rows per lane
  const int tq = lane >> 2, qd = lane & 3;
  const int vdim = HD == 128 ? 2 * lane : 2 * (lane & 31);
  const bool pos_ok = pos >= 0 && pos < d.max_pos;
  const int n = pos + 1;
  const int lo = pos_ok ? (int)((int64_t)sp * n / S) : 0;
  const int hi = pos_ok ? (int)((int64_t)(sp + 1) * n / S) : 0;
  const int chi = hi < pos ? hi : pos;  // cached keys [lo, chi)
  const int blk0 = lo / kPageSize, blk1 = chi > lo ? (chi - 1) / kPageSize : -1;
  // prefetch of this wave's first page
  u32x4 kr[KV4];
  uint32_t vr[VPOS];
  int pg_first = -1;
  if (blk0 + wave <= blk1) {
    pg_first = uni(ldg(d.page_table + (size_t)b * d.maxp + blk0 + wave));
    if (pg_first >= 0 && pg_first < d.npages) {
      const size_t pbase = (((size_t)l * d.npages + pg_first) * nkv + g) * kPageSize * HD;
#pragma unroll
      for (int i = 0; i < KV4; ++i)
        kr[i] = ldg((const u32x4 *)(d.k_pool + pbase + tq * HD + qd * DQ + i * 8));
#pragma unroll
      for (int i = 0; i < VPOS; ++i) {
        const int tt = HD == 128 ? i : 2 * i + (lane >> 5);
        vr[i] = ldg((const uint32_t *)(d.v_pool + pbase + tt * HD + vdim));
      }
    }
  }
  if (persistent && !wait_deps(sm, d, ca, t, ws)) return false;
  trace_start(d, t);
  if (!pos_ok) {
    if (pos >= d.max_pos && tid == 0)
      set_error(d, DEVERR_BAD_INPUT, tix, -1, (uint32_t)pos, (uint32_t)d.max_pos);
    for (int idx = tid; idx < G * HD; idx += kThreads) {
      const int h = idx / HD, dd = idx - h * HD;
      if (S == 1) {
        sta(d.attn + (head0 + h) * HD + dd, 0.f);
      } else {
        float *pp = d.part + ((head0 + h) * S + sp) * PS;
        sta(pp + dd, 0.f);
        if (dd == 0) { sta(pp + HD, -INFINITY); sta(pp + HD + 1, 0.f); }
      }
    }
    return true;
  }
  const bool has_cur = (hi == n);
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  const float *cs = d.rope_cos + (size_t)pos * (HD / 2);
  const float *sn = d.rope_sin + (size_t)pos * (HD / 2);
  const float *qg = d.q + head0 * HD;
  for (int idx = tid; idx < G * HD; idx += kThreads) {
    const int h = idx / HD, i = idx - h * HD, i0 = i & (HD / 2 - 1);
    const float a = lda(qg + h * HD + i0), c2 = lda(qg + h * HD + i0 + HD / 2);
    const float cv = ldg(cs + i0), sv = ldg(sn + i0);
    const float r = (i < HD / 2) ? a * cv - c2 * sv : a * sv + c2 * cv;
    qs[h * HD + i] = r * scale;
  }
  if (has_cur) {
    const size_t kvo = (((size_t)l * B + b) * nkv + g) * HD;
    const int pg = uni(ldg(d.page_table + (size_t)b * d.maxp + pos / kPageSize));
    const bool pg_ok = pg >= 0 && pg < d.npages;
    if (!pg_ok && tid == 0) set_error(d, DEVERR_BAD_INPUT, tix, -2, (uint32_t)pg, (uint32_t)d.npages);
    for (int i = tid; i < HD; i += kThreads) {
      const int i0 = i & (HD / 2 - 1);
      const float a = lda(d.k + kvo + i0), c2 = lda(d.k + kvo + i0 + HD / 2);
      const float cv = ldg(cs + i0), sv = ldg(sn + i0);
      const float kr = (i < HD / 2) ? a * cv - c2 * sv : a * sv + c2 * cv;
      const uint16_t kb = f2bf(kr), vb = f2bf(lda(d.v + kvo + i));
      kc[i] = bf1(kb);
      vc[i] = bf1(vb);
      if (pg_ok) {
        const size_t off =
            ((((size_t)l * d.npages + pg) * nkv + g) * kPageSize + (pos & (kPageSize - 1))) * HD + i;
        stg(d.k_pool + off, kb);
        stg(d.v_pool + off, vb);
      }
    }
  }
  __syncthreads();

  // --- page loop: wave w takes pages blk0+w, blk0+w+kWaves, ... (the first
  // one already loaded)
  float m[kMaxGroup], ls[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) { m[h] = -INFINITY; ls[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }
  if (chi > lo) {
    for (int blk = blk0 + wave; blk <= blk1; blk += kWaves) {
      const int pg = blk == blk0 + wave ? pg_first
                                        : uni(ldg(d.page_table + (size_t)b * d.maxp + blk));
      if (pg < 0 || pg >= d.npages) {
        if (lane == 0) set_error(d, DEVERR_BAD_INPUT, tix, -2, (uint32_t)pg, (uint32_t)d.npages);
        break;
      }
      if (blk != blk0 + wave) {
        const size_t pbase = (((size_t)l * d.npages + pg) * nkv + g) * kPageSize * HD;
#pragma unroll
        for (int i = 0; i < KV4; ++i)
          kr[i] = ldg((const u32x4 *)(d.k_pool + pbase + tq * HD + qd * DQ + i * 8));
#pragma unroll
        for (int i = 0; i < VPOS; ++i) {
          const int tt = HD == 128 ? i : 2 * i + (lane >> 5);
          vr[i] = ldg((const uint32_t *)(d.v_pool + pbase + tt * HD + vdim));
        }
      }
      const int p = blk * kPageSize + tq;
      const bool valid = p >= lo && p < chi;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h >= G) break;
        const float *qh = qs + h * HD + qd * DQ;
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < KV4; ++i) {
          const f32x4 x0 = *(const f32x4 *)(qh + i * 8), x1 = *(const f32x4 *)(qh + i * 8 + 4);
          a = fmaf(bf_lo(kr[i].x), x0.x, a);
          a = fmaf(bf_hi(kr[i].x), x0.y, a);
          a = fmaf(bf_lo(kr[i].y), x0.z, a);
          a = fmaf(bf_hi(kr[i].y), x0.w, a);
          a = fmaf(bf_lo(kr[i].z), x1.x, a);
          a = fmaf(bf_hi(kr[i].z), x1.y, a);
          a = fmaf(bf_lo(kr[i].w), x1.z, a);
          a = fmaf(bf_hi(kr[i].w), x1.w, a);
        }
        a = quad_sum(a);
        const float s = valid ? a : -INFINITY;
        const float mb = quads_max(s);
        const float mn = fmaxf(m[h], mb);
        if (mn == -INFINITY) continue;
        const float alpha = exp2f(m[h] - mn);
        const float pe = exp2f(s - mn);
        const float psum = quads_sum(pe);
        ls[h] = ls[h] * alpha + psum;
        m[h] = mn;
        float a0 = o0[h] * alpha, a1 = o1[h] * alpha;
#pragma unroll
        for (int i = 0; i < VPOS; ++i) {
          float pt;
          if (HD == 128) {
            pt = lanef(pe, i * 4);
          } else {  // lanes 0-31 take even positions, 32-63 odd ones
            const float pe_even = lanef(pe, 8 * i), pe_odd = lanef(pe, 8 * i + 4);
            pt = (lane >> 5) ? pe_odd : pe_even;
          }
          a0 = fmaf(pt, bf_lo(vr[i]), a0);
          a1 = fmaf(pt, bf_hi(vr[i]), a1);
        }
        o0[h] = a0;
        o1[h] = a1;
      }
    }
  }
  // per-wave state to LDS
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) break;
    float a0 = o0[h], a1 = o1[h];
    if (HD == 64) { a0 += __shfl_xor(a0, 32, 64); a1 += __shfl_xor(a1, 32, 64); }
    if (lane == 0) { wm[wave * kMaxGroup + h] = m[h]; wl[wave * kMaxGroup + h] = ls[h]; }
    if (HD == 128 || lane < 32) {
      wo[(wave * kMaxGroup + h) * HD + vdim] = a0;
      wo[(wave * kMaxGroup + h) * HD + vdim + 1] = a1;
    }
  }
  if (has_cur && wave < G) {  // score of the current key for head `wave`
    float a = 0.f;
    for (int i = lane; i < HD; i += 64) a = fmaf(qs[wave * HD + i], kc[i], a);
    a = wave_sum(a);
    if (lane == 0) scur[wave] = a;
  }
  __syncthreads();
  // merge the waves (fixed order) and the current key
  for (int idx = tid; idx < G * HD; idx += kThreads) {
    const int h = idx / HD, dd = idx - h * HD;
    float M = -INFINITY;
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, wm[w2 * kMaxGroup + h]);
    if (has_cur) M = fmaxf(M, scur[h]);
    float Ls = 0.f, Os = 0.f;
    if (M != -INFINITY) {
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float mw = wm[w2 * kMaxGroup + h];
        if (mw == -INFINITY) continue;
        const float f = exp2f(mw - M);
        Ls = fmaf(f, wl[w2 * kMaxGroup + h], Ls);
        Os = fmaf(f, wo[(w2 * kMaxGroup + h) * HD + dd], Os);
      }
      if (has_cur) {
        const float f = exp2f(scur[h] - M);
        Ls += f;
        Os = fmaf(f, vc[dd], Os);
      }
    }
    if (S == 1) {
      sta(d.attn + (head0 + h) * HD + dd, Ls > 0.f ? Os / Ls : 0.f);
    } else {
      float *pp = d.part + ((head0 + h) * S + sp) * PS;
      sta(pp + dd, Os);
      if (dd == 0) { sta(pp + HD, M); sta(pp + HD + 1, Ls); }
    }
  }
  return true;
}

// Log-sum-exp merge of the S split partials (o[HD], m, l) of one (slot, KV
// head): the group's G query heads.  One round of loads: every split's
// (m, l) and each thread's output vector's partials of up to 8 splits are in
// flight together; one wave per head turns (m, l) into the weights
// 2^(m_s - M) / L in LDS; each output is the weighted sum.
DEV void run_merge(Smem &sm, CP &d, const TD &t) {
  const int l = t.layer, b = t.a0, g = t.a1, G = d.G, S = d.S, HD = d.hd;
  const int PS = HD + 4, hv = HD / 4, nvec = G * hv, npairs = G * S, s8 = min(S, 8);
  const int tid = tidx(), lane = tid & 63, wave = uni(tid >> 6);
  const size_t head0 = ((size_t)l * d.B + b) * d.nq + (size_t)g * G;
  const float *part0 = d.part + head0 * S * PS;
  const __amdgpu_buffer_rsrc_t r = rsrc(part0);
  auto vec_at = [&](int h, int sp, int dd) {
    return lda4(r, (uint32_t)((((size_t)h * S + sp) * PS + dd) * 4));
  };
  const int h = tid / hv, dd = (tid - h * hv) * 4;
  f32x4 ov[8];
#pragma unroll
  for (int sp = 0; sp < 8; ++sp)
    ov[sp] = (tid < nvec && sp < s8) ? vec_at(h, sp, dd) : (f32x4){0.f, 0.f, 0.f, 0.f};
  float2 *ml = (float2 *)&sm.red[0][0];  // [G * S]: (m, l), then (weight, -)
  for (int i = tid; i < npairs; i += kThreads) {
    const float *pp = part0 + (size_t)i * PS + HD;  // pair i = head * S + split
    ml[i] = make_float2(lda(pp), lda(pp + 1));
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
  for (int v = tid; v < nvec; v += kThreads) {
    const int hh = v / hv, d0 = (v - hh * hv) * 4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (v == tid) {
#pragma unroll
      for (int sp = 0; sp < 8; ++sp)
        if (sp < s8) o += ml[hh * S + sp].x * ov[sp];
    }
    for (int sp = v == tid ? s8 : 0; sp < S; ++sp) o += ml[hh * S + sp].x * vec_at(hh, sp, d0);
    float *dst = d.attn + (head0 + hh) * HD + d0;
    sta(dst + 0, o.x);
    sta(dst + 1, o.y);
    sta(dst + 2, o.z);
    sta(dst + 3, o.w);
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
  float *x = d.x + (size_t)b * H;
  const uint16_t *e = d.embed + (size_t)(ok ? tok : 0) * H;
  for (int i = tidx(); i < H; i += kThreads) sta(x + i, ok ? bf1(ldg(e + i)) : 0.f);
}

// Softmax router top-k: k rounds of (max, lowest index) over the logits not
// yet taken; weights = softmax over the chosen logits; ids ascending.
DEV void run_topk(Smem &sm, CP &d, const TD &t) {
  const int l = t.layer, b = t.a0, E = d.E, K = d.topk;
  const int tid = tidx(), lane = tid & 63, wave = tid >> 6;
  const float *r = d.rl + ((size_t)l * d.B + b) * E;
  float *vals = sm.xs;
  int *taken = (int *)(sm.xs + kThreads);
  int *ids = sm.imisc + 8;            // [16]
  float *lg = sm.misc + 32;           // [16]
  for (int i = tid; i < E; i += kThreads) { vals[i] = lda(r + i); taken[i] = 0; }
  __syncthreads();
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = tid; i < E; i += kThreads)
      if (!taken[i] && better(vals[i], i, bv, bi)) { bv = vals[i]; bi = i; }
    wave_argmax(bv, bi);
    if (lane == 0) { sm.misc[wave] = bv; sm.imisc[32 + wave] = bi; }
    __syncthreads();
    if (tid == 0) {
      float cv = sm.misc[0];
      int ci = sm.imisc[32];
      for (int w2 = 1; w2 < kWaves; ++w2)
        if (better(sm.misc[w2], sm.imisc[32 + w2], cv, ci)) { cv = sm.misc[w2]; ci = sm.imisc[32 + w2]; }
      if (ci < 0 || ci >= E) ci = 0;  // all NaN: keep indices valid
      ids[j] = ci;
      lg[j] = vals[ci];
      taken[ci] = 1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    for (int a = 1; a < K; ++a)  // insertion sort by expert id
      for (int c = a; c > 0 && ids[c - 1] > ids[c]; --c) {
        const int ti = ids[c]; ids[c] = ids[c - 1]; ids[c - 1] = ti;
        const float tv = lg[c]; lg[c] = lg[c - 1]; lg[c - 1] = tv;
      }
    float mx = lg[0];
    for (int j = 1; j < K; ++j) mx = fmaxf(mx, lg[j]);
    float wsum = 0.f;
    for (int j = 0; j < K; ++j) { sm.misc[48 + j] = expf(lg[j] - mx); wsum += sm.misc[48 + j]; }
    const size_t o = ((size_t)l * d.B + b) * K;
    for (int j = 0; j < K; ++j) {
      stai(d.tk_ids + o + j, ids[j]);
      sta(d.tk_w + o + j, sm.misc[48 + j] / wsum);
    }
  }
}

DEV void run_combine(CP &d, const CallArgs &ca, const TD &t) {
  const int l = t.layer, b = t.a0, H = d.H, K = d.topk, B = d.B;
  const bool active = ldg(ca.positions + b) >= 0;
  const size_t xo = ((size_t)l * B + b) * H;
  const float *w = d.tk_w + ((size_t)l * B + b) * K;
  const float *y = d.ye + ((size_t)l * B + b) * K * H;
  const int r0 = t.a1, r1 = t.a1 + t.a2;
  for (int i = r0 + tidx(); i < r1; i += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < K; ++j) acc = fmaf(lda(w + j), lda(y + (size_t)j * H + i), acc);
    sta(d.x + xo + (size_t)B * H + i, active ? lda(d.xmid + xo + i) + acc : 0.f);
  }
}

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
    case OP_EMBED: run_embed(d, ca, t); break;
    case OP_TOPK: run_topk(sm, d, t); break;
    case OP_COMBINE: run_combine(d, ca, t); break;
    case OP_ARGMAX: run_argmax(sm, d, ca, t); break;
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
          d.att_cnt + ((size_t)t.layer * d.B + t.a0) * d.nkv + t.a1, 1u, __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT);
      sm.imisc[1] = old == (ca.epoch + 1u) * (uint32_t)d.S - 1u;
    }
    __syncthreads();
    const bool last = sm.imisc[1] != 0;
    if (last) {
      run_merge(sm, d, t);
      vm_drain();
    }
    __syncthreads();
    if (persistent) signal_count(d, t, last ? 1 : 0);
    return true;
  }
  if (persistent) vm_drain();
  __syncthreads();
  if (persistent) {
    trace_finish(d, t);
    signal_done(d, t);
  }
  return true;
}

// Run task t; `w` holds its weights when w_loaded.  When the worker's next
// task has static weights (pre), their tile geometry is gn and this task
// leaves them loading into `w`.  Returns whether it did; `alive` turns false
// when the step is drained after an error.  Uniform across waves.
// One task of the kernel-per-op executor (all waves of one workgroup).
DEV void run_task_once(Smem &sm, CP &d, const CallArgs &ca, const TD &t, WState &ws) {
  if (!is_gemv(t.op)) {
    run_small(sm, d, ca, t, false, ws);
  } else if (uni(tidx() >> 6) == 0) {
    gemv_ctl<false>(sm, d, ca, t, false, ws);
  } else {
    Buf w;
    Geo gn;
    gemv_cmp<false>(sm, d, ca, t, false, ws, w, false, false, gn);
  }
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
template <bool B1>
__global__ void __launch_bounds__(kThreads)
    mk_persistent_kernel(const DevPlan *__restrict__ dplan, CallArgs ca) {
  __shared__ Smem sm;
  CP &d = *(CP *)dplan;
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
      const bool alive = is_gemv(t.op) ? gemv_ctl<B1>(sm, d, ca, t, true, ws)
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
    if (static_weights(t.op)) {
      Buf w;
      load_slots(static_geo(t), w, cw);
      for (;;) {
        Geo gn;
        const bool pre = k + 1 < end && next_geo(sm.ring[(k + 1 - beg) % kRing], gn);
        if (!gemv_cmp<B1>(sm, d, ca, t, true, ws, w, true, pre, gn)) return;
        refill(k);
        ++k;
        if (!pre) break;
        t = td_from_ring(sm.ring[(k - beg) % kRing]);
      }
    } else {
      bool alive;
      if (is_gemv(t.op)) {
        Buf w;
        Geo gn;
        alive = gemv_cmp<B1>(sm, d, ca, t, true, ws, w, false, false, gn);
      } else {
        alive = run_small(sm, d, ca, t, true, ws);
      }
      if (!alive) return;
      refill(k);
      ++k;
    }
  }
}

__global__ void __launch_bounds__(kThreads)
    mk_phase_kernel(const DevPlan *__restrict__ dplan, CallArgs ca, int first) {
  __shared__ Smem sm;
  CP &d = *(CP *)dplan;
  const int pos = ((const AS4 int *)d.task_pos)[first + (int)blockIdx.x];
  const TD t = td_from_table(d.tasks, pos);
  WState ws;
  init_ws(ws);
  run_task_once(sm, d, ca, t, ws);
}

__global__ void mk_stage_kernel(int32_t *tok, int32_t *pos, int B, int slot,
                                const int32_t *tokens, int i, int start) {
  const int b = threadIdx.x + blockIdx.x * blockDim.x;
  if (b >= B) return;
  tok[b] = b == slot ? tokens[i] : 0;
  pos[b] = b == slot ? start + i : -1;
}

__global__ void mk_zero_kernel(uint32_t *p, int n) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------- launch --
// All workers must be resident at once (each may wait on any other), which a
// cooperative launch guarantees or refuses.
hipError_t launch_persistent(const DevPlan *d, const CallArgs &ca, int grid, int batch,
                             hipStream_t s) {
  void *args[] = {(void *)&d, (void *)&ca};
  const void *k = batch == 1 ? (const void *)mk_persistent_kernel<true>
                             : (const void *)mk_persistent_kernel<false>;
  return hipLaunchCooperativeKernel(k, dim3(grid), dim3(kThreads),
                                    args, 0, s);
}

hipError_t launch_phase(const DevPlan *d, const CallArgs &ca, int first, int count,
                        hipStream_t s) {
  hipLaunchKernelGGL(mk_phase_kernel, dim3(count), dim3(kThreads), 0, s, d, ca, first);
  return hipGetLastError();
}

hipError_t launch_stage(int32_t *stage_tok, int32_t *stage_pos, int B, int slot,
                        const int32_t *tokens, int i, int start, hipStream_t s) {
  hipLaunchKernelGGL(mk_stage_kernel, dim3((B + 255) / 256), dim3(256), 0, s, stage_tok,
                     stage_pos, B, slot, tokens, i, start);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

int persistent_lds_bytes() { return (int)sizeof(Smem); }

}  // namespace mk
