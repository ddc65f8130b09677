// kernels.hip -- device code of the decode-step megakernel for gfx950.
//
// The persistent kernel follows the Cohere megakernel article ("Egyetlen
// tartós kernelre épül a kiszolgálás"): exactly one workgroup per CU stays
// resident for the whole step and works from the host-prepared task list;
// dependencies are counters in global memory.  The worker loop is the one the
// Mirage MPK summary describes ("Part 2. Runtime", Worker): take the next
// task, run it, notify its event, repeat.  Tasks are taken from one atomic
// ticket counter in list order, which the planner makes a topological order,
// so the lowest unfinished ticket always has its inputs ready and the loop is
// deadlock-free even without co-residency guarantees.
//
// Before a task waits for its producers it already issues the loads of its
// own weight tile (weights never change, so they may be read early): the
// Cohere article's weight prefetch ("Honnan jön a gyorsulás?").
//
// Memory ordering: a producer's outputs are made visible with an agent-scope
// release fence before its counter increment; a consumer polls the counter
// with relaxed loads and then issues an agent-scope acquire fence (on the
// multi-XCD MI355X this writes back / invalidates the per-XCD L2 as needed).
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
DEV int vec_bytes(int K) { return ((K * 2) % 1024 == 0) ? 16 : 8; }

struct Smem {
  float xs[kLdsXBytes / 4];                                // staged activations
  float red[kMaxBatchGemv][kWaves][2 * kMaxChunks + 1];    // GEMV partial sums
  float ybuf[kMaxBatchGemv][256];                          // LM-head tile rows
  float misc[64];
  int imisc[64];
};

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
// Thread 0 polls each counter until it reaches (epoch+1)*threshold, then
// issues one acquire fence; the barrier hands the result to the workgroup.
// Returns false when the step is being drained after an error.
DEV bool wait_deps(Smem &sm, CP &d, const CallArgs &ca, CT &t, int tix) {
  if (threadIdx.x == 0) {
    int ok = 1;
    for (int i = 0; i < t.n_wait && ok; ++i) {
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
            set_error(d, DEVERR_TIMEOUT, tix, t.wait_ev[i], seen, want);
            ok = 0;
            break;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (ok && d.trace) {
      uint32_t *tr = d.trace + (size_t)tix * 6;
      stg(tr + 0, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
      atomicAdd(&tr[2], 1u);
      stg(tr + 3, (uint32_t)blockIdx.x);
      stg(tr + 4, (uint32_t)wall_clock64());
    }
    sm.imisc[0] = ok;
  }
  __syncthreads();
  return sm.imisc[0] != 0;
}

// All threads' outputs are complete after the barrier; thread 0 releases
// them at agent scope and bumps the task's counters.
DEV void signal_done(CP &d, CT &t, int tix) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (d.trace) {
      uint32_t *tr = d.trace + (size_t)tix * 6;
      stg(tr + 1, atomicAdd(&d.ctrl[CTRL_CLOCK], 1u));
      stg(tr + 5, (uint32_t)wall_clock64());
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int i = 0; i < t.n_sig; ++i)
      __hip_atomic_fetch_add(d.ev + t.sig_ev[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ GEMV tiles --
// A tile is `nseg` blocks of `seg_rows` consecutive rows (row length K bf16)
// cut at the same row offset (gate and up share a tile).  Its bytes are
// streamed as wave-chunks: 64 lanes x one VW-byte load, contiguous in memory
// (rows are a whole number of wave-chunks).  Wave w owns chunks
// [w*cpw, (w+1)*cpw); every lane keeps its loads in registers (the prefetch),
// multiplies them with the activations staged in LDS, and each wave reduces
// the partial dot product of each row it touched; rows are then summed over
// the waves that share them in fixed wave order (deterministic).
template <int VW> struct VT;
template <> struct VT<16> { typedef u32x4 T; static constexpr int N = kMaxChunks; };
template <> struct VT<8> { typedef u32x2 T; static constexpr int N = 2 * kMaxChunks; };

struct Geo {
  const uint16_t *seg0, *seg1;
  int seg_rows, K, wc, units, cpw;
};

DEV Geo make_geo(const uint16_t *s0, const uint16_t *s1, int seg_rows, int nseg, int K, int vw) {
  Geo g;
  g.seg0 = s0;
  g.seg1 = s1;
  g.seg_rows = seg_rows;
  g.K = K;
  g.wc = (K * 2) / (64 * vw);
  g.units = nseg * seg_rows * g.wc;
  g.cpw = (g.units + kWaves - 1) / kWaves;
  return g;
}

template <int VW>
DEV void gemv_load(const Geo &g, typename VT<VW>::T *w) {
  constexpr int N = VT<VW>::N;
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int u0 = wave * g.cpw;
  const int cnt = min(g.cpw, g.units - u0);
  int r = u0 / g.wc, c = u0 - r * g.wc;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (j < cnt) {
      const bool s1 = r >= g.seg_rows;
      const uint16_t *base = s1 ? g.seg1 : g.seg0;
      const int rr = s1 ? r - g.seg_rows : r;
      const uint16_t *p = base + (size_t)rr * g.K + c * (32 * VW) + lane * (VW / 2);
      w[j] = ldnt((const typename VT<VW>::T *)p);
    }
    if (++c == g.wc) { c = 0; ++r; }
  }
}

DEV float chunk_dot(const u32x4 &w, const float *x) {
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
DEV float chunk_dot(const u32x2 &w, const float *x) {
  const f32x4 a = *(const f32x4 *)x;
  float s = bf_lo(w.x) * a.x;
  s = fmaf(bf_hi(w.x), a.y, s);
  s = fmaf(bf_lo(w.y), a.z, s);
  s = fmaf(bf_hi(w.y), a.w, s);
  return s;
}

template <int VW>
DEV void gemv_dot(const Geo &g, const typename VT<VW>::T *w, const float *xs, float *red) {
  constexpr int N = VT<VW>::N;
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int u0 = wave * g.cpw;
  const int cnt = min(g.cpw, g.units - u0);
  int c = u0 % g.wc;
  float carry = 0.f;
  int slot = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (j < cnt) {
      carry += chunk_dot(w[j], xs + c * (32 * VW) + lane * (VW / 2));
      if (c == g.wc - 1 || j == cnt - 1) {
        const float s = wave_sum(carry);
        if (lane == 0) red[wave * (N + 1) + slot] = s;
        ++slot;
        carry = 0.f;
      }
    }
    if (++c == g.wc) c = 0;
  }
}

template <int VW>
DEV float gemv_row(const Geo &g, const float *red, int row) {
  constexpr int N = VT<VW>::N;
  const int uf = row * g.wc, ul = uf + g.wc - 1;
  const int w0 = uf / g.cpw, w1 = ul / g.cpw;
  float s = 0.f;
  for (int w = w0; w <= w1; ++w) s += red[w * (N + 1) + (row - (w * g.cpw) / g.wc)];
  return s;
}

// Copy nb activation rows src[b*stride + 0..K) into LDS; with a gain vector,
// RMS-normalise each row: x / sqrt(mean(x^2) + eps) * gain.
DEV void stage_x(Smem &sm, const float *src, size_t stride, int K, int nb, const uint16_t *gain,
                 float eps) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = 0; b < nb; ++b) {
    const f32x4 *s4 = (const f32x4 *)(src + (size_t)b * stride);
    f32x4 *d4 = (f32x4 *)(sm.xs + (size_t)b * K);
    float ss = 0.f;
    for (int i = tid; i < K / 4; i += kThreads) {
      const f32x4 v = ldg(s4 + i);
      d4[i] = v;
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
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
      float *xb = sm.xs + (size_t)b * K;
      for (int i = tid; i < K; i += kThreads) xb[i] = xb[i] * rs * bf1(ldg(gain + i));
    }
    __syncthreads();
  }
}

// One GEMV task: resolve the tile, prefetch its weights, wait, stage the
// input, multiply, reduce, run the operation's epilogue, signal.
template <int VW>
DEV void run_gemv(Smem &sm, CP &d, const CallArgs &ca, CT &t, int tix, bool persistent) {
  constexpr int N = VT<VW>::N;
  typename VT<VW>::T w[N];
  const int op = t.op, l = t.layer, B = d.B, H = d.H;
  const int a0 = t.a0, a1 = t.a1, seg_rows = t.a2, a3 = t.a3, a4 = t.a4;
  const int QD = d.nq * d.hd;
  const uint16_t *s0 = nullptr, *s1 = nullptr;
  int nseg = 1, K = H, nb = B, bfirst = 0;
  const float *src = nullptr;
  const uint16_t *gain = nullptr;
  const bool expert = (op == OP_EGATEUP || op == OP_EDOWN);

  if (!expert) {
    switch (op) {
      case OP_QKV: {
        const uint16_t *W = a0 == 0 ? tab(d.wq, l) : (a0 == 1 ? tab(d.wk, l) : tab(d.wv, l));
        s0 = W + (size_t)a1 * H;
        src = d.x + (size_t)l * B * H;
        gain = tab(d.attn_norm, l);
        break;
      }
      case OP_OPROJ:
        K = QD;
        s0 = tab(d.wo, l) + (size_t)a1 * K;
        src = d.attn + (size_t)l * B * K;
        break;
      case OP_GATEUP:
        s0 = tab(d.w_gate, l) + (size_t)a1 * H;
        s1 = tab(d.w_up, l) + (size_t)a1 * H;
        nseg = 2;
        src = d.xmid + (size_t)l * B * H;
        gain = tab(d.ffn_norm, l);
        break;
      case OP_DOWN:
        K = d.F;
        s0 = tab(d.w_down, l) + (size_t)a1 * K;
        src = d.h + (size_t)l * B * K;
        break;
      case OP_ROUTER:
        s0 = tab(d.router, l) + (size_t)a1 * H;
        src = d.xmid + (size_t)l * B * H;
        gain = tab(d.ffn_norm, l);
        break;
      default:  // OP_LMHEAD
        s0 = d.lm_head + (size_t)a1 * H;
        src = d.x + (size_t)d.L * B * H;
        gain = d.final_norm;
        break;
    }
    const Geo g0 = make_geo(s0, s1, seg_rows, nseg, K, VW);
    gemv_load<VW>(g0, w);  // weight prefetch: before the dependency wait
    if (persistent && !wait_deps(sm, d, ca, t, tix)) return;
  } else {
    if (persistent && !wait_deps(sm, d, ca, t, tix)) return;
    bfirst = a0;
    nb = 1;
    const int pos = ldg(ca.positions + bfirst);
    if (pos < 0) {  // empty slot: nothing to compute
      if (persistent) signal_done(d, t, tix);
      return;
    }
    const int e = uni(ldg(d.tk_ids + ((size_t)l * B + bfirst) * d.topk + a3));
    if (e < 0 || e >= d.E) {
      if (threadIdx.x == 0) set_error(d, DEVERR_BAD_INPUT, tix, -1, (uint32_t)e, (uint32_t)d.E);
      if (persistent) signal_done(d, t, tix);
      return;
    }
    const size_t le = (size_t)l * d.E + e;
    if (op == OP_EGATEUP) {
      s0 = tab(d.e_gate, le) + (size_t)a1 * H;
      s1 = tab(d.e_up, le) + (size_t)a1 * H;
      nseg = 2;
      src = d.xmid + ((size_t)l * B + bfirst) * H;
      gain = tab(d.ffn_norm, l);
    } else {
      K = d.Fe;
      s0 = tab(d.e_down, le) + (size_t)a1 * K;
      src = d.he + (((size_t)l * B + bfirst) * d.topk + a3) * K;
    }
    const Geo g0 = make_geo(s0, s1, seg_rows, nseg, K, VW);
    gemv_load<VW>(g0, w);
  }

  const Geo g = make_geo(s0, s1, seg_rows, nseg, K, VW);
  const int bb_max = min(kMaxBatchGemv, kLdsXBytes / (K * 4));
  const int tid = threadIdx.x;
  for (int b0 = 0; b0 < nb; b0 += bb_max) {
    const int n = min(bb_max, nb - b0);
    stage_x(sm, src + (size_t)b0 * K, K, K, n, gain, d.eps);
    for (int bi = 0; bi < n; ++bi) gemv_dot<VW>(g, w, sm.xs + (size_t)bi * K, &sm.red[bi][0][0]);
    __syncthreads();
    for (int idx = tid; idx < n * seg_rows; idx += kThreads) {
      const int bi = idx / seg_rows, i = idx - bi * seg_rows;
      const int b = bfirst + b0 + bi;
      const float *red = &sm.red[bi][0][0];
      const float y = gemv_row<VW>(g, red, i);
      const int r = a1 + i;
      switch (op) {
        case OP_QKV: {
          const int Nm = a0 == 0 ? QD : d.nkv * d.hd;
          float *dst = a0 == 0 ? d.q : (a0 == 1 ? d.k : d.v);
          stg(dst + ((size_t)l * B + b) * Nm + r, y);
          break;
        }
        case OP_OPROJ: {
          const size_t o = ((size_t)l * B + b) * H + r;
          stg(d.xmid + o, ldg(d.x + o) + y);
          break;
        }
        case OP_GATEUP: {
          const float u = gemv_row<VW>(g, red, seg_rows + i);
          stg(d.h + ((size_t)l * B + b) * d.F + r, silu(y) * u);
          break;
        }
        case OP_DOWN: {
          const size_t o = ((size_t)l * B + b) * H + r;
          stg(d.x + o + (size_t)B * H, ldg(d.xmid + o) + y);
          break;
        }
        case OP_ROUTER:
          stg(d.rl + ((size_t)l * B + b) * d.E + r, y);
          break;
        case OP_EGATEUP: {
          const float u = gemv_row<VW>(g, red, seg_rows + i);
          stg(d.he + (((size_t)l * B + b) * d.topk + a3) * d.Fe + r, silu(y) * u);
          break;
        }
        case OP_EDOWN:
          stg(d.ye + (((size_t)l * B + b) * d.topk + a3) * H + r, y);
          break;
        default:  // OP_LMHEAD
          if (ca.logits) stg(ca.logits + (size_t)b * d.V + r, y);
          sm.ybuf[bi][i] = y;
          break;
      }
    }
    if (op == OP_LMHEAD) {
      __syncthreads();
      // per-slot (max, lowest index) over this tile's rows, one wave per slot
      const int wave = uni(tid >> 6), lane = tid & 63;
      if (wave < n) {
        float bv = -INFINITY;
        int bix = 0x7fffffff;
        for (int i = lane; i < seg_rows; i += 64) {
          const float v = sm.ybuf[wave][i];
          if (better(v, a1 + i, bv, bix)) { bv = v; bix = a1 + i; }
        }
        wave_argmax(bv, bix);
        if (lane == 0) {
          const size_t o = (size_t)(bfirst + b0 + wave) * d.n_lm_tiles + a4;
          stg(d.amax_v + o, bv);
          stg(d.amax_i + o, bix);
        }
      }
    }
    __syncthreads();
  }
  if (persistent) signal_done(d, t, tix);
}

// -------------------------------------------------------------- attention --
// One (slot, KV head, split) task: the query heads of the group attend to
// the cached keys of positions [lo, min(hi, pos)) of the split, read page by
// page (16 positions) from the paged pools; the split that contains the
// current position also rotates and stores the new key/value (bf16) and
// attends to it.  Softmax runs online in base 2 on log2(e)/sqrt(hd)-scaled
// scores; the task leaves (max, sum, weighted values) for the merge, or the
// normalised output when there is a single split.
template <int HD>
DEV void run_attn(Smem &sm, CP &d, const CallArgs &ca, CT &t, int tix) {
  const int l = t.layer, b = t.a0, g = t.a1, sp = t.a2;
  const int G = d.G, S = d.S, B = d.B, nkv = d.nkv, nq = d.nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
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
  if (pos < 0 || pos >= d.max_pos) {
    if (pos >= d.max_pos && tid == 0)
      set_error(d, DEVERR_BAD_INPUT, tix, -1, (uint32_t)pos, (uint32_t)d.max_pos);
    for (int idx = tid; idx < G * HD; idx += kThreads) {
      const int h = idx / HD, dd = idx - h * HD;
      if (S == 1) {
        stg(d.attn + (head0 + h) * HD + dd, 0.f);
      } else {
        float *pp = d.part + ((head0 + h) * S + sp) * PS;
        stg(pp + dd, 0.f);
        if (dd == 0) { stg(pp + HD, -INFINITY); stg(pp + HD + 1, 0.f); }
      }
    }
    return;
  }
  const int n = pos + 1;
  const int lo = (int)((int64_t)sp * n / S), hi = (int)((int64_t)(sp + 1) * n / S);
  const bool has_cur = (hi == n);
  const int chi = hi < pos ? hi : pos;  // cached keys [lo, chi)
  const float scale = 1.4426950408889634f / sqrtf((float)HD);
  const float *cs = d.rope_cos + (size_t)pos * (HD / 2);
  const float *sn = d.rope_sin + (size_t)pos * (HD / 2);
  const float *qg = d.q + head0 * HD;
  for (int idx = tid; idx < G * HD; idx += kThreads) {
    const int h = idx / HD, i = idx - h * HD, i0 = i & (HD / 2 - 1);
    const float a = ldg(qg + h * HD + i0), c2 = ldg(qg + h * HD + i0 + HD / 2);
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
      const float a = ldg(d.k + kvo + i0), c2 = ldg(d.k + kvo + i0 + HD / 2);
      const float cv = ldg(cs + i0), sv = ldg(sn + i0);
      const float kr = (i < HD / 2) ? a * cv - c2 * sv : a * sv + c2 * cv;
      const uint16_t kb = f2bf(kr), vb = f2bf(ldg(d.v + kvo + i));
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

  // --- page loop: wave w takes pages blk0+w, blk0+w+kWaves, ...
  float m[kMaxGroup], ls[kMaxGroup], o0[kMaxGroup], o1[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) { m[h] = -INFINITY; ls[h] = 0.f; o0[h] = 0.f; o1[h] = 0.f; }
  constexpr int DQ = HD / 4;                  // key dims per lane
  constexpr int KV4 = DQ / 8;                 // 16-byte loads per lane
  constexpr int VPOS = HD == 128 ? 16 : 8;    // value rows per lane
  const int tq = lane >> 2, qd = lane & 3;
  const int vdim = HD == 128 ? 2 * lane : 2 * (lane & 31);
  if (chi > lo) {
    const int blk0 = lo / kPageSize, blk1 = (chi - 1) / kPageSize;
    for (int blk = blk0 + wave; blk <= blk1; blk += kWaves) {
      const int pg = uni(ldg(d.page_table + (size_t)b * d.maxp + blk));
      if (pg < 0 || pg >= d.npages) {
        if (lane == 0) set_error(d, DEVERR_BAD_INPUT, tix, -2, (uint32_t)pg, (uint32_t)d.npages);
        break;
      }
      const size_t pbase = (((size_t)l * d.npages + pg) * nkv + g) * kPageSize * HD;
      const uint16_t *kb = d.k_pool + pbase;
      const uint16_t *vb = d.v_pool + pbase;
      u32x4 kr[KV4];
#pragma unroll
      for (int i = 0; i < KV4; ++i) kr[i] = ldg((const u32x4 *)(kb + tq * HD + qd * DQ + i * 8));
      uint32_t vr[VPOS];
#pragma unroll
      for (int i = 0; i < VPOS; ++i) {
        const int tt = HD == 128 ? i : 2 * i + (lane >> 5);
        vr[i] = ldg((const uint32_t *)(vb + tt * HD + vdim));
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
      stg(d.attn + (head0 + h) * HD + dd, Ls > 0.f ? Os / Ls : 0.f);
    } else {
      float *pp = d.part + ((head0 + h) * S + sp) * PS;
      stg(pp + dd, Os);
      if (dd == 0) { stg(pp + HD, M); stg(pp + HD + 1, Ls); }
    }
  }
}

// Log-sum-exp merge of the S split partials of one (slot, KV head).
DEV void run_merge(CP &d, CT &t) {
  const int l = t.layer, b = t.a0, g = t.a1, G = d.G, S = d.S, HD = d.hd;
  const int PS = HD + 4;
  const size_t head0 = ((size_t)l * d.B + b) * d.nq + (size_t)g * G;
  for (int idx = threadIdx.x; idx < G * HD; idx += kThreads) {
    const int h = idx / HD, dd = idx - h * HD;
    const float *pp = d.part + (head0 + h) * S * PS;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ldg(pp + s * PS + HD));
    float Ls = 0.f, Os = 0.f;
    if (M != -INFINITY)
      for (int s = 0; s < S; ++s) {
        const float ms = ldg(pp + s * PS + HD);
        if (ms == -INFINITY) continue;
        const float f = exp2f(ms - M);
        Ls = fmaf(f, ldg(pp + s * PS + HD + 1), Ls);
        Os = fmaf(f, ldg(pp + s * PS + dd), Os);
      }
    stg(d.attn + (head0 + h) * HD + dd, Ls > 0.f ? Os / Ls : 0.f);
  }
}

// ------------------------------------------------------------- small ops --
DEV void run_embed(CP &d, const CallArgs &ca, CT &t, int tix) {
  const int b = t.a0, H = d.H;
  const int pos = uni(ldg(ca.positions + b));
  const int tok = uni(ldg(ca.tokens + b));
  const bool ok = pos >= 0 && tok >= 0 && tok < d.V;
  if (pos >= 0 && !ok && threadIdx.x == 0)
    set_error(d, DEVERR_BAD_INPUT, tix, -3, (uint32_t)tok, (uint32_t)d.V);
  float *x = d.x + (size_t)b * H;
  const uint16_t *e = d.embed + (size_t)(ok ? tok : 0) * H;
  for (int i = threadIdx.x; i < H; i += kThreads) stg(x + i, ok ? bf1(ldg(e + i)) : 0.f);
}

// Softmax router top-k: k rounds of (max, lowest index) over the logits not
// yet taken; weights = softmax over the chosen logits; ids ascending.
DEV void run_topk(Smem &sm, CP &d, CT &t) {
  const int l = t.layer, b = t.a0, E = d.E, K = d.topk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *r = d.rl + ((size_t)l * d.B + b) * E;
  float *vals = sm.xs;
  int *taken = (int *)(sm.xs + kThreads);
  int *ids = sm.imisc + 8;            // [16]
  float *lg = sm.misc + 32;           // [16]
  for (int i = tid; i < E; i += kThreads) { vals[i] = ldg(r + i); taken[i] = 0; }
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
      stg(d.tk_ids + o + j, ids[j]);
      stg(d.tk_w + o + j, sm.misc[48 + j] / wsum);
    }
  }
}

DEV void run_combine(CP &d, const CallArgs &ca, CT &t) {
  const int l = t.layer, b = t.a0, H = d.H, K = d.topk, B = d.B;
  const bool active = ldg(ca.positions + b) >= 0;
  const size_t xo = ((size_t)l * B + b) * H;
  const float *w = d.tk_w + ((size_t)l * B + b) * K;
  const float *y = d.ye + ((size_t)l * B + b) * K * H;
  const int r0 = t.a1, r1 = t.a1 + t.a2;
  for (int i = r0 + threadIdx.x; i < r1; i += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < K; ++j) acc = fmaf(ldg(w + j), ldg(y + (size_t)j * H + i), acc);
    stg(d.x + xo + (size_t)B * H + i, active ? ldg(d.xmid + xo + i) + acc : 0.f);
  }
}

DEV void run_argmax(Smem &sm, CP &d, const CallArgs &ca, CT &t) {
  const int b = t.a0, nt = d.n_lm_tiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < nt; i += kThreads) {
    const float v = ldg(d.amax_v + (size_t)b * nt + i);
    const int ix = ldg(d.amax_i + (size_t)b * nt + i);
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

// ------------------------------------------------------------- dispatcher --
DEV void run_task(Smem &sm, CP &d, const CallArgs &ca, int tix, bool persistent) {
  CT &t = ((CT *)d.tasks)[tix];
  const int op = t.op;
  switch (op) {
    case OP_QKV: case OP_OPROJ: case OP_GATEUP: case OP_DOWN: case OP_ROUTER:
    case OP_LMHEAD: case OP_EGATEUP: case OP_EDOWN: {
      int K = d.H;
      if (op == OP_OPROJ) K = d.nq * d.hd;
      else if (op == OP_DOWN) K = d.F;
      else if (op == OP_EDOWN) K = d.Fe;
      if (vec_bytes(K) == 16) run_gemv<16>(sm, d, ca, t, tix, persistent);
      else run_gemv<8>(sm, d, ca, t, tix, persistent);
      return;
    }
    default: break;
  }
  if (persistent && !wait_deps(sm, d, ca, t, tix)) return;
  switch (op) {
    case OP_EMBED: run_embed(d, ca, t, tix); break;
    case OP_ATTN:
      if (d.hd == 128) run_attn<128>(sm, d, ca, t, tix);
      else run_attn<64>(sm, d, ca, t, tix);
      break;
    case OP_MERGE: run_merge(d, t); break;
    case OP_TOPK: run_topk(sm, d, t); break;
    case OP_COMBINE: run_combine(d, ca, t); break;
    case OP_ARGMAX: run_argmax(sm, d, ca, t); break;
    default: break;
  }
  if (persistent) signal_done(d, t, tix);
}

__global__ void __launch_bounds__(kThreads)
    mk_persistent_kernel(const DevPlan *__restrict__ dplan, CallArgs ca) {
  __shared__ Smem sm;
  __shared__ uint32_t s_ticket;
  for (;;) {
    // Re-read the plan through an opaque pointer every task so the compiler
    // does not keep it live in registers across the loop.
    CP *dp = (CP *)dplan;
    asm volatile("" : "+s"(dp));
    CP &d = *dp;
    if (threadIdx.x == 0) {
      uint32_t tk = atomicAdd(&d.ctrl[CTRL_TICKET], 1u);
      if (error_set(d)) tk = 0xffffffffu;
      s_ticket = tk;
    }
    __syncthreads();
    const uint32_t t = (uint32_t)uni((int)s_ticket);
    __syncthreads();
    if (t >= (uint32_t)d.n_tasks) break;
    run_task(sm, d, ca, (int)t, true);
  }
  // the last workgroup out re-arms the ticket counter for the next step
  if (threadIdx.x == 0) {
    uint32_t *ctrl = ((CP *)dplan)->ctrl;
    const uint32_t prev = atomicAdd(&ctrl[CTRL_DONE], 1u);
    if (prev == gridDim.x - 1) {
      atomicExch(&ctrl[CTRL_TICKET], 0u);
      atomicExch(&ctrl[CTRL_DONE], 0u);
    }
  }
}

__global__ void __launch_bounds__(kThreads)
    mk_phase_kernel(const DevPlan *__restrict__ dplan, CallArgs ca, int first) {
  __shared__ Smem sm;
  run_task(sm, *(CP *)dplan, ca, first + (int)blockIdx.x, false);
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
hipError_t launch_persistent(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s) {
  hipLaunchKernelGGL(mk_persistent_kernel, dim3(grid), dim3(kThreads), 0, s, d, ca);
  return hipGetLastError();
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

int persistent_lds_bytes() { return (int)sizeof(Smem) + 4; }

}  // namespace mk
