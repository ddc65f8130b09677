// planner.cpp -- lowers one decode step into per-tile tasks and events.
//
// Task granularity follows the MPK author's answer in the Hacker News thread
// (post #58): one task does about the work of one thread block of a
// kernel-per-operator design, and task B depends on task A exactly when A
// writes elements that B reads.  For a full-K matrix-vector product every
// output tile reads the whole input vector, so it depends on every producer
// tile of that vector; where an operation reads only part of its input the
// planner uses the narrower dependency, as the Cohere article suggests
// ("Honnan jön a gyorsulás?"): the attention of one KV head waits only for the
// QKV tiles of that head's group, and an expert's down projection waits only
// for that expert's gate/up tiles.
//
// Tile sizes are chosen for the CU count (the same section's wave-quantization
// argument): among the row counts that fit one workgroup's load registers,
// pick the one with the least time counting whole waves of tiles plus a fixed
// per-tile cost.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace mk {

int vec_bytes_for(int K) {
  long rb = (long)K * 2;
  if (K <= 0) return 0;
  if (rb % 1024 == 0) return 16;
  if (rb % 512 == 0) return 8;
  return 0;
}

static int units_per_row(int K, int vw) { return (int)((long)K * 2 / (64L * vw)); }
static int max_units(int vw) { return kMaxTileUnits16 * 16 / vw; }

// Rows per tile for an operation over `total_rows` rows of K elements, with
// `nseg` matrices cut at the same rows (gate and up).  If align > 0 the row
// count must divide it (tiles never straddle a head boundary).
static bool choose_tile(long total_rows, int K, int nseg, int n_cus, int align,
                        GemvShape &s) {
  s.vec_bytes = vec_bytes_for(K);
  if (!s.vec_bytes) return false;
  int wc = units_per_row(K, s.vec_bytes);
  int rmax = max_units(s.vec_bytes) / (wc * nseg);
  if (rmax < 1) return false;
  double best = 0;
  int best_r = 0;
  for (int r = 1; r <= rmax; ++r) {
    if (align > 0 && align % r) continue;
    long tiles = (total_rows + r - 1) / r;
    long waves = (tiles + n_cus - 1) / n_cus;
    double cost = (double)waves * ((double)r * nseg * K * 2 + 24576.0);
    if (best_r == 0 || cost < best * (1 - 1e-12) ||
        (cost <= best * (1 + 1e-12) && r > best_r)) {
      best = cost;
      best_r = r;
    }
  }
  if (!best_r) return false;
  s.rows_per_tile = best_r;
  s.tiles = (int)((total_rows + best_r - 1) / best_r);
  return true;
}

int check_config(const mk_config &c, std::string &err) {
  char buf[256];
  auto bad = [&](const char *m) { err = m; return (int)MK_ERR_INVALID_CONFIG; };
  if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 ||
      c.vocab < 1 || c.max_batch < 1 || c.max_pages_per_seq < 1 || c.n_pages < 1)
    return bad("non-positive dimension in mk_config");
  if (c.page_size != kPageSize) return bad("page_size must be 16");
  if (c.head_dim != 64 && c.head_dim != 128)
    return bad("head_dim must be 64 or 128");
  if (c.n_q_heads % c.n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (c.n_q_heads / c.n_kv_heads > kMaxGroup) return bad("more than 8 query heads per KV head");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.0)) return bad("rms_eps and rope_theta must be > 0");
  if (c.n_experts < 0) return bad("n_experts < 0");
  if (c.n_experts == 0) {
    if (c.ffn_dim < 1) return bad("dense model needs ffn_dim > 0");
  } else {
    if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 16)
      return bad("top_k must be in [1, min(n_experts, 16)]");
    if (c.n_experts > kThreads) return bad("at most 512 experts");
    if (c.expert_ffn_dim < 1) return bad("MoE model needs expert_ffn_dim > 0");
  }
  const int Ks[4] = {c.hidden, c.n_q_heads * c.head_dim,
                     c.n_experts ? c.expert_ffn_dim : c.ffn_dim, 0};
  for (int i = 0; i < 3; ++i) {
    if (!vec_bytes_for(Ks[i])) {
      snprintf(buf, sizeof buf, "row length %d is not a multiple of 256 elements", Ks[i]);
      err = buf;
      return MK_ERR_UNSUPPORTED;
    }
    if ((long)Ks[i] * 4 > kLdsXBytes) {
      snprintf(buf, sizeof buf, "row length %d does not fit the LDS activation stage", Ks[i]);
      err = buf;
      return MK_ERR_UNSUPPORTED;
    }
  }
  if ((long)c.max_pages_per_seq * kPageSize > (1L << 24))
    return bad("max_pages_per_seq too large");
  return MK_OK;
}

namespace {

struct Builder {
  HostPlan &p;
  int phase = -1;
  explicit Builder(HostPlan &pp) : p(pp) {}
  int ev() {
    p.ev_thr.push_back(0);
    return (int)p.ev_thr.size() - 1;
  }
  void begin_phase() {
    int n = (int)p.tasks.size();
    if (phase >= 0 && p.phases.back().first == n) return;  // empty phase
    if (phase >= 0) p.phases.back().second = n;
    p.phases.push_back({n, n});
    phase = (int)p.phases.size() - 1;
  }
  void end() {
    if (phase >= 0) p.phases.back().second = (int)p.tasks.size();
  }
  void add(int op, int layer, int a0, int a1, int a2, int a3, int a4,
           std::initializer_list<int> waits, std::initializer_list<int> sigs,
           int64_t bytes) {
    Task t{};
    t.op = (int16_t)op;
    t.layer = (int16_t)layer;
    t.a0 = a0; t.a1 = a1; t.a2 = a2; t.a3 = a3; t.a4 = a4; t.a5 = 0;
    t.n_wait = 0;
    for (int e : waits) t.wait_ev[t.n_wait++] = e;
    t.n_sig = 0;
    for (int e : sigs) {
      t.sig_ev[t.n_sig++] = e;
      p.ev_thr[e] += 1;
    }
    p.tasks.push_back(t);
    p.task_phase.push_back(phase);
    p.task_bytes.push_back(bytes);
  }
};

}  // namespace

int build_host_plan(const mk_config &c, const mk_plan_options &o, int n_cus,
                    HostPlan &p, std::string &err) {
  int rc = check_config(c, err);
  if (rc != MK_OK) return rc;
  if (n_cus < 1) { err = "n_cus < 1"; return MK_ERR_INVALID_ARG; }
  p = HostPlan{};
  p.cfg = c;
  p.n_cus = n_cus;
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads,
            hd = c.head_dim, B = c.max_batch;
  const bool moe = c.n_experts > 0;
  p.G = nq / nkv;
  p.max_pos = c.max_pages_per_seq * kPageSize;

  // attention splits: enough (slot, KV head, split) tasks to cover the CUs,
  // but at least about 64 keys per split
  int ctx = o.planned_ctx > 0 ? std::min(o.planned_ctx, p.max_pos) : p.max_pos;
  int want = std::max(1, n_cus / (nkv * B));
  int by_len = std::max(1, ctx / 64);
  p.S = std::max(1, std::min(std::min(want, by_len), 64));
  if (o.attn_splits > 0) p.S = std::min(o.attn_splits, 256);

  // tile shapes
  bool ok = choose_tile((long)(nq + 2 * nkv) * hd, H, 1, n_cus, hd, p.qkv) &&
            choose_tile(H, nq * hd, 1, n_cus, 0, p.oproj) &&
            choose_tile(c.vocab, H, 1, n_cus, 0, p.lmhead);
  if (!moe) {
    ok = ok && choose_tile(c.ffn_dim, H, 2, n_cus, 0, p.gateup) &&
         choose_tile(H, c.ffn_dim, 1, n_cus, 0, p.down);
  } else {
    const int Fe = c.expert_ffn_dim;
    ok = ok && choose_tile(c.n_experts, H, 1, n_cus, 0, p.router) &&
         choose_tile((long)Fe * c.top_k * B, H, 2, n_cus, 0, p.egateup) &&
         choose_tile((long)H * c.top_k * B, Fe, 1, n_cus, 0, p.edown);
    // expert tiles must not straddle experts: round rows to divisors
    auto fit = [&](GemvShape &s, int rows) {
      int r = std::min(s.rows_per_tile, rows);
      while (rows % r) --r;
      s.rows_per_tile = r;
      s.tiles = rows / r;
    };
    if (ok) {
      fit(p.egateup, Fe);
      fit(p.edown, H);
    }
  }
  if (!ok) { err = "no tile shape fits the row lengths"; return MK_ERR_UNSUPPORTED; }
  p.n_lm_tiles = p.lmhead.tiles;

  // scratch sizes
  p.n_x = (int64_t)(L + 1) * B * H;
  p.n_xmid = (int64_t)L * B * H;
  p.n_q = (int64_t)L * B * nq * hd;
  p.n_k = (int64_t)L * B * nkv * hd;
  p.n_part = (int64_t)L * B * nq * p.S * part_stride(hd);
  p.n_attn = (int64_t)L * B * nq * hd;
  p.n_h = moe ? 0 : (int64_t)L * B * c.ffn_dim;
  if (moe) {
    p.n_rl = (int64_t)L * B * c.n_experts;
    p.n_tk = (int64_t)L * B * c.top_k;
    p.n_he = (int64_t)L * B * c.top_k * c.expert_ffn_dim;
    p.n_ye = (int64_t)L * B * c.top_k * H;
  }
  p.n_amax = (int64_t)B * p.n_lm_tiles;

  Builder b(p);
  std::vector<int> x_ev(L + 1);
  for (int l = 0; l <= L; ++l) x_ev[l] = b.ev();

  b.begin_phase();
  for (int s = 0; s < B; ++s)
    b.add(OP_EMBED, 0, s, 0, 0, 0, 0, {}, {x_ev[0]}, (int64_t)H * 2);

  const int G = p.G;
  for (int l = 0; l < L; ++l) {
    // QKV, group by group so a KV head's attention can start early
    std::vector<int> grp(nkv);
    for (int g = 0; g < nkv; ++g) grp[g] = b.ev();
    b.begin_phase();
    const int rq = p.qkv.rows_per_tile;
    for (int g = 0; g < nkv; ++g) {
      for (int r = g * G * hd; r < (g + 1) * G * hd; r += rq)
        b.add(OP_QKV, l, 0, r, rq, 0, 0, {x_ev[l]}, {grp[g]}, (int64_t)rq * H * 2);
      for (int m = 1; m <= 2; ++m)
        for (int r = g * hd; r < (g + 1) * hd; r += rq)
          b.add(OP_QKV, l, m, r, rq, 0, 0, {x_ev[l]}, {grp[g]}, (int64_t)rq * H * 2);
    }
    // attention splits (+ merge when split)
    int mrg = b.ev();
    std::vector<int> att(B * nkv, -1);
    b.begin_phase();
    for (int s = 0; s < B; ++s)
      for (int g = 0; g < nkv; ++g) {
        if (p.S > 1) att[s * nkv + g] = b.ev();
        for (int sp = 0; sp < p.S; ++sp)
          b.add(OP_ATTN, l, s, g, sp, 0, 0, {grp[g]},
                {p.S > 1 ? att[s * nkv + g] : mrg}, 0);
      }
    if (p.S > 1) {
      b.begin_phase();
      for (int s = 0; s < B; ++s)
        for (int g = 0; g < nkv; ++g)
          b.add(OP_MERGE, l, s, g, 0, 0, 0, {att[s * nkv + g]}, {mrg}, 0);
    }
    // O projection + residual
    int xo = b.ev();
    b.begin_phase();
    const int ro = p.oproj.rows_per_tile;
    for (int r = 0; r < H; r += ro) {
      int n = std::min(ro, H - r);
      b.add(OP_OPROJ, l, 0, r, n, 0, 0, {mrg}, {xo}, (int64_t)n * nq * hd * 2);
    }
    if (!moe) {
      int hev = b.ev();
      b.begin_phase();
      const int rg = p.gateup.rows_per_tile;
      for (int r = 0; r < c.ffn_dim; r += rg) {
        int n = std::min(rg, c.ffn_dim - r);
        b.add(OP_GATEUP, l, 0, r, n, 0, 0, {xo}, {hev}, (int64_t)2 * n * H * 2);
      }
      b.begin_phase();
      const int rd = p.down.rows_per_tile;
      for (int r = 0; r < H; r += rd) {
        int n = std::min(rd, H - r);
        b.add(OP_DOWN, l, 0, r, n, 0, 0, {hev}, {x_ev[l + 1]},
              (int64_t)n * c.ffn_dim * 2);
      }
    } else {
      const int E = c.n_experts, K = c.top_k, Fe = c.expert_ffn_dim;
      int rlev = b.ev();
      b.begin_phase();
      const int rr = p.router.rows_per_tile;
      for (int r = 0; r < E; r += rr) {
        int n = std::min(rr, E - r);
        b.add(OP_ROUTER, l, 0, r, n, 0, 0, {xo}, {rlev}, (int64_t)n * H * 2);
      }
      std::vector<int> tk(B);
      b.begin_phase();
      for (int s = 0; s < B; ++s) {
        tk[s] = b.ev();
        b.add(OP_TOPK, l, s, 0, 0, 0, 0, {rlev}, {tk[s]}, 0);
      }
      std::vector<int> eh(B * K), ey(B);
      b.begin_phase();
      const int re = p.egateup.rows_per_tile;
      for (int s = 0; s < B; ++s)
        for (int j = 0; j < K; ++j) {
          eh[s * K + j] = b.ev();
          for (int r = 0; r < Fe; r += re)
            b.add(OP_EGATEUP, l, s, r, re, j, 0, {tk[s]}, {eh[s * K + j]},
                  (int64_t)2 * re * H * 2);
        }
      b.begin_phase();
      const int rdn = p.edown.rows_per_tile;
      for (int s = 0; s < B; ++s) {
        ey[s] = b.ev();
        for (int j = 0; j < K; ++j)
          for (int r = 0; r < H; r += rdn)
            b.add(OP_EDOWN, l, s, r, rdn, j, 0, {eh[s * K + j]}, {ey[s]},
                  (int64_t)rdn * Fe * 2);
      }
      b.begin_phase();
      const int rc2 = std::max(256, H / 8);
      for (int s = 0; s < B; ++s)
        for (int r = 0; r < H; r += rc2)
          b.add(OP_COMBINE, l, s, r, std::min(rc2, H - r), 0, 0, {ey[s]},
                {x_ev[l + 1]}, 0);
    }
  }
  // final norm + LM head (+ per-tile argmax partials), then argmax
  int lm = b.ev();
  b.begin_phase();
  const int rl = p.lmhead.rows_per_tile;
  int tile = 0;
  for (int r = 0; r < c.vocab; r += rl, ++tile) {
    int n = std::min(rl, c.vocab - r);
    b.add(OP_LMHEAD, L, 0, r, n, 0, tile, {x_ev[L]}, {lm}, (int64_t)n * H * 2 + H * 2);
  }
  b.begin_phase();
  for (int s = 0; s < B; ++s) b.add(OP_ARGMAX, L, s, 0, 0, 0, 0, {lm}, {}, 0);
  b.end();

  // per-task thresholds
  for (auto &t : p.tasks)
    for (int i = 0; i < t.n_wait; ++i) t.wait_thr[i] = p.ev_thr[t.wait_ev[i]];
  return validate_plan(p, err);
}

int validate_plan(const HostPlan &p, std::string &err) {
  char buf[256];
  const int T = (int)p.tasks.size(), E = (int)p.ev_thr.size();
  std::vector<int> last_sig(E, -1), n_sig(E, 0), sig_phase(E, -1), n_wait(E, 0);
  for (int i = 0; i < T; ++i) {
    const Task &t = p.tasks[i];
    for (int k = 0; k < t.n_sig; ++k) {
      int e = t.sig_ev[k];
      if (e < 0 || e >= E) { err = "signal of an unknown event"; return MK_ERR_PLAN; }
      last_sig[e] = i;
      n_sig[e]++;
      sig_phase[e] = std::max(sig_phase[e], p.task_phase[i]);
    }
  }
  for (int i = 0; i < T; ++i) {
    const Task &t = p.tasks[i];
    for (int k = 0; k < t.n_wait; ++k) {
      int e = t.wait_ev[k];
      if (e < 0 || e >= E) { err = "wait on an unknown event"; return MK_ERR_PLAN; }
      n_wait[e]++;
      if (n_sig[e] == 0) {
        snprintf(buf, sizeof buf, "task %d waits on event %d that nothing signals", i, e);
        err = buf;
        return MK_ERR_PLAN;
      }
      if (last_sig[e] >= i) {
        snprintf(buf, sizeof buf,
                 "task %d waits on event %d signalled by later task %d (ticket order "
                 "is not topological)", i, e, last_sig[e]);
        err = buf;
        return MK_ERR_PLAN;
      }
      if (t.wait_thr[k] != n_sig[e] || p.ev_thr[e] != n_sig[e]) {
        snprintf(buf, sizeof buf, "task %d: threshold %d of event %d != %d signallers",
                 i, t.wait_thr[k], e, n_sig[e]);
        err = buf;
        return MK_ERR_PLAN;
      }
      if (sig_phase[e] >= p.task_phase[i]) {
        snprintf(buf, sizeof buf, "task %d waits on an event of its own launch", i);
        err = buf;
        return MK_ERR_PLAN;
      }
    }
  }
  for (int e = 0; e < E; ++e)
    if (n_sig[e] > 0 && n_wait[e] == 0) {
      snprintf(buf, sizeof buf, "event %d is signalled but never waited on", e);
      err = buf;
      return MK_ERR_PLAN;
    }
  // phases tile the task list
  int pos = 0;
  for (auto &ph : p.phases) {
    if (ph.first != pos || ph.second <= ph.first) { err = "bad phase ranges"; return MK_ERR_PLAN; }
    pos = ph.second;
  }
  if (pos != T) { err = "phases do not cover the task list"; return MK_ERR_PLAN; }
  return MK_OK;
}

}  // namespace mk
