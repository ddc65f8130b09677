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
  // rows are streamed in 16-byte lanes; 1 KiB chunks may straddle one row
  // boundary at lane 32, which needs rows of a multiple of 512 bytes
  if (K <= 0 || (K % 256) != 0) return 0;
  return 16;
}

// Rows per tile for an operation over `total_rows` rows of K elements, with
// `nseg` matrices cut at the same rows (gate and up).  A tile holds at most
// kMaxTileUnits16 chunks of 1 KiB and a whole number of them.  If align > 0
// the row count must divide it (tiles never straddle a head boundary).
static bool choose_tile(long total_rows, int K, int nseg, int n_cus, int align,
                        GemvShape &s) {
  s.vec_bytes = vec_bytes_for(K);
  if (!s.vec_bytes) return false;
  double best = 0;
  int best_r = 0;
  for (int r = 1; (long)nseg * r * K <= (long)kMaxTileUnits16 * 512; ++r) {
    if (((long)nseg * r * K) % 512) continue;
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
    if (c.n_experts > 512) return bad("at most 512 experts");
    if (c.expert_ffn_dim < 1) return bad("MoE model needs expert_ffn_dim > 0");
    if ((long)c.top_k * c.expert_ffn_dim * 4 > kLdsXBytes)
      return bad("top_k * expert_ffn_dim fp32 values must fit the LDS activation stage");
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
           const std::vector<int> &waits, std::initializer_list<int> sigs,
           int64_t bytes, int worker = -1, int rpp = 0) {
    Task t{};
    t.rpp = rpp;
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
    p.task_hint.push_back(worker);
  }
};

// One contiguous row range of one weight matrix (or of the gate/up pair)
// inside a GEMV operation, with what its tasks carry and signal.
struct RowSeg {
  int a0;     // QKV: matrix (0 q, 1 k, 2 v); expert GEMVs: slot; else 0
  int row0, rows;
  int sig;    // event the segment's tasks signal
  int a3 = 0; // expert gate/up: expert slot
};

// Matrix-core lowering of a static-weight GEMV for a batch of 16..64 slots.
// A tile is a block of whole 16-row groups (at most kMfmaGroups; gate/up: at
// most half of them per matrix) times a range of K.  Every slot's
// activations are read by every tile that covers their columns, so the
// operation is cut along K as well (split-K): with NB row blocks, each block
// is split into ns column ranges, NB * ns <= n_workers, so that a tile's
// activation slice is not much larger than its weights.  The ns tiles of a
// block leave their partial products in a shared buffer; each then waits for
// its siblings (an arrival counter per block) and adds up, in split order,
// one ns-th of the block's rows, which it writes as the operation's output.
// Task fields: a1 = first row, a2 = rows (per matrix), a3 = first column k0,
// rpp = kc | rb << 16 (columns per split, block index within the
// operation), a4 = the block's arrival counter (LM head: tile index; it is
// never split).  Tiles are placed one per worker, those of one column range
// on one XCD where possible (worker w runs on XCD w % 8), so the XCD's L2
// holds that slice of the activations for all of them.
static int add_gemv_mfma(Builder &b, int op, int layer, const std::vector<RowSeg> &segs, int K,
                         int nseg, int n_workers, int wait_ev, int64_t extra_bytes,
                         int *lm_index) {
  const int Rmax = (nseg == 2 ? kMfmaGroups / 2 : kMfmaGroups) * 16;
  struct Block { size_t seg; int row0, rows; };
  std::vector<Block> blocks;
  for (size_t i = 0; i < segs.size(); ++i) {
    const int rows = segs[i].rows;
    if (rows % 16) return -1;
    const int g = rows / 16;
    int nb = (rows + Rmax - 1) / Rmax;
    // more blocks than workers (the LM head): a whole number of blocks per
    // worker, so every worker streams the same share
    if (segs.size() == 1 && nb > n_workers)
      nb = std::min(g, (nb + n_workers - 1) / n_workers * n_workers);
    for (int k = 0; k < nb; ++k) {
      const int g0 = (int)((int64_t)g * k / nb), g1 = (int)((int64_t)g * (k + 1) / nb);
      blocks.push_back({i, segs[i].row0 + 16 * g0, 16 * (g1 - g0)});
    }
  }
  const int NB = (int)blocks.size();
  const int64_t row_bytes = (int64_t)nseg * K * 2;
  int ns = 1;
  if (op != OP_LMHEAD && NB < n_workers)
    ns = std::max(1, std::min({n_workers / NB, K / 256, kMaxKSplit}));
  int kc = (K + ns - 1) / ns;
  kc = (kc + 63) / 64 * 64;  // whole 64-column pairs (a tile loads 128-byte lines)
  ns = (K + kc - 1) / kc;
  if (ns > 1) {
    if (kc > 0xffff || NB > 0x7fff) return -1;
    b.p.n_kpart = std::max<int64_t>(b.p.n_kpart, (int64_t)NB * ns);
  }
  // workers: the tiles of column range ks prefer XCD ks % 8
  std::vector<std::vector<int>> free_w(8);
  for (int w = n_workers - 1; w >= 0; --w) free_w[w % 8].push_back(w);
  auto take_worker = [&](int pref) {
    int x = pref;
    if (free_w[x].empty())
      for (int y = 0; y < 8; ++y)
        if (free_w[y].size() > free_w[x].size()) x = y;
    const int w = free_w[x].back();
    free_w[x].pop_back();
    return w;
  };
  int added = 0;
  for (int rb = 0; rb < NB; ++rb) {
    const Block &bl = blocks[rb];
    const RowSeg &sg = segs[bl.seg];
    const int cnt = ns > 1 ? b.p.n_kcnt++ : 0;
    for (int ks = 0; ks < ns; ++ks) {
      const int k0 = ks * kc, kw = std::min(kc, K - k0);
      int w = -1;
      if (ns > 1) w = take_worker(ks % 8);
      else if (NB <= n_workers) w = rb;  // one tile per worker
      const int a4 = ns > 1 ? cnt : (lm_index ? (*lm_index)++ : 0);
      b.add(op, layer, sg.a0, bl.row0, bl.rows, k0, a4, {wait_ev}, {sg.sig},
            (int64_t)bl.rows * nseg * kw * 2 + extra_bytes, w, ns > 1 ? (kc | rb << 16) : K);
      ++added;
    }
  }
  (void)row_bytes;
  return added;
}

// Lower a static-weight GEMV operation: its rows (all of nseg * K bf16) are
// cut into one contiguous, near-equal share per worker (the balance is in
// bytes, as every row has the same length); a share becomes one task per
// segment piece, streamed in passes of at most one register tile, at most
// pmax passes per task.  With several segments the shares follow segment
// boundaries instead (see below).  Row counts are multiples of `min_unit`.
// Returns the number of tasks added, or -1 when a row does not fit one
// register tile.
int add_gemv(Builder &b, int op, int layer, const std::vector<RowSeg> &segs, int K, int nseg,
             int n_workers, int pmax, int wait_ev, int64_t extra_bytes, int *lm_index,
             int min_unit = 1, int early_ev = -1, const std::vector<int> *only = nullptr) {
  const int64_t row_bytes = (int64_t)nseg * K * 2;
  int unit = 1;
  while ((row_bytes * unit) % 1024 || unit % min_unit) ++unit;
  // the expert down projection keeps register-only passes
  const int units = op == OP_EDOWN ? kMaxTileUnits16 : b.p.tile_units;
  int R = (int)((int64_t)units * 1024 / row_bytes);
  R -= R % unit;
  if (b.p.mfma && op != OP_EGATEUP && op != OP_EDOWN)
    return add_gemv_mfma(b, op, layer, segs, K, nseg, n_workers, wait_ev, extra_bytes, lm_index);
  // the waits of every task: an earlier-stage event first when given (the
  // expert down projection routes from the router logits before its inputs)
  const std::vector<int> waits =
      early_ev >= 0 ? std::vector<int>{early_ev, wait_ev} : std::vector<int>{wait_ev};
  if (R < unit) return -1;
  int64_t total = 0;
  for (auto &sg : segs) total += sg.rows;
  int added = 0;
  const int nwk = only ? (int)only->size() : n_workers;  // the workers taking rows
  if (segs.size() > 1 && (int64_t)segs.size() <= nwk) {
    // Several matrices (the q, k, v rows of each KV group): workers are
    // shared out over the segments in proportion to their rows (largest
    // remainder, at least one each), and each segment's rows evenly over its
    // workers, so no worker's share straddles two matrices (one task each).
    const int ns = (int)segs.size();
    std::vector<int> nw(ns);
    int given = 0;
    for (int i = 0; i < ns; ++i) {
      nw[i] = std::max(1, (int)((double)segs[i].rows * nwk / (double)total));
      given += nw[i];
    }
    // then one worker at a time to the segment with the largest share per
    // worker (or away from the one whose share grows least)
    auto share = [&](int i, int k) { return (double)segs[i].rows / k; };
    while (given < nwk) {
      int bi = 0;
      for (int i = 1; i < ns; ++i)
        if (share(i, nw[i]) > share(bi, nw[bi])) bi = i;
      nw[bi]++, given++;
    }
    while (given > nwk) {
      int bi = -1;
      for (int i = 0; i < ns; ++i)
        if (nw[i] > 1 && (bi < 0 || share(i, nw[i] - 1) < share(bi, nw[bi] - 1))) bi = i;
      nw[bi]--, given--;
    }
    int w = 0;
    for (int i = 0; i < ns; ++i) {
      const RowSeg &sg = segs[i];
      for (int k = 0; k < nw[i]; ++k, ++w) {
        int64_t lo = (int64_t)sg.rows * k / nw[i], hi = (int64_t)sg.rows * (k + 1) / nw[i];
        lo -= lo % unit;
        hi = (k + 1 == nw[i]) ? sg.rows : hi - hi % unit;
        while (lo < hi) {
          int64_t n = std::min<int64_t>(hi - lo, (int64_t)pmax * R);
          const int P = (int)((n + R - 1) / R);
          int rpp = (int)((n + P - 1) / P);
          rpp += (unit - rpp % unit) % unit;
          b.add(op, layer, sg.a0, (int)(sg.row0 + lo), (int)n, sg.a3, 0, waits, {sg.sig},
                n * row_bytes + extra_bytes, only ? (*only)[w] : w, rpp);
          ++added;
          lo += n;
        }
      }
    }
    return added;
  }
  // (a single matrix: the workers in `only` when given, else all of them)
  const int nw = nwk;
  size_t si = 0;
  int64_t seg_base = 0;  // rows before segs[si]
  for (int i = 0; i < nw; ++i) {
    const int w = only ? (*only)[i] : i;
    int64_t lo = total * i / nw, hi = total * (i + 1) / nw;
    lo -= lo % unit;
    hi = (i + 1 == nw) ? total : hi - hi % unit;
    while (lo < hi) {
      while (lo >= seg_base + segs[si].rows) seg_base += segs[si++].rows;
      const RowSeg &sg = segs[si];
      const int64_t end = std::min<int64_t>(hi, seg_base + sg.rows);
      int64_t n = end - lo;
      const int64_t cap = (int64_t)pmax * R;
      if (n > cap) n = cap;
      const int P = (int)((n + R - 1) / R);
      int rpp = (int)((n + P - 1) / P);
      rpp += (unit - rpp % unit) % unit;
      const int row0 = (int)(sg.row0 + (lo - seg_base));
      const int a4 = lm_index ? (*lm_index)++ : 0;
      b.add(op, layer, sg.a0, row0, (int)n, sg.a3, a4, waits, {sg.sig},
            n * row_bytes + extra_bytes, w, rpp);
      ++added;
      lo += n;
    }
  }
  return added;
}

}  // namespace

int build_host_plan(const mk_config &c, const mk_plan_options &o, int n_cus,
                    int n_workers, HostPlan &p, std::string &err) {
  int rc = check_config(c, err);
  if (rc != MK_OK) return rc;
  if (n_cus < 1 || n_workers < 1) { err = "n_cus and n_workers must be >= 1"; return MK_ERR_INVALID_ARG; }
  p = HostPlan{};
  p.cfg = c;
  p.n_cus = n_cus;
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads,
            hd = c.head_dim, B = c.max_batch;
  const bool moe = c.n_experts > 0;
  p.G = nq / nkv;
  p.kv_first = o.shared_seqs > 0;
  p.max_pos = c.max_pages_per_seq * kPageSize;

  // attention splits: enough (slot, KV head, split) tasks to cover the CUs,
  // but at least 128 keys per split (a page for each of a task's waves) and
  // at most 128 partials (G heads x S splits) for the merging split to read
  // (measured on the MoE shape, G = 8, 8192 keys: 16 splits 3.37 ms/step,
  // 32 splits 3.42, 12 splits 3.50; on the 8B shape, G = 4, 32 splits stay
  // ahead of 16 at 131072 keys, 6.24 against 7.07 ms)
  int ctx = o.planned_ctx > 0 ? std::min(o.planned_ctx, p.max_pos) : p.max_pos;
  int want = std::max(1, n_cus / (nkv * B));
  int by_len = std::max(1, ctx / 128);
  p.S = std::max(1, std::min({want, by_len, std::max(1, 128 / (nq / nkv)), 64}));
  // a single sequence with a short context (at most 48 pages, six per wave
  // of one task): one split, as the merge's extra hop costs more than the
  // shorter page loops save (measured on the 8B shape: one split ahead at
  // contexts up to 551, the split count above ahead from 1047)
  if (B == 1 && ctx <= 768) p.S = 1;
  // Large batches (Cohere "Folyamatos batchkezelés": sequences of different
  // and changing lengths): the persistent workers claim a layer's attention
  // tasks at run time from a shared counter, longest first; about two tasks
  // per worker keep the last ones to finish short without multiplying the
  // per-task cost (8B shape, contexts U[128, 16384]: 8 splits best at 8
  // slots, 6.72 against 6.97 ms/step with 4; 4 at 16 slots, 9.06 against
  // 9.44 with 8; 2 at 32, 12.89 against 13.24 with 4; 1 at 64, where 2
  // splits took 2.3 % longer per step; at 4 slots the covering count, 8,
  // stays ahead of 16, 5.93 against 6.29).
  if (o.attn_pool >= 0 && B >= 8)
    p.S = std::max(1, std::min({2 * n_workers / (nkv * B), std::max(1, ctx / 256), 64}));
  if (o.attn_splits > 0) p.S = std::min(o.attn_splits, 128);  // merge keeps G*S pairs in LDS
  // (the scheduled executor dispatches tasks one by one: no claimed pool, no
  // split-K tiles that wait for their siblings, every edge a counter event)
  const bool sched = o.executor == MK_EXEC_SCHEDULED;
  p.attn_pool = !sched && (o.attn_pool > 0 ||
                           (o.attn_pool == 0 && B > 1 && (int64_t)B * nkv * p.S > n_workers));
  if (p.attn_pool && (int64_t)B * nkv * p.S > 0x7fff) {
    err = "too many attention tasks per layer for a claimed pool";
    return MK_ERR_UNSUPPORTED;
  }

  bool ok = true;
  // batched decode: matrix-core GEMV tiles when every static row count is a
  // whole number of 16-row groups and every input row a whole number of
  // 64-column pairs (a tile loads whole 128-byte lines)
  {
    const bool rows16 = H % 64 == 0 && (nq * hd) % 64 == 0 && hd % 16 == 0 &&
                        c.vocab % 16 == 0 && (moe ? c.n_experts % 16 == 0 : c.ffn_dim % 64 == 0);
    p.mfma = !sched && B <= kMfmaMaxBatch && rows16 &&
             (o.batched_mfma > 0 ? B >= 2 : o.batched_mfma == 0 && B >= 3);
  }
  // single slot: GEMV passes extend into the LDS above the staged
  // activations when the longest staged row leaves that space free.  Auto
  // for dense models only: a MoE layer is a chain of short tasks, where the
  // slots' extra waits cost more than the deeper prefetch saves (measured).
  {
    const int64_t kx = std::max<int64_t>(std::max<int64_t>(H, (int64_t)nq * hd),
                                         moe ? (int64_t)c.top_k * c.expert_ffn_dim : c.ffn_dim);
    const bool want = o.weight_lds > 0 || (o.weight_lds == 0 && !moe);
    p.lds_slots = (B == 1 && want && kx * 4 <= kLdsWbufOff) ? kLdsSlots : 0;
    p.tile_units = kCW * (kMaxChunks + p.lds_slots);
  }
  // passes per task: slots x passes share the LDS partial buffers; when the
  // slots of a step do not fit one activation stage the weights of a pass
  // are reused across slot chunks, so such tasks keep a single pass
  auto pmax_for = [&](int K) {
    const int bb = std::max(1, std::min(kMaxBatchGemv, (int)(kLdsXBytes / ((int64_t)K * 4))));
    if (B > bb) return 1;
    return std::max(1, kMaxPass / std::min(B, kMaxBatchGemv));
  };

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
  }

  Builder b(p);
  std::vector<int> x_ev(L + 1);
  for (int l = 0; l <= L; ++l) x_ev[l] = b.ev();
  // events of edges into tasks that read a whole tagged vector (x, attn,
  // xmid, h): data edges unless the batch runs on matrix cores
  std::vector<int> data_ev(x_ev);

  b.begin_phase();
  for (int s = 0; s < B; ++s)
    b.add(OP_EMBED, 0, s, 0, 0, 0, 0, {}, {x_ev[0]}, (int64_t)H * 2);

  const int G = p.G;
  // When a layer's attention tasks fill at most a quarter of the workers and
  // a worker's share of the output projection is one pass, attention runs
  // on workers of their own (the highest indices, which spread over the
  // XCDs) and the projection's rows go to the others: a worker that runs
  // attention cannot load its projection rows ahead, so its share would
  // finish last and hold back the next operation.  (Longer shares stream
  // mostly after the wait anyway; there the attention workers would idle.)
  // The QKV rows go to the others as well, so an attention task starts
  // waiting for its query, key and value while they are computed: after a
  // QKV tile of its own, its first loads would queue behind that tile's
  // output stores, which the memory side acknowledges only after their
  // write-through, and the task would start polling after the last
  // projection tile had finished (measured: 8B 3.24 -> 3.12 ms/step, MoE
  // 3.39 -> 3.24).
  const int n_attn = B * nkv * p.S;
  const int64_t oproj_share = (int64_t)H * nq * hd * 2 / n_workers;
  std::vector<int> attn_w, oproj_w;
  if (!p.mfma && !p.attn_pool && n_attn * 4 <= n_workers &&
      oproj_share * n_workers / (n_workers - n_attn) <= (int64_t)p.tile_units * 1024) {
    for (int i = 0; i < n_attn; ++i) attn_w.push_back(n_workers - 1 - i);
    for (int w = 0; w < n_workers - n_attn; ++w) oproj_w.push_back(w);
  }
  for (int l = 0; l < L; ++l) {
    // QKV, group by group so a KV head's attention can start early (in
    // shared-sequence plans one event for all groups: the key/value stores
    // wait for every group)
    std::vector<int> grp(nkv);
    for (int g = 0; g < nkv; ++g) {
      grp[g] = (p.kv_first && g > 0) ? grp[0] : b.ev();
      if (!p.kv_first || g == 0) data_ev.push_back(grp[g]);  // q, k, v are tagged
    }
    b.begin_phase();
    {
      std::vector<RowSeg> segs;
      for (int g = 0; g < nkv; ++g) {
        segs.push_back({0, g * G * hd, G * hd, grp[g]});
        segs.push_back({1, g * hd, hd, grp[g]});
        segs.push_back({2, g * hd, hd, grp[g]});
      }
      if (add_gemv(b, OP_QKV, l, segs, H, 1, n_workers, pmax_for(H), x_ev[l], 0, nullptr, 1,
                   -1, oproj_w.empty() ? nullptr : &oproj_w) < 0)
        ok = false;
    }
    // Shared-sequence plans: every slot's key and value go into the cache
    // before any attention task of the layer reads it (a prompt chunk's
    // slots attend to each other's positions), a counter edge.
    int app = -1;
    if (p.kv_first) {
      app = b.ev();
      b.begin_phase();
      for (int s = 0; s < B; ++s)
        b.add(OP_KVAPP, l, s, 0, 0, 0, 0, {grp[0]}, {app}, 0);
    }
    // attention splits; with several splits, the split that arrives last
    // for its (slot, KV head) merges them and reports the head group's one
    // completion (statically: the last split carries it)
    int mrg = b.ev();
    b.begin_phase();
    for (int s = 0; s < B; ++s)
      for (int g = 0; g < nkv; ++g)
        for (int sp = 0; sp < p.S; ++sp) {
          std::vector<int> waits{grp[g]};
          if (app >= 0) waits.push_back(app);
          b.add(OP_ATTN, l, s, g, sp, 0, 0, waits, {mrg}, 0,
                attn_w.empty() ? -1 : attn_w[(s * nkv + g) * p.S + sp]);
        }
    if (p.S > 1) p.ev_thr[mrg] = B * nkv;  // one merged group per (slot, KV head)
    // O projection + residual
    int xo = b.ev();
    data_ev.push_back(mrg);
    data_ev.push_back(xo);
    b.begin_phase();
    if (add_gemv(b, OP_OPROJ, l, {{0, 0, H, xo}}, nq * hd, 1, n_workers, pmax_for(nq * hd), mrg,
                 0, nullptr, 1, -1, oproj_w.empty() ? nullptr : &oproj_w) < 0)
      ok = false;
    if (!moe) {
      int hev = b.ev();
      data_ev.push_back(hev);
      b.begin_phase();
      if (add_gemv(b, OP_GATEUP, l, {{0, 0, c.ffn_dim, hev}}, H, 2, n_workers, pmax_for(H), xo,
                   0, nullptr) < 0)
        ok = false;
      b.begin_phase();
      if (add_gemv(b, OP_DOWN, l, {{0, 0, H, x_ev[l + 1]}}, c.ffn_dim, 1, n_workers,
                   pmax_for(c.ffn_dim), hev, 0, nullptr) < 0)
        ok = false;
    } else {
      // MoE: router logits; every expert gate/up task selects the top-k
      // itself from them (no separate routing task); the down projection of
      // a row range covers all k experts and adds their weighted sum to the
      // residual (no separate combine task).
      const int E = c.n_experts, K = c.top_k, Fe = c.expert_ffn_dim;
      int rlev = b.ev();
      data_ev.push_back(rlev);  // the router logits are tagged
      b.begin_phase();
      // (the router rows go to the attention workers when there are some:
      // they hold no output projection rows, so no output stores of theirs
      // are still in flight ahead of the staging loads; 3.25 -> 3.21 ms/step)
      if (add_gemv(b, OP_ROUTER, l, {{0, 0, E, rlev}}, H, 1, n_workers, pmax_for(H), xo, 0,
                   nullptr, 1, -1, attn_w.empty() ? nullptr : &attn_w) < 0)
        ok = false;
      int eh = b.ev();
      b.begin_phase();
      {
        std::vector<RowSeg> segs;
        for (int s = 0; s < B; ++s)
          for (int j = 0; j < K; ++j) segs.push_back({s, 0, Fe, eh, j});
        if (add_gemv(b, OP_EGATEUP, l, segs, H, 2, n_workers, pmax_for(H), rlev, 0, nullptr) < 0)
          ok = false;
      }
      b.begin_phase();
      {
        // k segments per task (one per expert), each a whole number of 1 KiB
        // chunks: rows * Fe * 2 bytes divisible by 1024
        int unit = 1;
        while (((int64_t)unit * Fe * 2) % 1024) ++unit;
        std::vector<RowSeg> segs;
        for (int s = 0; s < B; ++s) segs.push_back({s, 0, H, x_ev[l + 1]});
        if (add_gemv(b, OP_EDOWN, l, segs, Fe, K, n_workers, 1, eh, 0, nullptr, unit, rlev) < 0)
          ok = false;
      }
    }
  }
  // final norm + LM head (+ per-tile argmax partials), then argmax
  int lm = b.ev();
  b.begin_phase();
  int n_lm = 0;
  if (add_gemv(b, OP_LMHEAD, L, {{0, 0, c.vocab, lm}}, H, 1, n_workers, pmax_for(H), x_ev[L],
               (int64_t)H * 2, &n_lm) < 0)
    ok = false;
  if (!ok) { err = "a row does not fit one register tile"; return MK_ERR_UNSUPPORTED; }
  p.n_lm_tiles = n_lm;
  p.n_amax = (int64_t)B * p.n_lm_tiles;
  b.begin_phase();
  for (int s = 0; s < B; ++s) b.add(OP_ARGMAX, L, s, 0, 0, 0, 0, {lm}, {}, 0);
  b.end();

  // per-task thresholds
  for (auto &t : p.tasks)
    for (int i = 0; i < t.n_wait; ++i) t.wait_thr[i] = p.ev_thr[t.wait_ev[i]];

  // Worker queues (the MPK runtime's per-worker task queues).  Each launch
  // phase's tasks are dealt in contiguous blocks, so a worker's consecutive
  // tiles are neighbours in memory (weight streams stay within DRAM and
  // translation pages); when a phase does not divide evenly, the extra tasks
  // go to the workers with the least bytes so far.  Every queue is a
  // subsequence of the list order, which is topological, so with all workers
  // resident the lowest unfinished task always has its inputs ready.
  const int T = (int)p.tasks.size();
  p.n_workers = n_workers;
  p.task_worker.assign(T, 0);
  std::vector<std::vector<int32_t>> q(n_workers);
  std::vector<int64_t> load(n_workers, 0);
  std::vector<int> order(n_workers);
  for (auto &ph : p.phases) {
    const int n = ph.second - ph.first;
    if (p.task_hint[ph.first] >= 0) {  // per-worker shares chosen by the lowering
      for (int i = ph.first; i < ph.second; ++i) {
        const int w = p.task_hint[i];
        q[w].push_back(i);
        p.task_worker[i] = w;
        load[w] += std::max<int64_t>(p.task_bytes[i], 16384);
      }
      continue;
    }
    const int base = n / n_workers, extra = n % n_workers;
    // least-loaded workers take the extra tasks (ties: lower index)
    for (int w = 0; w < n_workers; ++w) order[w] = w;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return load[a] < load[b]; });
    std::vector<int> cnt(n_workers, base);
    for (int k = 0; k < extra; ++k) cnt[order[k]]++;
    int i = ph.first;
    for (int w = 0; w < n_workers; ++w)
      for (int k = 0; k < cnt[w]; ++k, ++i) {
        q[w].push_back(i);
        p.task_worker[i] = w;
        load[w] += std::max<int64_t>(p.task_bytes[i], 16384);
      }
  }
  // A run of consecutive tasks in one queue that signal the same events
  // reports all its completions once, from its last task.
  const bool split_attn = p.S > 1;
  auto same_sig = [&](const Task &a, const Task &b) {
    if ((split_attn || p.attn_pool) && (a.op == OP_ATTN || b.op == OP_ATTN)) return false;
    if (a.n_sig != b.n_sig || a.n_sig == 0) return false;
    for (int k = 0; k < a.n_sig; ++k)
      if (a.sig_ev[k] != b.sig_ev[k]) return false;
    return true;
  };
  p.worker_off.assign(n_workers + 1, 0);
  p.worker_list.clear();
  p.worker_list.reserve(T);
  for (int w = 0; w < n_workers; ++w) {
    const auto &lst = q[w];
    size_t k = 0;
    while (k < lst.size()) {
      size_t j = k;
      while (j + 1 < lst.size() && same_sig(p.tasks[lst[j]], p.tasks[lst[j + 1]])) ++j;
      for (size_t m = k; m < j; ++m) p.tasks[lst[m]].a5 = 0;
      p.tasks[lst[j]].a5 = (int)(j - k + 1);
      if (split_attn && p.tasks[lst[j]].op == OP_ATTN)
        p.tasks[lst[j]].a5 = p.tasks[lst[j]].a2 == p.S - 1 ? 1 : 0;
      k = j + 1;
    }
    p.worker_off[w] = (int32_t)p.worker_list.size();
    p.worker_list.insert(p.worker_list.end(), lst.begin(), lst.end());
  }
  p.worker_off[n_workers] = (int32_t)p.worker_list.size();
  if (p.attn_pool) {
    // Claimed attention: every ATTN task carries its layer's first ATTN task
    // (a4) and rpp = count | claims per step << 16, where a step's claims are
    // the count plus one failed claim by each worker holding entries of the
    // layer; the first of a worker's consecutive entries of a layer carries
    // their number (a3): that worker claims from the pool there and skips
    // the rest of them.
    std::vector<int> first(L, -1), cnt(L, 0), holders(L, 0);
    for (int i = 0; i < T; ++i)
      if (p.tasks[i].op == OP_ATTN) {
        const int l = p.tasks[i].layer;
        if (first[l] < 0) first[l] = i;
        cnt[l]++;
      }
    for (int w = 0; w < n_workers; ++w) {
      for (int k = p.worker_off[w]; k < p.worker_off[w + 1];) {
        Task &t = p.tasks[p.worker_list[k]];
        if (t.op != OP_ATTN) { ++k; continue; }
        int j = k + 1;
        while (j < p.worker_off[w + 1] && p.tasks[p.worker_list[j]].op == OP_ATTN &&
               p.tasks[p.worker_list[j]].layer == t.layer)
          ++j;
        t.a3 = j - k;
        holders[t.layer]++;
        k = j;
      }
    }
    for (auto &t : p.tasks)
      if (t.op == OP_ATTN) {
        t.a4 = first[t.layer];
        t.rpp = cnt[t.layer] | (cnt[t.layer] + holders[t.layer]) << 16;
      }
  }
  rc = validate_plan(p, err);
  if (rc != MK_OK) return rc;
  // Data edges: the reader checks the tags of the vector it stages instead of
  // waiting for the counter, and the writers do not signal.  (Matrix-core
  // batches stage their activations in slices, so they keep the counters.)
  if (!p.mfma && !sched) {
    std::vector<char> is_data(p.ev_thr.size(), 0);
    for (int e : data_ev) is_data[e] = 1;
    for (auto &t : p.tasks) {
      for (int i = 0; i < t.n_wait; ++i)
        if (is_data[t.wait_ev[i]]) t.wait_ev[i] |= kDataEdge;
      for (int i = 0; i < t.n_sig; ++i)
        if (is_data[t.sig_ev[i]]) t.sig_ev[i] |= kDataEdge;
    }
  }
  return MK_OK;
}

int validate_plan(const HostPlan &p, std::string &err) {
  char buf[256];
  const int T = (int)p.tasks.size(), E = (int)p.ev_thr.size();
  std::vector<int> last_sig(E, -1), n_sig(E, 0), sig_phase(E, -1), n_wait(E, 0);
  for (int i = 0; i < T; ++i) {
    const Task &t = p.tasks[i];
    // the splits of one (slot, KV head) report one completion between them
    // (the last to arrive, after merging); any of them may be that one
    const bool split = t.op == OP_ATTN && p.S > 1;
    for (int k = 0; k < t.n_sig; ++k) {
      int e = t.sig_ev[k];
      if (e < 0 || e >= E) { err = "signal of an unknown event"; return MK_ERR_PLAN; }
      last_sig[e] = i;
      n_sig[e] += split ? (t.a2 == p.S - 1) : 1;
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
  // completions reported per event equal its threshold; no self-waits
  std::vector<int64_t> reported(E, 0);
  for (int i = 0; i < T; ++i) {
    const Task &t = p.tasks[i];
    for (int k = 0; k < t.n_sig; ++k) {
      reported[t.sig_ev[k]] += t.a5;
      for (int m = 0; m < t.n_wait; ++m)
        if (t.wait_ev[m] == t.sig_ev[k]) { err = "a task waits on an event it signals"; return MK_ERR_PLAN; }
    }
  }
  for (int e = 0; e < E; ++e)
    if (reported[e] != p.ev_thr[e]) {
      snprintf(buf, sizeof buf, "event %d: %lld completions reported, threshold %d", e,
               (long long)reported[e], p.ev_thr[e]);
      err = buf;
      return MK_ERR_PLAN;
    }
  // worker queues: a partition of the tasks, each queue increasing
  if ((int)p.worker_off.size() != p.n_workers + 1 || (int)p.worker_list.size() != T) {
    err = "worker queues do not partition the tasks";
    return MK_ERR_PLAN;
  }
  std::vector<char> seen(T, 0);
  for (int w = 0; w < p.n_workers; ++w)
    for (int k = p.worker_off[w]; k < p.worker_off[w + 1]; ++k) {
      const int ti = p.worker_list[k];
      if (ti < 0 || ti >= T || seen[ti]) { err = "worker queues do not partition the tasks"; return MK_ERR_PLAN; }
      seen[ti] = 1;
      if (k > p.worker_off[w] && p.worker_list[k - 1] >= ti) {
        err = "a worker queue is not in list order";
        return MK_ERR_PLAN;
      }
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
