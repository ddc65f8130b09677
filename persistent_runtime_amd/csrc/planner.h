// planner.h -- host-side lowering of a decode step into the task graph.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_task.h"

namespace mk {

struct GemvShape {       // how one operation's rows are cut into tiles
  int rows_per_tile;     // rows per matrix segment
  int vec_bytes;         // 16 or 8: per-lane load width
  int tiles;
};

struct HostPlan {
  mk_config cfg{};
  int n_cus = 0;
  int S = 1;                        // attention splits per (slot, KV head)
  int G = 1;                        // query heads per KV head
  int n_lm_tiles = 0;
  int max_pos = 0;
  bool mfma = false;                // static GEMVs as matrix-core tiles (16-row groups)
  bool attn_pool = false;           // attention tasks claimed at run time (persistent)
  bool kv_first = false;            // several slots may hold one sequence: KVAPP
                                    // tasks store keys/values before attention
  int lds_slots = 0;                // kLdsSlots when GEMV passes extend into LDS
  int tile_units = kMaxTileUnits16; // 1 KiB units per GEMV pass
  std::vector<Task> tasks;
  std::vector<int32_t> ev_thr;      // per-step threshold of each event
  std::vector<int32_t> task_phase;  // launch index under kernel-per-op
  std::vector<std::pair<int32_t, int32_t>> phases;  // [begin, end) per launch
  std::vector<int64_t> task_bytes;  // algorithmic bytes read per task
  std::vector<int32_t> task_hint;   // worker chosen by the lowering, or -1
  int n_workers = 0;                // persistent workgroups (one per CU)
  std::vector<int32_t> task_worker; // worker that runs each task
  std::vector<int32_t> worker_off;  // [n_workers + 1]
  std::vector<int32_t> worker_list; // task indices per worker, in list order
  // scratch sizes in elements
  int64_t n_x = 0, n_xmid = 0, n_q = 0, n_k = 0, n_part = 0, n_attn = 0,
          n_h = 0, n_rl = 0, n_tk = 0, n_he = 0, n_amax = 0;
  // split-K matrix-core tiles: arrival counters (one per row block of every
  // split operation in the step) and partial-product slots (the most tiles
  // of one split operation; every operation reuses them)
  int n_kcnt = 0;
  int64_t n_kpart = 0;
};

// Vector width (bytes per lane load) for rows of K bf16 elements, or 0 when
// a row is not a multiple of 512 bytes.
int vec_bytes_for(int K);

// Check a configuration; returns MK_OK or MK_ERR_INVALID_CONFIG /
// MK_ERR_UNSUPPORTED with a message.
int check_config(const mk_config &c, std::string &err);

// Lower cfg into a task graph sized for n_cus CUs and give every one of
// n_workers persistent workgroups its task queue.
int build_host_plan(const mk_config &c, const mk_plan_options &o, int n_cus,
                    int n_workers, HostPlan &p, std::string &err);

// Structural checks: every waited event is signalled only by earlier tasks
// (list order is a topological order), thresholds equal the number of
// completions reported, no task waits on an event it signals, every worker
// queue is increasing in list order and reports each of its runs once.
int validate_plan(const HostPlan &p, std::string &err);

}  // namespace mk
