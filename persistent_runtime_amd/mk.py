"""ctypes binding of libmk.so (include/mk.h), same names as the C ABI.

Argument marshalling only: every step of the decode path runs in the HIP
library.  PyTorch is used by callers for device memory and streams; this
module takes raw device pointers (ints) or torch tensors and passes them on.
Importing this module loads the library and raises if it is missing: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MK_LIB", os.path.join(HERE, "libmk.so"))

MK_OK = 0
MK_ERR_INVALID_CONFIG = -1
MK_ERR_INVALID_ARG = -2
MK_ERR_HIP = -3
MK_ERR_OOM = -4
MK_ERR_PLAN = -5
MK_ERR_TIMEOUT = -6
MK_ERR_UNSUPPORTED = -7
MK_EXEC_PERSISTENT = 0
MK_EXEC_KERNEL_PER_OP = 1
MK_EXEC_SCHEDULED = 2

OPS = {1: "EMBED", 2: "QKV", 3: "ATTN", 4: "MERGE", 5: "OPROJ", 6: "GATEUP",
       7: "DOWN", 8: "ROUTER", 9: "TOPK", 10: "EGATEUP", 11: "EDOWN",
       12: "COMBINE", 13: "LMHEAD", 14: "ARGMAX", 15: "KVAPP"}
OP_ID = {v: k for k, v in OPS.items()}

# every function include/mk.h declares
EXPORTS = ["mk_plan_options_default", "mk_build_plan", "mk_decode_step",
           "mk_prefill", "mk_plan_status", "mk_free", "mk_last_error",
           "mk_build_id", "mk_inspect_plan", "mk_read_trace", "mk_plan_info",
           "mk_read_routing", "mk_build_plan_noalloc", "mk_batch_step"]


class mk_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_double), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("expert_ffn_dim", C.c_int32),
                ("max_batch", C.c_int32), ("page_size", C.c_int32),
                ("max_pages_per_seq", C.c_int32), ("n_pages", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class mk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p),
                ("final_norm", C.c_void_p), ("attn_norm", _PP),
                ("ffn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP),
                ("wo", _PP), ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP),
                ("router", _PP), ("e_gate", _PP), ("e_up", _PP),
                ("e_down", _PP)]


class mk_kv(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
                ("page_table", C.c_void_p)]


class mk_plan_options(C.Structure):
    _fields_ = [("executor", C.c_int32), ("n_workgroups", C.c_int32),
                ("attn_splits", C.c_int32), ("planned_ctx", C.c_int32),
                ("debug_trace", C.c_int32), ("device", C.c_int32),
                ("spin_budget", C.c_int64), ("n_cus", C.c_int32),
                ("graph_replay", C.c_int32), ("batched_mfma", C.c_int32),
                ("attn_pool", C.c_int32), ("weight_lds", C.c_int32),
                ("debug_withhold", C.c_int32), ("shared_seqs", C.c_int32),
                ("prefill_chunk", C.c_int32), ("attn_order", C.c_int32)]


class mk_task_info(C.Structure):
    _fields_ = [("op", C.c_int32), ("layer", C.c_int32), ("a0", C.c_int32),
                ("a1", C.c_int32), ("a2", C.c_int32), ("a3", C.c_int32),
                ("a4", C.c_int32), ("sig_count", C.c_int32), ("n_wait", C.c_int32),
                ("wait_ev", C.c_int32 * 3), ("n_sig", C.c_int32),
                ("sig_ev", C.c_int32 * 2), ("phase", C.c_int32),
                ("worker", C.c_int32), ("rows_per_pass", C.c_int32),
                ("bytes", C.c_int64), ("data_edges", C.c_int32), ("pad_", C.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmk.so not found at {LIB_PATH}; build it with "
            "`python -m persistent_runtime_amd.build` (there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    lib.mk_build_id.restype = C.c_char_p
    from .build import source_hash
    built, want = lib.mk_build_id().decode(), source_hash()
    if built != want and not os.environ.get("MK_LIB"):
        raise ImportError(
            f"{LIB_PATH} was built from other sources (build id {built}, sources {want}); "
            "rebuild it with `python -m persistent_runtime_amd.build`")
    vp, i32, pi32 = C.c_void_p, C.c_int32, C.POINTER(C.c_int32)
    lib.mk_plan_options_default.argtypes = [C.POINTER(mk_plan_options)]
    lib.mk_plan_options_default.restype = None
    lib.mk_build_plan.argtypes = [C.POINTER(mk_config), C.POINTER(mk_weights),
                                  C.POINTER(mk_kv), C.POINTER(mk_plan_options),
                                  C.POINTER(vp)]
    lib.mk_build_plan_noalloc.argtypes = lib.mk_build_plan.argtypes
    lib.mk_decode_step.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.mk_prefill.argtypes = [vp, i32, vp, i32, i32, vp, vp, vp]
    lib.mk_batch_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mk_plan_status.argtypes = [vp, vp]
    lib.mk_free.argtypes = [vp]
    lib.mk_free.restype = None
    lib.mk_last_error.restype = C.c_char_p
    lib.mk_inspect_plan.argtypes = [C.POINTER(mk_config), C.POINTER(mk_plan_options),
                                    C.POINTER(mk_task_info), i32, pi32, pi32, i32, pi32]
    lib.mk_read_trace.argtypes = [vp, vp, C.POINTER(C.c_uint32), i32]
    lib.mk_plan_info.argtypes = [vp, pi32, pi32, pi32, pi32]
    lib.mk_read_routing.argtypes = [vp, vp, pi32, C.POINTER(C.c_float), i32]
    for f in ("mk_build_plan", "mk_build_plan_noalloc", "mk_decode_step", "mk_prefill",
              "mk_plan_status", "mk_batch_step",
              "mk_inspect_plan", "mk_read_trace", "mk_plan_info", "mk_read_routing"):
        getattr(lib, f).restype = C.c_int
    return lib


lib = _load()


class MkError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != MK_OK:
        raise MkError(rc, lib.mk_last_error().decode())
    return rc


def last_error() -> str:
    return lib.mk_last_error().decode()


def make_config(model: dict, max_batch=1, max_pages_per_seq=64, n_pages=None) -> mk_config:
    c = mk_config()
    c.n_layers, c.hidden = model["n_layers"], model["hidden"]
    c.n_q_heads, c.n_kv_heads = model["n_q_heads"], model["n_kv_heads"]
    c.head_dim, c.ffn_dim, c.vocab = model["head_dim"], model["ffn_dim"], model["vocab"]
    c.rms_eps, c.rope_theta = model["rms_eps"], model["rope_theta"]
    c.n_experts, c.top_k = model["n_experts"], model["top_k"]
    c.expert_ffn_dim = model["expert_ffn_dim"]
    c.max_batch, c.page_size = max_batch, 16
    c.max_pages_per_seq = max_pages_per_seq
    c.n_pages = n_pages if n_pages is not None else max_batch * max_pages_per_seq
    return c


def default_options(**kw) -> mk_plan_options:
    o = mk_plan_options()
    lib.mk_plan_options_default(C.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def inspect_plan(cfg: mk_config, opts: mk_plan_options | None = None):
    """Run the planner on the host only; returns (tasks, thresholds) as lists."""
    nt, ne = C.c_int32(0), C.c_int32(0)
    o = C.byref(opts) if opts is not None else None
    _check(lib.mk_inspect_plan(C.byref(cfg), o, None, 0, C.byref(nt), None, 0, C.byref(ne)))
    tasks = (mk_task_info * nt.value)()
    thr = (C.c_int32 * ne.value)()
    _check(lib.mk_inspect_plan(C.byref(cfg), o, tasks, nt.value, C.byref(nt), thr,
                               ne.value, C.byref(ne)))
    return list(tasks), list(thr)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ptr_array(ptrs):
    arr = (C.c_void_p * len(ptrs))(*ptrs)
    return arr


class Plan:
    """A built plan over torch-owned device tensors.

    `W` is the synth weight dictionary (bf16 tensors on the device, per-layer
    tensors stacked on axis 0); `k_pool`, `v_pool` bf16
    [L, n_pages, nkv, 16, hd] and [L, n_pages, nkv, hd, 16] (values transposed
    within a page, as include/mk.h states); `page_table` int32
    [max_batch, max_pages].
    The Plan keeps references to all of them.
    """

    def __init__(self, model: dict, W: dict, k_pool, v_pool, page_table,
                 max_batch=1, opts: mk_plan_options | None = None, noalloc=False):
        L = model["n_layers"]
        self.model, self.W = model, W
        self.k_pool, self.v_pool, self.page_table = k_pool, v_pool, page_table
        self.cfg = make_config(model, max_batch, page_table.shape[1], k_pool.shape[1])
        w = mk_weights()
        w.embed, w.lm_head, w.final_norm = _ptr(W["embed"]), _ptr(W["lm_head"]), _ptr(W["final_norm"])
        keep = []

        def per_layer(name):
            t = W[name]
            a = _ptr_array([t[l].data_ptr() for l in range(L)])
            keep.append(a)
            return C.cast(a, _PP)

        def per_expert(name):
            t = W[name]
            E = t.shape[1]
            a = _ptr_array([t[l, e].data_ptr() for l in range(L) for e in range(E)])
            keep.append(a)
            return C.cast(a, _PP)

        for n in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo"):
            setattr(w, n, per_layer(n))
        if model["n_experts"] == 0:
            for n in ("w_gate", "w_up", "w_down"):
                setattr(w, n, per_layer(n))
        else:
            w.router = per_layer("router")
            for n in ("e_gate", "e_up", "e_down"):
                setattr(w, n, per_expert(n))
        kv = mk_kv(k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr())
        self.opts = opts if opts is not None else default_options()
        h = C.c_void_p()
        build = lib.mk_build_plan_noalloc if noalloc else lib.mk_build_plan
        _check(build(C.byref(self.cfg), C.byref(w), C.byref(kv), C.byref(self.opts),
                     C.byref(h)))
        self.handle = h

    @staticmethod
    def _stream(stream):
        if stream is None:
            import torch
            return C.c_void_p(torch.cuda.current_stream().cuda_stream)
        return C.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)

    def decode_step(self, tokens, positions, next_tokens, logits=None, stream=None):
        _check(lib.mk_decode_step(self.handle, _ptr(tokens), _ptr(positions),
                                  self._stream(stream), _ptr(next_tokens), _ptr(logits)))

    def batch_step(self, tokens, positions, seq_rows, next_tokens, logits=None, stream=None,
                   priorities=None):
        _check(lib.mk_batch_step(self.handle, _ptr(tokens), _ptr(positions), _ptr(seq_rows),
                                 _ptr(priorities), self._stream(stream), _ptr(next_tokens),
                                 _ptr(logits)))

    def prefill(self, slot, tokens, n, start_pos, next_token=None, logits=None, stream=None):
        _check(lib.mk_prefill(self.handle, slot, _ptr(tokens), n, start_pos,
                              self._stream(stream), _ptr(next_token), _ptr(logits)))

    def status(self, stream=None):
        return lib.mk_plan_status(self.handle, self._stream(stream))

    def check(self, stream=None):
        _check(self.status(stream))

    def info(self):
        a, b, c, d = (C.c_int32(), C.c_int32(), C.c_int32(), C.c_int32())
        _check(lib.mk_plan_info(self.handle, C.byref(a), C.byref(b), C.byref(c), C.byref(d)))
        return dict(n_tasks=a.value, n_events=b.value, n_cus=c.value, n_phases=d.value)

    def read_trace(self, stream=None):
        import numpy as np
        n = self.info()["n_tasks"]
        buf = (C.c_uint32 * (6 * n))()
        _check(lib.mk_read_trace(self.handle, self._stream(stream), buf, n))
        return np.frombuffer(buf, dtype=np.uint32).reshape(n, 6).copy()

    def read_routing(self, stream=None):
        """Expert ids and weights of the last step: ([L, B, top_k] int32, float32)."""
        import numpy as np
        m = self.model
        n = m["n_layers"] * self.cfg.max_batch * m["top_k"]
        ids = (C.c_int32 * n)()
        w = (C.c_float * n)()
        _check(lib.mk_read_routing(self.handle, self._stream(stream), ids, w, n))
        shape = (m["n_layers"], self.cfg.max_batch, m["top_k"])
        return (np.frombuffer(ids, dtype=np.int32).reshape(shape).copy(),
                np.frombuffer(w, dtype=np.float32).reshape(shape).copy())

    def free(self):
        if getattr(self, "handle", None):
            lib.mk_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
