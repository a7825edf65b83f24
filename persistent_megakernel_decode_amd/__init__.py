"""Python binding of libmk.so (include/mk.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; PyTorch is
used for device memory and streams.  Importing this package loads the
in-tree ``libmk.so`` and raises if it is missing -- there is no fallback.

    import persistent_megakernel_decode_amd as mk
    plan = mk.Plan.build(desc, batch, kv_len)       # mk_plan_build
    plan.run(weights, kv_cache, tokens)             # mk_run (one persistent launch)
    plan.run_layerwise(weights, kv_cache, tokens)   # mk_run_layerwise (one launch per op)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK, MK_E_INVALID, MK_E_UNSUPPORTED, MK_E_NOMEM, MK_E_HIP, MK_E_TIMEOUT, MK_E_STATE = 0, -1, -2, -3, -4, -5, -6
MK_ABI_VERSION = 2
MK_ARCH_LLAMA, MK_ARCH_QWEN3, MK_ARCH_GLM_PREATTN = 1, 2, 3
MK_BF16, MK_FP8_E4M3_B128 = 0, 1
MK_LAYER_SLOTS = 11
MK_GLM_SLOTS = 13
MK_OUT_LOGITS, MK_OUT_NEXT_TOKEN, MK_OUT_QKV, MK_OUT_HIDDEN = 0, 1, 2, 3
(MK_OUT_GLM_R, MK_OUT_GLM_Q, MK_OUT_GLM_QIDX, MK_OUT_GLM_GATE, MK_OUT_GLM_NORM, MK_OUT_GLM_ACT,
 MK_OUT_GLM_ACT_SCALE, MK_OUT_GLM_QKVA, MK_OUT_GLM_QA, MK_OUT_GLM_QA_SCALE) = range(4, 14)
# element type of each output: "f32", "i32", "bf16" (returned as int16 bit patterns) or "u8"
OUTPUT_TYPES = {MK_OUT_LOGITS: "f32", MK_OUT_NEXT_TOKEN: "i32", MK_OUT_QKV: "f32", MK_OUT_HIDDEN: "f32",
                MK_OUT_GLM_R: "bf16", MK_OUT_GLM_Q: "bf16", MK_OUT_GLM_QIDX: "bf16", MK_OUT_GLM_GATE: "f32",
                MK_OUT_GLM_NORM: "f32", MK_OUT_GLM_ACT: "u8", MK_OUT_GLM_ACT_SCALE: "f32", MK_OUT_GLM_QKVA: "f32",
                MK_OUT_GLM_QA: "u8", MK_OUT_GLM_QA_SCALE: "f32"}
GLM_SLOTS = ("attn_norm", "w_qkva", "s_qkva", "w_gate", "s_gate", "w_idxk", "s_idxk", "q_a_norm", "kv_a_norm",
             "w_qb", "s_qb", "w_idxq", "s_idxq")
LAYER_SLOTS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
EXPORTED = ("mk_last_error", "mk_abi_version", "mk_plan_build", "mk_graph_plan", "mk_pair_plan", "mk_plan_export",
            "mk_run",
            "mk_run_layerwise", "mk_plan_output", "mk_plan_copy_output", "mk_plan_check", "mk_plan_set_trace",
            "mk_plan_trace", "mk_plan_free", "mk_plan_set_kv_len", "mk_run_steps", "mk_plan_debug_raise_wait",
            "mk_run_noalloc", "mk_noalloc_bytes", "mk_plan_poison_workspace", "mk_stream_probe")

# operand-table slot kinds (mk.h MK_SLOT_*)
MK_SLOT_NONE = 0
MK_SLOT_ATTN_NORM = 1
MK_SLOT_WQ = 2
MK_SLOT_WK = 3
MK_SLOT_WV = 4
MK_SLOT_Q_NORM = 5
MK_SLOT_K_NORM = 6
MK_SLOT_WO = 7
MK_SLOT_FFN_NORM = 8
MK_SLOT_W_GATE = 9
MK_SLOT_W_UP = 10
MK_SLOT_W_DOWN = 11
MK_SLOT_EMBED = 12
MK_SLOT_FINAL_NORM = 13
MK_SLOT_LM_HEAD = 14
MK_SLOT_TOKENS = 20
MK_SLOT_K_CACHE = 21
MK_SLOT_V_CACHE = 22
MK_SLOT_ROPE = 30
MK_SLOT_QKV = 31
MK_SLOT_ATTN_PART = 32
MK_SLOT_ATTN_OUT = 33
MK_SLOT_HIDDEN_ATTN = 34
MK_SLOT_HIDDEN_FFN = 35
MK_SLOT_FFN_ACT = 36
MK_SLOT_LOGITS = 37
MK_SLOT_LM_MAX = 38
MK_SLOT_NEXT_TOKEN = 39
MK_SLOT_SPLIT_ATTN, MK_SLOT_SPLIT_FFN, MK_SLOT_SUMSQ_ATTN, MK_SLOT_SUMSQ_FFN = 40, 41, 42, 43
MK_SLOT_G_X = 50
MK_SLOT_G_R = 51
MK_SLOT_G_ATTN_NORM = 52
MK_SLOT_G_W = 53
MK_SLOT_G_W_SCALE = 54
MK_SLOT_G_Q_A_NORM = 55
MK_SLOT_G_KV_A_NORM = 56
MK_SLOT_G_KV_CACHE = 57
MK_SLOT_G_IDX_CACHE = 58
MK_SLOT_G_ROWS = 59
MK_SLOT_G_R_OUT = 60
MK_SLOT_G_NORM = 61
MK_SLOT_G_ACT = 62
MK_SLOT_G_ACT_SCALE = 63
MK_SLOT_G_QKVA = 64
MK_SLOT_G_QA = 65
MK_SLOT_G_QA_SCALE = 66
MK_SLOT_G_Q = 67
MK_SLOT_G_QIDX = 68
MK_SLOT_G_GATE = 69
MK_SLOT_G_GATE_PART = 70
# mk_plan_view.tile_opts, in order
TILE_OPTS = ("num_cus", "gemv_rows", "gateup_outs", "down_rows", "lm_rows", "attn_splits")

i32, u32, f32, vp, sz = ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class ModelDesc(ctypes.Structure):
    _fields_ = [("abi_version", u32), ("struct_size", u32), ("arch", i32), ("n_layers", i32), ("hidden", i32),
                ("n_q_heads", i32), ("n_kv_heads", i32), ("head_dim", i32), ("ffn", i32), ("vocab", i32),
                ("tied_lm_head", i32), ("qk_norm", i32), ("weight_dtype", i32), ("max_kv_len", i32),
                ("rms_eps", f32), ("rope_theta", f32), ("q_lora", i32), ("kv_lora", i32), ("rope_dim", i32),
                ("n_idx_heads", i32), ("idx_head_dim", i32), ("n_gate", i32), ("rows_per_seq", i32)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("num_cus", i32), ("gemv_rows", i32), ("gateup_outs", i32), ("down_rows", i32), ("lm_rows", i32),
                ("attn_splits", i32), ("timeout_ms", i32), ("dma_pages", i32), ("lw_streams", i32), ("pairing", i32),
                ("attn_order", i32), ("reserved", i32)]


class GraphOp(ctypes.Structure):
    _fields_ = [("opcode", i32), ("spec", i32), ("layer", i32), ("grid", i32 * 3)]


class GraphEdge(ctypes.Structure):
    _fields_ = [("prod", i32), ("cons", i32), ("out_map", i32 * 3), ("in_map", i32 * 3), ("has_extent", i32),
                ("extent", i32 * 4), ("ptile", i32 * 4), ("ctile", i32 * 4)]


# pairing strategies (mk.h MK_PAIR_*)
MK_PAIR_WHOLE, MK_PAIR_TILE, MK_PAIR_TILE_COVER, MK_PAIR_TILE_REDUCE = range(4)


class PairPub(ctypes.Structure):
    _fields_ = [("op", i32), ("map", i32 * 3), ("div", i32 * 3), ("sel", i32 * 3)]


class PairEdge(ctypes.Structure):
    _fields_ = [("pub", i32), ("cons", i32), ("strategy", i32), ("map", i32 * 3), ("div", i32 * 3)]


class PlanView(ctypes.Structure):
    _fields_ = [("num_cus", i32), ("max_len", i32), ("num_tasks", i32), ("num_events", i32), ("num_ops", i32),
                ("num_edges", i32), ("queue", vp), ("event_target", vp), ("event_first", vp), ("event_last", vp),
                ("task_trigger", vp), ("task_wait", vp), ("op_table", vp), ("edge_kept", vp),
                ("tile_opts", i32 * 6), ("op_slots", vp), ("task_trigger2", vp), ("task_wait2", vp),
                ("pairing", i32), ("attn_order", i32)]


class Weights(ctypes.Structure):
    _fields_ = [("layer_ptrs", vp), ("embed", vp), ("final_norm", vp), ("lm_head", vp)]


class Check(ctypes.Structure):
    _fields_ = [("epoch", u32), ("counters_ok", i32), ("bad_counters", i32), ("err_kind", i32), ("err_cu", i32),
                ("err_slot", i32), ("err_event", i32), ("err_value", u32), ("err_target", u32)]


class MKError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (status %d)" % (msg, status))
        self.status = status


_lib = None


def lib():
    """Load libmk.so (built by ``python -m persistent_megakernel_decode_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmk.so is not built: run python -m persistent_megakernel_decode_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.mk_last_error.restype = ctypes.c_char_p
        L.mk_abi_version.restype = ctypes.c_int
        L.mk_plan_build.argtypes = [P(ModelDesc), i32, vp, P(PlanOpts), P(vp)]
        L.mk_graph_plan.argtypes = [vp, i32, vp, i32, i32, P(vp)]
        L.mk_pair_plan.argtypes = [vp, i32, vp, i32, vp, i32, i32, P(vp)]
        L.mk_plan_export.argtypes = [vp, P(PlanView)]
        L.mk_run.argtypes = [vp, P(Weights), vp, vp, vp]
        L.mk_run_layerwise.argtypes = [vp, P(Weights), vp, vp, vp]
        L.mk_plan_set_kv_len.argtypes = [vp, vp, vp]
        L.mk_run_steps.argtypes = [vp, P(Weights), vp, vp, i32, vp, i32, vp]
        L.mk_plan_output.argtypes = [vp, i32, P(vp), P(sz)]
        L.mk_plan_copy_output.argtypes = [vp, i32, vp, sz, vp]
        L.mk_plan_check.argtypes = [vp, vp, P(Check)]
        L.mk_plan_set_trace.argtypes = [vp, i32]
        L.mk_plan_trace.argtypes = [vp, vp, vp, sz, P(ctypes.c_double)]
        L.mk_plan_debug_raise_wait.argtypes = [vp, i32, i32, i32]
        L.mk_plan_poison_workspace.argtypes = [vp, vp]
        L.mk_stream_probe.argtypes = [vp, sz, i32, i32, i32, i32, vp, vp]
        L.mk_run_noalloc.argtypes = [vp, P(Weights), vp, vp, vp, vp, vp]
        L.mk_noalloc_bytes.argtypes = [vp, P(sz), P(sz)]
        L.mk_plan_free.argtypes = [vp]
        L.mk_plan_free.restype = None
        for n in EXPORTED:
            if n not in ("mk_last_error", "mk_abi_version", "mk_plan_free"):
                getattr(L, n).restype = ctypes.c_int
        if L.mk_abi_version() != MK_ABI_VERSION:
            raise ImportError("libmk.so ABI version mismatch")
        _lib = L
    return _lib


def _check(st):
    if st != MK_OK:
        raise MKError(st, lib().mk_last_error().decode())


def model_desc(cfg, max_kv_len):
    """mk_model_desc from a workload dict (synth.config format)."""
    if cfg.get("arch") == "glm":
        d = ModelDesc(MK_ABI_VERSION, ctypes.sizeof(ModelDesc), MK_ARCH_GLM_PREATTN, 1, cfg["hidden"],
                      cfg["n_q_heads"], 0, cfg["head_dim"], 0, 0, 0, 0, MK_FP8_E4M3_B128, int(max_kv_len),
                      cfg["rms_eps"], cfg["rope_theta"])
        for k in ("q_lora", "kv_lora", "rope_dim", "n_idx_heads", "idx_head_dim", "n_gate", "rows_per_seq"):
            setattr(d, k, int(cfg[k]))
        return d
    return ModelDesc(MK_ABI_VERSION, ctypes.sizeof(ModelDesc),
                     MK_ARCH_QWEN3 if cfg.get("qk_norm") else MK_ARCH_LLAMA, cfg["n_layers"], cfg["hidden"],
                     cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"], cfg["vocab"],
                     int(cfg["tied"]), int(cfg["qk_norm"]), MK_BF16, int(max_kv_len), cfg["rms_eps"],
                     cfg["rope_theta"])


def _arr(view_ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype=dtype)
    buf = (ctypes.c_char * (n * np.dtype(dtype).itemsize)).from_address(view_ptr)
    return np.frombuffer(buf, dtype=dtype).copy()


class Plan:
    """An mk_plan: static schedule plus the device buffers it owns."""

    def __init__(self, handle, batch=None, vocab=None):
        self._h = vp(handle)
        self.batch, self.vocab = batch, vocab
        self._keep = None

    @classmethod
    def build(cls, cfg, batch, kv_len, max_kv_len, **opts):
        desc = model_desc(cfg, max_kv_len)
        kv = np.ascontiguousarray(kv_len, dtype=np.int32)
        o = PlanOpts()
        for k, v in opts.items():
            setattr(o, k, int(v))
        h = vp()
        _check(lib().mk_plan_build(ctypes.byref(desc), int(batch), kv.ctypes.data, ctypes.byref(o), ctypes.byref(h)))
        return cls(h.value, batch, cfg.get("vocab"))

    @classmethod
    def graph(cls, ops, edges, num_cus):
        """ops: [(opcode, grid[, spec, layer])],
        edges: [(prod, cons, out_map, in_map, extent|None, ptile, ctile)]"""
        OA = (GraphOp * max(1, len(ops)))()
        for i, op in enumerate(ops):
            opcode, grid = op[0], op[1]
            spec, layer = (op[2], op[3]) if len(op) > 2 else (0, 0)
            g = tuple(grid) + (1,) * (3 - len(grid))
            OA[i] = GraphOp(opcode, spec, layer, (i32 * 3)(*g))
        EA = (GraphEdge * max(1, len(edges)))()
        for i, (p, c, om, im, ext, pt, ct) in enumerate(edges):
            om = tuple(om) + (-1,) * (3 - len(om))
            im = tuple(im) + (-1,) * (3 - len(im))
            e = GraphEdge(p, c, (i32 * 3)(*om), (i32 * 3)(*im), 1 if ext is not None else 0)
            if ext is not None:
                pad = lambda v: tuple(v) + (1,) * (4 - len(v))
                e.extent, e.ptile, e.ctile = (i32 * 4)(*pad(ext)), (i32 * 4)(*pad(pt)), (i32 * 4)(*pad(ct))
            EA[i] = e
        h = vp()
        _check(lib().mk_graph_plan(OA, len(ops), EA, len(edges), num_cus, ctypes.byref(h)))
        return cls(h.value)

    @classmethod
    def pairs(cls, ops, pubs, edges, num_cus):
        """mk_pair_plan.  ops: [(opcode, grid)], pubs: [(op, map, div, sel)],
        edges: [(pub, cons, strategy, map, div)]; short tuples are padded (map
        and sel with -1, div with 1)."""
        pad = lambda v, f: tuple(v) + (f,) * (3 - len(v))
        OA = (GraphOp * max(1, len(ops)))()
        for i, (opcode, grid) in enumerate(ops):
            OA[i] = GraphOp(opcode, 0, 0, (i32 * 3)(*pad(grid, 1)))
        PA = (PairPub * max(1, len(pubs)))()
        for i, (op, mp, dv, sl) in enumerate(pubs):
            PA[i] = PairPub(op, (i32 * 3)(*pad(mp, -1)), (i32 * 3)(*pad(dv, 1)), (i32 * 3)(*pad(sl, -1)))
        EA = (PairEdge * max(1, len(edges)))()
        for i, (pb, c, st, mp, dv) in enumerate(edges):
            EA[i] = PairEdge(pb, c, st, (i32 * 3)(*pad(mp, -1)), (i32 * 3)(*pad(dv, 1)))
        h = vp()
        _check(lib().mk_pair_plan(OA, len(ops), PA, len(pubs), EA, len(edges), num_cus, ctypes.byref(h)))
        return cls(h.value)

    def export(self):
        v = PlanView()
        _check(lib().mk_plan_export(self._h, ctypes.byref(v)))
        C, L, T, E = v.num_cus, v.max_len, v.num_tasks, v.num_events
        return dict(num_cus=C, max_len=L, num_tasks=T, num_events=E,
                    queue=_arr(v.queue, C * L * 32, np.int32).reshape(C, L, 32),
                    event_target=_arr(v.event_target, E, np.uint32), event_first=_arr(v.event_first, E, np.int32),
                    event_last=_arr(v.event_last, E, np.int32), task_trigger=_arr(v.task_trigger, T, np.int32),
                    task_wait=_arr(v.task_wait, T, np.int32),
                    op_table=_arr(v.op_table, v.num_ops * 8, np.int32).reshape(v.num_ops, 8),
                    edge_kept=_arr(v.edge_kept, v.num_edges, np.uint8),
                    tile_opts=dict(zip(TILE_OPTS, list(v.tile_opts))),
                    op_slots=_arr(v.op_slots, v.num_ops * 16, np.int32).reshape(v.num_ops, 16),
                    task_trigger2=_arr(v.task_trigger2, T, np.int32), task_wait2=_arr(v.task_wait2, T, np.int32),
                    pairing=v.pairing, attn_order=v.attn_order)

    def run(self, weights, kv_cache, tokens, stream=None, layerwise=False):
        w = weights.struct if isinstance(weights, (DeviceWeights, GlmDeviceWeights)) else weights
        s = vp(stream.cuda_stream if stream is not None else current_stream())
        fn = lib().mk_run_layerwise if layerwise else lib().mk_run
        _check(fn(self._h, ctypes.byref(w), vp(kv_cache.data_ptr()), vp(tokens.data_ptr()), s))

    def run_layerwise(self, weights, kv_cache, tokens, stream=None):
        self.run(weights, kv_cache, tokens, stream, layerwise=True)

    def run_noalloc(self, weights, kv_cache, tokens, logits, next_tokens, stream=None):
        """mk_run_noalloc: the step with the plan's device state in the library's
        static buffer; logits (float32 [batch * vocab]) and next_tokens (int32
        [batch]) are the caller's device tensors."""
        w = weights.struct if isinstance(weights, DeviceWeights) else weights
        s = vp(stream.cuda_stream if stream is not None else current_stream())
        _check(lib().mk_run_noalloc(self._h, ctypes.byref(w), vp(kv_cache.data_ptr()), vp(tokens.data_ptr()),
                                    vp(logits.data_ptr()), vp(next_tokens.data_ptr()), s))

    def noalloc_bytes(self):
        """(bytes of the static buffer this plan needs, the buffer's size)"""
        need, limit = sz(), sz()
        _check(lib().mk_noalloc_bytes(self._h, ctypes.byref(need), ctypes.byref(limit)))
        return need.value, limit.value

    def poison_workspace(self, stream=None):
        """mk_plan_poison_workspace: every intermediate and output to NaN."""
        _check(lib().mk_plan_poison_workspace(self._h, vp(stream.cuda_stream if stream is not None
                                                            else current_stream())))

    def debug_raise_wait(self, event, delta, slot=0):
        """mk_plan_debug_raise_wait (tests of the watchdog); slot 0 every wait on
        the event, 1 first waits only, 2 second waits only."""
        _check(lib().mk_plan_debug_raise_wait(self._h, int(event), int(delta), int(slot)))

    def set_kv_len(self, kv_len, stream=None):
        """mk_plan_set_kv_len: the next step's sequence lengths, without replanning."""
        import torch
        kv = np.ascontiguousarray(kv_len, dtype=np.int32)
        if stream is not None:
            s = vp(stream.cuda_stream)
        else:  # a plan that has not run needs no stream (host-side patch only)
            s = vp(current_stream() if torch.cuda.is_available() else 0)
        _check(lib().mk_plan_set_kv_len(self._h, kv.ctypes.data, s))

    def run_steps(self, weights, kv_cache, tokens, n_steps, out_tokens=None, stream=None, layerwise=False):
        """mk_run_steps: n_steps decode steps, each fed the previous step's argmax;
        out_tokens: a device int32 tensor of n_steps * batch elements, or None."""
        w = weights.struct if isinstance(weights, (DeviceWeights, GlmDeviceWeights)) else weights
        s = vp(stream.cuda_stream if stream is not None else current_stream())
        o = vp(out_tokens.data_ptr()) if out_tokens is not None else vp(0)
        _check(lib().mk_run_steps(self._h, ctypes.byref(w), vp(kv_cache.data_ptr()), vp(tokens.data_ptr()),
                                  int(n_steps), o, 1 if layerwise else 0, s))

    def output(self, which):
        """Copy an output into a new flat torch tensor (on the current stream):
        float32, int32, int16 (bf16 bit patterns) or uint8 (E4M3 codes)."""
        import torch
        p, n = vp(), sz()
        _check(lib().mk_plan_output(self._h, which, ctypes.byref(p), ctypes.byref(n)))
        dt, isz = {"f32": (torch.float32, 4), "i32": (torch.int32, 4), "bf16": (torch.int16, 2),
                   "u8": (torch.uint8, 1)}[OUTPUT_TYPES[which]]
        out = torch.empty(n.value // isz, dtype=dt, device="cuda")
        _check(lib().mk_plan_copy_output(self._h, which, vp(out.data_ptr()), n.value, vp(current_stream())))
        return out

    def check(self, stream=None):
        c = Check()
        st = lib().mk_plan_check(self._h, vp(stream.cuda_stream if stream is not None else current_stream()),
                                 ctypes.byref(c))
        return st, c

    def set_trace(self, enable):
        _check(lib().mk_plan_set_trace(self._h, 1 if enable else 0))

    def trace(self, stream=None):
        ex = self.export()
        out = np.zeros((ex["num_cus"], ex["max_len"], 16), dtype=np.uint64)
        tpu = ctypes.c_double()
        _check(lib().mk_plan_trace(self._h, vp(stream.cuda_stream if stream is not None else current_stream()),
                                   out.ctypes.data, out.nbytes, ctypes.byref(tpu)))
        return out, tpu.value

    def free(self):
        if self._h:
            lib().mk_plan_free(self._h)
            self._h = vp()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def current_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


class DeviceWeights:
    """Upload host weights (synth.make_weights format: uint16 bf16 bits) to the
    current GPU as bf16 tensors and hold the mk_weights pointer table."""

    def __init__(self, host_weights, cfg):
        import torch

        def dev(a):
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
            return t.to("cuda", non_blocking=False)

        self.tensors = []
        L = cfg["n_layers"]
        self.table = (vp * (L * MK_LAYER_SLOTS))()
        for l in range(L):
            for s, name in enumerate(LAYER_SLOTS):
                a = host_weights["layers"][l].get(name)
                if a is not None:
                    t = dev(a)
                    self.tensors.append(t)
                    self.table[l * MK_LAYER_SLOTS + s] = t.data_ptr()
        self.embed = dev(host_weights["embed"])
        self.final_norm = dev(host_weights["final_norm"])
        self.lm_head = dev(host_weights["lm_head"]) if "lm_head" in host_weights else None
        self.struct = Weights(ctypes.cast(self.table, vp), self.embed.data_ptr(), self.final_norm.data_ptr(),
                              self.lm_head.data_ptr() if self.lm_head is not None else None)


def kv_to_device(kv_host):
    import torch
    return torch.from_numpy(np.ascontiguousarray(kv_host).view(np.int16)).view(torch.bfloat16).to("cuda")


def tokens_to_device(tokens):
    import torch
    return torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to("cuda")


class GlmDeviceWeights:
    """Upload GLM pre-attention weights (synth.make_glm_inputs format: bf16 norm
    bits, E4M3 codes, fp32 block scales) and hold the mk_weights table."""

    def __init__(self, host_weights):
        import torch
        self.tensors = []
        self.table = (vp * MK_GLM_SLOTS)()
        for k, name in enumerate(GLM_SLOTS):
            a = np.ascontiguousarray(host_weights[name])
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            t = torch.from_numpy(a).to("cuda")
            self.tensors.append(t)
            self.table[k] = t.data_ptr()
        self.struct = Weights(ctypes.cast(self.table, vp), None, None, None)


def glm_inputs_to_device(x, r):
    """bf16 [2][M][hidden] device tensor (x, then r) from uint16 bit arrays."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.stack([x, r])).view(np.int16)).to("cuda")


def glm_caches_to_device(kv_cache, idx_cache):
    """One bf16 device buffer: the KV cache followed by the indexer cache."""
    import torch
    flat = np.concatenate([np.ascontiguousarray(kv_cache).ravel(), np.ascontiguousarray(idx_cache).ravel()])
    return torch.from_numpy(flat.view(np.int16)).to("cuda")


def stream_probe(buf, lds_dma, workgroups, waves, depth, sink, stream=None):
    """mk_stream_probe: one streaming read of the device tensor buf."""
    s = vp(stream.cuda_stream if stream is not None else current_stream())
    _check(lib().mk_stream_probe(vp(buf.data_ptr()), buf.numel() * buf.element_size(), int(lds_dma),
                                 int(workgroups), int(waves), int(depth), vp(sink.data_ptr()), s))
