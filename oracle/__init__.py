"""CPU oracle for the decode step and the tile plan -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP library
(``persistent_megakernel_decode_amd``) and never imports it; the two meet only
through the seeded inputs of ``synth``.

* ``oracle.c``    -- the decode step in plain C (fp64; an fp32 build of the same
                     source is kept beside it), with per-op functions for pins.
* ``planner.py``  -- the tile-plan reference (DAG -> events -> queues).
* ``replay.py``   -- executes a plan's queues on the CPU (serial or random
                     interleavings) with a happens-before checker.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB64 = os.path.join(_HERE, "liboracle.so")
LIB32 = os.path.join(_HERE, "liboracle_f32.so")
N_SLOTS = 11
SLOT_NAMES = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def build(force=False):
    """Compile the fp64 and fp32 builds of oracle.c with gcc."""
    src = os.path.join(_HERE, "oracle.c")
    for path, real in ((LIB64, "double"), (LIB32, "float")):
        if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            tmp = path + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                                   "-DORACLE_REAL=" + real, "-o", tmp, src, "-lm"])
            os.replace(tmp, path)


class _Model(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("tied", ctypes.c_int), ("qk_norm", ctypes.c_int),
                ("kv_capacity", ctypes.c_int), ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double),
                ("round_new_kv", ctypes.c_int)]


_libs = {}


def lib(precision="f64"):
    if precision not in _libs:
        path = LIB64 if precision == "f64" else LIB32
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        vp, ci, cd = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.oracle_decode_step.argtypes = [ctypes.POINTER(_Model), vp, ci, vp, vp, vp, vp, vp]
        L.oracle_decode_step.restype = ci
        L.oracle_decode_step_ex.argtypes = [ctypes.POINTER(_Model), vp, ci, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_decode_step_ex.restype = ci
        L.oracle_rmsnorm.argtypes = [ci, vp, vp, cd, vp]
        L.oracle_matvec.argtypes = [ci, ci, vp, vp, vp]
        L.oracle_rope.argtypes = [ci, ci, cd, vp]
        L.oracle_attend.argtypes = [ci, ci, vp, vp, vp, ci, vp, vp, vp]
        L.oracle_argmax.argtypes = [ci, vp]
        L.oracle_argmax.restype = ci
        L.oracle_to_bf16.argtypes = [cd]
        L.oracle_to_bf16.restype = ctypes.c_uint16
        L.oracle_real_bytes.restype = ci
        _libs[precision] = L
    return _libs[precision]


def _dt(precision):
    return np.float64 if precision == "f64" else np.float32


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16 array) to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(v, precision="f64"):
    return int(lib(precision).oracle_to_bf16(float(v)))


def rmsnorm(x, w_bits, eps, precision="f64"):
    x = np.ascontiguousarray(x, dtype=_dt(precision))
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    y = np.empty_like(x)
    lib(precision).oracle_rmsnorm(x.size, _p(x), _p(w), eps, _p(y))
    return y


def matvec(W_bits, x, precision="f64"):
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=_dt(precision))
    out = np.empty(W.shape[0], dtype=_dt(precision))
    lib(precision).oracle_matvec(W.shape[0], W.shape[1], _p(W), _p(x), _p(out))
    return out


def rope(v, pos, theta, precision="f64"):
    v = np.array(v, dtype=_dt(precision))
    lib(precision).oracle_rope(v.size, pos, theta, _p(v))
    return v


def attend(q, K_bits, V_bits, special=-1, knew=None, vnew=None, precision="f64"):
    dt = _dt(precision)
    q = np.ascontiguousarray(q, dtype=dt)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    d = q.size
    kn = np.ascontiguousarray(knew if knew is not None else np.zeros(d), dtype=dt)
    vn = np.ascontiguousarray(vnew if vnew is not None else np.zeros(d), dtype=dt)
    out = np.empty(d, dtype=dt)
    lib(precision).oracle_attend(d, K.shape[0], _p(q), _p(K), _p(V), special, _p(kn), _p(vn), _p(out))
    return out


def argmax(v, precision="f64"):
    v = np.ascontiguousarray(v, dtype=_dt(precision))
    return int(lib(precision).oracle_argmax(v.size, _p(v)))


def decode_step(inputs, precision="f64", round_new_kv=True, kv_cache=None, intermediates=False):
    """Run one decode step on the host.

    ``inputs`` is the dict made by ``synth.make_inputs``.  The KV cache is
    copied (or ``kv_cache`` is updated in place when given).  Returns
    dict(logits [B, V], next [B] int32, kv_cache), and with ``intermediates``
    also hidden [L, 2, B, H] (residual stream after each layer's attention and
    FFN blocks) and qkv [L, B, n_q + 2 n_kv, head_dim] (projections before the
    q/k norm and RoPE).
    """
    cfg, w = inputs["cfg"], inputs["weights"]
    L, B = cfg["n_layers"], cfg["batch"]
    kv = inputs["kv_cache"].copy() if kv_cache is None else kv_cache
    m = _Model(L, cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"],
               cfg["vocab"], int(cfg["tied"]), int(cfg["qk_norm"]), kv.shape[4], cfg["rms_eps"],
               cfg["rope_theta"], 1 if round_new_kv else 0)
    keep = []
    table = (ctypes.c_void_p * (L * N_SLOTS + 3))()
    for l in range(L):
        for s, name in enumerate(SLOT_NAMES):
            a = w["layers"][l].get(name)
            if a is not None:
                a = np.ascontiguousarray(a)
                keep.append(a)
                table[l * N_SLOTS + s] = a.ctypes.data
    for j, name in enumerate(("embed", "final_norm", "lm_head")):
        a = w.get(name)
        if a is not None:
            a = np.ascontiguousarray(a)
            keep.append(a)
            table[L * N_SLOTS + j] = a.ctypes.data
    kv_len = np.ascontiguousarray(inputs["kv_len"], dtype=np.int32)
    tokens = np.ascontiguousarray(inputs["tokens"], dtype=np.int32)
    logits = np.empty((B, cfg["vocab"]), dtype=_dt(precision))
    nxt = np.empty(B, dtype=np.int32)
    hid = qkv = None
    if intermediates:
        nh = cfg["n_q_heads"] + 2 * cfg["n_kv_heads"]
        hid = np.empty((L, 2, B, cfg["hidden"]), dtype=_dt(precision))
        qkv = np.empty((L, B, nh, cfg["head_dim"]), dtype=_dt(precision))
    rc = lib(precision).oracle_decode_step_ex(ctypes.byref(m), ctypes.cast(table, ctypes.c_void_p), B,
                                              _p(kv_len), _p(tokens), _p(kv), _p(logits), _p(nxt),
                                              _p(hid) if hid is not None else None,
                                              _p(qkv) if qkv is not None else None)
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    out = dict(logits=logits, next=nxt, kv_cache=kv)
    if intermediates:
        out.update(hidden=hid, qkv=qkv)
    return out
