"""Seeded synthetic inputs for the decode-step workloads.

This package is shared by the CPU oracle (``oracle/``) and the HIP library's
tests and benchmark.  It holds no arithmetic of the decode step itself: only
the workload shapes and the seeded random draws (see ``synth.c`` for the
stream definition), returned as host numpy arrays.  bf16 values are carried
as ``uint16`` bit patterns.

Workloads (weights ~N(0, 0.02) bf16, norm weights 1.0, prior KV rows ~N(0, 1)
bf16, KV rows at and beyond ``kv_len`` poisoned with NaN, token ids uniform):

* ``tiny``        2 layers, hidden 256, 4 q / 2 kv heads, head_dim 64, FFN 688,
                  vocab 4096, tied LM head, batch 1, 128 prior KV rows.
* ``llama1b``     Llama-3.2-1B shape: 16 layers, hidden 2048, 32 q / 8 kv heads,
                  head_dim 64, FFN 8192, vocab 128256, tied, batch 1, KV 1024.
* ``llama1b_b16`` the same shape at batch 16, per-sequence KV length uniform
                  in [512, 2048].
* ``qwen3_8b``    Qwen3-8B shape: 36 layers, hidden 4096, 32 q / 8 kv heads,
                  head_dim 128, per-head q/k RMSNorm, FFN 12288, vocab 151936,
                  untied LM head, batch 1, KV 4096.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

BF16_ONE = 0x3F80
BF16_NAN = 0x7FC0
KV_POS_STRIDE = 1 << 20  # stream positions reserved per (seq, kv head) for KV rows


def build(force=False):
    """Compile libsynth.so with gcc (OpenMP for speed; results do not depend on threads)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [u64, u64, dbl, dbl, u64, u64, vp]
        lib.synth_normal_bf16_2d.argtypes = [u64, u64, dbl, dbl, u64, u64, u64, u64, vp]
        lib.synth_normal_f64.argtypes = [u64, u64, dbl, dbl, u64, u64, vp]
        lib.synth_uniform_i32.argtypes = [u64, u64, i64, i64, u64, vp]
        lib.synth_fill_u16.argtypes = [ctypes.c_uint16, u64, vp]
        lib.synth_mix.argtypes = [u64]
        lib.synth_mix.restype = u64
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.synth_f32_to_bf16.restype = ctypes.c_uint16
        lib.synth_fp8_weights.argtypes = [u64, u64, dbl, u64, u64, vp, vp]
        lib.synth_e4m3_code.argtypes = [dbl]
        lib.synth_e4m3_code.restype = ctypes.c_uint8
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_bf16(seed, tid, shape, sigma, mean=0.0, offset=0, out=None):
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(seed, tid, mean, sigma, offset, n, _ptr(out))
    return out


def normal_f64(seed, tid, shape, sigma=1.0, mean=0.0, offset=0):
    out = np.empty(shape, dtype=np.float64)
    _load().synth_normal_f64(seed, tid, mean, sigma, offset, out.size, _ptr(out))
    return out


def uniform_i32(seed, tid, lo, hi, n):
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_i32(seed, tid, lo, hi, n, _ptr(out))
    return out


def mix64(x):
    return int(_load().synth_mix(x))


def f32_to_bf16_bits(f):
    return int(_load().synth_f32_to_bf16(float(f)))


def fp8_weights(seed, tid, N, K, sigma=0.02):
    """[N, K] OCP e4m3 codes (uint8) and [ceil(N/128), K/128] fp32 block scales."""
    assert K % 128 == 0
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty(((N + 127) // 128, K // 128), dtype=np.float32)
    _load().synth_fp8_weights(seed, tid, sigma, N, K, _ptr(codes), _ptr(scales))
    return codes, scales


def e4m3_code(v):
    return int(_load().synth_e4m3_code(float(v)))


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------
CONFIGS = {
    "tiny": dict(arch="llama", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 ffn=688, vocab=4096, tied=1, qk_norm=0, rms_eps=1e-5, rope_theta=1e4,
                 batch=1, kv_len=128, seed=1000),
    "llama1b": dict(arch="llama", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                    ffn=8192, vocab=128256, tied=1, qk_norm=0, rms_eps=1e-5, rope_theta=1e4,
                    batch=1, kv_len=1024, seed=1001),
    "llama1b_b16": dict(arch="llama", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                        ffn=8192, vocab=128256, tied=1, qk_norm=0, rms_eps=1e-5, rope_theta=1e4,
                        batch=16, kv_len=(512, 2048), seed=1002),
    "qwen3_8b": dict(arch="qwen3", n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     ffn=12288, vocab=151936, tied=0, qk_norm=1, rms_eps=1e-5, rope_theta=1e4,
                     batch=1, kv_len=4096, seed=1003),
}

# GLM-style pre-attention path (one layer's prologue before sparse MLA):
# M token rows = n_seqs requests x rows_per_seq tokens, token t of request r at
# cache position pos0 + t.  Column layout of the QKV-A output:
# [q_lora | kv_lora | rope_dim]; each query head is head_dim = nope + rope_dim.
GLM_CONFIGS = {
    "glm_preattn": dict(arch="glm", hidden=6144, q_lora=1536, kv_lora=512, rope_dim=64, n_q_heads=64,
                        head_dim=192, n_idx_heads=32, idx_head_dim=128, n_gate=64, n_seqs=2, rows_per_seq=8,
                        pos0=8192, rms_eps=1e-5, rope_theta=1e4, seed=1004),
    "glm_tiny": dict(arch="glm", hidden=512, q_lora=256, kv_lora=128, rope_dim=64, n_q_heads=4,
                     head_dim=192, n_idx_heads=2, idx_head_dim=128, n_gate=16, n_seqs=2, rows_per_seq=3,
                     pos0=100, rms_eps=1e-5, rope_theta=1e4, seed=1005),
}
CONFIGS.update(GLM_CONFIGS)
# GLM weight slots, in this fixed order: norms bf16, linear weights fp8 [out, in]
# with fp32 [ceil(out/128), in/128] block scales.
GLM_SLOTS = ("attn_norm", "w_qkva", "s_qkva", "w_gate", "s_gate", "w_idxk", "s_idxk", "q_a_norm", "kv_a_norm",
             "w_qb", "s_qb", "w_idxq", "s_idxq")
TID_GLM = 30000


def glm_dims(cfg):
    """(M, N_qkva, N_qb, N_idxq) of a GLM config."""
    M = cfg["n_seqs"] * cfg["rows_per_seq"]
    return (M, cfg["q_lora"] + cfg["kv_lora"] + cfg["rope_dim"], cfg["n_q_heads"] * cfg["head_dim"],
            cfg["n_idx_heads"] * cfg["idx_head_dim"])


def glm_positions(cfg):
    """cache position and request of each token row"""
    M = cfg["n_seqs"] * cfg["rows_per_seq"]
    m = np.arange(M)
    return (cfg["pos0"] + m % cfg["rows_per_seq"]).astype(np.int32), (m // cfg["rows_per_seq"]).astype(np.int32)


def glm_capacity(cfg):
    return int((cfg["pos0"] + cfg["rows_per_seq"] + 15) // 16 * 16)


def make_glm_inputs(name, norm_sigma=0.0, **overrides):
    """All inputs of the GLM pre-attention step: dict(cfg, weights, x, r, pos, req,
    kv_cache [n_seqs][cap][kv_lora + rope_dim], idx_cache [n_seqs][cap][idx_head_dim]).
    x, r ~N(0,1) bf16 [M, hidden]; fp8 weights ~N(0, 0.02) quantized per block;
    norm weights 1.0 (or ~N(1, norm_sigma)); both caches all NaN (the step
    writes only the rows of its tokens)."""
    cfg = config(name, **overrides)
    seed, H, QL = cfg["seed"], cfg["hidden"], cfg["q_lora"]
    M, Nqkva, Nqb, Niq = glm_dims(cfg)
    shapes = {"w_qkva": (Nqkva, H), "w_gate": (cfg["n_gate"], H), "w_idxk": (cfg["idx_head_dim"], H),
              "w_qb": (Nqb, QL), "w_idxq": (Niq, QL)}
    norms = {"attn_norm": H, "q_a_norm": QL, "kv_a_norm": cfg["kv_lora"]}
    w = {}
    for i, s in enumerate(GLM_SLOTS):
        if s in shapes:
            w[s], w["s_" + s[2:]] = fp8_weights(seed, TID_GLM + i, *shapes[s])
        elif s in norms:
            w[s] = (np.full(norms[s], BF16_ONE, dtype=np.uint16) if norm_sigma == 0.0 else
                    normal_bf16(seed, TID_GLM + i, (norms[s],), norm_sigma, mean=1.0))
    x = normal_bf16(seed, TID_GLM + 100, (M, H), 1.0)
    r = normal_bf16(seed, TID_GLM + 101, (M, H), 1.0)
    pos, req = glm_positions(cfg)
    cap = glm_capacity(cfg)
    kvc = np.full((cfg["n_seqs"], cap, cfg["kv_lora"] + cfg["rope_dim"]), BF16_NAN, dtype=np.uint16)
    idc = np.full((cfg["n_seqs"], cap, cfg["idx_head_dim"]), BF16_NAN, dtype=np.uint16)
    return dict(cfg=cfg, weights=w, x=x, r=r, pos=pos, req=req, kv_cache=kvc, idx_cache=idc)


# Per-layer weight slots, in this fixed order.  Shapes are [out, in] row-major.
LAYER_SLOTS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate", "w_up", "w_down")

TID_EMBED, TID_FINAL_NORM, TID_LM_HEAD = 1, 2, 3
TID_TOKENS, TID_KV_LEN = 20000, 20001


def tid_layer(layer, slot):
    return 100 + layer * 16 + LAYER_SLOTS.index(slot)


def tid_kv(layer, kind):
    return 10000 + layer * 2 + kind


def config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def slot_shape(cfg, slot):
    H, hd, F = cfg["hidden"], cfg["head_dim"], cfg["ffn"]
    nq, nkv = cfg["n_q_heads"], cfg["n_kv_heads"]
    return {
        "attn_norm": (H,), "ffn_norm": (H,), "q_norm": (hd,), "k_norm": (hd,),
        "wq": (nq * hd, H), "wk": (nkv * hd, H), "wv": (nkv * hd, H), "wo": (H, nq * hd),
        "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
    }[slot]


def kv_lengths(cfg):
    kl = cfg["kv_len"]
    if isinstance(kl, tuple):
        return uniform_i32(cfg["seed"], TID_KV_LEN, kl[0], kl[1], cfg["batch"])
    if isinstance(kl, list):  # explicit per-sequence lengths
        assert len(kl) == cfg["batch"]
        return np.array(kl, dtype=np.int32)
    return np.full(cfg["batch"], kl, dtype=np.int32)


def kv_capacity(kv_len):
    """Cache rows per sequence: room for the new row plus a poisoned margin."""
    return int((int(np.max(kv_len)) + 1 + 15 + 15) // 16 * 16)


def make_weights(cfg, norm_sigma=0.0, zero_slots=()):
    """Random-init weights of the workload's shape.

    Linear weights ~N(0, 0.02) bf16.  Norm weights are 1.0 (``norm_sigma`` = 0)
    or ~N(1, norm_sigma) when a test wants them to matter.  ``zero_slots``
    names linear slots to set to exactly zero (used by closed-form tests).
    Returns a dict: 'embed', 'final_norm', 'lm_head' (absent when tied) and
    'layers' (list of dicts keyed by LAYER_SLOTS; q_norm/k_norm only with qk_norm).
    """
    seed = cfg["seed"]
    H, V = cfg["hidden"], cfg["vocab"]
    w = {"embed": normal_bf16(seed, TID_EMBED, (V, H), 0.02)}

    def norm_vec(tid, n):
        if norm_sigma == 0.0:
            return np.full(n, BF16_ONE, dtype=np.uint16)
        return normal_bf16(seed, tid, (n,), norm_sigma, mean=1.0)

    w["final_norm"] = norm_vec(TID_FINAL_NORM, H)
    if not cfg["tied"]:
        w["lm_head"] = normal_bf16(seed, TID_LM_HEAD, (V, H), 0.02)
    layers = []
    for l in range(cfg["n_layers"]):
        d = {}
        for s in LAYER_SLOTS:
            if s in ("q_norm", "k_norm") and not cfg["qk_norm"]:
                continue
            shp = slot_shape(cfg, s)
            if s.endswith("norm"):
                d[s] = norm_vec(tid_layer(l, s), shp[0])
            elif s in zero_slots:
                d[s] = np.zeros(shp, dtype=np.uint16)
            else:
                d[s] = normal_bf16(seed, tid_layer(l, s), shp, 0.02)
        layers.append(d)
    w["layers"] = layers
    return w


def make_kv_cache(cfg, kv_len, capacity=None):
    """KV cache [L][2][B][n_kv][capacity][head_dim] bf16 bits.

    Rows pos < kv_len[b] hold ~N(0,1) draws (element (b, g, pos, d) takes stream
    index ((b * n_kv + g) * 2^20 + pos) * head_dim + d of tensor (layer, K|V));
    every other row is NaN so that any read outside the attended range shows.
    """
    L, B, nkv, hd = cfg["n_layers"], cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"]
    cap = capacity or kv_capacity(kv_len)
    kv = np.empty((L, 2, B, nkv, cap, hd), dtype=np.uint16)
    lib = _load()
    for l in range(L):
        for kind in range(2):
            for b in range(B):
                for g in range(nkv):
                    blk = kv[l, kind, b, g]
                    n = int(kv_len[b])
                    blk[n:] = BF16_NAN
                    if n:
                        rows = np.ascontiguousarray(blk[:n])
                        lib.synth_normal_bf16_2d(cfg["seed"], tid_kv(l, kind), 0.0, 1.0,
                                                 (b * nkv + g) * KV_POS_STRIDE * hd, hd, n, hd, _ptr(rows))
                        blk[:n] = rows
    return kv


def make_tokens(cfg):
    return uniform_i32(cfg["seed"], TID_TOKENS, 0, cfg["vocab"] - 1, cfg["batch"])


def make_inputs(name, norm_sigma=0.0, zero_slots=(), **overrides):
    """All inputs of one decode step: dict(cfg, weights, kv_len, kv_cache, tokens)."""
    cfg = config(name, **overrides)
    kv_len = kv_lengths(cfg)
    return dict(cfg=cfg, weights=make_weights(cfg, norm_sigma, zero_slots), kv_len=kv_len,
                kv_cache=make_kv_cache(cfg, kv_len), tokens=make_tokens(cfg))

