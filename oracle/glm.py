"""CPU oracle of the GLM-style pre-attention step -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this module.  It shares no code with the HIP library and never
imports it; both sides meet only through the seeded inputs of ``synth``.
Plain numpy in fp64: every value is widened exactly from its storage format,
every product and sum is fp64, and storage roundings (bf16, e4m3) are written
out from their definitions below.

What it computes follows the MegaRTP article (tahou.com): section 1 lists the
path before sparse MLA as fused Add + RMSNorm + Quant, then GEMMs, RoPE and a
cache write-back, at M = 16 (two requests of eight tokens) and KV = 8192;
section 4 ("OpGraph" / "TaskGraph") says the Add+RMSNorm+Quant operator (A0)
works one row per tile and publishes two results, the fp8 hidden state with
its scales and the norm output, and that the QKV-A, head-gate and indexer-K
branches depend on A0 but not on each other, while the q path's final Q/scale
tiles feed the next GEMMs.  The operator list and shapes are the workload's:
QKV-A 6144 -> 1536 + 576, head gate 6144 -> 64, indexer-K 6144 -> 128, QKV-B
1536 -> 64 x 192 with RoPE on 64 dims, KV-cache write, indexer-Q 1536 -> 32 x 128,
fp8 e4m3 weights with fp32 scales per 128 x 128 block.

Readings where the pages leave a step open (each listed in the design notes):
  - RMSNorm: y = h / sqrt(mean(h^2) + eps) * w, in full precision.
  - Activation quantization: per (row, 128-column block), s = max(amax, 1e-4) / 448,
    code = e4m3(y / s) rounded to nearest even and saturated at +-448.  The
    quotient is evaluated as 448 * u / max|u| with u = the row before its 1/rms
    factor (h * w), which is the same number (the factor cancels) but exact for
    bf16-derived u, so that exact ties -- frequent when u has few significant
    bits -- resolve to the even code by definition, not by rounding noise.
  - Weights: W = e4m3 value * scale of the weight's 128 x 128 block.
  - QKV-A, indexer-K, QKV-B and indexer-Q take the dequantized fp8 activation
    (code value * scale); the head gate takes the unquantized norm output.
  - The QKV-A output splits as [q (q_lora) | kv (kv_lora) | k_rope (rope_dim)];
    q is RMSNorm'd (weight q_a_norm) and quantized like A0 before QKV-B and
    indexer-Q; the KV row is [RMSNorm(kv) * kv_a_norm | RoPE(k_rope)], rounded
    to bf16 and written at the token's position of its request's cache.
  - The indexer-K output is rounded to bf16 and written to the request's
    indexer cache at the token's position; q, the indexer q and the gate are
    outputs (q and indexer q in bf16, the gate in fp32).
  - RoPE: rotate-half pairs (i, i + d/2) of the rope_dim part, angle
    pos * theta^(-2i/d); on QKV-B it applies to the last rope_dim dims of each
    head.
  - r_out = bf16(x + r) (the residual carried to the next block).
"""
import numpy as np

E4M3_MAX = 448.0
ACT_SCALE_FLOOR = 1e-4
BLOCK = 128


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def e4m3_decode(codes):
    """OCP FP8 E4M3 (e4m3fn): sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _round_grid(v, mant_bits, min_exp):
    """Round fp64 values to a binary format with mant_bits fraction bits and
    smallest normal exponent min_exp, to nearest with ties to even (no
    overflow handling): the grid spacing is 2^(E - mant_bits) for values of
    exponent E >= min_exp, and 2^(min_exp - mant_bits) below."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)  # v = f * 2^ex, |f| in [0.5, 1)
    E = np.maximum(ex - 1, min_exp)
    q = np.exp2((E - mant_bits).astype(np.float64))
    return np.round(v / q) * q  # np.round rounds halves to even


def e4m3_round(v):
    """Nearest e4m3 value, ties to even, saturated to +-448."""
    r = _round_grid(v, 3, -6)
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(v):
    """e4m3 codes of e4m3_round(v)."""
    r = e4m3_round(v)
    a = np.abs(r)
    _, ex = np.frexp(a)
    E = ex - 1
    sub = a < 2.0 ** -6
    m_sub = np.round(a * 512.0)
    m_nrm = np.round((a / np.exp2(np.where(sub, 0, E).astype(np.float64)) - 1.0) * 8.0)
    code = np.where(sub, m_sub, ((E + 7) << 3) + m_nrm)
    code = np.where(a == 0, 0, code).astype(np.int64)
    return (code | np.where(np.signbit(r), 0x80, 0)).astype(np.uint8)


def bf16_round(v):
    """Nearest bf16 value (8 significant bits, fp32 exponent range), ties to even."""
    return _round_grid(v, 7, -126)


def bf16_bits(v):
    r = bf16_round(v).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_decode(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# operators
# ---------------------------------------------------------------------------
def rms_inv(h, eps):
    """1 / sqrt(mean(h^2) + eps) per row."""
    h = np.asarray(h, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(h * h, axis=-1) + eps)


def rmsnorm(h, w, eps):
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * w


def norm_quant(h, w, eps):
    """RMSNorm then quant: (norm output, codes, scales)."""
    h = np.asarray(h, dtype=np.float64)
    inv = rms_inv(h, eps)
    u = h * w
    codes, scales = quantize_rows(u, inv)
    return u * inv[:, None], codes, scales


def quantize_rows(u, inv=None, floor=ACT_SCALE_FLOOR):
    """Quantize the rows n = u * inv (inv: one factor per row, default 1): per
    (row, 128-column block) scale s = max(max|n|, floor) / 448 and codes
    e4m3(n / s), the quotient taken as 448 * u / max|u| while the floor is not
    active.  Returns (codes uint8 [M, K], scales fp64 [M, K / 128])."""
    M, K = u.shape
    inv = np.ones(M) if inv is None else np.asarray(inv, dtype=np.float64).reshape(M)
    ub = u.reshape(M, K // BLOCK, BLOCK)
    amu = np.max(np.abs(ub), axis=2)
    amn = amu * inv[:, None]
    s = np.maximum(amn, floor) / E4M3_MAX
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where((amn >= floor)[:, :, None], E4M3_MAX * ub / amu[:, :, None],
                     ub * inv[:, None, None] / s[:, :, None])
    codes = e4m3_encode(q).reshape(M, K)
    return codes, s


def dequant_rows(codes, scales):
    M, K = codes.shape
    return (e4m3_decode(codes).reshape(M, K // BLOCK, BLOCK) * scales[:, :, None]).reshape(M, K)


_E4M3_TABLE = None


def dequant_weight(codes, scales):
    """W[n, k] = e4m3(codes[n, k]) * scales[n / 128, k / 128]."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_decode(np.arange(256))
    N, K = codes.shape
    NB = -(-N // BLOCK)
    v = np.zeros((NB * BLOCK, K), dtype=np.float64)
    v[:N] = _E4M3_TABLE[codes]
    v = v.reshape(NB, BLOCK, K // BLOCK, BLOCK) * np.asarray(scales, dtype=np.float64)[:, None, :, None]
    return v.reshape(NB * BLOCK, K)[:N]


def block_gemm(a, w_codes, w_scales):
    """a [M, K] (fp64) times the dequantized fp8 weight [N, K], transposed."""
    return a @ dequant_weight(w_codes, w_scales).T


def rope(v, pos, theta):
    """Rotate-half RoPE of the last axis (d) of v at positions pos (one per row)."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64).reshape(-1, *([1] * (v.ndim - 1))) * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------
def a0(x_bits, r_bits, norm_bits, eps):
    """Add + RMSNorm + quant: (r_out bf16 bits, norm output, codes, scales)."""
    h = bf16_decode(x_bits) + bf16_decode(r_bits)
    n, codes, scales = norm_quant(h, bf16_decode(norm_bits), eps)
    return bf16_bits(h), n, codes, scales


def glm_step(inp):
    """All results of one pre-attention step for the inputs of synth.make_glm_inputs.
    Returns a dict; the caches come back as updated copies."""
    cfg, w = inp["cfg"], inp["weights"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    QL, KL, RD = cfg["q_lora"], cfg["kv_lora"], cfg["rope_dim"]
    nh, hd = cfg["n_q_heads"], cfg["head_dim"]
    pos, req = inp["pos"], inp["req"]
    M = len(pos)
    out = {}
    r_out, n, a8, a_s = a0(inp["x"], inp["r"], w["attn_norm"], eps)
    out.update(r_out=r_out, norm=n, act_codes=a8, act_scales=a_s)
    a = dequant_rows(a8, a_s)
    # three independent branches on A0's results
    qkva = block_gemm(a, w["w_qkva"], w["s_qkva"])
    out["qkva"] = qkva
    out["gate"] = n @ dequant_weight(w["w_gate"], w["s_gate"]).T
    kidx = bf16_bits(block_gemm(a, w["w_idxk"], w["s_idxk"]))
    out["kidx"] = kidx
    # q path: RMSNorm + quant, then QKV-B (RoPE on each head's last RD dims) and indexer-Q
    _, q8, q_s = norm_quant(qkva[:, :QL], bf16_decode(w["q_a_norm"]), eps)
    out.update(qa_codes=q8, qa_scales=q_s)
    qa = dequant_rows(q8, q_s)
    q = block_gemm(qa, w["w_qb"], w["s_qb"]).reshape(M, nh, hd)
    q = np.concatenate([q[:, :, : hd - RD], rope(q[:, :, hd - RD:], pos, theta)], axis=-1)
    out["q"] = bf16_bits(q)
    out["qidx"] = bf16_bits(block_gemm(qa, w["w_idxq"], w["s_idxq"])).reshape(M, cfg["n_idx_heads"],
                                                                             cfg["idx_head_dim"])
    # KV row: [RMSNorm(kv) | RoPE(k_rope)] in bf16
    kv = rmsnorm(qkva[:, QL:QL + KL], bf16_decode(w["kv_a_norm"]), eps)
    kr = rope(qkva[:, QL + KL:QL + KL + RD], pos, theta)
    kv_rows = bf16_bits(np.concatenate([kv, kr], axis=-1))
    out["kv_rows"] = kv_rows
    kvc, idc = inp["kv_cache"].copy(), inp["idx_cache"].copy()
    for m in range(M):
        kvc[req[m], pos[m]] = kv_rows[m]
        idc[req[m], pos[m]] = kidx[m]
    out.update(kv_cache=kvc, idx_cache=idc)
    return out
