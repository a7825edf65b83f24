"""Pins of the GLM pre-attention oracle (oracle/glm.py) to things other than
itself: the OCP e4m3 and bf16 definitions as implemented by torch's dtypes, a
nearest-code search over the whole e4m3 table, brute-force loops on shrunk
shapes, closed forms (selection weights, RoPE at position 0, scale invariance
of RMSNorm) and the storage contract of the two caches."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import glm as G


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def test_e4m3_decode_matches_definition_and_torch():
    # hand-listed values of the OCP FP8 E4M3 format
    spots = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in spots.items():
        assert G.e4m3_decode(np.array([c]))[0] == v, hex(c)
    assert np.isnan(G.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert math.copysign(1.0, G.e4m3_decode(np.array([0x80]))[0]) == -1.0
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = G.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])


def _nearest_code(v):
    """Brute force: scan every finite positive code for the nearest value, ties
    to the code with an even mantissa; saturate; sign from v."""
    table = [(c, G.e4m3_decode(np.array([c]))[0]) for c in range(0x7F)]
    a = min(abs(v), 448.0)
    best = None
    for c, x in table:
        d = abs(x - a)
        if best is None or d < best[1] or (d == best[1] and (c & 1) == 0):
            best = (c, d)
    return best[0] | (0x80 if v < 0 or (v == 0 and math.copysign(1.0, v) < 0) else 0)


def test_e4m3_encode_round_trip_ties_saturation():
    codes = np.arange(256, dtype=np.uint8)
    vals = G.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(G.e4m3_encode(vals[fin]), codes[fin])
    # midpoints between neighbouring positive codes go to the even code
    pos = np.arange(0x7E)
    mids = (G.e4m3_decode(pos) + G.e4m3_decode(pos + 1)) / 2
    got = G.e4m3_encode(mids)
    want = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(got, want)
    assert np.array_equal(G.e4m3_encode(-mids), want | 0x80)
    # saturation at +-448
    assert list(G.e4m3_encode(np.array([448.0, 460.0, 464.0, 1e6, -500.0, -1e30]))) == [0x7E] * 4 + [0xFE] * 2
    # brute-force nearest search on a sweep through every binade
    rng = np.random.default_rng(3)
    sweep = np.concatenate([rng.uniform(-1, 1, 400) * 2.0 ** rng.integers(-12, 10, 400), mids[:40], -mids[40:80]])
    assert [int(c) for c in G.e4m3_encode(sweep)] == [_nearest_code(v) for v in sweep]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 9, 200000)).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(G.e4m3_encode(x.astype(np.float64)), ref)


def test_generator_fp8_encoder_agrees_with_oracle_codec():
    """The seeded weight generator has its own (C) encoder; it must give the
    same codes as the oracle's, or the oracle would read different weights."""
    rng = np.random.default_rng(5)
    pos = np.arange(0x7E)
    mids = (G.e4m3_decode(pos) + G.e4m3_decode(pos + 1)) / 2
    vals = np.concatenate([rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 10, 3000), mids, -mids,
                           [0.0, 447.9, 448.0, 470.0, -1e5, 2.0 ** -10, 2.0 ** -9.5]])
    assert [synth.e4m3_code(v) for v in vals] == [int(c) for c in G.e4m3_encode(vals)]
    codes, scales = synth.fp8_weights(9, 1, 136, 256)
    assert scales.shape == (2, 2)
    dq = G.dequant_weight(codes, scales)
    # every block reaches its amax at one element: |dq| max per block == 448 * scale
    for nb in range(2):
        for kb in range(2):
            blk = dq[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert np.max(np.abs(blk)) == pytest.approx(448.0 * float(scales[nb, kb]), rel=1e-12)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(100000) * 2.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    # exact ties: low 16 bits 0x8000
    ties = ((rng.integers(0, 2 ** 7, 2000).astype(np.uint32) << 16) | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(G.bf16_bits(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# operators, against brute force
# ---------------------------------------------------------------------------
def test_a0_exact_ties_resolve_to_even():
    """With unit norm weights the quantizer's quotient 448 h / max|h| of
    bf16-derived values often lands exactly on an e4m3 midpoint; exact rational
    arithmetic and a nearest-code search with ties to the even code decide every
    such element the way the oracle does."""
    from fractions import Fraction
    M, H, eps = 2, 512, 1e-5
    x = synth.normal_bf16(13, 1, (M, H), 1.0)
    r = synth.normal_bf16(13, 2, (M, H), 1.0)
    w = np.full(H, synth.BF16_ONE, dtype=np.uint16)
    _, _, codes, _ = G.a0(x, r, w, eps)
    table = [(c, Fraction(G.e4m3_decode(np.array([c]))[0])) for c in range(0x7F)]
    ties = 0
    for m in range(M):
        h = [Fraction(G.bf16_decode(x[m, k])) + Fraction(G.bf16_decode(r[m, k])) for k in range(H)]
        for b in range(H // 128):
            amax = max(abs(v) for v in h[b * 128:(b + 1) * 128])
            for k in range(b * 128, (b + 1) * 128):
                q = 448 * h[k] / amax
                a = abs(q)
                best = min(table, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
                d = sorted(abs(v - a) for _, v in table)
                ties += d[0] == d[1]
                assert codes[m, k] == (best[0] | (0x80 if q < 0 else 0)), (m, k, q)
    assert ties > 0  # the case this test is about does occur


def test_a0_brute_force():
    M, H, eps = 2, 256, 1e-5
    x = synth.normal_bf16(11, 1, (M, H), 1.0)
    r = synth.normal_bf16(11, 2, (M, H), 1.0)
    w = synth.normal_bf16(11, 3, (H,), 0.2, mean=1.0)
    r_out, n, codes, scales = G.a0(x, r, w, eps)
    for m in range(M):
        h = [G.bf16_decode(x[m, k]) + G.bf16_decode(r[m, k]) for k in range(H)]
        ms = sum(v * v for v in h) / H
        inv = 1.0 / math.sqrt(ms + eps)
        y = [h[k] * inv * G.bf16_decode(w[k]) for k in range(H)]
        for k in range(H):
            # r_out: bf16 of the exact sum, by torch's fp32 -> bf16 (the sum of two bf16 is exact in fp32)
            want = torch.tensor([h[k]], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF
            assert r_out[m, k] == want
            assert n[m, k] == pytest.approx(y[k], rel=1e-13)
        for b in range(H // 128):
            amax = max(abs(v) for v in y[b * 128:(b + 1) * 128])
            s = max(amax, 1e-4) / 448.0
            assert scales[m, b] == pytest.approx(s, rel=1e-13)
            for k in range(b * 128, (b + 1) * 128):
                assert codes[m, k] == _nearest_code(y[k] / s), (m, k)


def test_block_gemm_brute_force_ragged_rows():
    rng = np.random.default_rng(8)
    M, K, N = 2, 256, 136  # two row blocks (the second partial), two column blocks
    codes = rng.integers(0, 256, (N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes in weights
    scales = rng.uniform(1e-4, 1e-2, (2, 2))
    a = rng.standard_normal((M, K))
    got = G.block_gemm(a, codes, scales)
    table = [G.e4m3_decode(np.array([c]))[0] for c in range(256)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += a[m, k] * table[codes[n, k]] * scales[n // 128, k // 128]
            assert got[m, n] == pytest.approx(acc, rel=1e-9, abs=1e-12)


def test_quantize_rows_error_bound_and_scale_invariance():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((3, 512)) * np.exp(rng.uniform(-4, 4, (3, 512)))
    codes, s = G.quantize_rows(y)
    dq = G.dequant_rows(codes, s)
    S = np.repeat(s, 128, axis=1)
    a = np.abs(y) / S
    # normal range: half a grid step, 2^-4 relative; subnormal range: 2^-10 absolute (in units of s)
    bound = np.where(a >= 2.0 ** -6, a * 2.0 ** -4, 2.0 ** -10) * S
    assert np.all(np.abs(dq - y) <= bound * (1 + 1e-12))
    # every block's largest element maps to 448 exactly
    assert np.all(np.max(np.abs(dq).reshape(3, 4, 128), axis=2) == pytest.approx(448.0 * s, rel=1e-12))
    # RMSNorm without eps is invariant under scaling by a power of two: codes and scales repeat
    h = rng.standard_normal((2, 256))
    w = np.ones(256)
    c1, s1 = G.quantize_rows(G.rmsnorm(h, w, 0.0))
    c2, s2 = G.quantize_rows(G.rmsnorm(4.0 * h, w, 0.0))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # the scale floor: an all-zero block gets scale 1e-4 / 448 and zero codes
    cz, sz = G.quantize_rows(np.zeros((1, 128)))
    assert sz[0, 0] == 1e-4 / 448.0 and not cz.any()


def test_rope_closed_forms():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 64))
    assert np.array_equal(G.rope(v, np.zeros(3), 1e4), v)
    r = G.rope(v, np.array([5, 100, 8199]), 1e4)
    # each pair (i, i + 32) keeps its length
    assert np.allclose(v[:, :32] ** 2 + v[:, 32:] ** 2, r[:, :32] ** 2 + r[:, 32:] ** 2, rtol=1e-12)
    # one pair at position 1 rotates by 1 radian
    e = G.rope(np.array([[1.0, 0.0]]), np.array([1]), 1e4)
    assert e[0, 0] == pytest.approx(math.cos(1.0)) and e[0, 1] == pytest.approx(math.sin(1.0))


# ---------------------------------------------------------------------------
# the step: which branch consumes what, and what the caches receive
# ---------------------------------------------------------------------------
def _select_weight(N, K, cols):
    """fp8 weight whose row n is 1.0 at column cols[n] (scale 1): W a = a[cols]."""
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[np.arange(N), cols] = 0x38
    return codes, np.ones(((N + 127) // 128, K // 128))


def test_step_with_selection_weights():
    inp = synth.make_glm_inputs("glm_tiny", norm_sigma=0.1)
    cfg, w = inp["cfg"], inp["weights"]
    H, QL, KL, RD = cfg["hidden"], cfg["q_lora"], cfg["kv_lora"], cfg["rope_dim"]
    M, Nqkva, Nqb, Niq = synth.glm_dims(cfg)
    rng = np.random.default_rng(9)
    sel_a = rng.integers(0, H, Nqkva)
    sel_g = rng.integers(0, H, cfg["n_gate"])
    sel_k = rng.integers(0, H, cfg["idx_head_dim"])
    sel_q = rng.integers(0, QL, Nqb)
    sel_i = rng.integers(0, QL, Niq)
    w["w_qkva"], w["s_qkva"] = _select_weight(Nqkva, H, sel_a)
    w["w_gate"], w["s_gate"] = _select_weight(cfg["n_gate"], H, sel_g)
    w["w_idxk"], w["s_idxk"] = _select_weight(cfg["idx_head_dim"], H, sel_k)
    w["w_qb"], w["s_qb"] = _select_weight(Nqb, QL, sel_q)
    w["w_idxq"], w["s_idxq"] = _select_weight(Niq, QL, sel_i)
    o = G.glm_step(inp)
    a = G.dequant_rows(o["act_codes"], o["act_scales"])
    # QKV-A and indexer-K read the quantized activation, the gate the norm output
    assert np.array_equal(o["qkva"], a[:, sel_a])
    assert np.array_equal(o["gate"], o["norm"][:, sel_g])
    assert not np.array_equal(o["gate"], a[:, sel_g])
    assert np.array_equal(o["kidx"], G.bf16_bits(a[:, sel_k]))
    # the q path: RMSNorm of the q part, quantized, then selected
    _, qc, qs = G.norm_quant(o["qkva"][:, :QL], G.bf16_decode(w["q_a_norm"]), cfg["rms_eps"])
    assert np.array_equal(qc, o["qa_codes"])
    qa = G.dequant_rows(qc, qs)
    qi = G.bf16_decode(o["qidx"].reshape(M, Niq))
    assert np.array_equal(qi, G.bf16_decode(G.bf16_bits(qa[:, sel_i])))
    # QKV-B: nope dims are plain selections, rope dims rotate at each token's position
    hd, nh = cfg["head_dim"], cfg["n_q_heads"]
    q = G.bf16_decode(o["q"]).reshape(M, nh, hd)
    raw = qa[:, sel_q].reshape(M, nh, hd)
    assert np.array_equal(q[:, :, :hd - RD], G.bf16_decode(G.bf16_bits(raw[:, :, :hd - RD])))
    want = G.rope(raw[:, :, hd - RD:], inp["pos"], cfg["rope_theta"])
    assert np.array_equal(q[:, :, hd - RD:], G.bf16_decode(G.bf16_bits(want)))
    # the KV row
    kvn = G.rmsnorm(o["qkva"][:, QL:QL + KL], G.bf16_decode(w["kv_a_norm"]), cfg["rms_eps"])
    kr = G.rope(o["qkva"][:, QL + KL:], inp["pos"], cfg["rope_theta"])
    assert np.array_equal(o["kv_rows"], G.bf16_bits(np.concatenate([kvn, kr], axis=1)))


def test_step_cache_writes():
    inp = synth.make_glm_inputs("glm_tiny")
    o = G.glm_step(inp)
    cfg = inp["cfg"]
    kvc, idc = o["kv_cache"], o["idx_cache"]
    written = np.zeros(kvc.shape[:2], dtype=bool)
    for m, (p, q) in enumerate(zip(inp["pos"], inp["req"])):
        written[q, p] = True
        assert np.array_equal(kvc[q, p], o["kv_rows"][m]) and np.array_equal(idc[q, p], o["kidx"][m])
    assert written.sum() == cfg["n_seqs"] * cfg["rows_per_seq"]
    # everything else keeps its (NaN) contents
    assert np.all(kvc[~written] == synth.BF16_NAN) and np.all(idc[~written] == synth.BF16_NAN)
    assert np.all(np.isfinite(G.bf16_decode(o["q"]))) and np.all(np.isfinite(o["gate"]))
