"""Pins of the CPU oracle's decode step to things other than itself.

* a third-party implementation: the float64 Llama and Qwen3 models of the
  ``transformers`` library, loaded with the same synthetic weights and KV rows
  (this fixes the RoPE pairing, GQA head mapping, RMSNorm form, SwiGLU, the
  tied LM head and the per-head q/k norm);
* closed forms and invariants of each step (RMSNorm scale invariance, RoPE
  identity / unit-vector images / relative-position property, attention
  special cases, the all-zero-projection model);
* library routines for single steps (numpy matmul and softmax, scipy expit);
* bf16 rounding against the round-to-nearest-even bit formula on every
  exponent and every tie pattern.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import bf16_to_f64


def _hf_model(cfg, weights, qwen3=False):
    if qwen3:
        from transformers import Qwen3Config as C, Qwen3ForCausalLM as M
    else:
        from transformers import LlamaConfig as C, LlamaForCausalLM as M
    kw = dict(vocab_size=cfg["vocab"], hidden_size=cfg["hidden"], intermediate_size=cfg["ffn"],
              num_hidden_layers=cfg["n_layers"], num_attention_heads=cfg["n_q_heads"],
              num_key_value_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], rms_norm_eps=cfg["rms_eps"],
              rope_theta=cfg["rope_theta"], tie_word_embeddings=bool(cfg["tied"]), max_position_embeddings=8192,
              attention_bias=False)
    hc = C(**kw)
    hc._attn_implementation = "eager"
    m = M(hc).double().eval()
    T = lambda a: torch.from_numpy(bf16_to_f64(a))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(T(weights["embed"]))
        m.model.norm.weight.copy_(T(weights["final_norm"]))
        if not cfg["tied"]:
            m.lm_head.weight.copy_(T(weights["lm_head"]))
        for l, lay in enumerate(m.model.layers):
            d = weights["layers"][l]
            lay.input_layernorm.weight.copy_(T(d["attn_norm"]))
            lay.post_attention_layernorm.weight.copy_(T(d["ffn_norm"]))
            a = lay.self_attn
            a.q_proj.weight.copy_(T(d["wq"]))
            a.k_proj.weight.copy_(T(d["wk"]))
            a.v_proj.weight.copy_(T(d["wv"]))
            a.o_proj.weight.copy_(T(d["wo"]))
            if qwen3:
                a.q_norm.weight.copy_(T(d["q_norm"]))
                a.k_norm.weight.copy_(T(d["k_norm"]))
            lay.mlp.gate_proj.weight.copy_(T(d["w_gate"]))
            lay.mlp.up_proj.weight.copy_(T(d["w_up"]))
            lay.mlp.down_proj.weight.copy_(T(d["w_down"]))
    return m, hc


def _hf_step(inp, qwen3=False):
    """Decode one token per sequence with the library model; returns logits and new K/V rows."""
    from transformers import DynamicCache
    cfg = inp["cfg"]
    m, hc = _hf_model(cfg, inp["weights"], qwen3)
    logits, newk, newv = [], [], []
    for b in range(cfg["batch"]):
        p = int(inp["kv_len"][b])
        cache = DynamicCache(config=hc)
        kv = inp["kv_cache"]
        with torch.no_grad():
            for l in range(cfg["n_layers"]):
                k = torch.from_numpy(bf16_to_f64(kv[l, 0, b:b + 1, :, :p, :]))
                v = torch.from_numpy(bf16_to_f64(kv[l, 1, b:b + 1, :, :p, :]))
                cache.update(k, v, l)
            out = m(input_ids=torch.tensor([[int(inp["tokens"][b])]]), past_key_values=cache,
                    position_ids=torch.tensor([[p]]), cache_position=torch.tensor([p]), use_cache=True)
        logits.append(out.logits[0, -1].numpy())
        c = out.past_key_values
        newk.append(np.stack([c.layers[l].keys[0, :, p, :].numpy() for l in range(cfg["n_layers"])]))
        newv.append(np.stack([c.layers[l].values[0, :, p, :].numpy() for l in range(cfg["n_layers"])]))
    return np.stack(logits), newk, newv


def _bf16_vec(a):
    return np.array([oracle.to_bf16(x) for x in np.ravel(a)], dtype=np.uint16).reshape(np.shape(a))


def _rel(a, b):
    return float(np.linalg.norm(np.ravel(a) - np.ravel(b)) / np.linalg.norm(np.ravel(b)))


@pytest.mark.parametrize("name,overrides,qwen3", [
    ("tiny", {}, False),
    ("tiny", dict(batch=2, kv_len=(5, 40), seed=77), False),
    ("tiny", dict(arch="qwen3", qk_norm=1, tied=0, head_dim=128, n_q_heads=4, n_kv_heads=2, seed=78), True),
])
def test_oracle_matches_transformers_fp64(name, overrides, qwen3):
    inp = synth.make_inputs(name, norm_sigma=0.1, **overrides)
    ref_logits, newk, newv = _hf_step(inp, qwen3=qwen3)
    r = oracle.decode_step(inp, round_new_kv=False)
    # The library computes RoPE angles in fp32; everything else is fp64.
    assert _rel(r["logits"], ref_logits) < 1e-5
    assert np.array_equal(r["next"], ref_logits.argmax(axis=1))
    L = inp["cfg"]["n_layers"]
    for b in range(inp["cfg"]["batch"]):
        p = int(inp["kv_len"][b])
        for l in range(L):
            got_k = r["kv_cache"][l, 0, b, :, p, :]
            got_v = r["kv_cache"][l, 1, b, :, p, :]
            # K/V rows: bf16 of the library's rows; the fp32 RoPE table may move a
            # K value across a rounding boundary, so allow one unit in the last place.
            assert np.array_equal(got_v, _bf16_vec(newv[b][l]))
            dk = np.abs(got_k.astype(np.int32) - _bf16_vec(newk[b][l]).astype(np.int32))
            assert dk.max() <= 1 and (dk > 0).mean() < 0.01


def test_round_new_kv_reading_changes_little():
    inp = synth.make_inputs("tiny", norm_sigma=0.1)
    a = oracle.decode_step(inp, round_new_kv=True)
    b = oracle.decode_step(inp, round_new_kv=False)
    # layer 0's new row does not depend on the reading; later layers see a different input
    assert np.array_equal(a["kv_cache"][0], b["kv_cache"][0])
    assert 0 < _rel(a["logits"], b["logits"]) < 1e-2


def test_fp32_build_tracks_fp64_build():
    assert oracle.lib("f64").oracle_real_bytes() == 8 and oracle.lib("f32").oracle_real_bytes() == 4
    inp = synth.make_inputs("tiny", norm_sigma=0.1)
    a = oracle.decode_step(inp, precision="f64")
    b = oracle.decode_step(inp, precision="f32")
    assert _rel(b["logits"], a["logits"]) < 2e-5
    assert np.array_equal(a["next"], b["next"])


def test_zero_projections_give_embedding_logits():
    """All attention and FFN projections zero: every layer is the identity, so the
    logits are rmsnorm(E[t]) * w_final . E^T (closed form, numpy)."""
    inp = synth.make_inputs("tiny", norm_sigma=0.1, zero_slots=("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"))
    r = oracle.decode_step(inp)
    cfg, w = inp["cfg"], inp["weights"]
    E = bf16_to_f64(w["embed"])
    x = E[int(inp["tokens"][0])]
    y = x / np.sqrt(np.mean(x * x) + cfg["rms_eps"]) * bf16_to_f64(w["final_norm"])
    ref = E @ y
    assert _rel(r["logits"][0], ref) < 1e-13
    assert r["next"][0] == int(np.argmax(ref))


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(512)
    one = np.full(512, synth.BF16_ONE, np.uint16)
    y = oracle.rmsnorm(x, one, 1e-5)
    ms = np.mean(x * x)
    assert abs(np.mean(y * y) - ms / (ms + 1e-5)) < 1e-14
    # scaling: rmsnorm(c x) = y * sqrt(ms + eps) / sqrt(ms + eps / c^2)
    f = np.sqrt(ms + 1e-5) / np.sqrt(ms + 1e-5 / 1e6)
    assert np.allclose(oracle.rmsnorm(1000 * x, one, 1e-5), y * f, rtol=1e-13, atol=0)
    # weights multiply element-wise
    w = synth.normal_bf16(3, 4, (512,), 0.3, mean=1.0)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-5), y * bf16_to_f64(w), rtol=1e-14, atol=1e-15)
    # eps enters under the root: a constant vector c gives c / sqrt(c^2 + eps)
    c = np.full(8, 0.01)
    assert np.allclose(oracle.rmsnorm(c, one[:8], 1e-5), 0.01 / np.sqrt(1e-4 + 1e-5), rtol=1e-14)


def test_rope_closed_forms():
    d, theta = 64, 1e4
    rng = np.random.default_rng(1)
    v = rng.standard_normal(d)
    assert np.array_equal(oracle.rope(v, 0, theta), v)  # position 0 is the identity
    # unit vector e_i (i < d/2) rotates within the pair (i, i + d/2)
    for i in (0, 5, 31):
        e = np.zeros(d)
        e[i] = 1.0
        ang = 7 * theta ** (-2.0 * i / d)
        r = oracle.rope(e, 7, theta)
        ref = np.zeros(d)
        ref[i], ref[i + d // 2] = np.cos(ang), np.sin(ang)
        assert np.allclose(r, ref, atol=1e-15)
    # norm-preserving and relative: <R_p q, R_p' k> = <q, R_(p'-p) k>
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    assert abs(np.linalg.norm(oracle.rope(q, 1234, theta)) - np.linalg.norm(q)) < 1e-12
    lhs = oracle.rope(q, 300, theta) @ oracle.rope(k, 1000, theta)
    rhs = q @ oracle.rope(k, 700, theta)
    assert abs(lhs - rhs) < 1e-10


def test_attention_special_cases():
    d, n = 64, 37
    K = synth.normal_bf16(5, 1, (n, d), 1.0)
    V = synth.normal_bf16(5, 2, (n, d), 1.0)
    Kf, Vf = bf16_to_f64(K), bf16_to_f64(V)
    q = np.random.default_rng(2).standard_normal(d)
    # library softmax
    s = Kf @ q / np.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert np.allclose(oracle.attend(q, K, V), p @ Vf, rtol=1e-12, atol=1e-13)
    # zero query: uniform weights, output = mean of V rows
    assert np.allclose(oracle.attend(np.zeros(d), K, V), Vf.mean(axis=0), rtol=1e-12, atol=1e-14)
    # a single row: output is that row exactly
    assert np.array_equal(oracle.attend(q, K[:1], V[:1]), Vf[0])
    # the special row is taken from knew/vnew
    kn, vn = np.random.default_rng(3).standard_normal((2, d))
    K2, V2 = K.copy(), V.copy()
    K2[4] = synth.BF16_NAN
    V2[4] = synth.BF16_NAN
    Kf2, Vf2 = Kf.copy(), Vf.copy()
    Kf2[4], Vf2[4] = kn, vn
    s = Kf2 @ q / np.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert np.allclose(oracle.attend(q, K2, V2, special=4, knew=kn, vnew=vn), p @ Vf2, rtol=1e-12, atol=1e-13)


def test_empty_prior_kv_attends_only_the_new_row():
    """kv_len = 0: softmax over one position, so layer 0's attention output is
    bf16(v_new) exactly; checked by running one layer of the step with numpy."""
    inp = synth.make_inputs("tiny", norm_sigma=0.1, kv_len=0, n_layers=1)
    r = oracle.decode_step(inp)
    cfg, w = inp["cfg"], inp["weights"]
    d0 = w["layers"][0]
    x = bf16_to_f64(w["embed"])[int(inp["tokens"][0])]
    y = x / np.sqrt(np.mean(x * x) + cfg["rms_eps"]) * bf16_to_f64(d0["attn_norm"])
    v = bf16_to_f64(d0["wv"]) @ y
    vb = bf16_to_f64(_bf16_vec(v))
    assert np.array_equal(r["kv_cache"][0, 1, 0, :, 0, :].ravel(), _bf16_vec(v))
    hpg = cfg["n_q_heads"] // cfg["n_kv_heads"]
    o = np.concatenate([vb[(h // hpg) * 64:(h // hpg + 1) * 64] for h in range(cfg["n_q_heads"])])
    x1 = x + bf16_to_f64(d0["wo"]) @ o
    y2 = x1 / np.sqrt(np.mean(x1 * x1) + cfg["rms_eps"]) * bf16_to_f64(d0["ffn_norm"])
    g, u = bf16_to_f64(d0["w_gate"]) @ y2, bf16_to_f64(d0["w_up"]) @ y2
    from scipy.special import expit
    x2 = x1 + bf16_to_f64(d0["w_down"]) @ (g * expit(g) * u)
    yf = x2 / np.sqrt(np.mean(x2 * x2) + cfg["rms_eps"]) * bf16_to_f64(w["final_norm"])
    assert _rel(r["logits"][0], bf16_to_f64(w["embed"]) @ yf) < 1e-12


def test_matvec_is_the_matrix_product():
    W = synth.normal_bf16(9, 9, (300, 257), 0.02)
    x = np.random.default_rng(4).standard_normal(257)
    assert np.allclose(oracle.matvec(W, x), bf16_to_f64(W) @ x, rtol=1e-12, atol=1e-14)


def test_argmax_lowest_index_on_ties():
    v = np.array([1.0, 3.0, -2.0, 3.0, 3.0])
    assert oracle.argmax(v) == 1
    assert oracle.argmax(np.zeros(7)) == 0


def test_bf16_rounding_all_exponents_and_tie_patterns():
    """Every fp32 exponent/sign (high 16 bits) with the low-half patterns that
    decide rounding, against the textbook RNE bit formula, plus doubles that
    sit just off a tie (one rounding, not two)."""
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    highs = np.arange(0, 1 << 16, dtype=np.uint32)
    highs = highs[((highs >> 7) & 0xFF) != 0xFF]  # finite values only
    bits = (highs[:, None] << 16 | lows[None, :]).ravel()
    sample = bits[:: max(1, bits.size // 60000)]
    f = sample.view(np.float32)
    exp_bits = ((sample + 0x7FFF + ((sample >> 16) & 1)) >> 16).astype(np.uint16)
    # values whose rounding overflows the finite range become inf
    got = np.array([oracle.to_bf16(float(x)) for x in f], dtype=np.uint16)
    assert np.array_equal(got, exp_bits)
    # a double just above a tie rounds up; the same value through fp32 would tie to even
    tie = 1.0 + 2.0 ** -8  # halfway between bf16 1.0 and 1.0078125
    assert oracle.to_bf16(tie) == 0x3F80
    assert oracle.to_bf16(tie + 2.0 ** -40) == 0x3F81
    assert oracle.to_bf16(-(tie + 2.0 ** -40)) == 0xBF81
    assert oracle.to_bf16(float("nan")) == 0x7FC0
    assert oracle.to_bf16(3.5e38) == 0x7F80


def test_new_k_row_is_rounded_before_it_is_attended():
    """Reading A5 (the new K and V rows are rounded to bf16 before they are
    attended), its K half, by a closed form at kv_len = 1.  One layer, one head;
    the normed input is exactly all ones (embedding row of ones, eps 1e-30), so
    q, k and v are chosen columns of Wq, Wk, Wv.  The prior cache row is set to
    bf16(RoPE(k)) -- the row the step itself writes -- with V = 0, and Wo is the
    identity with a zero FFN.  Attending the rounded new k gives two equal
    scores, weights exactly 1/2, so the post-attention stream is exactly
    1 + v / 2; attending the unrounded k gives the logistic weight of the score
    gap instead (the rotated q is chosen along the rounding error, so the gap
    is positive).  RoPE and bf16 rounding, pinned on their own above, build the
    prior row."""
    d, V, t = 64, 8, 3
    cfg = synth.config("tiny", n_layers=1, hidden=d, n_q_heads=1, n_kv_heads=1, head_dim=d, ffn=16, vocab=V,
                       kv_len=1, rms_eps=1e-30, seed=91)
    one = 0x3F80
    kappa = synth.normal_bf16(91, 1, (d,), 1.0)
    z = bf16_to_f64(synth.normal_bf16(91, 2, (d,), 1.0))
    nu = _bf16_vec(np.sign(z) * np.clip(np.round(np.abs(z) * 8), 1, 16) / 16)  # nonzero multiples of 1/16
    k_rot = oracle.rope(bf16_to_f64(kappa), 1, cfg["rope_theta"])
    K0 = _bf16_vec(k_rot)
    err = k_rot - bf16_to_f64(K0)
    assert np.count_nonzero(err) > d // 2
    # q is rotated too: pick the sign that makes the rotated q's gap positive
    q = _bf16_vec(64.0 * np.sign(err))
    if oracle.rope(bf16_to_f64(q), 1, cfg["rope_theta"]) @ err < 0:
        q = _bf16_vec(-64.0 * np.sign(err))

    def col0(v):
        W = np.zeros((d, d), dtype=np.uint16)
        W[:, 0] = v
        return W
    zeros = lambda shp: np.zeros(shp, dtype=np.uint16)
    layer = dict(attn_norm=np.full(d, one, np.uint16), wq=col0(q), wk=col0(kappa), wv=col0(nu),
                 wo=np.diag(np.full(d, one, np.uint16)).astype(np.uint16), ffn_norm=np.full(d, one, np.uint16),
                 w_gate=zeros((16, d)), w_up=zeros((16, d)), w_down=zeros((d, 16)))
    embed = zeros((V, d))
    embed[t] = one
    w = dict(embed=embed, final_norm=np.full(d, one, np.uint16), layers=[layer])
    cap = 16
    kv = np.full((1, 2, 1, 1, cap, d), 0x7FC0, dtype=np.uint16)
    kv[0, 0, 0, 0, 0] = K0
    kv[0, 1, 0, 0, 0] = 0
    inp = dict(cfg=cfg, weights=w, kv_len=np.array([1], np.int32), kv_cache=kv, tokens=np.array([t], np.int32))
    r = oracle.decode_step(inp, intermediates=True)
    nuf = bf16_to_f64(nu)
    assert np.array_equal(r["kv_cache"][0, 0, 0, 0, 1], K0)  # the step writes bf16(RoPE(k)) at row 1
    assert np.array_equal(r["kv_cache"][0, 1, 0, 0, 1], nu)
    assert np.array_equal(r["hidden"][0, 0, 0], 1.0 + nuf / 2)  # exact: weights 1/2 each
    # the other reading (the new k unrounded) moves the weight by the score gap
    u = oracle.decode_step(inp, round_new_kv=False, intermediates=True)
    gap = float(oracle.rope(bf16_to_f64(q), 1, cfg["rope_theta"]) @ err) / np.sqrt(d)
    assert gap > 0
    want = 1.0 + nuf / (1.0 + np.exp(-gap))
    assert np.allclose(u["hidden"][0, 0, 0], want, rtol=1e-14, atol=1e-14)
    assert not np.array_equal(u["hidden"][0, 0, 0], r["hidden"][0, 0, 0])


def test_intermediates_are_the_steps_own_values():
    """The per-layer intermediates the oracle reports are the values its step
    uses: the last layer's FFN output is the input of the final norm (logits by
    numpy from it), layer 0's q/k/v are the projections of the normed embedding
    row, and each layer's attention output feeds its FFN block."""
    inp = synth.make_inputs("tiny", norm_sigma=0.1, batch=2, kv_len=(3, 60), seed=44)
    cfg, w = inp["cfg"], inp["weights"]
    r = oracle.decode_step(inp, intermediates=True)
    plain = oracle.decode_step(inp)
    assert np.array_equal(r["logits"], plain["logits"])
    E = bf16_to_f64(w["embed"])
    for b in range(cfg["batch"]):
        xf = r["hidden"][-1, 1, b]
        yf = xf / np.sqrt(np.mean(xf * xf) + cfg["rms_eps"]) * bf16_to_f64(w["final_norm"])
        assert _rel(r["logits"][b], E @ yf) < 1e-12
        x0 = E[int(inp["tokens"][b])]
        d0 = w["layers"][0]
        y0 = x0 / np.sqrt(np.mean(x0 * x0) + cfg["rms_eps"]) * bf16_to_f64(d0["attn_norm"])
        proj = np.concatenate([bf16_to_f64(d0[k]) @ y0 for k in ("wq", "wk", "wv")])
        assert _rel(r["qkv"][0, b].ravel(), proj) < 1e-12
        for l in range(cfg["n_layers"]):
            dl = w["layers"][l]
            x1 = r["hidden"][l, 0, b]
            y2 = x1 / np.sqrt(np.mean(x1 * x1) + cfg["rms_eps"]) * bf16_to_f64(dl["ffn_norm"])
            g, u = bf16_to_f64(dl["w_gate"]) @ y2, bf16_to_f64(dl["w_up"]) @ y2
            from scipy.special import expit
            x2 = x1 + bf16_to_f64(dl["w_down"]) @ (g * expit(g) * u)
            assert _rel(r["hidden"][l, 1, b], x2) < 1e-12
