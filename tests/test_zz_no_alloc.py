"""mk_run_noalloc (the allocation-free entry point) against mk_run, through the
C ABI: two calls in a row on one GPU, the second with a smaller input, each
compared with mk_run's result on the same plan and inputs (identical tokens,
logits within the 2e-3 relative-L2 bar -- the same kernels run, so they are
expected bit-identical) and with the oracle's argmax.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-3


def _one(mk, name, **overrides):
    inp = synth.make_inputs(name, norm_sigma=0.1, **overrides)
    cfg = inp["cfg"]
    B, V = cfg["batch"], cfg["vocab"]
    w = mk.DeviceWeights(inp["weights"], cfg)
    tok = mk.tokens_to_device(inp["tokens"])
    plan = mk.Plan.build(cfg, B, inp["kv_len"], inp["kv_cache"].shape[4])
    try:
        need, limit = plan.noalloc_bytes()
        print("  %s batch %d: scratch %d of %d bytes" % (name, B, need, limit), flush=True)
        assert 0 < need <= limit
        # the existing entry point
        kv_a = mk.kv_to_device(inp["kv_cache"])
        plan.run(w, kv_a, tok)
        torch.cuda.synchronize()
        st, chk = plan.check()
        assert st == mk.MK_OK and chk.counters_ok == 1
        want_logits = plan.output(mk.MK_OUT_LOGITS).cpu().numpy().reshape(B, V)
        want_next = plan.output(mk.MK_OUT_NEXT_TOKEN).cpu().numpy()
        # the allocation-free one, straight through the C ABI, into caller buffers
        kv_b = mk.kv_to_device(inp["kv_cache"])
        logits = torch.full((B * V,), float("nan"), dtype=torch.float32, device="cuda")
        nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        s = mk.vp(torch.cuda.current_stream().cuda_stream)
        rc = mk.lib().mk_run_noalloc(plan._h, ctypes.byref(w.struct), mk.vp(kv_b.data_ptr()), mk.vp(tok.data_ptr()),
                                     mk.vp(logits.data_ptr()), mk.vp(nxt.data_ptr()), s)
        assert rc == mk.MK_OK, mk.lib().mk_last_error().decode()
        torch.cuda.synchronize()
        got_logits = logits.cpu().numpy().reshape(B, V)
        got_next = nxt.cpu().numpy()
        rel = np.linalg.norm(got_logits - want_logits) / np.linalg.norm(want_logits)
        print("  noalloc vs mk_run: rel-L2 %.3g, tokens %s / %s" % (rel, got_next, want_next), flush=True)
        assert np.isfinite(got_logits).all()
        assert rel <= LOGIT_TOL
        assert np.array_equal(got_next, want_next)
        assert np.array_equal(got_logits, want_logits)  # same kernels, same order
        assert np.array_equal(kv_a.cpu().view(torch.int16).numpy(), kv_b.cpu().view(torch.int16).numpy())
        assert np.array_equal(got_next, oracle.decode_step(inp)["next"])
    finally:
        plan.free()


def test_gpu_noalloc_matches_mk_run_two_calls():
    mk = pytest.importorskip("persistent_megakernel_decode_amd")
    # first a batch-4 step with long KV, then a smaller one: batch 1, shorter KV
    _one(mk, "tiny", batch=4, kv_len=(100, 600), seed=31)
    _one(mk, "tiny", kv_len=57, seed=32)


def test_gpu_noalloc_rejects_oversized_and_glm_plans():
    mk = pytest.importorskip("persistent_megakernel_decode_amd")
    cfg = synth.config("qwen3_8b")
    plan = mk.Plan.build(cfg, 1, np.array([4096], dtype=np.int32), 4097, num_cus=256)
    try:
        need, limit = plan.noalloc_bytes()
        if need > limit:
            z = torch.zeros(1, dtype=torch.int32, device="cuda")
            rc = mk.lib().mk_run_noalloc(plan._h, None, mk.vp(0), mk.vp(0), mk.vp(z.data_ptr()),
                                         mk.vp(z.data_ptr()), mk.vp(torch.cuda.current_stream().cuda_stream))
            assert rc == mk.MK_E_UNSUPPORTED
            assert "scratch" in mk.lib().mk_last_error().decode()
    finally:
        plan.free()
