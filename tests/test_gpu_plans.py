"""GPU tests of the plan variants: the pairing-strategy plan (MegaRTP article,
section 4, "TaskGraph": O and down wait on two events each) and the attention
placement (longest first, the batched default, or plan order: CMU 15-779
lecture 7 notes, section 6.4).  Each runs
through the C-ABI against the oracle and, since every tile computes the same
arithmetic wherever it is placed, bit for bit against the default plan.  The
second-wait test forces its failure from the host (a threshold raised past its
event's producer count); every kernel still exits normally."""
import gc

import numpy as np
import pytest

from tests.lib_defaults import documented_choices
from tests.test_gpu_parity import Case, assert_layerwise_consistent

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _mk():
    import persistent_megakernel_decode_amd as mk
    return mk


def _free(*cases):
    for c in cases:
        c.plan.free()
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,overrides,extra", [
    ("tiny", {}, dict(pairing=1)),
    ("tiny", dict(batch=3, kv_len=(0, 200), seed=11), dict(pairing=1, attn_order=1)),
    ("tiny", dict(batch=16, kv_len=(100, 300), seed=12), dict(attn_order=-1)),
    ("llama1b", {}, dict(pairing=1)),
    ("llama1b", {}, dict(attn_order=1)),
    ("llama1b_b16", {}, dict(attn_order=-1)),
])
def test_gpu_plan_variant_matches_oracle_and_default_plan(name, overrides, extra):
    sigma = 0.0 if name.startswith("llama1b") else 0.1
    base = Case(name, norm_sigma=sigma, **overrides)
    var = Case(name, norm_sigma=sigma, opts=extra, **overrides)
    try:
        ex = var.plan.export()
        want = documented_choices(base.cfg["batch"], **extra)
        assert ex["pairing"] == want["pairing"] and ex["attn_order"] == want["attn_order"]
        if extra.get("pairing"):
            n2 = int((ex["queue"][:, :, 3] == 2).sum())
            print("  %d instructions with two waits" % n2, flush=True)
            assert n2 > 0
        r = var.run()
        var.assert_parity(r)
        r0 = base.run()
        assert np.array_equal(r["logits"], r0["logits"])
        assert np.array_equal(r["kv"], r0["kv"])
        lw = var.run(layerwise=True)
        assert_layerwise_consistent(var.cfg, lw, r)
    finally:
        _free(base, var)


def test_gpu_second_wait_is_honoured():
    """Pairing plan on tiny: raise only the second-wait thresholds on layer 0's
    down event (layer 1's O tiles wait on it after the attention output).  All
    other waits can be met, so the run times out only if the device polls
    second waits; restored, the next run is correct."""
    mk = _mk()
    c = Case("tiny", opts=dict(pairing=1, timeout_ms=50))
    try:
        r = c.run()
        c.assert_parity(r)
        ex = c.plan.export()
        q = ex["queue"].reshape(-1, 32)
        two = q[(q[:, 0] != 0) & (q[:, 3] == 2)]
        oproj1 = two[(two[:, 0] == 4) & (two[:, 10] == 1)]  # O-projection tiles of layer 1
        assert len(oproj1) > 0
        ev = int(oproj1[0, 24])
        assert (oproj1[:, 24] == ev).all()
        print("  raising the second-wait threshold of event %d by 1" % ev, flush=True)
        c.plan.debug_raise_wait(ev, 1, slot=2)
        c.plan.run(c.w, c.fresh_kv(), c.tokens)
        torch.cuda.synchronize()
        s, chk = c.plan.check()
        print("  status %d kind %d event %d value %d target %d" % (s, chk.err_kind, chk.err_event, chk.err_value,
                                                                  chk.err_target), flush=True)
        assert s == mk.MK_E_TIMEOUT and chk.err_kind != 0
        if chk.err_kind == 1:
            assert chk.err_event >= ev
        c.plan.debug_raise_wait(ev, -1, slot=2)
        r = c.run()
        c.assert_parity(r)
        assert r["check"].epoch == 1
    finally:
        _free(c)
