"""GPU tests of the runtime around the decode step: repeated runs over a
poisoned workspace, the watchdog, invalid token ids, stream-capture refusal and
the per-instruction trace.  Every failure here is forced from the host (a wait
threshold raised past its event's producer count, a token id out of range);
every kernel still exits normally.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-3


def _mk():
    import persistent_megakernel_decode_amd as mk
    return mk


class Setup:
    def __init__(self, name, norm_sigma=0.1, opts=None, **overrides):
        mk = _mk()
        self.inp = synth.make_inputs(name, norm_sigma=norm_sigma, **overrides)
        self.cfg = self.inp["cfg"]
        self.w = mk.DeviceWeights(self.inp["weights"], self.cfg)
        self.tokens = mk.tokens_to_device(self.inp["tokens"])
        self.kv = mk.kv_to_device(self.inp["kv_cache"])
        self.plan = mk.Plan.build(self.cfg, self.cfg["batch"], self.inp["kv_len"], self.inp["kv_cache"].shape[4],
                                  **(opts or {}))

    def logits(self):
        mk = _mk()
        return self.plan.output(mk.MK_OUT_LOGITS).cpu().numpy().reshape(self.cfg["batch"], -1)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,runs", [("tiny", 100), ("llama1b", 20)])
def test_gpu_repeated_runs_over_poisoned_workspace(name, runs):
    """Before every run the whole workspace (every intermediate and output) is
    set to NaN; each run must give the first run's logits bit for bit, with
    every counter at epoch * target.  A missing dependency would read NaN."""
    mk = _mk()
    st = Setup(name, norm_sigma=0.0 if name == "llama1b" else 0.1)
    try:
        ref = oracle.decode_step(st.inp)
        first = None
        for k in range(runs):
            if k:
                st.plan.poison_workspace()
            st.plan.run(st.w, st.kv, st.tokens)
            torch.cuda.synchronize()
            s, chk = st.plan.check()
            assert s == mk.MK_OK and chk.counters_ok == 1 and chk.epoch == k + 1, (k, s, chk.bad_counters)
            lg = st.logits()
            if first is None:
                first = lg
                rel = np.linalg.norm(lg - ref["logits"]) / np.linalg.norm(ref["logits"])
                print("  %s first run rel-L2 %.3g" % (name, rel), flush=True)
                assert rel <= LOGIT_TOL
            elif not np.array_equal(lg, first):
                pytest.fail("run %d differs from run 0 (max |diff| %g)" % (k, np.nanmax(np.abs(lg - first))))
        print("  %s: %d runs identical" % (name, runs), flush=True)
    finally:
        st.plan.free()


def test_gpu_watchdog_times_out_and_recovers():
    """A wait threshold raised by one above its event's producer count: the
    waiters' bounded waits give up, the grid drains and exits, and
    mk_plan_check reports MK_E_TIMEOUT with the record of the wait.  With the
    threshold restored, the next run (counters cleared) is correct again."""
    mk = _mk()
    st = Setup("tiny", opts=dict(timeout_ms=50))
    try:
        ref = oracle.decode_step(st.inp)
        st.plan.run(st.w, st.kv, st.tokens)
        s, chk = st.plan.check()
        assert s == mk.MK_OK and chk.counters_ok == 1
        ex = st.plan.export()
        waits = ex["task_wait"][ex["task_wait"] >= 0]
        ev = int(waits[len(waits) // 2])  # an event mid-step
        print("  raising the wait threshold of event %d by 1" % ev, flush=True)
        st.plan.debug_raise_wait(ev, 1)
        st.plan.run(st.w, st.kv, st.tokens)
        torch.cuda.synchronize()
        s, chk = st.plan.check()
        print("  status %d kind %d cu %d slot %d event %d value %d target %d" % (
            s, chk.err_kind, chk.err_cu, chk.err_slot, chk.err_event, chk.err_value, chk.err_target), flush=True)
        assert s == mk.MK_E_TIMEOUT and chk.err_kind != 0
        # the first wait to give up may be one on an event downstream of ev (its
        # producers wait on ev; events are numbered in consumer order), never an
        # event that does not depend on ev
        if chk.err_kind == 1:
            assert chk.err_event >= ev
            if chk.err_event == ev:
                assert chk.err_target == chk.epoch * (int(ex["event_target"][ev]) + 1)
        st.plan.debug_raise_wait(ev, -1)
        st.plan.run(st.w, st.kv, st.tokens)
        torch.cuda.synchronize()
        s, chk = st.plan.check()
        assert s == mk.MK_OK and chk.counters_ok == 1 and chk.epoch == 1
        lg = st.logits()
        assert np.linalg.norm(lg - ref["logits"]) / np.linalg.norm(ref["logits"]) <= LOGIT_TOL
    finally:
        st.plan.free()


def test_gpu_token_out_of_range_fails_the_run():
    """A token id outside [0, vocab) fails the run (mk_plan_check returns
    MK_E_INVALID) on both paths; a valid id afterwards runs clean."""
    mk = _mk()
    st = Setup("tiny")
    try:
        V = st.cfg["vocab"]
        for bad in (V, -1):
            for lw in (False, True):
                st.plan.run(st.w, st.kv, mk.tokens_to_device(np.array([bad], dtype=np.int32)), layerwise=lw)
                torch.cuda.synchronize()
                s, _ = st.plan.check()
                assert s == mk.MK_E_INVALID, (bad, lw, s)
                assert "token" in mk.lib().mk_last_error().decode()
        st.plan.run(st.w, st.kv, st.tokens)
        s, chk = st.plan.check()
        assert s == mk.MK_OK and chk.counters_ok == 1
    finally:
        st.plan.free()


def test_gpu_megakernel_refuses_stream_capture():
    """mk_run carries its epoch in the launch arguments, so it refuses capture
    (MK_E_UNSUPPORTED, nothing enqueued); the layerwise path captures."""
    mk = _mk()
    st = Setup("tiny")
    try:
        st.plan.run(st.w, st.kv, st.tokens, layerwise=True)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        err = None
        with torch.cuda.graph(g, stream=s):
            try:
                st.plan.run(st.w, st.kv, st.tokens, stream=s)
            except mk.MKError as e:
                err = e
            st.plan.run(st.w, st.kv, st.tokens, stream=s, layerwise=True)
        assert err is not None and err.status == mk.MK_E_UNSUPPORTED
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.decode_step(st.inp)
        assert np.array_equal(st.plan.output(mk.MK_OUT_NEXT_TOKEN).cpu().numpy(), ref["next"])
    finally:
        st.plan.free()


@pytest.mark.parametrize("name", ["tiny", "llama1b"])
def test_gpu_trace_stamps_every_instruction(name):
    """The trace of one step: every instruction slot of every queue is stamped
    (compute end and signal), NoOp slots are not, each queue's stamps are
    monotone, and the clock rate is the device's constant clock."""
    mk = _mk()
    st = Setup(name, norm_sigma=0.0 if name == "llama1b" else 0.1)
    try:
        st.plan.set_trace(True)
        st.plan.run(st.w, st.kv, st.tokens)
        torch.cuda.synchronize()
        s, chk = st.plan.check()
        assert s == mk.MK_OK and chk.counters_ok == 1
        tr, tpu = st.plan.trace()
        print("  ticks per us %.3f" % tpu, flush=True)
        assert 1.0 <= tpu <= 10000.0
        q = st.plan.export()["queue"]
        live = q[:, :, 0] != 0
        assert (tr[live][:, 2] > 0).all() and (tr[live][:, 3] > 0).all()
        assert (tr[~live] == 0).all()
        for c in range(q.shape[0]):
            n = int(live[c].sum())
            assert live[c, :n].all()  # each queue ends at its first NoOp
            done = tr[c, :n, 2].astype(np.int64)
            assert (np.diff(done) >= 0).all()
            assert (tr[c, :n, 3].astype(np.int64) >= done).all()
        span_us = (tr[live][:, 3].max() - tr[live][:, 0][tr[live][:, 0] > 0].min()) / tpu
        print("  %s traced step %.1f us" % (name, span_us), flush=True)
        assert 0 < span_us < 1e5
        st.plan.set_trace(False)
    finally:
        st.plan.free()
