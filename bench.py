"""Benchmark of one decode step: persistent megakernel vs the layerwise baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama1b | llama1b_b16 | qwen3_8b |
                                                           glm_preattn]

Prints ONE JSON line.  ``value`` is the megakernel's decode-step latency (us,
median over the timed steps, lower is better) on the Llama-3.2-1B-shaped
workload at batch 1 (hidden 2048, 16 layers, 32 q / 8 kv heads, head_dim 64,
FFN 8192, vocab 128256, tied LM head, KV length 1024), with inputs resident in
HBM.  ``roofline`` relates the algorithmic bytes of one step (every weight
once, the KV rows read and written, logits written) to that latency against
MI355X's 8 TB/s HBM peak.  The layerwise baseline (one launch per operator) is
timed the same way.  ``cpu_baseline`` is the CPU oracle (fp64 C, OpenMP over
output rows) timed on this host on whole steps of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-step latency (µs) + achieved HBM GB/s vs peak, Llama-1B-shape bs=1"
PEAK_GBPS = 8000.0
SHAPES = {"tiny": "tiny Llama-style", "llama1b": "Llama-3.2-1B-shaped", "llama1b_b16": "Llama-3.2-1B-shaped",
          "qwen3_8b": "Qwen3-8B-shaped"}
KERNEL_SOURCES = ["persistent_megakernel_decode_amd/csrc/mk_kernels.hip",
                  "persistent_megakernel_decode_amd/csrc/mk_device.hpp",
                  "persistent_megakernel_decode_amd/csrc/mk_glm.hpp"]


def algorithmic_bytes(cfg, kv_len):
    """Bytes one decode step must move: each weight once (norms included), the
    embedding row per sequence, KV rows read (kv_len[b] per layer, K and V),
    the new K/V rows written, fp32 logits written."""
    H, nq, nkv, hd, F, V, L = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                                "n_layers"))
    per_layer = (nq * hd * H + 2 * nkv * hd * H + H * nq * hd + 3 * F * H) + 2 * H
    if cfg["qk_norm"]:
        per_layer += 2 * hd
    weights = 2 * (L * per_layer + H + V * H)
    B = cfg["batch"]
    emb = 2 * B * H
    kv_read = sum(2 * L * nkv * int(k) * hd * 2 for k in kv_len)
    kv_write = 2 * L * nkv * hd * 2 * B
    logits = 4 * B * V
    return weights + emb + kv_read + kv_write + logits


def glm_algorithmic_bytes(cfg, w):
    """Bytes one GLM pre-attention step must move: every fp8 weight and its fp32
    block scales once, the bf16 norm weights, x and r in, and out: r_out, q,
    indexer q (bf16), the gate (fp32), the KV and indexer cache rows (bf16)."""
    import synth
    M, Na, Nqb, Niq = synth.glm_dims(cfg)
    weights = sum(int(a.nbytes) for a in w.values())
    io = 2 * M * cfg["hidden"] * 2 + M * cfg["hidden"] * 2
    out = M * (Nqb + Niq) * 2 + M * cfg["n_gate"] * 4 + M * (cfg["kv_lora"] + cfg["rope_dim"] + cfg["idx_head_dim"]) * 2
    return weights + io + out


def sources_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes per megakernel launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel calibration), or None when
    absent or taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic_%s_megakernel.json" % workload)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sources_sha256_16") != sources_hash():
        return None
    return d.get("bytes_per_launch")


def time_launches(fn, stream, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    outer0.record(stream)
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    outer1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])  # us
    return dict(median=float(np.median(per)), p10=float(np.percentile(per, 10)), p90=float(np.percentile(per, 90)),
                mean=float(per.mean()), outer_us_per_step=outer0.elapsed_time(outer1) * 1e3 / steps,
                wall_us_per_step=wall * 1e6 / steps)


def time_cold(fn, flush, stream, steps, warmup):
    """Like time_launches, with flush() (reads and writes a buffer larger
    than the L2s and the memory-side cache) issued before each timed launch,
    outside its events: every step then finds its weights and caches in HBM."""
    import torch
    for _ in range(warmup):
        flush()
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, e in ev:
        flush()
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])  # us
    return dict(median=float(np.median(per)), p10=float(np.percentile(per, 10)), p90=float(np.percentile(per, 90)),
                mean=float(per.mean()))


def capture(run):
    """Capture run(stream) (one step's launches) in a graph; returns its replay.
    The run is made once eagerly first so that the plan has bound its operand
    table (the capture then records kernel launches only, no copies or fills)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    torch.cuda.synchronize()
    return g.replay


OP_NAMES = {1: "qkv", 2: "attn", 3: "combine", 4: "oproj", 5: "gateup", 6: "down", 7: "lmhead", 8: "argmax",
            9: "glm_a0", 10: "glm_qkva", 11: "glm_gate", 12: "glm_idxk", 13: "glm_qanorm", 14: "glm_qkvb",
            15: "glm_idxq", 16: "glm_gate_red"}


def trace_report(tr, tpu, queue):
    """Decode one step's per-instruction trace (mk_plan_trace) into the
    measures of the MegaRTP article, sections 1 and 6: the active-CU fraction
    (time the compute units spend inside an instruction, from its input being
    ready to its outputs stored, over CUs x the step's span), the bubbles
    between consecutive instructions of a CU (median and share of the span),
    and per event the hand-off: the tail of its producers (last signal minus
    median signal) and its detection (median consumer start minus last signal).
    Times in us from the first stamp."""
    live = queue[:, :, 0] != 0
    C = queue.shape[0]
    ready, done, sig = tr[:, :, 1].astype(np.float64), tr[:, :, 2].astype(np.float64), tr[:, :, 3].astype(np.float64)
    evs = tr[:, :, 0].astype(np.float64)
    t0 = min(evs[live].min(), ready[live & (ready > 0)].min())
    us = lambda t: (t - t0) / tpu
    start = np.where(ready > 0, ready, evs)  # instructions without a compute stamp start at their event
    span = us(sig[live].max())
    busy, gaps = 0.0, []
    for c in range(C):
        n = int(live[c].sum())
        if n == 0:
            continue
        st, en = us(start[c, :n]), us(done[c, :n])
        # union of the CU's busy intervals (with two compute groups consecutive
        # instructions overlap); the gaps between them are its bubbles
        order = np.argsort(st, kind="stable")
        cur_s, cur_e = st[order[0]], en[order[0]]
        for k in order[1:]:
            if st[k] <= cur_e:
                cur_e = max(cur_e, en[k])
            else:
                busy += cur_e - cur_s
                gaps.append(st[k] - cur_e)
                cur_s, cur_e = st[k], en[k]
        busy += cur_e - cur_s
    gaps = np.array(gaps) if gaps else np.zeros(1)
    ops = {}
    hop_tail, hop_detect = [], []
    wait_ev, sig_ev = queue[:, :, 4], queue[:, :, 7]
    has_wait, has_sig = queue[:, :, 3] != 0, queue[:, :, 6] != 0
    E = int(max(wait_ev[live & has_wait].max(initial=-1), sig_ev[live & has_sig].max(initial=-1))) + 1
    for e in range(E):
        prod = live & has_sig & (sig_ev == e)
        cons = live & has_wait & (wait_ev == e)
        if not prod.any() or not cons.any():
            continue
        ps = us(sig[prod])
        hop_tail.append(float(ps.max() - np.median(ps)))
        hop_detect.append(float(np.median(us(evs[cons])) - ps.max()))
    for c in range(C):
        for i in range(int(live[c].sum())):
            key = (int(queue[c, i, 10]), OP_NAMES.get(int(queue[c, i, 0]), str(int(queue[c, i, 0]))))
            o = ops.setdefault(key, dict(first=1e30, last=0.0, dur=[]))
            o["first"] = min(o["first"], us(start[c, i]))
            o["last"] = max(o["last"], us(sig[c, i]))
            o["dur"].append(us(done[c, i]) - us(start[c, i]))
    per_op = {}
    for (layer, name), o in ops.items():
        a = per_op.setdefault(name, dict(tasks=0, task_us=[], span_us=[]))
        a["tasks"] += len(o["dur"])
        a["task_us"].append(float(np.median(o["dur"])))
        a["span_us"].append(o["last"] - o["first"])
    per_op = {k: dict(tasks=v["tasks"], median_task_us=round(float(np.median(v["task_us"])), 3),
                      median_span_us=round(float(np.median(v["span_us"])), 3)) for k, v in per_op.items()}
    span, busy = float(span), float(busy)
    return dict(traced_step_us=round(span, 2), active_cu_frac=round(busy / (C * span), 4),
                bubble_median_us=round(float(np.median(gaps)), 3),
                bubble_share=round(float(gaps.sum()) / (C * span), 4),
                hop_tail_median_us=round(float(np.median(hop_tail)), 3) if hop_tail else None,
                hop_detect_median_us=round(float(np.median(hop_detect)), 3) if hop_detect else None,
                events=len(hop_tail), per_op=per_op)


def traced_step(plan, run, dump=None):
    """One traced run of the megakernel after the timed ones (the trace stamps
    cost a few percent, so the timed steps run untraced); its decoded report.
    dump: a path to save the raw trace and queue (npz) to."""
    import torch
    plan.set_trace(True)
    run()
    torch.cuda.synchronize()
    tr, tpu = plan.trace()
    plan.set_trace(False)
    q = plan.export()["queue"]
    if dump:
        np.savez_compressed(dump, trace=tr, ticks_per_us=tpu, queue=q)
    return trace_report(tr, tpu, q)


def stream_ceiling(full=False, gib=2):
    """Streaming-read ceiling of the device (mk_stream_probe over a 2 GiB buffer,
    8x the memory-side cache): GB/s per configuration (median of 5 reads) and
    the best.  The default set covers the megakernel's own loader layout (2
    waves, 1 page in flight, LDS-DMA) and the best layouts of the full sweep."""
    import torch
    import persistent_megakernel_decode_amd as mk
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    if full:
        cfgs = [(1, 256, w, d) for w in (1, 2, 4, 8) for d in (1, 2, 3, 4) if w * d <= 8]
        cfgs += [(1, 512, 4, d) for d in (1, 2)] + [(0, g, w, d) for g in (256, 512, 1024) for w in (4, 8) for d in (1, 2)]
    else:
        cfgs = [(1, 256, 2, 1), (1, 256, 4, 2), (1, 256, 8, 1), (0, 256, 8, 2), (0, 1024, 8, 1)]
    stream = torch.cuda.current_stream()
    out = []
    for lds, g, w, d in cfgs:
        ts = []
        for k in range(7):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mk.stream_probe(buf, lds, g, w, d, sink)
            b.record(stream)
            b.synchronize()
            if k >= 2:
                ts.append(a.elapsed_time(b) * 1e-3)
        gbps = buf.numel() / float(np.median(ts)) / 1e9
        out.append(dict(mode="lds_dma" if lds else "registers", workgroups=g, waves=w, depth=d, GBps=round(gbps, 1)))
    del buf
    best = max(out, key=lambda r: r["GBps"])
    return dict(best_GBps=best["GBps"], best=best, configs=out)


def cpu_model():
    """The host CPU's model name (what lscpu reports), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _omp():
    """The OpenMP runtime the CPU oracle runs on (libgomp, loaded with it)."""
    import ctypes
    g = ctypes.CDLL("libgomp.so.1")
    g.omp_get_max_threads.restype = ctypes.c_int
    g.omp_set_num_threads.argtypes = [ctypes.c_int]
    return g


def cpu_baseline(inp, budget_s=20.0):
    """The fp64 C oracle on this host's cores: whole decode steps with every
    OpenMP thread (the reported value), then one step on one thread."""
    import oracle
    oracle.lib()
    omp = _omp()
    threads = int(omp.omp_get_max_threads())
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.decode_step(inp)
        n += 1
        if time.perf_counter() - t0 > budget_s * 0.5 or n >= 3:
            break
    dt = (time.perf_counter() - t0) / n
    omp.omp_set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.decode_step(inp)
        one = time.perf_counter() - t1
    finally:
        omp.omp_set_num_threads(threads)
    return dict(value=dt * 1e6, unit="us", cores=threads, kind="oracle",
                sample="%d whole decode step(s) of the same workload (fp64 C oracle, OpenMP over output rows), "
                       "then 1 step on 1 thread" % n,
                cpu_model=cpu_model(), one_thread_us=round(one * 1e6, 1))


def bench_glm(args):
    """The GLM-style pre-attention step (fp8 weights, 16 token rows).  Its 40 MB
    of weights fit the 256 MiB MALL, so it is timed warm (one weight copy, as a
    loop over one layer would see it) and cold (eight weight copies in turn, one
    plan each, 315 MB per round: every step's weights come from HBM)."""
    import torch
    import synth
    import persistent_megakernel_decode_amd as mk
    torch.cuda.set_device(0)
    name = args.workload
    inp = synth.make_glm_inputs(name)
    cfg = inp["cfg"]
    M = len(inp["pos"])
    cap = synth.glm_capacity(cfg)
    xr = mk.glm_inputs_to_device(inp["x"], inp["r"])
    caches = mk.glm_caches_to_device(inp["kv_cache"], inp["idx_cache"])
    ncopy = 8
    ws = [mk.GlmDeviceWeights(inp["weights"]) for _ in range(ncopy)]
    plans = [mk.Plan.build(cfg, M, inp["pos"], cap) for _ in range(ncopy)]
    stream = torch.cuda.current_stream()
    nbytes = glm_algorithmic_bytes(cfg, inp["weights"])
    res = {}
    for key, lw in (("mk", False), ("lw", True)):
        if args.only == "megakernel" and lw or args.only == "layerwise" and not lw:
            continue
        print("[bench] timing %s (warm, cold)" % ("layerwise" if lw else "megakernel"), file=sys.stderr, flush=True)
        res[key + "_warm"] = time_launches(lambda: plans[0].run(ws[0], caches, xr, layerwise=lw), stream,
                                           args.steps, args.warmup)
        it = [0]

        def cold():
            k = it[0] % ncopy
            it[0] += 1
            plans[k].run(ws[k], caches, xr, layerwise=lw)
        for p_, w_ in zip(plans, ws):  # bind every plan once (operand-table upload) before timing
            p_.run(w_, caches, xr, layerwise=lw)
        res[key + "_cold"] = time_launches(cold, stream, args.steps, args.warmup)
        if lw and not args.no_graph:
            print("[bench] timing layerwise as a captured graph", file=sys.stderr, flush=True)
            res["lw_graph_warm"] = time_launches(
                capture(lambda s: plans[0].run(ws[0], caches, xr, stream=s, layerwise=True)), stream,
                args.steps, args.warmup)
            # the pages' strongest baseline: graph + the independent branches on
            # streams of their own (QKV-A / gate / indexer-K; QKV-B / indexer-Q)
            print("[bench] timing layerwise as a captured graph with branch streams", file=sys.stderr, flush=True)
            pms = mk.Plan.build(cfg, M, inp["pos"], cap, lw_streams=3)
            res["lw_graph_ms_warm"] = time_launches(
                capture(lambda s: pms.run(ws[0], caches, xr, stream=s, layerwise=True)), stream,
                args.steps, args.warmup)
            pms.free()
        if not lw:
            st, chk = plans[0].check()
            if st != mk.MK_OK or not chk.counters_ok:
                raise RuntimeError("megakernel check failed: %s" % mk.lib().mk_last_error().decode())
            print("[bench] one traced megakernel step", file=sys.stderr, flush=True)
            res_trace = traced_step(plans[0], lambda: plans[0].run(ws[0], caches, xr), args.trace_dump)
    main_key = "mk_cold" if "mk_cold" in res else "lw_cold"
    lat = res[main_key]["median"]
    achieved = nbytes / (res[main_key]["mean"] * 1e-6) / 1e9
    out = {
        "metric": "GLM pre-attention step latency (µs), cold weights, + achieved HBM GB/s vs peak",
        "value": round(lat, 2), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res[main_key]["outer_us_per_step"] / 1e3, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 weights (fp32 128x128 block scales), fp8 activations, fp32 accumulate",
        "data": "synthetic (seeded, random-init weights of the workload's shape)",
        "config": {"workload": "%s: GLM-style pre-attention, M=%d (%d requests x %d tokens), hidden %d, fp8 weights, "
                               "KV position %d" % (name, M, cfg["n_seqs"], cfg["rows_per_seq"], cfg["hidden"],
                                                   cfg["pos0"]),
                   "weight_copies_cold": ncopy,
                   "persistent_grid": "%d workgroups x 512 threads" % plans[0].export()["num_cus"]},
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": None},
    }
    for k, v in res.items():
        out[k + "_us"] = {a: round(b, 2) for a, b in v.items()}
    if args.only != "layerwise":
        out["trace"] = res_trace
    if "mk_cold" in res and "lw_cold" in res:
        out["speedup_vs_layerwise_cold"] = round(res["lw_cold"]["median"] / res["mk_cold"]["median"], 3)
        out["speedup_vs_layerwise_warm"] = round(res["lw_warm"]["median"] / res["mk_warm"]["median"], 3)
    if "mk_warm" in res and "lw_graph_warm" in res:
        out["speedup_vs_layerwise_graph_warm"] = round(res["lw_graph_warm"]["median"] / res["mk_warm"]["median"], 3)
    if "mk_warm" in res and "lw_graph_ms_warm" in res:
        out["speedup_vs_layerwise_graph_branches_warm"] = round(
            res["lw_graph_ms_warm"]["median"] / res["mk_warm"]["median"], 3)
    if not args.no_cpu_baseline:
        from oracle import glm as G
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        n = 0
        while n < 3 and (n == 0 or time.perf_counter() - t0 < 10.0):
            G.glm_step(inp)
            n += 1
        out["cpu_baseline"] = dict(value=(time.perf_counter() - t0) / n * 1e6, unit="us",
                                   cores=int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), kind="oracle",
                                   sample="%d whole step(s) of the same workload (fp64 numpy oracle)" % n,
                                   cpu_model=cpu_model())
    for p_ in plans:
        p_.free()
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-captured layerwise baseline")
    ap.add_argument("--only", choices=["megakernel", "layerwise", "both"], default="both")
    ap.add_argument("--trace-dump", default=None, help="save the traced step's raw trace and queue (npz) here")
    ap.add_argument("--pairing", type=int, default=0, choices=[0, 1],
                    help="plan with the pairing strategies (mk_plan_opts.pairing) instead of the gcd/lcm rules")
    ap.add_argument("--dma-pages", type=int, default=0, choices=[0, 1, 2, 3],
                    help="weight pages each loader wave keeps in flight (mk_plan_opts.dma_pages; 0: default)")
    ap.add_argument("--attn-order", type=int, default=0, choices=[-1, 0, 1],
                    help="attention placement (mk_plan_opts.attn_order): 1 longest first, -1 plan order, "
                         "0 the default (longest first at batch > 1)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only sweep the streaming-read probe (mk_stream_probe) and print its JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first launch one device-to-device copy of 256 MiB (read 256 MiB, write 256 MiB), so that "
                         "a profiler run can scale its HBM byte counters by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode megakernel is a single-GPU design here "
              "(no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.stream_ceiling:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(stream_ceiling(full=True)))
        return
    if args.workload.startswith("glm"):
        return bench_glm(args)
    import torch
    import synth
    import persistent_megakernel_decode_amd as mk

    torch.cuda.set_device(0)
    print("[bench] generating %s inputs" % args.workload, file=sys.stderr, flush=True)
    inp = synth.make_inputs(args.workload)
    cfg = inp["cfg"]
    w = mk.DeviceWeights(inp["weights"], cfg)
    kv = mk.kv_to_device(inp["kv_cache"])
    tok = mk.tokens_to_device(inp["tokens"])
    plan = mk.Plan.build(cfg, cfg["batch"], inp["kv_len"], inp["kv_cache"].shape[4], pairing=args.pairing,
                         attn_order=args.attn_order, dma_pages=args.dma_pages)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    nbytes = algorithmic_bytes(cfg, inp["kv_len"])
    res = {}
    if args.only in ("megakernel", "both"):
        print("[bench] timing megakernel", file=sys.stderr, flush=True)
        res["mk"] = time_launches(lambda: plan.run(w, kv, tok), stream, args.steps, args.warmup)
        st, chk = plan.check()
        if st != mk.MK_OK or not chk.counters_ok:
            raise RuntimeError("megakernel check failed: %s" % mk.lib().mk_last_error().decode())
        print("[bench] one traced megakernel step", file=sys.stderr, flush=True)
        res["trace"] = traced_step(plan, lambda: plan.run(w, kv, tok), args.trace_dump)
        # a decode loop: 8 steps per call (mk_run_steps), each step's argmax fed to
        # the next, the plan moved to each step's lengths without replanning
        print("[bench] timing an 8-step decode loop", file=sys.stderr, flush=True)
        kv_loop = mk.kv_to_device(inp["kv_cache"])
        kv0 = inp["kv_len"]

        def loop():
            plan.set_kv_len(kv0)
            plan.run_steps(w, kv_loop, tok, 8)
        r = time_launches(loop, stream, max(2, args.steps // 8), 2)
        res["mk_loop"] = {k: v / 8 for k, v in r.items()}
        plan.set_kv_len(kv0)
    if args.only in ("layerwise", "both"):
        print("[bench] timing layerwise", file=sys.stderr, flush=True)
        # the baseline's own best split count: its attention reads K/V in place,
        # so the megakernel's split rule (set by the LDS page ring) need not suit
        # it; batched plans are also timed with twice the splits
        S = plan.export()["tile_opts"]["attn_splits"]
        lw_plan, lw_S = plan, S
        res["lw"] = time_launches(lambda: plan.run_layerwise(w, kv, tok), stream, args.steps, args.warmup)
        if cfg["batch"] > 1:
            alt = mk.Plan.build(cfg, cfg["batch"], inp["kv_len"], inp["kv_cache"].shape[4], attn_splits=2 * S)
            r2 = time_launches(lambda: alt.run_layerwise(w, kv, tok), stream, args.steps, args.warmup)
            if r2["median"] < res["lw"]["median"]:
                res["lw"], lw_plan, lw_S = r2, alt, 2 * S
        res["lw_splits"] = lw_S
        if not args.no_graph:
            # the stronger baseline: the same launches captured once in a HIP graph
            # and replayed (no per-launch host cost)
            print("[bench] timing layerwise as a captured graph", file=sys.stderr, flush=True)
            res["lw_graph"] = time_launches(capture(lambda s: lw_plan.run_layerwise(w, kv, tok, stream=s)), stream,
                                            args.steps, args.warmup)
    if args.workload == "tiny":
        # the tiny model (2.4 MB of weights) stays in the caches between steps;
        # it is also timed cold, every step after a 512 MiB cache flush
        big = torch.empty(256 << 20, dtype=torch.float16, device="cuda")
        flush = lambda: big.add_(1)
        for key, lwf in (("mk_cold", False), ("lw_cold", True)):
            if args.only == "megakernel" and lwf or args.only == "layerwise" and not lwf:
                continue
            print("[bench] timing %s cold" % ("layerwise" if lwf else "megakernel"), file=sys.stderr, flush=True)
            run = (lambda: plan.run_layerwise(w, kv, tok)) if lwf else (lambda: plan.run(w, kv, tok))
            res[key] = time_cold(run, flush, stream, args.steps, args.warmup)
        del big
    torch.cuda.synchronize()
    print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
    ceil = stream_ceiling()
    main_key = "mk" if "mk" in res else "lw"
    lat = res[main_key]["median"]
    # roofline: algorithmic bytes per launch over the kernel's average launch
    # duration (HIP events on the launch stream, every timed step)
    achieved = nbytes / (res[main_key]["mean"] * 1e-6) / 1e9
    traffic = traffic_from_profiles(args.workload) if main_key == "mk" else None
    out = {
        "metric": METRIC,
        "value": round(lat, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res[main_key]["outer_us_per_step"] / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 accumulate",
        "data": "synthetic (seeded, random-init weights of the workload's shape)",
        "config": {"workload": "%s: %s decode step, batch %d, KV %s, %d layers, hidden %d"
                   % (args.workload, SHAPES.get(args.workload, "Llama-family"), cfg["batch"],
                      str(int(inp["kv_len"][0])) if cfg["batch"] == 1 else "%d..%d" % (min(inp["kv_len"]), max(inp["kv_len"])),
                      cfg["n_layers"], cfg["hidden"]),
                   "batch": int(cfg["batch"]), "kv_len": [int(k) for k in inp["kv_len"]],
                   "persistent_grid": "%d workgroups x %d threads" % (plan.export()["num_cus"],
                                                                      512 if cfg["batch"] == 1 else 768),
                   "plan": {"pairing": args.pairing, "attn_order": plan.export()["attn_order"]}},
        "algorithmic_bytes": nbytes,
        "achieved_GBps": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
        # second denominator: the best plain streaming read measured on this device
        "stream_ceiling": {"GBps": ceil["best_GBps"], "config": ceil["best"],
                           "loader_layout_GBps": ceil["configs"][0]["GBps"],
                           "frac_of_ceiling": round(achieved / ceil["best_GBps"], 4)},
    }
    if "mk" in res:
        out["megakernel_us"] = {k: round(v, 2) for k, v in res["mk"].items()}
    if "trace" in res:
        out["trace"] = res["trace"]
    if "mk_loop" in res:
        # per step of an 8-step mk_run_steps call (includes each step's queue
        # patch, RoPE copy and token hand-over; per-step percentiles are of calls / 8)
        out["decode_loop_us_per_step"] = {k: round(v, 2) for k, v in res["mk_loop"].items()}
    if "lw" in res:
        out["layerwise_us"] = {k: round(v, 2) for k, v in res["lw"].items()}
        out["layerwise_attn_splits"] = res["lw_splits"]
        lwl = res["lw"]["median"]
        out["layerwise_achieved_GBps"] = round(nbytes / (lwl * 1e-6) / 1e9, 1)
        if "mk" in res:
            out["speedup_vs_layerwise"] = round(lwl / lat, 3)
    if "mk_cold" in res:
        out["megakernel_cold_us"] = {k: round(v, 2) for k, v in res["mk_cold"].items()}
    if "lw_cold" in res:
        out["layerwise_cold_us"] = {k: round(v, 2) for k, v in res["lw_cold"].items()}
        if "mk_cold" in res:
            out["speedup_vs_layerwise_cold"] = round(res["lw_cold"]["median"] / res["mk_cold"]["median"], 3)
    if "lw_graph" in res:
        out["layerwise_graph_us"] = {k: round(v, 2) for k, v in res["lw_graph"].items()}
        if "mk" in res:
            out["speedup_vs_layerwise_graph"] = round(res["lw_graph"]["median"] / lat, 3)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp)
    plan.free()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
