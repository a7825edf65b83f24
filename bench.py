"""Benchmark of one decode step: persistent megakernel vs the layerwise baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload llama1b]

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
                  "persistent_megakernel_decode_amd/csrc/mk_device.hpp"]


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


def cpu_baseline(inp, budget_s=20.0):
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.decode_step(inp)
        n += 1
        if time.perf_counter() - t0 > budget_s * 0.5 or n >= 3:
            break
    dt = (time.perf_counter() - t0) / n
    return dict(value=dt * 1e6, unit="us", cores=threads, kind="oracle",
                sample="%d whole decode step(s) of the same workload (fp64 C oracle, OpenMP over output rows)" % n)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["megakernel", "layerwise", "both"], default="both")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first launch one device-to-device copy of 256 MiB (read 256 MiB, write 256 MiB), so that "
                         "a profiler run can scale its HBM byte counters by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the decode megakernel is a single-GPU design here "
              "(no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)
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
    plan = mk.Plan.build(cfg, cfg["batch"], inp["kv_len"], inp["kv_cache"].shape[4])
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
    if args.only in ("layerwise", "both"):
        print("[bench] timing layerwise", file=sys.stderr, flush=True)
        res["lw"] = time_launches(lambda: plan.run_layerwise(w, kv, tok), stream, args.steps, args.warmup)
    torch.cuda.synchronize()
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
                   "persistent_grid": "%d workgroups x 512 threads" % plan.export()["num_cus"]},
        "algorithmic_bytes": nbytes,
        "achieved_GBps": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
    }
    if "mk" in res:
        out["megakernel_us"] = {k: round(v, 2) for k, v in res["mk"].items()}
    if "lw" in res:
        out["layerwise_us"] = {k: round(v, 2) for k, v in res["lw"].items()}
        lwl = res["lw"]["median"]
        out["layerwise_achieved_GBps"] = round(nbytes / (lwl * 1e-6) / 1e9, 1)
        if "mk" in res:
            out["speedup_vs_layerwise"] = round(lwl / lat, 3)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp)
    plan.free()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
