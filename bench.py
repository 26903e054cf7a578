#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

Measures decode tokens/s and achieved HBM bandwidth of the hipGraph-replayed
fused decode step on seeded synthetic inputs, and prints one JSON line.

Workload (default): the 8B-class dense decoder -- 32 layers, d_model 4096, 32
query / 8 KV heads of 128, SwiGLU 14336, vocab 128256, bf16 weights N(0, 0.02),
bf16 paged KV (blocks of 16) -- at batch 1, per-sequence context lengths
uniform in [256, 1024] (context K/V drawn N(0, 1) straight into the cache),
teacher-forced token ids uniform in [0, vocab), 40 decode steps.  The same
model at batch 32 is measured as the metric's second batch size.

A step is one dec_step call: host packing of ids / positions / block tables,
one H2D copy into the static buffers, one graph replay.  `value` is decode
tokens/s = batch x steps / wall time of the timed loop (inputs resident in HBM,
torch.cuda.synchronize() on both sides).  Bandwidth counts the algorithmic
bytes of each step: all weights once (only the batch's embedding rows), the KV
read over every position plus the new token's K/V, and the fp32 logits.

Extra objects on the line:
  roofline      the dominant kernel (gate+up projection with SiLU x mul, about
                54% of the step's bytes at batch 1), timed alone with events on
                the library's stream: algorithmic bytes per launch / duration
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the
                same step (two layers + final norm + LM head, extrapolated)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec at batch 1 and 32; achieved HBM GB/s vs ~8 TB/s peak"
REPS_CPU = 5  # repeats of the CPU oracle's timed truncations (about 10 s of host work at 8B)
PEAK_GBPS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gate_up_bytes(cfg, B: int, mfma: bool) -> int:
    """Algorithmic bytes of one gate+up launch: the weights once (+ fp8 row scales),
    the input read once -- the fp32 residual rows and the norm gain where the
    matrix-vector kernel normalizes its own input, else (MFMA tiles) the bf16
    activations -- and the bf16 SiLU x mul output written."""
    b = 1 if cfg.weight_dtype == "fp8" else 2
    w = 2 * cfg.d_ff * cfg.d_model * b + (2 * cfg.d_ff * 4 if cfg.weight_dtype == "fp8" else 0)
    x = B * cfg.d_model * 2 if mfma else B * cfg.d_model * 4 + cfg.d_model * 4
    return w + x + B * cfg.d_ff * 2


def traffic_file(workload: str, B: int) -> str:
    return os.path.join(ROOT, "profiles", f"k_gemv_norm_gate_up_{workload}_b{B}_traffic.txt")


def measured_traffic(workload: str, B: int):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    or None when there is none or it was taken on other kernel sources."""
    from memory_bound_transformer_decode_amd import profile_summary as ps

    path = traffic_file(workload, B)
    if not os.path.exists(path):
        return None
    t = ps.read_traffic(path)
    if t.get("source_sha256") != ps.kernel_source_sha256():
        log(f"{os.path.basename(path)} was measured on other kernel sources: traffic not reported")
        return None
    return int(float(t["traffic_bytes_per_dispatch"]))


def copy_calibration(nbytes: int) -> int:
    """Device-to-device copies of a known size, for scaling the HBM byte counters."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "copies": 3}), flush=True)
    return 0


def run_batch(wl, B: int, steps: int, warmup: int, seed: int, want_eager: bool, want_kernel: bool,
              weights=None, base_flags: int = 0):
    import torch

    from memory_bound_transformer_decode_amd import dec, perfmodel, synth

    cfg = wl.model
    max_seq = wl.ctx_hi + steps
    bps = synth.blocks_per_seq(max_seq)
    nb = B * bps
    if weights is None:
        t0 = time.time()
        weights = synth.make_weights(cfg, seed=seed, device="cuda")
        torch.cuda.synchronize()
        log(f"drew {cfg.name} weights ({weights.nbytes() / 1e9:.2f} GB) in {time.time() - t0:.1f}s")
    lens0 = synth.make_context_lengths(wl, B, seed=seed)
    bt = synth.make_block_tables(cfg, B, max_seq, nb, seed=seed)
    pool = synth.empty_kv_pool(cfg, nb, device="cuda", canary=False)
    synth.fill_context_kv(cfg, pool, bt, lens0, seed=seed)
    ids = synth.make_token_ids(cfg, max(steps, warmup), B, seed=seed)
    d = dec.Decoder(cfg, weights, num_blocks=nb, max_batch=dec.ladder_bucket(B), max_seq_len=max_seq,
                    kv_pool=pool)
    shape = perfmodel.Shape.of(cfg)

    def timed(flags: int):
        d.set_flags(flags)
        for t in range(warmup):  # rewrites the first timed step's slots; captures the graph
            d.step(ids[t], lens0, bt)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for t in range(steps):
            d.step(ids[t], lens0 + t, bt)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) / 1e3

    wall, ev = timed(base_flags)
    info = d.info()
    step_bytes = sum(shape.step_bytes(lens0 + t) for t in range(steps))
    res = {
        "batch": B, "steps": steps, "wall_s": wall, "event_s": ev,
        "tok_s": B * steps / wall, "ms_per_step": 1e3 * wall / steps,
        "bytes_per_step": step_bytes / steps, "achieved_gbps": step_bytes / wall / 1e9,
        "kernels_per_step": info.kernels_per_step, "bucket": info.bucket, "used_mfma": info.used_mfma,
        "persistent": bool(info.persistent),
        "attn_splits": info.attn_splits, "graph": bool(info.used_graph),
        "flops_per_step": sum(shape.step_flops(lens0 + t) for t in range(steps)) / steps,
    }
    res["frac_of_peak"] = res["achieved_gbps"] / PEAK_GBPS
    if info.persistent:
        # the step is a single kernel: its duration is the event time per step (which
        # also holds the small H2D copy of the step inputs that precedes the kernel)
        res["kernel"] = {"name": "k_step (whole step, one persistent kernel)", "avg_s": ev / steps,
                         "bytes": step_bytes / steps, "gbps": step_bytes / ev / 1e9, "launches": steps}
    if want_eager:
        plans = {}
        for name, flags in (("persistent_graph", dec.FLAG_PERSISTENT),
                            ("multi_kernel_eager", dec.FLAG_EAGER),
                            ("fused_qkv_attention_graph", dec.FLAG_FUSED_QKV_ATTN),
                            ("unfused_graph", dec.FLAG_UNFUSED),
                            ("unfused_eager", dec.FLAG_UNFUSED | dec.FLAG_EAGER)):
            w2, _ = timed(flags)
            plans[name] = {"tok_s": B * steps / w2, "ms_per_step": 1e3 * w2 / steps,
                           "kernels_per_step": d.info().kernels_per_step}
        res["plans"] = plans
        d.set_flags(0)
    if want_kernel and "kernel" not in res:
        # the dominant kernel alone: one launch per layer back to back (distinct weights
        # each launch, so no launch is served from a cache), timed with events on the
        # library's stream (the torch stream the decoder was created on) around all L
        # launches; the average includes the short gaps between launches
        L = cfg.n_layers
        durs = []
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(L):
                d.launch_matmul(dec.MAT_GATE_UP, l)
            e1.record()
            torch.cuda.synchronize()
            if rep > 0:
                durs.append(e0.elapsed_time(e1) / 1e3 / L)
        avg = float(np.mean(durs))
        nbytes = gate_up_bytes(cfg, B, bool(info.used_mfma))
        res["kernel"] = {"name": ("k_gemm_lds" if info.used_mfma else "k_gemv_norm") + " gate+up + SiLU x mul",
                         "avg_s": avg, "bytes": nbytes, "gbps": nbytes / avg / 1e9, "launches": len(durs) * L}
    d.close()
    del pool
    return res, weights


def cpu_baseline(wl, B: int, weights, seed: int, budget_s: float):
    """fp64 oracle on the host: time 1-layer and 2-layer truncations of the same step
    (embedding, layers, final norm, LM head; weights already on the host) and
    extrapolate linearly to the full depth."""
    import torch

    from memory_bound_transformer_decode_amd import synth
    from oracle import decoder as OD
    from oracle import inputs as OI

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    cfg = wl.model
    max_seq = wl.ctx_hi + 1
    nb = B * synth.blocks_per_seq(max_seq)
    lens = synth.make_context_lengths(wl, B, seed=seed)
    bt = synth.make_block_tables(cfg, B, max_seq, nb, seed=seed)
    # the context KV of the first two layers, drawn by the same generator as on the GPU
    c2 = cfg.with_layers(2)
    pool = synth.empty_kv_pool(c2, nb, device="cuda", canary=False)
    synth.fill_context_kv(c2, pool, bt, lens, seed=seed)
    codes = synth.kv_codes_numpy(pool)
    del pool
    m = OI.model(weights, n_layers=2)  # host copies of the codes (transfer not timed)
    ids = synth.make_token_ids(cfg, 1, B, seed=seed)[0]
    times = {1: float("inf"), 2: float("inf")}
    for rep in range(REPS_CPU):  # best of a few repeats of each truncation
        for L in (1, 2):
            cache = OI.cache(c2, codes)
            t0 = time.perf_counter()
            OD.decode_step(m, cache, ids, lens, bt, n_layers=L)
            times[L] = min(times[L], time.perf_counter() - t0)
    per_layer = max(times[2] - times[1], 1e-9)
    step = times[1] + (cfg.n_layers - 1) * per_layer
    torch.cuda.empty_cache()
    return {"value": B / step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"one {cfg.name} decode step at batch {B}: embedding, 1 and 2 layers, final "
                       f"norm and LM head, best of {REPS_CPU} runs each ({times[1]:.1f}s, {times[2]:.1f}s), "
                       f"extrapolated linearly to {cfg.n_layers} layers = {step:.1f}s per step"),
            "host_cpus": os.cpu_count()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8B", help="tiny | 1B | 8B | 32B | 70B")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--second-batch", type=int, default=32, help="0 to skip")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip eager, kernel and probe legs")
    ap.add_argument("--eager", action="store_true",
                    help="launch the main leg's kernels one by one (for counter collection)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES device-to-device 3 times (scales the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode step here runs on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        return 2

    import torch

    from memory_bound_transformer_decode_amd import dec, synth

    dec.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    wl = synth.WORKLOADS[args.workload]
    cfg = wl.model
    extras = not args.no_extras
    log(f"workload {args.workload} batch {args.batch}, {args.steps} steps, {args.warmup} warmup")
    main_res, weights = run_batch(wl, args.batch, args.steps, args.warmup, args.seed,
                                  want_eager=extras, want_kernel=True,
                                  base_flags=dec.FLAG_EAGER if args.eager else 0)
    log(f"batch {args.batch}: {main_res['tok_s']:.1f} tok/s, {main_res['ms_per_step']:.3f} ms/step, "
        f"{main_res['achieved_gbps']:.0f} GB/s ({100 * main_res['frac_of_peak']:.1f}% of 8 TB/s)")
    second = None
    if args.second_batch and args.second_batch != args.batch and args.second_batch in wl.batches:
        second, _ = run_batch(wl, args.second_batch, args.steps, args.warmup, args.seed,
                              want_eager=False, want_kernel=False, weights=weights)
        log(f"batch {args.second_batch}: {second['tok_s']:.1f} tok/s, {second['ms_per_step']:.3f} ms/step, "
            f"{second['achieved_gbps']:.0f} GB/s")
    probe = None
    if extras:
        buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        probe = dec.bw_probe(buf, reps=5) / 1e9
        del buf
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.batch, weights, args.seed, 20.0)
        log(f"cpu oracle: {cpu['value']:.4f} tok/s on {cpu['cores']} threads")

    k = main_res["kernel"]
    line = {
        "metric": METRIC,
        "value": round(main_res["tok_s"], 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.weight_dtype,
        "data": "synthetic: seeded N(0,0.02) weights, N(0,1) context K/V, uniform token ids",
        "config": {
            "workload": (f"{cfg.name}-class dense decoder: {cfg.n_layers} layers, d_model {cfg.d_model}, "
                         f"{cfg.n_q_heads} q / {cfg.n_kv_heads} kv heads x {cfg.d_head}, SwiGLU {cfg.d_ff}, "
                         f"vocab {cfg.vocab}, {cfg.weight_dtype} weights, {cfg.kv_dtype} paged KV (16/block); "
                         f"batch {args.batch}; context U[{wl.ctx_lo},{wl.ctx_hi}] per sequence; "
                         f"{args.steps} decode steps; hipGraph replay per step"),
            "batch": args.batch,
            "kernels_per_step": main_res["kernels_per_step"],
            "persistent_step": main_res["persistent"],
            "attn_splits": main_res["attn_splits"],
        },
        "hbm": {"achieved_gbps": round(main_res["achieved_gbps"], 1),
                "frac_of_peak": round(main_res["frac_of_peak"], 4),
                "bytes_per_step": int(main_res["bytes_per_step"]),
                "probe_read_gbps": round(probe, 1) if probe else None},
        "roofline": {"bound": "hbm", "achieved": round(k["gbps"], 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k["gbps"] / PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.workload, args.batch) if args.batch <= 8 else None,
                     "kernel": k["name"],
                     "bytes_per_launch": int(k["bytes"]), "avg_us": round(k["avg_s"] * 1e6, 2),
                     "launches": k["launches"]},
        "cpu_baseline": cpu,
    }
    if "plans" in main_res:
        pl = {"persistent_graph" if main_res["persistent"] else "multi_kernel_graph":
              {"tok_s": round(main_res["tok_s"], 3), "ms_per_step": round(main_res["ms_per_step"], 4),
               "kernels_per_step": main_res["kernels_per_step"]}}
        for k2, v in main_res["plans"].items():
            pl[k2] = {"tok_s": round(v["tok_s"], 3), "ms_per_step": round(v["ms_per_step"], 4),
                      "kernels_per_step": v["kernels_per_step"]}
        line["plans"] = pl
    if second:
        line[f"batch{second['batch']}"] = {
            "value": round(second["tok_s"], 2), "unit": "tokens/s",
            "ms_per_step": round(second["ms_per_step"], 4),
            "achieved_gbps": round(second["achieved_gbps"], 1),
            "frac_of_peak": round(second["frac_of_peak"], 4), "used_mfma": second["used_mfma"],
            "kernels_per_step": second["kernels_per_step"]}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
