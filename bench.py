#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

Measures decode tokens/s and achieved HBM bandwidth of the hipGraph-replayed
fused decode step on seeded synthetic inputs, and prints one JSON line.

Headline (`value`): the 8B-class dense decoder -- 32 layers, d_model 4096, 32
query / 8 KV heads of 128, SwiGLU 14336, vocab 128256, bf16 weights N(0, 0.02),
bf16 paged KV (blocks of 16) -- at batch 1, per-sequence context lengths
uniform in [256, 1024] (context K/V drawn N(0, 1) straight into the cache),
teacher-forced token ids uniform in [0, vocab): decode tokens/s, the median of
REPEATS timed loops of `--steps` steps.

A step is one dec_step call: host packing of ids / positions / block tables,
one H2D copy into the static buffers, one graph replay.  tokens/s = batch x
steps / wall time of the timed loop (inputs resident in HBM,
torch.cuda.synchronize() on both sides).  Bandwidth counts the algorithmic
bytes of each step: all weights once (only the batch's embedding rows), the KV
read over every position plus the new tokens' K/V, and the fp32 logits.

Further legs on the same line (each a dict; `--legs none` skips them):
  batch32      the 8B model at batch 32 (the metric's second batch size)
  plans        8B batch 1: eager launches, attention and O as separate launches, and
               the unfused plan (graph and eager)
  workloads    1B batch 1 (graph and eager: the launch-bound regime), 32B and 70B
               at batch 1, 70B at batch 64, the 8B model with int8 weights; each
               with its dominant kernel's roofline
  prefill      time to first token of a 1024-token 8B prompt (chunks of 64)
  verify       the 8B k-token verify step at k = 4 and 8
  roofline     the dominant kernel of the headline (gate+up + SiLU x mul, 54 % of
               the bytes at batch 1) timed alone with HIP events on the library's
               stream: algorithmic bytes per launch / average duration; traffic
               from the committed counter summary when it was taken on these sources
  cpu_baseline the fp64 oracle on the host cores, on a bounded sample of the same
               step (1 and 2 layers + final norm + LM head, extrapolated)
  pages        the pages' own figures, with the hardware they were quoted on
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
REPEATS = 5  # timed loops per headline leg (median and best reported)
REPS_CPU = 5  # repeats of the CPU oracle's timed truncations (about 10 s of host work at 8B)
PEAK_GBPS = 8000.0
ALL_LEGS = ("batch32", "plans", "workloads", "prefill", "verify")

# The pages' figures, quoted with their hardware (context, not targets).
PAGES = {
    "h100_sxm_hbm_tb_s": 3.35,
    "h100_70b_fp8_weight_only_bound_tok_s": 48,
    "mi355x_70b_fp8_weight_only_bound_tok_s_at_8tb_s": round(8e12 / 69.874e9, 1),
    "study_32b_fp8_tok_s_before_after": [120, 195],
    "study_bandwidth_utilization_before_after": [0.52, 0.76],
    "study_whole_stack_gain": 1.7,
    "study_note": ("H100 80 GB SXM, FP8 weights and KV, 32B-class model; the study calls itself "
                   "hypothetical; the 1.7x is fusion + FlashAttention + CUDA graphs + batching + FP8 together"),
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gate_up_bytes(cfg, B: int, mfma: bool) -> int:
    """Algorithmic bytes of one gate+up launch: the weights once (+ one-byte row scales),
    the input read once -- the fp32 residual rows and the norm gain where the
    matrix-vector kernel normalizes its own input, else (MFMA tiles) the bf16
    activations -- and the bf16 SiLU x mul output written."""
    b = 2 if cfg.weight_dtype == "bf16" else 1
    w = 2 * cfg.d_ff * cfg.d_model * b + (0 if cfg.weight_dtype == "bf16" else 2 * cfg.d_ff * 4)
    x = B * cfg.d_model * 2 if mfma else B * cfg.d_model * 4 + cfg.d_model * 4
    return w + x + B * cfg.d_ff * 2


def measured_traffic(name: str, family: str):
    """HBM bytes per launch of a kernel from the committed counter summary
    profiles/<name>_traffic.txt, or None when there is none or it was taken on other
    kernel sources."""
    from memory_bound_transformer_decode_amd import profile_summary as ps

    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = ps.read_traffic(path)
    if t.get("source_sha256") != ps.kernel_source_sha256(family):
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


def draw_weights(cfg, seed: int):
    import torch

    from memory_bound_transformer_decode_amd import synth

    t0 = time.time()
    w = synth.make_weights(cfg, seed=seed, device="cuda")
    torch.cuda.synchronize()
    log(f"drew {cfg.name} weights ({w.nbytes() / 1e9:.2f} GB) in {time.time() - t0:.1f}s")
    return w


class Leg:
    """One (model, batch) decode context with its context KV drawn into the pool."""

    def __init__(self, wl, B: int, steps: int, seed: int, weights, flags: int = 0, max_batch: int = 0):
        import torch

        from memory_bound_transformer_decode_amd import dec, perfmodel, synth

        self.wl, self.B, self.steps = wl, B, steps
        cfg = self.cfg = wl.model
        self.max_seq = wl.ctx_hi + steps + 8
        nb = B * synth.blocks_per_seq(self.max_seq)
        self.lens0 = synth.make_context_lengths(wl, B, seed=seed)
        self.bt = synth.make_block_tables(cfg, B, self.max_seq, nb, seed=seed)
        self.pool = synth.empty_kv_pool(cfg, nb, device="cuda", canary=False)
        synth.fill_context_kv(cfg, self.pool, self.bt, self.lens0, seed=seed)
        self.ids = synth.make_token_ids(cfg, steps + 8, B, seed=seed)
        # the decoder's stream: a stream of its own, so that its launches can be captured
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            self.d = dec.Decoder(cfg, weights, num_blocks=nb, max_batch=max(max_batch, dec.ladder_bucket(B)),
                                 max_seq_len=self.max_seq, kv_pool=self.pool, flags=flags)
        self.shape = perfmodel.Shape.of(cfg)
        torch.cuda.synchronize()

    def timed(self, flags: int, warmup: int, per_step: bool = False):
        """One timed loop of self.steps steps after `warmup` untimed ones (which also
        capture the graph): (wall seconds, per-step seconds or None)."""
        import torch

        d = self.d
        d.set_flags(flags)
        for t in range(warmup):
            d.step(self.ids[t], self.lens0, self.bt)
        torch.cuda.synchronize()
        evs = None
        if per_step:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(self.steps + 1)]
            evs[0].record(self.stream)
        t0 = time.perf_counter()
        for t in range(self.steps):
            d.step(self.ids[t], self.lens0 + t, self.bt)
            if per_step:
                evs[t + 1].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps_s = [evs[t].elapsed_time(evs[t + 1]) / 1e3 for t in range(self.steps)] if per_step else None
        return wall, steps_s

    def step_bytes(self) -> float:
        return sum(self.shape.step_bytes(self.lens0 + t) for t in range(self.steps)) / self.steps

    def measure(self, flags: int, warmup: int, repeats: int, per_step: bool = False) -> dict:
        walls, dist = [], None
        for r in range(repeats):
            w, st = self.timed(flags, warmup if r == 0 else 1, per_step=per_step and r == 0)
            walls.append(w)
            if st:
                dist = st
        info = self.d.info()
        med = float(np.median(walls))
        best = float(np.min(walls))
        sb = self.step_bytes()
        res = {"tok_s": self.B * self.steps / med, "tok_s_best": self.B * self.steps / best,
               "ms_per_step": 1e3 * med / self.steps, "repeats": repeats,
               "tok_s_all": [round(self.B * self.steps / w, 2) for w in walls],
               "achieved_gbps": sb * self.steps / med / 1e9, "bytes_per_step": sb,
               "kernels_per_step": info.kernels_per_step, "used_mfma": info.used_mfma,
               "attn_splits": info.attn_splits, "graph": bool(info.used_graph)}
        res["frac_of_peak"] = res["achieved_gbps"] / PEAK_GBPS
        if dist:
            a = np.array(dist) * 1e3
            res["step_ms_p50"], res["step_ms_p90"], res["step_ms_max"] = (
                float(np.percentile(a, 50)), float(np.percentile(a, 90)), float(a.max()))
        return res

    def gate_up_kernel(self) -> dict:
        """The gate+up kernel alone: one launch per layer (distinct weights each launch,
        so none is served from a cache), the L launches captured into a graph on the
        decoder's stream -- as the step runs them -- and the graph's replays timed with
        events on that stream (three, after one warm-up replay); the average includes
        the graph's short gaps between kernels."""
        import torch

        from memory_bound_transformer_decode_amd import dec

        L = self.cfg.n_layers
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for l in range(L):
                self.d.launch_matmul(dec.MAT_GATE_UP, l)
        durs = []
        with torch.cuda.stream(self.stream):
            for rep in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                g.replay()
                e1.record(self.stream)
                torch.cuda.synchronize()
                if rep > 0:
                    durs.append(e0.elapsed_time(e1) / 1e3 / L)
        del g
        avg = float(np.mean(durs))
        mfma = bool(self.d.info().used_mfma)
        nbytes = gate_up_bytes(self.cfg, self.B, mfma)
        return {"name": ("k_gemm_lds" if mfma else "k_gemv_norm") + " gate+up + SiLU x mul",
                "avg_us": round(avg * 1e6, 2), "bytes_per_launch": nbytes, "gbps": round(nbytes / avg / 1e9, 1),
                "frac": round(nbytes / avg / 1e9 / PEAK_GBPS, 4), "launches": len(durs) * L}

    def close(self) -> None:
        import torch

        self.d.check()  # every device-side wait of the measured steps ended normally
        self.d.close()
        del self.pool
        torch.cuda.empty_cache()


def summary(res: dict) -> dict:
    keys = ("tok_s", "tok_s_best", "ms_per_step", "achieved_gbps", "frac_of_peak", "kernels_per_step",
            "used_mfma", "repeats", "tok_s_all", "step_ms_p50", "step_ms_p90", "step_ms_max")
    out = {}
    for k in keys:
        if k in res:
            v = res[k]
            out[k] = round(v, 4) if isinstance(v, float) else v
    return out


def cpu_baseline(wl, B: int, weights, seed: int):
    """fp64 oracle on the host: time 1-layer and 2-layer truncations of the same step
    (embedding, layers, final norm, LM head; weights already on the host) and
    extrapolate linearly to the full depth."""
    import torch

    from memory_bound_transformer_decode_amd import synth
    from oracle import decoder as OD
    from oracle import inputs as OI

    threads = OD._THREADS
    try:
        from threadpoolctl import threadpool_info
        threads = max([threads] + [i.get("num_threads", 1) for i in threadpool_info()])
    except Exception:  # noqa: BLE001
        pass
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
                       f"norm and LM head, best of {REPS_CPU} runs each ({times[1]:.2f}s, {times[2]:.2f}s), "
                       f"extrapolated linearly to {cfg.n_layers} layers = {step:.2f}s per step"),
            "host_cpus": os.cpu_count()}


def prefill_leg(cfg, weights, n_tokens: int, chunk: int, repeats: int, seed: int) -> dict:
    """Time to first token of one prompt: dec_prefill of n_tokens from an empty cache
    (chunks of `chunk` tokens, only the last chunk runs the LM head), graph replay."""
    import torch

    from memory_bound_transformer_decode_amd import dec, perfmodel, synth

    max_seq = n_tokens + 16
    bt = synth.make_block_tables(cfg, 1, max_seq, synth.blocks_per_seq(max_seq), seed=seed)
    pool = synth.empty_kv_pool(cfg, bt.shape[1], device="cuda", canary=False)
    toks = synth.make_token_ids(cfg, n_tokens, 1, seed=seed)[:, 0].copy()
    d = dec.Decoder(cfg, weights, num_blocks=bt.shape[1], max_batch=chunk, max_seq_len=max_seq, kv_pool=pool)
    d.prefill(toks, 0, bt[0])  # captures the graphs
    torch.cuda.synchronize()
    walls = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        d.prefill(toks, 0, bt[0])
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    info = d.info()
    d.close()
    del pool
    torch.cuda.empty_cache()
    med = float(np.median(walls))
    shape = perfmodel.Shape.of(cfg)
    flops = 2.0 * n_tokens * shape.matmul_params() + sum(
        4.0 * cfg.n_q_heads * cfg.d_head * (p + 1) * cfg.n_layers for p in range(n_tokens))
    return {"tokens": n_tokens, "chunk": chunk, "chunks": info.launches, "ttft_ms": round(1e3 * med, 3),
            "ttft_ms_best": round(1e3 * min(walls), 3), "prompt_tok_s": round(n_tokens / med, 1),
            "tflop_s": round(flops / med / 1e12, 1), "repeats": repeats}


def verify_leg(leg: "Leg", k: int, repeats: int) -> dict:
    """The k-token verify step at the leg's batch: tokens checked per second."""
    import torch

    d = leg.d
    d.set_flags(0)
    toks = np.stack([leg.ids[j] for j in range(k)], axis=1)  # [B][k]
    d.verify(toks, leg.lens0, leg.bt)
    torch.cuda.synchronize()
    n = 20
    walls = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        for _ in range(n):
            d.verify(toks, leg.lens0, leg.bt)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) / n)
    med = float(np.median(walls))
    return {"k": k, "batch": leg.B, "ms_per_verify": round(1e3 * med, 4),
            "tokens_checked_per_s": round(leg.B * k / med, 1), "repeats": repeats}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8B", help="tiny | 1B | 8B | 32B | 70B | 8B-int8")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--repeats", type=int, default=REPEATS)
    ap.add_argument("--legs", default="all", help="comma list of " + ", ".join(ALL_LEGS) + "; all; none")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    legs = set(ALL_LEGS) if args.legs == "all" else set() if args.legs == "none" else set(args.legs.split(","))
    if args.workload != "8B":  # a single workload's step (profiling runs)
        legs -= {"batch32", "workloads", "prefill", "verify"}
    wl = synth.WORKLOADS[args.workload]
    cfg = wl.model
    t_start = time.time()
    log(f"workload {args.workload} batch {args.batch}, {args.steps} steps, {args.warmup} warmup, "
        f"{args.repeats} repeats, legs {sorted(legs)}")
    weights = draw_weights(cfg, args.seed)
    base = dec.FLAG_EAGER if args.eager else 0
    # room for the verify leg's B x 8 rows (steps of B rows replay the bucket of B)
    main_leg = Leg(wl, args.batch, args.steps, args.seed, weights,
                   max_batch=dec.ladder_bucket(8 * args.batch) if "verify" in legs and args.batch <= 8 else 0)
    main_res = main_leg.measure(base, args.warmup, args.repeats, per_step=True)
    kern = main_leg.gate_up_kernel()
    log(f"batch {args.batch}: {main_res['tok_s']:.1f} tok/s (best {main_res['tok_s_best']:.1f}), "
        f"{main_res['ms_per_step']:.3f} ms/step, {main_res['achieved_gbps']:.0f} GB/s "
        f"({100 * main_res['frac_of_peak']:.1f}% of 8 TB/s); gate+up {kern['avg_us']} us")
    plans = None
    if "plans" in legs:
        plans = {"multi_kernel_graph": summary(main_res)}
        for name, flags in (("multi_kernel_eager", dec.FLAG_EAGER),
                            ("separate_attention_o_graph", dec.FLAG_NO_ATTN_O),
                            ("unfused_graph", dec.FLAG_UNFUSED),
                            ("unfused_eager", dec.FLAG_UNFUSED | dec.FLAG_EAGER)):
            plans[name] = summary(main_leg.measure(flags, args.warmup, 2))
        main_leg.d.set_flags(0)
        log("plans: " + ", ".join(f"{k} {v['tok_s']:.1f}" for k, v in plans.items()))
    verify = None
    if "verify" in legs:
        verify = {f"k{k}": verify_leg(main_leg, k, 3) for k in (4, 8)}
        log("verify: " + ", ".join(f"k={v['k']} {v['ms_per_verify']} ms" for v in verify.values()))
    main_leg.close()

    second = None
    if "batch32" in legs:
        leg = Leg(wl, 32, args.steps, args.seed, weights)
        r = leg.measure(0, args.warmup, args.repeats)
        second = summary(r)
        second["kernel"] = leg.gate_up_kernel()
        second["kernel"]["traffic"] = measured_traffic("k_gemm_lds_gate_up_8B_b32", "gemm")
        second["attention_traffic"] = measured_traffic("k_attn_mfma_8B_b32", "attn")
        leg.close()
        log(f"batch 32: {second['tok_s']:.1f} tok/s, {second['ms_per_step']:.3f} ms/step")

    prefill = None
    if "prefill" in legs:
        prefill = prefill_leg(cfg, weights, 1024, 64, 3, args.seed)
        log(f"prefill: {prefill}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.batch, weights, args.seed)
        log(f"cpu oracle: {cpu['value']:.4f} tok/s on {cpu['cores']} threads")
    del weights
    torch.cuda.empty_cache()

    workloads = None
    if "workloads" in legs:
        workloads = {}
        for name, batches, flag_sets in (("1B", (1,), (("graph", 0), ("eager", dec.FLAG_EAGER))),
                                         ("8B-int8", (1,), (("graph", 0),)),
                                         ("32B", (1,), (("graph", 0),)),
                                         ("70B", (1, 64), (("graph", 0),))):
            w2 = synth.WORKLOADS[name]
            wts = draw_weights(w2.model, args.seed)
            for B in batches:
                leg = Leg(w2, B, args.steps, args.seed, wts)
                entry = {}
                for tag, fl in flag_sets:
                    entry[tag] = summary(leg.measure(fl, args.warmup, 3))
                entry["kernel"] = leg.gate_up_kernel()
                if name == "70B" and B == 64:
                    entry["attention_traffic"] = measured_traffic("k_attn_mfma_70B_b64", "attn")
                leg.close()
                workloads[f"{name}_b{B}"] = entry
                log(f"{name} batch {B}: " + ", ".join(f"{t} {entry[t]['tok_s']:.1f} tok/s" for t, _ in flag_sets))
            del wts
            torch.cuda.empty_cache()
    log(f"bench wall {time.time() - t_start:.0f}s")

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
                         f"{args.steps} decode steps; {'eager launches' if args.eager else 'hipGraph replay'} "
                         f"per step; median of {args.repeats} timed loops"),
            "batch": args.batch,
            "kernels_per_step": main_res["kernels_per_step"],
            "attn_splits": main_res["attn_splits"],
        },
        "repeats": summary(main_res),
        "hbm": {"achieved_gbps": round(main_res["achieved_gbps"], 1),
                "frac_of_peak": round(main_res["frac_of_peak"], 4),
                "bytes_per_step": int(main_res["bytes_per_step"])},
        "roofline": {"bound": "hbm", "achieved": kern["gbps"], "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": kern["frac"],
                     "traffic": (measured_traffic(f"k_gemv_norm_gate_up_{args.workload}_b{args.batch}", "gemv")
                                 if args.batch <= 8 else
                                 measured_traffic(f"k_gemm_lds_gate_up_{args.workload}_b{args.batch}", "gemm")),
                     "kernel": kern["name"], "bytes_per_launch": kern["bytes_per_launch"],
                     "avg_us": kern["avg_us"], "launches": kern["launches"]},
        "cpu_baseline": cpu,
        "pages": PAGES,
    }
    if plans:
        line["plans"] = plans
    if second:
        line["batch32"] = second
    if workloads:
        line["workloads"] = workloads
    if prefill:
        line["prefill"] = prefill
    if verify:
        line["verify"] = verify
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
