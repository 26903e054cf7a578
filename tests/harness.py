"""Shared machinery of the GPU parity tests: draw a case, run the HIP path and the
oracle on the same seeded inputs, compare logits and KV-cache bits.

Tolerances (relative to each row's oracle logit range R = max - min):
  bf16 or int8 weights with a bf16 cache: max |z_gpu - z_oracle| <= 2e-2 R; fp8
  weights or fp8 cache: <= 6e-2 R.  (int8 storage is part of the model both sides
  compute, so what differs is the same bf16 activation rounding as for bf16
  weights; the fp8 bar is kept for an fp8 cache.)
Greedy agreement: wherever the oracle's top-1 minus top-2 exceeds tol * R, the
HIP path's argmax equals the oracle's.
KV cache: placement is exact -- every slot the oracle never wrote still holds
the canary and every slot it wrote holds a value.  Values: each element the step
wrote must be the oracle's code or an adjacent one, or lie within tol * R of the
oracle's value, R = max - min of the oracle's K (or V) values that layer wrote in
the step -- the logits' own bar (max |dz| relative to the range of the output it
belongs to), applied to each layer's K and V output.  The K/V of layer l carry
the drift that the bf16 rounding of earlier activations left in the residual
stream, the same drift the logits carry at the end of the step, so the same
relative bar holds them at every depth.  The worst error per layer is logged,
and also relative to the largest |v| of each head vector.
"""

from __future__ import annotations

import dataclasses
import os
import sys
import time
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from memory_bound_transformer_decode_amd import synth
from oracle import decoder as OD
from oracle import inputs as OI

TOL = {"bf16": 2e-2, "int8": 2e-2, "fp8": 6e-2}


def tol_of(cfg: synth.ModelConfig) -> float:
    """The bf16 bar for bf16 / int8 weights and a bf16 cache, the fp8 bar as soon as
    weights or cache are fp8."""
    return max(TOL[cfg.weight_dtype], TOL[cfg.kv_dtype])


def log(msg: str) -> None:
    print(f"[harness {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from memory_bound_transformer_decode_amd import dec
    dec.load_library()  # raises if the HIP library is missing: no fallback
    return dec


@dataclass
class Case:
    cfg: synth.ModelConfig
    weights: synth.ModelWeights
    pool: torch.Tensor  # device pool with the context written (canary elsewhere)
    block_tables: np.ndarray
    ctx_lens: np.ndarray
    max_seq_len: int
    num_blocks: int
    seed: int = 0


def make_case(cfg: synth.ModelConfig, ctx_lens: Sequence[int], max_seq_len: int, seed: int = 0,
              gains: str = "ones", spare_blocks: int = 3) -> Case:
    B = len(ctx_lens)
    bps = synth.blocks_per_seq(max_seq_len)
    nb = B * bps + spare_blocks
    w = synth.make_weights(cfg, seed=seed, device="cuda", gains=gains)
    bt = synth.make_block_tables(cfg, B, max_seq_len, nb, seed=seed)
    pool = synth.empty_kv_pool(cfg, nb, device="cuda", canary=True)
    lens = np.asarray(ctx_lens, dtype=np.int32)
    synth.fill_context_kv(cfg, pool, bt, lens, seed=seed)
    torch.cuda.synchronize()
    return Case(cfg, w, pool, bt, lens, max_seq_len, nb, seed)


def ordered(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Map sign-magnitude codes to integers whose order is the value order."""
    c = codes.astype(np.int64)
    if fmt == "bf16":
        return np.where(c & 0x8000, -(c & 0x7FFF), c)
    return np.where(c & 0x80, -(c & 0x7F), c)


@dataclass
class Report:
    max_rel_err: float = 0.0
    worst_step: int = -1
    argmax_checked: int = 0
    argmax_mismatch: int = 0
    kv_neighbour: int = 0  # written elements that differ from the oracle's code
    kv_worst: float = 0.0  # largest |dv| / R (R: range of the layer's K or V written in the step)
    kv_worst_layer: int = -1
    kv_worst_absmax: float = 0.0  # largest |dv| / max|v|
    kv_worst_far: float = 0.0  # largest |dv| / R over elements two or more codes away
    kv_by_layer: dict = field(default_factory=dict)  # layer -> largest |dv| / R
    rows: int = 0
    errs: List[float] = field(default_factory=list)


def compare_logits(z: np.ndarray, zo: np.ndarray, tol: float, rep: Report, step: int) -> None:
    for r in range(zo.shape[0]):
        R = float(zo[r].max() - zo[r].min())
        err = float(np.max(np.abs(z[r] - zo[r]))) / R
        rep.errs.append(err)
        rep.rows += 1
        if err > rep.max_rel_err:
            rep.max_rel_err, rep.worst_step = err, step
        top = np.argsort(zo[r])[-2:]
        if zo[r][top[1]] - zo[r][top[0]] > tol * R:
            rep.argmax_checked += 1
            if int(np.argmax(z[r])) != int(top[1]):
                rep.argmax_mismatch += 1


def compare_kv(pool_gpu: torch.Tensor, ocache: OD.PagedKVCache, fmt: str, rep: Report,
               tol: float, before: Optional[np.ndarray] = None) -> None:
    """before: the pool codes before the compared steps (the slots they wrote are the
    ones that differ from it in the oracle's cache); default: the differing vectors."""
    from oracle import codecs
    g = synth.kv_codes_numpy(pool_gpu)
    o = ocache.pool
    assert g.shape == o.shape
    diff = g != o
    if not diff.any():
        return
    canary = synth.KV_CANARY_BF16 if fmt == "bf16" else synth.KV_CANARY_FP8
    # a canary on one side only is a misplaced or missing write
    bad = diff & ((g == canary) | (o == canary))
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"KV write misplaced or missing at {idx} (layer, K/V, block, head, slot, e)")
    vec = np.any(diff, axis=-1)  # head vectors with any difference
    gv = codecs.decode(g[vec], fmt)
    ov = codecs.decode(o[vec], fmt)
    gap = np.abs(ordered(g[vec], fmt) - ordered(o[vec], fmt))
    idx = np.argwhere(vec)  # (layer, K/V, block, head, slot) of each such vector
    # R per (layer, K/V): the range of the oracle's values written in this step, over
    # the slots this step changed in the oracle's cache
    written = np.any(o != before, axis=-1) if before is not None else vec
    R = {}
    for l, kv in {(int(a), int(b)) for a, b in idx[:, :2]}:
        vals = codecs.decode(o[l, kv][written[l, kv]], fmt)
        R[(l, kv)] = float(vals.max() - vals.min()) if vals.size else 1.0
    rng = np.array([R[(int(a), int(b))] for a, b in idx[:, :2]])[:, None]
    amax = np.max(np.abs(ov), axis=-1, keepdims=True)
    err = np.abs(gv - ov)
    rel = err / rng
    layer = idx[:, 0]
    worst = rel.max(axis=-1)
    for l in np.unique(layer):
        wl = float(worst[layer == l].max())
        rep.kv_by_layer[int(l)] = max(wl, rep.kv_by_layer.get(int(l), 0.0))
        if wl > rep.kv_worst:
            rep.kv_worst, rep.kv_worst_layer = wl, int(l)
    rep.kv_worst_absmax = max(rep.kv_worst_absmax, float(np.max(err / amax)))
    far = gap > 1
    if far.any():
        rep.kv_worst_far = max(rep.kv_worst_far, float(np.max(rel[far])))
    ok = ~far | (rel <= tol)
    if not ok.all():
        where = idx[np.argwhere(~ok)[0][0]].tolist()
        bad_rel = float(np.max(np.where(ok, 0.0, rel)))
        raise AssertionError(f"KV values differ beyond tolerance ({bad_rel:.3e} of the layer's K/V range, "
                             f"more than one code away) e.g. at {where}")
    rep.kv_neighbour += int(diff.sum())


def progress(cfg: synth.ModelConfig, step: int):
    """A per-layer progress line every 8 layers for deep models (long oracle runs)."""
    if cfg.n_layers < 16:
        return None
    return lambda l: log(f"{cfg.name} step {step}: oracle layer {l + 1}/{cfg.n_layers}") if (l + 1) % 8 == 0 else None


def run_parity(case: Case, batch_ids: np.ndarray, *, flags: int = 0, max_batch: Optional[int] = None,
               keep_decoded: bool = True, stream_weights: bool = False, kv_every_step: bool = True,
               n_layers_oracle: Optional[int] = None) -> Report:
    """Teacher-forced decode of batch_ids [steps][B] on both sides from the same context."""
    from memory_bound_transformer_decode_amd import dec
    cfg = case.cfg
    steps, B = batch_ids.shape
    mb = max_batch or dec.ladder_bucket(B)
    tol = tol_of(cfg)
    d = dec.Decoder(cfg, case.weights, num_blocks=case.num_blocks, max_batch=mb,
                    max_seq_len=case.max_seq_len, flags=flags, kv_pool=case.pool.clone())
    om = OI.model(case.weights, keep=keep_decoded and not stream_weights, stream=stream_weights)
    oc = OI.cache(cfg, synth.kv_codes_numpy(case.pool))
    lens = case.ctx_lens.copy()
    rep = Report()
    before = oc.pool.copy()
    for t in range(steps):
        z = d.step(batch_ids[t], lens, case.block_tables).double().cpu().numpy()
        t0 = time.time()
        zo = OD.decode_step(om, oc, batch_ids[t], lens, case.block_tables, on_layer=progress(cfg, t))
        if cfg.n_layers >= 8:
            log(f"{cfg.name} step {t}: oracle {time.time() - t0:.1f}s")
        assert np.all(np.isfinite(z)), f"non-finite logits at step {t}"
        compare_logits(z, zo, tol, rep, t)
        if cfg.n_layers > 0 and (kv_every_step or t == steps - 1):
            compare_kv(d.kv_pool, oc, cfg.kv_dtype, rep, tol, before)
            before = oc.pool.copy()
        lens = lens + 1
    d.check()  # no device-side wait gave up
    info = d.info()
    d.close()
    log(f"{cfg.name} B={B} steps={steps} flags={flags} "
        f"mfma={info.used_mfma}: max rel err {rep.max_rel_err:.3e} "
        f"(tol {tol}), argmax {rep.argmax_checked - rep.argmax_mismatch}/{rep.argmax_checked}, "
        f"kv elements off the oracle's code {rep.kv_neighbour}, worst kv |dv|/R "
        f"{rep.kv_worst:.3e} (layer {rep.kv_worst_layer}; {rep.kv_worst_far:.3e} two or more codes away; "
        f"{rep.kv_worst_absmax:.3e} of max|v|)")
    if len(rep.kv_by_layer) > 2:
        log(f"{cfg.name} worst kv |dv|/R by layer: " +
            " ".join(f"{l}:{v:.2e}" for l, v in sorted(rep.kv_by_layer.items())))
    return rep


def assert_ok(rep: Report, cfg: synth.ModelConfig) -> None:
    tol = tol_of(cfg)
    assert rep.max_rel_err <= tol, f"max rel err {rep.max_rel_err:.3e} > {tol}"
    assert rep.argmax_mismatch == 0, f"{rep.argmax_mismatch} argmax mismatches"
