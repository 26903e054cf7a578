"""Full-depth parity of the benchmarked workloads (needs an MI355X).

The step the benchmark times, at every layer of the 8B (32 layers), 32B (64) and 70B
(80) models, against the fp64 oracle streaming the weights from the device tensors:
the cross-layer hand-offs (the residual product of layer l folding the RMSNorm that the
QKV product of layer l + 1 applies), every layer's region of the KV pool, and the bf16
activation drift over the whole depth, against the same bars as every other case.
Plus the 32B and 70B widths at two layers and batch 64 (the folded norm across a layer
boundary at E4M3 widths with four column tiles).  Each case logs the oracle's progress.
"""

import numpy as np
import pytest

from memory_bound_transformer_decode_amd import synth

from harness import assert_ok, log, make_case, require_gpu, run_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dec():
    return require_gpu()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers,B,steps", [("8B", None, 1, 2), ("8B", None, 32, 1),
                                                 ("32B", 2, 64, 1), ("70B", 2, 64, 1),
                                                 ("32B", None, 1, 1), ("70B", None, 1, 1)])
def test_workload_depth(dec, name, layers, B, steps):
    wl = synth.WORKLOADS[name]
    cfg = wl.model if layers is None else wl.model.with_layers(layers)
    lens = synth.make_context_lengths(wl, B, seed=0)
    log(f"{cfg.name}: {cfg.n_layers} layers, B={B}, {steps} step(s), contexts {lens.min()}..{lens.max()}")
    case = make_case(cfg, lens, wl.max_seq_len, seed=0)
    ids = synth.make_token_ids(cfg, steps, B, seed=0)
    rep = run_parity(case, ids, stream_weights=True, kv_every_step=False)
    log(f"{cfg.name} B={B}: max rel err {rep.max_rel_err:.3e}, worst KV {rep.kv_worst:.3e} "
        f"(layer {rep.kv_worst_layer})")
    del case
    assert_ok(rep, cfg)
