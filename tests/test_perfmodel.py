"""Pins for the measurement ledgers against the pages' worked examples (CPU only).

The expected values live in tests/golden/pages_worked_examples.json, each with
the page and section that prints it.
"""

import json
import os

import pytest

from memory_bound_transformer_decode_amd import perfmodel as P
from memory_bound_transformer_decode_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_worked_examples.json")))


def _page_model(weight_gib, n_kernels=430, tau_us=5.0, bw=1e12):
    return P.weight_streaming_launch_tax(weight_gib * 2 ** 30, bw, n_kernels, tau_us * 1e-6)


def test_launch_tax_printed_outputs():
    """The page's model at its printed inputs gives its printed figures (ms, 1 decimal;
    the gain to 2 decimals)."""
    g = GOLD["launch_tax_step_ms"]
    for c in g["cases"]:
        t = _page_model(c["weight_gib"], **g["params"])
        assert f"{1e3 * t.compute_s:.1f}" == f"{c['compute_ms']:.1f}"
        assert f"{1e3 * t.eager_s:.1f}" == f"{c['eager_ms']:.1f}"
        assert f"{1e3 * t.graph_s:.1f}" == f"{c['graph_ms']:.1f}"
        assert f"{t.graph_gain:.2f}" == f"{c['speedup']:.2f}"


def test_launch_tax_is_additive():
    t = P.launch_tax(2e-3, 100, 4e-6)
    assert t.eager_s == pytest.approx(2.4e-3) and t.graph_s == pytest.approx(2.004e-3)
    assert t.tax_share == pytest.approx(0.2)
    assert P.launch_tax(1.0, 0, 1e-6).eager_s == 1.0


def test_launch_tax_direct_answer_and_share():
    g = GOLD["launch_tax_direct_answer"]
    tax_ms = g["n_kernels"] * g["tau_us"] / 1e3
    assert tax_ms == pytest.approx(2.15)
    assert round(tax_ms) == g["approx_ms"]
    for c in GOLD["launch_share_quantized"]["cases"]:
        t = _page_model(c["weight_gib"])
        assert round(100 * t.tax_share) == c["share_pct"]  # share of the compute time


def test_machine_balance_h100():
    g = GOLD["machine_balance_h100"]
    for c in g["cases"]:
        assert round(P.machine_balance(c["peak"], g["bandwidth"]), -1) == pytest.approx(
            c["balance"], abs=5)


def test_batch1_70b_fp8_roofline():
    g = GOLD["decode_batch1_70b_fp8"]
    flops = 2 * g["params"]
    assert flops == g["flops"]
    inten = flops / (g["params"] * g["bytes_per_weight"])
    assert inten == g["intensity"]
    bal = P.machine_balance(1979e12, 3.35e12)
    assert round(bal / inten, -1) == pytest.approx(g["below_balance"], abs=5)
    assert round(P.single_stream_ceiling(g["bandwidth"], g["params"])) == g["ceiling_tok_s"]


def test_balance_crossover_batch():
    b16 = P.balance_crossover_batch(989e12, 3.35e12, 2)
    b8 = P.balance_crossover_batch(1979e12, 3.35e12, 1)
    assert round(b16) == pytest.approx(GOLD["balance_crossover_batch"]["batch"], abs=1)
    assert round(b8) == pytest.approx(GOLD["balance_crossover_batch"]["batch"], abs=1)
    assert P.weight_only_intensity(1, 2) == 1.0


def test_kv_ledger():
    g = GOLD["kv_ledger_70b_bf16"]
    k = P.kv_bytes_per_token(g["n_layers"], g["n_kv_heads"], g["d_head"], g["bytes"])
    assert k == g["bytes_per_token"]
    assert k * g["context"] == g["context_gib"] * 2 ** 30
    h = GOLD["kv_vs_weights_batch32_16k"]
    assert round(h["batch"] * h["tokens"] * h["kb_per_token"] * 1000 / 1e9) == h["approx_gb"]


def test_naive_attention_traffic():
    g = GOLD["naive_attention_scores"]
    mb = g["n"] ** 2 * g["bytes"] / 1e6
    assert round(mb) == g["approx_mb"]
    assert round(4 * mb / 1e3, 1) == g["approx_traffic_gb"]


def test_overlap_model():
    # launch-bound: 430 launches x 8 us beats 2 GB / 3.35 TB/s of GPU work
    t = P.overlapped_eager_step_s(2e9, 4e9, 3.35e12, 989e12, 430, 8e-6)
    assert t == pytest.approx(430 * 8e-6)
    t = P.overlapped_eager_step_s(70e9, 140e9, 3.35e12, 989e12, 430, 8e-6)
    assert t == pytest.approx(70e9 / 3.35e12)


def test_roofline_step_time():
    assert P.roofline_step_time(140e9, 70e9, 1979e12, 3.35e12) == pytest.approx(70e9 / 3.35e12)
    assert P.roofline_step_time(1e15, 1e9, 1e15, 1e12, eta_c=0.5) == pytest.approx(2.0)


@pytest.mark.parametrize("name,expect_gb", [("1B", 2.078), ("8B", 15.010), ("32B", 32.006),
                                            ("70B", 69.534)])
def test_config_weight_bytes(name, expect_gb):
    """Per-step weight bytes of each workload's model at batch 1."""
    s = P.Shape.of(synth.MODELS[name])
    assert s.weight_bytes_per_step(1) / 1e9 == pytest.approx(expect_gb, abs=1.5e-3)


def test_8b_step_flops_about_2p():
    s = P.Shape.of(synth.M8B)
    f = s.step_flops([640])
    assert f / 1e9 == pytest.approx(15.36, abs=0.05)
    assert 2 * s.matmul_params() / 1e9 == pytest.approx(15.01, abs=0.01)
