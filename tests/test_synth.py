"""Seeded input generation: determinism and structure (CPU only)."""

import dataclasses

import numpy as np
import torch

from memory_bound_transformer_decode_amd import synth
from oracle import codecs, inputs


def test_weights_deterministic_per_seed():
    a = synth.make_weights(synth.TINY, seed=0)
    b = synth.make_weights(synth.TINY, seed=0)
    c = synth.make_weights(synth.TINY, seed=1)
    assert torch.equal(a.qkv[0].w.view(torch.int16), b.qkv[0].w.view(torch.int16))
    assert torch.equal(a.lm_head.w.view(torch.int16), b.lm_head.w.view(torch.int16))
    assert not torch.equal(a.qkv[0].w.view(torch.int16), c.qkv[0].w.view(torch.int16))
    # distinct tensors draw from distinct streams
    assert not torch.equal(a.embed.w.view(torch.int16), a.lm_head.w.view(torch.int16))


def test_weight_statistics_and_formats():
    w = synth.make_weights(synth.TINY, seed=0)
    x = w.gate_up[0].w.float()
    assert abs(x.std().item() - 0.02) < 1e-3 and abs(x.mean().item()) < 1e-3
    assert torch.all(w.attn_norm == 1.0)
    f8 = synth.make_weights(dataclasses.replace(synth.TINY, weight_dtype="fp8"), seed=0)
    assert f8.qkv[0].w.dtype == torch.float8_e4m3fn and f8.qkv[0].scale is not None
    # per-row absmax maps to +-448 exactly
    amax = f8.qkv[0].w.float().abs().amax(dim=1)
    assert torch.all(amax == 448.0)
    rg = synth.make_weights(synth.TINY, seed=0, gains="random")
    assert abs((rg.attn_norm - 1).std().item() - 0.1) < 0.02


def test_block_tables_disjoint_permutation():
    bt = synth.make_block_tables(synth.M8B, 32, 1064, 2200, seed=0)
    assert bt.shape == (32, 67) and bt.dtype == np.int32
    assert len(np.unique(bt)) == bt.size and bt.min() >= 0 and bt.max() < 2200
    assert not np.array_equal(bt.ravel(), np.arange(bt.size))


def test_context_fill_touches_only_context_slots():
    cfg = synth.TINY
    pool = synth.empty_kv_pool(cfg, 8)
    bt = synth.make_block_tables(cfg, 2, 40, 8, seed=0)
    lens = [19, 5]
    synth.fill_context_kv(cfg, pool, bt, lens, seed=0)
    codes = synth.kv_codes_numpy(pool)
    written = codes != synth.KV_CANARY_BF16
    expect = np.zeros_like(written)
    for b, n in enumerate(lens):
        for p in range(n):
            expect[:, :, bt[b][p // 16], :, p % 16, :] = True
    assert np.array_equal(written, expect)
    vals = codecs.bf16_decode(codes[written])
    assert abs(vals.std() - 1.0) < 0.05


def test_token_ids_in_range():
    ids = synth.make_token_ids(synth.M1B, 40, 4, seed=0)
    assert ids.shape == (40, 4) and ids.min() >= 0 and ids.max() < 32000


def test_oracle_runs_tiny_workload():
    """The oracle consumes the drawn tiny model and cache bits end to end."""
    cfg = synth.TINY
    w = synth.make_weights(cfg, seed=0)
    pool = synth.empty_kv_pool(cfg, 4)
    bt = synth.make_block_tables(cfg, 1, 48, 4, seed=0)
    synth.fill_context_kv(cfg, pool, bt, [32], seed=0)
    m = inputs.model(w, keep=True)
    cache = inputs.cache(cfg, synth.kv_codes_numpy(pool))
    z = __import__("oracle").decoder.decode_step(m, cache, [17], [32], bt)
    assert z.shape == (1, cfg.vocab) and np.all(np.isfinite(z))
