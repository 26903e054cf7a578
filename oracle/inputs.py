"""Adapters from the seeded inputs to the oracle's stored-model objects.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Reads only the raw
storage bits the input generator drew (bf16 bit patterns, E4M3 codes, fp32
scales and gains) and hands them to the oracle, which decodes them itself.
"""

from __future__ import annotations

import numpy as np

from memory_bound_transformer_decode_amd import synth

from .decoder import Matrix, Model, PagedKVCache


def matrix(sm: "synth.StoredMatrix", keep: bool = False, stream: bool = False) -> Matrix:
    rows, cols = sm.w.shape
    fmt = sm.fmt
    scale = sm.scale_numpy()
    if stream:
        m = Matrix(rows, cols, fmt, codes=None, scale=scale,
                   fetch=lambda r0, r1, sm=sm: sm.codes_numpy(r0, r1))
    else:
        m = Matrix(rows, cols, fmt, codes=sm.codes_numpy(), scale=scale)
    if keep:
        m.keep_decoded()
    return m


def model(w: "synth.ModelWeights", keep: bool = False, stream: bool = False,
          n_layers: int | None = None) -> Model:
    """Oracle model from drawn weights.  keep: hold float64 copies (small models);
    stream: fetch rows from the (possibly device-resident) tensors on use."""
    cfg = w.cfg
    L = cfg.n_layers if n_layers is None else n_layers
    mk = lambda sm: matrix(sm, keep=keep, stream=stream)  # noqa: E731
    return Model(
        n_layers=L, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
        n_kv_heads=cfg.n_kv_heads, d_head=cfg.d_head, d_ff=cfg.d_ff, vocab=cfg.vocab,
        rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
        embed=matrix(w.embed, keep=False, stream=stream),
        attn_norm=w.attn_norm[:L].cpu().numpy().astype(np.float64),
        qkv=[mk(m) for m in w.qkv[:L]], o=[mk(m) for m in w.o[:L]],
        mlp_norm=w.mlp_norm[:L].cpu().numpy().astype(np.float64),
        gate_up=[mk(m) for m in w.gate_up[:L]], down=[mk(m) for m in w.down[:L]],
        final_norm=w.final_norm.cpu().numpy().astype(np.float64),
        lm_head=mk(w.lm_head),
    )


def cache(cfg: "synth.ModelConfig", pool_codes: np.ndarray) -> PagedKVCache:
    """The oracle's own cache, initialised from a copy of the drawn pool bits."""
    return PagedKVCache(np.array(pool_codes, copy=True), cfg.kv_dtype, cfg.block_size)
