"""fp64 decode step of a dense pre-norm decoder over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy only.

The step follows the layer sequence the pages describe for a decode forward
pass -- norm, projection, rotary embedding, attention, activation, residual
add, repeated per layer ("Kernels, Fusion & CUDA Graphs", opening section;
"CUDA graphs & kernel fusion", Direct answer) -- in the pre-norm reading:

  h = E[id]                                              (embedding row)
  for each layer l:
     x = RMSNorm(h, g_attn[l])
     [q; k; v] = W_qkv[l] x                               (fused QKV rows)
     q, k = RoPE(q, p), RoPE(k, p)       p = seq_len = tokens already cached
     cache[l][K/V][BT[p // 16]][head][p % 16] = round_cache(k), round_cache(v)
     o_j = sum_i softmax_i(q_j . K_c[i] / sqrt(dh)) V_c[i],  i = 0..p,  c = j // g
     h = h + W_o[l] concat_j o_j
     x = RMSNorm(h, g_mlp[l])
     h = h + W_down[l] (silu(W_gate[l] x) * (W_up[l] x))
  logits = W_lm RMSNorm(h, g_final)

Definitions (each by the paper the architecture study's reference list cites):
  RMSNorm (Zhang & Sennrich): y_i = g_i v_i / sqrt(mean_j v_j^2 + eps).
  RoPE (Su et al., RoFormer): adjacent pairs (2i, 2i+1) rotated by p * theta_i,
      theta_i = theta^(-2i/dh), 0-based position p; v is not rotated.
  SwiGLU (Shazeer): FFN(x) = (silu(x W) * x V) W2, silu(z) = z / (1 + e^-z).
  Attention: exact softmax attention (FlashAttention computes exactly this;
      "GPU Inference Internals", section "Kernels: FlashAttention and the
      Memory Hierarchy").  Grouped-query attention maps query head j to KV
      head j // (Hq / Hkv) ("GPU Inference Internals", The KV-Cache Ledger).
  Paged cache: a per-sequence block table maps logical block p // 16 to a
      physical block of 16 slots (PagedAttention, Kwon et al.).

Readings where the pages are silent (each listed with its reason in the
design notes): no biases; untied embedding and LM head; no embedding scale;
eps and theta as given for the tiny config apply to all; K/V are written to
the cache before attention and the new token attends to itself through the
rounded cached values; weights are the stored (already-quantized) values.

Parity status: every component is pinned by the CPU tests (closed forms,
invariants, the pages' worked examples, brute force against a cache-free full
recompute on tiny shapes).  Whole-model logits at the 1B-and-larger shapes
are "parity unpinned" beyond those component pins: no page prints a
forward-pass value.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence

import numpy as np
from threadpoolctl import threadpool_limits

from . import codecs

# Host threads for the matrix products: row chunks of a product are independent, so
# they are decoded and multiplied in parallel (each output row's sum is the same
# computation whichever thread runs it), each chunk's product by a single-threaded BLAS
# call (a threaded BLAS inside every worker would oversubscribe the cores).
_THREADS = max(1, min(16, os.cpu_count() or 1))
_POOL: Optional[ThreadPoolExecutor] = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=_THREADS)
    return _POOL


# ---------------------------------------------------------------- building blocks

def rmsnorm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * v / sqrt(mean(v^2) + eps) over the last axis (no centring, no bias)."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * v / np.sqrt(ms + eps)


def rope_angles(pos: int, dh: int, theta: float) -> np.ndarray:
    """phi_i = pos * theta^(-2i/dh) for i = 0 .. dh/2 - 1."""
    i = np.arange(dh // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * i / dh)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate adjacent pairs (x_2i, x_2i+1) of the last axis by phi_i."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    phi = rope_angles(pos, dh, theta)
    c, s = np.cos(phi), np.sin(phi)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(K q / sqrt(dh)) V for one query vector q [dh], keys/values [n][dh]."""
    dh = q.shape[-1]
    a = softmax(K @ q / np.sqrt(dh))
    return a @ V


# ---------------------------------------------------------------- stored model

@dataclass
class Matrix:
    """A stored weight matrix [rows][cols]: codes in `fmt` plus optional per-row scale.

    `fetch(r0, r1)` may stream rows from elsewhere (a device tensor) instead of
    holding them; it must return the raw codes of rows [r0, r1).
    """

    rows: int
    cols: int
    fmt: str  # "bf16" | "fp8" | "int8" | "f64"
    codes: Optional[np.ndarray] = None
    scale: Optional[np.ndarray] = None  # float32 [rows] or None (implicit 1)
    fetch: Optional[Callable[[int, int], np.ndarray]] = None
    chunk_rows: int = 512
    _cache: Optional[np.ndarray] = field(default=None, repr=False)

    def _codes(self, r0: int, r1: int) -> np.ndarray:
        return self.codes[r0:r1] if self.codes is not None else self.fetch(r0, r1)

    def decoded(self, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
        """Rows [r0, r1) as float64 values, scale applied (exact: an E4M3 value has at
        most 4 significant bits, an int8 value 7, and the scale 24, well inside float64)."""
        r1 = self.rows if r1 is None else r1
        if self._cache is not None:
            return self._cache[r0:r1]
        w = codecs.decode(self._codes(r0, r1), self.fmt)
        if self.scale is not None:
            w = w * self.scale[r0:r1].astype(np.float64)[:, None]
        return w

    def keep_decoded(self) -> "Matrix":
        """Hold the float64 copy in memory (small models only)."""
        self._cache = self.decoded()
        return self

    def matvec(self, X: np.ndarray, ledger: Optional["Ledger"] = None) -> np.ndarray:
        """Y[b] = s (.) (C X[b]) for X [B][cols] -> Y [B][rows]: the stored values C
        times X, each output row times its scale s (1 without scales) -- the per-row
        scale written as the definition of the scaled format.  Row chunks are fetched,
        decoded and multiplied independently (in parallel)."""
        X = np.asarray(X, dtype=np.float64)
        Y = np.empty((X.shape[0], self.rows), dtype=np.float64)
        # a streamed matrix is fetched once per product, then decoded chunk by chunk
        codes = self.codes if self.codes is not None or self._cache is not None else self.fetch(0, self.rows)

        def chunk(r0: int) -> None:
            r1 = min(self.rows, r0 + self.chunk_rows)
            if self._cache is not None:
                Y[:, r0:r1] = X @ self._cache[r0:r1].T
                return
            Y[:, r0:r1] = X @ codecs.decode(codes[r0:r1], self.fmt).T
            if self.scale is not None:
                Y[:, r0:r1] *= self.scale[r0:r1].astype(np.float64)[None, :]

        with threadpool_limits(limits=1, user_api="blas"):
            list(_pool().map(chunk, range(0, self.rows, self.chunk_rows)))
        if ledger is not None:
            ledger.macs += X.shape[0] * self.rows * self.cols
        return Y

    def row(self, r: int) -> np.ndarray:
        return self.decoded(r, r + 1)[0]


@dataclass
class Model:
    """Dimensions plus stored weights (the names follow the pages' op list)."""

    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    d_ff: int
    vocab: int
    rms_eps: float
    rope_theta: float
    embed: Matrix  # [V][d]
    attn_norm: np.ndarray  # [L][d]
    qkv: List[Matrix]  # [(Hq + 2 Hkv) dh][d]: rows of Q heads, then K heads, then V heads
    o: List[Matrix]  # [d][Hq dh]
    mlp_norm: np.ndarray  # [L][d]
    gate_up: List[Matrix]  # [2 d_ff][d]: gate rows [0, d_ff), up rows [d_ff, 2 d_ff)
    down: List[Matrix]  # [d][d_ff]
    final_norm: np.ndarray  # [d]
    lm_head: Matrix  # [V][d]

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclass
class Ledger:
    """Multiply-accumulates performed by the matrix products and by attention."""

    macs: int = 0
    attn_macs: int = 0


# ---------------------------------------------------------------- paged KV cache

class PagedKVCache:
    """Pool [layer][K=0,V=1][block][kv head][slot][dh] of codes in `fmt`.

    `fmt` is the cache storage format ("bf16", "fp8" or "f64" for an unrounded
    cache used by the brute-force comparisons).  Writes round to that format
    (RNE; E4M3 saturates); reads decode the stored codes.
    """

    def __init__(self, pool_codes: np.ndarray, fmt: str, block_size: int = 16):
        self.pool = pool_codes
        self.fmt = fmt
        self.bs = block_size

    def write(self, layer: int, kv: int, block_table: Sequence[int], pos: int, head: int,
              values: np.ndarray) -> None:
        blk = int(block_table[pos // self.bs])
        self.pool[layer, kv, blk, head, pos % self.bs, :] = codecs.encode(values, self.fmt)

    def read(self, layer: int, kv: int, block_table: Sequence[int], n_tokens: int,
             head: int) -> np.ndarray:
        """Positions 0 .. n_tokens-1 of one sequence and KV head, as float64 [n][dh]."""
        nb = (n_tokens + self.bs - 1) // self.bs
        blks = np.asarray(block_table[:nb], dtype=np.int64)
        codes = self.pool[layer, kv, blks, head]  # [nb][bs][dh]
        codes = codes.reshape(nb * self.bs, -1)[:n_tokens]
        return codecs.decode(codes, self.fmt)


# ---------------------------------------------------------------- the step

def decode_step(m: Model, cache: PagedKVCache, token_ids: Sequence[int],
                seq_lens: Sequence[int], block_tables: np.ndarray,
                ledger: Optional[Ledger] = None, n_layers: Optional[int] = None,
                on_layer: Optional[Callable[[int], None]] = None) -> np.ndarray:
    """One pass of the model over B rows; returns logits [B][V] (float64).

    Row b is token token_ids[b] at 0-based position seq_lens[b] (= tokens of its
    sequence already cached) of the sequence whose block table is block_tables[b].
    In a decode step every row is a different sequence.  Rows may also be several
    tokens of one sequence at consecutive positions (the verify step, a prefill
    chunk): in every layer the K and V of all rows are written first, then each row
    attends to positions 0 .. p of its sequence, so a token sees itself and the
    tokens before it and none after -- the causal mask, from the positions alone.
    Writes every row's K and V of every layer into `cache`.
    n_layers: run only the first n layers (default: all).
    on_layer: called with l after each layer (progress reports of long runs).
    """
    B = len(token_ids)
    L = m.n_layers if n_layers is None else n_layers
    Hq, Hkv, dh, g = m.n_q_heads, m.n_kv_heads, m.d_head, m.group
    eps, theta = m.rms_eps, m.rope_theta

    h = np.stack([m.embed.row(int(t)) for t in token_ids])  # [B][d]
    for l in range(L):
        x = rmsnorm(h, m.attn_norm[l], eps)
        qkv = m.qkv[l].matvec(x, ledger)
        qs = []
        for b in range(B):
            p = int(seq_lens[b])
            bt = block_tables[b]
            qs.append(rope(qkv[b, : Hq * dh].reshape(Hq, dh), p, theta))
            k = rope(qkv[b, Hq * dh:(Hq + Hkv) * dh].reshape(Hkv, dh), p, theta)
            v = qkv[b, (Hq + Hkv) * dh:].reshape(Hkv, dh)
            for c in range(Hkv):
                cache.write(l, 0, bt, p, c, k[c])
                cache.write(l, 1, bt, p, c, v[c])
        o = np.zeros((B, Hq, dh), dtype=np.float64)
        for b in range(B):
            p = int(seq_lens[b])
            bt = block_tables[b]
            for c in range(Hkv):
                Kc = cache.read(l, 0, bt, p + 1, c)
                Vc = cache.read(l, 1, bt, p + 1, c)
                for j in range(c * g, (c + 1) * g):
                    o[b, j] = attend(qs[b][j], Kc, Vc)
            if ledger is not None:
                ledger.attn_macs += 2 * Hq * dh * (p + 1)
        h = h + m.o[l].matvec(o.reshape(B, Hq * dh), ledger)
        x = rmsnorm(h, m.mlp_norm[l], eps)
        gu = m.gate_up[l].matvec(x, ledger)
        a = silu(gu[:, : m.d_ff]) * gu[:, m.d_ff:]
        h = h + m.down[l].matvec(a, ledger)
        if on_layer is not None:
            on_layer(l)
    xf = rmsnorm(h, m.final_norm, eps)
    return m.lm_head.matvec(xf, ledger)


def verify_step(m: Model, cache: PagedKVCache, tokens: np.ndarray, seq_lens: Sequence[int],
                block_tables: np.ndarray) -> np.ndarray:
    """The verification step of speculative decoding ("GPU Inference Internals",
    Roofline: Why Decode Is Memory-Bound, speculative-decoding paragraph): k tokens
    per sequence, tokens[s][j] at position seq_lens[s] + j, in one pass.  Returns
    logits [n][k][V]: row (s, j) is the distribution after token j of sequence s."""
    tokens = np.asarray(tokens)
    n, k = tokens.shape
    rows_ids = [int(tokens[s, j]) for s in range(n) for j in range(k)]
    rows_pos = [int(seq_lens[s]) + j for s in range(n) for j in range(k)]
    rows_bt = np.stack([block_tables[s] for s in range(n) for _ in range(k)])
    z = decode_step(m, cache, rows_ids, rows_pos, rows_bt)
    return z.reshape(n, k, -1)


def prefill(m: Model, cache: PagedKVCache, tokens: Sequence[int], start_pos: int,
            block_table: Sequence[int]) -> np.ndarray:
    """Prefill of one sequence's prompt ("GPU Inference Internals", Roofline: Why
    Decode Is Memory-Bound, the Prefill paragraph): every prompt token at positions
    start_pos, start_pos + 1, ... in one causal pass, writing its K and V into the
    cache.  Returns the logits after the last prompt token [V]."""
    n = len(tokens)
    bts = np.stack([np.asarray(block_table)] * n)
    z = decode_step(m, cache, [int(t) for t in tokens], [start_pos + i for i in range(n)], bts)
    return z[-1]


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, bytes_per_elem: int) -> int:
    """K and V of one token over all layers and KV heads ("GPU Inference Internals",
    The KV-Cache Ledger: 2 x layers x kv_heads x head_dim x bytes)."""
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_elem
