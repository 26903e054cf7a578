"""Seeded synthetic inputs for the decode step.

This module defines the workloads (model shapes, batch sizes, context-length
mixes) and draws every input both sides of a parity check consume: stored
weights, norm gains, the prefilled paged KV cache, block tables and token ids.
It holds none of the decode step's arithmetic; it only draws random numbers
and stores them in the formats the model is defined in.

Storage formats (the model *is* what is stored; both the HIP path and the
CPU oracle decode these bits themselves):
  * bf16 weights: N(0, 0.02) drawn in fp32, rounded to bf16 (RNE).
  * fp8 weights: N(0, 0.02) drawn in fp32, then per output row
    s = max|w| / 448 (s = 1 for an all-zero row), code = RNE_e4m3(w / s)
    with |w / s| clamped to 448 first; scales kept as fp32.  The FP8 format
    is E4M3 as defined by Micikevicius et al., "FP8 Formats for Deep
    Learning" (cited by the kernel-fusion architecture study's reference
    list): bias 7, max 448, no infinities.
  * int8 weights (weight-only INT8): N(0, 0.02) drawn in fp32, then per output
    row s = max|w| / 127 (s = 1 for an all-zero row), code = round-half-even
    (w / s) clamped to [-127, 127]; scales kept as fp32.
  * context K/V: N(0, 1) rounded to the cache dtype.
  * block tables: a seeded random permutation of the pool's block ids.

Every tensor has its own stream: numpy SeedSequence(seed, spawn_key=(config
id, layer, tensor id)) seeds a torch.Generator on the device the tensor is
drawn on.  The same (seed, config, device) gives the same bytes.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

BLOCK = 16  # KV positions per paged block

# tensor ids for the per-tensor seed streams
_T_EMBED, _T_ATTN_NORM, _T_QKV, _T_O, _T_MLP_NORM, _T_GU, _T_DOWN = 0, 1, 2, 3, 4, 5, 6
_T_FINAL_NORM, _T_LM, _T_CTX, _T_BT, _T_IDS, _T_LENS = 7, 8, 9, 10, 11, 12


@dataclass(frozen=True)
class ModelConfig:
    """Shape and storage formats of a dense pre-norm decoder."""

    name: str
    config_id: int
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    d_ff: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4
    weight_dtype: str = "bf16"  # "bf16" | "fp8" | "int8"
    kv_dtype: str = "bf16"  # "bf16" | "fp8"
    block_size: int = BLOCK

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.d_head

    def with_layers(self, n_layers: int) -> "ModelConfig":
        """Same widths and vocabulary, different depth (truncated-depth parity runs)."""
        return dataclasses.replace(self, n_layers=n_layers,
                                   name=f"{self.name}-L{n_layers}")


@dataclass(frozen=True)
class Workload:
    """A decode workload: model, batch sizes, context-length mix, steps."""

    model: ModelConfig
    batches: Sequence[int]
    ctx_lo: int  # context length drawn uniformly per sequence in [ctx_lo, ctx_hi]
    ctx_hi: int
    decode_steps: int
    description: str

    @property
    def max_seq_len(self) -> int:
        return self.ctx_hi + self.decode_steps


# The five workload classes: tiny (1 layer), ~1B, 8B, 32B and 70B dense decoders.
TINY = ModelConfig("tiny", 0, n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=4,
                   d_head=64, d_ff=1024, vocab=1024)
M1B = ModelConfig("1B", 1, n_layers=16, d_model=2048, n_q_heads=32, n_kv_heads=8,
                  d_head=64, d_ff=8192, vocab=32000)
M8B = ModelConfig("8B", 2, n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8,
                  d_head=128, d_ff=14336, vocab=128256)
M32B = ModelConfig("32B", 3, n_layers=64, d_model=5120, n_q_heads=40, n_kv_heads=8,
                   d_head=128, d_ff=27648, vocab=152064,
                   weight_dtype="fp8", kv_dtype="fp8")
M70B = ModelConfig("70B", 4, n_layers=80, d_model=8192, n_q_heads=64, n_kv_heads=8,
                   d_head=128, d_ff=28672, vocab=128256,
                   weight_dtype="fp8", kv_dtype="fp8")

# The 8B shape with weight-only INT8 (per-row scales) and a bf16 cache: the second
# one-byte weight format through the same dequantizing kernels.
M8B_I8 = dataclasses.replace(M8B, name="8B-int8", config_id=5, weight_dtype="int8")

MODELS: Dict[str, ModelConfig] = {m.name: m for m in (TINY, M1B, M8B, M32B, M70B, M8B_I8)}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(TINY, (1,), 32, 32, 8,
                     "tiny 1-layer decoder, batch 1, 32 prefilled positions, 8 decode steps"),
    "1B": Workload(M1B, (1,), 128, 128, 40,
                   "1B-class decoder, batch 1, 128-token context, 40 decode steps"),
    "8B": Workload(M8B, (1, 8, 32), 256, 1024, 40,
                   "8B-class decoder, bf16, context U[256,1024] per sequence, 40 decode steps"),
    "32B": Workload(M32B, (1, 2, 4, 8, 13, 16, 24, 32, 48, 64), 64, 256, 40,
                    "32B-class decoder, fp8 weights and KV, prompts U[64,256], 40 decode steps"),
    "70B": Workload(M70B, (1, 64), 2048, 2048, 40,
                    "70B-class decoder, fp8 weights and KV, context 2048, 40 decode steps"),
    "8B-int8": Workload(M8B_I8, (1, 8, 32), 256, 1024, 40,
                        "8B-class decoder, int8 weights, bf16 KV, context U[256,1024], 40 decode steps"),
}


def blocks_per_seq(max_seq_len: int, block: int = BLOCK) -> int:
    return (max_seq_len + block - 1) // block


# --------------------------------------------------------------------------
# seeded streams
# --------------------------------------------------------------------------

def _stream(seed: int, config_id: int, layer: int, tensor_id: int,
            device: torch.device | str) -> torch.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(config_id, layer, tensor_id))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def _np_rng(seed: int, config_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(config_id, layer, tensor_id)))


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def quantize_rows_fp8(w32: torch.Tensor):
    """Per-output-row absmax scaling to E4M3: returns (codes as float8_e4m3fn, fp32 scales)."""
    amax = w32.abs().amax(dim=1)
    # tensor / tensor keeps this a true (correctly rounded) binary32 division on
    # every device; dividing by a Python scalar may become a reciprocal multiply
    s = torch.where(amax > 0, amax / torch.full_like(amax, 448.0), torch.ones_like(amax))
    q = (w32 / s[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, s.to(torch.float32)


def quantize_rows_int8(w32: torch.Tensor):
    """Per-output-row absmax scaling to symmetric int8: returns (int8 codes, fp32 scales)."""
    amax = w32.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / torch.full_like(amax, 127.0), torch.ones_like(amax))
    q = torch.round(w32 / s[:, None]).clamp_(-127.0, 127.0).to(torch.int8)
    return q, s.to(torch.float32)


_FMT_OF_DTYPE = {torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8", torch.int8: "int8"}
_DTYPE_OF_FMT = {v: k for k, v in _FMT_OF_DTYPE.items()}


@dataclass
class StoredMatrix:
    """A weight matrix [rows][cols] in its storage format (row = output channel)."""

    w: torch.Tensor  # torch.bfloat16, torch.float8_e4m3fn or torch.int8, contiguous
    scale: Optional[torch.Tensor]  # fp32 [rows] for fp8 / int8, None for bf16

    @property
    def fmt(self) -> str:
        return _FMT_OF_DTYPE[self.w.dtype]

    def codes_numpy(self, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
        """Raw storage bits of rows [r0, r1) as uint16 (bf16) or uint8 (fp8, int8), on the host."""
        part = self.w[r0:r1]
        if self.fmt == "bf16":
            return part.view(torch.int16).cpu().numpy().view(np.uint16)
        return part.view(torch.uint8).cpu().numpy()

    def scale_numpy(self, r0: int = 0, r1: Optional[int] = None) -> Optional[np.ndarray]:
        if self.scale is None:
            return None
        return self.scale[r0:r1].cpu().numpy()


def _draw_matrix(rows: int, cols: int, fmt: str, gen: torch.Generator,
                 device, std: float = 0.02, chunk_rows: int = 8192) -> StoredMatrix:
    """N(0, std) in fp32, stored as bf16 or fp8 / int8 + per-row scale, drawn in row chunks."""
    out = torch.empty(rows, cols, dtype=_DTYPE_OF_FMT[fmt], device=device)
    if fmt != "bf16":
        scale = torch.empty(rows, dtype=torch.float32, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        w32 = torch.randn(r1 - r0, cols, generator=gen, device=device, dtype=torch.float32)
        w32.mul_(std)
        if fmt == "bf16":
            out[r0:r1] = w32.to(torch.bfloat16)
        else:
            q, s = quantize_rows_fp8(w32) if fmt == "fp8" else quantize_rows_int8(w32)
            out[r0:r1] = q
            scale[r0:r1] = s
        del w32
    return StoredMatrix(out, None if fmt == "bf16" else scale)


@dataclass
class ModelWeights:
    cfg: ModelConfig
    embed: StoredMatrix  # [V][d]
    attn_norm: torch.Tensor  # fp32 [L][d]
    qkv: List[StoredMatrix]  # [(Hq+2Hkv)dh][d]: Q heads, then K heads, then V heads
    o: List[StoredMatrix]  # [d][Hq dh]
    mlp_norm: torch.Tensor  # fp32 [L][d]
    gate_up: List[StoredMatrix]  # [2 d_ff][d]: gate rows then up rows
    down: List[StoredMatrix]  # [d][d_ff]
    final_norm: torch.Tensor  # fp32 [d]
    lm_head: StoredMatrix  # [V][d]

    def nbytes(self) -> int:
        def mb(m: StoredMatrix) -> int:
            return m.w.numel() * m.w.element_size() + (0 if m.scale is None else m.scale.numel() * 4)
        tot = mb(self.embed) + mb(self.lm_head)
        for lst in (self.qkv, self.o, self.gate_up, self.down):
            tot += sum(mb(m) for m in lst)
        tot += 4 * (self.attn_norm.numel() + self.mlp_norm.numel() + self.final_norm.numel())
        return tot


def make_weights(cfg: ModelConfig, seed: int = 0, device="cpu",
                 gains: str = "ones") -> ModelWeights:
    """Draw a model.  gains="ones" gives norm gains 1.0; "random" gives 1 + N(0, 0.1)."""
    dev = torch.device(device)
    fmt = cfg.weight_dtype
    L, d = cfg.n_layers, cfg.d_model
    cid = cfg.config_id

    def mat(layer, tid, rows, cols):
        return _draw_matrix(rows, cols, fmt, _stream(seed, cid, layer, tid, dev), dev)

    def gain(layer, tid, n):
        if gains == "ones":
            return torch.ones(n, dtype=torch.float32, device=dev)
        g = _stream(seed, cid, layer, tid, dev)
        return 1.0 + 0.1 * torch.randn(n, generator=g, device=dev, dtype=torch.float32)

    embed = mat(-1 & 0xFFFF, _T_EMBED, cfg.vocab, d)
    qkv, o, gu, down = [], [], [], []
    attn_norm = torch.empty(L, d, dtype=torch.float32, device=dev)
    mlp_norm = torch.empty(L, d, dtype=torch.float32, device=dev)
    for l in range(L):
        attn_norm[l] = gain(l, _T_ATTN_NORM, d)
        qkv.append(mat(l, _T_QKV, cfg.qkv_rows, d))
        o.append(mat(l, _T_O, d, cfg.n_q_heads * cfg.d_head))
        mlp_norm[l] = gain(l, _T_MLP_NORM, d)
        gu.append(mat(l, _T_GU, 2 * cfg.d_ff, d))
        down.append(mat(l, _T_DOWN, d, cfg.d_ff))
    final_norm = gain(0xFFFF, _T_FINAL_NORM, d)
    lm = mat(0xFFFF, _T_LM, cfg.vocab, d)
    return ModelWeights(cfg, embed, attn_norm, qkv, o, mlp_norm, gu, down, final_norm, lm)


# --------------------------------------------------------------------------
# paged KV cache and batch metadata
# --------------------------------------------------------------------------

KV_CANARY_BF16 = 0x7FC1  # a quiet-NaN bit pattern no kernel produces
KV_CANARY_FP8 = 0x7F  # the E4M3 NaN code


def kv_torch_dtype(kv_dtype: str) -> torch.dtype:
    return torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn


def kv_pool_shape(cfg: ModelConfig, num_blocks: int):
    """Pool layout [layer][K=0,V=1][block][kv head][slot 0..15][d_head]."""
    return (cfg.n_layers, 2, num_blocks, cfg.n_kv_heads, cfg.block_size, cfg.d_head)


def empty_kv_pool(cfg: ModelConfig, num_blocks: int, device="cpu", canary: bool = True) -> torch.Tensor:
    pool = torch.empty(kv_pool_shape(cfg, num_blocks), dtype=kv_torch_dtype(cfg.kv_dtype),
                       device=device)
    if canary:
        if cfg.kv_dtype == "bf16":
            pool.view(torch.int16).fill_(KV_CANARY_BF16)
        else:
            pool.view(torch.uint8).fill_(KV_CANARY_FP8)
    else:
        pool.view(torch.uint8).zero_()
    return pool


def make_block_tables(cfg: ModelConfig, batch: int, max_seq_len: int, num_blocks: int,
                      seed: int = 0) -> np.ndarray:
    """[batch][blocks_per_seq] int32: disjoint physical blocks from a seeded permutation."""
    nb = blocks_per_seq(max_seq_len, cfg.block_size)
    if batch * nb > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {batch} x {nb}")
    perm = _np_rng(seed, cfg.config_id, 0, _T_BT).permutation(num_blocks).astype(np.int32)
    return perm[: batch * nb].reshape(batch, nb).copy()


def make_context_lengths(wl: Workload, batch: int, seed: int = 0) -> np.ndarray:
    rng = _np_rng(seed, wl.model.config_id, batch, _T_LENS)
    return rng.integers(wl.ctx_lo, wl.ctx_hi + 1, size=batch).astype(np.int32)


def fill_context_kv(cfg: ModelConfig, pool: torch.Tensor, block_tables: np.ndarray,
                    ctx_lens: Sequence[int], seed: int = 0) -> None:
    """Write N(0,1) K and V (rounded to the cache dtype) into positions [0, ctx_len) of
    every sequence, for every layer and kv head; other slots are left untouched."""
    dev = pool.device
    bs = cfg.block_size
    for l in range(cfg.n_layers):
        g = _stream(seed, cfg.config_id, l, _T_CTX, dev)
        for b, n in enumerate(ctx_lens):
            n = int(n)
            if n == 0:
                continue
            nblk = (n + bs - 1) // bs
            vals = torch.randn(2, nblk, cfg.n_kv_heads, bs, cfg.d_head, generator=g,
                               device=dev, dtype=torch.float32)
            if cfg.kv_dtype == "fp8":
                vals.clamp_(-448.0, 448.0)
            vals = vals.to(pool.dtype)
            blks = torch.as_tensor(block_tables[b, :nblk].astype(np.int64), device=dev)
            full = n // bs
            if full:
                pool[l, :, blks[:full]] = vals[:, :full]
            rem = n - full * bs
            if rem:
                pool[l, :, blks[full], :, :rem] = vals[:, full, :, :rem]


def make_token_ids(cfg: ModelConfig, steps: int, batch: int, seed: int = 0) -> np.ndarray:
    """[steps][batch] int32 teacher-forced decode inputs, uniform in [0, vocab)."""
    rng = _np_rng(seed, cfg.config_id, batch, _T_IDS)
    return rng.integers(0, cfg.vocab, size=(steps, batch)).astype(np.int32)


def pool_blocks_needed(batch: int, max_seq_len: int, block: int = BLOCK) -> int:
    return batch * blocks_per_seq(max_seq_len, block)


def kv_codes_numpy(pool: torch.Tensor) -> np.ndarray:
    """Host copy of a pool's raw bits: uint16 for bf16, uint8 for fp8."""
    if pool.dtype == torch.bfloat16:
        return pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return pool.view(torch.uint8).cpu().numpy()


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

