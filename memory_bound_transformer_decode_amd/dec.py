"""ctypes binding over the C ABI in include/dec.h (argument marshalling only).

Every step of the decode path runs in the HIP kernels behind libdec.so; this
module only allocates device memory through torch, passes raw pointers and the
current HIP stream across the ABI, and turns status codes into exceptions.
Importing it loads the library and raises if it has not been built (there is
no fallback path).
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_double, c_float, c_int, c_int32, c_size_t, c_uint32, c_void_p
from typing import Optional, Sequence

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdec.so")

DEC_OK, DEC_E_INVALID, DEC_E_STATE, DEC_E_CAPACITY, DEC_E_UNSUPPORTED, DEC_E_HIP = 0, -1, -2, -3, -4, -5
DEC_BF16, DEC_FP8_E4M3, DEC_INT8 = 0, 1, 2
FLAG_EAGER, FLAG_UNFUSED, FLAG_NO_MFMA, FLAG_CAPTURE_ALL, FLAG_NO_ATTN_O = 1, 2, 4, 8, 16
PATH_GRAPH, PATH_MFMA_PRODUCTS, PATH_MFMA_ATTENTION, PATH_FOLDED_NORM, PATH_UNFUSED, PATH_ATTN_O = 1, 2, 4, 8, 16, 32
LADDER = (1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64)
BLOCK = 16


class DecConfig(Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("d_head", c_int32), ("d_ff", c_int32), ("vocab", c_int32),
                ("rms_eps", c_float), ("rope_theta", c_float), ("weight_dtype", c_int32),
                ("kv_dtype", c_int32), ("block_size", c_int32), ("num_blocks", c_int32),
                ("max_batch", c_int32), ("max_seq_len", c_int32), ("flags", c_uint32)]


class DecMat(Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p)]


class DecWeights(Structure):
    _fields_ = [("embed", DecMat), ("attn_norm", c_void_p), ("qkv", POINTER(DecMat)),
                ("o", POINTER(DecMat)), ("mlp_norm", c_void_p), ("gate_up", POINTER(DecMat)),
                ("down", POINTER(DecMat)), ("final_norm", c_void_p), ("lm_head", DecMat)]


class DecStepArgs(Structure):
    _fields_ = [("n_seqs", c_int32), ("token_ids", POINTER(c_int32)),
                ("seq_lens", POINTER(c_int32)), ("block_tables", POINTER(c_int32))]


class DecVerifyArgs(Structure):
    _fields_ = [("n_seqs", c_int32), ("k", c_int32), ("token_ids", POINTER(c_int32)),
                ("seq_lens", POINTER(c_int32)), ("block_tables", POINTER(c_int32))]


class DecPrefillArgs(Structure):
    _fields_ = [("n_tokens", c_int32), ("token_ids", POINTER(c_int32)), ("start_pos", c_int32),
                ("block_table", POINTER(c_int32))]


class DecInfo(Structure):
    _fields_ = [("kernels_per_step", c_int32), ("bucket", c_int32), ("attn_splits", c_int32),
                ("used_mfma", c_int32), ("used_graph", c_int32), ("graphs_captured", c_int32),
                ("flags", c_uint32), ("rows", c_int32), ("launches", c_int32)]


class DecAttnDesc(Structure):
    _fields_ = [("n_rows", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("d_head", c_int32),
                ("kv_dtype", c_int32), ("n_layers", c_int32), ("layer", c_int32), ("num_blocks", c_int32),
                ("max_blocks_per_seq", c_int32)]


class DecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dec error {code}: {msg}")
        self.code = code


EXPORTS = ("dec_workspace_bytes", "dec_create", "dec_load_weights", "dec_step", "dec_verify",
           "dec_prefill", "dec_set_flags", "dec_check", "dec_set_wait_limit", "dec_get_info",
           "dec_get_step_info", "dec_destroy", "dec_last_error", "dec_bw_probe", "dec_launch_matmul", "dec_sample_greedy", "dec_sample",
           "dec_attention_workspace_bytes", "dec_attention", "dec_attention_noalloc")
MAT_QKV, MAT_O, MAT_GATE_UP, MAT_DOWN, MAT_LM_HEAD = 0, 1, 2, 3, 4

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdec.so (raises if it is missing: build it with
    `python -m memory_bound_transformer_decode_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} is missing "
                          "(run python -m memory_bound_transformer_decode_amd.build)")
    lib = ctypes.CDLL(path)
    lib.dec_workspace_bytes.argtypes = [POINTER(DecConfig)]
    lib.dec_workspace_bytes.restype = c_size_t
    lib.dec_create.argtypes = [POINTER(DecConfig), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                               POINTER(c_void_p)]
    lib.dec_create.restype = c_int
    lib.dec_load_weights.argtypes = [c_void_p, POINTER(DecWeights)]
    lib.dec_load_weights.restype = c_int
    lib.dec_step.argtypes = [c_void_p, POINTER(DecStepArgs)]
    lib.dec_step.restype = c_int
    lib.dec_verify.argtypes = [c_void_p, POINTER(DecVerifyArgs)]
    lib.dec_verify.restype = c_int
    lib.dec_prefill.argtypes = [c_void_p, POINTER(DecPrefillArgs), POINTER(c_int32)]
    lib.dec_prefill.restype = c_int
    lib.dec_set_flags.argtypes = [c_void_p, c_uint32]
    lib.dec_set_flags.restype = c_int
    lib.dec_check.argtypes = [c_void_p]
    lib.dec_check.restype = c_int
    lib.dec_set_wait_limit.argtypes = [c_void_p, c_int32]
    lib.dec_set_wait_limit.restype = c_int
    lib.dec_get_info.argtypes = [c_void_p, POINTER(c_int32), POINTER(c_int32)]
    lib.dec_get_info.restype = c_int
    lib.dec_get_step_info.argtypes = [c_void_p, POINTER(DecInfo)]
    lib.dec_get_step_info.restype = c_int
    lib.dec_destroy.argtypes = [c_void_p]
    lib.dec_destroy.restype = c_int
    lib.dec_last_error.argtypes = []
    lib.dec_last_error.restype = ctypes.c_char_p
    lib.dec_bw_probe.argtypes = [c_void_p, c_size_t, c_int, c_void_p, POINTER(c_double)]
    lib.dec_bw_probe.restype = c_int
    lib.dec_sample_greedy.argtypes = [c_void_p, c_void_p]
    lib.dec_sample_greedy.restype = c_int
    lib.dec_sample.argtypes = [c_void_p, c_void_p, c_float, c_int, c_float, c_void_p]
    lib.dec_sample.restype = c_int
    lib.dec_launch_matmul.argtypes = [c_void_p, c_int, c_int]
    lib.dec_launch_matmul.restype = c_int
    lib.dec_attention_workspace_bytes.argtypes = [POINTER(DecAttnDesc)]
    lib.dec_attention_workspace_bytes.restype = c_size_t
    lib.dec_attention.argtypes = [POINTER(DecAttnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]
    lib.dec_attention.restype = c_int
    lib.dec_attention_noalloc.argtypes = [POINTER(DecAttnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p]
    lib.dec_attention_noalloc.restype = c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != DEC_OK:
        raise DecError(rc, load_library().dec_last_error().decode())


def _dtype_code(name: str) -> int:
    return {"bf16": DEC_BF16, "fp8": DEC_FP8_E4M3, "int8": DEC_INT8}[name]


def make_config(model, *, num_blocks: int, max_batch: int, max_seq_len: int, flags: int = 0) -> DecConfig:
    """DecConfig from a model description with the fields of synth.ModelConfig."""
    return DecConfig(model.n_layers, model.d_model, model.n_q_heads, model.n_kv_heads, model.d_head,
                     model.d_ff, model.vocab, float(model.rms_eps), float(model.rope_theta),
                     _dtype_code(model.weight_dtype), _dtype_code(model.kv_dtype), BLOCK,
                     num_blocks, max_batch, max_seq_len, flags)


def workspace_bytes(cfg: DecConfig) -> int:
    n = load_library().dec_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        _check(DEC_E_INVALID)
    return n


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _mat(m) -> DecMat:
    return DecMat(_ptr(m.w), _ptr(m.scale))


def ladder_bucket(n: int) -> int:
    for b in LADDER:
        if b >= n:
            return b
    raise ValueError(n)


class Decoder:
    """One decode-step context over caller-visible torch buffers.

    model: an object with the fields of synth.ModelConfig; weights: an object with
    the fields of synth.ModelWeights (device tensors).  The KV pool is
    [layers][2][num_blocks][kv_heads][16][d_head] in the cache dtype.
    """

    def __init__(self, model, weights, *, num_blocks: int, max_batch: int, max_seq_len: int,
                 flags: int = 0, kv_pool: Optional[torch.Tensor] = None, device="cuda"):
        self.lib = load_library()
        self.model = model
        self.cfg = make_config(model, num_blocks=num_blocks, max_batch=max_batch,
                               max_seq_len=max_seq_len, flags=flags)
        self.bps = (max_seq_len + BLOCK - 1) // BLOCK
        self.device = torch.device(device)
        ws_n = workspace_bytes(self.cfg)
        kv_dt = torch.bfloat16 if model.kv_dtype == "bf16" else torch.float8_e4m3fn
        shape = (model.n_layers, 2, num_blocks, model.n_kv_heads, BLOCK, model.d_head)
        if model.n_layers == 0:  # no cache is touched; the ABI still wants a valid pointer
            kv_pool = torch.zeros(16, dtype=torch.uint8, device=self.device)
        elif kv_pool is None:
            kv_pool = torch.zeros(shape, dtype=kv_dt, device=self.device)
        elif tuple(kv_pool.shape) != shape or kv_pool.dtype != kv_dt or not kv_pool.is_contiguous():
            raise ValueError(f"kv_pool must be a contiguous {kv_dt} tensor of shape {shape}")
        self.kv_pool = kv_pool
        self.workspace = torch.empty(ws_n, dtype=torch.uint8, device=self.device)
        self.logits = torch.empty(max_batch, model.vocab, dtype=torch.float32, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        self._last_n = 0
        ctx = c_void_p()
        _check(self.lib.dec_create(ctypes.byref(self.cfg), c_void_p(self.stream.cuda_stream),
                                   c_void_p(kv_pool.data_ptr()), c_void_p(self.workspace.data_ptr()),
                                   ws_n, c_void_p(self.logits.data_ptr()), ctypes.byref(ctx)))
        self.ctx = ctx
        self.load_weights(weights)

    def load_weights(self, w) -> None:
        L = self.model.n_layers
        self._w = w  # keep the tensors alive
        self._arrays = [(DecMat * max(L, 1))(*[_mat(m) for m in lst]) for lst in
                        (w.qkv, w.o, w.gate_up, w.down)]
        self._dw = DecWeights(_mat(w.embed), _ptr(w.attn_norm), self._arrays[0], self._arrays[1],
                              _ptr(w.mlp_norm), self._arrays[2], self._arrays[3], _ptr(w.final_norm),
                              _mat(w.lm_head))
        _check(self.lib.dec_load_weights(self.ctx, ctypes.byref(self._dw)))

    def step(self, token_ids: Sequence[int], seq_lens: Sequence[int], block_tables) -> torch.Tensor:
        """Enqueue one step; returns the [n, vocab] fp32 logits view (valid once the
        stream reaches it, e.g. after .cpu() or a synchronize)."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        n = ids.shape[0]
        if lens.shape != (n,) or bt.shape != (n, self.bps):
            raise ValueError(f"expected seq_lens [{n}] and block_tables [{n}][{self.bps}]")
        P = POINTER(c_int32)
        args = DecStepArgs(n, ids.ctypes.data_as(P), lens.ctypes.data_as(P), bt.ctypes.data_as(P))
        _check(self.lib.dec_step(self.ctx, ctypes.byref(args)))
        self._last_n = n
        return self.logits[:n]

    def verify(self, token_ids, seq_lens: Sequence[int], block_tables) -> torch.Tensor:
        """Enqueue the k-token verify step: token_ids [n][k], seq_lens [n] (position of
        each sequence's first token), block_tables [n][bps].  Returns the [n, k, vocab]
        fp32 logits view (row (s, j): after token j of sequence s)."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        if ids.ndim != 2:
            raise ValueError("token_ids must be [n][k]")
        n, k = ids.shape
        if lens.shape != (n,) or bt.shape != (n, self.bps):
            raise ValueError(f"expected seq_lens [{n}] and block_tables [{n}][{self.bps}]")
        P = POINTER(c_int32)
        args = DecVerifyArgs(n, k, ids.ctypes.data_as(P), lens.ctypes.data_as(P), bt.ctypes.data_as(P))
        _check(self.lib.dec_verify(self.ctx, ctypes.byref(args)))
        self._last_n = n * k
        return self.logits[: n * k].view(n, k, -1)

    def prefill(self, token_ids: Sequence[int], start_pos: int, block_table) -> torch.Tensor:
        """Enqueue chunked prefill of one prompt at positions start_pos, start_pos + 1, ...;
        returns the [vocab] fp32 logits view after the prompt's last token."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if ids.ndim != 1 or bt.shape != (self.bps,):
            raise ValueError(f"expected token_ids [n] and block_table [{self.bps}]")
        P = POINTER(c_int32)
        row = c_int32(-1)
        args = DecPrefillArgs(ids.shape[0], ids.ctypes.data_as(P), int(start_pos), bt.ctypes.data_as(P))
        _check(self.lib.dec_prefill(self.ctx, ctypes.byref(args), ctypes.byref(row)))
        self._last_n = row.value + 1
        return self.logits[row.value]

    def sample_greedy(self) -> torch.Tensor:
        """Enqueue greedy sampling of the last step: int32 [n] token ids on the device."""
        n = self._last_n
        out = torch.empty(n, dtype=torch.int32, device=self.device)
        _check(self.lib.dec_sample_greedy(self.ctx, c_void_p(out.data_ptr())))
        return out

    def sample(self, uniforms: torch.Tensor, temperature: float, top_k: int, top_p: float) -> torch.Tensor:
        """Enqueue top-k / top-p sampling of the last step with the draws `uniforms`
        (float32 [n] on the device, in [0, 1)): int32 [n] token ids on the device."""
        n = self._last_n
        out = torch.empty(n, dtype=torch.int32, device=self.device)
        _check(self.lib.dec_sample(self.ctx, c_void_p(uniforms.data_ptr()), float(temperature), int(top_k),
                                   float(top_p), c_void_p(out.data_ptr())))
        return out

    def launch_matmul(self, which: int, layer: int = 0) -> None:
        """Enqueue one matrix kernel of the step alone (for timing; clobbers intermediates)."""
        _check(self.lib.dec_launch_matmul(self.ctx, which, layer))

    def set_flags(self, flags: int) -> None:
        _check(self.lib.dec_set_flags(self.ctx, flags))

    def check(self) -> None:
        """dec_check: wait for the stream; raise if a device-side wait gave up."""
        _check(self.lib.dec_check(self.ctx))

    def set_wait_limit(self, polls: int) -> None:
        _check(self.lib.dec_set_wait_limit(self.ctx, polls))

    def info(self) -> DecInfo:
        out = DecInfo()
        _check(self.lib.dec_get_step_info(self.ctx, ctypes.byref(out)))
        return out

    def path(self):
        """(kernels per plan, PATH_* bits) of the last call (dec_get_info)."""
        k, f = c_int32(), c_int32()
        _check(self.lib.dec_get_info(self.ctx, ctypes.byref(k), ctypes.byref(f)))
        return k.value, f.value

    def close(self) -> None:
        if getattr(self, "ctx", None):
            rc = self.lib.dec_destroy(self.ctx)
            self.ctx = None
            _check(rc)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def attn_desc(q: torch.Tensor, pool: torch.Tensor, layer: int, block_tables: torch.Tensor) -> DecAttnDesc:
    """Descriptor of an attention call from q [n][Hq][dh] fp32, the pool
    [L][2][num_blocks][Hkv][16][dh] and block tables [n][max_blocks_per_seq]."""
    n, Hq, dh = q.shape
    L, _, nb, Hkv, _, dh2 = pool.shape
    if dh2 != dh:
        raise ValueError("q and pool disagree on d_head")
    kv = DEC_BF16 if pool.dtype == torch.bfloat16 else DEC_FP8_E4M3
    return DecAttnDesc(n, Hq, Hkv, dh, kv, L, layer, nb, block_tables.shape[1])


def attention(q: torch.Tensor, pool: torch.Tensor, layer: int, seq_lens: torch.Tensor,
              block_tables: torch.Tensor, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dec_attention on the current stream: o [n][Hq * dh] bf16 (device tensors in)."""
    lib = load_library()
    desc = attn_desc(q, pool, layer, block_tables)
    n = load_library().dec_attention_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        _check(DEC_E_INVALID)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1] * q.shape[2], dtype=torch.bfloat16, device=q.device)
    _check(lib.dec_attention(ctypes.byref(desc), c_void_p(q.data_ptr()), c_void_p(pool.data_ptr()),
                             c_void_p(seq_lens.data_ptr()), c_void_p(block_tables.data_ptr()),
                             c_void_p(out.data_ptr()), c_void_p(workspace.data_ptr()),
                             workspace.numel() * workspace.element_size(),
                             c_void_p(torch.cuda.current_stream(q.device).cuda_stream)))
    return out


def bw_probe(buf: torch.Tensor, reps: int = 5) -> float:
    """Best streaming-read bandwidth (bytes/s) over `buf` measured on the current stream."""
    lib = load_library()
    out = c_double()
    n = buf.numel() * buf.element_size() // 16 * 16
    _check(lib.dec_bw_probe(c_void_p(buf.data_ptr()), n, reps,
                            c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(out)))
    return out.value
