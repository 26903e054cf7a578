"""Byte, FLOP and launch-overhead ledgers for the decode step.

These are the closed-form models the pages use to reason about decode, applied
to this library's workloads; the benchmark prices its measurements against
them.

* Roofline step bound ("GPU Inference Internals", TL;DR equation): a step
  takes at least max(F / (eta_c C), D_HBM / (eta_b B_HBM), D_link / B_link);
  on one GPU the link term is zero.
* Machine balance = peak compute / memory bandwidth ("GPU Inference
  Internals", The Hardware Ledger).
* About 2 P FLOPs per token; batch-1 intensity about 2 FLOP/B for an FP8 70B
  model; single-stream ceiling = bandwidth / bytes per token; weight-only
  intensity 2B/b_w ("GPU Inference Internals", Roofline: Why Decode Is
  Memory-Bound).
* KV bytes per token = 2 x layers x kv_heads x head_dim x bytes ("GPU
  Inference Internals", The KV-Cache Ledger).
* Step ledger D_step(B, S) ~ W + B S K + D_activation, F_step ~ 2 P B
  ("GPU Inference Internals", Batching Economics).
* Launch tax, two forms: T_eager ~ T_compute + N tau, T_graph ~ T_compute +
  tau ("CUDA graphs & kernel fusion", Direct answer); and eager step
  = max(GPU work, launches x CPU cost per launch) ("Kernels, Fusion & CUDA
  Graphs", Fix 2: CUDA graphs).

Algorithmic bytes of one step (what the method must move; activations are left
out, so fractions of peak computed from it are conservative):
  W_step = all layer matrices + fp8 scales + norm gains + LM head
           + only the B embedding rows read
  KV     = sum_s (p_s + 1) K_tok read + B K_tok written, K_tok = 2 L Hkv dh b_kv
  logits = B V 4 bytes written
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

MI355X_HBM_BYTES_PER_S = 8.0e12  # published peak HBM3E bandwidth
MI355X_BF16_DENSE_FLOPS = 2.5e15  # dense MFMA bf16
MI355X_FP8_DENSE_FLOPS = 5.0e15  # dense MFMA fp8
MI355X_FP32_VECTOR_FLOPS = 157.3e12


def wbytes(dtype: str) -> int:
    return {"bf16": 2, "fp8": 1, "fp16": 2, "fp32": 4, "int8": 1}[dtype]


@dataclass(frozen=True)
class Shape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    d_ff: int
    vocab: int
    weight_dtype: str = "bf16"
    kv_dtype: str = "bf16"

    @classmethod
    def of(cls, cfg) -> "Shape":
        return cls(cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.d_head,
                   cfg.d_ff, cfg.vocab, cfg.weight_dtype, cfg.kv_dtype)

    # matrix shapes (rows x cols, row = output channel)
    def layer_matrices(self):
        d, dh = self.d_model, self.d_head
        return [((self.n_q_heads + 2 * self.n_kv_heads) * dh, d),  # W_qkv
                (d, self.n_q_heads * dh),  # W_o
                (2 * self.d_ff, d),  # W_gate_up
                (d, self.d_ff)]  # W_down

    def layer_params(self) -> int:
        return sum(r * c for r, c in self.layer_matrices())

    def matmul_params(self) -> int:
        """Parameters that take part in a matrix product per token (all layer matrices
        and the LM head; the embedding is a row lookup)."""
        return self.n_layers * self.layer_params() + self.vocab * self.d_model

    def total_params(self) -> int:
        return self.matmul_params() + self.vocab * self.d_model + \
            (2 * self.n_layers + 1) * self.d_model

    def layer_rows(self) -> int:
        return sum(r for r, _ in self.layer_matrices())

    def kv_bytes_per_token(self) -> int:
        return kv_bytes_per_token(self.n_layers, self.n_kv_heads, self.d_head,
                                  wbytes(self.kv_dtype))

    def weight_bytes_per_step(self, batch: int) -> int:
        """Weight bytes one step must stream: every layer matrix, the LM head, fp8
        per-row scales, fp32 norm gains, and only the `batch` embedding rows."""
        b = wbytes(self.weight_dtype)
        scaled = self.weight_dtype == "fp8"
        tot = self.n_layers * self.layer_params() * b
        tot += self.vocab * self.d_model * b
        if scaled:
            tot += 4 * (self.n_layers * self.layer_rows() + self.vocab)
        tot += batch * self.d_model * b + (4 * batch if scaled else 0)
        tot += 4 * (2 * self.n_layers + 1) * self.d_model
        return tot

    def step_bytes(self, seq_lens: Sequence[int]) -> int:
        """Algorithmic HBM bytes of one step for live sequences at positions seq_lens."""
        B = len(seq_lens)
        k_tok = self.kv_bytes_per_token()
        kv = sum(int(p) + 1 for p in seq_lens) * k_tok + B * k_tok
        return self.weight_bytes_per_step(B) + kv + B * self.vocab * 4

    def step_flops(self, seq_lens: Sequence[int]) -> int:
        """2 x (matrix-product MACs + attention MACs) for one step."""
        macs = len(seq_lens) * self.matmul_params()
        macs += sum(2 * self.n_q_heads * self.d_head * (int(p) + 1) * self.n_layers
                    for p in seq_lens)
        return 2 * macs


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, bytes_per_elem: int) -> int:
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_elem


def machine_balance(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth


def weight_only_intensity(batch: int, bytes_per_weight: float) -> float:
    return 2.0 * batch / bytes_per_weight


def balance_crossover_batch(peak_flops: float, bandwidth: float, bytes_per_weight: float) -> float:
    """Batch at which weight-only intensity 2B/b_w reaches machine balance."""
    return machine_balance(peak_flops, bandwidth) * bytes_per_weight / 2.0


def single_stream_ceiling(bandwidth: float, bytes_per_token: float) -> float:
    return bandwidth / bytes_per_token


def roofline_step_time(flops: float, hbm_bytes: float, peak_flops: float, bandwidth: float,
                       eta_c: float = 1.0, eta_b: float = 1.0,
                       link_bytes: float = 0.0, link_bw: float = float("inf")) -> float:
    return max(flops / (eta_c * peak_flops), hbm_bytes / (eta_b * bandwidth),
               link_bytes / link_bw if link_bytes else 0.0)


@dataclass(frozen=True)
class LaunchTax:
    """Seconds per step: the GPU work alone, with one launch per kernel, with one graph launch."""

    compute_s: float
    eager_s: float
    graph_s: float

    @property
    def graph_gain(self) -> float:
        return self.eager_s / self.graph_s

    @property
    def tax_share(self) -> float:
        """Launch overhead of the eager step relative to the GPU work."""
        return (self.eager_s - self.compute_s) / self.compute_s


def launch_tax(compute_s: float, kernels: int, per_launch_s: float) -> LaunchTax:
    """The additive launch-tax model ("CUDA graphs & kernel fusion", Direct answer): a
    step launched kernel by kernel costs its GPU work plus one launch cost per kernel;
    replayed as one graph it costs the GPU work plus a single launch."""
    return LaunchTax(compute_s, compute_s + kernels * per_launch_s, compute_s + per_launch_s)


def weight_streaming_launch_tax(weight_bytes: float, bandwidth: float, kernels: int,
                                per_launch_s: float) -> LaunchTax:
    """launch_tax for a step whose GPU work is one read of the weights at `bandwidth`
    (the memory term of roofline_step_time, no compute term)."""
    return launch_tax(roofline_step_time(0.0, weight_bytes, float("inf"), bandwidth), kernels, per_launch_s)


def overlapped_eager_step_s(weight_bytes: float, flops: float, bw: float, peak_flops: float,
                            n_launches: int, cpu_cost_per_launch_s: float) -> float:
    """Overlap model: eager step = max(GPU work, launches x CPU cost per launch)."""
    gpu = max(weight_bytes / bw, flops / peak_flops)
    return max(gpu, n_launches * cpu_cost_per_launch_s)
