"""fp64 CPU oracle for one decode step of a dense decoder-only transformer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path (no kernels, headers, tables or
helpers); the only thing both sides consume is the seeded input generator,
which holds none of the step's arithmetic.

What it computes is the plain definition of one decode step (pre-norm blocks,
RMSNorm, QKV projection, rotary embedding, cached grouped-query attention,
O projection, SwiGLU MLP, final norm, LM head), in float64, from the stored
bits of the weights and the KV cache, decoded by this package's own codecs.
The pages this follows state that fusion, FlashAttention and CUDA graphs
change how the mathematics executes, not what it computes (kernel-fusion
architecture study, section 11 "Kernel-fusion strategy" and Figure 4), so the
plain definition is the reference; FP8 storage is the one change to *what* is
computed (as is INT8 weight-only storage), and the oracle therefore takes the
already-quantized model as the model's definition.

Modules:
  codecs   -- bf16, FP8-E4M3 and int8 decode/encode from the bit definitions
  decoder  -- the fp64 decode step over a paged KV cache, the multi-token step
              (verify, prefill) as its causal generalisation, plus the MAC ledger
  sampling -- the top-k / top-p rule after the LM head
  inputs   -- adapters from the seeded inputs to the oracle's objects

Every function is pinned by the `-m "not gpu"` tests against closed forms,
worked examples printed on the pages, invariants and brute force; the one
result with no such pin (whole-model logits beyond the brute-forced tiny
shapes) is marked "parity unpinned" in decoder.py.
"""

from . import codecs, decoder  # noqa: F401
