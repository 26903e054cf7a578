"""MI355X-native decode step of a dense decoder-only transformer.

The step runs in hand-written HIP kernels for gfx950 behind a C ABI
(include/dec.h); `dec` is the thin ctypes binding over it.  Importing this
package loads nothing native: `from memory_bound_transformer_decode_amd import
dec` does, and raises if the HIP library has not been built.

Submodules:
  dec        -- binding: Decoder, config/weight marshalling (needs the built library)
  synth      -- seeded synthetic workloads and inputs
  perfmodel  -- byte / FLOP / launch-tax ledgers used to price measurements
"""

__all__ = ["dec", "synth", "perfmodel"]
