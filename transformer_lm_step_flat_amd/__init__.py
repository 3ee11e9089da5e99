"""MI355X-native fp32 GPT-2 training step: hand-written gfx950 HIP kernels
behind a C ABI (``include/gpt2.h``), with a thin ctypes binding.

Submodules:
  synth  -- seeded synthetic shapes, weights and token batches (no step arithmetic)
  gpt2   -- the binding to ``libgpt2mi.so`` (imports torch for memory and streams)
  build  -- compiles the HIP library for gfx950
"""
