"""Gated DeltaNet ReplaySSM verify / rollback / flush on MI355X (gfx950).

The work runs in libgdnreplay.so (hand-written HIP kernels behind the C ABI of
include/gdn_replay.h); the Python side only marshals arguments.

  build    compiles csrc/ for gfx950 into libgdnreplay.so (in-tree).
  binding  ctypes declarations of the C entry points; raises if the library is
           missing (there is no CPU fallback).
  cache    one layer's replay cache (state, ring, pointers, counters) as torch
           device tensors, with the verify / rollback / flush calls and their
           fused forms (verify_flush, rollback_verify_flush, step_norm_fp8).
  conv     the causal convolution before the recurrence, with its input ring.
  norm     the gated RMSNorm + FP8 quantisation of the recurrence's outputs.
  synth    seeded synthetic inputs and the named workloads (no method arithmetic).
"""
