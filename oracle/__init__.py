"""CPU oracle for the Gated DeltaNet ReplaySSM verify / rollback / flush path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package. Only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

  gdn_oracle   fp64 token-by-token recurrence, full-state snapshot / restore on
               rejection, and an independent replay mode.
  bookkeeping  pure-integer model of the ring pointers and error bits.
  wy_check     fp64 chunk (WY / UT) form of the same replay, used only to pin
               the algebra that the HIP kernels implement.
  norm_oracle  fp64 gated RMSNorm of the GDN output and its FP8 (OCP E4M3)
               quantisation with one scale per (token, head).
  conv_oracle  fp64 short causal convolution before the recurrence, its input
               history kept in a ring that shares the recurrence's pointers.
"""
