"""fp64 CPU oracle of the short causal convolution of GDN layers under block
speculative decoding, with its history kept in a ring and rolled back by pointer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
"The inference stack behind OCRia" (LlamaIndex): GDN layers run a causal
convolution before the recurrence (the post lists a faster causal convolution
for GDN layers among its fused kernels), and the section "Making speculative
verification cheaper" replaces state restores on rejection by buffers whose
pointer moves. The convolution's state is the last K - 1 inputs of the
committed stream, so it gets the same treatment as the recurrence's inputs:

* every input x_t (one channel vector per token: the concatenated q, k, v
  projections before the convolution) is appended to a ring that shares the
  slot's head / len with the recurrence's ring: the draft tokens of a step go to
  positions (head + len + j) mod C, exactly where the recurrence appends them;
* a rollback is len += a (no state to restore), a flush moves head / len (the
  inputs before head stay in the ring, so the history survives it);
* the output of draft token j, per channel c (depthwise, width K):

      y_j[c] = silu( b[c] + sum_{i=0}^{K-1} w[c][i] * x_{j-(K-1)+i}[c] )

  where x with a negative index is the committed input that many tokens before
  the draft, read from the ring at (head + len + index) mod C; a slot starts with
  a zero ring, which gives the usual zero padding of a causal convolution.

Readings taken (listed in the design notes): depthwise, width K, bias optional,
silu after the convolution, fp32 weights, bf16 inputs; the ring needs
C >= D + K - 1 so that the draft never overwrites the history it reads. Only the
last K - 1 committed inputs are ever read, so (unlike the recurrence's ring,
whose committed rows wait for the flush) len + D may exceed C: the draft then
overwrites committed inputs that no step reads again. This lets the step run
before a verify_flush that folds the due slots first.
"""
from __future__ import annotations

import numpy as np

from .gdn_oracle import ERR_POINTER, ERR_SLOT, to_f64


def silu(x):
    return x / (1.0 + np.exp(-x))


class ConvOracle:
    """The input ring of one layer's convolution; pointers come from the
    recurrence's cache model (head, len arrays of the same slots)."""

    def __init__(self, ring: np.ndarray, cap: int):
        self.ring = np.array(ring)          # [slots][C][CH] (bf16 bits or fp32)
        self.cap = int(cap)
        self.err = 0

    def update(self, head, length, slot_idx, x, weight, bias=None, magnitudes=False):
        """Outputs [R, D, CH] (NaN for skipped requests) of the draft x [R, D, CH];
        appends x to the ring. head / length: the slots' pointers before the
        step's rollback (they are not changed here). With magnitudes=True also
        returns |b| + sum_i |w_i x_i| per output (the scale of the rounding
        error of any evaluation of the sum)."""
        slot_idx = np.asarray(slot_idx)
        R, D, CH = np.asarray(x).shape
        w = np.asarray(weight, dtype=np.float64)          # [CH, K]
        K = w.shape[1]
        b = np.zeros(CH) if bias is None else np.asarray(bias, dtype=np.float64)
        out = np.full((R, D, CH), np.nan)
        mag = np.full((R, D, CH), np.nan)
        for i in range(R):
            s = int(slot_idx[i])
            if s < 0 or s >= self.ring.shape[0]:
                self.err |= ERR_SLOT
                continue
            h, n = int(head[s]), int(length[s])
            if not (0 <= h < self.cap and 0 <= n <= self.cap):
                self.err |= ERR_POINTER
                continue
            # history: the K - 1 inputs before the draft, oldest first
            hist = [to_f64(self.ring[s, (h + n - (K - 1) + m) % self.cap]) for m in range(K - 1)]
            seq = hist + [to_f64(np.asarray(x[i, j])) for j in range(D)]
            for j in range(D):
                acc = b.copy()
                m = np.abs(b)
                for t in range(K):
                    acc = acc + w[:, t] * seq[j + t]
                    m = m + np.abs(w[:, t] * seq[j + t])
                out[i, j] = silu(acc)
                mag[i, j] = m
            for j in range(D):
                self.ring[s, (h + n + j) % self.cap] = x[i, j]
        return (out, mag) if magnitudes else out
