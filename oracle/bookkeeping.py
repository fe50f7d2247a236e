"""Pure-integer model of the replay ring pointers and the sticky error word.

TEST INFRASTRUCTURE ONLY. Follows "The inference stack behind OCRia"
(LlamaIndex), section "Making speculative verification cheaper": a rejection
only moves a buffer pointer so that the accepted prefix is kept; the full
checkpoint is written only at a periodic flush.

Per slot: head (ring position of the first committed token), len (number of
committed tokens not yet folded into the checkpoint), capacity C.

  verify(D):    needs len + D <= C; the draft occupies ring positions
                (head + len + j) mod C, j < D. Pointers unchanged.
  rollback(a):  needs 0 <= a <= D and len + a <= C; len += a.
  flush(m):     if len >= max(m, 1): head = (head + len) mod C, len = 0.
  verify_flush(D, m): flush(m), then verify(D).
D may be one value for every request or one per request (D_i in [0, D_max];
D_i = 1 is plain decode, D_i = 0 no draft). Violations set CAPACITY=1 /
ACCEPT=2 / SLOT=4 / POINTER=8 (head outside [0, C) or len outside [0, C]) /
DRAFT=16 (D_i outside [0, D_max]) and leave the slot untouched; they are checked
in the order slot, pointers, draft length, then capacity or accept count.
"""
from __future__ import annotations

ERR_CAPACITY = 1
ERR_ACCEPT = 2
ERR_SLOT = 4
ERR_POINTER = 8
ERR_DRAFT = 16


def _lengths(draft_len, n: int):
    """(per-request lengths, maximum): one int for all, or a sequence with the
    maximum given as draft_len_max."""
    if isinstance(draft_len, (int,)):
        return [int(draft_len)] * n
    return [int(d) for d in draft_len]


class RingPointers:
    def __init__(self, head, length, cap: int):
        self.head = [int(h) for h in head]
        self.len = [int(n) for n in length]
        self.cap = int(cap)
        self.err = 0

    def _ok(self, s: int) -> bool:
        if not 0 <= s < len(self.head):
            self.err |= ERR_SLOT
            return False
        if not (0 <= self.head[s] < self.cap and 0 <= self.len[s] <= self.cap):
            self.err |= ERR_POINTER
            return False
        return True

    def verify(self, slots, draft_len, d_max: int | None = None):
        """Returns {slot: [ring positions written]} for the requests accepted.
        draft_len: one length for all requests, or one per request (then d_max
        bounds them)."""
        slots = [int(s) for s in slots]
        Ds = _lengths(draft_len, len(slots))
        d_max = max(Ds + [0]) if d_max is None else int(d_max)
        written = {}
        for s, D in zip(slots, Ds):
            if not self._ok(s):
                continue
            if not 0 <= D <= d_max:
                self.err |= ERR_DRAFT
                continue
            if self.len[s] + D > self.cap:
                self.err |= ERR_CAPACITY
                continue
            written[s] = [(self.head[s] + self.len[s] + j) % self.cap for j in range(D)]
        return written

    def rollback(self, slots, draft_len, accepted, d_max: int | None = None):
        slots = [int(s) for s in slots]
        Ds = _lengths(draft_len, len(slots))
        d_max = max(Ds + [0]) if d_max is None else int(d_max)
        for s, a, D in zip(slots, accepted, Ds):
            a = int(a)
            if not self._ok(s):
                continue
            if not 0 <= D <= d_max:
                self.err |= ERR_DRAFT
                continue
            if not 0 <= a <= D:
                self.err |= ERR_ACCEPT
                continue
            if self.len[s] + a > self.cap:
                self.err |= ERR_CAPACITY
                continue
            self.len[s] += a

    def flush(self, slots, min_len: int):
        """Returns {slot: number of tokens folded} for the slots that were due."""
        folded = {}
        for s in slots:
            s = int(s)
            if not self._ok(s):
                continue
            n = self.len[s]
            if n >= max(int(min_len), 1):
                folded[s] = n
                self.head[s] = (self.head[s] + n) % self.cap
                self.len[s] = 0
        return folded

    def verify_flush(self, slots, draft_len, min_len: int, d_max: int | None = None):
        """flush(min_len) then verify(draft_len): (folded, written) of the two. A
        request with a draft length outside [0, d_max] is not flushed either."""
        slots = [int(s) for s in slots]
        Ds = _lengths(draft_len, len(slots))
        d_max = max(Ds + [0]) if d_max is None else int(d_max)
        valid = [0 <= s < len(self.head) and 0 <= self.head[s] < self.cap
                 and 0 <= self.len[s] <= self.cap for s in slots]
        flushable = [s for s, D, ok in zip(slots, Ds, valid) if not (ok and not 0 <= D <= d_max)]
        folded = self.flush(flushable, min_len)
        return folded, self.verify(slots, Ds, d_max)
