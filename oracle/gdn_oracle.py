"""fp64 CPU oracle of the ReplaySSM verify / rollback / flush step for GDN layers.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy in float64,
one token at a time, one request at a time (heads vectorised).

What it follows
---------------
* The recurrence is the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated
  Delta Networks: Improving Mamba2 with Delta Rule", 2025), per value head:
      S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
      o_t = S_t q_t                      (output taken after the update)
  S is d_v x d_k. The stored checkpoint is its transpose H = S^T (d_k x d_v).
* The ReplaySSM scheme: "The inference stack behind OCRia" (LlamaIndex),
  section "Making speculative verification cheaper". A GDN layer's fixed-size
  recurrent state is read, updated and written back per token, which makes a
  rejected speculative token expensive to undo. ReplaySSM keeps a state
  checkpoint plus a small buffer of recent inputs, computes outputs from the
  checkpoint and the buffered inputs, writes the full checkpoint only at a
  periodic flush, and on rejection only moves a buffer pointer so that the
  accepted prefix is kept.
* Accept rule: a draft block is accepted up to its first rejected token, all
  later tokens are rejected ("Inference Engineering", chapter 5, section 5.2
  "Speculative decoding"); the caller passes the accepted count.

Two ways of computing the same thing
------------------------------------
mode="snapshot": keeps a live state per (slot, head) equal to the checkpoint
advanced over the committed tokens. verify takes an explicit full-state
snapshot, advances the live state over the draft, and rollback restores the
snapshot and re-advances over the accepted prefix. flush copies the live state
into the checkpoint. This is the "restore the state on rejection" scheme that
ReplaySSM avoids, written out literally.

mode="replay": holds only the checkpoint and the ring. verify recomputes from
the checkpoint over the committed ring records and then the draft; flush folds
the committed ring records into the checkpoint. This is ReplaySSM itself.

Both modes run the same fp64 steps in the same order, so they agree bitwise.

Readings taken where the pages are silent (each listed in the design notes)
--------------------------------------------------------------------------
* alpha is a direct multiplicative decay, beta a write strength; no clamping,
  no q scaling, no in-kernel normalisation.
* value head h uses key head h // (HV // HK) (consecutive grouping).
* verify appends the whole draft behind the committed tokens, at ring
  positions (head + len + j) mod C; rollback commits the accepted prefix by
  len += a; flush folds all committed tokens of slots with
  len >= max(min_len, 1) and sets head = (head + len) mod C, len = 0.
* contract violations skip the request and OR a bit into a sticky error word:
  CAPACITY (len + D > C at verify, len + a > C at rollback), ACCEPT
  (a outside [0, D]), SLOT (slot index outside [0, num_slots)), POINTER
  (head outside [0, C) or len outside [0, C]), DRAFT (a per-request draft
  length outside [0, D_max]).
* a buffered token's q is never read.
* per-request draft lengths: request i drafts D_i <= D_max tokens, the first
  D_i rows of its D_max-row block; D_i = 1 is plain (non-speculative) decode
  and D_i = 0 leaves the request without a draft (nothing appended, no outputs,
  its flush still happens in verify_flush). Rows past D_i are neither read nor
  written.
"""
from __future__ import annotations

import numpy as np

ERR_CAPACITY = 1
ERR_ACCEPT = 2
ERR_SLOT = 4
ERR_POINTER = 8
ERR_DRAFT = 16


def per_request_lengths(draft_lens, num_reqs: int, d_max: int) -> np.ndarray:
    """Draft length of every request: d_max for all, or the given per-request
    values (checked against [0, d_max] by the calls)."""
    if draft_lens is None:
        return np.full(num_reqs, d_max, dtype=np.int64)
    out = np.asarray(draft_lens, dtype=np.int64).reshape(-1)
    assert out.shape[0] == num_reqs
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the bits are the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# one step of the gated delta rule
# ---------------------------------------------------------------------------
def gdn_step_literal(S, k, v, alpha, beta):
    """S_t = alpha S (I - beta k k^T) + beta v k^T, with the dense d_k x d_k matrix.

    S: [..., dv, dk]; k: [..., dk]; v: [..., dv]; alpha, beta: [...]."""
    dk = S.shape[-1]
    eye = np.eye(dk)
    M = eye - beta[..., None, None] * (k[..., :, None] * k[..., None, :])
    return alpha[..., None, None] * (S @ M) + beta[..., None, None] * (v[..., :, None] * k[..., None, :])


def gdn_step(S, k, v, alpha, beta):
    """Same step in its rank-1 form: S_t = alpha S + beta (v - alpha S k) k^T.

    Expanding alpha S (I - beta k k^T) + beta v k^T gives exactly this."""
    Sk = np.einsum("...ij,...j->...i", S, k)
    u = beta[..., None] * (v - alpha[..., None] * Sk)
    return alpha[..., None, None] * S + u[..., :, None] * k[..., None, :]


def gdn_output(S, q):
    """o = S q."""
    return np.einsum("...ij,...j->...i", S, q)


class ReplayOracle:
    """fp64 model of one layer's replay cache and of the three calls on it."""

    def __init__(self, init: dict, hv: int, hk: int, dk: int, dv: int, cap: int,
                 mode: str = "snapshot", literal: bool | None = None):
        assert mode in ("snapshot", "replay")
        assert hv % hk == 0
        self.hv, self.hk, self.dk, self.dv, self.cap = hv, hk, dk, dv, cap
        self.group = hv // hk
        self.mode = mode
        self.literal = (dk <= 32) if literal is None else literal
        st = np.asarray(init["state"])
        self.num_slots = st.shape[0]
        # checkpoint in math orientation: S[s, h] = H[s, h]^T
        self.S_ckpt = np.swapaxes(st.astype(np.float64), -1, -2).copy()
        self.ring_q = np.array(init["ring_q"]) if init.get("ring_q") is not None else None
        self.ring_k = np.array(init["ring_k"])
        self.ring_v = np.array(init["ring_v"])
        self.ring_alpha = np.array(init["ring_alpha"])
        self.ring_beta = np.array(init["ring_beta"])
        self.head = np.array(init["head"], dtype=np.int64)
        self.len = np.array(init["len"], dtype=np.int64)
        self.err = 0
        self.snap = {}
        if mode == "snapshot":
            self.S_live = self.S_ckpt.copy()
            for s in range(self.num_slots):
                self.S_live[s] = self._advance_ring(self.S_ckpt[s], s, 0, int(self.len[s]))

    # -- helpers ------------------------------------------------------------
    def _step(self, S, k, v, a, b):
        f = gdn_step_literal if self.literal else gdn_step
        return f(S, k, v, a, b)

    def _kv_heads(self, kh_vec):
        """Per-key-head vectors [HK, d] -> per-value-head vectors [HV, d]."""
        return np.repeat(kh_vec, self.group, axis=0)

    def _ring_record(self, s, pos):
        k = self._kv_heads(to_f64(self.ring_k[s, :, pos]))
        v = to_f64(self.ring_v[s, :, pos])
        a = to_f64(self.ring_alpha[s, :, pos])
        b = to_f64(self.ring_beta[s, :, pos])
        return k, v, a, b

    def _advance_ring(self, S, s, start, count):
        """Advance S [HV, dv, dk] over ring tokens head+start .. head+start+count-1."""
        for t in range(count):
            pos = (int(self.head[s]) + start + t) % self.cap
            S = self._step(S, *self._ring_record(s, pos))
        return S

    def _slot_ok(self, s) -> bool:
        if s < 0 or s >= self.num_slots:
            self.err |= ERR_SLOT
            return False
        if not (0 <= self.head[s] < self.cap and 0 <= self.len[s] <= self.cap):
            self.err |= ERR_POINTER
            return False
        return True

    # -- the three calls ------------------------------------------------------
    def verify(self, slot_idx, q, k, v, alpha, beta, draft_lens=None) -> np.ndarray:
        """Outputs of the draft block [R, D, HV, dv] (NaN rows for skipped requests
        and for rows past a request's draft length).

        out[i, j, h] = S q_j for the state after draft token j of request i,
        starting from the state after the committed tokens. The draft is
        appended to the ring; checkpoint, head and len are not changed."""
        slot_idx = np.asarray(slot_idx)
        R, Dmax = np.asarray(alpha).shape[:2]
        Ds = per_request_lengths(draft_lens, R, Dmax)
        assert len(set(int(s) for s in slot_idx)) == len(slot_idx), "slots must be unique"
        out = np.full((R, Dmax, self.hv, self.dv), np.nan)
        for i in range(R):
            s = int(slot_idx[i])
            if not self._slot_ok(s):
                continue
            D = int(Ds[i])
            if D < 0 or D > Dmax:
                self.err |= ERR_DRAFT
                continue
            n = int(self.len[s])
            if n + D > self.cap:
                self.err |= ERR_CAPACITY
                continue
            # tentative append of the whole draft behind the committed window
            for j in range(D):
                pos = (int(self.head[s]) + n + j) % self.cap
                if self.ring_q is not None:
                    self.ring_q[s, :, pos] = q[i, j]
                self.ring_k[s, :, pos] = k[i, j]
                self.ring_v[s, :, pos] = v[i, j]
                self.ring_alpha[s, :, pos] = alpha[i, j]
                self.ring_beta[s, :, pos] = beta[i, j]
            if self.mode == "snapshot":
                if s in self.snap:                      # abandoned earlier speculation
                    self.S_live[s] = self.snap.pop(s)
                self.snap[s] = self.S_live[s].copy()    # explicit full-state snapshot
                S = self.S_live[s]
            else:
                S = self._advance_ring(self.S_ckpt[s], s, 0, n)
            for j in range(D):
                kj = self._kv_heads(to_f64(k[i, j]))
                qj = self._kv_heads(to_f64(q[i, j]))
                S = self._step(S, kj, to_f64(v[i, j]), to_f64(alpha[i, j]), to_f64(beta[i, j]))
                out[i, j] = gdn_output(S, qj)
            if self.mode == "snapshot":
                self.S_live[s] = S                      # live state moved speculatively
        return out

    def rollback(self, slot_idx, draft_len: int, num_accepted, draft_lens=None) -> None:
        """Commit the first a tokens of the last appended draft: len += a, with
        0 <= a <= the request's draft length."""
        slot_idx = np.asarray(slot_idx)
        Ds = per_request_lengths(draft_lens, len(slot_idx), draft_len)
        for s, a, D in zip(slot_idx, np.asarray(num_accepted), Ds):
            s, a, D = int(s), int(a), int(D)
            if not self._slot_ok(s):
                continue
            if D < 0 or D > draft_len:
                self.err |= ERR_DRAFT
                continue
            if a < 0 or a > D:
                self.err |= ERR_ACCEPT
                continue
            n = int(self.len[s])
            if n + a > self.cap:
                self.err |= ERR_CAPACITY
                continue
            if self.mode == "snapshot":
                if s in self.snap:                      # explicit full-state restore
                    self.S_live[s] = self.snap.pop(s)
                self.S_live[s] = self._advance_ring(self.S_live[s], s, n, a)
            self.len[s] = n + a

    def flush(self, slot_idx, min_len: int) -> None:
        """Fold all committed tokens of due slots into the checkpoint."""
        for s in np.asarray(slot_idx):
            s = int(s)
            if not self._slot_ok(s):
                continue
            n = int(self.len[s])
            if n < max(int(min_len), 1):
                continue
            if self.mode == "snapshot":
                if s in self.snap:
                    self.S_live[s] = self.snap.pop(s)
                self.S_ckpt[s] = self.S_live[s].copy()
            else:
                self.S_ckpt[s] = self._advance_ring(self.S_ckpt[s], s, 0, n)
            self.head[s] = (int(self.head[s]) + n) % self.cap
            self.len[s] = 0

    def verify_flush(self, slot_idx, min_len: int, q, k, v, alpha, beta,
                     draft_lens=None) -> np.ndarray:
        """The periodic flush folded into the next verify: flush(min_len), then
        verify from the resulting checkpoint, pointers and ring. A slot that is
        not due and has len + D > C is skipped by verify (CAPACITY) after a flush
        that did not touch it, so the call writes nothing for it. A request whose
        draft length is outside [0, D_max] is skipped entirely (DRAFT, no flush)."""
        slot_idx = np.asarray(slot_idx)
        R, Dmax = np.asarray(alpha).shape[:2]
        Ds = per_request_lengths(draft_lens, R, Dmax)
        # checks in the order slot, pointers, draft length: a request with a bad
        # length is flushed by nobody; verify then flags it (DRAFT) and skips it
        slot_ok = np.array([0 <= int(s) < self.num_slots
                            and 0 <= self.head[int(s)] < self.cap
                            and 0 <= self.len[int(s)] <= self.cap for s in slot_idx], dtype=bool)
        bad = slot_ok & ((Ds < 0) | (Ds > Dmax))
        self.flush(slot_idx[~bad], min_len)
        return self.verify(slot_idx, q, k, v, alpha, beta, draft_lens=Ds)

    # -- views in the library's layouts -----------------------------------------
    def state_abi(self) -> np.ndarray:
        """Checkpoint as [slots][HV][d_k][d_v] (H = S^T), float64."""
        return np.swapaxes(self.S_ckpt, -1, -2).copy()

    def committed_stream(self, s: int):
        """The committed ring records of slot s in order (for checks)."""
        return [(int(self.head[s]) + t) % self.cap for t in range(int(self.len[s]))]
