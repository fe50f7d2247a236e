"""One layer's replay cache as torch device tensors, and the calls on it.

Marshalling only: shapes, dtypes, devices and contiguity are checked here, the
pointers are handed to libgdnreplay.so, and every step runs in its HIP kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding
from .synth import BF16, F32

_TORCH_IN = {BF16: torch.bfloat16, F32: torch.float32}


def _from_np(x: np.ndarray, device) -> torch.Tensor:
    if x.dtype == np.uint16:                       # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def _to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy (bf16 as uint16 bits, fp32, int32) -> device tensor with the same bits."""
    return _from_np(x, device)


def to_host(t: torch.Tensor) -> np.ndarray:
    return _to_np(t)


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class ReplayCache:
    """Device tensors of one GDN layer's replay cache (layouts of include/gdn_replay.h)."""

    def __init__(self, num_slots, hv, hk, dk, dv, cap, in_dtype=BF16, device="cuda",
                 with_q=True):
        self.num_slots, self.hv, self.hk, self.dk, self.dv, self.cap = (
            num_slots, hv, hk, dk, dv, cap)
        self.in_dtype = in_dtype
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        tin = _TORCH_IN[in_dtype]
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=self.device)
        self.state = z((num_slots, hv, dk, dv), torch.float32)
        self.ring_q = z((num_slots, hk, cap, dk), tin) if with_q else None
        self.ring_k = z((num_slots, hk, cap, dk), tin)
        self.ring_v = z((num_slots, hv, cap, dv), tin)
        self.ring_alpha = z((num_slots, hv, cap), torch.float32)
        self.ring_beta = z((num_slots, hv, cap), torch.float32)
        self.head = z((num_slots,), torch.int32)
        self.len = z((num_slots,), torch.int32)
        # slot counters, then the per-(slot, key head) and grid counters of verify_flush
        self.sync = z((binding.sync_entries(num_slots, hk),), torch.int32)
        self.err = z((1,), torch.int32)
        self._struct = None

    @classmethod
    def from_numpy(cls, init: dict, hv, hk, dk, dv, cap, in_dtype, device="cuda",
                   with_q=True) -> "ReplayCache":
        c = cls(init["state"].shape[0], hv, hk, dk, dv, cap, in_dtype, device, with_q)
        c.load(init)
        return c

    def load(self, init: dict) -> None:
        for name in ("state", "ring_k", "ring_v", "ring_alpha", "ring_beta", "head", "len"):
            getattr(self, name).copy_(_from_np(init[name], self.device))
        if self.ring_q is not None and init.get("ring_q") is not None:
            self.ring_q.copy_(_from_np(init["ring_q"], self.device))
        self._struct = None

    def to_numpy(self) -> dict:
        out = {n: _to_np(getattr(self, n)) for n in
               ("state", "ring_k", "ring_v", "ring_alpha", "ring_beta", "head", "len", "sync", "err")}
        out["ring_q"] = None if self.ring_q is None else _to_np(self.ring_q)
        return out

    def struct(self) -> binding.GdnReplayCache:
        if self._struct is None:
            p = lambda t: None if t is None else t.data_ptr()
            self._struct = binding.GdnReplayCache(
                self.num_slots, self.hv, self.hk, self.dk, self.dv, self.cap,
                binding.GDN_BF16 if self.in_dtype == BF16 else binding.GDN_F32,
                self.sync.numel(),
                p(self.state), p(self.ring_q), p(self.ring_k), p(self.ring_v),
                p(self.ring_alpha), p(self.ring_beta), p(self.head), p(self.len),
                p(self.sync), p(self.err))
        return self._struct

    # -- the calls ---------------------------------------------------------------
    def _draft_args(self, slot_idx, q, k, v, alpha, beta, out):
        R = slot_idx.shape[0]
        D = alpha.shape[1] if alpha.dim() == 3 else 0
        tin = _TORCH_IN[self.in_dtype]
        dev = self.device
        _need(slot_idx, "slot_idx", torch.int32, (R,), dev)
        _need(q, "q", tin, (R, D, self.hk, self.dk), dev)
        _need(k, "k", tin, (R, D, self.hk, self.dk), dev)
        _need(v, "v", tin, (R, D, self.hv, self.dv), dev)
        _need(alpha, "alpha", torch.float32, (R, D, self.hv), dev)
        _need(beta, "beta", torch.float32, (R, D, self.hv), dev)
        if out is None:
            out = torch.empty((R, D, self.hv, self.dv), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, (R, D, self.hv, self.dv), dev)
        return R, D, out

    def _lens(self, draft_lens, R):
        if draft_lens is not None:
            _need(draft_lens, "draft_lens", torch.int32, (R,), self.device)
        return draft_lens

    def verify(self, slot_idx, q, k, v, alpha, beta, out=None, stream=None,
               draft_lens=None) -> torch.Tensor:
        """Outputs of the draft block. draft_lens ([R] int32, device): per-request
        draft lengths in [0, D] (the *_varlen entry point); rows past a request's
        length are left untouched."""
        R, D, out = self._draft_args(slot_idx, q, k, v, alpha, beta, out)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
                out.data_ptr(), _stream_handle(stream))
        if self._lens(draft_lens, R) is None:
            binding.verify(self.struct(), R, slot_idx.data_ptr(), D, *args)
        else:
            binding.verify_varlen(self.struct(), R, slot_idx.data_ptr(), draft_lens.data_ptr(), D,
                                  *args)
        return out

    def verify_flush(self, slot_idx, min_len: int, q, k, v, alpha, beta, out=None,
                     stream=None, draft_lens=None) -> torch.Tensor:
        """flush(min_len) then verify, in one pass (gdn_replay_verify_flush)."""
        R, D, out = self._draft_args(slot_idx, q, k, v, alpha, beta, out)
        args = (int(min_len), q.data_ptr(), k.data_ptr(), v.data_ptr(), alpha.data_ptr(),
                beta.data_ptr(), out.data_ptr(), _stream_handle(stream))
        if self._lens(draft_lens, R) is None:
            binding.verify_flush(self.struct(), R, slot_idx.data_ptr(), D, *args)
        else:
            binding.verify_flush_varlen(self.struct(), R, slot_idx.data_ptr(),
                                        draft_lens.data_ptr(), D, *args)
        return out

    def rollback_verify_flush(self, slot_idx, num_accepted, prev_draft: int, min_len: int, q, k,
                              v, alpha, beta, out=None, stream=None, prev_draft_lens=None,
                              draft_lens=None) -> torch.Tensor:
        """rollback(prev_draft, num_accepted) then verify_flush(min_len) of this
        step's draft, in one call (gdn_replay_rollback_verify_flush)."""
        R, D, out = self._draft_args(slot_idx, q, k, v, alpha, beta, out)
        _need(num_accepted, "num_accepted", torch.int32, (R,), self.device)
        lens = self._lens(draft_lens, R)
        plens = self._lens(prev_draft_lens, R)
        binding.rollback_verify_flush(
            self.struct(), R, slot_idx.data_ptr(), num_accepted.data_ptr(),
            None if plens is None else plens.data_ptr(), int(prev_draft),
            None if lens is None else lens.data_ptr(), D, int(min_len), q.data_ptr(), k.data_ptr(),
            v.data_ptr(), alpha.data_ptr(), beta.data_ptr(), out.data_ptr(),
            _stream_handle(stream))
        return out

    def step_norm_fp8(self, slot_idx, num_accepted, prev_draft: int, min_len: int, q, k, v,
                      alpha, beta, z, weight, eps: float, out=None, codes=None, scale=None,
                      write_out=True, stream=None, prev_draft_lens=None, draft_lens=None):
        """rollback_verify_flush with the gated RMSNorm + FP8 of its outputs in the
        same kernel (gdn_replay_step_norm_fp8). z [R, D, HV, dv] bf16 gate, weight
        [dv] fp32. Returns (out or None when write_out is False, codes uint8
        [R, D, HV, dv], scale fp32 [R, D, HV])."""
        R = slot_idx.shape[0]
        D = alpha.shape[1] if alpha.dim() == 3 else 0
        dev = self.device
        if write_out:
            R, D, out = self._draft_args(slot_idx, q, k, v, alpha, beta, out)
        else:
            tin = _TORCH_IN[self.in_dtype]
            _need(slot_idx, "slot_idx", torch.int32, (R,), dev)
            for t, name, dt, shape in ((q, "q", tin, (R, D, self.hk, self.dk)),
                                       (k, "k", tin, (R, D, self.hk, self.dk)),
                                       (v, "v", tin, (R, D, self.hv, self.dv)),
                                       (alpha, "alpha", torch.float32, (R, D, self.hv)),
                                       (beta, "beta", torch.float32, (R, D, self.hv))):
                _need(t, name, dt, shape, dev)
            out = None
        _need(num_accepted, "num_accepted", torch.int32, (R,), dev)
        _need(z, "z", torch.bfloat16, (R, D, self.hv, self.dv), dev)
        _need(weight, "weight", torch.float32, (self.dv,), dev)
        if codes is None:
            codes = torch.empty((R, D, self.hv, self.dv), dtype=torch.uint8, device=dev)
        if scale is None:
            scale = torch.empty((R, D, self.hv), dtype=torch.float32, device=dev)
        _need(codes, "codes", torch.uint8, (R, D, self.hv, self.dv), dev)
        _need(scale, "scale", torch.float32, (R, D, self.hv), dev)
        lens = self._lens(draft_lens, R)
        plens = self._lens(prev_draft_lens, R)
        norm = binding.GdnNormFp8(z.data_ptr(), weight.data_ptr(), float(eps), codes.data_ptr(),
                                  scale.data_ptr())
        binding.step_norm_fp8(
            self.struct(), R, slot_idx.data_ptr(), num_accepted.data_ptr(),
            None if plens is None else plens.data_ptr(), int(prev_draft),
            None if lens is None else lens.data_ptr(), D, int(min_len), q.data_ptr(), k.data_ptr(),
            v.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
            None if out is None else out.data_ptr(), norm, _stream_handle(stream))
        return out, codes, scale

    def rollback(self, slot_idx, draft_len: int, num_accepted, stream=None,
                 draft_lens=None) -> None:
        R = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (R,), self.device)
        _need(num_accepted, "num_accepted", torch.int32, (R,), self.device)
        if self._lens(draft_lens, R) is None:
            binding.rollback(self.struct(), R, slot_idx.data_ptr(), int(draft_len),
                             num_accepted.data_ptr(), _stream_handle(stream))
        else:
            binding.rollback_varlen(self.struct(), R, slot_idx.data_ptr(), draft_lens.data_ptr(),
                                    int(draft_len), num_accepted.data_ptr(),
                                    _stream_handle(stream))

    def flush(self, slot_idx, min_len: int, stream=None) -> None:
        R = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (R,), self.device)
        binding.flush(self.struct(), R, slot_idx.data_ptr(), int(min_len), _stream_handle(stream))
