"""The causal convolution before the recurrence, with its input ring, on torch
device tensors. Marshalling only: shapes, dtypes, devices and contiguity are
checked here and the work runs in libgdnreplay.so (gdn_causal_conv_update)."""
from __future__ import annotations

import torch

from . import binding
from .cache import ReplayCache, _need, _stream_handle


class ConvRing:
    """The input ring [num_slots][C][channels] bf16 of one layer's convolution; it
    shares head / len with the layer's ReplayCache."""

    def __init__(self, cache: ReplayCache, channels: int, width: int):
        self.cache, self.channels, self.width = cache, int(channels), int(width)
        self.ring = torch.zeros((cache.num_slots, cache.cap, channels), dtype=torch.bfloat16,
                                device=cache.device)

    def update(self, slot_idx, x, weight, bias=None, y=None, stream=None, num_accepted=None,
               prev_draft=0, prev_draft_lens=None) -> torch.Tensor:
        """y = silu(causal depthwise conv) of the draft x [R, D, channels] (bf16);
        appends x to the ring (call before the step's verify). With the one-call
        step, whose rollback of the previous draft comes after this call, pass
        that step's num_accepted [R] (and prev_draft / prev_draft_lens [R])."""
        R, D = slot_idx.shape[0], x.shape[1] if x.dim() == 3 else 0
        dev = self.cache.device
        _need(slot_idx, "slot_idx", torch.int32, (R,), dev)
        _need(x, "x", torch.bfloat16, (R, D, self.channels), dev)
        _need(weight, "weight", torch.float32, (self.channels, self.width), dev)
        if bias is not None:
            _need(bias, "bias", torch.float32, (self.channels,), dev)
        if y is None:
            y = torch.empty_like(x)
        _need(y, "y", torch.bfloat16, (R, D, self.channels), dev)
        acc = plens = None
        if num_accepted is not None:
            _need(num_accepted, "num_accepted", torch.int32, (R,), dev)
            acc = num_accepted.data_ptr()
            if prev_draft_lens is not None:
                _need(prev_draft_lens, "prev_draft_lens", torch.int32, (R,), dev)
                plens = prev_draft_lens.data_ptr()
        binding.causal_conv_update(self.cache.struct(), self.ring.data_ptr(), self.channels,
                                   self.width, R, slot_idx.data_ptr(), D, x.data_ptr(),
                                   weight.data_ptr(), None if bias is None else bias.data_ptr(),
                                   y.data_ptr(), _stream_handle(stream), acc, plens,
                                   int(prev_draft))
        return y
