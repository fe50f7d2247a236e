"""Gated RMSNorm + FP8 (OCP E4M3) quantisation of the GDN output, on torch device
tensors. Marshalling only: shapes, dtypes, devices and contiguity are checked
here and the work runs in libgdnreplay.so (gdn_gated_rmsnorm_fp8)."""
from __future__ import annotations

import torch

from . import binding
from .cache import _need, _stream_handle


def gated_rmsnorm_fp8(o: torch.Tensor, z: torch.Tensor, weight: torch.Tensor, eps: float,
                      q: torch.Tensor | None = None, scale: torch.Tensor | None = None,
                      stream=None):
    """o [..., H, d_v] fp32, z [..., H, d_v] bf16, weight [d_v] fp32 -> (q uint8 codes
    [..., H, d_v], scale fp32 [..., H]); a group dequantises as code value * scale."""
    if o.dim() < 2:
        raise ValueError("o must be [..., heads, d_v]")
    H, dv = o.shape[-2], o.shape[-1]
    rows = o.numel() // (H * dv) if o.numel() else 0
    dev = o.device
    _need(o, "o", torch.float32, o.shape, dev)
    _need(z, "z", torch.bfloat16, o.shape, dev)
    _need(weight, "weight", torch.float32, (dv,), dev)
    if q is None:
        q = torch.empty(o.shape, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(o.shape[:-1], dtype=torch.float32, device=dev)
    _need(q, "q", torch.uint8, o.shape, dev)
    _need(scale, "scale", torch.float32, o.shape[:-1], dev)
    binding.gated_rmsnorm_fp8(rows, H, dv, o.data_ptr(), z.data_ptr(), weight.data_ptr(),
                              float(eps), q.data_ptr(), scale.data_ptr(), _stream_handle(stream))
    return q, scale
