"""MI355X-native fused RNN-T loss (forward and backward) on packed logits.

The compute path is librnnt (``csrc/``: C ABI in ``include/rnnt.h``, gfx950
HIP kernels); this package binds it for PyTorch tensors.
"""
from .loss import (RNNTLoss, device_flags, rnnt_loss, rnnt_loss_fused, rnnt_loss_multiblank,  # noqa: F401
                   rnnt_multiblank_fused, workspace_bytes)
from . import _lib  # noqa: F401

__all__ = ["rnnt_loss", "RNNTLoss", "rnnt_loss_fused", "workspace_bytes", "device_flags", "rnnt_loss_multiblank",
           "rnnt_multiblank_fused"]
