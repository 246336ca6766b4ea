"""Model weights on disk and the linear() dispatch between W4A16 and fp32.

The pages' engine loads each quantized weight from a pair of raw files, a
`.qw` of packed int32 words and a `.sc` of fp32 group scales, into maps kept
beside the fp32 weights and a group-size field; its linear() runs a weight
through the W4A16 kernel when the weight has a quantized counterpart and
through the existing fp32 GEMM otherwise ("The Quiet Commit: How a Single
Documentation Edit Marks the Completion of a Major Engineering Milestone",
section "The INT4 Milestone: From FP32 to Production-Ready Quantization").
The presence of the `.qw` file is the whole test ("The Silence of Success: A
Single Line That Speaks Volumes", section "Assumptions Embedded in the Code"),
so a `.qw` without its `.sc`, or files of the wrong size, are errors rather
than a silent fall back to fp32.

Files of a bundle directory, per weight name (shapes come from the caller:
the files carry none):
  <name>.qw, <name>.sc   a quantized weight, read by w4a16_load_quantized
  <name>.f32             a plain weight W[N][K]: raw little-endian fp32,
                         row-major (the pages keep these in the engine's
                         fp32 format, which they do not describe; this raw
                         form is the reading taken here)
A name with both a `.qw` and a `.f32` file is quantized.
"""

from __future__ import annotations

import os
from typing import Mapping

import numpy as np

from .binding import GROUP, w4a16_gemm, w4a16_load_quantized, w4a16_save_quantized


class WeightBundle:
    """Device-resident weights by name, int4 (qweight, scales) or fp32."""

    def __init__(self, device="cuda"):
        import torch
        self.device = torch.device(device)
        self.group = GROUP
        self.qweight: dict[str, object] = {}
        self.scales: dict[str, object] = {}
        self.fp32: dict[str, object] = {}
        self.calls = {"int4": 0, "fp32": 0}

    # ---------------------------------------------------------------- loading
    @classmethod
    def from_directory(cls, directory, shapes: Mapping[str, tuple[int, int]], device="cuda"):
        """Load every weight named in `shapes` ({name: (N, K)}) from `directory`."""
        import torch
        b = cls(device)
        for name, (N, K) in shapes.items():
            base = os.path.join(directory, name)
            if os.path.exists(base + ".qw"):
                qw, sc = w4a16_load_quantized(base + ".qw", base + ".sc", N, K)
                b.add_quantized(name, torch.from_numpy(qw), torch.from_numpy(sc))
            elif os.path.exists(base + ".f32"):
                b.add_fp32(name, torch.from_numpy(_read_f32(base + ".f32", N, K)))
            else:
                raise FileNotFoundError(f"weight {name!r}: neither {base}.qw nor {base}.f32")
        return b

    def add_quantized(self, name: str, qweight, scales) -> None:
        """Register a quantized weight (qweight int32 [N][K/8], scales fp32 [N][K/32])."""
        import torch
        if qweight.dtype != torch.int32 or scales.dtype != torch.float32 or qweight.dim() != 2:
            raise TypeError(f"{name}: qweight must be 2-D int32 and scales float32")
        N, K = qweight.shape[0], 8 * qweight.shape[1]
        if K % GROUP or tuple(scales.shape) != (N, K // GROUP):
            raise ValueError(f"{name}: scales shape {tuple(scales.shape)} != {(N, K // GROUP)}")
        self.fp32.pop(name, None)
        self.qweight[name] = qweight.to(self.device).contiguous()
        self.scales[name] = scales.to(self.device).contiguous()

    def add_fp32(self, name: str, W) -> None:
        """Register a plain fp32 weight W[N][K] (ignored for dispatch if `name` is quantized)."""
        import torch
        if W.dtype != torch.float32 or W.dim() != 2:
            raise TypeError(f"{name}: W must be a 2-D float32 tensor")
        self.fp32[name] = W.to(self.device).contiguous()

    def save(self, directory) -> None:
        """Write every weight as `.qw`/`.sc` (quantized) or `.f32` (plain) files."""
        os.makedirs(directory, exist_ok=True)
        for name in self.qweight:
            base = os.path.join(directory, name)
            w4a16_save_quantized(base + ".qw", base + ".sc", self.qweight[name].cpu().numpy(),
                                 self.scales[name].cpu().numpy())
        for name, W in self.fp32.items():
            if name not in self.qweight:
                W.cpu().numpy().astype("<f4").tofile(os.path.join(directory, name + ".f32"))

    # --------------------------------------------------------------- dispatch
    def is_int4(self, name: str) -> bool:
        """True when `name` has a quantized counterpart (the pages' `.qw` test)."""
        if name in self.qweight:
            return True
        if name in self.fp32:
            return False
        raise KeyError(f"no weight named {name!r}")

    def shape(self, name: str) -> tuple[int, int]:
        """(N, K) of the weight."""
        if self.is_int4(name):
            return self.qweight[name].shape[0], 8 * self.qweight[name].shape[1]
        return tuple(self.fp32[name].shape)

    def linear(self, name: str, x, out=None):
        """y[..., N] = x[..., K] . W^T: W4A16 kernel for a quantized weight, the
        fp32 GEMM (torch on the device, full fp32) otherwise.  x must be fp32 on
        the bundle's device; no host fallback exists."""
        import torch
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise TypeError("x must be a tensor on a ROCm device")
        if x.dtype != torch.float32:
            raise TypeError("x must be float32")
        N, K = self.shape(name)
        if x.shape[-1] != K:
            raise ValueError(f"{name}: x has {x.shape[-1]} features, the weight takes {K}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, K).contiguous()
        y2 = None if out is None else out.view(-1, N)
        if self.is_int4(name):
            self.calls["int4"] += 1
            y2 = w4a16_gemm(x2, self.qweight[name], self.scales[name], y2)
        else:
            self.calls["fp32"] += 1
            W = self.fp32[name]
            if y2 is None:
                y2 = torch.matmul(x2, W.t())
            else:
                torch.matmul(x2, W.t(), out=y2)
        return y2.view(*lead, N)


def _read_f32(path: str, N: int, K: int) -> np.ndarray:
    """A raw little-endian fp32 [N][K] file, size checked."""
    need = 4 * N * K
    size = os.path.getsize(path)
    if size != need:
        raise ValueError(f"{path}: {size} bytes, expected {need} for a {N} x {K} fp32 weight")
    return np.fromfile(path, dtype="<f4").astype(np.float32).reshape(N, K)
