"""Seeded synthetic workloads (shapes and random inputs only).

This module draws the random inputs that both the HIP path and the oracle
consume.  It contains none of the attention arithmetic: it only knows tensor
shapes, dtypes and how to draw numbers.

The shapes stand in for the workloads on the pages (no trained weights or
images are available): Swin window attention ["Training and inference
acceleration for large vision models", section 1], SAM image-encoder
attention with decomposed relative position ["Accelerating Generative AI with
PyTorch: Segment Anything, Fast", sections "Bfloat16" and "SDPA"], and the
Stable Diffusion v1.5 UNet self/cross attention ["Accelerated Diffusers with
PyTorch 2.0", section "Stable Diffusion benchmark"].

Recipe: every tensor is drawn with ``numpy.random.Generator(PCG64(
SeedSequence([16, cfg_id, tensor_id])))`` as float32 standard normals
(tensor_id q=0, k=1, v=2, table/Rh=3, Rw=4); Q, K, V ~ N(0, 1); table, Rh, Rw
~ N(0, 0.02^2).  Values are then rounded to the device dtype with torch on
the CPU (round to nearest even).  An optional ``seed`` offsets the sequence so
tests can draw independent cases.

Workloads with 8-bit inputs (``qkv="e4m3"``) draw q, k and v the same way
and store each as E4M3 codes with one scale per tensor, the scale being the
tensor's largest magnitude / 448 (the largest finite E4M3 value): torch
divides by the scale and rounds to E4M3 (nearest even) on the CPU.  Their
tables and output use the compute dtype.  This is input preparation, as a
quantizing producer would do it; the attention consumes the codes and scales.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    cfg_id: int
    dtype: str
    B: int                       # batch items as the kernel sees them (windows included)
    H: int
    Nq: int
    Nk: int
    d: int
    bias: str = "none"           # none | table | relpos | additive
    grid: Optional[tuple] = None
    kgrid: Optional[tuple] = None    # relpos: key grid when it differs from grid
    mask: str = "none"           # none | shift | additive
    layout: str = "batched"      # batched | image
    images: Optional[int] = None
    window: Optional[tuple] = None   # (img_h, img_w, win_h, win_w, shift_h, shift_w)
    note: str = ""
    qkv: str = "same"            # same (q, k, v in dtype) | e4m3 (8-bit codes + scales)

    @property
    def q_shape(self):
        if self.layout == "image":
            ih, iw = self.window[0], self.window[1]
            return (self.images, self.H, ih * iw, self.d)
        return (self.B, self.H, self.Nq, self.d)

    @property
    def kv_shape(self):
        if self.layout == "image":
            return self.q_shape
        return (self.B, self.H, self.Nk, self.d)

    @property
    def flops(self) -> int:
        """4*B*H*Nq*Nk*d (two contractions of 2*Nq*Nk*d each)."""
        return 4 * self.B * self.H * self.Nq * self.Nk * self.d

    def bytes_per_elem(self) -> int:
        return {F32: 4, F16: 2, BF16: 2}[self.dtype]

    def input_bytes_per_elem(self) -> int:
        """Bytes of one q, k or v element (1 for 8-bit codes)."""
        return 1 if self.qkv == "e4m3" else self.bytes_per_elem()

    @property
    def algorithmic_bytes(self) -> int:
        """Q + K + V read once, O written once, plus the bias tables."""
        e = self.bytes_per_elem()
        if self.qkv == "e4m3":
            n_q = int(np.prod(self.q_shape))
            n_kv = int(np.prod(self.kv_shape))
            return 2 * n_kv + n_q + n_q * e + self.algorithmic_bytes_tables()
        qo = 2 * int(np.prod(self.q_shape))
        kv = 2 * int(np.prod(self.kv_shape))
        return (qo + kv) * e + self.algorithmic_bytes_tables()

    def algorithmic_bytes_tables(self) -> int:
        """Bytes of the bias tables (read once)."""
        e = self.bytes_per_elem()
        tables = 0
        if self.bias == "table":
            gh, gw = self.grid
            tables = (2 * gh - 1) * (2 * gw - 1) * self.H
        elif self.bias == "relpos":
            gh, gw = self.grid
            tables = (2 * gh - 1 + 2 * gw - 1) * self.d
        return tables * e


WORKLOADS = {
    "C1": Workload("C1", "swin_window_tiny_f32", 1, F32, B=4, H=3, Nq=49, Nk=49, d=32,
                   bias="table", grid=(7, 7),
                   note="4 windows of 7x7 tokens, 3 heads, d=32, table bias"),
    "C2": Workload("C2", "swin_t_stage1_shifted_f16", 2, F16, B=8 * 64, H=3, Nq=49, Nk=49,
                   d=32, bias="table", grid=(7, 7), mask="shift", layout="image",
                   images=8, window=(56, 56, 7, 7, 3, 3),
                   note="8 images of 56x56 tokens, 7x7 windows, cyclic shift 3"),
    "C3": Workload("C3", "sam_b_windowed_bf16", 3, BF16, B=8 * 25, H=12, Nq=196, Nk=196,
                   d=64, bias="relpos", grid=(14, 14),
                   note="SAM ViT-B windowed: 64x64 grid padded to 70x70, 25 windows of 14x14"),
    "C3i": Workload("C3i", "sam_b_windowed_image_bf16", 33, BF16, B=8 * 25, H=12, Nq=196, Nk=196,
                    d=64, bias="relpos", grid=(14, 14), layout="image", images=8,
                    window=(64, 64, 14, 14, 0, 0),
                    note="SAM ViT-B windowed from the 64x64 token image: zero padding to 70x70 and "
                         "the 25 windows of 14x14 folded into the addressing"),
    "C4": Workload("C4", "sam_b_global_bf16", 4, BF16, B=8, H=12, Nq=4096, Nk=4096, d=64,
                   bias="relpos", grid=(64, 64), note="SAM ViT-B global attention, 64x64 grid"),
    "C4h": Workload("C4h", "sam_h_global_bf16", 44, BF16, B=8, H=16, Nq=4096, Nk=4096, d=80,
                    bias="relpos", grid=(64, 64), note="SAM ViT-H global attention"),
    "C5s": Workload("C5s", "sd15_unet_self_f16", 5, F16, B=16, H=8, Nq=4096, Nk=4096, d=40,
                    note="SD 1.5 UNet self-attention at 64x64 latent, CFG batch 16"),
    "C5x": Workload("C5x", "sd15_unet_cross_f16", 55, F16, B=16, H=8, Nq=4096, Nk=77, d=40,
                    note="SD 1.5 UNet cross-attention, 77 context tokens"),
    # 8-bit inputs (E4M3 codes, one scale per tensor), f16 compute and output.
    "C2f8": Workload("C2f8", "swin_t_stage1_shifted_e4m3_f16", 62, F16, B=8 * 64, H=3, Nq=49,
                     Nk=49, d=32, bias="table", grid=(7, 7), mask="shift", layout="image",
                     images=8, window=(56, 56, 7, 7, 3, 3), qkv="e4m3",
                     note="the Swin-T stage-1 workload with q, k, v as E4M3 codes"),
    "C5sf8": Workload("C5sf8", "sd15_unet_self_e4m3_f16", 65, F16, B=16, H=8, Nq=4096, Nk=4096,
                      d=40, qkv="e4m3", note="SD 1.5 UNet self-attention, q, k, v as E4M3 codes"),
    "C5xf8": Workload("C5xf8", "sd15_unet_cross_e4m3_f16", 66, F16, B=16, H=8, Nq=4096, Nk=77,
                      d=40, qkv="e4m3", note="SD 1.5 UNet cross-attention, q, k, v as E4M3 codes"),
}


def _rng(cfg_id: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    parts = [16, cfg_id, tensor_id] + ([seed] if seed else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(parts)))


def normal(shape, cfg_id: int, tensor_id: int, std: float = 1.0, seed: int = 0) -> np.ndarray:
    """float32 N(0, std^2) draws of the given shape."""
    x = _rng(cfg_id, tensor_id, seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_dtype(x: np.ndarray, dtype: str):
    """Round float32 values to the device dtype (torch CPU, round to nearest even)."""
    import torch

    tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(tdt)


def to_e4m3(x: np.ndarray):
    """float32 values -> (E4M3 codes as a uint8 tensor, float32 scale): the
    scale is max|x| / 448 (1 for an all-zero tensor), and x / scale is
    rounded to E4M3 by torch on the CPU (nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = float(t.abs().max()) if t.numel() else 0.0
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    codes = (t / torch.tensor(scale)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), float(scale)


def make_inputs(w: Workload, seed: int = 0, std_qkv: float = 1.0, std_table: float = 0.02) -> dict:
    """Draw the inputs of workload ``w`` as torch CPU tensors in its dtype.

    Returns q, k, v and, depending on the bias kind, table or rh/rw.
    ``std_table`` (default 0.02, the workloads' recipe) sets the standard
    deviation of the bias tables; tests raise it so that the bias is large
    next to the tolerance.  For 8-bit inputs q, k, v are uint8 tensors of
    E4M3 codes and ``descale`` a float32 tensor of their three scales.
    """
    draws = {"q": normal(w.q_shape, w.cfg_id, 0, std_qkv, seed),
             "k": normal(w.kv_shape, w.cfg_id, 1, std_qkv, seed),
             "v": normal(w.kv_shape, w.cfg_id, 2, std_qkv, seed)}
    if w.qkv == "e4m3":
        import torch

        out, scales = {}, []
        for name in ("q", "k", "v"):
            out[name], s = to_e4m3(draws[name])
            scales.append(s)
        out["descale"] = torch.tensor(scales, dtype=torch.float32)
    else:
        out = {name: to_dtype(x, w.dtype) for name, x in draws.items()}
    if w.bias == "table":
        gh, gw = w.grid
        out["table"] = to_dtype(normal(((2 * gh - 1) * (2 * gw - 1), w.H), w.cfg_id, 3,
                                       std_table, seed), w.dtype)
    elif w.bias == "relpos":
        gh, gw = w.grid
        kgh, kgw = w.kgrid or w.grid
        out["rh"] = to_dtype(normal((2 * max(gh, kgh) - 1, w.d), w.cfg_id, 3, std_table, seed), w.dtype)
        out["rw"] = to_dtype(normal((2 * max(gw, kgw) - 1, w.d), w.cfg_id, 4, std_table, seed), w.dtype)
    return out


def custom(dtype: str, B: int, H: int, Nq: int, Nk: int, d: int, bias: str = "none",
           grid=None, mask: str = "none", layout: str = "batched", images=None,
           window=None, cfg_id: int = 900, key: str = "custom", kgrid=None,
           qkv: str = "same") -> Workload:
    """A workload of arbitrary shape for tests (same drawing recipe)."""
    return Workload(key, key, cfg_id, dtype, B=B, H=H, Nq=Nq, Nk=Nk, d=d, bias=bias,
                    grid=grid, kgrid=kgrid, mask=mask, layout=layout, images=images,
                    window=window, qkv=qkv)


def device_args(w: Workload, t: dict) -> dict:
    """Keyword arguments of ``binding.fwd`` for workload ``w``.

    ``t`` holds the workload's tensors already on the device (see
    :func:`make_inputs`).  Only descriptors are built here.
    """
    from . import binding as B

    kw: dict = {"layout": w.layout}
    if w.bias == "table":
        kw["bias"] = B.TableBias(t["table"], w.grid)
    elif w.bias == "relpos":
        kw["bias"] = B.RelposBias(t["rh"], t["rw"], w.grid, w.kgrid)
    elif w.bias == "additive":
        kw["bias"] = B.AdditiveBias(t["bias_add"])
    win = B.Window(*w.window) if w.window is not None else None
    if w.mask == "shift":
        kw["mask"] = B.ShiftMask(win)
    elif w.mask == "additive":
        kw["mask"] = B.AdditiveMask(t["mask_add"])
    if w.layout == "image":
        kw["window"] = win
    if w.qkv == "e4m3":
        import torch

        kw["qkv_descale"] = tuple(float(x) for x in t["descale"].to("cpu"))
        kw["out_dtype"] = {F16: torch.float16, BF16: torch.bfloat16}[w.dtype]
    return kw
