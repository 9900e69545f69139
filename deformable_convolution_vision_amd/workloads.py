"""Seeded synthetic inputs for the deformable-convolution forward.

This module only draws random tensors.  It holds none of the method's arithmetic
(no sampling positions, no interpolation, no output-size formula: the output
size of each named workload is stated in the table as data, and callers pass it
in for other shapes).  Both the HIP path's tests and bench and the oracle's
tests take their inputs from here.

The named workloads stand in for ResNet-50 / Faster R-CNN backbone activations
on COCO-sized images (deformable 3x3 layers in stages c3-c5, res5 with
dilation 2) and for the single 224x224 RGB example of the torchvision
deform_conv2d tutorial (agent.csdn.net/6a744b3d10ee7a33f2973402.html, section
2.2).  No dataset is read: only shapes and value distributions are reproduced.

Draw order per workload, all in float32 on the CPU from
``torch.Generator().manual_seed(seed)``: x, weight, offset, mask, bias.  For
bf16 workloads every tensor is then rounded to bfloat16 (round to nearest
even), and the oracle reads back exactly those rounded values.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": element type of every tensor
    B: int
    Cin: int
    H: int
    W: int
    Cout: int
    K: int
    stride: int
    pad: int
    dilation: int
    Ho: int               # stated output size (data, not computed here)
    Wo: int
    offset: str           # "uniform:a" U(-a,a) | "normal:s" s*N(0,1) | "tanh:s" s*tanh(N(0,1))
                          # | "frac:n:lo:hi" an integer uniform in [-n, n] plus U(lo, hi)
    mask: str | None      # "sigmoid" = sigmoid(N(0,1)) | "ones" | None (DCNv1)
    bias: str | None      # "zeros" | "normal:s" s*N(0,1) | None
    seed: int = 0
    x: str = "normal"     # "normal" = N(0,1) | "checker:e" = (-1)^(row+col) * (1 + e*N(0,1))
    groups: int = 1       # offset groups: offset has 2*groups*K^2 channels, mask groups*K^2
    op: str = "forward"   # "forward" | "offset_mask" (the DCNv2 offset/mask convolution; Cout = 3*groups*K^2)
    weight: str = "kaiming"   # "kaiming" = Kaiming-normal | "kaiming_abs" = its absolute value

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def flops(self) -> int:
        """2*B*Cout*Ho*Wo*Cin*K^2: the multiply-adds of the contraction."""
        return 2 * self.B * self.Cout * self.Ho * self.Wo * self.Cin * self.K * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Each tensor crossing the boundary counted once, at its element size."""
        es = 4 if self.dtype == "f32" else 2
        KK = self.K * self.K
        if self.op == "offset_mask":   # x, weight, bias in; offsets and mask (Cout channels) out
            return es * (self.B * self.Cin * self.H * self.W + self.Cout * self.Cin * KK
                         + (self.Cout if self.bias is not None else 0) + self.B * self.Cout * self.Ho * self.Wo)
        n = (self.B * self.Cin * self.H * self.W
             + self.B * 2 * KK * self.groups * self.Ho * self.Wo
             + (self.B * KK * self.groups * self.Ho * self.Wo if self.mask is not None else 0)
             + self.Cout * self.Cin * KK
             + (self.Cout if self.bias is not None else 0)
             + self.B * self.Cout * self.Ho * self.Wo)
        return n * es


# The five workloads: tiny smoke case, the 224x224 single image, and the
# ResNet-50 c3 / c4 (stride-2 downsampling) / c5 (DCNv1, dilation 2) layers.
WORKLOADS = {
    "tiny": Workload("tiny", "f32", 1, 3, 32, 32, 8, 3, 1, 1, 1, 32, 32,
                     offset="uniform:2", mask="sigmoid", bias="zeros", seed=1000),
    "single224": Workload("single224", "f32", 1, 3, 224, 224, 64, 3, 1, 1, 1, 224, 224,
                          offset="tanh:0.5", mask="sigmoid", bias=None, seed=1001),
    "c3": Workload("c3", "bf16", 2, 128, 100, 168, 128, 3, 1, 1, 1, 100, 168,
                   offset="normal:2", mask="sigmoid", bias=None, seed=1002),
    "c4": Workload("c4", "bf16", 2, 256, 100, 168, 256, 3, 2, 1, 1, 50, 84,
                   offset="normal:1", mask="sigmoid", bias=None, seed=1003),
    "c5": Workload("c5", "bf16", 8, 512, 25, 42, 512, 3, 1, 2, 2, 25, 42,
                   offset="uniform:8", mask=None, bias="normal:0.01", seed=1004),
    # the c4 layer with four offset groups of 64 channels (deformable groups)
    "c4_g4": Workload("c4_g4", "bf16", 2, 256, 100, 168, 256, 3, 2, 1, 1, 50, 84,
                      offset="normal:1", mask="sigmoid", bias=None, seed=1005, groups=4),
    # the c4 layer's offset/mask convolution: 3*K^2 = 27 outputs (offset field and mask)
    "c4_bwd": Workload("c4_bwd", "bf16", 2, 256, 100, 168, 256, 3, 2, 1, 1, 50, 84,
                       offset="normal:1", mask="sigmoid", bias=None, seed=1007, op="backward"),
    # deformable RoI pooling on the c4 feature map (stride 16 of an 800 x 1344 image):
    # 256 RoIs per image, 7 x 7 bins, 2 x 2 samples per bin
    "roi_c4": Workload("roi_c4", "bf16", 2, 256, 50, 84, 256, 7, 1, 0, 1, 7, 7,
                       offset="normal:0.1", mask="sigmoid", bias=None, seed=1008, op="roi_pool"),
    # deformable position-sensitive RoI pooling on R-FCN-style score maps of the c4 grid:
    # 81 classes (80 + background) x 7 x 7 bins = 3969 maps at 50 x 84, 256 RoIs per image,
    # 2 x 2 samples per bin, one offset per bin shared by all classes, and a mask
    "psroi_c4": Workload("psroi_c4", "bf16", 2, 3969, 50, 84, 81, 7, 1, 0, 1, 7, 7,
                         offset="normal:0.1", mask="sigmoid", bias=None, seed=1010, op="ps_roi_pool"),
    # the c4 layer with its offset/mask branch in one call (the branch's weight and bias
    # are c4_om's, the layer's weight c4's; x is c4_om's)
    "c4_layer": Workload("c4_layer", "bf16", 2, 256, 100, 168, 256, 3, 2, 1, 1, 50, 84,
                         offset="normal:1", mask="sigmoid", bias=None, seed=1003, op="layer"),
    "c4_om": Workload("c4_om", "bf16", 2, 256, 100, 168, 27, 3, 2, 1, 1, 50, 84,
                      offset="normal:1", mask=None, bias="normal:0.1", seed=1006, op="offset_mask"),
    # the c4 layer on inputs whose four corners nearly cancel: x of alternating sign
    # and almost equal magnitude, sample fractions in [0.45, 0.55], weights of one sign
    # (a parity case for the interpolation's precision, not a bench workload)
    "c4_cancel": Workload("c4_cancel", "bf16", 2, 256, 100, 168, 256, 3, 2, 1, 1, 50, 84,
                          offset="frac:2:0.45:0.55", mask="sigmoid", bias=None, seed=1009,
                          x="checker:0.01", weight="kaiming_abs"),
}
ORDER = ["tiny", "single224", "c3", "c4", "c5", "c4_g4", "c4_om", "c4_layer", "c4_bwd", "roi_c4", "psroi_c4"]


def _draw(kind: str, shape, g: torch.Generator) -> torch.Tensor:
    name, _, arg = kind.partition(":")
    if name == "normal":
        s = float(arg) if arg else 1.0
        return torch.randn(shape, generator=g) * s
    if name == "uniform":
        a = float(arg)
        return (torch.rand(shape, generator=g) * 2.0 - 1.0) * a
    if name == "tanh":
        return torch.tanh(torch.randn(shape, generator=g)) * float(arg)
    if name == "sigmoid":
        return torch.sigmoid(torch.randn(shape, generator=g))
    if name == "frac":   # integer part uniform in [-n, n], fractional part U(lo, hi)
        n, lo, hi = arg.split(":")
        ip = torch.randint(-int(n), int(n) + 1, shape, generator=g).float()
        return ip + float(lo) + torch.rand(shape, generator=g) * (float(hi) - float(lo))
    if name == "checker":   # signs alternating like a checkerboard over the last two axes
        e = float(arg)
        sign = 1.0 - 2.0 * ((torch.arange(shape[-2])[:, None] + torch.arange(shape[-1])[None, :]) % 2).float()
        return sign * (1.0 + e * torch.randn(shape, generator=g))
    if name == "ones":
        return torch.ones(shape)
    if name == "zeros":
        return torch.zeros(shape)
    raise ValueError(f"unknown distribution {kind!r}")


def generate(w: Workload, seed: int | None = None) -> dict[str, torch.Tensor | None]:
    """Seeded CPU tensors for one workload, in the workload's element type.

    Weight: Kaiming-normal, fan-in mode with gain sqrt(2): std = sqrt(2 / (Cin*K*K)).
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    KK = w.K * w.K
    x = _draw(w.x, (w.B, w.Cin, w.H, w.W), g)
    weight = torch.randn((w.Cout, w.Cin, w.K, w.K), generator=g) * math.sqrt(2.0 / (w.Cin * KK))
    if w.weight == "kaiming_abs":
        weight = weight.abs()
    if w.op == "offset_mask":   # x, the 3GK^2-output weight, its bias
        bias = _draw(w.bias, (w.Cout,), g) if w.bias is not None else None
        dt = w.torch_dtype
        cast = (lambda t: None if t is None else t.to(dt).contiguous())
        return {"x": cast(x), "offset": None, "mask": None, "weight": cast(weight), "bias": cast(bias)}
    offset = _draw(w.offset, (w.B, 2 * KK * w.groups, w.Ho, w.Wo), g)
    mask = _draw(w.mask, (w.B, KK * w.groups, w.Ho, w.Wo), g) if w.mask is not None else None
    bias = _draw(w.bias, (w.Cout,), g) if w.bias is not None else None
    dt = w.torch_dtype
    cast = (lambda t: None if t is None else t.to(dt).contiguous())
    return {"x": cast(x), "offset": cast(offset), "mask": cast(mask), "weight": cast(weight),
            "bias": cast(bias)}


def grad_output(w: Workload, seed: int | None = None) -> torch.Tensor:
    """Seeded upstream gradient [B, Cout, Ho, Wo] for a backward call: N(0, 1) in the
    workload's element type (CPU)."""
    g = torch.Generator().manual_seed((w.seed if seed is None else seed) + 7919)
    gy = torch.randn((w.B, w.Cout, w.Ho, w.Wo), generator=g, dtype=torch.float32)
    return gy.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def roi_inputs(w: Workload, num_rois: int, k: int, image_hw: tuple[int, int], seed: int | None = None) -> dict:
    """Seeded inputs of deformable RoI pooling on the workload's feature map x [B,Cin,H,W]:
    num_rois boxes per batch image with sides drawn log-uniformly in [32, 512] image pixels,
    placed uniformly inside the image of size image_hw; offsets N(0, 0.1^2) per bin (row,
    column); the mask the sigmoid of N(0, 1).  rois are float32 [R,5] (batch index, x1, y1,
    x2, y2); the others in the workload's element type (CPU)."""
    g = torch.Generator().manual_seed((w.seed if seed is None else seed) + 104729)
    x = _draw(w.x, (w.B, w.Cin, w.H, w.W), g)
    R = num_rois * w.B
    ih, iw = image_hw
    side = torch.exp(torch.rand((R, 2), generator=g) * (math.log(512.0) - math.log(32.0)) + math.log(32.0))
    bw = torch.minimum(side[:, 0], torch.tensor(float(iw)))
    bh = torch.minimum(side[:, 1], torch.tensor(float(ih)))
    x1 = torch.rand(R, generator=g) * (iw - bw)
    y1 = torch.rand(R, generator=g) * (ih - bh)
    bidx = torch.arange(R) // num_rois
    rois = torch.stack([bidx.float(), x1, y1, x1 + bw, y1 + bh], 1).float().contiguous()
    offset = torch.randn((R, 2, k, k), generator=g) * 0.1
    mask = torch.sigmoid(torch.randn((R, k, k), generator=g))
    dt = w.torch_dtype
    return {"x": x.to(dt).contiguous(), "rois": rois, "offset": offset.to(dt).contiguous(),
            "mask": mask.to(dt).contiguous()}


def custom(name: str, dtype: str, B: int, Cin: int, H: int, W: int, Cout: int, K: int,
           stride: int, pad: int, dilation: int, Ho: int, Wo: int, offset: str = "normal:1",
           mask: str | None = "sigmoid", bias: str | None = "normal:0.1", seed: int = 0,
           x: str = "normal", groups: int = 1, op: str = "forward", weight: str = "kaiming") -> Workload:
    """A workload of any shape (used for edge cases); the caller supplies Ho, Wo."""
    return Workload(name, dtype, B, Cin, H, W, Cout, K, stride, pad, dilation, Ho, Wo,
                    offset=offset, mask=mask, bias=bias, seed=seed, x=x, groups=groups, op=op, weight=weight)
