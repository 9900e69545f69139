"""MI355X (gfx950) modulated deformable convolution forward (DCNv2; DCNv1 without mask).

A thin ctypes binding over ``libdcn_hip.so`` (C ABI in ``include/dcn.h``).  The
functions named like the C entry points marshal torch tensors into device
pointers and the current HIP stream; every step of the computation runs in the
library's kernels.  ``deform_conv2d`` mirrors torchvision's keyword order
(input, offset, weight, bias, stride, padding, dilation, mask) and allocates the
output and the workspace with torch.

There is no fallback: if the library is missing or no GPU is present the
calls raise.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["Desc", "dcn_output_hw", "dcn_workspace_bytes", "dcn_forward", "dcn_stage",
           "dcn_forward_staged", "dcn_variant_name", "dcn_plan_describe", "dcn_status_str", "deform_conv2d",
           "dcn_offset_mask_workspace_bytes", "dcn_offset_mask", "offset_mask", "dcn_forward_noalloc",
           "DcnError", "library_path", "load_library", "F32", "BF16"]

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdcn_hip.so")

F32, BF16 = 0, 1
OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_SCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20   # DCN_NOALLOC_SCRATCH_BYTES of dcn.h
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}
_EXPORTS = ("dcn_output_hw", "dcn_workspace_bytes", "dcn_forward", "dcn_stage", "dcn_forward_staged",
            "dcn_variant_name", "dcn_plan_describe", "dcn_status_str", "dcn_offset_mask_workspace_bytes",
            "dcn_offset_mask")


class DcnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dcn_status_str(status)} (status {status})")


class Desc(ctypes.Structure):
    """Mirror of ``dcn_desc``."""
    _fields_ = [("batch", ctypes.c_int64), ("in_channels", ctypes.c_int64), ("height", ctypes.c_int64),
                ("width", ctypes.c_int64), ("out_channels", ctypes.c_int64),
                ("kernel_size", ctypes.c_int64), ("stride", ctypes.c_int64), ("pad", ctypes.c_int64),
                ("dilation", ctypes.c_int64), ("dtype", ctypes.c_int32), ("offset_groups", ctypes.c_int32)]

    def __repr__(self):
        return "Desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class RoiDesc(ctypes.Structure):
    """Mirror of ``dcn_roi_desc``."""
    _fields_ = [("batch", ctypes.c_int64), ("channels", ctypes.c_int64), ("height", ctypes.c_int64),
                ("width", ctypes.c_int64), ("num_rois", ctypes.c_int64), ("pooled_size", ctypes.c_int64),
                ("samples", ctypes.c_int64), ("spatial_scale", ctypes.c_float), ("gamma", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PsRoiDesc(ctypes.Structure):
    """Mirror of ``dcn_ps_roi_desc``."""
    _fields_ = [("batch", ctypes.c_int64), ("out_channels", ctypes.c_int64), ("height", ctypes.c_int64),
                ("width", ctypes.c_int64), ("num_rois", ctypes.c_int64), ("pooled_size", ctypes.c_int64),
                ("samples", ctypes.c_int64), ("offset_groups", ctypes.c_int64), ("spatial_scale", ctypes.c_float),
                ("gamma", ctypes.c_float), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return os.environ.get("DCN_HIP_LIB", LIB_PATH)


def load_library() -> ctypes.CDLL:
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m deformable_convolution_vision_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Desc)
    lib.dcn_output_hw.argtypes = [D, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.dcn_workspace_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_forward.argtypes = [D, P, P, P, P, P, P, P, S, P]
    lib.dcn_forward_staged.argtypes = [D, P, P, P, P, P, P, P, S, P]
    lib.dcn_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P]
    lib.dcn_layer_workspace_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_layer_workspace_bytes.restype = ctypes.c_int
    lib.dcn_layer_forward.argtypes = [D, P, P, P, P, P, P, P, P, P, S, P]
    lib.dcn_layer_forward.restype = ctypes.c_int
    lib.dcn_forward_noalloc.restype = ctypes.c_int
    lib.dcn_stage.argtypes = [D, P, P, P, S, P]
    lib.dcn_variant_name.argtypes = [D]
    lib.dcn_variant_name.restype = ctypes.c_char_p
    lib.dcn_plan_describe.argtypes = [D, ctypes.c_char_p, ctypes.c_size_t]
    lib.dcn_plan_describe.restype = ctypes.c_int
    lib.dcn_status_str.argtypes = [ctypes.c_int]
    lib.dcn_status_str.restype = ctypes.c_char_p
    lib.dcn_offset_mask_workspace_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_offset_mask_workspace_bytes.restype = ctypes.c_int
    lib.dcn_offset_mask.argtypes = [D, P, P, P, P, P, P, S, P]
    lib.dcn_offset_mask.restype = ctypes.c_int
    lib.dcn_backward_workspace_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_backward_workspace_bytes.restype = ctypes.c_int
    lib.dcn_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.dcn_backward.restype = ctypes.c_int
    lib.dcn_roi_pool.argtypes = [ctypes.POINTER(RoiDesc), P, P, P, P, P, P, S, P]
    lib.dcn_roi_pool.restype = ctypes.c_int
    lib.dcn_roi_pool_workspace_bytes.argtypes = [ctypes.POINTER(RoiDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_roi_pool_workspace_bytes.restype = ctypes.c_int
    lib.dcn_ps_roi_pool.argtypes = [ctypes.POINTER(PsRoiDesc), P, P, P, P, P, P, S, P]
    lib.dcn_ps_roi_pool.restype = ctypes.c_int
    lib.dcn_ps_roi_pool_workspace_bytes.argtypes = [ctypes.POINTER(PsRoiDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.dcn_ps_roi_pool_workspace_bytes.restype = ctypes.c_int
    for name in ("dcn_output_hw", "dcn_workspace_bytes", "dcn_forward", "dcn_forward_staged", "dcn_stage"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def dcn_status_str(status: int) -> str:
    return load_library().dcn_status_str(int(status)).decode()


def make_desc(B, Cin, H, W, Cout, K, stride=1, pad=0, dilation=1, dtype=F32, offset_groups=1) -> Desc:
    return Desc(B, Cin, H, W, Cout, K, stride, pad, dilation, dtype, offset_groups)


def dcn_output_hw(desc: Desc) -> tuple[int, int]:
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    rc = load_library().dcn_output_hw(ctypes.byref(desc), ctypes.byref(ho), ctypes.byref(wo))
    if rc != OK:
        raise DcnError(rc, "dcn_output_hw")
    return ho.value, wo.value


def dcn_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_workspace_bytes")
    return n.value


def dcn_variant_name(desc: Desc) -> str:
    return load_library().dcn_variant_name(ctypes.byref(desc)).decode()


def dcn_plan_describe(desc: Desc) -> str:
    buf = ctypes.create_string_buffer(512)
    rc = load_library().dcn_plan_describe(ctypes.byref(desc), buf, len(buf))
    if rc != OK:
        raise DcnError(rc, "dcn_plan_describe")
    return buf.value.decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dcn_forward(desc: Desc, x, offset, mask, weight, bias, out, workspace, workspace_bytes: int,
                stream=None) -> None:
    """Raw call: tensors (or integer device addresses) already laid out as dcn.h states."""
    rc = load_library().dcn_forward(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                    _ptr(bias), _ptr(out), _ptr(workspace), workspace_bytes,
                                    _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_forward")


def dcn_stage(desc: Desc, x, weight, workspace, workspace_bytes: int, stream=None) -> None:
    rc = load_library().dcn_stage(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(workspace),
                                  workspace_bytes, _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_stage")


def dcn_forward_staged(desc: Desc, x, offset, mask, weight, bias, out, workspace, workspace_bytes: int,
                       stream=None) -> None:
    rc = load_library().dcn_forward_staged(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask),
                                           _ptr(weight), _ptr(bias), _ptr(out), _ptr(workspace),
                                           workspace_bytes, _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_forward_staged")


def dcn_forward_noalloc(desc: Desc, x, offset, mask, weight, bias, out, stream=None) -> None:
    """Raw call of the entry point that allocates nothing (its workspace is a device
    array of NOALLOC_SCRATCH_BYTES held by the library per GPU); tensors or device
    addresses as dcn.h states."""
    rc = load_library().dcn_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                            _ptr(bias), _ptr(out), _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_forward_noalloc")


def describe(input, weight, stride=1, padding=0, dilation=1, offset=None) -> Desc:
    """Descriptor of a call; the offset groups follow from the offset's channel count
    (2*G*K*K), as in torchvision, when offset is given."""
    if input.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {input.dtype}; use float32 or bfloat16")
    if input.dim() != 4 or weight.dim() != 4:
        raise ValueError("input must be [B,Cin,H,W] and weight [Cout,Cin,K,K]")
    B, Cin, H, W = input.shape
    Cout, Cin_w, K, K2 = weight.shape
    if Cin_w != Cin or K != K2:
        raise ValueError(f"weight {tuple(weight.shape)} does not match input {tuple(input.shape)}")
    G = 1
    if offset is not None:
        if offset.dim() != 4 or offset.shape[1] % (2 * K * K) != 0 or offset.shape[1] == 0:
            raise ValueError(f"offset must have 2*G*K*K channels, got {tuple(offset.shape)}")
        G = offset.shape[1] // (2 * K * K)
        if Cin % G != 0:
            raise ValueError(f"{Cin} input channels do not split into {G} offset groups")
    return make_desc(B, Cin, H, W, Cout, K, int(stride), int(padding), int(dilation), _DTYPES[input.dtype], G)


def check_tensors(desc: Desc, input, offset, weight, bias, mask) -> tuple[int, int]:
    """Shape, dtype, device and contiguity checks; returns (Ho, Wo)."""
    Ho, Wo = dcn_output_hw(desc)
    KK = desc.kernel_size ** 2 * max(desc.offset_groups, 1)
    expect = {"offset": (offset, (desc.batch, 2 * KK, Ho, Wo)),
              "mask": (mask, (desc.batch, KK, Ho, Wo)),
              "bias": (bias, (desc.out_channels,))}
    for name, t in (("input", input), ("offset", offset), ("weight", weight), ("bias", bias), ("mask", mask)):
        if t is None:
            continue
        if t.dtype != input.dtype:
            raise TypeError(f"{name} is {t.dtype}, input is {input.dtype}: all tensors share one dtype")
        if not t.is_cuda or t.device != input.device:
            raise ValueError(f"{name} must be on the input's GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if name in expect and tuple(t.shape) != expect[name][1]:
            raise ValueError(f"{name} must have shape {expect[name][1]}, got {tuple(t.shape)}")
    return Ho, Wo


def _check_out(out, shape, dtype, device, name="out"):
    """A caller-supplied output: the exact shape, dtype and device, contiguous."""
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {out.dtype}")
    if not out.is_cuda or out.device != device:
        raise ValueError(f"{name} must be on {device}, got {out.device}")
    if not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(workspace, nbytes: int, device):
    """The caller's workspace after checks (contiguous, on the device, at least nbytes),
    or a fresh one when none is given."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a tensor")
    if not workspace.is_cuda or workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    have = workspace.numel() * workspace.element_size()
    if have < nbytes:
        raise ValueError(f"workspace holds {have} bytes, the call needs {nbytes}")
    return workspace


def deform_conv2d(input, offset, weight, bias=None, stride=1, padding=0, dilation=1, mask=None,
                  out=None, workspace=None):
    """Deformable convolution forward on the GPU (torchvision's argument order).

    input [B,Cin,H,W], offset [B,2GK^2,Ho,Wo] (channel 2(gK^2+k) = dy, 2(gK^2+k)+1 =
    dx of kernel point k = i*K + j for offset group g; G = 1 by default), weight
    [Cout,Cin,K,K], bias [Cout] or None, mask [B,GK^2,Ho,Wo] or None.  float32 or
    bfloat16, contiguous, on one GPU.
    """
    desc = describe(input, weight, stride, padding, dilation, offset)
    Ho, Wo = check_tensors(desc, input, offset, weight, bias, mask)
    shape = (desc.batch, desc.out_channels, Ho, Wo)
    if out is None:
        out = torch.empty(shape, dtype=input.dtype, device=input.device)
    else:
        _check_out(out, shape, input.dtype, input.device)
    nbytes = dcn_workspace_bytes(desc)
    workspace = _workspace(workspace, nbytes, input.device)
    with torch.cuda.device(input.device):
        dcn_forward(desc, input, offset, mask, weight, bias, out, workspace if nbytes else None, nbytes)
    return out


def dcn_offset_mask_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_offset_mask_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_offset_mask_workspace_bytes")
    return n.value


def dcn_offset_mask(desc: Desc, x, weight_om, bias_om, offset, mask, workspace, workspace_bytes: int,
                    stream=None) -> None:
    rc = load_library().dcn_offset_mask(ctypes.byref(desc), _ptr(x), _ptr(weight_om), _ptr(bias_om),
                                        _ptr(offset), _ptr(mask), _ptr(workspace), workspace_bytes,
                                        _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_offset_mask")


def offset_mask(input, weight_om, bias_om=None, stride=1, padding=0, dilation=1, offset_groups=1,
                workspace=None):
    """The DCNv2 offset/mask branch on the GPU: returns (offset [B,2GK^2,Ho,Wo], mask
    [B,GK^2,Ho,Wo]) from the regular convolution of input with weight_om
    [3GK^2,Cin,K,K] (bias_om [3GK^2] or None), ready for deform_conv2d."""
    K = weight_om.shape[2]
    G = int(offset_groups)
    if weight_om.dim() != 4 or weight_om.shape[0] != 3 * G * K * K or weight_om.shape[3] != K:
        raise ValueError(f"weight_om must be [3*G*K*K, Cin, K, K], got {tuple(weight_om.shape)}")
    if input.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {input.dtype}; use float32 or bfloat16")
    B, Cin, H, W = input.shape
    if weight_om.shape[1] != Cin:
        raise ValueError("weight_om does not match the input channels")
    for name, t in (("weight_om", weight_om), ("bias_om", bias_om)):
        if t is None:
            continue
        if t.dtype != input.dtype or t.device != input.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {input.dtype} tensor on the input's device")
    if bias_om is not None and tuple(bias_om.shape) != (3 * G * K * K,):
        raise ValueError("bias_om must be [3*G*K*K]")
    if not input.is_cuda or not input.is_contiguous():
        raise ValueError("input must be a contiguous GPU tensor")
    desc = make_desc(B, Cin, H, W, 1, K, int(stride), int(padding), int(dilation), _DTYPES[input.dtype], G)
    Ho, Wo = dcn_output_hw(desc)
    offset = torch.empty((B, 2 * G * K * K, Ho, Wo), dtype=input.dtype, device=input.device)
    mask = torch.empty((B, G * K * K, Ho, Wo), dtype=input.dtype, device=input.device)
    nbytes = dcn_offset_mask_workspace_bytes(desc)
    workspace = _workspace(workspace, nbytes, input.device)
    with torch.cuda.device(input.device):
        dcn_offset_mask(desc, input, weight_om, bias_om, offset, mask, workspace if nbytes else None, nbytes)
    return offset, mask


def dcn_backward_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_backward_workspace_bytes")
    return n.value


def dcn_backward(desc: Desc, x, offset, mask, weight, grad_out, grad_x, grad_offset, grad_mask, grad_weight,
                 grad_bias, workspace, workspace_bytes: int, stream=None) -> None:
    """Raw call: tensors (or integer device addresses) laid out as dcn.h states; any
    gradient may be None (not computed)."""
    rc = load_library().dcn_backward(ctypes.byref(desc), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                                     _ptr(grad_out), _ptr(grad_x), _ptr(grad_offset), _ptr(grad_mask),
                                     _ptr(grad_weight), _ptr(grad_bias), _ptr(workspace), workspace_bytes,
                                     _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_backward")


def deform_conv2d_backward(grad_out, input, offset, weight, stride=1, padding=0, dilation=1, mask=None,
                           with_bias=True, workspace=None):
    """Gradients of deform_conv2d on the GPU: returns (grad_input, grad_offset, grad_weight,
    grad_bias or None, grad_mask or None) for the upstream gradient grad_out
    [B, Cout, Ho, Wo]."""
    desc = describe(input, weight, stride, padding, dilation, offset)
    Ho, Wo = check_tensors(desc, input, offset, weight, None, mask)
    if tuple(grad_out.shape) != (desc.batch, desc.out_channels, Ho, Wo):
        raise ValueError(f"grad_out must be {(desc.batch, desc.out_channels, Ho, Wo)}")
    if grad_out.dtype != input.dtype or grad_out.device != input.device or not grad_out.is_contiguous():
        raise ValueError("grad_out must be a contiguous tensor of the input's dtype and device")
    gx = torch.empty_like(input)
    goff = torch.empty_like(offset)
    gw = torch.empty_like(weight)
    gb = torch.empty(desc.out_channels, dtype=input.dtype, device=input.device) if with_bias else None
    gm = torch.empty_like(mask) if mask is not None else None
    nbytes = dcn_backward_workspace_bytes(desc)
    workspace = _workspace(workspace, nbytes, input.device)
    with torch.cuda.device(input.device):
        dcn_backward(desc, input, offset, mask, weight, grad_out, gx, goff, gm, gw, gb,
                     workspace if nbytes else None, nbytes)
    return gx, goff, gw, gb, gm


def dcn_roi_pool_workspace_bytes(desc: RoiDesc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_roi_pool_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_roi_pool_workspace_bytes")
    return n.value


def dcn_roi_pool(desc: RoiDesc, x, rois, offset, mask, out, workspace, workspace_bytes: int, stream=None) -> None:
    """Raw call: tensors (or integer device addresses) laid out as dcn.h states."""
    rc = load_library().dcn_roi_pool(ctypes.byref(desc), _ptr(x), _ptr(rois), _ptr(offset), _ptr(mask), _ptr(out),
                                     _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_roi_pool")


def deform_roi_pool(input, rois, offset=None, mask=None, output_size=7, sampling_ratio=2, spatial_scale=1.0,
                    gamma=0.1):
    """Deformable RoI pooling on the GPU: input [B,C,H,W]; rois [R,5] float32 (batch index,
    x1, y1, x2, y2 in image coordinates); offset [R,2,k,k] (row, column, normalised by the
    RoI's size) or None; mask [R,k,k] or None.  Returns [R,C,k,k] in the input's dtype."""
    if input.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {input.dtype}; use float32 or bfloat16")
    k = int(output_size)
    B, C, H, W = input.shape
    R = rois.shape[0]
    if rois.dtype != torch.float32 or tuple(rois.shape) != (R, 5):
        raise ValueError("rois must be a float32 [R, 5] tensor")
    for name, t, shape in (("offset", offset, (R, 2, k, k)), ("mask", mask, (R, k, k))):
        if t is None:
            continue
        if tuple(t.shape) != shape or t.dtype != input.dtype:
            raise ValueError(f"{name} must be {shape} of the input's dtype")
    for t in (input, rois, offset, mask):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.device != input.device):
            raise ValueError("tensors must be contiguous and on the input's GPU")
    desc = RoiDesc(B, C, H, W, R, k, int(sampling_ratio), float(spatial_scale), float(gamma), _DTYPES[input.dtype], 0)
    out = torch.empty((R, C, k, k), dtype=input.dtype, device=input.device)
    nbytes = dcn_roi_pool_workspace_bytes(desc)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=input.device) if nbytes else None
    with torch.cuda.device(input.device):
        dcn_roi_pool(desc, input, rois, offset, mask, out, ws, nbytes)
    return out


def dcn_ps_roi_pool_workspace_bytes(desc: PsRoiDesc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_ps_roi_pool_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_ps_roi_pool_workspace_bytes")
    return n.value


def dcn_ps_roi_pool(desc: PsRoiDesc, x, rois, offset, mask, out, workspace, workspace_bytes: int,
                    stream=None) -> None:
    """Raw call: tensors (or integer device addresses) laid out as dcn.h states."""
    rc = load_library().dcn_ps_roi_pool(ctypes.byref(desc), _ptr(x), _ptr(rois), _ptr(offset), _ptr(mask), _ptr(out),
                                        _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_ps_roi_pool")


def deform_ps_roi_pool(input, rois, offset=None, mask=None, output_size=7, sampling_ratio=2, spatial_scale=1.0,
                       gamma=0.1):
    """Deformable position-sensitive RoI pooling on the GPU: input [B, C*k*k, H, W] (k*k
    score maps per output channel); rois [R,5] float32; offset [R,2G,k,k] (G groups of
    output channels) or None; mask [R,k,k] or None.  Returns [R,C,k,k]."""
    if input.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {input.dtype}; use float32 or bfloat16")
    k = int(output_size)
    B, Cin, H, W = input.shape
    if Cin % (k * k) != 0:
        raise ValueError(f"input must have C*k*k channels (k = {k}), got {Cin}")
    C = Cin // (k * k)
    R = rois.shape[0]
    if rois.dtype != torch.float32 or tuple(rois.shape) != (R, 5):
        raise ValueError("rois must be a float32 [R, 5] tensor")
    G = 1
    if offset is not None:
        if offset.dim() != 4 or offset.shape[0] != R or offset.shape[1] % 2 or tuple(offset.shape[2:]) != (k, k):
            raise ValueError(f"offset must be [R, 2G, {k}, {k}]")
        G = offset.shape[1] // 2
        if C % G != 0:
            raise ValueError(f"{C} output channels do not split into {G} offset groups")
    for name, t in (("offset", offset), ("mask", mask)):
        if t is not None and t.dtype != input.dtype:
            raise ValueError(f"{name} must have the input's dtype")
    if mask is not None and tuple(mask.shape) != (R, k, k):
        raise ValueError(f"mask must be {(R, k, k)}")
    for t in (input, rois, offset, mask):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.device != input.device):
            raise ValueError("tensors must be contiguous and on the input's GPU")
    desc = PsRoiDesc(B, C, H, W, R, k, int(sampling_ratio), G, float(spatial_scale), float(gamma),
                     _DTYPES[input.dtype], 0)
    out = torch.empty((R, C, k, k), dtype=input.dtype, device=input.device)
    nbytes = dcn_ps_roi_pool_workspace_bytes(desc)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=input.device) if nbytes else None
    with torch.cuda.device(input.device):
        dcn_ps_roi_pool(desc, input, rois, offset, mask, out, ws, nbytes)
    return out


def dcn_layer_workspace_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t()
    rc = load_library().dcn_layer_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    if rc != OK:
        raise DcnError(rc, "dcn_layer_workspace_bytes")
    return n.value


def dcn_layer_forward(desc: Desc, x, weight_om, bias_om, weight, bias, offset, mask, out, workspace,
                      workspace_bytes: int, stream=None) -> None:
    """Raw call: tensors (or integer device addresses) laid out as dcn.h states."""
    rc = load_library().dcn_layer_forward(ctypes.byref(desc), _ptr(x), _ptr(weight_om), _ptr(bias_om), _ptr(weight),
                                          _ptr(bias), _ptr(offset), _ptr(mask), _ptr(out), _ptr(workspace),
                                          workspace_bytes, _stream(stream))
    if rc != OK:
        raise DcnError(rc, "dcn_layer_forward")


def deform_conv2d_layer(input, weight_om, bias_om, weight, bias=None, stride=1, padding=0, dilation=1,
                        offset_groups=1, workspace=None):
    """The whole DCNv2 layer on the GPU in one call: the offset/mask branch (weight_om
    [3GK^2,Cin,K,K], bias_om [3GK^2] or None) and the deformable convolution (weight
    [Cout,Cin,K,K], bias [Cout] or None) off one staged copy of input.  Returns (out
    [B,Cout,Ho,Wo], offset [B,2GK^2,Ho,Wo], mask [B,GK^2,Ho,Wo])."""
    if input.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {input.dtype}; use float32 or bfloat16")
    if input.dim() != 4 or weight.dim() != 4 or weight_om.dim() != 4:
        raise ValueError("input, weight and weight_om must be 4-D")
    B, Cin, H, W = input.shape
    Cout, K = weight.shape[0], weight.shape[2]
    G = int(offset_groups)
    if tuple(weight.shape) != (Cout, Cin, K, K) or tuple(weight_om.shape) != (3 * G * K * K, Cin, K, K):
        raise ValueError("weight must be [Cout, Cin, K, K] and weight_om [3*G*K*K, Cin, K, K]")
    for name, t, shape in (("bias", bias, (Cout,)), ("bias_om", bias_om, (3 * G * K * K,))):
        if t is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    for name, t in (("input", input), ("weight", weight), ("weight_om", weight_om), ("bias", bias),
                    ("bias_om", bias_om)):
        if t is None:
            continue
        if t.dtype != input.dtype or not t.is_cuda or t.device != input.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {input.dtype} tensor on the input's GPU")
    desc = make_desc(B, Cin, H, W, Cout, K, int(stride), int(padding), int(dilation), _DTYPES[input.dtype], G)
    Ho, Wo = dcn_output_hw(desc)
    out = torch.empty((B, Cout, Ho, Wo), dtype=input.dtype, device=input.device)
    offset = torch.empty((B, 2 * G * K * K, Ho, Wo), dtype=input.dtype, device=input.device)
    mask = torch.empty((B, G * K * K, Ho, Wo), dtype=input.dtype, device=input.device)
    nbytes = dcn_layer_workspace_bytes(desc)
    workspace = _workspace(workspace, nbytes, input.device)
    with torch.cuda.device(input.device):
        dcn_layer_forward(desc, input, weight_om, bias_om, weight, bias, offset, mask, out,
                          workspace if nbytes else None, nbytes)
    return out, offset, mask
