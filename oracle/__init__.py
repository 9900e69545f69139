"""CPU oracle for the modulated deformable convolution forward (DCNv2; DCNv1 when
the mask is absent) and its gradients.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
package ``deformable_convolution_vision_amd`` never imports it, and the two
share no code: this package wraps ``libdcn_oracle.so``, built by ``g++`` from
``dcn_oracle.cpp`` alone (see that file and ``dcn_oracle.h`` for the definition
and its sources on the pages).

Every function here takes host arrays that are already rounded to the element
type under test (fp32 values, or bf16 values widened to fp32) and returns
float64 results.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dcn_oracle.cpp")
LIB = os.path.join(HERE, "libdcn_oracle.so")


class _Desc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in
                ("B", "Cin", "H", "W", "Cout", "K", "stride", "pad", "dilation", "groups")]


class _RoiDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in ("B", "C", "H", "W", "R", "k", "S")] + \
               [("spatial_scale", ctypes.c_double), ("gamma", ctypes.c_double)]


class _PsRoiDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in ("B", "C", "H", "W", "R", "k", "S", "G")] + \
               [("spatial_scale", ctypes.c_double), ("gamma", ctypes.c_double)]


def build(out_path: str = LIB, extra_flags: tuple[str, ...] = (), src: str = SRC) -> str:
    """Compile the oracle with g++ (OpenMP, IEEE arithmetic: no fast-math)."""
    tmp = out_path + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           f"-I{HERE}", *extra_flags, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str = LIB) -> ctypes.CDLL:
    """Load the oracle library, building it only if it is not there yet."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_output_hw.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.oracle_output_hw.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [ctypes.POINTER(_Desc), P, P, P, P, P, ctypes.c_int64,
                                   ctypes.c_int64, P, P, ctypes.c_int]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_points.argtypes = [ctypes.POINTER(_Desc), P, P, P, P, P, P, ctypes.c_int64, P, P,
                                  ctypes.c_int]
    lib.oracle_points.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [ctypes.POINTER(_Desc), P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_roi_pool.argtypes = [ctypes.POINTER(_RoiDesc), P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_roi_pool.restype = ctypes.c_int
    lib.oracle_ps_roi_pool.argtypes = [ctypes.POINTER(_PsRoiDesc), P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_ps_roi_pool.restype = ctypes.c_int
    lib.oracle_threads.argtypes = [ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _f32(a):
    """Host float32 C-contiguous copy of an array-like (numpy or torch CPU)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen (bf16 -> fp32 is exact) on the host
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _desc(x, weight, stride, pad, dilation, offset=None):
    B, Cin, H, W = x.shape
    Cout, Cin_w, K, K2 = weight.shape
    if Cin_w != Cin or K != K2:
        raise ValueError("weight must be [Cout, Cin, K, K] with Cin matching x")
    G = 1
    if offset is not None:   # offset groups from the offset's channel count, as torchvision does
        if offset.ndim != 4 or offset.shape[1] % (2 * K * K) != 0:
            raise ValueError("offset must have 2*G*K*K channels")
        G = offset.shape[1] // (2 * K * K)
        if G < 1 or Cin % G != 0:
            raise ValueError("Cin must be a multiple of the offset groups")
    return _Desc(B, Cin, H, W, Cout, K, stride, pad, dilation, G)


def output_hw(B, Cin, H, W, Cout, K, stride=1, pad=0, dilation=1, lib_path: str = LIB):
    lib = load(lib_path)
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    rc = lib.oracle_output_hw(ctypes.byref(_Desc(B, Cin, H, W, Cout, K, stride, pad, dilation, 1)),
                              ctypes.byref(ho), ctypes.byref(wo))
    if rc != 0:
        raise ValueError("invalid geometry")
    return ho.value, wo.value


def _check(x, offset, mask, weight, bias, d, Ho, Wo):
    KK = d.K * d.K * d.groups
    if offset.shape != (d.B, 2 * KK, Ho, Wo):
        raise ValueError(f"offset must be {(d.B, 2 * KK, Ho, Wo)}, got {offset.shape}")
    if mask is not None and mask.shape != (d.B, KK, Ho, Wo):
        raise ValueError(f"mask must be {(d.B, KK, Ho, Wo)}, got {mask.shape}")
    if bias is not None and bias.shape != (d.Cout,):
        raise ValueError("bias must be [Cout]")


def forward(x, offset, weight, bias=None, stride=1, padding=0, dilation=1, mask=None,
            cout_range=None, threads=0, with_abs=True, lib_path: str = LIB):
    """y (and sum of |terms|) for the full output grid, float64 [B, Cout', Ho, Wo].

    ``cout_range=(o0, o1)`` restricts the output channels computed.
    """
    lib = load(lib_path)
    x, offset, weight, bias, mask = map(_f32, (x, offset, weight, bias, mask))
    d = _desc(x, weight, stride, padding, dilation, offset)
    Ho, Wo = output_hw(d.B, d.Cin, d.H, d.W, d.Cout, d.K, stride, padding, dilation, lib_path)
    _check(x, offset, mask, weight, bias, d, Ho, Wo)
    o0, o1 = (0, d.Cout) if cout_range is None else cout_range
    out = np.empty((d.B, o1 - o0, Ho, Wo), dtype=np.float64)
    ab = np.empty_like(out) if with_abs else None
    rc = lib.oracle_forward(ctypes.byref(d), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                            _ptr(bias), o0, o1, _ptr(out), _ptr(ab), threads)
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    return (out, ab) if with_abs else out


def points(x, offset, weight, pts, bias=None, stride=1, padding=0, dilation=1, mask=None,
           threads=0, lib_path: str = LIB):
    """y and sum of |terms| at individual outputs; pts is an int array [n, 4] of (b, o, oy, ox)."""
    lib = load(lib_path)
    x, offset, weight, bias, mask = map(_f32, (x, offset, weight, bias, mask))
    d = _desc(x, weight, stride, padding, dilation, offset)
    Ho, Wo = output_hw(d.B, d.Cin, d.H, d.W, d.Cout, d.K, stride, padding, dilation, lib_path)
    _check(x, offset, mask, weight, bias, d, Ho, Wo)
    pts = np.ascontiguousarray(np.asarray(pts, dtype=np.int64).reshape(-1, 4))
    out = np.empty(len(pts), dtype=np.float64)
    ab = np.empty(len(pts), dtype=np.float64)
    rc = lib.oracle_points(ctypes.byref(d), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight),
                           _ptr(bias), _ptr(pts), len(pts), _ptr(out), _ptr(ab), threads)
    if rc != 0:
        raise ValueError("oracle_points rejected its arguments")
    return out, ab


def backward(x, offset, weight, grad_out, stride=1, padding=0, dilation=1, mask=None, threads=0,
             want=("grad_x", "grad_offset", "grad_mask", "grad_weight", "grad_bias"), lib_path: str = LIB):
    """Gradients of the forward with respect to x, offset, mask, weight and bias for the
    upstream gradient ``grad_out`` [B, Cout, Ho, Wo] (the gradient equation of the
    csdn.net tags page "可变形卷积：Deformable ConvNets", part "Deformable Convolutional
    Networks", section 可变形卷积; the full definition is in dcn_oracle.h).

    Returns a dict of float64 arrays: grad_x, grad_offset, grad_mask (None without a
    mask), grad_weight, grad_bias; those not named in ``want`` are None (not computed)."""
    lib = load(lib_path)
    x, offset, weight, grad_out, mask = map(_f32, (x, offset, weight, grad_out, mask))
    d = _desc(x, weight, stride, padding, dilation, offset)
    Ho, Wo = output_hw(d.B, d.Cin, d.H, d.W, d.Cout, d.K, stride, padding, dilation, lib_path)
    _check(x, offset, mask, weight, None, d, Ho, Wo)
    if grad_out.shape != (d.B, d.Cout, Ho, Wo):
        raise ValueError(f"grad_out must be {(d.B, d.Cout, Ho, Wo)}, got {grad_out.shape}")
    gx = np.empty(x.shape, dtype=np.float64) if "grad_x" in want else None
    goff = np.empty(offset.shape, dtype=np.float64) if "grad_offset" in want else None
    gm = np.empty(mask.shape, dtype=np.float64) if mask is not None and "grad_mask" in want else None
    gw = np.empty(weight.shape, dtype=np.float64) if "grad_weight" in want else None
    gb = np.empty(d.Cout, dtype=np.float64) if "grad_bias" in want else None
    rc = lib.oracle_backward(ctypes.byref(d), _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(grad_out),
                             _ptr(gx), _ptr(goff), _ptr(gm), _ptr(gw), _ptr(gb), threads)
    if rc != 0:
        raise ValueError("oracle_backward rejected its arguments")
    return {"grad_x": gx, "grad_offset": goff, "grad_mask": gm, "grad_weight": gw, "grad_bias": gb}


def roi_pool(x, rois, k, S, spatial_scale=1.0, gamma=0.1, offset=None, mask=None, threads=0,
             with_abs=False, lib_path: str = LIB):
    """Deformable RoI pooling (definition and readings in dcn_oracle.h): x [B,C,H,W],
    rois [R,5] = (batch index, x1, y1, x2, y2), offset [R,2,k,k] (row, column; normalised
    by the RoI's height and width and scaled by gamma) or None, mask [R,k,k] or None.
    Returns float64 [R,C,k,k], and with ``with_abs`` also the sum of |terms| of each
    output (|m| / S^2 times the sum of |corner weight * value| over its samples)."""
    lib = load(lib_path)
    x, rois, offset, mask = map(_f32, (x, rois, offset, mask))
    B, C, H, W = x.shape
    R = rois.shape[0]
    if rois.shape != (R, 5):
        raise ValueError("rois must be [R, 5]")
    if offset is not None and offset.shape != (R, 2, k, k):
        raise ValueError(f"offset must be {(R, 2, k, k)}")
    if mask is not None and mask.shape != (R, k, k):
        raise ValueError(f"mask must be {(R, k, k)}")
    d = _RoiDesc(B, C, H, W, R, k, S, float(spatial_scale), float(gamma))
    out = np.empty((R, C, k, k), dtype=np.float64)
    ab = np.empty_like(out) if with_abs else None
    rc = lib.oracle_roi_pool(ctypes.byref(d), _ptr(x), _ptr(rois), _ptr(offset), _ptr(mask), _ptr(out),
                             _ptr(ab), threads)
    if rc != 0:
        raise ValueError("oracle_roi_pool rejected its arguments")
    return (out, ab) if with_abs else out


def ps_roi_pool(x, rois, k, S, spatial_scale=1.0, gamma=0.1, offset=None, mask=None, threads=0,
                with_abs=False, lib_path: str = LIB):
    """Deformable position-sensitive RoI pooling (definition and readings in
    dcn_oracle.h): x [B, C*k*k, H, W] (k*k score maps per output channel; bin (i, j) of
    output channel c pools input channel (c*k + i)*k + j), rois [R,5], offset [R,2G,k,k]
    (G groups of output channels, each with its own row/column offsets) or None, mask
    [R,k,k] or None.  Returns float64 [R,C,k,k], and with ``with_abs`` the sum of |terms|."""
    lib = load(lib_path)
    x, rois, offset, mask = map(_f32, (x, rois, offset, mask))
    B, Cin, H, W = x.shape
    if Cin % (k * k) != 0:
        raise ValueError("x must have C*k*k channels")
    C = Cin // (k * k)
    R = rois.shape[0]
    if rois.shape != (R, 5):
        raise ValueError("rois must be [R, 5]")
    G = 1
    if offset is not None:
        if offset.ndim != 4 or offset.shape[0] != R or offset.shape[1] % 2 or offset.shape[2:] != (k, k):
            raise ValueError(f"offset must be [R, 2G, {k}, {k}]")
        G = offset.shape[1] // 2
        if C % G:
            raise ValueError("the output channels must split into the offset groups")
    if mask is not None and mask.shape != (R, k, k):
        raise ValueError(f"mask must be {(R, k, k)}")
    d = _PsRoiDesc(B, C, H, W, R, k, S, G, float(spatial_scale), float(gamma))
    out = np.empty((R, C, k, k), dtype=np.float64)
    ab = np.empty_like(out) if with_abs else None
    rc = lib.oracle_ps_roi_pool(ctypes.byref(d), _ptr(x), _ptr(rois), _ptr(offset), _ptr(mask), _ptr(out),
                                _ptr(ab), threads)
    if rc != 0:
        raise ValueError("oracle_ps_roi_pool rejected its arguments")
    return (out, ab) if with_abs else out


def threads_used(threads: int = 0, lib_path: str = LIB) -> int:
    return load(lib_path).oracle_threads(threads)


def offset_mask(x, weight_om, bias_om=None, stride=1, padding=0, dilation=1, groups=1, threads=0,
                lib_path: str = LIB):
    """The offset/mask branch of DCNv2 (csdn.net tags page "可变形卷积：Deformable ConvNets",
    DCNv2 section 3.2: a separate regular convolution of the same input, at the layer's
    resolution, with 3K^2 outputs per offset group; the first 2K^2 are the offsets, the
    rest go through a sigmoid and are the modulation scalars).

    A regular convolution is the deformable one with zero offsets and no mask, so this
    is the oracle's forward with a zero offset field, followed by the channel split and
    a sigmoid written out in float64.  Returns (offset [B, 2GK^2, Ho, Wo], mask
    [B, GK^2, Ho, Wo], sum of |terms| of the convolution [B, 3GK^2, Ho, Wo])."""
    w = _f32(weight_om)
    K = w.shape[2]
    KK = K * K
    if w.shape[0] != 3 * groups * KK:
        raise ValueError(f"weight_om must have 3*G*K*K = {3 * groups * KK} output channels")
    xs = _f32(x)
    B, _, H, W = xs.shape
    Ho, Wo = output_hw(B, xs.shape[1], H, W, w.shape[0], K, stride, padding, dilation, lib_path)
    zero = np.zeros((B, 2 * KK, Ho, Wo), dtype=np.float32)
    y, a = forward(xs, zero, w, bias_om, stride, padding, dilation, mask=None, threads=threads,
                   lib_path=lib_path)
    n_off = 2 * groups * KK
    return y[:, :n_off], 1.0 / (1.0 + np.exp(-y[:, n_off:])), a
