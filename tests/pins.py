"""Checks that pin the CPU oracle to facts fixed outside itself.

Each ``pin_*`` function raises AssertionError when the oracle library at
``lib`` disagrees with what the pages and the mathematics fix.  The tests run
them against the real oracle (all must pass) and against copies of the oracle
with a mistake planted on purpose (at least one must fail for each).

What each pin reduces to (no pin restates the oracle's own formula):
  p1  zero offsets, mask 1   -> a separate direct-convolution loop and torch conv2d
  p2  integer offsets        -> shifted convolution by integer indexing
  p3  bilinear input field   -> closed form alpha+beta*y+gamma*x+delta*x*y at the position
  p4  every sample outside   -> bias exactly
  p5  linear in the mask     -> homogeneity and additivity
  p6  mask absent            -> identical to mask of ones
  p7  offsets (+.5, +.5)     -> mean of the four neighbours
  p8  constant input         -> C * sum of W*m, plus bias
  p9  general offsets        -> torch grid_sample (bilinear, zero padding, align_corners)
                                per kernel point, then a contraction with W
  p10 NaN / Inf / 1e30 offsets -> that sample contributes zero
  p11 offset groups           -> the sum over groups of one-group problems (each channel slice
                                with its own offset and mask slice) via the grid_sample
                                formulation; G copies of one offset field -> one group
  p12 offset/mask branch      -> torch conv2d (float64) split into 2GK^2 offset channels and
                                the sigmoid of the other GK^2
  p13 gradients               -> differences of sum(gy * y) from the FORWARD oracle: exact
                                along x, weight, mask, bias (linear); central differences
                                along the offsets inside a cell (bilinear), G = 1 and 2
  p14 gradients, zero offsets  -> torch autograd of conv2d (float64); unfold for the mask
                                gradient; one-sided input differences for the offsets
  p15 gradients, all outside   -> zero, except the bias gradient sum(gy)
  p16 RoI pooling, pixel bins   -> the input pixels (moved RoI, whole-pixel offsets, batch image)
  p17 RoI pooling, linear field -> the field at the shifted bin centre times the mask, any S
  p18 RoI pooling, outside      -> zeros; a constant image gives the constant times the mask
  p19 PS RoI pooling, constant score maps -> bin (i, j) of channel c reads map (c*k+i)*k+j only
  p20 PS RoI pooling, replicated maps     -> plain deformable RoI pooling (p16-p18), per offset group
  p21 PS RoI pooling, pixel bins          -> the score maps' pixels; past the batch -> zeros
  golden                      -> hand-worked examples in tests/golden/
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def out_hw(H, W, K, s, p, d):
    """Output size of a regular strided convolution (textbook formula)."""
    return (H + 2 * p - d * (K - 1) - 1) // s + 1, (W + 2 * p - d * (K - 1) - 1) // s + 1


def rand_case(rng, B, Cin, H, W, Cout, K, s, p, d, offset_scale=1.5, mask=True, bias=True):
    Ho, Wo = out_hw(H, W, K, s, p, d)
    x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
    w = rng.standard_normal((Cout, Cin, K, K)).astype(np.float32)
    off = (rng.standard_normal((B, 2 * K * K, Ho, Wo)) * offset_scale).astype(np.float32)
    m = rng.uniform(0.0, 1.0, (B, K * K, Ho, Wo)).astype(np.float32) if mask else None
    b = rng.standard_normal(Cout).astype(np.float32) if bias else None
    return x, off, m, w, b, Ho, Wo


def direct_conv(x, w, b, s, p, d):
    """Regular convolution, written as the textbook loop on a zero-padded input."""
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    Ho, Wo = out_hw(H, W, K, s, p, d)
    xp = np.zeros((B, Cin, H + 2 * p, W + 2 * p))
    xp[:, :, p:p + H, p:p + W] = x
    y = np.zeros((B, Cout, Ho, Wo))
    for oy in range(Ho):
        for ox in range(Wo):
            patch = xp[:, :, oy * s:oy * s + d * (K - 1) + 1:d, ox * s:ox * s + d * (K - 1) + 1:d]
            y[:, :, oy, ox] = np.einsum("bcij,ocij->bo", patch, w.astype(np.float64))
    if b is not None:
        y += b[None, :, None, None]
    return y


def _close(a, b, tol, what):
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.1e}"


def pin_p1_zero_offsets(lib):
    rng = np.random.default_rng(11)
    for K in (1, 3, 5):
        for s in (1, 2, 3):
            for p in (0, 1, 2):
                for d in (1, 2):
                    H, W = 9, 8
                    if out_hw(H, W, K, s, p, d)[0] < 1 or out_hw(H, W, K, s, p, d)[1] < 1:
                        continue
                    x, off, _, w, b, Ho, Wo = rand_case(rng, 2, 3, H, W, 4, K, s, p, d)
                    off[:] = 0.0
                    y = oracle.forward(x, off, w, b, s, p, d, mask=None, with_abs=False, lib_path=lib)
                    _close(y, direct_conv(x, w, b, s, p, d), 1e-12, f"p1 loop K{K} s{s} p{p} d{d}")
                    ref = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                                   torch.from_numpy(b).double(), stride=s, padding=p, dilation=d)
                    _close(y, ref.numpy(), 1e-12, f"p1 conv2d K{K} s{s} p{p} d{d}")


def pin_p2_integer_offsets(lib):
    rng = np.random.default_rng(12)
    for (K, s, p, d) in [(3, 1, 1, 1), (3, 2, 1, 1), (2, 1, 0, 2), (3, 1, 2, 2)]:
        B, Cin, H, W, Cout = 2, 3, 7, 9, 3
        x, _, m, w, b, Ho, Wo = rand_case(rng, B, Cin, H, W, Cout, K, s, p, d)
        off = rng.integers(-3, 4, (B, 2 * K * K, Ho, Wo)).astype(np.float32)
        y, a = oracle.forward(x, off, w, b, s, p, d, mask=m, lib_path=lib)
        # shifted convolution: read the integer position from a zero-padded copy
        M = 3 + p + d * K + 1
        xp = np.zeros((B, Cin, H + 2 * M, W + 2 * M))
        xp[:, :, M:M + H, M:M + W] = x
        ref = np.zeros((B, Cout, Ho, Wo))
        ref_abs = np.zeros((B, Cout, Ho, Wo))
        oy, ox = np.meshgrid(np.arange(Ho), np.arange(Wo), indexing="ij")
        for bb in range(B):
            for k in range(K * K):
                i, j = divmod(k, K)
                yy = oy * s - p + i * d + off[bb, 2 * k].astype(np.int64)
                xx = ox * s - p + j * d + off[bb, 2 * k + 1].astype(np.int64)
                vals = xp[bb][:, yy + M, xx + M]                        # [Cin, Ho, Wo]
                wk, mk = w[:, :, i, j].astype(np.float64), m[bb, k].astype(np.float64)
                ref[bb] += np.einsum("chw,oc,hw->ohw", vals, wk, mk)
                ref_abs[bb] += np.einsum("chw,oc,hw->ohw", np.abs(vals), np.abs(wk), np.abs(mk))
        ref += b[None, :, None, None]
        ref_abs += np.abs(b)[None, :, None, None]
        _close(y, ref, 1e-12, f"p2 K{K} s{s} p{p} d{d}")
        _close(a, ref_abs, 1e-12, f"p2 sum of |terms| K{K} s{s} p{p} d{d}")


def pin_p3_bilinear_field(lib):
    """X = a + b*y + c*x + e*x*y is reproduced exactly by bilinear interpolation."""
    rng = np.random.default_rng(13)
    B, Cin, H, W, Cout, K, s, p, d = 1, 2, 12, 13, 3, 3, 1, 0, 2
    Ho, Wo = out_hw(H, W, K, s, p, d)
    coef = rng.integers(-2, 3, (Cin, 4)).astype(np.float64)
    yy, xx = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    x = np.stack([c[0] + c[1] * yy + c[2] * xx + c[3] * xx * yy for c in coef])[None].astype(np.float32)
    w = rng.integers(-3, 4, (Cout, Cin, K, K)).astype(np.float32)
    m = (rng.integers(0, 5, (B, K * K, Ho, Wo)) / 4.0).astype(np.float32)
    ref = np.zeros((B, Cout, Ho, Wo))
    oy, ox = np.meshgrid(np.arange(Ho), np.arange(Wo), indexing="ij")
    off = np.zeros((B, 2 * K * K, Ho, Wo), dtype=np.float32)
    for k in range(K * K):
        i, j = divmod(k, K)
        by, bx = oy * s - p + i * d, ox * s - p + j * d
        # dyadic offsets keeping the position inside [0,H-1] x [0,W-1]
        py = np.clip(by + rng.integers(-96, 97, by.shape) / 64.0, 0, H - 1)
        px = np.clip(bx + rng.integers(-96, 97, bx.shape) / 64.0, 0, W - 1)
        off[0, 2 * k], off[0, 2 * k + 1] = py - by, px - bx
        field = np.stack([c[0] + c[1] * py + c[2] * px + c[3] * px * py for c in coef])   # [Cin,Ho,Wo]
        ref[0] += np.einsum("chw,oc,hw->ohw", field, w[:, :, i, j].astype(np.float64), m[0, k])
    y = oracle.forward(x, off, w, None, s, p, d, mask=m, with_abs=False, lib_path=lib)
    _close(y, ref, 1e-12, "p3 bilinear field")


def pin_p4_all_outside(lib):
    rng = np.random.default_rng(14)
    H, W = 6, 7
    x, off, m, w, b, Ho, Wo = rand_case(rng, 2, 3, H, W, 4, 3, 1, 1, 1)
    bias = np.broadcast_to(b.astype(np.float64)[None, :, None, None], (2, 4, Ho, Wo))
    for dy, dx in ((100.25, None), (None, -100.25), (-11.0, None), (None, 3e4)):
        o = off.copy()
        if dy is not None:
            o[:, 0::2] = dy
        if dx is not None:
            o[:, 1::2] = dx
        y, a = oracle.forward(x, o, w, b, 1, 1, 1, mask=m, lib_path=lib)
        assert np.array_equal(y, bias), f"p4 dy={dy} dx={dx}: output is not the bias"
        assert np.array_equal(a, np.abs(bias)), f"p4 dy={dy} dx={dx}: abs terms are not |bias|"
    # every row position exactly H (one past the last row) or exactly -1: the sample is zero
    for target in (float(H), -1.0):
        o = off.copy()
        oy = np.arange(Ho)[None, :, None]
        for k in range(9):
            i = k // 3
            o[:, 2 * k] = (target - (oy - 1 + i)).astype(np.float32)
        y = oracle.forward(x, o, w, b, 1, 1, 1, mask=m, with_abs=False, lib_path=lib)
        assert np.array_equal(y, bias), f"p4 row position exactly {target}: must contribute zero"


def pin_p5_linear_in_mask(lib):
    rng = np.random.default_rng(15)
    x, off, m, w, b, Ho, Wo = rand_case(rng, 1, 4, 8, 9, 3, 3, 2, 1, 1)
    m2 = rng.uniform(0, 1, m.shape).astype(np.float32)
    f = lambda mm: oracle.forward(x, off, w, b, 2, 1, 1, mask=mm, with_abs=False, lib_path=lib)
    bb = b.astype(np.float64)[None, :, None, None]
    y1, y2, y12 = f(m), f(m2), f((m.astype(np.float64) + m2).astype(np.float32))
    msum_exact = np.array_equal((m.astype(np.float64) + m2).astype(np.float32).astype(np.float64),
                                m.astype(np.float64) + m2)
    y2m = f(2.0 * m)
    _close(y2m - bb, 2.0 * (y1 - bb), 1e-12, "p5 homogeneity")
    if msum_exact:
        _close(y12 - bb, (y1 - bb) + (y2 - bb), 1e-12, "p5 additivity")
    else:
        _close(y12 - bb, (y1 - bb) + (y2 - bb), 1e-6, "p5 additivity (rounded mask sum)")
    y0 = f(np.zeros_like(m))
    assert np.array_equal(y0, np.broadcast_to(bb, y0.shape)), "p5 mask 0 must give the bias"


def pin_p6_mask_absent(lib):
    rng = np.random.default_rng(16)
    x, off, m, w, b, Ho, Wo = rand_case(rng, 2, 3, 7, 8, 3, 3, 1, 1, 1)
    y_none, a_none = oracle.forward(x, off, w, b, 1, 1, 1, mask=None, lib_path=lib)
    y_one, a_one = oracle.forward(x, off, w, b, 1, 1, 1, mask=np.ones_like(m), lib_path=lib)
    assert np.array_equal(y_none, y_one) and np.array_equal(a_none, a_one), "p6 mask None != ones"


def pin_p7_half_offsets(lib):
    rng = np.random.default_rng(17)
    B, Cin, H, W, Cout, K, s, p, d = 1, 3, 8, 9, 2, 3, 1, 0, 1
    x, off, m, w, b, Ho, Wo = rand_case(rng, B, Cin, H, W, Cout, K, s, p, d)
    off[:] = 0.5
    # choose an output region whose every neighbour is inside (pad 0 and one-pixel margin)
    y = oracle.forward(x, off, w, b, s, p, d, mask=m, with_abs=False, lib_path=lib)
    xd = x.astype(np.float64)
    mean4 = (xd[:, :, :-1, :-1] + xd[:, :, 1:, :-1] + xd[:, :, :-1, 1:] + xd[:, :, 1:, 1:]) / 4.0
    ref = np.zeros_like(y)
    for k in range(K * K):
        i, j = divmod(k, K)
        hh, ww = min(Ho, mean4.shape[2] - i), min(Wo, mean4.shape[3] - j)
        ref[:, :, :hh, :ww] += np.einsum("bchw,oc,bhw->bohw", mean4[:, :, i:i + hh, j:j + ww],
                                         w[:, :, i, j].astype(np.float64), m[:, k, :hh, :ww])
    ref += b[None, :, None, None]
    hh, ww = H - 1 - (K - 1), W - 1 - (K - 1)
    _close(y[:, :, :hh, :ww], ref[:, :, :hh, :ww], 1e-12, "p7 half-pixel mean")


def pin_p8_constant_input(lib):
    rng = np.random.default_rng(18)
    B, Cin, H, W, Cout, K, s, p, d = 2, 3, 10, 11, 4, 3, 1, 0, 1
    x, off, m, w, b, Ho, Wo = rand_case(rng, B, Cin, H, W, Cout, K, s, p, d)
    C = 1.75
    x[:] = C
    oy, ox = np.meshgrid(np.arange(Ho), np.arange(Wo), indexing="ij")
    for k in range(K * K):   # keep every position inside
        i, j = divmod(k, K)
        by, bx = oy * s - p + i * d, ox * s - p + j * d
        off[:, 2 * k] = np.clip(by + off[:, 2 * k], 0, H - 1) - by
        off[:, 2 * k + 1] = np.clip(bx + off[:, 2 * k + 1], 0, W - 1) - bx
    y = oracle.forward(x, off, w, b, s, p, d, mask=m, with_abs=False, lib_path=lib)
    wk = w.reshape(Cout, Cin, K * K).astype(np.float64).sum(1)          # [Cout, K^2]
    ref = C * np.einsum("ok,bkhw->bohw", wk, m.astype(np.float64)) + b[None, :, None, None]
    _close(y, ref, 1e-12, "p8 constant input")


def grid_sample_formulation(x, off, m, w, b, s, p, d):
    """The whole operation via torch grid_sample (bilinear, zeros, align_corners=True)."""
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    Ho, Wo = off.shape[2:]
    xt = torch.from_numpy(x).double()
    y = torch.zeros((B, Cout, Ho, Wo), dtype=torch.float64)
    oy, ox = torch.meshgrid(torch.arange(Ho, dtype=torch.float64),
                            torch.arange(Wo, dtype=torch.float64), indexing="ij")
    for k in range(K * K):
        i, j = divmod(k, K)
        py = oy * s - p + i * d + torch.from_numpy(off[:, 2 * k]).double()
        px = ox * s - p + j * d + torch.from_numpy(off[:, 2 * k + 1]).double()
        grid = torch.stack([2.0 * px / (W - 1) - 1.0, 2.0 * py / (H - 1) - 1.0], dim=-1)
        smp = F.grid_sample(xt, grid, mode="bilinear", padding_mode="zeros", align_corners=True)
        if m is not None:
            smp = smp * torch.from_numpy(m[:, k]).double()[:, None]
        y += torch.einsum("bchw,oc->bohw", smp, torch.from_numpy(w[:, :, i, j]).double())
    if b is not None:
        y += torch.from_numpy(b).double()[None, :, None, None]
    return y.numpy()


def pin_p9_grid_sample(lib, cases=None):
    rng = np.random.default_rng(19)
    if cases is None:
        cases = [(1, 3, 5, 6, 2, 3, 1, 1, 1), (2, 4, 9, 7, 3, 3, 2, 1, 1), (1, 2, 8, 8, 3, 5, 1, 2, 1),
                 (2, 3, 11, 10, 4, 3, 1, 2, 2), (1, 5, 6, 9, 2, 2, 3, 0, 1), (1, 3, 2, 2, 2, 1, 1, 0, 1)]
    for (B, Cin, H, W, Cout, K, s, p, d) in cases:
        for mask in (True, False):
            x, off, m, w, b, Ho, Wo = rand_case(rng, B, Cin, H, W, Cout, K, s, p, d,
                                                 offset_scale=2.5, mask=mask, bias=mask)
            y = oracle.forward(x, off, w, b, s, p, d, mask=m, with_abs=False, lib_path=lib)
            ref = grid_sample_formulation(x, off, m, w, b, s, p, d)
            _close(y, ref, 1e-10, f"p9 {(B, Cin, H, W, Cout, K, s, p, d)} mask={mask}")


def pin_p10_nonfinite_offsets(lib):
    rng = np.random.default_rng(20)
    x, off, m, w, b, Ho, Wo = rand_case(rng, 2, 3, 7, 8, 3, 3, 1, 1, 1)
    bad = rng.uniform(size=(2, 9, Ho, Wo)) < 0.3
    specials = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, 3e38], dtype=np.float32)
    o = off.copy()
    pick = rng.integers(0, len(specials), bad.shape)
    which = rng.integers(0, 3, bad.shape)    # 0: dy bad, 1: dx bad, 2: both
    for k in range(9):
        sel = bad[:, k]
        val = specials[pick[:, k]]
        o[:, 2 * k][sel & (which[:, k] != 1)] = val[sel & (which[:, k] != 1)]
        o[:, 2 * k + 1][sel & (which[:, k] != 0)] = val[sel & (which[:, k] != 0)]
    m0 = m.copy()
    m0[bad] = 0.0
    y_bad, a_bad = oracle.forward(x, o, w, b, 1, 1, 1, mask=m, lib_path=lib)
    y_ref, a_ref = oracle.forward(x, off, w, b, 1, 1, 1, mask=m0, lib_path=lib)
    assert np.all(np.isfinite(y_bad)), "p10: non-finite offsets leaked into the output"
    _close(y_bad, y_ref, 1e-12, "p10 non-finite offsets contribute zero")
    _close(a_bad, a_ref, 1e-12, "p10 abs terms")


def pin_p11_offset_groups(lib):
    rng = np.random.default_rng(21)
    cases = [(2, 6, 3, 7, 8, 4, 3, 1, 1, 1), (1, 4, 2, 9, 6, 3, 2, 2, 0, 1), (2, 4, 4, 6, 7, 2, 3, 1, 2, 2)]
    for (B, Cin, G, H, W, Cout, K, s, p, d) in cases:
        KK = K * K
        Cg = Cin // G
        for mask in (True, False):
            x, _, _, w, b, Ho, Wo = rand_case(rng, B, Cin, H, W, Cout, K, s, p, d, mask=mask, bias=mask)
            off = (rng.standard_normal((B, 2 * KK * G, Ho, Wo)) * 2.0).astype(np.float32)
            m = rng.uniform(0.0, 1.0, (B, KK * G, Ho, Wo)).astype(np.float32) if mask else None
            y = oracle.forward(x, off, w, b, s, p, d, mask=m, with_abs=False, lib_path=lib)
            # channels [g*Cg, (g+1)*Cg) use offset channels [2*KK*g, 2*KK*(g+1)) and mask [KK*g, KK*(g+1))
            ref = b[None, :, None, None].astype(np.float64) if b is not None else 0.0
            for g in range(G):
                ref = ref + grid_sample_formulation(
                    x[:, g * Cg:(g + 1) * Cg], off[:, 2 * KK * g:2 * KK * (g + 1)],
                    None if m is None else m[:, KK * g:KK * (g + 1)], w[:, g * Cg:(g + 1) * Cg], None, s, p, d)
            _close(y, ref, 1e-10, f"p11 groups {(B, Cin, G, H, W, Cout, K, s, p, d)} mask={mask}")
            # every group given the same field: the one-group result, exactly
            off1, m1 = off[:, :2 * KK], None if m is None else m[:, :KK]
            yg = oracle.forward(x, np.tile(off1, (1, G, 1, 1)), w, b, s, p, d,
                                mask=None if m1 is None else np.tile(m1, (1, G, 1, 1)), with_abs=False, lib_path=lib)
            y1 = oracle.forward(x, off1, w, b, s, p, d, mask=m1, with_abs=False, lib_path=lib)
            assert np.array_equal(yg, y1), "p11 replicated groups differ from one group"


def pin_p12_offset_mask_branch(lib):
    rng = np.random.default_rng(22)
    for (B, Cin, H, W, K, s, p, d, G) in [(2, 5, 9, 11, 3, 1, 1, 1, 1), (1, 4, 12, 10, 3, 2, 1, 1, 2),
                                          (2, 3, 8, 9, 1, 1, 0, 1, 1), (1, 6, 13, 12, 3, 1, 2, 2, 3)]:
        KK = K * K
        x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
        w = rng.standard_normal((3 * G * KK, Cin, K, K)).astype(np.float32)
        b = rng.standard_normal(3 * G * KK).astype(np.float32)
        off, msk, _ = oracle.offset_mask(x, w, b, s, p, d, groups=G, lib_path=lib)
        ref = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                       stride=s, padding=p, dilation=d).numpy()
        _close(off, ref[:, :2 * G * KK], 1e-12, f"p12 offsets {(B, Cin, H, W, K, s, p, d, G)}")
        _close(msk, torch.sigmoid(torch.from_numpy(ref[:, 2 * G * KK:])).numpy(), 1e-12,
               f"p12 mask {(B, Cin, H, W, K, s, p, d, G)}")


def pin_golden(lib):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], dtype=np.float32)[None, None]
    for ex in g["examples"]:
        K = ex["K"]
        Ho, Wo = out_hw(3, 3, K, ex["stride"], ex["pad"], ex["dilation"])
        w = np.array(ex["weight"], dtype=np.float32)
        b = None if ex["bias"] is None else np.array(ex["bias"], dtype=np.float32)
        off = np.zeros((1, 2 * K * K, Ho, Wo), dtype=np.float32)
        if "offset_dy" in ex:
            off[0, 0] = ex["offset_dy"]
            off[0, 1] = ex["offset_dx"]
        else:
            for k in range(K * K):
                off[0, 2 * k, 0, 0] = ex["offset_at_00"][f"k{k}_dy"]
                off[0, 2 * k + 1, 0, 0] = ex["offset_at_00"][f"k{k}_dx"]
        m = None if ex["mask"] is None else np.array(ex["mask"], dtype=np.float32)[None, None]
        y, a = oracle.forward(x, off, w, b, ex["stride"], ex["pad"], ex["dilation"], mask=m, lib_path=lib)
        assert np.array_equal(y[0, 0], np.array(ex["expected_y"])), f"golden {ex['name']}: {y[0, 0]}"
        assert np.array_equal(a[0, 0], np.array(ex["expected_abs"])), f"golden {ex['name']} abs"


def _off_cells(rng, B, KKG, Ho, Wo):
    """Offsets whose sampling positions sit inside a cell, at least 0.1 from its edges:
    an integer part plus a fraction in [0.1, 0.9] (the base positions are integers)."""
    whole = np.round(rng.standard_normal((B, 2 * KKG, Ho, Wo)) * 1.5)
    return (whole + rng.uniform(0.1, 0.9, whole.shape)).astype(np.float32)


def _loss(lib, x, off, m, w, b, gy, s, p, d):
    """L = sum(gy * y) with the oracle's forward (float64)."""
    y = oracle.forward(x, off, w, b, s, p, d, mask=m, with_abs=False, lib_path=lib)
    return float(np.sum(gy.astype(np.float64) * y))


def pin_p13_backward_directional(lib):
    """Gradients against differences of L = sum(gy * y) computed by the FORWARD oracle.
    L is linear in x, weight, mask and bias, so L(v + D) - L(v) = <grad, D> exactly for
    any perturbation D (taken as the float32 difference actually applied).  Along the
    offsets L is bilinear inside a cell, so the central difference (L(+D) - L(-D)) / 2
    equals <grad, D> up to the float32 rounding of the two perturbed fields."""
    for G, (B, Cin, H, W, Cout, K, s, p, d) in ((1, (2, 3, 6, 7, 4, 3, 1, 1, 1)),
                                                  (2, (1, 4, 7, 6, 3, 3, 2, 1, 1)),
                                                  (1, (1, 2, 8, 7, 3, 2, 1, 0, 2))):
        rng = np.random.default_rng(1300 + G * 10 + K)
        Ho, Wo = out_hw(H, W, K, s, p, d)
        x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
        w = rng.standard_normal((Cout, Cin, K, K)).astype(np.float32)
        b = rng.standard_normal(Cout).astype(np.float32)
        off = _off_cells(rng, B, G * K * K, Ho, Wo)
        m = rng.uniform(0.1, 1.0, (B, G * K * K, Ho, Wo)).astype(np.float32)
        gy = rng.standard_normal((B, Cout, Ho, Wo)).astype(np.float32)
        r = oracle.backward(x, off, w, gy, s, p, d, mask=m, lib_path=lib)
        L0 = _loss(lib, x, off, m, w, b, gy, s, p, d)
        scale = 1.0 + abs(L0)

        def lin(name, arr, grad, make):
            v = rng.standard_normal(arr.shape)
            moved = (arr + 0.5 * v).astype(np.float32)
            D = moved.astype(np.float64) - arr.astype(np.float64)
            got = _loss(lib, *make(moved)) - L0
            want = float(np.sum(grad * D))
            # the backward rounds positions to float32 (the forward keeps them in double):
            # sample values then differ by about 1e-7 of their size
            tol = 1e-5 * float(np.sum(np.abs(grad * D))) + 1e-9 * scale
            assert abs(got - want) <= tol, f"G={G} {name}: {got} vs {want}"

        lin("x", x, r["grad_x"], lambda a: (a, off, m, w, b, gy, s, p, d))
        lin("weight", w, r["grad_weight"], lambda a: (x, off, m, a, b, gy, s, p, d))
        lin("mask", m, r["grad_mask"], lambda a: (x, off, a, w, b, gy, s, p, d))
        lin("bias", b, r["grad_bias"], lambda a: (x, off, m, w, a, gy, s, p, d))
        v = rng.uniform(-1.0, 1.0, off.shape) * 0.02
        op = (off + v).astype(np.float32)
        om = (off - v).astype(np.float32)
        Dp = op.astype(np.float64) - off.astype(np.float64)
        Dm = off.astype(np.float64) - om.astype(np.float64)
        got = (_loss(lib, x, op, m, w, b, gy, s, p, d) - _loss(lib, x, om, m, w, b, gy, s, p, d))
        want = float(np.sum(r["grad_offset"] * (Dp + Dm)))
        tol = 1e-5 * float(np.sum(np.abs(r["grad_offset"] * (Dp + Dm)))) + 1e-9 * scale
        assert abs(got - want) <= tol, f"G={G} offset: {got} vs {want}"
        # every offset channel on its own (a sign or an axis swap in one channel shows here)
        for ch in (0, 1, 2 * G * K * K - 1):
            v1 = np.zeros_like(off)
            v1[:, ch] = 0.01
            op = (off + v1).astype(np.float32)
            om = (off - v1).astype(np.float32)
            D = (op.astype(np.float64) - om.astype(np.float64))
            got = _loss(lib, x, op, m, w, b, gy, s, p, d) - _loss(lib, x, om, m, w, b, gy, s, p, d)
            want = float(np.sum(r["grad_offset"] * D))
            tol = 1e-5 * float(np.sum(np.abs(r["grad_offset"] * D))) + 1e-9 * scale
            assert abs(got - want) <= tol, f"G={G} offset channel {ch}: {got} vs {want}"


def pin_p14_backward_zero_offsets(lib):
    """Zero offsets: the gradients of a regular convolution from torch autograd of
    F.conv2d in float64 (x, weight, bias); the mask gradient from torch's unfold (the
    column of each kernel point times the column gradient W^T gy); the offset gradient
    at these integer positions from the one-sided difference X[y+1] - X[y] (and
    X[x+1] - X[x]) of the zero-padded input, since S(y + t) = (1-t) X[y] + t X[y+1]."""
    rng = np.random.default_rng(1401)
    B, Cin, H, W, Cout, K, s, p, d = 2, 3, 7, 6, 4, 3, 2, 1, 1
    Ho, Wo = out_hw(H, W, K, s, p, d)
    x = rng.standard_normal((B, Cin, H, W)).astype(np.float32)
    w = rng.standard_normal((Cout, Cin, K, K)).astype(np.float32)
    gy = rng.standard_normal((B, Cout, Ho, Wo)).astype(np.float32)
    off = np.zeros((B, 2 * K * K, Ho, Wo), dtype=np.float32)
    m = rng.uniform(0.1, 1.0, (B, K * K, Ho, Wo)).astype(np.float32)
    r = oracle.backward(x, off, w, gy, s, p, d, mask=None, lib_path=lib)
    xt = torch.from_numpy(x).double().requires_grad_()
    wt = torch.from_numpy(w).double().requires_grad_()
    bt = torch.zeros(Cout, dtype=torch.float64, requires_grad=True)
    y = F.conv2d(xt, wt, bt, stride=s, padding=p, dilation=d)
    y.backward(torch.from_numpy(gy).double())
    _close(r["grad_x"], xt.grad.numpy(), 1e-10, "grad_x vs conv2d")
    _close(r["grad_weight"], wt.grad.numpy(), 1e-10, "grad_weight vs conv2d")
    _close(r["grad_bias"], bt.grad.numpy(), 1e-10, "grad_bias vs conv2d")
    # column gradient per (c, k) and the columns themselves (unfold zero-pads)
    gcol = np.einsum("ocij,bopq->bcijpq", w.astype(np.float64), gy.astype(np.float64)).reshape(B, Cin, K * K, Ho, Wo)
    cols = F.unfold(torch.from_numpy(x).double(), K, dilation=d, padding=p, stride=s).numpy()
    cols = cols.reshape(B, Cin, K * K, Ho, Wo)
    rm = oracle.backward(x, off, w, gy, s, p, d, mask=m, lib_path=lib)
    _close(rm["grad_mask"], np.sum(gcol * cols, axis=1), 1e-10, "grad_mask vs unfold")
    # offsets: one-sided differences of the zero-padded input, one row/column past the pad
    xp = np.zeros((B, Cin, H + 2 * p + 2, W + 2 * p + 2))
    xp[:, :, p:p + H, p:p + W] = x
    want = np.zeros((B, 2 * K * K, Ho, Wo))
    for i in range(K):
        for j in range(K):
            k = i * K + j
            ys = np.arange(Ho) * s + i * d          # row of the sample in padded coordinates
            xs = np.arange(Wo) * s + j * d
            X0 = xp[:, :, ys][:, :, :, xs]
            Xdy = xp[:, :, ys + 1][:, :, :, xs]
            Xdx = xp[:, :, ys][:, :, :, xs + 1]
            mk = m[:, k][:, None].astype(np.float64)
            want[:, 2 * k] = np.sum(gcol[:, :, k] * mk * (Xdy - X0), axis=1)
            want[:, 2 * k + 1] = np.sum(gcol[:, :, k] * mk * (Xdx - X0), axis=1)
    _close(rm["grad_offset"], want, 1e-10, "grad_offset at integer positions")


def pin_p15_backward_all_outside(lib):
    """Every sample far outside the image: the output is the bias alone, so every
    gradient is zero except the bias's, which is the sum of gy."""
    rng = np.random.default_rng(1501)
    x, off, m, w, b, Ho, Wo = rand_case(rng, 2, 3, 5, 6, 4, 3, 1, 1, 1)
    off = np.full_like(off, 1.0e3)
    gy = rng.standard_normal((2, 4, Ho, Wo)).astype(np.float32)
    r = oracle.backward(x, off, w, gy, 1, 1, 1, mask=m, lib_path=lib)
    for k in ("grad_x", "grad_offset", "grad_mask", "grad_weight"):
        assert np.all(r[k] == 0.0), f"{k} not zero with every sample outside"
    _close(r["grad_bias"], gy.astype(np.float64).sum(axis=(0, 2, 3)), 1e-12, "grad_bias")


def pin_p16_roi_pixel_bins(lib):
    """RoI pooling with one sample per bin on a RoI whose bins are single pixels: the
    output is the input pixels themselves, also for a RoI moved by whole pixels, for
    bin offsets worth whole pixels (gamma * size * offset an integer), and for the
    RoI's own batch image; spatial_scale maps image coordinates to the feature grid."""
    rng = np.random.default_rng(1601)
    B, C, H, W, k = 2, 3, 11, 13, 4
    x = rng.standard_normal((B, C, H, W)).astype(np.float32)
    # image coordinates at scale 0.5: bins [2j-1, 2j+1) map to pixel j
    rois = np.array([[0, -1, -1, 2 * k - 1, 2 * k - 1],
                     [1, -1 + 2 * 3, -1 + 2 * 2, 2 * k - 1 + 2 * 3, 2 * k - 1 + 2 * 2]], dtype=np.float32)
    y, ya = oracle.roi_pool(x, rois, k, 1, spatial_scale=0.5, with_abs=True, lib_path=lib)
    _close(y[0], x[0, :, 0:k, 0:k], 1e-12, "pixel bins")
    _close(y[1], x[1, :, 2:2 + k, 3:3 + k], 1e-12, "pixel bins moved by (2, 3)")
    # one term per output (the pixel itself): the sum of |terms| is |pixel|
    _close(ya[0], np.abs(x[0, :, 0:k, 0:k]), 1e-12, "sum of |terms| of pixel bins")
    # offsets of n whole pixels: gamma * k * off = n with gamma 0.1, k 4 -> off = 2.5 n
    off = np.zeros((2, 2, k, k), dtype=np.float32)
    off[:, 0] = 2.5 * 1    # one row down
    off[:, 1] = 2.5 * -1   # one column left
    y, ya = oracle.roi_pool(x, rois, k, 1, spatial_scale=0.5, gamma=0.1, offset=off, with_abs=True, lib_path=lib)
    want0 = np.zeros((C, k, k))
    want0[:, :, 1:] = x[0, :, 1:k + 1, 0:k - 1]   # column -1 is outside: zero
    _close(y[0], want0, 1e-12, "whole-pixel bin offsets")
    _close(ya[0], np.abs(want0), 1e-12, "sum of |terms| with whole-pixel bin offsets")
    _close(y[1], x[1, :, 3:3 + k, 2:2 + k], 1e-12, "whole-pixel bin offsets, moved RoI")


def pin_p17_roi_linear_field(lib):
    """On a linear field X = a + b*y + c*x every bilinear sample is exact and the mean of
    the S x S sub-cell centres is the bin centre, so each output is m times the field at
    the shifted bin centre: y1 + (i + 1/2) h/k + gamma h dy_hat (rows), likewise columns,
    for any S, non-square RoIs and both batch images."""
    rng = np.random.default_rng(1701)
    B, C, H, W, k, g = 2, 3, 40, 50, 3, 0.1
    a = rng.standard_normal((B, C))
    bb = rng.standard_normal((B, C))
    cc = rng.standard_normal((B, C))
    yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    x = (a[:, :, None, None] + bb[:, :, None, None] * yy + cc[:, :, None, None] * xx).astype(np.float32)
    # the field is stored in float32: the tolerance covers that rounding (about 1e-7 of 50)
    for S in (1, 2, 3):
        R = 6
        x1 = rng.uniform(8, 20, R)
        y1 = rng.uniform(8, 14, R)
        w = rng.uniform(4, 20, R)
        h = rng.uniform(4, 16, R)
        rois = np.stack([rng.integers(0, B, R), x1, y1, x1 + w, y1 + h], 1).astype(np.float32)
        off = rng.uniform(-0.5, 0.5, (R, 2, k, k)).astype(np.float32)
        m = rng.uniform(0.2, 1.0, (R, k, k)).astype(np.float32)
        out = oracle.roi_pool(x, rois, k, S, 1.0, g, off, m, lib_path=lib)
        r64 = rois.astype(np.float64)
        for r in range(R):
            bi = int(r64[r, 0])
            rw, rh = r64[r, 3] - r64[r, 1], r64[r, 4] - r64[r, 2]
            i = np.arange(k)[:, None]
            j = np.arange(k)[None, :]
            cy = r64[r, 2] + (i + 0.5) * rh / k + g * rh * off[r, 0].astype(np.float64)
            cx = r64[r, 1] + (j + 0.5) * rw / k + g * rw * off[r, 1].astype(np.float64)
            want = m[r][None].astype(np.float64) * (a[bi][:, None, None] + bb[bi][:, None, None] * cy[None]
                                                     + cc[bi][:, None, None] * cx[None])
            _close(out[r], want, 2e-5, f"linear field, S={S}, RoI {r}")


def pin_p18_roi_outside(lib):
    """A RoI far outside the image, or with a batch index outside [0, B), pools zeros;
    a constant image pools the constant times the mask inside."""
    rng = np.random.default_rng(1801)
    x = np.full((2, 2, 9, 9), 3.0, dtype=np.float32)
    rois = np.array([[0, 100, 100, 120, 130], [5, 1, 1, 6, 6], [-1, 1, 1, 6, 6], [1, 1, 1, 6, 7]], np.float32)
    m = rng.uniform(0.1, 1.0, (4, 2, 2)).astype(np.float32)
    y, ya = oracle.roi_pool(x, rois, 2, 2, mask=m, with_abs=True, lib_path=lib)
    assert np.all(y[:3] == 0.0), "RoIs outside the image or the batch must pool zeros"
    assert np.all(ya[:3] == 0.0), "RoIs outside the image or the batch have no terms"
    _close(y[3], 3.0 * np.broadcast_to(m[3].astype(np.float64), (2, 2, 2)), 1e-12, "constant image")
    # every term positive: the sum of |terms| is the output itself; with the image
    # negated the output changes sign and the sum does not
    _close(ya[3], y[3], 1e-12, "sum of |terms| of a positive image")
    yn, yan = oracle.roi_pool(-x, rois, 2, 2, mask=m, with_abs=True, lib_path=lib)
    _close(yn[3], -y[3], 1e-12, "negated image")
    _close(yan[3], ya[3], 1e-12, "sum of |terms| of a negated image")


def pin_p19_ps_roi_score_map_per_bin(lib):
    """Position-sensitive pooling: bin (i, j) of output channel c reads only score map
    (c*k + i)*k + j.  Every score map a distinct constant (per batch image) and every
    sample inside the image: each output is m times that constant (the bilinear weights
    of an inside sample sum to 1), for one and for two offset groups."""
    rng = np.random.default_rng(1901)
    B, C, H, W, k = 2, 3, 20, 24, 3
    vals = rng.permutation(B * C * k * k).astype(np.float32).reshape(B, C * k * k) / 8.0 + 0.125
    x = np.broadcast_to(vals[:, :, None, None], (B, C * k * k, H, W)).copy()
    R = 5
    x1 = rng.uniform(3, 8, R)
    y1 = rng.uniform(3, 7, R)
    rois = np.stack([rng.integers(0, B, R), x1, y1, x1 + rng.uniform(4, 10, R), y1 + rng.uniform(4, 9, R)],
                    1).astype(np.float32)
    m = rng.uniform(0.2, 1.0, (R, k, k)).astype(np.float32)
    for G in (1, 3):
        off = rng.uniform(-0.2, 0.2, (R, 2 * G, k, k)).astype(np.float32)
        y = oracle.ps_roi_pool(x, rois, k, 2, 1.0, 0.1, off, m, lib_path=lib)
        for r in range(R):
            b = int(rois[r, 0])
            want = vals[b].reshape(C, k, k).astype(np.float64) * m[r][None].astype(np.float64)
            _close(y[r], want, 1e-12, f"score map per bin, G={G}, RoI {r}")


def pin_p20_ps_roi_replicated_maps(lib):
    """With the k*k score maps of each output channel all equal to one plane z[c], the
    position-sensitive pooling is the plain deformable RoI pooling of z (pinned by
    p16-p18); with G offset groups, group g equals the plain pooling of its channel
    slice of z with offset channels 2g, 2g+1."""
    rng = np.random.default_rng(2001)
    B, C, H, W, k, S = 2, 4, 17, 21, 3, 2
    z = rng.standard_normal((B, C, H, W)).astype(np.float32)
    x = np.repeat(z, k * k, axis=1)   # channel (c*k + i)*k + j = z[c]
    R = 6
    x1 = rng.uniform(-4, 14, R)
    y1 = rng.uniform(-4, 10, R)
    rois = np.stack([rng.integers(0, B, R), x1, y1, x1 + rng.uniform(2, 12, R), y1 + rng.uniform(2, 10, R)],
                    1).astype(np.float32)
    m = rng.uniform(0.1, 1.0, (R, k, k)).astype(np.float32)
    for G in (1, 2):
        off = rng.uniform(-1.0, 1.0, (R, 2 * G, k, k)).astype(np.float32)
        y = oracle.ps_roi_pool(x, rois, k, S, 0.9, 0.2, off, m, lib_path=lib)
        Cg = C // G
        for g in range(G):
            want = oracle.roi_pool(z[:, g * Cg:(g + 1) * Cg], rois, k, S, 0.9, 0.2,
                                   np.ascontiguousarray(off[:, 2 * g:2 * g + 2]), m, lib_path=lib)
            _close(y[:, g * Cg:(g + 1) * Cg], want, 1e-12, f"replicated score maps, group {g} of {G}")


def pin_p21_ps_roi_pixel_bins_and_outside(lib):
    """One sample per bin on a RoI whose bins are single pixels: output (r, c, i, j) is
    pixel (y0 + i, x0 + j) of score map (c*k + i)*k + j; a RoI past the last batch image
    pools zeros (sum of |terms| zero too)."""
    rng = np.random.default_rng(2101)
    B, C, H, W, k = 2, 2, 9, 10, 3
    x = rng.standard_normal((B, C * k * k, H, W)).astype(np.float32)
    # scale 0.5: image coordinates [2j-1, 2j+1) map to pixel j
    rois = np.array([[1, -1 + 2 * 4, -1 + 2 * 2, 2 * k - 1 + 2 * 4, 2 * k - 1 + 2 * 2],
                     [2, 0, 0, 4, 4]], dtype=np.float32)
    y, ya = oracle.ps_roi_pool(x, rois, k, 1, 0.5, 0.1, None, None, with_abs=True, lib_path=lib)
    want = np.empty((C, k, k))
    for c in range(C):
        for i in range(k):
            for j in range(k):
                want[c, i, j] = x[1, (c * k + i) * k + j, 2 + i, 4 + j]
    _close(y[0], want, 1e-12, "pixel bins of the score maps")
    _close(ya[0], np.abs(want), 1e-12, "sum of |terms| of pixel bins")
    assert np.all(y[1] == 0.0) and np.all(ya[1] == 0.0), "a RoI past the last image pools zeros"


ALL_PINS = [pin_p1_zero_offsets, pin_p2_integer_offsets, pin_p3_bilinear_field, pin_p4_all_outside,
            pin_p5_linear_in_mask, pin_p6_mask_absent, pin_p7_half_offsets, pin_p8_constant_input,
            pin_p9_grid_sample, pin_p10_nonfinite_offsets, pin_p11_offset_groups, pin_p12_offset_mask_branch,
            pin_golden, pin_p13_backward_directional, pin_p14_backward_zero_offsets,
            pin_p15_backward_all_outside, pin_p16_roi_pixel_bins, pin_p17_roi_linear_field,
            pin_p18_roi_outside, pin_p19_ps_roi_score_map_per_bin, pin_p20_ps_roi_replicated_maps,
            pin_p21_ps_roi_pixel_bins_and_outside]
