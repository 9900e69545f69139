"""The HIP deformable RoI pooling (dcn_roi_pool through the C ABI) against the oracle,
element by element, on seeded inputs."""

import numpy as np
import pytest
import torch

import deformable_convolution_vision_amd as dcn
import oracle

pytestmark = pytest.mark.gpu

# |got - ref| <= tol * max|x| (the output is a weighted mean of input values)
TOL = {"f32": 1e-5, "bf16": 1e-2}

CASES = [
    # name, B, C, H, W, R, k, S, scale, gamma, offset, mask
    ("v1_no_offset", 2, 5, 17, 23, 9, 3, 2, 1.0, 0.1, False, False),
    ("v1_offsets", 2, 5, 17, 23, 9, 7, 2, 1.0, 0.1, True, False),
    ("v2_modulated", 1, 8, 20, 15, 12, 7, 2, 0.5, 0.1, True, True),
    ("scale_16", 2, 16, 25, 42, 20, 7, 3, 1.0 / 16, 0.1, True, True),
    ("one_sample", 1, 4, 9, 9, 6, 4, 1, 1.0, 0.2, True, True),
    ("large_gamma", 1, 3, 12, 14, 10, 5, 2, 1.0, 1.0, True, True),   # bins pushed past the image
    ("k1", 2, 6, 10, 10, 5, 1, 4, 1.0, 0.1, True, True),
    ("channels_70", 2, 70, 12, 16, 7, 5, 2, 0.5, 0.1, True, True),   # a partial 64-channel block
    ("k20_unstaged", 1, 4, 30, 30, 3, 20, 1, 1.0, 0.1, True, True),  # bf16 with k > 16: no staging
]


def make(B, C, H, W, R, k, S, scale, gamma, with_off, with_mask, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn((B, C, H, W), generator=g).to(tdt)
    ih, iw = H / scale, W / scale
    x1 = torch.rand(R, generator=g) * iw * 1.1 - 0.05 * iw   # some RoIs cross the border
    y1 = torch.rand(R, generator=g) * ih * 1.1 - 0.05 * ih
    bw = torch.rand(R, generator=g) * iw * 0.6 + 1.0 / scale
    bh = torch.rand(R, generator=g) * ih * 0.6 + 1.0 / scale
    bidx = torch.randint(0, B, (R,), generator=g).float()
    bidx[0] = B   # a batch index past the last image: zeros
    rois = torch.stack([bidx, x1, y1, x1 + bw, y1 + bh], 1).float().contiguous()
    off = (torch.randn((R, 2, k, k), generator=g) * 0.3).to(tdt) if with_off else None
    m = torch.sigmoid(torch.randn((R, k, k), generator=g)).to(tdt) if with_mask else None
    return x, rois, off, m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_roi_pool_parity(case, dtype):
    name, B, C, H, W, R, k, S, scale, gamma, wo, wm = case
    x, rois, off, m = make(B, C, H, W, R, k, S, scale, gamma, wo, wm, dtype, seed=hash(name) % 1000)
    print(f"[gpu-test] roi {name} {dtype}", flush=True)
    got = dcn.deform_roi_pool(x.cuda(), rois.cuda(), None if off is None else off.cuda(),
                              None if m is None else m.cuda(), k, S, scale, gamma)
    torch.cuda.synchronize()
    ref = oracle.roi_pool(x, rois, k, S, scale, gamma, off, m)
    got = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    tol = TOL[dtype] * float(x.float().abs().max())
    assert np.all(err <= tol), f"{name}/{dtype}: max error {err.max():.3e} > {tol:.3e}"
    assert np.all(got[0] == 0.0), "a RoI past the last image must pool zeros"


def test_roi_pool_empty_and_full_size():
    x = torch.randn((1, 4, 8, 8), device="cuda")
    out = dcn.deform_roi_pool(x, torch.zeros((0, 5), device="cuda"), output_size=3)
    assert out.shape == (0, 4, 3, 3)
    # the bench's layer: 256 RoIs per image on the c4 feature map, full parity
    from deformable_convolution_vision_amd.workloads import WORKLOADS, roi_inputs
    w = WORKLOADS["roi_c4"]
    inp = roi_inputs(w, 256, w.K, (800, 1344))
    g = {k: v.cuda() for k, v in inp.items()}
    got = dcn.deform_roi_pool(g["x"], g["rois"], g["offset"], g["mask"], w.K, 2, 1.0 / 16, 0.1)
    torch.cuda.synchronize()
    ref = oracle.roi_pool(inp["x"], inp["rois"], w.K, 2, 1.0 / 16, 0.1, inp["offset"], inp["mask"])
    err = np.abs(got.float().cpu().numpy() - ref)
    assert err.max() <= 1e-2 * float(inp["x"].float().abs().max())
