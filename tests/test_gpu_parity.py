"""The HIP path against the CPU oracle, through the C ABI, on an MI355X.

Tolerance: per output, |y_gpu - y_oracle| / sum|terms| <= 1e-4 (fp32) or 1e-2
(bf16), exact where the sum of |terms| is 0."""

import zlib

import numpy as np
import pytest
import torch

import deformable_convolution_vision_amd as dcn
import oracle
from deformable_convolution_vision_amd.workloads import WORKLOADS, custom, generate
from gpu_common import TOL, check, full_parity, run_hip, sample_points, sampled_parity, to_gpu

pytestmark = pytest.mark.gpu


def make(name, dtype, B, Cin, H, W, Cout, K, s, p, d, **kw):
    Ho, Wo = oracle.output_hw(B, Cin, H, W, Cout, K, s, p, d)
    return custom(name, dtype, B, Cin, H, W, Cout, K, s, p, d, Ho, Wo, **kw)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("name", ["tiny", "single224"])
def test_named_workload_full(name):
    print(f"[gpu-test] variant {variant_of(WORKLOADS[name])}", flush=True)
    full_parity(WORKLOADS[name])


@pytest.mark.parametrize("name", ["c3", "c4", "c5", "c4_g4"])
def test_named_workload_full_grid(name):
    """The full-size layers, every output against the oracle (all host cores)."""
    print(f"[gpu-test] variant {variant_of(WORKLOADS[name])}", flush=True)
    worst = full_parity(WORKLOADS[name], threads=0)
    print(f"[gpu-test] max relative error {worst:.2e}", flush=True)


# Inputs whose four corners nearly cancel: x of alternating sign and almost equal
# magnitude, sample fractions in [0.45, 0.55] and weights of one sign, so a sample is
# small next to its corner terms; an interpolation whose corner weights lose precision
# (bf16 weights) breaks the per-element rule here while random inputs hide it.
CANCEL = [
    ("c4_like", None, dict(B=1, Cin=256, H=30, W=34, Cout=256, K=3, s=2, p=1, d=1)),
    ("c3_like", None, dict(B=1, Cin=128, H=24, W=40, Cout=128, K=3, s=1, p=1, d=1)),
    ("c5_like_no_mask", None, dict(B=2, Cin=512, H=12, W=14, Cout=512, K=3, s=1, p=2, d=2, mask=None)),
    ("box_pw4", ("box_bf16_m256", "4,5,10", "4"), dict(B=1, Cin=256, H=30, W=34, Cout=256, K=3, s=2, p=1, d=1)),
    ("box_m128_two_samples", ("box_bf16_m128", "8,8,16", None), dict(B=1, Cin=64, H=24, W=40, Cout=128, K=3, s=1,
                                                                      p=1, d=1)),
    ("k5", None, dict(B=1, Cin=48, H=30, W=26, Cout=96, K=5, s=2, p=2, d=1)),
    ("box_k1", ("box_bf16_m128", None, None), dict(B=2, Cin=64, H=17, W=19, Cout=130, K=1, s=1, p=0, d=1)),
    ("box_groups", ("box_bf16_m256", None, None), dict(B=1, Cin=256, H=30, W=34, Cout=256, K=3, s=2, p=1, d=1,
                                                          G=4)),
    ("tile", ("tile_bf16_m128_n64", None, None), dict(B=2, Cin=40, H=12, W=14, Cout=70, K=3, s=1, p=1, d=1)),
]


# both element types for the planner's own choice; bf16 alone where a bf16 kernel is forced
CANCEL_CASES = [(name, force, kw, dtype) for name, force, kw in CANCEL
                for dtype in (("bf16",) if force is not None else ("f32", "bf16"))]


@pytest.mark.parametrize("name,force,kw,dtype", CANCEL_CASES, ids=[f"{c[0]}-{c[3]}" for c in CANCEL_CASES])
def test_corner_cancellation(name, force, kw, dtype, monkeypatch):
    if force is not None:
        variant, tile, pw = force
        monkeypatch.setenv("DCN_VARIANT", variant)
        if tile:
            monkeypatch.setenv("DCN_BOX_TILE", tile)
        if pw:
            monkeypatch.setenv("DCN_BOX_PW", pw)
    kw = dict(kw)
    G = kw.pop("G", 1)
    g = {k: kw.pop(k) for k in ("B", "Cin", "H", "W", "Cout", "K", "s", "p", "d")}
    w = make(name, dtype, g["B"], g["Cin"], g["H"], g["W"], g["Cout"], g["K"], g["s"], g["p"], g["d"],
             seed=zlib.crc32(name.encode()) % 1000, x="checker:0.01", offset="frac:2:0.45:0.55",
             weight="kaiming_abs", groups=G, bias=None, **kw)
    inp = generate(w)
    desc = dcn.describe(inp["x"], inp["weight"], w.stride, w.pad, w.dilation, inp["offset"])
    print(f"[gpu-test] {w} plan {dcn.dcn_plan_describe(desc)}", flush=True)
    worst = full_parity(w, inp)
    print(f"[gpu-test] max relative error {worst:.2e}", flush=True)


def test_corner_cancellation_c4_layer_full_grid():
    """The c4 layer at full size on the cancellation inputs, every output."""
    w = WORKLOADS["c4_cancel"]
    print(f"[gpu-test] variant {variant_of(w)}", flush=True)
    worst = full_parity(w, threads=0)
    print(f"[gpu-test] max relative error {worst:.2e}", flush=True)


def variant_of(w):
    return dcn.dcn_variant_name(dcn.make_desc(w.B, w.Cin, w.H, w.W, w.Cout, w.K, w.stride, w.pad, w.dilation,
                                              dcn.F32 if w.dtype == "f32" else dcn.BF16, w.groups))


EDGE = [
    ("ragged", dict(B=3, Cin=37, H=11, W=13, Cout=70, K=3, s=1, p=1, d=1, offset="normal:2")),
    ("k1", dict(B=2, Cin=16, H=9, W=7, Cout=24, K=1, s=1, p=0, d=1)),
    ("k5_s3_d2", dict(B=1, Cin=12, H=23, W=19, Cout=40, K=5, s=3, p=2, d=2, offset="normal:3")),
    ("hw1", dict(B=2, Cin=8, H=1, W=1, Cout=5, K=3, s=1, p=1, d=1)),
    ("no_mask_no_bias", dict(B=2, Cin=33, H=10, W=12, Cout=17, K=3, s=1, p=1, d=1, mask=None, bias=None)),
    ("odd_stride2", dict(B=1, Cin=40, H=15, W=17, Cout=66, K=3, s=2, p=1, d=1)),
    ("cin3", dict(B=2, Cin=3, H=20, W=21, Cout=9, K=3, s=1, p=1, d=1, offset="uniform:2")),
    # small-reduction kernel: rows of two 64-pixel segments with offsets that leave the
    # input window (its corners then come from x); stride 2 and dilation 2, whose window
    # does not fit (every corner from x); K = 2
    ("direct_far_offsets", dict(B=2, Cin=4, H=21, W=70, Cout=20, K=3, s=1, p=1, d=1, offset="uniform:6")),
    ("direct_s2_d2", dict(B=1, Cin=2, H=30, W=150, Cout=70, K=3, s=2, p=2, d=2)),
    ("direct_k2", dict(B=2, Cin=1, H=9, W=11, Cout=5, K=2, s=1, p=0, d=1, offset="normal:1.5")),
    ("cout300", dict(B=1, Cin=64, H=12, W=14, Cout=300, K=3, s=1, p=1, d=1)),
    ("far_offsets_d2", dict(B=2, Cin=24, H=13, W=11, Cout=20, K=3, s=1, p=2, d=2, offset="uniform:8",
                            mask=None)),
    ("many_pixels", dict(B=1, Cin=32, H=64, W=96, Cout=64, K=3, s=1, p=1, d=1)),
    ("pad0_k2", dict(B=2, Cin=8, H=6, W=9, Cout=3, K=2, s=1, p=0, d=1, offset="normal:1.5")),
    # offsets far beyond any LDS box: exercises the global-memory path of the box kernel
    ("huge_offsets", dict(B=1, Cin=64, H=48, W=64, Cout=128, K=3, s=1, p=1, d=1, offset="uniform:30")),
    ("k5_box", dict(B=1, Cin=48, H=30, W=26, Cout=96, K=5, s=2, p=2, d=1, offset="normal:2")),
    ("k1_box", dict(B=2, Cin=64, H=17, W=19, Cout=130, K=1, s=1, p=0, d=1)),
    # H*W a multiple of 8: the register-transpose staging; 70 channels pad to 96, so
    # the second 64-channel block is half padding
    ("stage_cp96", dict(B=3, Cin=70, H=8, W=12, Cout=40, K=3, s=1, p=1, d=1, offset="normal:1.5")),
    # staging tiles: 280 pixels (a multiple of 8, not of the 256-pixel tile) with an odd
    # channel count, with two full 64-channel blocks, and 130 pixels (2-pixel vectors,
    # full 64 x 64 tiles and a 2-pixel tail)
    ("stage_tail_odd_cin", dict(B=2, Cin=67, H=10, W=28, Cout=48, K=3, s=1, p=1, d=1)),
    ("stage_full_blocks", dict(B=2, Cin=128, H=10, W=28, Cout=64, K=3, s=1, p=1, d=1)),
    ("stage_vec2", dict(B=2, Cin=64, H=10, W=13, Cout=32, K=3, s=1, p=1, d=1)),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shape(name, kw, dtype):
    kw = dict(kw)
    g = {k: kw.pop(k) for k in ("B", "Cin", "H", "W", "Cout", "K", "s", "p", "d")}
    w = make(name, dtype, g["B"], g["Cin"], g["H"], g["W"], g["Cout"], g["K"], g["s"], g["p"], g["d"],
             seed=zlib.crc32(name.encode()) % 1000, **kw)
    print(f"[gpu-test] {w} variant {variant_of(w)}", flush=True)
    full_parity(w)


def _variants(dtype):
    names = []
    for v in ("tile_f32_m64_n64", "tile_f32_m128_n64", "tile_bf16_m64_n64", "tile_bf16_m128_n64",
              "tile_bf16_m128_n32", "tile_bf16_m256_n64", "box_bf16_m128", "box_bf16_m256",
              "direct_f32", "direct_bf16"):
        if ("bf16" in v) == (dtype == "bf16"):
            names.append(v)
    return names


@pytest.mark.parametrize("variant", _variants("f32") + _variants("bf16"))
def test_every_variant(variant, monkeypatch):
    dtype = "bf16" if "bf16" in variant else "f32"
    monkeypatch.setenv("DCN_VARIANT", variant)
    shapes = [(3, 37, 11, 13, 70, 3, 1, 1, 1), (2, 64, 9, 10, 260, 3, 2, 1, 1)]
    if variant.startswith("direct"):   # at most 4 input channels, K*K in {1, 4, 9}
        shapes = [(3, 3, 11, 13, 70, 3, 1, 1, 1), (2, 4, 9, 10, 37, 2, 2, 0, 1), (1, 1, 6, 7, 5, 1, 1, 0, 1)]
    for seed, shape in enumerate(shapes):
        w = make(f"sweep_{variant}", dtype, *shape, offset="normal:2", seed=seed)
        assert variant_of(w) == variant
        full_parity(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_samples_outside_gives_bias(dtype):
    w = make("outside", dtype, 2, 20, 9, 10, 12, 3, 1, 1, 1)
    inp = generate(w)
    inp["offset"] = torch.full_like(inp["offset"], 100.5)
    out = run_hip(w, to_gpu(inp)).cpu()
    assert torch.equal(out, inp["bias"][None, :, None, None].expand_as(out))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_offsets_contribute_zero(dtype):
    w = make("nonfinite", dtype, 2, 24, 9, 10, 12, 3, 1, 1, 1, offset="normal:2")
    inp = generate(w)
    off = inp["offset"].float().clone()
    g = torch.Generator().manual_seed(3)
    sel = torch.rand(off.shape, generator=g) < 0.2
    specials = torch.tensor([float("nan"), float("inf"), -float("inf"), 1e30, -1e30])
    pick = torch.randint(0, len(specials), off.shape, generator=g)
    off[sel] = specials[pick[sel]]
    inp["offset"] = off.to(inp["x"].dtype)
    out = run_hip(w, to_gpu(inp)).cpu()
    assert torch.isfinite(out).all()
    y, a = oracle.forward(inp["x"], inp["offset"], inp["weight"], inp["bias"], 1, 1, 1, mask=inp["mask"])
    check(out.float().numpy(), y, a, TOL[dtype], "nonfinite offsets")


def test_deterministic_and_stage_split_matches():
    w = WORKLOADS["c4"]
    g = to_gpu(generate(w))
    outs = [run_hip(w, g) for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    desc = dcn.describe(g["x"], g["weight"], w.stride, w.pad, w.dilation)
    nb = dcn.dcn_workspace_bytes(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(outs[0])
    dcn.dcn_stage(desc, g["x"], g["weight"], ws, nb)
    dcn.dcn_forward_staged(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out, outs[0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_untouched(dtype):
    w = make("guard", dtype, 2, 40, 11, 12, 70, 3, 1, 1, 1)
    g = to_gpu(generate(w))
    desc = dcn.describe(g["x"], g["weight"], w.stride, w.pad, w.dilation)
    nb = dcn.dcn_workspace_bytes(desc)
    G = 4096
    n_out = w.B * w.Cout * w.Ho * w.Wo
    tdt = g["x"].dtype
    out_buf = torch.full((n_out + 2 * G,), 1234.5, dtype=tdt, device="cuda")
    ws_buf = torch.full((nb + 2 * G * 4,), 77, dtype=torch.uint8, device="cuda")
    out_view = out_buf[G:G + n_out]
    ws_view = ws_buf[4 * G:4 * G + nb]
    assert ws_view.data_ptr() % 256 == 0
    dcn.dcn_forward(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out_view, ws_view, nb)
    torch.cuda.synchronize()
    assert torch.all(out_buf[:G] == 1234.5) and torch.all(out_buf[G + n_out:] == 1234.5)
    assert torch.all(ws_buf[:4 * G] == 77) and torch.all(ws_buf[4 * G + nb:] == 77)
    ref = run_hip(w, g)
    assert torch.equal(out_view.view_as(ref), ref)


def test_error_leaves_output_untouched():
    w = make("err", "bf16", 1, 8, 9, 9, 4, 3, 1, 1, 1)
    g = to_gpu(generate(w))
    desc = dcn.describe(g["x"], g["weight"], 1, 1, 1)
    nb = dcn.dcn_workspace_bytes(desc)
    out = torch.full((1, 4, 9, 9), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dcn.DcnError) as e:
        dcn.dcn_forward(desc, g["x"], g["offset"], g["mask"], g["weight"], None, out, None, nb)
    assert e.value.status == dcn.E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_empty_batch():
    x = torch.zeros(0, 8, 9, 9, device="cuda")
    out = dcn.deform_conv2d(x, torch.zeros(0, 18, 9, 9, device="cuda"), torch.zeros(4, 8, 3, 3, device="cuda"),
                            padding=1)
    assert out.shape == (0, 4, 9, 9)


@pytest.mark.parametrize("roles", ["0", "1"])
@pytest.mark.parametrize("variant,tile", [("box_bf16_m256", "4,5,10"), ("box_bf16_m256", "6,7,13"),
                                          ("box_bf16_m128", "8,8,16"), ("box_bf16_m128", "10,9,17")])
def test_box_role_placement(variant, tile, roles, monkeypatch):
    """Both placements of the box kernel's consumer and producer waves on the SIMDs,
    with one, two and three samples per producer thread and step."""
    monkeypatch.setenv("DCN_VARIANT", variant)
    monkeypatch.setenv("DCN_BOX_TILE", tile)
    monkeypatch.setenv("DCN_BOX_ROLES", roles)
    shapes = [(2, 64, 9, 10, 260, 3, 2, 1, 1), (2, 64, 17, 19, 130, 1, 1, 0, 1), (2, 40, 12, 14, 300, 3, 1, 2, 2)]
    for seed, shape in enumerate(shapes):
        w = make(f"roles_{variant}_{roles}", "bf16", *shape, offset="uniform:8", seed=seed)
        desc = dcn.make_desc(w.B, w.Cin, w.H, w.W, w.Cout, w.K, w.stride, w.pad, w.dilation, dcn.BF16)
        plan = dcn.dcn_plan_describe(desc)
        print(f"[gpu-test] {shape} {plan}", flush=True)
        assert ("roles=split" if roles == "1" else "roles=paired") in plan
        full_parity(w)


GROUPED = [
    ("g2_k3", dict(B=2, Cin=64, H=11, W=13, Cout=70, K=3, s=1, p=1, d=1, G=2, offset="normal:2")),
    ("g4_s2", dict(B=1, Cin=32, H=15, W=17, Cout=40, K=3, s=2, p=1, d=1, G=4, offset="normal:1.5")),
    ("g3_nomask", dict(B=2, Cin=48, H=9, W=10, Cout=33, K=3, s=1, p=2, d=2, G=3, offset="uniform:4",
                       mask=None)),
    ("g2_k1", dict(B=2, Cin=16, H=9, W=7, Cout=24, K=1, s=1, p=0, d=1, G=2)),
    ("g8_k5", dict(B=1, Cin=64, H=12, W=14, Cout=130, K=5, s=1, p=2, d=1, G=8, offset="normal:2")),
    ("g4_cout300", dict(B=3, Cin=96, H=8, W=12, Cout=300, K=3, s=1, p=1, d=1, G=4, offset="normal:1.5")),
    # 32-channel multiples per group: the box kernel (bf16), group tables swapped per group
    ("g4_box", dict(B=2, Cin=128, H=19, W=23, Cout=256, K=3, s=2, p=1, d=1, G=4, offset="normal:1.5")),
    ("g2_box_cpg4", dict(B=1, Cin=256, H=14, W=18, Cout=70, K=3, s=1, p=1, d=1, G=2, offset="normal:2")),
    ("g3_box_cpg2", dict(B=2, Cin=192, H=11, W=13, Cout=130, K=3, s=1, p=2, d=2, G=3, offset="uniform:6",
                         mask=None)),
    ("g8_box_far", dict(B=1, Cin=256, H=24, W=20, Cout=256, K=3, s=1, p=1, d=1, G=8, offset="uniform:12")),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,kw", GROUPED, ids=[e[0] for e in GROUPED])
def test_offset_groups(name, kw, dtype):
    kw = dict(kw)
    g = {k: kw.pop(k) for k in ("B", "Cin", "H", "W", "Cout", "K", "s", "p", "d", "G")}
    w = make(name, dtype, g["B"], g["Cin"], g["H"], g["W"], g["Cout"], g["K"], g["s"], g["p"], g["d"],
             seed=zlib.crc32(name.encode()) % 1000, groups=g["G"], **kw)
    inp = generate(w)
    desc = dcn.describe(inp["x"], inp["weight"], w.stride, w.pad, w.dilation, inp["offset"])
    assert desc.offset_groups == g["G"]
    print(f"[gpu-test] {w} plan {dcn.dcn_plan_describe(desc)}", flush=True)
    full_parity(w, inp)


@pytest.mark.parametrize("variant", ["tile_f32_m64_n64", "tile_f32_m128_n64", "tile_bf16_m64_n64",
                                     "tile_bf16_m128_n64", "tile_bf16_m128_n32", "tile_bf16_m256_n64"])
def test_offset_groups_every_tile_variant(variant, monkeypatch):
    dtype = "bf16" if "bf16" in variant else "f32"
    monkeypatch.setenv("DCN_VARIANT", variant)
    w = make(f"groups_{variant}", dtype, 2, 64, 9, 10, 260, 3, 2, 1, 1, offset="normal:2", seed=7, groups=4)
    full_parity(w)


@pytest.mark.parametrize("roles", ["0", "1"])
@pytest.mark.parametrize("variant,tile", [("box_bf16_m256", "4,5,10"), ("box_bf16_m128", "4,5,10"),
                                          ("box_bf16_m128", "6,7,13"), ("box_bf16_m128", "8,8,16")])
def test_offset_groups_box_tiles(variant, tile, roles, monkeypatch):
    """Offset groups on the box kernel with one and two samples per producer thread."""
    monkeypatch.setenv("DCN_VARIANT", variant)
    monkeypatch.setenv("DCN_BOX_TILE", tile)
    monkeypatch.setenv("DCN_BOX_ROLES", roles)
    for seed, (Cin, G) in enumerate([(128, 4), (192, 3)]):
        w = make(f"gbox_{variant}_{tile}", "bf16", 2, Cin, 13, 17, 150, 3, 1, 1, 1, offset="normal:2",
                 seed=seed, groups=G)
        inp = generate(w)
        desc = dcn.describe(inp["x"], inp["weight"], w.stride, w.pad, w.dilation, inp["offset"])
        plan = dcn.dcn_plan_describe(desc)
        print(f"[gpu-test] {plan}", flush=True)
        assert plan.startswith(variant) and f"offset groups={G}" in plan
        full_parity(w, inp)


@pytest.mark.parametrize("pw", ["4", "8"])
@pytest.mark.parametrize("variant,tile", [("box_bf16_m256", "4,5,10"), ("box_bf16_m256", "6,7,13"),
                                          ("box_bf16_m128", "8,8,16"), ("box_bf16_m128", "10,10,15")])
def test_box_producer_waves(variant, tile, pw, monkeypatch):
    """The box kernel with four and with eight producer waves, paired roles."""
    monkeypatch.setenv("DCN_VARIANT", variant)
    monkeypatch.setenv("DCN_BOX_TILE", tile)
    monkeypatch.setenv("DCN_BOX_ROLES", "0")
    monkeypatch.setenv("DCN_BOX_PW", pw)
    # the last shape: an image large enough for boxes at full capacity, and offsets that
    # reach the boxes' last rows (every box pixel must be copied)
    shapes = [(2, 64, 9, 10, 260, 3, 2, 1, 1), (2, 40, 12, 14, 300, 3, 1, 2, 2), (1, 256, 30, 34, 256, 3, 2, 1, 1),
              (1, 64, 44, 52, 128, 3, 1, 1, 1)]
    for seed, shape in enumerate(shapes):
        w = make(f"pw{pw}_{variant}_{tile}", "bf16", *shape, offset="uniform:9" if seed == 3 else "normal:2",
                 seed=seed)
        desc = dcn.make_desc(w.B, w.Cin, w.H, w.W, w.Cout, w.K, w.stride, w.pad, w.dilation, dcn.BF16)
        plan = dcn.dcn_plan_describe(desc)
        print(f"[gpu-test] {shape} {plan}", flush=True)
        assert f"producer waves={pw}" in plan
        full_parity(w)


# B, Cin, H, W, K, s, p, d, G.  The last shape's taps span more input than the LDS box
# of a 32-pixel block can hold (7x7 at dilation 8), so it runs the kernel that reads the
# staged copy directly; the others run the box kernel.
OM_SHAPES = [(2, 32, 13, 17, 3, 1, 1, 1, 1), (1, 64, 20, 24, 3, 2, 1, 1, 1), (2, 48, 11, 9, 3, 1, 2, 2, 3),
             (2, 16, 9, 10, 1, 1, 0, 1, 1), (1, 3, 12, 14, 3, 1, 1, 1, 1), (1, 256, 15, 21, 3, 2, 1, 1, 4),
             (1, 16, 60, 60, 7, 1, 24, 8, 1)]


def _offset_mask_case(dtype, shape, seed):
    B, Cin, H, W, K, s, p, d, G = shape
    Ho, Wo = oracle.output_hw(B, Cin, H, W, 1, K, s, p, d)
    w = custom("om", dtype, B, Cin, H, W, 3 * G * K * K, K, s, p, d, Ho, Wo, mask=None, bias="normal:0.1",
               seed=seed, groups=G, op="offset_mask")
    return w, generate(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", OM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_offset_mask_branch(shape, dtype):
    """dcn_offset_mask against the oracle's branch: offsets per element to the parity
    tolerance; the mask to the same tolerance through the sigmoid (1/4-Lipschitz) plus
    the rounding of a value in [0, 1] to the element type."""
    w, inp = _offset_mask_case(dtype, shape, zlib.crc32(repr(shape).encode()) % 1000)
    g = to_gpu(inp)
    off, msk = dcn.offset_mask(g["x"], g["weight"], g["bias"], w.stride, w.pad, w.dilation, offset_groups=w.groups)
    torch.cuda.synchronize()
    o_ref, m_ref, a = oracle.offset_mask(inp["x"], inp["weight"], inp["bias"], w.stride, w.pad, w.dilation,
                                         groups=w.groups)
    n_off = o_ref.shape[1]
    check(off.float().cpu().numpy(), o_ref, a[:, :n_off], TOL[dtype], "offset_mask offsets")
    round_err = 2.0 ** -9 if dtype == "bf16" else 1e-6
    err = np.abs(msk.float().cpu().numpy() - m_ref)
    bound = TOL[dtype] * a[:, n_off:] / 4 + round_err
    assert np.all(err <= bound), f"offset_mask mask: worst excess {float(np.max(err - bound)):.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_offset_mask_then_forward(dtype):
    """The branch's outputs fed to the deformable convolution: the forward matches the
    oracle run on those same (GPU-computed) offsets and mask."""
    w, inp = _offset_mask_case(dtype, (2, 64, 17, 19, 3, 1, 1, 1, 1), 5)
    g = to_gpu(inp)
    off, msk = dcn.offset_mask(g["x"], g["weight"], g["bias"], 1, 1, 1)
    wd = make("om_fwd", dtype, 2, 64, 17, 19, 70, 3, 1, 1, 1, seed=6)
    dcn_in = generate(wd)
    dcn_in["x"] = inp["x"]
    dcn_in["offset"] = off.cpu()
    dcn_in["mask"] = msk.cpu()
    out = run_hip(wd, to_gpu(dcn_in)).cpu()
    y, a = oracle.forward(dcn_in["x"], dcn_in["offset"], dcn_in["weight"], dcn_in["bias"], 1, 1, 1,
                          mask=dcn_in["mask"])
    check(out.float().numpy(), y, a, TOL[dtype], "offset_mask -> forward")


def test_offset_mask_c4_layer():
    """The c4 layer's branch (256 -> 27 channels, stride 2) against the oracle on every
    output: offsets to the parity tolerance, the mask through the sigmoid as above."""
    w = WORKLOADS["c4_om"]
    inp = generate(w)
    g = to_gpu(inp)
    off, msk = dcn.offset_mask(g["x"], g["weight"], g["bias"], w.stride, w.pad, w.dilation)
    torch.cuda.synchronize()
    o_ref, m_ref, a = oracle.offset_mask(inp["x"], inp["weight"], inp["bias"], w.stride, w.pad, w.dilation)
    n_off = o_ref.shape[1]
    check(off.float().cpu().numpy(), o_ref, a[:, :n_off], TOL["bf16"], "c4_om offsets")
    err = np.abs(msk.float().cpu().numpy() - m_ref)
    bound = TOL["bf16"] * a[:, n_off:] / 4 + 2.0 ** -9
    assert np.all(err <= bound), f"c4_om mask: worst excess {float(np.max(err - bound)):.3e}"


def test_binding_rejects_bad_out_and_workspace():
    """deform_conv2d checks a caller's out (shape, dtype, device, contiguity) and
    workspace (device, contiguity, byte size) before launching."""
    w = make("binding_checks", "bf16", 2, 40, 11, 12, 70, 3, 1, 1, 1)
    g = to_gpu(generate(w))
    args = (g["x"], g["offset"], g["weight"], g["bias"], 1, 1, 1)
    good = torch.empty((w.B, w.Cout, w.Ho, w.Wo), dtype=torch.bfloat16, device="cuda")
    bad_outs = [torch.empty((w.B, w.Cout, w.Ho, w.Wo + 1), dtype=torch.bfloat16, device="cuda"),
                torch.empty((w.B, w.Cout, w.Ho, w.Wo), dtype=torch.float32, device="cuda"),
                torch.empty((w.B, w.Cout, w.Ho, w.Wo), dtype=torch.bfloat16),
                torch.empty((w.B, w.Cout, w.Wo, w.Ho), dtype=torch.bfloat16, device="cuda").transpose(2, 3)]
    for o in bad_outs:
        with pytest.raises(ValueError):
            dcn.deform_conv2d(*args, mask=g["mask"], out=o)
    desc = dcn.describe(g["x"], g["weight"], 1, 1, 1)
    nb = dcn.dcn_workspace_bytes(desc)
    assert nb > 0
    bad_ws = [torch.empty(nb, dtype=torch.uint8), torch.empty(nb - 1, dtype=torch.uint8, device="cuda"),
              torch.empty(2 * nb, dtype=torch.uint8, device="cuda")[::2]]
    for ws in bad_ws:
        with pytest.raises(ValueError):
            dcn.deform_conv2d(*args, mask=g["mask"], out=good, workspace=ws)
    # a workspace of another element type is counted in bytes
    ws32 = torch.empty((nb + 3) // 4, dtype=torch.float32, device="cuda")
    out = dcn.deform_conv2d(*args, mask=g["mask"], out=good, workspace=ws32)
    assert torch.equal(out, run_hip(w, g))


LAYER_SHAPES = [  # B, Cin, H, W, Cout, K, s, p, d, G
    (2, 64, 17, 19, 70, 3, 1, 1, 1, 1),
    (1, 256, 30, 34, 256, 3, 2, 1, 1, 1),
    (2, 48, 11, 9, 33, 3, 1, 2, 2, 3),
    (2, 16, 9, 10, 24, 1, 1, 0, 1, 1),
    (1, 3, 12, 14, 8, 3, 1, 1, 1, 1),
    (1, 128, 15, 21, 130, 3, 2, 1, 1, 4),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", LAYER_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layer_forward(shape, dtype):
    """dcn_layer_forward (branch and deformable convolution off one staged x): offsets
    and mask against the oracle's branch, the output against the oracle's forward on the
    offsets and mask the call produced, and bit for bit against dcn_forward on them."""
    _layer_case(shape, dtype)


# The layer with the deformable convolution's box tile and producer-wave schedule pinned:
# edge tiles, four and eight producer waves, one and three 32-channel chunks, dilation 2,
# stride 2 without padding, two tiles of output channels.
LAYER_PINNED_CASES = [  # shape (B, Cin, H, W, Cout, K, s, p, d, G), DCN_BOX_TILE, DCN_BOX_PW
    ((1, 256, 30, 34, 256, 3, 2, 1, 1, 1), "4,5,10", "8"),
    ((1, 256, 30, 34, 256, 3, 2, 1, 1, 1), "4,5,10", "4"),
    ((2, 64, 17, 19, 70, 3, 1, 1, 1, 1), "4,4,16", "4"),
    ((1, 96, 23, 29, 300, 3, 1, 2, 2, 1), "4,8,8", "8"),
    ((2, 32, 13, 11, 64, 3, 2, 0, 1, 1), "4,6,10", "4"),
]


@pytest.mark.parametrize("case", LAYER_PINNED_CASES, ids=lambda c: "x".join(map(str, c[0])) + f"_t{c[1]}_pw{c[2]}")
def test_layer_forward_pinned_tiles(case, monkeypatch):
    """dcn_layer_forward on the box kernel with its tile and schedule pinned, against the
    oracle and bit for bit against dcn_forward on the offsets and mask it produced."""
    shape, tile, pw = case
    monkeypatch.setenv("DCN_BOX_TILE", tile)
    monkeypatch.setenv("DCN_BOX_PW", pw)
    plan = _layer_case(shape, "bf16")
    assert "(64 slots)" in plan, plan


def _layer_case(shape, dtype):
    B, Cin, H, W, Cout, K, s, p, d, G = shape
    seed = zlib.crc32(repr(shape).encode()) % 1000
    w_om, inp_om = _offset_mask_case(dtype, (B, Cin, H, W, K, s, p, d, G), seed)
    wd = make("layer", dtype, B, Cin, H, W, Cout, K, s, p, d, seed=seed + 1, groups=G)
    inp = generate(wd)
    inp["x"] = inp_om["x"]
    g = to_gpu(inp)
    go = to_gpu(inp_om)
    desc = dcn.make_desc(B, Cin, H, W, Cout, K, s, p, d, dcn.BF16 if dtype == "bf16" else dcn.F32, G)
    plan = dcn.dcn_plan_describe(desc)
    print(f"[gpu-test] layer {shape} {dtype}: {plan}", flush=True)
    out, off, msk = dcn.deform_conv2d_layer(g["x"], go["weight"], go["bias"], g["weight"], g["bias"], s, p, d,
                                            offset_groups=G)
    torch.cuda.synchronize()
    o_ref, m_ref, a = oracle.offset_mask(inp["x"], inp_om["weight"], inp_om["bias"], s, p, d, groups=G)
    n_off = o_ref.shape[1]
    check(off.float().cpu().numpy(), o_ref, a[:, :n_off], TOL[dtype], "layer offsets")
    round_err = 2.0 ** -9 if dtype == "bf16" else 1e-6
    err = np.abs(msk.float().cpu().numpy() - m_ref)
    assert np.all(err <= TOL[dtype] * a[:, n_off:] / 4 + round_err), "layer mask"
    y, ay = oracle.forward(inp["x"], off.cpu(), inp["weight"], inp["bias"], s, p, d, mask=msk.cpu())
    check(out.float().cpu().numpy(), y, ay, TOL[dtype], "layer output")
    ref = dcn.deform_conv2d(g["x"], off, g["weight"], g["bias"], s, p, d, mask=msk)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "dcn_layer_forward differs from dcn_forward on its own offsets and mask"
    return plan


def test_layer_forward_c4():
    """The c4 layer with its branch (256 -> 27 channels, then 256 -> 256) in one call,
    every output against the oracle."""
    w_om, w = WORKLOADS["c4_om"], WORKLOADS["c4"]
    inp_om, inp = generate(w_om), generate(w)
    inp["x"] = inp_om["x"]
    g, go = to_gpu(inp), to_gpu(inp_om)
    out, off, msk = dcn.deform_conv2d_layer(g["x"], go["weight"], go["bias"], g["weight"], None, 2, 1, 1)
    torch.cuda.synchronize()
    o_ref, m_ref, a = oracle.offset_mask(inp["x"], inp_om["weight"], inp_om["bias"], 2, 1, 1, threads=0)
    check(off.float().cpu().numpy(), o_ref, a[:, :18], TOL["bf16"], "c4 layer offsets")
    assert np.all(np.abs(msk.float().cpu().numpy() - m_ref) <= TOL["bf16"] * a[:, 18:] / 4 + 2.0 ** -9)
    y, ay = oracle.forward(inp["x"], off.cpu(), inp["weight"], None, 2, 1, 1, mask=msk.cpu(), threads=0)
    worst = check(out.float().cpu().numpy(), y, ay, TOL["bf16"], "c4 layer output")
    print(f"[gpu-test] max relative error {worst:.2e}", flush=True)
    ref = dcn.deform_conv2d(g["x"], off, g["weight"], None, 2, 1, 1, mask=msk)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "the c4 layer differs from dcn_forward on its own offsets and mask"
