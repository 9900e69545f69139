"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Every mutant is a textual edit of ``oracle/dcn_oracle.cpp`` compiled to a
temporary library (CPU only).  Its pins run in a child process, so a mutant
that reads out of bounds and crashes also counts as caught.  The real oracle
is never modified.
"""

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, [(old, new), ...]) -- each old string must occur in the source.
MUTANTS = [
    ("swap_dy_dx", [("const double dy = offset[((b * 2 * KK * G + 2 * gk) *",
                     "const double dy = offset[((b * 2 * KK * G + 2 * gk + 1) *"),
                    ("const double dx = offset[((b * 2 * KK * G + 2 * gk + 1) *",
                     "const double dx = offset[((b * 2 * KK * G + 2 * gk) *")]),
    ("ceil_upper_corner", [("const double yy = y0 + dy;",
                            "const double yy = (dy == 0) ? y0 : std::ceil(py);")]),
    ("truncate_not_floor", [("const double y0 = std::floor(py);", "const double y0 = std::trunc(py);")]),
    ("drop_mask", [("(mask != nullptr) ? static_cast<double>", "(false) ? static_cast<double>")]),
    ("pad_sign", [("oy * d->stride - d->pad", "oy * d->stride + d->pad")]),
    ("ignore_dilation", [("i * d->dilation", "i")]),
    ("ignore_stride_x", [("ox * d->stride - d->pad", "ox - d->pad")]),
    ("weight_ij_transposed", [("((o * d->Cin + c) * K + i) * K + j", "((o * d->Cin + c) * K + j) * K + i")]),
    ("kernel_points_column_major", [("const int64_t i = k / K, j = k % K;",
                                     "const int64_t i = k % K, j = k / K;")]),
    ("drop_one_corner", [("for (int dx = 0; dx < 2; ++dx)", "for (int dx = 0; dx < 1; ++dx)")]),
    ("complement_weight", [("(1.0 - std::fabs(py - yy))", "std::fabs(py - yy)")]),
    ("clamp_not_zero", [("if (!(yy >= 0.0 && yy <= static_cast<double>(H - 1))) continue;",
                         "const double yyc = std::fmin(std::fmax(yy, 0.0), static_cast<double>(H - 1));"),
                        ("const int64_t iy = static_cast<int64_t>(yy);",
                         "const int64_t iy = static_cast<int64_t>(yyc);")]),
    ("inside_bound_off_by_one", [("xx <= static_cast<double>(W - 1)", "xx < static_cast<double>(W - 1)")]),
    ("drop_bias", [("y = static_cast<double>(bias[o]);", "y = 0.0;")]),
    ("abs_terms_signed", [("a += std::fabs(term);", "a += term;")]),
    ("mask_kernel_point_reversed", [("mask[((b * KK * G + gk) * Ho + oy) * Wo + ox]",
                                     "mask[((b * KK * G + g * KK + (KK - 1 - k)) * Ho + oy) * Wo + ox]")]),
    ("offset_batch_stride", [("offset[((b * 2 * KK * G + 2 * gk) *", "offset[((b * KK * G + 2 * gk) *"),
                             ("offset[((b * 2 * KK * G + 2 * gk + 1) *", "offset[((b * KK * G + 2 * gk + 1) *")]),
    ("group_of_channel_modulo", [("const int64_t g = c / Cg;", "const int64_t g = c % G;")]),
    ("groups_interleaved_by_kernel_point", [("const int64_t gk = g * KK + k;", "const int64_t gk = k * G + g;")]),
    ("group_batch_stride_dropped", [("offset[((b * 2 * KK * G + 2 * gk) *", "offset[((b * 2 * KK + 2 * gk) *"),
                                    ("offset[((b * 2 * KK * G + 2 * gk + 1) *", "offset[((b * 2 * KK + 2 * gk + 1) *")]),
    ("mask_ignores_group", [("mask[((b * KK * G + gk) * Ho + oy) * Wo + ox]", "mask[((b * KK * G + k) * Ho + oy) * Wo + ox]")]),
    ("x_channel_stride", [("x + ((b * d->Cin + c) * d->H) * d->W", "x + ((b * d->Cin + c) * d->W) * d->W")]),
    # gradients
    ("bwd_dsy_sign", [("r.dsy += (dy == 0 ? -1.0 : 1.0) * tx * v;", "r.dsy += (dy == 0 ? 1.0 : -1.0) * tx * v;")]),
    ("bwd_dsx_uses_tx", [("r.dsx += (dx == 0 ? -1.0 : 1.0) * ty * v;", "r.dsx += (dx == 0 ? -1.0 : 1.0) * tx * v;")]),
    ("bwd_offset_without_mask", [("goy += gc * m * sg.dsy;", "goy += gc * sg.dsy;")]),
    ("bwd_grad_x_without_mask", [("const double t = col_grad(b, c, k, pix) * mask_of(b, g * KK + k, pix);",
                                  "const double t = col_grad(b, c, k, pix);")]),
    ("bwd_grad_mask_times_mask", [("gm += gc * sg.s;", "gm += gc * m * sg.s;")]),
    ("bwd_weight_ignores_group", [("const int64_t o = oc / Cin, c = oc % Cin, g = c / Cg;",
                                   "const int64_t o = oc / Cin, c = oc % Cin, g = 0;")]),
    ("bwd_offset_pair_swapped", [("grad_offset[(b * 2 * G * KK + 2 * gk) * HoWo + pix] = goy;",
                                  "grad_offset[(b * 2 * G * KK + 2 * gk) * HoWo + pix] = gox;"),
                                 ("grad_offset[(b * 2 * G * KK + 2 * gk + 1) * HoWo + pix] = gox;",
                                  "grad_offset[(b * 2 * G * KK + 2 * gk + 1) * HoWo + pix] = goy;")]),
    ("bwd_grad_x_corner_weight", [("if (sg.inside[n]) gx[sg.iy[n] * W + sg.ix[n]] += t * sg.g[n];",
                                   "if (sg.inside[n]) gx[sg.iy[n] * W + sg.ix[n]] += t * sg.g[3 - n];")]),
    # RoI pooling
    ("roi_offset_scaled_by_width", [("d->gamma * h * static_cast<double>(offset[((r * 2 + 0)",
                                     "d->gamma * w * static_cast<double>(offset[((r * 2 + 0)")]),
    ("roi_subcell_corner", [("(static_cast<double>(u) + 0.5)", "static_cast<double>(u)")]),
    ("roi_bins_transposed", [("double* y = out + (rc * k + i) * k + j;", "double* y = out + (rc * k + j) * k + i;")]),
    ("roi_batch_ignored", [("const int64_t b = batch_ok ? static_cast<int64_t>(bi) : 0;", "const int64_t b = 0;")]),
    ("roi_mask_ignored", [("mask != nullptr ? static_cast<double>(mask[(r * k + i) * k + j]) : 1.0", "1.0")]),
    ("roi_scale_not_on_x1", [("const double x1 = static_cast<double>(roi[1]) * d->spatial_scale,",
                              "const double x1 = static_cast<double>(roi[1]),")]),
    ("roi_mean_over_s", [("*y = m * acc / static_cast<double>(S * S);", "*y = m * acc / static_cast<double>(S);")]),
    ("roi_abs_signed", [("if (abs_sum != nullptr) *abs_sum += std::fabs(t);", "if (abs_sum != nullptr) *abs_sum += t;")]),
    ("roi_abs_without_mask", [("*ya = std::fabs(m) * acc_abs", "*ya = acc_abs")]),
    # position-sensitive RoI pooling
    ("ps_bins_transposed_in_map", [("const int64_t ch = (c * k + i) * k + j;", "const int64_t ch = (c * k + j) * k + i;")]),
    ("ps_bin_major_maps", [("const int64_t ch = (c * k + i) * k + j;", "const int64_t ch = (i * k + j) * C + c;")]),
    ("ps_offset_group_ignored", [("const int64_t r = rc / C, c = rc % C, g = c / Cg;",
                                  "const int64_t r = rc / C, c = rc % C, g = 0 * Cg;")]),
    ("ps_offset_group_by_modulo", [("const int64_t r = rc / C, c = rc % C, g = c / Cg;",
                                    "const int64_t r = rc / C, c = rc % C, g = c % G;")]),
    ("bwd_position_ignores_pad", [("static_cast<float>(oy * d->stride - d->pad + i * d->dilation) + dy;",
                                   "static_cast<float>(oy * d->stride + i * d->dilation) + dy;")]),
]

RUNNER = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import warnings; warnings.filterwarnings("ignore")
import pins
failed = []
for pin in pins.ALL_PINS:
    try:
        pin({lib!r})
    except AssertionError as e:
        failed.append(pin.__name__)
        break
print("CAUGHT" if failed else "SURVIVED", failed)
sys.exit(0)
"""


def _run_mutant(name, edits, workdir):
    with open(oracle.SRC) as f:
        src = f.read()
    for old, new in edits:
        assert old in src, f"mutant {name}: pattern not found: {old}"
        src = src.replace(old, new)
    path = os.path.join(workdir, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(workdir, f"lib_{name}.so")
    oracle.build(lib, src=path)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "1"})
    if r.returncode != 0:       # crashed (e.g. an out-of-bounds read): caught
        return name, "CAUGHT(crash)"
    return name, r.stdout.strip()


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as wd:
        with ThreadPoolExecutor(max_workers=6) as ex:
            results = list(ex.map(lambda m: _run_mutant(m[0], m[1], wd), MUTANTS))
    survivors = [(n, r) for n, r in results if not r.startswith("CAUGHT")]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
