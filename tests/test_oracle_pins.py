"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""

import json
import os

import numpy as np
import pytest

import oracle
import pins

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


@pytest.fixture(scope="module")
def lib():
    oracle.load()
    return oracle.LIB


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_shapes_from_pages(lib):
    with open(os.path.join(pins.GOLDEN, "shapes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        Ho, Wo = oracle.output_hw(c["B"], c["Cin"], c["H"], c["W"], c["Cout"], c["K"], c["stride"],
                                  c["pad"], c["dilation"])
        assert [c["B"], 2 * c["K"] ** 2, Ho, Wo] == c["offset_shape"]
        assert [c["B"], c["Cout"], Ho, Wo] == c["out_shape"]


def test_points_match_full_grid(lib):
    rng = np.random.default_rng(5)
    x, off, m, w, b, Ho, Wo = pins.rand_case(rng, 2, 3, 9, 10, 5, 3, 2, 1, 1)
    y, a = oracle.forward(x, off, w, b, 2, 1, 1, mask=m)
    pts = np.stack(np.meshgrid(np.arange(2), np.arange(5), np.arange(Ho), np.arange(Wo),
                               indexing="ij"), -1).reshape(-1, 4)
    yp, ap = oracle.points(x, off, w, pts, b, 2, 1, 1, mask=m)
    assert np.array_equal(yp, y.reshape(-1)) and np.array_equal(ap, a.reshape(-1))


def test_cout_range_and_thread_count_invariance(lib):
    rng = np.random.default_rng(6)
    x, off, m, w, b, Ho, Wo = pins.rand_case(rng, 2, 4, 8, 8, 6, 3, 1, 1, 1)
    y1 = oracle.forward(x, off, w, b, 1, 1, 1, mask=m, threads=1, with_abs=False)
    y8 = oracle.forward(x, off, w, b, 1, 1, 1, mask=m, threads=8, with_abs=False)
    ys = oracle.forward(x, off, w, b, 1, 1, 1, mask=m, cout_range=(2, 5), with_abs=False)
    assert np.array_equal(y1, y8)
    assert np.array_equal(ys, y1[:, 2:5])


def test_invalid_geometry_rejected(lib):
    with pytest.raises(ValueError):
        oracle.output_hw(1, 3, 2, 2, 4, 5, 1, 0, 1)   # kernel larger than the padded input
    with pytest.raises(ValueError):
        oracle.output_hw(1, 3, 8, 8, 4, 3, 0, 1, 1)   # stride 0


def test_abs_terms_bound_output(lib):
    rng = np.random.default_rng(7)
    x, off, m, w, b, Ho, Wo = pins.rand_case(rng, 1, 5, 9, 9, 4, 3, 1, 1, 1, offset_scale=3.0)
    y, a = oracle.forward(x, off, w, b, 1, 1, 1, mask=m)
    assert np.all(np.abs(y) <= a * (1 + 1e-12))
    assert np.all(a >= np.abs(b)[None, :, None, None])
