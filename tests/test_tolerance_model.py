"""The dQ tolerance of the GPU backward tests, derived on the CPU from a
model of the HIP path's bf16 roundings (tests/bf16_error_model.py): O, P, dS
and dQ rounded to bf16, float64 otherwise, against the float64 oracle.

The tolerance must admit the modelled error with at least 30 % headroom (for
fp32 accumulation order and the hardware exp2, which the model leaves out)
and stay within twice it, so that it is neither tighter than the arithmetic
allows nor loose enough to hide a real mistake. The cases are the ones that
set the bound: the 6 x 6 x 12 grid, where every axis is cut and blocks hold
16 to 128 tokens (the sharpest softmax), and the smooth-field 8 x 16 x 32
grid."""

import math

import numpy as np
import pytest

import oracle.bsa_oracle as O
from bf16_error_model import dq_with_gpu_roundings, round_bf16
from test_gpu_backward import TOL
from video_dit_block_bsa_amd.inputs import make_grad, make_qkv

SCALE = 1.0 / math.sqrt(128)
CASES = [((6, 6, 12), 3, 43), ((8, 16, 32), 6, 11)]  # (grid, top-k, seed), field inputs, 2 heads


def test_round_bf16_against_the_format():
    """round_bf16 keeps 8 significant bits, rounding ties to even."""
    one = 1.0
    ulp = 2.0 ** -7
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 1e-6, -2.5, 3.140625,
                  2.0 ** -133])
    want = np.array([one, one + 2 * ulp, one + ulp, -2.5, 3.140625, 2.0 ** -133])
    assert np.array_equal(round_bf16(x), want)


def _model_errors():
    worst_max, worst_mean = 0.0, 0.0
    for (T, H, W), ksel, seed in CASES:
        q, k, v = make_qkv(T, H, W, 2, kind="field", seed=seed)
        do = make_grad(T, H, W, 2, seed=seed)
        g = O.Geometry(T, H, W)
        for h in range(2):
            qf, kf, vf, dof = (O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v, do))
            idx, cnt, _ = O.select_head(qf, kf, g, O.SelectParams("topk", k=ksel), SCALE)
            ref = O.backward_head(qf, kf, vf, dof, g, idx, cnt, SCALE)[0]
            err = np.abs(dq_with_gpu_roundings(qf, kf, vf, dof, g, idx, cnt, SCALE) - ref)
            worst_max = max(worst_max, err.max() / np.abs(ref).max())
            worst_mean = max(worst_mean, err.mean() / np.abs(ref).mean())
    return worst_max, worst_mean


@pytest.fixture(scope="module")
def model():
    return _model_errors()


def test_dq_tolerance_follows_the_rounding_model(model):
    worst_max, worst_mean = model
    tol_max, tol_mean = TOL["dq"]
    print(f"modelled dQ error: max {worst_max:.4f}, mean {worst_mean:.4f}; "
          f"tolerance {tol_max}, {tol_mean}")
    assert 1.3 * worst_max <= tol_max <= 2.0 * worst_max
    assert 1.3 * worst_mean <= tol_mean <= 2.0 * worst_mean


def test_cut_grid_needs_more_than_one_percent(model):
    """The modelled mean error on the cut grid is above 1 %: a 1e-2 mean
    tolerance would reject a correct kernel."""
    assert model[1] > 1e-2
