"""Pins of the fp8 indexer oracle to facts other than its own code: torch's
float8_e4m3fn conversion (a library routine), values worked out from the
e4m3 definition, a hand-worked scored example, and the special case where
quantisation is exact and the fp8 score must equal the (separately pinned)
unquantised score. Each test names the mistake it would catch."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import index_scores
from oracle.fp8_indexer import E4M3_MAX, e4m3_round, index_scores_fp8, quantize_rows_fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_every_code_is_a_fixed_point_and_matches_torch():
    """All 254 finite e4m3 values round to themselves (catches a wrong bias,
    mantissa width or subnormal step)."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = codes[np.isfinite(codes)]
    assert codes.size == 254 and codes.max() == E4M3_MAX and np.min(codes[codes > 0]) == 2.0 ** -9
    assert np.array_equal(e4m3_round(codes), codes)


def test_random_and_tie_values_match_torch():
    """Random float32 magnitudes over the whole range, and every midpoint
    between neighbouring codes (ties to even), against torch."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-12, 8.5, 200000))).astype(np.float32)
    x = x[np.abs(x) <= 440]
    assert np.array_equal(e4m3_round(x), _torch_e4m3(x))
    codes = np.unique(np.abs(torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn)
                             .to(torch.float64).numpy()))
    codes = codes[np.isfinite(codes)]
    mids = ((codes[:-1] + codes[1:]) / 2).astype(np.float32)
    assert np.array_equal(e4m3_round(mids), _torch_e4m3(mids))
    assert np.array_equal(e4m3_round(-mids), _torch_e4m3(-mids))


@pytest.mark.parametrize("x,want", [(0.1, 0.1015625), (1.0625, 1.0), (1.1875, 1.25), (2.0 ** -10, 0.0),
                                    (3 * 2.0 ** -10, 2.0 ** -8), (447.0, 448.0), (460.0, 448.0),
                                    (470.0, 448.0), (-500.0, -448.0), (1.0e6, 448.0),
                                    (-149.33, -144.0), (0.0, 0.0)])
def test_worked_values(x, want):
    """From the definition: step 2^(e-3) for normal values, 2^-9 below 2^-6,
    ties to the even mantissa, saturation at 448 (460 is below the midpoint
    464 between 448 and 480 and rounds to 448 anyway; 470, -500 and 1e6 reach
    448 only by saturating)."""
    assert e4m3_round(np.float32(x)) == want


def test_row_scales_map_the_row_maximum_to_448():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    codes, scale = quantize_rows_fp8(x)
    assert scale.dtype == np.float32
    assert np.array_equal(np.max(np.abs(codes), axis=1), np.full(50, E4M3_MAX))
    # an all-zero row gets scale 1 and zero codes (no 0 / 0)
    c0, s0 = quantize_rows_fp8(np.zeros((1, 8), dtype=np.float32))
    assert s0[0] == 1.0 and not c0.any()


def test_hand_worked_score():
    """Catches a dropped key scale, a query scale not folded into w, or the
    ReLU taken after the scales with a sign error."""
    g = json.load(open(os.path.join(GOLDEN, "fp8_indexer_tiny.json")))
    s, q8, wq, k8, ks = index_scores_fp8(np.array(g["qidx"]), np.array(g["w"]), np.array(g["kidx"]), g["q_pos0"])
    assert np.array_equal(q8, np.array(g["q_codes"], dtype=np.float64))
    assert np.array_equal(k8, np.array(g["k_codes"], dtype=np.float64))
    np.testing.assert_allclose(s, np.array(g["scores"]), rtol=1e-6, atol=0)


def test_exact_inputs_reduce_to_the_unquantised_score():
    """Rows that already hold e4m3 values with maximum 448 quantise with
    scale 1, so the fp8 score is the pinned unquantised score exactly."""
    rng = np.random.default_rng(2)
    T, H, D, L = 5, 4, 32, 9
    q = e4m3_round(rng.uniform(-448, 448, (T, H, D)))
    k = e4m3_round(rng.uniform(-448, 448, (L, D)))
    q[..., 0] = E4M3_MAX
    k[:, 0] = E4M3_MAX
    w = rng.standard_normal((T, H)).astype(np.float32)
    s8, q8, wq, k8, ks = index_scores_fp8(q, w, k, q_pos0=L - T)
    assert np.all(ks == 1.0) and np.array_equal(q8, q) and np.array_equal(wq, w)
    assert np.array_equal(s8, index_scores(q, w, k, L - T))
