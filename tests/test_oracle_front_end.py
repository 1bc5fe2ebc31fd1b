"""Pins of the indexer front-end oracle to facts other than its own code: a
hand-worked fixture, special cases with a known answer, torch's float64
linear layer, and linearity. Each test names the mistake it would catch."""
import json
import os

import numpy as np
import torch

from oracle import indexer_front_end

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_fixture():
    """Catches a transposed weight, a dim-major instead of head-major split of
    q_b's output, and x / q_lat swapped between the maps."""
    g = json.load(open(os.path.join(GOLDEN, "front_end_tiny.json")))
    qidx, kidx, w = indexer_front_end(np.array(g["x"]), np.array(g["q_lat"]), np.array(g["w_qb"]),
                                      np.array(g["w_k"]), np.array(g["w_proj"]), g["idx_heads"], g["idx_dim"])
    assert np.array_equal(qidx, np.array(g["qidx"], dtype=np.float64))
    assert np.array_equal(kidx, np.array(g["kidx"], dtype=np.float64))
    assert np.array_equal(w, np.array(g["w"], dtype=np.float64))


def test_identity_q_b_splits_heads_major():
    """With w_qb = I the query of head h is q_lat[h*D_I : (h+1)*D_I]."""
    HI, DI, T = 3, 4, 5
    rng = np.random.default_rng(0)
    q_lat = rng.standard_normal((T, HI * DI))
    x = rng.standard_normal((T, 8))
    qidx, _, _ = indexer_front_end(x, q_lat, np.eye(HI * DI), np.zeros((DI, 8)), np.zeros((HI, 8)), HI, DI)
    for h in range(HI):
        assert np.array_equal(qidx[:, h, :], q_lat[:, h * DI : (h + 1) * DI])


def test_selector_rows_pick_input_columns():
    """w_k / w_proj rows that are unit vectors copy the chosen activation
    columns (catches an index mix-up between output and input dims)."""
    T, hidden, HI, DI = 4, 9, 2, 3
    x = np.arange(T * hidden, dtype=np.float64).reshape(T, hidden)
    wk = np.zeros((DI, hidden))
    wp = np.zeros((HI, hidden))
    for d, j in enumerate((7, 0, 4)):
        wk[d, j] = 1.0
    for h, j in enumerate((8, 2)):
        wp[h, j] = -2.0
    _, kidx, w = indexer_front_end(x, np.zeros((T, 2)), np.zeros((HI * DI, 2)), wk, wp, HI, DI)
    assert np.array_equal(kidx, x[:, [7, 0, 4]])
    assert np.array_equal(w, -2.0 * x[:, [8, 2]])


def test_matches_torch_linear_float64():
    """torch.nn.functional.linear (y = x W^T) in float64 on the CPU."""
    T, hidden, rank, HI, DI = 6, 40, 24, 4, 8
    g = torch.Generator().manual_seed(3)
    x = torch.randn(T, hidden, generator=g, dtype=torch.float64)
    ql = torch.randn(T, rank, generator=g, dtype=torch.float64)
    wqb = torch.randn(HI * DI, rank, generator=g, dtype=torch.float64)
    wk = torch.randn(DI, hidden, generator=g, dtype=torch.float64)
    wp = torch.randn(HI, hidden, generator=g, dtype=torch.float64)
    qidx, kidx, w = indexer_front_end(x.numpy(), ql.numpy(), wqb.numpy(), wk.numpy(), wp.numpy(), HI, DI)
    F = torch.nn.functional
    np.testing.assert_allclose(qidx, F.linear(ql, wqb).view(T, HI, DI).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kidx, F.linear(x, wk).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(w, F.linear(x, wp).numpy(), rtol=1e-12, atol=1e-12)


def test_linear_in_activations():
    """Doubling the activations doubles every output exactly (no bias, no
    norm, no hidden constant)."""
    rng = np.random.default_rng(5)
    T, hidden, rank, HI, DI = 3, 16, 8, 2, 4
    args = [rng.standard_normal(s) for s in ((T, hidden), (T, rank), (HI * DI, rank), (DI, hidden), (HI, hidden))]
    a = indexer_front_end(*args, HI, DI)
    b = indexer_front_end(2 * args[0], 2 * args[1], *args[2:], HI, DI)
    for u, v in zip(a, b):
        assert np.array_equal(2 * u, v)
