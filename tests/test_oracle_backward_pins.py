"""Pins of the oracle's backward (CPU only): each compares the hand-derived
gradients with something that does not use them -- central finite differences
of the oracle's forward, PyTorch autograd (CPU, float64) through a per-pair
formulation with no scatter or grouping, the split-fc1 formulation, and the
exact identities of duplicate routes ([VEOMNI] "Regression test pattern")."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def _problem(seed=3, T=12, H=16, E=4, k=2, I=8, dup_tokens=(1, 5), empty_expert=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W1 = rng.standard_normal((E, H, 2 * I)) / np.sqrt(H)
    W2 = rng.standard_normal((E, I, H)) / np.sqrt(I)
    ids = rng.integers(0, E, size=(T, k))
    ids[ids == empty_expert] = 0          # one expert receives no rows
    for t in dup_tokens:                  # duplicate routes: both slots name one expert
        ids[t, :] = ids[t, 0]
    w = rng.uniform(0.1, 1.0, size=(T, k))
    dy = rng.standard_normal((T, H))
    return x, W1, W2, ids, w, dy


def _loss(x, W1, W2, ids, w, dy):
    """L = sum(dy * y) for the routed layer, through the oracle's forward (float64)."""
    sc = O.build_scatter(ids, len(W1))
    Xs = O.scatter_rows(x, sc["row_token"])
    _, Ys = O.grouped_experts(Xs, sc["offsets"], list(W1), list(W2))
    y = O.gather_combine(Ys, sc["scatter_index"], w)
    return float(np.sum(dy * y))


def test_swiglu_grad_matches_central_differences():
    rng = np.random.default_rng(0)
    g = np.concatenate([rng.standard_normal(200) * 3, [0.0, -20.0, 20.0, 1e-3]])
    u = rng.standard_normal(g.shape)
    dA = rng.standard_normal(g.shape)
    dG, dU = O.swiglu_grad(g, u, dA)
    f = lambda gg, uu: O.silu(gg) * uu
    h = 1e-6
    fd_g = (f(g + h, u) - f(g - h, u)) / (2 * h) * dA
    fd_u = (f(g, u + h) - f(g, u - h)) / (2 * h) * dA
    np.testing.assert_allclose(dG, fd_g, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(dU, fd_u, rtol=1e-7, atol=1e-9)
    # closed forms at g = 0: silu'(0) = 1/2 and silu(0) = 0
    dG0, dU0 = O.swiglu_grad(np.zeros(1), np.ones(1), np.ones(1))
    assert dG0[0] == 0.5 and dU0[0] == 0.0


@pytest.mark.parametrize("which", ["x", "W1", "W2", "w"])
def test_gradients_match_directional_derivatives(which):
    x, W1, W2, ids, w, dy = _problem()
    g = O.moe_backward(x, list(W1), list(W2), (ids, w), dy)
    grad = {"x": g["dx"], "W1": g["dW1"], "W2": g["dW2"], "w": g["dweights"]}[which]
    params = {"x": x, "W1": W1, "W2": W2, "w": w}
    rng = np.random.default_rng(11)
    d = rng.standard_normal(params[which].shape)
    eps = 1e-5

    def at(sign):
        p = dict(params)
        p[which] = params[which] + sign * eps * d
        return _loss(p["x"], p["W1"], p["W2"], ids, p["w"], dy)

    fd = (at(+1) - at(-1)) / (2 * eps)
    an = float(np.sum(grad * d))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_gradients_match_torch_autograd_per_pair():
    """Eager per-(token, slot) formulation with no scatter, grouping or gather."""
    x, W1, W2, ids, w, dy = _problem(seed=5, T=10, H=24, E=5, k=3, I=16)
    tx = torch.tensor(x, requires_grad=True)
    tW1 = torch.tensor(W1, requires_grad=True)
    tW2 = torch.tensor(W2, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    I = W2.shape[1]
    rows = []
    for t in range(x.shape[0]):
        yt = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            h = tx[t] @ tW1[e]
            a = torch.nn.functional.silu(h[:I]) * h[I:]
            yt = yt + tw[t, j] * (a @ tW2[e])
        rows.append(yt)
    L = (torch.stack(rows) * torch.tensor(dy)).sum()
    L.backward()
    g = O.moe_backward(x, list(W1), list(W2), (ids, w), dy)
    for name, ref in [("dx", tx.grad), ("dW1", tW1.grad), ("dW2", tW2.grad), ("dweights", tw.grad)]:
        np.testing.assert_allclose(g[name], ref.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_split_and_merged_fc1_agree():
    x, W1, W2, ids, w, dy = _problem(seed=7, T=16, H=32, E=4, k=2, I=12)
    merged = O.moe_backward(x, list(W1), list(W2), (ids, w), dy)
    split = O.moe_backward(x, list(W1), list(W2), (ids, w), dy, split_fc1=True)
    for name in ("dx", "dW1", "dW2", "dweights"):
        np.testing.assert_allclose(split[name], merged[name], rtol=1e-12, atol=1e-12, err_msg=name)


def _all_duplicate(k, weight, T=128, H=32, E=3, I=16, seed=9):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W1 = rng.standard_normal((E, H, 2 * I)) / np.sqrt(H)
    W2 = rng.standard_normal((E, I, H)) / np.sqrt(I)
    dy = rng.standard_normal((T, H))
    ids = np.zeros((T, k), np.int64)          # selected_experts = zeros([tokens, topk])
    w = np.full((T, k), weight)               # routing_weights = full([tokens, topk], weight)
    return x, list(W1), list(W2), ids, w, dy


def test_all_duplicate_routes_equal_one_route_of_summed_weight():
    """[VEOMNI] "Duplicate top-k routes": tokens=128, topk=2, every slot on expert 0
    (a group of 256 rows).  Since y = sum_j w f_0(x) = (k w) f_0(x), the gradients
    equal those of a single route of weight k*w, and all are finite."""
    k, weight = 2, 0.3
    x, W1, W2, ids, w, dy = _all_duplicate(k, weight)
    dup = O.moe_backward(x, W1, W2, (ids, w), dy)
    assert dup["max_group"] == 2 * x.shape[0]
    one = O.moe_backward(x, W1, W2, (ids[:, :1], np.full((x.shape[0], 1), k * weight)), dy)
    for name in ("dx", "dW1", "dW2"):
        assert np.isfinite(dup[name]).all(), name
        np.testing.assert_allclose(dup[name], one[name], rtol=1e-12, atol=1e-12, err_msg=name)
    # every slot of a token sees the same expert output, so the same weight gradient
    np.testing.assert_allclose(dup["dweights"][:, 0], dup["dweights"][:, 1], rtol=0, atol=0)
    np.testing.assert_allclose(dup["dweights"][:, 0], one["dweights"][:, 0], rtol=1e-12, atol=1e-12)


def test_stale_token_bound_is_caught_by_the_finiteness_check():
    """Mutation: a launch bound of `tokens` rows per group leaves rows 128..255 of
    expert 0 uncomputed; the finiteness check above must then fail."""
    x, W1, W2, ids, w, dy = _all_duplicate(2, 0.3)
    bad = O.moe_backward(x, W1, W2, (ids, w), dy, _stale_row_bound=x.shape[0])
    assert not np.isfinite(bad["dx"]).all()
    good = O.moe_backward(x, W1, W2, (ids, w), dy)
    assert not np.allclose(bad["dW1"], good["dW1"])


def test_empty_expert_has_zero_weight_gradients_and_bad_ids_add_nothing():
    x, W1, W2, ids, w, dy = _problem()
    ids = ids.copy()
    ids[0, 1] = 99                       # out of range: no row, no gradient
    g = O.moe_backward(x, list(W1), list(W2), (ids, w), dy)
    assert g["counts"][3] == 0
    assert not g["dW1"][3].any() and not g["dW2"][3].any()
    assert g["dweights"][0, 1] == 0.0
    assert np.isfinite(g["dx"]).all()


def test_contract_mode_rounds_stored_intermediates_only():
    x, W1, W2, ids, w, dy = _problem(seed=4, T=20, H=32, E=4, k=2, I=16)
    c = O.moe_backward(x, list(W1), list(W2), (ids, w), dy, contract=True)
    e = O.moe_backward(x, list(W1), list(W2), (ids, w), dy)
    valid = c["row_token"] >= 0
    for name in ("H_pre", "A", "dYs", "dH"):
        v = c[name][valid].astype(np.float32)
        assert np.array_equal(O.bf16_rne(v), v), name
    for name in ("dx", "dW1", "dW2", "dweights"):
        rel = np.linalg.norm(c[name] - e[name]) / np.linalg.norm(e[name])
        assert rel < 1e-2, (name, rel)


def test_skipping_weight_gradients_changes_nothing_else():
    x, W1, W2, ids, w, dy = _problem(seed=8)
    full = O.moe_backward(x, list(W1), list(W2), (ids, w), dy, contract=True)
    part = O.moe_backward(x, list(W1), list(W2), (ids, w), dy, contract=True, weight_grads=False)
    assert part["dW1"] is None and part["dW2"] is None
    for name in ("dx", "dweights", "dH", "dXs", "dYs"):
        np.testing.assert_array_equal(part[name], full[name], err_msg=name)
