"""Pins for the CPU oracle: each test checks an oracle function against something
other than itself -- hand-derived examples, closed forms, brute force on tiny
inputs, invariants, or an independent library routine.  CPU only."""

import itertools
import math
from collections import Counter

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

F32_EPS = 2.0 ** -24


# ----------------------------------------------------------------------------- bf16
def test_bf16_rne_known_values():
    cases = {
        1.0 + 2.0 ** -8: 1.0,                       # exact tie, lower neighbour even
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,       # exact tie, upper neighbour even
        -(1.0 + 2.0 ** -8): -1.0,
        1.0 + 2.0 ** -8 + 2.0 ** -20: 1.0 + 2.0 ** -7,   # just above the tie
        1.0 + 2.0 ** -8 - 2.0 ** -20: 1.0,              # just below the tie
        0.0: 0.0,
        3.0: 3.0,
        float(np.finfo(np.float32).max): math.inf,  # rounds past the largest bf16
    }
    src = np.array(list(cases.keys()), np.float32)
    want = np.array(list(cases.values()), np.float32)
    got = O.bf16_rne(src)
    assert np.array_equal(got, want)
    assert np.isnan(O.bf16_rne(np.array([np.nan], np.float32)))[0]


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
        (rng.standard_normal(50000) * 1e-38).astype(np.float32),   # subnormals
        rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    v = v[~np.isnan(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_rne(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------------------- router
def test_router_logits_integer_brute_force():
    rng = np.random.default_rng(2)
    T, H, E = 5, 7, 4
    x = rng.integers(-3, 4, (T, H))
    w = rng.integers(-3, 4, (H, E))
    want = [[sum(int(x[t, h]) * int(w[h, e]) for h in range(H)) for e in range(E)] for t in range(T)]
    got = O.router_logits(x.astype(np.float32), w.astype(np.float32))
    assert got.dtype == np.float32
    assert np.array_equal(got, np.array(want, np.float32))
    b = np.array([0.5, -1.0, 0.0, 2.0], np.float32)
    got_b = O.router_logits(x.astype(np.float32), w.astype(np.float32), b)
    assert np.array_equal(got_b, np.array(want, np.float32) + b)


def test_routing_hand_example(golden):
    g = golden["routing"]
    L, ids, w = O.route(np.array(g["x"], np.float32), np.array(g["w_router"], np.float32), g["top_k"])
    assert np.array_equal(L, np.array(g["logits"], np.float32))
    assert np.array_equal(ids, np.array(g["ids"]))
    assert np.allclose(w, np.array(g["weights"]), rtol=0, atol=1e-7)


@pytest.mark.parametrize("E", list(range(1, 11)))
def test_topk_brute_force_with_forced_ties(E):
    rng = np.random.default_rng(100 + E)
    for k in range(1, min(3, E) + 1):
        L = rng.integers(0, 3, (40, E)).astype(np.float32)     # values {0,1,2}: many ties
        ids = O.topk_select(L, k)
        for t in range(L.shape[0]):
            def beats(a, b):   # a ranks before b: larger value, then lower index
                return (L[t, a] > L[t, b]) or (L[t, a] == L[t, b] and a < b)
            dominating = [set(S) for S in itertools.combinations(range(E), k)
                          if all(beats(a, b) for a in S for b in range(E) if b not in S)]
            assert len(dominating) == 1
            assert set(ids[t].tolist()) == dominating[0]
            order = sorted(dominating[0], key=lambda e: (-float(L[t, e]), e))
            assert ids[t].tolist() == order


def test_topk_deepseek_v3_width_selects_expert_255():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((16, 256)).astype(np.float32)
    L[:, 255] = L.max(axis=1) + 1.0
    ids = O.topk_select(L, 8)
    assert (ids[:, 0] == 255).all()
    assert all(len(set(r)) == 8 for r in ids.tolist())


def test_topk_rejects_nonpositive_k():
    with pytest.raises(ValueError):
        O.topk_select(np.zeros((2, 4), np.float32), 0)


def test_route_weights_properties():
    rng = np.random.default_rng(4)
    for E, k in [(16, 1), (60, 4), (64, 6), (256, 8), (8, 2)]:
        L = (rng.standard_normal((64, E)) * 2).astype(np.float32)
        ids = O.topk_select(L, k)
        w = O.route_weights(L, ids)
        assert w.dtype == np.float32
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 4 * F32_EPS)
        if k == 1:
            assert np.all(w == 1.0)
        # renormalised softmax over all E experts (different formula, float64)
        p = np.exp(L.astype(np.float64) - L.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        sel = np.take_along_axis(p, ids.astype(np.int64), 1)
        ref = sel / sel.sum(1, keepdims=True)
        assert np.max(np.abs(w - ref)) <= 6e-8
        assert np.all(np.diff(w, axis=1) <= 0)     # slot order: weights non-increasing


def _fp32_sums(x, w, order):
    """x @ w accumulated in float32 one product at a time, in the given order of h."""
    acc = np.zeros((x.shape[0], w.shape[1]), np.float32)
    for h in order:
        acc = (acc + (x[:, h:h + 1] * w[h:h + 1, :]).astype(np.float32)).astype(np.float32)
    return acc


def test_router_logit_bound_covers_float32_accumulation_orders():
    # float32 sums in three orders (forward, reverse, and blocked partial sums
    # added at the end, as split-K kernels do) against the float64 product:
    # every error lies inside the bound, including under heavy cancellation.
    rng = np.random.default_rng(11)
    H, E = 512, 16
    x = torch.from_numpy(rng.standard_normal((24, H)).astype(np.float32)).bfloat16().float().numpy()
    w = torch.from_numpy((rng.standard_normal((H, E)) * 0.02).astype(np.float32)).bfloat16().float().numpy()
    x[:4] = np.abs(x[:4]) * 1e3                     # large same-sign terms
    w[:, :2] = np.abs(w[:, :2])
    x[4:8, 1::2] = -x[4:8, 0::2]                    # exact cancellation pairs
    bias = (rng.standard_normal(E) * 3).astype(np.float32)
    exact = O.router_logits(x, w, bias).astype(np.float64)
    bound = O.router_logit_bound(x, w, bias)
    for order in (range(H), range(H - 1, -1, -1)):
        got = (_fp32_sums(x, w, order) + bias[None, :]).astype(np.float32)
        assert np.all(np.abs(got - exact) <= bound)
    blocks = [_fp32_sums(x[:, b:b + 64], w[b:b + 64], range(64)) for b in range(0, H, 64)]
    got = np.zeros_like(blocks[0])
    for part in blocks:
        got = (got + part).astype(np.float32)
    got = (got + bias[None, :]).astype(np.float32)
    assert np.all(np.abs(got - exact) <= bound)


def test_router_logit_bound_closed_form():
    # one term: gamma_1 |x||w| doubled plus four units of |value| + |bias|
    u = 2.0 ** -24
    b = O.router_logit_bound(np.array([[3.0]]), np.array([[-2.0]]), np.array([5.0], np.float32))
    gamma = u / (1 - u)
    assert b[0, 0] == pytest.approx(2 * gamma * 6.0 + 4 * u * (6.0 + 5.0) + 1e-30, rel=1e-12)
    # H equal terms: gamma_H grows with H and so does the magnitude
    for H in (100, 200):
        gH = H * u / (1 - H * u)
        b = O.router_logit_bound(np.ones((1, H)), np.ones((H, 1)))
        assert b[0, 0] == pytest.approx(2 * gH * H + 4 * u * H + 1e-30, rel=1e-12)


# ----------------------------------------------------------------------------- scatter
def _check_scatter_invariants(ids, E, sc):
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    cnt = Counter(int(e) for e in flat[valid])
    assert [cnt.get(e, 0) for e in range(E)] == sc["counts"].tolist()
    assert sc["offsets"][0] == 0
    assert np.array_equal(np.diff(sc["offsets"]), sc["counts"])
    assert sc["max_group"] == max(cnt.values(), default=0)
    assert sc["n_bad"] == int((~valid).sum())
    si = sc["scatter_index"].reshape(-1)
    assert np.all(si[~valid] == -1)
    nvalid = int(valid.sum())
    assert sorted(si[valid].tolist()) == list(range(nvalid))          # a permutation
    for p in np.nonzero(valid)[0]:
        e = flat[p]
        assert sc["offsets"][e] <= si[p] < sc["offsets"][e + 1]       # inside its group
        assert sc["row_token"][si[p]] == p // k
    for e in range(E):                                                # stable within a group
        ps = [p for p in range(T * k) if flat[p] == e]
        assert si[ps].tolist() == list(range(sc["offsets"][e], sc["offsets"][e + 1]))


def test_scatter_hand_example(golden):
    g = golden["scatter"]
    sc = O.build_scatter(np.array(g["ids"]), g["num_experts"])
    for key in ("counts", "offsets", "scatter_index", "row_token"):
        assert sc[key].tolist() == g[key], key
    assert sc["max_group"] == g["max_group"]


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (37, 8, 2), (64, 60, 4), (33, 256, 8), (20, 3, 5)])
def test_scatter_invariants_random_with_duplicates(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)          # duplicates allowed
    _check_scatter_invariants(ids, E, O.build_scatter(ids, E))


def test_scatter_counts_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 1], [2, 2]], np.int32)
    sc = O.build_scatter(ids, 3)
    _check_scatter_invariants(ids, 3, sc)
    assert sc["n_bad"] == 2 and sc["offsets"][-1] == 4


def test_scatter_duplicate_and_balanced_patterns(golden):
    g = golden["duplicate_routes"]
    T, k = g["tokens"], g["top_k"]
    dup = np.zeros((T, k), np.int32)
    sc = O.build_scatter(dup, 8)
    assert sc["counts"][0] == g["duplicate_group_rows"]["0"] == 2 * T
    assert sc["max_group"] == 256
    assert np.array_equal(sc["scatter_index"], np.arange(T * k).reshape(T, k))   # 2t + j
    bal = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    sc = O.build_scatter(bal, 8)
    assert sc["counts"][0] == g["balanced_group_rows"]["0"]
    assert sc["counts"][1] == g["balanced_group_rows"]["1"]
    assert sc["max_group"] == T


def test_scatter_rows_copies_token_rows_bitwise():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 16)).astype(np.float32)
    ids = rng.integers(0, 6, (30, 3)).astype(np.int32)
    sc = O.build_scatter(ids, 6)
    Xs = O.scatter_rows(x, sc["row_token"])
    for t in range(30):
        for j in range(3):
            assert np.array_equal(Xs[sc["scatter_index"][t, j]].view(np.uint32), x[t].view(np.uint32))


# ----------------------------------------------------------------------------- experts
def test_silu_closed_forms():
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 1.0, -800.0, 800.0])
    s = O.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(s[2] - (-0.25 * math.log(3.0))) < 1e-15
    assert abs(s[3] - math.e / (1 + math.e)) < 1e-15
    assert s[4] == 0.0 or abs(s[4]) < 1e-300
    assert s[5] == 800.0


def test_swiglu_ffn_hand_example(golden):
    g = golden["swiglu_ffn"]
    a, y = O.expert_ffn(np.array(g["x"], float), np.array(g["w1"], float), np.array(g["w2"], float))
    assert np.allclose(a, g["a"], rtol=1e-15, atol=0)
    assert np.allclose(y, g["y"], rtol=1e-15, atol=0)


def test_swiglu_contract_mode_rounds_activation():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((9, 32)).astype(np.float32)
    w1 = (rng.standard_normal((32, 48)) * 0.2).astype(np.float32)
    w2 = (rng.standard_normal((24, 32)) * 0.2).astype(np.float32)
    a, y = O.expert_ffn(x, w1, w2, contract=True, dtype=np.float32)
    assert np.array_equal(O.bf16_rne(a), a)
    a_exact, _ = O.expert_ffn(x, w1, w2, dtype=np.float64)
    assert np.max(np.abs(a - a_exact) / (np.abs(a_exact) + 1e-30)) <= 2.0 ** -8 + 1e-6


def _tiny_layer(rng, T=24, H=16, E=5, I=8, scale=0.3):
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((H, E)) * scale
    W1 = [rng.standard_normal((H, 2 * I)) * scale for _ in range(E)]
    W2 = [rng.standard_normal((I, H)) * scale for _ in range(E)]
    return x, wr, W1, W2


@pytest.mark.parametrize("k", [1, 2, 3])
def test_forward_equals_dense_mask_formulation(k):
    rng = np.random.default_rng(7 + k)
    x, wr, W1, W2 = _tiny_layer(rng)
    out = O.moe_forward(x, wr, W1, W2, k)
    ref = O.dense_mask_forward(x, W1, W2, out["ids"], out["weights"])
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())
    # fed-in routes with duplicates and arbitrary weights
    ids = rng.integers(0, 5, (24, k)).astype(np.int32)
    w = rng.random((24, k)).astype(np.float32)
    out = O.moe_forward(x, None, W1, W2, k, routes=(ids, w))
    ref = O.dense_mask_forward(x, W1, W2, ids, w)
    assert np.max(np.abs(out["y"] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


def test_all_duplicate_routes_zero_error_all_rows_computed(golden):
    g = golden["duplicate_routes"]
    rng = np.random.default_rng(8)
    T, k = g["tokens"], g["top_k"]
    x, _, W1, W2 = _tiny_layer(rng, T=T, H=32, E=4, I=16)
    ids = np.zeros((T, k), np.int32)
    w = np.full((T, k), 0.5, np.float32)
    for dt in (np.float64, np.float32):
        out = O.moe_forward(x.astype(dt), None, W1, W2, k, routes=(ids, w), dtype=dt)
        assert not np.isnan(out["A"][: 2 * T]).any() and not np.isnan(out["Ys"][: 2 * T]).any()
        _, y0 = O.expert_ffn(x.astype(dt), W1[0], W2[0], dtype=dt)
        assert np.array_equal(out["y"], y0)                       # 0.5a + 0.5a == a exactly
        assert np.array_equal(out["Ys"][0::2], out["Ys"][1::2])


def test_stale_bound_mutation_is_caught_only_by_duplicates(golden):
    """Plant the stale per-group bound (rows per group capped at T) in the oracle:
    the all-duplicate all-rows check must fail, the balanced control must not."""
    g = golden["duplicate_routes"]
    rng = np.random.default_rng(9)
    T, k = g["tokens"], g["top_k"]
    x, _, W1, W2 = _tiny_layer(rng, T=T, H=16, E=2, I=8)
    w = np.full((T, k), 0.5, np.float32)
    bal = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    good = O.moe_forward(x, None, W1, W2, k, routes=(bal, w))
    stale = O.moe_forward(x, None, W1, W2, k, routes=(bal, w), _stale_row_bound=T)
    assert np.array_equal(good["y"], stale["y"])
    dup = np.zeros((T, k), np.int32)
    stale = O.moe_forward(x, None, W1, W2, k, routes=(dup, w), _stale_row_bound=T)
    assert np.isnan(stale["Ys"][:2 * T]).any() and np.isnan(stale["y"]).any()


def test_out_of_range_fed_ids_contribute_nothing():
    rng = np.random.default_rng(10)
    x, _, W1, W2 = _tiny_layer(rng, T=6, E=3)
    ids = np.array([[0, 7]] * 6, np.int32)
    w = np.full((6, 2), 0.5, np.float32)
    out = O.moe_forward(x, None, W1, W2, 2, routes=(ids, w))
    _, y0 = O.expert_ffn(x, W1[0], W2[0])
    assert out["n_bad"] == 6
    assert np.allclose(out["y"], 0.5 * y0, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- shared
def test_fusion_identity():
    rng = np.random.default_rng(11)
    H, I, T = 24, 12, 10
    x = rng.standard_normal((T, H))
    experts = [(rng.standard_normal((H, 2 * I)) * 0.3, rng.standard_normal((I, H)) * 0.3) for _ in range(2)]
    ws1, ws2 = O.fuse_shared(experts)
    assert ws1.shape == (H, 4 * I) and ws2.shape == (2 * I, H)
    fused = O.shared_expert(x, ws1, ws2)
    summed = sum(O.expert_ffn(x, w1, w2)[1] for w1, w2 in experts)
    assert np.max(np.abs(fused - summed)) <= 1e-12 * np.abs(summed).max()
    x32 = x.astype(np.float32)
    e32 = [(a.astype(np.float32), b.astype(np.float32)) for a, b in experts]
    f32 = O.shared_expert(x32, *O.fuse_shared(e32), dtype=np.float32)
    s32 = sum(O.expert_ffn(x32, a, b, dtype=np.float32)[1] for a, b in e32)
    assert np.max(np.abs(f32 - s32)) <= 1e-5 * np.abs(s32).max()


def test_shared_gate_closed_forms(golden):
    g = golden["sigmoid_gate"]
    rng = np.random.default_rng(12)
    H, I = 8, 4
    ws1 = rng.standard_normal((H, 2 * I))
    ws2 = rng.standard_normal((I, H))
    x = np.zeros((2, H))
    x[0, 0] = math.log(3.0)
    x[1, 1] = 1.0
    x[1, 0] = 0.0
    wg = np.zeros(H)
    wg[0] = 1.0
    ungated = O.shared_expert(x, ws1, ws2)
    gated = O.shared_expert(x, ws1, ws2, wg)
    assert np.allclose(gated[0], g["gate_at_ln3"] * ungated[0], rtol=1e-15, atol=0)
    assert np.array_equal(gated[1], g["gate_at_0"] * ungated[1])
    assert np.array_equal(O.shared_expert(x, ws1, ws2, np.zeros(H)), 0.5 * ungated)


def test_scout_shaped_top1_closed_form():
    rng = np.random.default_rng(13)
    x, wr, W1, W2 = _tiny_layer(rng, T=20, E=4)
    ws1 = rng.standard_normal((16, 2 * 8)) * 0.3
    ws2 = rng.standard_normal((8, 16)) * 0.3
    out = O.moe_forward(x, wr, W1, W2, 1, shared=(ws1, ws2, None))
    assert np.all(out["weights"] == 1.0)
    _, ys = O.expert_ffn(x, ws1, ws2)
    for t in range(20):
        _, ye = O.expert_ffn(x[t:t + 1], W1[out["ids"][t, 0]], W2[out["ids"][t, 0]])
        assert np.allclose(out["y"][t], ys[t] + ye[0], rtol=1e-13, atol=1e-13)


def test_token_outputs_matches_forward():
    rng = np.random.default_rng(14)
    x, wr, W1, W2 = _tiny_layer(rng, T=30, E=6)
    ws1 = rng.standard_normal((16, 2 * 8)) * 0.3
    ws2 = rng.standard_normal((8, 16)) * 0.3
    wg = rng.standard_normal(16) * 0.3
    out = O.moe_forward(x, wr, W1, W2, 2, shared=(ws1, ws2, wg), contract=True)
    sel = np.array([0, 7, 29])
    tok = O.token_outputs(x[sel], out["ids"][sel], out["weights"][sel], lambda e: (W1[e], W2[e]),
                          shared=(ws1, ws2, wg), contract=True)
    assert np.allclose(tok["y"], out["y"][sel], rtol=1e-12, atol=1e-12)
    for n, t in enumerate(sel):
        for j in range(2):
            assert np.allclose(tok["per_slot"][n, j], out["Ys"][out["scatter_index"][t, j]], rtol=1e-12, atol=1e-12)


# ---- MXFP8 expert weights ([PLENA-C] "Group C -- shared experts", fusion-identity paragraph:
# e4m3 values, one e8m0 scale per block of 8 along the intermediate axis; OCP encodings)

def test_e4m3_decode_matches_torch_float8_on_every_code():
    import torch
    v = O.e4m3_decode(np.arange(256))
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    assert np.isnan(v).sum() == 2                     # only S.1111.111


def test_e4m3_and_e8m0_known_values():
    known = {0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0xB8: -1.0, 0x7E: 448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x00: 0.0}
    for code, val in known.items():
        assert O.e4m3_decode(code) == val, hex(code)
    neg0 = O.e4m3_decode(0x80)
    assert neg0 == 0.0 and np.signbit(neg0)
    assert np.isnan(O.e4m3_decode(0x7F)) and np.isnan(O.e4m3_decode(0xFF))
    assert O.e8m0_decode(127) == 1.0 and O.e8m0_decode(120) == 2.0 ** -7
    assert O.e8m0_decode(0) == 2.0 ** -127 and O.e8m0_decode(254) == 2.0 ** 127
    assert np.isnan(O.e8m0_decode(255))


def test_mx_dequant_blocks_run_along_the_given_axis():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 0x7F, (24, 40))           # no NaN codes
    codes[rng.random(codes.shape) < 0.5] |= 0x80      # both signs
    for axis in (0, 1):
        sshape = (24 // 8, 40) if axis == 0 else (24, 40 // 8)
        scales = rng.integers(110, 140, sshape)
        W = O.mx_dequant(codes, scales, axis)
        # one element by hand
        r, c = 13, 29
        s = scales[r // 8, c] if axis == 0 else scales[r, c // 8]
        assert W[r, c] == O.e4m3_decode(codes[r, c]) * 2.0 ** (int(s) - 127)
        # raising one scale by 1 doubles exactly its block of 8 along `axis`
        bumped = scales.copy()
        bumped[1, 2] += 1
        W2 = O.mx_dequant(codes, bumped, axis)
        changed = W2 != W
        block = np.zeros_like(changed)
        if axis == 0:
            block[8:16, 2] = True
        else:
            block[1, 16:24] = True
        assert np.array_equal(changed, block & (W != 0))
        assert np.array_equal(W2[block], 2 * W[block])
    with pytest.raises(ValueError):
        O.mx_dequant(codes, np.ones((3, 41), np.int64), 0)
