"""Full-size GPU parity for every layer workload, in the launch configuration
the benchmark times (the same binding calls on the same buffers: routing and
scatter through moe_route_and_scatter; routed and shared experts through the
*_and_shared calls; expert weights stored [K, N]).

Checked on each workload:
  * routing: logits within the certified fp32 bound of the oracle's; top-k
    bit-exact against the oracle's top-k of the GPU logits; route weights
    within 1e-6;
  * scatter: scatter_index, row_token, expert_offsets and the status words
    bit-exact against the oracle; a sample of scattered rows bitwise equal to
    their token rows;
  * outputs: for sampled tokens, y and the tokens' expert rows Y_s against the
    oracle's per-token evaluation of the layer equation (float32, bf16
    activation rounding), within max|err| <= 2e-2 and relative Frobenius
    error <= 1e-2.
"""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_05_amd import binding as B
from mixture_experts_ffn_05_amd import workloads as wl
from oracle import moe_oracle as O
from tests.gpu_helpers import assert_grad_close, assert_output_close, check_routing, host

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FULL = ["scout", "qwen2", "v2l", "v2l_decode1", "v2l_decode16", "v2l_decode64", "v3", "v3_decode64"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    picks = {0, T - 1}
    picks.update(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(picks))


# every workload in the benchmark's configuration (routed rows gathered by fc1), two with the row copy
FULL_ROWS = [(n, "gather") for n in FULL] + [("v2l", "copy"), ("v3_decode64", "copy")]


@pytest.mark.parametrize("name,rows", FULL_ROWS, ids=[f"{n}-{r}" for n, r in FULL_ROWS])
def test_full_size_layer(name, rows):
    cfg = wl.WORKLOADS[name]
    print(f"[full] {name} ({rows}) T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.top_k} I={cfg.I} I_s={cfg.I_s}", flush=True)
    layer = wl.make_layer(cfg, DEV)
    x, wr = layer["x"], layer["w_router"]
    bias = layer["bias"]
    bias_t = torch.from_numpy(bias).to(DEV) if bias is not None else None
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s, x.dtype, DEV)
    bufs.y_rows.fill_(float("nan"))
    bufs.y.fill_(float("nan"))
    B.moe_layer_forward(x, wr, bias_t, layer["W1"], layer["W2"], cfg.top_k, shared=layer["shared"], bufs=bufs,
                        fused_shared=True, fused_route=True, gather=rows == "gather")
    torch.cuda.synchronize()

    # routing
    xh, wrh = host(x), host(wr)
    ids, w = host(bufs.topk_ids), host(bufs.topk_weights)
    near_ties = check_routing(host(bufs.logits), ids, w, xh, wrh, bias, cfg.top_k, O)
    print(f"[full] {name}: tokens whose oracle routes differ at near-ties: {near_ties}", flush=True)

    # scatter, bit-exact
    sc = O.build_scatter(ids, cfg.E)
    assert np.array_equal(host(bufs.scatter_index), sc["scatter_index"])
    assert np.array_equal(host(bufs.row_token), sc["row_token"])
    assert np.array_equal(host(bufs.expert_offsets), sc["offsets"])
    assert host(bufs.status_words).tolist() == [sc["max_group"], 0]
    if rows == "copy":
        pick = np.unique(np.concatenate([[0, cfg.R - 1], np.random.default_rng(1).integers(0, cfg.R, 256)]))
        xs = host(bufs.x_scattered[torch.from_numpy(pick).to(DEV)])
        assert np.array_equal(xs.view(np.uint32), xh[sc["row_token"][pick]].view(np.uint32))

    # every routed row and every output was written (the buffers were NaN-filled)
    assert torch.isfinite(bufs.y_rows[:cfg.R]).all().item(), f"{name}: a routed row was not computed"
    assert torch.isfinite(bufs.y).all().item(), f"{name}: non-finite output"

    # outputs on sampled tokens
    toks = _sample_tokens(cfg.T, 10 if cfg.E >= 256 else 24, seed=cfg.T)
    W1, W2 = layer["W1"], layer["W2"]
    shared = None
    if layer["shared"] is not None:
        ws1, ws2, wg = layer["shared"]
        shared = (host(ws1), host(ws2), host(wg) if wg is not None else None)
    ref = O.token_outputs(xh[toks], ids[toks], w[toks], lambda e: (host(W1[e]), host(W2[e])), shared=shared,
                          contract=True, dtype=np.float32)
    y = host(bufs.y)[toks]
    mx, rel = assert_output_close(y, ref["y"], "bf16", f"{name} y")
    Ys = host(bufs.y_rows)
    per_slot = np.stack([Ys[sc["scatter_index"][t]] for t in toks])
    assert_output_close(per_slot.reshape(-1, cfg.H), ref["per_slot"].reshape(-1, cfg.H), "bf16", f"{name} Y_s")
    print(f"[full] {name}: y max|err| {mx:.3e} rel_fro {rel:.3e} over {len(toks)} tokens", flush=True)


def _bench_layer(cfg):
    layer = wl.make_layer(cfg, DEV)
    layer["layout"] = B.MOE_W_KN
    layer["gather"] = True
    bias_t = torch.from_numpy(layer["bias"]).to(DEV) if layer["bias"] is not None else None
    return layer, bias_t


def _host_shared(layer):
    if layer["shared"] is None:
        return None
    ws1, ws2, wg = layer["shared"]
    return host(ws1), host(ws2), host(wg) if wg is not None else None


def _check_sampled_outputs(name, cfg, layer, bufs, ids, w, toks):
    """y and the sampled tokens' Y_s rows against the oracle's per-token layer equation."""
    xh = host(layer["x"])
    W1, W2 = layer["W1"], layer["W2"]
    ref = O.token_outputs(xh[toks], ids[toks], w[toks], lambda e: (host(W1[e]), host(W2[e])),
                          shared=_host_shared(layer), contract=True, dtype=np.float32)
    mx, rel = assert_output_close(host(bufs.y)[toks], ref["y"], "bf16", f"{name} y")
    si = host(bufs.scatter_index)
    Ys = host(bufs.y_rows)
    per_slot = np.stack([Ys[si[t]] for t in toks])
    assert_output_close(per_slot.reshape(-1, cfg.H), ref["per_slot"].reshape(-1, cfg.H), "bf16", f"{name} Y_s")
    return mx, rel


# The end-to-end contract: the oracle's routes (computed on the host from the
# oracle's own logits) fed into the GPU layer, in the benchmark's launch
# configuration after routing (scatter build, fc1 gathering rows from x with the
# shared expert, fc2 with the shared expert, combine).
FED = ["scout", "qwen2", "v2l", "v3", "v2l_decode1", "v2l_decode16", "v3_decode64"]


@pytest.mark.parametrize("name", FED)
def test_full_size_layer_oracle_routes_fed(name):
    import bench

    cfg = wl.WORKLOADS[name]
    print(f"[full-fed] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.top_k} I={cfg.I} I_s={cfg.I_s}", flush=True)
    layer, bias_t = _bench_layer(cfg)
    _, ids, w = O.route(host(layer["x"]), host(layer["w_router"]), cfg.top_k, layer["bias"])
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s, layer["x"].dtype, DEV)
    bufs.y_rows.fill_(float("nan"))
    bufs.y.fill_(float("nan"))
    bench.run_step(layer, bufs, cfg, bias_t, routes=(torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)))
    torch.cuda.synchronize()
    sc = O.build_scatter(ids, cfg.E)
    assert np.array_equal(host(bufs.scatter_index), sc["scatter_index"])
    assert np.array_equal(host(bufs.row_token), sc["row_token"])
    assert np.array_equal(host(bufs.expert_offsets), sc["offsets"])
    assert host(bufs.status_words).tolist() == [sc["max_group"], 0]
    assert torch.isfinite(bufs.y_rows[:cfg.R]).all().item(), f"{name}: a routed row was not computed"
    assert torch.isfinite(bufs.y).all().item(), f"{name}: non-finite output"
    toks = _sample_tokens(cfg.T, 10 if cfg.E >= 256 else 24, seed=cfg.T + 5)
    mx, rel = _check_sampled_outputs(name, cfg, layer, bufs, ids, w, toks)
    print(f"[full-fed] {name}: y max|err| {mx:.3e} rel_fro {rel:.3e} over {len(toks)} tokens", flush=True)


# HIP-graph replay, the launch mode of the benchmark's decode lines: one step of
# bench.run_step captured as bench.py captures it, replayed several times with
# eager work and synchronisations in between; every replay must reproduce the
# eager step bit for bit (all the kernels reduce in a fixed order), also after
# x changes in place, and the replayed outputs must match the oracle.
GRAPH = ["v2l_decode1", "v2l_decode16", "v2l_decode64", "v3_decode64"]


@pytest.mark.parametrize("name", GRAPH)
def test_graph_replay_decode(name):
    import bench

    cfg = wl.WORKLOADS[name]
    print(f"[graph] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.top_k}", flush=True)
    layer, bias_t = _bench_layer(cfg)
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s, layer["x"].dtype, DEV)
    outs = ("y", "y_rows", "topk_ids", "topk_weights", "logits", "scatter_index", "row_token", "expert_offsets",
            "status_words", "act")

    def eager():
        bench.run_step(layer, bufs, cfg, bias_t)
        torch.cuda.synchronize()
        return {k: getattr(bufs, k).clone() for k in outs}

    ref0 = eager()
    capture_stream = torch.cuda.Stream()
    capture_stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(capture_stream):
        with torch.cuda.graph(graph, stream=capture_stream):
            bench.run_step(layer, bufs, cfg, bias_t)
    torch.cuda.current_stream().wait_stream(capture_stream)
    torch.cuda.synchronize()

    def replay_matches(ref, what):
        for key in ("y", "y_rows", "act"):
            getattr(bufs, key).fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            a, b = getattr(bufs, k), ref[k]
            if a.is_floating_point():
                assert torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                                   b.view(torch.int16 if b.element_size() == 2 else torch.int32)), f"{what}: {k}"
            else:
                assert torch.equal(a, b), f"{what}: {k}"

    for rep in range(3):
        replay_matches(ref0, f"{name} replay {rep}")
        _ = torch.randn(1024, device=DEV).sum().item()   # eager work between replays

    # new tokens in place: the next T rows of the prefill draw
    base = wl.WORKLOADS[name.split("_")[0]]
    x2 = wl.make_x(base, DEV)[cfg.T:2 * cfg.T]
    layer["x"].copy_(x2)
    ref1 = eager()
    assert not torch.equal(ref1["y"], ref0["y"])
    for rep in range(2):
        replay_matches(ref1, f"{name} replay on new x {rep}")

    xh = host(layer["x"])
    ids, w = host(bufs.topk_ids), host(bufs.topk_weights)
    check_routing(host(bufs.logits), ids, w, xh, host(layer["w_router"]), layer["bias"], cfg.top_k, O)
    sc = O.build_scatter(ids, cfg.E)
    assert np.array_equal(host(bufs.scatter_index), sc["scatter_index"])
    assert np.array_equal(host(bufs.row_token), sc["row_token"])
    assert np.array_equal(host(bufs.expert_offsets), sc["offsets"])
    assert torch.isfinite(bufs.y_rows[:cfg.R]).all().item() and torch.isfinite(bufs.y).all().item()
    toks = _sample_tokens(cfg.T, 6 if cfg.E >= 256 else 12, seed=cfg.T + 9)
    mx, rel = _check_sampled_outputs(name, cfg, layer, bufs, ids, w, toks)
    print(f"[graph] {name}: replays bitwise equal to eager; y max|err| {mx:.3e} rel_fro {rel:.3e} over "
          f"{len(toks)} tokens", flush=True)


MX_FULL = ["v2l_decode1", "v2l_decode64", "v3_decode64"]


@pytest.mark.parametrize("name", MX_FULL)
def test_full_size_layer_mxfp8(name):
    """The benchmark's MXFP8 step (moe_route_and_scatter, the routed and shared experts through
    the *_and_shared_mx8 calls, combine) at full size; sampled tokens against the oracle on the
    dequantized weights."""
    cfg = wl.WORKLOADS[name]
    print(f"[full-mx] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.top_k} I={cfg.I} I_s={cfg.I_s}", flush=True)
    layer = wl.make_layer(cfg, DEV)
    mx = wl.mx_layer_weights(layer)
    del layer["W1"], layer["W2"]
    torch.cuda.empty_cache()
    x, wr = layer["x"], layer["w_router"]
    bias = layer["bias"]
    bias_t = torch.from_numpy(bias).to(DEV) if bias is not None else None
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s, x.dtype, DEV)
    bufs.y_rows.fill_(float("nan"))
    B.moe_route_and_scatter(x, wr, bias_t, cfg.top_k, bufs.topk_ids, bufs.topk_weights, bufs.logits,
                            bufs.scatter_index, bufs.row_token, bufs.expert_offsets, bufs.status_words,
                            bufs.x_scattered, bufs.route_scatter_ws)
    q1, s1, q2, s2, wg = mx["shared"]
    B.moe_grouped_swiglu_fc1_and_shared_mx8(bufs.x_scattered, bufs.expert_offsets, mx["W1q"], mx["W1s"], bufs.act,
                                            x, q1, s1, bufs.act_shared)
    B.moe_grouped_fc2_and_shared_mx8(bufs.act, bufs.expert_offsets, mx["W2q"], mx["W2s"], bufs.y_rows,
                                     bufs.act_shared, q2, s2, x, wg, bufs.y, bufs.shared_ws, accumulate=False)
    B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y, True)
    torch.cuda.synchronize()

    xh = host(x)
    ids, w = host(bufs.topk_ids), host(bufs.topk_weights)
    check_routing(host(bufs.logits), ids, w, xh, host(wr), bias, cfg.top_k, O)
    sc = O.build_scatter(ids, cfg.E)
    assert np.array_equal(host(bufs.scatter_index), sc["scatter_index"])
    assert np.array_equal(host(bufs.expert_offsets), sc["offsets"])

    def expert(e):   # K x N matrices, dequantized exactly by the oracle
        w1 = O.mx_dequant(host(mx["W1q"][e]), host(mx["W1s"][e]), axis=0).T.astype(np.float32)
        w2 = O.mx_dequant(host(mx["W2q"][e]), host(mx["W2s"][e]), axis=1).T.astype(np.float32)
        return np.ascontiguousarray(w1), np.ascontiguousarray(w2)

    shared = (np.ascontiguousarray(O.mx_dequant(host(q1), host(s1), axis=0).T.astype(np.float32)),
              np.ascontiguousarray(O.mx_dequant(host(q2), host(s2), axis=1).T.astype(np.float32)),
              host(wg) if wg is not None else None)
    toks = _sample_tokens(cfg.T, 4 if cfg.E >= 256 else 12, seed=cfg.T + 1)
    ref = O.token_outputs(xh[toks], ids[toks], w[toks], expert, shared=shared, contract=True, dtype=np.float32)
    mxe, rel = assert_output_close(host(bufs.y)[toks], ref["y"], "bf16", f"{name} mx y")
    print(f"[full-mx] {name}: y max|err| {mxe:.3e} rel_fro {rel:.3e} over {len(toks)} tokens", flush=True)


BWD_FULL = ["scout", "qwen2", "v2l_decode64", "v3_decode64", "v3"]


class _LazyExperts:
    """Expert weights as K x N host matrices, copied from the device on first use."""

    def __init__(self, w):
        self.w, self.cache = w, {}

    def __len__(self):
        return self.w.shape[0]

    def __getitem__(self, e):
        if e not in self.cache:
            self.cache[e] = host(self.w[e])
        return self.cache[e]


@pytest.mark.parametrize("name", BWD_FULL)
def test_full_size_backward(name):
    """The benchmark's backward step (bench.backward_setup, then bench.run_backward_step) at
    full size.  d_x and the route-weight gradients of sampled tokens depend on those tokens'
    rows only, so the oracle's backward over the sampled tokens gives them exactly; the weight
    gradients of the smallest non-empty expert group are recomputed from that group's rows."""
    import bench

    cfg = wl.WORKLOADS[name]
    print(f"[full-bwd] {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.top_k} I={cfg.I}", flush=True)
    layer = wl.make_layer(cfg, DEV)
    layer["shared"] = None
    layer["layout"] = B.MOE_W_KN
    torch.cuda.empty_cache()
    bias_t = torch.from_numpy(layer["bias"]).to(DEV) if layer["bias"] is not None else None
    bufs, bwd, dy = bench.backward_setup(cfg, layer, bias_t, DEV)
    for t in (bwd.d_rows, bwd.d_h, bwd.d_x, bwd.d_w1, bwd.d_w2, bwd.d_topk_weights):
        t.fill_(float("nan"))
    bench.run_backward_step(layer, bufs, bwd, dy)
    torch.cuda.synchronize()

    xh = host(layer["x"])
    ids, w = host(bufs.topk_ids), host(bufs.topk_weights)
    check_routing(host(bufs.logits), ids, w, xh, host(layer["w_router"]), layer["bias"], cfg.top_k, O)
    sc = O.build_scatter(ids, cfg.E)
    assert np.array_equal(host(bufs.scatter_index), sc["scatter_index"])
    dyh = host(dy)
    W1, W2 = _LazyExperts(layer["W1"]), _LazyExperts(layer["W2"])

    toks = _sample_tokens(cfg.T, 8 if cfg.E >= 256 else 16, seed=cfg.T + 2)
    ref = O.moe_backward(xh[toks], W1, W2, (ids[toks], w[toks]), dyh[toks], contract=True, dtype=np.float32,
                         weight_grads=False)
    assert_grad_close(host(bwd.d_x)[toks], ref["dx"], "bf16", f"{name} d_x")
    assert_grad_close(host(bwd.d_topk_weights)[toks], ref["dweights"], "bf16", f"{name} d_topk_weights")

    counts = sc["counts"]
    e = int(np.flatnonzero(counts)[np.argmin(counts[counts > 0])])
    sub = np.flatnonzero((ids == e).any(axis=1))
    ids_e = np.where(ids[sub] == e, 0, -1)            # expert e as the only expert; other slots dropped
    ref_e = O.moe_backward(xh[sub], [W1[e]], [W2[e]], (ids_e, w[sub]), dyh[sub], contract=True, dtype=np.float32)
    assert_grad_close(host(bwd.d_w1[e]), ref_e["dW1"][0], "bf16", f"{name} d_w1[{e}] ({counts[e]} rows)")
    assert_grad_close(host(bwd.d_w2[e]), ref_e["dW2"][0], "bf16", f"{name} d_w2[{e}] ({counts[e]} rows)")
    empty = np.flatnonzero(counts == 0)
    if empty.size:
        assert not host(bwd.d_w1[int(empty[0])]).any() and not host(bwd.d_w2[int(empty[0])]).any()
    assert torch.isfinite(bwd.d_x).all() and torch.isfinite(bwd.d_w1.float()).all()
    print(f"[full-bwd] {name}: sampled {len(toks)} tokens, expert {e} with {counts[e]} rows; "
          f"{empty.size} empty experts", flush=True)
