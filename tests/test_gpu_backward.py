"""GPU parity of the routed experts' backward against the CPU oracle
(moe_backward), through the C ABI: the training forward (fc1 keeping its
pre-activation), the scattered output gradient and route-weight gradient, the
same-N/K input-gradient GEMMs with SwiGLU' in the epilogue, the same-M/N
weight-gradient GEMMs and the gather of input gradients back to tokens.

Cases span several tiles, ragged row/column/reduction tails, T = 1 with most
experts empty, 256 experts, groups of >= 512 rows, both weight layouts, and the
duplicate-route regression pattern ([VEOMNI] "Regression test pattern": every
slot of every token on expert 0, a group of twice the token count; split-fc1,
merged-fc1 and eager results compared, every gradient finite)."""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_05_amd import binding as B
from mixture_experts_ffn_05_amd import workloads as wl
from oracle import moe_oracle as O
from tests.gpu_helpers import assert_grad_close, host

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    wl.TINY,
    wl.LayerConfig("ragged_bf16", "bf16", T=300, H=264, E=7, top_k=2, I=200),
    wl.LayerConfig("mid_bf16", "bf16", T=517, H=512, E=16, top_k=4, I=136),
    wl.LayerConfig("decode1_bf16", "bf16", T=1, H=256, E=64, top_k=6, I=128),
    wl.LayerConfig("wide_bf16", "bf16", T=96, H=384, E=256, top_k=8, I=64),
    wl.LayerConfig("big_groups_bf16", "bf16", T=1100, H=512, E=2, top_k=1, I=320),
    wl.LayerConfig("ragged_f32", "f32", T=77, H=136, E=5, top_k=3, I=40, fan_in_init=True),
]
LAYOUTS = [B.MOE_W_KN, B.MOE_W_NK]
LAYOUT_IDS = ["kn", "nk"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _routes(cfg, seed=21):
    """Seeded fed-in routes: a fat group, an empty expert, tokens whose slots repeat an expert."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, cfg.E, (cfg.T, cfg.top_k)).astype(np.int32)
    ids[: min(cfg.T, 5)] = 0
    if cfg.E > 3:
        ids[ids == 2] = 1
    if cfg.top_k > 1 and cfg.T > 8:
        ids[6:9, :] = ids[6:9, :1]
    w = rng.uniform(0.05, 1.0, (cfg.T, cfg.top_k)).astype(np.float32)
    return ids, w


def _dy(cfg, seed=22):
    return np.random.default_rng(seed).standard_normal((cfg.T, cfg.H)).astype(np.float32)


def _to_kn(w, layout):
    """Per-expert weight (or weight gradient) as [K, N] for comparison."""
    return w if layout == B.MOE_W_KN else np.swapaxes(w, -1, -2)


def _run(cfg, layout, ids, w, dy):
    print(f"[case] {cfg.name} layout={layout}", flush=True)
    layer = wl.make_layer(cfg, DEV)
    x = layer["x"]
    W1d, W2d = layer["W1"], layer["W2"]
    if layout == B.MOE_W_NK:
        W1d, W2d = W1d.transpose(-1, -2).contiguous(), W2d.transpose(-1, -2).contiguous()
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, 0, x.dtype, DEV)
    bwd = B.MoEBackwardBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, x.dtype, DEV, layout)
    for t in (bufs.act, bufs.y_rows, bwd.h_pre, bwd.d_rows, bwd.d_h, bwd.d_x, bwd.d_w1, bwd.d_w2,
              bwd.d_topk_weights):
        t.fill_(float("nan"))
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    B.moe_routed_train_forward(x, W1d, W2d, (ids_d, w_d), bufs, bwd, layout=layout)
    B.moe_routed_backward(torch.from_numpy(dy).to(DEV), W1d, W2d, w_d, bufs, bwd, layout=layout)
    torch.cuda.synchronize()
    W1 = host(layer["W1"])
    W2 = host(layer["W2"])
    return layer, bufs, bwd, [W1[e] for e in range(cfg.E)], [W2[e] for e in range(cfg.E)]


def _check(cfg, layout, bufs, bwd, ref):
    dt = cfg.dtype
    valid = ref["row_token"] >= 0
    assert np.array_equal(host(bufs.scatter_index), ref["scatter_index"])
    # the training forward's pre-activation: one bf16 rounding step at most apart
    hp = host(bwd.h_pre)[valid]
    hp_ref = ref["H_pre"][valid]
    tol = np.abs(hp_ref) * (2.0 ** -7 if dt == "bf16" else 1e-5) + 1e-4
    assert (np.abs(hp - hp_ref) <= tol).all(), "h_pre"
    assert_grad_close(host(bwd.d_topk_weights), ref["dweights"], dt, "d_topk_weights")
    assert_grad_close(host(bwd.d_rows)[valid], ref["dYs"][valid], dt, "d_rows")
    assert_grad_close(host(bwd.d_h)[valid], ref["dH"][valid], dt, "d_h")
    assert_grad_close(_to_kn(host(bwd.d_w2), layout), ref["dW2"], dt, "d_w2")
    assert_grad_close(_to_kn(host(bwd.d_w1), layout), ref["dW1"], dt, "d_w1")
    assert_grad_close(host(bwd.d_x), ref["dx"], dt, "d_x")


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_parity(cfg, layout):
    ids, w = _routes(cfg)
    dy = _dy(cfg)
    layer, bufs, bwd, W1, W2 = _run(cfg, layout, ids, w, dy)
    ref = O.moe_backward(host(layer["x"]), W1, W2, (ids, w), dy, contract=cfg.dtype == "bf16")
    _check(cfg, layout, bufs, bwd, ref)
    if cfg.E > 3:   # the empty expert's weight gradients are written, as zeros
        assert not host(bwd.d_w1)[2].any() and not host(bwd.d_w2)[2].any()


@pytest.mark.parametrize("layout", LAYOUTS, ids=LAYOUT_IDS)
@pytest.mark.parametrize("cfg", [wl.TINY_DUP, wl.LayerConfig("dup_bf16", "bf16", T=128, H=256, E=4, top_k=2,
                                                                 I=128, routes="all_dup")], ids=lambda c: c.name)
def test_backward_all_duplicate_routes(cfg, layout):
    """[VEOMNI] "Regression test pattern": selected_experts = zeros([tokens, topk]),
    routing_weights = full([tokens, topk], weight).  Expert 0 holds 256 rows for
    128 tokens; every row's gradient is computed (a bound of `tokens` rows would
    leave rows 128..255 stale), all gradients are finite, and they match the
    oracle's merged-fc1 and split-fc1 backward."""
    ids, w = wl.all_duplicate_routes(cfg)
    dy = _dy(cfg)
    layer, bufs, bwd, W1, W2 = _run(cfg, layout, ids, w, dy)
    assert host(bufs.expert_offsets).tolist()[:2] == [0, 2 * cfg.T]
    for name in ("h_pre", "d_rows", "d_h", "d_x", "d_w1", "d_w2", "d_topk_weights"):
        assert torch.isfinite(getattr(bwd, name).float()).all(), name
    x = host(layer["x"])
    contract = cfg.dtype == "bf16"
    merged = O.moe_backward(x, W1, W2, (ids, w), dy, contract=contract)
    split = O.moe_backward(x, W1, W2, (ids, w), dy, contract=contract, split_fc1=True)
    _check(cfg, layout, bufs, bwd, merged)
    _check(cfg, layout, bufs, bwd, split)
    # both slots of a token see the same expert output
    dw = host(bwd.d_topk_weights)
    assert np.array_equal(dw[:, 0], dw[:, 1])


def test_fc1_backward_accumulates_into_d_x():
    cfg = wl.LayerConfig("acc_bf16", "bf16", T=64, H=256, E=4, top_k=2, I=128)
    ids, w = _routes(cfg)
    dy = _dy(cfg)
    layer, bufs, bwd, W1, W2 = _run(cfg, B.MOE_W_KN, ids, w, dy)
    first = host(bwd.d_x).copy()
    B.moe_grouped_fc1_backward(bwd.d_h, bufs.x_scattered, bufs.expert_offsets, layer["W1"], bufs.scatter_index,
                               bwd.d_x, bwd.d_w1, bwd.ws, accumulate=True)
    torch.cuda.synchronize()
    # the slots are added onto the existing d_x one at a time: (d_x + r0) + r1, not bitwise 2 d_x
    np.testing.assert_allclose(host(bwd.d_x), first + first, rtol=1e-5, atol=1e-6)
