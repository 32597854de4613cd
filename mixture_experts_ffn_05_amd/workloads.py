"""Seeded synthetic inputs for the MoE FFN layer workloads.

This module only draws and lays out input tensors.  It holds none of the
layer's arithmetic (no routing, no expert maths), so both the HIP path and the
CPU oracle can take their inputs from it.

Shapes follow the routing table of the PLENA pages (section "Group A --
C_SET_TOPK_REG": Llama-4 Scout 16/top-1, Qwen2-MoE 60/top-4, DeepSeek-V2-Lite
64/top-6, DeepSeek-V3 256/top-8) and the shared-expert table of section
"Group C -- shared experts" (DeepSeek: moe_inter x n_shared, ungated; Qwen2-MoE:
independent width, sigmoid gate; Llama-4: width equal to the routed one).

Recipe (all tensors row-major, contiguous):

* x [T, H] and the router weight W_r [H, E] are drawn on the host with NumPy
  PCG64 streams keyed by SeedSequence(seed, spawn_key=(tensor_id,)), so they
  are identical on every machine.  Decode workloads take the first T rows of
  the prefill draw.
* Expert weights W1 [E, H, 2I] (gate columns [0, I), up columns [I, 2I)),
  W2 [E, I, H], and the shared weights Ws1 [H, 2 I_s], Ws2 [I_s, H], w_gate [H]
  are drawn with torch's generator on the device where they will live, one
  generator per (tensor, expert) seeded from the same SeedSequence keys.  A
  parity check always hands the oracle host copies of exactly these tensors.
* Values are float32 normals times the stated standard deviation, then rounded
  to bfloat16 (round-to-nearest-even, by torch's conversion) for bf16 workloads.
* Skewed routing uses a per-expert float32 logit bias stored in
  route_bias.json next to this file.  That file is written by a script in the
  oracle directory which fits the bias on these same x and W_r draws.
* MXFP8 expert weights (e4m3 codes, one e8m0 scale per 8 consecutive elements
  along the intermediate axis; PLENA_Compiler PR #69, section "Group C -- shared
  experts") are made from the bf16 weights above by mx_quantize: per block, the
  scale is the smallest power of two that brings max |w| to at most 448 (the
  largest e4m3 value), so nothing saturates and the block maximum lands in
  (224, 448]; each value divided by its scale is rounded to e4m3 by torch's
  conversion.  This is input preparation only: the
  layer consumes the codes and scales as given, and both the HIP path and the
  oracle dequantize them.  They are stored [N, K] per weight (K contiguous):
  W1q [E, 2I, H] with scales [E, 2I/8, H] (blocks along the output axis), W2q
  [E, H, I] with scales [E, H, I/8] (blocks along the reduction axis), and the
  shared Ws1q [2 I_s, H] / [2 I_s/8, H], Ws2q [H, I_s] / [H, I_s/8].
"""

from __future__ import annotations

import json
import os
from dataclasses import dataclass, field, replace

import numpy as np
import torch

TENSOR_X, TENSOR_WR, TENSOR_W1, TENSOR_W2, TENSOR_WS1, TENSOR_WS2, TENSOR_WG = range(7)

_BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "route_bias.json")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    dtype: str            # "f32" or "bf16": dtype of x, weights and the activation
    T: int                # tokens
    H: int                # hidden size
    E: int                # routed experts
    top_k: int
    I: int                # routed expert intermediate size
    I_s: int = 0          # shared intermediate width (0 = no shared expert)
    gated: bool = False   # sigmoid gate on the shared branch
    std: float = 0.02     # weight std for bf16 workloads
    fan_in_init: bool = False  # std = 1/sqrt(fan_in) instead (tiny workload)
    skew: str | None = None    # key into route_bias.json, or None for natural routing
    routes: str | None = None  # "all_dup": every token to expert 0 in every slot
    T_draw: int = 0       # rows drawn for x (decode takes the first T of these)
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.top_k

    def at_tokens(self, T: int, suffix: str) -> "LayerConfig":
        return replace(self, name=f"{self.name}_{suffix}", T=T,
                       T_draw=self.T_draw or self.T)


TINY = LayerConfig("tiny", "f32", T=128, H=256, E=8, top_k=2, I=128, fan_in_init=True,
                   notes="fp32 correctness workload")
TINY_DUP = replace(TINY, name="tiny_dup", routes="all_dup",
                   notes="every token sends both slots to expert 0 (one 256-row group)")
SCOUT = LayerConfig("scout", "bf16", T=2048, H=5120, E=16, top_k=1, I=8192, I_s=8192,
                    skew="scout_zipf", notes="Llama-4-Scout-shaped, Zipf-skewed routing")
QWEN2 = LayerConfig("qwen2", "bf16", T=4096, H=2048, E=60, top_k=4, I=1408, I_s=5632,
                    gated=True, notes="Qwen2-MoE-shaped, sigmoid-gated shared expert")
V2L = LayerConfig("v2l", "bf16", T=8192, H=2048, E=64, top_k=6, I=1408, I_s=2816,
                  notes="DeepSeek-V2-Lite-shaped, 2 shared experts stored fused")
V3 = LayerConfig("v3", "bf16", T=4096, H=7168, E=256, top_k=8, I=2048, I_s=2048,
                 skew="v3_top4", notes="DeepSeek-V3-shaped, top-4 experts take 25% of routes")

WORKLOADS = {c.name: c for c in (TINY, TINY_DUP, SCOUT, QWEN2, V2L, V3)}
for _T in (1, 16, 64):
    WORKLOADS[f"v2l_decode{_T}"] = V2L.at_tokens(_T, f"decode{_T}")
WORKLOADS["v3_decode64"] = V3.at_tokens(64, "decode64")


def _seed_sequence(cfg: LayerConfig, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(cfg.seed, spawn_key=tuple(int(k) for k in key))


def _numpy_normal(cfg: LayerConfig, shape, std: float, *key: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(_seed_sequence(cfg, *key)))
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _torch_seed(cfg: LayerConfig, *key: int) -> int:
    return int(_seed_sequence(cfg, *key).generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def torch_dtype(cfg: LayerConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def weight_stds(cfg: LayerConfig) -> dict:
    if cfg.fan_in_init:
        return {"wr": cfg.H ** -0.5, "w1": cfg.H ** -0.5, "w2": cfg.I ** -0.5,
                "ws1": cfg.H ** -0.5, "ws2": max(cfg.I_s, 1) ** -0.5, "wg": cfg.H ** -0.5}
    s = cfg.std
    return {"wr": s, "w1": s, "w2": s, "ws1": s, "ws2": s, "wg": s}


def make_x(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    T_draw = cfg.T_draw or cfg.T
    xd = _numpy_normal(cfg, (T_draw, cfg.H), 1.0, TENSOR_X)[: cfg.T]
    return torch.from_numpy(np.ascontiguousarray(xd)).to(torch_dtype(cfg)).to(device)


def make_router(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    wr = _numpy_normal(cfg, (cfg.H, cfg.E), weight_stds(cfg)["wr"], TENSOR_WR)
    return torch.from_numpy(wr).to(torch_dtype(cfg)).to(device)


def _torch_normal(cfg: LayerConfig, shape, std: float, device, *key: int) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg, *key))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return v.mul_(std).to(torch_dtype(cfg))


def make_expert_weights(cfg: LayerConfig, device="cpu"):
    """(W1 [E, H, 2I], W2 [E, I, H]), generated one expert at a time."""
    std = weight_stds(cfg)
    dt = torch_dtype(cfg)
    W1 = torch.empty((cfg.E, cfg.H, 2 * cfg.I), dtype=dt, device=device)
    W2 = torch.empty((cfg.E, cfg.I, cfg.H), dtype=dt, device=device)
    for e in range(cfg.E):
        W1[e].copy_(_torch_normal(cfg, (cfg.H, 2 * cfg.I), std["w1"], device, TENSOR_W1, e))
        W2[e].copy_(_torch_normal(cfg, (cfg.I, cfg.H), std["w2"], device, TENSOR_W2, e))
    return W1, W2


def make_shared_weights(cfg: LayerConfig, device="cpu"):
    """(Ws1 [H, 2 I_s], Ws2 [I_s, H], w_gate [H] or None), or None without a shared expert."""
    if cfg.I_s <= 0:
        return None
    std = weight_stds(cfg)
    ws1 = _torch_normal(cfg, (cfg.H, 2 * cfg.I_s), std["ws1"], device, TENSOR_WS1)
    ws2 = _torch_normal(cfg, (cfg.I_s, cfg.H), std["ws2"], device, TENSOR_WS2)
    wg = _torch_normal(cfg, (cfg.H,), std["wg"], device, TENSOR_WG) if cfg.gated else None
    return ws1, ws2, wg


def load_route_bias(cfg: LayerConfig):
    """Per-expert float32 logit bias for skewed workloads (None for natural routing)."""
    if cfg.skew is None:
        return None
    with open(_BIAS_FILE) as f:
        data = json.load(f)
    entry = data[cfg.skew]
    b = np.asarray(entry["bias"], dtype=np.float32)
    if b.shape != (cfg.E,):
        raise ValueError(f"bias {cfg.skew} has shape {b.shape}, expected ({cfg.E},)")
    return b


def all_duplicate_routes(cfg: LayerConfig):
    """Fed-in routes for the duplicate pattern: every slot of every token names
    expert 0 with weight 1/top_k ([VEOMNI] "Fused MoE Kernel Notes", section
    "Duplicate top-k routes" and "Regression test pattern")."""
    ids = np.zeros((cfg.T, cfg.top_k), np.int32)
    w = np.full((cfg.T, cfg.top_k), 1.0 / cfg.top_k, np.float32)
    return ids, w


def mx_quantize(w: torch.Tensor, axis: int, block: int = 8):
    """(codes uint8, scales uint8) of w with one e8m0 scale per `block`
    consecutive elements along `axis` (see the module notes)."""
    axis = axis % w.dim()
    wf = w.float()
    shape = list(wf.shape)
    shape[axis:axis + 1] = [shape[axis] // block, block]
    blocks = wf.reshape(shape)
    amax = blocks.abs().amax(dim=axis + 1, keepdim=True)
    exp = torch.ceil(torch.log2(torch.where(amax > 0, amax, torch.full_like(amax, 448.0)) / 448.0))
    sbyte = (exp + 127).clamp(1, 254)
    scaled = (blocks / torch.exp2(sbyte - 127)).clamp(-448.0, 448.0)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(wf.shape)
    return codes.contiguous(), sbyte.squeeze(axis + 1).to(torch.uint8).contiguous()


def mx_layer_weights(layer: dict) -> dict:
    """MXFP8 codes and scales of a layer's expert and shared weights, stored [N, K]."""
    t = lambda w: w.transpose(-1, -2).contiguous()
    out = {}
    out["W1q"], out["W1s"] = mx_quantize(t(layer["W1"]), axis=-2)   # [E, 2I, H]; blocks along 2I
    out["W2q"], out["W2s"] = mx_quantize(t(layer["W2"]), axis=-1)   # [E, H, I]; blocks along I
    sh = layer.get("shared")
    if sh is not None:
        ws1q, ws1s = mx_quantize(t(sh[0]), axis=-2)                  # [2 I_s, H]
        ws2q, ws2s = mx_quantize(t(sh[1]), axis=-1)                  # [H, I_s]
        out["shared"] = (ws1q, ws1s, ws2q, ws2s, sh[2])
    else:
        out["shared"] = None
    return out


def make_layer(cfg: LayerConfig, device="cpu", with_experts: bool = True) -> dict:
    """All inputs of one layer: x, w_router, bias, W1, W2, shared."""
    layer = {"cfg": cfg, "x": make_x(cfg, device), "w_router": make_router(cfg, device),
             "bias": load_route_bias(cfg)}
    if with_experts:
        layer["W1"], layer["W2"] = make_expert_weights(cfg, device)
        layer["shared"] = make_shared_weights(cfg, device)
    return layer
