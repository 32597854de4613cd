"""Helpers shared by the GPU parity tests (comparison metrics and tolerances)."""

from __future__ import annotations

import numpy as np
import torch

# Output tolerances: bf16 workloads against the oracle in contract mode
# (the SwiGLU output rounded to bf16 where the kernels round it), float32
# workloads against the plain oracle.
TOL = {"bf16": {"max_abs": 2e-2, "rel_fro": 1e-2}, "f32": {"max_abs": 1e-4, "rel_fro": 1e-4}}


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float32 (or integer) host copy of a device tensor."""
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def err_metrics(y, ref) -> tuple[float, float]:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    d = y - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_output_close(y, ref, dtype: str, what: str = "y"):
    assert np.isfinite(y).all(), f"{what}: non-finite values"
    mx, rel = err_metrics(y, ref)
    tol = TOL[dtype]
    assert mx <= tol["max_abs"] and rel <= tol["rel_fro"], \
        f"{what}: max|err| {mx:.3e} (tol {tol['max_abs']}), rel_fro {rel:.3e} (tol {tol['rel_fro']})"
    return mx, rel


def check_routing(logits_gpu, ids_gpu, w_gpu, x, wr, bias, top_k, oracle):
    """Route parity: logits within the certified bound of the oracle's; top-k
    bit-exact against the oracle applied to the GPU's own logits; weights
    within 1e-6 of the oracle's softmax of those logits."""
    ref_logits = oracle.router_logits(x, wr, bias)
    bound = oracle.router_logit_bound(x, wr, bias)
    excess = np.abs(logits_gpu.astype(np.float64) - ref_logits) - bound
    assert excess.max() <= 0, f"logits outside the certified bound by {excess.max():.3e}"
    ids_ref = oracle.topk_select(logits_gpu, top_k)
    assert np.array_equal(ids_gpu, ids_ref), f"top-k differs on {int((ids_gpu != ids_ref).any(1).sum())} tokens"
    w_ref = oracle.route_weights(logits_gpu, ids_gpu)
    assert np.max(np.abs(w_gpu - w_ref)) <= 1e-6
    # how many tokens' routes would flip under the oracle's own logits (near ties)
    return int((oracle.topk_select(ref_logits, top_k) != ids_gpu).any(1).sum())


# Gradient tolerances: a gradient's scale follows the incoming gradient's, so
# the largest error is measured against the largest reference magnitude.  The
# bf16 bar is the forward's (2e-2 max, 1e-2 relative Frobenius); a stored bf16
# gradient alone carries up to 2^-9 relative rounding, and the bf16 h_pre, A,
# d_rows and d_h it is computed from each carry one more.
GRAD_TOL = {"bf16": {"max_rel": 2e-2, "rel_fro": 1e-2}, "f32": {"max_rel": 1e-4, "rel_fro": 1e-4}}


def assert_grad_close(g, ref, dtype: str, what: str):
    g = np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    d = np.abs(g - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    mx = float(d.max()) / scale
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    tol = GRAD_TOL[dtype]
    assert mx <= tol["max_rel"] and rel <= tol["rel_fro"], \
        f"{what}: max|err|/max|ref| {mx:.3e} (tol {tol['max_rel']}), rel_fro {rel:.3e} (tol {tol['rel_fro']})"
    return mx, rel
