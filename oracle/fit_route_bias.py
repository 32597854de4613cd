"""Fit the per-expert logit biases that skew routing for two workloads.

Writes mixture_experts_ffn_05_amd/route_bias.json.  Calls only the oracle
(router logits and top-k) on the seeded x and W_r draws of the workload module.

* scout_zipf (T=2048, E=16, top-1): target counts proportional to 1/rank
  (expert e has rank e+1), rounded by largest remainder to sum to T.  Fit by
  200 steps of b_e += 0.3 * (ln target_e - ln max(count_e, 1)).
* v3_top4 (T=4096, E=256, top-8): one bias beta on experts 0..3, found by
  bisection so those four experts take 25% of the T*k routes.

Run from the repository root:  python -m oracle.fit_route_bias
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from oracle.moe_oracle import router_logits, topk_select  # noqa: E402
from mixture_experts_ffn_05_amd import workloads as wl  # noqa: E402


def _counts(L0, bias, top_k, E):
    L = (L0 + bias[None, :].astype(np.float32)).astype(np.float32)
    ids = topk_select(L, top_k)
    return np.bincount(ids.reshape(-1), minlength=E)


def zipf_targets(T, E):
    raw = np.array([T / (e + 1) for e in range(E)])
    raw = raw / raw.sum() * T
    base = np.floor(raw).astype(np.int64)
    rem = raw - base
    for i in np.argsort(-rem, kind="stable")[: T - base.sum()]:
        base[i] += 1
    return base


def fit_scout():
    cfg = wl.SCOUT
    x = wl.make_x(cfg).float().numpy()
    wr = wl.make_router(cfg).float().numpy()
    L0 = router_logits(x, wr)
    target = zipf_targets(cfg.T, cfg.E)
    b = np.zeros(cfg.E, np.float64)
    for _ in range(200):
        c = _counts(L0, b.astype(np.float32), cfg.top_k, cfg.E)
        b += 0.3 * (np.log(target) - np.log(np.maximum(c, 1)))
    b32 = b.astype(np.float32)
    c = _counts(L0, b32, cfg.top_k, cfg.E)
    return {"bias": [float(v) for v in b32], "target_counts": target.tolist(),
            "oracle_counts": c.tolist(), "workload": cfg.name}


def fit_v3():
    cfg = wl.V3
    x = wl.make_x(cfg).float().numpy()
    wr = wl.make_router(cfg).float().numpy()
    L0 = router_logits(x, wr)
    R = cfg.T * cfg.top_k

    def share(beta):
        b = np.zeros(cfg.E, np.float32)
        b[:4] = beta
        c = _counts(L0, b, cfg.top_k, cfg.E)
        return c[:4].sum() / R, c

    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        s, _ = share(np.float32(mid))
        if s < 0.25:
            lo = mid
        else:
            hi = mid
    beta = np.float32(hi)
    s, c = share(beta)
    b = np.zeros(cfg.E, np.float32)
    b[:4] = beta
    return {"bias": [float(v) for v in b], "top4_share": float(s), "beta": float(beta),
            "oracle_counts": c.tolist(), "active_experts": int((c > 0).sum()),
            "workload": cfg.name}


def main():
    out = {"_note": "written by oracle/fit_route_bias.py; per-expert float32 logit biases",
           "scout_zipf": fit_scout(), "v3_top4": fit_v3()}
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "mixture_experts_ffn_05_amd", "route_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)
    print("scout counts", out["scout_zipf"]["oracle_counts"])
    print("v3 top4 share", out["v3_top4"]["top4_share"], "beta", out["v3_top4"]["beta"])


if __name__ == "__main__":
    main()
