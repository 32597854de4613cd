"""Benchmark: forward pass of one MoE FFN layer through libmoe on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3]
                    [--launch auto|eager|graph] [--no-evict] [--no-cpu-baseline]
                    [--cpu-sample TOKENS]

One step = the whole layer through libmoe (routing and scatter build in one
call, with no copy of the routed rows: fc1 gathers them from x on load;
grouped fc1 + SwiGLU with the shared expert's fc1 in the same launch,
grouped fc2 with the shared expert's fc2 and gate in the same launch,
gather/combine) over one batch of synthetic input already resident in HBM.
The default workload is the DeepSeek-V3-shaped prefill (T=4096, H=7168,
E=256, top-8, I=2048, one shared expert), the largest layer that fits one GPU.

Timing: W untimed warm-up steps, then exactly K steps (default 50 for prefill,
200 for decode shapes) between two stream synchronisations.  Before every
timed step, outside its events, an ordinary reduction kernel reads 1 GiB so
the 256 MiB last-level cache holds none of the step's inputs (--no-evict skips
this).  HIP events on the launch stream bracket each step and each call; the
line reports the median step time (value = T / median) with p10/p90, and the
mean duration of the dominant call (the fc1 launch) for the roofline object.
Decode shapes (T <= 64) replay a HIP graph of the step by default (--launch
auto); their per-call times come from an eager pass with the same eviction.
A warm-cache figure (the same steps back to back, nothing evicted) is
reported separately and labelled.

The CPU baseline runs the NumPy oracle (float32, bf16 contract mode) on a
bounded sample of the same workload (the first --cpu-sample tokens) on the
host cores, after the GPU timing.  Parity, checked in the same run: routing
of all T tokens certified against the oracle's logits; the GPU layer run
again with the oracle's routes fed in and compared with the oracle on the
sample; the timed run's own output compared on the sampled tokens whose
routes agree.  A parity failure makes the run exit non-zero.

With --backward, one step is instead the backward of the routed experts for the
routes a forward pass realized (moe_scatter_grad, moe_grouped_fc2_backward,
moe_grouped_fc1_backward), with the forward's saved tensors resident; the
roofline object covers the moe_grouped_fc1_backward call.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from mixture_experts_ffn_05_amd import binding as B  # noqa: E402
from mixture_experts_ffn_05_amd import workloads as wl  # noqa: E402

METRIC = "MoE-layer tokens/s and grouped-GEMM TFLOP/s (% bf16 MFMA peak; decode % HBM BW)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
CALLS = ("route_scatter", "fc1", "fc2", "combine")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(cfg, counts, shared_in_gemms=True, weight_bytes=None):
    """FLOPs and bytes the layer must do for the realized routes (counts per expert).
    fc1/fc2 figures cover what the timed fc1/fc2 launches carry: the routed
    groups and, with shared_in_gemms and a shared expert, the shared expert.
    weight_bytes: bytes per expert-weight element (MXFP8: 1 + 1/8); activations
    keep the workload's element size."""
    T, H, E, k, I, I_s = cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s
    R = int(counts.sum())
    active = int((counts > 0).sum())
    el = 2 if cfg.dtype == "bf16" else 4
    wel = weight_bytes if weight_bytes is not None else el
    S = I_s if shared_in_gemms else 0
    fc1_flops = 4.0 * R * H * I + 4.0 * T * H * S
    fc2_flops = 2.0 * R * I * H + 2.0 * T * S * H
    fc1_bytes = (active * H * 2 * I * wel + R * H * el + R * I * el         # routed weights + X_s read + A write
                 + (H * 2 * S * wel + T * H * el + T * S * el if S else 0))
    fc2_bytes = (active * I * H * wel + R * I * el + R * H * 4              # routed weights + A read + Y_s write
                 + (S * H * wel + T * S * el + T * H * 4 if S else 0))
    shared_flops = 6.0 * T * H * I_s + (2.0 * T * H if cfg.gated else 0.0)
    layer_flops = 2.0 * T * H * E + 4.0 * R * H * I + 2.0 * R * I * H + shared_flops
    layer_bytes = (active * 3 * H * I * wel + 3 * H * I_s * wel + H * E * el + T * H * el + T * H * 4)
    return {"R": R, "active_experts": active, "fc1_flops": fc1_flops, "fc2_flops": fc2_flops,
            "fc1_bytes": fc1_bytes, "fc2_bytes": fc2_bytes, "shared_flops": shared_flops,
            "layer_flops": layer_flops, "layer_bytes": layer_bytes}


def roofline(flops, nbytes, seconds):
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if flops / nbytes >= ridge:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBPS, 4)}


def committed_traffic(workload, backward=False):
    """Calibrated HBM bytes of one timed call from the committed rocprofv3 counter
    summary (profiles/hbm_counters_<workload>[_backward]_pmc.md), or None if
    absent or taken on a different kernel source."""
    import re
    from mixture_experts_ffn_05_amd import prof_summary
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}{'_backward' if backward else ''}_pmc.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^TRAFFIC_JSON (.*)$", open(path).read(), re.M)
    rec = json.loads(m.group(1)) if m else None
    if rec and rec.get("gemm_source_hash") == prof_summary.kernel_source_hash():
        return rec
    return None


def committed_trace(workload, backward=False):
    """Average duration (us) of the timed call's kernels from the committed rocprofv3
    kernel-trace summary (profiles/kernel_trace_<workload>[_backward].md), or None if
    absent or taken on a different kernel source."""
    import re
    from mixture_experts_ffn_05_amd import prof_summary
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}{'_backward' if backward else ''}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^TRACE_JSON (.*)$", open(path).read(), re.M)
    rec = json.loads(m.group(1)) if m else None
    if rec and rec.get("gemm_source_hash") == prof_summary.kernel_source_hash():
        return rec
    return None


def add_profile_fraction(roof, rec):
    """The roofline fraction recomputed from the committed kernel trace's average
    duration of the same call, next to the live event-based one."""
    if rec is None:
        roof["profile_avg_us"] = roof["frac_profile"] = None
        return
    us = rec["avg_us_per_call"]
    roof["profile_avg_us"] = round(us, 2)
    work = roof["algorithmic_bytes"] if roof["bound"] == "hbm" else roof["algorithmic_flops"]
    scale = 1e9 if roof["bound"] == "hbm" else 1e12
    roof["frac_profile"] = round(work / (us * 1e-6) / scale / roof["peak"], 4)


class Evictor:
    """Reads 1 GiB with an ordinary reduction kernel (torch's sum), so the 256 MiB
    last-level cache (and every L2) holds none of the next step's inputs, only
    clean lines of this buffer: an eviction that wrote its buffer would leave
    dirty lines whose write-back then competes with the step's reads.  Enqueued
    outside the timed events and outside any captured graph."""

    def __init__(self, dev, enabled=True):
        # float32, so the sum reads the buffer in place (an integer sum would first widen it to a new buffer)
        self.buf = torch.ones((1 << 28,), dtype=torch.float32, device=dev) if enabled else None
        self.sink = None

    def __call__(self):
        if self.buf is not None:
            self.sink = self.buf.sum()


def step_stats(ms):
    ms = np.asarray(ms, np.float64)
    return {"median_ms": round(float(np.median(ms)), 5), "p10_ms": round(float(np.percentile(ms, 10)), 5),
            "p90_ms": round(float(np.percentile(ms, 90)), 5), "mean_ms": round(float(ms.mean()), 5),
            "min_ms": round(float(ms.min()), 5), "max_ms": round(float(ms.max()), 5), "n": int(ms.size)}


def host_info():
    """CPU model, CPUs this process may run on, BLAS library, and the thread count
    the CPU baseline uses (the CPUs in the affinity mask, capped by OMP_NUM_THREADS
    when the environment sets it)."""
    import threadpoolctl
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else affinity
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpoolctl.threadpool_info()
            if i.get("user_api") == "blas"]
    return {"cpu_model": model, "affinity_cpus": affinity, "threads": threads,
            "blas": ", ".join(blas) or "unknown"}


def route_and_scatter(layer, bufs, cfg, bias_t, routes=None, copy_rows=False):
    """Step 1-2: routing and the scatter build, or, with `routes` = (ids, weights)
    device tensors, the scatter build of those fed-in routes."""
    x = layer["x"]
    if routes is None:
        B.moe_route_and_scatter(x, layer["w_router"], bias_t, cfg.top_k, bufs.topk_ids, bufs.topk_weights,
                                bufs.logits, bufs.scatter_index, bufs.row_token, bufs.expert_offsets,
                                bufs.status_words, bufs.x_scattered if copy_rows else None, bufs.route_scatter_ws)
    else:
        bufs.topk_ids.copy_(routes[0])
        bufs.topk_weights.copy_(routes[1])
        B.moe_build_scatter(x, bufs.topk_ids, cfg.E, bufs.scatter_index, bufs.row_token, bufs.expert_offsets,
                            bufs.status_words, bufs.x_scattered if copy_rows else None, bufs.scatter_ws)


def run_step(layer, bufs, cfg, bias_t, events=None, side=None, routes=None):
    """One layer forward: route + scatter, fc1 (+ shared fc1), fc2 (+ shared fc2, gate), combine.
    With `routes` ((ids, weights) device tensors) the routes are fed in and only
    the scatter build runs in the first call.
    With `side` (a second stream) and a shared expert, the shared expert runs on
    `side` (y = shared(x)) while routing and the routed experts run on the
    current stream, which waits for it before the combine adds onto y.
    With `events`, records one HIP event before each call on the current stream
    and one after the last."""
    lay = layer["layout"]
    x, W1, W2 = layer["x"], layer["W1"], layer["W2"]
    rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
    shared = layer["shared"]
    mx = layer.get("mx")
    if mx is not None:  # MXFP8 expert weights: routed and shared experts together, then the combine
        rec(0)
        route_and_scatter(layer, bufs, cfg, bias_t, routes, copy_rows=True)
        rec(1)
        if mx["shared"] is not None:
            q1, s1, q2, s2, wg = mx["shared"]
            B.moe_grouped_swiglu_fc1_and_shared_mx8(bufs.x_scattered, bufs.expert_offsets, mx["W1q"], mx["W1s"],
                                                    bufs.act, x, q1, s1, bufs.act_shared)
            rec(2)
            B.moe_grouped_fc2_and_shared_mx8(bufs.act, bufs.expert_offsets, mx["W2q"], mx["W2s"], bufs.y_rows,
                                             bufs.act_shared, q2, s2, x, wg, bufs.y, bufs.shared_ws,
                                             accumulate=False)
        else:
            B.moe_grouped_swiglu_fc1_mx8(bufs.x_scattered, bufs.expert_offsets, mx["W1q"], mx["W1s"], bufs.act)
            rec(2)
            B.moe_grouped_fc2_mx8(bufs.act, bufs.expert_offsets, mx["W2q"], mx["W2s"], bufs.y_rows)
        rec(3)
        B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y,
                             mx["shared"] is not None)
        rec(4)
        return
    if side is not None and shared is not None:
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        ws1, ws2, wg = shared
        B.moe_shared_expert(x, ws1, ws2, wg, bufs.y, bufs.shared_ws, False, stream=side, layout=lay)
        rec(0)
        route_and_scatter(layer, bufs, cfg, bias_t, routes, copy_rows=True)
        rec(1)
        B.moe_grouped_swiglu_fc1(bufs.x_scattered, bufs.expert_offsets, W1, bufs.act, layout=lay)
        rec(2)
        B.moe_grouped_fc2(bufs.act, bufs.expert_offsets, W2, bufs.y_rows, layout=lay)
        rec(3)
        main.wait_stream(side)
        B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y, True)
        rec(4)
        return
    gather = layer.get("gather", False)   # fc1 reads the routed rows from x through row_token
    rec(0)
    route_and_scatter(layer, bufs, cfg, bias_t, routes, copy_rows=not gather)
    rec(1)
    if shared is not None:
        ws1, ws2, wg = shared
        if gather:
            B.moe_grouped_swiglu_fc1_and_shared_gather(x, bufs.row_token, bufs.expert_offsets, W1, bufs.act, ws1,
                                                       bufs.act_shared, layout=lay)
        else:
            B.moe_grouped_swiglu_fc1_and_shared(bufs.x_scattered, bufs.expert_offsets, W1, bufs.act, x, ws1,
                                                bufs.act_shared, layout=lay)
        rec(2)
        B.moe_grouped_fc2_and_shared(bufs.act, bufs.expert_offsets, W2, bufs.y_rows, bufs.act_shared, ws2, x, wg,
                                     bufs.y, bufs.shared_ws, False, layout=lay)
        rec(3)
        B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y, True)
    else:
        if gather:
            B.moe_grouped_swiglu_fc1_gather(x, bufs.row_token, bufs.expert_offsets, W1, bufs.act, layout=lay)
        else:
            B.moe_grouped_swiglu_fc1(bufs.x_scattered, bufs.expert_offsets, W1, bufs.act, layout=lay)
        rec(2)
        B.moe_grouped_fc2(bufs.act, bufs.expert_offsets, W2, bufs.y_rows, layout=lay)
        rec(3)
        B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y, False)
    rec(4)


class HostExperts:
    """Expert weights as the K x N float32 host matrices the oracle takes (x @ W),
    copied from the device one expert at a time when the oracle first asks for it.
    Nothing is cached, so host memory holds about one expert; the time spent
    moving and upcasting weights is kept in `copy_s`, apart from the oracle's own
    time.  With MXFP8 codes the oracle's exact dequantization runs on access (its
    own arithmetic, so it is not counted in `copy_s`)."""

    def __init__(self, w=None, layout=None, q=None, sc=None, axis=None, name="W"):
        self.w, self.layout, self.q, self.sc, self.axis, self.name = w, layout, q, sc, axis, name
        self.copy_s = 0.0
        self.fetched = 0

    def __len__(self):
        return (self.w if self.w is not None else self.q).shape[0]

    def __getitem__(self, e):
        from oracle import moe_oracle as O
        self.fetched += 1
        if self.fetched % 64 == 0:
            log(f"cpu baseline: {self.name} of {self.fetched} experts fetched so far")
        t0 = time.perf_counter()
        if self.q is not None:
            q, sc = self.q[e].cpu().numpy(), self.sc[e].cpu().numpy()
            self.copy_s += time.perf_counter() - t0
            return np.ascontiguousarray(O.mx_dequant(q, sc, axis=self.axis).T.astype(np.float32))
        a = self.w[e].cpu().float().numpy()
        if self.layout == B.MOE_W_NK:
            a = np.ascontiguousarray(a.T)
        self.copy_s += time.perf_counter() - t0
        return a


def _host(t):
    return t.detach().cpu().float().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def cpu_baseline(layer, cfg, sample_tokens, info):
    """Time the oracle (the whole layer, routing included) on the first
    `sample_tokens` tokens on the host cores; returns (record, oracle output)."""
    import threadpoolctl
    from oracle import moe_oracle as O

    S = min(sample_tokens, cfg.T)
    contract = cfg.dtype == "bf16"
    nk = layer["layout"] == B.MOE_W_NK
    x = _host(layer["x"][:S])
    wr = _host(layer["w_router"])
    mx = layer.get("mx")
    if mx is not None:
        W1 = HostExperts(q=mx["W1q"], sc=mx["W1s"], axis=0, name="W1")
        W2 = HostExperts(q=mx["W2q"], sc=mx["W2s"], axis=1, name="W2")
        shared = None
        if mx["shared"] is not None:
            q1, s1, q2, s2, wg = mx["shared"]
            u = lambda t: t.cpu().numpy()
            shared = (np.ascontiguousarray(O.mx_dequant(u(q1), u(s1), axis=0).T.astype(np.float32)),
                      np.ascontiguousarray(O.mx_dequant(u(q2), u(s2), axis=1).T.astype(np.float32)),
                      _host(wg) if wg is not None else None)
    else:
        W1 = HostExperts(layer["W1"], layer["layout"], name="W1")
        W2 = HostExperts(layer["W2"], layer["layout"], name="W2")
        shared = None
        if layer["shared"] is not None:
            ws1, ws2, wg = layer["shared"]
            fw = (lambda t: np.ascontiguousarray(_host(t).T)) if nk else _host
            shared = (fw(ws1), fw(ws2), _host(wg) if wg is not None else None)
    threads = info["threads"]
    log(f"cpu baseline: oracle over {S} of {cfg.T} tokens, {threads} BLAS threads ({info['blas']}), "
        f"{info['cpu_model']}")
    runs, walls = [], []
    with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
        while True:  # up to 3 runs within about 20 s of wall time; the median is reported
            c0 = W1.copy_s + W2.copy_s
            t0 = time.perf_counter()
            ref = O.moe_forward(x, wr, W1, W2, cfg.top_k, bias=layer["bias"], shared=shared, contract=contract,
                                dtype=np.float32)
            wall = time.perf_counter() - t0
            walls.append(wall)
            runs.append(wall - (W1.copy_s + W2.copy_s - c0))
            if len(runs) >= 3 or sum(walls) >= 20.0:
                break
    dt = float(np.median(runs))
    log(f"cpu baseline: {len(runs)} runs, median {dt:.2f} s of oracle time "
        f"(+ {W1.copy_s + W2.copy_s:.1f} s moving weights to the host, not counted)")
    base = {"value": round(S / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"first {S} of {cfg.T} tokens of the {cfg.name} workload, whole layer (routing, scatter, "
                       f"routed experts, combine, shared expert), NumPy float32"
                       f"{' with bf16 activation rounding' if contract else ''}; median of {len(runs)} runs "
                       f"({', '.join(f'{r:.2f}' for r in runs)} s); expert weights are fetched from the device "
                       f"one expert at a time and that transfer is not counted"),
            "cpu_model": info["cpu_model"], "affinity_cpus": info["affinity_cpus"], "blas": info["blas"]}
    return base, ref


def parity_check(layer, cfg, bufs, bias_t, dev, side, ref, S):
    """Parity of the run just timed, against the oracle:
    * routing of all T tokens: GPU logits within the oracle's certified float32
      bound, top-k bit-exact on the GPU's own logits, weights within 1e-6; tokens
      whose oracle routes differ (certified near ties) at most 1% of T;
    * the whole GPU layer run again with the oracle's routes fed in: scatter
      structures bit-exact, every routed row and output finite, y on the first S
      tokens within the tolerance of the oracle's y;
    * the timed run's own y on the first S tokens whose routes agree with the
      oracle's, within the same tolerance (and at least one token compared)."""
    from oracle import moe_oracle as O

    tol = {"max_abs": 2e-2, "rel_fro": 1e-2} if cfg.dtype == "bf16" else {"max_abs": 1e-4, "rel_fro": 1e-4}
    T, k, E = cfg.T, cfg.top_k, cfg.E
    xh, wrh = _host(layer["x"]), _host(layer["w_router"])
    L_o = O.router_logits(xh, wrh, layer["bias"])
    bound = O.router_logit_bound(xh, wrh, layer["bias"])
    Lg = bufs.logits.cpu().numpy()
    ids_g, w_g = bufs.topk_ids.cpu().numpy(), bufs.topk_weights.cpu().numpy()
    ids_o = O.topk_select(L_o, k)
    w_o = O.route_weights(L_o, ids_o)
    near_tie = (ids_o != ids_g).any(1)
    routing = {"tokens": T,
               "logits_within_certified_bound": bool((np.abs(Lg.astype(np.float64) - L_o) <= bound).all()),
               "topk_bit_exact_on_gpu_logits": bool(np.array_equal(ids_g, O.topk_select(Lg, k))),
               "weights_max_abs_err": float(np.abs(w_g - O.route_weights(Lg, ids_g)).max()),
               "near_tie_tokens": int(near_tie.sum())}
    routing_ok = (routing["logits_within_certified_bound"] and routing["topk_bit_exact_on_gpu_logits"]
                  and routing["weights_max_abs_err"] <= 1e-6 and near_tie.mean() <= 0.01)

    def err(a, b):
        d = a.astype(np.float64) - b
        return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(b), 1e-30))

    # the GPU layer with the oracle's routes fed in
    fb = B.MoELayerBuffers(T, cfg.H, E, k, cfg.I, cfg.I_s, layer["x"].dtype, dev)
    fb.y_rows.fill_(float("nan"))
    fb.y.fill_(float("nan"))
    run_step(layer, fb, cfg, bias_t, side=side,
             routes=(torch.from_numpy(ids_o).to(dev), torch.from_numpy(w_o).to(dev)))
    torch.cuda.synchronize()
    sc = O.build_scatter(ids_o, E)
    R = T * k
    scatter_ok = (np.array_equal(fb.scatter_index.cpu().numpy(), sc["scatter_index"])
                  and np.array_equal(fb.row_token.cpu().numpy(), sc["row_token"])
                  and np.array_equal(fb.expert_offsets.cpu().numpy(), sc["offsets"])
                  and fb.status_words.cpu().tolist() == [sc["max_group"], 0])
    fed_finite = bool(torch.isfinite(fb.y_rows[:R]).all().item() and torch.isfinite(fb.y).all().item())
    same_o = (ref["ids"] == ids_o[:S]).all(1)    # the oracle's routes of the sample, computed alone
    y_fed = fb.y[:S].cpu().numpy()[same_o]
    fmx, frel = err(y_fed, ref["y"][same_o]) if same_o.any() else (float("inf"), float("inf"))
    fed = {"tokens_compared": int(same_o.sum()), "max_abs_err": fmx, "rel_fro_err": frel,
           "scatter_bit_exact": bool(scatter_ok), "all_rows_finite": fed_finite}
    fed_ok = (scatter_ok and fed_finite and same_o.sum() > 0 and (~same_o).mean() <= 0.01 and fmx <= tol["max_abs"]
              and frel <= tol["rel_fro"])
    del fb

    # the timed run's own output
    own_finite = bool(torch.isfinite(bufs.y_rows[:R]).all().item() and torch.isfinite(bufs.y).all().item())
    same = (ids_g[:S] == ref["ids"]).all(1)
    omx, orel = err(bufs.y[:S].cpu().numpy()[same], ref["y"][same]) if same.any() else (float("inf"),) * 2
    own = {"tokens_compared": int(same.sum()), "tokens_excluded_near_tie": int((~same).sum()),
           "max_abs_err": omx, "rel_fro_err": orel, "all_rows_finite": own_finite}
    own_ok = own_finite and same.sum() > 0 and (~same).mean() <= 0.01 and omx <= tol["max_abs"] and \
        orel <= tol["rel_fro"]
    return {"routing": routing, "oracle_routes_fed": fed, "own_routes": own, "tolerance": tol,
            "pass": bool(routing_ok and fed_ok and own_ok)}


BWD_CALLS = ("scatter_grad", "fc2_backward", "fc1_backward")


def backward_work(cfg, counts):
    """FLOPs and algorithmic bytes of the three backward calls for the realized routes."""
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    R = int(counts.sum())
    active = int((counts > 0).sum())
    el = 2 if cfg.dtype == "bf16" else 4
    k = cfg.top_k
    scat_bytes = T * H * 4 + R * H * 4 + R * H * el + 3 * T * k * 4            # dy, y_rows, d_rows, index/weights
    fc2_flops = 4.0 * R * H * I                                                 # dgrad + wgrad
    fc2_bytes = (active * I * H * el + R * H * el + 2 * R * 2 * I * el          # W2, d_rows, h_pre, d_h (dgrad)
                 + R * I * el + R * H * el + E * I * H * el)                    # act, d_rows, d_w2 (wgrad)
    fc1_flops = 8.0 * R * H * I                                                 # dgrad + wgrad
    fc1_bytes = (active * H * 2 * I * el + R * 2 * I * el + R * H * 4           # W1, d_h, d_xs (dgrad)
                 + R * H * 4 + T * H * 4                                        # gather
                 + R * H * el + R * 2 * I * el + E * H * 2 * I * el)            # x_s, d_h, d_w1 (wgrad)
    return {"R": R, "active_experts": active, "scatter_bytes": scat_bytes, "fc2_flops": fc2_flops,
            "fc2_bytes": fc2_bytes, "fc1_flops": fc1_flops, "fc1_bytes": fc1_bytes,
            "flops": fc1_flops + fc2_flops, "bytes": scat_bytes + fc1_bytes + fc2_bytes}


def run_backward_step(layer, bufs, bwd, dy, events=None):
    lay = layer["layout"]
    rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)
    rec(0)
    B.moe_scatter_grad(dy, bufs.y_rows, bufs.topk_weights, bufs.scatter_index, bwd.d_rows, bwd.d_topk_weights)
    rec(1)
    B.moe_grouped_fc2_backward(bwd.d_rows, bufs.act, bwd.h_pre, bufs.expert_offsets, layer["W2"], bwd.d_h, bwd.d_w2,
                               layout=lay)
    rec(2)
    B.moe_grouped_fc1_backward(bwd.d_h, bufs.x_scattered, bufs.expert_offsets, layer["W1"], bufs.scatter_index,
                               bwd.d_x, bwd.d_w1, bwd.ws, False, layout=lay)
    rec(3)


def cpu_baseline_backward(layer, cfg, bufs, bwd, dy, sample_tokens, info):
    """Time the oracle's backward on the first `sample_tokens` tokens (their GPU
    routes) and check the GPU's d_x and route-weight gradients on them: both
    depend on a token's own rows only, so they are exact on a sample."""
    import threadpoolctl
    from oracle import moe_oracle as O

    S = min(sample_tokens, cfg.T)
    f = _host
    x = f(layer["x"][:S])
    W1 = HostExperts(layer["W1"], layer["layout"])
    W2 = HostExperts(layer["W2"], layer["layout"])
    ids = bufs.topk_ids[:S].cpu().numpy()
    w = bufs.topk_weights[:S].cpu().numpy()
    dys = f(dy[:S])
    threads = info["threads"]
    log(f"cpu baseline (backward): oracle over {S} tokens with {threads} BLAS threads ({info['blas']})")
    runs, walls = [], []
    with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
        while True:
            c0 = W1.copy_s + W2.copy_s
            t0 = time.perf_counter()
            ref = O.moe_backward(x, W1, W2, (ids, w), dys, contract=True, dtype=np.float32)
            wall = time.perf_counter() - t0
            walls.append(wall)
            runs.append(wall - (W1.copy_s + W2.copy_s - c0))
            if len(runs) >= 3 or sum(walls) >= 20.0:
                break
    dt = float(np.median(runs))
    log(f"cpu baseline (backward): {len(runs)} runs, median {dt:.2f} s")
    parity = {}
    ok = True
    for name, gpu, r in (("d_x", f(bwd.d_x[:S]), ref["dx"]), ("d_topk_weights", f(bwd.d_topk_weights[:S]),
                                                               ref["dweights"])):
        d = gpu.astype(np.float64) - r
        mx = float(np.abs(d).max() / max(np.abs(r).max(), 1e-30))
        rel = float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-30))
        parity[name] = {"max_err_over_max_ref": mx, "rel_fro_err": rel}
        ok = ok and np.isfinite(gpu).all() and mx <= 2e-2 and rel <= 1e-2
    parity["tokens_compared"] = S
    parity["pass"] = bool(ok)
    base = {"value": round(S / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of the {cfg.name} workload with their GPU routes: routed "
                      f"experts' training forward and backward (moe_backward, NumPy float32, bf16 storage "
                      f"rounding); median of {len(runs)} runs ({', '.join(f'{r:.2f}' for r in runs)} s); expert "
                      f"weights are fetched from the device one expert at a time and that transfer is not counted",
            "cpu_model": info["cpu_model"], "affinity_cpus": info["affinity_cpus"], "blas": info["blas"]}
    return base, parity


def backward_setup(cfg, layer, bias_t, dev):
    """State the timed backward steps start from: routes from the router, the
    routed experts' training forward (fc1 keeping h_pre), and a seeded output
    gradient dy = N(0, 1) / sqrt(H).  Returns (bufs, bwd, dy)."""
    lay = layer["layout"]
    x = layer["x"]
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, 0, x.dtype, dev)
    bwd = B.MoEBackwardBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, x.dtype, dev, lay)
    B.moe_route_and_scatter(x, layer["w_router"], bias_t, cfg.top_k, bufs.topk_ids, bufs.topk_weights, bufs.logits,
                            bufs.scatter_index, bufs.row_token, bufs.expert_offsets, bufs.status_words,
                            bufs.x_scattered, bufs.route_scatter_ws)
    B.moe_grouped_swiglu_fc1_save(bufs.x_scattered, bufs.expert_offsets, layer["W1"], bufs.act, bwd.h_pre,
                                  layout=lay)
    B.moe_grouped_fc2(bufs.act, bufs.expert_offsets, layer["W2"], bufs.y_rows, layout=lay)
    B.moe_gather_combine(bufs.y_rows, bufs.scatter_index, bufs.topk_weights, bufs.y, False)
    g = torch.Generator(device="cpu").manual_seed(1234)
    dy = (torch.randn((cfg.T, cfg.H), generator=g, dtype=torch.float32) / np.sqrt(cfg.H)).to(dev)
    return bufs, bwd, dy


def bench_backward(args, cfg, layer, bias_t, dev, evict, info):
    lay = layer["layout"]
    bufs, bwd, dy = backward_setup(cfg, layer, bias_t, dev)
    torch.cuda.synchronize()
    counts = np.diff(bufs.expert_offsets.cpu().numpy())
    steps = args.steps or 50
    for _ in range(args.warmup):
        run_backward_step(layer, bufs, bwd, dy)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(BWD_CALLS) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        evict()
        run_backward_step(layer, bufs, bwd, dy, ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [ev[s][0].elapsed_time(ev[s][len(BWD_CALLS)]) for s in range(steps)]
    stats = step_stats(step_ms)
    ms_per_step = stats["median_ms"]
    per_call = {c: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                for i, c in enumerate(BWD_CALLS)}
    log("per-call ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per_call.items()))
    work = backward_work(cfg, counts)
    roof = roofline(work["fc1_flops"], work["fc1_bytes"], per_call["fc1_backward"] / 1e3)
    roof["algorithmic_bytes"] = work["fc1_bytes"]
    roof["algorithmic_flops"] = work["fc1_flops"]
    tr = committed_traffic(cfg.name, backward=True) if lay == B.MOE_W_KN else None
    roof["traffic"] = round(tr["hbm_bytes_per_call"] / 1e9, 4) if tr else None
    roof["traffic_unit"] = "GB per fc1_backward call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    add_profile_fraction(roof, committed_trace(cfg.name, backward=True) if lay == B.MOE_W_KN else None)
    roof["kernel"] = ("fc1_backward call = grouped_gemm_bf16_pipe<StoreF32, ROLE 2> (input gradient) + "
                      "gather_combine_k + grouped_wgrad_bf16<ROLE 1> (weight gradient)")
    step_s = ms_per_step / 1e3
    t_roof = max(work["flops"] / (PEAK_BF16_TFLOPS * 1e12), work["bytes"] / (PEAK_HBM_GBPS * 1e9))
    result = {
        "metric": "MoE-layer backward (routed experts) tokens/s",
        "value": round(cfg.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normals; random-init weights of the layer shape; dy seeded normal / sqrt(H))",
        "timing": {"step": stats, "cache": "evicted" if evict.buf is not None else "warm",
                   "wall_ms_per_step": round(wall * 1e3 / steps, 4),
                   "note": "step = HIP events around the three calls; value uses the median; the wall time also "
                           "covers the 1 GiB eviction read before each step"},
        "config": {"workload": cfg.name, "pass": "backward of the routed experts (routes fixed)", "T": cfg.T,
                   "H": cfg.H, "E": cfg.E, "top_k": cfg.top_k, "I": cfg.I, "routing": cfg.skew or "natural",
                   "shared_expert": "not included", "realized_rows_per_expert": counts.tolist()},
        "roofline": roof,
        "step": {"flops": work["flops"], "bytes_alg": work["bytes"],
                 "tflops": round(work["flops"] / step_s / 1e12, 2),
                 "gbps_alg": round(work["bytes"] / step_s / 1e9, 1),
                 "frac_roofline": round(t_roof / step_s, 4), "roofline_ms": round(t_roof * 1e3, 4)},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "weight_layout": "[N, K] per expert (torch.nn.Linear)" if args.layout == "nk" else "[K, N] per expert",
        "cpu_baseline": None,
    }
    rc = 0
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_backward(layer, cfg, bufs, bwd, dy, args.cpu_sample or 512, info)
        result["cpu_baseline"] = base
        result["parity"] = parity
        if not parity["pass"]:
            log(f"PARITY FAILURE: {parity}")
            rc = 1
    print(json.dumps(result), flush=True)
    sys.exit(rc)


def library_reference(cfg, layer, counts, evict, dev, reps=20):
    """The same GEMM shapes through torch's bf16 bmm/matmul (the vendor GEMM library), as a reference for the
    grouped GEMMs: every active expert gets the mean group size (a uniform routing, no partial tiles), fc1 without
    the SwiGLU epilogue and fc2 with a bf16 output (libmoe's fc2 writes fp32).  Each call is timed after the same
    1 GiB eviction; median of `reps`."""
    active = np.flatnonzero(counts > 0)
    ea = len(active)
    m = max(1, int(round(cfg.R / max(ea, 1))))
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    sel = lambda w: w if ea == cfg.E else w[torch.from_numpy(active).to(dev)].contiguous()

    def timed(fn, flops, name, shape):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ms = float(np.median(ts))
        tf = flops / (ms / 1e3) / 1e12
        log(f"library reference {name} {shape}: {ms:.4f} ms, {tf:.1f} TFLOP/s ({tf / PEAK_BF16_TFLOPS:.1%} of peak)")
        return {"shape": shape, "ms": round(ms, 4), "tflops": round(tf, 1),
                "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}

    out = {"note": "torch bf16 bmm/matmul (hipBLASLt) on the layer's own [K, N] weights, every active expert with "
                   f"the mean group size {m} (uniform routing); fc1 without SwiGLU, bf16 outputs"}
    for name, w, K, N in (("routed_fc1", layer["W1"], cfg.H, 2 * cfg.I), ("routed_fc2", layer["W2"], cfg.I, cfg.H)):
        wb = sel(w)
        x = torch.randn((ea, m, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        y = torch.empty((ea, m, N), device=dev, dtype=torch.bfloat16)
        out[name] = timed(lambda: torch.bmm(x, wb, out=y), 2.0 * ea * m * K * N, name, [ea, m, K, N])
        del wb, x, y
    if layer["shared"] is not None:
        ws1, ws2, _ = layer["shared"]
        for name, w, K, N in (("shared_fc1", ws1, cfg.H, 2 * cfg.I_s), ("shared_fc2", ws2, cfg.I_s, cfg.H)):
            x = torch.randn((cfg.T, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            y = torch.empty((cfg.T, N), device=dev, dtype=torch.bfloat16)
            out[name] = timed(lambda: torch.matmul(x, w, out=y), 2.0 * cfg.T * K * N, name, [cfg.T, K, N])
            del x, y
    torch.cuda.empty_cache()
    return out


def default_cpu_sample(cfg, mxfp8=False):
    """Tokens in the CPU-baseline sample: all of a decode batch, at most 2048 of a
    prefill batch (about 1-15 s of oracle time on 16 host threads).  With MXFP8
    weights the oracle decodes every expert it touches in float64 (about 1 s per
    DeepSeek-V3-sized expert), so 256-expert layers sample 4 tokens (at most 32
    experts) and the others at most 256 tokens."""
    if mxfp8:
        return min(cfg.T, 4 if cfg.E >= 256 else 256)
    return cfg.T if cfg.T <= 64 else min(cfg.T, 2048)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50 for prefill shapes, 200 for decode shapes, T <= 64)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens in the CPU-baseline sample (default: all tokens of a decode batch, 2048 of a "
                         "prefill batch; 512 for --backward)")
    ap.add_argument("--launch", choices=("auto", "eager", "graph"), default="auto",
                    help="eager launches, or replays of a HIP graph of one step; auto = graph for decode shapes "
                         "(T <= 64), eager otherwise")
    ap.add_argument("--graph", action="store_true", help="same as --launch graph")
    ap.add_argument("--no-evict", action="store_true",
                    help="do not evict the last-level cache before each timed step (warm-cache figures)")
    ap.add_argument("--shared", choices=("fused", "overlap"), default="fused",
                    help="shared expert inside the routed fc1/fc2 launches (fused, the default: measured faster "
                         "on every workload) or on a second stream concurrent with routing (overlap)")
    ap.add_argument("--weights", choices=("bf16", "mxfp8"), default="bf16",
                    help="expert weight format: bf16, or MXFP8 (e4m3 codes, one e8m0 scale per 8 along the "
                         "intermediate axis, dequantized exactly in the kernels; activations stay bf16)")
    ap.add_argument("--layout", choices=("kn", "nk"), default="kn",
                    help="expert weight storage: kn = [K, N] per expert (the x @ W form, the default), "
                         "nk = [N, K] (torch.nn.Linear layout)")
    ap.add_argument("--rows", choices=("gather", "copy"), default="gather",
                    help="routed rows for fc1: gathered from x through row_token on load (default), or copied to "
                         "x_scattered by the scatter build (the MXFP8 and overlap paths always copy)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the routed experts (for the routes a forward realized) instead of "
                         "the forward")
    ap.add_argument("--library-reference", action="store_true",
                    help="also time the same GEMM shapes through torch's bf16 bmm/matmul (the vendor GEMM library) "
                         "at uniform group sizes, as a reference (bf16 weights in the [K, N] layout)")
    ap.add_argument("--copy-reference-mb", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libmoe has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load()
    dev = torch.device("cuda:0")
    cfg = wl.WORKLOADS[args.workload]
    decode = cfg.T <= 64
    launch = "graph" if args.graph else args.launch
    if launch == "auto":
        launch = "graph" if decode else "eager"
    steps = args.steps or (200 if decode else 50)
    info = host_info()
    log(f"workload {cfg}")
    layer = wl.make_layer(cfg, dev)
    layer["layout"] = B.MOE_W_NK if args.layout == "nk" else B.MOE_W_KN
    if args.weights == "mxfp8":
        if cfg.dtype != "bf16":
            print("--weights mxfp8 needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        layer["mx"] = wl.mx_layer_weights(layer)
        layer["W1"] = layer["W2"] = layer["shared"] = None   # only the MXFP8 copies stay on the device
        torch.cuda.empty_cache()
    elif args.layout == "nk":  # the same matrices, stored [N, K]
        t = lambda w: w.transpose(-1, -2).contiguous()
        for key in ("W1", "W2"):
            layer[key] = t(layer[key])
            torch.cuda.empty_cache()
        if layer["shared"] is not None:
            ws1, ws2, wg = layer["shared"]
            layer["shared"] = (t(ws1), t(ws2), wg)
    bias_t = torch.from_numpy(layer["bias"]).to(dev) if layer["bias"] is not None else None
    bufs = B.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.top_k, cfg.I, cfg.I_s, layer["x"].dtype, dev)
    evict = Evictor(dev, enabled=not args.no_evict)
    torch.cuda.synchronize()
    if args.copy_reference_mb > 0:
        n = args.copy_reference_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy reference: {n} bytes read and {n} bytes written by one device copy")
        del src, dst

    if args.backward:
        if args.weights != "bf16" or args.graph or args.launch == "graph":
            print("--backward runs with bf16 weights and eager launches", file=sys.stderr)
            sys.exit(2)
        bench_backward(args, cfg, layer, bias_t, dev, evict, info)

    mode = args.shared
    if not cfg.I_s:
        mode = "none"
    if args.weights == "mxfp8":
        mode = "mx"
    side = torch.cuda.Stream() if mode == "overlap" else None
    layer["gather"] = args.rows == "gather" and mode in ("fused", "none")
    for _ in range(args.warmup):
        run_step(layer, bufs, cfg, bias_t, side=side)
    torch.cuda.synchronize()
    status = bufs.status_words.cpu().tolist()
    if status[1] != 0:
        raise RuntimeError(f"router produced {status[1]} out-of-range expert ids")
    counts = np.diff(bufs.expert_offsets.cpu().numpy())

    mk = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ev = [mk(len(CALLS) + 1) for _ in range(steps)]
    if launch == "graph":
        # Per-call times come from an eager pass (same eviction); the timed steps replay a captured graph.
        torch.cuda.synchronize()
        for s in range(steps):
            evict()
            run_step(layer, bufs, cfg, bias_t, ev[s], side=side)
        torch.cuda.synchronize()
        capture_stream = torch.cuda.Stream()
        capture_stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(capture_stream):
            with torch.cuda.graph(graph, stream=capture_stream):
                run_step(layer, bufs, cfg, bias_t, side=side)
        torch.cuda.current_stream().wait_stream(capture_stream)
        for _ in range(args.warmup):
            graph.replay()
        step_fn = lambda e: (e[0].record(), graph.replay(), e[1].record())
    else:
        step_fn = lambda e: run_step(layer, bufs, cfg, bias_t, e, side=side)
    sev = [mk(2) for _ in range(steps)] if launch == "graph" else [(e[0], e[len(CALLS)]) for e in ev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        evict()
        step_fn(sev[s] if launch == "graph" else ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stats = step_stats([a.elapsed_time(b) for a, b in sev])
    # warm cache, labelled: the same steps back to back with nothing evicted
    wev = [mk(2) for _ in range(min(steps, 50))]
    for e in wev:
        if launch == "graph":
            e[0].record()
            graph.replay()
            e[1].record()
        else:
            e[0].record()
            run_step(layer, bufs, cfg, bias_t, side=side)
            e[1].record()
    torch.cuda.synchronize()
    warm = step_stats([a.elapsed_time(b) for a, b in wev])
    ms_per_step = stats["median_ms"]
    per_call = {c: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                for i, c in enumerate(CALLS)}
    log(f"step ms median {stats['median_ms']:.4f} p10 {stats['p10_ms']:.4f} p90 {stats['p90_ms']:.4f} "
        f"(warm {warm['median_ms']:.4f}); per-call ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per_call.items()))

    work = algorithmic_work(cfg, counts, shared_in_gemms=(mode in ("fused", "mx")),
                            weight_bytes=1.125 if args.weights == "mxfp8" else None)
    fc1_s = per_call["fc1"] / 1e3
    fc2_s = per_call["fc2"] / 1e3
    roof = roofline(work["fc1_flops"], work["fc1_bytes"], fc1_s)
    roof["algorithmic_bytes"] = work["fc1_bytes"]
    roof["algorithmic_flops"] = work["fc1_flops"]
    roof["avg_us"] = round(per_call["fc1"] * 1e3, 2)
    # the committed profiles were taken in the default configuration (fused shared expert, [K, N], gathered rows,
    # bf16 weights, eviction before every step)
    default_cfg = mode == "fused" and args.layout == "kn" and layer["gather"] and not args.no_evict
    tr = committed_traffic(cfg.name) if default_cfg else None
    roof["traffic"] = round(tr["hbm_bytes_per_call"] / 1e9, 4) if tr else None
    roof["traffic_unit"] = "GB per fc1 call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    add_profile_fraction(roof, committed_trace(cfg.name) if default_cfg else None)
    one_launch = bool(cfg.I_s) and B.moe_and_shared_launches(layer["x"].dtype, cfg.R, cfg.H, cfg.E, cfg.I, cfg.T,
                                                               cfg.I_s) == 1
    if mode == "fused" and one_launch:
        roof["kernel"] = ("fc1 call = one launch of grouped_gemm_bf16_fused<SwiGLU> (moe_grouped_swiglu_fc1_and_shared:"
                          " routed experts and shared expert together)")
    elif mode == "fused":
        roof["kernel"] = ("fc1 call = two launches of grouped_gemm_bf16_pipe<SwiGLU> (moe_grouped_swiglu_fc1_and_shared:"
                          " routed experts, then the shared expert)")
    elif mode == "mx":
        roof["kernel"] = ("fc1 call = one launch of grouped_gemm_mx8_fused<SwiGLU> (moe_grouped_swiglu_fc1_and_shared_mx8:"
                          " routed and shared experts, MXFP8 weights)")
    else:
        roof["kernel"] = "fc1 call = grouped_gemm_bf16_pipe<SwiGLU> (moe_grouped_swiglu_fc1: routed experts)"
    gg_s = fc1_s + fc2_s
    gg_tflops = (work["fc1_flops"] + work["fc2_flops"]) / gg_s / 1e12
    gg_gbps = (work["fc1_bytes"] + work["fc2_bytes"]) / gg_s / 1e9
    layer_s = ms_per_step / 1e3
    t_roof = max(work["layer_flops"] / (PEAK_BF16_TFLOPS * 1e12), work["layer_bytes"] / (PEAK_HBM_GBPS * 1e9))

    result = {
        "metric": METRIC,
        "value": round(cfg.T / layer_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normals; random-init weights of the layer shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "top_k": cfg.top_k, "I": cfg.I,
                   "I_s": cfg.I_s, "shared_gate": cfg.gated, "routing": cfg.skew or "natural",
                   "realized_rows_per_expert": counts.tolist()},
        "roofline": roof,
        "timing": {"launch": "hip graph replay" if launch == "graph" else "eager launches",
                   "cache": "evicted" if evict.buf is not None else "warm",
                   "step": stats, "warm_cache_step": warm,
                   "wall_ms_per_step": round(wall * 1e3 / steps, 4),
                   "note": ("value and ms_per_step use the median of the per-step HIP-event times; before every "
                            "timed step a reduction kernel reading 1 GiB (outside the events) evicts the 256 MiB "
                            "last-level cache, so the wall time per step also covers it; warm_cache_step repeats "
                            "the step back to back without eviction")},
        "grouped_gemm": {"tflops": round(gg_tflops, 2), "frac_mfma_peak": round(gg_tflops / PEAK_BF16_TFLOPS, 4),
                         "gbps": round(gg_gbps, 1), "frac_hbm_peak": round(gg_gbps / PEAK_HBM_GBPS, 4),
                         "fc1_ms": round(per_call["fc1"], 4), "fc2_ms": round(per_call["fc2"], 4),
                         "fc1_frac": roof["frac"],
                         "fc2": roofline(work["fc2_flops"], work["fc2_bytes"], fc2_s)},
        "layer": {"flops": work["layer_flops"], "bytes_alg": work["layer_bytes"],
                  "tflops": round(work["layer_flops"] / layer_s / 1e12, 2),
                  "gbps_alg": round(work["layer_bytes"] / layer_s / 1e9, 1),
                  "frac_roofline": round(t_roof / layer_s, 4), "roofline_ms": round(t_roof * 1e3, 4),
                  "active_experts": work["active_experts"]},
        "per_call_ms": {k: round(v, 4) for k, v in per_call.items()},
        "per_call_note": ("fc1/fc2 carry the shared expert too (see shared_expert)" if mode in ("fused", "mx")
                          else "fc1/fc2 are the routed experts only"),
        "weight_layout": "[N, K] per expert (torch.nn.Linear)" if args.layout == "nk" else "[K, N] per expert",
        "routed_rows": ("gathered from x through row_token by fc1" if layer["gather"]
                        else "copied to x_scattered by the scatter build"),
        "weights": ("MXFP8 (e4m3 + e8m0 per 8 along the intermediate axis), dequantized to bf16 in the kernels"
                    if args.weights == "mxfp8" else "bf16"),
        "shared_expert": {"mx": "inside the routed fc1/fc2 launches (MXFP8 *_and_shared_mx8 calls)",
                          "fused": "inside the routed fc1/fc2 launches",
                          "overlap": "moe_shared_expert on a second stream, concurrent with routing and the "
                                     "routed experts; the combine waits for it",
                          "none": "layer has no shared expert"}[mode],
        "cpu_baseline": None,
    }
    if args.library_reference:
        if args.weights != "bf16" or args.layout != "kn" or cfg.dtype != "bf16":
            print("--library-reference needs bf16 weights in the [K, N] layout", file=sys.stderr)
            sys.exit(2)
        result["library_reference"] = library_reference(cfg, layer, counts, evict, dev)
    rc = 0
    if not args.no_cpu_baseline:
        S = min(args.cpu_sample or default_cpu_sample(cfg, args.weights == "mxfp8"), cfg.T)
        base, ref = cpu_baseline(layer, cfg, S, info)
        result["cpu_baseline"] = base
        parity = parity_check(layer, cfg, bufs, bias_t, dev, side, ref, S)
        result["parity"] = parity
        if not parity["pass"]:
            log(f"PARITY FAILURE: {parity}")
            rc = 1
    print(json.dumps(result), flush=True)
    sys.exit(rc)


if __name__ == "__main__":
    main()
