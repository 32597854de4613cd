"""Plain CPU oracle for the forward pass of one MoE FFN layer, and for the
backward of its routed experts (NumPy).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU-baseline
leg of the benchmark.  It shares no code with the HIP library and never imports it.

The pages this follows, cited by title and section:

* [PLENA-C]  PLENA_Compiler PR #69, "MoE: shared experts, arbitrary V_TOPK expert
  shapes, and an enforced stage-marker contract".
* [PLENA-S]  PLENA_Simulator PR #97, "MoE: timing-replay harnesses, shared experts,
  parameterized V_TOPK routing".
* [SPYRE]    hf-adapters PR #2, "Add persistent dense-expert MoE path via spyre::moe_ffn".
* [VEOMNI]   VeOmni docs, "Fused MoE Kernel Notes".

The layer (both PLENA pages, section "Group C -- shared experts" / "Part 2 -- Shared
experts"):

    y = shared(x) + sum_k route_weight_k * routed_expert_k(x)

computed in five steps: router logits and top-k softmax; scatter of tokens into
expert-grouped rows through a scatter_index ([VEOMNI] "Scatter/gather layout");
per-expert SwiGLU FFN; weighted gather back to token order; optional (optionally
sigmoid-gated) shared expert.

Precision.  ``dtype`` selects the arithmetic: float64 (default; used by the
property pins) or float32 (used for timing and large parity runs).  ``contract``
rounds the SwiGLU output to bfloat16 (round-to-nearest-even) at the point where a
bf16 implementation feeds it to the down projection; [PLENA-S] section "Tests"
describes a reference that mirrors BF16 rounding step by step for the same reason.
Router logits are always produced as float32 (accumulated in float64, rounded
once) because top-k is decided on float32 values.

Readings taken where the pages are silent (each is also listed in the design notes):

* top-k is taken over the float32 logits; softmax is monotone so this equals
  top-k over probabilities in exact arithmetic;
* ties go to the lower expert index; slots are ordered by descending logit, ties
  lower index first;
* route weights are the softmax over the k selected logits (equal to softmax
  over all E experts, then renormalised over the selected ones);
* fc1 columns [0, I) are the gate projection and [I, 2I) the up projection;
  SwiGLU is silu(gate) * up with silu(g) = g * sigmoid(g);
* rows inside an expert group are ordered by the flattened pair index
  p = t * top_k + j (a stable counting sort); groups are in ascending expert id;
* expert ids outside [0, E) in fed-in routes are errors: they are counted,
  receive scatter_index -1 and contribute nothing;
* the combine adds routed slots in ascending j, in the working precision;
* the shared gate is sigmoid(x . w_gate), one scalar per token, scaling only the
  shared branch;
* the backward (section "Backward of the routed experts" below) holds the routes
  fixed and follows the chain rule of the forward steps.

Parity status: every function below is pinned by a CPU test against something
other than itself (closed forms, hand-derived examples, brute force, invariants,
independent library routines); see the pin tests under tests/.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_rne",
    "router_logits",
    "topk_select",
    "route_weights",
    "route",
    "router_logit_bound",
    "build_scatter",
    "scatter_rows",
    "silu",
    "expert_ffn",
    "grouped_swiglu_up",
    "grouped_down",
    "grouped_experts",
    "gather_combine",
    "shared_expert",
    "fuse_shared",
    "moe_forward",
    "dense_mask_forward",
    "token_outputs",
    "e4m3_decode",
    "e8m0_decode",
    "mx_dequant",
    "swiglu_grad",
    "grouped_fc1_saved",
    "scatter_grad",
    "grouped_experts_backward",
    "gather_sum",
    "moe_backward",
]


# ----------------------------------------------------------------------------
# bfloat16 rounding
# ----------------------------------------------------------------------------
def bf16_rne(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  Written
    from the IEEE-754 definition: bfloat16 keeps the top 16 bits of a float32,
    so round-to-nearest-even adds 0x7FFF plus the lowest kept bit to the
    32-bit pattern and truncates.  NaN stays NaN.
    """
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    bits = a32.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(a32), np.float32(np.nan), out)
    return out.reshape(a32.shape)


# ----------------------------------------------------------------------------
# MXFP8 expert weights
# ----------------------------------------------------------------------------
# [PLENA-C], section "Group C -- shared experts" (the paragraph on the fusion
# identity): expert weights are MXFP8 -- e4m3 values with one e8m0 scale per
# block of 8 consecutive elements along the intermediate axis.  The pages name
# the two encodings without spelling out their bits; the reading taken here is
# the OCP microscaling definition: e4m3 has a sign bit, a 4-bit exponent with
# bias 7 and a 3-bit mantissa, subnormals at exponent 0, no infinities, and
# only S.1111.111 is NaN (largest finite value 448); e8m0 is a bare exponent
# with bias 127 whose all-ones code is NaN.  Dequantization is exact: value =
# e4m3(code) * 2**(scale - 127), evaluated in float64.

def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each e4m3 byte."""
    b = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & (m == 7), np.nan, out)


def e8m0_decode(scales) -> np.ndarray:
    """float64 value 2**(s - 127) of each e8m0 byte (255 is NaN)."""
    s = np.asarray(scales).astype(np.int64) & 0xFF
    return np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))


def mx_dequant(codes, scales, axis: int, block: int = 8) -> np.ndarray:
    """Exact float64 weights from e4m3 codes and their e8m0 block scales.

    ``scales`` has the shape of ``codes`` with dimension ``axis`` divided by
    ``block``: element i along that axis takes the scale of block i // block."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if codes.shape[axis] != scales.shape[axis] * block:
        raise ValueError(f"scales cover {scales.shape[axis] * block} elements along axis {axis}, "
                         f"codes have {codes.shape[axis]}")
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), block, axis=axis)


# ----------------------------------------------------------------------------
# Step 1: router GEMM and top-k softmax
# ----------------------------------------------------------------------------
def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Router logits L = x @ W_r (+ b).

    [PLENA-C] section "Group E" (the router GEMM, moe_router_logits_bf16_v0).
    The product is accumulated in float64 and rounded once to float32; an
    optional per-expert float32 bias is then added in float32.
    """
    L = (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)).astype(np.float32)
    if bias is not None:
        L = (L + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    return L


def topk_select(logits, top_k: int) -> np.ndarray:
    """Indices of the top_k experts per token, in slot order.

    [PLENA-S] section "C_SET_TOPK_REG": topk_softmax is generic in the expert
    count and k, and k must be positive.  Order key per token: (logit
    descending, expert index ascending); NaN logits rank below every number.
    A stable lexicographic sort provides the order.
    """
    L = np.asarray(logits, np.float32)
    if top_k < 1:
        raise ValueError("topk must be positive")
    T, E = L.shape
    if top_k > E:
        raise ValueError("top_k exceeds the number of experts")
    key = np.where(np.isnan(L), -np.inf, L).astype(np.float64)
    index = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((index, -key), axis=-1)
    return order[:, :top_k].astype(np.int32)


def route_weights(logits, ids) -> np.ndarray:
    """Route weights: softmax over the k selected logits, in float64, stored as float32.

    Slot 0 holds the largest selected logit, which is subtracted before exp.
    """
    L = np.asarray(logits, np.float64)
    sel = np.take_along_axis(L, np.asarray(ids, np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x, w_router, top_k: int, bias=None):
    """Step 1 in full: (logits float32 [T,E], ids int32 [T,k], weights float32 [T,k])."""
    L = router_logits(x, w_router, bias)
    ids = topk_select(L, top_k)
    return L, ids, route_weights(L, ids)


def router_logit_bound(x, w_router, bias=None) -> np.ndarray:
    """Largest distance [T,E] between router_logits and logits accumulated in float32.

    The pages fix no precision for the router GEMM ([PLENA-C] section "Group E"
    names it only), so a float32-accumulating implementation may sum the H
    products in any order.  Every order obeys the forward error bound of a
    summed dot product, |fl(sum_h x_h w_h) - sum_h x_h w_h| <= gamma_H *
    sum_h |x_h| |w_h| with gamma_n = n u / (1 - n u) and u = 2^-24 (Higham,
    "Accuracy and Stability of Numerical Algorithms", section 3.1; products of
    bf16 or float32 inputs taken exactly or rounded once are covered by the
    same gamma).  Returned: twice that term, plus four float32 units of
    |value| + |bias| for the rounding of router_logits itself and of the bias
    add on either side.  A near tie between the k-th and (k+1)-th logit closer
    than this bound may legitimately order differently.
    """
    u = 2.0 ** -24
    ax = np.abs(np.asarray(x, np.float64))
    aw = np.abs(np.asarray(w_router, np.float64))
    H = ax.shape[1]
    gamma = H * u / (1.0 - H * u)
    mag = ax @ aw
    b = 0.0 if bias is None else np.abs(np.asarray(bias, np.float64))[None, :]
    return 2.0 * gamma * mag + 4.0 * u * (mag + b) + 1e-30


# ----------------------------------------------------------------------------
# Step 2: scatter into expert-grouped rows
# ----------------------------------------------------------------------------
def build_scatter(ids, num_experts: int) -> dict:
    """Expert-grouped row layout for routed pairs.

    [VEOMNI] section "Scatter/gather layout": tokens [T, H] expand to
    [T * top_k, H] rows grouped by expert; scatter_index maps each
    (token, slot) pair to its row.  Section "Duplicate top-k routes": several
    slots of one token may name the same expert, so a group can hold more
    than T rows.

    Pairs p = t * top_k + j are visited in increasing p; each valid pair takes
    the next free row of its expert's group (a stable counting sort).  Pairs
    whose expert id lies outside [0, E) are counted in ``n_bad`` and get
    scatter_index -1.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    E = int(num_experts)
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.zeros(E, np.int64)
    n_bad = 0
    for e in flat:
        if 0 <= e < E:
            counts[e] += 1
        else:
            n_bad += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = offsets[:-1].copy()
    scatter_index = np.full(T * k, -1, np.int64)
    row_token = np.full(T * k, -1, np.int64)
    for p, e in enumerate(flat):
        if 0 <= e < E:
            r = next_row[e]
            next_row[e] += 1
            scatter_index[p] = r
            row_token[r] = p // k
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "scatter_index": scatter_index.reshape(T, k).astype(np.int32),
        "row_token": row_token.astype(np.int32),
        "max_group": int(counts.max()) if E > 0 else 0,
        "n_bad": int(n_bad),
    }


def scatter_rows(x, row_token) -> np.ndarray:
    """X_s[r] = x[row_token[r]] for assigned rows; unassigned rows (token -1) stay NaN."""
    x = np.asarray(x)
    rt = np.asarray(row_token)
    Xs = np.full((rt.shape[0], x.shape[1]), np.nan, dtype=x.dtype)
    ok = rt >= 0
    Xs[ok] = x[rt[ok]]
    return Xs


# ----------------------------------------------------------------------------
# Step 3: SwiGLU expert FFN
# ----------------------------------------------------------------------------
def silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(xrows, w1, w2, *, contract: bool = False, dtype=np.float64):
    """One expert: a = silu(x W1[:, :I]) * (x W1[:, I:]); y = a W2.

    [PLENA-C] section "Group C -- shared experts" (SwiGLU along the
    intermediate axis, then the down projection); [PLENA-S] section "Tests"
    (silu(g)*u).  W1 is [H, 2I] with the gate in columns [0, I) and the up
    projection in [I, 2I); W2 is [I, H].  With ``contract`` the activation is
    rounded to bfloat16 before the down projection.  Returns (a, y).
    """
    X = np.asarray(xrows, dtype)
    W1 = np.asarray(w1, dtype)
    W2 = np.asarray(w2, dtype)
    I = W2.shape[0]
    if W1.shape[1] != 2 * I:
        raise ValueError("w1 must be [H, 2I] for w2 [I, H]")
    h = X @ W1
    a = silu(h[:, :I]) * h[:, I:]
    if contract:
        a = bf16_rne(a.astype(np.float32)).astype(dtype)
    return a, a @ W2


def _group_bounds(offsets, stale_row_bound=None):
    off = np.asarray(offsets, np.int64)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if stale_row_bound is not None:
            hi = min(hi, lo + int(stale_row_bound))
        yield e, lo, hi


def grouped_swiglu_up(Xs, offsets, W1, *, contract: bool = False, dtype=np.float64,
                      _stale_row_bound: int | None = None) -> np.ndarray:
    """First half of every expert over its group: A[r] = silu(X_s[r] W1[e][:, :I]) * (X_s[r] W1[e][:, I:]).

    Group e is rows [offsets[e], offsets[e+1]); rows outside every group stay NaN.
    ``_stale_row_bound`` exists only for the mutation test (see grouped_experts).
    """
    Xs = np.asarray(Xs)
    I = np.asarray(W1[0]).shape[1] // 2
    A = np.full((Xs.shape[0], I), np.nan, dtype)
    for e, lo, hi in _group_bounds(offsets, _stale_row_bound):
        if hi > lo:
            h = np.asarray(Xs[lo:hi], dtype) @ np.asarray(W1[e], dtype)
            a = silu(h[:, :I]) * h[:, I:]
            if contract:
                a = bf16_rne(a.astype(np.float32)).astype(dtype)
            A[lo:hi] = a
    return A


def grouped_down(A, offsets, W2, *, dtype=np.float64, _stale_row_bound: int | None = None) -> np.ndarray:
    """Second half of every expert over its group: Y_s[r] = A[r] W2[e]; other rows stay NaN."""
    A = np.asarray(A)
    H = np.asarray(W2[0]).shape[1]
    Ys = np.full((A.shape[0], H), np.nan, dtype)
    for e, lo, hi in _group_bounds(offsets, _stale_row_bound):
        if hi > lo:
            Ys[lo:hi] = np.asarray(A[lo:hi], dtype) @ np.asarray(W2[e], dtype)
    return Ys


def grouped_experts(Xs, offsets, W1, W2, *, contract: bool = False, dtype=np.float64,
                    _stale_row_bound: int | None = None):
    """Per-expert FFN over the expert-grouped rows.

    Group e is rows [offsets[e], offsets[e+1]).  Every row of every group is
    computed; [VEOMNI] section "Backward grouped-GEMM launch bound" explains why
    the bound must come from the largest group, not the token count.  Rows
    outside every group stay NaN in the outputs.

    ``_stale_row_bound`` exists only for the mutation test: it computes at most
    that many rows per group, emulating the stale bound that page describes.
    Returns (A [R, I], Y_s [R, H]).
    """
    A = grouped_swiglu_up(Xs, offsets, W1, contract=contract, dtype=dtype,
                          _stale_row_bound=_stale_row_bound)
    Ys = grouped_down(A, offsets, W2, dtype=dtype, _stale_row_bound=_stale_row_bound)
    return A, Ys


# ----------------------------------------------------------------------------
# Step 4: weighted gather back to token order
# ----------------------------------------------------------------------------
def gather_combine(Ys, scatter_index, weights, *, dtype=np.float64) -> np.ndarray:
    """y[t] = sum over j ascending of w[t, j] * Y_s[scatter_index[t, j]].

    [VEOMNI] section "Scatter/gather layout" (moe_gather sums routed outputs
    back to [tokens, hidden]).  Pull form: each output row reads its own k
    rows, so duplicate routes of one token need no read-modify-write ([SPYRE],
    commit on the loop-on-topk decode combine).  Pairs with index -1 add nothing.
    """
    Ys = np.asarray(Ys, dtype)
    si = np.asarray(scatter_index, np.int64)
    w = np.asarray(weights, dtype)
    T, k = si.shape
    y = np.zeros((T, Ys.shape[1]), dtype)
    for j in range(k):
        r = si[:, j]
        ok = r >= 0
        y[ok] = y[ok] + w[ok, j:j + 1] * Ys[r[ok]]
    return y


# ----------------------------------------------------------------------------
# Step 5: shared expert
# ----------------------------------------------------------------------------
def shared_expert(x, ws1, ws2, w_gate=None, *, contract: bool = False, dtype=np.float64):
    """Shared expert over all tokens, optionally sigmoid-gated.

    [PLENA-C] section "Group C -- shared experts": a dense FFN every token
    passes through, added unweighted; Qwen2-MoE's variant scales it by
    sigmoid(x @ w_gate), one scalar per token broadcast over hidden.  Returns
    the shared branch output [T, H] (not yet added to anything).
    """
    _, ys = expert_ffn(x, ws1, ws2, contract=contract, dtype=dtype)
    if w_gate is not None:
        z = np.asarray(x, dtype) @ np.asarray(w_gate, dtype).reshape(-1)
        gate = 1.0 / (1.0 + np.exp(-z))
        ys = ys * gate[:, None]
    return ys


def fuse_shared(experts):
    """Fuse n shared experts into one MLP of width sum(I_i).

    [PLENA-C] section "Group C -- shared experts" (fused_shared_intermediate):
    SwiGLU is elementwise along the intermediate axis and the down projection
    sums over it, so concatenating the experts along that axis gives exactly
    (in real arithmetic) the sum of the individual experts.  ``experts`` is a
    list of (w1 [H, 2I_i], w2 [I_i, H]); the result is (Ws1 [H, 2*sum I_i]
    laid out [gate_1 .. gate_n | up_1 .. up_n], Ws2 [sum I_i, H]).
    """
    gates, ups, downs = [], [], []
    for w1, w2 in experts:
        I = np.asarray(w2).shape[0]
        gates.append(np.asarray(w1)[:, :I])
        ups.append(np.asarray(w1)[:, I:])
        downs.append(np.asarray(w2))
    return np.concatenate(gates + ups, axis=1), np.concatenate(downs, axis=0)


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------
def moe_forward(x, w_router, W1, W2, top_k: int, *, bias=None, routes=None,
                shared=None, contract: bool = False, dtype=np.float64,
                _stale_row_bound: int | None = None) -> dict:
    """Forward pass of one MoE FFN layer, step by step.

    ``routes`` = (ids [T,k] int, weights [T,k]) feeds routes in and skips step 1
    (duplicates allowed).  ``shared`` = (ws1, ws2, w_gate or None) or None.
    Returns every intermediate of the pass in a dict.
    """
    x = np.asarray(x)
    E = len(W1)
    out = {}
    if routes is None:
        L, ids, w = route(x, w_router, top_k, bias)
        out["logits"] = L
    else:
        ids = np.asarray(routes[0], np.int32)
        w = np.asarray(routes[1], np.float32)
    out["ids"], out["weights"] = ids, w
    sc = build_scatter(ids, E)
    out.update(sc)
    Xs = scatter_rows(x, sc["row_token"])
    out["Xs"] = Xs
    A, Ys = grouped_experts(Xs, sc["offsets"], W1, W2, contract=contract, dtype=dtype,
                            _stale_row_bound=_stale_row_bound)
    out["A"], out["Ys"] = A, Ys
    y = gather_combine(Ys, sc["scatter_index"], w, dtype=dtype)
    if shared is not None:
        ws1, ws2, wg = shared
        ys = shared_expert(x, ws1, ws2, wg, contract=contract, dtype=dtype)
        out["y_shared"] = ys
        y = y + ys
    out["y"] = y
    return out


def dense_mask_forward(x, W1, W2, ids, weights, *, dtype=np.float64) -> np.ndarray:
    """Dense all-expert formulation of the routed part (no scatter at all).

    y[t] = sum_e r[t, e] * expert_e(x[t]) with r[t, e] = sum of w[t, j] over
    slots j that chose e.  This is the dense persistent formulation of [SPYRE]
    (router once, every expert over every token, one routing scalar per
    (token, expert)); it costs E/k times the routed work and serves only as a
    brute-force cross-check on tiny shapes.
    """
    x = np.asarray(x, dtype)
    ids = np.asarray(ids)
    w = np.asarray(weights, dtype)
    T, k = ids.shape
    E = len(W1)
    r = np.zeros((T, E), dtype)
    for t in range(T):
        for j in range(k):
            if 0 <= ids[t, j] < E:
                r[t, ids[t, j]] += w[t, j]
    y = np.zeros((T, np.asarray(W2[0]).shape[1]), dtype)
    for e in range(E):
        _, ye = expert_ffn(x, W1[e], W2[e], dtype=dtype)
        y = y + r[:, e:e + 1] * ye
    return y


def token_outputs(x_rows, ids_rows, w_rows, get_expert, *, shared=None,
                  contract: bool = False, dtype=np.float64) -> dict:
    """Layer output for a sample of tokens, straight from the layer equation.

    y[t] = sum_j w[t, j] * expert_{ids[t, j]}(x[t]) (+ shared(x[t])), used to
    check full-size runs on sampled tokens.  ``get_expert(e)`` returns
    (w1 [H, 2I], w2 [I, H]) for expert e.  Returns {"y": [S, H],
    "per_slot": [S, k, H]} (the latter = expert_{ids[t,j]}(x[t]), i.e. the
    Y_s row that pair (t, j) must produce).
    """
    X = np.asarray(x_rows, dtype)
    ids = np.asarray(ids_rows)
    w = np.asarray(w_rows, dtype)
    S, k = ids.shape
    per_slot = np.zeros((S, k, X.shape[1]), dtype)
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        w1, w2 = get_expert(e)
        mask = ids == e
        rows = np.nonzero(mask.any(axis=1))[0]
        _, ye = expert_ffn(X[rows], w1, w2, contract=contract, dtype=dtype)
        for n, t in enumerate(rows):
            for j in range(k):
                if ids[t, j] == e:
                    per_slot[t, j] = ye[n]
    y = np.zeros((S, X.shape[1]), dtype)
    for j in range(k):
        y = y + w[:, j:j + 1] * per_slot[:, j]
    out = {"per_slot": per_slot}
    if shared is not None:
        ws1, ws2, wg = shared
        ys = shared_expert(X, ws1, ws2, wg, contract=contract, dtype=dtype)
        out["y_shared"] = ys
        y = y + ys
    out["y"] = y
    return out


# ----------------------------------------------------------------------------
# Backward of the routed experts (routes held fixed)
# ----------------------------------------------------------------------------
# [VEOMNI], sections "Backward grouped-GEMM launch bound", "Duplicate top-k
# routes" and "Regression test pattern": the backward scatters the output
# gradient into the expert-grouped rows (grad_fc2_output is moe_scatter of
# grad_output through scatter_index), runs same-N/K grouped GEMMs for the input
# gradients (every row of the largest group covered, not only the first
# `tokens` rows) and same-M/N grouped GEMMs for the weight gradients (the
# reduction runs over a group's rows), and its results must stay finite when
# every slot of every token names the same expert.  The page gives no
# formulas; the ones below are the chain rule applied to the forward above:
#
# * row r = scatter_index[t, j] receives dYs[r] = w[t, j] * dy[t], because the
#   combine weights that row by w[t, j];
# * the route weight's gradient is dw[t, j] = dy[t] . Ys[r]; the routes
#   themselves are constants (no gradient flows through the top-k choice, and
#   the softmax's own backward to the router logits is not part of this step);
# * d[silu(g) u]/dg = u s (1 + g (1 - s)) with s = sigmoid(g), d/du = silu(g);
# * dA = dYs W2[e]^T, dH = [dG | dU], dXs = dH W1[e]^T, dW2[e] = A^T dYs and
#   dW1[e] = Xs^T dH over the rows of group e;
# * x's gradient through the routed experts is the unweighted sum of the dXs
#   rows of its k slots (the weights were applied to dYs already).
#
# Precision with ``contract``: values are rounded to bfloat16 where a bf16
# implementation stores them before they feed a later product -- the fc1
# pre-activation H_pre and the SwiGLU output A (each from the unrounded
# fc1 result), the scattered gradient dYs (formed in float32, then rounded) and
# the fc1 gradient dH.  Everything else is left in the working precision.
def swiglu_grad(g, u, dA):
    """Gradient of silu(g) * u: returns (dG, dU) = (dA u s (1 + g (1 - s)), dA silu(g)), s = sigmoid(g)."""
    g = np.asarray(g)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    dG = dA * u * s * (1.0 + g * (1.0 - s))
    dU = dA * g * s
    return dG, dU


def grouped_fc1_saved(Xs, offsets, W1, *, contract: bool = False, dtype=np.float64,
                      _stale_row_bound: int | None = None):
    """fc1 of every group, keeping what the backward needs: (H_pre [R, 2I], A [R, I]).

    H_pre[r] = X_s[r] W1[e] (gate columns [0, I), up columns [I, 2I)) and
    A[r] = silu(gate) * up, both from the unrounded product; with ``contract``
    each is then rounded to bfloat16.  Rows outside every group stay NaN.
    """
    Xs = np.asarray(Xs)
    I = np.asarray(W1[0]).shape[1] // 2
    Hp = np.full((Xs.shape[0], 2 * I), np.nan, dtype)
    A = np.full((Xs.shape[0], I), np.nan, dtype)
    for e, lo, hi in _group_bounds(offsets, _stale_row_bound):
        if hi > lo:
            h = np.asarray(Xs[lo:hi], dtype) @ np.asarray(W1[e], dtype)
            a = silu(h[:, :I]) * h[:, I:]
            if contract:
                h = bf16_rne(h.astype(np.float32)).astype(dtype)
                a = bf16_rne(a.astype(np.float32)).astype(dtype)
            Hp[lo:hi] = h
            A[lo:hi] = a
    return Hp, A


def scatter_grad(dy, Ys, scatter_index, weights, *, contract: bool = False, dtype=np.float64):
    """Output gradient into the expert-grouped rows, and the route weights' gradient.

    For every pair (t, j) with r = scatter_index[t, j] >= 0:
    dYs[r] = w[t, j] * dy[t] and dw[t, j] = dy[t] . Ys[r].  Rows that no pair
    names stay NaN; pairs with index -1 get dw = 0.  With ``contract`` the
    product w * dy is formed in float32 and rounded to bfloat16.
    """
    dy = np.asarray(dy, dtype)
    Ys = np.asarray(Ys, dtype)
    si = np.asarray(scatter_index, np.int64)
    w = np.asarray(weights)
    T, k = si.shape
    dYs = np.full((Ys.shape[0], dy.shape[1]), np.nan, dtype)
    dw = np.zeros((T, k), dtype)
    for t in range(T):
        for j in range(k):
            r = si[t, j]
            if r < 0:
                continue
            if contract:
                prod = np.float32(w[t, j]) * dy[t].astype(np.float32)
                dYs[r] = bf16_rne(prod).astype(dtype)
            else:
                dYs[r] = np.asarray(w[t, j], dtype) * dy[t]
            dw[t, j] = dy[t] @ Ys[r]
    return dYs, dw


def grouped_experts_backward(Xs, offsets, W1, W2, H_pre, A, dYs, *, contract: bool = False,
                             dtype=np.float64, split_fc1: bool = False, weight_grads: bool = True,
                             _stale_row_bound: int | None = None) -> dict:
    """Input and weight gradients of every expert over its group.

    For group e (rows [offsets[e], offsets[e+1])): dA = dYs W2[e]^T, then
    (dG, dU) = swiglu_grad(gate, up, dA) on H_pre, dH = [dG | dU],
    dXs = dH W1[e]^T, dW2[e] = A^T dYs and dW1[e] = Xs^T dH.

    ``split_fc1`` treats fc1 as two separate projections (gate weights
    W1[e][:, :I], up weights W1[e][:, I:]): dXs = dG Wg^T + dU Wu^T and the two
    weight gradients are computed apart and placed side by side -- the split
    formulation that the merged one must match.  An empty group gets zero
    weight gradients.  Rows outside every group stay NaN in dH and dXs.
    With ``weight_grads`` False the weight gradients are not formed (dW1 and
    dW2 are None; nothing else changes).
    Returns {"dA", "dH", "dXs", "dW1" [E, H, 2I], "dW2" [E, I, H]}.
    """
    Xs = np.asarray(Xs)
    E = len(W1)
    Hd = np.asarray(W1[0]).shape[0]
    I = np.asarray(W2[0]).shape[0]
    R = Xs.shape[0]
    dA_all = np.full((R, I), np.nan, dtype)
    dH_all = np.full((R, 2 * I), np.nan, dtype)
    dXs = np.full((R, Hd), np.nan, dtype)
    dW1 = np.zeros((E, Hd, 2 * I), dtype) if weight_grads else None
    dW2 = np.zeros((E, I, np.asarray(W2[0]).shape[1]), dtype) if weight_grads else None
    for e, lo, hi in _group_bounds(offsets, _stale_row_bound):
        if hi <= lo:
            continue
        w1 = np.asarray(W1[e], dtype)
        w2 = np.asarray(W2[e], dtype)
        x = np.asarray(Xs[lo:hi], dtype)
        dy = np.asarray(dYs[lo:hi], dtype)
        dA = dy @ w2.T
        hp = np.asarray(H_pre[lo:hi], dtype)
        dG, dU = swiglu_grad(hp[:, :I], hp[:, I:], dA)
        if contract:
            dG = bf16_rne(dG.astype(np.float32)).astype(dtype)
            dU = bf16_rne(dU.astype(np.float32)).astype(dtype)
        dA_all[lo:hi] = dA
        dH_all[lo:hi, :I] = dG
        dH_all[lo:hi, I:] = dU
        if weight_grads:
            dW2[e] = np.asarray(A[lo:hi], dtype).T @ dy
        if split_fc1:
            wg, wu = w1[:, :I], w1[:, I:]
            dXs[lo:hi] = dG @ wg.T + dU @ wu.T
            if weight_grads:
                dW1[e, :, :I] = x.T @ dG
                dW1[e, :, I:] = x.T @ dU
        else:
            dH = np.concatenate([dG, dU], axis=1)
            dXs[lo:hi] = dH @ w1.T
            if weight_grads:
                dW1[e] = x.T @ dH
    return {"dA": dA_all, "dH": dH_all, "dXs": dXs, "dW1": dW1, "dW2": dW2}


def gather_sum(dXs, scatter_index, *, dtype=np.float64) -> np.ndarray:
    """dx[t] = sum over j ascending of dXs[scatter_index[t, j]] (pairs with index -1 add nothing)."""
    si = np.asarray(scatter_index, np.int64)
    return gather_combine(dXs, si, np.ones(si.shape, dtype), dtype=dtype)


def moe_backward(x, W1, W2, routes, dy, *, contract: bool = False, dtype=np.float64,
                 split_fc1: bool = False, weight_grads: bool = True,
                 _stale_row_bound: int | None = None) -> dict:
    """Gradients of the routed part of the layer for fixed routes.

    ``routes`` = (ids [T, k], weights [T, k]); ``dy`` [T, H] is the gradient of
    the loss with respect to the layer output y.  Runs the forward steps
    (scatter, fc1 keeping H_pre and A, fc2) and then the backward steps above.
    Returns every intermediate plus dx [T, H], dW1 [E, H, 2I], dW2 [E, I, H]
    and dweights [T, k].  ``_stale_row_bound`` exists only for the mutation
    test: it limits every group to that many rows, as a launch bound of
    `tokens` rows would.  ``weight_grads`` False skips dW1 / dW2 (for checks
    of dx and dweights on a sample of tokens of a large layer).
    """
    ids = np.asarray(routes[0], np.int64)
    w = np.asarray(routes[1])
    E = len(W1)
    sc = build_scatter(ids, E)
    Xs = scatter_rows(x, sc["row_token"])
    Hp, A = grouped_fc1_saved(Xs, sc["offsets"], W1, contract=contract, dtype=dtype,
                              _stale_row_bound=_stale_row_bound)
    Ys = grouped_down(A, sc["offsets"], W2, dtype=dtype, _stale_row_bound=_stale_row_bound)
    dYs, dw = scatter_grad(dy, Ys, sc["scatter_index"], w, contract=contract, dtype=dtype)
    g = grouped_experts_backward(Xs, sc["offsets"], W1, W2, Hp, A, dYs, contract=contract, dtype=dtype,
                                 split_fc1=split_fc1, weight_grads=weight_grads,
                                 _stale_row_bound=_stale_row_bound)
    out = dict(sc)
    out.update({"Xs": Xs, "H_pre": Hp, "A": A, "Ys": Ys, "dYs": dYs, "dweights": dw})
    out.update(g)
    out["dx"] = gather_sum(g["dXs"], sc["scatter_index"], dtype=dtype)
    return out
