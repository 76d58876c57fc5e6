"""CPU oracle for the forward pass of the sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module: only the tests, the smoke check and the bench's CPU-baseline leg do.  It
shares no code with the HIP library and imports nothing from it.

It is a plain, slow, obviously correct numpy implementation written from the pages:

  [book ch.30]   "Chapter 30: Mixture of Experts", LLM Transformer book, Japanese
                 edition (waylandz.com)
  [MoE guide]    "Mixture of Experts guide" (ai-native-b2y.pages.dev)
  [MoE memo]     "Mixture of Experts (MoE) memo" (iwashi.co)
  [MoE practice] "Mixture-of-experts in practice: routing, load balancing and parallel
                 configuration" (deepseekmodel.com blog)

Precision.  Inputs arrive as float32 arrays holding bf16 (or fp32) values and are
widened exactly to float64.  Every dot product and reduction runs in float64 and is
rounded once to float32 where the layer has a float32 boundary: the router
probabilities, the selection score, the mixing weights, the expert intermediate h
(rounded further to bf16 for the bf16 workloads, because h is the down projection's
input) and the expert output o.  Decisions that floating point makes for an integer
(the top-k choice) are taken in float32, the precision the layer computes them in.

Readings where the pages are silent or disagree (each one is listed in the design
notes of the repository):
  * the selection bias is added to the softmax probabilities, not the logits;
  * ties in the selection score go to the lower expert index, and slots are ordered
    by selection score, highest first;
  * f_e counts top-k assignments before any capacity drop and is normalised by T*k;
  * capacity C = max(floor(cf * k * T / E), k), the product taken exactly on the
    float32 value of cf (C above T*k reported as T*k); assignments are ranked per expert
    in row-major (token, slot) order and the first C are kept;
  * a dropped assignment contributes zero; the layer adds no residual;
  * overflow handed to the next-best expert ([book ch.30] 30.5.2) is one redirect round:
    each assignment dropped by the capacity goes to its token's next unused expert by
    selection score, which takes such offers in row-major order while it has room; the
    slot keeps its weight;
  * 8-bit expert weights (an extension past the pages' layer: [book ch.30] 30.4.6 counts
    FP8 among the measures that halve the memory traffic of each operation, and
    [MoE practice], section on quantisation and routing, keeps the router in high
    precision while the expert weights take the quantisation) are e4m3 "fn" codes with
    one float32 scale per output row, dequantised exactly before the same arithmetic;
    the router, x and h stay as in the bf16 layer;
  * expert-choice routing (the second routing of the pages: [MoE memo] routing-design
    table, [MoE practice] top-k section) scores tokens by the softmax probabilities,
    gives each expert the C = min(T, max(floor(cf * k * T / E), k)) tokens with the
    largest score (ties to the lower token index), and weights each output by that
    probability without renormalisation.

Pins: tests/test_oracle_pins.py checks each function against values the pages print,
closed forms, library routines and brute force.  Large-shape absolute values are
"parity unpinned" except through these functions.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------- numerics
def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; returns float32.

    bfloat16 keeps the top 16 bits of an IEEE float32.  Round-to-nearest-even adds
    0x7FFF plus the lowest kept bit, then truncates.  Inputs are finite here.
    """
    u = np.ascontiguousarray(a, dtype=F32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F32)


def e4m3_decode(q) -> np.ndarray:
    """Value of each 8-bit float in the e4m3 "fn" encoding; returns float64.

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the mantissa.  An
    exponent field of 0 is subnormal: m/8 * 2^-6.  Otherwise (1 + m/8) * 2^(e - 7),
    except that e = 15 with m = 7 is NaN (the encoding has no infinities, so the
    largest finite value is 1.75 * 2^8 = 448).
    """
    q = np.asarray(q, np.uint8).astype(np.int64)
    sign = np.where(q & 0x80, -1.0, 1.0)
    e = (q >> 3) & 0xF
    m = (q & 0x7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def dequant_rows(q, scale) -> np.ndarray:
    """Weights stored as e4m3 codes with one float32 scale per output row:
    W[n, :] = scale[n] * decode(q[n, :]), in float64 (exact: no rounding happens)."""
    return np.asarray(scale, F64)[:, None] * e4m3_decode(q)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))   ([book ch.30] 30.2.4)."""
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------- router
def router_probs(x: np.ndarray, W_router: np.ndarray) -> np.ndarray:
    """Router linear layer without bias, then softmax over the experts.

    logits[t, e] = sum_i x[t, i] * W_router[e, i]     ([book ch.30] 30.2.3 step 1;
    [MoE practice] routing-math section: the gate is a bias-free linear layer)
    p[t, :] = softmax(logits[t, :])                   ([book ch.30] 30.2.3 step 2)
    Computed in float64, returned rounded to float32.
    """
    logits = x.astype(F64) @ W_router.astype(F64).T
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(F32)


def select_topk(p: np.ndarray, k: int, bias: np.ndarray | None = None):
    """Top-k expert choice on the selection score s = p + bias.

    [book ch.30] 30.2.3 step 3 picks the k largest probabilities; with the
    aux-loss-free bias ([MoE memo] DeepSeek-V3 section; [MoE practice] load-balancing
    section, bias-balanced router) the bias enters the choice only.  s is formed in
    float32.  Order: s descending, ties to the lower expert index.

    Returns (idx [T,k] int32, s [T,E] float32, margin [T] float64) where margin is the
    smallest difference between neighbouring scores among the first k+1 in sorted
    order (the k-th/(k+1)-th gap, and the gaps that fix the order of the k slots);
    +inf when k == E == 1.
    """
    T, E = p.shape
    s = p.astype(F32) if bias is None else (p.astype(F32) + bias.astype(F32)[None, :])
    s = s.astype(F32)
    # stable sort on (-s) keeps the lower index first among equal scores
    order = np.argsort(-s.astype(F64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    m = min(k + 1, E)
    srt = np.take_along_axis(s, order[:, :m], axis=1).astype(F64)
    if m >= 2:
        margin = (srt[:, :-1] - srt[:, 1:]).min(axis=1)
    else:
        margin = np.full(T, np.inf)
    return idx, s, margin


def renorm_weights(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] on the unbiased probabilities.

    [book ch.30] 30.2.3 step 4; [MoE practice] routing-math section (renormalise
    always) and bias-balanced router (weights from the raw distribution).
    """
    sel = np.take_along_axis(p.astype(F64), idx.astype(np.int64), axis=1)
    return (sel / sel.sum(axis=1, keepdims=True)).astype(F32)


def route(x, W_router, k, bias=None):
    """Router + top-k + renorm.  Returns dict(p, idx, w, s, margin)."""
    p = router_probs(x, W_router)
    idx, s, margin = select_topk(p, k, bias)
    w = renorm_weights(p, idx)
    return {"p": p, "idx": idx, "w": w, "s": s, "margin": margin}


def aux_stats(p: np.ndarray, idx: np.ndarray, E: int):
    """Switch-style statistics f and P.

    f_e = share of the T*k top-k assignments that went to expert e (before capacity)
    P_e = mean over tokens of the router probability of expert e
    ([MoE memo] auxiliary-loss section, worked 2-expert example; [book ch.30] 30.2.6;
    [MoE practice] load-balancing section).  The loss itself is E * sum_e f_e * P_e.
    """
    T, k = idx.shape
    counts = np.bincount(idx.ravel().astype(np.int64), minlength=E)
    f = (counts.astype(F64) / float(T * k)).astype(F32)
    P = p.astype(F64).mean(axis=0).astype(F32)
    return f, P


def balance_loss(f, P) -> float:
    """E * sum_e f_e * P_e; equals 1 under uniform routing ([MoE memo] aux-loss section)."""
    return float(len(f) * np.sum(np.asarray(f, F64) * np.asarray(P, F64)))


# ----------------------------------------------------------------------------- dispatch
def capacity(T: int, k: int, E: int, cf: float):
    """Per-expert capacity C = max(floor(cf * k * T / E), k); None when cf <= 0.

    [MoE practice] routing-math section (capacity from the expected load k*T/E times the
    capacity factor, truncated, at least k); [book ch.30] 30.5.2 and [MoE guide]
    expert-capacity section give (T/E)*cf, the same number for top-1.

    The pages write the product in three orders, which round differently in binary
    floating point.  Reading taken: cf is the float32 value the layer's descriptor
    carries, and the product is exact (rational arithmetic, floored once), so no
    evaluation order enters.  A C above T*k keeps every assignment (an expert holds at
    most one slot of each token), so such a C is reported as T*k.
    """
    if cf is None or not cf > 0:
        return None
    cf32 = Fraction(float(np.float32(cf)))          # the exact binary value carried
    raw = math.floor(cf32 * k * T / E)
    return max(min(raw, T * k), k)


def dispatch(idx: np.ndarray, E: int, C=None):
    """Group the (token, slot) assignments by expert, stably, with the capacity cut.

    The T*k assignments are flattened row-major (i = t*k + j) and stably sorted by
    expert id ([MoE practice] expert-parallel section: flatten, stable argsort,
    bincount).  The r-th assignment of expert e in that order has rank r; it is kept
    iff r < C.  Kept rows of expert e occupy [offsets[e], offsets[e+1]).

    Returns dict(counts [E], kept [E], offsets [E+1], perm_src [N], slot_pos [T*k]):
    perm_src[pos] = i of the assignment in row pos; slot_pos[i] = pos or -1 (dropped).
    """
    flat = idx.reshape(-1).astype(np.int64)
    n = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty(n, np.int64)
    rank[order] = np.arange(n) - start[flat[order]]
    kept = counts if C is None else np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    keep = np.ones(n, bool) if C is None else rank < C
    slot_pos = np.where(keep, offsets[flat] + rank, -1)
    perm_src = np.empty(int(offsets[-1]), np.int64)
    perm_src[slot_pos[keep]] = np.nonzero(keep)[0]
    return {
        "counts": counts.astype(np.int32), "kept": kept.astype(np.int32),
        "offsets": offsets.astype(np.int32), "perm_src": perm_src.astype(np.int32),
        "slot_pos": slot_pos.astype(np.int32),
    }


# ----------------------------------------------------------------------------- experts
def expert_ffn(x_rows, Wg, Wu, Wd, h_bf16: bool, return_h: bool = False):
    """One SwiGLU expert on a block of rows: o = W2( SiLU(W1 x) * W3 x ).

    [book ch.30] 30.2.4 and 30.6.1: w1 (gate) goes through SiLU, w3 (up) is linear,
    w2 (down) projects back; no biases.  Here Wg = w1 [F,d], Wu = w3 [F,d],
    Wd = w2 [d,F].  h = fp32(SiLU(g) * u), rounded to bf16 when the layer's
    activations are bf16; o = fp32(W2 h).  With return_h, also returns the float64 g, u
    and h before any rounding (the tests use them to bound where a bf16 rounding of h
    may legitimately go either way).
    """
    xr = np.asarray(x_rows, F64)
    g = xr @ np.asarray(Wg, F64).T
    u = xr @ np.asarray(Wu, F64).T
    h64 = silu(g) * u
    h = h64.astype(F32)
    if h_bf16:
        h = bf16_round(h)
    o = (h.astype(F64) @ np.asarray(Wd, F64).T).astype(F32)
    return (o, {"g": g, "u": u, "h": h64}) if return_h else o


def combine(T, d, w, slot_pos, Y, shared=None) -> np.ndarray:
    """y[t] = sum over kept slots j (ascending) of w[t,j] * Y[slot_pos[t,j]] (+ shared[t]).

    [book ch.30] 30.6.1 (weighted accumulation per token); a dropped slot contributes
    zero ([MoE practice] capacity section: the FFN branch of a dropped token is 0);
    the shared expert is added with weight 1 ([book ch.30] 30.4.5).  float64 sums,
    rounded to float32.
    """
    k = w.shape[1]
    y = np.zeros((T, d), F64)
    sp = slot_pos.reshape(T, k)
    for j in range(k):
        rows = np.nonzero(sp[:, j] >= 0)[0]
        y[rows] += w[rows, j].astype(F64)[:, None] * Y[sp[rows, j]].astype(F64)
    if shared is not None:
        y += shared.astype(F64)
    return y.astype(F32)


# ----------------------------------------------------------------------------- layer
def _np(a):
    """torch tensor or array -> float32 numpy array (bf16 widens exactly)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float32).numpy()
    return np.asarray(a, F32)


def expert_weights(inputs: dict, e: int):
    """(W_gate[e], W_up[e], W_down[e]) of expert e.  With 8-bit expert weights (inputs
    holding Wq_gate, Wq_up, Wq_down as e4m3 codes and s_gate, s_up, s_down as per-row
    scales) they are dequantised exactly in float64; otherwise widened from float32."""
    if "Wq_gate" in inputs:
        q = lambda name: np.asarray(inputs[name][e].numpy() if hasattr(inputs[name], "numpy")
                                    else inputs[name][e], np.uint8)
        sc = lambda name: _np(inputs[name][e])
        return (dequant_rows(q("Wq_gate"), sc("s_gate")), dequant_rows(q("Wq_up"), sc("s_up")),
                dequant_rows(q("Wq_down"), sc("s_down")))
    return (_np(inputs["W_gate"][e]), _np(inputs["W_up"][e]), _np(inputs["W_down"][e]))


def forward(inputs: dict, k: int, capacity_factor: float = 0.0, n_shared: int = 0,
            h_bf16: bool = True, idx_override=None, next_best: bool = False,
            cand_override=None) -> dict:
    """The whole layer: route -> stats -> dispatch -> grouped experts -> combine.

    ``inputs`` holds x, W_router, router_bias (or None), W_gate, W_up, W_down as torch
    tensors or float32 arrays.  ``idx_override`` replaces the top-k choice (used where
    near-tied tokens have more than one correct routing); the weights are then
    renormalised from the same unbiased probabilities.  ``next_best`` hands assignments
    that overflow an expert's capacity to their token's next-best experts
    (``dispatch_next_best``) instead of dropping them; ``cand_override`` replaces their
    candidates (near-tied scores).
    """
    x = _np(inputs["x"])
    Wr = _np(inputs["W_router"])
    b = _np(inputs.get("router_bias"))
    T, d = x.shape
    E = Wr.shape[0]
    r = route(x, Wr, k, b)
    if idx_override is not None:
        r["idx"] = np.asarray(idx_override, np.int32)
        r["w"] = renorm_weights(r["p"], r["idx"])
    f, P = aux_stats(r["p"], r["idx"], E)
    C = capacity(T, k, E, capacity_factor)
    if next_best:
        r["cand"] = (next_best_candidates(r["s"], k, r["idx"]) if cand_override is None
                     else np.asarray(cand_override, np.int32))
        disp = dispatch_next_best(r["idx"], r["cand"], E, C)
    else:
        disp = dispatch(r["idx"], E, C)
    Y = np.zeros((int(disp["offsets"][-1]), d), F32)
    for e in range(E):
        lo, hi = int(disp["offsets"][e]), int(disp["offsets"][e + 1])
        if hi == lo:
            continue
        tok = disp["perm_src"][lo:hi] // k
        Y[lo:hi] = expert_ffn(x[tok], *expert_weights(inputs, e), h_bf16)
    shared = None
    if n_shared:
        shared = expert_ffn(x, *expert_weights(inputs, E), h_bf16)
    y = combine(T, d, r["w"], disp["slot_pos"], Y, shared)
    return {"y": y, "f": f, "p": P, "route": r, "dispatch": disp, "C": C}


def forward_rows(inputs: dict, rows, k: int, capacity_factor: float = 0.0,
                 n_shared: int = 0, h_bf16: bool = True, routing: dict | None = None,
                 disp: dict | None = None) -> np.ndarray:
    """Output rows y[rows] of the whole layer, computing experts only for those rows.

    Routing and dispatch (which decide drops under a capacity) are computed for every
    token, exactly as in ``forward``; the expert FFNs run only for the requested
    tokens.  Used where the full layer is too large for the CPU.
    """
    x = _np(inputs["x"])
    T, d = x.shape
    if routing is None:
        routing = route(x, _np(inputs["W_router"]), k, _np(inputs.get("router_bias")))
    E = routing["p"].shape[1]
    if disp is None:
        disp = dispatch(routing["idx"], E, capacity(T, k, E, capacity_factor))
    rows = np.asarray(rows, np.int64)
    sp = disp["slot_pos"].reshape(T, k)[rows]
    # the expert that processes each slot (differs from the top-k choice for redirected
    # slots)
    idx = disp["expert"].reshape(T, k)[rows] if "expert" in disp else routing["idx"][rows]
    w = routing["w"][rows]
    y = np.zeros((rows.size, d), F64)
    for e in np.unique(idx[sp >= 0]):
        sel = np.argwhere((idx == e) & (sp >= 0))        # (row-in-sample, slot)
        o = expert_ffn(x[rows[sel[:, 0]]], *expert_weights(inputs, int(e)), h_bf16)
        y[sel[:, 0]] += w[sel[:, 0], sel[:, 1]].astype(F64)[:, None] * o.astype(F64)
    if n_shared:
        y += expert_ffn(x[rows], *expert_weights(inputs, E), h_bf16).astype(F64)
    return y.astype(F32)


# ----------------------------------------------------------------------------- expert choice
def expert_choice_capacity(T: int, k: int, E: int, cf: float) -> int:
    """Tokens each expert takes under expert-choice routing: the per-expert capacity of
    ``capacity`` (C = max(floor(cf * k * T / E), k), k read as the average number of
    experts per token), at most T.  cf must be > 0.

    [MoE practice] top-k section: each expert takes its top-C tokens according to its
    capacity; the capacity is the routing-math section's.
    """
    if cf is None or cf <= 0:
        raise ValueError("expert-choice routing needs a capacity factor > 0")
    return min(T, capacity(T, k, E, cf))


def expert_choice_select(p: np.ndarray, C: int):
    """Each expert takes the C tokens with the largest router probability p[t, e].

    [MoE memo] routing section (the expert-choice row of the routing-design table: each
    expert picks the tokens that suit it, so every expert's load is equal); [MoE
    practice] top-k section (each expert picks its top-C tokens).  The scores are the
    token-wise softmax probabilities of ``router_probs`` (no bias), compared in float32;
    equal scores go to the lower token index.

    Returns (sel [E, C] int32: expert e's tokens in ascending token order, margin [E]
    float64: the gap between the C-th and the (C+1)-th largest p of the column, +inf when
    C == T; a column with margin < 1e-6 may be chosen either way in float32).
    """
    T, E = p.shape
    sel = np.empty((E, C), np.int32)
    margin = np.full(E, np.inf)
    for e in range(E):
        col = p[:, e].astype(F32).astype(F64)
        order = np.argsort(-col, kind="stable")    # stable: lower token first on ties
        sel[e] = np.sort(order[:C])
        if C < T:
            margin[e] = col[order[C - 1]] - col[order[C]]
    return sel, margin


def expert_choice_dispatch(sel: np.ndarray, T: int) -> dict:
    """Rows and slots of an expert-choice selection: expert e's rows are
    [e*C, (e+1)*C), holding its tokens in ascending order; slot[t, e] is the row of
    (t, e) or -1 when expert e did not take token t."""
    E, C = sel.shape
    offsets = (np.arange(E + 1, dtype=np.int64) * C).astype(np.int32)
    perm_src = sel.reshape(-1).astype(np.int32)
    slot = np.full((T, E), -1, np.int32)
    for e in range(E):
        slot[sel[e], e] = e * C + np.arange(C, dtype=np.int32)
    return {"offsets": offsets, "perm_src": perm_src, "slot": slot}


def forward_expert_choice(inputs: dict, k: int, capacity_factor: float, n_shared: int = 0,
                          h_bf16: bool = True, sel_override=None) -> dict:
    """The layer with expert-choice routing.

    p = router_probs(x, W_router); each expert takes its top-C tokens
    (``expert_choice_select``); every expert runs the SwiGLU FFN on its C tokens;
    y[t] = sum over the experts e that took t, in ascending e, of p[t, e] * o_e(t), plus
    the shared expert with weight 1.  The weights are the probabilities themselves (the
    pages give no renormalisation for this routing); a token no expert took outputs 0
    (+ shared).  P_e = mean_t p[t, e] as for token choice; f_e = share of the E*C
    assignments, 1/E.  ``sel_override`` replaces the selection (near-tied columns).
    """
    x = _np(inputs["x"])
    Wr = _np(inputs["W_router"])
    T, d = x.shape
    E = Wr.shape[0]
    p = router_probs(x, Wr)
    C = expert_choice_capacity(T, k, E, capacity_factor)
    sel, margin = expert_choice_select(p, C)
    if sel_override is not None:
        sel = np.asarray(sel_override, np.int32)
    disp = expert_choice_dispatch(sel, T)
    Y = np.zeros((E * C, d), F32)
    for e in range(E):
        if C:
            Y[e * C:(e + 1) * C] = expert_ffn(x[sel[e]], *expert_weights(inputs, e), h_bf16)
    shared = expert_ffn(x, *expert_weights(inputs, E), h_bf16) if n_shared else None
    y = combine(T, d, p, disp["slot"].reshape(-1), Y, shared)
    counts = np.full(E, C, np.int64)
    f = (counts.astype(F64) / float(max(E * C, 1))).astype(F32)
    P = p.astype(F64).mean(axis=0).astype(F32)
    return {"y": y, "f": f, "p": P, "probs": p, "sel": sel, "margin": margin, "C": C,
            "dispatch": disp}


# ----------------------------------------------------------------------------- next best
def next_best_candidates(s: np.ndarray, k: int, idx: np.ndarray | None = None) -> np.ndarray:
    """The experts each token would take after its k chosen ones: its best selection
    scores outside its top-k (descending, ties to the lower expert index), at most k of
    them, -1 where fewer than k experts remain.  With ``idx`` (a given top-k choice) the
    candidates are the best-scored experts outside idx."""
    T, E = s.shape
    s2 = s.astype(F64).copy()
    if idx is None:
        idx = np.argsort(-s2, axis=1, kind="stable")[:, :k]
    np.put_along_axis(s2, np.asarray(idx, np.int64), -np.inf, axis=1)
    order = np.argsort(-s2, axis=1, kind="stable")     # the chosen experts sort last
    cand = np.full((T, k), -1, np.int32)
    m = min(k, E - k)
    cand[:, :m] = order[:, :m]
    return cand


def dispatch_next_best(idx: np.ndarray, cand: np.ndarray, E: int, C: int) -> dict:
    """Capacity overflow handed to the next-best expert instead of dropped.

    [book ch.30] 30.5.2: tokens past an expert's capacity are dropped or redirected to
    the next-best expert.  Reading: one redirect round.  Round 0 is ``dispatch``: each
    expert keeps its first C assignments in row-major (token, slot) order.  Every
    assignment dropped there is offered to its token's next-best expert: the m-th dropped
    slot of token t (in slot order) goes to cand[t, m], the token's (k+1+m)-th best
    expert.  Each expert takes these offers in row-major order while its total stays
    within C; the rest are dropped.  An expert's rows are its round-0 assignments, then the
    redirected ones, each in row-major order.  The slot keeps its mixing weight.

    Returns the fields of ``dispatch`` (counts = the top-k histogram, kept = rows per
    expert) plus expert [T*k]: the expert that processes each assignment (-1 dropped).
    """
    if C is None:
        raise ValueError("redirecting overflow needs a capacity")
    T, k = idx.shape
    d0 = dispatch(idx, E, C)
    flat = idx.reshape(-1).astype(np.int64)
    sp0 = d0["slot_pos"].astype(np.int64)
    kept0 = d0["kept"].astype(np.int64)
    rank0 = np.where(sp0 >= 0, sp0 - d0["offsets"].astype(np.int64)[np.clip(flat, 0, E - 1)], -1)
    dropped = (sp0 < 0).reshape(T, k)
    m = np.cumsum(dropped, axis=1) - dropped                  # earlier dropped slots of t
    cand = np.asarray(cand, np.int64)
    mm = np.minimum(m, cand.shape[1] - 1)
    prop = np.where(dropped & (m < cand.shape[1]), np.take_along_axis(cand, mm, axis=1), -1)
    prop = prop.reshape(-1)
    # stable rank of each offer among the offers to the same expert, row-major order
    offered = np.nonzero(prop >= 0)[0]
    tgt = prop[offered]
    order = np.argsort(tgt, kind="stable")
    pcount = np.bincount(tgt, minlength=E).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(pcount)[:-1]])
    rank1 = np.empty(offered.size, np.int64)
    rank1[order] = np.arange(offered.size) - start[tgt[order]]
    room = C - kept0
    acc = rank1 < room[tgt]
    acc_count = np.bincount(tgt[acc], minlength=E).astype(np.int64)
    kept = kept0 + acc_count
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)
    slot_pos = np.full(T * k, -1, np.int64)
    expert = np.full(T * k, -1, np.int64)
    keep0 = sp0 >= 0
    slot_pos[keep0] = offsets[flat[keep0]] + rank0[keep0]
    expert[keep0] = flat[keep0]
    a_i, a_e = offered[acc], tgt[acc]
    slot_pos[a_i] = offsets[a_e] + kept0[a_e] + rank1[acc]
    expert[a_i] = a_e
    perm_src = np.empty(int(offsets[-1]), np.int64)
    perm_src[slot_pos[slot_pos >= 0]] = np.nonzero(slot_pos >= 0)[0]
    return {
        "counts": d0["counts"], "kept": kept.astype(np.int32),
        "offsets": offsets.astype(np.int32), "perm_src": perm_src.astype(np.int32),
        "slot_pos": slot_pos.astype(np.int32), "expert": expert.astype(np.int32),
        "redirected": int(acc.sum()),
    }
