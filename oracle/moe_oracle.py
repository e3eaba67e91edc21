"""Plain CPU oracle for the forward pass of a top-k routed MoE SwiGLU FFN layer.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code with the HIP path and imports nothing from it.

Everything is computed in float64 from the (bf16-rounded, exactly widened)
input values, except where a floating-point value decides an integer: the
top-k choice is taken on the logits rounded to float32, the precision the
routing kernel holds them in.

Pages cited (no page has a usable title line, so each is named by its address):

* P1  cf-1.com/news/5914943
* P2  hotelren.com/news/5904824
* P3  devpress.csdn.net/awstech/6a91abf42b83d06f0ec71b09.html
* P4  2kiu.com/news/2885792
* P5  hotelren.com/news/3071227

Readings of points the pages leave open (each also listed in the design notes):

* gate weights are a softmax over the k selected logits (P1 §2.1, P5 §4.1);
  P3 §4.1's order (softmax over all N experts, then keep the top k and
  renormalise them) gives the same values;
* ties go to the lower expert index and slot order is (logit desc, index asc)
  (P4 §5.3);
* capacity C = floor((T*k)/N * CF) with the operation order of P4 §3.1's
  formula; CF <= 0 means "no limit" (C = T);
* the first C tokens in token order keep their place at an expert (P4 §3.1);
  a dropped assignment contributes nothing and the surviving weights are not
  renormalised, so a fully dropped token has y = 0 and only the caller's
  residual carries it (P1 §2.3 tip);
* the expert FFN is SwiGLU, FFN(x) = (silu(x W1) * (x W3)) W2 with
  silu(z) = z / (1 + exp(-z)), W1 being the gated branch, no biases (P4 §2.2
  names SwiGLU; the formula is the standard GLU-variant one);
* aux = N * sum_e f_e * P_e with f_e = counts_e / (T*k) from the router's
  pre-drop assignments and P_e the mean over tokens of the full-N softmax of
  the logits (P1 §2.3, P2 §3.2); the 0.01-style coefficient is the caller's;
* overflow re-routing (the alternative to dropping that P3 §2.3, P4 §2.2 and
  P5 §2.2 mention, and P5 §4.2's capacity-aware routing sketches in code by
  masking the full expert and taking the next-best one): one second dispatch round after the
  capacity cut.  Each dropped assignment, in slot order within its token,
  proposes the highest-logit expert that is not among the token's top-k picks,
  not already proposed by an earlier dropped slot of the same token, and still
  had room after the first round (kept_e < C); ties go to the lower index.
  Proposals are admitted per expert in token order up to the room left
  (C - kept_e); the rest are dropped.  A re-routed assignment keeps its gate
  weight.  Inside an expert, first-round rows come before second-round rows,
  each token-ascending.  Counts and the aux loss stay on the router's own
  (pre-drop) assignments;
* shared experts (P2 §3.3: experts every token calls unconditionally, next to
  the routed ones): each is a SwiGLU FFN of its own applied to every token,
  dropped or not, and added to the routed sum with weight 1;
* FP8 expert weights (P1 §3.1: the experts are stored in FP8): each expert
  matrix is quantised per output column to OCP FP8 E4M3 (1 sign, 4 exponent
  bits with bias 7, 3 mantissa bits, subnormals, largest finite 448, no
  infinity): scale = amax / 448 over the column (1 for an all-zero column),
  code = round-to-nearest-even of w / scale, clamped to +-448, both divisions
  in float32; the layer then runs on code * scale;
* backward pass (the training step the aux loss exists for: P1 §2.3, P2 §3.2;
  every expert keeps gradients of its own: P4 §2.2; only the selected experts
  receive any: P4 §5.1): gradients of L = <dy, y> + aux_coef * aux with respect to hidden,
  W_router, bias, W1, W3, W2.  The top-k choice, the capacity cut and the
  counts f_e are piecewise constant (no gradient); gradients reach the router
  through the softmax over the k selected logits and through P_e in the aux
  loss.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "router_logits", "select_topk", "gate_weights", "expert_counts", "capacity",
    "dispatch", "dispatch_reroute", "silu", "swiglu_ffn", "aux_loss", "moe_forward",
    "moe_forward_per_token", "e4m3_decode", "e4m3_encode", "quantize_fp8_columns",
    "dequantize_fp8_columns", "swiglu_backward", "moe_backward", "moe_backward_sampled",
]


def router_logits(hidden, w_router, bias=None) -> np.ndarray:
    """Router linear layer: logits[t, e] = sum_i hidden[t, i] * W_router[i, e] (+ bias[e]).

    P1 §2.1 (router scores every expert with one small linear layer, W_router
    [hidden_dim, num_experts]); P4 §3.1 (the router contracts the hidden dimension with W_router); optional
    bias per P3 §4.1 (nn.Linear with bias) and P4 §5.2 (per-expert offset).
    """
    L = np.asarray(hidden, np.float64) @ np.asarray(w_router, np.float64)
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def select_topk(logits, k: int) -> np.ndarray:
    """Indices [T, k] of the k largest logits per token, in slot order.

    P1 §2.1 / §2.2 (top-k experts by router score, k = 2 typical); P4 §5.3
    (equal logits are ranked by ascending expert id).  The decision is made on
    the float32-rounded logits.
    """
    L32 = np.asarray(logits).astype(np.float32)
    T, N = L32.shape
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= N")
    ids = np.broadcast_to(np.arange(N), (T, N))
    order = np.lexsort((ids, -L32.astype(np.float64)), axis=-1)   # primary: -logit, then id
    return order[:, :k].astype(np.int64)


def gate_weights(logits, idx) -> np.ndarray:
    """Softmax over the k selected logits of each token (P1 §2.1 code; P5 §4.1)."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), idx, axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


def expert_counts(idx, N: int) -> np.ndarray:
    """Tokens assigned to each expert before any capacity drop (P1 §2.3)."""
    return np.bincount(np.asarray(idx).ravel(), minlength=N).astype(np.int64)


def capacity(T: int, k: int, N: int, capacity_factor: float) -> int:
    """Expert capacity C = floor((T*k)/N * CF) (P4 §3.1; worked example P5 §2.2).

    CF <= 0 stands for "no capacity limit": C = T, which no expert can exceed
    since a token never picks the same expert twice.
    """
    if capacity_factor is None or capacity_factor <= 0:
        return int(T)
    return int(math.floor((T * k) / N * float(capacity_factor)))


def dispatch(idx, N: int, C: int) -> dict:
    """Per-expert queues after the capacity cut.

    Tokens are visited in order t = 0..T-1; at each selected expert the token
    takes the next place, and it keeps its place only if fewer than C tokens
    came before it (P4 §3.1 "keep the first capacity tokens per expert").
    Kept rows are laid out expert-major, token-ascending inside an expert.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    place = np.empty((T, k), np.int64)
    running = np.zeros(N, np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            place[t, j] = running[e]
            running[e] += 1
    keep = place < C
    kept = np.array([min(int(running[e]), C) for e in range(N)], np.int64)
    offsets = np.zeros(N + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    slot_row = np.where(keep, offsets[idx] + place, -1)
    perm_src = np.empty(int(offsets[-1]), np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                perm_src[slot_row[t, j]] = t
    return {"place": place, "keep": keep, "kept": kept, "offsets": offsets,
            "slot_row": slot_row, "perm_src": perm_src}


def dispatch_reroute(idx, logits, N: int, C: int) -> dict:
    """Capacity cut, then one re-routing round for the dropped assignments.

    First round exactly as :func:`dispatch`.  Second round: every dropped
    (t, j), in token order and slot order inside a token, proposes the best
    expert by the float32 logits (larger first, lower index on ties) among
    those that are not in token t's top-k, not proposed by an earlier dropped
    slot of t, and had kept_e < C after the first round.  Each expert admits
    proposals in token order while it has room left (C - kept_e).  P5 §4.2
    (capacity-aware routing: mask the original pick, take the next best), P4
    §2.2 and P5 §2.2 (over-capacity tokens are dropped or sent to the
    next-best expert), P3 §2.3 (overflow is handed to other, idle experts).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    L32 = np.asarray(logits, np.float64).astype(np.float32)
    first = dispatch(idx, N, C)
    keep1, kept1 = first["keep"], first["kept"]
    room = kept1 < C
    prop = np.full((T, k), -1, np.int64)
    for t in range(T):
        taken = set(int(e) for e in idx[t])
        for j in range(k):
            if keep1[t, j]:
                continue
            best = -1
            for e in range(N):
                if e in taken or not room[e]:
                    continue
                if best < 0 or L32[t, e] > L32[t, best]:
                    best = e
            if best >= 0:
                prop[t, j] = best
                taken.add(best)
    # admission, per expert in token order
    place2 = np.full((T, k), -1, np.int64)
    used = np.zeros(N, np.int64)
    for t in range(T):
        for j in range(k):
            e = prop[t, j]
            if e >= 0:
                place2[t, j] = used[e]
                used[e] += 1
    keep2 = (prop >= 0) & (place2 < (C - kept1)[np.maximum(prop, 0)])
    kept2 = np.array([min(int(used[e]), C - int(kept1[e])) for e in range(N)], np.int64)
    kept = kept1 + kept2
    offsets = np.zeros(N + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    expert = np.where(keep1, idx, np.where(keep2, prop, -1))
    slot_row = np.full((T, k), -1, np.int64)
    slot_row[keep1] = (offsets[idx] + first["place"])[keep1]
    e2 = np.maximum(prop, 0)
    slot_row[keep2] = (offsets[e2] + kept1[e2] + place2)[keep2]
    perm_src = np.empty(int(offsets[-1]), np.int64)
    for t in range(T):
        for j in range(k):
            if slot_row[t, j] >= 0:
                perm_src[slot_row[t, j]] = t
    return {"keep1": keep1, "proposal": prop, "keep2": keep2, "kept1": kept1, "kept": kept,
            "offsets": offsets, "slot_row": slot_row, "perm_src": perm_src, "expert": expert}


def e4m3_decode(code):
    """Value of OCP FP8 E4M3 codes (uint8 array): (-1)^s 2^(E-7) (1 + M/8), subnormal
    2^-6 M/8 for E = 0, NaN for E = 15, M = 7."""
    c = np.asarray(code, np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 15
    M = c & 7
    v = np.where(E == 0, M / 8.0 * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    v = np.where((E == 15) & (M == 7), np.nan, v)
    return s * v


def e4m3_encode(x):
    """Nearest OCP FP8 E4M3 code of float values with |x| <= 448 (ties to the even
    mantissa).  Written from the format: the spacing of representable values is
    2^(e-3) in binade [2^e, 2^(e+1)) for e >= -6, and 2^-9 below 2^-6."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > 448) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode expects finite values within +-448")
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    n = a / quantum                       # exact: a power-of-two rescale
    r = np.floor(n)
    frac = n - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (r % 2 == 1)), r + 1, r)
    q = r * quantum                       # the rounded magnitude (may step into the next binade)
    # encode q: subnormal when q < 2^-6
    code = np.zeros(x.shape, np.int64)
    sub = q < 2.0 ** -6
    code = np.where(sub, np.round(q / 2.0 ** -9).astype(np.int64), code)
    with np.errstate(divide="ignore"):
        eq = np.floor(np.log2(np.where(sub, 1.0, q)))
    mant = np.where(sub, 0, np.round((q / np.exp2(eq) - 1.0) * 8.0)).astype(np.int64)
    code = np.where(sub, code, ((eq + 7).astype(np.int64) << 3) | mant)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_fp8_columns(w):
    """Per-column FP8 quantisation of one expert matrix w [K, M] (float32 values).

    scale[m] = amax_k |w[k, m]| / 448 in float32 (1 for an all-zero column);
    code[k, m] = e4m3_encode(clamp(float32(w[k, m] / scale[m]), -448, 448)).
    P1 §3.1 (expert weights stored in FP8 to save memory and bandwidth).
    """
    w = np.asarray(w, np.float32)
    amax = np.abs(w).max(axis=0)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = (w / scale[None, :]).astype(np.float32)
    r = np.clip(r, np.float32(-448.0), np.float32(448.0))
    return e4m3_encode(r), scale


def dequantize_fp8_columns(code, scale):
    """The weights the FP8 layer computes with: code value * column scale (float64)."""
    return e4m3_decode(code) * np.asarray(scale, np.float64)[None, :]


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(x, w1, w3, w2) -> np.ndarray:
    """One expert: (silu(x W1) * (x W3)) W2 (P4 §2.2 names SwiGLU experts)."""
    x = np.asarray(x, np.float64)
    h1 = x @ np.asarray(w1, np.float64)
    h3 = x @ np.asarray(w3, np.float64)
    return (silu(h1) * h3) @ np.asarray(w2, np.float64)


def aux_loss(logits, counts, k: int) -> float:
    """Load-balancing loss N * sum_e f_e * P_e (P1 §2.3; P2 §3.2).

    P_e: mean over tokens of the softmax over all N logits.  f_e: share of
    the T*k router assignments that went to expert e, before capacity drop,
    so that sum_e f_e = 1 and a uniform router scores exactly 1.
    """
    L = np.asarray(logits, np.float64)
    T, N = L.shape
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    probs = ex / ex.sum(axis=1, keepdims=True)
    P = probs.mean(axis=0)
    f = np.asarray(counts, np.float64) / float(T * k)
    return float(N * np.sum(f * P))


def moe_forward(hidden, w_router, w1, w3, w2, k: int, capacity_factor: float = 0.0,
                bias=None, tokens=None, overflow: str = "drop", shared=None) -> dict:
    """The layer forward, per expert (the page's gather -> FFN -> weighted add loop).

    ``w1[e]``, ``w3[e]``, ``w2[e]`` are indexed one expert at a time, so the
    caller may hand in lazy per-expert views.  If ``tokens`` is given, routing,
    counts, dispatch and aux cover every token but the expert FFN and the
    combine are evaluated only for those tokens (``y`` then has one row per
    listed token).  ``overflow`` is "drop" (the default) or "reroute"
    (:func:`dispatch_reroute`).  ``shared`` is None or ``(w1s, w3s, w2s)``
    indexable by shared expert: y_t += sum_s FFN_s(x_t) (P2 §3.3).

    P1 §2.1 (route, top-k, softmax, weighted sum), P3 §4.1 (per-expert loop;
    its shortcut that weights every expert by the sum of both gate values is
    not reproduced), P1 §2.3 (aux, capacity).
    """
    hidden = np.asarray(hidden)
    T, d = hidden.shape
    L = router_logits(hidden, w_router, bias)
    N = L.shape[1]
    idx = select_topk(L, k)
    w = gate_weights(L, idx)
    counts = expert_counts(idx, N)
    C = capacity(T, k, N, capacity_factor)
    if overflow == "drop":
        disp = dispatch(idx, N, C)
    elif overflow == "reroute":
        disp = dispatch_reroute(idx, L, N, C)
    else:
        raise ValueError(f"unknown overflow policy {overflow!r}")
    slot_row, offsets, perm_src = disp["slot_row"], disp["offsets"], disp["perm_src"]

    tok = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    want = np.zeros(T, bool)
    want[tok] = True
    A = int(offsets[-1])
    y_perm = np.full((A, d), np.nan)
    for e in range(N):
        rows = np.arange(offsets[e], offsets[e + 1])
        rows = rows[want[perm_src[rows]]]
        if rows.size == 0:
            continue
        y_perm[rows] = swiglu_ffn(hidden[perm_src[rows]], w1[e], w3[e], w2[e])
    y = np.zeros((tok.size, d))
    for n, t in enumerate(tok):
        for j in range(k):
            r = slot_row[t, j]
            if r >= 0:
                y[n] += w[t, j] * y_perm[r]
    y_shared = None
    if shared is not None:
        w1s, w3s, w2s = shared
        y_shared = np.zeros((tok.size, d))
        for q in range(len(w1s)):
            y_shared += swiglu_ffn(hidden[tok], w1s[q], w3s[q], w2s[q])
        y = y + y_shared
    return {"y_shared": y_shared, "logits": L, "topk_idx": idx, "topk_w": w, "counts": counts, "capacity": C,
            "kept": disp["kept"], "offsets": offsets, "slot_row": slot_row, "perm_src": perm_src,
            "y_perm": y_perm, "y": y, "tokens": tok, "aux": aux_loss(L, counts, k)}


def moe_forward_per_token(hidden, w_router, w1, w3, w2, k: int, capacity_factor: float = 0.0,
                          bias=None, overflow: str = "drop", shared=None) -> np.ndarray:
    """Brute force for tiny inputs: y_t = sum over kept slots j of w_tj * FFN_{i_tj}(x_t).

    One token and one slot at a time, with its own running per-expert counter
    for the capacity cut; no permutation, no grouping.  With
    overflow="reroute" a second pass walks the dropped slots in token order,
    each scanning the experts in logit order for one that is not the token's
    and had room after the first pass, and keeps it while that expert's
    second-pass count stays within its room.
    """
    hidden = np.asarray(hidden, np.float64)
    T, d = hidden.shape
    L = router_logits(hidden, w_router, bias)
    N = L.shape[1]
    idx = select_topk(L, k)
    w = gate_weights(L, idx)
    C = capacity(T, k, N, capacity_factor)
    seen = [0] * N
    y = np.zeros((T, d))
    dropped = []
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if seen[e] < C:
                y[t] += w[t, j] * swiglu_ffn(hidden[t:t + 1], w1[e], w3[e], w2[e])[0]
            else:
                dropped.append((t, j))
            seen[e] += 1
    if overflow == "reroute":
        full = [min(c, C) for c in seen]            # rows each expert kept in the first pass
        second = [0] * N
        L32 = L.astype(np.float32)
        chosen = {}
        for t, j in dropped:
            mine = set(int(e) for e in idx[t]) | chosen.setdefault(t, set())
            order = sorted(range(N), key=lambda e: (-float(L32[t, e]), e))
            cand = next((e for e in order if e not in mine and full[e] < C), None)
            if cand is None:
                continue
            chosen[t].add(cand)
            if second[cand] < C - full[cand]:
                y[t] += w[t, j] * swiglu_ffn(hidden[t:t + 1], w1[cand], w3[cand], w2[cand])[0]
            second[cand] += 1
    elif overflow != "drop":
        raise ValueError(f"unknown overflow policy {overflow!r}")
    if shared is not None:
        w1s, w3s, w2s = shared
        for t in range(T):
            for q in range(len(w1s)):
                y[t] += swiglu_ffn(hidden[t:t + 1], w1s[q], w3s[q], w2s[q])[0]
    return y


def swiglu_backward(X, G, W1, W3, W2, cols=None) -> dict:
    """One expert's SwiGLU FFN backward for rows X [n, d] whose output gradient is G [n, d].

    h1 = X W1, h3 = X W3, s = sigmoid(h1), a = h1 s h3 (= silu(h1) * h3), y = a W2;
    da = G W2^T;  dh3 = da * h1 s;  dh1 = da * h3 * (s + h1 s (1 - s))  (silu'(z) = s + z s (1 - s));
    dW1 = X^T dh1, dW3 = X^T dh3, dW2 = a^T G, dX = dh1 W1^T + dh3 W3^T.
    With ``cols`` (indices into f) only dW1[:, cols], dW3[:, cols] and dW2[cols, :] are
    formed: every step above is local to a column of f, so they equal the same entries of
    the full result.  Without ``cols`` dX and y are returned as well.
    """
    X = np.asarray(X, np.float64)
    G = np.asarray(G, np.float64)
    c = slice(None) if cols is None else np.asarray(cols)
    W1c = np.asarray(np.asarray(W1)[:, c], np.float64)
    W3c = np.asarray(np.asarray(W3)[:, c], np.float64)
    W2c = np.asarray(np.asarray(W2)[c, :], np.float64)
    h1, h3 = X @ W1c, X @ W3c
    s = 1.0 / (1.0 + np.exp(-h1))
    a = h1 * s * h3
    da = G @ W2c.T
    dh3 = da * (h1 * s)
    dh1 = da * h3 * (s + h1 * s * (1.0 - s))
    out = {"dw1": X.T @ dh1, "dw3": X.T @ dh3, "dw2": a.T @ G}
    if cols is None:
        out["dx"] = dh1 @ W1c.T + dh3 @ W3c.T
        out["y"] = a @ W2c
    return out


def _routing(hidden, w_router, k, capacity_factor, bias, overflow):
    L = router_logits(hidden, w_router, bias)
    T, N = L.shape
    idx = select_topk(L, k)
    w = gate_weights(L, idx)
    counts = expert_counts(idx, N)
    C = capacity(T, k, N, capacity_factor)
    if overflow == "drop":
        disp = dispatch(idx, N, C)
    elif overflow == "reroute":
        disp = dispatch_reroute(idx, L, N, C)
    else:
        raise ValueError(f"unknown overflow policy {overflow!r}")
    slot_row, offsets = disp["slot_row"], disp["offsets"]
    A = int(offsets[-1])
    row_tok = np.empty(A, np.int64)
    row_j = np.empty(A, np.int64)
    for t in range(T):
        for j in range(k):
            r = slot_row[t, j]
            if r >= 0:
                row_tok[r], row_j[r] = t, j
    return {"L": L, "idx": idx, "w": w, "counts": counts, "slot_row": slot_row,
            "offsets": offsets, "row_tok": row_tok, "row_j": row_j, "N": N, "T": T}


def _dlogits(L, idx, w, dgate, counts, T, k, aux_coef):
    """Logit gradient of the rows given: softmax over the k selected logits, plus
    aux_coef times d aux / d logits = (N / T) p (f - sum_m p_m f_m), p = softmax of all N."""
    n, N = L.shape
    dlog = np.zeros((n, N))
    inner = np.sum(w * dgate, axis=1, keepdims=True)
    np.put_along_axis(dlog, idx, w * (dgate - inner), axis=1)
    if aux_coef != 0.0:
        p = np.exp(L - L.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        fe = counts.astype(np.float64) / float(T * k)
        dlog += aux_coef * (N / T) * p * (fe[None, :] - np.sum(p * fe[None, :], axis=1, keepdims=True))
    return dlog


def moe_backward(hidden, w_router, w1, w3, w2, k: int, dy, capacity_factor: float = 0.0,
                 bias=None, aux_coef: float = 0.0, overflow: str = "drop", shared=None) -> dict:
    """Gradients of L = sum(dy * y) + aux_coef * aux (float64, from the definitions).

    Per kept slot (t, j) at expert e with gate weight w: g = w * dy[t] is the gradient
    reaching the expert's output (:func:`swiglu_backward` for the expert's rows gives
    dW1_e, dW3_e, dW2_e and each row's dX), and dgate[t, j] = <dy[t], FFN_e(x_t)>.
    Softmax over the selected logits: dlogit[t, i_j] = w_j (dgate_j - sum_m w_m dgate_m).
    Aux loss: d aux / d logits[t, e] = (N / T) p_te (f_e - sum_m p_tm f_m), p = full softmax.
    Router: dW_router = hidden^T dlogits, dbias = sum_t dlogits,
    dhidden[t] = sum of its slots' dX rows + dlogits[t] W_router^T.
    Shared experts (``shared`` = (w1s, w3s, w2s), P2 §3.3, weight 1 on every token):
    :func:`swiglu_backward` over all T rows with g = dy gives dw1s/dw3s/dw2s, and
    their dX rows are added to dhidden.
    """
    hidden = np.asarray(hidden, np.float64)
    T, d = hidden.shape
    dy = np.asarray(dy, np.float64)
    Wr = np.asarray(w_router, np.float64)
    R = _routing(hidden, w_router, k, capacity_factor, bias, overflow)
    N, offsets = R["N"], R["offsets"]
    f = np.asarray(w1[0]).shape[1]
    dW1 = np.zeros((N, d, f))
    dW3 = np.zeros((N, d, f))
    dW2 = np.zeros((N, f, d))
    dhidden = np.zeros((T, d))
    dgate = np.zeros((T, k))
    for e in range(N):
        rows = np.arange(offsets[e], offsets[e + 1])
        if rows.size == 0:
            continue
        tok, slot = R["row_tok"][rows], R["row_j"][rows]
        G = R["w"][tok, slot][:, None] * dy[tok]
        out = swiglu_backward(hidden[tok], G, w1[e], w3[e], w2[e])
        dgate[tok, slot] = np.sum(dy[tok] * out["y"], axis=1)
        dW1[e], dW3[e], dW2[e] = out["dw1"], out["dw3"], out["dw2"]
        np.add.at(dhidden, tok, out["dx"])
    dlog = _dlogits(R["L"], R["idx"], R["w"], dgate, R["counts"], T, k, aux_coef)
    dW_router = hidden.T @ dlog
    dbias = dlog.sum(axis=0)
    dhidden += dlog @ Wr.T
    res = {"dhidden": dhidden, "dw_router": dW_router, "dbias": dbias, "dw1": dW1, "dw3": dW3,
           "dw2": dW2, "dgate": dgate, "dlogits": dlog, "topk_idx": R["idx"],
           "slot_row": R["slot_row"], "offsets": offsets}
    if shared is not None:
        w1s, w3s, w2s = shared
        outs = [swiglu_backward(hidden, dy, w1s[q], w3s[q], w2s[q]) for q in range(len(w1s))]
        for o in outs:
            dhidden += o["dx"]
        res["dw1s"] = np.stack([o["dw1"] for o in outs])
        res["dw3s"] = np.stack([o["dw3"] for o in outs])
        res["dw2s"] = np.stack([o["dw2"] for o in outs])
    return res


def moe_backward_sampled(hidden, w_router, w1, w3, w2, k: int, dy, capacity_factor: float = 0.0,
                         bias=None, aux_coef: float = 0.0, overflow: str = "drop", tokens=(),
                         expert_cols=(), router: bool = False) -> dict:
    """Entries of :func:`moe_backward` at sizes where the whole is too slow on a CPU.

    Routing, counts and dispatch cover every token (they are cheap); then
    * ``dhidden[t]`` for each t in ``tokens``: only the token's own slots are run
      (dX and dgate are local to a row), plus its logit gradient;
    * for each ``(e, cols)`` in ``expert_cols``: dW1_e[:, cols], dW3_e[:, cols] and
      dW2_e[cols, :] over all of expert e's rows (local to a column of f);
    * with ``router``: dW_router and dbias in full.  They need every token's logit
      gradient, hence every kept slot's dgate = <dy[t], FFN_e(x_t)>: one forward of
      the experts over their rows (no expert backward).
    Returns {"dhidden": {t: [d]}, "dw": {(e, tuple(cols)): (dW1 cols, dW3 cols, dW2 rows)},
    "topk_idx", "slot_row", "offsets"} (+ "dw_router", "dbias", "dgate" with ``router``).
    """
    hidden = np.asarray(hidden)
    T, d = hidden.shape
    dy = np.asarray(dy)
    R = _routing(hidden, w_router, k, capacity_factor, bias, overflow)
    offsets = R["offsets"]
    Wr = np.asarray(w_router, np.float64)
    res = {"dhidden": {}, "dw": {}, "topk_idx": R["idx"], "slot_row": R["slot_row"],
           "offsets": offsets}
    for t in tokens:
        x = np.asarray(hidden[t], np.float64)[None]
        g_dy = np.asarray(dy[t], np.float64)
        acc = np.zeros(d)
        dg = np.zeros((1, k))
        for j in range(k):
            r = R["slot_row"][t, j]
            if r < 0:
                continue
            e = int(np.searchsorted(offsets, r, side="right") - 1)
            out = swiglu_backward(x, R["w"][t, j] * g_dy[None], w1[e], w3[e], w2[e])
            acc += out["dx"][0]
            dg[0, j] = float(g_dy @ out["y"][0])
        dl = _dlogits(R["L"][t:t + 1], R["idx"][t:t + 1], R["w"][t:t + 1], dg, R["counts"], T, k,
                      aux_coef)
        res["dhidden"][int(t)] = acc + (dl @ Wr.T)[0]
    for e, cols in expert_cols:
        rows = np.arange(offsets[e], offsets[e + 1])
        tok, slot = R["row_tok"][rows], R["row_j"][rows]
        G = R["w"][tok, slot][:, None] * np.asarray(dy[tok], np.float64)
        out = swiglu_backward(np.asarray(hidden[tok], np.float64), G, w1[e], w3[e], w2[e], cols)
        res["dw"][(int(e), tuple(int(c) for c in cols))] = (out["dw1"], out["dw3"], out["dw2"])
    if router:
        dgate = np.zeros((T, k))
        for e in range(R["N"]):
            rows = np.arange(offsets[e], offsets[e + 1])
            if rows.size == 0:
                continue
            tok, slot = R["row_tok"][rows], R["row_j"][rows]
            ye = swiglu_ffn(hidden[tok], w1[e], w3[e], w2[e])
            dgate[tok, slot] = np.sum(np.asarray(dy[tok], np.float64) * ye, axis=1)
        dlog = _dlogits(R["L"], R["idx"], R["w"], dgate, R["counts"], T, k, aux_coef)
        res["dw_router"] = np.asarray(hidden, np.float64).T @ dlog
        res["dbias"] = dlog.sum(axis=0)
        res["dgate"] = dgate
    return res
