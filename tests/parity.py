"""Parity checks between the HIP path (through the C ABI) and the CPU oracle.

Bars (stated for this layer): exact expert indices, counts, capacity cut,
permutation and copied rows; layer output y within a max relative error of
2e-2 for bf16 and 1e-4 for fp32 (max |y_gpu - y_ref| / max |y_ref|); aux loss
within 1e-4 relative.  A token whose k-th and (k+1)-th oracle logits differ by
less than 1e-5 is a near tie: both choices are correct, so it is excluded from
the index comparison and reported, and the dispatch is then compared against
the oracle's dispatch of the GPU's own indices.
"""
from __future__ import annotations

import time

import numpy as np

import oracle.moe_oracle as O
from mixture_experts_layer_sum_amd import synth

NEAR_TIE = 1e-5
Y_TOL = {"bf16": 2e-2, "f32": 1e-4}
AUX_TOL = 1e-4


def log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)


class ExpertView:
    """Lazy per-expert float32 values of a weight tensor (for the oracle)."""

    def __init__(self, inp, name):
        self.inp, self.name = inp, name

    def __getitem__(self, e):
        return self.inp.expert_values(self.name, e)


def to_device(inp, device="cuda"):
    import torch

    def t(a):
        if a is None:
            return None
        if inp.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {"hidden": t(inp.hidden), "w_router": t(inp.w_router), "w1": t(inp.w1),
            "w3": t(inp.w3), "w2": t(inp.w2), "w1s": t(inp.w1s), "w3s": t(inp.w3s),
            "w2s": t(inp.w2s),
            "bias": None if inp.bias is None else t(inp.bias.astype(np.float32))}


def run_gpu(inp, dev, bufs=None, overflow="drop"):
    """One forward through the C ABI; returns (host results, buffers)."""
    import torch
    from mixture_experts_layer_sum_amd import moe
    shared = None if inp.n_shared == 0 else (dev["w1s"], dev["w3s"], dev["w2s"])
    b = moe.moe_forward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"], inp.k,
                        inp.capacity_factor, dev["bias"], bufs, overflow=overflow, shared=shared)
    torch.cuda.synchronize()
    return host_results(b), b


def host_results(b):
    import torch

    def h(x):
        if x.dtype == torch.bfloat16:
            return synth.bf16_bits_to_f32(x.view(torch.int16).cpu().numpy().view(np.uint16))
        return x.cpu().numpy()

    A = int(b.offsets[-1].item())
    return {"logits": h(b.logits), "topk_idx": h(b.topk_idx).astype(np.int64),
            "topk_w": h(b.topk_w), "counts": h(b.counts).astype(np.int64),
            "kept": h(b.kept).astype(np.int64), "offsets": h(b.offsets).astype(np.int64),
            "slot_row": h(b.slot_row).astype(np.int64), "perm_src": h(b.perm_src)[:A].astype(np.int64),
            "x_perm": h(b.x_perm[:A]), "y_perm": h(b.y_perm[:A]), "y": h(b.y),
            "aux": float(b.aux.item()), "A": A,
            "y_shared": h(b.y_shared) if getattr(b, "n_shared", 0) else None}


def near_ties(logits32, k):
    """Tokens whose k-th and (k+1)-th largest float32 logits are closer than NEAR_TIE."""
    T, N = logits32.shape
    if k >= N:
        return np.zeros(T, bool)
    s = -np.sort(-logits32.astype(np.float64), axis=1)
    return (s[:, k - 1] - s[:, k]) < NEAR_TIE


def slot_experts(slot_row, offsets):
    """Expert of every slot's row (-1 for dropped slots)."""
    rows = np.asarray(slot_row)
    e = np.searchsorted(np.asarray(offsets), rows, side="right") - 1
    return np.where(rows >= 0, e, -1)


def check(inp, g, sample=None, label="", audit=True, y_tol=None, overflow="drop"):
    """Compare GPU results `g` with the oracle.  Returns a small report dict.

    With overflow="reroute" the dispatch is checked exactly against the
    oracle's re-routing of the GPU's own top-k and fp32 logits, and y on the
    tokens whose slots ended on the same experts as in the oracle's own run
    (a near-tie in a second-round choice can move later admissions).
    """
    T, k, N = inp.T, inp.k, inp.N
    t0 = time.time()
    ref = O.moe_forward(inp.values("hidden"), inp.values("w_router"), ExpertView(inp, "w1"),
                        ExpertView(inp, "w3"), ExpertView(inp, "w2"), k, inp.capacity_factor,
                        inp.bias, tokens=sample, overflow=overflow,
                        shared=None if inp.n_shared == 0 else
                        (inp.values("w1s"), inp.values("w3s"), inp.values("w2s")))
    log(f"{label}: oracle {time.time() - t0:.1f}s")
    L32 = ref["logits"].astype(np.float32)
    # logits: fp32 accumulation vs fp64 -- a loose sanity bar, the decision audit is below
    scale = max(1.0, float(np.abs(ref["logits"]).max()))
    assert np.abs(g["logits"] - ref["logits"]).max() <= 1e-4 * scale, label

    excl = near_ties(L32, k) if audit else np.zeros(T, bool)
    keep = ~excl
    gi, ri = g["topk_idx"], ref["topk_idx"]
    assert gi.shape == ri.shape
    assert ((gi >= 0) & (gi < N)).all(), label
    assert np.array_equal(np.sort(gi[keep], 1), np.sort(ri[keep], 1)), f"{label}: top-k sets differ"
    # slot order where the adjacent selected logits are not near-tied
    sel = np.take_along_axis(L32.astype(np.float64), ri, 1)
    ordered = keep.copy()
    if k > 1:
        ordered &= (np.diff(-sel, axis=1) >= NEAR_TIE).all(1)
    assert np.array_equal(gi[ordered], ri[ordered]), f"{label}: slot order differs"

    # dispatch: exact, against the oracle's dispatch of the GPU's own indices
    counts = O.expert_counts(gi, N)
    C = O.capacity(T, k, N, inp.capacity_factor)
    disp = O.dispatch(gi, N, C) if overflow == "drop" else O.dispatch_reroute(gi, g["logits"], N, C)
    assert np.array_equal(g["counts"], counts), f"{label}: counts"
    assert g["counts"].sum() == T * k
    assert np.array_equal(g["kept"], disp["kept"]), f"{label}: kept"
    assert np.array_equal(g["offsets"], disp["offsets"]), f"{label}: offsets"
    assert np.array_equal(g["slot_row"], disp["slot_row"]), f"{label}: slot_row"
    assert np.array_equal(g["perm_src"], disp["perm_src"]), f"{label}: perm_src"
    if not excl.any() and overflow == "drop":
        assert np.array_equal(gi, ri)
        assert np.array_equal(g["slot_row"], ref["slot_row"])
    same_experts = (slot_experts(g["slot_row"], g["offsets"]) ==
                    slot_experts(ref["slot_row"], ref["offsets"])).all(1)
    # rows of x_perm are exact copies of hidden rows
    hv = inp.values("hidden")
    rows = np.arange(g["A"]) if sample is None else np.unique(
        np.concatenate([g["slot_row"][t][g["slot_row"][t] >= 0] for t in ref["tokens"]] + [[0]]))
    rows = rows[rows < g["A"]]
    assert np.array_equal(g["x_perm"][rows], hv[g["perm_src"][rows]]), f"{label}: x_perm"

    # gate weights
    wok = keep & (g["topk_idx"] == ri).all(1)
    assert np.abs(g["topk_w"][wok] - ref["topk_w"][wok]).max(initial=0) <= 1e-5, f"{label}: topk_w"

    # layer output (on the tokens the oracle evaluated, all of them if sample is None)
    tol = Y_TOL[inp.dtype] if y_tol is None else y_tol
    toks = ref["tokens"]
    yref = ref["y"]
    ygpu = g["y"][toks]
    tok_ok = keep[toks] & (g["topk_idx"][toks] == ri[toks]).all(1) & same_experts[toks]
    den = float(np.abs(yref[tok_ok]).max(initial=0.0))
    err = float(np.abs(ygpu[tok_ok] - yref[tok_ok]).max(initial=0.0))
    rel = err / den if den > 0 else err
    # diagnostic only: elementwise relative error where |y_ref| >= 1e-3 max |y_ref|
    yr_ok, yg_ok = yref[tok_ok], ygpu[tok_ok]
    big = (np.abs(yr_ok) >= 1e-3 * den) & (np.abs(yr_ok) > 0)
    elem = float((np.abs(yg_ok - yr_ok)[big] / np.abs(yr_ok)[big]).max(initial=0.0))
    assert rel <= tol, f"{label}: y max rel err {rel:.3e} > {tol}"
    # tokens with every slot dropped are exactly zero (without shared experts)
    dropped = (g["slot_row"] < 0).all(1)
    if inp.n_shared == 0:
        assert (g["y"][dropped] == 0).all(), f"{label}: dropped tokens not zero"
    else:
        # the shared experts' outputs on the evaluated tokens, summed over experts
        ys = g["y_shared"].sum(0)[toks]
        yr = ref["y_shared"]
        den_s = float(np.abs(yr).max())
        rel_s = float(np.abs(ys - yr).max()) / den_s if den_s > 0 else 0.0
        assert rel_s <= tol, f"{label}: y_shared rel {rel_s:.3e}"
    # y_perm rows the oracle evaluated
    yp_rows = np.where(~np.isnan(ref["y_perm"][:, 0]))[0]
    if yp_rows.size and not excl.any() and same_experts.all():
        yr = ref["y_perm"][yp_rows]
        den_p = float(np.abs(yr).max())
        errp = float(np.abs(g["y_perm"][yp_rows] - yr).max())
        relp = errp / den_p if den_p > 0 else errp
        assert relp <= tol, f"{label}: y_perm rel {relp:.3e}"
    aux_rel = abs(g["aux"] - ref["aux"]) / abs(ref["aux"])
    assert aux_rel <= AUX_TOL, f"{label}: aux {g['aux']} vs {ref['aux']}"
    rep = {"label": label, "excluded_near_ties": int(excl.sum()), "y_rel": rel,
           "y_elem_rel_diag": elem, "tokens_compared": int(tok_ok.sum()), "aux": g["aux"],
           "aux_ref": ref["aux"], "aux_rel": aux_rel, "rows": g["A"], "C": C,
           "dropped_assignments": int((g["slot_row"] < 0).sum()),
           "tokens_on_other_experts": int((~same_experts).sum())}
    log(f"{label}: {rep}")
    return rep
