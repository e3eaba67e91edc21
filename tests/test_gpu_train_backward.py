"""GPU parity of the backward pass: the HIP path through the C ABI against the
oracle's gradients (oracle.moe_backward, fp64).

Bar: for every gradient tensor, max |gpu - oracle| / max |oracle| <= 2e-2 for
bf16 layers (the HIP path rounds g = w dy, dh1, dh3 and a to bf16 before the
GEMMs that consume them, as the forward rounds its activations) and <= 1e-4 for
fp32 layers; experts that receive no rows get weight gradients that are exactly
zero; the routing the gradients are taken at is compared exactly first.
"""
import numpy as np
import pytest

from mixture_experts_layer_sum_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRAD_TOL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from mixture_experts_layer_sum_amd import moe as m   # raises if the library is missing
    return m


def _dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel(gpu, ref):
    den = float(np.abs(ref).max(initial=0.0))
    err = float(np.abs(gpu - ref).max(initial=0.0))
    return err / den if den > 0 else err


def _forward(moe, inp, dev, overflow, saved):
    from tests import parity
    sh = (dev["w1s"], dev["w3s"], dev["w2s"]) if inp.n_shared else None
    b = moe.moe_forward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"], inp.k,
                        inp.capacity_factor, dev["bias"], overflow=overflow, shared=sh,
                        save_for_backward=saved)
    torch.cuda.synchronize()
    return parity.host_results(b), b


def run_backward(moe, inp, coef, overflow="drop", label="",
                 modes=("recompute", "saved", "saved_recompute_act")):
    """The expert-backward paths against one oracle backward: h1 / h3 recomputed; saved
    by the forward, with dW2 from the forward's activations; saved, with the activations
    recomputed from h1 / h3 (moe_expert_backward_saved with act = NULL)."""
    import oracle.moe_oracle as O
    from tests import parity
    parity.log(f"{label}: T={inp.T} d={inp.d} N={inp.N} k={inp.k} f={inp.f} {inp.dtype} "
               f"cf={inp.capacity_factor} aux_coef={coef} overflow={overflow}")
    dev = parity.to_device(inp)
    dy = synth.make_dy(inp.T, inp.d, inp.dtype, seed=11)
    sh = (dev["w1s"], dev["w3s"], dev["w2s"]) if inp.n_shared else None
    dyv = synth.bf16_bits_to_f32(dy) if inp.dtype == "bf16" else dy
    ref = None
    reps = {}
    for mode in modes:
        g, b = _forward(moe, inp, dev, overflow, mode.startswith("saved"))
        if mode == "saved_recompute_act":
            b.act = None        # moe_backward then passes no activations
        gr = moe.moe_backward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"],
                              _dev(dy, inp.dtype), b, coef, want_dbias=inp.bias is not None,
                              shared=sh)
        torch.cuda.synchronize()
        if ref is None:
            ref = O.moe_backward(inp.values("hidden"), inp.values("w_router"),
                                 parity.ExpertView(inp, "w1"), parity.ExpertView(inp, "w3"),
                                 parity.ExpertView(inp, "w2"), inp.k, dyv, inp.capacity_factor,
                                 inp.bias, aux_coef=coef, overflow=overflow,
                                 shared=(inp.values("w1s"), inp.values("w3s"), inp.values("w2s"))
                                 if inp.n_shared else None)
        reps[mode] = _compare(inp, g, gr, ref, f"{label}/{mode}")
    return reps


def _compare(inp, g, gr, ref, label):
    from tests import parity
    # the gradients are taken at one routing: it must be the oracle's
    assert np.array_equal(g["topk_idx"], ref["topk_idx"]), f"{label}: routing differs"
    assert np.array_equal(g["slot_row"], ref["slot_row"]), f"{label}: dispatch differs"
    tol = GRAD_TOL[inp.dtype]
    host = {"dhidden": gr.dhidden, "dw_router": gr.dw_router, "dw1": gr.dw1, "dw3": gr.dw3,
            "dw2": gr.dw2, "dgate": gr.dgate}
    if inp.bias is not None:
        host["dbias"] = gr.dbias
    if inp.n_shared:
        host.update({"dw1s": gr.dw1s, "dw3s": gr.dw3s, "dw2s": gr.dw2s})
    rep = {}
    for name, t in host.items():
        got = t.cpu().numpy().astype(np.float64)
        rel = _rel(got, ref[name])
        rep[name] = rel
        assert rel <= tol, f"{label}: {name} max rel err {rel:.3e} > {tol}"
    # experts with no rows: weight gradients exactly zero
    empty = np.where(np.diff(g["offsets"]) == 0)[0]
    for e in empty:
        for name in ("dw1", "dw3", "dw2"):
            assert (host[name][e] == 0).all().item(), f"{label}: {name}[{e}] of an empty expert"
    parity.log(f"{label}: rel errors {rep}; empty experts {empty.tolist()}")
    return rep


SMALL = [
    # label, T, d, N, k, f, dtype, cf, bias, aux_coef, overflow
    ("f32_tiny", 64, 128, 8, 2, 192, "f32", 0.0, None, 0.0, "drop"),
    ("f32_drop_aux", 300, 128, 8, 2, 128, "f32", 1.0, "skew", 0.01, "drop"),
    ("f32_k1", 77, 64, 4, 1, 64, "f32", 0.0, None, 0.5, "drop"),
    ("bf16_ragged", 300, 256, 4, 2, 512, "bf16", 0.0, None, 0.0, "drop"),
    ("bf16_drop_aux_bias", 1000, 512, 8, 2, 256, "bf16", 1.0, "skew", 0.01, "drop"),
    ("bf16_empty_experts", 200, 256, 16, 2, 256, "bf16", 0.0, "hot", 0.1, "drop"),
    ("bf16_reroute", 600, 256, 8, 2, 256, "bf16", 0.8, "skew", 0.01, "reroute"),
    ("bf16_multi_tile_rows", 1500, 256, 2, 2, 256, "bf16", 0.0, None, 0.0, "drop"),
    # edge shapes: k = 4, N not a multiple of 8 with k = 3, one token, N = 64 and 256 (most
    # experts empty), k = N (dense softmax), f = 3 * 256
    ("bf16_k4_N16", 200, 256, 16, 4, 256, "bf16", 0.0, None, 0.05, "drop"),
    ("bf16_N12_k3_cap", 130, 256, 12, 3, 256, "bf16", 0.8, None, 0.01, "drop"),
    ("bf16_single_token", 1, 256, 8, 2, 256, "bf16", 0.0, None, 0.01, "drop"),
    ("bf16_N64_sparse", 100, 256, 64, 2, 256, "bf16", 0.0, None, 0.01, "drop"),
    ("bf16_N256", 70, 256, 256, 2, 256, "bf16", 0.0, None, 0.01, "drop"),
    ("f32_k_eq_N", 40, 64, 4, 4, 64, "f32", 0.0, None, 0.1, "drop"),
    ("bf16_d512_f768", 300, 512, 8, 2, 768, "bf16", 1.25, None, 0.01, "drop"),
    # f = 4096: the dx GEMM is 2f = 8192 deep (128 k-steps) and its 4 tiles fill a few of
    # the CUs, so each tile is split over k into 4 ranges whose partials meet in the
    # workspace
    ("bf16_dx_ksplit", 300, 256, 2, 2, 4096, "bf16", 0.0, None, 0.01, "drop"),
    # shared experts: every token, weight 1; two of them, and one with all routed slots dropped
    ("f32_two_shared", 100, 128, 8, 2, 128, "f32", 1.0, None, 0.01, "drop", 2, 64),
    ("bf16_shared", 400, 256, 8, 2, 256, "bf16", 1.0, "skew", 0.01, "drop", 1, 512),
    ("bf16_shared_all_dropped", 64, 256, 8, 2, 256, "bf16", 0.01, "skew", 0.0, "drop", 1, 256),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_small(moe, case):
    label, T, d, N, k, f, dt, cf, bias, coef, overflow = case[:11]
    ns, fs = case[11:] if len(case) > 11 else (0, None)
    b = None
    if bias == "skew":
        b = np.zeros(N, np.float32)
        b[:3] = [1.5, 1.0, 0.5]
    elif bias == "hot":
        b = np.full(N, -4.0, np.float32)
        b[:4] = 2.0                        # experts 4.. get (almost) nothing
    inp = synth.make_inputs(T, d, N, k, f, dt, cf, 0, bias=b, n_shared=ns, f_shared=fs)
    run_backward(moe, inp, coef, overflow, label)


def _random_configs(n=12, seed=20261204):
    """Seeded draws across the backward's limits (bf16: d a multiple of 256 and f of
    256; fp32: multiples of 64): 1 to 64 experts, k up to 4 (k = N included), token
    counts that are no multiple of a tile, both overflow policies, with and without
    the aux term and a router bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "bf16" if rng.random() < 0.7 else "f32"
        N = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 64]))
        if dt == "bf16":
            d = int(rng.choice([256, 512]))
            f = int(rng.choice([256, 512])) if N <= 16 else 256
        else:
            d = int(rng.choice([64, 128, 192]))
            f = int(rng.choice([64, 128, 192])) if N <= 16 else 64
        k = int(rng.integers(1, min(N, 4) + 1))
        T = int(rng.integers(1, 600))
        cf = float(rng.choice([0.0, 0.8, 1.0, 1.25]))
        bias = str(rng.choice(["none", "skew"]))
        coef = float(rng.choice([0.0, 0.01, 0.1]))
        overflow = "reroute" if (cf > 0 and rng.random() < 0.35) else "drop"
        out.append((f"rand{i:02d}_{dt}_T{T}_d{d}_N{N}_k{k}_f{f}_cf{cf}_{bias}_aux{coef}_{overflow}",
                    T, d, N, k, f, dt, cf, bias, coef, overflow, i))
    return out


RANDOM = _random_configs()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_backward_random_configs(moe, case):
    label, T, d, N, k, f, dt, cf, bias, coef, overflow, seed = case
    b = None
    if bias == "skew":
        b = np.zeros(N, np.float32)
        b[: min(3, N)] = [1.5, 1.0, 0.5][: min(3, N)]
    inp = synth.make_inputs(T, d, N, k, f, dt, cf, 200 + seed, bias=b)
    run_backward(moe, inp, coef, overflow, label)


@pytest.mark.parametrize("saved", [False, True])
def test_backward_is_deterministic(moe, saved):
    inp = synth.make_inputs(500, 256, 8, 2, 256, "bf16", 1.0, 3)
    from tests import parity
    dev = parity.to_device(inp)
    outs = []
    for _ in range(2):
        _, b = _forward(moe, inp, dev, "drop", saved)
        dy = _dev(synth.make_dy(inp.T, inp.d, "bf16", 5), "bf16")
        gr = moe.moe_backward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"], dy,
                              b, 0.01)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (gr.dhidden, gr.dw_router, gr.dw1, gr.dw3, gr.dw2)])
    for a, c in zip(*outs):
        assert torch.equal(a, c)


def test_up_save_stores_both_projections(moe):
    """moe_expert_up_save: act as moe_expert_up, and h13 = [x W1 | x W3] per row against
    the oracle's fp64 products (bf16: one rounding of an fp32 sum)."""
    import oracle.moe_oracle as O
    from tests import parity
    for dt, T, N in (("bf16", 300, 8), ("bf16", 37, 64), ("f32", 100, 8)):
        inp = synth.make_inputs(T, 256 if dt == "bf16" else 128, N, 2, 256, dt, 0.0, 2)
        dev = parity.to_device(inp)
        g, b = _forward(moe, inp, dev, "drop", True)
        act2 = moe.moe_expert_up(b.x_perm, b.offsets, dev["w1"], dev["w3"])
        torch.cuda.synchronize()
        A = g["A"]
        h13 = b.h13[:A].float().cpu().numpy().astype(np.float64)
        hv = inp.values("hidden")
        f = inp.f
        src = g["perm_src"]
        h1 = np.zeros((A, f))
        h3 = np.zeros((A, f))
        off = g["offsets"]
        for e in range(N):
            rows = np.arange(off[e], off[e + 1])
            if rows.size:
                x = hv[src[rows]].astype(np.float64)
                h1[rows] = x @ inp.expert_values("w1", e).astype(np.float64)
                h3[rows] = x @ inp.expert_values("w3", e).astype(np.float64)
        tol = 2e-2 if dt == "bf16" else 1e-5
        assert _rel(h13[:, :f], h1) <= tol and _rel(h13[:, f:], h3) <= tol, dt
        a1 = b.act[:A].float().cpu().numpy()
        a2 = act2[:A].float().cpu().numpy()
        assert _rel(a1, a2) <= (1e-2 if dt == "bf16" else 1e-6), dt
        ref = O.moe_forward(hv, inp.values("w_router"), parity.ExpertView(inp, "w1"),
                            parity.ExpertView(inp, "w3"), parity.ExpertView(inp, "w2"), inp.k)
        assert _rel(g["y"], ref["y"]) <= parity.Y_TOL[dt], dt


@pytest.mark.parametrize("key", ["mixtral", "skewed_zipf"])
def test_backward_workload_full_size(moe, key):
    """Full-size workload in the launch configuration the benchmark times, with h1 / h3
    recomputed and with them saved by the forward: routing exact for every token;
    dhidden on sampled tokens and dW1/dW3 columns and dW2 rows of sampled experts from
    the oracle entry by entry; dW_router and dbias in full against the oracle's (every
    token's logit gradient: one oracle forward of the experts), and by the softmax shift
    invariance (each row of dW_router sums to 0)."""
    import oracle.moe_oracle as O
    from tests import parity
    inp = synth.make_workload_inputs(key, seed=0)
    coef = 0.01
    dev = parity.to_device(inp)
    dy = synth.make_dy(inp.T, inp.d, inp.dtype, seed=11)
    T, N, f = inp.T, inp.N, inp.f
    toks = [0, 1, T // 2 + 1, T - 1]
    got = {}
    for mode in ("recompute", "saved"):
        parity.log(f"backward_{key}/{mode}: forward + backward on the GPU")
        g, b = _forward(moe, inp, dev, "drop", mode == "saved")
        gr = moe.moe_backward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"],
                              _dev(dy, inp.dtype), b, coef, want_dbias=inp.bias is not None)
        torch.cuda.synchronize()
        rows = np.diff(g["offsets"])
        busiest, idlest = int(rows.argmax()), int(rows.argmin())
        ec = [(busiest, [0, 1, f // 2 + 3, f - 1]), (idlest, [5, f - 2])]
        got[mode] = {"g": g, "ec": ec, "dh": gr.dhidden[toks].cpu().numpy(),
                     "dw": {(e, tuple(c)): (gr.dw1[e][:, c].cpu().numpy(),
                                             gr.dw3[e][:, c].cpu().numpy(),
                                             gr.dw2[e][c, :].cpu().numpy()) for e, c in ec},
                     "dw_router": gr.dw_router.cpu().numpy().astype(np.float64),
                     "dbias": gr.dbias.cpu().numpy().astype(np.float64)
                     if inp.bias is not None else None}
        del gr, b
        torch.cuda.empty_cache()
    ec = got["recompute"]["ec"]
    assert ec == got["saved"]["ec"]
    parity.log(f"backward_{key}: oracle on tokens {toks}, experts/columns {ec}")
    smp = O.moe_backward_sampled(inp.values("hidden"), inp.values("w_router"),
                                 parity.ExpertView(inp, "w1"), parity.ExpertView(inp, "w3"),
                                 parity.ExpertView(inp, "w2"), inp.k,
                                 synth.bf16_bits_to_f32(dy), inp.capacity_factor, inp.bias,
                                 aux_coef=coef, tokens=toks, expert_cols=ec, router=True)
    tol = GRAD_TOL[inp.dtype]
    ref = np.stack([smp["dhidden"][t] for t in toks])
    for mode, r in got.items():
        assert np.array_equal(r["g"]["topk_idx"], smp["topk_idx"]), "routing differs"
        assert np.array_equal(r["g"]["slot_row"], smp["slot_row"]), "dispatch differs"
        rep = {"dhidden": _rel(r["dh"], ref)}
        for e, cols in ec:
            r1, r3, r2 = smp["dw"][(e, tuple(cols))]
            d1, d3, d2 = r["dw"][(e, tuple(cols))]
            rep[f"dw1[{e}]"] = _rel(d1, r1)
            rep[f"dw3[{e}]"] = _rel(d3, r3)
            rep[f"dw2[{e}]"] = _rel(d2, r2)
        wr = r["dw_router"]
        rep["dw_router"] = _rel(wr, smp["dw_router"])
        if inp.bias is not None:
            rep["dbias"] = _rel(r["dbias"], smp["dbias"])
        for name, rel in rep.items():
            assert rel <= tol, f"backward_{key}/{mode}: {name} max rel err {rel:.3e} > {tol}"
        assert np.abs(wr).max() > 0
        assert np.abs(wr.sum(1)).max() <= 1e-4 * np.abs(wr).max(), "dW_router rows do not sum to 0"
        if inp.bias is not None:
            assert abs(r["dbias"].sum()) <= 1e-4 * np.abs(r["dbias"]).max()
        parity.log(f"backward_{key}/{mode}: rel errors {rep}")
