"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of the oracle's code.

Each check either compares against a value the pages print (fixtures under
tests/golden/), a closed form, an invariant, a special case that reduces to a
textbook formula, or brute force on tiny inputs.  The last group plants
plausible mistakes in a copy of the oracle and shows that a pin catches each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle.moe_oracle as O
from mixture_experts_layer_sum_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(T=24, d=16, N=8, k=2, f=32, seed=0, cf=0.0, bias=None, n_shared=0, f_shared=None):
    inp = synth.make_inputs(T, d, N, k, f, "f32", cf, seed, bias=bias, n_shared=n_shared,
                            f_shared=f_shared)
    return inp


def _fwd(inp, k=None, cf=None, mod=O):
    return mod.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2,
                           inp.k if k is None else k,
                           inp.capacity_factor if cf is None else cf, inp.bias)


# ---------------------------------------------------------------- top-k choice
@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_matches_brute_force_over_subsets(k):
    """The chosen set maximises the summed logit, with ties resolved by lower ids."""
    rng = np.random.default_rng(1)
    N = 8
    # small integers force many exact ties
    L = rng.integers(-3, 4, size=(200, N)).astype(np.float64)
    idx = O.select_topk(L, k)
    for t in range(L.shape[0]):
        best = None
        for sub in itertools.combinations(range(N), k):
            # preference: larger sum; on equal sums, the lexicographically smaller id
            # multiset sorted by (value desc, id asc) wins
            key = (sum(L[t, list(sub)]), tuple(-e for e in sub))
            if best is None or key > best[0]:
                best = (key, sub)
        assert set(idx[t]) == set(best[1]), (t, L[t], idx[t], best)
        # slot order: value descending, ids ascending among equal values
        vals = L[t, idx[t]]
        for a in range(k - 1):
            assert vals[a] > vals[a + 1] or (vals[a] == vals[a + 1] and idx[t, a] < idx[t, a + 1])
        # nothing outside the set beats a member, and an outside tie has a larger id
        rest = [e for e in range(N) if e not in set(idx[t])]
        for e in rest:
            assert L[t, e] <= vals.min()
            if L[t, e] == vals.min():
                assert e > max(i for i in idx[t] if L[t, i] == vals.min())


def test_zero_router_routes_every_token_to_lowest_ids():
    """W_router = 0: all logits tie, so every token picks experts 0..k-1 with weight 1/k."""
    inp = _rand(T=10, N=8, k=3)
    inp.w_router[:] = 0
    out = _fwd(inp)
    assert (out["topk_idx"] == np.arange(3)[None, :]).all()
    assert np.array_equal(out["topk_w"], np.full((10, 3), 1.0 / 3.0))


def test_bias_moves_the_choice():
    inp = _rand(T=12, N=8, k=2)
    bias = np.zeros(8, np.float32)
    bias[5] = 1e3
    inp.bias = bias
    out = _fwd(inp)
    assert (out["topk_idx"][:, 0] == 5).all()


# ---------------------------------------------------------------- gate weights
def test_weights_sum_to_one_and_k1_is_exactly_one():
    inp = _rand(T=40, N=8, k=3, seed=2)
    out = _fwd(inp)
    assert np.allclose(out["topk_w"].sum(1), 1.0, rtol=0, atol=1e-15)
    assert (np.diff(out["topk_w"], axis=1) <= 1e-15).all()   # slot order is by logit
    out1 = _fwd(inp, k=1)
    assert (out1["topk_w"] == 1.0).all()


def test_weights_equal_renormalised_full_softmax():
    """P3's form (softmax over all N, keep the top-k, divide by their sum) gives the same weights."""
    inp = _rand(T=30, N=8, k=2, seed=3)
    out = _fwd(inp)
    L = out["logits"]
    probs = np.exp(L) / np.exp(L).sum(1, keepdims=True)
    p_sel = np.take_along_axis(probs, out["topk_idx"], 1)
    assert np.allclose(out["topk_w"], p_sel / p_sel.sum(1, keepdims=True), rtol=1e-13, atol=0)


def test_two_expert_weight_is_logistic_of_gap():
    """For k = 2, w_0 = 1 / (1 + exp(-(l_0 - l_1))) (closed form of a 2-way softmax)."""
    inp = _rand(T=30, N=8, k=2, seed=4)
    out = _fwd(inp)
    l = np.take_along_axis(out["logits"], out["topk_idx"], 1)
    assert np.allclose(out["topk_w"][:, 0], 1 / (1 + np.exp(-(l[:, 0] - l[:, 1]))), rtol=1e-13)


# ---------------------------------------------------------------- expert FFN
def test_silu_values():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(40.0) - 40.0) < 1e-12
    assert abs(O.silu(-40.0)) < 1e-15
    assert O.silu(-1e4) == 0.0 or abs(O.silu(-1e4)) < 1e-300


def test_swiglu_closed_form_identity_and_permutation():
    """W1 = I, W3 = 2I, W2 = P (a permutation): FFN(x) = P applied to silu(x) * 2x.

    Distinct W1 / W3 catch a swapped gate; a non-symmetric W2 catches a transpose.
    """
    d = 6
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, d))
    P = np.eye(d)[[2, 0, 5, 1, 3, 4]]
    y = O.swiglu_ffn(x, np.eye(d), 2 * np.eye(d), P)
    g = (x / (1 + np.exp(-x))) * (2 * x)
    assert np.allclose(y, g @ P, rtol=1e-14, atol=0)
    assert np.allclose(y[:, 0], g[:, 1])      # column 0 of P picks row 1


def test_zero_input_gives_zero_output():
    inp = _rand(T=8, seed=6)
    inp.hidden[:] = 0
    out = _fwd(inp)
    assert (out["y"] == 0).all()


# ---------------------------------------------------------------- counts / capacity
def test_counts_sum_to_T_times_k():
    inp = _rand(T=33, N=8, k=3, seed=7)
    out = _fwd(inp)
    assert out["counts"].sum() == 33 * 3


def test_activation_ratio_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "activation_ratio.json")))
    for case in g["cases"]:
        N, k = case["experts"], case["top_k"]
        rng = np.random.default_rng(N)
        L = rng.standard_normal((50, N))
        idx = O.select_topk(L, k)
        counts = O.expert_counts(idx, N)
        assert len(set(map(tuple, np.sort(idx, 1)))) >= 1
        assert all(len(set(r)) == k for r in idx)             # k distinct experts per token
        assert counts.sum() / (50 * N) == pytest.approx(case["ratio"], abs=1e-15)


def test_capacity_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "capacity_worked_example.json")))
    T = g["batch"] * g["seq_len"]
    assert T == g["tokens"]
    assert T // g["experts"] == g["mean_tokens_per_expert"]
    assert O.capacity(T, g["top_k"], g["experts"], g["capacity_factor"]) == g["capacity"]


def test_capacity_of_the_workloads_and_no_limit():
    assert O.capacity(4096, 2, 16, 1.25) == 640
    assert O.capacity(16384, 2, 64, 1.5) == 768
    assert O.capacity(8192, 2, 8, 0.0) == 8192
    assert O.capacity(256, 2, 128, -1.0) == 256


def _running_places(idx, N):
    """Place of each (t, j) at its expert via a cumulative sum over a one-hot mask."""
    T, k = idx.shape
    onehot = np.zeros((T, N), np.int64)
    for j in range(k):
        onehot[np.arange(T), idx[:, j]] += 1
    before = np.cumsum(onehot, axis=0) - onehot              # tokens strictly before t
    return np.take_along_axis(before, idx, 1)


@pytest.mark.parametrize("cf", [0.0, 0.5, 1.0, 1.25])
def test_dispatch_characterisation(cf):
    inp = _rand(T=64, N=8, k=2, seed=8, cf=cf)
    bias = np.zeros(8, np.float32)
    bias[:3] = [2.0, 1.0, 0.5]                  # skew so that capacity bites
    inp.bias = bias
    out = _fwd(inp)
    idx, C = out["topk_idx"], out["capacity"]
    place = _running_places(idx, 8)
    keep = place < C
    assert np.array_equal(out["slot_row"] >= 0, keep)
    assert np.array_equal(out["kept"], np.minimum(out["counts"], C))
    offs = out["offsets"]
    assert offs[0] == 0 and np.array_equal(np.diff(offs), out["kept"])
    # rows form a permutation of the kept (t, j); expert-major, token-ascending
    rows = out["slot_row"][keep]
    assert np.array_equal(np.sort(rows), np.arange(offs[-1]))
    src = out["perm_src"]
    for e in range(8):
        seg = src[offs[e]:offs[e + 1]]
        assert (np.diff(seg) > 0).all()
        for r, t in zip(range(offs[e], offs[e + 1]), seg):
            j = int(np.where(idx[t] == e)[0][0])
            assert out["slot_row"][t, j] == r
    if cf > 0:
        assert (~keep).any() or cf >= 1.0


# ---------------------------------------------------------------- whole layer
@pytest.mark.parametrize("cf", [0.0, 0.75])
def test_per_expert_path_equals_per_token_brute_force(cf):
    inp = _rand(T=48, d=16, N=8, k=2, f=24, seed=9, cf=cf)
    out = _fwd(inp)
    y_bf = O.moe_forward_per_token(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, cf)
    assert np.allclose(out["y"], y_bf, rtol=1e-12, atol=1e-14)


def test_k_equals_N_is_dense_softmax_mixture():
    """k = N: y_t = sum_e softmax(l_t)_e * FFN_e(x_t), the dense mixture of experts."""
    inp = _rand(T=20, d=12, N=4, k=4, f=16, seed=10)
    out = _fwd(inp)
    x = inp.hidden.astype(np.float64)
    L = x @ inp.w_router.astype(np.float64)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    y = np.zeros_like(x)
    for e in range(4):
        h1 = x @ inp.w1[e].astype(np.float64)
        h3 = x @ inp.w3[e].astype(np.float64)
        y += p[:, e:e + 1] * ((h1 * (1 / (1 + np.exp(-h1))) * h3) @ inp.w2[e].astype(np.float64))
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-14)


def test_k1_no_cap_is_the_chosen_expert_output():
    inp = _rand(T=16, N=8, k=1, seed=11)
    out = _fwd(inp, k=1)
    for t in range(16):
        e = out["topk_idx"][t, 0]
        ref = O.swiglu_ffn(inp.hidden[t:t + 1], inp.w1[e], inp.w3[e], inp.w2[e])[0]
        assert np.allclose(out["y"][t], ref, rtol=1e-13, atol=0)


def test_dropped_tokens_are_zero_and_weights_not_renormalised():
    inp = _rand(T=32, N=8, k=2, seed=12)
    inp.w_router[:] = 0            # everyone wants experts 0 and 1
    out = _fwd(inp, cf=0.5)        # C = floor(64/8*0.5) = 4
    assert out["capacity"] == 4
    kept_tok = set(range(4))
    for t in range(32):
        if t in kept_tok:
            ref = 0.5 * O.swiglu_ffn(inp.hidden[t:t + 1], inp.w1[0], inp.w3[0], inp.w2[0])[0] \
                + 0.5 * O.swiglu_ffn(inp.hidden[t:t + 1], inp.w1[1], inp.w3[1], inp.w2[1])[0]
            assert np.allclose(out["y"][t], ref, rtol=1e-13, atol=0)
        else:
            assert (out["y"][t] == 0).all()
    # one slot dropped, the other kept: the kept one keeps its own weight
    inp2 = _rand(T=16, N=8, k=2, seed=13)
    inp2.w_router[:] = 0
    bias = np.zeros(8, np.float32)
    bias[0], bias[1] = 1.0, 0.0
    inp2.bias = bias
    hid = inp2.hidden.copy()
    inp2.hidden[:] = 0
    inp2.hidden[:8] = hid[:8]
    out2 = _fwd(inp2, cf=0.5)      # C = 1: token 0 keeps both, later tokens lose both
    w0 = 1 / (1 + math.exp(-1.0))
    assert out2["topk_w"][0, 0] == pytest.approx(w0, rel=1e-14)
    t = 0
    ref = w0 * O.swiglu_ffn(inp2.hidden[t:t + 1], inp2.w1[0], inp2.w3[0], inp2.w2[0])[0] \
        + (1 - w0) * O.swiglu_ffn(inp2.hidden[t:t + 1], inp2.w1[1], inp2.w3[1], inp2.w2[1])[0]
    assert np.allclose(out2["y"][0], ref, rtol=1e-13)


def test_one_slot_dropped_keeps_unnormalised_weight():
    """Token 1 loses its first choice to capacity but keeps its second at the original weight."""
    T, d, N, f = 2, 8, 4, 8
    inp = _rand(T=T, d=d, N=N, k=2, f=f, seed=14)
    inp.w_router[:] = 0
    inp.bias = np.array([0.0, 3.0, 1.0, 2.0], np.float32)
    # token 0 -> (1, 3); token 1 -> (1, 3) as well, C = floor(4/4*1.0) = 1
    out = _fwd(inp, cf=1.0)
    assert out["capacity"] == 1
    assert (out["topk_idx"] == np.array([[1, 3], [1, 3]])).all()
    assert out["slot_row"][1, 0] == -1 and out["slot_row"][1, 1] == -1
    inp.bias = np.array([0.0, 3.0, 1.0, 2.0], np.float32)
    out = _fwd(inp, cf=2.0)        # C = 2: nothing dropped
    assert (out["slot_row"] >= 0).all()
    # now make token 1 pick (1, 2) by its own hidden: give expert 2 a token-dependent score
    inp.w_router[:] = 0
    inp.w_router[0, 2] = 10.0
    inp.hidden[:, 0] = [-1.0, 1.0]  # token 0: expert 2 at -10, token 1: expert 2 at +10
    out = _fwd(inp, cf=1.0)        # C = 1
    assert list(out["topk_idx"][0]) == [1, 3] and list(out["topk_idx"][1]) == [2, 1]
    # token 1: expert 2 kept (first at 2), expert 1 dropped (token 0 holds the one place)
    assert out["slot_row"][1, 0] >= 0 and out["slot_row"][1, 1] == -1
    w = out["topk_w"][1, 0]
    ref = w * O.swiglu_ffn(inp.hidden[1:2], inp.w1[2], inp.w3[2], inp.w2[2])[0]
    assert w < 1.0
    assert np.allclose(out["y"][1], ref, rtol=1e-13)


# ---------------------------------------------------------------- overflow re-routing
def test_reroute_hand_example_single_choice():
    """Four tokens all pick expert 0 with room for one each (C = 1): the first
    keeps it, the next two move to their best other expert, the fourth finds
    its best other expert already taken and is dropped."""
    idx = np.array([[0], [0], [0], [0]])
    L = np.array([[3, 2, 1], [3, 1, 2], [3, 2, 1], [3, 1, 2]], np.float64)
    r = O.dispatch_reroute(idx, L, 3, 1)
    assert r["expert"].ravel().tolist() == [0, 2, 1, -1]
    assert r["kept"].tolist() == [1, 1, 1]
    assert r["offsets"].tolist() == [0, 1, 2, 3]
    assert r["slot_row"].ravel().tolist() == [0, 2, 1, -1]
    assert r["perm_src"].tolist() == [0, 2, 1]


def test_reroute_hand_example_two_dropped_slots_take_distinct_experts():
    """Both slots of a token dropped: they propose the two best other experts
    (never the same one twice); a later token proposing the same experts finds
    them full."""
    idx = np.array([[0, 1], [0, 1], [0, 1]])
    L = np.array([[4, 3, 2, 1]] * 3, np.float64)
    r = O.dispatch_reroute(idx, L, 4, 1)
    assert r["proposal"].tolist() == [[-1, -1], [2, 3], [2, 3]]
    assert r["expert"].tolist() == [[0, 1], [2, 3], [-1, -1]]
    assert r["slot_row"].tolist() == [[0, 1], [2, 3], [-1, -1]]


def test_reroute_only_to_experts_with_room_after_the_first_round():
    """An expert that is full after the first round is never proposed, even
    when it has the best remaining logit."""
    idx = np.array([[0], [1], [0]])
    L = np.array([[5, 1, 0], [0, 5, 1], [5, 4, 1]], np.float64)
    r = O.dispatch_reroute(idx, L, 3, 1)
    # token 2 drops at expert 0; expert 1 (logit 4) is full, so it goes to 2
    assert r["proposal"][2, 0] == 2
    assert r["expert"].ravel().tolist() == [0, 1, 2]


def test_reroute_without_overflow_is_the_drop_dispatch():
    inp = _rand(T=40, N=8, k=2, seed=21)
    a = _fwd(inp)
    b = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.0, None,
                      overflow="reroute")
    for key in ("slot_row", "perm_src", "offsets", "kept"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["y"], b["y"])


@pytest.mark.parametrize("seed,cf", [(0, 0.5), (1, 1.0), (2, 0.25), (3, 1.5)])
def test_reroute_invariants(seed, cf):
    """Capacity holds, first-round places are untouched, re-routed slots land
    on experts outside the token's picks (distinct within a token), and no
    slot that the drop policy keeps is lost."""
    bias = np.zeros(16, np.float32)
    bias[:3] = [3.0, 2.0, 1.0]
    inp = _rand(T=96, N=16, k=2, seed=seed, cf=cf, bias=bias)
    L = O.router_logits(inp.hidden, inp.w_router, inp.bias)
    idx = O.select_topk(L, 2)
    C = O.capacity(96, 2, 16, cf)
    d0 = O.dispatch(idx, 16, C)
    r = O.dispatch_reroute(idx, L, 16, C)
    assert (r["kept"] <= C).all()
    assert np.array_equal(r["keep1"], d0["keep"])
    moved = r["keep2"]
    for t, j in zip(*np.nonzero(moved)):
        assert r["expert"][t, j] not in idx[t]
    for t in range(96):
        ex = [e for e in r["expert"][t] if e >= 0]
        assert len(ex) == len(set(ex))
    # every row's expert is the one its slot names
    for t in range(96):
        for j in range(2):
            row = r["slot_row"][t, j]
            if row >= 0:
                e = r["expert"][t, j]
                assert r["offsets"][e] <= row < r["offsets"][e + 1]
                assert r["perm_src"][row] == t
    assert r["kept"].sum() >= d0["kept"].sum()
    if (~d0["keep"]).any():
        assert moved.any()


@pytest.mark.parametrize("cf", [0.25, 0.75])
def test_reroute_per_expert_path_equals_per_token_brute_force(cf):
    bias = np.zeros(8, np.float32)
    bias[:2] = [4.0, 3.0]                       # experts 0 and 1 overflow, the others have room
    inp = _rand(T=40, N=8, k=2, seed=5, cf=cf, bias=bias)
    a = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, cf, inp.bias,
                      overflow="reroute")
    b = O.moe_forward_per_token(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, cf,
                                inp.bias, overflow="reroute")
    assert np.allclose(a["y"], b, rtol=1e-12, atol=1e-12)
    d = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, cf, inp.bias)
    moved = (a["slot_row"] >= 0) & (d["slot_row"] < 0)
    assert moved.any()
    assert not np.allclose(a["y"][moved.any(1)], d["y"][moved.any(1)])


# ---------------------------------------------------------------- shared experts
def test_shared_expert_closed_form_with_silent_routed_experts():
    """Routed experts with W2 = 0 contribute nothing; a shared expert with W1 = I,
    W3 = 2I, W2 = a permutation gives (silu(x) * 2x) P for every token."""
    d = 8
    inp = _rand(T=12, d=d, N=4, k=2, f=16, seed=31)
    inp.w2[:] = 0
    Pm = np.eye(d)[[3, 1, 7, 0, 2, 6, 4, 5]]
    shared = (np.eye(d)[None], 2 * np.eye(d)[None], Pm[None])
    out = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, shared=shared)
    x = inp.hidden.astype(np.float64)
    ref = ((x / (1 + np.exp(-x))) * (2 * x)) @ Pm
    assert np.allclose(out["y"], ref, rtol=1e-14, atol=1e-14)


def test_shared_expert_adds_to_every_token_even_when_all_slots_drop():
    inp = _rand(T=24, N=8, k=2, seed=33, cf=0.1, n_shared=1, f_shared=24)
    shared = (inp.w1s, inp.w3s, inp.w2s)
    a = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.1, shared=shared)
    b = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.1)
    direct = O.swiglu_ffn(inp.hidden, inp.w1s[0], inp.w3s[0], inp.w2s[0])
    assert np.allclose(a["y"] - b["y"], direct, rtol=1e-12, atol=1e-13)
    dropped = (a["slot_row"] < 0).all(1)
    assert dropped.any()
    assert np.allclose(a["y"][dropped], direct[dropped], rtol=1e-13, atol=1e-14)


def test_two_shared_experts_sum_and_match_brute_force():
    inp = _rand(T=20, N=4, k=2, seed=35, cf=0.75, n_shared=2, f_shared=16)
    sh = (inp.w1s, inp.w3s, inp.w2s)
    a = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.75, shared=sh)
    one = [O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.75,
                         shared=(inp.w1s[q:q + 1], inp.w3s[q:q + 1], inp.w2s[q:q + 1]))["y"]
           for q in range(2)]
    none = O.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.75)["y"]
    assert np.allclose(a["y"], one[0] + one[1] - none, rtol=1e-12, atol=1e-13)
    b = O.moe_forward_per_token(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.75,
                                shared=sh)
    assert np.allclose(a["y"], b, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- FP8 (OCP E4M3) weights
def test_e4m3_code_values_from_the_format():
    """Landmarks of OCP FP8 E4M3 (bias 7, 3 mantissa bits, no infinity)."""
    dec = O.e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x7E, 0xFE, 0x7F, 0xFF],
                                 np.uint8))
    assert dec[0] == 0.0 and dec[1] == 0.0 and np.signbit(dec[1])
    assert dec[2] == 2.0 ** -9                    # smallest subnormal
    assert dec[3] == 7 * 2.0 ** -9                # largest subnormal
    assert dec[4] == 2.0 ** -6                    # smallest normal
    assert dec[5] == 1.0
    assert dec[6] == 1.875
    assert dec[7] == 448.0 and dec[8] == -448.0   # largest finite
    assert np.isnan(dec[9]) and np.isnan(dec[10])


def test_e4m3_encode_is_the_nearest_code_by_brute_force():
    """Against a table search over all finite codes: nearest value, ties to the
    code with an even mantissa."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.e4m3_decode(codes)
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 3000),
                        vals, (vals[:-1] + vals[1:]) / 2])          # includes exact midpoints
    x = x[np.abs(x) <= 448]
    got = O.e4m3_encode(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:                       # tie: the even mantissa wins
            best = [b for b in best if codes[b] & 1 == 0]
        ref = codes[best[0]]
        if vals[best[0]] == 0.0:                # +-0: the sign of x decides
            assert O.e4m3_decode(np.array([gi], np.uint8))[0] == 0.0
        else:
            assert gi == ref, (xi, gi, ref)


def test_e4m3_roundtrip_and_ties_to_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)
    # halfway cases: 1.0625 between 1.0 (even) and 1.125; 1.1875 between 1.125 and
    # 1.25 (even); 17 between 16 (even) and 18; 2^-10 between 0 (even) and 2^-9
    assert O.e4m3_encode(np.array([1.0625, 1.1875, 17.0, 2.0 ** -10])).tolist() == \
        [0x38, 0x3A, 0x58, 0x00]


def test_fp8_column_quantisation():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((64, 5)) * [1e-3, 1.0, 30.0, 0.0, 5e2]).astype(np.float32)
    q, scale = O.quantize_fp8_columns(w)
    assert scale[3] == 1.0 and (q[:, 3] & 0x7F == 0).all()          # an all-zero column (+-0)
    for m in (0, 1, 2, 4):
        amax = np.abs(w[:, m]).max()
        assert scale[m] == np.float32(amax) / np.float32(448.0)
        k = int(np.abs(w[:, m]).argmax())
        assert q[k, m] & 0x7F == 0x7E                               # the column's amax -> 448
    wd = O.dequantize_fp8_columns(q, scale)
    # relative error of a normal code is at most half a mantissa step: 2^-4
    big = np.abs(w) >= 2.0 ** -6 * scale[None, :]
    assert (np.abs(wd - w)[big] <= 2.0 ** -4 * np.abs(w)[big] + 1e-12).all()


# ---------------------------------------------------------------- aux loss
def test_aux_uniform_router_is_exactly_one():
    """W_router = 0 gives P_e = 1/N; with f summing to 1 the loss is exactly 1, also under drops."""
    for N, k, cf in [(8, 2, 0.0), (16, 2, 1.25), (4, 1, 0.5)]:
        inp = _rand(T=32, N=N, k=k, seed=15, cf=cf)
        inp.w_router[:] = 0
        out = _fwd(inp)
        assert out["aux"] == 1.0


def test_aux_balanced_assignment_is_one():
    """Each expert gets the same share of assignments: f_e = 1/N, so aux = sum_e P_e = 1."""
    N, T, k = 8, 64, 2
    d = N
    hidden = np.zeros((T, d), np.float32)
    for t in range(T):
        hidden[t, t % N] = 2.0
        hidden[t, (t + 1) % N] = 1.0
    w_router = np.eye(d, N, dtype=np.float32)
    L = O.router_logits(hidden, w_router)
    idx = O.select_topk(L, k)
    counts = O.expert_counts(idx, N)
    assert (counts == T * k // N).all()
    assert O.aux_loss(L, counts, k) == pytest.approx(1.0, abs=1e-15)


def test_aux_collapse_reaches_N():
    """Every token on one expert with near-certain probability: aux -> N."""
    N, T = 8, 16
    L = np.full((T, N), -50.0)
    L[:, 3] = 50.0
    idx = O.select_topk(L, 1)
    counts = O.expert_counts(idx, N)
    assert O.aux_loss(L, counts, 1) == pytest.approx(N, rel=1e-12)


# ---------------------------------------------------------------- planted mistakes
class _Mutant:
    """A copy of the oracle's namespace with one function replaced."""

    def __init__(self, **repl):
        self.__dict__.update({k: getattr(O, k) for k in O.__all__})
        self.__dict__.update(repl)
        src = O.moe_forward

        def moe_forward(*a, **kw):
            g = dict(src.__globals__)
            g.update(repl)
            fn = type(src)(src.__code__, g, src.__name__, src.__defaults__, src.__closure__)
            return fn(*a, **kw)

        self.moe_forward = moe_forward


def test_pins_catch_planted_mistakes():
    def swapped_gate(x, w1, w3, w2):
        return O.swiglu_ffn(x, w3, w1, w2)

    def high_index_ties(L, k):
        L32 = np.asarray(L).astype(np.float32)
        T, N = L32.shape
        ids = np.broadcast_to(-np.arange(N), (T, N))
        return np.lexsort((ids, -L32.astype(np.float64)), axis=-1)[:, :k]

    def unnormalised_f(L, counts, k):
        return O.aux_loss(L, counts, 1)

    def capacity_without_k(T, k, N, cf):
        return O.capacity(T, 1, N, cf)

    def last_tokens_kept(idx, N, C):
        rev = O.dispatch(np.asarray(idx)[::-1], N, C)
        keep = rev["keep"][::-1]
        T, k = idx.shape
        # rebuild rows in token order from the reversed keep decision
        kept = np.bincount(np.asarray(idx)[keep], minlength=N)
        offsets = np.concatenate([[0], np.cumsum(kept)])
        slot_row = -np.ones((T, k), np.int64)
        fill = offsets[:-1].copy()
        perm_src = np.empty(offsets[-1], np.int64)
        for t in range(T):
            for j in range(k):
                if keep[t, j]:
                    e = idx[t, j]
                    slot_row[t, j] = fill[e]
                    perm_src[fill[e]] = t
                    fill[e] += 1
        return {"keep": keep, "kept": kept, "offsets": offsets, "slot_row": slot_row,
                "perm_src": perm_src, "place": None}

    def full_softmax_weights(L, idx):
        p = np.exp(L - L.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return np.take_along_axis(p, idx, 1)

    # swapped gate: closed-form SwiGLU pin (through the per-expert path)
    d = 6
    P = np.eye(d)[[2, 0, 5, 1, 3, 4]]
    x = np.random.default_rng(0).standard_normal((3, d))
    g = (x / (1 + np.exp(-x))) * (2 * x)
    assert not np.allclose(swapped_gate(x, np.eye(d), 2 * np.eye(d), P), g @ P)

    # tie rule: zero router must pick 0..k-1
    inp = _rand(T=6, N=8, k=2)
    inp.w_router[:] = 0
    m = _Mutant(select_topk=high_index_ties)
    assert not (m.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2)["topk_idx"]
                == np.arange(2)).all()

    # f without /k: the uniform router no longer scores 1
    m = _Mutant(aux_loss=unnormalised_f)
    assert m.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2)["aux"] != 1.0

    # capacity without k: the workload capacities no longer come out
    assert capacity_without_k(4096, 2, 16, 1.25) != 640

    # re-routing that ignores the first round's fill sends token 2 of the
    # room example to the full expert 1
    def reroute_ignoring_room(idx, L, N, C):
        big = O.dispatch_reroute(idx, L, N, C + 10 ** 6)
        return big
    r = reroute_ignoring_room(np.array([[0], [1], [0]]),
                              np.array([[5, 1, 0], [0, 5, 1], [5, 4, 1]], np.float64), 3, 1)
    assert r["expert"].ravel().tolist() != [0, 1, 2]

    # keeping the last C tokens instead of the first: characterisation fails
    inp = _rand(T=64, N=8, k=2, seed=8)
    inp.bias = np.array([2.0, 1.0, 0.5, 0, 0, 0, 0, 0], np.float32)
    m = _Mutant(dispatch=last_tokens_kept)
    out = m.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, 0.5, inp.bias)
    place = _running_places(out["topk_idx"], 8)
    assert not np.array_equal(out["slot_row"] >= 0, place < out["capacity"])

    # softmax over all N without renormalising: weights no longer sum to 1
    m = _Mutant(gate_weights=full_softmax_weights)
    out = m.moe_forward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2)
    assert not np.allclose(out["topk_w"].sum(1), 1.0)


# ---------------------------------------------------------------- backward pass
def _loss_and_fd(inp, k, cf, dy, coef, overflow, eps=1e-6):
    """Central differences of L = <dy, y> + coef * aux through the forward oracle.

    Entries whose perturbation changes the top-k choice are NaN (the choice is
    piecewise constant, so the derivative there is one-sided)."""
    P = {"hidden": inp.hidden, "w_router": inp.w_router, "w1": inp.w1, "w3": inp.w3,
         "w2": inp.w2, "bias": inp.bias}
    if inp.n_shared:
        P.update({"w1s": inp.w1s, "w3s": inp.w3s, "w2s": inp.w2s})
    P = {n: np.asarray(v, np.float64) for n, v in P.items()}

    def loss(Q):
        sh = (Q["w1s"], Q["w3s"], Q["w2s"]) if inp.n_shared else None
        out = O.moe_forward(Q["hidden"], Q["w_router"], Q["w1"], Q["w3"], Q["w2"], k, cf,
                            Q["bias"], overflow=overflow, shared=sh)
        return float(np.sum(dy * out["y"])) + coef * float(out["aux"]), out

    _, base = loss(P)
    grads = {}
    for name, arr in P.items():
        G = np.full(arr.shape, np.nan)
        for i in np.ndindex(arr.shape):
            vals = []
            for sgn in (1.0, -1.0):
                Q = dict(P)
                Q[name] = arr.copy()
                Q[name][i] += sgn * eps
                l, out = loss(Q)
                if not np.array_equal(out["topk_idx"], base["topk_idx"]):
                    break
                vals.append(l)
            if len(vals) == 2:
                G[i] = (vals[0] - vals[1]) / (2 * eps)
        grads[name] = G
    return grads, base


_GRAD_KEYS = {"hidden": "dhidden", "w_router": "dw_router", "w1": "dw1", "w3": "dw3",
              "w2": "dw2", "bias": "dbias", "w1s": "dw1s", "w3s": "dw3s", "w2s": "dw2s"}


def _backward(inp, k, cf, dy, coef, overflow, mod=O):
    sh = (inp.w1s, inp.w3s, inp.w2s) if inp.n_shared else None
    return mod.moe_backward(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, k, dy, cf,
                            inp.bias, aux_coef=coef, overflow=overflow, shared=sh)


def _fd_agrees(inp, k, cf, dy, coef, overflow, g):
    fd, _ = _loss_and_fd(inp, k, cf, dy, coef, overflow)
    worst = 0.0
    for name, key in _GRAD_KEYS.items():
        if name not in fd:
            continue
        ok = ~np.isnan(fd[name])
        assert ok.mean() > 0.9
        scale = max(1.0, float(np.abs(fd[name][ok]).max()))
        worst = max(worst, float(np.abs(fd[name][ok] - g[key][ok]).max()) / scale)
    return worst


@pytest.mark.parametrize("cf,coef,overflow,seed,ns", [
    (0.0, 0.0, "drop", 0, 0),        # no capacity limit, no aux loss
    (0.8, 0.37, "drop", 1, 0),       # dropped slots and the aux-loss term
    (0.8, 0.05, "reroute", 2, 0),    # re-routed slots keep their gate weight
    (0.8, 0.1, "drop", 3, 2),        # two shared experts (weight 1 on every token)
])
def test_backward_matches_finite_differences_of_the_forward(cf, coef, overflow, seed, ns):
    """Every gradient equals the central difference of the pinned forward (fp64, eps 1e-6)."""
    inp = synth.make_inputs(10, 6, 4, 2, 5, "f32", cf, seed,
                            bias=np.array([0.5, 0.0, -0.3, 0.2], np.float32), n_shared=ns,
                            f_shared=3 if ns else None)
    dy = np.random.default_rng(100 + seed).standard_normal((10, 6))
    g = _backward(inp, 2, cf, dy, coef, overflow)
    if cf > 0:
        assert (g["slot_row"] < 0).any()          # the case really drops slots
    assert _fd_agrees(inp, 2, cf, dy, coef, overflow, g) < 1e-6


def test_backward_softmax_shift_invariance():
    """Adding one constant to a token's logits changes neither the top-k set, the
    weights nor P: each token's logit gradient sums to zero, so dbias sums to zero
    and every row of dW_router does too."""
    inp = _rand(T=32, d=8, N=8, k=2, f=16, seed=3, cf=1.0)
    dy = np.random.default_rng(4).standard_normal((32, 8))
    g = _backward(inp, 2, 1.0, dy, 0.1, "drop")
    assert np.abs(g["dlogits"].sum(1)).max() < 1e-12
    assert abs(g["dbias"].sum()) < 1e-12
    assert np.abs(g["dw_router"].sum(1)).max() < 1e-12


def test_backward_fully_dropped_token_has_no_gradient_without_aux():
    """A token whose every slot is dropped skips the layer (y = 0 there), so with
    no aux term nothing flows back to it or from it."""
    inp = _rand(T=16, d=8, N=4, k=1, f=8, seed=5, cf=0.25)
    inp.bias = np.array([6.0, 0.0, 0.0, 0.0], np.float32)    # everyone wants expert 0
    dy = np.random.default_rng(6).standard_normal((16, 8))
    g = _backward(inp, 1, 0.25, dy, 0.0, "drop")
    gone = (g["slot_row"] < 0).all(1)
    assert gone.any()
    assert np.abs(g["dhidden"][gone]).max() == 0.0
    assert np.abs(g["dlogits"][gone]).max() == 0.0
    # with k = 1 the single weight is exactly 1: the router gets nothing either
    assert np.abs(g["dlogits"]).max() == 0.0


def test_backward_pins_catch_planted_mistakes():
    """Plant a plausible mistake in a copy of the oracle's backward; the
    finite-difference pin must reject each."""
    import inspect
    fns = [O.swiglu_backward, O._dlogits, O.moe_backward]
    srcs = {fn.__name__: inspect.getsource(fn) for fn in fns}
    mistakes = [
        ("s + h1 * s * (1.0 - s)", "s"),                       # silu' without its second term
        ("w * (dgate - inner)", "w * dgate"),                  # softmax Jacobian without the mean
        ("(fe[None, :] - np.sum", "(fe[None, :] + np.sum"),    # aux gradient sign
        ('"dw2": a.T @ G', '"dw2": (h1 * h3).T @ G'),          # dW2 from h1 h3 instead of silu(h1) h3
        ("dhidden += dlog @ Wr.T", "pass"),                    # router path into dhidden dropped
        ("dh3 = da * (h1 * s)", "dh3 = da * h1"),              # dh3 without the sigmoid
    ]
    inp = synth.make_inputs(10, 6, 4, 2, 5, "f32", 0.8, 1,
                            bias=np.array([0.5, 0.0, -0.3, 0.2], np.float32))
    dy = np.random.default_rng(101).standard_normal((10, 6))
    for old, new in mistakes:
        hits = [n for n, src in srcs.items() if old in src]
        assert len(hits) == 1, old
        ns = dict(vars(O))
        for n, src in srcs.items():
            exec(compile(src.replace(old, new) if n == hits[0] else src, "<mutant>", "exec"), ns)

        class M:
            moe_backward = staticmethod(ns["moe_backward"])
        g = _backward(inp, 2, 0.8, dy, 0.37, "drop", mod=M)
        assert _fd_agrees(inp, 2, 0.8, dy, 0.37, "drop", g) > 1e-3, old


@pytest.mark.parametrize("overflow,cf,coef", [("drop", 1.0, 0.2), ("reroute", 0.8, 0.05)])
def test_backward_sampled_entries_equal_the_full_backward(overflow, cf, coef):
    """The row- and column-local entries the full-size tests use are the same
    numbers as the (finite-difference pinned) full backward."""
    inp = _rand(T=40, d=8, N=4, k=2, f=12, seed=9, cf=cf,
                bias=np.array([0.8, 0.2, 0.0, -0.5], np.float32))
    dy = np.random.default_rng(12).standard_normal((40, 8))
    full = _backward(inp, 2, cf, dy, coef, overflow)
    toks = [0, 7, 39]
    ec = [(0, [0, 5, 11]), (3, [2])]
    smp = O.moe_backward_sampled(inp.hidden, inp.w_router, inp.w1, inp.w3, inp.w2, 2, dy, cf,
                                 inp.bias, aux_coef=coef, overflow=overflow, tokens=toks,
                                 expert_cols=ec, router=True)
    assert np.allclose(smp["dw_router"], full["dw_router"], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dbias"], full["dbias"], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dgate"], full["dgate"], rtol=1e-12, atol=1e-12)
    for t in toks:
        assert np.allclose(smp["dhidden"][t], full["dhidden"][t], rtol=1e-12, atol=1e-12)
    for e, cols in ec:
        d1, d3, d2 = smp["dw"][(e, tuple(cols))]
        assert np.allclose(d1, full["dw1"][e][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(d3, full["dw3"][e][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(d2, full["dw2"][e][cols, :], rtol=1e-12, atol=1e-12)


def test_backward_shared_pin_catches_a_dropped_shared_path():
    """A copy of the oracle that forgets the shared experts' dX in dhidden fails
    the finite-difference pin."""
    import inspect
    src = inspect.getsource(O.moe_backward)
    old = 'dhidden += o["dx"]'
    assert old in src
    ns = dict(vars(O))
    exec(compile(src.replace(old, "pass"), "<mutant>", "exec"), ns)

    class M:
        moe_backward = staticmethod(ns["moe_backward"])
    inp = synth.make_inputs(10, 6, 4, 2, 5, "f32", 0.8, 3,
                            bias=np.array([0.5, 0.0, -0.3, 0.2], np.float32), n_shared=2,
                            f_shared=3)
    dy = np.random.default_rng(103).standard_normal((10, 6))
    g = _backward(inp, 2, 0.8, dy, 0.1, "drop", mod=M)
    assert _fd_agrees(inp, 2, 0.8, dy, 0.1, "drop", g) > 1e-3
