"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes are compared element by element (every token, every row); so are
the five workload shapes at full size, in the launch configuration bench.py
times, for two seeds: routing, counts and the permutation exact for every
token, and the layer output on every token.
"""
import numpy as np
import pytest

from mixture_experts_layer_sum_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from mixture_experts_layer_sum_amd import moe as m   # raises if the library is missing
    return m


def _run(inp, label, sample=None, audit=True, bufs=None, overflow="drop"):
    from tests import parity
    parity.log(f"{label}: T={inp.T} d={inp.d} N={inp.N} k={inp.k} f={inp.f} {inp.dtype} "
               f"cf={inp.capacity_factor} bias={'yes' if inp.bias is not None else 'no'} "
               f"overflow={overflow}")
    dev = parity.to_device(inp)
    g, b = parity.run_gpu(inp, dev, bufs, overflow=overflow)
    rep = parity.check(inp, g, sample=sample, label=label, audit=audit, overflow=overflow)
    return rep, g, dev, b


SMALL = [
    # label, T, d, N, k, f, dtype, cf, bias
    ("tiny_fp32_workload", 64, 128, 8, 2, 256, "f32", 0.0, None),
    ("f32_ragged_drop", 300, 128, 8, 2, 192, "f32", 1.0, "skew"),
    ("f32_k1", 77, 64, 4, 1, 64, "f32", 0.0, None),
    ("bf16_ragged_tail", 300, 256, 8, 2, 256, "bf16", 0.0, None),
    ("bf16_n16_cap", 1000, 512, 16, 2, 384, "bf16", 1.25, None),
    ("bf16_zipf_drops", 513, 256, 64, 2, 256, "bf16", 1.5, "zipf"),
    ("bf16_sparse_decode", 37, 256, 128, 2, 256, "bf16", 0.0, None),
    ("bf16_k4", 200, 256, 16, 4, 128, "bf16", 0.0, None),
    ("bf16_dense_k_eq_N", 96, 256, 8, 8, 128, "bf16", 0.0, None),
    ("bf16_single_token", 1, 256, 8, 2, 128, "bf16", 0.0, None),
    ("bf16_N_not_mult8", 130, 256, 12, 3, 128, "bf16", 0.8, None),
    ("bf16_N256", 70, 256, 256, 2, 128, "bf16", 0.0, None),
    ("bf16_all_dropped", 64, 256, 8, 2, 128, "bf16", 0.01, "skew"),
    ("bf16_big_expert_multi_tile", 1200, 256, 2, 2, 256, "bf16", 0.0, None),
    # 1025 rows per expert: five 256-row tiles balanced as 256, 256, 192, 192, 129 rows
    ("bf16_balanced_row_tiles", 1025, 256, 2, 2, 256, "bf16", 0.0, None),
    ("bf16_router_ksplit", 40, 1024, 64, 2, 128, "bf16", 0.0, None),
    ("bf16_router_ksplit_N200", 50, 1024, 200, 3, 128, "bf16", 0.0, None),
    # weight-streaming paths: 32-row tiles (some experts need two), 64-row tiles
    ("bf16_rows32_two_tiles", 300, 512, 32, 2, 256, "bf16", 0.0, None),
    ("bf16_rows64", 400, 512, 20, 2, 256, "bf16", 0.0, None),
    # up projection of the 32-row path: 256-column W1/W3 wave pairs (f % 256 == 0,
    # three column slices) and the 128-column kernel (f % 256 == 128)
    ("bf16_rows32_up_f768", 150, 256, 16, 2, 768, "bf16", 0.0, None),
    ("bf16_rows32_up_f384", 150, 256, 16, 2, 384, "bf16", 0.0, None),
    # 132 full row tiles x 2 column tiles = 264 tiles: on a 256-CU device the down
    # projection's last round (8 tiles) is split over k into 4 ranges each (f = 8192:
    # only tiles of at least 128 k-steps are split; every tile holds 256 rows, so the
    # grouped tile order applies rather than the heaviest-first one)
    ("bf16_down_ksplit4", 16896, 512, 2, 2, 8192, "bf16", 0.0, None),
    # short grids of unequal tiles run heaviest first: 7 experts of ~1400, ~1000,
    # ~300 and 47..71 rows (row tiles of 4, 3, 2 and 1 units of 64 rows)
    ("bf16_heaviest_first_mix", 1500, 256, 7, 2, 512, "bf16", 0.0, "skew"),
    # the large-batch router (>= 2048 tokens): 256 experts (16 expert tiles), 40 experts
    # (tiles padded to 4) with k = 3 and a capacity cut, and one token below the threshold
    ("bf16_router_wt_N256", 2048, 256, 256, 2, 128, "bf16", 0.0, None),
    ("bf16_router_wt_N40_k3", 2048, 256, 40, 3, 128, "bf16", 1.0, None),
    ("bf16_router_below_threshold", 2047, 256, 40, 3, 128, "bf16", 1.0, None),
    # capacity factors whose fp32 value lies below the decimal one, at shapes where
    # (T*k)/N * CF is a whole number (C = 21, 21, 7, 14): the capacity must follow
    # the double formula exactly (P2 §3.4's range starts at 1.05)
    ("bf16_cf105_T160_k1", 160, 256, 8, 1, 128, "bf16", 1.05, "skew"),
    ("bf16_cf105_T80_k2", 80, 256, 8, 2, 128, "bf16", 1.05, "skew"),
    ("bf16_cf07_T40_k2", 40, 256, 8, 2, 128, "bf16", 0.7, "skew"),
    ("f32_cf07_T160_N16_k1", 160, 128, 16, 1, 128, "f32", 0.7, "skew"),
    # the fp32 router: one wave per token up to 32 experts (24 experts: the 32-wide
    # accumulator set; k = 20: the token's top-k by the whole wave), the 64-token
    # block beyond 32 experts
    ("f32_router_N24", 100, 128, 24, 2, 128, "f32", 0.0, None),
    ("f32_router_N24_k20", 40, 64, 24, 20, 64, "f32", 0.0, None),
    ("f32_router_N40_k3", 90, 128, 40, 3, 128, "f32", 1.0, "skew"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(moe, case):
    label, T, d, N, k, f, dt, cf, bias = case
    b = None
    if bias == "zipf":
        b = synth.zipf_bias(N)
    elif bias == "skew":
        b = np.zeros(N, np.float32)
        b[: min(3, N)] = [3.0, 2.0, 1.0][: min(3, N)]
    for seed in (0, 1):
        inp = synth.make_inputs(T, d, N, k, f, dt, cf, seed, bias=b)
        _run(inp, f"{label}/seed{seed}")


@pytest.mark.parametrize("T", [64, 128])
def test_uniform_router_exact_ties(moe, T):
    """W_router = 0: every logit ties; lower ids win on both sides, aux is exactly 1
    (T = 64: the one-launch aux loss, T = 128: partial sums and a final pass)."""
    for dt in ("bf16", "f32"):
        inp = synth.make_inputs(T, 256, 8, 2, 128, dt, 1.25, 3)
        inp.w_router[:] = 0
        rep, g, _, _ = _run(inp, f"uniform_router_{dt}_T{T}", audit=False)
        assert (g["topk_idx"] == np.arange(2)).all()
        assert np.all(g["topk_w"] == 0.5)
        assert g["aux"] == 1.0


@pytest.mark.parametrize("T,N,k", [(2048, 8, 2), (4096, 64, 3), (2048, 40, 16), (2048, 24, 20)])
def test_uniform_router_exact_ties_large_batch(moe, T, N, k):
    """The large-batch router (transposed W_router, one thread per token for k <= 16,
    one wave per token above): with W_router = 0 every logit ties and experts
    0..k-1 win with weight 1/k."""
    inp = synth.make_inputs(T, 256, N, k, 128, "bf16", 0.0, 3)
    inp.w_router[:] = 0
    rep, g, _, _ = _run(inp, f"uniform_router_T{T}_N{N}_k{k}", audit=False)
    assert (g["topk_idx"] == np.arange(k)).all()
    assert np.all(np.abs(g["topk_w"] - 1.0 / k) <= 1e-7)
    assert abs(g["aux"] - 1.0) <= 1e-6


def test_zero_hidden_gives_zero(moe):
    inp = synth.make_inputs(64, 256, 8, 2, 128, "bf16", 0.0, 4)
    inp.hidden[:] = 0
    rep, g, _, _ = _run(inp, "zero_hidden", audit=False)
    assert (g["y"] == 0).all()


def test_deterministic_and_ffn_entry_matches_split(moe):
    """Two runs are bitwise identical; moe_expert_ffn equals moe_expert_up + moe_expert_down."""
    from tests import parity
    inp = synth.make_inputs(700, 512, 16, 2, 256, "bf16", 1.25, 5, bias=synth.zipf_bias(16))
    dev = parity.to_device(inp)
    g1, b = parity.run_gpu(inp, dev)
    g2, _ = parity.run_gpu(inp, dev, b)
    for key in g1:
        if isinstance(g1[key], np.ndarray):
            assert np.array_equal(g1[key], g2[key], equal_nan=True), key
    y_ffn = moe.moe_expert_ffn(b.x_perm, b.offsets, dev["w1"], dev["w3"], dev["w2"])
    torch.cuda.synchronize()
    A = g1["A"]
    assert torch.equal(y_ffn[:A], b.y_perm[:A])


def test_down_workspace_is_checked(moe):
    """The MFMA down projection needs its k-split workspace; a short one is refused."""
    import ctypes
    N, d, f, rows = 8, 256, 256, 4096
    need = moe.workspace_size(moe.MOE_OP_EXPERT_DOWN, rows, d, N, 1, f, torch.bfloat16)
    assert need > 0
    act = torch.zeros(rows, f, dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros(N, f, d, dtype=torch.bfloat16, device="cuda")
    offs = (torch.arange(N + 1, dtype=torch.int32, device="cuda") * (rows // N)).contiguous()
    y = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = moe._lib.moe_expert_down(act.data_ptr(), offs.data_ptr(), w2.data_ptr(), N, d, f, rows,
                                  moe.MOE_BF16, y.data_ptr(), ws.data_ptr(), need - 1,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == moe.MOE_ERR_WORKSPACE
    moe.moe_expert_down(act, offs, w2, y, ws)
    torch.cuda.synchronize()
    assert (y == 0).all()


REROUTE = [
    # label, T, d, N, k, f, dtype, cf, bias
    ("f32_reroute", 300, 128, 8, 2, 192, "f32", 1.0, "skew"),
    ("bf16_reroute_zipf", 513, 256, 64, 2, 256, "bf16", 1.5, "zipf"),
    ("bf16_reroute_k1", 200, 256, 8, 1, 128, "bf16", 0.6, "skew"),
    ("bf16_reroute_k4", 300, 256, 16, 4, 128, "bf16", 0.5, "skew"),
    ("bf16_reroute_no_room", 64, 256, 8, 2, 128, "bf16", 0.01, "skew"),
    ("bf16_reroute_many_chunks", 1500, 256, 16, 2, 128, "bf16", 0.75, "zipf"),
    # more experts than a wave has lanes: each lane holds several candidates
    ("bf16_reroute_N200", 400, 256, 200, 2, 128, "bf16", 0.8, "zipf"),
    ("bf16_reroute_N256_k3", 300, 256, 256, 3, 128, "bf16", 0.5, "skew"),
    # capacity factors below their decimal value in fp32 (C = 21, 21, 7)
    ("bf16_reroute_cf105_T160_k1", 160, 256, 8, 1, 128, "bf16", 1.05, "skew"),
    ("bf16_reroute_cf105_T80_k2", 80, 256, 8, 2, 128, "bf16", 1.05, "skew"),
    ("bf16_reroute_cf07_T40_k2", 40, 256, 8, 2, 128, "bf16", 0.7, "skew"),
]


@pytest.mark.parametrize("case", REROUTE, ids=[c[0] for c in REROUTE])
def test_reroute_small_shapes(moe, case):
    label, T, d, N, k, f, dt, cf, bias = case
    if bias == "zipf":
        b = synth.zipf_bias(N)
    else:
        b = np.zeros(N, np.float32)
        b[: min(3, N)] = [3.0, 2.0, 1.0][: min(3, N)]
    for seed in (0, 1):
        inp = synth.make_inputs(T, d, N, k, f, dt, cf, seed, bias=b)
        rep, g, _, _ = _run(inp, f"{label}/seed{seed}", overflow="reroute")
        import oracle.moe_oracle as O
        assert (g["kept"] <= O.capacity(T, k, N, cf)).all()


def _random_configs(n=24, seed=20261203):
    """Seeded draws across the documented limits: 1 to 256 experts (one expert, k = N
    and odd counts included), token counts that are not multiples of any tile, both
    dtypes, capacity factors with and without drops, both overflow policies.  The
    weight count N*d*f stays small enough for the oracle to finish in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "bf16" if rng.random() < 0.75 else "f32"
        N = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 64, 100, 256]))
        if dt == "bf16":
            d = int(rng.choice([256, 512, 768])) if N <= 16 else 256
            f = int(rng.choice([128, 256, 384, 512])) if N <= 16 else int(rng.choice([128, 256]))
        else:
            d = int(rng.choice([64, 128, 192, 256])) if N <= 16 else 64
            f = int(rng.choice([64, 128, 192])) if N <= 16 else 64
        k = int(rng.integers(1, min(N, 6) + 1))
        T = int(rng.integers(1, 800))
        cf = float(rng.choice([0.0, 0.5, 0.9, 1.0, 1.05, 1.25, 2.0]))
        bias = str(rng.choice(["none", "skew", "zipf"]))
        overflow = "reroute" if (cf > 0 and rng.random() < 0.35) else "drop"
        out.append((f"rand{i:02d}_{dt}_T{T}_d{d}_N{N}_k{k}_f{f}_cf{cf}_{bias}_{overflow}",
                    T, d, N, k, f, dt, cf, bias, overflow, i))
    return out


RANDOM = _random_configs()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_configs(moe, case):
    label, T, d, N, k, f, dt, cf, bias, overflow, seed = case
    b = None
    if bias == "zipf":
        b = synth.zipf_bias(N)
    elif bias == "skew":
        b = np.zeros(N, np.float32)
        b[: min(3, N)] = [3.0, 2.0, 1.0][: min(3, N)]
    inp = synth.make_inputs(T, d, N, k, f, dt, cf, 100 + seed, bias=b)
    _run(inp, label, overflow=overflow)


@pytest.mark.parametrize("N", [8, 130])
def test_reroute_exact_ties(moe, N):
    """W_router = 0: every logit ties, so experts 0..k-1 overflow and each dropped
    slot is re-routed to the lowest-id expert that has room and that the token
    does not hold yet (ties to the lower id, also across the lanes of a wave)."""
    inp = synth.make_inputs(64, 256, N, 2, 128, "bf16", 0.5 if N == 8 else 4.0, 3)
    inp.w_router[:] = 0
    rep, g, _, _ = _run(inp, f"reroute_ties_N{N}", audit=False, overflow="reroute")
    assert (g["topk_idx"] == np.arange(2)).all()
    assert (g["kept"][2:] > 0).any()


def test_reroute_workload_full_size(moe):
    """The skewed 64-expert workload (heavy overflow) with re-routing, y on sampled tokens."""
    inp = synth.make_workload_inputs("skewed_zipf", seed=0)
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, inp.T - 1], rng.choice(inp.T, 48, replace=False)]))
    rep, g, _, _ = _run(inp, "workload_skewed_zipf_reroute", sample=sample, overflow="reroute")
    assert rep["tokens_on_other_experts"] <= inp.T // 100


SHARED = [
    # label, T, d, N, k, f, dtype, cf, n_shared, f_shared, overflow
    ("f32_shared1", 64, 128, 8, 2, 256, "f32", 0.0, 1, 128, "drop"),
    ("bf16_shared1_drops", 300, 256, 8, 2, 256, "bf16", 1.0, 1, 384, "drop"),
    ("bf16_shared2_all_dropped", 64, 256, 8, 2, 128, "bf16", 0.01, 2, 256, "drop"),
    ("bf16_shared1_decode", 37, 256, 128, 2, 256, "bf16", 0.0, 1, 256, "drop"),
    ("bf16_shared1_reroute", 300, 256, 16, 2, 128, "bf16", 0.75, 1, 128, "reroute"),
]


@pytest.mark.parametrize("case", SHARED, ids=[c[0] for c in SHARED])
def test_shared_experts_small_shapes(moe, case):
    label, T, d, N, k, f, dt, cf, ns, fs, overflow = case
    b = np.zeros(N, np.float32)
    b[: min(3, N)] = [3.0, 2.0, 1.0][: min(3, N)]
    for seed in (0, 1):
        inp = synth.make_inputs(T, d, N, k, f, dt, cf, seed, bias=b, n_shared=ns, f_shared=fs)
        _run(inp, f"{label}/seed{seed}", overflow=overflow)


def test_shared_expert_mixtral_full_size(moe):
    """Mixtral-shaped layer plus one shared expert of the same size, y on sampled tokens."""
    inp = synth.make_workload_inputs("mixtral", seed=0, n_shared=1)
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([[0, inp.T - 1], rng.choice(inp.T, 32, replace=False)]))
    _run(inp, "workload_mixtral_shared1", sample=sample)


# ---------------------------------------------------------------- FP8 expert weights
def _dev_bf16(a):
    return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fp8_quantiser_is_bit_exact(moe, dt):
    """Codes and scales equal the oracle's own E4M3 quantisation, byte for byte."""
    import oracle.moe_oracle as O
    rng = np.random.default_rng(9)
    w = rng.standard_normal((3, 256, 384)).astype(np.float32)
    w[0, :, 5] = 0.0                                   # an all-zero column
    w[1, :, 7] *= 1e-6                                 # tiny values: subnormal codes
    w[2, :, 9] *= 300.0                                # large values
    w[2, 17, 11] = -w[2, :, 11].__abs__().max() * 2    # a lone negative peak
    if dt == "bf16":
        bits = synth.f32_to_bf16_bits(w)
        wv, wdev = synth.bf16_bits_to_f32(bits), _dev_bf16(bits)
    else:
        wv, wdev = w, torch.from_numpy(w).cuda()
    q, sc = moe.moe_quantize_fp8(wdev)
    torch.cuda.synchronize()
    q, sc = q.cpu().numpy(), sc.cpu().numpy()
    for e in range(3):
        rq, rs = O.quantize_fp8_columns(wv[e])
        assert np.array_equal(sc[e], rs), e
        assert np.array_equal(q[e], rq), e


def _fp8_layer(moe, inp, label, sample=None):
    """The layer with FP8 expert weights quantised on the GPU, against the oracle's layer on
    the oracle's own dequantised weights (same codes: the quantiser is bit-exact)."""
    import oracle.moe_oracle as O
    from tests import parity
    dev = parity.to_device(inp)
    q1, s1 = moe.moe_quantize_fp8(dev["w1"])
    q3, s3 = moe.moe_quantize_fp8(dev["w3"])
    q2, s2 = moe.moe_quantize_fp8(dev["w2"])
    b = moe.moe_forward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"], inp.k,
                        inp.capacity_factor, dev["bias"], fp8=(q1, q3, q2, s1, s3, s2))
    torch.cuda.synchronize()
    g = parity.host_results(b)

    class Deq:
        def __init__(self, name):
            self.name = name

        def __getitem__(self, e):
            qq, ss = O.quantize_fp8_columns(inp.expert_values(self.name, e))
            return O.dequantize_fp8_columns(qq, ss)

    ref = O.moe_forward(inp.values("hidden"), inp.values("w_router"), Deq("w1"), Deq("w3"),
                        Deq("w2"), inp.k, inp.capacity_factor, inp.bias, tokens=sample)
    same = (g["topk_idx"] == ref["topk_idx"]).all(1)
    # routing runs on the bf16 router (FP8 touches only the expert weights): a token
    # whose picks differ from the oracle's must be a near tie of the oracle's logits
    L32 = ref["logits"].astype(np.float32)
    ties = parity.near_ties(L32, inp.k)
    if inp.k > 1:
        sel = np.take_along_axis(L32.astype(np.float64), ref["topk_idx"], 1)
        ties = ties | (np.diff(-sel, axis=1) < parity.NEAR_TIE).any(1)
    assert (same | ties).all(), f"{label}: routing differs on tokens that are not near ties"
    parity.log(f"{label}: {int((~same).sum())} near-tie tokens left out of the y comparison")
    assert np.array_equal(g["slot_row"][same], ref["slot_row"][same]), label
    toks = ref["tokens"]
    ok = same[toks]
    yr, yg = ref["y"][ok], g["y"][toks][ok]
    rel = float(np.abs(yg - yr).max()) / float(np.abs(yr).max())
    parity.log(f"{label}: fp8 layer y rel {rel:.3e} on {ok.sum()} tokens")
    assert rel <= parity.Y_TOL["bf16"], f"{label}: y rel {rel:.3e}"
    return rel


@pytest.mark.parametrize("shape", [
    (37, 256, 16, 2, 256, None), (200, 512, 32, 2, 384, None), (1, 256, 8, 2, 128, None),
    (37, 512, 16, 2, 512, None), (1, 512, 8, 2, 512, None),
    # skewed routing: experts 0..2 take several 32-row tiles each
    (60, 1024, 16, 2, 1024, "skew")])
def test_fp8_layer_small(moe, shape):
    T, d, N, k, f, bias = shape
    b = None
    if bias == "skew":
        b = np.zeros(N, np.float32)
        b[:3] = [3.0, 2.0, 1.0]
    for seed in (0, 1):
        inp = synth.make_inputs(T, d, N, k, f, "bf16", 0.0, seed, bias=b)
        _fp8_layer(moe, inp, f"fp8_T{T}_d{d}_N{N}_f{f}/seed{seed}")


def test_fp8_decode_workload_full_size(moe):
    inp = synth.make_workload_inputs("decode", seed=0)
    _fp8_layer(moe, inp, "fp8_decode_T256", sample=np.arange(0, 256, 8))


WORKLOADS = ["tiny_fp32", "n16_cf125", "mixtral", "skewed_zipf", "decode"]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("key", WORKLOADS)
def test_workload_full_size(moe, key, seed):
    """Full-size workload, seeds 0 and 1, in the launch configuration the benchmark
    times: every token's routing and dispatch exact, every row of x_perm a bitwise
    copy, and y and y_perm compared with the oracle on every token and row."""
    inp = synth.make_workload_inputs(key, seed=seed)
    rep, g, dev, b = _run(inp, f"workload_{key}/seed{seed}", sample=None)
    # every token is compared unless a near tie (or a capacity cascade from one) moved it
    assert rep["tokens_compared"] + rep["excluded_near_ties"] + rep["tokens_on_other_experts"] >= inp.T
    if key == "skewed_zipf":
        assert rep["dropped_assignments"] > 0          # the Zipf bias makes capacity bite
