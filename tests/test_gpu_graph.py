"""The layer forward captured in a HIP graph: every replay matches the eager run.

All of the forward's work is the library's own kernels on the caller's stream
(counters are cleared by kernels, not memset nodes), so the whole step can be
captured once and replayed; each replay here is checked bitwise against the
eager result, with eager work and synchronisations between the replays.
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
    from mixture_experts_layer_sum_amd import moe as m
    return m


def _dev(a):
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("shape,overflow", [
    ((256, 1024, 64, 2, 512, 0.0), "drop"),          # decode-like: weight streaming kernels
    ((2048, 512, 8, 2, 512, 1.25), "drop"),          # MFMA tiles, capacity cut, k-split down
    ((1024, 512, 16, 2, 256, 0.8), "reroute"),       # second dispatch round
])
def test_forward_graph_replays_match_eager(moe, shape, overflow):
    T, d, N, k, f, cf = shape
    inp = synth.make_inputs(T, d, N, k, f, "bf16", cf, 4, zipf=True)
    h, wr, w1, w3, w2 = (_dev(inp.hidden), _dev(inp.w_router), _dev(inp.w1), _dev(inp.w3),
                         _dev(inp.w2))
    bias = torch.from_numpy(inp.bias).cuda()
    bufs = moe.MoEBuffers(T, d, N, k, f, torch.bfloat16)
    names = ("y", "logits", "topk_idx", "slot_row", "offsets", "y_perm", "aux")

    def run():
        moe.moe_forward(h, wr, w1, w3, w2, k, cf, bias, bufs, overflow=overflow)

    run()
    torch.cuda.synchronize()
    ref = {n: getattr(bufs, n).clone() for n in names}
    A = int(ref["offsets"][-1].item())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for n in names:                             # clobber the outputs between replays
            getattr(bufs, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            got, want = getattr(bufs, n), ref[n]
            if n in ("y_perm",):
                got, want = got[:A], want[:A]
            assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.uint8) if want.dtype == torch.bfloat16 else want), \
                f"replay {rep}: {n} differs from the eager run"


def test_training_step_graph_replays_match_eager(moe):
    """A training step -- the forward with moe_permute_noalloc (no workspace for the
    permutation) and h1 / h3 saved, then the backward that uses them -- captured in one
    graph: every replay matches the eager step bitwise."""
    T, d, N, k, f, cf = 1024, 512, 8, 2, 512, 1.25
    inp = synth.make_inputs(T, d, N, k, f, "bf16", cf, 6, zipf=True)
    h, wr, w1, w3, w2 = (_dev(inp.hidden), _dev(inp.w_router), _dev(inp.w1), _dev(inp.w3),
                         _dev(inp.w2))
    bias = torch.from_numpy(inp.bias).cuda()
    dy = _dev(synth.make_dy(T, d, "bf16", seed=6))
    b = moe.MoEBuffers(T, d, N, k, f, torch.bfloat16, save_for_backward=True)
    gb = moe.MoEGradBuffers(T, d, N, k, f, torch.bfloat16)

    def run():
        moe.moe_route(h, wr, k, bias, b.logits, b.topk_idx, b.topk_w, b.counts, b.ws_route)
        moe.moe_permute_noalloc(h, b.topk_idx, N, cf, b.x_perm, b.perm_src, b.slot_row, b.kept,
                                b.offsets)
        moe.moe_expert_up_save(b.x_perm, b.offsets, w1, w3, b.act, b.h13)
        moe.moe_expert_down(b.act, b.offsets, w2, b.y_perm, b.ws_down)
        moe.moe_combine(b.y_perm, b.slot_row, b.topk_w, torch.bfloat16, b.y)
        moe.moe_aux_loss(b.logits, b.counts, k, b.aux, b.ws_aux)
        moe.moe_combine_backward(dy, b.y_perm, b.slot_row, b.topk_w, gb.g_perm, gb.dgate)
        moe.moe_expert_backward_saved(b.x_perm, gb.g_perm, b.h13, b.offsets, w1, w3, w2,
                                      gb.dx_perm, gb.dw1, gb.dw3, gb.dw2, gb.ws_expert, act=b.act)
        moe.moe_router_backward(h, wr, b.logits, b.topk_idx, b.topk_w, b.counts, gb.dgate,
                                gb.dx_perm, b.slot_row, 0.01, gb.dhidden, gb.dw_router, gb.dbias,
                                True, gb.ws_router)

    outs = {"y": b, "aux": b, "slot_row": b, "dhidden": gb, "dw_router": gb, "dbias": gb,
            "dw1": gb, "dw3": gb, "dw2": gb}
    run()
    torch.cuda.synchronize()
    ref = {n: getattr(o, n).clone() for n, o in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for n, o in outs.items():
            getattr(o, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, o in outs.items():
            got, want = getattr(o, n), ref[n]
            if got.dtype == torch.bfloat16:
                got, want = got.view(torch.int16), want.view(torch.int16)
            assert torch.equal(got, want), f"replay {rep}: {n} differs from the eager step"
