"""The C ABI on the host: the library loads without a GPU, exports every symbol
include/moe.h declares, and rejects bad arguments before any HIP call.

Only argument-validation paths are exercised here (fake non-null pointers are
never dereferenced because validation fails first); nothing is launched.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("mixture_experts_layer_sum_amd.moe")
lib = moe._lib

OK, INV, UNS, WS = moe.MOE_OK, moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED, moe.MOE_ERR_WORKSPACE
BF16, F32 = moe.MOE_BF16, moe.MOE_F32
P = ctypes.c_void_p(4096)          # fake device address: never dereferenced
NUL = None
S = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_aux_loss"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.SIGNATURES)


def test_status_strings():
    for s in range(5):
        assert lib.moe_status_string(s).startswith(b"MOE_")
    assert lib.moe_status_string(99) == b"unknown moe_status"


def test_workspace_sizes():
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTE, 64, 128, 8, 2, 256, F32) == 0
    # bf16 router: partial logits when few token tiles split the hidden dim
    # bf16 batches of >= 2048 tokens: W_router transposed, 16 rows per expert tile
    # (tile count rounded up to a power of two)
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTE, 8192, 4096, 8, 2, 256, BF16) == 16 * 4096 * 2
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTE, 2048, 1024, 40, 2, 256, BF16) == 64 * 1024 * 2
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTE, 4096, 2048, 256, 2, 256, BF16) == 256 * 2048 * 2
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTE, 256, 4096, 128, 2, 256, BF16) == 16 * 256 * 128 * 4
    assert lib.moe_workspace_size(moe.MOE_OP_COMBINE, 64, 128, 8, 2, 256, F32) == 0
    # two int32 [chunks, N] tables, chunks of 256 tokens
    assert lib.moe_workspace_size(moe.MOE_OP_PERMUTE, 257, 128, 8, 2, 256, F32) == 2 * 2 * 8 * 4
    # re-routing: four chunk tables, first-round kept, three per-slot arrays
    assert lib.moe_workspace_size(moe.MOE_OP_PERMUTE_REROUTE, 257, 128, 8, 2, 256, F32) == \
        (4 * 2 * 8 + 8 + 3 * 257 * 2) * 4
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_FFN, 64, 128, 8, 2, 256, BF16) == 64 * 2 * 256 * 2
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_FFN, 64, 128, 8, 2, 256, F32) == 64 * 2 * 256 * 4
    # the k-split buffers of the down projection follow the current device (none here);
    # the fp32 path never uses them
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_DOWN, 64, 128, 8, 2, 256, F32) == 0
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_DOWN, 64, 128, 8, 0, 256, BF16) == 0
    # one fp32 [N] partial per 16 tokens
    assert lib.moe_workspace_size(moe.MOE_OP_AUX_LOSS, 256, 128, 8, 2, 256, F32) == 16 * 8 * 4
    assert lib.moe_workspace_size(moe.MOE_OP_AUX_LOSS, 65, 128, 8, 2, 256, F32) == 5 * 8 * 4
    assert lib.moe_workspace_size(17, 64, 128, 8, 2, 256, F32) == 0
    # backward: da fp32 [rows, f], [dh1 | dh3] [rows, 2f] and a [rows, f] in the layer dtype
    rows, f = 64 * 2, 256
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_BACKWARD, 64, 128, 8, 2, f, BF16) == \
        rows * f * 4 + rows * 2 * f * 2 + rows * f * 2
    assert lib.moe_workspace_size(moe.MOE_OP_EXPERT_BACKWARD, 64, 128, 8, 2, f, F32) == \
        rows * f * 4 + rows * 2 * f * 4 + rows * f * 4
    # router: dlogit [T, N], partial dW [ceil(T/64), d, N], partial dbias [ceil(T/64), N]
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTER_BACKWARD, 128, 256, 8, 2, 0, BF16) == \
        128 * 8 * 4 + 2 * 256 * 8 * 4 + 256
    assert lib.moe_workspace_size(moe.MOE_OP_ROUTER_BACKWARD, 128, 256, 300, 2, 0, BF16) == 0
    assert lib.moe_workspace_size(moe.MOE_OP_PERMUTE, 0, 128, 8, 2, 256, F32) == 0


def test_capacity_matches_oracle():
    """moe_capacity (the C the permute kernels apply) equals the oracle's
    capacity, floor((T*k)/N * CF) in double with P4 §3.1's operation order, at
    the pages' factors (P2 §3.4's working range 1.05-1.25, P4 §3.1's 1.5) and
    below 1, for every T below 70,000.  Narrowing the factor to fp32 before the
    product loses a row wherever (T*k)/N * CF is a whole number (CF 1.05:
    T 160, k 1, N 8 gives 21, fp32 gives 20), which the first asserts pin."""
    import oracle.moe_oracle as O
    assert lib.moe_capacity(160, 1, 8, 1.05) == O.capacity(160, 1, 8, 1.05) == 21
    assert lib.moe_capacity(80, 2, 8, 1.05) == O.capacity(80, 2, 8, 1.05) == 21
    assert math.floor(20 * float(ctypes.c_float(1.05).value)) == 20     # what fp32 would give
    assert lib.moe_capacity(65536, 1, 64, 1.2) == 1228                 # P5 §2.2 worked example
    assert lib.moe_capacity(4096, 2, 16, 1.25) == 640
    assert lib.moe_capacity(16384, 2, 64, 1.5) == 768
    cap = lib.moe_capacity
    for cf in (0.7, 1.05, 1.1, 1.2, 1.25, 1.5):
        for k in (1, 2):
            for N in (8, 16, 64, 128):
                bad = [T for T in range(1, 70000)
                       if cap(T, k, N, cf) != min(O.capacity(T, k, N, cf), T)]
                assert not bad, (cf, k, N, bad[:5])
    # no limit, and invalid arguments
    assert cap(300, 2, 8, 0.0) == 300 and cap(300, 2, 8, -1.0) == 300
    assert cap(10, 2, 8, 100.0) == 10                                  # clamped to T
    assert cap(0, 2, 8, 1.0) == -1 and cap(10, 9, 8, 1.0) == -1 and cap(10, 2, 8, math.nan) == -1


def route(**kw):
    a = dict(hidden=P, w_router=P, bias=NUL, T=64, d=128, N=8, k=2, dt=BF16, logits=P,
             topk_idx=P, topk_w=P, counts=P, ws=P, ws_bytes=1 << 30, stream=S)
    a.update(kw)
    return lib.moe_route(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=NUL), INV), (dict(w_router=NUL), INV), (dict(logits=NUL), INV),
    (dict(topk_idx=NUL), INV), (dict(topk_w=NUL), INV), (dict(counts=NUL), INV),
    (dict(T=0), INV), (dict(T=-3), INV), (dict(N=0), INV), (dict(k=0), INV), (dict(k=9), INV),
    (dict(d=0), INV), (dict(N=257, k=2), UNS), (dict(d=100), UNS), (dict(dt=2), UNS),
    (dict(T=2 ** 30, k=2), UNS), (dict(T=256, d=4096, N=128, ws_bytes=0), WS),
    (dict(T=256, d=4096, N=128, ws=NUL), INV),
])
def test_route_rejects(kw, status):
    assert route(**kw) == status


def permute(**kw):
    a = dict(hidden=P, topk_idx=P, T=300, d=128, N=8, k=2, cf=1.25, dt=BF16, x_perm=P,
             perm_src=P, slot_row=P, kept=P, offsets=P, ws=P, ws_bytes=1 << 20, stream=S)
    a.update(kw)
    return lib.moe_permute(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=NUL), INV), (dict(topk_idx=NUL), INV), (dict(x_perm=NUL), INV),
    (dict(perm_src=NUL), INV), (dict(slot_row=NUL), INV), (dict(kept=NUL), INV),
    (dict(offsets=NUL), INV), (dict(cf=math.nan), INV), (dict(k=0), INV), (dict(k=9), INV),
    (dict(T=0), INV), (dict(d=96), UNS), (dict(N=300), UNS), (dict(dt=7), UNS),
    (dict(ws_bytes=2 * 2 * 8 * 4 - 1), WS), (dict(ws=NUL), INV),
])
def test_permute_rejects(kw, status):
    assert permute(**kw) == status


def ffn(**kw):
    a = dict(x_perm=P, offsets=P, w1=P, w3=P, w2=P, N=8, d=256, f=256, max_rows=128, dt=BF16,
             y_perm=P, ws=P, ws_bytes=1 << 30, stream=S)
    a.update(kw)
    return lib.moe_expert_ffn(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x_perm=NUL), INV), (dict(offsets=NUL), INV), (dict(w1=NUL), INV), (dict(w3=NUL), INV),
    (dict(w2=NUL), INV), (dict(y_perm=NUL), INV), (dict(N=0), INV), (dict(d=0), INV),
    (dict(f=0), INV), (dict(max_rows=0), INV), (dict(N=257), UNS), (dict(d=320), UNS),
    (dict(f=192), UNS), (dict(d=128, dt=BF16), UNS), (dict(f=64, dt=F32, d=64), WS),
    (dict(dt=3), UNS), (dict(ws_bytes=128 * 256 * 2 - 1), WS), (dict(ws=NUL), INV),
])
def test_expert_ffn_rejects(kw, status):
    if kw.get("dt") == F32 and kw.get("f") == 64:
        # fp32 accepts d = f = 64; a too-small workspace is then the only error
        kw = dict(kw, ws_bytes=128 * 64 * 4 - 1)
    assert ffn(**kw) == status


M = ctypes.c_void_p(4096 + 8)      # fake device address, 8-byte but not 16-byte aligned


@pytest.mark.parametrize("call,names", [
    (route, ["hidden", "w_router", "bias", "logits", "topk_idx", "topk_w", "counts", "ws"]),
    (permute, ["hidden", "topk_idx", "x_perm", "perm_src", "slot_row", "kept", "offsets", "ws"]),
    (ffn, ["x_perm", "offsets", "w1", "w3", "w2", "y_perm", "ws"]),
], ids=["route", "permute", "expert_ffn"])
def test_misaligned_pointers_rejected(call, names):
    """Every device buffer must be 16-byte aligned (the kernels use 16-byte
    accesses); a misaligned one is an argument error caught before any launch."""
    for name in names:
        assert call(**{name: M}) == INV, name


def reroute(**kw):
    a = dict(hidden=P, topk_idx=P, logits=P, T=64, d=128, N=8, k=2, cf=1.0, dt=BF16, x_perm=P,
             perm_src=P, slot_row=P, kept=P, offsets=P, ws=P, ws_bytes=1 << 20, stream=S)
    a.update(kw)
    return lib.moe_permute_reroute(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(logits=NUL), INV), (dict(hidden=NUL), INV), (dict(ws=NUL), INV), (dict(cf=math.nan), INV),
    (dict(k=9), INV), (dict(T=0), INV), (dict(N=300), UNS), (dict(d=100), UNS), (dict(dt=7), UNS),
    (dict(ws_bytes=(4 * 1 * 8 + 8 + 3 * 64 * 2) * 4 - 1), WS),
])
def test_permute_reroute_rejects(kw, status):
    assert reroute(**kw) == status


def test_fp8_entry_points_reject():
    assert lib.moe_quantize_fp8(NUL, BF16, 2, 64, 64, P, P, S) == INV
    assert lib.moe_quantize_fp8(P, BF16, 0, 64, 64, P, P, S) == INV
    assert lib.moe_quantize_fp8(P, BF16, 2, 64, 64, NUL, P, S) == INV
    assert lib.moe_quantize_fp8(P, 5, 2, 64, 64, P, P, S) == UNS
    # up: null scale; too many rows per expert for the streaming kernel; d not a multiple of 256
    assert lib.moe_expert_up_fp8(P, P, P, P, NUL, P, 8, 256, 256, 64, P, S) == INV
    assert lib.moe_expert_up_fp8(P, P, P, P, P, P, 8, 256, 256, 8 * 33, P, S) == UNS
    assert lib.moe_expert_up_fp8(P, P, P, P, P, P, 8, 128, 256, 64, P, S) == UNS
    assert lib.moe_expert_down_fp8(P, P, P, NUL, 8, 256, 256, 64, P, S) == INV
    assert lib.moe_expert_down_fp8(P, P, P, P, 8, 256, 256, 8 * 33, P, S) == UNS
    assert lib.moe_expert_down_fp8(P, P, P, P, 8, 256, 192, 64, P, S) == UNS


def test_expert_matrix_size_limit():
    # d >= 2^21: a 256-row fp32 tile of y_perm is past the 32-bit offsets of the down projection
    assert lib.moe_expert_down(P, P, P, 8, 1 << 21, 128, 64, BF16, P, P, 1 << 40, S) == UNS
    # d * f * 2 bytes >= 2^31: one bf16 expert matrix is past the 31-bit resource range
    assert lib.moe_expert_up(P, P, P, P, 8, 32768, 32768, 64, BF16, P, S) == UNS
    assert lib.moe_expert_down(P, P, P, 8, 32768, 32768, 64, BF16, P, P, 1 << 40, S) == UNS
    assert lib.moe_expert_ffn(P, P, P, P, P, 8, 32768, 32768, 64, BF16, P, P, 1 << 40, S) == UNS


def test_expert_up_down_reject():
    assert lib.moe_expert_up(NUL, P, P, P, 8, 256, 256, 64, BF16, P, S) == INV
    assert lib.moe_expert_up(P, P, P, P, 8, 256, 200, 64, BF16, P, S) == UNS
    assert lib.moe_expert_down(P, P, NUL, 8, 256, 256, 64, BF16, P, P, 1 << 30, S) == INV
    assert lib.moe_expert_down(P, P, P, 8, 128, 256, 64, BF16, P, P, 1 << 30, S) == UNS
    assert lib.moe_expert_down(P, P, P, 8, 256, 256, 64, 3, P, P, 1 << 30, S) == UNS


@pytest.mark.parametrize("args,status", [
    ((NUL, P, P, NUL, 0, 64, 128, 2, BF16, P, S), INV), ((P, NUL, P, NUL, 0, 64, 128, 2, BF16, P, S), INV),
    ((P, P, NUL, NUL, 0, 64, 128, 2, BF16, P, S), INV), ((P, P, P, NUL, 0, 64, 128, 2, BF16, NUL, S), INV),
    ((P, P, P, NUL, 0, 0, 128, 2, BF16, P, S), INV), ((P, P, P, NUL, 0, 64, 128, 0, BF16, P, S), INV),
    ((P, P, P, NUL, 0, 64, 130, 2, BF16, P, S), UNS), ((P, P, P, NUL, 0, 64, 128, 2, 9, P, S), UNS),
    ((P, P, P, NUL, 0, 64, 128, 300, BF16, P, S), UNS),
    # shared experts: a count without outputs, or a negative count
    ((P, P, P, NUL, 1, 64, 128, 2, BF16, P, S), INV), ((P, P, P, P, -1, 64, 128, 2, BF16, P, S), INV),
])
def test_combine_rejects(args, status):
    assert lib.moe_combine(*args) == status


@pytest.mark.parametrize("args,status", [
    ((NUL, P, 64, 8, 2, P, P, 1024, S), INV), ((P, NUL, 64, 8, 2, P, P, 1024, S), INV),
    ((P, P, 64, 8, 2, NUL, P, 1024, S), INV), ((P, P, 64, 8, 9, P, P, 1024, S), INV),
    ((P, P, 0, 8, 2, P, P, 1024, S), INV), ((P, P, 64, 300, 2, P, P, 1 << 20, S), UNS),
    ((P, P, 64, 8, 2, P, P, 31, S), WS), ((P, P, 64, 8, 2, P, NUL, 1024, S), INV),
])
def test_aux_rejects(args, status):
    assert lib.moe_aux_loss(*args) == status


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        moe.load_library(str(tmp_path / "nope.so"))


def test_backward_entry_points_reject():
    # combine backward: null output, k = 0, d not a multiple of 64, unknown dtype
    assert lib.moe_combine_backward(P, P, P, P, 64, 128, 2, BF16, NUL, P, S) == INV
    assert lib.moe_combine_backward(P, P, P, P, 64, 128, 0, BF16, P, P, S) == INV
    assert lib.moe_combine_backward(P, P, P, P, 64, 100, 2, BF16, P, P, S) == UNS
    assert lib.moe_combine_backward(P, P, P, P, 64, 128, 2, 7, P, P, S) == UNS
    big = 1 << 40
    # expert backward: null gradient output; bf16 f not a multiple of 256; too many rows x f;
    # workspace too small; null workspace
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 256, 256, 64, BF16, P, NUL, P, P, P, big,
                                   S) == INV
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 256, 384, 64, BF16, P, P, P, P, P, big,
                                   S) == UNS
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 256, 16384, 1 << 15, BF16, P, P, P, P, P,
                                   big, S) == UNS
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 65536, 256, 1 << 14, BF16, P, P, P, P, P,
                                   big, S) == UNS
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 256, 256, 64, BF16, P, P, P, P, P, 1000,
                                   S) == WS
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 256, 256, 64, BF16, P, P, P, P, NUL, big,
                                   S) == INV
    # fp32 allows f a multiple of 64
    ws = lib.moe_workspace_size(moe.MOE_OP_EXPERT_BACKWARD, 64, 128, 8, 1, 192, F32)
    assert lib.moe_expert_backward(P, P, P, P, P, P, 8, 128, 192, 64, F32, P, P, P, P, P, ws - 1,
                                   S) == WS
    # backward with saved h1 / h3: null h13; bf16 f not a multiple of 256; workspace of
    # [dh1 | dh3] + a only (no da), one byte short; null workspace
    assert lib.moe_expert_backward_saved(P, P, NUL, P, P, P, P, P, 8, 256, 256, 64, BF16, P, P, P,
                                         P, P, big, S) == INV
    assert lib.moe_expert_backward_saved(P, P, P, P, P, P, P, P, 8, 256, 384, 64, BF16, P, P, P,
                                         P, P, big, S) == UNS
    rows, f = 64 * 2, 256
    wss = lib.moe_workspace_size(moe.MOE_OP_EXPERT_BACKWARD_SAVED, 64, 128, 8, 2, f, BF16)
    assert wss == rows * 2 * f * 2 + rows * f * 2
    assert lib.moe_expert_backward_saved(P, P, P, P, P, P, P, P, 8, 256, 256, rows, BF16, P, P, P,
                                         P, P, wss - 1, S) == WS
    assert lib.moe_expert_backward_saved(P, P, P, P, P, P, P, P, 8, 256, 256, rows, BF16, P, P, P,
                                         P, NUL, wss, S) == INV
    # the forward's activations are optional (NULL: recomputed): a null act alone is accepted
    # up to the workspace check
    assert lib.moe_expert_backward_saved(P, P, P, NUL, P, P, P, P, 8, 256, 256, rows, BF16, P, P,
                                         P, P, P, wss - 1, S) == WS
    # up projection that keeps h13: null h13; unsupported dtype
    assert lib.moe_expert_up_save(P, P, P, P, 8, 256, 256, 64, BF16, P, NUL, S) == INV
    assert lib.moe_expert_up_save(P, P, P, P, 8, 256, 256, 64, 5, P, P, S) == UNS
    # router backward: null dgate; NaN coefficient; k > N; workspace too small; null
    # workspace; shared count without their gradients; negative shared count
    args = [P, P, P, P, P, P, P, P, P, NUL, 0, 0.01, 64, 128, 8, 2, BF16, P, P, NUL, P, big, S]
    a = list(args); a[6] = NUL
    assert lib.moe_router_backward(*a) == INV
    a = list(args); a[11] = math.nan
    assert lib.moe_router_backward(*a) == INV
    a = list(args); a[15] = 9
    assert lib.moe_router_backward(*a) == INV
    a = list(args); a[21] = 100
    assert lib.moe_router_backward(*a) == WS
    a = list(args); a[20] = NUL
    assert lib.moe_router_backward(*a) == INV
    a = list(args); a[10] = 1
    assert lib.moe_router_backward(*a) == INV
    a = list(args); a[10] = -1; a[9] = P
    assert lib.moe_router_backward(*a) == INV


def test_plain_c_caller(tmp_path):
    """include/moe.h compiles as strict C99 and a C program linked against the library
    gets the documented capacities and argument errors (tests/c_abi_check.c)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    libdir = os.path.dirname(moe.LIB_PATH)
    libname = os.path.basename(moe.LIB_PATH)
    assert libname.startswith("lib") and libname.endswith(".so")
    exe = tmp_path / "c_abi_check"
    subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
                    "-L", libdir, "-l" + libname[3:-3], "-Wl,-rpath," + libdir, "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 failure(s)" in out.stdout
