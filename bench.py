"""Throughput of the top-k MoE SwiGLU layer forward on one MI355X.

A step is one pass of the whole layer (route, permute, up GEMM + SwiGLU, down
GEMM, combine, aux loss) over one batch of the Mixtral-shaped workload
(T 8192 = batch 4 x seq 2048, d 4096, 8 experts, top-2, f 14336, bf16, no
drop), with every input already resident in HBM and every buffer allocated
before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W]

Also reported in the same line:
  roofline      the up-projection grouped GEMM (the dominant kernel): its
                algorithmic flops per launch (4*A*d*f, A = routed rows) over
                its mean duration from HIP events on the launch stream,
                against the bf16 dense MFMA peak; HBM traffic per launch from
                rocprofv3 FETCH_SIZE/WRITE_SIZE when a committed counter
                summary matches the current kernel source, else null;
  backward      the backward pass of the Mixtral-shaped layer (gradients of
                <dy, y> + 0.01 * aux into hidden, the router and every expert's
                W1/W3/W2, fp32 gradients) after a training forward that keeps
                h1 / h3: its time, the expert GEMMs' rate (12*A*d*f flop: da
                with the SwiGLU backward, dx, dW1/dW3, dW2) against the bf16
                MFMA peak, the training forward, forward + backward per step,
                and the variant that recomputes h1 / h3 instead;
  decode_fp8    the decode-shaped layer with FP8 (OCP E4M3, per-column fp32
                scale) expert weights quantised on the GPU: bytes counted at one
                byte per weight plus the scales;
  shared_expert the Mixtral-shaped layer plus one always-on shared expert of
                the same size (f 14336), added with weight 1 in the combine;
  skewed_overflow  the skewed 64-expert workload (T 16384, d 4096, top-2, f 2048,
                CF 1.5, Zipf router bias): layer time with over-capacity
                assignments dropped and with them re-routed once;
  decode        the decode-shaped workload (T 256, d 4096, 128 experts, top-2,
                f 1536): layer time and the algorithmic bytes it must read
                (the weights of every expert that got a token, router weights,
                hidden and y) per second, against the HBM peak;
  n16_cf125     the 16-expert workload (T 4096, d 2048, top-2, f 5632, bf16,
                CF 1.25): time, tokens/s, TFLOP/s and % of the bf16 MFMA peak;
  tiny_fp32     the tiny fp32 layer (T 64, d 128, 8 experts, f 256): microseconds
                per layer (launch-latency bound);
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.

Helper modes for profiling (no timing claims):
  --copy-calibration MiB   also run a plain device copy of that size (read once,
                           written once) so rocprofv3 counters can be scaled
  --summarize-rocprof DIR  turn rocprofv3 csv output into a short text summary
  --write-traffic FETCH_DIR WRITE_DIR
                           turn two rocprofv3 --pmc runs (FETCH_SIZE, then
                           WRITE_SIZE, each with --copy-calibration) into the
                           per-launch HBM traffic record of the grouped GEMMs
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
UP_KERNEL = "grouped_gemm_bf16_kernel<true>"
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_sum_amd", "csrc", "expert_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "up_gemm_mixtral_T8192_traffic.json")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def src_hash(path=GEMM_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def upload(inp):
    import numpy as np
    import torch

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    return {k: t(getattr(inp, k)) for k in ("hidden", "w_router", "w1", "w3", "w2", "bias")}


def upload_shared(inp):
    import numpy as np
    import torch

    def t(a):
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)

    return (t(inp.w1s), t(inp.w3s), t(inp.w2s))


def time_layer(inp, dev, steps, warmup, overflow="drop", shared=None, fp8=None, save=False):
    """Warm up, then time `steps` forwards; per-step HIP events bracket the GEMMs.  With
    `save` the up projection also keeps h1 / h3 for the backward (training forward)."""
    import torch
    from mixture_experts_layer_sum_amd import moe
    T, d, N, k, f = inp.T, inp.d, inp.N, inp.k, inp.f
    ns = 0 if shared is None else shared[0].shape[0]
    b = moe.MoEBuffers(T, d, N, k, f, dev["hidden"].dtype, n_shared=ns,
                       f_shared=None if shared is None else shared[0].shape[2],
                       save_for_backward=save)
    s = torch.cuda.current_stream()

    def step(ev=None):
        moe.moe_route(dev["hidden"], dev["w_router"], k, dev["bias"], b.logits, b.topk_idx, b.topk_w,
                      b.counts, b.ws_route)
        if overflow == "drop":
            moe.moe_permute(dev["hidden"], b.topk_idx, N, inp.capacity_factor, b.x_perm,
                            b.perm_src, b.slot_row, b.kept, b.offsets, b.ws_permute)
        else:
            moe.moe_permute_reroute(dev["hidden"], b.topk_idx, b.logits, N, inp.capacity_factor,
                                    b.x_perm, b.perm_src, b.slot_row, b.kept, b.offsets,
                                    b.ws_permute)
        if ev:
            ev[0].record(s)
        if fp8 is None and save:
            moe.moe_expert_up_save(b.x_perm, b.offsets, dev["w1"], dev["w3"], b.act, b.h13)
        elif fp8 is None:
            moe.moe_expert_up(b.x_perm, b.offsets, dev["w1"], dev["w3"], b.act)
        else:
            moe.moe_expert_up_fp8(b.x_perm, b.offsets, fp8[0], fp8[1], fp8[3], fp8[4], b.act)
        if ev:
            ev[1].record(s)
        if fp8 is None:
            moe.moe_expert_down(b.act, b.offsets, dev["w2"], b.y_perm, b.ws_down)
        else:
            moe.moe_expert_down_fp8(b.act, b.offsets, fp8[2], fp8[5], b.y_perm)
        if ev:
            ev[2].record(s)
        if shared is not None:
            for q in range(shared[0].shape[0]):
                moe.moe_expert_ffn(dev["hidden"], b.shared_offsets, shared[0][q:q + 1],
                                   shared[1][q:q + 1], shared[2][q:q + 1], b.y_shared[q],
                                   b.ws_shared)
        moe.moe_combine(b.y_perm, b.slot_row, b.topk_w, dev["hidden"].dtype, b.y,
                        None if shared is None else b.y_shared)
        moe.moe_aux_loss(b.logits, b.counts, k, b.aux, b.ws_aux)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    up_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    down_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    kept = b.kept.cpu().numpy()
    A = int(b.offsets[-1].item())
    dropped = int((b.slot_row < 0).sum().item())
    return {"elapsed_s": elapsed, "ms_per_step": 1e3 * elapsed / steps, "up_ms": up_ms,
            "down_ms": down_ms, "A": A, "kept": kept, "aux": float(b.aux.item()),
            "dropped": dropped}


def time_backward(inp, dev, steps, warmup, coef=0.01, saved=True):
    """One forward (untimed), then `steps` backward passes; HIP events on the launch
    stream bracket the three backward entry points of each pass.  `saved`: the forward
    kept h1 / h3 and the expert backward uses them (else it recomputes them)."""
    import torch
    from mixture_experts_layer_sum_amd import moe, synth
    T, d, N, k, f = inp.T, inp.d, inp.N, inp.k, inp.f
    b = moe.moe_forward(dev["hidden"], dev["w_router"], dev["w1"], dev["w3"], dev["w2"], k,
                        inp.capacity_factor, dev["bias"], save_for_backward=saved)
    gb = moe.MoEGradBuffers(T, d, N, k, f, dev["hidden"].dtype)
    dyh = synth.make_dy(T, d, inp.dtype, seed=11)
    dy = (torch.from_numpy(dyh.view("int16")).cuda().view(torch.bfloat16) if inp.dtype == "bf16"
          else torch.from_numpy(dyh).cuda())
    s = torch.cuda.current_stream()
    want_db = dev["bias"] is not None

    def step(ev=None):
        if ev:
            ev[0].record(s)
        moe.moe_combine_backward(dy, b.y_perm, b.slot_row, b.topk_w, gb.g_perm, gb.dgate)
        if ev:
            ev[1].record(s)
        if saved:
            moe.moe_expert_backward_saved(b.x_perm, gb.g_perm, b.h13, b.offsets, dev["w1"],
                                          dev["w3"], dev["w2"], gb.dx_perm, gb.dw1, gb.dw3,
                                          gb.dw2, gb.ws_expert, act=b.act)
        else:
            moe.moe_expert_backward(b.x_perm, gb.g_perm, b.offsets, dev["w1"], dev["w3"],
                                    dev["w2"], gb.dx_perm, gb.dw1, gb.dw3, gb.dw2, gb.ws_expert)
        if ev:
            ev[2].record(s)
        moe.moe_router_backward(dev["hidden"], dev["w_router"], b.logits, b.topk_idx, b.topk_w,
                                b.counts, gb.dgate, gb.dx_perm, b.slot_row, coef, gb.dhidden,
                                gb.dw_router, gb.dbias, want_db, gb.ws_router)
        if ev:
            ev[3].record(s)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    part = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(3)]
    A = int(b.offsets[-1].item())
    del gb, b
    return {"ms_per_step": 1e3 * elapsed / steps, "combine_ms": part[0], "expert_ms": part[1],
            "router_ms": part[2], "A": A}


def layer_flops(inp, A):
    return 2.0 * inp.T * inp.d * inp.N + 6.0 * inp.d * inp.f * A


def layer_bytes(inp, kept, weight_bytes=None):
    s = 2 if inp.dtype == "bf16" else 4
    ws = s if weight_bytes is None else weight_bytes
    active = int((kept > 0).sum())
    return active * 3.0 * inp.d * inp.f * ws + inp.d * inp.N * s + 2.0 * inp.T * inp.d * s


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except Exception:  # pragma: no cover - informational only
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(inp, sample_tokens):
    """The oracle as it stands, on the first `sample_tokens` tokens of the same layer."""
    import oracle.moe_oracle as O
    from mixture_experts_layer_sum_amd import synth  # noqa: F401

    class View:
        def __init__(self, name):
            self.name = name

        def __getitem__(self, e):
            return inp.expert_values(self.name, e)

    S = min(sample_tokens, inp.T)
    hid = inp.values("hidden")[:S]
    t0 = time.perf_counter()
    O.moe_forward(hid, inp.values("w_router"), View("w1"), View("w3"), View("w2"), inp.k,
                  inp.capacity_factor, inp.bias)
    dt = time.perf_counter() - t0
    threads, api = blas_threads()
    return {"value": S / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full fp64 oracle forward (route, top-k, dispatch, per-expert SwiGLU, "
                      f"combine, aux) of the first {S} of {inp.T} tokens with the same weights; "
                      f"{dt:.1f} s; numpy BLAS {api}, {threads} threads"}


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB read + {mib} MiB written per copy, 3 copies")


def traffic_entry():
    """HBM bytes per launch of the up GEMM from committed counters, if they match this source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_source_sha256_16") != src_hash():
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(d, counter):
    import csv
    rows = []
    for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += [r for r in csv.DictReader(open(p)) if r.get("Counter_Name") == counter]
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def write_traffic(fetch_dir, write_dir, calib_mib, cmds):
    """HBM bytes per launch of both grouped GEMMs from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by what it reads for the calibration copy (`calib_mib` MiB read and
    written once, the largest __amd_rocclr_copyBuffer dispatches in the same run).
    """
    from mixture_experts_layer_sum_amd import synth
    w = synth.WORKLOADS["mixtral"]
    A = w.T * w.k                      # no capacity limit: every assignment is a routed row
    s = 2
    algo = {"up": A * w.d * s + 2 * w.N * w.d * w.f * s + A * w.f * s,
            "down": A * w.f * s + w.N * w.f * w.d * s + A * w.d * 4}
    names = {"up": "grouped_gemm_bf16_kernel<true>", "down": "grouped_gemm_bf16_kernel<false>"}
    calib_kib = calib_mib * 1024.0
    per = {}
    factor = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = [v for v in copies if v > 0.25 * calib_kib]
        if not big:
            raise SystemExit(f"no calibration copy found in {d}")
        factor[counter] = calib_kib / (sum(big) / len(big))
        for key, kname in names.items():
            vals = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
            per[(key, counter)] = sum(vals) / len(vals)
    src = os.path.relpath(GEMM_SRC, ROOT)
    recs = {}
    for key in ("up", "down"):
        rd = per[(key, "FETCH_SIZE")] * 1024 * factor["FETCH_SIZE"]
        wr = per[(key, "WRITE_SIZE")] * 1024 * factor["WRITE_SIZE"]
        recs[key] = {"kernel": names[key], "fetch_size_kib_per_dispatch": per[(key, "FETCH_SIZE")],
                     "write_size_kib_per_dispatch": per[(key, "WRITE_SIZE")],
                     "bytes_per_launch": rd + wr, "read_bytes_per_launch": rd,
                     "write_bytes_per_launch": wr, "algorithmic_bytes_per_launch": algo[key]}
    rec = dict(recs["up"])
    rec.update({"workload": f"{w.name} (seed 0, A = {A} routed rows)", "kernel_source": src,
                "kernel_source_sha256_16": src_hash(),
                "copy_calibration": {"mib": calib_mib, "fetch_factor": factor["FETCH_SIZE"],
                                     "write_factor": factor["WRITE_SIZE"]},
                "down": recs["down"], "commands": cmds})
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=2)
        fh.write("\n")
    md = [f"# HBM traffic of the grouped GEMMs, Mixtral-shaped layer (seed 0, A = {A} routed rows)",
          "", "Commands (repo root, on one MI355X; one counter per run):", ""]
    md += [f"    {c}" for c in cmds]
    md += ["", f"Calibration in the same processes: a plain {calib_mib} MiB device copy "
           f"(`--copy-calibration {calib_mib}`, torch `copy_`, runs as `__amd_rocclr_copyBuffer`); "
           f"FETCH_SIZE is scaled by {factor['FETCH_SIZE']:.3f} and WRITE_SIZE by "
           f"{factor['WRITE_SIZE']:.3f} so that the copy reads and writes its own size.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read GB | scaled write GB "
           "| algorithmic GB | traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
    for key in ("up", "down"):
        r = recs[key]
        md.append(f"| {key} `{r['kernel']}` | {r['fetch_size_kib_per_dispatch']:.0f} | "
                  f"{r['write_size_kib_per_dispatch']:.0f} | {r['read_bytes_per_launch']/1e9:.3f} | "
                  f"{r['write_bytes_per_launch']/1e9:.3f} | {r['algorithmic_bytes_per_launch']/1e9:.3f} | "
                  f"{r['bytes_per_launch']/r['algorithmic_bytes_per_launch']:.2f} |")
    md += ["", "Algorithmic bytes: up = x_perm rows (A*d) + W1 and W3 of the 8 experts (2*N*d*f) + "
           "activations written (A*f), bf16; down = activations (A*f) + W2 (N*f*d) bf16 + y_perm "
           "(A*d) fp32.  Reads above the algorithmic bytes are re-fetches of x_perm row tiles and "
           "weight column tiles that left the 4 MB per-XCD L2 between the tiles that use them.",
           f"Kernel source hash at collection time: {src_hash()} (`{src}`)."]
    out = os.path.join(ROOT, "profiles", "up_down_gemm_mixtral_T8192_hbm_traffic.md")
    with open(out, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


DECODE_KERNELS = {
    "bf16 up": "grouped_gemm_bf16_rows32_up2_kernel",
    "bf16 down": "grouped_gemm_bf16_rows32_kernel<false>",
    "fp8 up": "grouped_gemm_fp8_rows32_up2_kernel",
    "fp8 down": "grouped_gemm_fp8_rows32_kernel<false>",
}


def write_decode_traffic(fetch_dir, write_dir, calib_mib, active, cmds):
    """HBM bytes per launch of the decode-shaped layer's weight-streaming GEMMs (bf16 and FP8
    weights) from FETCH_SIZE / WRITE_SIZE, scaled by the calibration copy as in write_traffic."""
    from mixture_experts_layer_sum_amd import synth
    w = synth.WORKLOADS["decode"]
    A = w.T * w.k                      # no capacity limit
    algo = {"bf16 up": active * 2 * w.d * w.f * 2 + A * w.d * 2 + A * w.f * 2,
            "bf16 down": active * w.f * w.d * 2 + A * w.f * 2 + A * w.d * 4,
            "fp8 up": active * 2 * w.d * w.f + active * 2 * w.f * 4 + A * w.d * 2 + A * w.f * 2,
            "fp8 down": active * w.f * w.d + active * w.d * 4 + A * w.f * 2 + A * w.d * 4}
    weights = {"bf16 up": active * 2 * w.d * w.f * 2, "bf16 down": active * w.f * w.d * 2,
               "fp8 up": active * 2 * w.d * w.f, "fp8 down": active * w.f * w.d}
    calib_kib = calib_mib * 1024.0
    per, factor = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = [v for v in copies if v > 0.25 * calib_kib]
        if not big:
            raise SystemExit(f"no calibration copy found in {d}")
        factor[counter] = calib_kib / (sum(big) / len(big))
        for key, kname in DECODE_KERNELS.items():
            vals = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
            if not vals:
                raise SystemExit(f"no {kname} dispatches in {d}")
            per[(key, counter)] = sum(vals) / len(vals)
    md = [f"# HBM traffic of the decode-shaped layer's expert GEMMs ({w.name}, seed 0, "
          f"{active} active experts, A = {A} routed rows)", "",
          "Commands (repo root, on one MI355X; one counter per run):", ""]
    md += [f"    {c}" for c in cmds]
    md += ["", f"Calibration in the same processes: a plain {calib_mib} MiB device copy "
           f"(`--copy-calibration {calib_mib}`); FETCH_SIZE is scaled by "
           f"{factor['FETCH_SIZE']:.3f} and WRITE_SIZE by {factor['WRITE_SIZE']:.3f} so that the "
           "copy reads and writes its own size.  Values are means over every dispatch of the "
           "kernel in the run.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read GB | scaled write GB "
           "| algorithmic GB | weight bytes GB | traffic / algorithmic |",
           "|---|---|---|---|---|---|---|---|"]
    for key, kname in DECODE_KERNELS.items():
        rd = per[(key, "FETCH_SIZE")] * 1024 * factor["FETCH_SIZE"]
        wr = per[(key, "WRITE_SIZE")] * 1024 * factor["WRITE_SIZE"]
        md.append(f"| {key} `{kname}` | {per[(key, 'FETCH_SIZE')]:.0f} | "
                  f"{per[(key, 'WRITE_SIZE')]:.0f} | {rd/1e9:.4f} | {wr/1e9:.4f} | "
                  f"{algo[key]/1e9:.4f} | {weights[key]/1e9:.4f} | {(rd + wr)/algo[key]:.3f} |")
    md += ["", "Algorithmic bytes: the weights of every active expert (bf16: 2 bytes, FP8: 1 byte "
           "per weight, plus one fp32 scale per output column), the x_perm rows read and the "
           "activations written (up), the activations read and the fp32 y_perm written (down).",
           "The layer's HBM rate in bench.py's `decode` / `decode_fp8` objects is these "
           "algorithmic bytes over the event-timed layer."]
    out = os.path.join(ROOT, "profiles", "decode_T256_expert_gemm_hbm_traffic.md")
    with open(out, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_rocprof(d, out, skip_first=0):
    """Short text summary of rocprofv3 csv output in directory `d`.

    With `skip_first` W, a second table gives each kernel's mean over its dispatches after the
    first W (the warm-up forwards), the same dispatches bench.py's own events time.
    """
    import csv
    lines = []
    traces = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    for p in traces if skip_first else []:
        per = {}
        for r in csv.DictReader(open(p)):
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append(f"per-kernel mean after the first {skip_first} dispatches "
                     f"({os.path.relpath(p, d)}):")
        lines.append("| kernel | timed calls | mean us | min us | max us |")
        lines.append("|---|---|---|---|---|")
        for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            t = v[skip_first:]
            if t:
                lines.append(f"| {name[:90]} | {len(t)} | {sum(t)/len(t):.1f} | {min(t):.1f} | "
                             f"{max(t):.1f} |")
        lines.append("")
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    for p in stats:
        rows = list(csv.DictReader(open(p)))
        lines.append(f"kernel stats ({os.path.relpath(p, d)}):")
        lines.append("| kernel | calls | avg us | min us | max us | % time |")
        lines.append("|---|---|---|---|---|---|")
        for r in rows:
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                         f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                         f"{float(r['Percentage']):.2f} |")
    cc = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    for p in cc:
        rows = list(csv.DictReader(open(p)))
        agg = {}
        for r in rows:
            key = (r.get("Kernel_Name", "")[:90], r.get("Counter_Name", ""))
            agg.setdefault(key, []).append(float(r.get("Counter_Value", 0) or 0))
        lines.append(f"counters ({os.path.relpath(p, d)}), mean per dispatch:")
        lines.append("| kernel | counter | dispatches | mean value |")
        lines.append("|---|---|---|---|")
        for (kname, cname), vals in sorted(agg.items()):
            lines.append(f"| {kname} | {cname} | {len(vals)} | {sum(vals)/len(vals):.1f} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "a") as fh:
            fh.write(text)
    print(text)


def rates(inp, rs):
    """Rate fields of one timed layer: tokens/s, flops and algorithmic bytes per second,
    both roofline fractions, the routing outcome and the aux loss."""
    ms = rs["ms_per_step"]
    fl = layer_flops(inp, rs["A"])
    by = layer_bytes(inp, rs["kept"])
    tf = fl / (ms * 1e-3) / 1e12
    gbs = by / (ms * 1e-3) / 1e9
    return {"ms_per_step": ms, "us_per_step": 1e3 * ms, "tokens_per_s": inp.T / (ms * 1e-3),
            "layer_tflops": tf, "pct_mfma_peak": 100.0 * tf / PEAK_BF16_TFLOPS,
            "algorithmic_bytes": by, "GB_per_s": gbs, "pct_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS,
            "routed_rows": rs["A"], "dropped_assignments": rs["dropped"],
            "active_experts": int((rs["kept"] > 0).sum()), "aux": rs["aux"],
            "up_ms": rs["up_ms"], "down_ms": rs["down_ms"]}


def time_workload(key, args, steps):
    """One of the smaller workloads (tiny fp32, 16 experts with capacity), its own object."""
    import torch
    from mixture_experts_layer_sum_amd import synth
    wk = synth.WORKLOADS[key]
    log(f"generating {wk.name}")
    inp = synth.make_workload_inputs(key, seed=args.seed)
    devk = upload(inp)
    rs = time_layer(inp, devk, steps, args.warmup)
    out = {"workload": wk.name, "dtype": wk.dtype, "steps": steps}
    out.update(rates(inp, rs))
    if wk.dtype == "f32":
        # fp32 layers run on the VALU kernels: the fp32 vector peak is the matching roofline
        out["pct_fp32_peak"] = 100.0 * out["layer_tflops"] / PEAK_FP32_TFLOPS
        del out["pct_mfma_peak"]
    del devk
    torch.cuda.empty_cache()
    return out


def time_skewed(args):
    """The skewed-routing workload under both overflow policies."""
    import torch
    from mixture_experts_layer_sum_amd import synth
    ks = "skewed_zipf"
    wsk = synth.WORKLOADS[ks]
    log(f"generating {wsk.name}")
    inps = synth.make_workload_inputs(ks, seed=args.seed)
    devs = upload(inps)
    sk = {"workload": wsk.name}
    for pol in ("drop", "reroute"):
        rs = time_layer(inps, devs, max(args.steps, 20), args.warmup, overflow=pol)
        sk[pol] = rates(inps, rs)
    del devs
    torch.cuda.empty_cache()
    return sk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the Mixtral-shaped layer with one shared expert")
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the skewed 64-expert workload (drop vs re-route)")
    ap.add_argument("--only-skewed", action="store_true",
                    help="time only the skewed-routing workload (both overflow policies) and exit")
    ap.add_argument("--no-main", action="store_true",
                    help="profiling aid: time only the decode-shaped layer (no JSON line)")
    ap.add_argument("--fp8", action="store_true",
                    help="with --no-main: the decode-shaped layer with FP8 expert weights")
    ap.add_argument("--only-workload", default=None, choices=["n16_cf125", "tiny_fp32"],
                    help="time only that workload (log line, no JSON line) and exit")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the 16-expert (CF 1.25) and tiny fp32 workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass object")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    ap.add_argument("--summarize-rocprof", default=None, metavar="DIR")
    ap.add_argument("--summary-out", default=None)
    ap.add_argument("--skip-first", type=int, default=0,
                    help="with --summarize-rocprof: warm-up dispatches per kernel left out")
    ap.add_argument("--write-traffic", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--decode-both", action="store_true",
                    help="with --no-main: the decode-shaped layer with bf16, then FP8 weights")
    ap.add_argument("--write-decode-traffic", nargs=2, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--decode-active", type=int, default=0,
                    help="with --write-decode-traffic: active experts of the decode run")
    args = ap.parse_args()

    if args.write_decode_traffic:
        if args.decode_active < 1:
            raise SystemExit("--write-decode-traffic needs --decode-active (from the run's log)")
        cmds = [f"rocprofv3 --pmc {c} -d {dr} -o run --output-format csv -- python -u "
                f"bench.py --steps 3 --warmup 1 --no-main --decode-both "
                f"--copy-calibration {args.copy_calibration}"
                for c, dr in zip(("FETCH_SIZE", "WRITE_SIZE"), args.write_decode_traffic)]
        write_decode_traffic(*args.write_decode_traffic, args.copy_calibration,
                             args.decode_active, cmds)
        return 0

    if args.write_traffic:
        # the counter runs these two commands, with -d the directories given here
        cmds = [f"rocprofv3 --pmc {c} -d {dr} -o run --output-format csv -- python -u "
                f"bench.py --steps 2 --warmup 1 --no-decode --no-skewed --no-shared --no-backward "
                f"--no-small --no-cpu-baseline --copy-calibration {args.copy_calibration}"
                for c, dr in zip(("FETCH_SIZE", "WRITE_SIZE"), args.write_traffic)]
        write_traffic(*args.write_traffic, args.copy_calibration, cmds)
        return 0

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.summary_out, args.skip_first)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this layer's path runs on a single MI355X; "
              "a multi-GPU (expert-parallel) run is not built.", file=sys.stderr)
        return 2

    import torch
    from mixture_experts_layer_sum_amd import moe, synth  # noqa: F401  (fails loudly if unbuilt)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    if args.only_workload:
        r1 = time_workload(args.only_workload, args, max(args.steps, 20))
        log(f"{args.only_workload} only: " + json.dumps(r1))
        return 0

    if args.only_skewed:
        sk = time_skewed(args)
        log("skewed only: " + ", ".join(f"{p} {sk[p]['ms_per_step']:.3f} ms/step" for p in ("drop", "reroute")))
        return 0

    if args.no_main:
        kd = "decode"
        inpd = synth.make_workload_inputs(kd, seed=args.seed)
        devd = upload(inpd)
        variants = [False, True] if args.decode_both else [args.fp8]
        for use_fp8 in variants:
            fp8 = None
            if use_fp8:
                fq = [moe.moe_quantize_fp8(devd[n]) for n in ("w1", "w3", "w2")]
                fp8 = (fq[0][0], fq[1][0], fq[2][0], fq[0][1], fq[1][1], fq[2][1])
                torch.cuda.synchronize()
            rd = time_layer(inpd, devd, max(args.steps, 20) if not args.decode_both else args.steps,
                            args.warmup, fp8=fp8)
            log(f"decode only{' (fp8 weights)' if use_fp8 else ''}: {rd['ms_per_step']:.3f} ms/step, "
                f"up {rd['up_ms']:.3f} ms, down {rd['down_ms']:.3f} ms, "
                f"active experts {int((rd['kept'] > 0).sum())}, routed rows {rd['A']}")
        if args.copy_calibration:
            copy_calibration(args.copy_calibration)
        return 0

    key = "mixtral"
    w = synth.WORKLOADS[key]
    log(f"generating {w.name}")
    inp = synth.make_workload_inputs(key, seed=args.seed, n_shared=0 if args.no_shared else 1)
    dev = upload(inp)
    log("timing")
    r = time_layer(inp, dev, args.steps, args.warmup)
    A = r["A"]
    up_flops = 4.0 * A * inp.d * inp.f
    up_tflops = up_flops / (r["up_ms"] * 1e-3) / 1e12
    total_flops = layer_flops(inp, A)
    ms = r["ms_per_step"]
    value = inp.T / (ms * 1e-3)
    traffic = traffic_entry()
    out = {
        "metric": "MoE layer forward tokens/s (Mixtral-shaped layer)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded Gaussian, bf16)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "N": w.N, "k": w.k, "f": w.f,
                   "capacity_factor": w.capacity_factor, "seed": args.seed},
        "layer_tflops": total_flops / (ms * 1e-3) / 1e12,
        "layer_pct_mfma_peak": 100.0 * total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_ms": {"up_gemm_swiglu": r["up_ms"], "down_gemm": r["down_ms"],
                      "other_steps": ms - r["up_ms"] - r["down_ms"]},
        "roofline": {"kernel": UP_KERNEL, "bound": "mfma", "achieved": up_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": up_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "work_per_launch": f"4*A*d*f = {up_flops:.4e} flop, A={A}"},
    }
    if not args.no_shared:
        log("timing with one shared expert")
        sh = upload_shared(inp)
        rs = time_layer(inp, dev, args.steps, args.warmup, shared=sh)
        fl = layer_flops(inp, A) + 6.0 * inp.d * inp.w1s.shape[2] * inp.T
        out["shared_expert"] = {"workload": w.name + "_plus1shared_f" + str(inp.w1s.shape[2]),
                                "ms_per_step": rs["ms_per_step"],
                                "tokens_per_s": inp.T / (rs["ms_per_step"] * 1e-3),
                                "layer_tflops": fl / (rs["ms_per_step"] * 1e-3) / 1e12}
        del sh
    if not args.no_backward:
        log("timing the training forward and the backward pass")
        rt = time_layer(inp, dev, args.steps, args.warmup, save=True)
        rb = time_backward(inp, dev, args.steps, args.warmup, saved=True)
        rr = time_backward(inp, dev, args.steps, args.warmup, saved=False)
        # the expert backward's algorithmic flops: da, dx, dW2, dW1 | dW3 (12 A d f); the
        # recompute variant adds the 4 A d f of h1 / h3 again
        bfl = 12.0 * rb["A"] * inp.d * inp.f
        gt = bfl / (rb["expert_ms"] * 1e-3) / 1e12
        tfwd = rt["ms_per_step"]
        out["backward"] = {"workload": w.name + "_backward_auxcoef0.01",
                           "ms_per_step": rb["ms_per_step"],
                           "tokens_per_s": inp.T / (rb["ms_per_step"] * 1e-3),
                           "kernel_ms": {"combine_backward": rb["combine_ms"],
                                         "expert_backward": rb["expert_ms"],
                                         "router_backward": rb["router_ms"]},
                           "expert_gemm_tflops": gt, "expert_gemm_frac_mfma_peak": gt / PEAK_BF16_TFLOPS,
                           "work_per_launch": f"12*A*d*f = {bfl:.4e} flop over 4 GEMM launches "
                                              f"(h1 / h3 saved by the forward), A={rb['A']}",
                           "training_forward_ms": tfwd,
                           "training_forward_up_ms": rt["up_ms"],
                           "forward_plus_backward_ms": tfwd + rb["ms_per_step"],
                           "training_tokens_per_s": inp.T / ((tfwd + rb["ms_per_step"]) * 1e-3),
                           "recompute_variant": {
                               "ms_per_step": rr["ms_per_step"], "expert_backward_ms": rr["expert_ms"],
                               "forward_plus_backward_ms": ms + rr["ms_per_step"]}}
        torch.cuda.empty_cache()
    del dev
    torch.cuda.empty_cache()

    if not args.no_decode:
        kd = "decode"
        wd = synth.WORKLOADS[kd]
        log(f"generating {wd.name}")
        inpd = synth.make_workload_inputs(kd, seed=args.seed)
        devd = upload(inpd)
        rd = time_layer(inpd, devd, max(args.steps, 20), args.warmup)
        by = layer_bytes(inpd, rd["kept"])
        gbs = by / (rd["ms_per_step"] * 1e-3) / 1e9
        # the same layer with FP8 (E4M3, per-column scale) expert weights
        fq = [moe.moe_quantize_fp8(devd[n]) for n in ("w1", "w3", "w2")]
        fp8 = (fq[0][0], fq[1][0], fq[2][0], fq[0][1], fq[1][1], fq[2][1])
        torch.cuda.synchronize()
        rf = time_layer(inpd, devd, max(args.steps, 20), args.warmup, fp8=fp8)
        byf = layer_bytes(inpd, rf["kept"], weight_bytes=1) + \
            4.0 * int((rf["kept"] > 0).sum()) * (2 * inpd.f + inpd.d)        # column scales
        gbf = byf / (rf["ms_per_step"] * 1e-3) / 1e9
        out["decode_fp8"] = {"workload": wd.name + "_fp8e4m3_weights",
                             "ms_per_step": rf["ms_per_step"],
                             "tokens_per_s": wd.T / (rf["ms_per_step"] * 1e-3),
                             "algorithmic_bytes": byf, "GB_per_s": gbf,
                             "pct_hbm_peak": 100.0 * gbf / PEAK_HBM_GBS,
                             "up_ms": rf["up_ms"], "down_ms": rf["down_ms"]}
        del fq, fp8
        out["decode"] = {"workload": wd.name, "ms_per_step": rd["ms_per_step"],
                         "tokens_per_s": wd.T / (rd["ms_per_step"] * 1e-3),
                         "active_experts": int((rd["kept"] > 0).sum()), "algorithmic_bytes": by,
                         "GB_per_s": gbs, "pct_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS,
                         "up_ms": rd["up_ms"], "down_ms": rd["down_ms"]}
        del devd
        torch.cuda.empty_cache()

    if not args.no_skewed:
        out["skewed_overflow"] = time_skewed(args)
        torch.cuda.empty_cache()

    if not args.no_small:
        out["n16_cf125"] = time_workload("n16_cf125", args, max(args.steps, 20))
        out["tiny_fp32"] = time_workload("tiny_fp32", args, max(args.steps, 200))

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
