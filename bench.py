#!/usr/bin/env python3
"""Throughput of the STAPLE token-indexed FFN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (`value`): decode tokens/s of an OLMo-2-1B-shaped decode step, batch
64, through 12 augmented FFN layers whose 100352 x 8192 bf16 tables are all
resident in HBM; one step runs every layer back to back (the packed decode
gate/up kernel with the token-row gather in its epilogue, then the split-K
down-projection and its sum), timed both as eager launches and as replays of
one HIP graph; the faster is reported.

Also reported: `train`, tokens/s of one OLMo-2-1B-shaped training micro-batch
(32768 Zipf tokens) through one augmented layer (the timed step: dedup,
compact-row gather, forward, backward with the fp32 table-row segment-sum and
all weight and input gradients; the AdamW update of the touched table rows is
timed on its own and reported beside it, `adamw_table_rows`); `decode_stem`,
`train_stem`, the same two workloads for the STEM layer (no up-projection);
`decode_7b`, `train_7b` (OLMo-2-7B shapes: 16 decode layers over
100352 x 11008 tables, a 16384-token training batch); `train_lowrank` (the
1B training step with the low-rank r=512 table and its projection);
`offload_decode`, `offload_prefill` (64 prompts of 256 tokens through the 12
layers in chunks of 4096 or 8192 tokens, the faster reported; the next
chunk's rows fetched while the current chunk's layers run), `offload_train` (tables in
pinned host memory with a 5% HBM cache of the most frequent rows,
PCIe-inclusive).  Every workload carries its own `roofline`
object for its dominant kernel.  `--workloads` selects a subset (`prefill` is
the chunked prefill; it shares the pinned tables with `offload` when both run).

Every input is synthetic and seeded (staple_synth).  Inputs are resident in
HBM before timing starts.  The CPU oracle is timed on a bounded sample of the
same work on the host cores (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "STAPLE-FFN tokens/s (decode B=64; train fwd+bwd) + HBM GB/s / MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


WORKLOADS = ("decode", "train", "stem", "decode7b", "train7b", "offload", "prefill", "lowrank")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--train-steps", type=int, default=10)
    ap.add_argument("--train-warmup", type=int, default=3)
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="comma-separated subset of %(default)s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle baseline sample")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args(argv)
    unknown = sorted(set(args.workloads.split(",")) - set(WORKLOADS))
    if unknown:
        ap.error(f"unknown workloads {', '.join(unknown)}; choose from {', '.join(WORKLOADS)}")
    return args


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "token_indexed_ffn_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str, sha: str):
    """HBM bytes per launch of one kernel on one workload ("kernel/workload")
    from the committed counter summary, if it was taken on the current kernel
    source; otherwise None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return os.cpu_count() or 1


def host_cpu() -> dict:
    """The host the oracle runs on: logical CPUs the process may use, all
    logical CPUs, and the model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": usable, "cpus_total": os.cpu_count(), "cpu_model": model}


# ----------------------------------------------------------------------------
# Decode: 12 layers, batch 64, full tables in HBM
# ----------------------------------------------------------------------------
def setup_decode(torch, st, w, stem=False):
    """stem: the STEM layer (no up-projection, u = E[t]) instead of STAPLE's."""
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    L, n, d, f, v = w.n_layers, w.n_tokens, w.d_model, w.d_ff, w.vocab
    ids_np = w.ids()
    layers = []
    for l in range(L):
        s = w.layer_seeds(l)
        layers.append({
            "x": device_normal((n, d), w.x_std, s["x"], torch.bfloat16, dev),
            "w_gate": device_normal((f, d), w.w_std, s["w_gate"], torch.bfloat16, dev),
            "w_up": None if stem else device_normal((f, d), w.w_std, s["w_up"], torch.bfloat16, dev),
            "w_down": device_normal((d, f), w.w_std, s["w_down"], torch.bfloat16, dev),
            "table": device_normal((v, f), w.table_std, s["table"], torch.bfloat16, dev),
            "y": torch.empty(n, d, dtype=torch.bfloat16, device=dev),
        })
        lay = layers[-1]
        # the serving layout: packed once when the weights are loaded
        lay["pgu"], lay["pd"] = st.staple_decode_pack_weights(lay["w_gate"], lay["w_up"],
                                                              lay["w_down"], d_model=d, d_ff=f)
        torch.cuda.synchronize()
    ids = torch.from_numpy(ids_np).to(dev)
    h = torch.empty(n, f, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(st.lib().staple_ffn_fwd_workspace_bytes(n, d, f, 1), dtype=torch.uint8,
                     device=dev)
    return {"layers": layers, "ids": ids, "ids_np": ids_np, "h": h, "fwd_ws": ws}


def decode_step(st, D):
    ids = D["ids"]
    for lay in D["layers"]:
        st.staple_ffn_fwd_packed(lay["x"], lay["pgu"], lay["pd"], lay["table"], ids,
                                 d_ff=lay["w_gate"].shape[0], out={"y": lay["y"]},
                                 workspace=D["fwd_ws"])


def decode_step_row_major(st, D):
    ids = D["ids"]
    for lay in D["layers"]:
        st.staple_ffn_fwd(lay["x"], lay["w_gate"], lay["w_up"], lay["w_down"], lay["table"], ids,
                          out={"y": lay["y"]}, workspace=D["fwd_ws"])


def run_decode(torch, st, w, steps, warmup, stem=False):
    import numpy as np
    D = setup_decode(torch, st, w, stem)
    n, d, f = w.n_tokens, w.d_model, w.d_ff
    n_unique = int(len(np.unique(D["ids_np"])))
    for _ in range(3):
        decode_step(st, D)
    torch.cuda.synchronize()
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error during decode warmup")

    # eager launches, timed like the graph replays below
    for _ in range(warmup):
        decode_step(st, D)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        decode_step(st, D)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / steps * 1e3

    # the same step on the row-major weights, for comparison
    for _ in range(warmup):
        decode_step_row_major(st, D)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        decode_step_row_major(st, D)
    torch.cuda.synchronize()
    row_major_ms = (time.perf_counter() - t0) / steps * 1e3

    # one decode step captured as a HIP graph
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        decode_step(st, D)   # warm the capture stream
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            decode_step(st, D)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    graph_ms = elapsed / steps * 1e3
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error during decode timing")
    # the step's figure is the faster of the two ways of launching it
    launch = "HIP graph replay" if graph_ms <= eager_ms else "eager launches"
    ms = min(graph_ms, eager_ms)

    # dominant kernel: the fused gate/up kernel, one launch per layer
    gu_us = decode_gate_up_us(torch, st, [(lay["x"], lay["pgu"], lay["table"]) for lay in D["layers"]],
                              D["ids"], D["h"], max(20, steps // 2))

    n_w = 1 if stem else 2
    gu_bytes = (n_w * d * f + n * d + n_unique * f + n * f) * 2    # W_gate (+ W_up), x, rows, h
    down_bytes = (d * f + n * f + n * d) * 2                        # W_down, h, y
    step_bytes = w.n_layers * (gu_bytes + down_bytes)
    sha = source_sha("decode.hip", "common.h")
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    res = {
        "ms_per_step": ms,
        "tokens_per_s": n / (ms * 1e-3),
        "launch": launch,
        "graph_ms_per_step": graph_ms,
        "eager_ms_per_step": eager_ms,
        "row_major_eager_ms_per_step": row_major_ms,
        "weights": "packed decode layout (staple_decode_pack_weights, once at load)",
        "step_hbm_gb_s": step_bytes / (ms * 1e-3) / 1e9,
        "step_bytes": step_bytes,
        "n_unique": n_unique,
        "roofline": {
            "kernel": "decode_gateup_kernel (staple_ffn_gate_up_packed, 64 tokens"
                      + (", STEM gate-only)" if stem else ")"),
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_from_profile(f"decode_gate_up/{w.name}" + ("_stem" if stem else ""), sha),
            "avg_launch_us": gu_us, "algorithmic_bytes_per_launch": gu_bytes,
        },
    }
    return res, D


def decode_gate_up_us(torch, st, layers, index, h, reps):
    """Average duration of one decode gate/up launch: a HIP graph holds one
    staple_ffn_gate_up_packed per (x, packed weights, rows) of `layers`, all on
    the graph's capture stream, and HIP events on that stream bracket `reps`
    replays."""
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    gg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for x, pgu, rows in layers:        # warm the capture stream
            st.staple_ffn_gate_up_packed(x, pgu, rows, index, h)
        cap.synchronize()
        with torch.cuda.graph(gg, stream=cap):
            for x, pgu, rows in layers:
                st.staple_ffn_gate_up_packed(x, pgu, rows, index, h)
    torch.cuda.synchronize()
    for _ in range(5):
        gg.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cap):
        e0.record(cap)
        for _ in range(reps):
            gg.replay()
        e1.record(cap)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(layers)) * 1e3


def decode_cpu_baseline(torch, w, D, seconds):
    """Oracle forward of the decode step on the host, layer by layer, until
    `seconds` of CPU time have been spent in the oracle; tokens/s is scaled to
    the whole 12-layer step."""
    import numpy as np
    from oracle import staple_oracle as O
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    ids = D["ids_np"]
    uniq = np.unique(ids)
    cache = {}
    layer_times = []
    l = 0
    while sum(layer_times) < seconds and l < 4 * w.n_layers:
        li = l % w.n_layers
        if li not in cache:
            if len(cache) >= 3:
                cache.pop(next(iter(cache)))
            lay = D["layers"][li]
            idx = torch.from_numpy(uniq.astype(np.int64)).to(lay["table"].device)
            cache[li] = [f64(lay[k]) for k in ("x", "w_gate", "w_up", "w_down")] + \
                        [_Rows(uniq, f64(lay["table"][idx]))]
        x, wg, wu, wd, table = cache[li]
        t0 = time.perf_counter()
        O.ffn_forward(x, wg, wu, wd, table, ids, precision=O.BF16)
        layer_times.append(time.perf_counter() - t0)
        l += 1
    per_layer = float(np.mean(layer_times))
    return {"value": w.n_tokens / (per_layer * w.n_layers), "unit": "tokens/s",
            "cores": oracle_threads(), "kind": "oracle", **host_cpu(),
            "sample": f"{len(layer_times)} layer forwards of the 64-token decode batch "
                      f"(float64 numpy, bf16 rounding points), scaled to {w.n_layers} layers"}


class _Rows:
    """Table stand-in holding only the rows of the given sorted IDs."""

    def __init__(self, ids_sorted, rows):
        import numpy as np
        self.ids = np.asarray(ids_sorted)
        self.rows = rows

    def __getitem__(self, key):
        import numpy as np
        if isinstance(key, tuple):
            r, c = key
            r = np.asarray(r).reshape(-1)
            return self.rows[np.searchsorted(self.ids, r)][:, np.asarray(c).reshape(-1)]
        return self.rows[np.searchsorted(self.ids, np.asarray(key))]


# ----------------------------------------------------------------------------
# Training micro-batch: one layer, fwd + bwd
# ----------------------------------------------------------------------------
def setup_train(torch, st, w, stem=False):
    """stem: the STEM layer (no up-projection, u = E[t]) instead of STAPLE's."""
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v = w.n_tokens, w.d_model, w.d_ff, w.vocab
    s = w.layer_seeds(0)
    T = {
        "ids_np": w.ids(),
        "x": device_normal((n, d), w.x_std, s["x"], torch.bfloat16, dev),
        "w_gate": device_normal((f, d), w.w_std, s["w_gate"], torch.bfloat16, dev),
        "w_up": None if stem else device_normal((f, d), w.w_std, s["w_up"], torch.bfloat16, dev),
        "w_down": device_normal((d, f), w.w_std, s["w_down"], torch.bfloat16, dev),
        "table": device_normal((v, f), w.table_std, s["table"], torch.bfloat16, dev),
        "dy": device_normal((n, d), w.dy_std, s["dy"], torch.bfloat16, dev),
    }
    T["ids"] = torch.from_numpy(T["ids_np"]).to(dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    T["dd"] = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
               "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
               "n_unique": torch.empty(1, **i32)}
    T["dd_ws"] = torch.empty(max(st.lib().staple_dedup_workspace_bytes(n), 1), dtype=torch.uint8,
                             device=dev)
    T["rows"] = torch.empty(n, f, **bf)
    T["fwd"] = {"y": torch.empty(n, d, **bf), "g": torch.empty(n, f, **bf),
                "u": torch.empty(n, f, **bf), "h": torch.empty(n, f, **bf)}
    T["bwd"] = {"d_rows": torch.empty(n, f, **f32), "dx": torch.empty(n, d, **bf),
                "dw_gate": torch.empty(f, d, **f32),
                "dw_up": None if stem else torch.empty(f, d, **f32),
                "dw_down": torch.empty(d, f, **f32)}
    T["bwd_ws"] = torch.empty(st.lib().staple_ffn_bwd_workspace_bytes(n, d, f, 1), dtype=torch.uint8,
                              device=dev)
    torch.cuda.synchronize()
    return T


def train_step(st, T, vocab, events=None):
    dd = st.staple_dedup(T["ids"], vocab, out=T["dd"], workspace=T["dd_ws"])
    st.staple_gather_rows(T["table"], dd["uniq"], dd["n_unique"], out=T["rows"])
    fw = T["fwd"]
    if events:
        events[0].record()
    st.staple_ffn_gate_up(T["x"], T["w_gate"], T["w_up"], T["rows"], dd["inv"], fw["h"],
                          fw["g"], fw["u"])
    if events:
        events[1].record()
    st.staple_ffn_down(fw["h"], T["w_down"], fw["y"])
    st.staple_ffn_bwd_table_grad(T["dy"], T["x"], T["w_gate"], T["w_up"], T["w_down"], fw["g"],
                                 fw["u"], fw["h"], dd["sorted_pos"], dd["seg_start"],
                                 dd["n_unique"], inv=dd["inv"], out=T["bwd"],
                                 workspace=T["bwd_ws"])


def run_train(torch, st, w, steps, warmup, stem=False):
    T = setup_train(torch, st, w, stem)
    n, d, f = w.n_tokens, w.d_model, w.d_ff
    for _ in range(warmup):
        train_step(st, T, w.vocab)
    torch.cuda.synchronize()
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error during train warmup")
    t0 = time.perf_counter()
    for _ in range(steps):
        train_step(st, T, w.vocab)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    # dominant kernel timing: the fused gate/up GEMM, events around each launch
    durs = []
    for _ in range(max(3, steps // 2)):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        train_step(st, T, w.vocab, events=ev)
        torch.cuda.synchronize()
        durs.append(ev[0].elapsed_time(ev[1]) * 1e3)
    gu_us = sum(durs) / len(durs)
    # STAPLE: gate/up 4ndf + down 2ndf forward, twice that backward; STEM has
    # no up-projection: gate 2ndf + down 2ndf forward, twice that backward
    flops_total = (12 if stem else 18) * n * d * f
    gu_flops = (2 if stem else 4) * n * d * f
    achieved = gu_flops / (gu_us * 1e-6) / 1e12
    adamw = None if stem else run_device_adamw(torch, st, T, w, reps=max(5, steps))
    return {
        "workload": w.name, "tokens": n, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3),
        "step_tflops": flops_total / (ms * 1e-3) / 1e12,
        "step_mfma_frac": flops_total / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "n_unique": int(T["dd"]["n_unique"].item()),
        "roofline": {
            "kernel": ("gemm_kernel<bf16,GateStem> (staple_ffn_gate_up, w_up NULL, training batch)"
                       if stem else "gemm_kernel<bf16,GateUp> (staple_ffn_gate_up, training batch)"),
            "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / BF16_PEAK_TFLOPS,
            "traffic": traffic_from_profile(f"train_gate_up/{w.name}" + ("_stem" if stem else ""),
                                            source_sha("gemm.hip", "common.h")),
            "avg_launch_us": gu_us, "algorithmic_flops_per_launch": gu_flops,
        },
        **({"adamw_table_rows": adamw} if adamw else {}),
    }, T


def run_train_lowrank(torch, st, w, r, steps, warmup):
    """The training step of the low-rank table layer (table E_r of width r and
    projection P [d_ff x r]): dedup, R_r = E_r[uniq], Z = R_r P^T, the layer's
    forward and backward over Z, then dE_r and dP (staple_lowrank_bwd)."""
    import numpy as np
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v = w.n_tokens, w.d_model, w.d_ff, w.vocab
    T = setup_train(torch, st, w)
    s = w.layer_seeds(0)
    del T["table"]
    torch.cuda.empty_cache()
    T["table_r"] = device_normal((v, r), w.table_std, s["table"], torch.bfloat16, dev)
    T["proj"] = device_normal((f, r), w.w_std, s["w_up"] + 1000, torch.bfloat16, dev)
    T["rows_r"] = torch.empty(n, r, dtype=torch.bfloat16, device=dev)
    lr_out = {"d_rows_r": torch.empty(n, r, dtype=torch.float32, device=dev),
              "d_proj": torch.empty(f, r, dtype=torch.float32, device=dev)}
    lr_ws = torch.empty(max(st.lib().staple_lowrank_bwd_workspace_bytes(n, f, 1), 1),
                        dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(timed=False):
        dd = st.staple_dedup(T["ids"], v, out=T["dd"], workspace=T["dd_ws"])
        st.staple_gather_rows(T["table_r"], dd["uniq"], dd["n_unique"], out=T["rows_r"])
        if timed:
            ev[0].record()
        st.staple_lowrank_expand(T["rows_r"], dd["n_unique"], T["proj"], out=T["rows"])
        if timed:
            ev[1].record()
        fw = T["fwd"]
        st.staple_ffn_gate_up(T["x"], T["w_gate"], T["w_up"], T["rows"], dd["inv"], fw["h"],
                              fw["g"], fw["u"])
        st.staple_ffn_down(fw["h"], T["w_down"], fw["y"])
        st.staple_ffn_bwd_table_grad(T["dy"], T["x"], T["w_gate"], T["w_up"], T["w_down"], fw["g"],
                                     fw["u"], fw["h"], dd["sorted_pos"], dd["seg_start"],
                                     dd["n_unique"], inv=dd["inv"], out=T["bwd"],
                                     workspace=T["bwd_ws"])
        if timed:
            ev[2].record()
        st.staple_lowrank_bwd(T["bwd"]["d_rows"], T["rows_r"], dd["n_unique"], T["proj"],
                              out=lr_out, workspace=lr_ws)
        if timed:
            ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error in the low-rank training step")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    exp_us, bwd_us = [], []
    for _ in range(3):
        step(timed=True)
        torch.cuda.synchronize()
        exp_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
        bwd_us.append(ev[2].elapsed_time(ev[3]) * 1e3)
    u = int(T["dd"]["n_unique"].item())
    flops_total = 18 * n * d * f + 6 * u * r * f
    # dominant kernel: the gate/up GEMM, the same launch as the full-width
    # layer's (its rows are Z instead of E[uniq])
    gu_us = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        e0.record()
        st.staple_ffn_gate_up(T["x"], T["w_gate"], T["w_up"], T["rows"], T["dd"]["inv"],
                              T["fwd"]["h"], T["fwd"]["g"], T["fwd"]["u"])
        e1.record()
        torch.cuda.synchronize()
        gu_us.append(e0.elapsed_time(e1) * 1e3)
    gu = float(np.median(gu_us))
    gu_flops = 4 * n * d * f
    out = {"workload": w.name + f"_lowrank_r{r}", "tokens": n, "rank": r, "ms_per_step": ms,
           "tokens_per_s": n / (ms * 1e-3), "n_unique": u,
           "step_tflops": flops_total / (ms * 1e-3) / 1e12,
           "step_mfma_frac": flops_total / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
           "expand_us": float(np.median(exp_us)), "lowrank_bwd_us": float(np.median(bwd_us)),
           "table_bytes": v * r * 2, "full_width_table_bytes": v * f * 2,
           "roofline": {"kernel": "gemm_kernel<bf16,GateUp> (staple_ffn_gate_up over Z)",
                        "bound": "mfma", "achieved": gu_flops / (gu * 1e-6) / 1e12,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": gu_flops / (gu * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                        "traffic": traffic_from_profile(f"train_gate_up/{w.name}_lowrank_r{r}",
                                                        source_sha("gemm.hip", "common.h")),
                        "avg_launch_us": gu,
                        "algorithmic_flops_per_launch": gu_flops},
           "note": "step: dedup, R_r = E_r[uniq] (U x r), Z = R_r P^T (staple_lowrank_expand), "
                   "gate/up over Z, down, backward, dE_r and dP (staple_lowrank_bwd); FLOPs "
                   "18 N d f + 6 U r f"}
    del T, lr_out, lr_ws
    torch.cuda.empty_cache()
    return out


def run_device_adamw(torch, st, T, w, reps):
    """AdamW on the batch's unique table rows, table and fp32 moments in HBM,
    gradients from the step's d_rows; events around the launches."""
    dev = T["table"].device
    vocab, f = T["table"].shape
    m = torch.zeros(vocab, f, dtype=torch.float32, device=dev)
    v = torch.zeros(vocab, f, dtype=torch.float32, device=dev)
    dd, g = T["dd"], T["bwd"]["d_rows"]
    kw = dict(lr=3e-4, weight_decay=1e-4, n_rows=dd["n_unique"])
    st.staple_adamw_rows(T["table"], m, v, dd["uniq"], g, step=1, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        st.staple_adamw_rows(T["table"], m, v, dd["uniq"], g, step=2 + i, **kw)
    e1.record()
    torch.cuda.synchronize()
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error in AdamW")
    us = e0.elapsed_time(e1) / reps * 1e3
    u = int(dd["n_unique"].item())
    nbytes = u * f * (2 * 2 + 2 * 4 + 2 * 4 + 4)     # param, m, v read + written, gradient read
    del m, v
    torch.cuda.empty_cache()
    return {"rows": u, "us_per_step": us, "hbm_gb_s": nbytes / (us * 1e-6) / 1e9,
            "algorithmic_bytes": nbytes, "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "staple_adamw_rows over the batch's unique rows (bf16 table, fp32 moments in "
                    "HBM): 24 bytes moved per element"}


def train_cpu_baseline(torch, w, T, seconds):
    """Oracle fwd + bwd of the first S tokens of the batch; tokens/s = S / time."""
    import numpy as np
    from oracle import staple_oracle as O
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    wg, wu, wd = (f64(T[k]) for k in ("w_gate", "w_up", "w_down"))
    s_tokens = 64
    done = 0
    elapsed = 0.0
    while elapsed < seconds and done < w.n_tokens:
        sl = slice(done, done + s_tokens)
        ids = T["ids_np"][sl]
        uniq = np.unique(ids)
        idx = torch.from_numpy(uniq.astype(np.int64)).to(T["table"].device)
        table = _Rows(uniq, f64(T["table"][idx]))
        x, dy = f64(T["x"][sl]), f64(T["dy"][sl])
        t0 = time.perf_counter()
        O.dedup(ids)
        fw = O.ffn_forward(x, wg, wu, wd, table, ids, precision=O.BF16)
        O.ffn_backward(dy, x, wg, wu, wd, fw, ids, precision=O.BF16)
        elapsed += time.perf_counter() - t0
        done += s_tokens
    return {"value": done / elapsed, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            **host_cpu(),
            "sample": f"first {done} tokens of the 32768-token batch in chunks of {s_tokens} "
                      "(dedup + forward + backward, float64 numpy, bf16 rounding points)"}



# ----------------------------------------------------------------------------
# Host-offloaded tables with the HBM row cache (decode batch and training batch)
# ----------------------------------------------------------------------------
def _stream_pair(torch, k=2):
    """k streams for work that must overlap.  Streams share the process's few
    hardware queues (four on this machine), and two streams on one queue run
    one after the other; which of torch's pool streams share a queue depends
    on the order the process created them (measured: every sixteenth pair of
    consecutive pool streams did).  So each stream taken from the pool is
    checked against the ones already chosen: a four-workgroup GEMM on each
    (about 0.6 ms alone) must run side by side, else the stream is skipped.
    Where no stream does (a profiler that serialises the kernels), the first
    k candidates are returned."""
    import token_indexed_ffn_amd as st
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    kk = 65536
    h = device_normal((256, kk), 1.0, 1, torch.bfloat16, dev)
    w = device_normal((256, kk), 0.02, 2, torch.bfloat16, dev)
    ys = [torch.empty(256, 256, dtype=torch.bfloat16, device=dev) for _ in range(2)]

    def side_by_side(a, b):
        for s, y in ((a, ys[0]), (b, ys[1])):
            st.staple_ffn_down(h, w, y, stream=s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st.staple_ffn_down(h, w, ys[0], stream=a)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st.staple_ffn_down(h, w, ys[0], stream=a)
        st.staple_ffn_down(h, w, ys[1], stream=b)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        return (t2 - t1) < 1.5 * (t1 - t0)

    chosen, seen = [], []
    for _ in range(16):
        s = torch.cuda.Stream()
        seen.append(s)
        if all(side_by_side(c, s) for c in chosen):
            chosen.append(s)
            if len(chosen) == k:
                return tuple(chosen)
    print(f"[bench] no {k} streams ran side by side (kernels serialised?); using the first {k}",
          file=sys.stderr, flush=True)
    return tuple(seen[:k])


def setup_offload(torch, st, w, n_layers):
    """Pinned host tables (one per layer), the calibration-ranked HBM cache and
    per-layer cached rows."""
    import numpy as np
    import staple_synth as S
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    v, f = w.vocab, w.d_ff
    counts = torch.from_numpy(S.calibration_counts(v)).to(dev)
    cap = w.cache_capacity
    id_to_slot, slot_to_id = st.staple_cache_build(counts, cap)
    tables, cache_rows = [], []
    for l in range(n_layers):
        dtab = device_normal((v, f), w.table_std, w.layer_seeds(l)["table"], torch.bfloat16, dev)
        htab = torch.empty((v, f), dtype=torch.bfloat16, pin_memory=True)
        htab.copy_(dtab)
        del dtab
        tables.append(htab)
        cache_rows.append(st.staple_cache_fill(htab, slot_to_id, cap))
    torch.cuda.synchronize()
    return {"id_to_slot": id_to_slot, "slot_to_id": slot_to_id, "tables": tables,
            "cache_rows": cache_rows}


def _miss_list_to_host(torch, lk, host_buf, blocking=False):
    """Copies n_miss and the miss IDs to pinned host memory (one sync;
    blocking: the thread sleeps in the wait instead of spinning, leaving its
    core to host threads that work meanwhile)."""
    n = torch.empty(1, dtype=torch.int32, pin_memory=True)
    n.copy_(lk["n_miss"], non_blocking=True)
    host_buf[: lk["miss_ids"].numel()].copy_(lk["miss_ids"], non_blocking=True)
    if blocking:
        ev = torch.cuda.Event(blocking=True)
        ev.record()
        ev.synchronize()
    else:
        torch.cuda.current_stream().synchronize()
    return int(n.item())


def run_offload_decode(torch, st, w, steps, warmup, O=None):
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v, L = w.n_tokens, w.d_model, w.d_ff, w.vocab, w.n_layers
    if O is None:
        O = setup_offload(torch, st, w, L)
    ids = torch.from_numpy(w.ids()).to(dev)
    layers = []
    for l in range(L):
        s = w.layer_seeds(l)
        layers.append({k: device_normal(shape, std, s[k], torch.bfloat16, dev) for k, shape, std in (
            ("x", (n, d), w.x_std), ("w_gate", (f, d), w.w_std), ("w_up", (f, d), w.w_std),
            ("w_down", (d, f), w.w_std))})
        layers[-1]["y"] = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
        lay = layers[-1]
        lay["pgu"], lay["pd"] = st.staple_decode_pack_weights(lay["w_gate"], lay["w_up"],
                                                              lay["w_down"], d_model=d, d_ff=f)
        del lay["w_gate"], lay["w_up"], lay["w_down"]
    i32 = dict(dtype=torch.int32, device=dev)
    dd_out = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
              "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
              "n_unique": torch.empty(1, **i32)}
    lk_out = {k: torch.empty(n, **i32) for k in ("code", "miss_uidx", "miss_ids")}
    lk_out["n_miss"] = torch.empty(1, **i32)
    miss_host = torch.empty(n, dtype=torch.int32, pin_memory=True)
    staging = [torch.empty(n, f, dtype=torch.bfloat16, pin_memory=True) for _ in range(L)]
    dev_miss = [torch.empty(n, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    R = torch.empty(n, f, dtype=torch.bfloat16, device=dev)
    R_layers = [torch.empty(n, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ws = torch.empty(st.lib().staple_ffn_fwd_workspace_bytes(n, d, f, 1), dtype=torch.uint8,
                     device=dev)
    side = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(L)]
    main = torch.cuda.current_stream()

    def step_staged():
        dd = st.staple_dedup(ids, v, out=dd_out)
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], O["id_to_slot"], out=lk_out)
        m = _miss_list_to_host(torch, lk, miss_host)
        # layer l+1's miss rows are packed on the host and sent on the side
        # stream right after layer l's FFN is queued, so both overlap it
        side.wait_stream(main)

        def stage(l):
            st.staple_stage_misses(O["tables"][l], miss_host, m, staging[l], dev_miss[l], stream=side)
            events[l].record(side)

        stage(0)
        for l, lay in enumerate(layers):
            main.wait_event(events[l])
            st.staple_assemble_rows(O["cache_rows"][l], dev_miss[l], lk["code"], dd["n_unique"], out=R)
            st.staple_ffn_fwd_packed(lay["x"], lay["pgu"], lay["pd"], R, dd["inv"], d_ff=f,
                                     out={"y": lay["y"]}, workspace=ws)
            if l + 1 < L:
                stage(l + 1)
        return m

    def step_direct():
        # no host round trip: before each layer one kernel assembles R, the
        # hits from the HBM cache and the misses straight from the pinned host
        # table over PCIe, in stream order
        dd = st.staple_dedup(ids, v, out=dd_out)
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], O["id_to_slot"], out=lk_out)
        for l, lay in enumerate(layers):
            st.staple_assemble_rows_from_table(O["cache_rows"][l], O["tables"][l], dd["uniq"],
                                               lk["code"], dd["n_unique"], out=R,
                                               capacity=w.cache_capacity)
            st.staple_ffn_fwd_packed(lay["x"], lay["pgu"], lay["pd"], R, dd["inv"], d_ff=f,
                                     out={"y": lay["y"]}, workspace=ws)
        return None

    # the whole step (dedup, probe, every layer's rows in one launch, the
    # FFNs) enqueued by one native call
    stack = st.DecodeStack([{"x": lay["x"], "packed_gate_up": lay["pgu"], "packed_down": lay["pd"],
                             "cache_rows": O["cache_rows"][l], "table": O["tables"][l],
                             "rows": R_layers[l], "y": lay["y"]} for l, lay in enumerate(layers)],
                           d_model=d, d_ff=f, n_tokens=n)
    step_ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)

    def step_native():
        st.staple_decode_step_cached(stack, ids, O["id_to_slot"], w.cache_capacity,
                                     dedup_out=dd_out, lookup_out=lk_out, workspace=step_ws)

    # the same call with no compact rows: each layer's gate/up kernel reads
    # every token's row in place (cache slot, or the pinned host table over
    # PCIe) while its weights stream
    stack_inplace = st.DecodeStack([{"x": lay["x"], "packed_gate_up": lay["pgu"],
                                     "packed_down": lay["pd"], "cache_rows": O["cache_rows"][l],
                                     "table": O["tables"][l], "y": lay["y"]}
                                    for l, lay in enumerate(layers)],
                                   d_model=d, d_ff=f, n_tokens=n)

    def step_inplace():
        st.staple_decode_step_cached(stack_inplace, ids, O["id_to_slot"], w.cache_capacity,
                                     dedup_out=dd_out, lookup_out=lk_out, workspace=step_ws)

    # groups of layers: the first group's rows assembled before layer 0, each
    # later group's rows copied by the gate/up launches of the group before
    # it; groups of two over the separate tables, and groups of four over
    # tables interleaved token-major by fours in host memory (one contiguous
    # read per miss per group)
    def step_carried():
        st.staple_decode_step_cached(stack, ids, O["id_to_slot"], w.cache_capacity,
                                     dedup_out=dd_out, lookup_out=lk_out, workspace=step_ws, group=2)

    def step_carried1():
        st.staple_decode_step_cached(stack, ids, O["id_to_slot"], w.cache_capacity,
                                     dedup_out=dd_out, lookup_out=lk_out, workspace=step_ws, group=1)

    grouped = [st.staple_group_tables_host(O["tables"][g:g + 4]) for g in range(0, L, 4)]
    stack_grouped = st.DecodeStack(
        [{"x": lay["x"], "packed_gate_up": lay["pgu"], "packed_down": lay["pd"],
          "cache_rows": O["cache_rows"][l],
          "table": (grouped[l // 4], (l % 4) * f, min(4, L - (l // 4) * 4) * f),
          "rows": R_layers[l], "y": lay["y"]} for l, lay in enumerate(layers)],
        d_model=d, d_ff=f, n_tokens=n)

    def step_grouped():
        st.staple_decode_step_cached(stack_grouped, ids, O["id_to_slot"], w.cache_capacity,
                                     dedup_out=dd_out, lookup_out=lk_out, workspace=step_ws, group=4)

    def timed(step):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        if st.staple_get_device_error() != 0:
            raise RuntimeError("device error in offload decode")
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    ms_direct = timed(step_direct)
    ys = [lay["y"].clone() for lay in layers]
    ms_native = timed(step_native)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the native step driver's outputs differ from the per-layer calls")
    ms_inplace = timed(step_inplace)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the in-place row reads give other outputs than the per-layer calls")
    ms_carried = timed(step_carried)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the carried row copies give other outputs than the per-layer calls")
    ms_grouped = timed(step_grouped)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the grouped host tables give other outputs than the per-layer calls")
    ms_carried1 = timed(step_carried1)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the carried row copies give other outputs than the per-layer calls")
    # the carried step captured once in a HIP graph, replayed
    cap_s = torch.cuda.Stream()
    cap_s.wait_stream(main)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap_s):
        step_carried()
        cap_s.synchronize()
        with torch.cuda.graph(graph, stream=cap_s):
            step_carried()
    torch.cuda.synchronize()
    ms_graph = timed(graph.replay)
    torch.cuda.synchronize()
    if not all(torch.equal(a, lay["y"]) for a, lay in zip(ys, layers)):
        raise RuntimeError("the graph-replayed step gives other outputs than the per-layer calls")
    del graph
    ms_staged = timed(step_staged)
    m = _miss_list_to_host(torch, lk_out, miss_host)
    times = {"direct": ms_direct, "staged": ms_staged, "native": ms_native, "native_inplace": ms_inplace,
             "native_carried": ms_carried, "native_carried1": ms_carried1,
             "native_grouped": ms_grouped, "native_carried_graph": ms_graph}
    method = min(times, key=times.get)
    ms = times[method]
    n_unique = int(dd_out["n_unique"].item())
    # dominant kernel: the decode gate/up over each layer's compact rows (as
    # the native step runs it)
    step_native()
    torch.cuda.synchronize()
    h = torch.empty(n, f, dtype=torch.bfloat16, device=dev)
    gu_us = decode_gate_up_us(torch, st, [(lay["x"], lay["pgu"], R_layers[l]) for l, lay in enumerate(layers)],
                              dd_out["inv"], h, 20)
    gu_bytes = (2 * d * f + n * d + n_unique * f + n * f) * 2
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    # the miss rows' PCIe read: one layer's compact rows assembled from the
    # HBM cache and the pinned host table, HIP events around repeated launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        st.staple_assemble_rows_from_table(O["cache_rows"][0], O["tables"][0], dd_out["uniq"],
                                           lk_out["code"], dd_out["n_unique"], out=R,
                                           capacity=w.cache_capacity)
    e1.record()
    torch.cuda.synchronize()
    asm_us = e0.elapsed_time(e1) / reps * 1e3
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3),
            "method": method,
            "roofline": {
                "kernel": "decode_gateup_kernel (staple_ffn_gate_up_packed over the layer's compact rows)",
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic_from_profile(f"decode_gate_up/{w.name}",
                                                source_sha("decode.hip", "common.h")),
                "avg_launch_us": gu_us, "algorithmic_bytes_per_launch": gu_bytes},
            "pcie": {"kernel": "assemble_rows_table_kernel (one layer: hits from the HBM cache, "
                               "misses from the pinned host table)",
                     "avg_launch_us": asm_us, "pcie_bytes_per_launch": m * f * 2,
                     "pcie_gb_s": m * f * 2 / (asm_us * 1e-6) / 1e9, "pcie_peak_gb_s": 64.0},
            "direct_ms_per_step": ms_direct, "native_ms_per_step": ms_native,
            "native_inplace_ms_per_step": ms_inplace, "native_carried_ms_per_step": ms_carried,
            "native_carried1_ms_per_step": ms_carried1,
            "native_grouped_ms_per_step": ms_grouped, "staged_ms_per_step": ms_staged,
            "native_carried_graph_ms_per_step": ms_graph,
            "n_unique": n_unique, "misses_per_layer": m, "cache_capacity": w.cache_capacity,
            "pcie_bytes_per_step": m * f * 2 * L,
            "note": "eager steps, dedup + cache probe once per step. direct: per layer one kernel "
                    "assembles R with the hits from the HBM cache and the misses read from the "
                    "pinned host table over PCIe (no host sync, one stream), then gate/up, "
                    "down. native: one staple_decode_step_cached call per step (dedup, probe, "
                    "every layer's rows in one launch, the FFNs). native_inplace: the same call "
                    "with no compact rows, each gate/up kernel reading its tokens' rows in place "
                    "(cache slot or pinned host table). native_carried: the same call with groups "
                    "of two layers, the first group's rows assembled first and every later "
                    "group's rows copied by the copy waves of the gate/up launches of the group "
                    "before it (native_carried1: groups of one layer, each layer's rows copied "
                    "during the previous layer's gate/up). native_grouped: native_carried over "
                    "host tables interleaved "
                    "token-major by groups of four. native_carried_graph: native_carried "
                    "captured once in a HIP graph and replayed. staged: "
                    "one host sync for the miss list, host pack + H2D copy per layer on a side "
                    "stream one layer ahead"}


def run_offload_prefill_chunks(torch, st, w, O, steps, warmup, chunks=(4096, 8192)):
    """The chunked prefill at each chunk size (the pages do not print theirs);
    the fastest is reported, with every size's time."""
    runs = {}
    for c in chunks:
        runs[c] = run_offload_prefill(torch, st, w, O, steps, warmup, chunk=c)
        torch.cuda.empty_cache()
    best = min(runs, key=lambda c: runs[c]["ms_per_prefill"])
    out = runs[best]
    out["ms_by_chunk_tokens"] = {str(c): r["ms_per_prefill"] for c, r in runs.items()}
    return out


def run_offload_prefill(torch, st, w, O, steps, warmup, chunk=4096, workgroups=(16, 32, 64)):
    main, side = _stream_pair(torch)
    with torch.cuda.stream(main):
        out = _run_offload_prefill(torch, st, w, O, steps, warmup, chunk, workgroups, main, side)
    torch.cuda.synchronize()
    return out


def _run_offload_prefill(torch, st, w, O, steps, warmup, chunk, workgroups, main, side):
    """Prefill of w.n_tokens tokens through w.n_layers layers whose tables are in
    pinned host memory (top-5% rows cached in HBM), in chunks of `chunk` tokens.
    Each chunk's rows come from one staple_prefill_rows_cached call (dedup, cache
    probe, all layers' compact rows with the misses read over PCIe), then the
    layers' FFNs (staple_ffn_fwd: gate/up GEMM with the row epilogue, down GEMM).
    compute_only: every chunk's rows assembled beforehand (the FFNs alone).
    serial: each chunk's rows, then its FFNs, on one stream.  pipelined: chunk
    c + 1's rows on a side stream, on at most `workgroups` workgroups, while
    chunk c's FFNs run; in the first chunk, layer 0's rows come first (full
    grid) and each later layer's rows while the layer before it runs; two sets
    of row buffers, each reused only after the chunk that read it.  dma: the
    first chunk as in pipelined; every later chunk's miss rows packed on the
    host and copied by the GPU's DMA engines (staple_stage_misses_dma, no
    compute unit) while the chunk before it runs, then each layer's compact
    rows assembled from the cache and the staged misses.  The fastest schedule
    gives ms_per_prefill."""
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v, L = w.n_tokens, w.d_model, w.d_ff, w.vocab, w.n_layers
    C = chunk
    nc = n // C
    cap = w.cache_capacity
    ids = torch.from_numpy(w.ids()).to(dev)
    layers = []
    for l in range(L):
        s = w.layer_seeds(l)
        layers.append({k: device_normal(shape, std, s[k], torch.bfloat16, dev) for k, shape, std in (
            ("x", (n, d), w.x_std), ("w_gate", (f, d), w.w_std), ("w_up", (f, d), w.w_std),
            ("w_down", (d, f), w.w_std))})
        layers[-1]["y"] = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ws_bytes = st.prefill_rows_workspace_bytes(C)

    def buffers():
        B = {"dd": {"uniq": torch.empty(C, **i32), "inv": torch.empty(C, **i32),
                    "sorted_pos": torch.empty(C, **i32), "seg_start": torch.empty(C + 1, **i32),
                    "n_unique": torch.empty(1, **i32)},
             "lk": {"code": torch.empty(C, **i32), "miss_uidx": torch.empty(C, **i32),
                    "n_miss": torch.empty(1, **i32)},
             "rows": [torch.empty(C, f, dtype=torch.bfloat16, device=dev) for _ in range(L)],
             "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None}
        srcs = [{"table": O["tables"][l], "cache_rows": O["cache_rows"][l], "rows": B["rows"][l]}
                for l in range(L)]
        B["rs"] = st.RowSources(srcs, d_ff=f)
        B["rs_layer"] = [st.RowSources([src], d_ff=f) for src in srcs]
        return B

    bufs = [buffers() for _ in range(2)]
    pre = [buffers() for _ in range(nc)]
    fwd_ws = torch.empty(st.lib().staple_ffn_fwd_workspace_bytes(C, d, f, 1), dtype=torch.uint8,
                         device=dev)
    ready = [torch.cuda.Event() for _ in range(nc)]
    done = [torch.cuda.Event() for _ in range(nc)]
    layer_ready = [torch.cuda.Event() for _ in range(L)]

    def rows(B, c, stream, wg, rs=None, lookup=True):
        st.staple_prefill_rows_cached(B["rs"] if rs is None else rs, ids[c * C:(c + 1) * C],
                                      O["id_to_slot"], cap, dedup_out=B["dd"], lookup_out=B["lk"],
                                      workspace=B["ws"], max_workgroups=wg, lookup=lookup,
                                      stream=stream)

    def ffns(B, c, per_layer=None):
        for l, lay in enumerate(layers):
            if per_layer is not None:
                main.wait_event(per_layer[l])
            st.staple_ffn_fwd(lay["x"][c * C:(c + 1) * C], lay["w_gate"], lay["w_up"],
                              lay["w_down"], B["rows"][l], B["dd"]["inv"],
                              out={"y": lay["y"][c * C:(c + 1) * C]}, workspace=fwd_ws,
                              stream=main)

    def compute_only():
        for c in range(nc):
            ffns(pre[c], c)

    def serial():
        for c in range(nc):
            rows(bufs[0], c, main, 0)
            ffns(bufs[0], c)

    def pipelined(wg):
        side.wait_stream(main)          # the previous prefill has finished with the buffers

        def issue(c):
            if c >= 2:
                side.wait_event(done[c - 2])
            rows(bufs[c % 2], c, side, wg)
            ready[c].record(side)

        # the first chunk: layer 0's rows (with the dedup and the probe) on the
        # full grid, nothing else running yet; then each later layer's rows,
        # one call each, so that layer l + 1's rows arrive during layer l
        B0 = bufs[0]
        rows(B0, 0, side, 0, rs=B0["rs_layer"][0])
        layer_ready[0].record(side)
        for l in range(1, L):
            rows(B0, 0, side, wg, rs=B0["rs_layer"][l], lookup=False)
            layer_ready[l].record(side)
        for c in range(nc):
            if c + 1 < nc:
                issue(c + 1)
            if c == 0:
                ffns(B0, 0, per_layer=layer_ready)
            else:
                main.wait_event(ready[c])
                ffns(bufs[c % 2], c)
            done[c].record(main)

    # DMA-engine staging: each later chunk's miss rows packed on the host and
    # copied by the DMA engines (staple_stage_misses_dma) while the chunk
    # before it runs, then assembled with the cached rows by one HBM-only
    # kernel per layer; no compute unit reads PCIe
    dma_blocks = [[torch.empty(C, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
                  for _ in range(2)]
    dma_staging = torch.empty(L * C * f, dtype=torch.bfloat16, pin_memory=True)
    miss_ids_host = torch.empty(C, dtype=torch.int32, pin_memory=True)
    n_miss_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
    lk_ids = [torch.empty(C, **i32) for _ in range(2)]
    looked_up = torch.cuda.Event(blocking=True)
    done_host = [torch.cuda.Event(blocking=True) for _ in range(nc)]
    call_done = torch.cuda.Event(blocking=True)   # the previous prefill's last kernels

    def lookup_to_host(c, B):
        """dedup and probe of chunk c on the side stream, the miss list to the host"""
        lk = {"code": B["lk"]["code"], "miss_uidx": B["lk"]["miss_uidx"],
              "miss_ids": lk_ids[c % 2], "n_miss": B["lk"]["n_miss"]}
        with torch.cuda.stream(side):
            st.staple_dedup(ids[c * C:(c + 1) * C], v, out=B["dd"], workspace=B["ws"], stream=side)
            st.staple_cache_lookup(B["dd"]["uniq"], B["dd"]["n_unique"], O["id_to_slot"], out=lk,
                                   stream=side)
            n_miss_host.copy_(lk["n_miss"], non_blocking=True)
            miss_ids_host.copy_(lk["miss_ids"], non_blocking=True)
            looked_up.record(side)
        looked_up.synchronize()
        return int(n_miss_host.item())

    def dma(wg):
        side.wait_stream(main)
        call_done.synchronize()     # the previous prefill no longer reads any block
        # the first chunk as in pipelined(): its rows read over PCIe by kernels
        # (layer 0's on the full grid, each later layer's during the layer
        # before it), so that the host can stage the next chunk at once
        B0 = bufs[0]
        rows(B0, 0, side, 0, rs=B0["rs_layer"][0])
        layer_ready[0].record(side)
        for l in range(1, L):
            rows(B0, 0, side, wg, rs=B0["rs_layer"][l], lookup=False)
            layer_ready[l].record(side)
        # each later chunk: every layer's misses staged by the DMA engines while
        # the chunk before it runs, then assembled with the cached rows (HBM only)
        for c in range(nc):
            if c == 0:
                ffns(B0, 0, per_layer=layer_ready)
            else:
                main.wait_event(ready[c])
                ffns(bufs[c % 2], c)
            done_host[c].record(main)
            if c + 1 >= nc:
                continue
            p = (c + 1) % 2
            Bn = bufs[p]
            if c >= 1:
                side.wait_event(done_host[c - 1])   # chunk c - 1 read Bn last
            m = lookup_to_host(c + 1, Bn)
            if c >= 1:
                done_host[c - 1].synchronize()      # ... and its device blocks
            st.staple_stage_misses_dma(O["tables"], miss_ids_host, m, dma_staging, dma_blocks[p])
            for l in range(L):
                st.staple_assemble_rows(O["cache_rows"][l], dma_blocks[p][l], Bn["lk"]["code"],
                                        Bn["dd"]["n_unique"], out=Bn["rows"][l], stream=side)
            ready[c + 1].record(side)
        call_done.record(main)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if st.staple_get_device_error() != 0:
            raise RuntimeError("device error in offload prefill")
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    for c in range(nc):
        rows(pre[c], c, main, 0)
    torch.cuda.synchronize()
    misses = sum(int(B["lk"]["n_miss"].item()) for B in pre)
    uniques = sum(int(B["dd"]["n_unique"].item()) for B in pre)
    ms_compute = timed(compute_only)
    ref = [layers[0]["y"].clone(), layers[-1]["y"].clone()]
    ms_serial = timed(serial)
    same = lambda: torch.equal(ref[0], layers[0]["y"]) and torch.equal(ref[1], layers[-1]["y"])
    if not same():
        raise RuntimeError("serial prefill outputs differ from the precomputed-rows run")
    ms_pipe = {}
    for wg in workgroups:
        ms_pipe[wg] = timed(lambda: pipelined(wg))
        torch.cuda.synchronize()
        if not same():
            raise RuntimeError("pipelined prefill outputs differ from the serial run")
    ms_dma = {}
    for wg in workgroups:
        ms_dma[wg] = timed(lambda: dma(wg))
        torch.cuda.synchronize()
        if not same():
            raise RuntimeError("DMA-staged prefill outputs differ from the serial run")
    ms_all = {("chunk", k): t for k, t in ms_pipe.items()}
    ms_all.update({("dma", k): t for k, t in ms_dma.items()})
    best_sched, best_wg = min(ms_all, key=ms_all.get)
    ms = ms_all[(best_sched, best_wg)]
    # the rows of one chunk alone (all layers, full grid): what the pipeline hides
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in range(nc):
        rows(bufs[0], c, main, 0)
    e1.record()
    torch.cuda.synchronize()
    rows_ms = e0.elapsed_time(e1)
    # dominant kernel: the gate/up GEMM of one chunk (events around each launch)
    h = torch.empty(C, f, dtype=torch.bfloat16, device=dev)
    durs = []
    for rep in range(max(3, steps)):
        lay, B = layers[rep % L], pre[rep % nc]
        c = rep % nc
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        st.staple_ffn_gate_up(lay["x"][c * C:(c + 1) * C], lay["w_gate"], lay["w_up"],
                              B["rows"][rep % L], B["dd"]["inv"], h)
        ev[1].record()
        torch.cuda.synchronize()
        durs.append(ev[0].elapsed_time(ev[1]) * 1e3)
    gu_us = sum(durs) / len(durs)
    gu_flops = 4 * C * d * f
    achieved = gu_flops / (gu_us * 1e-6) / 1e12
    flops = 6 * n * d * f * L
    pcie = misses * L * f * 2
    return {"workload": w.name, "tokens": n, "chunk_tokens": C, "chunks": nc, "layers": L,
            "ms_per_prefill": ms, "tokens_per_s": n / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "pipelined_ms": {str(k): t for k, t in ms_pipe.items()},
            "dma_ms": {str(k): t for k, t in ms_dma.items()},
            "schedule": "rows read by kernels" if best_sched == "chunk" else "DMA-engine staging",
            "max_workgroups": best_wg,
            "serial_ms": ms_serial, "compute_only_ms": ms_compute,
            "ratio_to_compute_only": ms / ms_compute,
            "rows_alone_ms": rows_ms,
            "hidden_fraction_of_rows": 1.0 - (ms - ms_compute) / rows_ms,
            "unique_rows_per_chunk": uniques / nc, "miss_rows_per_chunk": misses / nc,
            "pcie_bytes_per_prefill": pcie, "cache_capacity": cap,
            "roofline": {
                "kernel": f"gemm_kernel<bf16,GateUp> (staple_ffn_gate_up, one {C}-token chunk)",
                "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS,
                "traffic": traffic_from_profile(f"prefill_gate_up/{w.name}_chunk{C}",
                                                source_sha("gemm.hip", "common.h")),
                "avg_launch_us": gu_us, "algorithmic_flops_per_launch": gu_flops},
            "note": "forward only (prefill), eager launches; FLOPs 6 N d f per layer. "
                    "rows_alone_ms: every chunk's rows on the full grid with nothing beside them; "
                    "hidden_fraction_of_rows = 1 - (ms_per_prefill - compute_only) / rows_alone_ms; "
                    "pipelined_ms: rows read over PCIe by kernels beside the FFNs, by workgroup cap; "
                    "dma_ms: later chunks' miss rows staged by the DMA engines, by the first "
                    "chunk's workgroup cap"}


def run_offload_train(torch, st, w, steps, warmup):
    # the step, the miss-row copy, the host update's refreshes
    main, side, copy = _stream_pair(torch, 3)
    with torch.cuda.stream(main):
        out = _run_offload_train(torch, st, w, steps, warmup, main, side, copy)
    torch.cuda.synchronize()
    return out


def _run_offload_train(torch, st, w, steps, warmup, main, side, copy):
    import numpy as np
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v = w.n_tokens, w.d_model, w.d_ff, w.vocab
    O = setup_offload(torch, st, w, 1)
    T = setup_train(torch, st, w)
    i32 = dict(dtype=torch.int32, device=dev)
    lk_out = {k: torch.empty(n, **i32) for k in ("code", "miss_uidx", "miss_ids")}
    lk_out["n_miss"] = torch.empty(1, **i32)
    miss_host = torch.empty(n, dtype=torch.int32, pin_memory=True)
    counts_host = torch.empty(2, dtype=torch.int32, pin_memory=True)
    sp_out = {k: torch.empty(n, **i32) for k in ("hit_pos", "miss_pos", "tok_row")}
    sp_out["counts"] = torch.empty(2, **i32)
    staging = torch.empty(n, f, dtype=torch.bfloat16, pin_memory=True)
    dev_miss = torch.empty(n, f, dtype=torch.bfloat16, device=dev)
    ev_copy0, ev_copy1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_gu0, ev_gu1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_ready = torch.cuda.Event()
    stats = {"pack_s": 0.0, "copy_ms": 0.0, "hit_tokens": 0, "gu_us": {}, "dma_ms": 0.0}

    def step(mode, B=None, before_rows=None, rows_event=None, blocking=False):
        """B: the step's own dedup, probe and row-gradient buffers (default:
        the shared ones); before_rows: called once the miss list is known and
        before anything reads the table's rows (the optimizer's finish)."""
        dd = st.staple_dedup(T["ids"], v, out=T["dd"] if B is None else B["dd"],
                             workspace=T["dd_ws"])
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], O["id_to_slot"],
                                    out=lk_out if B is None else B["lk"])
        sp = st.staple_split_tokens(dd["inv"], lk["code"], dd["n_unique"], out=sp_out)
        counts_host.copy_(sp["counts"], non_blocking=True)
        m = _miss_list_to_host(torch, lk, miss_host, blocking)   # one host sync for both
        n_hit, n_miss_tok = int(counts_host[0]), int(counts_host[1])
        stats["hit_tokens"] = n_hit
        side.wait_stream(main)
        if before_rows is not None:
            before_rows()
        fw = T["fwd"]

        def gate_up_cached():
            # the tokens whose rows are cached run while the miss rows are in flight
            ev_gu0.record(main)
            st.staple_ffn_gate_up_tokens(sp["hit_pos"], n_hit, T["x"], T["w_gate"], T["w_up"],
                                         O["cache_rows"][0], sp["tok_row"], fw["h"], fw["g"],
                                         fw["u"])
            ev_gu1.record(main)

        if mode == "dma":
            # the cached tokens' gate/up first; meanwhile the host packs the miss
            # rows and the DMA engines copy them (no compute unit); the missed
            # tokens' gate/up is enqueued once the copy is done.  The previous
            # step's readers of dev_miss finished before the miss-list sync.
            gate_up_cached()
            t0 = time.perf_counter()
            st.staple_stage_misses_dma([O["tables"][0]], miss_host, m, staging, [dev_miss])
            stats["dma_ms"] = (time.perf_counter() - t0) * 1e3
        else:
            t0 = time.perf_counter()
            with torch.cuda.stream(side):
                ev_copy0.record(side)
            if mode == "staged":      # host pack into pinned staging, one H2D copy
                st.staple_stage_misses(O["tables"][0], miss_host, m, staging, dev_miss, stream=side)
            elif mode == "direct":    # a kernel reads the rows from the pinned host table
                with torch.cuda.stream(side):
                    st.staple_gather_rows(O["tables"][0], lk["miss_ids"], lk["n_miss"],
                                          out=dev_miss, stream=side)
            # mode "resident": the miss rows are already in HBM (no copy; reference)
            with torch.cuda.stream(side):
                ev_copy1.record(side)
            stats["pack_s"] += time.perf_counter() - t0
            ev_ready.record(side)
            gate_up_cached()
            main.wait_event(ev_ready)
        st.staple_ffn_gate_up_tokens(sp["miss_pos"], n_miss_tok, T["x"], T["w_gate"], T["w_up"],
                                     dev_miss, sp["tok_row"], fw["h"], fw["g"], fw["u"])
        st.staple_ffn_down(fw["h"], T["w_down"], fw["y"])
        st.staple_ffn_bwd_table_grad(T["dy"], T["x"], T["w_gate"], T["w_up"], T["w_down"], fw["g"],
                                     fw["u"], fw["h"], dd["sorted_pos"], dd["seg_start"],
                                     dd["n_unique"], inv=dd["inv"],
                                     out=T["bwd"] if B is None else B["bwd"],
                                     workspace=T["bwd_ws"], rows_event=rows_event)
        return m

    def timed(mode):
        for _ in range(warmup):
            step(mode)
        torch.cuda.synchronize()
        if st.staple_get_device_error() != 0:
            raise RuntimeError("device error in offload train")
        stats["pack_s"] = 0.0
        copy_ms = []
        t0 = time.perf_counter()
        for _ in range(steps):
            m = step(mode)
            if mode == "dma":
                copy_ms.append(stats["dma_ms"])   # host pack and DMA copy, timed on the host
            else:
                ev_copy1.synchronize()
                copy_ms.append(ev_copy0.elapsed_time(ev_copy1))
            if mode in ("direct", "dma"):
                ev_gu1.synchronize()
                stats["gu_us"].setdefault(mode, []).append(ev_gu0.elapsed_time(ev_gu1) * 1e3)
        torch.cuda.synchronize()
        return ((time.perf_counter() - t0) / steps * 1e3, float(np.median(copy_ms)),
                stats["pack_s"] / steps * 1e3, m)

    # "resident" reuses the miss rows the step before it copied
    res, outs = {}, {}
    for k in ("staged", "resident", "direct", "dma"):
        res[k] = timed(k)
        outs[k] = (T["fwd"]["y"].clone(), T["bwd"]["d_rows"].clone())
        if not all(torch.equal(a, b) for a, b in zip(outs[k], outs["staged"])):
            raise RuntimeError(f"offloaded training step ({k}) differs from the staged one")
    del outs
    host_adamw = run_host_adamw(torch, st, O, T, lk_out)
    # the optimizer overlapped with each of the two faster row paths (their
    # optimizer-free times are within run-to-run noise); the faster counts
    opts = {k: run_offload_train_optimizer(torch, st, O, T, lk_out, step, k, steps, warmup, copy)
            for k in ("direct", "dma")}
    mode = min(opts, key=lambda k: opts[k]["overlapped_ms_per_step"])
    opt = opts[mode]
    opt["overlapped_ms_per_step_by_method"] = {k: o["overlapped_ms_per_step"] for k, o in opts.items()}
    ms_free, _, _, m = res[mode]
    ms_res = res["resident"][0]
    ms = opt["overlapped_ms_per_step"]
    opt["ratio_to_optimizer_free_step"] = ms / ms_free
    opt["serial_ratio_to_optimizer_free_step"] = opt["serial_ms_per_step"] / ms_free
    gu_us = float(np.median(stats["gu_us"]["dma" if mode == "dma" else "direct"]))
    gu_flops = 4 * stats["hit_tokens"] * d * f
    achieved = gu_flops / (gu_us * 1e-6) / 1e12
    out = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3),
           "optimizer_free_ms_per_step": ms_free,
           "optimizer_free_tokens_per_s": n / (ms_free * 1e-3), "optimizer": opt,
           "method": mode, "n_unique": int(T["dd"]["n_unique"].item()), "miss_rows": m,
           "roofline": {
               "kernel": "gemm_kernel<bf16,GateUp> (staple_ffn_gate_up_tokens over the cached "
                         "tokens, beside the miss-row copy)",
               "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": achieved / BF16_PEAK_TFLOPS,
               "traffic": traffic_from_profile(f"offload_gate_up/{w.name}",
                                               source_sha("gemm.hip", "common.h")),
               "avg_launch_us": gu_us, "algorithmic_flops_per_launch": gu_flops},
           "cache_capacity": w.cache_capacity, "token_hit_rate": stats["hit_tokens"] / n,
           "resident_ms_per_step": ms_res, "pcie_bytes_per_step": m * f * 2}
    out["adamw_host"] = host_adamw
    for k in ("staged", "direct", "dma"):
        ms_k, copy_k, pack_k, _ = res[k]
        out[k] = {"ms_per_step": ms_k, "copy_ms": copy_k, "host_pack_ms": pack_k,
                  "pcie_gb_s": m * f * 2 / (copy_k * 1e-3) / 1e9,
                  "hidden_fraction_of_copy": max(0.0, min(1.0, 1.0 - max(0.0, ms_k - ms_res) /
                                                          max(copy_k + pack_k, 1e-9)))}
    out["note"] = ("eager step: dedup + cache probe + token split, one host sync for the miss "
                   "list and the split counts; the miss rows move while the gate/up GEMM of the "
                   "cached tokens runs (rows from the cache slots): staged, host pack into pinned "
                   "staging + one H2D copy on a side stream; direct, a kernel on a side stream "
                   "reads them from the pinned host table; dma, host pack + a copy on the DMA "
                   "engines (staple_stage_misses_dma), its copy_ms the pack and copy timed on "
                   "the host; then the missed tokens' gate/up, down, backward. "
                   "ms_per_step and tokens_per_s include the table rows' AdamW update on the host "
                   "overlapped with the GPU (optimizer.overlapped); optimizer_free_*: the same "
                   "step without it. resident: the step with the miss rows already in HBM, for "
                   "the hidden fraction = 1 - (t - t_resident) / (host pack + copy time)")
    return out


def run_offload_train_optimizer(torch, st, O, T, lk_out, step, mode, steps, warmup, copy_s):
    """The offloaded training step with the AdamW update of the table rows on
    the host (bf16 table, fp32 moments in host memory; STAPLE Figure 4
    caption), in two schedules:
      serial: after the step, the row gradients come to the host, host threads
        update the rows, the cached copies are refreshed; then the next step.
      overlapped (staple_host_adamw_*): the row gradients leave in chunks on a
        copy stream as soon as the backward's segment sum has formed them, a
        host worker updates each chunk as it lands and refreshes its cached
        copies, all while the GPU runs the rest of the backward and the next
        step's dedup and probe; the next step waits for the update only
        before it reads table rows (miss copy, cached tokens' gate/up).
    Each step's dedup, probe and row gradients live in one of two buffer sets
    (alternating), so the update of one step reads buffers the next step does
    not write."""
    import numpy as np
    table, cache = O["tables"][0], O["cache_rows"][0]
    vocab, f = table.shape
    n = T["ids"].numel()
    m = torch.zeros(vocab, f, dtype=torch.float32)
    v = torch.zeros(vocab, f, dtype=torch.float32)
    hp = dict(lr=3e-4, weight_decay=1e-4)
    sets = [{"dd": {k: torch.empty_like(t) for k, t in T["dd"].items()},
             "lk": {k: torch.empty_like(t) for k, t in lk_out.items()},
             "bwd": dict(T["bwd"], d_rows=torch.empty_like(T["bwd"]["d_rows"]))}
            for _ in range(2)]
    main = torch.cuda.current_stream()
    grad_h = torch.empty(n, f, dtype=torch.float32, pin_memory=True)
    uniq_h = torch.empty(n, dtype=torch.int32, pin_memory=True)
    t_step = [0]

    def serial(k):
        B = sets[k % 2]
        step(mode, B)
        dd = B["dd"]
        u = int(dd["n_unique"].item())                 # synchronizes
        grad_h[:u].copy_(B["bwd"]["d_rows"][:u])
        uniq_h[:u].copy_(dd["uniq"][:u])
        t_step[0] += 1
        st.staple_adamw_rows_host(table, m, v, uniq_h[:u], grad_h[:u], step=t_step[0], **hp)
        st.staple_cache_refresh(table, dd["uniq"], B["lk"]["code"], dd["n_unique"], cache)

    ha = st.HostAdamW(n, f)
    pending = [False]

    def finish():
        if pending[0]:
            ha.finish(main)
            pending[0] = False

    def overlapped(k):
        B = sets[k % 2]
        step(mode, B, before_rows=finish, rows_event=ha.event, blocking=True)
        t_step[0] += 1
        ha.start(table, m, v, B["dd"]["uniq"], B["dd"]["n_unique"], B["bwd"]["d_rows"],
                 step=t_step[0], copy_stream=copy_s, code=B["lk"]["code"], cache_rows=cache, **hp)
        pending[0] = True

    def timed(fn):
        for k in range(warmup):
            fn(k)
        finish()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            fn(k)
        finish()
        torch.cuda.synchronize()
        if st.staple_get_device_error() != 0:
            raise RuntimeError("device error in offload train with the optimizer")
        return (time.perf_counter() - t0) / steps * 1e3

    ms_serial = timed(serial)
    ms_ovl = timed(overlapped)
    ha.close()
    return {"serial_ms_per_step": ms_serial, "overlapped_ms_per_step": ms_ovl,
            "rows_per_step": int(sets[0]["dd"]["n_unique"].item()),
            "note": "AdamW of the batch's unique table rows on the host (bf16 table, fp32 moments "
                    "in host memory) and the refresh of their cached copies, once per step: "
                    "serial after the step, or overlapped with it (staple_host_adamw_*)"}


def run_host_adamw(torch, st, O, T, lk, reps=3):
    """The pages' optimizer placement for offloaded tables: the table and its
    fp32 moments in host memory; after the backward the batch's row gradients
    come to the host over PCIe, host threads update the rows, and the cached
    copies of the updated rows are refreshed from the host table."""
    import numpy as np
    table = O["tables"][0]
    vocab, f = table.shape
    dd = T["dd"]
    u = int(dd["n_unique"].item())
    m = torch.zeros(vocab, f, dtype=torch.float32)
    v = torch.zeros(vocab, f, dtype=torch.float32)
    grad_h = torch.empty(u, f, dtype=torch.float32, pin_memory=True)
    uniq_h = dd["uniq"][:u].cpu().contiguous()
    t_copy, t_upd, t_ref = [], [], []
    for i in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        grad_h.copy_(T["bwd"]["d_rows"][:u], non_blocking=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st.staple_adamw_rows_host(table, m, v, uniq_h, grad_h, lr=3e-4, weight_decay=1e-4,
                                  step=i + 1)
        t2 = time.perf_counter()
        st.staple_cache_refresh(table, dd["uniq"], lk["code"], dd["n_unique"], O["cache_rows"][0])
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        t_copy.append(t1 - t0)
        t_upd.append(t2 - t1)
        t_ref.append(t3 - t2)
    if st.staple_get_device_error() != 0:
        raise RuntimeError("device error in the cache refresh")
    upd = float(np.median(t_upd))
    nbytes = u * f * (2 * 2 + 2 * 4 + 2 * 4 + 4)
    return {"rows": u, "grad_d2h_ms": float(np.median(t_copy)) * 1e3, "update_ms": upd * 1e3,
            "cache_refresh_ms": float(np.median(t_ref)) * 1e3,
            "host_gb_s": nbytes / upd / 1e9, "threads": min(16, os.cpu_count() or 1),
            "note": "staple_adamw_rows_host over the batch's unique rows (bf16 table, fp32 "
                    "moments in host memory), after a D2H copy of the fp32 row gradients; then "
                    "staple_cache_refresh of the cached rows among them"}


# ----------------------------------------------------------------------------
def copy_probe(torch):
    """A plain device copy of 1 GiB, five times: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    a = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": a.numel() * 2,
                      "copy_bytes_written_per_launch": b.numel() * 2}))


def _progress(msg: str) -> None:
    """One line per finished workload on stderr (the JSON line goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU path is not built.", file=sys.stderr)
        return 2
    import torch
    if args.mode == "copy":
        copy_probe(torch)
        return 0
    import staple_synth as S
    import token_indexed_ffn_amd as st
    st.lib()
    torch.cuda.set_device(0)
    wl = set(args.workloads.split(","))
    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: seeded Zipf(1.1) token IDs over vocab 100352 (fixed rank->ID "
                   "permutation), x ~ N(0,1), weights and tables ~ N(0,0.02), bf16"}
    w = S.OLMO1B_DECODE
    if "decode" in wl:
        dec, D = run_decode(torch, st, w, args.steps, args.warmup)
        out["value"] = dec["tokens_per_s"]
        out["ms_per_step"] = dec["ms_per_step"]
        out["config"] = {"workload": w.name, "d_model": w.d_model, "d_ff": w.d_ff,
                         "vocab": w.vocab, "batch": w.n_tokens, "layers": w.n_layers,
                         "tables": "12 x 100352 x 8192 bf16, HBM-resident",
                         "step": "12 x staple_ffn_fwd_packed (gate/up kernel, down kernel, split-K sum), "
                                 + dec["launch"]}
        out["roofline"] = dec["roofline"]
        out["decode"] = {k: v for k, v in dec.items() if k != "roofline"}
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = decode_cpu_baseline(torch, w, D, args.cpu_seconds)
        del D
        torch.cuda.empty_cache()
        _progress(f"decode: {out['value']:.0f} tokens/s")
    if "train" in wl:
        wt = S.OLMO1B_TRAIN
        tr, T = run_train(torch, st, wt, args.train_steps, args.train_warmup)
        if not args.no_cpu_baseline:
            tr["cpu_baseline"] = train_cpu_baseline(torch, wt, T, args.cpu_seconds)
        out["train"] = tr
        if out["value"] is None:
            out["value"] = tr["tokens_per_s"]
            out["ms_per_step"] = tr["ms_per_step"]
            out["roofline"] = tr["roofline"]
            out["config"] = {"workload": wt.name}
        del T
        torch.cuda.empty_cache()
        _progress(f"train: {tr['tokens_per_s']:.0f} tokens/s")
    if "decode7b" in wl:
        w7 = S.OLMO7B_DECODE
        dec7, D7 = run_decode(torch, st, w7, max(20, args.steps // 2), args.warmup)
        out["decode_7b"] = dict(dec7, workload=w7.name)
        del D7
        torch.cuda.empty_cache()
        _progress(f"decode7b: {dec7['tokens_per_s']:.0f} tokens/s")
    if "train7b" in wl:
        w7 = S.OLMO7B_TRAIN
        tr7, T7 = run_train(torch, st, w7, args.train_steps, args.train_warmup)
        out["train_7b"] = tr7
        del T7
        torch.cuda.empty_cache()
        _progress(f"train7b: {tr7['tokens_per_s']:.0f} tokens/s")
    if "stem" in wl:
        # the STEM layer STAPLE is compared against (no up-projection), same workloads
        dec_s, D_s = run_decode(torch, st, w, args.steps, args.warmup, stem=True)
        out["decode_stem"] = dict(dec_s, workload=w.name + "_stem")
        del D_s
        torch.cuda.empty_cache()
        _progress(f"decode stem: {dec_s['tokens_per_s']:.0f} tokens/s")
        tr_s, T_s = run_train(torch, st, S.OLMO1B_TRAIN, args.train_steps, args.train_warmup,
                              stem=True)
        out["train_stem"] = dict(tr_s, workload=S.OLMO1B_TRAIN.name + "_stem")
        del T_s
        torch.cuda.empty_cache()
        _progress(f"train stem: {tr_s['tokens_per_s']:.0f} tokens/s")
    if "lowrank" in wl:
        out["train_lowrank"] = run_train_lowrank(torch, st, S.OLMO1B_TRAIN, 512, args.train_steps,
                                                 args.train_warmup)
        _progress(f"lowrank: {out['train_lowrank']['tokens_per_s']:.0f} tokens/s")
    O12 = None
    if "offload" in wl or "prefill" in wl:
        # the 12 pinned host tables and their HBM cache, shared by both workloads
        O12 = setup_offload(torch, st, S.OLMO1B_OFFLOAD, S.OLMO1B_OFFLOAD.n_layers)
    if "offload" in wl:
        out["offload_decode"] = run_offload_decode(torch, st, S.OLMO1B_OFFLOAD, 20, 3, O=O12)
        torch.cuda.empty_cache()
        _progress(f"offload decode: {out['offload_decode']['tokens_per_s']:.0f} tokens/s")
    if "prefill" in wl:
        out["offload_prefill"] = run_offload_prefill_chunks(torch, st, S.OLMO1B_OFFLOAD_PREFILL,
                                                            O12, max(3, args.train_steps), 1)
        torch.cuda.empty_cache()
        _progress(f"offload prefill: {out['offload_prefill']['tokens_per_s']:.0f} tokens/s")
    del O12
    if "offload" in wl:
        out["offload_train"] = run_offload_train(torch, st, S.OLMO1B_OFFLOAD_TRAIN,
                                                 args.train_steps, args.train_warmup)
        torch.cuda.empty_cache()
        _progress(f"offload train: {out['offload_train']['tokens_per_s']:.0f} tokens/s")
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
