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
(32768 Zipf tokens) through one augmented layer (dedup, compact-row gather,
forward, backward with the fp32 table-row segment-sum and all weight and input
gradients, then AdamW on the touched table rows); `decode_stem`, `train_stem`,
the same two workloads for the STEM layer (no up-projection).  With
`--workloads`: `decode7b`, `train7b` (OLMo-2-7B shapes) and `offload` (tables in
pinned host memory with a 5% HBM cache of the most frequent rows, decode and
training, PCIe-inclusive).

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


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--train-steps", type=int, default=10)
    ap.add_argument("--train-warmup", type=int, default=3)
    ap.add_argument("--workloads", default="decode,train,stem")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle baseline sample")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args(argv)


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

    # dominant kernel: the fused gate/up GEMM, one launch per layer, timed with
    # HIP events around replays of a graph holding only those launches
    gg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gg, stream=cap):
            for lay in D["layers"]:
                st.staple_ffn_gate_up_packed(lay["x"], lay["pgu"], lay["table"], D["ids"], D["h"])
    torch.cuda.synchronize()
    reps = max(20, steps // 2)
    for _ in range(5):
        gg.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        gg.replay()
    e1.record()
    torch.cuda.synchronize()
    gu_us = e0.elapsed_time(e1) / (reps * w.n_layers) * 1e3

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
            "cores": oracle_threads(), "kind": "oracle",
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
            "sample": f"first {done} tokens of the 32768-token batch in chunks of {s_tokens} "
                      "(dedup + forward + backward, float64 numpy, bf16 rounding points)"}



# ----------------------------------------------------------------------------
# Host-offloaded tables with the HBM row cache (decode batch and training batch)
# ----------------------------------------------------------------------------
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


def _miss_list_to_host(torch, lk, host_buf):
    """Copies n_miss and the miss IDs to pinned host memory (one sync)."""
    n = torch.empty(1, dtype=torch.int32, pin_memory=True)
    n.copy_(lk["n_miss"], non_blocking=True)
    host_buf[: lk["miss_ids"].numel()].copy_(lk["miss_ids"], non_blocking=True)
    torch.cuda.current_stream().synchronize()
    return int(n.item())


def run_offload_decode(torch, st, w, steps, warmup):
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    n, d, f, v, L = w.n_tokens, w.d_model, w.d_ff, w.vocab, w.n_layers
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
    ms_staged = timed(step_staged)
    m = _miss_list_to_host(torch, lk_out, miss_host)
    times = {"direct": ms_direct, "staged": ms_staged, "native": ms_native, "native_inplace": ms_inplace}
    method = min(times, key=times.get)
    ms = times[method]
    n_unique = int(dd_out["n_unique"].item())
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3),
            "method": method,
            "direct_ms_per_step": ms_direct, "native_ms_per_step": ms_native,
            "native_inplace_ms_per_step": ms_inplace, "staged_ms_per_step": ms_staged,
            "n_unique": n_unique, "misses_per_layer": m, "cache_capacity": w.cache_capacity,
            "pcie_bytes_per_step": m * f * 2 * L,
            "note": "eager steps, dedup + cache probe once per step. direct: per layer one kernel "
                    "assembles R with the hits from the HBM cache and the misses read from the "
                    "pinned host table over PCIe (no host sync, one stream), then gate/up, "
                    "down. native: one staple_decode_step_cached call per step (dedup, probe, "
                    "every layer's rows in one launch, the FFNs). native_inplace: the same call "
                    "with no compact rows, each gate/up kernel reading its tokens' rows in place "
                    "(cache slot or pinned host table). staged: "
                    "one host sync for the miss list, host pack + H2D copy per layer on a side "
                    "stream one layer ahead"}


def run_offload_train(torch, st, w, steps, warmup):
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
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    ev_copy0, ev_copy1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev_ready = torch.cuda.Event()
    stats = {"pack_s": 0.0, "copy_ms": 0.0, "hit_tokens": 0}

    def step(mode):
        dd = st.staple_dedup(T["ids"], v, out=T["dd"], workspace=T["dd_ws"])
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], O["id_to_slot"], out=lk_out)
        sp = st.staple_split_tokens(dd["inv"], lk["code"], dd["n_unique"], out=sp_out)
        counts_host.copy_(sp["counts"], non_blocking=True)
        m = _miss_list_to_host(torch, lk, miss_host)        # one host sync for both
        n_hit, n_miss_tok = int(counts_host[0]), int(counts_host[1])
        stats["hit_tokens"] = n_hit
        side.wait_stream(main)
        t0 = time.perf_counter()
        with torch.cuda.stream(side):
            ev_copy0.record(side)
        if mode == "staged":      # host pack into pinned staging, one H2D copy
            st.staple_stage_misses(O["tables"][0], miss_host, m, staging, dev_miss, stream=side)
        elif mode == "direct":    # a kernel reads the rows from the pinned host table
            with torch.cuda.stream(side):
                st.staple_gather_rows(O["tables"][0], lk["miss_ids"], lk["n_miss"], out=dev_miss,
                                      stream=side)
        # mode "resident": the miss rows are already in HBM (no copy; reference)
        with torch.cuda.stream(side):
            ev_copy1.record(side)
        stats["pack_s"] += time.perf_counter() - t0
        ev_ready.record(side)
        fw = T["fwd"]
        # the tokens whose rows are cached run while the miss rows are in flight
        st.staple_ffn_gate_up_tokens(sp["hit_pos"], n_hit, T["x"], T["w_gate"], T["w_up"],
                                     O["cache_rows"][0], sp["tok_row"], fw["h"], fw["g"], fw["u"])
        main.wait_event(ev_ready)
        st.staple_ffn_gate_up_tokens(sp["miss_pos"], n_miss_tok, T["x"], T["w_gate"], T["w_up"],
                                     dev_miss, sp["tok_row"], fw["h"], fw["g"], fw["u"])
        st.staple_ffn_down(fw["h"], T["w_down"], fw["y"])
        st.staple_ffn_bwd_table_grad(T["dy"], T["x"], T["w_gate"], T["w_up"], T["w_down"], fw["g"],
                                     fw["u"], fw["h"], dd["sorted_pos"], dd["seg_start"],
                                     dd["n_unique"], inv=dd["inv"], out=T["bwd"],
                                     workspace=T["bwd_ws"])
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
            ev_copy1.synchronize()
            copy_ms.append(ev_copy0.elapsed_time(ev_copy1))
        torch.cuda.synchronize()
        return ((time.perf_counter() - t0) / steps * 1e3, float(np.median(copy_ms)),
                stats["pack_s"] / steps * 1e3, m)

    res = {k: timed(k) for k in ("staged", "direct", "resident")}
    host_adamw = run_host_adamw(torch, st, O, T, lk_out)
    mode = min(("staged", "direct"), key=lambda k: res[k][0])
    ms, _, _, m = res[mode]
    ms_res = res["resident"][0]
    out = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": n / (ms * 1e-3),
           "method": mode, "n_unique": int(T["dd"]["n_unique"].item()), "miss_rows": m,
           "cache_capacity": w.cache_capacity, "token_hit_rate": stats["hit_tokens"] / n,
           "resident_ms_per_step": ms_res, "pcie_bytes_per_step": m * f * 2}
    out["adamw_host"] = host_adamw
    for k in ("staged", "direct"):
        ms_k, copy_k, pack_k, _ = res[k]
        out[k] = {"ms_per_step": ms_k, "copy_ms": copy_k, "host_pack_ms": pack_k,
                  "pcie_gb_s": m * f * 2 / (copy_k * 1e-3) / 1e9,
                  "hidden_fraction_of_copy": max(0.0, min(1.0, 1.0 - max(0.0, ms_k - ms_res) /
                                                          max(copy_k + pack_k, 1e-9)))}
    out["note"] = ("eager step: dedup + cache probe + token split, one host sync for the miss "
                   "list and the split counts; the miss rows move on a side stream (staged: host "
                   "pack into pinned staging + one H2D copy; direct: a kernel reads them from the "
                   "pinned host table) while the gate/up GEMM of the cached tokens runs (rows "
                   "from the cache slots); then the missed tokens' gate/up, down, backward. "
                   "resident: the same step with the miss rows already in HBM, for the hidden "
                   "fraction = 1 - (t - t_resident) / (host pack + copy time)")
    return out


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
    if "decode7b" in wl:
        w7 = S.OLMO7B_DECODE
        dec7, D7 = run_decode(torch, st, w7, max(20, args.steps // 2), args.warmup)
        out["decode_7b"] = dict(dec7, workload=w7.name)
        del D7
        torch.cuda.empty_cache()
    if "train7b" in wl:
        w7 = S.OLMO7B_TRAIN
        tr7, T7 = run_train(torch, st, w7, args.train_steps, args.train_warmup)
        out["train_7b"] = tr7
        del T7
        torch.cuda.empty_cache()
    if "stem" in wl:
        # the STEM layer STAPLE is compared against (no up-projection), same workloads
        dec_s, D_s = run_decode(torch, st, w, args.steps, args.warmup, stem=True)
        out["decode_stem"] = dict(dec_s, workload=w.name + "_stem")
        del D_s
        torch.cuda.empty_cache()
        tr_s, T_s = run_train(torch, st, S.OLMO1B_TRAIN, args.train_steps, args.train_warmup,
                              stem=True)
        out["train_stem"] = dict(tr_s, workload=S.OLMO1B_TRAIN.name + "_stem")
        del T_s
        torch.cuda.empty_cache()
    if "offload" in wl:
        out["offload_decode"] = run_offload_decode(torch, st, S.OLMO1B_OFFLOAD, 20, 3)
        torch.cuda.empty_cache()
        out["offload_train"] = run_offload_train(torch, st, S.OLMO1B_OFFLOAD_TRAIN,
                                                 args.train_steps, args.train_warmup)
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
