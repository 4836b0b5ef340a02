"""Host-offloaded tables at full size (OLMo-2-1B shapes): twelve 100352 x 8192
bf16 tables in pinned host memory, the 5018 most frequent rows of each
(ranked by a seeded count pass) cached in HBM.

* The 64-token decode step through staple_decode_step_cached, with the rows
  assembled (misses read from the pinned tables) and read in place, against
  the oracle on every token and feature of every layer.
* The 32768-token training batch split by cache outcome: the cached tokens'
  gate/up reads the HBM cache, the others' the miss rows packed on the host
  and copied over PCIe; h, g, u have the bits of the whole-batch gate/up over
  the rows gathered from the host table, and h matches the oracle on sampled
  features.
* The 16384-token prefill in chunks of 4096 over two layers, the next
  chunk's rows assembled on a second stream: y has the bits of the whole
  batch in one pass and matches the oracle on sampled tokens.
"""
import sys

import numpy as np
import pytest

import staple_synth as S
from oracle import staple_oracle as O
from tests.helpers import assert_close, assert_close_stored_bf16, to_np

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def st():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_indexed_ffn_amd as st
    st.lib()
    return st


@pytest.fixture(scope="module")
def dev(st):
    import torch
    return torch.device("cuda:0")


class _Rows:
    """A [vocab x f] table that holds only the rows of some sorted IDs."""

    def __init__(self, ids_sorted, rows):
        self.ids = np.asarray(ids_sorted)
        self.rows = rows

    def __getitem__(self, key):
        if isinstance(key, tuple):
            r, c = key
            r = np.asarray(r).reshape(-1)
            return self.rows[np.searchsorted(self.ids, r)][:, np.asarray(c).reshape(-1)]
        return self.rows[np.searchsorted(self.ids, np.asarray(key))]


def _host_tables(torch, st, w, n_layers, dev):
    """Pinned host tables (drawn on the device, copied out), the count-ranked
    cache and every layer's cached rows."""
    from staple_synth import device_normal
    counts = torch.from_numpy(S.calibration_counts(w.vocab)).to(dev)
    cap = w.cache_capacity
    id_to_slot, slot_to_id = st.staple_cache_build(counts, cap)
    tables, cache_rows = [], []
    for l in range(n_layers):
        dtab = device_normal((w.vocab, w.d_ff), w.table_std, w.layer_seeds(l)["table"],
                             torch.bfloat16, dev)
        htab = torch.empty((w.vocab, w.d_ff), dtype=torch.bfloat16, pin_memory=True)
        htab.copy_(dtab)
        del dtab
        tables.append(htab)
        cache_rows.append(st.staple_cache_fill(htab, slot_to_id, cap))
    torch.cuda.synchronize()
    # the cache is the oracle's ranking of the same counts
    i2s, s2i = O.cache_build(S.calibration_counts(w.vocab), cap)
    np.testing.assert_array_equal(to_np(id_to_slot), i2s)
    np.testing.assert_array_equal(to_np(slot_to_id)[:cap], s2i)
    return id_to_slot, tables, cache_rows


@pytest.mark.timeout(900)
def test_offloaded_decode_step_full_size(st, dev):
    import torch
    from staple_synth import device_normal
    w = S.OLMO1B_OFFLOAD
    n, d, f, L = w.n_tokens, w.d_model, w.d_ff, w.n_layers
    _log(f"offloaded decode, {L} pinned {w.vocab} x {f} tables, cache {w.cache_capacity}")
    id_to_slot, tables, cache_rows = _host_tables(torch, st, w, L, dev)
    ids_np = w.ids()
    ids = torch.from_numpy(ids_np).to(dev)
    layers = []
    for l in range(L):
        s = w.layer_seeds(l)
        lay = {k: device_normal(shape, std, s[k], torch.bfloat16, dev) for k, shape, std in (
            ("x", (n, d), w.x_std), ("w_gate", (f, d), w.w_std), ("w_up", (f, d), w.w_std),
            ("w_down", (d, f), w.w_std))}
        lay["pgu"], lay["pd"] = st.staple_decode_pack_weights(lay["w_gate"], lay["w_up"],
                                                              lay["w_down"], d_model=d, d_ff=f)
        layers.append(lay)
    i32 = dict(dtype=torch.int32, device=dev)
    dd = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
          "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
          "n_unique": torch.empty(1, **i32)}
    lk = {k: torch.empty(n, **i32) for k in ("code", "miss_uidx")}
    lk["n_miss"] = torch.empty(1, **i32)
    ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)
    nan = lambda: torch.full((n, d), float("nan"), dtype=torch.float32, device=dev)
    R = [torch.empty(n, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ys_a = [nan() for _ in range(L)]
    ys_b = [nan() for _ in range(L)]
    common = lambda l: {"x": layers[l]["x"], "packed_gate_up": layers[l]["pgu"],
                        "packed_down": layers[l]["pd"], "cache_rows": cache_rows[l],
                        "table": tables[l]}
    assembled = st.DecodeStack([dict(common(l), rows=R[l], y=ys_a[l]) for l in range(L)],
                               d_model=d, d_ff=f, n_tokens=n)
    in_place = st.DecodeStack([dict(common(l), y=ys_b[l]) for l in range(L)],
                              d_model=d, d_ff=f, n_tokens=n)
    for stack in (assembled, in_place):
        st.staple_decode_step_cached(stack, ids, id_to_slot, w.cache_capacity, dedup_out=dd,
                                     lookup_out=lk, workspace=ws)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    # groups of four layers with carried row copies, over separate tables and
    # over tables interleaved token-major by groups of four
    grouped = [st.staple_group_tables_host(tables[g:g + 4]) for g in range(0, L, 4)]
    ys_c = [nan() for _ in range(L)]
    ys_g = [nan() for _ in range(L)]
    R_c = [torch.empty(n, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    R_g = [torch.empty(n, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    carried = st.DecodeStack([dict(common(l), rows=R_c[l], y=ys_c[l]) for l in range(L)],
                             d_model=d, d_ff=f, n_tokens=n)
    grouped_stack = st.DecodeStack(
        [dict(common(l), table=(grouped[l // 4], (l % 4) * f, 4 * f), rows=R_g[l], y=ys_g[l])
         for l in range(L)], d_model=d, d_ff=f, n_tokens=n)
    for stack in (carried, grouped_stack):
        st.staple_decode_step_cached(stack, ids, id_to_slot, w.cache_capacity, dedup_out=dd,
                                     lookup_out=lk, workspace=ws, group=4)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    nu = int(dd["n_unique"].item())
    for l in range(L):
        assert torch.equal(ys_c[l], ys_a[l]) and torch.equal(ys_g[l], ys_a[l]), f"layer {l}"
        assert torch.equal(R_c[l][:nu], R[l][:nu]) and torch.equal(R_g[l][:nu], R[l][:nu]), \
            f"layer {l} rows"
    uniq = np.unique(ids_np)
    u = len(uniq)
    assert int(dd["n_unique"].item()) == u
    np.testing.assert_array_equal(to_np(dd["uniq"])[:u], uniq)
    code, miss = O.cache_lookup(uniq, to_np(id_to_slot))
    np.testing.assert_array_equal(to_np(lk["code"])[:u], code)
    assert int(lk["n_miss"].item()) == len(miss)
    _log(f"  {u} unique IDs, {len(miss)} misses per layer")
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    for l in range(L):
        assert not bool(torch.isnan(ys_a[l]).any()), f"layer {l}: y has unwritten elements"
        assert torch.equal(ys_a[l], ys_b[l]), f"layer {l}: in-place rows give other bits"
        host_rows = tables[l][torch.from_numpy(uniq.astype(np.int64))]
        assert torch.equal(R[l][:u].cpu(), host_rows), f"layer {l}: compact rows"
        lay = layers[l]
        of = O.ffn_forward(f64(lay["x"]), f64(lay["w_gate"]), f64(lay["w_up"]), f64(lay["w_down"]),
                           _Rows(uniq, f64(host_rows)), ids_np, precision=O.BF16)
        assert_close(f64(ys_a[l]), of["y"], f"layer {l} y")


@pytest.mark.timeout(900)
def test_offloaded_training_split_full_size(st, dev):
    import torch
    from staple_synth import device_normal
    w = S.OLMO1B_OFFLOAD_TRAIN
    n, d, f, v = w.n_tokens, w.d_model, w.d_ff, w.vocab
    _log(f"offloaded training split, {n} tokens, cache {w.cache_capacity}")
    id_to_slot, tables, cache_rows = _host_tables(torch, st, w, 1, dev)
    htab, crows = tables[0], cache_rows[0]
    s = w.layer_seeds(0)
    x = device_normal((n, d), w.x_std, s["x"], torch.bfloat16, dev)
    wg = device_normal((f, d), w.w_std, s["w_gate"], torch.bfloat16, dev)
    wu = device_normal((f, d), w.w_std, s["w_up"], torch.bfloat16, dev)
    ids_np = w.ids()
    ids = torch.from_numpy(ids_np).to(dev)
    dd = st.staple_dedup(ids, v)
    lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], id_to_slot)
    sp = st.staple_split_tokens(dd["inv"], lk["code"], dd["n_unique"])
    torch.cuda.synchronize()
    n_miss = int(lk["n_miss"].item())
    n_hit, n_miss_tok = (int(c) for c in sp["counts"].cpu())
    _log(f"  {n_miss} miss rows, {n_hit} cached tokens, {n_miss_tok} others")
    miss_host = lk["miss_ids"][:max(n_miss, 1)].cpu().contiguous()
    staging = torch.empty(max(n_miss, 1), f, dtype=torch.bfloat16, pin_memory=True)
    dev_miss = torch.empty(max(n_miss, 1), f, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    st.staple_stage_misses(htab, miss_host, n_miss, staging, dev_miss, stream=side)
    ready = torch.cuda.Event()
    ready.record(side)
    bf = dict(dtype=torch.bfloat16, device=dev)
    h, g, u = (torch.full((n, f), float("nan"), **bf) for _ in range(3))
    st.staple_ffn_gate_up_tokens(sp["hit_pos"], n_hit, x, wg, wu, crows, sp["tok_row"], h, g, u)
    torch.cuda.current_stream().wait_event(ready)
    st.staple_ffn_gate_up_tokens(sp["miss_pos"], n_miss_tok, x, wg, wu, dev_miss, sp["tok_row"],
                                 h, g, u)
    # the whole batch over the compact rows gathered from the host table
    R = st.staple_gather_rows(htab, dd["uniq"], dd["n_unique"])
    h2, g2, u2 = (torch.empty(n, f, **bf) for _ in range(3))
    st.staple_ffn_gate_up(x, wg, wu, R, dd["inv"], h2, g2, u2)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    assert n_hit + n_miss_tok == n
    for a, b, k in ((h, h2, "h"), (g, g2, "g"), (u, u2, "u")):
        assert not bool(torch.isnan(a).any()), f"{k} has unwritten elements"
        assert torch.equal(a, b), f"split {k} differs from the whole batch"
    # h on sampled features against the oracle
    uniq = np.unique(ids_np)
    rng = np.random.default_rng(1)
    cols = np.unique(np.concatenate([[0, f - 1], rng.choice(f, 30, replace=False)]))
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    host_rows = f64(htab[torch.from_numpy(uniq.astype(np.int64))])
    of = O.ffn_forward(f64(x), f64(wg), f64(wu), None, _Rows(uniq, host_rows), ids_np,
                       precision=O.BF16, cols=cols)
    cs = torch.from_numpy(cols).to(dev)
    assert_close_stored_bf16(f64(h[:, cs]), of["h"], "split h[:, cols]")
    assert_close_stored_bf16(f64(u[:, cs]), of["u_saved"], "split u[:, cols]")


@pytest.mark.timeout(900)
def test_offloaded_prefill_pipeline_full_size(st, dev):
    """The prefill of 64 prompts x 256 tokens over two layers of pinned
    100352 x 8192 tables with the 5018-row cache, in chunks of 4096 tokens:
    chunk c + 1's rows assembled on a second stream on 16 workgroups while
    chunk c's layers run.  Every layer's y has the bits of the whole batch in
    one pass, and matches the oracle on one token of every 256."""
    import torch
    from staple_synth import device_normal
    w = S.OLMO1B_OFFLOAD_PREFILL
    n, d, f, L, C = w.n_tokens, w.d_model, w.d_ff, 2, 4096
    nc = n // C
    cap = w.cache_capacity
    _log(f"offloaded prefill, {n} tokens in chunks of {C}, {L} pinned tables, cache {cap}")
    id_to_slot, tables, cache_rows = _host_tables(torch, st, w, L, dev)
    ids_np = w.ids()
    ids = torch.from_numpy(ids_np).to(dev)
    layers = []
    for l in range(L):
        s = w.layer_seeds(l)
        layers.append({k: device_normal(shape, std, s[k], torch.bfloat16, dev) for k, shape, std in (
            ("x", (n, d), w.x_std), ("w_gate", (f, d), w.w_std), ("w_up", (f, d), w.w_std),
            ("w_down", (d, f), w.w_std))})
    # the whole batch in one pass
    dd = st.staple_dedup(ids, w.vocab)
    lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], id_to_slot)
    y_ref = []
    for l, lay in enumerate(layers):
        R = st.staple_assemble_rows_from_table(cache_rows[l], tables[l], dd["uniq"], lk["code"],
                                               dd["n_unique"], capacity=cap)
        y_ref.append(st.staple_ffn_fwd(lay["x"], lay["w_gate"], lay["w_up"], lay["w_down"], R,
                                       dd["inv"], out_dtype=torch.float32)["y"])
    torch.cuda.synchronize()
    # the pipelined chunks
    i32 = dict(dtype=torch.int32, device=dev)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    bufs = []
    for _ in range(2):
        B = {"dd": {"uniq": torch.empty(C, **i32), "inv": torch.empty(C, **i32),
                    "sorted_pos": torch.empty(C, **i32), "seg_start": torch.empty(C + 1, **i32),
                    "n_unique": torch.empty(1, **i32)},
             "lk": {"code": torch.empty(C, **i32), "miss_uidx": torch.empty(C, **i32),
                    "n_miss": torch.empty(1, **i32)},
             "rows": [torch.empty(C, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]}
        B["rs"] = st.RowSources([{"table": tables[l], "cache_rows": cache_rows[l],
                                  "rows": B["rows"][l]} for l in range(L)], d_ff=f)
        bufs.append(B)
    y = [torch.full((n, d), float("nan"), dtype=torch.float32, device=dev) for _ in range(L)]
    ready = [torch.cuda.Event() for _ in range(nc)]
    done = [torch.cuda.Event() for _ in range(nc)]
    main.wait_stream(torch.cuda.current_stream())
    side.wait_stream(torch.cuda.current_stream())

    def issue(c):
        if c >= 2:
            side.wait_event(done[c - 2])
        B = bufs[c % 2]
        st.staple_prefill_rows_cached(B["rs"], ids[c * C:(c + 1) * C], id_to_slot, cap,
                                      dedup_out=B["dd"], lookup_out=B["lk"], workspace=None,
                                      max_workgroups=16 if c > 0 else 0, stream=side)
        ready[c].record(side)

    issue(0)
    with torch.cuda.stream(main):
        for c in range(nc):
            if c + 1 < nc:
                issue(c + 1)
            main.wait_event(ready[c])
            B = bufs[c % 2]
            for l, lay in enumerate(layers):
                st.staple_ffn_fwd(lay["x"][c * C:(c + 1) * C], lay["w_gate"], lay["w_up"],
                                  lay["w_down"], B["rows"][l], B["dd"]["inv"],
                                  out={"y": y[l][c * C:(c + 1) * C]}, stream=main)
            done[c].record(main)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    toks = np.arange(0, n, 256)
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    for l, lay in enumerate(layers):
        assert not bool(torch.isnan(y[l]).any()), f"layer {l}: a chunk was not written"
        assert torch.equal(y[l], y_ref[l]), f"layer {l}: pipelined prefill differs"
        sel = np.unique(ids_np[toks])
        rows = f64(tables[l][torch.from_numpy(sel.astype(np.int64))])
        tk = torch.from_numpy(toks).to(dev)
        of = O.ffn_forward(f64(lay["x"][tk]), f64(lay["w_gate"]), f64(lay["w_up"]),
                           f64(lay["w_down"]), _Rows(sel, rows), ids_np[toks], precision=O.BF16)
        assert_close(f64(y[l][tk]), of["y"], f"prefill layer {l} y (sampled tokens)")
