"""Stack-level pipelining over host-offloaded tables, through the C ABI.

* staple_prefill_rows_cached (one call per prefill chunk: dedup, cache probe,
  every layer's compact rows in one launch with a workgroup cap) gives the
  same bits as the separate calls, and its rows are the table's rows.
* A chunked prefill pipelined over two streams (the next chunk's rows
  assembled on a side stream while the current chunk's layers run) gives
  every layer's y bit for bit as the whole batch in one pass, and within the
  parity tolerance of the oracle.
* The offloaded decode step captured in a HIP graph and replayed with new
  token IDs gives, on every replay, the same bits as the eager step.
"""
import sys

import numpy as np
import pytest

import staple_synth as S
from oracle import staple_oracle as O
from tests.helpers import assert_close, to_dev, to_np

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


def _no_device_error(st):
    assert st.staple_get_device_error() == 0


def _pinned_table(torch, inp):
    return torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()


def _outputs(torch, n, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    dd = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
          "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
          "n_unique": torch.empty(1, **i32)}
    lk = {"code": torch.empty(n, **i32), "miss_uidx": torch.empty(n, **i32),
          "n_miss": torch.empty(1, **i32)}
    return dd, lk


def _workspace(torch, st, n, dev):
    nb = st.prefill_rows_workspace_bytes(n)
    return torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None


@pytest.mark.parametrize("n,vocab,cap,wgs,layout", [
    (700, 500, 40, 0, "separate"),        # dedup in one workgroup, rows on the full grid
    (700, 500, 0, 3, "separate"),         # no cache: every row over PCIe, three workgroups
    (64, 500, 40, 1, "grouped"),          # a decode-sized chunk, one workgroup
    (5000, 3000, 40, 7, "grouped"),       # multi-workgroup dedup, interleaved tables
    (5000, 3000, 200, 0, "separate"),
])
def test_prefill_rows_match_the_separate_calls(st, dev, n, vocab, cap, wgs, layout):
    import torch
    L, f = 3, 256
    _log(f"prefill rows n={n} vocab={vocab} cap={cap} max_workgroups={wgs} layout={layout}")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 4)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    inps = [S.host_layer_inputs(8, 64, f, vocab, dtype="bf16", seed=300 + l, table_std=0.5)
            for l in range(L)]
    tables = [_pinned_table(torch, inp) for inp in inps]
    caches = [st.staple_cache_fill(t, s2i, cap) if cap else None for t in tables]
    grouped = st.staple_group_tables_host(tables) if layout == "grouped" else None
    srcs = []
    for l in range(L):
        tab = tables[l] if grouped is None else (grouped, l * f, L * f)
        srcs.append({"table": tab, "cache_rows": caches[l],
                     "rows": torch.zeros(n, f, dtype=torch.bfloat16, device=dev)})
    rs = st.RowSources(srcs, d_ff=f)
    ids_np = S.zipf_ids(n, vocab, 31 + n)
    ids = torch.from_numpy(ids_np).to(dev)
    dd, lk = _outputs(torch, n, dev)
    st.staple_prefill_rows_cached(rs, ids, i2s, cap, dedup_out=dd, lookup_out=lk,
                                  workspace=_workspace(torch, st, n, dev), max_workgroups=wgs)
    torch.cuda.synchronize()
    _no_device_error(st)
    # the separate calls
    rd = st.staple_dedup(ids, vocab)
    rl = st.staple_cache_lookup(rd["uniq"], rd["n_unique"], i2s)
    torch.cuda.synchronize()
    u = int(rd["n_unique"].item())
    assert int(dd["n_unique"].item()) == u == len(np.unique(ids_np))
    assert torch.equal(dd["uniq"][:u], rd["uniq"][:u])
    assert torch.equal(dd["sorted_pos"], rd["sorted_pos"])
    assert torch.equal(dd["inv"], rd["inv"])
    assert torch.equal(dd["seg_start"][:u + 1], rd["seg_start"][:u + 1])
    m = int(rl["n_miss"].item())
    assert int(lk["n_miss"].item()) == m
    assert torch.equal(lk["code"][:u], rl["code"][:u])
    assert torch.equal(lk["miss_uidx"][:m], rl["miss_uidx"][:m])
    uniq = rd["uniq"][:u].cpu().numpy()
    for l in range(L):
        ref = st.staple_assemble_rows_from_table(caches[l], tables[l], rd["uniq"], rl["code"],
                                                 rd["n_unique"], capacity=cap)
        torch.cuda.synchronize()
        assert torch.equal(srcs[l]["rows"][:u], ref[:u]), f"layer {l}"
        # the rows are the table's rows of the unique IDs
        got = srcs[l]["rows"][:u].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, inps[l].table[uniq]), f"layer {l} vs table"
    # lookup off: the rows again from the outputs left by the first call (the
    # IDs passed are not read), the dedup and probe outputs untouched
    kept = [srcs[l]["rows"][:u].clone() for l in range(L)]
    kept_dd = {k: t.clone() for k, t in dd.items()}
    for x in srcs:
        x["rows"].zero_()
    st.staple_prefill_rows_cached(rs, torch.flip(ids, [0]).contiguous(), i2s, cap, dedup_out=dd,
                                  lookup_out=lk, workspace=_workspace(torch, st, n, dev),
                                  max_workgroups=wgs, lookup=False)
    torch.cuda.synchronize()
    _no_device_error(st)
    for l in range(L):
        assert torch.equal(srcs[l]["rows"][:u], kept[l]), f"layer {l}, lookup off"
    for k, t in kept_dd.items():
        assert torch.equal(dd[k], t), k
    # the misses staged by the DMA engines instead, then assembled with the
    # cached rows: the same compact rows
    miss_h = rl["miss_ids"][:max(m, 1)].cpu().contiguous()
    staging = torch.empty(L * max(m, 1) * f, dtype=torch.bfloat16, pin_memory=True)
    blocks = [torch.empty(max(m, 1), f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    st.staple_stage_misses_dma([src["table"] for src in srcs], miss_h, m, staging, blocks)
    for l in range(L):
        cache = caches[l] if caches[l] is not None else torch.zeros(1, f, dtype=torch.bfloat16,
                                                                   device=dev)
        staged = st.staple_assemble_rows(cache, blocks[l], rl["code"], rd["n_unique"])
        torch.cuda.synchronize()
        assert torch.equal(staged[:u], kept[l]), f"layer {l}, DMA-staged misses"
    _no_device_error(st)


def test_chunked_prefill_pipeline_matches_the_whole_batch(st, dev):
    """Three chunks of 700 tokens through three layers: chunk c + 1's rows are
    assembled on a side stream (four workgroups, pinned host tables, an HBM
    cache) while chunk c's layers run on the main stream; row buffers are
    double-buffered and reused only after the chunk that read them.  In the
    first chunk each layer's rows come from a call of their own (the first
    with the dedup and probe, the others with lookup off), each awaited just
    before its layer."""
    import torch
    L, d, f, vocab, cap, C, n_chunks = 3, 128, 256, 500, 40, 700, 3
    n = C * n_chunks
    _log(f"chunked prefill pipeline: {n_chunks} chunks of {C} tokens, {L} layers")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 5)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    inps = [S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=340 + l, table_std=0.5)
            for l in range(L)]
    W = []
    for inp in inps:
        lay = {k: to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "w_down")}
        lay["table"] = _pinned_table(torch, inp)
        lay["cache"] = st.staple_cache_fill(lay["table"], s2i, cap)
        W.append(lay)
    ids_np = S.zipf_ids(n, vocab, 77)
    ids = torch.from_numpy(ids_np).to(dev)

    # the whole batch in one pass
    rd = st.staple_dedup(ids, vocab)
    rl = st.staple_cache_lookup(rd["uniq"], rd["n_unique"], i2s)
    y_ref = []
    for lay in W:
        R = st.staple_assemble_rows_from_table(lay["cache"], lay["table"], rd["uniq"], rl["code"],
                                               rd["n_unique"], capacity=cap)
        y_ref.append(st.staple_ffn_fwd(lay["x"], lay["w_gate"], lay["w_up"], lay["w_down"], R,
                                       rd["inv"], out_dtype=torch.float32)["y"])
    torch.cuda.synchronize()

    # the pipelined chunks
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    bufs = []
    for b in range(2):
        dd, lk = _outputs(torch, C, dev)
        rows = [torch.empty(C, f, dtype=torch.bfloat16, device=dev) for _ in range(L)]
        srcs = [{"table": lay["table"], "cache_rows": lay["cache"], "rows": r}
                for lay, r in zip(W, rows)]
        bufs.append({"dd": dd, "lk": lk, "rows": rows, "rs": st.RowSources(srcs, d_ff=f),
                     "rs_layer": [st.RowSources([x], d_ff=f) for x in srcs],
                     "ws": _workspace(torch, st, C, dev)})
    y = [torch.full((n, d), float("nan"), dtype=torch.float32, device=dev) for _ in range(L)]
    ready = [torch.cuda.Event() for _ in range(n_chunks)]
    done = [torch.cuda.Event() for _ in range(n_chunks)]
    side.wait_stream(main)

    def issue_rows(c):
        B = bufs[c % 2]
        if c >= 2:
            side.wait_event(done[c - 2])       # chunk c - 2 has finished reading these buffers
        st.staple_prefill_rows_cached(B["rs"], ids[c * C:(c + 1) * C], i2s, cap,
                                      dedup_out=B["dd"], lookup_out=B["lk"], workspace=B["ws"],
                                      max_workgroups=4, stream=side)
        ready[c].record(side)

    # chunk 0: layer 0's rows with the dedup and probe, then each later
    # layer's rows alone (lookup off), each awaited just before its layer
    layer_ready = [torch.cuda.Event() for _ in range(L)]
    B0 = bufs[0]
    for l in range(L):
        st.staple_prefill_rows_cached(B0["rs_layer"][l], ids[:C], i2s, cap, dedup_out=B0["dd"],
                                      lookup_out=B0["lk"], workspace=B0["ws"], max_workgroups=2,
                                      lookup=l == 0, stream=side)
        layer_ready[l].record(side)
    for c in range(n_chunks):
        if c + 1 < n_chunks:
            issue_rows(c + 1)
        if c > 0:
            main.wait_event(ready[c])
        B = bufs[c % 2]
        for l, lay in enumerate(W):
            if c == 0:
                main.wait_event(layer_ready[l])
            st.staple_ffn_fwd(lay["x"][c * C:(c + 1) * C], lay["w_gate"], lay["w_up"],
                              lay["w_down"], B["rows"][l], B["dd"]["inv"],
                              out={"y": y[l][c * C:(c + 1) * C]}, stream=main)
        done[c].record(main)
    torch.cuda.synchronize()
    _no_device_error(st)
    for l in range(L):
        assert not torch.isnan(y[l]).any(), f"layer {l}: a chunk was not written"
        assert torch.equal(y[l], y_ref[l]), f"layer {l}"
    # the oracle on the first and last layers
    for l in (0, L - 1):
        g = {k: inps[l].as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table")}
        of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], ids_np,
                           precision=O.BF16)
        assert_close(to_np(y[l]), of["y"], f"pipelined prefill y layer {l}")


@pytest.mark.parametrize("group,in_place", [(2, False), (0, True)])
def test_decode_step_graph_replays_match_eager(st, dev, group, in_place):
    """The offloaded decode step (pinned tables, an HBM cache; the rows of
    later groups carried by the previous group's launches, or read in place)
    captured once in a HIP graph over a static ID buffer, then replayed with
    new IDs four times, eager steps and synchronisations in between: every
    replay gives each layer's y (and compact rows) bit for bit as the eager
    step on the same IDs."""
    import torch
    L, n, d, f, vocab, cap = 5, 64, 64, 256, 300, 40
    _log(f"decode step graph capture group={group} in_place={in_place}")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 6)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    base = []
    for l in range(L):
        inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=360 + l, table_std=0.5)
        x, wg, wu, wd = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "w_down"))
        tab = _pinned_table(torch, inp)
        pgu, pd = st.staple_decode_pack_weights(wg, wu, wd, d_model=d, d_ff=f)
        base.append({"x": x, "packed_gate_up": pgu, "packed_down": pd, "table": tab,
                     "cache_rows": st.staple_cache_fill(tab, s2i, cap)})

    def make():
        lays = [dict(b, rows=None if in_place else torch.zeros(n, f, dtype=torch.bfloat16, device=dev),
                     y=torch.zeros(n, d, dtype=torch.float32, device=dev)) for b in base]
        dd, lk = _outputs(torch, n, dev)
        ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)
        return lays, st.DecodeStack(lays, d_model=d, d_ff=f, n_tokens=n), dd, lk, ws

    e_lays, e_stack, e_dd, e_lk, e_ws = make()
    g_lays, g_stack, g_dd, g_lk, g_ws = make()
    ids_static = torch.from_numpy(S.zipf_ids(n, vocab, 500)).to(dev)
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        # first call eagerly: per-kernel attributes are set outside the capture
        st.staple_decode_step_cached(g_stack, ids_static, i2s, cap, dedup_out=g_dd,
                                     lookup_out=g_lk, workspace=g_ws, group=group)
        cap_stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap_stream):
            st.staple_decode_step_cached(g_stack, ids_static, i2s, cap, dedup_out=g_dd,
                                         lookup_out=g_lk, workspace=g_ws, group=group)
    torch.cuda.synchronize()
    _no_device_error(st)
    for k in range(4):
        ids = torch.from_numpy(S.zipf_ids(n, vocab, 510 + k)).to(dev)
        st.staple_decode_step_cached(e_stack, ids, i2s, cap, dedup_out=e_dd, lookup_out=e_lk,
                                     workspace=e_ws, group=group)
        ids_static.copy_(ids)
        for lay in g_lays:
            lay["y"].fill_(float("nan"))
            if lay["rows"] is not None:
                lay["rows"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _no_device_error(st)
        u = int(e_dd["n_unique"].item())
        assert int(g_dd["n_unique"].item()) == u
        assert torch.equal(g_dd["inv"], e_dd["inv"]), k
        assert torch.equal(g_lk["code"][:u], e_lk["code"][:u]), k
        for l in range(L):
            assert torch.equal(g_lays[l]["y"], e_lays[l]["y"]), (k, l)
            if not in_place:
                assert torch.equal(g_lays[l]["rows"][:u], e_lays[l]["rows"][:u]), (k, l)
    # the last replay against the oracle on one layer
    ids_np = S.zipf_ids(n, vocab, 513)
    inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=360 + L - 1, table_std=0.5)
    g = {kk: inp.as_f64(kk) for kk in ("x", "w_gate", "w_up", "w_down", "table")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], ids_np,
                       precision=O.BF16)
    assert_close(to_np(g_lays[L - 1]["y"]), of["y"], "graph-replayed decode y")


def test_prefill_rows_refuses_short_outputs_and_mixed_dtypes(st, dev):
    """Outputs or rows shorter than the chunk, a cache shorter than the
    capacity, and tables of another dtype are refused on the host; nothing is
    written."""
    import torch
    n, f, vocab, cap = 100, 64, 50, 4
    table = torch.zeros(vocab, f, dtype=torch.bfloat16).pin_memory()
    cache = torch.zeros(cap, f, dtype=torch.bfloat16, device=dev)
    rows = torch.zeros(n, f, dtype=torch.bfloat16, device=dev)
    i2s = torch.full((vocab,), -1, dtype=torch.int32, device=dev)
    ids = torch.zeros(n, dtype=torch.int32, device=dev)
    rs = st.RowSources([{"table": table, "cache_rows": cache, "rows": rows}], d_ff=f)
    dd, lk = _outputs(torch, n, dev)
    kw = dict(dedup_out=dd, lookup_out=lk, workspace=None)
    short = dict(dd, uniq=dd["uniq"][: n - 1])
    with pytest.raises(ValueError, match="uniq"):
        st.staple_prefill_rows_cached(rs, ids, i2s, cap, **dict(kw, dedup_out=short))
    with pytest.raises(ValueError, match="seg_start"):
        st.staple_prefill_rows_cached(rs, ids, i2s, cap,
                                      **dict(kw, dedup_out=dict(dd, seg_start=dd["seg_start"][:n])))
    with pytest.raises(ValueError, match="cache_rows"):
        st.staple_prefill_rows_cached(rs, ids, i2s, cap + 1, **kw)
    with pytest.raises(ValueError, match="ids"):
        st.staple_prefill_rows_cached(rs, ids.to(torch.int64), i2s, cap, **kw)
    with pytest.raises(ValueError, match="rows"):
        st.staple_prefill_rows_cached(rs, torch.zeros(n + 1, dtype=torch.int32, device=dev), i2s,
                                      cap, **dict(kw, **{k: v for k, v in
                                                        zip(("dedup_out", "lookup_out"),
                                                            _outputs(torch, n + 1, dev))}))
    with pytest.raises(ValueError, match="dtype"):
        st.RowSources([{"table": table.float().pin_memory(), "cache_rows": cache, "rows": rows}],
                      d_ff=f)
    torch.cuda.synchronize()
    assert not rows.any()


def test_prefill_rows_of_a_stack_longer_than_one_launch(st, dev):
    """Forty layers: the rows are assembled in launches of at most 32 layers;
    every layer's rows are its own table's rows (some layers cached, the
    tables in pinned host memory and on the device)."""
    import torch
    L, n, f, vocab, cap = 40, 300, 64, 200, 10
    _log(f"prefill rows over {L} layers")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(5000, vocab, 8)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    rng = np.random.default_rng(5)
    hosts = [rng.integers(0, 1 << 16, size=(vocab, f), dtype=np.uint16) for _ in range(L)]
    srcs = []
    for l, tb in enumerate(hosts):
        t = torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16)
        tab = t.pin_memory() if l % 2 == 0 else t.to(dev)
        srcs.append({"table": tab, "cache_rows": st.staple_cache_fill(tab, s2i, cap),
                     "rows": torch.zeros(n, f, dtype=torch.bfloat16, device=dev)})
    rs = st.RowSources(srcs, d_ff=f)
    ids_np = S.zipf_ids(n, vocab, 41)
    dd, lk = _outputs(torch, n, dev)
    st.staple_prefill_rows_cached(rs, torch.from_numpy(ids_np).to(dev), i2s, cap, dedup_out=dd,
                                  lookup_out=lk, workspace=_workspace(torch, st, n, dev),
                                  max_workgroups=5)
    torch.cuda.synchronize()
    _no_device_error(st)
    uniq = np.unique(ids_np)
    u = len(uniq)
    assert int(dd["n_unique"].item()) == u
    for l in range(L):
        got = srcs[l]["rows"][:u].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, hosts[l][uniq]), f"layer {l}"


@pytest.mark.parametrize("grouped", [False, True])
def test_stage_misses_dma_rows_reach_the_device(st, dev, grouped):
    """staple_stage_misses_dma: every layer's miss rows land in its device block
    as the host tables' bytes (separate tables, and tables interleaved by fours);
    over several calls into the same blocks, each after a kernel has read the
    previous contents, a kernel reading the blocks (the compact-row assembly)
    sees the new rows."""
    import torch
    L, v, f = 4, 3000, 2048
    _log(f"stage misses dma grouped={grouped}")
    gen = torch.Generator().manual_seed(41)
    tables = [torch.randn(v, f, generator=gen).to(torch.bfloat16) for _ in range(L)]
    if grouped:
        inter = st.staple_group_tables_host(tables)
        srcs = [(inter, l * f, L * f) for l in range(L)]
    else:
        srcs = tables
    n_max = 700
    staging = torch.empty(L * n_max * f, dtype=torch.bfloat16, pin_memory=True)
    blocks = [torch.full((n_max, f), float("nan"), dtype=torch.bfloat16, device=dev)
              for _ in range(L)]
    cache = torch.zeros(4, f, dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(7)
    for call, n in enumerate((n_max, 333, 1, 610)):
        ids = rng.choice(v, size=n, replace=False).astype(np.int32)
        st.staple_stage_misses_dma(srcs, torch.from_numpy(ids), n, staging, blocks)
        code = torch.from_numpy(-1 - np.arange(n, dtype=np.int32)).to(dev)
        nu = torch.tensor([n], dtype=torch.int32, device=dev)
        for l in range(L):
            got = st.staple_assemble_rows(cache, blocks[l], code, nu)
            torch.cuda.synchronize()
            want = tables[l][torch.from_numpy(ids.astype(np.int64))]
            assert torch.equal(got.cpu().view(torch.int16), want.view(torch.int16)), \
                f"call {call} layer {l}: rows differ"
        _no_device_error(st)
    with pytest.raises(st.StapleError):
        bad = np.array([1, v], dtype=np.int32)
        st.staple_stage_misses_dma(srcs, torch.from_numpy(bad), 2, staging, blocks)
