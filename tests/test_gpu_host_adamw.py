"""The host AdamW update of offloaded tables overlapped with the GPU step
(staple_host_adamw_*): over three training steps it gives the host table,
its moments and the HBM cache rows bit for bit as the serial schedule (copy
the row gradients, update on the host, refresh the cache after every step),
and the rows agree with the oracle's AdamW."""
import sys

import numpy as np
import pytest

import staple_synth as S
from oracle import staple_oracle as O
from tests.helpers import to_dev

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


def _run(st, inp, ids_steps, cap, overlapped, refresh_in_worker=False, steps=3):
    import torch
    dev = torch.device("cuda:0")
    vocab, f = inp.table.shape
    n, d = inp.x.shape
    x, wg, wu, wd, dy = (to_dev(getattr(inp, k), "bf16", dev)
                         for k in ("x", "w_gate", "w_up", "w_down", "dy"))
    table = torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()
    m = torch.zeros(vocab, f, dtype=torch.float32)
    v = torch.zeros(vocab, f, dtype=torch.float32)
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(50_000, vocab, 9)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    cache = st.staple_cache_fill(table, s2i, cap)
    side = torch.cuda.Stream()
    ha = st.HostAdamW(n, f) if overlapped else None
    hp = dict(lr=1e-2, weight_decay=1e-2)
    ys = []
    grads = []
    for k in range(steps):
        ids = torch.from_numpy(ids_steps[k]).to(dev)
        dd = st.staple_dedup(ids, vocab)
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], i2s)
        if ha is not None and k > 0:
            ha.finish()                              # the previous step's rows are updated
            if not refresh_in_worker:
                st.staple_cache_refresh(table, prev["uniq"], prev["code"], prev["n_unique"], cache)
        rows = st.staple_assemble_rows_from_table(cache, table, dd["uniq"], lk["code"],
                                                  dd["n_unique"], capacity=cap)
        fwd = st.staple_ffn_fwd(x, wg, wu, wd, rows, dd["inv"], out_dtype=torch.float32, save=True)
        bwd = st.staple_ffn_bwd_table_grad(dy, x, wg, wu, wd, fwd["g"], fwd["u"], fwd["h"],
                                           dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                           inv=dd["inv"],
                                           rows_event=None if ha is None else ha.event)
        ys.append(fwd["y"])
        if ha is not None:
            extra = {"code": lk["code"], "cache_rows": cache} if refresh_in_worker else {}
            ha.start(table, m, v, dd["uniq"], dd["n_unique"], bwd["d_rows"], step=k + 1,
                     copy_stream=side, **extra, **hp)
            prev = {"uniq": dd["uniq"], "code": lk["code"], "n_unique": dd["n_unique"],
                    "d_rows": bwd["d_rows"], "keep": bwd}
        else:
            torch.cuda.synchronize()
            u = int(dd["n_unique"].item())
            g = bwd["d_rows"][:u].cpu().contiguous()
            st.staple_adamw_rows_host(table, m, v, dd["uniq"][:u].cpu().contiguous(), g,
                                      step=k + 1, **hp)
            st.staple_cache_refresh(table, dd["uniq"], lk["code"], dd["n_unique"], cache)
        grads.append((dd["uniq"][:int(dd["n_unique"].item())].cpu().numpy(),
                      bwd["d_rows"][:int(dd["n_unique"].item())].cpu().numpy()))
    if ha is not None:
        ha.finish()
        if not refresh_in_worker:
            st.staple_cache_refresh(table, prev["uniq"], prev["code"], prev["n_unique"], cache)
        ha.close()
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    return table, m, v, cache, ys, grads


@pytest.mark.parametrize("cap,in_worker", [(0, False), (60, False), (60, True), (2000, True)])
def test_overlapped_host_adamw_matches_the_serial_schedule(st, cap, in_worker):
    """cap 0: every row from the host table; 60: a few hot rows cached; 2000:
    the whole table cached.  in_worker: the handle refreshes the cached copies
    chunk by chunk, else one staple_cache_refresh after finish()."""
    import torch
    n, d, f, vocab = 700, 128, 256, 2000
    _log(f"overlapped host AdamW cap={cap} refresh_in_worker={in_worker}")
    inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=81)
    ids_steps = [S.zipf_ids(n, vocab, 900 + k) for k in range(3)]
    ser = _run(st, inp, ids_steps, cap, overlapped=False)
    ovl = _run(st, inp, ids_steps, cap, overlapped=True, refresh_in_worker=in_worker)
    for name, a, b in zip(("table", "m", "v", "cache"), ser[:4], ovl[:4]):
        if name == "cache":
            a, b = a[:cap], b[:cap]                  # capacity 0: a one-row unused buffer
        assert torch.equal(a, b), name
    for k, (a, b) in enumerate(zip(ser[4], ovl[4])):
        assert torch.equal(a, b), f"y of step {k}"
    # the rows against the oracle's AdamW over the same three gradients
    f32 = lambda z: float(np.float32(z))
    p = S.bf16_bits_to_f32(inp.table).astype(np.float64)
    mm, vv = np.zeros_like(p), np.zeros_like(p)
    for k, (uniq, g) in enumerate(ser[5]):
        p, mm, vv = O.adamw_rows(p, mm, vv, uniq, g.astype(np.float64), lr=f32(1e-2),
                                 weight_decay=f32(1e-2), step=k + 1, beta1=f32(0.9),
                                 beta2=f32(0.999), eps=f32(1e-8))
        p = O.bf16_round(p)
    got = ovl[0].float().numpy().astype(np.float64)
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(p), 1e-30))).astype(np.int64) - 7)
    assert np.mean(np.abs(got - p) <= step * 1.01) > 0.999


def test_overlapped_host_adamw_reports_an_id_outside_the_table(st):
    """A row ID past the table's end: finish() raises STAPLE_ERR_HOST, nothing
    is updated, and the same handle then runs a normal update."""
    import torch
    dev = torch.device("cuda:0")
    n, d, f, vocab = 300, 128, 256, 2000
    _log("overlapped host AdamW with an ID outside the table")
    inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=83)
    x, wg, wu, wd, dy = (to_dev(getattr(inp, k), "bf16", dev)
                         for k in ("x", "w_gate", "w_up", "w_down", "dy"))
    table = torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()
    ids = S.zipf_ids(n, vocab, 910)
    ids[0] = vocab - 1                                # above the short table's end
    ids_dev = torch.from_numpy(ids).to(dev)
    dd = st.staple_dedup(ids_dev, vocab)
    rows = st.staple_gather_rows(table, dd["uniq"], dd["n_unique"])
    fwd = st.staple_ffn_fwd(x, wg, wu, wd, rows, dd["inv"], out_dtype=torch.float32, save=True)
    ha = st.HostAdamW(n, f)
    bwd = st.staple_ffn_bwd_table_grad(dy, x, wg, wu, wd, fwd["g"], fwd["u"], fwd["h"],
                                       dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                       inv=dd["inv"], rows_event=ha.event)
    side = torch.cuda.Stream()
    short = table[: vocab // 2]                       # a pinned view of the first rows
    m = torch.zeros(vocab, f, dtype=torch.float32)
    v = torch.zeros(vocab, f, dtype=torch.float32)
    before = short.clone()
    ha.start(short, m[: vocab // 2], v[: vocab // 2], dd["uniq"], dd["n_unique"], bwd["d_rows"],
             lr=1e-2, weight_decay=1e-2, step=1, copy_stream=side)
    with pytest.raises(st.StapleError) as e:
        ha.finish()
    assert e.value.status == -6                       # STAPLE_ERR_HOST
    assert torch.equal(short, before)
    assert not m.any() and not v.any()
    # the handle is usable again: a full-size table, compared with the serial update
    bwd = st.staple_ffn_bwd_table_grad(dy, x, wg, wu, wd, fwd["g"], fwd["u"], fwd["h"],
                                       dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                       inv=dd["inv"], rows_event=ha.event)
    ref_t, ref_m, ref_v = table.clone(), m.clone(), v.clone()
    ha.start(table, m, v, dd["uniq"], dd["n_unique"], bwd["d_rows"], lr=1e-2, weight_decay=1e-2,
             step=1, copy_stream=side)
    ha.finish()
    ha.close()
    torch.cuda.synchronize()
    u = int(dd["n_unique"].item())
    st.staple_adamw_rows_host(ref_t, ref_m, ref_v, dd["uniq"][:u].cpu().contiguous(),
                              bwd["d_rows"][:u].cpu().contiguous(), step=1, lr=1e-2,
                              weight_decay=1e-2)
    assert torch.equal(table, ref_t) and torch.equal(m, ref_m) and torch.equal(v, ref_v)
    assert st.staple_get_device_error() == 0
