"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Integer outputs (dedup, inverse map, cache slots, miss lists, gathered rows)
must match bit for bit.  Floating-point outputs must be within relative L2
error 5e-3 and max-abs error 3e-2 of the oracle (bf16 inputs, fp32
accumulation; the oracle runs in float64 with bf16 rounding at the points
where the bf16 path stores bf16, and exactly for the fp32 workload).
"""
import sys

import numpy as np
import pytest

import staple_synth as S
from oracle import staple_oracle as O
from tests.helpers import (assert_close, assert_close_floor, assert_close_stored_bf16, errors,
                           to_dev, to_np)

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


# ---------------------------------------------------------------- dedup
DEDUP_CASES = [
    ("empty", 0, 10, None),
    ("one", 1, 10, None),
    ("decode64", 64, 100352, None),
    ("pow2_512", 512, 4096, None),
    ("tile_edge", 4096, 100352, None),
    ("tile_edge_plus1", 4097, 100352, None),
    ("ragged", 9999, 50, None),
    ("train32k", 32768, 100352, None),
    ("all_equal", 5000, 100352, "equal"),
    ("all_distinct", 6000, 100352, "distinct"),
    # radix-sort paths: one-wave (1-bit passes), one workgroup (LDS), and the
    # multi-workgroup passes with several 4096-pair steps per workgroup
    ("wave_ragged", 37, 100352, None),
    ("small_65", 65, 100352, None),
    ("vocab1", 700, 1, "zero"),
    ("wave_31bit", 64, 2**31 - 1, "wide"),
    ("group_31bit", 3000, 2**31 - 1, "wide"),
    ("multi_31bit", 20000, 2**31 - 1, "wide"),
    ("multi_step", 300_000, 100352, None),
]


@pytest.mark.parametrize("name,n,vocab,kind", DEDUP_CASES, ids=[c[0] for c in DEDUP_CASES])
def test_dedup_bit_exact(st, dev, name, n, vocab, kind):
    import torch
    _log(f"dedup case {name} n={n} vocab={vocab}")
    if kind == "equal":
        ids = np.full(n, 77, dtype=np.int32)
    elif kind == "zero":
        ids = np.zeros(n, dtype=np.int32)
    elif kind == "wide":   # IDs over 31 bits, a third of them repeated
        rng = np.random.default_rng(n)
        base = rng.integers(0, vocab, n, dtype=np.int64).astype(np.int32)
        ids = np.where(rng.random(n) < 0.33, base[rng.integers(0, max(n // 8, 1), n)], base)
    elif kind == "distinct":
        ids = np.random.default_rng(3).permutation(vocab)[:n].astype(np.int32)
    else:
        ids = S.zipf_ids(n, vocab, 500 + n)
    out = st.staple_dedup(torch.from_numpy(ids).to(dev), vocab)
    torch.cuda.synchronize()
    _no_device_error(st)
    uniq, inv, sp, ss = O.dedup(ids)
    u = len(uniq)
    assert int(out["n_unique"].item()) == u
    np.testing.assert_array_equal(to_np(out["uniq"])[:u], uniq)
    np.testing.assert_array_equal(to_np(out["inv"])[:n], inv)
    np.testing.assert_array_equal(to_np(out["sorted_pos"])[:n], sp)
    np.testing.assert_array_equal(to_np(out["seg_start"])[: u + 1], ss)


def test_dedup_flags_out_of_range_ids(st, dev):
    import torch
    ids = torch.tensor([3, 10, 2], dtype=torch.int32, device=dev)
    st.staple_dedup(ids, 10)
    assert st.staple_get_device_error() == -5
    _no_device_error(st)  # the word was cleared


# ---------------------------------------------------------------- cache
@pytest.mark.parametrize("vocab,capacity,n_cal", [(4096, 205, 50_000), (100352, 5018, 1 << 20),
                                                  (1000, 0, 5000), (1000, 1000, 5000),
                                                  (300_000, 15000, 1 << 20), (1, 1, 10)])
def test_cache_count_build_lookup_bit_exact(st, dev, vocab, capacity, n_cal):
    import torch
    _log(f"cache vocab={vocab} capacity={capacity}")
    cal = S.zipf_ids(n_cal, vocab, 8)
    counts = st.staple_cache_count(torch.from_numpy(cal).to(dev), vocab)
    ref_counts = np.bincount(cal, minlength=vocab)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref_counts)
    id_to_slot, slot_to_id = st.staple_cache_build(counts, capacity)
    torch.cuda.synchronize()
    _no_device_error(st)
    o_i2s, o_s2i = O.cache_build(ref_counts, capacity)
    np.testing.assert_array_equal(to_np(id_to_slot), o_i2s)
    if capacity:
        np.testing.assert_array_equal(to_np(slot_to_id)[:capacity], o_s2i)

    for n in (64, 32768):
        ids = S.zipf_ids(n, vocab, 900 + n)
        dd = st.staple_dedup(torch.from_numpy(ids).to(dev), vocab)
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], id_to_slot)
        torch.cuda.synchronize()
        _no_device_error(st)
        uniq, _, _, _ = O.dedup(ids)
        code, miss = O.cache_lookup(uniq, o_i2s)
        u, m = len(uniq), len(miss)
        assert int(lk["n_miss"].item()) == m
        np.testing.assert_array_equal(to_np(lk["code"])[:u], code)
        np.testing.assert_array_equal(to_np(lk["miss_uidx"])[:m], miss)
        np.testing.assert_array_equal(to_np(lk["miss_ids"])[:m], uniq[miss])


def test_compact_rows_hit_and_miss_paths_are_bit_identical(st, dev):
    """R = E[uniq] bitwise, whether rows come from the HBM cache, from pinned
    host staging, from a kernel reading the pinned host table, or from a
    device-resident table; capacity 0, 5% and full."""
    import torch
    vocab, f, n = 3000, 256, 2048
    table_bits = S.normal_bf16_bits((vocab, f), 0.02, 77)
    host_table = torch.from_numpy(table_bits.view(np.int16)).view(torch.bfloat16).pin_memory()
    dev_table = host_table.to(dev)
    ids = S.zipf_ids(n, vocab, 31)
    dd = st.staple_dedup(torch.from_numpy(ids).to(dev), vocab)
    uniq, _, _, _ = O.dedup(ids)
    u = len(uniq)
    expect = table_bits[uniq]
    direct = st.staple_gather_rows(dev_table, dd["uniq"], dd["n_unique"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(direct[:u].cpu().view(torch.int16).numpy().view(np.uint16), expect)
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(40_000, vocab, 8)).to(dev), vocab)
    for capacity in (0, 150, vocab):
        i2s, s2i = st.staple_cache_build(counts, capacity)
        cache_rows = st.staple_cache_fill(host_table, s2i, capacity)   # reads pinned host memory
        lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], i2s)
        torch.cuda.synchronize()
        m = int(lk["n_miss"].item())
        miss_ids = lk["miss_ids"][:m].cpu().contiguous()
        staging = torch.empty(max(m, 1), f, dtype=torch.bfloat16).pin_memory()
        miss_rows = torch.empty(max(m, 1), f, dtype=torch.bfloat16, device=dev)
        side = torch.cuda.Stream()
        st.staple_stage_misses(host_table, miss_ids, m, staging, miss_rows, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        rows = st.staple_assemble_rows(cache_rows, miss_rows, lk["code"], dd["n_unique"])
        # misses read by a kernel straight from the pinned host table, either
        # gathered first or read inside the assembly; and from the device table
        direct_miss = st.staple_gather_rows(host_table, lk["miss_ids"], lk["n_miss"])
        rows2 = st.staple_assemble_rows(cache_rows, direct_miss, lk["code"], dd["n_unique"])
        rows3 = st.staple_assemble_rows_from_table(cache_rows, host_table, dd["uniq"], lk["code"],
                                                   dd["n_unique"], capacity=capacity)
        rows4 = st.staple_assemble_rows_from_table(cache_rows, dev_table, dd["uniq"], lk["code"],
                                                   dd["n_unique"], capacity=capacity)
        torch.cuda.synchronize()
        _no_device_error(st)
        for name, r in (("staged", rows), ("gathered from host", rows2),
                        ("assembled from host table", rows3), ("assembled from device table", rows4)):
            got = r[:u].cpu().view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(got, expect, err_msg=f"capacity {capacity}, {name}")


@pytest.mark.parametrize("f", [8192, 9000])
def test_wide_row_copies_from_host_and_device(st, dev, f):
    """Rows of 16 KB and more (the copy loop's four-deep unrolled part plus a
    remainder) gathered and assembled from a pinned host table (a capped,
    grid-striding launch) and from a device table, bit for bit."""
    import torch
    vocab, n = 700, 300
    bits = S.normal_bf16_bits((vocab, f), 0.02, 5 + f)
    host_table = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).pin_memory()
    dev_table = host_table.to(dev)
    rng = np.random.default_rng(f)
    index = rng.integers(0, vocab, size=n).astype(np.int32)
    idx = torch.from_numpy(index).to(dev)
    cnt = torch.tensor([n - 7], dtype=torch.int32, device=dev)
    a = st.staple_gather_rows(host_table, idx, cnt)
    b = st.staple_gather_rows(dev_table, idx, cnt)
    code = torch.from_numpy(np.where(np.arange(n) % 3 == 0, np.arange(n) % 50, -1).astype(np.int32)).to(dev)
    cache_rows = dev_table[:50].contiguous()
    c = st.staple_assemble_rows_from_table(cache_rows, host_table, idx, code, cnt)
    torch.cuda.synchronize()
    _no_device_error(st)
    m = n - 7
    want = bits[index[:m]]
    for name, r in (("host gather", a), ("device gather", b)):
        np.testing.assert_array_equal(r[:m].cpu().view(torch.int16).numpy().view(np.uint16), want,
                                      err_msg=name)
    cpu_code = code.cpu().numpy()[:m]
    want_c = np.where((cpu_code >= 0)[:, None], bits[np.maximum(cpu_code, 0)], want)
    np.testing.assert_array_equal(c[:m].cpu().view(torch.int16).numpy().view(np.uint16), want_c)


def test_row_copies_refuse_pageable_host_memory(st, dev):
    """A pageable host buffer handed to a row copy (source or destination) is
    refused on the host with STAPLE_ERR_INVALID_ARGUMENT; nothing is launched."""
    import torch
    f = 256
    src = torch.zeros(8, f, dtype=torch.bfloat16, device=dev)
    idx = torch.arange(4, dtype=torch.int32, device=dev)
    pageable = torch.zeros(4, f, dtype=torch.bfloat16)
    lib = st.lib()
    rc = lib.staple_gather_rows(src.data_ptr(), 8, idx.data_ptr(), None, 4, f, 1,
                                pageable.data_ptr(), None)
    assert rc == -1
    rc = lib.staple_gather_rows(pageable.data_ptr(), 4, idx.data_ptr(), None, 4, f, 1,
                                src.data_ptr(), None)
    assert rc == -1
    slot_to_id = torch.arange(4, dtype=torch.int32, device=dev)
    rc = lib.staple_cache_fill(pageable.data_ptr(), 4, f, 1, slot_to_id.data_ptr(), 4,
                               src.data_ptr(), None)
    assert rc == -1
    torch.cuda.synchronize()
    _no_device_error(st)


# ---------------------------------------------------- cache-split gate/up
@pytest.mark.parametrize("n,d,f,dtype,capacity", [
    (1000, 256, 512, "bf16", 0), (1000, 256, 512, "bf16", 120), (1000, 256, 512, "bf16", 2000),
    (64, 256, 512, "bf16", 60), (20, 128, 256, "bf16", 2000), (37, 128, 256, "bf16", 0),
    (300, 128, 256, "f32", 90), (48, 64, 11008, "bf16", 300)])
def test_split_gate_up_matches_whole_batch_bitwise(st, dev, n, d, f, dtype, capacity):
    """The cached tokens' gate/up (rows from the cache slots) and the missed
    tokens' gate/up (rows from the staged misses) together give the bits of
    one gate/up over the whole batch with the assembled rows E[uniq]; the
    split lists are the oracle's dedup and cache probe, token by token."""
    import torch
    vocab = 2000
    _log(f"split gate/up n={n} d={d} f={f} {dtype} capacity={capacity}")
    inp = S.host_layer_inputs(n, d, f, vocab, dtype=dtype, seed=60 + n + capacity)
    x, wg, wu, tab = (to_dev(getattr(inp, k), dtype, dev) for k in ("x", "w_gate", "w_up", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    dd = st.staple_dedup(ids, vocab)
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 8)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, capacity)
    cache_rows = st.staple_cache_fill(tab, s2i, capacity)
    lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], i2s)
    sp = st.staple_split_tokens(dd["inv"], lk["code"], dd["n_unique"])
    torch.cuda.synchronize()
    m = int(lk["n_miss"].item())
    miss_rows = st.staple_gather_rows(tab, lk["miss_ids"], lk["n_miss"])
    # oracle's view of the split
    uniq, inv, _, _ = O.dedup(inp.ids)
    i2s_np = i2s.cpu().numpy()
    code, _ = O.cache_lookup(uniq, i2s_np)
    tcode = np.asarray(code)[np.asarray(inv)]
    hit_pos = np.nonzero(tcode >= 0)[0]
    miss_pos = np.nonzero(tcode < 0)[0]
    n_hit, n_miss = (int(v) for v in sp["counts"].cpu().numpy())
    assert (n_hit, n_miss) == (len(hit_pos), len(miss_pos))
    np.testing.assert_array_equal(sp["hit_pos"][:n_hit].cpu().numpy(), hit_pos)
    np.testing.assert_array_equal(sp["miss_pos"][:n_miss].cpu().numpy(), miss_pos)
    np.testing.assert_array_equal(sp["tok_row"][:n].cpu().numpy(),
                                  np.where(tcode >= 0, tcode, -1 - tcode))
    # whole batch with the assembled rows
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rows = st.staple_gather_rows(tab, dd["uniq"], dd["n_unique"])
    ref = {k: torch.empty(n, f, dtype=tdt, device=dev) for k in ("h", "g", "u")}
    st.staple_ffn_gate_up(x, wg, wu, rows, dd["inv"], ref["h"], ref["g"], ref["u"])
    # split: cached tokens first, then the misses
    got = {k: torch.full((n, f), float("nan"), dtype=tdt, device=dev) for k in ("h", "g", "u")}
    crow = cache_rows if capacity > 0 else torch.zeros(1, f, dtype=tdt, device=dev)
    st.staple_ffn_gate_up_tokens(sp["hit_pos"], n_hit, x, wg, wu, crow, sp["tok_row"], got["h"],
                                 got["g"], got["u"])
    st.staple_ffn_gate_up_tokens(sp["miss_pos"], n_miss, x, wg, wu, miss_rows, sp["tok_row"],
                                 got["h"], got["g"], got["u"])
    torch.cuda.synchronize()
    _no_device_error(st)
    for k in ("h", "g", "u"):
        assert torch.equal(got[k], ref[k]), f"{k} differs"


def test_gate_up_tokens_out_of_range_position_is_flagged(st, dev):
    """A token position outside the batch sets the device error word and
    writes nothing (host-side range is not checked for device lists)."""
    import torch
    n, d, f, vocab = 100, 128, 256, 50
    inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=5)
    x, wg, wu, tab = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    for n_sel in (3, 80):     # decode kernel, tiled GEMM
        pos = torch.tensor([0, n + 5, 2] + list(range(3, n_sel)), dtype=torch.int32, device=dev)[:n_sel]
        h = torch.zeros(n, f, dtype=torch.bfloat16, device=dev)
        st.staple_ffn_gate_up_tokens(pos, n_sel, x, wg, wu, tab, ids, h)
        torch.cuda.synchronize()
        assert st.staple_get_device_error() != 0      # reading it also clears it
        assert torch.count_nonzero(h[n_sel:]) == 0 and torch.count_nonzero(h[1]) == 0


@pytest.mark.parametrize("stem", [False, True])
@pytest.mark.parametrize("n_sel", [5, 80, 300])     # decode kernel, 128 and 256 GEMM tiles
def test_bad_table_row_index_is_flagged_and_reads_as_zero(st, dev, n_sel, stem):
    """A row index outside the rows block (past the end, or negative) sets the
    device error word and that token's table row counts as zeros: h, g, u equal
    bit for bit those of the same call with the token pointed at a zero row."""
    import torch
    d, vocab = 128, 50
    f = 8192 if n_sel == 300 else 256
    _log(f"bad row index n={n_sel} stem={stem}")
    inp = S.host_layer_inputs(n_sel, d, f, vocab, dtype="bf16", seed=11, table_std=0.5)
    x, wg, wu, tab = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "table"))
    wu = None if stem else wu
    ids = torch.from_numpy(inp.ids).to(dev)
    bad = ids.clone()
    bad[1], bad[2] = vocab + 7, -3
    zero_rows = torch.cat([tab, torch.zeros(1, f, dtype=torch.bfloat16, device=dev)])
    to_zero = ids.clone()
    to_zero[1], to_zero[2] = vocab, vocab

    def run(rows, index):
        o = {k: torch.zeros(n_sel, f, dtype=torch.bfloat16, device=dev) for k in ("h", "g", "u")}
        st.staple_ffn_gate_up(x, wg, wu, rows, index, o["h"], o["g"], o["u"])
        torch.cuda.synchronize()
        return o

    got = run(tab, bad)
    assert st.staple_get_device_error() != 0      # reading it also clears it
    ref = run(zero_rows, to_zero)
    _no_device_error(st)
    for k in ("h", "g", "u"):
        assert torch.equal(got[k], ref[k]), k


# ---------------------------------------------------------------- FFN helpers
def _run_layer(st, dev, inp, out_f32=True, freeze_up=False, backward=True, full_table=False):
    import torch
    dt = inp.dtype
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x, wg, wu, wd, tab, dy = (to_dev(getattr(inp, k), dt, dev)
                              for k in ("x", "w_gate", "w_up", "w_down", "table", "dy"))
    ids = torch.from_numpy(inp.ids).to(dev)
    vocab = tab.shape[0]
    dd = st.staple_dedup(ids, vocab)
    if full_table:
        rows, index = tab, ids
    else:
        rows = st.staple_gather_rows(tab, dd["uniq"], dd["n_unique"])
        index = dd["inv"]
    fwd = st.staple_ffn_fwd(x, wg, wu, wd, rows, index,
                            out_dtype=torch.float32 if out_f32 else tdt, save=backward)
    res = {"fwd": fwd, "dd": dd}
    if backward:
        out = None
        if freeze_up:
            n, f = inp.ids.shape[0], wg.shape[0]
            d = x.shape[1]
            out = {
                "d_rows": torch.empty(max(n, 1), f, dtype=torch.float32, device=dev),
                "dx": torch.empty(n, d, dtype=torch.float32 if out_f32 else tdt, device=dev),
                "dw_gate": torch.empty(f, d, dtype=torch.float32, device=dev),
                "dw_up": torch.full((f, d), float("nan"), dtype=torch.float32, device=dev),
                "dw_down": torch.empty(d, f, dtype=torch.float32, device=dev),
            }
        res["bwd"] = st.staple_ffn_bwd_table_grad(
            dy, x, wg, wu, wd, fwd["g"], fwd["u"], fwd["h"], dd["sorted_pos"], dd["seg_start"],
            dd["n_unique"], inv=dd["inv"], freeze_up=freeze_up,
            out_dtype=torch.float32 if out_f32 else tdt,
            out=out)
    torch.cuda.synchronize()
    _no_device_error(st)
    return res


def _oracle_layer(inp, precision, freeze_up=False):
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table", "dy")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], inp.ids,
                       precision=precision)
    uniq, _, _, _ = O.dedup(inp.ids)
    ob = O.ffn_backward(g["dy"], g["x"], g["w_gate"], g["w_up"], g["w_down"], of, inp.ids,
                        precision=precision, freeze_up=freeze_up, uniq=uniq)
    return of, ob, len(uniq)


def _compare_layer(res, of, ob, u, name, freeze_up=False):
    assert_close(to_np(res["fwd"]["y"]), of["y"], f"{name} y")
    b = res["bwd"]
    assert_close(to_np(b["dx"]), ob["dx"], f"{name} dx")
    assert_close(to_np(b["d_rows"])[:u], ob["d_rows"], f"{name} d_rows")
    assert_close(to_np(b["dw_gate"]), ob["dw_gate"], f"{name} dw_gate")
    assert_close(to_np(b["dw_down"]), ob["dw_down"], f"{name} dw_down")
    if freeze_up:
        assert np.all(np.isnan(to_np(b["dw_up"]))), "dw_up was written while frozen"
    else:
        assert_close(to_np(b["dw_up"]), ob["dw_up"], f"{name} dw_up")


# ---------------------------------------------------------------- FFN parity
def test_tiny_fp32_layer_matches_oracle(st, dev):
    """fp32 end to end: d_model 256, d_ff 1024, vocab 4096, 512 Zipf tokens."""
    w = S.TINY_F32
    _log("tiny fp32 layer")
    inp = S.host_layer_inputs(w.n_tokens, w.d_model, w.d_ff, w.vocab, dtype="f32", seed=0)
    res = _run_layer(st, dev, inp)
    of, ob, u = _oracle_layer(inp, O.EXACT)
    _compare_layer(res, of, ob, u, "tiny_f32")
    # the table's contribution on its own (it is ~2% of y, so check it separately)
    inp0 = S.host_layer_inputs(w.n_tokens, w.d_model, w.d_ff, w.vocab, dtype="f32", seed=0,
                               zero_table=True)
    res0 = _run_layer(st, dev, inp0)
    of0, ob0, _ = _oracle_layer(inp0, O.EXACT)
    _compare_layer(res0, of0, ob0, u, "tiny_f32_zero_table")
    assert_close(to_np(res["fwd"]["y"]) - to_np(res0["fwd"]["y"]), of["y"] - of0["y"], "delta_y")


@pytest.mark.parametrize("n,d,f,v,seed", [(300, 256, 512, 1000, 1), (1, 64, 128, 10, 2),
                                          (129, 192, 320, 50, 3), (700, 128, 256, 4, 4)])
def test_bf16_layer_matches_oracle(st, dev, n, d, f, v, seed):
    _log(f"bf16 layer n={n} d={d} f={f} v={v}")
    inp = S.host_layer_inputs(n, d, f, v, dtype="bf16", seed=seed)
    res = _run_layer(st, dev, inp)
    of, ob, u = _oracle_layer(inp, O.BF16)
    _compare_layer(res, of, ob, u, f"bf16 n={n}")


@pytest.mark.parametrize("n,d,f,seed", [(4096, 2048, 256, 5), (2600, 1984, 512, 6),
                                        (2048, 2048, 256, 7), (4608, 2048, 128, 8)])
def test_plain_gemm_tile_shapes_match_oracle(st, dev, n, d, f, seed):
    """Token counts at which the down projection and dx (plain stores of two
    K-major operands) change tile shape on a 256-CU device: 256 x 256 tiles
    that would fill at most half of the compute units give way to 256 x 128
    tiles (4096 x 2048, and 2600 x 1984 with ragged tails in both
    dimensions); with fewer tiles still, 128 x 128 (2048 x 2048); with more,
    256 x 256 (4608 x 2048).  y and dx on every token against the oracle,
    every element written (NaN-poisoned first)."""
    import torch
    _log(f"plain GEMM tile shapes n={n} d={d} f={f}")
    inp = S.host_layer_inputs(n, d, f, 3000, dtype="bf16", seed=seed)
    x, wg, wu, wd, tab, dy = (to_dev(getattr(inp, k), "bf16", dev)
                              for k in ("x", "w_gate", "w_up", "w_down", "table", "dy"))
    ids = torch.from_numpy(inp.ids).to(dev)
    dd = st.staple_dedup(ids, tab.shape[0])
    rows = st.staple_gather_rows(tab, dd["uniq"], dd["n_unique"])
    bf = torch.bfloat16
    fwd = st.staple_ffn_fwd(x, wg, wu, wd, rows, dd["inv"],
                            out={"y": _nan((n, d), torch.float32, dev), "g": _nan((n, f), bf, dev),
                                 "u": _nan((n, f), bf, dev), "h": _nan((n, f), bf, dev)})
    bwd = st.staple_ffn_bwd_table_grad(dy, x, wg, wu, wd, fwd["g"], fwd["u"], fwd["h"],
                                       dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                       inv=dd["inv"], out_dtype=torch.float32,
                                       out={"d_rows": torch.empty(n, f, dtype=torch.float32, device=dev),
                                            "dx": _nan((n, d), torch.float32, dev),
                                            "dw_gate": torch.empty(f, d, dtype=torch.float32, device=dev),
                                            "dw_up": torch.empty(f, d, dtype=torch.float32, device=dev),
                                            "dw_down": torch.empty(d, f, dtype=torch.float32, device=dev)})
    torch.cuda.synchronize()
    _no_device_error(st)
    for k, t in (("y", fwd["y"]), ("dx", bwd["dx"])):
        assert not bool(torch.isnan(t).any()), f"{k} has unwritten elements"
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table", "dy")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], inp.ids,
                       precision=O.BF16)
    ob = O.ffn_backward(g["dy"], g["x"], g["w_gate"], g["w_up"], g["w_down"], of, inp.ids,
                        precision=O.BF16, with_dw=False)
    assert_close(to_np(fwd["y"]), of["y"], f"n={n} y")
    assert_close(to_np(bwd["dx"]), ob["dx"], f"n={n} dx")


@pytest.mark.parametrize("n", [1, 17, 33, 63, 64, 65])
def test_decode_path_boundary(st, dev, n):
    """Batches of at most 64 bf16 tokens take the decode kernels, 65 the tiled
    GEMMs; both give the oracle's y, h and the saved g, u."""
    import torch
    _log(f"decode boundary n={n}")
    d, f, v = 256, 512, 300
    inp = S.host_layer_inputs(n, d, f, v, dtype="bf16", seed=20 + n)
    x, wg, wu, wd, tab = (to_dev(getattr(inp, k), "bf16", dev)
                          for k in ("x", "w_gate", "w_up", "w_down", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    fwd = st.staple_ffn_fwd(x, wg, wu, wd, tab, ids, out_dtype=torch.float32, save=True)
    torch.cuda.synchronize()
    _no_device_error(st)
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], inp.ids,
                       precision=O.BF16)
    assert_close(to_np(fwd["y"]), of["y"], f"y n={n}")
    assert_close(to_np(fwd["h"]), of["h"], f"h n={n}")
    assert_close(to_np(fwd["g"]), of["g_saved"], f"g n={n}")
    assert_close(to_np(fwd["u"]), of["u_saved"], f"u n={n}")
    # the split halves give the same bits as the fused call
    h2 = torch.empty_like(fwd["h"])
    st.staple_ffn_gate_up(x, wg, wu, tab, ids, h2)
    y2 = torch.empty_like(fwd["y"])
    st.staple_ffn_down(h2, wd, y2)
    torch.cuda.synchronize()
    assert torch.equal(h2, fwd["h"]) and torch.equal(y2, fwd["y"])


def _packed_expected(a, b, rows_per_block_from_a):
    """The documented packed order: steps of 64 columns, row blocks of 16 rows
    (8 of a then 8 of b, or 16 of a), two 32-column halves, 64 lanes = (q, r)
    with lane q * 16 + r holding columns 8 q .. 8 q + 8 of the half, row r."""
    k = a.shape[1]
    if rows_per_block_from_a == 8:
        m = np.concatenate([a.reshape(-1, 8, k), b.reshape(-1, 8, k)], axis=1)
    else:
        m = a.reshape(-1, 16, k)
    rb = m.shape[0]
    m = m.reshape(rb, 16, k // 64, 2, 4, 8)          # (b, r, s, j, q, e)
    return m.transpose(2, 0, 3, 4, 1, 5).reshape(-1)  # (s, b, j, q, r, e)


@pytest.mark.parametrize("d,f", [(64, 64), (192, 320), (256, 512)])
def test_decode_pack_is_the_documented_permutation(st, dev, d, f):
    """Packing moves bytes only: every bf16 bit pattern lands where the
    documented layout says (compared as raw 16-bit words)."""
    import torch
    _log(f"decode pack d={d} f={f}")
    rng = np.random.default_rng(d + f)
    raw = {k: rng.integers(-32768, 32768, size=sh, dtype=np.int16)
           for k, sh in (("wg", (f, d)), ("wu", (f, d)), ("wd", (d, f)))}
    t = {k: torch.from_numpy(v).to(dev).view(torch.bfloat16) for k, v in raw.items()}
    pgu, pd = st.staple_decode_pack_weights(t["wg"], t["wu"], t["wd"], d_model=d, d_ff=f)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pgu.view(torch.int16).cpu().numpy(),
                                  _packed_expected(raw["wg"], raw["wu"], 8))
    np.testing.assert_array_equal(pd.view(torch.int16).cpu().numpy(),
                                  _packed_expected(raw["wd"], None, 16))


@pytest.mark.parametrize("n,d,f", [(1, 256, 512), (17, 192, 320), (64, 256, 512), (33, 64, 64),
                                   (64, 128, 11008), (17, 64, 11008)])
def test_ffn_fwd_packed_matches_oracle_and_row_major_bitwise(st, dev, n, d, f):
    """The decode forward on packed weights gives the oracle's y, h, g, u and
    the same bits as staple_ffn_fwd on the row-major weights.  d_ff 11008 has
    more 8-feature groups than four per CU, so gate/up runs six groups per
    workgroup with a partly empty last workgroup."""
    import torch
    _log(f"packed decode n={n} d={d} f={f}")
    inp = S.host_layer_inputs(n, d, f, 300, dtype="bf16", seed=40 + n)
    x, wg, wu, wd, tab = (to_dev(getattr(inp, k), "bf16", dev)
                          for k in ("x", "w_gate", "w_up", "w_down", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    pgu, pd = st.staple_decode_pack_weights(wg, wu, wd, d_model=d, d_ff=f)
    ref = st.staple_ffn_fwd(x, wg, wu, wd, tab, ids, out_dtype=torch.float32, save=True)
    got = st.staple_ffn_fwd_packed(x, pgu, pd, tab, ids, d_ff=f, out_dtype=torch.float32, save=True)
    got16 = st.staple_ffn_fwd_packed(x, pgu, pd, tab, ids, d_ff=f)
    ref16 = st.staple_ffn_fwd(x, wg, wu, wd, tab, ids)
    torch.cuda.synchronize()
    _no_device_error(st)
    for k in ("y", "h", "g", "u"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(got16["y"], ref16["y"])
    # the two halves give the same bits as the fused call
    h2 = torch.empty_like(got["h"])
    st.staple_ffn_gate_up_packed(x, pgu, tab, ids, h2)
    y2 = torch.empty_like(got["y"])
    st.staple_ffn_down_packed(h2, pd, y2)
    torch.cuda.synchronize()
    assert torch.equal(h2, got["h"]) and torch.equal(y2, got["y"])
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], inp.ids,
                       precision=O.BF16)
    assert_close(to_np(got["y"]), of["y"], f"packed y n={n}")
    assert_close(to_np(got["h"]), of["h"], f"packed h n={n}")
    assert_close(to_np(got["u"]), of["u_saved"], f"packed u n={n}")


def test_ffn_fwd_packed_refuses_what_it_does_not_cover(st, dev):
    """More than 64 tokens or fp32 is refused; an empty batch is a no-op."""
    import torch
    d, f = 64, 64
    wg = torch.zeros(f, d, dtype=torch.bfloat16, device=dev)
    pgu, pd = st.staple_decode_pack_weights(wg, wg, wg.t().contiguous(), d_model=d, d_ff=f)
    tab = torch.zeros(4, f, dtype=torch.bfloat16, device=dev)
    for n in (65, 128):
        x = torch.zeros(n, d, dtype=torch.bfloat16, device=dev)
        ids = torch.zeros(n, dtype=torch.int32, device=dev)
        with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported"):
            st.staple_ffn_fwd_packed(x, pgu, pd, tab, ids, d_ff=f)
    x0 = torch.zeros(0, d, dtype=torch.bfloat16, device=dev)
    out = st.staple_ffn_fwd_packed(x0, pgu, pd, tab, torch.zeros(0, dtype=torch.int32, device=dev),
                                   d_ff=f)
    assert out["y"].shape == (0, d)
    with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported"):
        st.staple_decode_pack_weights(wg.float(), wg.float(), wg.float(), d_model=d, d_ff=f)


def test_bf16_table_contribution_and_large_table_values(st, dev):
    """Rows with E ~ N(0,1) dominate u, so wrong rows cannot hide in tolerance."""
    _log("bf16 strong table")
    inp = S.host_layer_inputs(400, 128, 256, 300, dtype="bf16", seed=5, table_std=1.0)
    res = _run_layer(st, dev, inp)
    of, ob, u = _oracle_layer(inp, O.BF16)
    _compare_layer(res, of, ob, u, "bf16 strong table")


def test_zero_table_equals_dense_path_bitwise(st, dev):
    """E = 0 reproduces the dense SwiGLU: the GPU y with a zero table equals
    the GPU y with the table rows replaced by zeros through a full table."""
    import torch
    inp = S.host_layer_inputs(256, 128, 256, 64, dtype="bf16", seed=6, zero_table=True)
    a = _run_layer(st, dev, inp, backward=False)
    b = _run_layer(st, dev, inp, backward=False, full_table=True)
    assert torch.equal(a["fwd"]["y"], b["fwd"]["y"])
    of, _, _ = _oracle_layer(inp, O.BF16)
    assert_close(to_np(a["fwd"]["y"]), of["y"], "zero-table y")


def test_freeze_up_leaves_dw_up_untouched_and_rest_identical(st, dev):
    import torch
    inp = S.host_layer_inputs(333, 128, 192, 40, dtype="bf16", seed=7)
    a = _run_layer(st, dev, inp)
    b = _run_layer(st, dev, inp, freeze_up=True)
    assert np.all(np.isnan(to_np(b["bwd"]["dw_up"])))
    u = int(a["dd"]["n_unique"].item())
    assert torch.equal(a["bwd"]["d_rows"][:u], b["bwd"]["d_rows"][:u])
    for k in ("dx", "dw_gate", "dw_down"):
        assert torch.equal(a["bwd"][k], b["bwd"][k]), k
    of, ob, u = _oracle_layer(inp, O.BF16, freeze_up=True)
    _compare_layer(b, of, ob, u, "frozen", freeze_up=True)


@pytest.mark.parametrize("dtype,n,d,f", [("bf16", 300, 256, 512), ("f32", 200, 128, 256)])
def test_backward_without_saved_h_recomputes_it(st, dev, dtype, n, d, f):
    """saved_h NULL: h is formed again from the saved g and u for dW_down; every
    other output has the bits of the call with the forward's h, and dW_down
    matches the oracle's backward with the recomputed h."""
    import torch
    _log(f"recomputed h {dtype} n={n}")
    inp = S.host_layer_inputs(n, d, f, 90, dtype=dtype, seed=9)
    res = _run_layer(st, dev, inp)
    x, wg, wu, wd, dy = (to_dev(getattr(inp, k), dtype, dev)
                         for k in ("x", "w_gate", "w_up", "w_down", "dy"))
    fwd, dd = res["fwd"], res["dd"]
    b = st.staple_ffn_bwd_table_grad(dy, x, wg, wu, wd, fwd["g"], fwd["u"], None,
                                     dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                     inv=dd["inv"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    _no_device_error(st)
    u = int(dd["n_unique"].item())
    assert torch.equal(b["d_rows"][:u], res["bwd"]["d_rows"][:u])
    for k in ("dx", "dw_gate", "dw_up"):
        assert torch.equal(b[k], res["bwd"][k]), k
    prec = O.BF16 if dtype == "bf16" else O.EXACT
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table", "dy")}
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], g["table"], inp.ids,
                       precision=prec)
    ob = O.ffn_backward(g["dy"], g["x"], g["w_gate"], g["w_up"], g["w_down"], of, inp.ids,
                        precision=prec, recompute_h=True)
    assert_close(to_np(b["dw_down"]), ob["dw_down"], f"recomputed-h dw_down {dtype}")


def test_bf16_outputs_stored_in_bf16(st, dev):
    inp = S.host_layer_inputs(256, 128, 256, 100, dtype="bf16", seed=8)
    res = _run_layer(st, dev, inp, out_f32=False)
    of, ob, u = _oracle_layer(inp, O.BF16)
    assert_close(to_np(res["fwd"]["y"]), of["y"], "y bf16 store")
    assert_close(to_np(res["bwd"]["dx"]), ob["dx"], "dx bf16 store")


def test_empty_batch(st, dev):
    import torch
    d, f = 64, 128
    z = torch.zeros(0, d, dtype=torch.bfloat16, device=dev)
    w = torch.randn(f, d, device=dev).to(torch.bfloat16)
    wd = torch.randn(d, f, device=dev).to(torch.bfloat16)
    tab = torch.randn(10, f, device=dev).to(torch.bfloat16)
    ids = torch.zeros(0, dtype=torch.int32, device=dev)
    dd = st.staple_dedup(ids, 10)
    fwd = st.staple_ffn_fwd(z, w, w, wd, tab, ids, save=True)
    for k in ("g", "u", "h"):
        assert fwd[k].shape == (0, f)
    b = st.staple_ffn_bwd_table_grad(z, z, w, w, wd, fwd["g"], fwd["u"], fwd["h"],
                                     dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                     inv=dd["inv"])
    torch.cuda.synchronize()
    assert int(dd["n_unique"].item()) == 0
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert torch.all(b[k] == 0), k


# ---------------------------------------------------------------- full-size, sampled
class RowSubset:
    """A [vocab x f] table that stores only some rows (fetched from the device)."""

    def __init__(self, ids_sorted, rows):
        self.ids = np.asarray(ids_sorted)
        self.rows = rows

    def __getitem__(self, key):
        if isinstance(key, tuple):
            r, c = key
            return self.rows[np.searchsorted(self.ids, np.asarray(r).reshape(-1))][:, np.asarray(c).reshape(-1)] \
                .reshape(np.asarray(r).shape[0], -1)
        return self.rows[np.searchsorted(self.ids, np.asarray(key))]


def _device_inputs(dev, w, n_tokens, seed_base=0):
    import torch
    from staple_synth import device_normal
    d, f, v = w.d_model, w.d_ff, w.vocab
    ids = S.zipf_ids(n_tokens, v, w.ids_seed + seed_base)
    t = {
        "x": device_normal((n_tokens, d), 1.0, 2000 + seed_base, torch.bfloat16, dev),
        "w_gate": device_normal((f, d), 0.02, 3000 + seed_base, torch.bfloat16, dev),
        "w_up": device_normal((f, d), 0.02, 3001 + seed_base, torch.bfloat16, dev),
        "w_down": device_normal((d, f), 0.02, 3002 + seed_base, torch.bfloat16, dev),
        "table": device_normal((v, f), 0.02, 4000 + seed_base, torch.bfloat16, dev),
        "dy": device_normal((n_tokens, d), 1.0, 5000 + seed_base, torch.bfloat16, dev),
    }
    return ids, t


def _tile_samples(total, block, rng):
    """One index in every block of `block` consecutive indices, plus the
    first and the last index: every tile of that size holds a sample."""
    starts = np.arange(0, total, block)
    idx = np.minimum(starts + rng.integers(0, block, size=len(starts)), total - 1)
    return np.unique(np.concatenate([[0, total - 1], idx]))


def _nan(shape, dtype, dev):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device=dev)


def _train_shape_check(st, dev, w, ids, t, rows_s, cols_s, label):
    """One full-size training batch: forward and backward on the GPU with
    every output NaN-poisoned first; returns the GPU and oracle y on the
    sampled tokens.  Integer outputs are compared in full, y, h, g, u and dx
    on the sampled tokens (every feature), d_rows and the weight gradients on
    the sampled features (every token), the sums over the whole batch against
    a bound measured from the oracle's float32 evaluation."""
    import torch
    n, d, f = w.n_tokens, w.d_model, w.d_ff
    bf = torch.bfloat16
    idt = torch.from_numpy(ids).to(dev)
    dd = st.staple_dedup(idt, w.vocab)
    rows = st.staple_gather_rows(t["table"], dd["uniq"], dd["n_unique"])
    fout = {"y": _nan((n, d), torch.float32, dev), "g": _nan((n, f), bf, dev),
            "u": _nan((n, f), bf, dev), "h": _nan((n, f), bf, dev)}
    fwd = st.staple_ffn_fwd(t["x"], t["w_gate"], t["w_up"], t["w_down"], rows, dd["inv"],
                            out=fout)
    bout = {"d_rows": _nan((n, f), torch.float32, dev), "dx": _nan((n, d), torch.float32, dev),
            "dw_gate": _nan((f, d), torch.float32, dev), "dw_up": _nan((f, d), torch.float32, dev),
            "dw_down": _nan((d, f), torch.float32, dev)}
    bwd = st.staple_ffn_bwd_table_grad(t["dy"], t["x"], t["w_gate"], t["w_up"], t["w_down"],
                                       fwd["g"], fwd["u"], fwd["h"], dd["sorted_pos"],
                                       dd["seg_start"], dd["n_unique"], inv=dd["inv"], out=bout)
    torch.cuda.synchronize()
    _no_device_error(st)
    uniq, inv, sp, ss = O.dedup(ids)
    u = len(uniq)
    assert int(dd["n_unique"].item()) == u
    np.testing.assert_array_equal(to_np(dd["uniq"])[:u], uniq)
    np.testing.assert_array_equal(to_np(dd["inv"]), inv)
    np.testing.assert_array_equal(to_np(dd["sorted_pos"]), sp)
    np.testing.assert_array_equal(to_np(dd["seg_start"])[: u + 1], ss)
    # no output element is left unwritten
    for k, v in fwd.items():
        assert not bool(torch.isnan(v).any()), f"{label}: {k} has unwritten elements"
    assert not bool(torch.isnan(bwd["d_rows"][:u]).any()), f"{label}: d_rows has unwritten rows"
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert not bool(torch.isnan(bwd[k]).any()), f"{label}: {k} has unwritten elements"
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    table = RowSubset(uniq, f64(t["table"][torch.from_numpy(uniq.astype(np.int64)).to(dev)]))
    x, wg, wu, wdn, dy = (f64(t[k]) for k in ("x", "w_gate", "w_up", "w_down", "dy"))
    rs = torch.from_numpy(rows_s).to(dev)
    # forward and dx on sampled tokens (all features)
    of_r = O.ffn_forward(x[rows_s], wg, wu, wdn, table, ids[rows_s], precision=O.BF16)
    y_gpu = f64(fwd["y"][rs])
    assert_close(y_gpu, of_r["y"], f"{label} y[rows]")
    assert_close_stored_bf16(f64(fwd["h"][rs]), of_r["h"], f"{label} h[rows]")
    assert_close_stored_bf16(f64(fwd["g"][rs]), of_r["g_saved"], f"{label} g[rows]")
    assert_close_stored_bf16(f64(fwd["u"][rs]), of_r["u_saved"], f"{label} u[rows]")
    ob_r = O.ffn_backward(dy[rows_s], x[rows_s], wg, wu, wdn, of_r, ids[rows_s], precision=O.BF16,
                          with_dw=False)
    assert_close(f64(bwd["dx"][rs]), ob_r["dx"], f"{label} dx[rows]")
    # table-row and weight gradients on sampled features (all tokens), with the
    # float32 evaluation giving the floor
    ob = {}
    for acc in ("f64", "f32"):
        of_c = O.ffn_forward(x, wg, wu, wdn, table, ids, precision=O.BF16, cols=cols_s, accum=acc)
        ob[acc] = O.ffn_backward(dy, x, wg, wu, wdn, of_c, ids, precision=O.BF16, cols=cols_s,
                                 uniq=uniq, accum=acc)
    cs = torch.from_numpy(cols_s).to(dev)
    got = {"d_rows": f64(bwd["d_rows"][:u][:, cs]), "dw_gate": f64(bwd["dw_gate"][cs]),
           "dw_up": f64(bwd["dw_up"][cs]), "dw_down": f64(bwd["dw_down"][:, cs])}
    for k, v in got.items():
        assert_close_floor(v, ob["f64"][k], ob["f32"][k], f"{label} {k}[cols]")
    return y_gpu, of_r["y"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wname", ["olmo1b", "olmo7b"])
def test_olmo_train_shape_sampled(st, dev, wname):
    """The training batch at full size, bf16 (1B: 32768 Zipf tokens, d_model
    2048, d_ff 8192; 7B: 16384 tokens, 4096, 11008; vocab 100352).  The
    sampled tokens hold one token of every 256 (an M-tile of the GEMMs), the
    sampled features one of every 128 (an N-tile of the gate/up GEMM, whose
    256 columns interleave 128 gate and 128 up features), so every tile of
    every GEMM has checked outputs.  The 1B batch runs a second time with an
    all-zero table (the dense layer the zero-initialised table starts from),
    and the table's own contribution y(E) - y(0) is compared on its own."""
    w = {"olmo1b": S.OLMO1B_TRAIN, "olmo7b": S.OLMO7B_TRAIN}[wname]
    n, f = w.n_tokens, w.d_ff
    _log(f"{wname} train-shape sampled parity")
    ids, t = _device_inputs(dev, w, n)
    rng = np.random.default_rng(0)
    rows_s = _tile_samples(n, 256, rng)
    cols_s = _tile_samples(f, 128, rng)
    y_e, ref_e = _train_shape_check(st, dev, w, ids, t, rows_s, cols_s, wname)
    if wname == "olmo1b":
        _log(f"{wname} train-shape sampled parity, zero table")
        t["table"].zero_()
        y_0, ref_0 = _train_shape_check(st, dev, w, ids, t, rows_s, cols_s, wname + " E=0")
        assert_close(y_e - y_0, ref_e - ref_0, f"{wname} y(E) - y(0)[rows]")


@pytest.mark.timeout(600)
def test_olmo1b_hot_row_gradients_on_every_feature(st, dev):
    """The table-row gradients of the ten most frequent IDs of the 32768-token
    batch (the hottest sums ~4400 positions), on all 8192 features, against
    the oracle's sum of the unrounded dL/du over each ID's positions."""
    import torch
    w = S.OLMO1B_TRAIN
    n, f = w.n_tokens, w.d_ff
    _log("olmo1b hot-row gradients")
    ids, t = _device_inputs(dev, w, n)
    idt = torch.from_numpy(ids).to(dev)
    dd = st.staple_dedup(idt, w.vocab)
    rows = st.staple_gather_rows(t["table"], dd["uniq"], dd["n_unique"])
    fwd = st.staple_ffn_fwd(t["x"], t["w_gate"], t["w_up"], t["w_down"], rows, dd["inv"], save=True)
    bwd = st.staple_ffn_bwd_table_grad(t["dy"], t["x"], t["w_gate"], t["w_up"], t["w_down"],
                                       fwd["g"], fwd["u"], fwd["h"], dd["sorted_pos"],
                                       dd["seg_start"], dd["n_unique"], inv=dd["inv"],
                                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    _no_device_error(st)
    uniq, counts = np.unique(ids, return_counts=True)
    order = np.argsort(-counts, kind="stable")[:10]
    top = uniq[order]
    _log(f"  counts of the ten IDs: {counts[order].tolist()}")
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    wg, wu, wdn = (f64(t[k]) for k in ("w_gate", "w_up", "w_down"))
    ref, alt = [], []
    for tok in top:
        pos = np.flatnonzero(ids == tok)
        pt = torch.from_numpy(pos).to(dev)
        x_p, dy_p = f64(t["x"][pt]), f64(t["dy"][pt])
        table = RowSubset(np.array([tok]), f64(t["table"][int(tok):int(tok) + 1]))
        for acc, dst in (("f64", ref), ("f32", alt)):
            fw = O.ffn_forward(x_p, wg, wu, wdn, table, ids[pos], precision=O.BF16, with_y=False,
                               accum=acc)
            bw = O.ffn_backward(dy_p, x_p, wg, wu, wdn, fw, ids[pos], precision=O.BF16,
                                uniq=[int(tok)], with_dx=False, with_dw=False, accum=acc)
            dst.append(bw["d_rows"][0])
    uidx = torch.from_numpy(np.searchsorted(uniq, top)).to(dev)
    got = f64(bwd["d_rows"][uidx])
    assert_close_floor(got, np.stack(ref), np.stack(alt), "hot-row d_rows (10 IDs x 8192)")


@pytest.mark.parametrize("wname", ["olmo1b", "olmo7b"])
def test_olmo_decode_layer_full(st, dev, wname):
    """Decode batch of 64 over a full 100352 x d_ff table in HBM (1B: d_model
    2048, d_ff 8192; 7B: 4096, 11008), rows gathered by token ID inside the
    fused epilogue; every output compared, and the packed serving layout gives
    the same bits."""
    import torch
    w = {"olmo1b": S.OLMO1B_DECODE, "olmo7b": S.OLMO7B_DECODE}[wname]
    _log(f"{wname} decode layer")
    ids, t = _device_inputs(dev, w, w.n_tokens)
    idt = torch.from_numpy(ids).to(dev)
    fwd = st.staple_ffn_fwd(t["x"], t["w_gate"], t["w_up"], t["w_down"], t["table"], idt,
                            out={"y": _nan((w.n_tokens, w.d_model), torch.float32, dev)})
    torch.cuda.synchronize()
    _no_device_error(st)
    assert not bool(torch.isnan(fwd["y"]).any())
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    uniq = np.unique(ids)
    table = RowSubset(uniq, f64(t["table"][torch.from_numpy(uniq.astype(np.int64)).to(dev)]))
    of = O.ffn_forward(f64(t["x"]), f64(t["w_gate"]), f64(t["w_up"]), f64(t["w_down"]), table,
                       ids, precision=O.BF16)
    assert_close(f64(fwd["y"]), of["y"], "decode y")
    # the packed weights (the serving layout) give the same bits
    pgu, pd = st.staple_decode_pack_weights(t["w_gate"], t["w_up"], t["w_down"], d_model=w.d_model,
                                            d_ff=w.d_ff)
    got = st.staple_ffn_fwd_packed(t["x"], pgu, pd, t["table"], idt, d_ff=w.d_ff,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    _no_device_error(st)
    assert torch.equal(got["y"], fwd["y"])


# ---------------------------------------------------------------- AdamW on table rows
def _bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("dtype,f", [("bf16", 8192), ("f32", 64), ("bf16", 11008)])
def test_device_adamw_rows_match_oracle(st, dev, dtype, f):
    """Three lazy steps of the device update (rows from staple_dedup's uniq,
    count from its device scalar) against the oracle's AdamW, with the oracle
    rounded to bf16 where the table stores bf16; untouched rows bit-identical."""
    import torch
    _log(f"device adamw {dtype} f={f}")
    rng = np.random.default_rng(21 + f)
    vocab = 300
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    table = torch.tensor(rng.normal(0, 0.02, (vocab, f)), dtype=tdt, device=dev)
    m = torch.zeros(vocab, f, dtype=torch.float32, device=dev)
    v = torch.zeros(vocab, f, dtype=torch.float32, device=dev)
    ref_p, ref_m, ref_v = table.double().cpu().numpy(), np.zeros((vocab, f)), np.zeros((vocab, f))
    f32 = lambda x: float(np.float32(x))
    ohp = dict(lr=f32(3e-4), weight_decay=f32(1e-4), beta1=f32(0.9), beta2=f32(0.999), eps=f32(1e-8))
    for step, n_tok in enumerate((200, 64, 500), start=1):
        ids = S.zipf_ids(n_tok, vocab, 90 + step)
        dd = st.staple_dedup(torch.from_numpy(ids).to(dev), vocab)
        torch.cuda.synchronize()
        u = int(dd["n_unique"].item())
        uniq = dd["uniq"][:u].cpu().numpy()
        grad = torch.tensor(rng.normal(0, 1.0, (n_tok, f)), dtype=torch.float32, device=dev)
        before = table.clone()
        st.staple_adamw_rows(table, m, v, dd["uniq"], grad, n_rows=dd["n_unique"], lr=3e-4,
                             weight_decay=1e-4, step=step)
        torch.cuda.synchronize()
        _no_device_error(st)
        ref_p, ref_m, ref_v = O.adamw_rows(ref_p, ref_m, ref_v, uniq,
                                           grad[:u].double().cpu().numpy(), step=step, **ohp)
        if dtype == "bf16":
            ref_p = O.bf16_round(ref_p)
        other = torch.from_numpy(np.setdiff1d(np.arange(vocab), uniq)).to(dev)
        assert torch.equal(table[other], before[other]), "untouched rows changed"
        got = table.double().cpu().numpy()
        if dtype == "f32":
            np.testing.assert_allclose(got, ref_p, rtol=2e-6, atol=1e-9)
        else:
            bad = np.abs(got - ref_p) > _bf16_ulp(ref_p) * 1.01
            assert not bad.any(), f"{bad.sum()} parameters beyond one bf16 ulp"
            # a one-ulp rounding flip must not carry into the next step's check
            ref_p = got.copy()
        np.testing.assert_allclose(m.double().cpu().numpy(), ref_m, rtol=2e-6, atol=2e-7)
        np.testing.assert_allclose(v.double().cpu().numpy(), ref_v, rtol=2e-6, atol=1e-8)


def test_device_adamw_flags_rows_outside_the_table(st, dev):
    import torch
    table = torch.zeros(16, 64, dtype=torch.bfloat16, device=dev)
    m = torch.zeros(16, 64, device=dev)
    v = torch.zeros(16, 64, device=dev)
    rows = torch.tensor([3, 16, 5], dtype=torch.int32, device=dev)
    grad = torch.ones(3, 64, device=dev)
    st.staple_adamw_rows(table, m, v, rows, grad, lr=1e-2, weight_decay=0.0, step=1)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() != 0
    assert m[3].abs().sum() > 0 and m[5].abs().sum() > 0
    assert torch.count_nonzero(m[torch.tensor([0, 1, 2, 4, 6, 15], device=dev)]) == 0


def test_cache_refresh_after_host_update(st, dev):
    """Host AdamW on a pinned table, then the cached copies of the updated rows
    are refreshed: every cache slot equals its table row again, bit for bit,
    and slots of rows not in the batch are untouched."""
    import torch
    vocab, f, cap = 3000, 256, 150
    bits = S.normal_bf16_bits((vocab, f), 0.02, 55)
    host = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).pin_memory()
    m = torch.zeros(vocab, f)
    v = torch.zeros(vocab, f)
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(40_000, vocab, 8)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    cache_rows = st.staple_cache_fill(host, s2i, cap)
    ids = S.zipf_ids(1024, vocab, 56)
    dd = st.staple_dedup(torch.from_numpy(ids).to(dev), vocab)
    lk = st.staple_cache_lookup(dd["uniq"], dd["n_unique"], i2s)
    torch.cuda.synchronize()
    u = int(dd["n_unique"].item())
    grad = torch.randn(u, f, generator=torch.Generator().manual_seed(3))
    st.staple_adamw_rows_host(host, m, v, dd["uniq"][:u].cpu().contiguous(), grad, lr=1e-2,
                              weight_decay=0.0, step=1)
    stale = cache_rows.clone()
    st.staple_cache_refresh(host, dd["uniq"], lk["code"], dd["n_unique"], cache_rows)
    torch.cuda.synchronize()
    _no_device_error(st)
    slot_ids = s2i.cpu().numpy()
    want = host[torch.from_numpy(slot_ids.astype(np.int64))].to(dev)
    assert torch.equal(cache_rows, want)
    touched = np.isin(slot_ids, dd["uniq"][:u].cpu().numpy())
    assert touched.any() and (~touched).any()
    keep = torch.from_numpy(np.nonzero(~touched)[0]).to(dev)
    assert torch.equal(cache_rows[keep], stale[keep])


# ---------------------------------------------------------------- STEM layer (w_up None)
def _run_stem(st, dev, inp, out_f32=True):
    import torch
    dt = inp.dtype
    x, wg, wd, tab, dy = (to_dev(getattr(inp, k), dt, dev)
                          for k in ("x", "w_gate", "w_down", "table", "dy"))
    ids = torch.from_numpy(inp.ids).to(dev)
    dd = st.staple_dedup(ids, tab.shape[0])
    rows = st.staple_gather_rows(tab, dd["uniq"], dd["n_unique"])
    odt = torch.float32 if out_f32 else x.dtype
    fwd = st.staple_ffn_fwd(x, wg, None, wd, rows, dd["inv"], out_dtype=odt, save=True)
    n, d = x.shape
    f = wg.shape[0]
    out = {
        "d_rows": torch.empty(max(n, 1), f, dtype=torch.float32, device=dev),
        "dx": torch.empty(n, d, dtype=odt, device=dev),
        "dw_gate": torch.empty(f, d, dtype=torch.float32, device=dev),
        "dw_up": torch.full((f, d), float("nan"), dtype=torch.float32, device=dev),
        "dw_down": torch.empty(d, f, dtype=torch.float32, device=dev),
    }
    bwd = st.staple_ffn_bwd_table_grad(dy, x, wg, None, wd, fwd["g"], fwd["u"], fwd["h"],
                                       dd["sorted_pos"], dd["seg_start"], dd["n_unique"],
                                       inv=dd["inv"], out_dtype=odt, out=out)
    torch.cuda.synchronize()
    _no_device_error(st)
    return fwd, bwd


@pytest.mark.parametrize("dtype,n,d,f,v,seed", [
    ("f32", 300, 256, 512, 1000, 60),     # tiled GEMMs, exact fp32 oracle
    ("bf16", 300, 256, 512, 1000, 61),    # tiled GEMMs
    ("bf16", 129, 192, 320, 50, 62),      # ragged tiles, repeated tokens
    ("bf16", 17, 256, 512, 300, 63),      # decode gate kernel (row-major weights)
    ("bf16", 64, 64, 64, 10, 64),         # decode, one row group per workgroup pair
    ("bf16", 1, 64, 128, 10, 65),
])
def test_stem_layer_matches_oracle(st, dev, dtype, n, d, f, v, seed):
    """The STEM layer (no up-projection, u = E[t]): forward y, h, g, u and the
    backward dx, d_rows, dw_gate, dw_down against the oracle with w_up None;
    dw_up is not written."""
    _log(f"stem layer {dtype} n={n} d={d} f={f}")
    inp = S.host_layer_inputs(n, d, f, v, dtype=dtype, seed=seed, table_std=1.0)
    fwd, bwd = _run_stem(st, dev, inp)
    prec = O.EXACT if dtype == "f32" else O.BF16
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_down", "table", "dy")}
    of = O.ffn_forward(g["x"], g["w_gate"], None, g["w_down"], g["table"], inp.ids, precision=prec)
    uniq, _, _, _ = O.dedup(inp.ids)
    ob = O.ffn_backward(g["dy"], g["x"], g["w_gate"], None, g["w_down"], of, inp.ids,
                        precision=prec, uniq=uniq)
    name = f"stem {dtype} n={n}"
    assert_close(to_np(fwd["y"]), of["y"], f"{name} y")
    assert_close(to_np(fwd["h"]), of["h"], f"{name} h")
    assert_close(to_np(fwd["g"]), of["g_saved"], f"{name} g")
    np.testing.assert_array_equal(to_np(fwd["u"]), of["u_saved"])   # u is the table row itself
    assert_close(to_np(bwd["dx"]), ob["dx"], f"{name} dx")
    assert_close(to_np(bwd["d_rows"])[:len(uniq)], ob["d_rows"], f"{name} d_rows")
    assert_close(to_np(bwd["dw_gate"]), ob["dw_gate"], f"{name} dw_gate")
    assert_close(to_np(bwd["dw_down"]), ob["dw_down"], f"{name} dw_down")
    assert "dw_up" not in ob
    assert np.all(np.isnan(to_np(bwd["dw_up"]))), "dw_up was written for the STEM layer"


@pytest.mark.parametrize("n", [40, 300])
def test_stem_split_gate_matches_whole_batch_bitwise(st, dev, n):
    """The gate-only kernels over two token subsets (the cached / staged-miss
    split) give the whole batch's h, g, u bit for bit (40 tokens: decode
    kernel; 300: tiled GEMM)."""
    import torch
    _log(f"stem split n={n}")
    d, f = 128, 320
    inp = S.host_layer_inputs(n, d, f, 200, dtype="bf16", seed=70 + n, table_std=1.0)
    x, wg, tab = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    out = {k: torch.zeros(n, f, dtype=torch.bfloat16, device=dev) for k in ("h", "g", "u")}
    st.staple_ffn_gate_up(x, wg, None, tab, ids, out["h"], out["g"], out["u"])
    perm = torch.from_numpy(np.random.default_rng(n).permutation(n).astype(np.int32)).to(dev)
    k = n // 3
    part = {kk: torch.zeros(n, f, dtype=torch.bfloat16, device=dev) for kk in ("h", "g", "u")}
    for sel in (perm[:k], perm[k:]):
        st.staple_ffn_gate_up_tokens(sel, sel.numel(), x, wg, None, tab, ids, part["h"],
                                     part["g"], part["u"])
    torch.cuda.synchronize()
    _no_device_error(st)
    for kk in ("h", "g", "u"):
        assert torch.equal(part[kk], out[kk]), kk


@pytest.mark.parametrize("d,f", [(64, 64), (192, 320)])
def test_stem_decode_pack_is_the_documented_permutation(st, dev, d, f):
    """Packing without w_up writes W_gate alone in 16-row blocks."""
    import torch
    rng = np.random.default_rng(d * f)
    raw = rng.integers(-32768, 32768, size=(f, d), dtype=np.int16)
    wg = torch.from_numpy(raw).to(dev).view(torch.bfloat16)
    pgu, pd = st.staple_decode_pack_weights(wg, None, None, d_model=d, d_ff=f)
    torch.cuda.synchronize()
    assert pd is None and pgu.numel() == f * d
    np.testing.assert_array_equal(pgu.view(torch.int16).cpu().numpy(), _packed_expected(raw, None, 16))


@pytest.mark.parametrize("n,d,f", [(17, 256, 512), (64, 64, 64), (1, 64, 8192), (64, 64, 11008),
                                   (33, 64, 16384), (17, 64, 16448)])
def test_stem_packed_matches_oracle_and_row_major_bitwise(st, dev, n, d, f):
    """The STEM decode forward on gate-only packed weights gives the same bits
    as the row-major call and the oracle's y, h.  The d_ff values cover every
    workgroup shape: 2 row groups per workgroup (64, 8192), 3 (11008), 4
    (16384) and 6 with a partly empty last workgroup (16448)."""
    import torch
    _log(f"stem packed n={n} d={d} f={f}")
    inp = S.host_layer_inputs(n, d, f, 300, dtype="bf16", seed=80 + n, table_std=1.0)
    x, wg, wd, tab = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_down", "table"))
    ids = torch.from_numpy(inp.ids).to(dev)
    pgu, pd = st.staple_decode_pack_weights(wg, None, wd, d_model=d, d_ff=f)
    ref = st.staple_ffn_fwd(x, wg, None, wd, tab, ids, out_dtype=torch.float32, save=True)
    got = st.staple_ffn_fwd_packed(x, pgu, pd, tab, ids, d_ff=f, out_dtype=torch.float32, save=True)
    h2 = torch.empty_like(got["h"])
    st.staple_ffn_gate_up_packed(x, pgu, tab, ids, h2)
    torch.cuda.synchronize()
    _no_device_error(st)
    for k in ("y", "h", "g", "u"):
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(h2, got["h"])
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_down", "table")}
    of = O.ffn_forward(g["x"], g["w_gate"], None, g["w_down"], g["table"], inp.ids, precision=O.BF16)
    assert_close(to_np(got["y"]), of["y"], f"stem packed y n={n} f={f}")
    assert_close(to_np(got["h"]), of["h"], f"stem packed h n={n} f={f}")
    np.testing.assert_array_equal(to_np(got["u"]), of["u_saved"])


# ---------------------------------------------------------------- native decode step driver
@pytest.mark.parametrize("stem", [False, True])
@pytest.mark.parametrize("rows_mode", ["assembled", "direct", "mixed", "direct_nocache"])
def test_decode_step_driver_matches_per_layer_calls(st, dev, stem, rows_mode):
    """staple_decode_step_cached (dedup, cache probe, every layer's rows from
    the HBM cache or the pinned host table in one launch, the packed FFNs)
    gives each layer's y and rows bit for bit as the separate calls over
    several steps, and y matches the oracle on the full table.  Layers
    without rows (rows_mode "direct", or every other layer in "mixed") read
    each token's row in place inside the gate/up kernel, with the same y
    ("direct_nocache": no HBM cache at all, every row read from the pinned
    table, cache_rows NULL)."""
    import torch
    L, n, d, f, vocab = 3, 33, 128, 256, 500
    cap = 0 if rows_mode == "direct_nocache" else 40
    _log(f"decode step driver stem={stem} rows={rows_mode}")
    keeps_rows = [rows_mode == "assembled" or (rows_mode == "mixed" and l % 2 == 1) for l in range(L)]
    cache_refs = []
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 3)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    layers, ref = [], []
    for l in range(L):
        inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=90 + l, table_std=0.5)
        x, wg, wu, wd = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "w_down"))
        host_table = torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()
        pgu, pd = st.staple_decode_pack_weights(wg, None if stem else wu, wd, d_model=d, d_ff=f)
        cache_refs.append(st.staple_cache_fill(host_table, s2i, cap))
        layers.append({"x": x, "packed_gate_up": pgu, "packed_down": pd,
                       "cache_rows": None if cap == 0 else cache_refs[-1], "table": host_table,
                       "rows": torch.zeros(n, f, dtype=torch.bfloat16, device=dev) if keeps_rows[l] else None,
                       "y": torch.zeros(n, d, dtype=torch.float32, device=dev)})
        ref.append(inp)
    stack = st.DecodeStack(layers, d_model=d, d_ff=f, n_tokens=n)
    i32 = dict(dtype=torch.int32, device=dev)
    dd = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
          "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
          "n_unique": torch.empty(1, **i32)}
    lk = {"code": torch.empty(n, **i32), "miss_uidx": torch.empty(n, **i32),
          "n_miss": torch.empty(1, **i32)}
    ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)
    for step in range(3):
        ids_np = S.zipf_ids(n, vocab, 500 + step)
        ids = torch.from_numpy(ids_np).to(dev)
        d2 = st.staple_dedup(ids, vocab)
        l2 = st.staple_cache_lookup(d2["uniq"], d2["n_unique"], i2s)
        want = []
        for l, lay in enumerate(layers):
            r = st.staple_assemble_rows_from_table(cache_refs[l], lay["table"], d2["uniq"],
                                                   l2["code"], d2["n_unique"], capacity=cap)
            y = st.staple_ffn_fwd_packed(lay["x"], lay["packed_gate_up"], lay["packed_down"], r,
                                         d2["inv"], d_ff=f, out_dtype=torch.float32)["y"]
            want.append((r, y))
        for lay in layers:
            lay["y"].zero_()
            if lay["rows"] is not None:
                lay["rows"].zero_()
        st.staple_decode_step_cached(stack, ids, i2s, cap, dedup_out=dd, lookup_out=lk, workspace=ws)
        torch.cuda.synchronize()
        _no_device_error(st)
        u = int(d2["n_unique"].item())
        assert int(dd["n_unique"].item()) == u
        assert torch.equal(dd["inv"], d2["inv"]) and torch.equal(lk["code"][:u], l2["code"][:u])
        for l, lay in enumerate(layers):
            assert torch.equal(lay["y"], want[l][1]), (step, l)
            if lay["rows"] is not None:
                assert torch.equal(lay["rows"][:u], want[l][0][:u]), (step, l)
            g = {k: ref[l].as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table")}
            of = O.ffn_forward(g["x"], g["w_gate"], None if stem else g["w_up"], g["w_down"],
                               g["table"], ids_np, precision=O.BF16)
            assert_close(to_np(lay["y"]), of["y"], f"driver y layer {l} step {step}")


@pytest.mark.parametrize("stem,n,f,cap", [(False, 64, 256, 40), (True, 33, 256, 40),
                                          (False, 64, 256, 0), (True, 64, 16448, 40)])
def test_decode_step_driver_carried_rows_and_grouped_tables(st, dev, stem, n, f, cap):
    """The decode step with the rows of each group of layers copied by the
    gate/up launches of the group before (group 1, 2, 3, 4; seven layers, so
    the last group is partial) and with the tables interleaved token-major by
    groups of four (staple_group_tables_host: one contiguous host read per
    miss per group) gives every layer's y and compact rows bit for bit as the
    step that assembles every row first from separate tables.  cap 0: no HBM
    cache, every row from the pinned tables.  STEM at d_ff 16448: six row
    groups per workgroup, whose copy waves cannot carry a part, so those
    groups are assembled first instead."""
    import torch
    L, d, vocab = 7, 64, 300
    _log(f"carried rows stem={stem} n={n} f={f} cap={cap}")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(20_000, vocab, 3)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    base, tables, caches = [], [], []
    for l in range(L):
        inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=120 + l, table_std=0.5)
        x, wg, wu, wd = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "w_down"))
        tab = torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()
        pgu, pd = st.staple_decode_pack_weights(wg, None if stem else wu, wd, d_model=d, d_ff=f)
        tables.append(tab)
        caches.append(st.staple_cache_fill(tab, s2i, cap))
        base.append({"x": x, "packed_gate_up": pgu, "packed_down": pd,
                     "cache_rows": None if cap == 0 else caches[-1]})
    grouped = [st.staple_group_tables_host(tables[g:g + 4]) for g in range(0, L, 4)]
    torch.testing.assert_close(grouped[0][:, 2], tables[2], rtol=0, atol=0)

    def stack(layout):
        lays = []
        for l in range(L):
            gsz = min(4, L - (l // 4) * 4)
            tab = tables[l] if layout == "separate" else (grouped[l // 4], (l % 4) * f, gsz * f)
            lays.append(dict(base[l], table=tab,
                             rows=torch.zeros(n, f, dtype=torch.bfloat16, device=dev),
                             y=torch.zeros(n, d, dtype=torch.float32, device=dev)))
        return lays, st.DecodeStack(lays, d_model=d, d_ff=f, n_tokens=n)

    i32 = dict(dtype=torch.int32, device=dev)
    dd = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
          "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
          "n_unique": torch.empty(1, **i32)}
    lk = {"code": torch.empty(n, **i32), "miss_uidx": torch.empty(n, **i32),
          "n_miss": torch.empty(1, **i32)}
    ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)
    ref_lays, ref_stack = stack("separate")
    for step in range(2):
        ids = torch.from_numpy(S.zipf_ids(n, vocab, 700 + step)).to(dev)
        st.staple_decode_step_cached(ref_stack, ids, i2s, cap, dedup_out=dd, lookup_out=lk,
                                     workspace=ws, group=0)
        torch.cuda.synchronize()
        _no_device_error(st)
        u = int(dd["n_unique"].item())
        for layout in ("separate", "grouped"):
            for group in (1, 2, 3, 4):
                lays, stk = stack(layout)
                st.staple_decode_step_cached(stk, ids, i2s, cap, dedup_out=dd, lookup_out=lk,
                                             workspace=ws, group=group)
                torch.cuda.synchronize()
                _no_device_error(st)
                for l in range(L):
                    assert torch.equal(lays[l]["y"], ref_lays[l]["y"]), (layout, group, step, l)
                    assert torch.equal(lays[l]["rows"][:u], ref_lays[l]["rows"][:u]), \
                        (layout, group, step, l)
    # the oracle on the last step
    ids_np = S.zipf_ids(n, vocab, 701)
    uniq = np.unique(ids_np)
    for l in (0, L - 1):
        inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=120 + l, table_std=0.5)
        g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "table")}
        of = O.ffn_forward(g["x"], g["w_gate"], None if stem else g["w_up"], g["w_down"],
                           g["table"], ids_np, precision=O.BF16)
        assert_close(to_np(ref_lays[l]["y"]), of["y"], f"carried y layer {l}")


def test_decode_step_driver_refuses_carried_rows_without_compact_rows(st, dev):
    import torch
    d, f, n, vocab = 64, 64, 8, 16
    wg = torch.zeros(f, d, dtype=torch.bfloat16, device=dev)
    pgu, pd = st.staple_decode_pack_weights(wg, wg, wg.t().contiguous(), d_model=d, d_ff=f)
    tab = torch.zeros(vocab, f, dtype=torch.bfloat16, device=dev)
    lay = {"x": torch.zeros(n, d, dtype=torch.bfloat16, device=dev), "packed_gate_up": pgu,
           "packed_down": pd, "cache_rows": None, "table": tab,
           "y": torch.zeros(n, d, dtype=torch.bfloat16, device=dev)}
    stk = st.DecodeStack([lay], d_model=d, d_ff=f, n_tokens=n)
    i32 = dict(dtype=torch.int32, device=dev)
    dd = {k: torch.empty(n + 1, **i32) for k in ("uniq", "inv", "sorted_pos", "seg_start")}
    dd["n_unique"] = torch.empty(1, **i32)
    lk = {k: torch.empty(n, **i32) for k in ("code", "miss_uidx")}
    lk["n_miss"] = torch.empty(1, **i32)
    ws = torch.empty(max(st.decode_step_workspace_bytes(n, d, f), 1), dtype=torch.uint8, device=dev)
    ids = torch.zeros(n, dtype=torch.int32, device=dev)
    i2s = torch.full((vocab,), -1, dtype=torch.int32, device=dev)
    for group in (2, 5):
        with pytest.raises(RuntimeError, match="invalid argument"):
            st.staple_decode_step_cached(stk, ids, i2s, 0, dedup_out=dd, lookup_out=lk,
                                         workspace=ws, group=group)


@pytest.mark.parametrize("stem", [False, True])
def test_decode_step_driver_in_place_bad_slot_is_flagged_and_reads_as_zero(st, dev, stem):
    """With rows read in place, a cache slot past the capacity (a corrupt
    id -> slot map) sets the device error word and the token's row counts as
    zeros, as in the per-layer call on rows whose row is zero."""
    import torch
    L, n, d, f, vocab, cap = 2, 20, 128, 256, 60, 8
    _log(f"decode step driver bad slot stem={stem}")
    counts = st.staple_cache_count(torch.from_numpy(S.zipf_ids(5_000, vocab, 4)).to(dev), vocab)
    i2s, s2i = st.staple_cache_build(counts, cap)
    ids_np = S.zipf_ids(n, vocab, 77)
    ids = torch.from_numpy(ids_np).to(dev)
    corrupt = i2s.clone()
    corrupt[int(ids_np[0])] = cap + 5                 # token 0's ID maps past the cache
    layers = []
    for l in range(L):
        inp = S.host_layer_inputs(n, d, f, vocab, dtype="bf16", seed=120 + l, table_std=0.5)
        x, wg, wu, wd = (to_dev(getattr(inp, k), "bf16", dev) for k in ("x", "w_gate", "w_up", "w_down"))
        host_table = torch.from_numpy(inp.table.view(np.int16)).view(torch.bfloat16).pin_memory()
        pgu, pd = st.staple_decode_pack_weights(wg, None if stem else wu, wd, d_model=d, d_ff=f)
        layers.append({"x": x, "packed_gate_up": pgu, "packed_down": pd,
                       "cache_rows": st.staple_cache_fill(host_table, s2i, cap), "table": host_table,
                       "y": torch.zeros(n, d, dtype=torch.float32, device=dev)})
    stack = st.DecodeStack(layers, d_model=d, d_ff=f, n_tokens=n)
    i32 = dict(dtype=torch.int32, device=dev)
    dd = {"uniq": torch.empty(n, **i32), "inv": torch.empty(n, **i32),
          "sorted_pos": torch.empty(n, **i32), "seg_start": torch.empty(n + 1, **i32),
          "n_unique": torch.empty(1, **i32)}
    lk = {"code": torch.empty(n, **i32), "miss_uidx": torch.empty(n, **i32),
          "n_miss": torch.empty(1, **i32)}
    ws = torch.empty(st.decode_step_workspace_bytes(n, d, f), dtype=torch.uint8, device=dev)
    st.staple_decode_step_cached(stack, ids, corrupt, cap, dedup_out=dd, lookup_out=lk, workspace=ws)
    torch.cuda.synchronize()
    assert st.staple_get_device_error() != 0
    # reference: the rows from the correct map, with token 0's row zeroed
    d2 = st.staple_dedup(ids, vocab)
    l2 = st.staple_cache_lookup(d2["uniq"], d2["n_unique"], i2s)
    u0 = int(d2["inv"][0].item())
    for lay in layers:
        r = st.staple_assemble_rows_from_table(lay["cache_rows"], lay["table"], d2["uniq"],
                                               l2["code"], d2["n_unique"], capacity=cap)
        r[u0].zero_()
        want = st.staple_ffn_fwd_packed(lay["x"], lay["packed_gate_up"], lay["packed_down"], r,
                                        d2["inv"], d_ff=f, out_dtype=torch.float32)["y"]
        torch.cuda.synchronize()
        assert torch.equal(lay["y"], want)
    _no_device_error(st)


def test_decode_step_driver_refuses_bad_arguments(st, dev):
    """Batches past 64 tokens and a layer without a table are refused before
    anything is enqueued."""
    import ctypes
    import torch
    d, f, vocab = 64, 64, 10
    t = lambda *sh, **kw: torch.zeros(*sh, dtype=kw.get("dtype", torch.bfloat16), device=dev)
    host_table = torch.zeros(vocab, f, dtype=torch.bfloat16).pin_memory()
    # buffers for 65 tokens, so that the library's own check of the batch is reached
    lay = {"x": t(65, d), "packed_gate_up": t(2 * f * d), "packed_down": t(f * d),
           "cache_rows": t(1, f), "table": host_table, "rows": t(65, f), "y": t(65, d)}
    stack = st.DecodeStack([lay], d_model=d, d_ff=f, n_tokens=64)
    i32 = dict(dtype=torch.int32)
    dd = {k: t(66, **i32) for k in ("uniq", "inv", "sorted_pos", "seg_start", "n_unique")}
    lk = {k: t(66, **i32) for k in ("code", "miss_uidx", "n_miss")}
    ws = t(1 << 20, dtype=torch.uint8)
    i2s = torch.full((vocab,), -1, dtype=torch.int32, device=dev)
    with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported"):
        st.staple_decode_step_cached(stack, t(65, **i32), i2s, 0, dedup_out=dd, lookup_out=lk,
                                     workspace=ws)
    stack.desc[0].table = None      # a layer without its table
    with pytest.raises(RuntimeError, match="INVALID|invalid"):
        st.staple_decode_step_cached(stack, t(64, **i32), i2s, 0, dedup_out=dd, lookup_out=lk,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dd["n_unique"]) == 0 and torch.count_nonzero(lay["y"]) == 0
