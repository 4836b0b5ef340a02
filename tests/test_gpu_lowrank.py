"""GPU parity of the low-rank table layer (u = W_up x + P E_r[t], E_r of width
r, P [d_ff x r]; STAPLE Table 2, r=512 row) against the oracle, through the
C ABI: the compact rows R_r = E_r[uniq] (staple_gather_rows), Z = R_r P^T
(staple_lowrank_expand), the full-width forward and backward over Z, and the
table-row and projection gradients (staple_lowrank_bwd)."""
import sys

import numpy as np
import pytest

import staple_synth as S
from oracle import staple_oracle as O
from tests.helpers import (assert_close, assert_close_floor, assert_close_stored_bf16, to_dev,
                           to_np)

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


def _gpu_layer(st, ids, t, vocab, out_dtype):
    """Dedup, R_r, Z, forward and backward of the layer, then the low-rank
    gradients; t holds the device tensors (x, w_gate, w_up, w_down, table_r,
    proj, dy)."""
    import torch
    dd = st.staple_dedup(ids, vocab)
    rows_r = st.staple_gather_rows(t["table_r"], dd["uniq"], dd["n_unique"])
    z = st.staple_lowrank_expand(rows_r, dd["n_unique"], t["proj"])
    fwd = st.staple_ffn_fwd(t["x"], t["w_gate"], t["w_up"], t["w_down"], z, dd["inv"],
                            out_dtype=out_dtype, save=True)
    bwd = st.staple_ffn_bwd_table_grad(t["dy"], t["x"], t["w_gate"], t["w_up"], t["w_down"],
                                       fwd["g"], fwd["u"], fwd["h"], dd["sorted_pos"],
                                       dd["seg_start"], dd["n_unique"], inv=dd["inv"],
                                       out_dtype=out_dtype)
    lr = st.staple_lowrank_bwd(bwd["d_rows"], rows_r, dd["n_unique"], t["proj"])
    torch.cuda.synchronize()
    assert st.staple_get_device_error() == 0
    return dd, z, fwd, bwd, lr


@pytest.mark.parametrize("dtype,n,d,f,r,v,seed", [
    ("f32", 300, 128, 256, 64, 500, 61),
    ("bf16", 700, 256, 512, 128, 400, 62),
    ("bf16", 129, 192, 320, 192, 40, 63),
])
def test_lowrank_layer_matches_oracle(st, dtype, n, d, f, r, v, seed):
    import torch
    dev = torch.device("cuda:0")
    _log(f"low-rank layer {dtype} n={n} d={d} f={f} r={r}")
    inp = S.host_layer_inputs(n, d, f, v, dtype=dtype, seed=seed)
    draw = S.normal_bf16_bits if dtype == "bf16" else S.normal_f32
    table_r = draw((v, r), 0.05, 7000 + seed)
    proj = draw((f, r), 0.05, 7100 + seed)
    t = {k: to_dev(getattr(inp, k), dtype, dev) for k in ("x", "w_gate", "w_up", "w_down", "dy")}
    t["table_r"] = to_dev(table_r, dtype, dev)
    t["proj"] = to_dev(proj, dtype, dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    dd, z, fwd, bwd, lr = _gpu_layer(st, ids, t, v, torch.float32)
    prec = O.BF16 if dtype == "bf16" else O.EXACT
    f64 = lambda a: (S.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)
    g = {k: inp.as_f64(k) for k in ("x", "w_gate", "w_up", "w_down", "dy")}
    er, p = f64(table_r), f64(proj)
    uniq = np.unique(inp.ids)
    u = len(uniq)
    assert int(dd["n_unique"].item()) == u
    tab = O.LowRankTable(er, p, prec)
    of = O.ffn_forward(g["x"], g["w_gate"], g["w_up"], g["w_down"], tab, inp.ids, precision=prec)
    ob = O.ffn_backward(g["dy"], g["x"], g["w_gate"], g["w_up"], g["w_down"], of, inp.ids,
                        precision=prec, uniq=uniq)
    ol = O.lowrank_backward(ob["d_rows"], er, p, uniq, precision=prec)
    assert_close(to_np(z)[:u], O.lowrank_rows(er, p, uniq, prec), f"{dtype} Z")
    assert_close(to_np(fwd["y"]), of["y"], f"{dtype} y")
    assert_close(to_np(bwd["dx"]), ob["dx"], f"{dtype} dx")
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert_close(to_np(bwd[k]), ob[k], f"{dtype} {k}")
    assert_close(to_np(bwd["d_rows"])[:u], ob["d_rows"], f"{dtype} dL/dZ")
    assert_close(to_np(lr["d_rows_r"])[:u], ol["d_rows_r"], f"{dtype} d_rows_r")
    assert_close(to_np(lr["d_proj"]), ol["d_proj"], f"{dtype} d_proj")


def test_lowrank_with_no_rows_zeroes_the_projection_gradient(st):
    import torch
    dev = torch.device("cuda:0")
    r, f = 64, 128
    rows_r = torch.randn(8, r, device=dev).to(torch.bfloat16)
    proj = torch.randn(f, r, device=dev).to(torch.bfloat16)
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    d_rows = torch.randn(8, f, device=dev)
    out = {"d_rows_r": torch.full((8, r), float("nan"), device=dev),
           "d_proj": torch.full((f, r), float("nan"), device=dev)}
    st.staple_lowrank_bwd(d_rows, rows_r, zero, proj, out=out)
    z = torch.full((8, f), float("nan"), device=dev).to(torch.bfloat16)
    st.staple_lowrank_expand(rows_r, zero, proj, out=z)
    torch.cuda.synchronize()
    assert bool((out["d_proj"] == 0).all())
    assert bool(torch.isnan(out["d_rows_r"]).all()) and bool(torch.isnan(z.float()).all())


@pytest.mark.timeout(600)
def test_lowrank_olmo1b_training_shape(st):
    """32768 Zipf tokens at d_model 2048, d_ff 8192, r 512, vocab 100352: Z on
    every unique row; y, dx on one token per 256; dL/dZ and dP on one feature
    per 128 (all unique rows); the row gradients of the ten hottest IDs and
    22 others on all r columns.  Sums over the batch are bounded by 3x the
    floor measured from the oracle's float32 evaluation."""
    import torch
    from staple_synth import device_normal
    dev = torch.device("cuda:0")
    w = S.OLMO1B_TRAIN
    n, d, f, v, r = w.n_tokens, w.d_model, w.d_ff, w.vocab, 512
    _log("low-rank layer, OLMo-2-1B training shape, r=512")
    bf = torch.bfloat16
    t = {"x": device_normal((n, d), 1.0, 2000, bf, dev),
         "w_gate": device_normal((f, d), 0.02, 3000, bf, dev),
         "w_up": device_normal((f, d), 0.02, 3001, bf, dev),
         "w_down": device_normal((d, f), 0.02, 3002, bf, dev),
         "table_r": device_normal((v, r), 0.02, 4000, bf, dev),
         "proj": device_normal((f, r), 0.02, 4100, bf, dev),
         "dy": device_normal((n, d), 1.0, 5000, bf, dev)}
    ids_np = S.zipf_ids(n, v, w.ids_seed)
    ids = torch.from_numpy(ids_np).to(dev)
    dd, z, fwd, bwd, lr = _gpu_layer(st, ids, t, v, torch.float32)
    f64 = lambda a: a.float().cpu().numpy().astype(np.float64)
    uniq, counts = np.unique(ids_np, return_counts=True)
    u = len(uniq)
    assert int(dd["n_unique"].item()) == u
    rows_r = f64(t["table_r"][torch.from_numpy(uniq.astype(np.int64)).to(dev)])

    class Er:
        def __getitem__(self, key):
            return rows_r[np.searchsorted(uniq, np.asarray(key).reshape(-1))]

    er = Er()
    p = f64(t["proj"])
    # Z for every unique row
    assert_close_stored_bf16(f64(z[:u]), O.lowrank_rows(er, p, uniq, O.BF16), "Z")
    x, wg, wu, wdn, dy = (f64(t[k]) for k in ("x", "w_gate", "w_up", "w_down", "dy"))
    rng = np.random.default_rng(3)
    rows_s = np.unique(np.concatenate([[0, n - 1], np.arange(0, n, 256) + rng.integers(0, 256, n // 256)]))
    cols_s = np.unique(np.concatenate([[0, f - 1], np.arange(0, f, 128) + rng.integers(0, 128, f // 128)]))
    rs = torch.from_numpy(rows_s).to(dev)
    of_r = O.ffn_forward(x[rows_s], wg, wu, wdn, O.LowRankTable(er, p, O.BF16), ids_np[rows_s],
                         precision=O.BF16)
    assert_close(f64(fwd["y"][rs]), of_r["y"], "y[rows]")
    ob_r = O.ffn_backward(dy[rows_s], x[rows_s], wg, wu, wdn, of_r, ids_np[rows_s],
                          precision=O.BF16, with_dw=False)
    assert_close(f64(bwd["dx"][rs]), ob_r["dx"], "dx[rows]")
    # dL/dZ and dP on sampled features (every unique row), f64 and f32 evaluations
    cs = torch.from_numpy(cols_s).to(dev)
    ref = {}
    for acc in ("f64", "f32"):
        of_c = O.ffn_forward(x, wg, wu, wdn, O.LowRankTable(er, p, O.BF16, acc), ids_np,
                             precision=O.BF16, cols=cols_s, accum=acc)
        ob_c = O.ffn_backward(dy, x, wg, wu, wdn, of_c, ids_np, precision=O.BF16, cols=cols_s,
                              uniq=uniq, accum=acc, with_dw=False)
        dz = ob_c["d_rows"]
        ref[acc] = {"dz": dz,
                    "d_proj": O.lowrank_backward(dz, er, p[cols_s], uniq, O.BF16, acc)["d_proj"]}
    assert_close_floor(f64(bwd["d_rows"][:u][:, cs]), ref["f64"]["dz"], ref["f32"]["dz"], "dL/dZ[:, cols]")
    assert_close_floor(f64(lr["d_proj"][cs]), ref["f64"]["d_proj"], ref["f32"]["d_proj"], "d_proj[cols]")
    # row gradients of the hottest and some other IDs on every column of r
    order = np.argsort(-counts, kind="stable")
    pick = np.unique(np.concatenate([order[:10], rng.choice(order[10:], 22, replace=False)]))
    got = f64(lr["d_rows_r"][torch.from_numpy(pick).to(dev)])
    want = {"f64": [], "f32": []}
    for k in pick:
        tok = uniq[k]
        pos = np.flatnonzero(ids_np == tok)
        pt = torch.from_numpy(pos).to(dev)
        x_p, dy_p = f64(t["x"][pt]), f64(t["dy"][pt])
        for acc in ("f64", "f32"):
            fw = O.ffn_forward(x_p, wg, wu, wdn, O.LowRankTable(er, p, O.BF16, acc), ids_np[pos],
                               precision=O.BF16, with_y=False, accum=acc)
            bw = O.ffn_backward(dy_p, x_p, wg, wu, wdn, fw, ids_np[pos], precision=O.BF16,
                                uniq=[int(tok)], with_dx=False, with_dw=False, accum=acc)
            want[acc].append(O.lowrank_backward(bw["d_rows"], er, p, [int(tok)], O.BF16, acc)["d_rows_r"][0])
    assert_close_floor(got, np.stack(want["f64"]), np.stack(want["f32"]), "d_rows_r (32 IDs x 512)")
