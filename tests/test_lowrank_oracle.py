"""Pins of the oracle's low-rank table layer (u = W_up x + P E_r[t], E_r of
width r, P [d_ff x r]): torch autograd of the same layer, finite
differences, and the closed forms P = 0 (the dense layer) and r = d_ff with
P = I (the full-width layer)."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import staple_oracle as O


def _layer(rng, n=40, d=12, f=24, r=6, v=9):
    x = rng.standard_normal((n, d))
    wg = rng.standard_normal((f, d)) * 0.3
    wu = rng.standard_normal((f, d)) * 0.3
    wd = rng.standard_normal((d, f)) * 0.3
    er = rng.standard_normal((v, r)) * 0.5
    p = rng.standard_normal((f, r)) * 0.4
    ids = rng.integers(0, v, size=n)
    dy = rng.standard_normal((n, d))
    return x, wg, wu, wd, er, p, ids, dy


def _oracle(x, wg, wu, wd, er, p, ids, dy, precision=O.EXACT):
    tab = O.LowRankTable(er, p, precision)
    uniq = np.unique(ids)
    fw = O.ffn_forward(x, wg, wu, wd, tab, ids, precision=precision)
    bw = O.ffn_backward(dy, x, wg, wu, wd, fw, ids, precision=precision, uniq=uniq)
    lr = O.lowrank_backward(bw["d_rows"], er, p, uniq, precision=precision)
    return fw, bw, lr, uniq


def test_lowrank_layer_matches_torch_autograd():
    rng = np.random.default_rng(51)
    x, wg, wu, wd, er, p, ids, dy = _layer(rng)
    fw, bw, lr, uniq = _oracle(x, wg, wu, wd, er, p, ids, dy)
    T = {k: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for k, a in (("x", x), ("wg", wg), ("wu", wu), ("wd", wd), ("er", er), ("p", p))}
    it = torch.from_numpy(ids)
    z = F.embedding(it, T["er"]) @ T["p"].T
    h = F.silu(T["x"] @ T["wg"].T) * (T["x"] @ T["wu"].T + z)
    y = h @ T["wd"].T
    y.backward(torch.from_numpy(dy))
    np.testing.assert_allclose(fw["y"], y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bw["dx"], T["x"].grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(bw["dw_up"], T["wu"].grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lr["d_rows_r"], T["er"].grad.numpy()[uniq], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lr["d_proj"], T["p"].grad.numpy(), rtol=1e-11, atol=1e-11)
    # rows of E_r whose token is absent get no gradient
    absent = np.setdiff1d(np.arange(er.shape[0]), uniq)
    assert np.all(T["er"].grad.numpy()[absent] == 0)


def test_lowrank_gradients_match_finite_differences():
    rng = np.random.default_rng(52)
    x, wg, wu, wd, er, p, ids, dy = _layer(rng, n=12, d=5, f=8, r=3, v=4)
    _, _, lr, uniq = _oracle(x, wg, wu, wd, er, p, ids, dy)
    loss = lambda er_, p_: float(np.sum(dy * O.ffn_forward(
        x, wg, wu, wd, O.LowRankTable(er_, p_), ids)["y"]))
    eps = 1e-5
    for (i, j) in [(0, 0), (3, 2), (7, 1)]:
        a, b = p.copy(), p.copy()
        a[i, j] += eps
        b[i, j] -= eps
        fd = (loss(er, a) - loss(er, b)) / (2 * eps)
        assert abs(fd - lr["d_proj"][i, j]) <= 1e-6 * max(1.0, abs(fd))
    for k, t in enumerate(uniq):
        for j in range(er.shape[1]):
            a, b = er.copy(), er.copy()
            a[t, j] += eps
            b[t, j] -= eps
            fd = (loss(a, p) - loss(b, p)) / (2 * eps)
            assert abs(fd - lr["d_rows_r"][k, j]) <= 1e-6 * max(1.0, abs(fd))


def test_zero_projection_is_the_dense_layer():
    """P = 0: Z = 0, so y, dx and the weight gradients are the dense layer's
    (a zero table) and the table rows get no gradient; P itself still does."""
    rng = np.random.default_rng(53)
    x, wg, wu, wd, er, p, ids, dy = _layer(rng)
    p0 = np.zeros_like(p)
    fw, bw, lr, uniq = _oracle(x, wg, wu, wd, er, p0, ids, dy)
    zero = np.zeros((er.shape[0], wg.shape[0]))
    fd = O.ffn_forward(x, wg, wu, wd, zero, ids)
    bd = O.ffn_backward(dy, x, wg, wu, wd, fd, ids, uniq=uniq)
    np.testing.assert_array_equal(fw["y"], fd["y"])
    for k in ("dx", "dw_gate", "dw_up", "dw_down", "d_rows"):
        np.testing.assert_array_equal(bw[k], bd[k])
    assert np.all(lr["d_rows_r"] == 0)
    np.testing.assert_allclose(lr["d_proj"], bd["d_rows"].T @ er[uniq], rtol=1e-13, atol=1e-13)


def test_full_width_identity_projection_is_the_full_width_layer():
    """r = d_ff and P = I: Z = E_r[t], the full-width STAPLE layer with table
    E_r, and the low-rank row gradient is its table-row gradient."""
    rng = np.random.default_rng(54)
    x, wg, wu, wd, _, _, ids, dy = _layer(rng)
    f = wg.shape[0]
    er = rng.standard_normal((9, f)) * 0.5
    eye = np.eye(f)
    for prec in (O.EXACT, O.BF16):
        fw, bw, lr, uniq = _oracle(x, wg, wu, wd, er, eye, ids, dy, precision=prec)
        ff = O.ffn_forward(x, wg, wu, wd, er, ids, precision=prec)
        bf = O.ffn_backward(dy, x, wg, wu, wd, ff, ids, precision=prec, uniq=uniq)
        if prec == O.EXACT:
            np.testing.assert_array_equal(fw["y"], ff["y"])
            np.testing.assert_array_equal(lr["d_rows_r"], bf["d_rows"])
        else:
            # the bf16 path rounds Z once (E_r values here are not bf16 values)
            np.testing.assert_array_equal(
                O.lowrank_rows(er, eye, ids, O.BF16), O.bf16_round(er[ids]))
            np.testing.assert_array_equal(lr["d_rows_r"], O.bf16_round(bw["d_rows"]))
