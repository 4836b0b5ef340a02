"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to an independent statement of what it must
produce: a library routine that computes the same thing (torch autograd,
numpy.unique / argsort / lexsort, torch's bfloat16 cast), finite differences,
closed forms of special cases, brute force on tiny inputs, or figures printed
on the STAPLE pages.  All CPU-only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import staple_oracle as O
import staple_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(rng, n, d, f, v, scale_w=0.3, zero_table=False):
    x = rng.standard_normal((n, d))
    wg = rng.standard_normal((f, d)) * scale_w
    wu = rng.standard_normal((f, d)) * scale_w
    wd = rng.standard_normal((d, f)) * scale_w
    e = np.zeros((v, f)) if zero_table else rng.standard_normal((v, f)) * 0.5
    ids = rng.integers(0, v, size=n)
    dy = rng.standard_normal((n, d))
    return x, wg, wu, wd, e, ids, dy


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_matches_torch_cast_on_float32():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(200_000).astype(np.float32),
            (rng.standard_normal(20_000) * 1e-39).astype(np.float32),   # fp32 subnormals
            (rng.standard_normal(20_000) * 1e37).astype(np.float32),
            np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, -3.3895314e38], dtype=np.float32)]
    # exact midpoints between neighbouring bf16 values (ties): bits xxxx8000
    bits = (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << 16) | 0x8000
    bits = bits[((bits >> 23) & 0xFF) < 0xFE]        # keep finite, below the top binade
    vals.append(bits.view(np.float32))
    v = np.concatenate(vals)
    ours = O.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_round_is_nearest_on_float64_by_brute_force():
    # every finite positive bf16 value, in order
    allbits = np.arange(0, 0x7F80, dtype=np.uint32)
    grid = (allbits << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(50_000) * 10.0 ** rng.integers(-30, 30, 50_000),
                        rng.standard_normal(1000) * 1e-40])
    a = np.abs(v)
    hi = np.searchsorted(grid, a, side="left")
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - grid[lo], grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((allbits[hi] & 1) == 0))
    expect = np.where(pick_hi, grid[hi], grid[lo]) * np.sign(v)
    expect = np.where(a == grid[hi], grid[hi] * np.sign(v), expect)
    np.testing.assert_array_equal(O.bf16_round(v), expect)


# ---------------------------------------------------------------- forward
def _torch_forward(x, wg, wu, wd, e, ids):
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    xt, wgt, wut, wdt, et = map(t, (x, wg, wu, wd, e))
    idt = torch.tensor(ids, dtype=torch.long)
    g = F.linear(xt, wgt)
    u = F.linear(xt, wut) + F.embedding(idt, et)
    h = F.silu(g) * u
    return g, u, h, F.linear(h, wdt)


@pytest.mark.parametrize("n,d,f,v", [(37, 16, 24, 11), (1, 8, 8, 1), (64, 32, 48, 5)])
def test_forward_exact_matches_torch(n, d, f, v):
    rng = np.random.default_rng(n + d)
    x, wg, wu, wd, e, ids, _ = _rand_layer(rng, n, d, f, v)
    out = O.ffn_forward(x, wg, wu, wd, e, ids)
    g, u, h, y = (a.numpy() for a in _torch_forward(x, wg, wu, wd, e, ids))
    for ours, ref in ((out["g"], g), (out["u"], u), (out["h"], h), (out["y"], y)):
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_zero_table_reduces_to_dense_swiglu():
    # Zero-initialised tables restore the seed model's computation (news synopsis
    # "Pretrained models gain sparse capacity without retraining", Interpretation).
    rng = np.random.default_rng(3)
    x, wg, wu, wd, e, ids, _ = _rand_layer(rng, 50, 16, 32, 7, zero_table=True)
    y = O.ffn_forward(x, wg, wu, wd, e, ids)["y"]
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    dense = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd)).numpy()
    np.testing.assert_allclose(y, dense, rtol=1e-13, atol=1e-13)
    # the zero row adds nothing: u equals the up-projection exactly
    np.testing.assert_array_equal(O.ffn_forward(x, wg, wu, wd, e, ids)["u"], x @ wu.T)


def test_forward_columns_and_rows_are_restrictions():
    rng = np.random.default_rng(4)
    x, wg, wu, wd, e, ids, _ = _rand_layer(rng, 40, 16, 32, 9)
    full = O.ffn_forward(x, wg, wu, wd, e, ids)
    cols = np.array([0, 5, 31, 7])
    part = O.ffn_forward(x, wg, wu, wd, e, ids, cols=cols)
    np.testing.assert_allclose(part["h"], full["h"][:, cols], rtol=1e-13, atol=1e-14)
    rows = np.array([3, 0, 39])
    sub = O.ffn_forward(x[rows], wg, wu, wd, e, ids[rows])
    np.testing.assert_allclose(sub["y"], full["y"][rows], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- backward
def _torch_grads(x, wg, wu, wd, e, ids, dy):
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    xt, wgt, wut, wdt, et = map(t, (x, wg, wu, wd, e))
    idt = torch.tensor(ids, dtype=torch.long)
    y = F.linear(F.silu(F.linear(xt, wgt)) * (F.linear(xt, wut) + F.embedding(idt, et)), wdt)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return {k: p.grad.numpy() for k, p in
            (("dx", xt), ("dw_gate", wgt), ("dw_up", wut), ("dw_down", wdt), ("de", et))}


@pytest.mark.parametrize("n,d,f,v", [(37, 16, 24, 11), (64, 8, 16, 3), (5, 4, 4, 50)])
def test_backward_exact_matches_torch_autograd(n, d, f, v):
    rng = np.random.default_rng(10 + n)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, n, d, f, v)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    uniq, _, _, _ = O.dedup(ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, uniq=uniq)
    ref = _torch_grads(x, wg, wu, wd, e, ids, dy)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        np.testing.assert_allclose(b[k], ref[k], rtol=1e-11, atol=1e-11, err_msg=k)
    np.testing.assert_allclose(b["d_rows"], ref["de"][uniq], rtol=1e-11, atol=1e-11)
    absent = np.setdiff1d(np.arange(v), uniq)
    assert np.all(ref["de"][absent] == 0)


def test_backward_matches_central_finite_differences():
    rng = np.random.default_rng(5)
    n, d, f, v = 6, 4, 5, 3
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, n, d, f, v)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    uniq, _, _, _ = O.dedup(ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, uniq=uniq)
    loss = lambda x, wg, wu, wd, e: float(np.sum(O.ffn_forward(x, wg, wu, wd, e, ids)["y"] * dy))
    params = dict(x=x, wg=wg, wu=wu, wd=wd, e=e)
    grads = dict(x=b["dx"], wg=b["dw_gate"], wu=b["dw_up"], wd=b["dw_down"])
    de = np.zeros_like(e)
    de[uniq] = b["d_rows"]
    grads["e"] = de
    eps = 1e-6
    for name in params:
        for trial in range(3):
            dirn = rng.standard_normal(params[name].shape)
            plus = dict(params); minus = dict(params)
            plus[name] = params[name] + eps * dirn
            minus[name] = params[name] - eps * dirn
            fd = (loss(**plus) - loss(**minus)) / (2 * eps)
            an = float(np.sum(grads[name] * dirn))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_silu_grad_matches_finite_difference():
    z = np.linspace(-30, 30, 2001)
    eps = 1e-6
    fd = (O.silu(z + eps) - O.silu(z - eps)) / (2 * eps)
    np.testing.assert_allclose(O.silu_grad(z), fd, rtol=1e-6, atol=1e-8)
    assert O.silu(0.0) == 0.0 and O.silu_grad(0.0) == 0.5


def test_closed_form_zero_input():
    # x = 0: g = a = 0, u = E[t], silu(0) = 0, silu'(0) = 1/2.
    rng = np.random.default_rng(6)
    _, wg, wu, wd, e, ids, dy = _rand_layer(rng, 20, 8, 12, 5)
    x = np.zeros((20, 8))
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids)
    assert np.all(fwd["y"] == 0)
    for k in ("d_rows", "dw_gate", "dw_up", "dw_down"):
        assert np.all(b[k] == 0), k
    expect_dx = np.stack([wg.T @ (0.5 * (wd.T @ dy[i]) * e[ids[i]]) for i in range(20)])
    np.testing.assert_allclose(b["dx"], expect_dx, rtol=1e-12, atol=1e-13)


def test_closed_form_zero_gate():
    rng = np.random.default_rng(7)
    x, _, wu, wd, e, ids, dy = _rand_layer(rng, 20, 8, 12, 5)
    wg = np.zeros((12, 8))
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids)
    assert np.all(fwd["y"] == 0)
    assert np.all(b["d_rows"] == 0) and np.all(b["dw_up"] == 0)
    u = x @ wu.T + e[ids]
    np.testing.assert_allclose(b["dg"], 0.5 * (dy @ wd) * u, rtol=1e-12, atol=1e-13)


def test_all_equal_ids_single_segment():
    rng = np.random.default_rng(8)
    x, wg, wu, wd, e, _, dy = _rand_layer(rng, 30, 8, 12, 5)
    ids = np.full(30, 3)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids)
    assert b["d_rows"].shape == (1, 12)
    np.testing.assert_allclose(b["d_rows"][0], b["du"].sum(axis=0), rtol=1e-13, atol=1e-14)


def test_singleton_ids_take_their_row_gradient_unchanged():
    rng = np.random.default_rng(9)
    x, wg, wu, wd, e, _, dy = _rand_layer(rng, 10, 8, 12, 40)
    ids = rng.permutation(40)[:10]
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    uniq, inv, _, _ = O.dedup(ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, uniq=uniq)
    np.testing.assert_array_equal(b["d_rows"][inv], b["du"])


def test_freeze_up_skips_only_the_up_gradient():
    # During warmup the pretrained up-projections of augmented layers are frozen
    # (STAPLE Table 3 caption); gradients still flow through them.
    rng = np.random.default_rng(11)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 25, 8, 12, 6)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    a = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, freeze_up=True)
    assert "dw_up" in a and "dw_up" not in b
    for k in ("dx", "dw_gate", "dw_down", "d_rows"):
        np.testing.assert_array_equal(a[k], b[k])


def test_backward_columns_are_restrictions():
    rng = np.random.default_rng(12)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 30, 8, 20, 6)
    full_f = O.ffn_forward(x, wg, wu, wd, e, ids, precision=O.BF16)
    full = O.ffn_backward(dy, x, wg, wu, wd, full_f, ids, precision=O.BF16)
    cols = np.array([19, 2, 7])
    pf = O.ffn_forward(x, wg, wu, wd, e, ids, precision=O.BF16, cols=cols)
    part = O.ffn_backward(dy, x, wg, wu, wd, pf, ids, precision=O.BF16, cols=cols)
    np.testing.assert_allclose(part["d_rows"], full["d_rows"][:, cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(part["dw_gate"], full["dw_gate"][cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(part["dw_up"], full["dw_up"][cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(part["dw_down"], full["dw_down"][:, cols], rtol=1e-13, atol=1e-14)


def test_bf16_mode_differs_from_exact_by_rounding_only():
    rng = np.random.default_rng(13)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 64, 16, 32, 9)
    ex = O.ffn_forward(x, wg, wu, wd, e, ids)
    bf = O.ffn_forward(x, wg, wu, wd, e, ids, precision=O.BF16)
    # h is rounded once: relative change at most 2^-8 per element
    assert np.all(np.abs(bf["h"] - ex["h"]) <= 2.0 ** -8 * np.abs(ex["h"]))
    assert np.all(O.bf16_round(bf["h"]) == bf["h"])
    assert np.all(O.bf16_round(bf["g_saved"]) == bf["g_saved"])
    assert np.all(bf["g"] == ex["g"]) and np.all(bf["u"] == ex["u"])
    b = O.ffn_backward(dy, x, wg, wu, wd, bf, ids, precision=O.BF16)
    assert np.all(O.bf16_round(b["du"]) == b["du"]) and np.all(O.bf16_round(b["dg"]) == b["dg"])
    # du, dg are computed from the saved (rounded) activations
    np.testing.assert_array_equal(b["du"], O.bf16_round(b["dh"] * O.silu(bf["g_saved"])))


def test_bf16_mode_rounding_points_on_a_scalar_layer():
    # One token, d = f = 1, values chosen so that every rounding point moves the
    # result; expected values use torch's own bfloat16 cast at the stated points.
    x, wg, wu, wd, e, dy = 1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6, 1.0 + 3 * 2 ** -7, 2 ** -9, 1.0 + 2 ** -7
    bf = lambda v: torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double().item()
    sg = 1.0 / (1.0 + math.exp(-wg * x))
    u = wu * x + e
    h = bf(wg * x * sg * u)
    y = h * wd
    fwd = O.ffn_forward([[x]], [[wg]], [[wu]], [[wd]], np.array([[e]]), [0], precision=O.BF16)
    assert fwd["h"][0, 0] == h and fwd["y"][0, 0] == y
    assert fwd["u_saved"][0, 0] == bf(u) and bf(u) != u
    dh = dy * wd
    gs, us = bf(wg * x), bf(u)
    s = 1.0 / (1.0 + math.exp(-gs))
    du = bf(dh * gs * s)
    dg = bf(dh * us * s * (1.0 + gs * (1.0 - s)))
    b = O.ffn_backward([[dy]], [[x]], [[wg]], [[wu]], [[wd]], fwd, [0], precision=O.BF16)
    assert b["du"][0, 0] == du and b["dg"][0, 0] == dg
    assert b["dw_up"][0, 0] == du * x and b["dw_gate"][0, 0] == dg * x
    assert b["dw_down"][0, 0] == dy * h
    # the table-row gradient sums dL/du before its bf16 rounding (an fp32 sum,
    # not a contraction operand): here the two differ
    du_sum = dh * gs * s
    assert bf(du_sum) != du_sum
    assert b["d_rows"][0, 0] == du_sum and b["du_sum"][0, 0] == du_sum
    # h recomputed from the saved (rounded) g and u for dW_down
    br = O.ffn_backward([[dy]], [[x]], [[wg]], [[wu]], [[wd]], fwd, [0], precision=O.BF16,
                        recompute_h=True)
    h_rec = bf(gs * s * us)
    assert br["dw_down"][0, 0] == dy * h_rec
    for k in ("du", "dg", "dw_up", "dw_gate", "d_rows", "dx"):
        assert br[k][0, 0] == b[k][0, 0], k


def test_recomputed_h_in_bf16_is_silu_of_the_saved_activations():
    rng = np.random.default_rng(33)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 64, 16, 32, 6)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids, precision=O.BF16)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, precision=O.BF16, recompute_h=True)
    g, u = fwd["g_saved"], fwd["u_saved"]
    h_rec = torch.tensor(g / (1 + np.exp(-g)) * u).to(torch.bfloat16).double().numpy()
    np.testing.assert_allclose(b["dw_down"], dy.T @ h_rec, rtol=1e-12, atol=1e-12)
    assert np.any(h_rec != fwd["h"])   # the saved activations' rounding shows


def test_recomputed_h_equals_the_forward_h_without_rounding():
    rng = np.random.default_rng(32)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 40, 8, 16, 5)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids)
    a = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, recompute_h=True)
    for k in ("dw_down", "dw_gate", "dw_up", "d_rows", "dx"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-13, atol=1e-13)


def test_bf16_table_row_gradient_sums_the_unrounded_du():
    # d_rows = sum over occurrences of dh * silu(g_saved), with no rounding of
    # the summands; a version that summed the rounded du would differ
    rng = np.random.default_rng(31)
    x, wg, wu, wd, e, _, dy = _rand_layer(rng, 200, 16, 24, 3)
    ids = rng.integers(0, 3, size=200)
    fwd = O.ffn_forward(x, wg, wu, wd, e, ids, precision=O.BF16)
    b = O.ffn_backward(dy, x, wg, wu, wd, fwd, ids, precision=O.BF16)
    dh = dy @ wd
    want = dh * O.silu(fwd["g_saved"])
    uniq = np.unique(ids)
    brute = np.stack([want[ids == t].sum(axis=0) for t in uniq])
    np.testing.assert_allclose(b["d_rows"], brute, rtol=1e-12, atol=1e-13)
    rounded = np.stack([O.bf16_round(want)[ids == t].sum(axis=0) for t in uniq])
    assert np.max(np.abs(rounded - brute)) > 1e-6


# ---------------------------------------------------------------- dedup
@pytest.mark.parametrize("n,v,seed", [(0, 10, 0), (1, 10, 1), (64, 100352, 2), (512, 4096, 3),
                                      (5000, 50, 4), (3000, 1, 5)])
def test_dedup_matches_numpy(n, v, seed):
    ids = S.zipf_ids(n, v, seed) if n else np.zeros(0, dtype=np.int32)
    uniq, inv, sorted_pos, seg_start = O.dedup(ids)
    nu, ninv = np.unique(ids, return_inverse=True)
    np.testing.assert_array_equal(uniq, nu)
    np.testing.assert_array_equal(inv, ninv.reshape(-1))
    np.testing.assert_array_equal(sorted_pos, np.argsort(ids, kind="stable"))
    sorted_ids = np.sort(ids, kind="stable")
    np.testing.assert_array_equal(seg_start, np.searchsorted(sorted_ids, np.append(nu, np.iinfo(np.int32).max)))
    assert seg_start[-1] == n


# ---------------------------------------------------------------- cache
@pytest.mark.parametrize("vocab,capacity", [(1000, 0), (1000, 50), (1000, 1000), (4096, 205)])
def test_cache_build_matches_lexsort(vocab, capacity):
    counts = S.calibration_counts(vocab, n_tokens=20_000, seed=8)
    counts[::7] = counts[1]          # force many ties
    id_to_slot, slot_to_id = O.cache_build(counts, capacity)
    order = np.lexsort((np.arange(vocab), -counts))
    np.testing.assert_array_equal(slot_to_id, order[:capacity])
    expect = np.full(vocab, -1)
    expect[order[:capacity]] = np.arange(capacity)
    np.testing.assert_array_equal(id_to_slot, expect)


def test_cache_build_fills_every_slot_when_counts_are_sparse():
    counts = np.zeros(100, dtype=np.int64)
    counts[[5, 60]] = [3, 9]
    _, slot_to_id = O.cache_build(counts, 10)
    assert list(slot_to_id) == [60, 5, 0, 1, 2, 3, 4, 6, 7, 8]


def test_cache_lookup_by_membership():
    rng = np.random.default_rng(14)
    vocab = 300
    counts = rng.integers(0, 50, vocab)
    id_to_slot, slot_to_id = O.cache_build(counts, 40)
    ids = rng.integers(0, vocab, 200)
    uniq, _, _, _ = O.dedup(ids)
    code, miss = O.cache_lookup(uniq, id_to_slot)
    cached = set(slot_to_id.tolist())
    expect_miss = [u for u, t in enumerate(uniq) if t not in cached]
    assert list(miss) == expect_miss
    for u, t in enumerate(uniq):
        if t in cached:
            assert slot_to_id[code[u]] == t
        else:
            assert miss[-1 - code[u]] == u


# ---------------------------------------------------------------- synthetic inputs
def test_zipf_stream_statistics():
    v, n = 100352, 1 << 18
    ids = S.zipf_ids(n, v, 123)
    perm = S.rank_permutation(v)
    h = np.sum(np.arange(1, v + 1, dtype=np.float64) ** -1.1)
    p1 = 1.0 / h
    share = np.mean(ids == perm[0])
    assert abs(share - p1) < 4 * math.sqrt(p1 * (1 - p1) / n)
    assert ids.min() >= 0 and ids.max() < v and ids.dtype == np.int32
    np.testing.assert_array_equal(ids, S.zipf_ids(n, v, 123))


def test_expected_unique_count_of_a_training_batch():
    v, n = 100352, 32768
    p = np.arange(1, v + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    expect_u = np.sum(1.0 - (1.0 - p) ** n)
    got = np.mean([len(np.unique(S.zipf_ids(n, v, s))) for s in range(4)])
    assert abs(got - expect_u) < 0.01 * expect_u


def test_bf16_input_encoding_is_round_to_nearest_even():
    a = S.normal_f32((1000,), 1.0, 0)
    np.testing.assert_array_equal(S.bf16_bits_to_f32(S.f32_to_bf16_bits(a)),
                                  torch.from_numpy(a).to(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------- page figures
def test_page_figures_fix_the_1b_workload_shapes():
    gold = json.load(open(os.path.join(GOLDEN, "page_closed_forms.json")))
    w = S.OLMO1B_DECODE
    sh = gold["shapes"]
    assert (w.d_model, w.d_ff, w.vocab, w.n_layers) == (sh["d_model"], sh["d_ff"], sh["vocab"],
                                                         sh["augmented_layers"])
    d, f, v, L, A = w.d_model, w.d_ff, w.vocab, sh["n_layers_model"], w.n_layers
    dense_flops = 2 * (L * (4 * d * d + 3 * d * f) + v * d)
    computed = {
        "offloaded_tables_bytes": A * v * f * 2 / 1e9,
        "host_tables_and_moments": A * v * f * (2 + 4 + 4) / 2 ** 30,
        "linear_gflops_per_token_dense": dense_flops / 1e9,
        "linear_gflops_per_token_stem": (dense_flops - 2 * A * d * f) / 1e9,
        "gpu_weights_dense": 2 * (L * (4 * d * d + 3 * d * f) + 2 * v * d) / 1e9,
        "gpu_weights_stem": 2 * (L * (4 * d * d + 3 * d * f) + 2 * v * d - A * d * f) / 1e9,
        "gpu_cache_bytes": A * S.OLMO1B_OFFLOAD.cache_capacity * f * 2 / 1e9,
        "decode_b64_tok_per_s_dense": 64 / 1.817e-3 / 1e3,
        "decode_b64_tok_per_s_staple": 64 / 1.845e-3 / 1e3,
    }
    for ent in gold["entries"]:
        got = round(computed[ent["name"]], ent["printed_decimals"])
        assert got == pytest.approx(ent["value"]), (ent["name"], computed[ent["name"]])
    assert S.OLMO1B_OFFLOAD.cache_capacity == 5018


# ---------------------------------------------------------------- AdamW on rows
def _adamw_case(seed, vocab=9, f=6, n_rows=4):
    rng = np.random.default_rng(seed)
    table = rng.normal(0, 0.5, (vocab, f))
    rows = rng.choice(vocab, n_rows, replace=False)
    grad = rng.normal(0, 1.0, (n_rows, f))
    return table, rows, grad


def test_adamw_first_step_closed_form():
    """From zero moments, step 1: m = (1-b1) g, v = (1-b2) g^2, and the bias
    corrections turn the update into lr * g / (|g| + eps) after the decay."""
    table, rows, grad = _adamw_case(0)
    lr, wd, b1, b2, eps = 3e-4, 1e-4, 0.9, 0.999, 1e-8
    p, m, v = O.adamw_rows(table, np.zeros_like(table), np.zeros_like(table), rows, grad,
                           lr=lr, weight_decay=wd, step=1, beta1=b1, beta2=b2, eps=eps)
    want_p = table.copy()
    want_p[rows] = table[rows] * (1 - lr * wd) - lr * grad / (np.abs(grad) + eps)
    np.testing.assert_allclose(p, want_p, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m[rows], (1 - b1) * grad, rtol=1e-15)
    np.testing.assert_allclose(v[rows], (1 - b2) * grad ** 2, rtol=1e-15)


def test_adamw_zero_gradient_row_only_decays():
    table, rows, grad = _adamw_case(1)
    grad[:] = 0.0
    p, m, v = O.adamw_rows(table, np.zeros_like(table), np.zeros_like(table), rows, grad,
                           lr=1e-2, weight_decay=0.5, step=1)
    np.testing.assert_array_equal(p[rows], table[rows] * (1 - 1e-2 * 0.5))
    assert not m.any() and not v.any()


def test_adamw_untouched_rows_are_bit_identical():
    table, rows, grad = _adamw_case(2)
    m0 = np.random.default_rng(3).normal(0, 0.1, table.shape)
    v0 = np.abs(np.random.default_rng(4).normal(0, 0.1, table.shape))
    p, m, v = O.adamw_rows(table, m0, v0, rows, grad, lr=1e-3, weight_decay=1e-4, step=7)
    other = np.setdiff1d(np.arange(table.shape[0]), rows)
    np.testing.assert_array_equal(p[other], table[other])
    np.testing.assert_array_equal(m[other], m0[other])
    np.testing.assert_array_equal(v[other], v0[other])


def test_adamw_all_rows_touched_matches_torch_adamw():
    """With every row in every step the update is torch.optim.AdamW's (float64)."""
    rng = np.random.default_rng(5)
    vocab, f = 7, 5
    table = rng.normal(0, 0.5, (vocab, f))
    lr, wd, b1, b2, eps = 4e-4, 1e-4, 0.9, 0.999, 1e-8
    w = torch.nn.Parameter(torch.tensor(table, dtype=torch.float64))
    opt = torch.optim.AdamW([w], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = table.copy(), np.zeros_like(table), np.zeros_like(table)
    for step in range(1, 4):
        g = rng.normal(0, 1.0, (vocab, f))
        w.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = O.adamw_rows(p, m, v, np.arange(vocab), g, lr=lr, weight_decay=wd,
                               step=step, beta1=b1, beta2=b2, eps=eps)
    np.testing.assert_allclose(p, w.detach().numpy(), rtol=1e-13, atol=1e-15)
    st = opt.state[w]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_adamw_sparse_rows_match_torch_sparse_adam():
    """Rows absent from a step keep their moments and parameters, and the bias
    correction counts global steps: torch.optim.SparseAdam's semantics (no
    weight decay there; it adds eps before the bias correction, so eps is
    made negligible and the comparison is to 1e-9)."""
    rng = np.random.default_rng(6)
    vocab, f = 10, 4
    table = rng.normal(0, 0.5, (vocab, f))
    lr, b1, b2, eps = 1e-2, 0.9, 0.999, 1e-30
    w = torch.nn.Parameter(torch.tensor(table, dtype=torch.float64))
    opt = torch.optim.SparseAdam([w], lr=lr, betas=(b1, b2), eps=eps)
    p, m, v = table.copy(), np.zeros_like(table), np.zeros_like(table)
    for step, rows in enumerate(([0, 3, 7], [3, 5], [0, 1, 3, 9], [5, 7]), start=1):
        rows = np.array(rows)
        g = rng.normal(0, 1.0, (len(rows), f))
        w.grad = torch.sparse_coo_tensor(torch.tensor(rows)[None], torch.tensor(g), (vocab, f))
        opt.step()
        p, m, v = O.adamw_rows(p, m, v, rows, g, lr=lr, weight_decay=0.0, step=step,
                               beta1=b1, beta2=b2, eps=eps)
    np.testing.assert_allclose(p, w.detach().numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(p[[2, 4, 6, 8]], table[[2, 4, 6, 8]])


# ---------------------------------------------------------------- STEM variant
def test_stem_is_staple_with_a_zero_up_projection():
    """STEM (up-projection replaced by the table row) equals the STAPLE layer
    with W_up = 0 in every output but dW_up, bit for bit in float64."""
    rng = np.random.default_rng(31)
    x, wg, wu, wd, e, ids, dy = _rand_layer(rng, 40, 16, 24, 9)
    zero = np.zeros_like(wu)
    for prec in (O.EXACT, O.BF16):
        fs = O.ffn_forward(x, wg, None, wd, e, ids, precision=prec)
        fz = O.ffn_forward(x, wg, zero, wd, e, ids, precision=prec)
        for k in ("g", "u", "h", "y", "g_saved", "u_saved"):
            np.testing.assert_array_equal(fs[k], fz[k], err_msg=k)
        bs = O.ffn_backward(dy, x, wg, None, wd, fs, ids, precision=prec)
        bz = O.ffn_backward(dy, x, wg, zero, wd, fz, ids, precision=prec)
        assert "dw_up" not in bs
        for k in ("dh", "du", "dg", "d_rows", "dw_down", "dw_gate", "dx"):
            np.testing.assert_array_equal(bs[k], bz[k], err_msg=k)


def test_stem_matches_torch_autograd():
    """y = W_down (silu(W_gate x) * E[t]) and its gradients, by autograd."""
    rng = np.random.default_rng(32)
    n, d, f, v = 33, 12, 20, 7
    x, wg, _, wd, e, ids, dy = _rand_layer(rng, n, d, f, v)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    xt, wgt, wdt, et = t(x), t(wg), t(wd), t(e)
    y = F.linear(F.silu(F.linear(xt, wgt)) * et[torch.tensor(ids)], wdt)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    fs = O.ffn_forward(x, wg, None, wd, e, ids)
    bs = O.ffn_backward(dy, x, wg, None, wd, fs, ids)
    uniq = np.unique(ids)
    np.testing.assert_allclose(fs["y"], y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bs["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bs["dw_gate"], wgt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bs["dw_down"], wdt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bs["d_rows"], et.grad.numpy()[uniq], rtol=1e-12, atol=1e-12)
