"""The host AdamW update of touched table rows (plain host code in
libstaple.so, no GPU needed) against the oracle's AdamW step."""
import numpy as np
import pytest

from oracle import staple_oracle as O


def _lib():
    st = pytest.importorskip("token_indexed_ffn_amd")
    try:
        st.lib()
    except RuntimeError as e:                      # library not built
        pytest.skip(str(e))
    return st


def _bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_host_adamw_rows_match_oracle_over_lazy_steps(dtype):
    import torch
    st = _lib()
    rng = np.random.default_rng(11)
    vocab, f = 40, 24
    p0 = rng.normal(0, 0.05, (vocab, f))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    table = torch.tensor(p0, dtype=tdt)
    m = torch.zeros(vocab, f, dtype=torch.float32)
    v = torch.zeros(vocab, f, dtype=torch.float32)
    ref_p = table.double().numpy()
    ref_m, ref_v = np.zeros((vocab, f)), np.zeros((vocab, f))
    hp = dict(lr=4e-4, weight_decay=1e-4)
    # the library takes its hyperparameters as float32: give the oracle the same values
    f32 = lambda x: float(np.float32(x))
    ohp = dict(lr=f32(4e-4), weight_decay=f32(1e-4), beta1=f32(0.9), beta2=f32(0.999), eps=f32(1e-8))
    for step, n in enumerate((13, 7, 21), start=1):
        rows = np.sort(rng.choice(vocab, n, replace=False)).astype(np.int32)
        grad = rng.normal(0, 1.0, (n, f)).astype(np.float32)
        before = table.clone()
        st.staple_adamw_rows_host(table, m, v, torch.from_numpy(rows), torch.from_numpy(grad),
                                  step=step, **hp)
        ref_p, ref_m, ref_v = O.adamw_rows(ref_p, ref_m, ref_v, rows, grad.astype(np.float64),
                                           step=step, **ohp)
        if dtype == "bf16":
            ref_p = O.bf16_round(ref_p)            # the table is stored in bf16 after each step
        other = np.setdiff1d(np.arange(vocab), rows)
        assert torch.equal(table[other], before[other]), "untouched rows changed"
        got = table.double().numpy()
        if dtype == "f32":
            np.testing.assert_allclose(got, ref_p, rtol=2e-6, atol=1e-9)
        else:
            assert np.all(np.abs(got - ref_p) <= _bf16_ulp(ref_p) * 1.01), "beyond one bf16 ulp"
            ref_p = got.copy()      # a one-ulp rounding flip must not carry into the next step
        # fp32 rounding of the terms (|(1-b1) g| <= ~0.5, |(1-b2) g^2| <= ~0.02):
        # a few float32 ulps of the terms, also where the new moment cancels
        np.testing.assert_allclose(m.double().numpy(), ref_m, rtol=2e-6, atol=2e-7)
        np.testing.assert_allclose(v.double().numpy(), ref_v, rtol=2e-6, atol=1e-8)


def test_host_adamw_refuses_rows_outside_the_table():
    import torch
    st = _lib()
    table = torch.zeros(8, 16, dtype=torch.bfloat16)
    m, v = torch.zeros(8, 16), torch.zeros(8, 16)
    grad = torch.ones(2, 16)
    before = table.clone()
    with pytest.raises(RuntimeError):
        st.staple_adamw_rows_host(table, m, v, torch.tensor([1, 8], dtype=torch.int32), grad,
                                  lr=1e-3, weight_decay=0.0, step=1)
    assert torch.equal(table, before) and not m.any()
    with pytest.raises(RuntimeError):       # step 0 has no bias correction
        st.staple_adamw_rows_host(table, m, v, torch.tensor([1, 2], dtype=torch.int32), grad,
                                  lr=1e-3, weight_decay=0.0, step=0)


def test_host_adamw_from_several_threads_at_once_matches_serial_calls():
    """The library's host threads are one persistent pool shared by every call:
    calls made at the same time from several threads (each on its own table)
    take turns and give the bits of the same calls made one after another."""
    import threading
    import torch
    st = _lib()
    rng = np.random.default_rng(12)
    vocab, f, n = 600, 512, 400
    jobs = []
    for k in range(6):
        rows = torch.from_numpy(np.sort(rng.choice(vocab, n, replace=False)).astype(np.int32))
        grad = torch.from_numpy(rng.normal(0, 1, (n, f)).astype(np.float32))
        p0 = torch.from_numpy(rng.normal(0, 0.05, (vocab, f)).astype(np.float32)).to(torch.bfloat16)
        jobs.append((rows, grad, p0))

    def run(rows, grad, p0):
        t, m, v = p0.clone(), torch.zeros(vocab, f), torch.zeros(vocab, f)
        for step in (1, 2):
            st.staple_adamw_rows_host(t, m, v, rows, grad, lr=1e-3, weight_decay=1e-2, step=step,
                                      n_threads=8)
        return t, m, v

    serial = [run(*j) for j in jobs]
    out = [None] * len(jobs)
    threads = [threading.Thread(target=lambda i=i: out.__setitem__(i, run(*jobs[i])))
               for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for a, b in zip(serial, out):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_stage_misses_packs_rows_on_the_host_threads():
    """staple_stage_misses packs host_table[ids] into the staging buffer on the
    library's host threads (a 9.4 MB pack uses several) before it queues the
    copy to the device; without a GPU the copy itself fails with
    STAPLE_ERR_HIP, after the pack."""
    import torch
    st = _lib()
    if torch.cuda.is_available():
        pytest.skip("checks the host pack only on a host without a GPU")
    rng = np.random.default_rng(13)
    vocab, f, n = 1000, 8192, 300
    table = rng.normal(0, 1, (vocab, f)).astype(np.float32)
    ids = rng.choice(vocab, n, replace=False).astype(np.int32)
    staging = np.zeros((n, f), dtype=np.float32)
    status = st.lib().staple_stage_misses(table.ctypes.data, vocab, f, 0, ids.ctypes.data, n,
                                          staging.ctypes.data, 16, None)
    assert status == -4
    np.testing.assert_array_equal(staging, table[ids])


def test_group_tables_host_interleaves_token_major():
    """staple_group_tables_host: grouped[t, j] = tables[j][t] (host threads)."""
    import torch
    st = _lib()
    rng = np.random.default_rng(14)
    vocab, f = 3000, 128
    tabs = [torch.from_numpy(rng.normal(0, 1, (vocab, f)).astype(np.float32)).to(torch.bfloat16)
            for _ in range(3)]
    out = torch.empty(vocab, 3, f, dtype=torch.bfloat16)
    st.staple_group_tables_host(tabs, out=out)
    for j in range(3):
        assert torch.equal(out[:, j], tabs[j])
