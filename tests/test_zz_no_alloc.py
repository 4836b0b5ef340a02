"""The allocation-free decode forward (staple_ffn_fwd_packed_noalloc) against
the workspace form it shares its kernels with (staple_ffn_fwd_packed): two
calls in a row on one GPU, the second with a smaller batch, give the bits of
the workspace form; a problem larger than the fixed scratch is refused before
any launch."""
import numpy as np
import pytest

import staple_synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def st():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_indexed_ffn_amd as st
    st.lib()
    return st


def _layer(torch, st, dev, d, f, up=True):
    from staple_synth import device_normal
    wg = device_normal((f, d), 0.02, 3000, torch.bfloat16, dev)
    wu = device_normal((f, d), 0.02, 3001, torch.bfloat16, dev) if up else None
    wd = device_normal((d, f), 0.02, 3002, torch.bfloat16, dev)
    table = device_normal((5000, f), 0.02, 4000, torch.bfloat16, dev)
    pgu, pd = st.staple_decode_pack_weights(wg, wu, wd, d_model=d, d_ff=f)
    return pgu, pd, table


@pytest.mark.parametrize("d,f,up", [(2048, 8192, True), (4096, 11008, True), (2048, 8192, False)])
def test_noalloc_forward_matches_the_workspace_form_on_two_calls(st, d, f, up):
    import torch
    dev = torch.device("cuda:0")
    print(f"noalloc forward d={d} f={f} up={up}", flush=True)
    pgu, pd, table = _layer(torch, st, dev, d, f, up)
    from staple_synth import device_normal
    for call, n in enumerate((64, 17)):
        x = device_normal((n, d), 1.0, 2000 + call, torch.bfloat16, dev)
        ids = torch.from_numpy(S.zipf_ids(n, table.shape[0], 1000 + call)).to(dev)
        nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device=dev)
        ref = st.staple_ffn_fwd_packed(x, pgu, pd, table, ids, d_ff=f, out_dtype=torch.float32,
                                       save=True)
        # call 1 keeps h in the scratch array; call 2 saves h, g, u
        out = {"y": nan((n, d), torch.float32)}
        if call == 1:
            out.update({k: nan((n, f), torch.bfloat16) for k in ("g", "u", "h")})
        got = st.staple_ffn_fwd_packed_noalloc(x, pgu, pd, table, ids, d_ff=f, out=out)
        torch.cuda.synchronize()
        assert st.staple_get_device_error() == 0
        assert torch.equal(got["y"], ref["y"]), f"call {call}: y"
        for k in ("g", "u", "h"):
            if k in got:
                assert torch.equal(got[k], ref[k]), f"call {call}: {k}"


def test_noalloc_forward_refuses_a_problem_beyond_its_scratch(st):
    import torch
    dev = torch.device("cuda:0")
    lib = st.lib()
    buf = torch.zeros(1 << 20, dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(64, dtype=torch.int32, device=dev)
    y = torch.full((64, 8192), float("nan"), dtype=torch.float32, device=dev)
    p = buf.data_ptr()
    # 64 tokens at d_model 8192: the partial sums alone take 16 MiB
    status = lib.staple_ffn_fwd_packed_noalloc(64, 8192, 8192, 1, 0, p, p, 1, p, p, 10,
                                               idx.data_ptr(), y.data_ptr(), None, None, None,
                                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert status == -7
    assert bool(torch.isnan(y).all()), "nothing may be written"
