"""Shared helpers of the GPU tests: host<->device marshalling and tolerances."""
import numpy as np

REL_L2 = 5e-3     # relative L2 error bound for floating-point outputs
MAX_ABS = 3e-2    # max-abs error bound for floating-point outputs


def to_dev(a, dtype, dev):
    """Host array (bf16 bits as uint16, or float32) -> device tensor of `dtype`."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_np(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 \
        else t.detach().cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    return rel, mx


def assert_close(got, ref, name, rel_l2=REL_L2, max_abs=MAX_ABS):
    rel, mx = errors(got, ref)
    print(f"  {name}: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= rel_l2 and mx <= max_abs, f"{name}: rel_l2={rel:.3e} (<= {rel_l2}), max_abs={mx:.3e} (<= {max_abs})"
    return rel, mx


def bf16_ulp(v):
    """Spacing of bfloat16 values at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def assert_close_long_sum(got, ref, name, rel_l2=REL_L2, max_abs=MAX_ABS):
    """Bound for outputs that are sums over a whole large batch (weight
    gradients of a 32768-token batch, |value| ~ 100): relative L2 <= rel_l2 and
    max-abs <= max(max_abs, one bf16 ulp at the output's RMS magnitude).

    Derivation: a bf16 intermediate (h, du, dg) computed in fp32 lands on the
    neighbouring bf16 value, relative to the float64 oracle's rounding, for a
    small fraction rho of elements (last-bit differences of fp32 accumulation
    order).  Each such flip moves one term of an N-term sum by ~2^-8 of that
    term, so the error has standard deviation ~ sqrt(rho) * 2^-8 * rms(output),
    independent of the element's own magnitude.  An absolute 3e-2 is below that
    floor once rms(output) reaches ~100; one bf16 ulp at the RMS magnitude sits
    above it for any rho < 1."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel, mx = errors(got, ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = max(max_abs, float(bf16_ulp(rms)))
    print(f"  {name}: rel_l2={rel:.3e} max_abs={mx:.3e} bound={bound:.3e} rms={rms:.3e}", flush=True)
    assert rel <= rel_l2 and mx <= bound, f"{name}: rel_l2={rel:.3e}, max_abs={mx:.3e} (<= {bound:.3e})"
    return rel, mx
