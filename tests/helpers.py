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


def bf16_step(v):
    """Spacing of bfloat16 values at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def assert_close_stored_bf16(got, ref, name, rel_l2=REL_L2, max_abs=MAX_ABS):
    """A tensor the bf16 path stores in bf16 (h, the saved g and u): relative
    L2 <= rel_l2 and, element by element, |got - ref| <= max(max_abs, one bf16
    step at |ref|): a value that lands on the neighbouring bf16 value of the
    oracle's is one step away, which exceeds 3e-2 once |ref| >= 4."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel, mx = errors(got, ref)
    over = np.abs(got - ref) > np.maximum(max_abs, bf16_step(ref))
    print(f"  {name}: rel_l2={rel:.3e} max_abs={mx:.3e} beyond max(3e-2, 1 bf16 step): "
          f"{int(over.sum())}", flush=True)
    assert rel <= rel_l2 and not over.any(), f"{name}: rel_l2={rel:.3e}, {int(over.sum())} elements out"
    return rel, mx


# Multiple of the measured floor allowed for the GPU's max-abs error on
# outputs that sum over a whole large batch.  The floor is how far two correct
# evaluations (float64 and float32 arithmetic, same bf16 rounding points) lie
# apart on the same inputs; the GPU accumulates each dot product in fp32
# through a longer sequential chain (one MFMA k-group after another) than a
# blocked BLAS, so its rounding flips of the bf16 intermediates are somewhat
# more frequent than the float32 evaluation's.
FLOOR_FACTOR = 3.0


def assert_close_floor(got, ref, alt, name, factor=FLOOR_FACTOR, rel_l2=REL_L2, max_abs=MAX_ABS):
    """GPU output `got` against the float64 oracle `ref`, with `alt` the
    oracle's float32 evaluation of the same definition on the same inputs:
    relative L2 <= rel_l2 and max-abs <= max(max_abs, factor * floor), where
    floor = max|alt - ref| is measured here, not assumed."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    alt = np.asarray(alt, dtype=np.float64)
    rel, mx = errors(got, ref)
    floor = float(np.max(np.abs(alt - ref))) if ref.size else 0.0
    bound = max(max_abs, factor * floor)
    print(f"  {name}: rel_l2={rel:.3e} max_abs={mx:.3e} floor={floor:.3e} "
          f"(x{mx / max(floor, 1e-300):.2f}) bound={bound:.3e}", flush=True)
    assert rel <= rel_l2 and mx <= bound, \
        f"{name}: rel_l2={rel:.3e}, max_abs={mx:.3e} (<= {bound:.3e}, floor {floor:.3e})"
    return rel, mx, floor
