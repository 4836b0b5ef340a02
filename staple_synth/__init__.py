"""Seeded synthetic inputs for the STAPLE token-indexed FFN.

This module is shared by the HIP path's tests and benchmark and by the oracle's
tests.  It holds none of the method's arithmetic: only random draws, the
truncated Zipf token distribution that stands in for real text, the bf16
encoding of generated inputs, and the named workload shapes.

Token streams stand in for the pages' training/serving text (Dolma 3 Dolmino
Mix and DCLM, STAPLE news synopsis, "Perspective"), which is not available
here.  Ranks are drawn from a Zipf(s) law truncated to the vocabulary and
mapped to token IDs through a fixed seeded permutation, so that the most
frequent IDs are not simply 0..C-1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Seed of the rank -> token-ID permutation.  Fixed for every workload so that
# a cache built from one stream's counts is meaningful for another stream.
PERM_SEED = 7


# --------------------------------------------------------------------------
# Token streams
# --------------------------------------------------------------------------
_CDF_CACHE: dict = {}


def zipf_cdf(vocab: int, s: float = 1.1) -> np.ndarray:
    """Cumulative distribution of p_k proportional to k^-s for k = 1..vocab."""
    key = (int(vocab), float(s))
    cdf = _CDF_CACHE.get(key)
    if cdf is None:
        k = np.arange(1, vocab + 1, dtype=np.float64)
        w = k ** (-s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        cdf[-1] = 1.0
        _CDF_CACHE[key] = cdf
    return cdf


def rank_permutation(vocab: int, perm_seed: int = PERM_SEED) -> np.ndarray:
    """Fixed map from frequency rank (0-based) to token ID."""
    return np.random.default_rng(perm_seed).permutation(vocab).astype(np.int32)


def zipf_ids(n: int, vocab: int, seed: int, s: float = 1.1,
             perm_seed: int = PERM_SEED) -> np.ndarray:
    """n token IDs in [0, vocab), rank ~ truncated Zipf(s), int32."""
    rng = np.random.default_rng(seed)
    cdf = zipf_cdf(vocab, s)
    rank = np.searchsorted(cdf, rng.random(n), side="right")
    rank = np.minimum(rank, vocab - 1)
    return rank_permutation(vocab, perm_seed)[rank].astype(np.int32)


def calibration_counts(vocab: int, n_tokens: int = 1 << 20, seed: int = 8,
                       s: float = 1.1) -> np.ndarray:
    """Per-ID occurrence counts of one seeded calibration stream (int64[vocab]).

    This is the count pass that ranks rows for the frequency-aware cache.
    """
    ids = zipf_ids(n_tokens, vocab, seed, s)
    return np.bincount(ids, minlength=vocab).astype(np.int64)


# --------------------------------------------------------------------------
# Values and their bf16 encoding
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    """N(0, std^2) samples in float32 from PCG64(seed)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16_bits(shape, std: float, seed: int) -> np.ndarray:
    """N(0, std^2) drawn in float32, then rounded once to bf16 (uint16 bits)."""
    return f32_to_bf16_bits(normal_f32(shape, std, seed))


def device_normal(shape, std: float, seed: int, dtype, device):
    """Large seeded N(0, std^2) tensors generated directly in device memory.

    Used for tensors too large to draw on the host (multi-GB tables).  The
    values come from torch's Philox generator on the device; a caller that
    needs some of them on the host copies those rows back.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, float(std), generator=g)
    return t.to(dtype)


# --------------------------------------------------------------------------
# Named workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shape and seeds of one synthetic workload."""

    name: str
    d_model: int
    d_ff: int
    vocab: int
    n_tokens: int            # tokens per batch (decode batch or training micro-batch)
    n_layers: int = 1        # augmented layers run in one step
    dtype: str = "bf16"      # "bf16" or "f32"
    zipf_s: float = 1.1
    cache_fraction: float = 0.0   # share of the vocabulary held in the HBM row cache
    ids_seed: int = 1000
    x_seed: int = 2000
    w_seed: int = 3000
    table_seed: int = 4000
    dy_seed: int = 5000
    x_std: float = 1.0
    w_std: float = 0.02
    table_std: float = 0.02
    dy_std: float = 1.0
    notes: str = ""

    @property
    def cache_capacity(self) -> int:
        return int(round(self.cache_fraction * self.vocab))

    def ids(self, seed_offset: int = 0) -> np.ndarray:
        return zipf_ids(self.n_tokens, self.vocab, self.ids_seed + seed_offset, self.zipf_s)

    def layer_seeds(self, layer: int) -> dict:
        return {
            "x": self.x_seed + layer,
            "w_gate": self.w_seed + 3 * layer + 0,
            "w_up": self.w_seed + 3 * layer + 1,
            "w_down": self.w_seed + 3 * layer + 2,
            "table": self.table_seed + layer,
            "dy": self.dy_seed + layer,
        }


TINY_F32 = Workload(
    name="tiny_f32", d_model=256, d_ff=1024, vocab=4096, n_tokens=512,
    dtype="f32", ids_seed=1000,
    notes="single layer, fp32 end to end; forward plus table-row gradients, "
          "also run with an all-zero table")

OLMO1B_DECODE = Workload(
    name="olmo2_1b_decode_b64_12L", d_model=2048, d_ff=8192, vocab=100352,
    n_tokens=64, n_layers=12, ids_seed=1001,
    notes="decode step: 12 augmented FFN layers, each with its own full "
          "100352x8192 bf16 table resident in HBM; forward only")

OLMO1B_TRAIN = Workload(
    name="olmo2_1b_train_32k", d_model=2048, d_ff=8192, vocab=100352,
    n_tokens=8 * 4096, n_layers=1, ids_seed=1002,
    notes="training micro-batch of 8 x 4096 tokens through one augmented "
          "layer: forward, backward, dedup and fp32 table-row gradient")

OLMO1B_OFFLOAD = Workload(
    name="olmo2_1b_offload_cache5", d_model=2048, d_ff=8192, vocab=100352,
    n_tokens=64, n_layers=12, cache_fraction=0.05, ids_seed=1003,
    notes="12 tables in pinned host memory, top-5% rows (by a calibration "
          "count pass) cached in HBM; decode batch 64 and a 32768-token "
          "training batch")

OLMO7B_TRAIN = Workload(
    name="olmo2_7b_train_16k", d_model=4096, d_ff=11008, vocab=100352,
    n_tokens=16384, n_layers=1, ids_seed=1004,
    notes="7B-shaped layer (the first 16 of 32 FFN layers are augmented): "
          "training batch of 16384 tokens, forward and backward")

OLMO7B_DECODE = Workload(
    name="olmo2_7b_decode_b64_16L", d_model=4096, d_ff=11008, vocab=100352,
    n_tokens=64, n_layers=16, ids_seed=1005,
    notes="7B-shaped decode step: 16 augmented layers, each with its own "
          "100352x11008 bf16 table in HBM; forward only")

OLMO1B_OFFLOAD_TRAIN = Workload(
    name="olmo2_1b_offload_cache5_train_32k", d_model=2048, d_ff=8192, vocab=100352,
    n_tokens=8 * 4096, n_layers=1, cache_fraction=0.05, ids_seed=1006,
    notes="training batch of 32768 tokens through one layer whose table is in "
          "pinned host memory with the top-5% rows cached in HBM")

OLMO1B_OFFLOAD_PREFILL = Workload(
    name="olmo2_1b_offload_cache5_prefill_16k", d_model=2048, d_ff=8192, vocab=100352,
    n_tokens=64 * 256, n_layers=12, cache_fraction=0.05, ids_seed=1007,
    notes="prefill of 64 prompts of 256 tokens (16384 tokens) through the 12 "
          "layers of the offloaded stack (the same tables and cache), in chunks")

WORKLOADS = {w.name: w for w in (TINY_F32, OLMO1B_DECODE, OLMO1B_TRAIN, OLMO1B_OFFLOAD,
                                 OLMO1B_OFFLOAD_TRAIN, OLMO7B_TRAIN, OLMO7B_DECODE,
                                 OLMO1B_OFFLOAD_PREFILL)}


@dataclass
class LayerInputs:
    """Host-side inputs of one layer (bf16 as uint16 bits, f32 as float32)."""

    ids: np.ndarray
    x: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    table: np.ndarray
    dy: np.ndarray
    dtype: str

    def as_f64(self, name: str) -> np.ndarray:
        """Exact values of one input as float64."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


def host_layer_inputs(n_tokens: int, d_model: int, d_ff: int, vocab: int,
                      dtype: str = "bf16", seed: int = 0, zipf_s: float = 1.1,
                      zero_table: bool = False, table_std: float = 0.02,
                      w_std: float = 0.02, ids: Optional[np.ndarray] = None) -> LayerInputs:
    """All inputs of one layer, drawn on the host (small and medium sizes)."""
    if ids is None:
        ids = zipf_ids(n_tokens, vocab, 1000 + seed, zipf_s)
    draw = normal_bf16_bits if dtype == "bf16" else normal_f32
    x = draw((n_tokens, d_model), 1.0, 2000 + seed)
    wg = draw((d_ff, d_model), w_std, 3000 + 3 * seed)
    wu = draw((d_ff, d_model), w_std, 3001 + 3 * seed)
    wd = draw((d_model, d_ff), w_std, 3002 + 3 * seed)
    if zero_table:
        table = np.zeros((vocab, d_ff), dtype=np.uint16 if dtype == "bf16" else np.float32)
    else:
        table = draw((vocab, d_ff), table_std, 4000 + seed)
    dy = draw((n_tokens, d_model), 1.0, 5000 + seed)
    return LayerInputs(ids=np.asarray(ids, dtype=np.int32), x=x, w_gate=wg, w_up=wu,
                       w_down=wd, table=table, dy=dy, dtype=dtype)
