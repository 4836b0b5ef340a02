"""CPU oracle of the STAPLE embedding-augmented gated FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library and does not import it.

It is a plain, slow, float64 statement of what one augmented FFN layer
computes, together with the batch dedup, the frequency-ranked row cache and
the table-row gradient.  Every function says which passage of the STAPLE
pages it follows.  Where the pages leave a step open, the reading taken is
stated next to the code.

Definition of one augmented layer (positions i = 0..N-1, token IDs t_i):

    g_i = W_gate x_i          a_i = W_up x_i
    u_i = a_i + E[t_i]        h_i = silu(g_i) * u_i        y_i = W_down h_i

* The up-projection is kept and the token's table row is added to it as a
  residual path (STAPLE abstract; news synopsis "Pretrained models gain
  sparse capacity without retraining", Synopsis and Interpretation).
* The gate branch multiplies the memory path (same synopsis, Perspective:
  a context-dependent gate controls how much the memory contributes).
* Reading: the gated FFN is the SwiGLU form with SiLU on the gate and no
  biases; the table row is indexed by the input token at the same position.

Two precisions:

* ``"exact"``: every intermediate is kept in float64.  The fp32 workload is
  checked against this mode.
* ``"bf16"``: float64 accumulation, with rounding to bf16 (nearest, ties to
  even) exactly where the bf16 path materialises a tensor between two
  contractions: h (operand of the down-projection), the activations g and u
  saved for the backward pass, and du, dg (operands of the weight-gradient
  and input-gradient contractions).  Reading: the pages fix bf16 tables and
  weights (STAPLE Table 4 caption; Figure 4 caption) but not where
  intermediates are rounded; these are the tensors a bf16 layer stores.
  The table-row gradient is a sum, not a contraction operand: it adds the
  unrounded dL/du (the "fp32 accumulate" of a bf16 layer), so its only
  rounding is that of the saved g it is computed from.

Arithmetic (``accum``): ``"f64"`` (the default, the oracle proper) evaluates
every product and sum in float64.  ``"f32"`` evaluates the same definition
with float32 arithmetic (float32 contractions and elementwise work) and the
same bf16 rounding points.  It is a second correct evaluation of a bf16
layer, used only to measure how far two correct evaluations of a long batch
sum lie apart: the floor of the weight-gradient tolerance.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

EXACT = "exact"
BF16 = "bf16"


# --------------------------------------------------------------------------
# Scalar building blocks
# --------------------------------------------------------------------------
def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range.  The value
    is split as m * 2^e with 0.5 <= |m| < 1, m is rounded to 8 bits with
    round-half-even (numpy's rint), and the result is scaled back.  Below the
    smallest normal (2^-126) the quantum is fixed at 2^-133.  Overflow past
    the largest finite bf16 value goes to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    e = np.maximum(e, -125)          # subnormal range: fixed quantum 2^(-125-8)
    q = np.rint(np.ldexp(v, 8 - e))  # value in units of the quantum 2^(e-8)
    out = np.ldexp(q, e - 8)
    big = np.abs(out) > 3.3895313892515355e38
    if np.any(big):
        out = np.where(big, np.copysign(np.inf, v), out)
    return out


def _real(a) -> np.ndarray:
    """float32 arrays stay float32 (the ``accum="f32"`` evaluation); anything
    else becomes float64."""
    a = np.asarray(a)
    return a if a.dtype == np.float32 else np.asarray(a, dtype=np.float64)


def sigmoid(z) -> np.ndarray:
    z = _real(z)
    with np.errstate(over="ignore"):
        return 1 / (1 + np.exp(-z))


def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z)."""
    z = _real(z)
    return z * sigmoid(z)


def silu_grad(z) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = _real(z)
    s = sigmoid(z)
    return s * (1 + z * (1 - s))


def _maybe_round(a: np.ndarray, precision: str) -> np.ndarray:
    if precision == BF16:
        # every bf16 value is a float32 value: the f32 evaluation stays float32
        return bf16_round(a).astype(a.dtype, copy=False)
    if precision == EXACT:
        return a
    raise ValueError(f"unknown precision {precision!r}")


def _ftype(accum: str):
    if accum == "f64":
        return np.float64
    if accum == "f32":
        return np.float32
    raise ValueError(f"unknown accum {accum!r}")


def _table_rows(table, ids: np.ndarray, cols: Optional[np.ndarray], ft=np.float64) -> np.ndarray:
    """E[t_i] for every position, restricted to the given feature columns."""
    if cols is None:
        return np.asarray(table[ids], dtype=ft)
    return np.asarray(table[np.ix_(ids, cols)], dtype=ft)


# --------------------------------------------------------------------------
# Batch dedup (STAPLE retrieval-path table, Prefill row: the prompt tokens
# are deduplicated once and one inverse token map serves every STAPLE layer;
# AI Radio episode on STAPLE: only the U x d_ff active rows live on the GPU.)
# --------------------------------------------------------------------------
def dedup(ids: Sequence[int]):
    """Unique IDs, inverse map, stably sorted positions and segment offsets.

    Readings: unique IDs are listed in ascending order; positions sharing an
    ID keep ascending position order; segment u of ``sorted_pos`` is
    ``sorted_pos[seg_start[u]:seg_start[u+1]]``.

    Returns (uniq int32[U], inv int32[N], sorted_pos int32[N], seg_start int32[U+1]).
    """
    ids = [int(t) for t in ids]
    n = len(ids)
    uniq = sorted(set(ids))
    index_of = {t: k for k, t in enumerate(uniq)}
    inv = [index_of[t] for t in ids]
    sorted_pos = sorted(range(n), key=lambda i: (ids[i], i))
    seg_start = [0] * (len(uniq) + 1)
    counts = [0] * len(uniq)
    for t in ids:
        counts[index_of[t]] += 1
    for k in range(len(uniq)):
        seg_start[k + 1] = seg_start[k] + counts[k]
    as32 = lambda a: np.asarray(a, dtype=np.int32).reshape(-1)
    return as32(uniq), as32(inv), as32(sorted_pos), as32(seg_start)


# --------------------------------------------------------------------------
# Frequency-aware row cache (AI Radio episode: about 5-6% of the vocabulary
# cached with a frequency-aware policy; STAPLE retrieval-path table, Decode
# row: a GPU lookup probes the LFU cache.)
# --------------------------------------------------------------------------
def cache_build(counts: Sequence[int], capacity: int):
    """Static top-`capacity` cache by count.

    Readings: the cache is built once from a count pass (no eviction is
    described); IDs are ranked by count, larger first, ties by smaller ID; slot
    s holds the ID of rank s; when fewer IDs than `capacity` have non-zero
    counts the ranking still fills every slot.

    Returns (id_to_slot int32[V] with -1 for uncached IDs, slot_to_id int32[C]).
    """
    counts = [int(c) for c in counts]
    vocab = len(counts)
    if not 0 <= capacity <= vocab:
        raise ValueError("capacity out of range")
    ranking = sorted(range(vocab), key=lambda v: (-counts[v], v))
    slot_to_id = ranking[:capacity]
    id_to_slot = [-1] * vocab
    for s, v in enumerate(slot_to_id):
        id_to_slot[v] = s
    return np.asarray(id_to_slot, dtype=np.int32), np.asarray(slot_to_id, dtype=np.int32)


def cache_lookup(uniq: Sequence[int], id_to_slot: Sequence[int]):
    """Probe the cache for each unique ID and list the misses.

    Returns (code int32[U], miss_uidx int32[M]).  ``code[u]`` is the cache slot
    of ``uniq[u]`` on a hit and ``-1 - m`` on a miss, where m is the position of
    u in the miss list; ``miss_uidx`` lists the missing unique indices in
    ascending order (reading: the pages do not fix an order).
    """
    code = []
    miss = []
    for u, t in enumerate(uniq):
        s = int(id_to_slot[int(t)])
        if s >= 0:
            code.append(s)
        else:
            code.append(-1 - len(miss))
            miss.append(u)
    return np.asarray(code, dtype=np.int32), np.asarray(miss, dtype=np.int32)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------
def ffn_forward(x, w_gate, w_up, w_down, table, ids, precision: str = EXACT,
                cols: Optional[np.ndarray] = None, with_y: bool = True,
                accum: str = "f64") -> dict:
    """Forward of one augmented layer.

    x [N, d]; w_gate, w_up [f, d]; w_down [d, f]; table [V, f] (anything that
    supports ``table[ids]`` and ``table[np.ix_(ids, cols)]``); ids [N].

    ``cols`` restricts the feature dimension to a subset (g, u, h for those
    columns only; y needs every column and is then not returned).

    Returns g, u (pre-rounding), g_saved, u_saved (as stored for backward),
    h, and y (when every column is present).

    ``w_up=None`` is the STEM layer the pages compare against: the
    up-projection is replaced by the token's table row, u = E[t] (STAPLE
    abstract: STEM replaces the FFN up-projections with token-indexed
    embeddings, STAPLE keeps them and adds the embeddings as a residual).

    ``accum`` selects float64 (the oracle) or float32 arithmetic (see the
    module docstring).
    """
    ft = _ftype(accum)
    x = np.asarray(x, dtype=ft)
    ids = np.asarray(ids, dtype=np.int64)
    wg = np.asarray(w_gate, dtype=ft)
    wu = None if w_up is None else np.asarray(w_up, dtype=ft)
    if cols is not None:
        wg = wg[cols]
        wu = None if wu is None else wu[cols]
    g = x @ wg.T
    rows = _table_rows(table, ids, cols, ft)
    u = rows if wu is None else x @ wu.T + rows
    h = _maybe_round(silu(g) * u, precision)
    out = {"g": g, "u": u, "h": h,
           "g_saved": _maybe_round(g, precision),
           "u_saved": _maybe_round(u, precision)}
    if cols is None and with_y:
        out["y"] = h @ np.asarray(w_down, dtype=ft).T
    return out


# --------------------------------------------------------------------------
# Backward, including the table-row gradient
# --------------------------------------------------------------------------
def table_row_grad(du: np.ndarray, ids: Sequence[int], uniq: Sequence[int]) -> np.ndarray:
    """dR[u] = sum of du_i over positions whose token is uniq[u].

    The gradient of the compact leaf block (AI Radio episode: active rows as an
    autograd leaf; STAPLE abstract: token-specific updates).  Reading: a plain
    sum over occurrences, no averaging by count.
    """
    du = _real(du)
    index_of = {int(t): k for k, t in enumerate(uniq)}
    out = np.zeros((len(index_of),) + du.shape[1:], dtype=du.dtype)
    for i, t in enumerate(ids):
        out[index_of[int(t)]] += du[i]
    return out


def ffn_backward(dy, x, w_gate, w_up, w_down, fwd: dict, ids, precision: str = EXACT,
                 freeze_up: bool = False, cols: Optional[np.ndarray] = None,
                 uniq: Optional[Sequence[int]] = None, with_dx: bool = True,
                 accum: str = "f64", recompute_h: bool = False,
                 with_dw: bool = True) -> dict:
    """Backward of one augmented layer given the upstream gradient dy [N, d].

    With ``cols`` set, ``fwd`` must come from ``ffn_forward(..., cols=cols)`` and
    every feature-indexed result is restricted to those columns (dx needs every
    column and is then not returned).

    Returns dh, du, dg, d_rows (one row per unique ID, ascending), dw_down,
    dw_gate, dw_up (absent when ``freeze_up``: during warmup the up-projections
    of augmented layers are frozen, STAPLE Table 3 caption; the gradient still
    flows through them into dx and the table rows) and dx.

    ``w_up=None`` (STEM, see ffn_forward): there is no dw_up and dx has no
    up-projection term.

    In the bf16 precision du and dg are rounded where they become operands of
    the weight- and input-gradient contractions, while the table-row
    gradient sums the unrounded dL/du (returned as ``du_sum``): a sum of
    fp32 values accumulated in fp32 (reading of "bf16 in, fp32 accumulate").

    ``recompute_h``: the backward of a caller that kept no h forms it again
    from the saved activations, h = silu(g_saved) * u_saved (rounded as h is),
    for dw_down; everything else is unchanged.  ``with_dw=False`` leaves the
    weight gradients out (for callers that check only the row gradients).
    """
    ft = _ftype(accum)
    dy = np.asarray(dy, dtype=ft)
    x = np.asarray(x, dtype=ft)
    wd = np.asarray(w_down, dtype=ft)
    wg = np.asarray(w_gate, dtype=ft)
    wu = None if w_up is None else np.asarray(w_up, dtype=ft)
    if cols is not None:
        wd = wd[:, cols]
        wg = wg[cols]
        wu = None if wu is None else wu[cols]
    g = np.asarray(fwd["g_saved"], dtype=ft)
    u = np.asarray(fwd["u_saved"], dtype=ft)
    if recompute_h:
        h = _maybe_round(silu(g) * u, precision)
    else:
        h = np.asarray(fwd["h"], dtype=ft)

    dh = dy @ wd                                     # dL/dh = W_down^T dy
    du_sum = dh * silu(g)                            # dL/du = dh * silu(g)
    du = _maybe_round(du_sum, precision)
    dg = _maybe_round(dh * u * silu_grad(g), precision)  # dL/dg = dh * u * silu'(g)

    if uniq is None:
        uniq = sorted(set(int(t) for t in ids))
    out = {
        "dh": dh, "du": du, "dg": dg, "du_sum": du_sum,
        "d_rows": table_row_grad(du_sum, ids, uniq),  # dL/dE[t] summed over occurrences
    }
    if with_dw:
        out["dw_down"] = dy.T @ h                    # dL/dW_down = sum_i dy_i h_i^T
        out["dw_gate"] = dg.T @ x                    # dL/dW_gate = sum_i dg_i x_i^T
    if with_dw and not freeze_up and wu is not None:
        out["dw_up"] = du.T @ x                      # dL/dW_up = sum_i du_i x_i^T
    if cols is None and with_dx:
        out["dx"] = dg @ wg                          # dL/dx = W_gate^T dg (+ W_up^T du)
        if wu is not None:
            out["dx"] = out["dx"] + du @ wu
    return out


# --------------------------------------------------------------------------
# Low-rank table (STAPLE Table 2, row L=12, r=512: the embedding dimension r
# is a capacity axis next to the number of augmented layers, r=512 being the
# low-rank variant; AI Radio episode, paper summary: rank 512 shrinks the
# token-indexed table sixteen times, i.e. d_ff / r at d_ff = 8192).
# Reading: each layer keeps a table E_r of width r and a learned projection
# P [d_ff x r] that maps a row to d_ff, so the up branch becomes
# u = W_up x + P E_r[t]; the pages do not print the map, a bias-free linear
# one is the plainest reading.
# --------------------------------------------------------------------------
def lowrank_rows(table_r, proj, ids, precision: str = EXACT, accum: str = "f64") -> np.ndarray:
    """Z_i = P E_r[t_i] for every position: the d_ff-wide row that the
    low-rank table adds to the up branch.  In the bf16 precision Z is rounded
    once, where the bf16 path stores it (the row block the gate/up reads)."""
    ft = _ftype(accum)
    ids = np.asarray(ids, dtype=np.int64)
    e = np.asarray(table_r[ids], dtype=ft)
    return _maybe_round(e @ np.asarray(proj, dtype=ft).T, precision)


class LowRankTable:
    """The low-rank layer's rows as ffn_forward reads a table: ``t[ids]`` is
    Z_i = P E_r[t_i] for each position and ``t[np.ix_(ids, cols)]`` its
    restriction to some features (rounded as lowrank_rows rounds)."""

    def __init__(self, table_r, proj, precision: str = EXACT, accum: str = "f64"):
        self.table_r = table_r
        self.proj = np.asarray(proj, dtype=np.float64)
        self.precision = precision
        self.accum = accum

    def __getitem__(self, key):
        if isinstance(key, tuple):
            ids, cols = key
            ids = np.asarray(ids).reshape(-1)
            cols = np.asarray(cols).reshape(-1)
            return lowrank_rows(self.table_r, self.proj[cols], ids, self.precision, self.accum)
        return lowrank_rows(self.table_r, self.proj, np.asarray(key).reshape(-1), self.precision,
                            self.accum)


def lowrank_backward(d_rows, table_r, proj, uniq, precision: str = EXACT,
                     accum: str = "f64") -> dict:
    """Gradients of the low-rank table rows and of the projection, given
    d_rows[u] = dL/dZ summed over the positions of uniq[u] (ffn_backward's
    table-row gradient with the Z rows as the table):

        dE_r[uniq[u]] = P^T d_rows[u]          dP = sum_u d_rows[u] E_r[uniq[u]]^T

    (the sums over positions collapse to sums over unique IDs because Z_i
    depends on t_i alone).  In the bf16 precision d_rows is rounded to bf16
    where it becomes the operand of these two contractions."""
    ft = _ftype(accum)
    dz = _maybe_round(np.asarray(d_rows, dtype=ft), precision)
    e = np.asarray(table_r[np.asarray(uniq, dtype=np.int64)], dtype=ft)
    p = np.asarray(proj, dtype=ft)
    return {"d_rows_r": dz @ p, "d_proj": dz.T @ e}


# --------------------------------------------------------------------------
# Optimizer step on the touched table rows
# --------------------------------------------------------------------------
ADAMW_DEFAULTS = dict(beta1=0.9, beta2=0.999, eps=1e-8)


def adamw_rows(table, m, v, rows: Sequence[int], grad, lr: float, weight_decay: float,
               step: int, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8):
    """One AdamW step applied to the listed rows of a table and its moments.

    The tables are trained with AdamW, their moments kept in fp32 beside the
    bf16 table (Figure 4 caption: bf16 tables and fp32 AdamW moments in host
    DRAM; Table 3: peak learning rate and weight decay of the table group).
    For each listed row r with gradient g (decoupled weight decay, bias
    correction with the global step t):

        p <- p (1 - lr wd)
        m <- beta1 m + (1 - beta1) g          v <- beta2 v + (1 - beta2) g^2
        p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)

    Readings: the pages give neither the betas nor epsilon, so they default
    to (0.9, 0.999) and 1e-8; rows outside `rows` are not touched at all,
    neither the parameters nor the moments (a row absent from the batch has
    no gradient, and decaying every row of a 100352-row table in host memory
    at every step is not what an offloaded sparse update does); the step
    count is global, as in a sparse Adam over an embedding.
    Returns new float64 arrays (table, m, v); the inputs are not modified.
    """
    p = np.array(table, dtype=np.float64, copy=True)
    m = np.array(m, dtype=np.float64, copy=True)
    v = np.array(v, dtype=np.float64, copy=True)
    g = np.asarray(grad, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    assert len(np.unique(rows)) == len(rows), "rows must be distinct"
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    for k, r in enumerate(rows):
        p[r] *= 1.0 - lr * weight_decay
        m[r] = beta1 * m[r] + (1.0 - beta1) * g[k]
        v[r] = beta2 * v[r] + (1.0 - beta2) * g[k] * g[k]
        p[r] -= lr / bc1 * m[r] / (np.sqrt(v[r]) / math.sqrt(bc2) + eps)
    return p, m, v
