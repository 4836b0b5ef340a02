"""Python binding of libstaple, the gfx950 hot path of the STAPLE
embedding-augmented gated FFN.

Each function here has the name of the C entry point it calls and does
argument marshalling only: it checks tensor placement, allocates outputs with
torch when the caller passes none, and forwards raw device pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's kernels; there is no Python or CPU fallback.
"""
from __future__ import annotations

from typing import Optional

import ctypes

import torch

from . import _lib

F32 = 0
BF16 = 1

_DT = {torch.float32: F32, torch.bfloat16: BF16}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}


class StapleError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_lib.load().staple_status_string(status).decode()})")


def lib():
    return _lib.load()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise StapleError(status, what)


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32") from None


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(*ts) -> None:
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("expected contiguous device tensors")


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(nbytes: int, workspace: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace of {nbytes} bytes required")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_size(w: Optional[torch.Tensor]) -> int:
    return 0 if w is None else w.numel() * w.element_size()


def _need(t: torch.Tensor, n: int, what: str, dtype=torch.int32) -> None:
    """A caller-provided output or index array: dtype and at least n elements (the
    kernels write up to that many; a shorter buffer would be written past its end)."""
    if t.dtype != dtype or t.numel() < n:
        raise ValueError(f"{what}: needs {n} {dtype} elements, got {t.numel()} {t.dtype}")


def _step_outputs(dd: dict, lk: dict, n: int) -> None:
    for k in ("uniq", "inv", "sorted_pos"):
        _need(dd[k], n, k)
    _need(dd["seg_start"], n + 1, "seg_start")
    _need(dd["n_unique"], 1, "n_unique")
    for k in ("code", "miss_uidx"):
        _need(lk[k], n, k)
    _need(lk["n_miss"], 1, "n_miss")


# ----------------------------------------------------------------------------
def staple_get_device_error(stream=None) -> int:
    """Synchronises the stream and returns (and clears) the device error status."""
    return lib().staple_get_device_error(_stream(stream))


def staple_dedup(ids: torch.Tensor, vocab: int, *, out: Optional[dict] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Dedup of one batch: uniq, inv, sorted_pos, seg_start, n_unique (device)."""
    _dev(ids)
    assert ids.dtype == torch.int32
    n = ids.numel()
    dev = ids.device
    if out is None:
        out = {
            "uniq": torch.empty(max(n, 1), dtype=torch.int32, device=dev),
            "inv": torch.empty(max(n, 1), dtype=torch.int32, device=dev),
            "sorted_pos": torch.empty(max(n, 1), dtype=torch.int32, device=dev),
            "seg_start": torch.empty(n + 1, dtype=torch.int32, device=dev),
            "n_unique": torch.empty(1, dtype=torch.int32, device=dev),
        }
    ws = _ws(lib().staple_dedup_workspace_bytes(n), workspace, dev)
    _check(lib().staple_dedup(_p(ids), n, int(vocab), _p(out["uniq"]), _p(out["inv"]),
                              _p(out["sorted_pos"]), _p(out["seg_start"]), _p(out["n_unique"]),
                              _p(ws), _ws_size(ws), _stream(stream)), "staple_dedup")
    return out


def staple_cache_count(ids: torch.Tensor, vocab: int, counts: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    _dev(ids, counts)
    if counts is None:
        counts = torch.zeros(vocab, dtype=torch.int64, device=ids.device)
    _check(lib().staple_cache_count(_p(ids), ids.numel(), int(vocab), _p(counts), _stream(stream)),
           "staple_cache_count")
    return counts


def staple_cache_build(counts: torch.Tensor, capacity: int, *, out: Optional[tuple] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (id_to_slot int32[vocab], slot_to_id int32[capacity])."""
    _dev(counts)
    assert counts.dtype == torch.int64
    vocab = counts.numel()
    if out is None:
        out = (torch.empty(vocab, dtype=torch.int32, device=counts.device),
               torch.empty(max(capacity, 1), dtype=torch.int32, device=counts.device))
    ws = _ws(lib().staple_cache_build_workspace_bytes(vocab), workspace, counts.device)
    _check(lib().staple_cache_build(_p(counts), vocab, int(capacity), _p(out[0]), _p(out[1]),
                                    _p(ws), _ws_size(ws), _stream(stream)), "staple_cache_build")
    return out


def staple_cache_fill(table: torch.Tensor, slot_to_id: torch.Tensor, capacity: int,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """slot_rows[s] = table[slot_to_id[s]]; `table` on the device or pinned host memory."""
    _dev(slot_to_id, out)
    vocab, d_ff = table.shape
    if out is None:
        out = torch.empty(max(capacity, 1), d_ff, dtype=table.dtype, device=slot_to_id.device)
    _check(lib().staple_cache_fill(_p(table), vocab, d_ff, _dt(table), _p(slot_to_id), int(capacity),
                                   _p(out), _stream(stream)), "staple_cache_fill")
    return out


def staple_cache_lookup(uniq: torch.Tensor, n_unique: torch.Tensor, id_to_slot: torch.Tensor, *,
                        out: Optional[dict] = None, stream=None) -> dict:
    """code, miss_uidx, miss_ids, n_miss for the first *n_unique unique IDs."""
    _dev(uniq, n_unique, id_to_slot)
    mu = uniq.numel()
    if out is None:
        out = {k: torch.empty(max(mu, 1), dtype=torch.int32, device=uniq.device)
               for k in ("code", "miss_uidx", "miss_ids")}
        out["n_miss"] = torch.empty(1, dtype=torch.int32, device=uniq.device)
    _check(lib().staple_cache_lookup(_p(uniq), _p(n_unique), mu, _p(id_to_slot), id_to_slot.numel(),
                                     _p(out["code"]), _p(out["miss_uidx"]), _p(out.get("miss_ids")),
                                     _p(out["n_miss"]), _stream(stream)), "staple_cache_lookup")
    return out


def staple_split_tokens(inv: torch.Tensor, code: torch.Tensor, n_unique: torch.Tensor, *,
                        out: Optional[dict] = None, stream=None) -> dict:
    """hit_pos, miss_pos, tok_row and counts {hits, misses} of the batch's tokens."""
    _dev(inv, code, n_unique)
    n = inv.numel()
    max_unique = min(code.numel(), n)
    if out is None:
        out = {k: torch.empty(max(n, 1), dtype=torch.int32, device=inv.device)
               for k in ("hit_pos", "miss_pos", "tok_row")}
        out["counts"] = torch.empty(2, dtype=torch.int32, device=inv.device)
    _check(lib().staple_split_tokens(_p(inv), n, _p(code), _p(n_unique), max_unique,
                                     _p(out["hit_pos"]), _p(out["miss_pos"]), _p(out["tok_row"]),
                                     _p(out["counts"]), _stream(stream)), "staple_split_tokens")
    return out


def staple_stage_misses(host_table: torch.Tensor, host_miss_ids: torch.Tensor, n_miss: int,
                        host_staging: torch.Tensor, dev_miss_rows: torch.Tensor,
                        stream=None) -> None:
    """Pack host_table[host_miss_ids[:n_miss]] into pinned staging, then one async H2D copy."""
    assert not host_table.is_cuda and not host_miss_ids.is_cuda and not host_staging.is_cuda
    assert host_miss_ids.dtype == torch.int32 and host_table.is_contiguous()
    vocab, d_ff = host_table.shape
    _check(lib().staple_stage_misses(_p(host_table), vocab, d_ff, _dt(host_table), _p(host_miss_ids),
                                     int(n_miss), _p(host_staging), _p(dev_miss_rows),
                                     _stream(stream)), "staple_stage_misses")


def staple_stage_misses_dma(host_tables: list, host_miss_ids: torch.Tensor, n_miss: int,
                            host_staging: torch.Tensor, dev_miss_rows: list) -> None:
    """Every layer's miss rows host_tables[l][host_miss_ids[:n_miss]] packed into pinned
    staging and copied to dev_miss_rows[l] on the GPU's DMA engines; returns when the
    copies have completed.  host_tables: [vocab x d_ff] host tensors, or (tensor,
    element offset, row stride) triples for tables interleaved by
    staple_group_tables_host (one stride for all)."""
    if not host_tables or len(host_tables) != len(dev_miss_rows):
        raise ValueError("one device block per table")
    trip = [t if isinstance(t, tuple) else (t, 0, 0) for t in host_tables]
    strides = {s for _, _, s in trip}
    if len(strides) != 1:
        raise ValueError("the tables share one row stride")
    stride = strides.pop()
    dt = trip[0][0].dtype
    d_ff = dev_miss_rows[0].shape[1]
    vocab = None
    for tab, off, s in trip:
        if tab.is_cuda or tab.dtype != dt:
            raise ValueError("tables are host tensors of one dtype")
        v = tab.shape[0] if s == 0 else tab.numel() // s
        vocab = v if vocab is None else min(vocab, v)
        if s == 0 and (tab.dim() != 2 or tab.shape[1] != d_ff or not tab.is_contiguous()):
            raise ValueError("table is a contiguous [vocab x d_ff] tensor")
    for r in dev_miss_rows:
        if not r.is_cuda or r.dtype != dt or r.dim() != 2 or r.shape[1] != d_ff or r.shape[0] < n_miss:
            raise ValueError(f"each device block is [>= {n_miss} x {d_ff}] of the tables' dtype")
    if host_miss_ids.is_cuda or host_miss_ids.dtype != torch.int32:
        raise ValueError("host_miss_ids is a host int32 tensor")
    _need(host_miss_ids, n_miss, "host_miss_ids")
    if host_staging.is_cuda or not host_staging.is_pinned() or host_staging.dtype != dt:
        raise ValueError("host_staging is pinned host memory of the tables' dtype")
    _need(host_staging, len(trip) * n_miss * d_ff, "host_staging", dtype=dt)
    tabs = (ctypes.c_void_p * len(trip))(*[t.data_ptr() + off * t.element_size() for t, off, _ in trip])
    dst = (ctypes.c_void_p * len(trip))(*[r.data_ptr() for r in dev_miss_rows])
    _check(lib().staple_stage_misses_dma(len(trip), ctypes.cast(tabs, ctypes.c_void_p), stride, vocab,
                                         d_ff, _DT[dt], _p(host_miss_ids), int(n_miss),
                                         _p(host_staging), ctypes.cast(dst, ctypes.c_void_p)),
           "staple_stage_misses_dma")


def staple_assemble_rows(cache_rows: torch.Tensor, miss_rows: torch.Tensor, code: torch.Tensor,
                         n_unique: torch.Tensor, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    _dev(cache_rows, miss_rows, code, n_unique, out)
    d_ff = cache_rows.shape[1]
    mu = code.numel()
    if out is None:
        out = torch.empty(mu, d_ff, dtype=cache_rows.dtype, device=code.device)
    _check(lib().staple_assemble_rows(_p(cache_rows), cache_rows.shape[0], _p(miss_rows),
                                      miss_rows.shape[0], _p(code), _p(n_unique), mu, d_ff,
                                      _dt(cache_rows), _p(out), _stream(stream)),
           "staple_assemble_rows")
    return out


def staple_assemble_rows_from_table(cache_rows: torch.Tensor, table: torch.Tensor,
                                    uniq: torch.Tensor, code: torch.Tensor,
                                    n_unique: torch.Tensor, out: Optional[torch.Tensor] = None,
                                    capacity: Optional[int] = None, stream=None) -> torch.Tensor:
    """R[u] = cache_rows[code[u]] on a hit, table[uniq[u]] on a miss (`table` on the device
    or in pinned host memory)."""
    if not (table.is_cuda or table.is_pinned()) or not table.is_contiguous():
        raise ValueError("table must be a contiguous device or pinned host tensor")
    _dev(cache_rows, uniq, code, n_unique, out)
    vocab, d_ff = table.shape
    mu = uniq.numel()
    cap = cache_rows.shape[0] if capacity is None else capacity
    if out is None:
        out = torch.empty(max(mu, 1), d_ff, dtype=table.dtype, device=uniq.device)
    _check(lib().staple_assemble_rows_from_table(_p(cache_rows), cap, _p(table), vocab, _p(uniq),
                                                 _p(code), _p(n_unique), mu, d_ff, _dt(table),
                                                 _p(out), _stream(stream)),
           "staple_assemble_rows_from_table")
    return out


def staple_gather_rows(src: torch.Tensor, index: torch.Tensor, n_rows: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dst[r] = src[index[r]]; `src` on the device or in pinned host memory."""
    if not (src.is_cuda or src.is_pinned()) or not src.is_contiguous():
        raise ValueError("src must be a contiguous device or pinned host tensor")
    _dev(index, n_rows, out)
    d_ff = src.shape[1]
    mr = index.numel()
    if out is None:
        out = torch.empty(mr, d_ff, dtype=src.dtype, device=index.device)
    _check(lib().staple_gather_rows(_p(src), src.shape[0], _p(index), _p(n_rows), mr, d_ff,
                                    _dt(src), _p(out), _stream(stream)), "staple_gather_rows")
    return out


def staple_ffn_fwd(x: torch.Tensor, w_gate: torch.Tensor, w_up: Optional[torch.Tensor],
                   w_down: torch.Tensor, rows: torch.Tensor, row_index: torch.Tensor, *,
                   out_dtype: Optional[torch.dtype] = None, save: bool = False,
                   out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> dict:
    """Forward of one augmented layer (w_up None: the STEM layer, u = rows[row_index]).
    Returns {"y"} (+ "g", "u", "h" when save)."""
    _dev(x, w_gate, w_up, w_down, rows, row_index)
    n, d = x.shape
    f = w_gate.shape[0]
    dt = _dt(x)
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = {"y": torch.empty(n, d, dtype=out_dtype, device=x.device)}
        if save:
            for k in ("g", "u", "h"):
                out[k] = torch.empty(n, f, dtype=x.dtype, device=x.device)
    ws = _ws(lib().staple_ffn_fwd_workspace_bytes(n, d, f, dt), workspace, x.device)
    _check(lib().staple_ffn_fwd(n, d, f, dt, _DT[out["y"].dtype], _p(x), _p(w_gate), _p(w_up),
                                _p(w_down), _p(rows), rows.shape[0], _p(row_index), _p(out["y"]),
                                _p(out.get("g")), _p(out.get("u")), _p(out.get("h")), _p(ws),
                                _ws_size(ws), _stream(stream)), "staple_ffn_fwd")
    return out


def staple_decode_pack_weights(w_gate: Optional[torch.Tensor], w_up: Optional[torch.Tensor],
                               w_down: Optional[torch.Tensor], *, d_model: int, d_ff: int,
                               stream=None) -> tuple:
    """Packed copies of (w_gate, w_up) and of w_down in the decode kernels' read order
    (bf16).  Returns (packed_gate_up, packed_down); packed_gate_up is None without w_gate
    and the gate-only (STEM) operand, d_ff * d_model elements, when w_up is None;
    packed_down is None without w_down."""
    _dev(w_gate, w_up, w_down)
    ref = next(t for t in (w_gate, w_up, w_down) if t is not None)
    pgu = pd = None
    if w_gate is not None:
        pgu = torch.empty((1 if w_up is None else 2) * d_ff * d_model, dtype=ref.dtype,
                          device=ref.device)
    if w_down is not None:
        pd = torch.empty(d_model * d_ff, dtype=ref.dtype, device=ref.device)
    _check(lib().staple_decode_pack_weights(d_model, d_ff, _dt(ref), _p(w_gate), _p(w_up),
                                            _p(w_down), _p(pgu), _p(pd), _stream(stream)),
           "staple_decode_pack_weights")
    return pgu, pd


def _up_proj(packed_gate_up: torch.Tensor, d: int, f: int) -> int:
    """1 for a packed STAPLE gate/up operand (2 f d elements), 0 for a gate-only one (f d)."""
    if packed_gate_up.numel() == 2 * f * d:
        return 1
    if packed_gate_up.numel() == f * d:
        return 0
    raise ValueError("packed_gate_up has neither the gate/up nor the gate-only size")


def staple_ffn_fwd_packed(x: torch.Tensor, packed_gate_up: torch.Tensor,
                          packed_down: torch.Tensor, rows: torch.Tensor, row_index: torch.Tensor,
                          *, d_ff: int, out_dtype: Optional[torch.dtype] = None,
                          save: bool = False, out: Optional[dict] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """staple_ffn_fwd for a decode batch (<= 64 tokens) on packed weights (a gate-only
    packed operand runs the STEM layer)."""
    _dev(x, packed_gate_up, packed_down, rows, row_index)
    n, d = x.shape
    f = d_ff
    up = _up_proj(packed_gate_up, d, f)
    dt = _dt(x)
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = {"y": torch.empty(n, d, dtype=out_dtype, device=x.device)}
        if save:
            for k in ("g", "u", "h"):
                out[k] = torch.empty(n, f, dtype=x.dtype, device=x.device)
    ws = _ws(lib().staple_ffn_fwd_workspace_bytes(n, d, f, dt), workspace, x.device)
    _check(lib().staple_ffn_fwd_packed(n, d, f, dt, _DT[out["y"].dtype], _p(x), _p(packed_gate_up),
                                       up, _p(packed_down), _p(rows), rows.shape[0], _p(row_index),
                                       _p(out["y"]), _p(out.get("g")), _p(out.get("u")),
                                       _p(out.get("h")), _p(ws), _ws_size(ws), _stream(stream)),
           "staple_ffn_fwd_packed")
    return out


def staple_ffn_fwd_packed_noalloc(x: torch.Tensor, packed_gate_up: torch.Tensor,
                                  packed_down: torch.Tensor, rows: torch.Tensor,
                                  row_index: torch.Tensor, *, d_ff: int, out: dict,
                                  stream=None) -> dict:
    """staple_ffn_fwd_packed with its scratch in the library's fixed device array:
    the call allocates nothing, so the caller passes every output in `out`
    ("y", and optionally "g", "u", "h")."""
    _dev(x, packed_gate_up, packed_down, rows, row_index, *out.values())
    n, d = x.shape
    f = d_ff
    _check(lib().staple_ffn_fwd_packed_noalloc(
        n, d, f, _dt(x), _DT[out["y"].dtype], _p(x), _p(packed_gate_up),
        _up_proj(packed_gate_up, d, f), _p(packed_down), _p(rows), rows.shape[0], _p(row_index),
        _p(out["y"]), _p(out.get("g")), _p(out.get("u")), _p(out.get("h")), _stream(stream)),
        "staple_ffn_fwd_packed_noalloc")
    return out


def staple_ffn_gate_up_packed(x: torch.Tensor, packed_gate_up: torch.Tensor, rows: torch.Tensor,
                              row_index: torch.Tensor, h: torch.Tensor,
                              save_g: Optional[torch.Tensor] = None,
                              save_u: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """staple_ffn_gate_up for a decode batch on the packed gate/up weights."""
    _dev(x, packed_gate_up, rows, row_index, h, save_g, save_u)
    n, d = x.shape
    f = h.shape[1]
    _check(lib().staple_ffn_gate_up_packed(n, d, f, _dt(x), _p(x), _p(packed_gate_up),
                                           _up_proj(packed_gate_up, d, f), _p(rows),
                                           rows.shape[0], _p(row_index), _p(h), _p(save_g),
                                           _p(save_u), _stream(stream)),
           "staple_ffn_gate_up_packed")
    return h


def staple_ffn_down_packed(h: torch.Tensor, packed_down: torch.Tensor, y: torch.Tensor,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """staple_ffn_down for a decode batch on the packed down weights."""
    _dev(h, packed_down, y)
    n, f = h.shape
    d = y.shape[1]
    ws = _ws(lib().staple_ffn_down_workspace_bytes(n, d, f, _dt(h)), workspace, h.device)
    _check(lib().staple_ffn_down_packed(n, d, f, _dt(h), _DT[y.dtype], _p(h), _p(packed_down),
                                        _p(y), _p(ws), _ws_size(ws), _stream(stream)),
           "staple_ffn_down_packed")
    return y


def staple_ffn_gate_up(x: torch.Tensor, w_gate: torch.Tensor, w_up: Optional[torch.Tensor],
                       rows: torch.Tensor, row_index: torch.Tensor, h: torch.Tensor,
                       save_g: Optional[torch.Tensor] = None, save_u: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """h = silu(x W_gate^T) * (x W_up^T + rows[row_index]) (fused gather epilogue);
    w_up None: h = silu(x W_gate^T) * rows[row_index] (the STEM layer)."""
    _dev(x, w_gate, w_up, rows, row_index, h, save_g, save_u)
    n, d = x.shape
    f = w_gate.shape[0]
    _check(lib().staple_ffn_gate_up(n, d, f, _dt(x), _p(x), _p(w_gate), _p(w_up), _p(rows),
                                    rows.shape[0], _p(row_index), _p(h), _p(save_g), _p(save_u),
                                    _stream(stream)), "staple_ffn_gate_up")
    return h


def staple_ffn_gate_up_tokens(token_pos: torch.Tensor, n_sel: int, x: torch.Tensor,
                              w_gate: torch.Tensor, w_up: Optional[torch.Tensor],
                              rows: torch.Tensor, row_index: torch.Tensor, h: torch.Tensor,
                              save_g: Optional[torch.Tensor] = None,
                              save_u: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """staple_ffn_gate_up for the tokens token_pos[:n_sel] only (rows of x, h, g, u)."""
    _dev(token_pos, x, w_gate, w_up, rows, row_index, h, save_g, save_u)
    n, d = x.shape
    f = w_gate.shape[0]
    _check(lib().staple_ffn_gate_up_tokens(int(n_sel), _p(token_pos), n, d, f, _dt(x), _p(x),
                                           _p(w_gate), _p(w_up), _p(rows), rows.shape[0],
                                           _p(row_index), _p(h), _p(save_g), _p(save_u),
                                           _stream(stream)), "staple_ffn_gate_up_tokens")
    return h


def staple_ffn_down(h: torch.Tensor, w_down: torch.Tensor, y: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = h W_down^T."""
    _dev(h, w_down, y)
    n, f = h.shape
    d = w_down.shape[0]
    ws = _ws(lib().staple_ffn_down_workspace_bytes(n, d, f, _dt(h)), workspace, h.device)
    _check(lib().staple_ffn_down(n, d, f, _dt(h), _DT[y.dtype], _p(h), _p(w_down), _p(y), _p(ws),
                                 _ws_size(ws), _stream(stream)), "staple_ffn_down")
    return y


class _DecodeLayer(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("x", "packed_gate_up", "packed_down", "cache_rows", "table", "rows", "y")] + \
               [("table_stride", ctypes.c_int64)]


class DecodeStack:
    """The per-layer tensors of staple_decode_step_cached, marshalled once
    (the descriptor array is rebuilt only when this object is)."""

    def __init__(self, layers: list, *, d_model: int, d_ff: int, n_tokens: int):
        keys = ("x", "packed_gate_up", "packed_down", "cache_rows", "table", "rows", "y")
        # keeps the tensors alive; a layer without "rows" (or rows None) reads
        # each token's row in place.  "table" is a [vocab x d_ff] tensor, or a
        # (tensor, element offset, row stride) triple for a layer whose table
        # is interleaved with others' (staple_group_tables_host).
        self.layers = [{k: lay.get(k) for k in keys} for lay in layers]
        ptrs = []
        for lay in self.layers:
            _dev(lay["x"], lay["packed_gate_up"], lay["packed_down"], lay["cache_rows"],
                 lay["rows"], lay["y"])
            tab, off, stride = (lay["table"] if isinstance(lay["table"], tuple)
                                else (lay["table"], 0, 0))
            if not (tab.is_cuda or tab.is_pinned()):
                raise ValueError("table must be a device or pinned host tensor")
            ptrs.append((tab.data_ptr() + off * tab.element_size(), stride))
        self.n_layers = len(layers)
        self.d_model, self.d_ff, self.n_tokens = d_model, d_ff, n_tokens
        self.up_proj = _up_proj(self.layers[0]["packed_gate_up"], d_model, d_ff)
        self.out_dtype = _DT[self.layers[0]["y"].dtype]
        self.desc = (_DecodeLayer * self.n_layers)(
            *[_DecodeLayer(*[(_p(lay[k]) if k != "table" else tp) for k in keys], stride)
              for lay, (tp, stride) in zip(self.layers, ptrs)])


def staple_decode_step_cached(stack: DecodeStack, ids: torch.Tensor, id_to_slot: torch.Tensor,
                              capacity: int, *, dedup_out: dict, lookup_out: dict,
                              workspace: torch.Tensor, group: int = 0, stream=None) -> None:
    """One decode step over the stack: dedup + cache probe, the layers' compact rows
    (group 0: all before the first layer; group G: the first G layers' before, the
    others carried by the gate/up launches of the group before), each layer's
    packed FFN."""
    n = ids.numel()
    vocab = id_to_slot.numel()
    dd, lk = dedup_out, lookup_out
    _dev(ids, id_to_slot, workspace)
    _need(ids, n, "ids")
    _need(id_to_slot, vocab, "id_to_slot")
    _step_outputs(dd, lk, n)
    for lay in stack.layers:
        if lay["x"].numel() < n * stack.d_model:
            raise ValueError(f"each layer's x needs {n} rows")
        if lay["rows"] is not None and lay["rows"].numel() < n * stack.d_ff:
            raise ValueError(f"each layer's rows need {n} rows")
        if lay["y"].numel() < n * stack.d_model:
            raise ValueError(f"each layer's y needs {n} rows")
        if capacity > 0 and (lay["cache_rows"] is None
                             or lay["cache_rows"].numel() < capacity * stack.d_ff):
            raise ValueError("each layer's cache_rows need `capacity` rows")
    _check(lib().staple_decode_step_cached(
        stack.n_layers, ctypes.cast(stack.desc, ctypes.c_void_p), n, stack.d_model, stack.d_ff,
        stack.up_proj, stack.out_dtype, _p(ids), vocab, _p(id_to_slot), int(capacity), int(group),
        _p(dd["uniq"]), _p(dd["inv"]), _p(dd["sorted_pos"]), _p(dd["seg_start"]),
        _p(dd["n_unique"]), _p(lk["code"]), _p(lk["miss_uidx"]), _p(lk["n_miss"]), _p(workspace),
        _ws_size(workspace), _stream(stream)), "staple_decode_step_cached")


class _RowSource(ctypes.Structure):
    _fields_ = [("cache_rows", ctypes.c_void_p), ("table", ctypes.c_void_p),
                ("table_stride", ctypes.c_int64), ("rows", ctypes.c_void_p)]


class RowSources:
    """The per-layer row sources of staple_prefill_rows_cached, marshalled once:
    dicts with "table" (a [vocab x d_ff] device or pinned host tensor, or a
    (tensor, element offset, row stride) triple for tables interleaved by
    staple_group_tables_host), "cache_rows" (device, or None without a cache)
    and "rows" (device [n x d_ff], the layer's compact rows)."""

    def __init__(self, layers: list, *, d_ff: int):
        self.layers = [{k: lay.get(k) for k in ("cache_rows", "table", "rows")} for lay in layers]
        if not self.layers or self.layers[0]["rows"] is None:
            raise ValueError("every layer needs its rows")
        dt = self.layers[0]["rows"].dtype
        descs = []
        for lay in self.layers:
            _dev(lay["cache_rows"], lay["rows"])
            if lay["rows"] is None:
                raise ValueError("every layer needs its rows")
            tab, off, stride = (lay["table"] if isinstance(lay["table"], tuple)
                                else (lay["table"], 0, 0))
            if not (tab.is_cuda or tab.is_pinned()):
                raise ValueError("table must be a device or pinned host tensor")
            for t in (lay["rows"], lay["cache_rows"], tab):
                if t is not None and t.dtype != dt:
                    raise ValueError("tables, caches and rows must share one dtype")
            for t in (lay["rows"], lay["cache_rows"]):
                if t is not None and (t.dim() != 2 or t.shape[1] != d_ff):
                    raise ValueError("rows and cache_rows are [rows x d_ff]")
            if not isinstance(lay["table"], tuple) and (tab.dim() != 2 or tab.shape[1] != d_ff):
                raise ValueError("table is [vocab x d_ff]")
            descs.append(_RowSource(_p(lay["cache_rows"]), tab.data_ptr() + off * tab.element_size(),
                                    stride, _p(lay["rows"])))
        self.n_layers, self.d_ff = len(layers), d_ff
        self.dtype = _dt(self.layers[0]["rows"])
        self.desc = (_RowSource * self.n_layers)(*descs)


def prefill_rows_workspace_bytes(n_tokens: int) -> int:
    return int(lib().staple_prefill_rows_workspace_bytes(n_tokens))


def staple_prefill_rows_cached(sources: RowSources, ids: torch.Tensor, id_to_slot: torch.Tensor,
                               capacity: int, *, dedup_out: dict, lookup_out: dict,
                               workspace: Optional[torch.Tensor], max_workgroups: int = 0,
                               lookup: bool = True, stream=None) -> None:
    """The rows of one prefill chunk for every layer: dedup of `ids`, cache probe,
    then each layer's compact rows (hits from its cache, misses from its table) in
    one launch of at most max_workgroups workgroups (0: enough to fill the GPU).
    lookup False: no dedup or probe; the rows from the uniq, code and n_unique an
    earlier call on the same chunk left in dedup_out / lookup_out."""
    _dev(ids, id_to_slot, workspace)
    n, vocab = ids.numel(), id_to_slot.numel()
    dd, lk = dedup_out, lookup_out
    _need(ids, n, "ids")
    _need(id_to_slot, vocab, "id_to_slot")
    _step_outputs(dd, lk, n)
    for lay in sources.layers:
        if lay["rows"].shape[0] < n:
            raise ValueError(f"each layer's rows need {n} rows")
        if capacity > 0 and (lay["cache_rows"] is None or lay["cache_rows"].shape[0] < capacity):
            raise ValueError("each layer's cache_rows need `capacity` rows")
        if not isinstance(lay["table"], tuple) and lay["table"].shape[0] < vocab:
            raise ValueError("each layer's table needs id_to_slot's vocabulary")
    _check(lib().staple_prefill_rows_cached(
        sources.n_layers, ctypes.cast(sources.desc, ctypes.c_void_p), n, sources.d_ff,
        sources.dtype, _p(ids), vocab, _p(id_to_slot), int(capacity), int(bool(lookup)),
        int(max_workgroups),
        _p(dd["uniq"]), _p(dd["inv"]), _p(dd["sorted_pos"]), _p(dd["seg_start"]),
        _p(dd["n_unique"]), _p(lk["code"]), _p(lk["miss_uidx"]), _p(lk["n_miss"]), _p(workspace),
        _ws_size(workspace), _stream(stream)), "staple_prefill_rows_cached")


def staple_group_tables_host(tables: list, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The tables' rows interleaved token-major: out[t, j] = tables[j][t] (host tensors;
    out pinned when none is given)."""
    for t in tables:
        if t.is_cuda or not t.is_contiguous():
            raise ValueError("expected contiguous host tensors")
    vocab, d_ff = tables[0].shape
    if out is None:
        out = torch.empty(vocab, len(tables), d_ff, dtype=tables[0].dtype, pin_memory=True)
    arr = (ctypes.c_void_p * len(tables))(*[t.data_ptr() for t in tables])
    _check(lib().staple_group_tables_host(ctypes.cast(arr, ctypes.c_void_p), len(tables), vocab,
                                          d_ff, _dt(tables[0]), out.data_ptr()),
           "staple_group_tables_host")
    return out


def decode_step_workspace_bytes(n: int, d: int, f: int) -> int:
    return lib().staple_decode_step_workspace_bytes(n, d, f)


def staple_lowrank_expand(rows_r: torch.Tensor, n_rows: torch.Tensor, proj: torch.Tensor,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Z[u] = proj @ rows_r[u] for u < *n_rows (the low-rank table's d_ff-wide rows)."""
    _dev(rows_r, n_rows, proj, out)
    max_rows, r = rows_r.shape
    f = proj.shape[0]
    if out is None:
        out = torch.empty(max(max_rows, 1), f, dtype=rows_r.dtype, device=rows_r.device)
    _check(lib().staple_lowrank_expand(_p(rows_r), _p(n_rows), max_rows, r, f, _dt(rows_r),
                                       _p(proj), _p(out), _stream(stream)), "staple_lowrank_expand")
    return out


def staple_lowrank_bwd(d_rows: torch.Tensor, rows_r: torch.Tensor, n_rows: torch.Tensor,
                       proj: torch.Tensor, *, out: Optional[dict] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """The low-rank table-row gradient d_rows_r = d_rows @ proj and the projection's
    gradient d_proj = d_rows^T @ rows_r over the first *n_rows rows."""
    _dev(d_rows, rows_r, n_rows, proj)
    max_rows, r = rows_r.shape
    f = proj.shape[0]
    dev = rows_r.device
    if out is None:
        out = {"d_rows_r": torch.empty(max(max_rows, 1), r, dtype=torch.float32, device=dev),
               "d_proj": torch.empty(f, r, dtype=torch.float32, device=dev)}
    ws = _ws(lib().staple_lowrank_bwd_workspace_bytes(max_rows, f, _dt(rows_r)), workspace, dev)
    _check(lib().staple_lowrank_bwd(_p(d_rows), _p(rows_r), _p(n_rows), max_rows, r, f, _dt(rows_r),
                                    _p(proj), _p(out["d_rows_r"]), _p(out["d_proj"]), _p(ws),
                                    _ws_size(ws), _stream(stream)), "staple_lowrank_bwd")
    return out


def staple_adamw_rows(table: torch.Tensor, m: torch.Tensor, v: torch.Tensor, rows: torch.Tensor,
                      grad: torch.Tensor, *, lr: float, weight_decay: float, step: int,
                      n_rows: Optional[torch.Tensor] = None, beta1: float = 0.9,
                      beta2: float = 0.999, eps: float = 1e-8, stream=None) -> None:
    """AdamW on table rows rows[:n] (device tensors; n from the device scalar when given)."""
    _dev(table, m, v, rows, grad, n_rows)
    vocab, d_ff = table.shape
    _check(lib().staple_adamw_rows(_p(table), _p(m), _p(v), vocab, d_ff, _dt(table), _p(rows),
                                   _p(n_rows), rows.numel(), _p(grad), lr, beta1, beta2, eps,
                                   weight_decay, step, _stream(stream)), "staple_adamw_rows")


def staple_adamw_rows_host(table: torch.Tensor, m: torch.Tensor, v: torch.Tensor,
                           rows: torch.Tensor, grad: torch.Tensor, *, lr: float,
                           weight_decay: float, step: int, beta1: float = 0.9,
                           beta2: float = 0.999, eps: float = 1e-8, n_threads: int = 0) -> None:
    """The same update on host tensors with host threads (synchronous)."""
    for t in (table, m, v, rows, grad):
        if t.is_cuda or not t.is_contiguous():
            raise ValueError("expected contiguous host tensors")
    if m.dtype != torch.float32 or v.dtype != torch.float32 or grad.dtype != torch.float32:
        raise TypeError("moments and gradients are float32")
    vocab, d_ff = table.shape
    _check(lib().staple_adamw_rows_host(_p(table), _p(m), _p(v), vocab, d_ff, _dt(table), _p(rows),
                                        rows.numel(), _p(grad), lr, beta1, beta2, eps,
                                        weight_decay, step, n_threads), "staple_adamw_rows_host")


class HostAdamW:
    """The host AdamW update overlapped with the GPU (staple_host_adamw_*): the
    gradient rows leave for the host right after the backward's segment sum
    (pass `event` to staple_ffn_bwd_table_grad as rows_event), a worker
    updates them as they land and, given the batch's cache probe, refreshes
    their cached copies on `copy_stream` (a stream that does not carry the
    step); finish() waits for the host update and orders `stream` after the
    refreshes."""

    def __init__(self, max_rows: int, d_ff: int):
        h = ctypes.c_void_p()
        _check(lib().staple_host_adamw_create(int(max_rows), int(d_ff), ctypes.byref(h)),
               "staple_host_adamw_create")
        self._h = h
        self.max_rows, self.d_ff = int(max_rows), int(d_ff)
        self.event = lib().staple_host_adamw_event(h)

    def start(self, table: torch.Tensor, m: torch.Tensor, v: torch.Tensor, uniq: torch.Tensor,
              n_unique: torch.Tensor, grad: torch.Tensor, *, lr: float, weight_decay: float,
              step: int, copy_stream, code: Optional[torch.Tensor] = None,
              cache_rows: Optional[torch.Tensor] = None, beta1: float = 0.9,
              beta2: float = 0.999, eps: float = 1e-8, n_threads: int = 0) -> None:
        for t in (table, m, v):
            if t.is_cuda or not t.is_contiguous():
                raise ValueError("table and moments are contiguous host tensors")
        _dev(uniq, n_unique, grad)
        if uniq.numel() < self.max_rows or grad.dim() != 2 or grad.shape[1] != self.d_ff \
                or grad.shape[0] < self.max_rows or table.shape[1] != self.d_ff:
            raise ValueError("uniq and grad must hold max_rows rows of the handle's width")
        if (code is None) != (cache_rows is None):
            raise ValueError("code and cache_rows go together")
        if code is not None:
            _dev(code, cache_rows)
            if code.numel() < self.max_rows or cache_rows.shape[-1] != self.d_ff \
                    or not table.is_pinned():
                raise ValueError("a refresh needs the batch's code, the cache of the table's "
                                 "width and a pinned table")
        vocab = table.shape[0]
        cap = 0 if cache_rows is None else cache_rows.shape[0]
        _check(lib().staple_host_adamw_start(self._h, _p(table), _p(m), _p(v), vocab, _dt(table),
                                             _p(uniq), _p(n_unique), _p(grad), lr, beta1, beta2,
                                             eps, weight_decay, step, n_threads, _p(code),
                                             _p(cache_rows), cap, _stream(copy_stream)),
               "staple_host_adamw_start")

    def finish(self, stream=None) -> None:
        _check(lib().staple_host_adamw_finish(self._h, _stream(stream)),
               "staple_host_adamw_finish")

    def close(self) -> None:
        if self._h:
            lib().staple_host_adamw_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def staple_cache_refresh(table: torch.Tensor, uniq: torch.Tensor, code: torch.Tensor,
                         n_unique: torch.Tensor, cache_rows: torch.Tensor, stream=None) -> None:
    """cache_rows[code[u]] = table[uniq[u]] for the cached rows among uniq[:n_unique]."""
    if not (table.is_cuda or table.is_pinned()) or not table.is_contiguous():
        raise ValueError("table must be a contiguous device or pinned host tensor")
    _dev(uniq, code, n_unique, cache_rows)
    vocab, d_ff = table.shape
    _check(lib().staple_cache_refresh(_p(table), vocab, d_ff, _dt(table), _p(uniq), _p(code),
                                      _p(n_unique), uniq.numel(), _p(cache_rows),
                                      cache_rows.shape[0], _stream(stream)), "staple_cache_refresh")


def staple_ffn_bwd_table_grad(dy: torch.Tensor, x: torch.Tensor, w_gate: torch.Tensor,
                              w_up: Optional[torch.Tensor], w_down: torch.Tensor,
                              saved_g: torch.Tensor,
                              saved_u: torch.Tensor, saved_h: Optional[torch.Tensor],
                              sorted_pos: torch.Tensor, seg_start: torch.Tensor,
                              n_unique: torch.Tensor, *, inv: torch.Tensor,
                              max_unique: Optional[int] = None,
                              freeze_up: bool = False, out_dtype: Optional[torch.dtype] = None,
                              out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                              rows_event: Optional[int] = None, stream=None) -> dict:
    """Backward with the table-row gradient: d_rows, dx, dw_gate, dw_up, dw_down
    (w_up None: the STEM layer, no dw_up).  sorted_pos, inv, seg_start, n_unique are
    staple_dedup's outputs for the batch; saved_h None recomputes h from saved_g,
    saved_u."""
    _dev(dy, x, w_gate, w_up, w_down, saved_g, saved_u, saved_h, sorted_pos, inv, seg_start,
         n_unique)
    n, d = x.shape
    f = w_gate.shape[0]
    dt = _dt(x)
    mu = n if max_unique is None else int(max_unique)
    dev = x.device
    if out is None:
        out = {
            "d_rows": torch.empty(max(mu, 1), f, dtype=torch.float32, device=dev),
            "dx": torch.empty(n, d, dtype=out_dtype or x.dtype, device=dev),
            "dw_gate": torch.empty(f, d, dtype=torch.float32, device=dev),
            "dw_up": None if freeze_up or w_up is None
            else torch.empty(f, d, dtype=torch.float32, device=dev),
            "dw_down": torch.empty(d, f, dtype=torch.float32, device=dev),
        }
    ws = _ws(lib().staple_ffn_bwd_workspace_bytes(n, d, f, dt), workspace, dev)
    _check(lib().staple_ffn_bwd_table_grad(
        n, d, f, dt, _DT[out["dx"].dtype], _p(dy), _p(x), _p(w_gate), _p(w_up), _p(w_down),
        _p(saved_g), _p(saved_u), _p(saved_h), _p(sorted_pos), _p(inv), _p(seg_start),
        _p(n_unique), mu,
        _p(out["d_rows"]), _p(out["dx"]), _p(out["dw_gate"]), _p(out.get("dw_up")),
        _p(out["dw_down"]), int(bool(freeze_up)), _p(ws), _ws_size(ws), rows_event,
        _stream(stream)), "staple_ffn_bwd_table_grad")
    return out


def ffn_workspace_bytes(n: int, d: int, f: int, dtype: torch.dtype) -> dict:
    return {"fwd": lib().staple_ffn_fwd_workspace_bytes(n, d, f, _DT[dtype]),
            "bwd": lib().staple_ffn_bwd_workspace_bytes(n, d, f, _DT[dtype]),
            "dedup": lib().staple_dedup_workspace_bytes(n)}
