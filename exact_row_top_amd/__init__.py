"""Exact per-row top-K for MI355X (gfx950): thin Python binding of the C ABI.

Every step of the selection runs in the HIP kernels of ``libexact_row_top.so``;
this module only marshals torch tensors (device memory and the current HIP
stream) into the C calls declared in ``include/exact_row_top.h``.  There is no
CPU fallback: if the library is missing or the device is not gfx950 the calls
raise.

    out = topk_decode(logits, n_valid, k)               # logits [rows, stride] fp32
    out = topk_prefill(logits, row_starts, row_ends, k)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexact_row_top.so")

TOPK_OK, TOPK_EINVAL, TOPK_ELAYOUT, TOPK_EWORKSPACE, TOPK_EDEVICE, TOPK_ELAUNCH = range(6)
STATS_WORDS = 9
VALID_K = (512, 1024, 2048)

_lib = None


class TopKError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"exact_row_top status {status}: {msg}")
        self.status = status


class _Options(ctypes.Structure):
    _fields_ = [("force_wgs_per_row", ctypes.c_int32),
                ("force_rescue", ctypes.c_int32),
                ("row_stats", ctypes.c_void_p),
                ("values", ctypes.c_void_p),
                ("flags", ctypes.c_uint32),
                ("pre_idx", ctypes.c_void_p),
                ("pre_idx_stride", ctypes.c_int64),
                ("bmax", ctypes.c_void_p),
                ("bmax_stride", ctypes.c_int64),
                ("blockskip", ctypes.c_int32),
                ("barrier_spins", ctypes.c_int32)]


TOPK_SORTED = 1
TOPK_DETERMINISTIC = 2


def load_library():
    """Load the C ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_row_top_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.topk_decode.argtypes = [P, I64, P, I32, I32, P, P, SZ, P]
    lib.topk_decode.restype = ctypes.c_int
    lib.topk_prefill.argtypes = [P, I64, P, P, I32, I32, P, I64, P, SZ, P]
    lib.topk_prefill.restype = ctypes.c_int
    lib.topk_decode_v.argtypes = [P, I64, P, I32, I32, P, P, ctypes.c_uint32, P, SZ, P]
    lib.topk_decode_v.restype = ctypes.c_int
    lib.topk_prefill_v.argtypes = [P, I64, P, P, I32, I32, P, P, ctypes.c_uint32, I64, P, SZ, P]
    lib.topk_prefill_v.restype = ctypes.c_int
    lib.topk_decode_varlen.argtypes = [P, I64, P, I32, I32, I32, I32, P, P, ctypes.c_uint32, P,
                                       SZ, P]
    lib.topk_decode_varlen.restype = ctypes.c_int
    lib.topk_decode_hinted.argtypes = [P, I64, P, P, I64, I32, I32, P, P, ctypes.c_uint32, P,
                                       SZ, P]
    lib.topk_decode_hinted.restype = ctypes.c_int
    lib.topk_decode_varlen_hinted.argtypes = [P, I64, P, P, I64, I32, I32, I32, I32, P, P,
                                              ctypes.c_uint32, P, SZ, P]
    lib.topk_decode_varlen_hinted.restype = ctypes.c_int
    lib.topk_decode_blockskip.argtypes = [P, I64, P, P, I64, I32, I32, P, P, ctypes.c_uint32, P,
                                          SZ, P]
    lib.topk_decode_blockskip.restype = ctypes.c_int
    lib.topk_block_max.argtypes = [P, I64, I32, P, I64, P]
    lib.topk_block_max.restype = ctypes.c_int
    lib.topk_decode_varlen_ex.argtypes = [P, I64, P, I32, I32, I32, I32, P, P, SZ, P,
                                          ctypes.POINTER(_Options)]
    lib.topk_decode_varlen_ex.restype = ctypes.c_int
    lib.topk_decode_ex.argtypes = [P, I64, P, I32, I32, P, P, SZ, P, ctypes.POINTER(_Options)]
    lib.topk_decode_ex.restype = ctypes.c_int
    lib.topk_prefill_ex.argtypes = [P, I64, P, P, I32, I32, P, I64, P, SZ, P,
                                    ctypes.POINTER(_Options)]
    lib.topk_prefill_ex.restype = ctypes.c_int
    lib.topk_workspace_bytes.argtypes = [I32, I64, I32]
    lib.topk_workspace_bytes.restype = SZ
    lib.topk_workspace_init.argtypes = [P, SZ, P]
    lib.topk_workspace_init.restype = ctypes.c_int
    lib.topk_decode_noalloc.argtypes = [P, I64, P, I32, I32, P, P]
    lib.topk_decode_noalloc.restype = ctypes.c_int
    lib.topk_read_floor.argtypes = [I32, P, I64, P, P, I32, I32, P, P]
    lib.topk_read_floor.restype = ctypes.c_int
    lib.topk_status.argtypes = [P, P]
    lib.topk_status.restype = ctypes.c_int
    lib.topk_strerror.argtypes = [ctypes.c_int]
    lib.topk_strerror.restype = ctypes.c_char_p
    lib.topk_plan_query.argtypes = [I32, I64, I64, I32, I32, I32, I32, ctypes.POINTER(I64)]
    lib.topk_plan_query.restype = ctypes.c_int
    lib.topk_device_query.argtypes = [ctypes.POINTER(I64)]
    lib.topk_device_query.restype = ctypes.c_int
    lib.topk_workspace_layout.argtypes = [ctypes.POINTER(I64)]
    lib.topk_workspace_layout.restype = ctypes.c_int
    lib.topk_validate.argtypes = [I32, P, I64, P, P, I32, I32, P, P, SZ, I64]
    lib.topk_validate.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().topk_strerror(int(status)).decode()


def _check(status: int):
    if status != TOPK_OK:
        raise TopKError(status, strerror(status))


def workspace_bytes(num_rows: int, row_stride: int, k: int) -> int:
    return int(load_library().topk_workspace_bytes(int(num_rows), int(row_stride), int(k)))


def plan_query(num_rows: int, row_stride: int, k: int, force_wgs_per_row: int = 0,
               cu_count: int = 256, wgs_per_cu: int = 2) -> dict:
    """The launch plan the library would use (host-only, no GPU needed)."""
    out = (ctypes.c_int64 * 7)()
    _check(load_library().topk_plan_query(num_rows, row_stride, 0, k, force_wgs_per_row,
                                          cu_count, wgs_per_cu, out))
    keys = ("wgs_per_row", "quads_per_thread", "rows_per_launch", "launches", "workspace_bytes",
            "cap", "block")
    return dict(zip(keys, (int(x) for x in out)))


def workspace_layout() -> dict:
    """Byte layout of a split-tier workspace (host-only)."""
    out = (ctypes.c_int64 * 6)()
    _check(load_library().topk_workspace_layout(out))
    keys = ("header_bytes", "slot_fixed_bytes", "slots", "data_offset", "slice_bytes",
            "list_bytes")
    return dict(zip(keys, (int(x) for x in out)))


def device_query() -> dict:
    """Compute units and split-tier residency the planner sees (needs a GPU)."""
    out = (ctypes.c_int64 * 37)()
    _check(load_library().topk_device_query(out))
    def tab(off):
        return {k: [int(out[off + 3 * ki + qi]) for qi in range(3)] for ki, k in enumerate(VALID_K)}
    return {"cus": int(out[0]), "split_wgs_per_cu": tab(1), "runtime_wgs_per_cu": tab(10),
            "vgprs": tab(19), "lds_bytes": tab(28)}


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _stream_ptr(stream, device) -> Optional[int]:
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return int(raw(device.index if device.index is not None else torch.cuda.current_device())) or None
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def _require(t, name, dtype, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")


def _logits_layout(logits):
    import torch
    _require(logits, "logits", torch.float32, 2)
    if logits.stride(1) != 1:
        raise ValueError("logits must have unit inner stride")
    rows, width = logits.shape
    row_stride = logits.stride(0) if rows > 1 else width
    if rows > 1 and row_stride < width:
        raise ValueError("logits rows overlap")
    if row_stride != width:
        # a column-sliced view: the kernel may read any aligned float4 of a
        # row's full stride, so the storage must hold the whole last row
        need = (logits.storage_offset() + rows * row_stride) * 4
        if rows and logits.untyped_storage().nbytes() < need:
            raise ValueError("logits storage must hold rows x row_stride floats (full last row)")
    return rows, int(row_stride)


def _out(indices, rows, k, device):
    import torch
    if indices is None:
        return torch.empty((rows, k), dtype=torch.int32, device=device)
    _require(indices, "indices", torch.int32, 2)
    if tuple(indices.shape) != (rows, k) or not indices.is_contiguous():
        raise ValueError(f"indices must be a contiguous int32 [{rows}, {k}] tensor")
    return indices


def _opts(force_wgs_per_row, force_rescue, row_stats, rows, values=None, flags=0, hints=None,
          bmax=None, blockskip=0, barrier_spins=0):
    import torch
    if not (force_wgs_per_row or force_rescue or row_stats is not None or blockskip
            or barrier_spins):
        return None
    if row_stats is not None:
        _require(row_stats, "row_stats", torch.int32, 2)
        if tuple(row_stats.shape) != (rows, STATS_WORDS) or not row_stats.is_contiguous():
            raise ValueError(f"row_stats must be a contiguous int32 [{rows}, {STATS_WORDS}] tensor")
    o = _Options(int(force_wgs_per_row), int(bool(force_rescue)),
                 row_stats.data_ptr() if row_stats is not None else None,
                 values.data_ptr() if values is not None else None, int(flags),
                 hints[0] if hints else None, hints[1] if hints else 0,
                 bmax[0] if bmax else None, bmax[1] if bmax else 0, int(blockskip),
                 int(barrier_spins))
    return ctypes.pointer(o)


def _values(values, return_values, rows, k, device):
    """The values output tensor (float32 [rows, k]) or None."""
    import torch
    if values is None:
        if not return_values:
            return None
        return torch.empty((rows, k), dtype=torch.float32, device=device)
    _require(values, "values", torch.float32, 2)
    if tuple(values.shape) != (rows, k) or not values.is_contiguous() or values.device != device:
        raise ValueError(f"values must be a contiguous float32 [{rows}, {k}] tensor on {device}")
    return values


def _hints(pre_idx, requests, k, device):
    """(pointer, stride) of a hint tensor: int32 [>= requests, >= k], unit
    inner stride; or None."""
    import torch
    if pre_idx is None:
        return None
    _require(pre_idx, "pre_idx", torch.int32, 2)
    if pre_idx.device != device:
        raise ValueError(f"pre_idx must be on {device}")
    if pre_idx.shape[0] < requests or pre_idx.shape[1] < k or pre_idx.stride(1) != 1:
        raise ValueError(f"pre_idx must be int32 [>= {requests}, >= {k}] with unit inner stride")
    stride = pre_idx.stride(0) if pre_idx.shape[0] > 1 else pre_idx.shape[1]
    return pre_idx.data_ptr(), int(stride)


def _bmax(bmax, rows, row_stride, device):
    """(pointer, stride) of a block-maxima tensor: float32 [rows, >=
    ceil(row_stride / 32)] with unit inner stride; or None."""
    import torch
    if bmax is None:
        return None
    _require(bmax, "bmax", torch.float32, 2)
    nb = (row_stride + 31) // 32
    if bmax.device != device or bmax.shape[0] != rows or bmax.shape[1] < nb or bmax.stride(1) != 1:
        raise ValueError(f"bmax must be float32 [{rows}, >= {nb}] with unit inner stride on {device}")
    return bmax.data_ptr(), int(bmax.stride(0) if rows > 1 else bmax.shape[1])


def block_max(logits, bmax=None, *, stream=None):
    """Per-32-score block maxima of every row (the side input of the
    block-skip pass): float32 [rows, ceil(row_stride / 32)]."""
    import torch
    rows, row_stride = _logits_layout(logits)
    nb = (row_stride + 31) // 32
    if bmax is None:
        bmax = torch.empty((rows, nb), dtype=torch.float32, device=logits.device)
    bp = _bmax(bmax, rows, row_stride, logits.device)
    _check(load_library().topk_block_max(logits.data_ptr(), row_stride, rows, bp[0], bp[1],
                                         _stream_ptr(stream, logits.device)))
    return bmax


def _flags(sorted_, deterministic):
    return (TOPK_SORTED if sorted_ else 0) | (TOPK_DETERMINISTIC if deterministic else 0)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def topk_decode(logits, n_valid, k: int, indices=None, *, workspace=None, stream=None,
                values=None, return_values: bool = False, sorted: bool = False,
                deterministic: bool = False, pre_idx=None, bmax=None, blockskip: int = 0,
                force_wgs_per_row: int = 0, force_rescue: bool = False, row_stats=None,
                barrier_spins: int = 0):
    """Exact top-k of logits[r, :n_valid[r]] per row (local indices, -1 pad).

    values / return_values: also the selected scores (-FLT_MAX pad); sorted:
    long rows ordered by value descending, then index ascending;
    deterministic: the k-th value's ties resolved by smallest index; pre_idx:
    optional int32 [rows, >= k] hints (the previous step's top-k positions),
    which steer the guess only; bmax: optional per-32-score block maxima
    (see block_max) for the block-skip pass, taken when the batch passes its
    size gate (blockskip=1 forces it, -1 never).  Returns the indices, or
    (indices, values) when values are asked for."""
    import torch
    lib = load_library()
    rows, row_stride = _logits_layout(logits)
    _require(n_valid, "n_valid", torch.int32, 1)
    if n_valid.shape[0] != rows or not n_valid.is_contiguous():
        raise ValueError("n_valid must be a contiguous int32 [rows] tensor")
    out = _out(indices, rows, k, logits.device)
    vals = _values(values, return_values, rows, k, logits.device)
    flags = _flags(sorted, deterministic)
    hints = _hints(pre_idx, rows, k, logits.device)
    bm = _bmax(bmax, rows, row_stride, logits.device)
    wp, wb = _ws(workspace)
    opts = _opts(force_wgs_per_row, force_rescue, row_stats, rows, vals, flags, hints, bm,
                 blockskip, barrier_spins)
    s = _stream_ptr(stream, logits.device)
    if opts is not None:
        rc = lib.topk_decode_ex(logits.data_ptr(), row_stride, n_valid.data_ptr(), rows, k,
                                out.data_ptr(), wp, wb, s, opts)
    elif bm is not None and hints is None:
        rc = lib.topk_decode_blockskip(logits.data_ptr(), row_stride, n_valid.data_ptr(), bm[0],
                                       bm[1], rows, k, out.data_ptr(),
                                       vals.data_ptr() if vals is not None else None, flags, wp,
                                       wb, s)
    elif bm is not None:
        o = _Options(0, 0, None, vals.data_ptr() if vals is not None else None, int(flags),
                     hints[0], hints[1], bm[0], bm[1], 0)
        rc = lib.topk_decode_ex(logits.data_ptr(), row_stride, n_valid.data_ptr(), rows, k,
                                out.data_ptr(), wp, wb, s, ctypes.pointer(o))
    elif hints is not None:
        rc = lib.topk_decode_hinted(logits.data_ptr(), row_stride, n_valid.data_ptr(), hints[0],
                                    hints[1], rows, k, out.data_ptr(),
                                    vals.data_ptr() if vals is not None else None, flags, wp, wb,
                                    s)
    elif vals is not None or flags:
        rc = lib.topk_decode_v(logits.data_ptr(), row_stride, n_valid.data_ptr(), rows, k,
                               out.data_ptr(), vals.data_ptr() if vals is not None else None,
                               flags, wp, wb, s)
    else:
        rc = lib.topk_decode(logits.data_ptr(), row_stride, n_valid.data_ptr(), rows, k,
                             out.data_ptr(), wp, wb, s)
    _check(rc)
    return (out, vals) if vals is not None else out


def topk_prefill(logits, row_starts, row_ends, k: int, indices=None, *, max_row_len: int = 0,
                 workspace=None, stream=None, values=None, return_values: bool = False,
                 sorted: bool = False, deterministic: bool = False, force_wgs_per_row: int = 0,
                 force_rescue: bool = False, row_stats=None, barrier_spins: int = 0):
    """Exact top-k of logits[r, row_starts[r]:row_ends[r]] per row (ks-relative).

    Output options as for topk_decode."""
    import torch
    lib = load_library()
    rows, row_stride = _logits_layout(logits)
    for name, t in (("row_starts", row_starts), ("row_ends", row_ends)):
        _require(t, name, torch.int32, 1)
        if t.shape[0] != rows or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 [rows] tensor")
    out = _out(indices, rows, k, logits.device)
    vals = _values(values, return_values, rows, k, logits.device)
    flags = _flags(sorted, deterministic)
    wp, wb = _ws(workspace)
    opts = _opts(force_wgs_per_row, force_rescue, row_stats, rows, vals, flags,
                 barrier_spins=barrier_spins)
    s = _stream_ptr(stream, logits.device)
    if opts is not None:
        rc = lib.topk_prefill_ex(logits.data_ptr(), row_stride, row_starts.data_ptr(),
                                 row_ends.data_ptr(), rows, k, out.data_ptr(), int(max_row_len),
                                 wp, wb, s, opts)
    elif vals is not None or flags:
        rc = lib.topk_prefill_v(logits.data_ptr(), row_stride, row_starts.data_ptr(),
                                row_ends.data_ptr(), rows, k, out.data_ptr(),
                                vals.data_ptr() if vals is not None else None, flags,
                                int(max_row_len), wp, wb, s)
    else:
        rc = lib.topk_prefill(logits.data_ptr(), row_stride, row_starts.data_ptr(),
                              row_ends.data_ptr(), rows, k, out.data_ptr(), int(max_row_len),
                              wp, wb, s)
    _check(rc)
    return (out, vals) if vals is not None else out


def topk_decode_varlen(logits, kv_lens, k: int, next_n: int = 1, compress_ratio: int = 1,
                       indices=None, *, workspace=None, stream=None, values=None,
                       return_values: bool = False, sorted: bool = False,
                       deterministic: bool = False, pre_idx=None, bmax=None, blockskip: int = 0,
                       force_wgs_per_row: int = 0, force_rescue: bool = False, row_stats=None,
                       barrier_spins: int = 0):
    """Exact top-k of the varlen / MTP decode form: row r selects from
    logits[r, :n] with n = (kv_lens[r // next_n] - next_n + r % next_n + 1) //
    compress_ratio (no window when kv_lens[r // next_n] < next_n), computed on
    the device from the per-request kv_lens.  pre_idx: optional int32
    [requests, >= k] hints, one row per request shared by its next_n rows.
    bmax / blockskip and the output options as for topk_decode."""
    import torch
    lib = load_library()
    rows, row_stride = _logits_layout(logits)
    _require(kv_lens, "kv_lens", torch.int32, 1)
    need = (rows + int(next_n) - 1) // int(next_n) if next_n >= 1 else 0
    if not kv_lens.is_contiguous() or kv_lens.shape[0] < need:
        raise ValueError(f"kv_lens must be a contiguous int32 tensor of >= {need} requests")
    out = _out(indices, rows, k, logits.device)
    vals = _values(values, return_values, rows, k, logits.device)
    flags = _flags(sorted, deterministic)
    hints = _hints(pre_idx, need, k, logits.device)
    bm = _bmax(bmax, rows, row_stride, logits.device)
    wp, wb = _ws(workspace)
    opts = _opts(force_wgs_per_row, force_rescue, row_stats, rows, vals, flags, hints, bm,
                 blockskip, barrier_spins)
    if opts is None and bm is not None:
        opts = ctypes.pointer(_Options(0, 0, None, vals.data_ptr() if vals is not None else None,
                                       int(flags), hints[0] if hints else None,
                                       hints[1] if hints else 0, bm[0], bm[1], 0))
    s = _stream_ptr(stream, logits.device)
    if opts is not None:
        rc = lib.topk_decode_varlen_ex(logits.data_ptr(), row_stride, kv_lens.data_ptr(), rows,
                                       int(next_n), int(compress_ratio), k, out.data_ptr(), wp, wb,
                                       s, opts)
    elif hints is not None:
        rc = lib.topk_decode_varlen_hinted(logits.data_ptr(), row_stride, kv_lens.data_ptr(),
                                           hints[0], hints[1], rows, int(next_n),
                                           int(compress_ratio), k, out.data_ptr(),
                                           vals.data_ptr() if vals is not None else None, flags,
                                           wp, wb, s)
    else:
        rc = lib.topk_decode_varlen(logits.data_ptr(), row_stride, kv_lens.data_ptr(), rows,
                                    int(next_n), int(compress_ratio), k, out.data_ptr(),
                                    vals.data_ptr() if vals is not None else None, flags, wp, wb,
                                    s)
    _check(rc)
    return (out, vals) if vals is not None else out


def status(device="cuda", stream=None):
    """Stream-ordered count of split-tier row-barrier waits that gave up since
    the previous status() on this device (their calls' results are undefined),
    as an int32 [1] device tensor; the count is reset.  A non-zero count also
    re-zeroes the library-owned slab (caller workspaces need
    topk_workspace_init)."""
    import torch
    out = torch.zeros(1, dtype=torch.int32, device=device)
    _check(load_library().topk_status(out.data_ptr(), _stream_ptr(stream, out.device)))
    return out


def read_floor(logits, extents, k: int, extents2=None, *, sink=None, stream=None):
    """Measurement aid: read exactly the scores a selection of these rows would
    read, in its launch shape, and nothing else (decode: extents = n_valid;
    prefill: extents, extents2 = row_starts, row_ends)."""
    import torch
    rows, row_stride = _logits_layout(logits)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=logits.device)
    mode = 0 if extents2 is None else 1
    _check(load_library().topk_read_floor(
        mode, logits.data_ptr(), row_stride, extents.data_ptr(),
        extents2.data_ptr() if extents2 is not None else None, rows, int(k), sink.data_ptr(),
        _stream_ptr(stream, logits.device)))
    return sink


def new_workspace(num_rows: int, row_stride: int, k: int, device="cuda", stream=None):
    """Allocate and zero a caller-owned workspace (None when the plan needs none)."""
    import torch
    nbytes = workspace_bytes(num_rows, row_stride, k)
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(load_library().topk_workspace_init(ws.data_ptr(), nbytes, _stream_ptr(stream, ws.device)))
    return ws


__all__ = ["topk_decode", "topk_prefill", "topk_decode_varlen", "block_max", "workspace_bytes",
           "new_workspace", "status", "plan_query",
           "strerror", "load_library", "TopKError", "STATS_WORDS", "VALID_K", "TOPK_SORTED",
           "TOPK_DETERMINISTIC"]
