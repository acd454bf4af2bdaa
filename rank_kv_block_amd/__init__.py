"""Python binding of the MI355X block predictor (libpred.so, C ABI in include/pred.h).

The functions carry the C names and only marshal arguments: torch tensors give
device pointers (``data_ptr``) and the current HIP stream; every step of the
path runs in the library's HIP kernels.  torch supplies device memory and
streams, nothing else.
"""

import ctypes

import numpy as np

from . import _lib
from ._lib import (PRED_FLAG_ZERO_AG, PRED_OK, PredDims, ERROR_NAMES, PRED_NOALLOC_SCRATCH_BYTES,  # noqa: F401
                   PRED_SCORE_PATH_AUTO, PRED_SCORE_PATH_DECODE, PRED_SCORE_PATH_GENERIC,
                   PRED_ERR_INVALID_DIMS, PRED_ERR_OUT_OF_RANGE, PRED_ERR_OOM, PRED_ERR_UNSUPPORTED,
                   PRED_ERR_NULL_ARG, PRED_ERR_HIP, PRED_ERR_WORKSPACE, PRED_ERR_DEVICE)


class PredError(RuntimeError):
    def __init__(self, code, message):
        self.code = code
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")


def lib():
    return _lib.load()


def _check(rc):
    if rc != PRED_OK:
        raise PredError(rc, lib().pred_last_error().decode())
    return rc


def dims(num_layers, num_q_heads, num_kv_heads, head_dim, r, block_size, max_blocks):
    return PredDims(num_layers, num_q_heads, num_kv_heads, head_dim, r, block_size, max_blocks)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, what, dtypes=None, device=True):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if device and t.device.type != "cuda":
        raise ValueError(f"{what}: tensor must live on the GPU")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


# ------------------------------------------------------------------ pure functions

def pred_a_g_bytes(d):
    v = lib().pred_a_g_bytes(ctypes.byref(d))
    if v < 0:
        _check(int(v))
    return v


def pred_check_fit(d, free_bytes):
    return _check(lib().pred_check_fit(ctypes.byref(d), free_bytes))


def pred_rank_workspace_bytes(n_blocks, n_segments):
    return lib().pred_rank_workspace_bytes(n_blocks, n_segments)


def pred_projection_host(head_dim, r, seed):
    out = np.empty((head_dim, r), np.uint16)
    _check(lib().pred_projection_host(head_dim, r, seed, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def pred_limits():
    return lib().pred_limits().decode()


def pred_version():
    return lib().pred_version().decode()


def pred_last_error():
    return lib().pred_last_error().decode()


# ------------------------------------------------------------------ lifetime

def pred_create(d, seed, flags=0, stream=None):
    h = ctypes.c_void_p()
    _check(lib().pred_create(ctypes.byref(d), seed, flags, _stream(stream), ctypes.byref(h)))
    return h


def pred_create_with_projection(d, p_host, flags=0, stream=None):
    p = np.ascontiguousarray(p_host, dtype=np.uint16)
    if p.shape != (d.head_dim, d.r):
        raise ValueError(f"P must be [{d.head_dim}, {d.r}]")
    h = ctypes.c_void_p()
    _check(lib().pred_create_with_projection(ctypes.byref(d), p.ctypes.data_as(ctypes.c_void_p), flags,
                                             _stream(stream), ctypes.byref(h)))
    return h


def pred_destroy(h):
    lib().pred_destroy(h)


# ------------------------------------------------------------------ hot path

def pred_project_q(h, q, q_proj, stream=None):
    """q [n_vec, Hq, D] bf16 -> q_proj [n_vec, Hq, R] bf16 (any leading shape, flattened)."""
    bt = _bf16_types()
    d = pred_get_dims(h)
    if q.numel() % (d.num_q_heads * d.head_dim) or q_proj.numel() % (d.num_q_heads * d.r):
        raise ValueError("q / q_proj sizes do not match [*, num_q_heads, head_dim / r]")
    n_vec = q.numel() // (d.num_q_heads * d.head_dim)
    if q_proj.numel() != n_vec * d.num_q_heads * d.r:
        raise ValueError("q_proj has the wrong number of elements")
    _check(lib().pred_project_q(h, _ptr(q, "q", bt), n_vec, _ptr(q_proj, "q_proj", bt), _stream(stream)))


def pred_project_kv_block(h, layer0, k, block_table=None, stream=None):
    """k [n_layers, n_blocks, B, Hk, D] bf16; block_table [n_layers, n_blocks] int32 or None."""
    import torch
    d = pred_get_dims(h)
    if k.dim() != 5 or tuple(k.shape[2:]) != (d.block_size, d.num_kv_heads, d.head_dim):
        raise ValueError(f"k must be [n_layers, n_blocks, {d.block_size}, {d.num_kv_heads}, {d.head_dim}]")
    n_layers, n_blocks = k.shape[0], k.shape[1]
    if block_table is not None and tuple(block_table.shape) != (n_layers, n_blocks):
        raise ValueError("block_table must be [n_layers, n_blocks]")
    _check(lib().pred_project_kv_block(h, layer0, n_layers, _ptr(k, "k", _bf16_types()),
                                       _ptr(block_table, "block_table", (torch.int32,)), n_blocks,
                                       _stream(stream)))


def pred_project_step(h, layer0, k_new, new_table, q, q_proj, stream=None):
    """pred_project_kv_block(h, layer0, k_new, new_table) then pred_project_q(h, q, q_proj), in one call:
    k_new [n_layers, n_new, B, Hk, D] bf16 (new_table [n_layers, n_new] int32 or None); q [n_vec, Hq, D]
    -> q_proj [n_vec, Hq, R] (any leading shape, flattened)."""
    import torch
    d = pred_get_dims(h)
    bt = _bf16_types()
    if k_new.dim() != 5 or tuple(k_new.shape[2:]) != (d.block_size, d.num_kv_heads, d.head_dim):
        raise ValueError(f"k_new must be [n_layers, n_new, {d.block_size}, {d.num_kv_heads}, {d.head_dim}]")
    n_layers, n_new = k_new.shape[0], k_new.shape[1]
    if new_table is not None and tuple(new_table.shape) != (n_layers, n_new):
        raise ValueError("new_table must be [n_layers, n_new]")
    if q.numel() % (d.num_q_heads * d.head_dim):
        raise ValueError("q size does not match [*, num_q_heads, head_dim]")
    n_vec = q.numel() // (d.num_q_heads * d.head_dim)
    if q_proj.numel() != n_vec * d.num_q_heads * d.r:
        raise ValueError("q_proj has the wrong number of elements")
    _check(lib().pred_project_step(h, layer0, n_layers, _ptr(k_new, "k_new", bt),
                                   _ptr(new_table, "new_table", (torch.int32,)), n_new, _ptr(q, "q", bt), n_vec,
                                   _ptr(q_proj, "q_proj", bt), _stream(stream)))


def pred_score_blocks(h, layer0, q_proj, block_tables, scores, stream=None):
    """q_proj [n_layers, n_seqs, n_rows, Hq, R]; block_tables [n_seqs, n_blocks] int32 or None;
    scores [n_layers, n_seqs, n_blocks] float32."""
    import torch
    d = pred_get_dims(h)
    if q_proj.dim() != 5 or tuple(q_proj.shape[3:]) != (d.num_q_heads, d.r):
        raise ValueError(f"q_proj must be [n_layers, n_seqs, n_rows, {d.num_q_heads}, {d.r}]")
    n_layers, n_seqs, n_rows = q_proj.shape[:3]
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (n_layers, n_seqs):
        raise ValueError("scores must be [n_layers, n_seqs, n_blocks]")
    n_blocks = scores.shape[2]
    if block_tables is not None and tuple(block_tables.shape) != (n_seqs, n_blocks):
        raise ValueError("block_tables must be [n_seqs, n_blocks]")
    _check(lib().pred_score_blocks(h, layer0, n_layers, _ptr(q_proj, "q_proj", _bf16_types()), n_rows,
                                   _ptr(block_tables, "block_tables", (torch.int32,)), n_blocks, n_seqs,
                                   _ptr(scores, "scores", (torch.float32,)), _stream(stream)))


def pred_score_blocks_masked(h, layer0, q_proj, block_tables, last_fill, scores, stream=None):
    """As pred_score_blocks; last_fill [n_seqs] int32 (or None) = tokens held by each sequence's last block."""
    import torch
    d = pred_get_dims(h)
    if q_proj.dim() != 5 or tuple(q_proj.shape[3:]) != (d.num_q_heads, d.r):
        raise ValueError(f"q_proj must be [n_layers, n_seqs, n_rows, {d.num_q_heads}, {d.r}]")
    n_layers, n_seqs, n_rows = q_proj.shape[:3]
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (n_layers, n_seqs):
        raise ValueError("scores must be [n_layers, n_seqs, n_blocks]")
    n_blocks = scores.shape[2]
    if block_tables is not None and tuple(block_tables.shape) != (n_seqs, n_blocks):
        raise ValueError("block_tables must be [n_seqs, n_blocks]")
    if last_fill is not None and tuple(last_fill.shape) != (n_seqs,):
        raise ValueError("last_fill must be [n_seqs]")
    _check(lib().pred_score_blocks_masked(h, layer0, n_layers, _ptr(q_proj, "q_proj", _bf16_types()), n_rows,
                                          _ptr(block_tables, "block_tables", (torch.int32,)), n_blocks, n_seqs,
                                          _ptr(last_fill, "last_fill", (torch.int32,)),
                                          _ptr(scores, "scores", (torch.float32,)), _stream(stream)))


def pred_rank_victims(h, scores, victims, workspace=None, stream=None):
    """scores [n_segments, n_blocks] float32 -> victims [n_segments, n_blocks] int32."""
    import torch
    if scores.dim() != 2 or tuple(victims.shape) != tuple(scores.shape):
        raise ValueError("scores and victims must both be [n_segments, n_blocks]")
    n_seg, n = scores.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pred_rank_victims(h, _ptr(scores, "scores", (torch.float32,)), n, n_seg,
                                   _ptr(victims, "victims", (torch.int32,)), _ptr(workspace, "workspace"),
                                   ws_bytes, _stream(stream)))


def pred_rank_victims_noalloc(h, scores, victims, stream=None):
    """pred_rank_victims with the library's static device scratch instead of a workspace."""
    import torch
    if scores.dim() != 2 or tuple(victims.shape) != tuple(scores.shape):
        raise ValueError("scores and victims must both be [n_segments, n_blocks]")
    n_seg, n = scores.shape
    _check(lib().pred_rank_victims_noalloc(h, _ptr(scores, "scores", (torch.float32,)), n, n_seg,
                                           _ptr(victims, "victims", (torch.int32,)), _stream(stream)))


def pred_select_victims(h, scores, k, victims, workspace=None, stream=None):
    """scores [n_segments, n_blocks] float32 -> victims [n_segments, k] int32: the k lowest of each row,
    in eviction order (the first k of pred_rank_victims)."""
    import torch
    if scores.dim() != 2 or victims.dim() != 2 or victims.shape[0] != scores.shape[0] or victims.shape[1] != k:
        raise ValueError("scores must be [n_segments, n_blocks] and victims [n_segments, k]")
    n_seg, n = scores.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pred_select_victims(h, _ptr(scores, "scores", (torch.float32,)), n, n_seg, k,
                                     _ptr(victims, "victims", (torch.int32,)), _ptr(workspace, "workspace"),
                                     ws_bytes, _stream(stream)))


def pred_score_rows(h, layer, q_proj, first_pos, block_table, n_blocks, scores, stream=None):
    """Per-row causal scores: q_proj [rows, Hq, R] bf16 (row i at position first_pos + i);
    block_table [n_blocks] int32 or None; scores [rows, stride] float32."""
    import torch
    d = pred_get_dims(h)
    if q_proj.dim() != 3 or tuple(q_proj.shape[1:]) != (d.num_q_heads, d.r):
        raise ValueError(f"q_proj must be [rows, {d.num_q_heads}, {d.r}]")
    rows = q_proj.shape[0]
    if scores.dim() != 2 or scores.shape[0] != rows:
        raise ValueError("scores must be [rows, stride]")
    if block_table is not None and tuple(block_table.shape) != (n_blocks,):
        raise ValueError("block_table must be [n_blocks]")
    _check(lib().pred_score_rows(h, layer, _ptr(q_proj, "q_proj", _bf16_types()), rows, first_pos,
                                 _ptr(block_table, "block_table", (torch.int32,)), n_blocks,
                                 _ptr(scores, "scores", (torch.float32,)), scores.shape[1], _stream(stream)))


def pred_select_keep(h, scores, first_pos, ratio, topk, keep, workspace=None, stream=None):
    """scores [rows, stride] float32 -> keep [rows, topk] int32: per row, the top-k of the blocks complete
    at its position (descending, lower index on ties, -1 past the complete ones)."""
    import torch
    if scores.dim() != 2 or keep.dim() != 2 or keep.shape[0] != scores.shape[0] or keep.shape[1] != topk:
        raise ValueError("scores must be [rows, stride] and keep [rows, topk]")
    rows, stride = scores.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pred_select_keep(h, _ptr(scores, "scores", (torch.float32,)), rows, stride, first_pos, ratio,
                                  topk, _ptr(keep, "keep", (torch.int32,)), _ptr(workspace, "workspace"),
                                  ws_bytes, _stream(stream)))


def pred_decode_step(h, layer0, k_new, new_table, q, q_proj, block_tables, last_fill, scores, k, victims,
                     workspace=None, stream=None):
    """One decode step: k_new [n_layers, n_new, B, Hk, D] (+ new_table [n_layers, n_new] or None) into A_g,
    q [n_layers, n_seqs, n_rows, Hq, D] -> q_proj, scores [n_layers, n_seqs, n_blocks], victims
    [n_layers * n_seqs, k] (the k lowest of each row in eviction order)."""
    import torch
    d = pred_get_dims(h)
    bt = _bf16_types()
    if q.dim() != 5 or tuple(q.shape[3:]) != (d.num_q_heads, d.head_dim):
        raise ValueError(f"q must be [n_layers, n_seqs, n_rows, {d.num_q_heads}, {d.head_dim}]")
    n_layers, n_seqs, n_rows = q.shape[:3]
    if tuple(q_proj.shape) != (n_layers, n_seqs, n_rows, d.num_q_heads, d.r):
        raise ValueError("q_proj must be [n_layers, n_seqs, n_rows, num_q_heads, r]")
    if k_new.dim() != 5 or k_new.shape[0] != n_layers or tuple(k_new.shape[2:]) != (d.block_size, d.num_kv_heads,
                                                                                    d.head_dim):
        raise ValueError("k_new must be [n_layers, n_new, block_size, num_kv_heads, head_dim]")
    n_new = k_new.shape[1]
    if new_table is not None and tuple(new_table.shape) != (n_layers, n_new):
        raise ValueError("new_table must be [n_layers, n_new]")
    if scores.dim() != 3 or tuple(scores.shape[:2]) != (n_layers, n_seqs):
        raise ValueError("scores must be [n_layers, n_seqs, n_blocks]")
    n_blocks = scores.shape[2]
    if block_tables is not None and tuple(block_tables.shape) != (n_seqs, n_blocks):
        raise ValueError("block_tables must be [n_seqs, n_blocks]")
    if last_fill is not None and tuple(last_fill.shape) != (n_seqs,):
        raise ValueError("last_fill must be [n_seqs]")
    if tuple(victims.shape) != (n_layers * n_seqs, k):
        raise ValueError("victims must be [n_layers * n_seqs, k]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pred_decode_step(h, layer0, n_layers, _ptr(k_new, "k_new", bt),
                                  _ptr(new_table, "new_table", (torch.int32,)), n_new, _ptr(q, "q", bt), n_rows,
                                  _ptr(q_proj, "q_proj", bt), _ptr(block_tables, "block_tables", (torch.int32,)),
                                  n_blocks, n_seqs, _ptr(last_fill, "last_fill", (torch.int32,)),
                                  _ptr(scores, "scores", (torch.float32,)), k, _ptr(victims, "victims", (torch.int32,)),
                                  _ptr(workspace, "workspace"), ws_bytes, _stream(stream)))


# ------------------------------------------------------------------ inspection

def pred_score_kernel_name(h, n_rows=1):
    """The kernel pred_score_blocks runs for this handle with n_rows query rows per sequence."""
    name = lib().pred_score_kernel_name(h, n_rows)
    if name is None:
        raise PredError(PRED_ERR_NULL_ARG if not h else PRED_ERR_OUT_OF_RANGE, pred_last_error())
    return name.decode()


def pred_score_kernel_variant(h, n_rows=1, n_blocks=1):
    """The kernel and template arguments pred_score_blocks runs for n_rows rows and n_blocks blocks."""
    name = lib().pred_score_kernel_variant(h, n_rows, n_blocks)
    if name is None:
        raise PredError(PRED_ERR_NULL_ARG if not h else PRED_ERR_OUT_OF_RANGE, pred_last_error())
    return name.decode()


def pred_set_score_path(path):
    """Route score calls through one kernel family (PRED_SCORE_PATH_AUTO / _DECODE / _GENERIC)."""
    return _check(lib().pred_set_score_path(path))


def pred_get_score_path():
    return lib().pred_get_score_path()


def pred_copy_projection(h):
    d = pred_get_dims(h)
    out = np.empty((d.head_dim, d.r), np.uint16)
    _check(lib().pred_copy_projection(h, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def pred_a_g_ptr(h):
    return lib().pred_a_g_ptr(h)


def pred_read_slot(h, layer, block, stream=None):
    d = pred_get_dims(h)
    out = np.empty((d.num_kv_heads, d.block_size, d.r), np.uint16)
    _check(lib().pred_read_slot(h, layer, block, out.ctypes.data_as(ctypes.c_void_p), _stream(stream)))
    return out


def pred_get_dims(h):
    d = PredDims()
    _check(lib().pred_get_dims(h, ctypes.byref(d)))
    return d


def pred_device_error(h, stream=None):
    return _check(lib().pred_device_error(h, _stream(stream)))


def a_g_view(h):
    """A torch view [L, N, Hk, B, R] (int16 bit patterns) of the library-owned A_g, for tests."""
    import torch
    d = pred_get_dims(h)
    shape = (d.num_layers, d.max_blocks, d.num_kv_heads, d.block_size, d.r)
    n = int(np.prod(shape))
    ptr = pred_a_g_ptr(h)
    # wrap the device pointer without copying (no ownership taken)
    class _Holder:
        __cuda_array_interface__ = {
            "shape": (n,), "typestr": "<i2", "data": (ptr, False), "version": 2, "strides": None,
        }
    return torch.as_tensor(_Holder(), device="cuda").view(shape)


class Predictor:
    """Owning wrapper: ``Predictor(dims, seed)`` ... ``close()``."""

    def __init__(self, d, seed=0, flags=0, projection=None, stream=None):
        self.dims = d
        if projection is None:
            self.handle = pred_create(d, seed, flags, stream)
        else:
            self.handle = pred_create_with_projection(d, projection, flags, stream)

    def close(self):
        if self.handle is not None:
            pred_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
