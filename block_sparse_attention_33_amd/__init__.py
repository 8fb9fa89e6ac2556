"""MiniMax Sparse Attention (MSA) hot path for AMD MI355X (gfx950).

Thin PyTorch binding over the C ABI of libmsa.so (include/msa.h): it checks
tensor shapes and dtypes, allocates outputs and workspaces with torch, and
passes raw device pointers plus torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.

Layouts: q/out [B, S, Hq, D] bf16; k, v [B, G, S, D] bf16; q_idx, k_idx
[B, G, S, 64] int8; block_keys [B, G, nb, 64] int8; sel [B, G, S, top_k]
int32 (ascending, -1 padded).  Decode: q [B, Hq, D], q_idx [B, G, 64],
k_cache / v_cache [B, G, L, D], block_keys [B, G, nb, 64].
"""
import ctypes

import torch

from . import _lib
from ._lib import (MSA_OP_BACKWARD, MSA_OP_DECODE, MSA_OP_INDEX, MSA_OP_POOL, MSA_OP_PREFILL,  # noqa: F401
                   MSA_OP_PREFILL_VARLEN, MsaDims)

__all__ = [
    "MsaError", "make_dims", "profile_enable", "profile_read", "msa_workspace_bytes", "msa_backward_pass_rows", "msa_prefill_chunk_workspace_bytes", "msa_plan_check",
    "msa_pool_block_keys", "msa_index_select",
    "msa_prefill", "msa_prefill_varlen", "msa_prefill_switched", "msa_prefill_lse", "msa_prefill_backward", "msa_prefill_chunk", "msa_prefill_chunk_varlen", "msa_decode", "msa_decode_noalloc", "msa_decode_init", "msa_decode_step", "msa_decode_varlen", "msa_decode_init_varlen", "msa_decode_step_varlen", "MSA_OP_POOL", "MSA_OP_INDEX", "MSA_OP_PREFILL", "MSA_OP_DECODE", "MSA_OP_BACKWARD",
]


class MsaError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where}: {_lib.status_string(code)} ({code})")
        self.code = code


def _check(code, where):
    if code != _lib.MSA_OK:
        raise MsaError(code, where)


def make_dims(batch, seq_len, n_q_heads, n_kv_heads, block_size, top_k, head_dim=128, idx_dim=64,
              softmax_scale=0.0) -> MsaDims:
    return MsaDims(batch, seq_len, n_q_heads, n_kv_heads, head_dim, idx_dim, block_size, top_k,
                   float(softmax_scale))


def msa_workspace_bytes(op, dims: MsaDims):
    """(min_bytes, full_bytes) of workspace for an operation."""
    lo, hi = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.load().msa_workspace_bytes(op, ctypes.byref(dims), ctypes.byref(lo), ctypes.byref(hi)),
           "msa_workspace_bytes")
    return lo.value, hi.value


def msa_probe_mfma_bf16(n_workgroups: int, iters: int, out: torch.Tensor) -> float:
    """Enqueue the matrix-core probe (a kernel of bf16 MFMAs only) on the
    current stream; out: float32 [n_workgroups * 256] on the GPU.  Returns
    the FLOP the launch performs (time it with events on the stream)."""
    _need(out, "out", torch.float32, 1)
    if out.numel() < n_workgroups * 256:
        raise ValueError("out needs n_workgroups * 256 floats")
    flop = ctypes.c_double(0.0)
    _check(_lib.load().msa_probe_mfma_bf16(int(n_workgroups), int(iters), _ptr(out), ctypes.byref(flop),
                                           _stream(out.device)), "msa_probe_mfma_bf16")
    return flop.value


def profile_enable(on: bool = True):
    """Record every launch of the library's kernels with HIP events."""
    _check(_lib.load().msa_profile_enable(1 if on else 0), "msa_profile_enable")


def msa_backward_pass_rows(dims: MsaDims, ws_bytes: int) -> int:
    """Query rows per backward pass with a workspace of ws_bytes (seq_len:
    one pass; 0: below the minimum)."""
    rows = ctypes.c_int32(0)
    _check(_lib.load().msa_backward_pass_rows(ctypes.byref(dims), ctypes.c_size_t(ws_bytes), ctypes.byref(rows)),
           "msa_backward_pass_rows")
    return rows.value


def msa_prefill_chunk_workspace_bytes(dims: MsaDims, count: int):
    """(minimum, full) workspace bytes of msa_prefill_chunk for count queries."""
    lo, hi = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.load().msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), count, ctypes.byref(lo),
                                                         ctypes.byref(hi)), "msa_prefill_chunk_workspace_bytes")
    return lo.value, hi.value


def msa_plan_check(op, dims: MsaDims, ws_bytes: int) -> int:
    """Launches the call would make with a workspace of ws_bytes (host only;
    raises MsaError when the workspace is too small)."""
    n = ctypes.c_int32(0)
    _check(_lib.load().msa_plan_check(op, ctypes.byref(dims), ctypes.c_size_t(ws_bytes), ctypes.byref(n)),
           "msa_plan_check")
    return n.value


def profile_read():
    """{kernel name: (launches, total_ms)} recorded since the last read
    (waits for the recorded launches)."""
    arr = (_lib.MsaKernelTime * 64)()
    n = ctypes.c_int(0)
    _check(_lib.load().msa_profile_read(arr, 64, ctypes.byref(n)), "msa_profile_read")
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n.value, 64))}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(op, dims, device, workspace, sizes=None):
    lo, hi = sizes if sizes is not None else msa_workspace_bytes(op, dims)
    if lo == 0:
        return None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, device)
        return workspace, workspace.numel()
    size = hi
    if op in (MSA_OP_PREFILL, MSA_OP_BACKWARD):
        free, _ = torch.cuda.mem_get_info(device)
        budget = int(free * 0.8)
        if size > budget:
            size = max(lo, budget)
    return torch.empty(size, dtype=torch.uint8, device=device), size


def msa_pool_block_keys(k_idx: torch.Tensor, block_size: int, block_keys=None) -> torch.Tensor:
    """Block summary keys [B, G, nb, 64] (floor-mean of each block's index keys)."""
    _need(k_idx, "k_idx", torch.int8, 4)
    B, G, S, di = k_idx.shape
    nb = -(-S // block_size)
    if block_keys is None:
        block_keys = torch.empty((B, G, nb, di), dtype=torch.int8, device=k_idx.device)
    _need(block_keys, "block_keys", torch.int8, 4, k_idx.device)
    dims = make_dims(B, S, G, G, block_size, 1, idx_dim=di)
    _check(_lib.load().msa_pool_block_keys(ctypes.byref(dims), _ptr(k_idx), _ptr(block_keys),
                                           _stream(k_idx.device)), "msa_pool_block_keys")
    return block_keys


def msa_index_select(q_idx: torch.Tensor, k_idx: torch.Tensor, block_size: int, top_k: int):
    """Index branch: (block_keys [B, G, nb, 64] int8, sel [B, G, S, top_k] int32)."""
    _need(q_idx, "q_idx", torch.int8, 4)
    _need(k_idx, "k_idx", torch.int8, 4, q_idx.device)
    if q_idx.shape != k_idx.shape:
        raise ValueError("q_idx and k_idx must have the same shape")
    B, G, S, di = q_idx.shape
    nb = -(-S // block_size)
    dev = q_idx.device
    block_keys = torch.empty((B, G, nb, di), dtype=torch.int8, device=dev)
    sel = torch.empty((B, G, S, top_k), dtype=torch.int32, device=dev)
    dims = make_dims(B, S, G, G, block_size, top_k, idx_dim=di)
    ws, ws_bytes = _workspace(MSA_OP_INDEX, dims, dev, None)
    _check(_lib.load().msa_index_select(ctypes.byref(dims), _ptr(q_idx), _ptr(k_idx), _ptr(block_keys),
                                        _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)), "msa_index_select")
    return block_keys, sel


def msa_prefill(q, k, v, q_idx, k_idx, block_size: int, top_k: int, softmax_scale: float = 0.0,
                out=None, sel=None, return_sel: bool = False, workspace=None):
    """MSA prefill -> out [B, S, Hq, D] bf16 (and sel when return_sel)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    _need(q_idx, "q_idx", torch.int8, 4, dev)
    _need(k_idx, "k_idx", torch.int8, 4, dev)
    B, S, Hq, D = q.shape
    G = k.shape[1]
    if k.shape != (B, G, S, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [B, G, S, D] = {(B, G, S, D)}")
    if q_idx.shape[:3] != (B, G, S) or k_idx.shape != q_idx.shape:
        raise ValueError("q_idx/k_idx must be [B, G, S, di]")
    dims = make_dims(B, S, Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[3],
                     softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, S, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 4, dev)
    ws, ws_bytes = _workspace(MSA_OP_PREFILL, dims, dev, workspace)
    _check(_lib.load().msa_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx),
                                   _ptr(out), _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)), "msa_prefill")
    return (out, sel) if return_sel else out


def msa_prefill_varlen(q, k, v, q_idx, k_idx, cu_seqlens, block_size: int, top_k: int, softmax_scale: float = 0.0,
                       out=None, sel=None, return_sel: bool = False, workspace=None):
    """Ragged batch of sequences packed along the token axis -> out [T, Hq, D]
    bf16 (and sel [G, T, top_k] when return_sel).  q [T, Hq, D]; k, v [G, T, D];
    q_idx, k_idx [G, T, di]; cu_seqlens: host sequence offsets (list or CPU
    tensor, n + 1 entries from 0 to T)."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_idx, "k_idx", torch.int8, 3, dev)
    T, Hq, D = q.shape
    G = k.shape[0]
    if k.shape != (G, T, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [G, T, D] = {(G, T, D)}")
    if q_idx.shape[:2] != (G, T) or k_idx.shape != q_idx.shape:
        raise ValueError("q_idx/k_idx must be [G, T, di]")
    cu = [int(x) for x in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens)]
    if len(cu) < 2 or cu[-1] != T:
        raise ValueError("cu_seqlens must have n + 1 entries ending at T")
    n = len(cu) - 1
    longest = max(b - a for a, b in zip(cu[:-1], cu[1:]))
    dims = make_dims(n, max(1, longest), Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[2],
                     softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((G, T, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    ws, ws_bytes = _workspace(MSA_OP_PREFILL_VARLEN, dims, dev, workspace)
    cu_arr = (ctypes.c_int32 * len(cu))(*cu)
    _check(_lib.load().msa_prefill_varlen(ctypes.byref(dims), cu_arr, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx),
                                          _ptr(k_idx), _ptr(out), _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)),
           "msa_prefill_varlen")
    return (out, sel) if return_sel else out


def msa_prefill_switched(q, k, v, q_idx, k_idx, block_size: int, top_k: int, dense_below: int = 0,
                         softmax_scale: float = 0.0, out=None, sel=None, workspace=None):
    """msa_prefill, or -- for sequences shorter than dense_below tokens (0:
    8192) -- standard causal GQA attention (not MSA; sel filled with -1).
    Returns (out, took_dense)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    _need(q_idx, "q_idx", torch.int8, 4, dev)
    _need(k_idx, "k_idx", torch.int8, 4, dev)
    B, S, Hq, D = q.shape
    G = k.shape[1]
    if k.shape != (B, G, S, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [B, G, S, D] = {(B, G, S, D)}")
    dims = make_dims(B, S, Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[3],
                     softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4, dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 4, dev)
    below = dense_below if dense_below > 0 else 8192
    ws, ws_bytes = (None, 0) if S < below else _workspace(MSA_OP_PREFILL, dims, dev, workspace)
    took = ctypes.c_int32(-1)
    _check(_lib.load().msa_prefill_switched(ctypes.byref(dims), int(dense_below), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(q_idx), _ptr(k_idx), _ptr(out), _ptr(sel), _ptr(ws), ws_bytes,
                                            _stream(dev), ctypes.byref(took)), "msa_prefill_switched")
    return out, bool(took.value)


def msa_prefill_lse(q, k, v, q_idx, k_idx, block_size: int, top_k: int, softmax_scale: float = 0.0,
                    workspace=None):
    """Prefill for training -> (out [B, S, Hq, D] bf16, sel [B, G, S, top_k]
    int32, lse [B, S, Hq] fp32: natural log-sum-exp of each row's scaled
    scores)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    _need(q_idx, "q_idx", torch.int8, 4, dev)
    _need(k_idx, "k_idx", torch.int8, 4, dev)
    B, S, Hq, D = q.shape
    G = k.shape[1]
    if k.shape != (B, G, S, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [B, G, S, D] = {(B, G, S, D)}")
    if q_idx.shape[:3] != (B, G, S) or k_idx.shape != q_idx.shape:
        raise ValueError("q_idx/k_idx must be [B, G, S, di]")
    dims = make_dims(B, S, Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[3],
                     softmax_scale=softmax_scale)
    out = torch.empty_like(q)
    sel = torch.empty((B, G, S, top_k), dtype=torch.int32, device=dev)
    lse = torch.empty((B, S, Hq), dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(MSA_OP_PREFILL, dims, dev, workspace)
    _check(_lib.load().msa_prefill_lse(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx),
                                       _ptr(out), _ptr(sel), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)),
           "msa_prefill_lse")
    return out, sel, lse


def msa_prefill_backward(q, k, v, out, dout, lse, sel, block_size: int, softmax_scale: float = 0.0,
                         workspace=None):
    """Gradients of the main branch with the selection fixed -> (dq [B, S, Hq, D],
    dk [B, G, S, D], dv [B, G, S, D]) bf16, from the forward's out, lse and sel.
    Without a workspace, one of the full size is allocated when it fits in 80 %
    of the free device memory, else the largest that does (the library then
    runs the query rows in passes; at least the minimum size is needed)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, S, Hq, D = q.shape
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 4, dev)
    _need(out, "out", torch.bfloat16, 4, dev)
    _need(dout, "dout", torch.bfloat16, 4, dev)
    _need(lse, "lse", torch.float32, 3, dev)
    _need(sel, "sel", torch.int32, 4, dev)
    G = k.shape[1]
    top_k = sel.shape[3]
    if k.shape != (B, G, S, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [B, G, S, D] = {(B, G, S, D)}")
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (B, S, Hq) or sel.shape[:3] != (B, G, S):
        raise ValueError("out/dout must be [B, S, Hq, D], lse [B, S, Hq], sel [B, G, S, top_k]")
    dims = make_dims(B, S, Hq, G, block_size, top_k, head_dim=D, softmax_scale=softmax_scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws, ws_bytes = _workspace(MSA_OP_BACKWARD, dims, dev, workspace)
    _check(_lib.load().msa_prefill_backward(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                            _ptr(lse), _ptr(sel), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes,
                                            _stream(dev)), "msa_prefill_backward")
    return dq, dk, dv


def msa_decode(q, q_idx, k_cache, v_cache, block_keys, block_size: int, top_k: int,
               softmax_scale: float = 0.0, out=None, sel=None, return_sel: bool = False, workspace=None):
    """One decode step at position L - 1 -> out [B, Hq, D] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    B, Hq, D = q.shape
    _, G, L, _ = k_cache.shape
    nb = -(-L // block_size)
    if k_cache.shape != (B, G, L, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, L, D]")
    if q_idx.shape[:2] != (B, G) or block_keys.shape != (B, G, nb, q_idx.shape[2]):
        raise ValueError("q_idx must be [B, G, di] and block_keys [B, G, nb, di]")
    dims = make_dims(B, L, Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[2],
                     softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    ws, ws_bytes = _workspace(MSA_OP_DECODE, dims, dev, workspace)
    _check(_lib.load().msa_decode(ctypes.byref(dims), _ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_keys), _ptr(out), _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)),
           "msa_decode")
    return (out, sel) if return_sel else out


def msa_decode_noalloc(q, q_idx, k_cache, v_cache, block_keys, block_size: int, top_k: int, out,
                       softmax_scale: float = 0.0, sel=None):
    """msa_decode through the entry point that allocates nothing: the caller
    passes the output (and optionally sel); the library's scratch is a fixed
    per-device array.  Returns out (and sel when given)."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    _need(out, "out", torch.bfloat16, 3, dev)
    B, Hq, D = q.shape
    _, G, L, _ = k_cache.shape
    nb = -(-L // block_size)
    if k_cache.shape != (B, G, L, D) or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("k_cache/v_cache must be [B, G, L, D] and out shaped like q")
    if q_idx.shape[:2] != (B, G) or block_keys.shape != (B, G, nb, q_idx.shape[2]):
        raise ValueError("q_idx must be [B, G, di] and block_keys [B, G, nb, di]")
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    dims = make_dims(B, L, Hq, G, block_size, top_k, head_dim=D, idx_dim=q_idx.shape[2],
                     softmax_scale=softmax_scale)
    _check(_lib.load().msa_decode_noalloc(ctypes.byref(dims), _ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(block_keys), _ptr(out), _ptr(sel), _stream(dev)),
           "msa_decode_noalloc")
    return (out, sel) if sel is not None else out


def _cache_dims(k_cache, block_size, top_k, n_q_heads, idx_dim, softmax_scale=0.0):
    B, G, C, D = k_cache.shape
    return make_dims(B, C, n_q_heads, G, block_size, top_k, head_dim=D, idx_dim=idx_dim,
                     softmax_scale=softmax_scale)


def msa_decode_init(k_idx, length: int, block_size: int, block_keys=None, open_sums=None):
    """Summaries and open-block sums of caches holding `length` tokens.
    k_idx [B, G, C, di] int8 (capacity C) -> (block_keys [B, G, ceil(C/bs), di]
    int8, open_sums [B, G, di] int32)."""
    _need(k_idx, "k_idx", torch.int8, 4)
    dev = k_idx.device
    B, G, C, di = k_idx.shape
    nbc = -(-C // block_size)
    if block_keys is None:
        block_keys = torch.zeros((B, G, nbc, di), dtype=torch.int8, device=dev)
    if open_sums is None:
        open_sums = torch.zeros((B, G, di), dtype=torch.int32, device=dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    _need(open_sums, "open_sums", torch.int32, 3, dev)
    if block_keys.shape != (B, G, nbc, di) or open_sums.shape != (B, G, di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di] and open_sums [B, G, di]")
    dims = make_dims(B, C, G, G, block_size, 1, idx_dim=di)
    _check(_lib.load().msa_decode_init(ctypes.byref(dims), int(length), _ptr(k_idx), _ptr(block_keys),
                                       _ptr(open_sums), _stream(dev)), "msa_decode_init")
    return block_keys, open_sums


def msa_decode_step(q, q_idx, k_new, v_new, k_idx_new, k_cache, v_cache, open_sums, block_keys, length: int,
                    block_size: int, top_k: int, softmax_scale: float = 0.0, out=None, sel=None,
                    return_sel: bool = False, workspace=None):
    """Append token length - 1 (k_new, v_new [B, G, D], k_idx_new [B, G, di])
    to caches of capacity C ([B, G, C, D]), refresh its block's summary, then
    decode q [B, Hq, D] at that position -> out [B, Hq, D] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_new, "k_new", torch.bfloat16, 3, dev)
    _need(v_new, "v_new", torch.bfloat16, 3, dev)
    _need(k_idx_new, "k_idx_new", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(open_sums, "open_sums", torch.int32, 3, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    B, Hq, D = q.shape
    _, G, C, _ = k_cache.shape
    di = q_idx.shape[2]
    if k_cache.shape != (B, G, C, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, C, D]")
    if k_new.shape != (B, G, D) or v_new.shape != (B, G, D):
        raise ValueError("k_new/v_new must be [B, G, D]")
    if q_idx.shape != (B, G, di) or k_idx_new.shape != (B, G, di) or open_sums.shape != (B, G, di):
        raise ValueError("q_idx, k_idx_new and open_sums must be [B, G, di]")
    if block_keys.shape != (B, G, -(-C // block_size), di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di]")
    dims = _cache_dims(k_cache, block_size, top_k, Hq, di, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    ws, ws_bytes = _workspace(MSA_OP_DECODE, dims, dev, workspace)
    _check(_lib.load().msa_decode_step(ctypes.byref(dims), int(length), _ptr(q), _ptr(q_idx), _ptr(k_new),
                                       _ptr(v_new), _ptr(k_idx_new), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(open_sums), _ptr(block_keys), _ptr(out), _ptr(sel), _ptr(ws),
                                       ws_bytes, _stream(dev)), "msa_decode_step")
    return (out, sel) if return_sel else out


def _on_device(lengths, B, dev):
    """True for an int32 [B] tensor on the GPU (read by the kernels)."""
    if isinstance(lengths, torch.Tensor) and lengths.device.type == "cuda":
        _need(lengths, "lengths", torch.int32, 1, dev)
        if lengths.shape[0] != B or not lengths.is_contiguous():
            raise ValueError(f"device lengths must be a contiguous int32 tensor of {B} entries")
        return True
    return False


def _lengths(lengths, B):
    vals = [int(x) for x in (lengths.tolist() if isinstance(lengths, torch.Tensor) else lengths)]
    if len(vals) != B:
        raise ValueError(f"lengths needs one entry per sequence ({B})")
    return (ctypes.c_int32 * B)(*vals)


def msa_decode_varlen(q, q_idx, k_cache, v_cache, block_keys, lengths, block_size: int, top_k: int,
                      softmax_scale: float = 0.0, out=None, sel=None, return_sel: bool = False, workspace=None):
    """Decode of a ragged batch: sequence b's query at position lengths[b] -
    1 over its first lengths[b] cached tokens (caches [B, G, C, D] of
    capacity C, block_keys [B, G, ceil(C/bs), di]); lengths: host list or
    CPU tensor, or an int32 [B] tensor on the GPU read by the kernels (a
    length outside 1 .. C then gives a zero row and sel -1) -> out
    [B, Hq, D] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    B, Hq, D = q.shape
    _, G, C, _ = k_cache.shape
    di = q_idx.shape[2]
    if k_cache.shape != (B, G, C, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, C, D]")
    if q_idx.shape != (B, G, di) or block_keys.shape != (B, G, -(-C // block_size), di):
        raise ValueError("q_idx must be [B, G, di] and block_keys [B, G, ceil(C/bs), di]")
    dims = _cache_dims(k_cache, block_size, top_k, Hq, di, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    ws, ws_bytes = _workspace(MSA_OP_DECODE, dims, dev, workspace)
    if _on_device(lengths, B, dev):
        _check(_lib.load().msa_decode_varlen_device(ctypes.byref(dims), _ptr(lengths), _ptr(q), _ptr(q_idx),
                                                    _ptr(k_cache), _ptr(v_cache), _ptr(block_keys), _ptr(out),
                                                    _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)),
               "msa_decode_varlen_device")
        return (out, sel) if return_sel else out
    _check(_lib.load().msa_decode_varlen(ctypes.byref(dims), _lengths(lengths, B), _ptr(q), _ptr(q_idx),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(block_keys), _ptr(out), _ptr(sel),
                                         _ptr(ws), ws_bytes, _stream(dev)), "msa_decode_varlen")
    return (out, sel) if return_sel else out


def msa_decode_init_varlen(k_idx, lengths, block_size: int, block_keys=None, open_sums=None):
    """msa_decode_init with each sequence's own cached length (host list or
    CPU tensor of B values in 0 .. C) -> (block_keys, open_sums)."""
    _need(k_idx, "k_idx", torch.int8, 4)
    dev = k_idx.device
    B, G, C, di = k_idx.shape
    nbc = -(-C // block_size)
    if block_keys is None:
        block_keys = torch.zeros((B, G, nbc, di), dtype=torch.int8, device=dev)
    if open_sums is None:
        open_sums = torch.zeros((B, G, di), dtype=torch.int32, device=dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    _need(open_sums, "open_sums", torch.int32, 3, dev)
    if block_keys.shape != (B, G, nbc, di) or open_sums.shape != (B, G, di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di] and open_sums [B, G, di]")
    dims = make_dims(B, C, G, G, block_size, 1, idx_dim=di)
    _check(_lib.load().msa_decode_init_varlen(ctypes.byref(dims), _lengths(lengths, B), _ptr(k_idx),
                                              _ptr(block_keys), _ptr(open_sums), _stream(dev)),
           "msa_decode_init_varlen")
    return block_keys, open_sums


def msa_decode_step_varlen(q, q_idx, k_new, v_new, k_idx_new, k_cache, v_cache, open_sums, block_keys, lengths,
                           block_size: int, top_k: int, softmax_scale: float = 0.0, out=None, sel=None,
                           return_sel: bool = False, workspace=None):
    """msa_decode_step with each sequence's own length (host list or CPU
    tensor, or an int32 [B] tensor on the GPU read by the kernels):
    sequence b's new token goes to row lengths[b] - 1 of its caches, then
    its query there is decoded -> out [B, Hq, D] bf16."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_new, "k_new", torch.bfloat16, 3, dev)
    _need(v_new, "v_new", torch.bfloat16, 3, dev)
    _need(k_idx_new, "k_idx_new", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(open_sums, "open_sums", torch.int32, 3, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    B, Hq, D = q.shape
    _, G, C, _ = k_cache.shape
    di = q_idx.shape[2]
    if k_cache.shape != (B, G, C, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, C, D]")
    if k_new.shape != (B, G, D) or v_new.shape != (B, G, D):
        raise ValueError("k_new/v_new must be [B, G, D]")
    if q_idx.shape != (B, G, di) or k_idx_new.shape != (B, G, di) or open_sums.shape != (B, G, di):
        raise ValueError("q_idx, k_idx_new and open_sums must be [B, G, di]")
    if block_keys.shape != (B, G, -(-C // block_size), di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di]")
    dims = _cache_dims(k_cache, block_size, top_k, Hq, di, softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    ws, ws_bytes = _workspace(MSA_OP_DECODE, dims, dev, workspace)
    if _on_device(lengths, B, dev):
        _check(_lib.load().msa_decode_step_varlen_device(ctypes.byref(dims), _ptr(lengths), _ptr(q), _ptr(q_idx),
                                                         _ptr(k_new), _ptr(v_new), _ptr(k_idx_new), _ptr(k_cache),
                                                         _ptr(v_cache), _ptr(open_sums), _ptr(block_keys),
                                                         _ptr(out), _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)),
               "msa_decode_step_varlen_device")
        return (out, sel) if return_sel else out
    _check(_lib.load().msa_decode_step_varlen(ctypes.byref(dims), _lengths(lengths, B), _ptr(q), _ptr(q_idx),
                                              _ptr(k_new), _ptr(v_new), _ptr(k_idx_new), _ptr(k_cache),
                                              _ptr(v_cache), _ptr(open_sums), _ptr(block_keys), _ptr(out),
                                              _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)), "msa_decode_step_varlen")
    return (out, sel) if return_sel else out


def msa_prefill_chunk(q, q_idx, k_cache, v_cache, k_idx, block_keys, start: int, block_size: int, top_k: int,
                      softmax_scale: float = 0.0, out=None, sel=None, return_sel: bool = False, workspace=None):
    """Prefill of the count = q.shape[1] queries at positions start .. start +
    count - 1 against caches of capacity C that already hold tokens 0 ..
    start + count - 1: k_cache/v_cache [B, G, C, D] bf16, k_idx [B, G, C, di]
    int8; block_keys [B, G, ceil(C/bs), di] int8 holds the summaries of the
    blocks before start / bs and receives those of the chunk's blocks.
    q [B, count, Hq, D], q_idx [B, G, count, di] -> out [B, count, Hq, D]."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 4, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(k_idx, "k_idx", torch.int8, 4, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    B, T, Hq, D = q.shape
    _, G, C, _ = k_cache.shape
    di = q_idx.shape[3]
    if k_cache.shape != (B, G, C, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, C, D]")
    if q_idx.shape != (B, G, T, di) or k_idx.shape != (B, G, C, di):
        raise ValueError("q_idx must be [B, G, count, di] and k_idx [B, G, C, di]")
    if block_keys.shape != (B, G, -(-C // block_size), di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di]")
    dims = make_dims(B, C, Hq, G, block_size, top_k, head_dim=D, idx_dim=di, softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4, dev)
    if sel is None and return_sel:
        sel = torch.empty((B, G, T, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 4, dev)
    lo, hi = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.load().msa_prefill_chunk_workspace_bytes(ctypes.byref(dims), int(T), ctypes.byref(lo),
                                                         ctypes.byref(hi)), "msa_prefill_chunk_workspace_bytes")
    ws, ws_bytes = _workspace(MSA_OP_PREFILL, dims, dev, workspace, sizes=(lo.value, hi.value))
    _check(_lib.load().msa_prefill_chunk(ctypes.byref(dims), int(start), int(T), _ptr(q), _ptr(q_idx),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(k_idx), _ptr(block_keys), _ptr(out),
                                         _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)), "msa_prefill_chunk")
    return (out, sel) if return_sel else out


def msa_prefill_chunk_varlen(q, q_idx, k_cache, v_cache, k_idx, block_keys, starts, counts, block_size: int,
                             top_k: int, softmax_scale: float = 0.0, out=None, sel=None, return_sel: bool = False,
                             workspace=None):
    """Each sequence b of the caches (k_cache/v_cache [B, G, C, D] bf16, k_idx
    [B, G, C, di] int8, block_keys [B, G, ceil(C/bs), di] int8) adds counts[b]
    queries at positions starts[b] .. starts[b] + counts[b] - 1; the queries
    are packed along the token axis in sequence order: q [T, Hq, D], q_idx
    [G, T, di] with T = sum(counts) -> out [T, Hq, D] bf16 (and sel [G, T,
    top_k] when return_sel).  starts, counts: host lists or CPU tensors."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(q_idx, "q_idx", torch.int8, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(k_idx, "k_idx", torch.int8, 4, dev)
    _need(block_keys, "block_keys", torch.int8, 4, dev)
    T, Hq, D = q.shape
    B, G, C, _ = k_cache.shape
    di = q_idx.shape[2]
    st = [int(x) for x in (starts.tolist() if isinstance(starts, torch.Tensor) else starts)]
    ct = [int(x) for x in (counts.tolist() if isinstance(counts, torch.Tensor) else counts)]
    if len(st) != B or len(ct) != B or sum(ct) != T:
        raise ValueError("starts and counts need one entry per sequence, and the counts must sum to q.shape[0]")
    if k_cache.shape != (B, G, C, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [B, G, C, D]")
    if q_idx.shape != (G, T, di) or k_idx.shape != (B, G, C, di):
        raise ValueError("q_idx must be [G, T, di] and k_idx [B, G, C, di]")
    if block_keys.shape != (B, G, -(-C // block_size), di):
        raise ValueError("block_keys must be [B, G, ceil(C/bs), di]")
    dims = make_dims(B, C, Hq, G, block_size, top_k, head_dim=D, idx_dim=di, softmax_scale=softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 3, dev)
    if sel is None and return_sel:
        sel = torch.empty((G, T, top_k), dtype=torch.int32, device=dev)
    if sel is not None:
        _need(sel, "sel", torch.int32, 3, dev)
    one = make_dims(1, C, Hq, G, block_size, top_k, head_dim=D, idx_dim=di, softmax_scale=softmax_scale)
    lo, hi = msa_prefill_chunk_workspace_bytes(one, max(1, max(ct)))
    ws, ws_bytes = _workspace(MSA_OP_PREFILL, dims, dev, workspace, sizes=(lo, hi))
    st_arr = (ctypes.c_int32 * B)(*st)
    ct_arr = (ctypes.c_int32 * B)(*ct)
    _check(_lib.load().msa_prefill_chunk_varlen(ctypes.byref(dims), st_arr, ct_arr, _ptr(q), _ptr(q_idx),
                                                _ptr(k_cache), _ptr(v_cache), _ptr(k_idx), _ptr(block_keys),
                                                _ptr(out), _ptr(sel), _ptr(ws), ws_bytes, _stream(dev)),
           "msa_prefill_chunk_varlen")
    return (out, sel) if return_sel else out
