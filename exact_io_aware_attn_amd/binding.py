"""ctypes binding of libmiattn.so (the C ABI in include/miattn.h).

Argument marshalling only: tensors become device pointers and element
strides, outputs and the workspace are allocated with torch when the caller
does not pass them, and the call is enqueued on torch's current stream. Every
step of the computation runs in the library's HIP kernels. If the library is
not built, or there is no GPU, the calls raise; there is no fallback.
"""

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmiattn.so")

MIATTN_BF16, MIATTN_F32 = 0, 1
MIATTN_MASK_NONE, MIATTN_MASK_CAUSAL, MIATTN_MASK_BLOCK = 0, 1, 2
SOFTMAX_MODES = {"online": 0, "fixed_max": 1, "fixed_max_centered": 2}

_EXPORTS = ("attn_fwd", "attn_fwd_workspace_bytes", "attn_decode", "attn_decode_noalloc",
            "attn_decode_workspace_bytes", "attn_decode_multi",
            "attn_decode_multi_workspace_bytes", "attn_decode_paged", "attn_bwd",
            "attn_bwd_workspace_bytes",
            "attn_status_str")


class MiattnError(RuntimeError):
    def __init__(self, status, fn):
        self.status = int(status)
        super().__init__(f"{fn} failed with status {status}: {attn_status_str(status)}")


class _Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64)]


_lib = None


def library():
    """Load libmiattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_io_aware_attn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_str.argtypes = [I]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I, I]
    lib.attn_fwd_workspace_bytes.restype = Z
    lib.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, I, I, I,
                             ctypes.POINTER(_Strides), P, Z, P]
    lib.attn_fwd.restype = I
    lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_workspace_bytes.restype = Z
    lib.attn_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I,
                                ctypes.POINTER(_Strides), P, Z, P]
    lib.attn_decode.restype = I
    lib.attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I,
                                        ctypes.POINTER(_Strides), P]
    lib.attn_decode_noalloc.restype = I
    lib.attn_decode_multi_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_decode_multi_workspace_bytes.restype = Z
    lib.attn_decode_multi.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I,
                                      ctypes.POINTER(_Strides), P, Z, P]
    lib.attn_decode_multi.restype = I
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I,
                                      ctypes.POINTER(_Strides), P, Z, P]
    lib.attn_decode_paged.restype = I
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.attn_bwd_workspace_bytes.restype = Z
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, I, I,
                             ctypes.POINTER(_Strides), P, Z, P]
    lib.attn_bwd.restype = I
    _lib = lib
    return lib


def attn_status_str(status):
    """Static description of a status code returned by the library."""
    return library().attn_status_str(int(status)).decode()


def attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, mask_kind, block_q, block_k, softmax_mode):
    """Workspace bytes attn_fwd needs for these arguments (0 for the plain online mode)."""
    return int(library().attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, mask_kind, block_q,
                                                  block_k, softmax_mode))


def attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d, kv_splits=0):
    """Workspace bytes attn_decode needs (the split-K partial results)."""
    return int(library().attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d, kv_splits))


def attn_decode_multi_workspace_bytes(B, n_new, Hq, Hkv, max_len, d, kv_splits=0):
    """Workspace bytes attn_decode_multi and attn_decode_paged need."""
    return int(library().attn_decode_multi_workspace_bytes(B, n_new, Hq, Hkv, max_len, d,
                                                           kv_splits))


def attn_bwd_workspace_bytes(B, Hq, Nq):
    """Workspace bytes attn_bwd needs (per-row statistics of the backward pass)."""
    return int(library().attn_bwd_workspace_bytes(B, Hq, Nq))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MIATTN_BF16
    if t.dtype == torch.float32:
        return MIATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_gpu(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.device != dev:
            raise ValueError("tensors must be on one device")


def _strides4(t):
    sb, ss, sh, sd = t.stride()
    if sd != 1 and t.shape[3] > 1:
        raise ValueError("the last (head) dimension must be contiguous")
    return _Strides(sb, ss, sh)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _fwd_setup(q, k, v, causal, block_mask, block, scale, softmax, return_lse, out, lse_out,
               workspace):
    """Validate, allocate what the caller did not pass, and marshal the C
    arguments of attn_fwd. Returns (args, o, lse, keep): keep holds every
    object the arguments point into."""
    _check_gpu(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Nq,Hq,d]; k and v [B,Nk,Hkv,d]")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share a dtype")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    mode = SOFTMAX_MODES[softmax]
    mask_kind = MIATTN_MASK_CAUSAL if causal else MIATTN_MASK_NONE
    bm = None
    bq = bk = 0
    if block_mask is not None:
        mask_kind |= MIATTN_MASK_BLOCK
        bq, bk = block
        if isinstance(block_mask, np.ndarray):
            block_mask = torch.from_numpy(np.ascontiguousarray(block_mask, dtype=np.uint8))
        bm = block_mask.to(device=dev, dtype=torch.uint8).contiguous()
    o = torch.empty_like(q) if out is None else out
    _check_gpu(o)
    lse = None
    if return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    need = attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, mask_kind, bq, bk, mode)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = (_Strides * 4)(_strides4(q), _strides4(k), _strides4(v), _strides4(o))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), B, Hq, Hkv, Nq, Nk, d,
            scale, mask_kind, _ptr(bm), bq, bk, mode, st, _ptr(workspace), ws_bytes, _stream(dev))
    return args, o, lse, (q, k, v, o, lse, bm, workspace, st)


def attn_fwd(q, k, v, *, causal=False, block_mask=None, block=None, scale=None,
             softmax="online", return_lse=True, out=None, lse_out=None, workspace=None):
    """Exact attention of q [B,Nq,Hq,d] against k, v [B,Nk,Hkv,d] (GPU tensors,
    bf16 or fp32). block_mask: uint8 [Nq/bq, Nk/bk] (GPU tensor or array),
    block = (bq, bk). Returns (o, lse) with lse [B,Hq,Nq] fp32 (or None)."""
    args, o, lse, _ = _fwd_setup(q, k, v, causal, block_mask, block, scale, softmax, return_lse,
                                 out, lse_out, workspace)
    rc = library().attn_fwd(*args)
    if rc != 0:
        raise MiattnError(rc, "attn_fwd")
    return o, lse


def fixed_max_decisions(workspace, B, Hq, Hkv, Nq, Nk):
    """The per-row choices attn_fwd recorded in a fixed-max call's workspace
    (the layout include/miattn.h documents): a uint8 [B, Hq, Nq] view, 1 where
    the row took the fixed max, 0 where it fell back to the running max."""
    off = (B * Hkv * Nk * 4 + 255) // 256 * 256
    return workspace[off:off + B * Hq * Nq].view(B, Hq, Nq)


class PreparedCall:
    """One entry point with its C arguments marshalled once: calling it
    enqueues the same work again (same tensors, the stream current when it
    was prepared) with a single foreign call. The tensors it was prepared
    with must stay alive and keep their storage."""

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            raise MiattnError(rc, self._name)


def prepare_fwd(q, k, v, *, causal=False, block_mask=None, block=None, scale=None,
                softmax="online", return_lse=True, out=None, lse_out=None, workspace=None):
    """attn_fwd as a PreparedCall: returns (call, o, lse); every call() writes
    o (and lse) again."""
    args, o, lse, keep = _fwd_setup(q, k, v, causal, block_mask, block, scale, softmax,
                                    return_lse, out, lse_out, workspace)
    return PreparedCall(library().attn_fwd, args, "attn_fwd", keep), o, lse


def _decode_setup(q, k_cache, v_cache, seqlens, scale, kv_splits, return_lse, out, lse_out,
                  workspace):
    _check_gpu(q, k_cache, v_cache, seqlens)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,d]; caches [B,max_len,Hkv,d]")
    if seqlens.dtype != torch.int32:
        raise TypeError("seqlens must be int32")
    B, Hq, d = q.shape
    _, max_len, Hkv, _ = k_cache.shape
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q = q.contiguous()
    seqlens = seqlens.contiguous()
    o = torch.empty_like(q) if out is None else out
    lse = None
    if return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    need = attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d, kv_splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = (_Strides * 2)(_strides4(k_cache), _strides4(v_cache))
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse),
            _dtype_code(q), B, Hq, Hkv, max_len, d, scale, kv_splits, st, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    return args, o, lse, (q, k_cache, v_cache, seqlens, o, lse, workspace, st)


def attn_decode(q, k_cache, v_cache, seqlens, *, scale=None, kv_splits=0, return_lse=True,
                out=None, lse_out=None, workspace=None):
    """Decode attention: q [B,Hq,d] bf16 against caches [B,max_len,Hkv,d] bf16 with
    seqlens int32 [B] (all GPU tensors). Returns (o [B,Hq,d], lse [B,Hq] or None)."""
    args, o, lse, _ = _decode_setup(q, k_cache, v_cache, seqlens, scale, kv_splits, return_lse,
                                    out, lse_out, workspace)
    rc = library().attn_decode(*args)
    if rc != 0:
        raise MiattnError(rc, "attn_decode")
    return o, lse


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse=None, *, scale=None, kv_splits=0):
    """attn_decode through the entry point that allocates nothing: the caller
    passes the outputs o [B,Hq,d] bf16 and (optionally) lse [B,Hq] fp32; the
    split-K partials go to the library's static per-device scratch. q must be
    contiguous [B,Hq,d] and seqlens contiguous int32 [B]. Nothing is allocated
    here either. Returns (o, lse)."""
    _check_gpu(q, k_cache, v_cache, seqlens, o)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,Hq,d]; caches [B,max_len,Hkv,d]")
    if not q.is_contiguous() or not o.is_contiguous() or not seqlens.is_contiguous():
        raise ValueError("q, o and seqlens must be contiguous")
    if seqlens.dtype != torch.int32:
        raise TypeError("seqlens must be int32")
    B, Hq, d = q.shape
    _, max_len, Hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = (_Strides * 2)(_strides4(k_cache), _strides4(v_cache))
    rc = library().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
                                       _ptr(o), _ptr(lse), _dtype_code(q), B, Hq, Hkv, max_len,
                                       d, scale, kv_splits, st, _stream(q.device))
    if rc != 0:
        raise MiattnError(rc, "attn_decode_noalloc")
    return o, lse


def prepare_decode(q, k_cache, v_cache, seqlens, *, scale=None, kv_splits=0, return_lse=True,
                   out=None, lse_out=None, workspace=None):
    """attn_decode as a PreparedCall: returns (call, o, lse)."""
    args, o, lse, keep = _decode_setup(q, k_cache, v_cache, seqlens, scale, kv_splits,
                                       return_lse, out, lse_out, workspace)
    return PreparedCall(library().attn_decode, args, "attn_decode", keep), o, lse


def _bwd_setup(q, k, v, o, lse, dout, causal, block_mask, block, scale, dq, dk, dv, workspace):
    _check_gpu(q, k, v, o, lse, dout)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape \
            or dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B,Nq,Hq,d]; k and v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if lse.shape != (B, Hq, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B,Hq,Nq]")
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lse = lse.contiguous()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_gpu(dq, dk, dv)
    need = attn_bwd_workspace_bytes(B, Hq, Nq)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = (_Strides * 8)(*[_strides4(t) for t in (q, k, v, o, dout, dq, dk, dv)])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    mask_kind = MIATTN_MASK_CAUSAL if causal else MIATTN_MASK_NONE
    bm = None
    bq = bk = 0
    if block_mask is not None:
        mask_kind |= MIATTN_MASK_BLOCK
        bq, bk = block
        if isinstance(block_mask, np.ndarray):
            block_mask = torch.from_numpy(np.ascontiguousarray(block_mask, dtype=np.uint8))
        bm = block_mask.to(device=dev, dtype=torch.uint8).contiguous()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
            _ptr(dv), _dtype_code(q), B, Hq, Hkv, Nq, Nk, d, scale, mask_kind, _ptr(bm), bq, bk,
            st, _ptr(workspace), ws_bytes, _stream(dev))
    return args, (dq, dk, dv), (q, k, v, o, lse, dout, dq, dk, dv, bm, workspace, st)


def attn_bwd(q, k, v, o, lse, dout, *, causal=False, block_mask=None, block=None, scale=None,
             dq=None, dk=None, dv=None, workspace=None):
    """Gradients of attention with respect to q, k, v (bf16 GPU tensors) for the
    upstream gradient dout, given the forward's o and lse [B,Hq,Nq] (float32) and
    the forward's mask. Returns (dq, dk, dv)."""
    args, grads, _ = _bwd_setup(q, k, v, o, lse, dout, causal, block_mask, block, scale, dq, dk,
                                dv, workspace)
    rc = library().attn_bwd(*args)
    if rc != 0:
        raise MiattnError(rc, "attn_bwd")
    return grads


def prepare_bwd(q, k, v, o, lse, dout, *, causal=False, block_mask=None, block=None, scale=None,
                dq=None, dk=None, dv=None, workspace=None):
    """attn_bwd as a PreparedCall: returns (call, (dq, dk, dv))."""
    args, grads, keep = _bwd_setup(q, k, v, o, lse, dout, causal, block_mask, block, scale, dq,
                                   dk, dv, workspace)
    return PreparedCall(library().attn_bwd, args, "attn_bwd", keep), grads


def _decode_multi_setup(q, k_cache, v_cache, seqlens, scale, kv_splits, return_lse, out,
                        lse_out, workspace):
    _check_gpu(q, k_cache, v_cache, seqlens)
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,n_new,Hq,d]; caches [B,max_len,Hkv,d]")
    if seqlens.dtype != torch.int32:
        raise TypeError("seqlens must be int32")
    B, nt, Hq, d = q.shape
    _, max_len, Hkv, _ = k_cache.shape
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q = q.contiguous()
    seqlens = seqlens.contiguous()
    o = torch.empty_like(q) if out is None else out
    lse = None
    if return_lse:
        lse = torch.empty((B, nt, Hq), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    need = attn_decode_multi_workspace_bytes(B, nt, Hq, Hkv, max_len, d, kv_splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = (_Strides * 2)(_strides4(k_cache), _strides4(v_cache))
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse),
            _dtype_code(q), B, nt, Hq, Hkv, max_len, d, scale, kv_splits, st, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    return args, o, lse, (q, k_cache, v_cache, seqlens, o, lse, workspace, st)


def attn_decode_multi(q, k_cache, v_cache, seqlens, *, scale=None, kv_splits=0, return_lse=True,
                      out=None, lse_out=None, workspace=None):
    """Decode of n_new tokens per sequence: q [B,n_new,Hq,d] bf16 against caches
    [B,max_len,Hkv,d] whose last seqlens[b] rows include the new tokens' own keys.
    Returns (o [B,n_new,Hq,d], lse [B,n_new,Hq] or None)."""
    args, o, lse, _ = _decode_multi_setup(q, k_cache, v_cache, seqlens, scale, kv_splits,
                                          return_lse, out, lse_out, workspace)
    rc = library().attn_decode_multi(*args)
    if rc != 0:
        raise MiattnError(rc, "attn_decode_multi")
    return o, lse


def prepare_decode_multi(q, k_cache, v_cache, seqlens, *, scale=None, kv_splits=0,
                         return_lse=True, out=None, lse_out=None, workspace=None):
    """attn_decode_multi as a PreparedCall: returns (call, o, lse)."""
    args, o, lse, keep = _decode_multi_setup(q, k_cache, v_cache, seqlens, scale, kv_splits,
                                             return_lse, out, lse_out, workspace)
    return PreparedCall(library().attn_decode_multi, args, "attn_decode_multi", keep), o, lse


def _decode_paged_setup(q, k_pages, v_pages, block_table, seqlens, scale, kv_splits, return_lse,
                        out, lse_out, workspace):
    _check_gpu(q, k_pages, v_pages, block_table, seqlens)
    if q.dim() == 3:
        q = q[:, None]
    if q.dim() != 4 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B,n_new,Hq,d] (or [B,Hq,d]); pages [num_pages,page_size,Hkv,d]")
    if seqlens.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise TypeError("seqlens and block_table must be int32")
    B, nt, Hq, d = q.shape
    _, page_size, Hkv, _ = k_pages.shape
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    max_pages = block_table.shape[1]
    dev = q.device
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q = q.contiguous()
    seqlens = seqlens.contiguous()
    block_table = block_table.contiguous()
    o = torch.empty_like(q) if out is None else out
    lse = None
    if return_lse:
        lse = torch.empty((B, nt, Hq), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    need = attn_decode_multi_workspace_bytes(B, nt, Hq, Hkv, page_size * max_pages, d, kv_splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = (_Strides * 2)(_strides4(k_pages), _strides4(v_pages))
    args = (_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens), _ptr(o),
            _ptr(lse), _dtype_code(q), B, nt, Hq, Hkv, page_size, max_pages, d, scale, kv_splits,
            st, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    return args, o, lse, (q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, st)


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens, *, scale=None, kv_splits=0,
                      return_lse=True, out=None, lse_out=None, workspace=None):
    """Decode against a paged cache: q [B,n_new,Hq,d] (or [B,Hq,d]) bf16, pages
    [num_pages,page_size,Hkv,d] bf16, block_table int32 [B,max_pages], seqlens int32
    [B]. Returns (o [B,n_new,Hq,d], lse [B,n_new,Hq] or None)."""
    args, o, lse, _ = _decode_paged_setup(q, k_pages, v_pages, block_table, seqlens, scale,
                                          kv_splits, return_lse, out, lse_out, workspace)
    rc = library().attn_decode_paged(*args)
    if rc != 0:
        raise MiattnError(rc, "attn_decode_paged")
    return o, lse


def prepare_decode_paged(q, k_pages, v_pages, block_table, seqlens, *, scale=None, kv_splits=0,
                         return_lse=True, out=None, lse_out=None, workspace=None):
    """attn_decode_paged as a PreparedCall: returns (call, o, lse)."""
    args, o, lse, keep = _decode_paged_setup(q, k_pages, v_pages, block_table, seqlens, scale,
                                             kv_splits, return_lse, out, lse_out, workspace)
    return PreparedCall(library().attn_decode_paged, args, "attn_decode_paged", keep), o, lse
