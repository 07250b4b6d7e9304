"""Exact attention prefill for AMD MI355X (gfx950): thin Python binding.

The work is done by ``libattn_prefill.so`` (HIP kernels behind a C ABI, see
include/attn_prefill.h); this module only marshals torch tensors to it.  The
functions carry the C entry points' names:

* ``attn_prefill(q, k, v, cu_seqlens, mask="causal", scale=None, out=None)``
* ``attn_prefill_kv(q, k, v, cu_seqlens_q, cu_seqlens_k, mask="causal",
  scale=None, out=None, lse=False)`` -- queries that end a longer key
  sequence (chunked prefill, decode), optionally with the log-sum-exp
* ``attn_decode(q, k, v, cu_seqlens_k, mask="causal", scale=None, out=None,
  lse=False, workspace=None)`` -- one query per sequence over its cache
* ``attn_decode_noalloc(q, k, v, cu_seqlens_k, mask="causal", scale=None,
  out=None, lse=False)`` -- the same with the library's static device
  workspace (for callers that cannot allocate; calls on one GPU must not
  overlap)
* ``attn_prefill_check(...)``, ``attn_prefill_kv_check(...)``,
  ``attn_decode_workspace_size(...)``, ``attn_strerror(status)``,
  ``attn_version()``
* ``gdn_prefill(q, k, v, g, beta, cu_seqlens, scale=None, initial_state=None,
  out=None, final_state=False, workspace=None)`` -- chunked gated-delta-rule
  prefill (include/gdn_prefill.h), and ``gdn_prefill_workspace_size(...)``
* ``proj_dequantize_int8(q, scale, out=None)`` and ``proj_linear(x, w,
  out=None)`` -- int8 weights dequantized once to bf16, and y = x w^T by the
  vendor GEMM (include/proj.h)
* ``vision_attention_block(x, w_qkv, b_qkv, w_o, b_o, cu_seqlens, n_heads,
  mask="full", scale=None, out=None, workspace=None)`` -- QKV projection,
  attention and output projection in one call (include/vision_block.h), and
  ``vision_attention_block_workspace_size(...)``

There is no fallback: if the library is missing or cannot be loaded, the
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["attn_prefill", "attn_prefill_check", "attn_prefill_kv", "attn_prefill_kv_check",
           "attn_decode", "attn_decode_noalloc", "attn_decode_workspace_size", "attn_strerror",
           "attn_version",
           "gdn_prefill", "gdn_prefill_workspace_size", "proj_dequantize_int8", "proj_linear",
           "vision_attention_block", "vision_attention_block_workspace_size",
           "AttnError", "library_path", "load_library", "ATTN_OK", "ATTN_EINVAL",
           "ATTN_EUNSUPPORTED", "ATTN_ELAUNCH", "ATTN_BF16", "ATTN_F32", "ATTN_CAUSAL",
           "ATTN_FULL", "ATTN_WINDOW", "ATTN_DECODE_SCRATCH_BYTES"]

# values of include/attn_prefill.h
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ELAUNCH = 0, -1, -2, -3
ATTN_BF16, ATTN_F32 = 1, 2
ATTN_CAUSAL, ATTN_FULL, ATTN_WINDOW = 0, 1, 2
ATTN_DECODE_SCRATCH_BYTES = 16777216

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str = "attn_prefill"):
        self.status = status
        super().__init__(f"{what} failed: {attn_strerror(status)} (status {status})")


def library_path() -> str:
    return os.environ.get("ATTN_PREFILL_LIBRARY", os.path.join(_HERE, "libattn_prefill.so"))


def load_library() -> ctypes.CDLL:
    """Load the HIP library (after torch, so both share one HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  -- binds libamdhip64 before the library does

    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m long_context_attention_prefill_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.attn_prefill.argtypes = [vp, vp, vp, vp, ip, i32, i32, i32, i32, i32, i32, i32,
                                 ctypes.c_float, vp]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill_check.argtypes = [vp, vp, vp, vp, ip, i32, i32, i32, i32, i32, i32, i32,
                                       ctypes.c_float]
    lib.attn_prefill_check.restype = ctypes.c_int
    lib.attn_prefill_kv.argtypes = [vp, vp, vp, vp, vp, ip, ip, i32, i32, i32, i32, i32, i32,
                                    i32, ctypes.c_float, vp]
    lib.attn_prefill_kv.restype = ctypes.c_int
    lib.attn_prefill_kv_check.argtypes = [vp, vp, vp, vp, vp, ip, ip, i32, i32, i32, i32, i32,
                                          i32, i32, ctypes.c_float]
    lib.attn_prefill_kv_check.restype = ctypes.c_int
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, ip, i32, i32, i32, i32, i32, i32, i32,
                                ctypes.c_float, vp, ctypes.c_uint64, vp]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ip, i32, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_float, vp]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_workspace_size.argtypes = [ip, i32, i32, i32, i32, i32, i32, i32,
                                               ctypes.POINTER(ctypes.c_uint64)]
    lib.attn_decode_workspace_size.restype = ctypes.c_int
    fp = ctypes.c_void_p
    lib.gdn_prefill.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32, i32, i32, i32,
                                ctypes.c_float, vp, ctypes.c_uint64, vp]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_prefill_check.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, ip, i32, i32, i32, i32,
                                      i32, ctypes.c_float, vp, ctypes.c_uint64]
    lib.gdn_prefill_check.restype = ctypes.c_int
    lib.gdn_prefill_workspace_size.argtypes = [ip, i32, i32, i32, i32, i32,
                                               ctypes.POINTER(ctypes.c_uint64)]
    lib.gdn_prefill_workspace_size.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.proj_dequantize_int8.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.proj_dequantize_int8.restype = ctypes.c_int
    lib.proj_linear.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.proj_linear.restype = ctypes.c_int
    f32, u64 = ctypes.c_float, ctypes.c_uint64
    lib.vision_attention_block.argtypes = [vp, vp, vp, vp, vp, vp, ip, i32, i32, i32, i32, i32, i32,
                                           i32, f32, vp, u64, vp]
    lib.vision_attention_block.restype = ctypes.c_int
    lib.vision_attention_block_workspace_size.argtypes = [i64, i32, i32, i32, i32,
                                                          ctypes.POINTER(u64)]
    lib.vision_attention_block_workspace_size.restype = ctypes.c_int
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(int(status)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


def _mask_args(mask):
    if mask == "causal":
        return ATTN_CAUSAL, 0
    if mask == "full":
        return ATTN_FULL, 0
    if isinstance(mask, (tuple, list)) and len(mask) == 2 and mask[0] == "window":
        return ATTN_WINDOW, int(mask[1])
    raise ValueError(f"mask must be 'causal', 'full' or ('window', W), not {mask!r}")


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _cu_array(cu_seqlens):
    vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    arr = (ctypes.c_int32 * max(len(vals), 1))(*vals)
    return arr, len(vals) - 1


def _stream_of(stream, device):
    """The torch stream a call's kernels run on: ``stream`` (a torch stream or
    a raw hipStream_t handle), else torch's current stream.  Tensors a call
    allocates (outputs, workspaces) are allocated on this stream, so the
    caching allocator never hands their memory to other work before the
    call's kernels are done with it."""
    import torch

    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = int(stream)
    if handle == 0:
        return torch.cuda.default_stream(device)
    return torch.cuda.ExternalStream(handle, device=device)


def _args(q, k, v, out, cu_seqlens, mask, scale):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [T, Hq, d]; k and v [T, Hkv, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("q, k, v shapes disagree")
    if out.shape != q.shape or out.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v and out must share dtype; out must have q's shape")
    kind, window = _mask_args(mask)
    d = int(q.shape[2])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu, n_seqs = _cu_array(cu_seqlens)
    if n_seqs >= 0 and int(cu[n_seqs]) != q.shape[0]:
        raise ValueError("cu_seqlens[-1] must equal the number of packed tokens")
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu, n_seqs,
            int(q.shape[1]), int(k.shape[1]), d, _dtype_code(q), kind, window, float(scale))


def attn_prefill(q, k, v, cu_seqlens, mask="causal", scale=None, out=None, stream=None):
    """Exact attention over a packed batch; returns ``out`` ([T, Hq, d], q's dtype).

    q: [T, Hq, d], k/v: [T, Hkv, d] contiguous device tensors (bf16 or fp32);
    cu_seqlens: host sequence of n_seqs+1 ints; mask: "causal", "full" or
    ("window", W); scale defaults to 1/sqrt(d).  Runs on ``stream`` (default:
    torch's current stream) and returns without synchronising.
    """
    import torch

    lib = load_library()
    st = _stream_of(stream, q.device)
    if out is None:
        with torch.cuda.stream(st):
            out = torch.empty_like(q)
    a = _args(q, k, v, out, cu_seqlens, mask, scale)
    status = lib.attn_prefill(*a, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status)
    return out


def attn_prefill_check(q, k, v, cu_seqlens, mask="causal", scale=None, out=None) -> int:
    """Status attn_prefill would return for these arguments (host-only)."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    a = _args(q, k, v, out, cu_seqlens, mask, scale)
    return int(load_library().attn_prefill_check(*a))


def _args_kv(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, mask, scale):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [Tq, Hq, d]; k and v [Tk, Hkv, d]")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q, k, v shapes disagree")
    if out.shape != q.shape or out.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v and out must share dtype; out must have q's shape")
    if lse is not None:
        import torch

        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:2]) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [Tq, Hq] tensor")
    kind, window = _mask_args(mask)
    d = int(q.shape[2])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu_q, n_q = _cu_array(cu_seqlens_q)
    cu_k, n_k = _cu_array(cu_seqlens_k)
    if n_q != n_k:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if n_q >= 0 and (int(cu_q[n_q]) != q.shape[0] or int(cu_k[n_k]) != k.shape[0]):
        raise ValueError("cu_seqlens_q[-1] must equal Tq and cu_seqlens_k[-1] must equal Tk")
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(), cu_q, cu_k, n_q, int(q.shape[1]),
            int(k.shape[1]), d, _dtype_code(q), kind, window, float(scale))


def attn_prefill_kv(q, k, v, cu_seqlens_q, cu_seqlens_k, mask="causal", scale=None, out=None,
                    lse=False, stream=None):
    """Exact attention of queries that end longer key sequences.

    q: [Tq, Hq, d], k/v: [Tk, Hkv, d]; sequence b has its last
    cu_seqlens_q[b+1]-cu_seqlens_q[b] positions as queries over
    cu_seqlens_k[b+1]-cu_seqlens_k[b] keys.  ``lse``: False (not computed),
    True (allocated and returned) or a float32 [Tq, Hq] tensor to fill.
    Returns ``out``, or ``(out, lse)`` when lse is requested.
    """
    import torch

    lib = load_library()
    st = _stream_of(stream, q.device)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty_like(q)
        lse_t = None
        if lse is True:
            lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        elif lse is not False and lse is not None:
            lse_t = lse
    a = _args_kv(q, k, v, out, lse_t, cu_seqlens_q, cu_seqlens_k, mask, scale)
    status = lib.attn_prefill_kv(*a, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_prefill_kv")
    return out if lse_t is None else (out, lse_t)


def attn_prefill_kv_check(q, k, v, cu_seqlens_q, cu_seqlens_k, mask="causal", scale=None,
                          out=None, lse=None) -> int:
    """Status attn_prefill_kv would return for these arguments (host-only)."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    a = _args_kv(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, mask, scale)
    return int(load_library().attn_prefill_kv_check(*a))


def attn_decode_workspace_size(cu_seqlens_k, n_q_heads, n_kv_heads, head_dim, dtype=ATTN_BF16,
                               mask="causal") -> int:
    """Workspace bytes attn_decode needs for this shape (host-only)."""
    kind, window = _mask_args(mask)
    cu, n = _cu_array(cu_seqlens_k)
    out = ctypes.c_uint64(0)
    status = load_library().attn_decode_workspace_size(cu, n, int(n_q_heads), int(n_kv_heads),
                                                       int(head_dim), int(dtype), kind, window,
                                                       ctypes.byref(out))
    if status != ATTN_OK:
        raise AttnError(status, "attn_decode_workspace_size")
    return int(out.value)


def attn_decode(q, k, v, cu_seqlens_k, mask="causal", scale=None, out=None, lse=False,
                workspace=None, stream=None):
    """Attention of each sequence's newest token (row b of q) over its cache.

    q: [n_seqs, Hq, d]; k/v: [Tk, Hkv, d] packed by cu_seqlens_k (host ints,
    every sequence non-empty).  ``workspace``: a device tensor of at least
    attn_decode_workspace_size(...) bytes, or None to allocate one here.
    ``lse`` as for attn_prefill_kv.  Returns ``out`` or ``(out, lse)``.
    """
    import torch

    lib = load_library()
    st = _stream_of(stream, q.device)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty_like(q)
        lse_t = None
        if lse is True:
            lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        elif lse is not False and lse is not None:
            lse_t = lse
    n = q.shape[0]
    cu_q = list(range(n + 1))
    a = _args_kv(q, k, v, out, lse_t, cu_q, cu_seqlens_k, mask, scale)
    qp, kp, vp_, op, lp, _, cu_k, n_seqs, hq, hkv, d, dt, kind, window, sc = a
    if workspace is None:
        need = attn_decode_workspace_size(cu_seqlens_k, hq, hkv, d, dt, mask)
        if need > 0:
            with torch.cuda.stream(st):
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib.attn_decode(qp, kp, vp_, op, lp, cu_k, n_seqs, hq, hkv, d, dt, kind, window, sc,
                             ws_ptr, ws_bytes, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_decode")
    return out if lse_t is None else (out, lse_t)


def attn_decode_noalloc(q, k, v, cu_seqlens_k, mask="causal", scale=None, out=None, lse=False,
                        stream=None):
    """attn_decode without a workspace argument: the library's static device
    array serves as the workspace (include/attn_prefill.h).  Pass ``out``
    (and an ``lse`` tensor) to keep the call free of allocations."""
    import torch

    lib = load_library()
    st = _stream_of(stream, q.device)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty_like(q)
        lse_t = None
        if lse is True:
            lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        elif lse is not False and lse is not None:
            lse_t = lse
    n = q.shape[0]
    a = _args_kv(q, k, v, out, lse_t, list(range(n + 1)), cu_seqlens_k, mask, scale)
    qp, kp, vp_, op, lp, _, cu_k, n_seqs, hq, hkv, d, dt, kind, window, sc = a
    status = lib.attn_decode_noalloc(qp, kp, vp_, op, lp, cu_k, n_seqs, hq, hkv, d, dt, kind, window,
                                     sc, ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "attn_decode_noalloc")
    return out if lse_t is None else (out, lse_t)


def gdn_prefill_workspace_size(cu_seqlens, n_heads, head_dim_k=128, head_dim_v=128,
                               dtype=ATTN_BF16) -> int:
    """Workspace bytes gdn_prefill needs for this shape (host-only)."""
    cu, n = _cu_array(cu_seqlens)
    out = ctypes.c_uint64(0)
    status = load_library().gdn_prefill_workspace_size(cu, n, int(n_heads), int(head_dim_k),
                                                       int(head_dim_v), int(dtype),
                                                       ctypes.byref(out))
    if status != ATTN_OK:
        raise AttnError(status, "gdn_prefill_workspace_size")
    return int(out.value)


def gdn_prefill(q, k, v, g, beta, cu_seqlens, scale=None, initial_state=None, out=None,
                final_state=False, workspace=None, stream=None):
    """Chunked gated-delta-rule prefill over a packed batch.

    q, k: [T, H, dk] bf16; v: [T, H, dv] bf16; g (log decay) and beta:
    [T, H] float32; initial_state: None or float32 [n_seqs, H, dv, dk].
    ``final_state``: False (not computed), True (allocated and returned) or a
    float32 tensor to fill (may be ``initial_state`` itself, updated in
    place).  ``workspace``: a device tensor of at least
    gdn_prefill_workspace_size(...) bytes, or None to allocate one here.
    Returns ``out`` or ``(out, final_state)``.
    """
    import torch

    lib = load_library()
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [T, H, dk] and v [T, H, dv]")
    T, H, dk = (int(x) for x in q.shape)
    dv = int(v.shape[2])
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if tuple(g.shape) != (T, H) or tuple(beta.shape) != (T, H):
        raise ValueError("g and beta must be [T, H]")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise ValueError("g and beta must be float32")
    cu, n = _cu_array(cu_seqlens)
    if n >= 0 and int(cu[n]) != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    st = _stream_of(stream, q.device)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty_like(v)
        fin = None
        if final_state is True:
            fin = torch.empty((max(n, 0), H, dv, dk), dtype=torch.float32, device=q.device)
        elif final_state is not False and final_state is not None:
            fin = final_state
    for name, t in (("initial_state", initial_state), ("final_state", fin)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (n, H, dv, dk)
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [n_seqs, H, dv, dk] tensor")
    if workspace is None:
        need = gdn_prefill_workspace_size(cu_seqlens, H, dk, dv, _dtype_code(q))
        if need > 0:
            with torch.cuda.stream(st):
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    handle = st.cuda_stream
    status = lib.gdn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                             beta.data_ptr(),
                             None if initial_state is None else initial_state.data_ptr(),
                             out.data_ptr(), None if fin is None else fin.data_ptr(), cu, n, H,
                             dk, dv, _dtype_code(q), float(1.0 / math.sqrt(dk) if scale is None
                                                           else scale),
                             ws_ptr, ws_bytes, ctypes.c_void_p(handle))
    if status != ATTN_OK:
        raise AttnError(status, "gdn_prefill")
    return out if fin is None else (out, fin)


def _handle(stream, device):
    return ctypes.c_void_p(_stream_of(stream, device).cuda_stream)


def proj_dequantize_int8(q, scale, out=None, stream=None):
    """bf16 weights w[n][k] = scale[n] * q[n][k] from int8 q [N, K] and float32 scale [N]."""
    import torch

    if q.dim() != 2 or q.dtype != torch.int8 or not q.is_contiguous():
        raise ValueError("q must be a contiguous int8 [N, K] tensor")
    if scale.dtype != torch.float32 or tuple(scale.shape) != (q.shape[0],) or not scale.is_contiguous():
        raise ValueError("scale must be a contiguous float32 [N] tensor")
    if out is None:
        with torch.cuda.stream(_stream_of(stream, q.device)):
            out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor of q's shape")
    status = load_library().proj_dequantize_int8(q.data_ptr(), scale.data_ptr(), out.data_ptr(),
                                                 int(q.shape[0]), int(q.shape[1]),
                                                 _handle(stream, q.device))
    if status != ATTN_OK:
        raise AttnError(status, "proj_dequantize_int8")
    return out


def proj_linear(x, w, out=None, stream=None):
    """y = x w^T: x bf16 [T, K], w bf16 [N, K] -> y bf16 [T, N] (vendor GEMM, fp32 accumulation)."""
    import torch

    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T, K] and w [N, K]")
    for name, t in (("x", x), ("w", w)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
    T, K = (int(s) for s in x.shape)
    N = int(w.shape[0])
    if out is None:
        with torch.cuda.stream(_stream_of(stream, x.device)):
            out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (T, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [T, N] tensor")
    status = load_library().proj_linear(x.data_ptr(), w.data_ptr(), out.data_ptr(), T, N, K,
                                        _handle(stream, x.device))
    if status != ATTN_OK:
        raise AttnError(status, "proj_linear")
    return out


def vision_attention_block_workspace_size(tokens, n_heads, head_dim, hidden, dtype=ATTN_BF16) -> int:
    """Workspace bytes vision_attention_block needs for ``tokens`` packed tokens."""
    out = ctypes.c_uint64(0)
    status = load_library().vision_attention_block_workspace_size(int(tokens), int(n_heads), int(head_dim),
                                                                  int(hidden), int(dtype), ctypes.byref(out))
    if status != ATTN_OK:
        raise AttnError(status, "vision_attention_block_workspace_size")
    return int(out.value)


def vision_attention_block(x, w_qkv, b_qkv, w_o, b_o, cu_seqlens, n_heads, mask="full", scale=None,
                           out=None, workspace=None, stream=None):
    """out = attention(x W_qkv^T + b_qkv) W_o^T + b_o over packed images.

    x [T, hidden]; w_qkv [3 H d, hidden] (q, k, v row blocks, heads contiguous);
    b_qkv [3 H d]; w_o [hidden, H d]; b_o [hidden]; all contiguous, one dtype
    (bf16 or fp32).  cu_seqlens: host sequence of n_images+1 ints; mask "full",
    "causal" or ("window", W); scale defaults to 1/sqrt(d).  A workspace tensor
    (uint8, at least vision_attention_block_workspace_size bytes) is allocated
    when none is given.
    """
    import torch

    if x.dim() != 2 or w_qkv.dim() != 2 or w_o.dim() != 2 or b_qkv.dim() != 1 or b_o.dim() != 1:
        raise ValueError("x, w_qkv, w_o must be 2-d and the biases 1-d")
    T, hidden = (int(s) for s in x.shape)
    H = int(n_heads)
    if H <= 0 or w_qkv.shape[0] % (3 * H) != 0:
        raise ValueError("w_qkv must have 3 * n_heads * head_dim rows")
    d = int(w_qkv.shape[0]) // (3 * H)
    if tuple(w_qkv.shape) != (3 * H * d, hidden) or tuple(b_qkv.shape) != (3 * H * d,) \
            or tuple(w_o.shape) != (hidden, H * d) or tuple(b_o.shape) != (hidden,):
        raise ValueError("weight shapes disagree with x and n_heads")
    st = _stream_of(stream, x.device)
    if out is None:
        with torch.cuda.stream(st):
            out = torch.empty_like(x)
    for name, t in (("x", x), ("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o), ("out", out)):
        if t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous and of x's dtype")
    if tuple(out.shape) != (T, hidden):
        raise ValueError("out must be [T, hidden]")
    kind, window = _mask_args(mask)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(x)
    cu, n_seqs = _cu_array(cu_seqlens)
    if n_seqs >= 0 and int(cu[n_seqs]) != T:
        raise ValueError("cu_seqlens[-1] must equal the number of packed tokens")
    if workspace is None:
        need = vision_attention_block_workspace_size(T, H, d, hidden, code)
        with torch.cuda.stream(st):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    status = load_library().vision_attention_block(
        x.data_ptr(), w_qkv.data_ptr(), b_qkv.data_ptr(), w_o.data_ptr(), b_o.data_ptr(), out.data_ptr(),
        cu, n_seqs, H, d, hidden, code, kind, window, float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), ctypes.c_void_p(st.cuda_stream))
    if status != ATTN_OK:
        raise AttnError(status, "vision_attention_block")
    return out
