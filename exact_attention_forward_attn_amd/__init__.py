"""Exact attention forward on MI355X (gfx950): Python binding of libattn.so.

The binding only marshals arguments: it checks tensor shapes, dtypes and
devices, takes device pointers and the current HIP stream from PyTorch, and
calls the C ABI declared in ``include/attn.h``. Every step of the attention
computation runs in the HIP kernels of ``libattn.so``; there is no fallback
path, and a missing library raises instead of computing anything elsewhere.

Functions (same names as the C ABI):

``attn_fwd(q, k, v, o, lse, causal=False, alpha=None, stream=None)``
    16-bit (bf16 / f16) forward; q, k, v, o are [B, N, H, d] tensors, lse is
    float32 [B, H, N].
``attn_fp8_prepare(x, x8, descale, block_rows=128, hadamard=False, seed=0, stream=None)``
    Hadamard transform (optional) + block quantisation of a bf16 tensor to
    e4m3 codes (uint8) and float32 descales.
``attn_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=False,
alpha=None, block_rows=128, hadamard_seed=0, stream=None)``
    Forward on e4m3 inputs with a bf16 output.
``attn_fwd_fp8_ex(...)``
    The same with k8/v8 (and their descales) over fewer key/value heads.
``attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, causal=False, alpha=None, stream=None)``
    16-bit backward (d = 64, 128 or 256): gradients dq, dk, dv of the forward's
    O = softmax(alpha q k^T) v for an upstream gradient dout; o and lse are
    the forward's outputs; delta is a float32 [B, H, N] workspace the call
    fills with rowsum(dout * o).
``attn_fwd_ex(q, k, v, o, lse, causal=False, alpha=None, cu_seqlens_q=None, cu_seqlens_k=None,
max_seqlen_q=None, max_seqlen_k=None, pack_gqa=-1, num_splits=1, workspace=None, stream=None)``
    16-bit forward with Hq query heads over Hkv key/value heads, N_q != N_k,
    packed variable-length batches (int32 cu_seqlens) and split-KV. Dense:
    q, o [B, Nq, Hq, d], k, v [B, Nk, Hkv, d], lse [B, Hq, Nq]. Packed:
    q, o [total_q, Hq, d], k, v [total_k, Hkv, d], lse [Hq, total_q].
``attn_fwd_ex_noalloc(q, k, v, o, lse, ...)``
    attn_fwd_ex without the workspace argument (for callers that cannot
    allocate): split-KV states go to a static 16 MiB array per GPU.
``attn_splitkv_workspace_bytes``, ``attn_pack_gqa_heuristic``,
``attn_num_splits_heuristic``
    Sizing helpers of attn_fwd_ex (pure host functions).
``attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, causal=False, alpha=None, stream=None,
  cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, window=(-1, -1))``
    Backward with grouped heads, N_q != N_k, packed batches and windows.
``attn_last_error()``
    Message of the last failed call on this thread.

Convenience wrappers that allocate the outputs with torch: ``attention``,
``attention_ex``, ``attention_backward`` and ``fp8_prepare``/``attention_fp8``.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "AttnError", "load", "lib_path", "attn_fwd", "attn_fp8_prepare", "attn_fwd_fp8", "attn_fwd_fp8_ex", "attn_bwd",
    "attn_bwd_ex",
    "attention_backward_ex", "attn_fwd_ex", "attn_fwd_ex_noalloc", "STATIC_WORKSPACE_BYTES",
    "attn_splitkv_workspace_bytes", "attn_pack_gqa_heuristic", "attn_num_splits_heuristic",
    "attn_last_error", "attention", "attention_ex", "attention_backward", "fp8_prepare", "attention_fp8",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libattn.so")
_lib = None

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, -1, -2, -3
DTYPE_BF16, DTYPE_F16 = 0, 1
EXPORTED_SYMBOLS = ("attn_fwd", "attn_fp8_prepare", "attn_fwd_fp8", "attn_fwd_fp8_ex", "attn_bwd", "attn_bwd_ex",
                    "attn_fwd_ex", "attn_fwd_ex_noalloc",
                    "attn_splitkv_workspace_bytes", "attn_pack_gqa_heuristic", "attn_num_splits_heuristic",
                    "attn_last_error", "attn_version")


class AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"attn status {status}: {msg}")
        self.status = status


def load():
    """Load libattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build it with "
                           "`python -m exact_attention_forward_attn_amd.build`")
    # torch first: the library then binds to the HIP runtime torch has
    # loaded (opened the other way round, the two can end up on different
    # runtime instances and launches report no device)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(lib_path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fp8_prepare.argtypes = [vp, vp, vp, i, i, i, i, i, i, ctypes.c_uint64, vp]
    lib.attn_fp8_prepare.restype = i
    u64 = ctypes.c_uint64
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, vp, i, u64, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_fp8_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, i, u64, vp]
    lib.attn_fwd_fp8_ex.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, i, i, i, i, i,
                                f, i, vp]
    lib.attn_bwd_ex.restype = i
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, i, i, i, i, i, f, i, i, i, vp,
                                ctypes.c_int64, vp]
    lib.attn_fwd_ex.restype = i
    lib.attn_fwd_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.attn_fwd_ex_noalloc.restype = i
    lib.attn_splitkv_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_splitkv_workspace_bytes.restype = ctypes.c_int64
    lib.attn_pack_gqa_heuristic.argtypes = [i, i, i]
    lib.attn_pack_gqa_heuristic.restype = i
    lib.attn_num_splits_heuristic.argtypes = [i, i, i, i, i, i, i, i]
    lib.attn_num_splits_heuristic.restype = i
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _default_alpha(d, alpha):
    return 1.0 / math.sqrt(d) if alpha is None else float(alpha)


def attn_fwd(q, k, v, o, lse, causal=False, alpha=None, stream=None):
    """O = softmax(alpha q k^T) v and LSE for [B, N, H, d] bf16/f16 tensors."""
    torch = _torch()
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    B, N, H, d = q.shape
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    for t, n in ((k, "k"), (v, "v"), (o, "o")):
        _require(t, n, q.dtype, q.shape, q.device)
    _require(q, "q", q.dtype, q.shape, q.device)
    _require(lse, "lse", torch.float32, (B, H, N), q.device)
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                        _default_alpha(d, alpha), dt, _stream_handle(stream)))
    return o, lse


def attn_splitkv_workspace_bytes(num_splits, total_q, Hq, d):
    return int(load().attn_splitkv_workspace_bytes(int(num_splits), int(total_q), int(Hq), int(d)))


def attn_pack_gqa_heuristic(Hq, Hkv, Nq):
    return int(load().attn_pack_gqa_heuristic(int(Hq), int(Hkv), int(Nq)))


def attn_num_splits_heuristic(B, Hq, Hkv, Nq, Nk, d, pack_gqa=-1, num_cus=None):
    if num_cus is None:
        num_cus = _torch().cuda.get_device_properties(0).multi_processor_count
    return int(load().attn_num_splits_heuristic(int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d),
                                                int(pack_gqa), int(num_cus)))


def _ex_shapes(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k):
    """(B, Hq, Hkv, Nq, Nk, d, total_q, total_k, lse shape) of an attn_fwd_ex call."""
    if cu_seqlens_q is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense inputs: q must be [B, Nq, Hq, d] and k [B, Nk, Hkv, d]")
        B, Nq, Hq, d = q.shape
        Nk, Hkv = k.shape[1], k.shape[2]
        return B, Hq, Hkv, Nq, Nk, d, B * Nq, B * Nk, (B, Hq, Nq)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed inputs: q must be [total_q, Hq, d] and k [total_k, Hkv, d]")
    if max_seqlen_q is None or max_seqlen_k is None:
        raise ValueError("packed inputs need max_seqlen_q and max_seqlen_k")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    return B, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), d, total_q, total_k, (Hq, total_q)


def attn_fwd_ex(q, k, v, o, lse, causal=False, alpha=None, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q=None, max_seqlen_k=None, pack_gqa=-1, num_splits=1, workspace=None, stream=None,
                window=(-1, -1)):
    """Forward with grouped heads, N_q != N_k, packed batches, split-KV and a
    (left, right) sliding window (-1 = unbounded side)."""
    torch = _torch()
    lib = load()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    B, Hq, Hkv, Nq, Nk, d, total_q, total_k, lse_shape = _ex_shapes(q, k, cu_seqlens_q, cu_seqlens_k,
                                                                    max_seqlen_q, max_seqlen_k)
    _require(q, "q", q.dtype, q.shape, q.device)
    _require(o, "o", q.dtype, q.shape, q.device)
    _require(k, "k", q.dtype, k.shape, q.device)
    _require(v, "v", q.dtype, k.shape, q.device)
    _require(lse, "lse", torch.float32, lse_shape, q.device)
    cu_q = cu_k = ctypes.c_void_p(0)
    if cu_seqlens_q is not None:
        _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,), q.device)
        _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, (B + 1,), q.device)
        cu_q, cu_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    ws, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        if workspace.dtype != torch.float32 or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous float32 tensor on the device of q")
        ws, ws_bytes = _ptr(workspace), workspace.numel() * 4
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    _check(lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, cu_q, cu_k,
                           total_q, total_k, int(bool(causal)), int(window[0]), int(window[1]),
                           _default_alpha(d, alpha), dt, int(pack_gqa),
                           int(num_splits), ws, ctypes.c_int64(ws_bytes), _stream_handle(stream)))
    return o, lse


STATIC_WORKSPACE_BYTES = 16 << 20  # ATTN_STATIC_WORKSPACE_BYTES of include/attn.h


def attn_fwd_ex_noalloc(q, k, v, o, lse, causal=False, alpha=None, cu_seqlens_q=None, cu_seqlens_k=None,
                        max_seqlen_q=None, max_seqlen_k=None, pack_gqa=-1, num_splits=1, stream=None,
                        window=(-1, -1)):
    """attn_fwd_ex without a workspace argument: the split-KV range states go
    to the library's static per-GPU array (STATIC_WORKSPACE_BYTES), so the
    call allocates no device memory. Calls that overlap in time on one GPU
    race on that array."""
    torch = _torch()
    lib = load()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    B, Hq, Hkv, Nq, Nk, d, total_q, total_k, lse_shape = _ex_shapes(q, k, cu_seqlens_q, cu_seqlens_k,
                                                                    max_seqlen_q, max_seqlen_k)
    _require(q, "q", q.dtype, q.shape, q.device)
    _require(o, "o", q.dtype, q.shape, q.device)
    _require(k, "k", q.dtype, k.shape, q.device)
    _require(v, "v", q.dtype, k.shape, q.device)
    _require(lse, "lse", torch.float32, lse_shape, q.device)
    cu_q = cu_k = ctypes.c_void_p(0)
    if cu_seqlens_q is not None:
        _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,), q.device)
        _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, (B + 1,), q.device)
        cu_q, cu_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    _check(lib.attn_fwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, cu_q, cu_k,
                                   total_q, total_k, int(bool(causal)), int(window[0]), int(window[1]),
                                   _default_alpha(d, alpha), dt, int(pack_gqa), int(num_splits),
                                   _stream_handle(stream)))
    return o, lse


def attention_ex(q, k, v, causal=False, alpha=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                 max_seqlen_k=None, pack_gqa=-1, num_splits=None, stream=None, window=(-1, -1)):
    """Allocate O, LSE and the split-KV workspace with torch and run attn_fwd_ex.

    ``num_splits=None`` takes attn_num_splits_heuristic for this device.
    """
    torch = _torch()
    B, Hq, Hkv, Nq, Nk, d, total_q, _, lse_shape = _ex_shapes(q, k, cu_seqlens_q, cu_seqlens_k,
                                                              max_seqlen_q, max_seqlen_k)
    if num_splits is None:
        num_splits = attn_num_splits_heuristic(B, Hq, Hkv, Nq, Nk, d, pack_gqa,
                                               torch.cuda.get_device_properties(q.device).multi_processor_count)
    o = torch.empty_like(q)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    nbytes = attn_splitkv_workspace_bytes(num_splits, total_q, Hq, d)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device) if nbytes else None
    return attn_fwd_ex(q, k, v, o, lse, causal, alpha, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                       pack_gqa, num_splits, ws, stream, window)


def attn_fp8_prepare(x, x8, descale, block_rows=128, hadamard=False, seed=0, stream=None):
    """Block quantisation (and optional Hadamard transform) of bf16 x to e4m3."""
    torch = _torch()
    lib = load()
    B, N, H, d = x.shape
    _require(x, "x", torch.bfloat16, x.shape, x.device)
    _require(x8, "x8", torch.uint8, x.shape, x.device)
    nd = (B, H, (N + block_rows - 1) // block_rows) if block_rows else (1,)
    _require(descale, "descale", torch.float32, nd, x.device)
    _check(lib.attn_fp8_prepare(_ptr(x), _ptr(x8), _ptr(descale), B, H, N, d, int(block_rows),
                                int(bool(hadamard)), ctypes.c_uint64(int(seed) & (2 ** 64 - 1)),
                                _stream_handle(stream)))
    return x8, descale


def _seed(seed):
    return ctypes.c_uint64(int(seed) & (2 ** 64 - 1))


def attn_fwd_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=False, alpha=None,
                 block_rows=128, hadamard_seed=0, stream=None):
    """Forward on e4m3 codes from attn_fp8_prepare; o is bf16. hadamard_seed
    is the seed q8 and k8 were prepared with (a contract the library cannot
    check: the forward never applies the transform)."""
    torch = _torch()
    lib = load()
    B, N, H, d = q8.shape
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _require(t, n, torch.uint8, q8.shape, q8.device)
    _require(o, "o", torch.bfloat16, q8.shape, q8.device)
    _require(lse, "lse", torch.float32, (B, H, N), q8.device)
    nd = (B, H, (N + block_rows - 1) // block_rows) if block_rows else (1,)
    for t, n in ((descale_q, "descale_q"), (descale_k, "descale_k"), (descale_v, "descale_v")):
        _require(t, n, torch.float32, nd, q8.device)
    _check(lib.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, H, N, d,
                            int(bool(causal)), _default_alpha(d, alpha), _ptr(descale_q), _ptr(descale_k),
                            _ptr(descale_v), int(block_rows), _seed(hadamard_seed), _stream_handle(stream)))
    return o, lse


def attn_fwd_fp8_ex(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal=False, alpha=None,
                    block_rows=128, hadamard_seed=0, stream=None):
    """attn_fwd_fp8 with k8/v8 of shape [B, N, Hkv, d], Hq a multiple of Hkv."""
    torch = _torch()
    lib = load()
    B, N, Hq, d = q8.shape
    Hkv = k8.shape[2] if k8.dim() == 4 else 0
    _require(q8, "q8", torch.uint8, q8.shape, q8.device)
    for t, n in ((k8, "k8"), (v8, "v8")):
        _require(t, n, torch.uint8, (B, N, Hkv, d), q8.device)
    _require(o, "o", torch.bfloat16, q8.shape, q8.device)
    _require(lse, "lse", torch.float32, (B, Hq, N), q8.device)
    nb = (N + block_rows - 1) // block_rows if block_rows else 0
    _require(descale_q, "descale_q", torch.float32, (B, Hq, nb) if block_rows else (1,), q8.device)
    for t, n in ((descale_k, "descale_k"), (descale_v, "descale_v")):
        _require(t, n, torch.float32, (B, Hkv, nb) if block_rows else (1,), q8.device)
    _check(lib.attn_fwd_fp8_ex(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                               int(bool(causal)), _default_alpha(d, alpha), _ptr(descale_q), _ptr(descale_k),
                               _ptr(descale_v), int(block_rows), _seed(hadamard_seed), _stream_handle(stream)))
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, causal=False, alpha=None, stream=None):
    """Gradients of O = softmax(alpha q k^T) v: fills dq, dk, dv (and delta)."""
    torch = _torch()
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    B, N, H, d = q.shape
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _require(t, n, q.dtype, q.shape, q.device)
    _require(lse, "lse", torch.float32, (B, H, N), q.device)
    _require(delta, "delta", torch.float32, (B, H, N), q.device)
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(delta), B, H, N, d, int(bool(causal)), _default_alpha(d, alpha), dt,
                        _stream_handle(stream)))
    return dq, dk, dv


def attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, causal=False, alpha=None, stream=None,
                cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, window=(-1, -1)):
    """Backward with Hq query heads over Hkv key/value heads, N_q != N_k,
    packed batches and a (left, right) sliding window. Dense: q, o, dout, dq
    [B, Nq, Hq, d]; k, v, dk, dv [B, Nk, Hkv, d]; lse and delta float32
    [B, Hq, Nq]. Packed: [total_q, Hq, d], [total_k, Hkv, d], [Hq, total_q]."""
    torch = _torch()
    lib = load()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    B, Hq, Hkv, Nq, Nk, d, total_q, total_k, lse_shape = _ex_shapes(q, k, cu_seqlens_q, cu_seqlens_k,
                                                                    max_seqlen_q, max_seqlen_k)
    for t, n in ((q, "q"), (o, "o"), (dout, "dout"), (dq, "dq")):
        _require(t, n, q.dtype, q.shape, q.device)
    for t, n in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _require(t, n, q.dtype, k.shape, q.device)
    _require(lse, "lse", torch.float32, lse_shape, q.device)
    _require(delta, "delta", torch.float32, lse_shape, q.device)
    cu_q = cu_k = ctypes.c_void_p(0)
    if cu_seqlens_q is not None:
        _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,), q.device)
        _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, (B + 1,), q.device)
        cu_q, cu_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_F16
    _check(lib.attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(delta), B, Hq, Hkv, Nq, Nk, d, cu_q, cu_k, total_q, total_k, int(bool(causal)),
                           int(window[0]), int(window[1]), _default_alpha(d, alpha), dt, _stream_handle(stream)))
    return dq, dk, dv


def attention_backward_ex(q, k, v, o, lse, dout, causal=False, alpha=None, stream=None, cu_seqlens_q=None,
                          cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None, window=(-1, -1)):
    """Allocate dq, dk, dv and the workspace with torch and run attn_bwd_ex."""
    torch = _torch()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(lse.shape, dtype=torch.float32, device=q.device)
    return attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, causal, alpha, stream, cu_seqlens_q, cu_seqlens_k,
                       max_seqlen_q, max_seqlen_k, window)


def attention_backward(q, k, v, o, lse, dout, causal=False, alpha=None, stream=None):
    """Allocate dq, dk, dv and the workspace with torch and run attn_bwd."""
    torch = _torch()
    B, N, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    return attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, causal, alpha, stream)


def attention(q, k, v, causal=False, alpha=None, stream=None):
    """Allocate O and LSE with torch and run attn_fwd."""
    torch = _torch()
    B, N, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    return attn_fwd(q, k, v, o, lse, causal, alpha, stream)


def fp8_prepare(x, block_rows=128, hadamard=False, seed=0, stream=None):
    torch = _torch()
    B, N, H, d = x.shape
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    nd = (B, H, (N + block_rows - 1) // block_rows) if block_rows else (1,)
    descale = torch.empty(nd, dtype=torch.float32, device=x.device)
    return attn_fp8_prepare(x, x8, descale, block_rows, hadamard, seed, stream)


def attention_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, alpha=None, block_rows=128,
                  hadamard_seed=0, stream=None):
    torch = _torch()
    B, N, H, d = q8.shape
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    fwd = attn_fwd_fp8 if k8.shape == q8.shape else attn_fwd_fp8_ex
    return fwd(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal, alpha, block_rows, hadamard_seed,
               stream)
