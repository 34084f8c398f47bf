"""ctypes binding of libattn.so: argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI declared in
include/attn.h, include/attn_block.h, include/attn_decode.h,
include/attn_dropout.h and include/attn_rope.h. PyTorch is used only to own device memory and to provide the
stream handle. There is no fallback: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
# TAM_LIBATTN_PATH selects another build of the same library (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("TAM_LIBATTN_PATH") or os.path.join(_PKG, "lib", "libattn.so")

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL_POINTER", 2: "ATTN_ERR_BAD_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED_HEAD_DIM", 4: "ATTN_ERR_BAD_SCALE", 5: "ATTN_ERR_MISALIGNED",
    6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_HIP", 8: "ATTN_ERR_BAD_FLAG", 9: "ATTN_ERR_ALIAS",
    10: "ATTN_ERR_SCRATCH_LIMIT",
}

EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_timed", "attn_bwd_workspace_bytes", "attn_status_string",
           "attn_version", "attn_fwd_block", "attn_merge", "attn_bwd_block_workspace_bytes",
           "attn_bwd_block_begin", "attn_bwd_block_dq", "attn_bwd_block_dq_end", "attn_bwd_block_dkdv",
           "attn_decode_workspace_bytes", "attn_decode", "attn_fwd_dropout", "attn_bwd_dropout",
           "attn_rope_workspace_bytes", "attn_fwd_rope", "attn_bwd_rope", "attn_bwd_noalloc")
NOALLOC_SCRATCH_BYTES = 256 << 20
BWD_EVENTS = 5
MAX_MERGE = 16

_lock = threading.Lock()
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({attn_status_string(status)})")


def load() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by tiled_attention_memory_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m tiled_attention_memory_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        lib.attn_fwd.restype = i
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                 i, i, i, i, i, i, f, vp]
        lib.attn_bwd.restype = i
        lib.attn_bwd_timed.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       i, i, i, i, i, i, f, vp, vp]
        lib.attn_bwd_timed.restype = i
        lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        lib.attn_bwd_noalloc.restype = i
        lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
        lib.attn_bwd_workspace_bytes.restype = i
        lib.attn_status_string.argtypes = [i]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_version.argtypes = []
        lib.attn_version.restype = i
        ll = ctypes.c_longlong
        lib.attn_fwd_block.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, ll, ll, f, vp]
        lib.attn_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i, vp, vp, i, i, i, i, vp]
        lib.attn_bwd_block_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(sz)]
        lib.attn_bwd_block_begin.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, i, vp]
        lib.attn_bwd_block_dq.argtypes = [vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, ll, ll, f, vp]
        lib.attn_bwd_block_dq_end.argtypes = [vp, vp, sz, i, i, i, i, i, i, f, vp]
        lib.attn_bwd_block_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, ll, ll, f, vp]
        lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(sz)]
        lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, vp]
        ull = ctypes.c_ulonglong
        lib.attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, ull, vp]
        lib.attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, f, ull, vp]
        lib.attn_rope_workspace_bytes.argtypes = [i, i, i, i, i, ctypes.POINTER(sz)]
        lib.attn_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, f, vp]
        lib.attn_bwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, f, vp]
        for name in ("attn_fwd_block", "attn_merge", "attn_bwd_block_workspace_bytes", "attn_bwd_block_begin",
                     "attn_bwd_block_dq", "attn_bwd_block_dq_end", "attn_bwd_block_dkdv",
                     "attn_decode_workspace_bytes", "attn_decode", "attn_fwd_dropout", "attn_bwd_dropout",
                     "attn_rope_workspace_bytes", "attn_fwd_rope", "attn_bwd_rope"):
            getattr(lib, name).restype = i
        _lib = lib
        return lib


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return load().attn_version()


# ---------------------------------------------------------------------------
# raw entry points: plain integers for pointers (used for the C ABI contract)
# ---------------------------------------------------------------------------
def attn_fwd_raw(q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, stream=0) -> int:
    return load().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, S, D, int(causal), float(scale), stream)


def attn_bwd_raw(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, S, D, causal,
                 scale, stream=0) -> int:
    return load().attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, S, D,
                           int(causal), float(scale), stream)


def attn_bwd_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, D: int) -> int:
    out = ctypes.c_size_t(0)
    st = load().attn_bwd_workspace_bytes(B, Hq, Hkv, S, D, ctypes.byref(out))
    if st != 0:
        raise AttnError(st, "attn_bwd_workspace_bytes")
    return out.value


# ---------------------------------------------------------------------------
# torch-tensor entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def _shape(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, S, D]")
    B, Hq, S, D = q.shape
    if k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    return B, Hq, k.shape[1], S, D


def _check(t, name, dtype, shape):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def attn_fwd(q, k, v, o, lse, causal=True, scale=None, stream=None) -> None:
    """Enqueue the forward pass: writes o (bf16) and lse (fp32) in place."""
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
         _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
         _check(lse, "lse", torch.float32, (B, Hq, S))]
    st = load().attn_fwd(*p, B, Hq, Hkv, S, D, int(bool(causal)), _scale(scale, D), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd")


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal=True, scale=None,
             stream=None, events=None) -> None:
    """Enqueue the backward pass: writes dq, dk, dv (bf16) in place.

    events: optional ctypes array of BWD_EVENTS hipEvent_t handles; when given,
    the call goes through attn_bwd_timed and records them between the kernels.
    """
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
         _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
         _check(dout, "dout", bf, (B, Hq, S, D)), _check(lse, "lse", torch.float32, (B, Hq, S)),
         _check(dq, "dq", bf, (B, Hq, S, D)), _check(dk, "dk", bf, (B, Hkv, S, D)),
         _check(dv, "dv", bf, (B, Hkv, S, D))]
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    args = (*p, workspace.data_ptr(), workspace.numel(), B, Hq, Hkv, S, D, int(bool(causal)),
            _scale(scale, D), _stream(stream))
    if events is None:
        st = load().attn_bwd(*args)
    else:
        st = load().attn_bwd_timed(*args, ctypes.cast(events, ctypes.c_void_p))
    if st != 0:
        raise AttnError(st, "attn_bwd")


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal=True, scale=None, stream=None) -> None:
    """Enqueue the backward pass without a workspace (the library's fixed scratch):
    writes dq, dk, dv (bf16) in place. Calls on one GPU must not overlap in time."""
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
         _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
         _check(dout, "dout", bf, (B, Hq, S, D)), _check(lse, "lse", torch.float32, (B, Hq, S)),
         _check(dq, "dq", bf, (B, Hq, S, D)), _check(dk, "dk", bf, (B, Hkv, S, D)),
         _check(dv, "dv", bf, (B, Hkv, S, D))]
    st = load().attn_bwd_noalloc(*p, B, Hq, Hkv, S, D, int(bool(causal)), _scale(scale, D), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")


# ---------------------------------------------------------------------------
# conveniences that allocate outputs with torch, then call the entry points
# ---------------------------------------------------------------------------
def forward(q, k, v, causal=True, scale=None, stream=None):
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def workspace_for(q, k):
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    return torch.empty(attn_bwd_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8,
                       device=q.device)


def backward(q, k, v, o, dout, lse, causal=True, scale=None, stream=None, workspace=None):
    import torch
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = workspace_for(q, k) if workspace is None else workspace
    attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, causal, scale, stream)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# context-parallel building block (include/attn_block.h)
# ---------------------------------------------------------------------------
def _block_shape(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q shape {tuple(q.shape)}")
    return B, Hq, k.shape[1], Sq, k.shape[2], D


def _ws_ptr(workspace):
    import torch
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    return workspace.data_ptr(), workspace.numel()


def _raise(st, what):
    if st != 0:
        raise AttnError(st, what)


def attn_fwd_block(q, k, v, o_part, lse_part, q_pos0, k_pos0, causal=True, scale=None, stream=None) -> None:
    """Partial output (fp32) and log-sum-exp of one (query block, key block) pair."""
    import torch
    B, Hq, Hkv, Sq, Sk, D = _block_shape(q, k)
    bf, f32 = torch.bfloat16, torch.float32
    p = [_check(q, "q", bf, (B, Hq, Sq, D)), _check(k, "k", bf, (B, Hkv, Sk, D)),
         _check(v, "v", bf, (B, Hkv, Sk, D)), _check(o_part, "o_part", f32, (B, Hq, Sq, D)),
         _check(lse_part, "lse_part", f32, (B, Hq, Sq))]
    _raise(load().attn_fwd_block(*p, B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), int(q_pos0), int(k_pos0),
                                 _scale(scale, D), _stream(stream)), "attn_fwd_block")


def attn_merge(o_parts, lse_parts, o, lse, stream=None) -> None:
    """Merge partial results over disjoint key blocks into o (bf16) and lse."""
    import torch
    n = len(o_parts)
    if n != len(lse_parts):
        raise ValueError("o_parts and lse_parts differ in length")
    B, Hq, Sq, D = o.shape
    op = [_check(t, "o_parts[i]", torch.float32, (B, Hq, Sq, D)) for t in o_parts]
    lp = [_check(t, "lse_parts[i]", torch.float32, (B, Hq, Sq)) for t in lse_parts]
    arr = ctypes.c_void_p * max(n, 1)
    _raise(load().attn_merge(arr(*op), arr(*lp), n, _check(o, "o", torch.bfloat16, (B, Hq, Sq, D)),
                             _check(lse, "lse", torch.float32, (B, Hq, Sq)), B, Hq, Sq, D, _stream(stream)),
           "attn_merge")


def attn_bwd_block_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int) -> int:
    out = ctypes.c_size_t(0)
    _raise(load().attn_bwd_block_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, ctypes.byref(out)),
           "attn_bwd_block_workspace_bytes")
    return out.value


def attn_bwd_block_begin(o, dout, lse, workspace, Hkv, Sk, stream=None) -> None:
    import torch
    B, Hq, Sq, D = o.shape
    bf = torch.bfloat16
    p = [_check(o, "o", bf, (B, Hq, Sq, D)), _check(dout, "dout", bf, (B, Hq, Sq, D)),
         _check(lse, "lse", torch.float32, (B, Hq, Sq))]
    _raise(load().attn_bwd_block_begin(*p, *_ws_ptr(workspace), B, Hq, Hkv, Sq, Sk, D, _stream(stream)),
           "attn_bwd_block_begin")


def attn_bwd_block_dq(q, k, v, dout, workspace, q_pos0, k_pos0, causal=True, scale=None, stream=None) -> None:
    import torch
    B, Hq, Hkv, Sq, Sk, D = _block_shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, Sq, D)), _check(k, "k", bf, (B, Hkv, Sk, D)),
         _check(v, "v", bf, (B, Hkv, Sk, D)), _check(dout, "dout", bf, (B, Hq, Sq, D))]
    _raise(load().attn_bwd_block_dq(*p, *_ws_ptr(workspace), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                    int(q_pos0), int(k_pos0), _scale(scale, D), _stream(stream)),
           "attn_bwd_block_dq")


def attn_bwd_block_dq_end(dq, workspace, Hkv, Sk, scale=None, stream=None) -> None:
    import torch
    B, Hq, Sq, D = dq.shape
    _raise(load().attn_bwd_block_dq_end(_check(dq, "dq", torch.bfloat16, (B, Hq, Sq, D)), *_ws_ptr(workspace),
                                        B, Hq, Hkv, Sq, Sk, D, _scale(scale, D), _stream(stream)),
           "attn_bwd_block_dq_end")


def attn_bwd_block_dkdv(q, k, v, dout, dk, dv, workspace, q_pos0, k_pos0, causal=True, scale=None,
                        stream=None) -> None:
    import torch
    B, Hq, Hkv, Sq, Sk, D = _block_shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, Sq, D)), _check(k, "k", bf, (B, Hkv, Sk, D)),
         _check(v, "v", bf, (B, Hkv, Sk, D)), _check(dout, "dout", bf, (B, Hq, Sq, D)),
         _check(dk, "dk", bf, (B, Hkv, Sk, D)), _check(dv, "dv", bf, (B, Hkv, Sk, D))]
    _raise(load().attn_bwd_block_dkdv(*p, *_ws_ptr(workspace), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                      int(q_pos0), int(k_pos0), _scale(scale, D), _stream(stream)),
           "attn_bwd_block_dkdv")


# ---------------------------------------------------------------------------
# decode against a key/value cache (include/attn_decode.h)
# ---------------------------------------------------------------------------
def attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int) -> int:
    out = ctypes.c_size_t(0)
    _raise(load().attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, ctypes.byref(out)),
           "attn_decode_workspace_bytes")
    return out.value


def attn_decode(q, k, v, o, lse, workspace, causal=True, scale=None, stream=None) -> None:
    """Sq new tokens per head (the last Sq positions) against the Sk-key cache k, v."""
    import torch
    B, Hq, Hkv, Sq, Sk, D = _block_shape(q, k)
    bf = torch.bfloat16
    p = [_check(q, "q", bf, (B, Hq, Sq, D)), _check(k, "k", bf, (B, Hkv, Sk, D)),
         _check(v, "v", bf, (B, Hkv, Sk, D)), _check(o, "o", bf, (B, Hq, Sq, D)),
         _check(lse, "lse", torch.float32, (B, Hq, Sq))]
    _raise(load().attn_decode(*p, *_ws_ptr(workspace), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                              _scale(scale, D), _stream(stream)), "attn_decode")


# ---------------------------------------------------------------------------
# dropout on the probabilities (include/attn_dropout.h)
# ---------------------------------------------------------------------------
def attn_fwd_dropout(q, k, v, o, lse, p, seed, causal=True, scale=None, stream=None) -> None:
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    ptrs = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
            _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
            _check(lse, "lse", torch.float32, (B, Hq, S))]
    _raise(load().attn_fwd_dropout(*ptrs, B, Hq, Hkv, S, D, int(bool(causal)), _scale(scale, D), float(p),
                                   int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(stream)), "attn_fwd_dropout")


def attn_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, p, seed, causal=True, scale=None,
                     stream=None) -> None:
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    ptrs = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
            _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
            _check(dout, "dout", bf, (B, Hq, S, D)), _check(lse, "lse", torch.float32, (B, Hq, S)),
            _check(dq, "dq", bf, (B, Hq, S, D)), _check(dk, "dk", bf, (B, Hkv, S, D)),
            _check(dv, "dv", bf, (B, Hkv, S, D))]
    _raise(load().attn_bwd_dropout(*ptrs, *_ws_ptr(workspace), B, Hq, Hkv, S, D, int(bool(causal)),
                                   _scale(scale, D), float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(stream)),
           "attn_bwd_dropout")


# ---------------------------------------------------------------------------
# rotary position embedding (include/attn_rope.h)
# ---------------------------------------------------------------------------
def attn_rope_workspace_bytes(B: int, Hq: int, Hkv: int, S: int, D: int) -> int:
    out = ctypes.c_size_t(0)
    _raise(load().attn_rope_workspace_bytes(B, Hq, Hkv, S, D, ctypes.byref(out)), "attn_rope_workspace_bytes")
    return out.value


def rope_workspace_for(q, k):
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    return torch.empty(attn_rope_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device=q.device)


def attn_fwd_rope(q, k, v, o, lse, workspace, base, causal=True, scale=None, stream=None) -> None:
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    ptrs = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
            _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
            _check(lse, "lse", torch.float32, (B, Hq, S))]
    _raise(load().attn_fwd_rope(*ptrs, *_ws_ptr(workspace), B, Hq, Hkv, S, D, int(bool(causal)), _scale(scale, D),
                                float(base), _stream(stream)), "attn_fwd_rope")


def attn_bwd_rope(q, k, v, o, dout, lse, dq, dk, dv, workspace, base, causal=True, scale=None, stream=None) -> None:
    import torch
    B, Hq, Hkv, S, D = _shape(q, k)
    bf = torch.bfloat16
    ptrs = [_check(q, "q", bf, (B, Hq, S, D)), _check(k, "k", bf, (B, Hkv, S, D)),
            _check(v, "v", bf, (B, Hkv, S, D)), _check(o, "o", bf, (B, Hq, S, D)),
            _check(dout, "dout", bf, (B, Hq, S, D)), _check(lse, "lse", torch.float32, (B, Hq, S)),
            _check(dq, "dq", bf, (B, Hq, S, D)), _check(dk, "dk", bf, (B, Hkv, S, D)),
            _check(dv, "dv", bf, (B, Hkv, S, D))]
    _raise(load().attn_bwd_rope(*ptrs, *_ws_ptr(workspace), B, Hq, Hkv, S, D, int(bool(causal)), _scale(scale, D),
                                float(base), _stream(stream)), "attn_bwd_rope")
