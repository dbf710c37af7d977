"""Python binding of libtpshard (one GPU's shard of a Megatron-LM TP layer).

Argument marshalling only: every function takes torch tensors that live on
the GPU, reads their sizes and device pointers, and calls the C entry point
of the same name in libtpshard.so on the current (or given) HIP stream.  All
arithmetic runs in the library's gfx950 kernels; there is no fallback, and
importing the binding without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "TPError", "lib", "LIB_PATH", "TP_DT_F32", "TP_DT_BF16",
    "tp_mlp_fwd", "tp_mlp_bwd", "tp_mlp_bwd_workspace_bytes", "tp_mlp_bwd_noalloc", "MLP_BWD_NOALLOC_MAX_WORKSPACE",
    "tp_mlp_fwd_shards", "tp_mlp_bwd_shards", "tp_mlp_bwd_shards_workspace_bytes",
    "tp_swiglu_fwd", "tp_swiglu_bwd", "tp_swiglu_bwd_workspace_bytes",
    "tp_attn_shard_fwd", "tp_attn_gqa_shard_fwd", "tp_attn_shard_bwd", "tp_attn_shard_bwd_workspace_bytes",
    "tp_attn_gqa_shard_bwd", "tp_attn_gqa_shard_bwd_workspace_bytes",
    "tp_shard_reduce", "tp_shard_range", "tp_sp_reduce_scatter_ln", "tp_sp_all_gather", "tp_sp_ln_bwd_reduce_scatter",
    "tp_sp_ln_bwd_workspace_bytes",
    "tp_vocab_embed_fwd", "tp_vocab_embed_bwd", "tp_vocab_ce_fwd", "tp_vocab_ce_fwd_workspace_bytes", "tp_vocab_ce_combine", "tp_vocab_ce_bwd",
    "tp_vocab_ce_bwd_workspace_bytes",
    "tp_abi_version", "EXPORTS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# TPSHARD_LIB selects another build of the same library (the host-sanitizer
# build of the CPU ABI checks); unset, the in-tree library is loaded.
LIB_PATH = os.environ.get("TPSHARD_LIB") or os.path.join(HERE, "libtpshard.so")
ABI_VERSION = 11         # TP_ABI_VERSION of include/tp_shard.h these wrappers are written for

TP_DT_F32 = 0
TP_DT_BF16 = 1
MLP_BWD_NOALLOC_MAX_WORKSPACE = 64 << 20    # TP_MLP_BWD_NOALLOC_MAX_WORKSPACE

STATUS = {0: "TP_OK", -1: "TP_E_NULL", -2: "TP_E_DIM", -3: "TP_E_DIVIS", -4: "TP_E_DTYPE",
          -5: "TP_E_ALIGN", -6: "TP_E_ALIAS", -7: "TP_E_WORKSPACE", -8: "TP_E_HIP"}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tp_shard.h
EXPORTS = {
    "tp_shard_range": (_i32, [_i64, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tp_mlp_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "tp_mlp_bwd": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "tp_mlp_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_mlp_bwd_noalloc": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tp_mlp_fwd_shards": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "tp_mlp_bwd_shards": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "tp_mlp_bwd_shards_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i64]),
    "tp_swiglu_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tp_swiglu_bwd": (_i32, [_p, _i32, _i64, _i64, _i64] + [_p] * 8 + [_p] * 4 + [_p, _sz]),
    "tp_swiglu_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_attn_shard_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _i64, _i32, ctypes.c_float]
                          + [_p] * 5 + [_p] * 5 + [_p]),
    "tp_attn_gqa_shard_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i32, ctypes.c_float]
                              + [_p] * 5 + [_p] * 5 + [_p]),
    "tp_attn_shard_bwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _i64, _i32, ctypes.c_float]
                          + [_p] * 5 + [_p] * 5 + [_p] + [_p] * 5 + [_p, _sz]),
    "tp_attn_shard_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i64, _i64]),
    "tp_attn_gqa_shard_bwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _i64, _i64, _i32, ctypes.c_float]
                              + [_p] * 5 + [_p] * 5 + [_p] + [_p] * 5 + [_p, _sz]),
    "tp_attn_gqa_shard_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64, _i64, _i64, _i64]),
    "tp_shard_reduce": (_i32, [_p, _i32, _i32, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "tp_sp_reduce_scatter_ln": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _i64, _p, _p, _p, ctypes.c_float,
                                       _p, _p, ctypes.c_float, _p, _p]),
    "tp_sp_all_gather": (_i32, [_p, _i32, _i64, _i64, _i64, ctypes.POINTER(_p), _p]),
    "tp_sp_ln_bwd_reduce_scatter": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _i64, _p, _p, ctypes.c_float, _p,
                                           ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "tp_sp_ln_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_vocab_embed_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "tp_vocab_embed_bwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "tp_vocab_ce_fwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _sz]),
    "tp_vocab_ce_fwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_vocab_ce_combine": (_i32, [_p, _i64, _i64, _p, _i64, _p, _p]),
    "tp_vocab_ce_bwd": (_i32, [_p, _i32, _i64, _i64, _i64, _i64] + [_p] * 6 + [_p, _p, _p, _sz]),
    "tp_vocab_ce_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64, _i64]),
    "tp_strerror": (ctypes.c_char_p, [_i32]),
    "tp_last_error_detail": (ctypes.c_char_p, []),
    "tp_abi_version": (_i32, []),
    "tp_profile_begin": (_i32, [ctypes.POINTER(_p), ctypes.POINTER(_p), _i32]),
    "tp_profile_only": (_i32, [ctypes.c_char_p]),
    "tp_profile_end": (_i32, []),
    "tp_profile_label": (ctypes.c_char_p, [_i32]),
}

_LIB = None


class TPError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def lib() -> ctypes.CDLL:
    """Load libtpshard.so (built in-tree by build.build())."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "megatron_tensor_transformer_fwd_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            try:
                fn = getattr(L, name)
            except AttributeError:
                raise ImportError(f"{LIB_PATH} does not export {name}: it is stale, rebuild it") from None
            fn.restype, fn.argtypes = res, args
        if L.tp_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {L.tp_abi_version()}, the binding expects "
                              f"{ABI_VERSION}: rebuild it")
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        raise TPError(status, lib().tp_last_error_detail().decode())


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TP_DT_BF16
    if t.dtype == torch.float32:
        return TP_DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _need(name: str, t, numel: int, dtype=None, optional: bool = False, at_least: bool = False) -> None:
    """Refuse a tensor whose element count or dtype differs from what the
    call's sizes imply, before its address reaches the library (the C layer
    can check extents only against the sizes it is given)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        raise ValueError(f"{name} has {n} elements, the call needs {'at least ' if at_least else ''}{numel}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, the call needs {dtype}")


def _f32():
    import torch
    return torch.float32


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def tp_abi_version() -> int:
    return lib().tp_abi_version()


def tp_shard_range(total: int, n_shards: int, index: int):
    s, n = _i64(), _i64()
    _check(lib().tp_shard_range(total, n_shards, index, ctypes.byref(s), ctypes.byref(n)))
    return s.value, n.value


def tp_mlp_fwd(X, W1, W2, A, H, Z, stream=None) -> None:
    """A = X W1, H = GeLU(A), Z = H W2 (see include/tp_shard.h)."""
    M, d = X.shape
    f = W1.shape[1]
    dt = X.dtype
    _need("W1", W1, d * f, dt)
    _need("W2", W2, f * d, dt)
    _need("A", A, M * f, dt, optional=True)
    _need("H", H, M * f, dt)
    _need("Z", Z, M * d, dt)
    _check(lib().tp_mlp_fwd(_stream(stream), _dt(X), M, d, f, _ptr(X), _ptr(W1), _ptr(W2),
                            _ptr(A), _ptr(H), _ptr(Z)))


def tp_mlp_bwd_workspace_bytes(dtype: int, M: int, d: int, f: int) -> int:
    return lib().tp_mlp_bwd_workspace_bytes(dtype, M, d, f)


def tp_mlp_bwd(X, W1, W2, A, H, dY, dX, dW1, dW2, ws, stream=None) -> None:
    M, d = X.shape
    f = W1.shape[1]
    dt = X.dtype
    _need("W1", W1, d * f, dt)
    _need("W2", W2, f * d, dt)
    for name, t in (("A", A), ("H", H)):
        _need(name, t, M * f, dt)
    for name, t in (("dY", dY), ("dX", dX)):
        _need(name, t, M * d, dt)
    _need("dW1", dW1, d * f, _f32())
    _need("dW2", dW2, f * d, _f32())
    _check(lib().tp_mlp_bwd(_stream(stream), _dt(X), M, d, f, _ptr(X), _ptr(W1), _ptr(W2), _ptr(A),
                            _ptr(H), _ptr(dY), _ptr(dX), _ptr(dW1), _ptr(dW2), _ptr(ws),
                            ws.numel() * ws.element_size()))


def tp_mlp_bwd_noalloc(X, W1, W2, A, H, dY, dX, dW1, dW2, stream=None) -> None:
    """tp_mlp_bwd with the library's own per-GPU scratch instead of ws."""
    M, d = X.shape
    f = W1.shape[1]
    dt = X.dtype
    _need("W1", W1, d * f, dt)
    _need("W2", W2, f * d, dt)
    for name, t in (("A", A), ("H", H)):
        _need(name, t, M * f, dt)
    for name, t in (("dY", dY), ("dX", dX)):
        _need(name, t, M * d, dt)
    _need("dW1", dW1, d * f, _f32())
    _need("dW2", dW2, f * d, _f32())
    _check(lib().tp_mlp_bwd_noalloc(_stream(stream), _dt(X), M, d, f, _ptr(X), _ptr(W1), _ptr(W2), _ptr(A),
                                    _ptr(H), _ptr(dY), _ptr(dX), _ptr(dW1), _ptr(dW2)))


def tp_mlp_fwd_shards(X, W1s, W2s, A, H, Z, stream=None) -> None:
    """Every shard at once: W1s [n x d x f], W2s [n x f x d]; A, H [n x M x f];
    Z [n x M x d] (the partials)."""
    n, d, f = W1s.shape
    M = X.shape[0]
    dt = X.dtype
    _need("X", X, M * d, dt)
    _need("W2s", W2s, n * f * d, dt)
    _need("A", A, n * M * f, dt, optional=True)
    _need("H", H, n * M * f, dt)
    _need("Z", Z, n * M * d, dt)
    _check(lib().tp_mlp_fwd_shards(_stream(stream), _dt(X), n, M, d, f, _ptr(X), _ptr(W1s), _ptr(W2s), _ptr(A),
                                   _ptr(H), _ptr(Z)))


def tp_mlp_bwd_shards_workspace_bytes(dtype: int, n_shards: int, M: int, d: int, f: int) -> int:
    return lib().tp_mlp_bwd_shards_workspace_bytes(dtype, n_shards, M, d, f)


def tp_mlp_bwd_shards(X, W1s, W2s, A, H, dY, dX, dW1s, dW2s, ws, stream=None) -> None:
    """Every shard's backward at once: dX [n x M x d] (summands), dW1s
    [n x d x f] and dW2s [n x f x d] fp32."""
    n, d, f = W1s.shape
    M = X.shape[0]
    dt = X.dtype
    _need("X", X, M * d, dt)
    _need("W2s", W2s, n * f * d, dt)
    for name, t in (("A", A), ("H", H)):
        _need(name, t, n * M * f, dt)
    _need("dY", dY, M * d, dt)
    _need("dX", dX, n * M * d, dt)
    _need("dW1s", dW1s, n * d * f, _f32())
    _need("dW2s", dW2s, n * f * d, _f32())
    _check(lib().tp_mlp_bwd_shards(_stream(stream), _dt(X), n, M, d, f, _ptr(X), _ptr(W1s), _ptr(W2s), _ptr(A),
                                   _ptr(H), _ptr(dY), _ptr(dX), _ptr(dW1s), _ptr(dW2s), _ptr(ws),
                                   ws.numel() * ws.element_size()))


def tp_swiglu_fwd(X, W1, W3, W2, G, U, H, Z, stream=None) -> None:
    M, d = X.shape
    f = W1.shape[1]
    dt = X.dtype
    _need("W3", W3, d * f, dt)
    _need("W2", W2, f * d, dt)
    _need("G", G, M * f, dt, optional=True)
    _need("U", U, M * f, dt, optional=True)
    _need("H", H, M * f, dt)
    _need("Z", Z, M * d, dt)
    _check(lib().tp_swiglu_fwd(_stream(stream), _dt(X), M, d, f, _ptr(X), _ptr(W1), _ptr(W3), _ptr(W2),
                               _ptr(G), _ptr(U), _ptr(H), _ptr(Z)))


def tp_swiglu_bwd_workspace_bytes(dtype: int, M: int, d: int, f: int) -> int:
    return lib().tp_swiglu_bwd_workspace_bytes(dtype, M, d, f)


def tp_swiglu_bwd(X, W1, W3, W2, G, U, H, dY, dX, dW1, dW3, dW2, ws, stream=None) -> None:
    M, d = X.shape
    f = W1.shape[1]
    dt = X.dtype
    _need("W3", W3, d * f, dt)
    _need("W2", W2, f * d, dt)
    for name, t in (("G", G), ("U", U), ("H", H)):
        _need(name, t, M * f, dt)
    for name, t in (("dY", dY), ("dX", dX)):
        _need(name, t, M * d, dt)
    _need("dW1", dW1, d * f, _f32())
    _need("dW3", dW3, d * f, _f32())
    _need("dW2", dW2, f * d, _f32())
    _check(lib().tp_swiglu_bwd(_stream(stream), _dt(X), M, d, f, _ptr(X), _ptr(W1), _ptr(W3), _ptr(W2),
                               _ptr(G), _ptr(U), _ptr(H), _ptr(dY), _ptr(dX), _ptr(dW1), _ptr(dW3),
                               _ptr(dW2), _ptr(ws), ws.numel() * ws.element_size()))


def _attn_need(X, Wq, Wk, Wv, Wo, Q, K, V, O, b, s, h_local, h_kv, d_head, L=None, L_optional=True):
    M, d = X.shape
    if M != b * s:
        raise ValueError(f"X has {M} rows, b*s is {b * s}")
    dt = X.dtype
    N, Nkv = h_local * d_head, h_kv * d_head
    _need("Wq", Wq, d * N, dt)
    _need("Wk", Wk, d * Nkv, dt)
    _need("Wv", Wv, d * Nkv, dt)
    _need("Wo", Wo, N * d, dt)
    _need("Q", Q, b * h_local * s * d_head, dt)
    _need("K", K, b * h_kv * s * d_head, dt)
    _need("V", V, b * h_kv * s * d_head, dt)
    _need("O", O, M * N, dt)
    _need("L", L, b * h_local * s, _f32(), optional=L_optional)
    return M, d, N, Nkv


def _attn_grads_need(dt, M, d, N, Nkv, dY, dX, dWq, dWk, dWv, dWo):
    _need("dY", dY, M * d, dt)
    _need("dX", dX, M * d, dt)
    _need("dWq", dWq, d * N, _f32())
    _need("dWk", dWk, d * Nkv, _f32())
    _need("dWv", dWv, d * Nkv, _f32())
    _need("dWo", dWo, N * d, _f32())


def tp_attn_shard_fwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, Z, b: int, s: int, h_local: int, d_head: int,
                      causal: bool = True, scale: float = 0.0, L=None, stream=None) -> None:
    M, d, _, _ = _attn_need(X, Wq, Wk, Wv, Wo, Q, K, V, O, b, s, h_local, h_local, d_head, L)
    _need("Z", Z, M * d, X.dtype)
    _check(lib().tp_attn_shard_fwd(_stream(stream), _dt(X), b, s, d, h_local, d_head, int(causal),
                                   float(scale), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                   _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(Z), _ptr(L)))


def tp_attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, Z, b: int, s: int, h_local: int, h_kv_local: int,
                          d_head: int, causal: bool = True, scale: float = 0.0, L=None, stream=None) -> None:
    M, d, _, _ = _attn_need(X, Wq, Wk, Wv, Wo, Q, K, V, O, b, s, h_local, h_kv_local, d_head, L)
    _need("Z", Z, M * d, X.dtype)
    _check(lib().tp_attn_gqa_shard_fwd(_stream(stream), _dt(X), b, s, d, h_local, h_kv_local, d_head, int(causal),
                                       float(scale), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                       _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(Z), _ptr(L)))


def tp_attn_shard_bwd_workspace_bytes(dtype: int, b: int, s: int, d: int, h_local: int, d_head: int) -> int:
    return lib().tp_attn_shard_bwd_workspace_bytes(dtype, b, s, d, h_local, d_head)


def tp_attn_shard_bwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, L, dY, dX, dWq, dWk, dWv, dWo, ws, b: int, s: int,
                      h_local: int, d_head: int, causal: bool = True, scale: float = 0.0, stream=None) -> None:
    M, d, N, Nkv = _attn_need(X, Wq, Wk, Wv, Wo, Q, K, V, O, b, s, h_local, h_local, d_head, L, L_optional=False)
    _attn_grads_need(X.dtype, M, d, N, Nkv, dY, dX, dWq, dWk, dWv, dWo)
    _check(lib().tp_attn_shard_bwd(_stream(stream), _dt(X), b, s, d, h_local, d_head, int(causal),
                                   float(scale), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                   _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dY), _ptr(dX),
                                   _ptr(dWq), _ptr(dWk), _ptr(dWv), _ptr(dWo), _ptr(ws),
                                   ws.numel() * ws.element_size()))


def tp_attn_gqa_shard_bwd_workspace_bytes(dtype: int, b: int, s: int, d: int, h_local: int, h_kv_local: int,
                                          d_head: int) -> int:
    return lib().tp_attn_gqa_shard_bwd_workspace_bytes(dtype, b, s, d, h_local, h_kv_local, d_head)


def tp_attn_gqa_shard_bwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, L, dY, dX, dWq, dWk, dWv, dWo, ws, b: int, s: int,
                          h_local: int, h_kv_local: int, d_head: int, causal: bool = True, scale: float = 0.0,
                          stream=None) -> None:
    M, d, N, Nkv = _attn_need(X, Wq, Wk, Wv, Wo, Q, K, V, O, b, s, h_local, h_kv_local, d_head, L,
                              L_optional=False)
    _attn_grads_need(X.dtype, M, d, N, Nkv, dY, dX, dWq, dWk, dWv, dWo)
    _check(lib().tp_attn_gqa_shard_bwd(_stream(stream), _dt(X), b, s, d, h_local, h_kv_local, d_head, int(causal),
                                       float(scale), _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                       _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dY), _ptr(dX),
                                       _ptr(dWq), _ptr(dWk), _ptr(dWv), _ptr(dWo), _ptr(ws),
                                       ws.numel() * ws.element_size()))


def tp_shard_reduce(partials, out, n_shards: int, numel: int, shard_stride: Optional[int] = None,
                    bias=None, stream=None) -> None:
    """out[e] = sum_i partials[i*stride + e] (+ bias[e % len(bias)])."""
    stride = numel if shard_stride is None else shard_stride
    _need("partials", partials, (n_shards - 1) * stride + numel, at_least=True)
    _need("out", out, numel, at_least=True)
    if bias is not None and bias.dtype != partials.dtype:
        raise ValueError(f"bias is {bias.dtype}, the partials are {partials.dtype}")
    _check(lib().tp_shard_reduce(_stream(stream), _dt(partials), _dt(out), n_shards, numel, _ptr(partials),
                                 stride, _ptr(bias), 0 if bias is None else bias.numel(), _ptr(out)))


def tp_sp_reduce_scatter_ln(partials, residual, gamma, beta, h_out, x_out, n_shards: int, index: int,
                            rows: int, cols: int, shard_stride: Optional[int] = None, bias=None, keep=None,
                            p_drop: float = 0.0, eps: float = 1e-5, stream=None) -> None:
    """Stripe `index` of sum_i partials_i (+ bias), inverted dropout with the
    uint8 mask `keep`, + residual -> h_out, LayerNorm(h) -> x_out."""
    import torch
    if keep is not None and keep.dtype != torch.uint8:
        raise TypeError("keep must be a uint8 tensor")
    stride = rows * cols if shard_stride is None else shard_stride
    dt, k = partials.dtype, rows // n_shards if n_shards > 0 else 0
    _need("partials", partials, (n_shards - 1) * stride + rows * cols, at_least=True)
    for name, t in (("residual", residual), ("h_out", h_out), ("x_out", x_out)):
        _need(name, t, k * cols, dt)
    for name, t in (("gamma", gamma), ("beta", beta)):
        _need(name, t, cols, dt)
    _need("bias", bias, cols, dt, optional=True)
    _need("keep", keep, k * cols, optional=True)
    _check(lib().tp_sp_reduce_scatter_ln(_stream(stream), _dt(partials), n_shards, rows, cols, index,
                                         _ptr(partials), stride, _ptr(bias), _ptr(residual), _ptr(keep),
                                         float(p_drop), _ptr(gamma), _ptr(beta), float(eps), _ptr(h_out),
                                         _ptr(x_out)))


def tp_sp_ln_bwd_workspace_bytes(dtype: int, n_shards: int, rows: int, cols: int) -> int:
    return lib().tp_sp_ln_bwd_workspace_bytes(dtype, n_shards, rows, cols)


def tp_sp_ln_bwd_reduce_scatter(dx_partials, h, gamma, dh_out, dy_out, dgamma, dbeta, ws, n_shards: int,
                                index: int, rows: int, cols: int, shard_stride: Optional[int] = None, keep=None,
                                p_drop: float = 0.0, dres=None, dbias=None, eps: float = 1e-5,
                                stream=None) -> None:
    """Backward of tp_sp_reduce_scatter_ln on stripe `index`: the stripe's
    LayerNorm backward of the summed input gradients (+ dres) -> dh_out,
    dropout backward -> dy_out, and this stripe's gamma/beta/bias gradients."""
    import torch
    if keep is not None and keep.dtype != torch.uint8:
        raise TypeError("keep must be a uint8 tensor")
    stride = rows * cols if shard_stride is None else shard_stride
    dt, k = h.dtype, rows // n_shards if n_shards > 0 else 0
    _need("dx_partials", dx_partials, (n_shards - 1) * stride + rows * cols, dt, at_least=True)
    for name, t in (("h", h), ("dh_out", dh_out), ("dy_out", dy_out)):
        _need(name, t, k * cols, dt)
    _need("dres", dres, k * cols, dt, optional=True)
    _need("keep", keep, k * cols, optional=True)
    _need("gamma", gamma, cols, dt)
    for name, t in (("dgamma", dgamma), ("dbeta", dbeta)):
        _need(name, t, cols, _f32())
    _need("dbias", dbias, cols, _f32(), optional=True)
    _check(lib().tp_sp_ln_bwd_reduce_scatter(_stream(stream), _dt(h), n_shards, rows, cols, index,
                                             _ptr(dx_partials), stride, _ptr(h), _ptr(gamma), float(eps), _ptr(keep),
                                             float(p_drop), _ptr(dres), _ptr(dh_out), _ptr(dy_out), _ptr(dgamma),
                                             _ptr(dbeta), _ptr(dbias), _ptr(ws), ws.numel() * ws.element_size()))


def tp_sp_all_gather(stripes, full, stream=None) -> None:
    """full = concatenation of the [stripe_rows x cols] stripes along rows.
    A stripe that is already the matching row block of `full` (a view at
    its place) is not copied."""
    n = len(stripes)
    rows, cols = stripes[0].shape
    for j, t in enumerate(stripes):
        _need(f"stripes[{j}]", t, rows * cols, full.dtype)
    _need("full", full, n * rows * cols)
    arr = (_p * n)(*[_ptr(t) for t in stripes])
    _check(lib().tp_sp_all_gather(_stream(stream), _dt(full), n, rows, cols, arr, _ptr(full)))


def _ids(t):
    import torch
    if t.dtype != torch.int64:
        raise TypeError("token ids must be an int64 tensor")
    return _ptr(t)


def tp_vocab_embed_fwd(ids, E_local, Y, vocab_start: int, stream=None) -> None:
    """Y = this shard's partial of the input embedding (rows of E_local for
    the ids it holds, zero rows for the rest)."""
    vl, d = E_local.shape
    _need("Y", Y, ids.numel() * d, E_local.dtype)
    _check(lib().tp_vocab_embed_fwd(_stream(stream), _dt(E_local), ids.numel(), d, vl, vocab_start, _ids(ids),
                                    _ptr(E_local), _ptr(Y)))


def tp_vocab_embed_bwd(ids, dY, dE_local, vocab_start: int, stream=None) -> None:
    """dE_local[v] = sum of dY over the tokens whose id is vocab_start + v."""
    vl, d = dE_local.shape
    _need("dY", dY, ids.numel() * d)
    _need("dE_local", dE_local, vl * d, _f32())
    _check(lib().tp_vocab_embed_bwd(_stream(stream), _dt(dY), ids.numel(), d, vl, vocab_start, _ids(ids), _ptr(dY),
                                    _ptr(dE_local)))


def tp_vocab_ce_fwd_workspace_bytes(dtype: int, n_tokens: int, d: int, vocab_local: int) -> int:
    return lib().tp_vocab_ce_fwd_workspace_bytes(dtype, n_tokens, d, vocab_local)


def tp_vocab_ce_fwd(X, E_local, targets, logits, stats, vocab_start: int, ws=None, stream=None) -> None:
    """logits = X E_local^T and the per-token (max, sum-exp, target logit)."""
    n_tokens, d = X.shape
    vl = E_local.shape[0]
    _need("E_local", E_local, vl * d, X.dtype)
    _need("targets", targets, n_tokens)
    _need("logits", logits, n_tokens * vl, X.dtype)
    _need("stats", stats, n_tokens * 3, _f32())
    _check(lib().tp_vocab_ce_fwd(_stream(stream), _dt(X), n_tokens, d, vl, vocab_start, _ptr(X), _ptr(E_local),
                                 _ids(targets), _ptr(logits), _ptr(stats), _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size()))


def tp_vocab_ce_combine(stats, loss, lse, stream=None) -> None:
    """stats [n_shards x n_tokens x 3] fp32 -> per-token loss and log-sum-exp."""
    n, n_tokens = stats.shape[0], stats.shape[1]
    _need("stats", stats, n * n_tokens * 3, _f32())
    _need("loss", loss, n_tokens, _f32())
    _need("lse", lse, n_tokens, _f32())
    _check(lib().tp_vocab_ce_combine(_stream(stream), n, n_tokens, _ptr(stats), n_tokens * 3, _ptr(loss),
                                     _ptr(lse)))


def tp_vocab_ce_bwd_workspace_bytes(dtype: int, n_tokens: int, d: int, vocab_local: int) -> int:
    return lib().tp_vocab_ce_bwd_workspace_bytes(dtype, n_tokens, d, vocab_local)


def tp_vocab_ce_bwd(X, E_local, targets, logits, lse, dloss, dX, dE, ws, vocab_start: int, stream=None) -> None:
    n_tokens, d = X.shape
    vl = E_local.shape[0]
    _need("E_local", E_local, vl * d, X.dtype)
    _need("targets", targets, n_tokens)
    _need("logits", logits, n_tokens * vl, X.dtype)
    for name, t in (("lse", lse), ("dloss", dloss)):
        _need(name, t, n_tokens, _f32())
    _need("dX", dX, n_tokens * d, X.dtype)
    _need("dE", dE, vl * d, _f32())
    _check(lib().tp_vocab_ce_bwd(_stream(stream), _dt(X), n_tokens, d, vl, vocab_start, _ptr(X), _ptr(E_local),
                                 _ids(targets), _ptr(logits), _ptr(lse), _ptr(dloss), _ptr(dX), _ptr(dE),
                                 _ptr(ws), ws.numel() * ws.element_size()))
