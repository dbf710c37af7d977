"""fp64 CPU oracle for one GPU's shard of a Megatron-LM tensor-parallel layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Everything here is the plain definition written out in numpy float64
(``np.matmul`` is the only library step, plus ``scipy.special.erf``); there is
no tiling, fusion or reordering.  Sources (the pages these definitions come
from):

* [JY] "Parallelism on Jiang Yi's Homepage", note "megatron-lm": sections
  FFN (Y = GeLU(X W1) W2, the column split of W1 and the row split of W2, the
  f/g table, the SwiGLU split), Attention (per-head outputs, O = [o_1..o_h] W_O),
  Embedding (the vocabulary split of the input embedding with its all-reduce,
  the output embedding fused with the cross-entropy) and Implementation
  (ParallelEmbedding: mask, shift, look up, zero the masked rows).
* [HC] "Splitting the model: five parallelisms and the traffic they make",
  section 3.4 "Tensor parallelism", Figures 3.4-3.6 (Z = sum_k Z_k; g
  all-reduces the partial sums forward, f all-reduces dX backward; heads are
  assigned to GPUs in contiguous groups).
* [BM] "tensor-parallelism" (brunomaga.github.io), section "Megatron-LM tensor
  parallelism" (Megatron_f / Megatron_g, the feed-forward block with its bias
  added after the reduction, the attention block with its causal mask and
  1/sqrt(head_dim) scale).
* [DW] "Chapter 8: Distributed Training", section 8.4.2 NCCL (all-reduce SUM).

Readings taken where the pages are silent or garbled are listed in the
repository's design notes; the ones that change arithmetic are: the exact
erf form of GeLU, 1/sqrt(d_h) as the softmax scale ([JY]'s attention equation
prints d_h without the root), W1 as the Swish'd gate of SwiGLU, the causal
mask keeping u <= t, and weights laid out [in x out] with Y = X W.

Every function returns float64 arrays.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

try:  # scipy's erfc; math.erfc is the fallback and the brute-force cross-check
    from scipy.special import erfc as _erfc
except Exception:  # pragma: no cover
    _erfc = np.vectorize(math.erfc, otypes=[np.float64])

__all__ = [
    "gelu", "gelu_prime", "swish", "swish_prime",
    "mlp_shard_fwd", "mlp_shard_bwd", "mlp_unsharded", "mlp_unsharded_bwd",
    "swiglu_shard_fwd", "swiglu_shard_bwd", "swiglu_unsharded",
    "attn_shard_fwd", "attn_unsharded", "attn_core", "attn_core_lse", "attn_core_bwd", "attn_shard_bwd",
    "attn_gqa_shard_fwd", "attn_gqa_query_rows", "attn_gqa_shard_bwd",
    "shard_reduce", "shard_range",
    "stripe_rows", "reduce_scatter", "all_gather", "layer_norm", "sp_block_end", "layer_norm_bwd",
    "sp_block_end_bwd",
    "vocab_embed_shard", "vocab_embed", "vocab_embed_shard_bwd", "vocab_ce_shard", "vocab_ce_combine", "vocab_ce_fwd",
    "vocab_ce_shard_bwd",
]

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Activations.  GeLU is named on the pages ([JY] FFN; [HC] 3.4; [BM] MLP
# block) and called as PyTorch's default (erf) form in the code listings.
# ----------------------------------------------------------------------------

def _norm_cdf(x):
    """Phi(x) = (1 + erf(x / sqrt 2)) / 2, written as erfc(-x / sqrt 2) / 2: the
    same function, without the cancellation of 1 + erf in the lower tail
    (below x = -6 the sum rounds to 0 in fp64 while Phi(-10) is 7.6e-24)."""
    return 0.5 * _erfc(-_f64(x) / _SQRT2)


def gelu(x):
    """GeLU(x) = x * Phi(x), Phi the standard normal CDF (exact erf form)."""
    x = _f64(x)
    return x * _norm_cdf(x)


def gelu_prime(x):
    """dGeLU/dx = Phi(x) + x * phi(x), phi the standard normal density."""
    x = _f64(x)
    return _norm_cdf(x) + x * _INV_SQRT_2PI * np.exp(-0.5 * x * x)


def _sigmoid(x):
    x = _f64(x)
    # exp of a non-positive argument only: no overflow for large |x|
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def swish(x):
    """Swish(x) = x * sigmoid(x) ([JY] SwiGLU section; ``F.silu`` in its code)."""
    x = _f64(x)
    return x * _sigmoid(x)


def swish_prime(x):
    """dSwish/dx = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    x = _f64(x)
    s = _sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ----------------------------------------------------------------------------
# GeLU MLP shard.  [JY] FFN: W1 = [W11, W12] split by columns, GeLU applied
# per slice, W2 split by rows, Y = sum_i GeLU(X W1_i) W2_i.  [HC] Figure 3.4.
# ----------------------------------------------------------------------------

def mlp_shard_fwd(X, W1_i, W2_i) -> Dict[str, np.ndarray]:
    """A_i = X W1_i; H_i = GeLU(A_i); Z_i = H_i W2_i (this shard's summand)."""
    X, W1_i, W2_i = _f64(X), _f64(W1_i), _f64(W2_i)
    A = X @ W1_i
    H = gelu(A)
    Z = H @ W2_i
    return {"A": A, "H": H, "Z": Z}


def mlp_shard_bwd(X, W1_i, W2_i, dY) -> Dict[str, np.ndarray]:
    """Gradients of this shard given the full upstream gradient dY.

    g is the identity in the backward pass ([JY] f/g table; [BM] Megatron_g),
    so every shard sees the whole dY.  Chain rule through Z_i = GeLU(X W1_i) W2_i:
    dH = dY W2_i^T, dA = dH * GeLU'(A), dW2_i = H^T dY, dW1_i = X^T dA,
    dX_i = dA W1_i^T (the summand that f all-reduces, [HC] 3.4).
    """
    X, W1_i, W2_i, dY = _f64(X), _f64(W1_i), _f64(W2_i), _f64(dY)
    A = X @ W1_i
    H = gelu(A)
    dH = dY @ W2_i.T
    dA = dH * gelu_prime(A)
    return {"dH": dH, "dA": dA, "dW2": H.T @ dY, "dW1": X.T @ dA, "dX": dA @ W1_i.T}


def mlp_unsharded(X, W1, W2) -> np.ndarray:
    """Y = GeLU(X W1) W2 on one device ([JY] FFN, first equation)."""
    return gelu(_f64(X) @ _f64(W1)) @ _f64(W2)


def mlp_unsharded_bwd(X, W1, W2, dY) -> Dict[str, np.ndarray]:
    """Unsharded gradients of Y = GeLU(X W1) W2."""
    return mlp_shard_bwd(X, W1, W2, dY)


# ----------------------------------------------------------------------------
# SwiGLU shard.  [JY] FFN, SwiGLU part: Y = (X W3 (.) Swish(X W1)) W2 with
# W1, W3 split by columns and W2 by rows; the code computes
# w2(silu(w1(x)) * w3(x)), so W1 is the Swish'd gate and W3 the multiplier.
# ----------------------------------------------------------------------------

def swiglu_shard_fwd(X, W1_i, W3_i, W2_i) -> Dict[str, np.ndarray]:
    """G = X W1_i; U = X W3_i; H = Swish(G) * U; Z_i = H W2_i."""
    X = _f64(X)
    G = X @ _f64(W1_i)
    U = X @ _f64(W3_i)
    H = swish(G) * U
    Z = H @ _f64(W2_i)
    return {"G": G, "U": U, "H": H, "Z": Z}


def swiglu_shard_bwd(X, W1_i, W3_i, W2_i, dY) -> Dict[str, np.ndarray]:
    """dH = dY W2_i^T; dU = dH * Swish(G); dG = dH * U * Swish'(G);
    dW2 = H^T dY; dW1 = X^T dG; dW3 = X^T dU; dX_i = dG W1_i^T + dU W3_i^T."""
    X, W1_i, W3_i, W2_i, dY = map(_f64, (X, W1_i, W3_i, W2_i, dY))
    G = X @ W1_i
    U = X @ W3_i
    H = swish(G) * U
    dH = dY @ W2_i.T
    dU = dH * swish(G)
    dG = dH * U * swish_prime(G)
    return {"dH": dH, "dG": dG, "dU": dU, "dW2": H.T @ dY, "dW1": X.T @ dG,
            "dW3": X.T @ dU, "dX": dG @ W1_i.T + dU @ W3_i.T}


def swiglu_unsharded(X, W1, W3, W2) -> np.ndarray:
    X = _f64(X)
    return (swish(X @ _f64(W1)) * (X @ _f64(W3))) @ _f64(W2)


# ----------------------------------------------------------------------------
# Attention head-group shard.  [JY] Attention: o_i = softmax(Q_i K_i^T / s) V_i,
# O = [o_1..o_h] W_O.  [BM] Megatron_MHA: Q/K/V column-parallel by heads,
# local causal softmax with masked_fill(tril == 0, -inf), scale head_dim^-0.5,
# heads concatenated in order, row-parallel output projection.  [HC] Figure
# 3.5: shard i owns a contiguous group of heads.
# ----------------------------------------------------------------------------

def attn_core(Q, K, V, causal: bool = True, scale: Optional[float] = None) -> np.ndarray:
    """softmax(Q K^T * scale, masked) V for one head; Q, K, V are [s x d_h].

    Masked entries (u > t when causal) are -inf before the softmax, so they
    get weight exactly zero.  The softmax is taken directly over the row.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    s, dh = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    S = (Q @ K.T) * scale
    if causal:
        S = np.where(np.tril(np.ones((s, K.shape[0]), dtype=bool)), S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=1, keepdims=True)
    return P @ V


def attn_core_lse(Q, K, V, causal: bool = True, scale: Optional[float] = None):
    """attn_core plus the log-sum-exp of each query's scaled, masked scores:
    L_t = log sum_{u allowed} exp(S[t, u]), so that P[t, u] = exp(S[t, u] - L_t)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    s, dh = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    S = (Q @ K.T) * scale
    if causal:
        S = np.where(np.tril(np.ones((s, K.shape[0]), dtype=bool)), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    tot = E.sum(axis=1, keepdims=True)
    L = (m + np.log(tot))[:, 0]
    return (E / tot) @ V, L


def attn_core_bwd(Q, K, V, dO, causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gradients of O = softmax(mask(Q K^T * scale)) V for one head, by the
    chain rule on that definition: with P the softmax,
      dV = P^T dO,  dP = dO V^T,
      dS = P * (dP - rowsum(P * dP))     (the softmax Jacobian applied row by row),
      dQ = dS K * scale,  dK = dS^T Q * scale.
    Masked entries have P = 0 and so carry no gradient."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    s, dh = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    S = (Q @ K.T) * scale
    if causal:
        S = np.where(np.tril(np.ones((s, K.shape[0]), dtype=bool)), S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return {"dQ": dS @ K * scale, "dK": dS.T @ Q * scale, "dV": dV}


def _split_heads(T, b, s, h, dh):
    return T.reshape(b, s, h, dh).transpose(0, 2, 1, 3)


def attn_shard_fwd(X, Wq, Wk, Wv, Wo, b: int, s: int, h_local: int, d_head: int,
                   causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """One shard's attention: returns Q, K, V as [b, h_l, s, d_h], the
    concatenated head outputs O [b*s, h_l*d_h], the partial Z = O W_O,i and
    the per-query log-sum-exp L [b, h_l, s] (natural log, of the scaled,
    masked scores).

    Local head j uses columns [j*d_h, (j+1)*d_h) of the shard's W_Q/W_K/W_V
    and rows [j*d_h, (j+1)*d_h) of its W_O slice.
    """
    X = _f64(X).reshape(b, s, -1)
    hd = h_local * d_head
    Q = _split_heads(X @ _f64(Wq), b, s, h_local, d_head)
    K = _split_heads(X @ _f64(Wk), b, s, h_local, d_head)
    V = _split_heads(X @ _f64(Wv), b, s, h_local, d_head)
    O = np.empty((b, s, h_local, d_head))
    L = np.empty((b, h_local, s))
    for bi in range(b):
        for j in range(h_local):
            O[bi, :, j, :], L[bi, j] = attn_core_lse(Q[bi, j], K[bi, j], V[bi, j], causal, scale)
    O = O.reshape(b * s, hd)
    Z = O @ _f64(Wo)
    return {"Q": Q, "K": K, "V": V, "O": O, "Z": Z, "L": L}


def attn_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b: int, s: int, h_local: int, d_head: int,
                   causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Backward of one attention shard ([BM] Megatron_MHA: the input passes
    Megatron_f, identity forward, so dX is this shard's summand of the full
    dX and is summed over shards (the f all-reduce, [HC] 3.4); Z's gradient
    is the full upstream dY because g's backward is the identity).

      dO = dY W_O^T,  dW_O = O^T dY                      (row-parallel product)
      per head: dQ, dK, dV from attn_core_bwd
      dX = dQ W_Q^T + dK W_K^T + dV W_V^T                 (this shard's partial)
      dW_Q = X^T dQ,  dW_K = X^T dK,  dW_V = X^T dV       (column slices)

    dQ, dK, dV are returned token-major [b*s, h_l*d_h] like O.
    """
    f = attn_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, h_local, d_head, causal, scale)
    X2 = _f64(X).reshape(b * s, -1)
    dY = _f64(dY)
    hd = h_local * d_head
    dO = dY @ _f64(Wo).T
    dOh = _split_heads(dO, b, s, h_local, d_head)
    dQ = np.empty((b, s, h_local, d_head))
    dK = np.empty_like(dQ)
    dV = np.empty_like(dQ)
    for bi in range(b):
        for j in range(h_local):
            g = attn_core_bwd(f["Q"][bi, j], f["K"][bi, j], f["V"][bi, j], dOh[bi, j], causal, scale)
            dQ[bi, :, j, :], dK[bi, :, j, :], dV[bi, :, j, :] = g["dQ"], g["dK"], g["dV"]
    dQ, dK, dV = (t.reshape(b * s, hd) for t in (dQ, dK, dV))
    return {"dO": dO, "dQ": dQ, "dK": dK, "dV": dV,
            "dX": dQ @ _f64(Wq).T + dK @ _f64(Wk).T + dV @ _f64(Wv).T,
            "dWq": X2.T @ dQ, "dWk": X2.T @ dK, "dWv": X2.T @ dV, "dWo": f["O"].T @ dY}


def attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, b: int, s: int, h_local: int, h_kv: int, d_head: int,
                       causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Grouped-query attention shard ([HC] 3.4, the Llama-3 example: the
    shard's query heads share its key/value heads in equal groups).  Query
    head j uses columns [j*d_h, (j+1)*d_h) of W_Q and K/V head j // (h_local /
    h_kv), i.e. columns [g*d_h, (g+1)*d_h) of W_K and W_V; everything else is
    attn_shard_fwd.  Returns Q [b, h_local, s, d_h], K and V [b, h_kv, s, d_h],
    O, Z and L as attn_shard_fwd."""
    assert h_local % h_kv == 0
    group = h_local // h_kv
    X = _f64(X).reshape(b, s, -1)
    Q = _split_heads(X @ _f64(Wq), b, s, h_local, d_head)
    K = _split_heads(X @ _f64(Wk), b, s, h_kv, d_head)
    V = _split_heads(X @ _f64(Wv), b, s, h_kv, d_head)
    O = np.empty((b, s, h_local, d_head))
    L = np.empty((b, h_local, s))
    for bi in range(b):
        for j in range(h_local):
            O[bi, :, j, :], L[bi, j] = attn_core_lse(Q[bi, j], K[bi, j // group], V[bi, j // group], causal, scale)
    O = O.reshape(b * s, h_local * d_head)
    return {"Q": Q, "K": K, "V": V, "O": O, "Z": O @ _f64(Wo), "L": L}


def attn_gqa_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b: int, s: int, h_local: int, h_kv: int, d_head: int,
                       causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Backward of the grouped-query shard: attn_shard_bwd's chain rule with
    query head j reading K/V head j // (h_local / h_kv).  A K/V head feeds
    every query head of its group, so its dK and dV are the sums of the
    group's per-head contributions.  dQ is [b*s, h_local*d_h]; dK and dV are
    [b*s, h_kv*d_h]; dX, dW_Q, dW_K, dW_V, dW_O as attn_shard_bwd."""
    assert h_local % h_kv == 0
    group = h_local // h_kv
    f = attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, h_local, h_kv, d_head, causal, scale)
    X2 = _f64(X).reshape(b * s, -1)
    dY = _f64(dY)
    dO = dY @ _f64(Wo).T
    dOh = _split_heads(dO, b, s, h_local, d_head)
    dQ = np.zeros((b, s, h_local, d_head))
    dK = np.zeros((b, s, h_kv, d_head))
    dV = np.zeros((b, s, h_kv, d_head))
    for bi in range(b):
        for j in range(h_local):
            g = attn_core_bwd(f["Q"][bi, j], f["K"][bi, j // group], f["V"][bi, j // group], dOh[bi, j], causal,
                              scale)
            dQ[bi, :, j, :] = g["dQ"]
            dK[bi, :, j // group, :] += g["dK"]
            dV[bi, :, j // group, :] += g["dV"]
    dQ = dQ.reshape(b * s, h_local * d_head)
    dK, dV = (t.reshape(b * s, h_kv * d_head) for t in (dK, dV))
    return {"dO": dO, "dQ": dQ, "dK": dK, "dV": dV,
            "dX": dQ @ _f64(Wq).T + dK @ _f64(Wk).T + dV @ _f64(Wv).T,
            "dWq": X2.T @ dQ, "dWk": X2.T @ dK, "dWv": X2.T @ dV, "dWo": f["O"].T @ dY}


def attn_gqa_query_rows(Xb, Wq, Wk, Wv, Wo, rows, h_local: int, h_kv: int, d_head: int,
                        causal: bool = True, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """attn_gqa_shard_fwd for one batch row Xb [s x d], evaluated only at the
    query positions `rows` (each query still sees every allowed key of the
    row): O[rows] and Z[rows], by the same definitions."""
    Xb = _f64(Xb)
    rows = np.asarray(rows)
    s = Xb.shape[0]
    group = h_local // h_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d_head)
    Qr = (Xb[rows] @ _f64(Wq)).reshape(len(rows), h_local, d_head)
    K = (Xb @ _f64(Wk)).reshape(s, h_kv, d_head)
    V = (Xb @ _f64(Wv)).reshape(s, h_kv, d_head)
    O = np.empty((len(rows), h_local, d_head))
    for j in range(h_local):
        Kj, Vj = K[:, j // group], V[:, j // group]
        S = (Qr[:, j] @ Kj.T) * scale
        if causal:
            S = np.where(np.arange(s)[None, :] <= rows[:, None], S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        O[:, j] = (P / P.sum(axis=1, keepdims=True)) @ Vj
    O = O.reshape(len(rows), h_local * d_head)
    return {"O": O, "Z": O @ _f64(Wo)}


def attn_unsharded(X, Wq, Wk, Wv, Wo, b: int, s: int, heads: int, d_head: int,
                   causal: bool = True) -> Dict[str, np.ndarray]:
    """All heads on one device: O = [o_1..o_h] W_O ([JY] Attention)."""
    return attn_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, heads, d_head, causal)


# ----------------------------------------------------------------------------
# Shard-reduce: the sum that g performs in the forward pass and f in the
# backward pass ([JY] f/g table; [HC] 3.4 Z = sum_k Z_k; [DW] 8.4.2 all_reduce
# with ReduceOp.SUM).  The row-parallel bias is added once, after the sum
# ([BM] Megatron_FeedForward: the bias is added after Megatron_g).
# ----------------------------------------------------------------------------

def shard_reduce(partials: Sequence, bias=None) -> np.ndarray:
    """out = sum_i P_i (+ bias broadcast over the trailing dimension, once)."""
    P = [_f64(p) for p in partials]
    out = np.zeros_like(P[0])
    for p in P:
        out = out + p
    if bias is not None:
        bias = _f64(bias).reshape(-1)
        flat = out.reshape(-1)
        flat += np.resize(bias, flat.shape)   # element e gets bias[e % len]
        out = flat.reshape(out.shape)
    return out


# ----------------------------------------------------------------------------
# Sequence parallelism ([HC] 3.4, Figure 3.7; [BM] "Sharding activations to
# reduce memory"): the all-reduce at g becomes a reduce-scatter that sums the
# partial outputs and leaves each GPU one stripe of tokens, dropout and the
# residual add run on that stripe, then LayerNorm for the next block, and an
# all-gather rebuilds the full input.  all-reduce = reduce-scatter + all-gather.
# ----------------------------------------------------------------------------

def stripe_rows(rows: int, n_shards: int, index: int):
    """Token stripe `index` of `rows` tokens over n_shards GPUs (contiguous, equal)."""
    return shard_range(rows, n_shards, index)


def reduce_scatter(partials: Sequence, n_shards: int, index: int, bias=None) -> np.ndarray:
    """Stripe `index` of sum_i P_i (rows split equally and contiguously), plus
    the bias once."""
    P = [_f64(p) for p in partials]
    r0, k = stripe_rows(P[0].shape[0], n_shards, index)
    return shard_reduce([p[r0:r0 + k] for p in P], bias)


def all_gather(stripes: Sequence) -> np.ndarray:
    """The stripes of every GPU stacked in order into the full tensor."""
    return np.concatenate([_f64(x) for x in stripes], axis=0)


def layer_norm(h, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """Per row: (h - mean) / sqrt(var + eps) * gamma + beta, var the biased
    (population) variance over the row."""
    h = _f64(h)
    mu = h.mean(axis=1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=1, keepdims=True)
    return (h - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def sp_block_end(partials: Sequence, n_shards: int, index: int, residual, gamma, beta, bias=None,
                 keep=None, p_drop: float = 0.0, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """One GPU's sequence-parallel block end on its stripe: y = the
    reduce-scattered sum (+ bias); inverted dropout with the given keep mask,
    y * keep / (1 - p); the residual stream h = residual + y; and x =
    LayerNorm(h), the stripe of the next block's input."""
    y = reduce_scatter(partials, n_shards, index, bias)
    if keep is not None:
        y = y * _f64(keep) / (1.0 - p_drop)
    h = _f64(residual) + y
    return {"h": h, "x": layer_norm(h, gamma, beta, eps)}

def layer_norm_bwd(dx, h, gamma, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """Backward of layer_norm by the chain rule on its definition, per row:
    with xhat = (h - mean) / sqrt(var + eps) and g = dx * gamma,
      dh = (g - mean(g) - xhat * mean(g * xhat)) / sqrt(var + eps),
      dgamma = sum over rows of dx * xhat,  dbeta = sum over rows of dx."""
    dx, h, gamma = _f64(dx), _f64(h), _f64(gamma)
    mu = h.mean(axis=1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (h - mu) * rstd
    g = dx * gamma
    dh = (g - g.mean(axis=1, keepdims=True) - xhat * (g * xhat).mean(axis=1, keepdims=True)) * rstd
    return {"dh": dh, "dgamma": (dx * xhat).sum(axis=0), "dbeta": dx.sum(axis=0)}


def sp_block_end_bwd(dx_partials: Sequence, n_shards: int, index: int, h, gamma, keep=None,
                     p_drop: float = 0.0, dres=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """Backward of sp_block_end on one GPU's stripe ([HC] Figure 3.7: the
    backward pass mirrors the forward, a reduce-scatter where the forward
    gathered).  dx: the stripe of the sum of every shard's gradient of the
    next block's input (reduce_scatter of the summands); h: the stripe's
    residual stream as the forward produced it; dres: gradient reaching h
    through the skip connection (or None).
      dh = LayerNorm backward of dx (+ dres)      -> the previous residual's gradient
      dy = dh * keep / (1 - p)                    -> the gradient of the reduce-scattered sum
      dbias = sum over the stripe's rows of dy; dgamma, dbeta this stripe's parts.
    Every shard's row-parallel partial then receives the all-gather of the
    stripes' dy as its output gradient."""
    dx = reduce_scatter(dx_partials, n_shards, index)
    ln = layer_norm_bwd(dx, h, gamma, eps)
    dh = ln["dh"] + (_f64(dres) if dres is not None else 0.0)
    dy = dh * _f64(keep) / (1.0 - p_drop) if keep is not None else dh
    return {"dh": dh, "dy": dy, "dbias": dy.sum(axis=0), "dgamma": ln["dgamma"], "dbeta": ln["dbeta"]}


# ----------------------------------------------------------------------------
# Vocabulary-parallel embeddings ([JY] Embedding and Implementation)
# ----------------------------------------------------------------------------

def vocab_embed_shard(ids, E_local, vocab_start: int) -> np.ndarray:
    """One shard's partial of the input embedding: the shard holds rows
    [vocab_start, vocab_start + V_local) of the table.  Ids outside that range
    are masked: they are shifted like the rest, looked up at row 0 and their
    output rows then set to zero; the others read row id - vocab_start."""
    ids = np.asarray(ids, dtype=np.int64)
    E = _f64(E_local)
    mask = (ids < vocab_start) | (ids >= vocab_start + E.shape[0])
    local = ids - vocab_start
    local[mask] = 0
    y = E[local]
    y[mask] = 0.0
    return y


def vocab_embed(ids, E_shards: Sequence) -> np.ndarray:
    """The input embedding over all shards: the all-reduce SUM of every
    shard's partial.  Shard i holds the i-th contiguous block of rows."""
    start, parts = 0, []
    for E in E_shards:
        parts.append(vocab_embed_shard(ids, E, start))
        start += np.asarray(E).shape[0]
    return shard_reduce(parts)


def vocab_embed_shard_bwd(ids, dY, vocab_local: int, vocab_start: int) -> np.ndarray:
    """Gradient of the shard's table rows: the forward's all-reduce has an
    identity backward, so every shard receives the whole output gradient dY
    and row v of dE_local is the sum of dY over the tokens whose id is
    vocab_start + v (ids outside the shard contribute nothing).  Summed in
    token order."""
    ids = np.asarray(ids, dtype=np.int64)
    dY = _f64(dY)
    dE = np.zeros((vocab_local, dY.shape[1]))
    for t, v in enumerate(ids):
        if vocab_start <= v < vocab_start + vocab_local:
            dE[v - vocab_start] += dY[t]
    return dE


def vocab_ce_shard(X, E_local, targets, vocab_start: int) -> Dict[str, np.ndarray]:
    """One shard's part of the output embedding fused with the cross-entropy:
    logits z = X E_local^T over the shard's V_local vocabulary columns, and per
    token the shard's three numbers: m = max_v z, s = sum_v exp(z - m), and
    z_t = the target's logit when the target falls in this shard (else 0)."""
    z = _f64(X) @ _f64(E_local).T
    t = np.asarray(targets, dtype=np.int64)
    m = z.max(axis=1)
    ssum = np.exp(z - m[:, None]).sum(axis=1)
    inside = (t >= vocab_start) & (t < vocab_start + z.shape[1])
    zt = np.zeros(z.shape[0])
    rows = np.nonzero(inside)[0]
    zt[rows] = z[rows, t[rows] - vocab_start]
    return {"logits": z, "m": m, "s": ssum, "zt": zt}


def vocab_ce_combine(stats: Sequence[Dict[str, np.ndarray]]) -> Dict[str, np.ndarray]:
    """The exchange of the fused cross-entropy: per token only (m, s, z_t) of
    each shard cross GPUs.  M = max_i m_i, S = sum_i s_i exp(m_i - M),
    log-sum-exp = M + log S, loss = log-sum-exp - sum_i z_t,i."""
    m = np.stack([_f64(st["m"]) for st in stats])
    ssum = np.stack([_f64(st["s"]) for st in stats])
    zt = np.stack([_f64(st["zt"]) for st in stats]).sum(axis=0)
    M = m.max(axis=0)
    S = (ssum * np.exp(m - M)).sum(axis=0)
    lse = M + np.log(S)
    return {"lse": lse, "loss": lse - zt}


def vocab_ce_fwd(X, E_shards: Sequence, targets) -> Dict[str, np.ndarray]:
    """Per-token cross-entropy of the vocabulary-parallel output embedding."""
    start, stats = 0, []
    for E in E_shards:
        stats.append(vocab_ce_shard(X, E, targets, start))
        start += np.asarray(E).shape[0]
    return vocab_ce_combine(stats)


def vocab_ce_shard_bwd(X, E_local, targets, vocab_start: int, lse, dloss) -> Dict[str, np.ndarray]:
    """Backward of one shard given the combined log-sum-exp and the upstream
    gradient of every token's loss: dz = (softmax(z) - onehot(target)) dloss
    on the shard's columns, dX_i = dz E_local (this shard's summand of dX),
    dE_local = dz^T X."""
    Xf, E = _f64(X), _f64(E_local)
    z = Xf @ E.T
    p = np.exp(z - _f64(lse)[:, None])
    t = np.asarray(targets, dtype=np.int64)
    inside = (t >= vocab_start) & (t < vocab_start + z.shape[1])
    rows = np.nonzero(inside)[0]
    p[rows, t[rows] - vocab_start] -= 1.0
    dz = p * _f64(dloss)[:, None]
    return {"dlogits": dz, "dX": dz @ E, "dE": dz.T @ Xf}



def shard_range(total: int, n_shards: int, index: int):
    """Contiguous equal split: shard ``index`` owns [index*k, (index+1)*k),
    k = total / n_shards.  Indivisible totals are an error, as the pages'
    listings assert ([JY] Implementation: divisibility asserts on features,
    heads and vocabulary; [BM] Megatron_MHA raises ValueError)."""
    if n_shards <= 0 or total <= 0 or not (0 <= index < n_shards):
        raise ValueError("bad shard arguments")
    if total % n_shards:
        raise ValueError(f"{total} is not divisible by {n_shards}")
    k = total // n_shards
    return index * k, k


def max_rel_err(y, ref) -> float:
    """||y - ref||_inf / ||ref||_inf over all elements (0 when both are 0)."""
    y, ref = _f64(y), _f64(ref)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def per_element_rel_err(y, ref, floor: float = 1e-3) -> float:
    """max_e |y_e - ref_e| / max(|ref_e|, floor * ||ref||_inf): the relative
    error of each element, with entries far below the tensor's largest
    measured against floor * ||ref||_inf instead of their own size."""
    y, ref = _f64(y), _f64(ref)
    if not ref.size:
        return 0.0
    big = float(np.max(np.abs(ref)))
    den = np.maximum(np.abs(ref), floor * big)
    num = np.abs(y - ref)
    if big == 0.0:
        return float(np.max(num))
    return float(np.max(num / den))


__all__ += ["max_rel_err", "per_element_rel_err"]
