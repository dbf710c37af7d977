"""Seeded synthetic inputs for one GPU's tensor-parallel shard.

This module only draws numbers and slices them. It holds none of the shard's
arithmetic, so both the fp64 oracle side and the HIP side take their inputs
from here without sharing any computation.

Workloads (the problem statement of the Megatron-LM reading note on
"Parallelism on Jiang Yi's Homepage", section FFN: X in R^{bs x d},
W1 in R^{d x d_ff}, W2 in R^{d_ff x d}; section Attention: W_Q, W_K, W_V in
R^{d x h d_h}):

* ``C1`` tiny fp32 GeLU MLP, 2 shards: X[32x64], W1[64x256], W2[256x64].
* ``C2`` GPT-2-medium-shaped bf16 MLP, b 8, s 1024, d 1024, d_ff 4096, 8 shards.
* ``C3`` SwiGLU bf16 shard, b 4, s 2048, d 4096, d_ff 11008, 4 shards.
* ``C4`` causal attention bf16 shard, b 4, s 2048, 32 heads of 128, 4 shards.
* ``C5`` large GeLU MLP bf16 shard, b 2, s 4096, d 8192, d_ff 32768, 8 shards.
* ``G1`` grouped-query causal attention bf16 shard shaped as the Llama-3-405B
  example of "Splitting the model" section 3.4 at TP 8: d 16384, 128 query
  heads and 8 key/value heads of 128, so one GPU holds 16 query heads sharing
  1 key/value head (W_Q [16384 x 2048], W_K and W_V [16384 x 128]); b 2,
  s 4096 like C5.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64); normals drawn in float64,
scaled by the stated standard deviation, cast to float32, and for bf16
workloads rounded to the nearest bf16 value (ties to even).  Draw order:
MLP X, W1, (W3), W2, dY; attention X, W_Q, W_K, W_V, W_O.  C1 and C2 draw the
full weight matrices and slice every shard from them; C3, C4 and C5 draw only
shard 0's slices (a shard's result does not depend on the other shards).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "round_to_bf16", "normal",
    "mlp_inputs", "swiglu_inputs", "attn_inputs", "reduce_inputs",
    "random_mlp", "random_swiglu", "random_attn", "gqa_inputs", "random_gqa",
    "sp_inputs", "random_sp", "vocab_inputs", "random_vocab", "zipf_token_ids",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "mlp" | "swiglu" | "attn" | "gqa" | "sp" | "vocab"
    dtype: str              # "f32" | "bf16"
    b: int
    s: int
    d: int
    n_shards: int
    d_ff: int = 0
    heads: int = 0
    d_head: int = 0
    kv_heads: int = 0            # grouped-query attention: key/value heads (0: = heads)
    w_std: float = 0.02
    p_drop: float = 0.0          # dropout probability (sequence-parallel block end)
    vocab: int = 0               # vocabulary rows of the embedding table (padded)
    vocab_used: int = 0          # ids drawn below this (the tokenizer's real vocabulary)
    full_weights: bool = False   # draw every shard's weights (else shard 0 only)
    backward: bool = True
    description: str = ""

    @property
    def M(self) -> int:
        return self.b * self.s

    @property
    def f_local(self) -> int:
        return self.d_ff // self.n_shards

    @property
    def h_local(self) -> int:
        return self.heads // self.n_shards

    @property
    def h_kv_local(self) -> int:
        return (self.kv_heads or self.heads) // self.n_shards


WORKLOADS: Dict[str, Workload] = {
    "C1": Workload("C1", "mlp", "f32", b=1, s=32, d=64, d_ff=256, n_shards=2,
                   w_std=0.02, full_weights=True,
                   description="tiny fp32 GeLU MLP, 2 shards of 128"),
    "C2": Workload("C2", "mlp", "bf16", b=8, s=1024, d=1024, d_ff=4096, n_shards=8,
                   w_std=0.02, full_weights=True,
                   description="GPT-2-medium-shaped GeLU MLP, TP 8, slice 512"),
    "C3": Workload("C3", "swiglu", "bf16", b=4, s=2048, d=4096, d_ff=11008, n_shards=4,
                   w_std=0.02, description="SwiGLU MLP shard, TP 4, slice 2752"),
    "C4": Workload("C4", "attn", "bf16", b=4, s=2048, d=4096, heads=32, d_head=128,
                   n_shards=4, w_std=0.02, backward=False,
                   description="causal self-attention, 8 of 32 heads of 128"),
    "C5": Workload("C5", "mlp", "bf16", b=2, s=4096, d=8192, d_ff=32768, n_shards=8,
                   w_std=0.01, description="large GeLU MLP shard, TP 8, slice 4096"),
    "G1": Workload("G1", "gqa", "bf16", b=2, s=4096, d=16384, heads=128, kv_heads=8, d_head=128,
                   n_shards=8, w_std=0.01, backward=False,
                   description="grouped-query causal attention shard, 16 query heads sharing 1 KV head"),
    "S1": Workload("S1", "sp", "bf16", b=2, s=4096, d=8192, n_shards=8, p_drop=0.1, backward=False,
                   description="sequence-parallel block end, 8192 tokens x 8192 over TP 8: "
                               "reduce-scatter to a 1024-token stripe, dropout, residual, LayerNorm"),
    "E1": Workload("E1", "vocab", "bf16", b=8, s=1024, d=1024, n_shards=8, vocab=51200, vocab_used=50257,
                   w_std=0.02,
                   description="vocabulary-parallel input embedding and output embedding + cross-entropy, "
                               "GPT-2-medium width, vocabulary 50257 padded to 51200, TP 8 -> 6400 rows here"),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, ties to even.

    Returns float32 values that are exactly representable in bf16. NaN and
    Inf are not expected from the generators and are not treated specially.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    """One N(0, std^2) draw in float64, cast to float32, rounded for bf16."""
    x = (rng.standard_normal(size=shape) * std).astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def _cols(w: np.ndarray, n: int, i: int) -> np.ndarray:
    k = w.shape[1] // n
    return np.ascontiguousarray(w[:, i * k:(i + 1) * k])


def _rows(w: np.ndarray, n: int, i: int) -> np.ndarray:
    k = w.shape[0] // n
    return np.ascontiguousarray(w[i * k:(i + 1) * k, :])


def mlp_inputs(wl: Workload, seed: int = 0) -> dict:
    """GeLU MLP inputs: X, dY and per-shard W1 column slices / W2 row slices.

    ``W1s[i]`` is [d x f_i] and ``W2s[i]`` is [f_i x d].  When the workload
    draws full weights, ``W1``/``W2`` hold the unsharded matrices too.
    """
    assert wl.kind == "mlp"
    rng = np.random.default_rng(seed)
    M, d = wl.M, wl.d
    f_draw = wl.d_ff if wl.full_weights else wl.f_local
    X = normal(rng, (M, d), 1.0, wl.dtype)
    W1 = normal(rng, (d, f_draw), wl.w_std, wl.dtype)
    W2 = normal(rng, (f_draw, d), wl.w_std, wl.dtype)
    dY = normal(rng, (M, d), 1.0, wl.dtype) if wl.backward else None
    out = {"X": X, "dY": dY}
    if wl.full_weights:
        out["W1"], out["W2"] = W1, W2
        out["W1s"] = [_cols(W1, wl.n_shards, i) for i in range(wl.n_shards)]
        out["W2s"] = [_rows(W2, wl.n_shards, i) for i in range(wl.n_shards)]
    else:
        out["W1s"], out["W2s"] = [W1], [W2]
    return out


def swiglu_inputs(wl: Workload, seed: int = 0) -> dict:
    """SwiGLU inputs: X, shard W1 (gate, the Swish'd one), W3 (up), W2, dY."""
    assert wl.kind == "swiglu"
    rng = np.random.default_rng(seed)
    M, d, f = wl.M, wl.d, wl.f_local
    X = normal(rng, (M, d), 1.0, wl.dtype)
    W1 = normal(rng, (d, f), wl.w_std, wl.dtype)
    W3 = normal(rng, (d, f), wl.w_std, wl.dtype)
    W2 = normal(rng, (f, d), wl.w_std, wl.dtype)
    dY = normal(rng, (M, d), 1.0, wl.dtype) if wl.backward else None
    return {"X": X, "W1": W1, "W3": W3, "W2": W2, "dY": dY}


def attn_inputs(wl: Workload, seed: int = 0) -> dict:
    """Attention shard inputs: X[b*s x d], W_Q/W_K/W_V [d x h_l*d_h], W_O [h_l*d_h x d]."""
    assert wl.kind == "attn"
    rng = np.random.default_rng(seed)
    hd = wl.h_local * wl.d_head
    X = normal(rng, (wl.M, wl.d), 1.0, wl.dtype)
    Wq = normal(rng, (wl.d, hd), wl.w_std, wl.dtype)
    Wk = normal(rng, (wl.d, hd), wl.w_std, wl.dtype)
    Wv = normal(rng, (wl.d, hd), wl.w_std, wl.dtype)
    Wo = normal(rng, (hd, wl.d), wl.w_std, wl.dtype)
    return {"X": X, "Wq": Wq, "Wk": Wk, "Wv": Wv, "Wo": Wo}


def gqa_inputs(wl: Workload, seed: int = 0) -> dict:
    """Grouped-query shard inputs: X[b*s x d], W_Q [d x h_l*d_h],
    W_K/W_V [d x h_kv*d_h], W_O [h_l*d_h x d]; draw order X, W_Q, W_K, W_V, W_O."""
    assert wl.kind == "gqa"
    return random_gqa(wl.b, wl.s, wl.d, wl.h_local, wl.h_kv_local, wl.d_head, wl.dtype, seed, wl.w_std)


def random_gqa(b: int, s: int, d: int, h_local: int, h_kv: int, d_head: int, dtype: str,
               seed: int = 0, w_std: float = 0.02) -> dict:
    rng = np.random.default_rng(seed)
    X = normal(rng, (b * s, d), 1.0, dtype)
    Wq = normal(rng, (d, h_local * d_head), w_std, dtype)
    Wk = normal(rng, (d, h_kv * d_head), w_std, dtype)
    Wv = normal(rng, (d, h_kv * d_head), w_std, dtype)
    Wo = normal(rng, (h_local * d_head, d), w_std, dtype)
    return {"X": X, "Wq": Wq, "Wk": Wk, "Wv": Wv, "Wo": Wo}


def reduce_inputs(n_shards: int, numel: int, dtype: str, seed: int = 0,
                  bias_len: int = 0) -> dict:
    """Stacked partials [n_shards x numel] ~ N(0,1) and an optional bias."""
    rng = np.random.default_rng(seed)
    P = normal(rng, (n_shards, numel), 1.0, dtype)
    bias = normal(rng, (bias_len,), 1.0, dtype) if bias_len else None
    return {"P": P, "bias": bias}


def random_mlp(M: int, d: int, f: int, dtype: str, seed: int = 0,
               w_std: float = 0.02, x_std: float = 1.0) -> dict:
    """One shard of arbitrary shape (for ragged and edge cases)."""
    rng = np.random.default_rng(seed)
    X = normal(rng, (M, d), x_std, dtype)
    W1 = normal(rng, (d, f), w_std, dtype)
    W2 = normal(rng, (f, d), w_std, dtype)
    dY = normal(rng, (M, d), 1.0, dtype)
    return {"X": X, "W1": W1, "W2": W2, "dY": dY}


def random_swiglu(M: int, d: int, f: int, dtype: str, seed: int = 0,
                  w_std: float = 0.02) -> dict:
    rng = np.random.default_rng(seed)
    X = normal(rng, (M, d), 1.0, dtype)
    W1 = normal(rng, (d, f), w_std, dtype)
    W3 = normal(rng, (d, f), w_std, dtype)
    W2 = normal(rng, (f, d), w_std, dtype)
    dY = normal(rng, (M, d), 1.0, dtype)
    return {"X": X, "W1": W1, "W3": W3, "W2": W2, "dY": dY}


def random_attn(b: int, s: int, d: int, h_local: int, d_head: int, dtype: str,
                seed: int = 0, w_std: float = 0.02,
                n_shards: Optional[int] = None) -> dict:
    """Attention inputs of arbitrary shape.  With ``n_shards`` the full
    projection matrices for ``n_shards * h_local`` heads are drawn and every
    shard's slices are returned as lists."""
    rng = np.random.default_rng(seed)
    n = n_shards or 1
    hd = h_local * d_head * n
    X = normal(rng, (b * s, d), 1.0, dtype)
    Wq = normal(rng, (d, hd), w_std, dtype)
    Wk = normal(rng, (d, hd), w_std, dtype)
    Wv = normal(rng, (d, hd), w_std, dtype)
    Wo = normal(rng, (hd, d), w_std, dtype)
    out = {"X": X, "Wq": Wq, "Wk": Wk, "Wv": Wv, "Wo": Wo}
    if n_shards:
        out["Wqs"] = [_cols(Wq, n, i) for i in range(n)]
        out["Wks"] = [_cols(Wk, n, i) for i in range(n)]
        out["Wvs"] = [_cols(Wv, n, i) for i in range(n)]
        out["Wos"] = [_rows(Wo, n, i) for i in range(n)]
    return out


def sp_inputs(wl: Workload, seed: int = 0) -> dict:
    """Sequence-parallel block end inputs at the workload's shape: rows = b*s
    tokens of width d, over n_shards GPUs (see random_sp)."""
    assert wl.kind == "sp"
    return random_sp(wl.n_shards, wl.M, wl.d, wl.dtype, seed, wl.p_drop)


def random_sp(n_shards: int, rows: int, cols: int, dtype: str, seed: int = 0,
              p_drop: float = 0.1, with_bias: bool = True) -> dict:
    """P [n_shards x rows x cols] ~ N(0,1): every shard's partial output of the
    row-parallel product; residual [rows x cols] ~ N(0,1): the residual stream
    (a GPU uses its stripe); bias ~ N(0, 0.1^2) or None; gamma ~ 1 + N(0,
    0.1^2), beta ~ N(0, 0.1^2); keep [rows x cols] uint8, 1 with probability
    1 - p_drop (dropout's random draw, handed to both sides).  Draw order P
    (shard by shard), residual, bias, gamma, beta, keep."""
    rng = np.random.default_rng(seed)
    P = np.empty((n_shards, rows, cols), dtype=np.float32)
    for i in range(n_shards):
        P[i] = normal(rng, (rows, cols), 1.0, dtype)
    residual = normal(rng, (rows, cols), 1.0, dtype)
    bias = normal(rng, (cols,), 0.1, dtype) if with_bias else None
    gamma = (1.0 + normal(rng, (cols,), 0.1, "f32")).astype(np.float32)
    gamma = round_to_bf16(gamma) if dtype == "bf16" else gamma
    beta = normal(rng, (cols,), 0.1, dtype)
    keep = (rng.random((rows, cols), dtype=np.float32) >= p_drop).astype(np.uint8)
    return {"P": P, "residual": residual, "bias": bias, "gamma": gamma, "beta": beta, "keep": keep,
            "p_drop": p_drop}


def zipf_token_ids(rng: np.random.Generator, n: int, vocab_used: int, a: float = 1.1) -> np.ndarray:
    """Token ids with a heavy-tailed (Zipf, exponent a) frequency: rank r has
    probability proportional to 1 / r^a, and ranks map to ids through one
    fixed random permutation of [0, vocab_used), so frequent tokens fall in
    every shard's rows."""
    ranks = np.arange(1, vocab_used + 1, dtype=np.float64)
    p = ranks ** -a
    p /= p.sum()
    perm = np.random.default_rng(12345).permutation(vocab_used)
    return perm[rng.choice(vocab_used, size=n, p=p)].astype(np.int64)


def vocab_inputs(wl: Workload, seed: int = 0) -> dict:
    """Vocabulary-parallel inputs at the workload's shape (see random_vocab)."""
    assert wl.kind == "vocab"
    return random_vocab(wl.M, wl.d, wl.vocab, wl.vocab_used, wl.n_shards, wl.dtype, seed, wl.w_std)


def random_vocab(T: int, d: int, vocab: int, vocab_used: int, n_shards: int, dtype: str, seed: int = 0,
                 w_std: float = 0.02) -> dict:
    """E [vocab x d] ~ N(0, w_std^2), the table shared by the input and the
    output embedding (shard i holds rows [i V/n, (i+1) V/n)); ids and targets
    [T] Zipf-distributed below vocab_used; X [T x d] ~ N(0,1), the hidden
    states entering the output embedding; dloss [T] ~ U(0.5, 1.5) / T, the
    upstream gradient of each token's loss.  Draw order E, ids, targets, X,
    dloss."""
    rng = np.random.default_rng(seed)
    E = normal(rng, (vocab, d), w_std, dtype)
    ids = zipf_token_ids(rng, T, vocab_used)
    targets = zipf_token_ids(rng, T, vocab_used)
    X = normal(rng, (T, d), 1.0, dtype)
    dloss = (rng.uniform(0.5, 1.5, size=T) / T).astype(np.float32)
    return {"E": E, "Es": [_rows(E, n_shards, i) for i in range(n_shards)], "ids": ids, "targets": targets,
            "X": X, "dloss": dloss}
