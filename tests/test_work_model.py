"""The bench's FLOP and byte model, pinned to what the pages and counting fix.

* The worked GPT-3 175B example of "Splitting the model: five parallelisms and
  the traffic they make", section 3.4 (subsection "Why TP usually stays inside
  the server" and its table), stored in tests/golden/tp_traffic_gpt3.txt: the
  model's per-GPU layer FLOPs, all-reduce message, ring traffic and the times
  they give at the page's assumed rates must round to the printed values.
* The same page's rule that a backward pass costs twice its forward pass, for
  every product list the model holds.
* The causal pair count against brute-force counting of the kept mask entries.
* Byte counts against the sizes of the tensors each kernel reads and writes.
"""
import os

import numpy as np
import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tp_traffic_gpt3.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = float(v)
    return vals


def test_gpt3_tp_layer_example():
    g = _golden()
    tokens, h, t = int(g["tokens"]), int(g["hidden"]), int(g["tp"])
    msg = bench.allreduce_message_bytes(tokens, h, int(g["bytes_per_elem"]))
    assert round(msg / 1e6, 1) == g["message_mb"]
    ring = bench.ring_bytes_per_gpu(msg, t)
    assert round(ring / 1e6) == g["layer_ring_mb"]
    flops = bench.tp_layer_flops(tokens, h, t)
    compute_ms = flops / (g["assumed_tflops"] * 1e12) * 1e3
    assert round(compute_ms, 1) == g["compute_ms"]
    nvlink_ms = ring / (g["nvlink_gbps"] * 1e9) * 1e3
    nic_ms = ring / (g["nic_gbps"] * 1e9) * 1e3
    assert round(nvlink_ms, 2) == g["nvlink_comm_ms"]
    assert round(nic_ms, 1) == g["nic_comm_ms"]
    assert round(100 * nvlink_ms / (compute_ms + nvlink_ms)) == g["nvlink_share_pct"]
    assert round(100 * nic_ms / (compute_ms + nic_ms)) == g["nic_share_pct"]


@pytest.mark.parametrize("fn,args", [
    (bench.mlp_products, (8192, 8192, 4096)),
    (bench.mlp_products, (8192, 1024, 512)),
    (bench.swiglu_products, (8192, 4096, 2752)),
    (bench.attn_products, (8192, 4096, 1024, 1024)),
    (bench.attn_products, (8192, 16384, 2048, 128)),
])
def test_backward_is_twice_forward(fn, args):
    pr = fn(*args)
    assert bench.products_flops(pr["bwd"]) == 2 * bench.products_flops(pr["fwd"])


def test_attention_core_counts():
    for s in (1, 2, 7, 64, 129):
        kept = int(np.tril(np.ones((s, s), dtype=np.int64)).sum())
        assert bench.attn_pairs(s) == kept
        assert bench.attn_pairs(s, causal=False) == s * s
    f = bench.attn_core_flops(4, 8, 2048, 128)
    # two products over the kept pairs: 2 * d_head FLOPs each per pair
    assert f == 4 * 8 * bench.attn_pairs(2048) * 2 * (2 * 128)
    # backward = the page's twice-the-forward for the four gradient products,
    # plus the recomputed scores (one of the forward's two products)
    assert bench.attn_core_flops(4, 8, 2048, 128, backward=True) == 2 * f + f / 2


def test_headline_flops():
    fl = bench.mlp_product_flops(8192, 8192, 4096)
    assert set(fl) == set(bench.C5_LABELS)
    assert all(v == 549755813888.0 for v in fl.values())
    assert round(sum(fl.values()) / 1e9, 2) == 3298.53


def test_product_bytes_are_tensor_sizes():
    M, d, f = 96, 64, 32
    bf, fp = np.zeros(1, np.float16).itemsize, np.zeros(1, np.float32).itemsize
    X, dY, Z, dX = (np.zeros((M, d), np.float16) for _ in range(4))
    W1, dW1 = np.zeros((d, f), np.float16), np.zeros((d, f), np.float32)
    W2, dW2 = np.zeros((f, d), np.float16), np.zeros((f, d), np.float32)
    A, H, dA = (np.zeros((M, f), np.float16) for _ in range(3))
    size = lambda *ts: sum(t.nbytes for t in ts)
    want = {"mlp_fwd.xw1_gelu": size(X, W1, A, H), "mlp_fwd.hw2": size(H, W2, Z),
            "mlp_bwd.htdy": size(H, dY, dW2), "mlp_bwd.dyw2t_dgelu": size(dY, W2, A, dA),
            "mlp_bwd.daw1t": size(dA, W1, dX), "mlp_bwd.xtda": size(X, dA, dW1)}
    assert bf == 2 and fp == 4
    assert bench.mlp_product_bytes(M, d, f) == want


def test_hbm_kernel_bytes_are_tensor_sizes():
    n, k, cols = 8, 16, 64
    e = k * cols
    stripe = lambda dt=np.float16: np.zeros((k, cols), dt)
    vec = lambda dt=np.float16: np.zeros(cols, dt)
    size = lambda *ts: sum(t.nbytes for t in ts)
    parts = [stripe() for _ in range(n)]
    # reduce-scatter + LayerNorm: partial stripes, residual, mask, bias, gamma, beta -> h, x
    assert bench.sp_rs_ln_bytes(n, e, cols) == size(*parts, stripe(), stripe(np.uint8), vec(), vec(), vec(),
                                                    stripe(), stripe())
    # all-gather: n stripes read and written
    assert bench.sp_all_gather_bytes(n, e) == 2 * size(*parts)
    # backward: dx partial stripes, h, mask, dres, gamma -> dh, dy, dgamma, dbeta, dbias (fp32)
    assert bench.sp_ln_bwd_bytes(n, e, cols) == size(*parts, stripe(), stripe(np.uint8), stripe(), vec(),
                                                     stripe(), stripe(), vec(np.float32), vec(np.float32),
                                                     vec(np.float32))
    assert bench.shard_reduce_bytes(n, e) == size(*parts, stripe())
    T, d, vl, owned = 32, 64, 40, 5
    ids = np.zeros(T, np.int64)
    rows = np.zeros((owned, d), np.float16)
    assert bench.vocab_embed_bytes(T, d, owned) == size(ids, rows, np.zeros((T, d), np.float16))
    assert bench.vocab_embed_bwd_bytes(T, d, vl, owned) == size(ids, rows, np.zeros((vl, d), np.float32))


def test_oracle_step_flops_count_the_oracles_products(monkeypatch):
    """The CPU baseline's FLOP count equals what the oracle's MLP forward and
    backward actually multiply: every matrix product they perform is recorded
    (2 m n k each) through an ndarray subclass handed in for their inputs."""
    import oracle.tp_oracle as T
    seen = []

    class Counted(np.ndarray):
        def __matmul__(self, other):
            a, b = np.asarray(self), np.asarray(other)
            seen.append(2 * a.shape[0] * a.shape[1] * b.shape[1])
            return (a @ b).view(Counted)

    monkeypatch.setattr(T, "_f64", lambda a: np.asarray(a, dtype=np.float64).view(Counted))
    M, d, f = 24, 16, 8
    r = np.random.default_rng(0)
    X, W1, W2, dY = r.standard_normal((M, d)), r.standard_normal((d, f)), r.standard_normal((f, d)), \
        r.standard_normal((M, d))
    T.mlp_shard_fwd(X, W1, W2)
    fwd = sum(seen)
    T.mlp_shard_bwd(X, W1, W2, dY)
    step, executed = bench.oracle_mlp_step_flops(M, d, f)
    assert len(seen) == 7
    assert sum(seen) == executed
    assert executed - step == fwd / 2         # the one recomputed forward product
