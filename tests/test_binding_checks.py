"""The Python binding refuses tensors whose element count or dtype differs
from what the call's sizes imply, before any address reaches the library.

CPU tensors stand in for device tensors: every check runs before the binding
reads a device pointer or a stream, so a refused call raises ValueError naming
the tensor, and nothing is launched."""
import pytest
import torch

import megatron_tensor_transformer_fwd_amd as tp

bf, f32 = torch.bfloat16, torch.float32
M, d, f = 32, 16, 24


def _mlp():
    e = lambda *sh, dt=bf: torch.zeros(*sh, dtype=dt)
    return dict(X=e(M, d), W1=e(d, f), W2=e(f, d), A=e(M, f), H=e(M, f), Z=e(M, d), dY=e(M, d),
                dX=e(M, d), dW1=e(d, f, dt=f32), dW2=e(f, d, dt=f32), ws=torch.zeros(64, dtype=torch.uint8))


def _raises(fn, name, **kw):
    with pytest.raises(ValueError, match=name):
        fn(**kw)


@pytest.mark.parametrize("name,bad", [
    ("W2", torch.zeros(f, d + 8, dtype=bf)), ("H", torch.zeros(M - 1, f, dtype=bf)),
    ("Z", torch.zeros(M, d, dtype=f32)), ("A", torch.zeros(M, f + 1, dtype=bf))])
def test_mlp_fwd_refuses(name, bad):
    t = _mlp()
    t[name] = bad
    _raises(tp.tp_mlp_fwd, name, **{k: t[k] for k in ("X", "W1", "W2", "A", "H", "Z")})


@pytest.mark.parametrize("name,bad", [
    ("dW1", torch.zeros(d, f, dtype=bf)),          # bf16 where fp32 is written: half the bytes
    ("dW2", torch.zeros(f, d - 8, dtype=f32)), ("dX", torch.zeros(M // 2, d, dtype=bf)),
    ("dY", torch.zeros(M, d, dtype=f32)), ("A", torch.zeros(M, f // 2, dtype=bf))])
def test_mlp_bwd_refuses(name, bad):
    t = _mlp()
    t[name] = bad
    _raises(tp.tp_mlp_bwd, name, **{k: t[k] for k in ("X", "W1", "W2", "A", "H", "dY", "dX", "dW1", "dW2", "ws")})


def test_swiglu_refuses():
    e = lambda *sh, dt=bf: torch.zeros(*sh, dtype=dt)
    kw = dict(X=e(M, d), W1=e(d, f), W3=e(d, f), W2=e(f, d), G=e(M, f), U=e(M, f), H=e(M, f), Z=e(M, d))
    _raises(tp.tp_swiglu_fwd, "W3", **{**kw, "W3": e(d, f - 8)})
    _raises(tp.tp_swiglu_fwd, "U", **{**kw, "U": e(M, f, dt=f32)})
    bw = dict(kw, dY=e(M, d), dX=e(M, d), dW1=e(d, f, dt=f32), dW3=e(d, f, dt=f32), dW2=e(f, d, dt=f32),
              ws=e(8, dt=torch.uint8))
    del bw["Z"]
    _raises(tp.tp_swiglu_bwd, "dW3", **{**bw, "dW3": e(d, f)})
    _raises(tp.tp_swiglu_bwd, "dX", **{**bw, "dX": e(M, d + 8)})


def _attn(b=2, s=8, dm=16, hl=2, hkv=2, dh=8):
    e = lambda *sh, dt=bf: torch.zeros(*sh, dtype=dt)
    N, Nkv = hl * dh, hkv * dh
    return dict(X=e(b * s, dm), Wq=e(dm, N), Wk=e(dm, Nkv), Wv=e(dm, Nkv), Wo=e(N, dm), Q=e(b, hl, s, dh),
                K=e(b, hkv, s, dh), V=e(b, hkv, s, dh), O=e(b * s, N), Z=e(b * s, dm), L=e(b, hl, s, dt=f32),
                dY=e(b * s, dm), dX=e(b * s, dm), dWq=e(dm, N, dt=f32), dWk=e(dm, Nkv, dt=f32),
                dWv=e(dm, Nkv, dt=f32), dWo=e(N, dm, dt=f32), ws=e(8, dt=torch.uint8))


FWD = ("X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "Z")
BWD = ("X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "L", "dY", "dX", "dWq", "dWk", "dWv", "dWo", "ws")


def test_attention_refuses():
    t = _attn()
    with pytest.raises(ValueError, match="b\\*s"):
        tp.tp_attn_shard_fwd(*[t[k] for k in FWD], b=2, s=4, h_local=2, d_head=8, L=t["L"])
    for name, bad in (("Q", torch.zeros(2, 2, 4, 8, dtype=bf)), ("Wo", torch.zeros(16, 8, dtype=bf)),
                      ("L", torch.zeros(2, 2, 8, dtype=bf)), ("Z", torch.zeros(16, 8, dtype=bf))):
        u = dict(t, **{name: bad})
        with pytest.raises(ValueError, match=name):
            tp.tp_attn_shard_fwd(*[u[k] for k in FWD], b=2, s=8, h_local=2, d_head=8, L=u["L"])
    for name, bad in (("dWq", torch.zeros(16, 16, dtype=bf)), ("dX", torch.zeros(8, 16, dtype=bf)),
                      ("L", None)):
        u = dict(t, **{name: bad})
        with pytest.raises(ValueError, match=name):
            tp.tp_attn_shard_bwd(*[u[k] for k in BWD], b=2, s=8, h_local=2, d_head=8)
    g = _attn(hl=4, hkv=1)
    u = dict(g, K=torch.zeros(2, 4, 8, 8, dtype=bf))      # K sized for 4 heads, the call has 1
    with pytest.raises(ValueError, match="K"):
        tp.tp_attn_gqa_shard_fwd(*[u[k] for k in FWD], b=2, s=8, h_local=4, h_kv_local=1, d_head=8, L=u["L"])
    u = dict(g, dWk=torch.zeros(16, 32, dtype=f32))
    with pytest.raises(ValueError, match="dWk"):
        tp.tp_attn_gqa_shard_bwd(*[u[k] for k in BWD], b=2, s=8, h_local=4, h_kv_local=1, d_head=8)


def test_shard_reduce_refuses():
    P = torch.zeros(4, 64, dtype=bf)
    with pytest.raises(ValueError, match="partials"):
        tp.tp_shard_reduce(P, torch.zeros(64, dtype=bf), 5, 64)           # 5 shards in 4 blocks
    with pytest.raises(ValueError, match="partials"):
        tp.tp_shard_reduce(P, torch.zeros(64, dtype=bf), 4, 64, shard_stride=72)
    with pytest.raises(ValueError, match="out"):
        tp.tp_shard_reduce(P, torch.zeros(32, dtype=bf), 4, 64)
    with pytest.raises(ValueError, match="bias"):
        tp.tp_shard_reduce(P, torch.zeros(64, dtype=bf), 4, 64, bias=torch.zeros(8, dtype=f32))


def test_sequence_parallel_refuses():
    n, rows, cols = 4, 16, 8
    k = rows // n
    e = lambda *sh, dt=bf: torch.zeros(*sh, dtype=dt)
    kw = dict(partials=e(n, rows, cols), residual=e(k, cols), gamma=e(cols), beta=e(cols), h_out=e(k, cols),
              x_out=e(k, cols), n_shards=n, index=0, rows=rows, cols=cols)
    for name, bad in (("partials", e(n - 1, rows, cols)), ("residual", e(rows, cols)), ("x_out", e(k, cols, dt=f32)),
                      ("gamma", e(cols + 8))):
        with pytest.raises(ValueError, match=name):
            tp.tp_sp_reduce_scatter_ln(**dict(kw, **{name: bad}))
    with pytest.raises(ValueError, match="keep"):
        tp.tp_sp_reduce_scatter_ln(**kw, keep=e(rows, cols, dt=torch.uint8))
    bw = dict(dx_partials=e(n, rows, cols), h=e(k, cols), gamma=e(cols), dh_out=e(k, cols), dy_out=e(k, cols),
              dgamma=e(cols, dt=f32), dbeta=e(cols, dt=f32), ws=e(8, dt=torch.uint8), n_shards=n, index=0, rows=rows,
              cols=cols)
    for name, bad in (("dgamma", e(cols)), ("dy_out", e(k - 1, cols)), ("dx_partials", e(n, k, cols))):
        with pytest.raises(ValueError, match=name):
            tp.tp_sp_ln_bwd_reduce_scatter(**dict(bw, **{name: bad}))
    with pytest.raises(ValueError, match="stripes"):
        tp.tp_sp_all_gather([e(k, cols), e(k, cols + 8)], e(2 * k, cols))
    with pytest.raises(ValueError, match="full"):
        tp.tp_sp_all_gather([e(k, cols), e(k, cols)], e(3 * k, cols))


def test_vocab_refuses():
    T, dm, vl = 16, 8, 24
    e = lambda *sh, dt=bf: torch.zeros(*sh, dtype=dt)
    ids = torch.zeros(T, dtype=torch.int64)
    with pytest.raises(ValueError, match="Y"):
        tp.tp_vocab_embed_fwd(ids, e(vl, dm), e(T - 1, dm), 0)
    with pytest.raises(ValueError, match="dE_local"):
        tp.tp_vocab_embed_bwd(ids, e(T, dm), e(vl, dm), 0)
    with pytest.raises(ValueError, match="logits"):
        tp.tp_vocab_ce_fwd(e(T, dm), e(vl, dm), ids, e(T, vl - 8), e(T, 3, dt=f32), 0)
    with pytest.raises(ValueError, match="stats"):
        tp.tp_vocab_ce_fwd(e(T, dm), e(vl, dm), ids, e(T, vl), e(T, 3), 0)
    with pytest.raises(ValueError, match="lse"):
        tp.tp_vocab_ce_combine(e(2, T, 3, dt=f32), e(T, dt=f32), e(T - 1, dt=f32))
    with pytest.raises(ValueError, match="dE"):
        tp.tp_vocab_ce_bwd(e(T, dm), e(vl, dm), ids, e(T, vl), e(T, dt=f32), e(T, dt=f32), e(T, dm), e(vl, dm), e(8), 0)
