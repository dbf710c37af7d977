"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph): each
path's step is captured once and replayed several times, with eager work,
poisoned outputs and synchronisations between the replays; every replay must
reproduce the eager outputs bit for bit (all kernels are deterministic)."""
import sys

import numpy as np
import pytest

import tpsynth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import megatron_tensor_transformer_fwd_amd as m
    m.lib()
    return m


def dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).cuda()


def capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def check_replays(g, outputs, eager_other):
    ref = [t.clone() for t in outputs]
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs, ref)):
            assert torch.equal(t, e), f"replay {r}: output {i} differs from the eager result"


def _busy(tp):
    """Unrelated eager library work between replays."""
    P = torch.randn(3, 4096, device="cuda").to(torch.bfloat16)
    out = torch.empty(4096, dtype=torch.bfloat16, device="cuda")
    return lambda: tp.tp_shard_reduce(P, out, 3, 4096)


def test_graph_mlp_two_shards_and_reduces(tp):
    _say("graph: GeLU MLP 2 shards fwd+bwd + reduces")
    M, d, f, n = 300, 128, 192, 2
    inp = tpsynth.random_mlp(M, d, f * n, "bf16", seed=80)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    W1s = [dev(inp["W1"][:, i * f:(i + 1) * f]) for i in range(n)]
    W2s = [dev(inp["W2"][i * f:(i + 1) * f]) for i in range(n)]
    bf = torch.bfloat16
    A, H = torch.empty((n, M, f), dtype=bf, device="cuda"), torch.empty((n, M, f), dtype=bf, device="cuda")
    Zp, dXp = torch.empty((n, M, d), dtype=bf, device="cuda"), torch.empty((n, M, d), dtype=bf, device="cuda")
    Z, dX = torch.empty((M, d), dtype=bf, device="cuda"), torch.empty((M, d), dtype=bf, device="cuda")
    dW1 = torch.empty((n, d, f), device="cuda")
    dW2 = torch.empty((n, f, d), device="cuda")
    ws = torch.empty(tp.tp_mlp_bwd_workspace_bytes(tp.TP_DT_BF16, M, d, f), dtype=torch.uint8, device="cuda")

    def step():
        for i in range(n):
            tp.tp_mlp_fwd(X, W1s[i], W2s[i], A[i], H[i], Zp[i])
        tp.tp_shard_reduce(Zp, Z, n, M * d)
        for i in range(n):
            tp.tp_mlp_bwd(X, W1s[i], W2s[i], A[i], H[i], dY, dXp[i], dW1[i], dW2[i], ws)
        tp.tp_shard_reduce(dXp, dX, n, M * d)

    step()
    torch.cuda.synchronize()
    check_replays(capture(step), [A, H, Zp, Z, dXp, dX, dW1, dW2], _busy(tp))


def test_graph_attention_fwd_bwd(tp):
    _say("graph: attention shard fwd+bwd")
    b, s, d, hl, dh = 2, 130, 64, 2, 128
    inp = tpsynth.random_attn(b, s, d, hl, dh, "bf16", seed=81)
    X, Wq, Wk, Wv, Wo = (dev(inp[k]) for k in ("X", "Wq", "Wk", "Wv", "Wo"))
    dY = dev(np.random.default_rng(82).standard_normal((b * s, d)))
    bf = torch.bfloat16
    Q, K, V = (torch.empty((b, hl, s, dh), dtype=bf, device="cuda") for _ in range(3))
    O = torch.empty((b * s, hl * dh), dtype=bf, device="cuda")
    Z = torch.empty((b * s, d), dtype=bf, device="cuda")
    L = torch.empty((b, hl, s), device="cuda")
    dX = torch.empty((b * s, d), dtype=bf, device="cuda")
    dWq, dWk, dWv = (torch.empty((d, hl * dh), device="cuda") for _ in range(3))
    dWo = torch.empty((hl * dh, d), device="cuda")
    ws = torch.empty(tp.tp_attn_shard_bwd_workspace_bytes(tp.TP_DT_BF16, b, s, d, hl, dh), dtype=torch.uint8,
                     device="cuda")

    def step():
        tp.tp_attn_shard_fwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, Z, b, s, hl, dh, causal=True, L=L)
        tp.tp_attn_shard_bwd(X, Wq, Wk, Wv, Wo, Q, K, V, O, L, dY, dX, dWq, dWk, dWv, dWo, ws, b, s, hl, dh,
                             causal=True)

    step()
    torch.cuda.synchronize()
    check_replays(capture(step), [Q, K, V, O, Z, L, dX, dWq, dWk, dWv, dWo], _busy(tp))


def test_graph_sequence_parallel_and_vocab(tp):
    _say("graph: sequence-parallel block end + all-gather, vocabulary embeddings + cross-entropy")
    n, rows, cols = 4, 64, 1024
    sp = tpsynth.random_sp(n, rows, cols, "bf16", seed=83)
    P, res, bias, gamma, beta = (dev(sp[k]) for k in ("P", "residual", "bias", "gamma", "beta"))
    keep = torch.from_numpy(sp["keep"]).cuda()
    k = rows // n
    hs = [torch.empty((k, cols), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    xs = [torch.empty((k, cols), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    full = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    T, d, V, nv = 200, 128, 512, 2
    vo = tpsynth.random_vocab(T, d, V, V, nv, "bf16", seed=84)
    vl = V // nv
    Es = [dev(e) for e in vo["Es"]]
    Xv = dev(vo["X"])
    ids, tg = torch.from_numpy(vo["ids"]).cuda(), torch.from_numpy(vo["targets"]).cuda()
    dloss = torch.from_numpy(vo["dloss"]).cuda()
    emb_p = torch.empty((nv, T, d), dtype=torch.bfloat16, device="cuda")
    emb = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((nv, T, vl), dtype=torch.bfloat16, device="cuda")
    stats = torch.empty((nv, T, 3), device="cuda")
    loss, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    dXv = torch.empty((nv, T, d), dtype=torch.bfloat16, device="cuda")
    dE = torch.empty((nv, vl, d), device="cuda")
    ws = torch.empty(tp.tp_vocab_ce_bwd_workspace_bytes(tp.TP_DT_BF16, T, d, vl), dtype=torch.uint8, device="cuda")
    fws = torch.empty(tp.tp_vocab_ce_fwd_workspace_bytes(tp.TP_DT_BF16, T, d, vl), dtype=torch.uint8,
                      device="cuda")

    def step():
        for i in range(n):
            tp.tp_sp_reduce_scatter_ln(P, res[i * k:(i + 1) * k], gamma, beta, hs[i], xs[i], n, i, rows, cols,
                                       bias=bias, keep=keep[i * k:(i + 1) * k], p_drop=sp["p_drop"])
        tp.tp_sp_all_gather(hs, full)
        for i in range(nv):
            tp.tp_vocab_embed_fwd(ids, Es[i], emb_p[i], i * vl)
            tp.tp_vocab_ce_fwd(Xv, Es[i], tg, logits[i], stats[i], i * vl, ws=fws)
        tp.tp_shard_reduce(emb_p, emb, nv, T * d)
        tp.tp_vocab_ce_combine(stats, loss, lse)
        for i in range(nv):
            tp.tp_vocab_ce_bwd(Xv, Es[i], tg, logits[i], lse, dloss, dXv[i], dE[i], ws, i * vl)

    step()
    torch.cuda.synchronize()
    check_replays(capture(step), hs + xs + [full, emb_p, emb, logits, stats, loss, lse, dXv, dE], _busy(tp))
