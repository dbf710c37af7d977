"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: textbook values of
the normal distribution, closed-form identities, central finite differences,
brute-force loops on tiny inputs (``math.fsum``/``math.erf``/``math.exp``, not
numpy), the pages' sharding identities and their printed worked examples.
"""
import math
import os

import numpy as np
import pytest

import oracle as O
import tpsynth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- activations

def test_gelu_textbook_values():
    # Phi(1), Phi(2), phi(1) from standard normal tables (e.g. Abramowitz &
    # Stegun, Table 26.1): GeLU(x) = x Phi(x); GeLU'(x) = Phi(x) + x phi(x).
    phi1, Phi1, Phi2 = 0.24197072451914337, 0.8413447460685429, 0.9772498680518208
    assert O.gelu(1.0) == pytest.approx(Phi1, abs=1e-15)
    assert O.gelu(2.0) == pytest.approx(2 * Phi2, abs=1e-15)
    assert O.gelu(-1.0) == pytest.approx(-(1 - Phi1), abs=1e-15)
    assert O.gelu(0.0) == 0.0
    assert O.gelu_prime(0.0) == pytest.approx(0.5, abs=1e-15)
    assert O.gelu_prime(1.0) == pytest.approx(Phi1 + phi1, abs=1e-15)
    assert O.gelu(10.0) == pytest.approx(10.0, abs=1e-15)
    assert abs(O.gelu(-10.0)) < 1e-20


def test_gelu_lower_tail_relative():
    # Upper-tail probabilities Q(x) = Phi(-x) of the standard normal from
    # tables of the normal distribution: Q(5) = 2.8665157187919e-7,
    # Q(10) = 7.6198530241605e-24.  GeLU(-x) = -x Q(x) must hold to relative
    # accuracy, not just be small, because the products store these values
    # in floating point with their own exponent.
    assert O.gelu(-5.0) == pytest.approx(-5 * 2.8665157187919e-7, rel=1e-12)
    assert O.gelu(-10.0) == pytest.approx(-10 * 7.6198530241605e-24, rel=1e-12)
    # GeLU'(-10) = Phi(-10) - 10 phi(-10), phi(10) = exp(-50) / sqrt(2 pi)
    phi10 = math.exp(-50.0) / math.sqrt(2 * math.pi)
    assert O.gelu_prime(-10.0) == pytest.approx(7.6198530241605e-24 - 10 * phi10, rel=1e-12)


def test_swish_closed_forms():
    sig1 = 1.0 / (1.0 + math.exp(-1.0))
    assert O.swish(1.0) == pytest.approx(sig1, abs=1e-15)
    assert O.swish(1.0) == pytest.approx(0.7310585786300049, abs=1e-15)
    assert O.swish_prime(0.0) == pytest.approx(0.5, abs=1e-15)
    assert O.swish_prime(1.0) == pytest.approx(0.9276705118714869, abs=1e-14)
    assert O.swish(0.0) == 0.0
    # no overflow far out on either side
    assert O.swish(-800.0) == pytest.approx(0.0, abs=1e-300)
    assert O.swish(800.0) == pytest.approx(800.0)


def test_activation_reflection_identities():
    x = np.random.default_rng(1).standard_normal(1000) * 4
    # Phi(-x) = 1 - Phi(x)  =>  GeLU(-x) = GeLU(x) - x ; likewise for Swish
    np.testing.assert_allclose(O.gelu(-x), O.gelu(x) - x, atol=1e-13)
    np.testing.assert_allclose(O.swish(-x), O.swish(x) - x, atol=1e-13)


def test_activation_derivatives_match_finite_differences():
    x = np.linspace(-6, 6, 241)
    h = 1e-5
    fd_g = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    fd_s = (O.swish(x + h) - O.swish(x - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_prime(x), fd_g, atol=1e-9)
    np.testing.assert_allclose(O.swish_prime(x), fd_s, atol=1e-9)


def test_erf_matches_math_erf():
    x = np.linspace(-5, 5, 101)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    np.testing.assert_allclose(O.gelu(x), ref, rtol=0, atol=1e-15)


# ------------------------------------------------------- brute-force helpers

def _bf_matmul(A, B):
    A, B = np.asarray(A, float), np.asarray(B, float)
    n, k = A.shape
    k2, m = B.shape
    assert k == k2
    return np.array([[math.fsum(A[i, t] * B[t, j] for t in range(k)) for j in range(m)]
                     for i in range(n)])


def _bf_gelu(v):
    return v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0)))


def _bf_swish(v):
    return v / (1.0 + math.exp(-v))


def _tiny(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ------------------------------------------------------------------ GeLU MLP

def test_mlp_fwd_brute_force():
    X, W1, W2 = _tiny((3, 4), 0), _tiny((4, 5), 1), _tiny((5, 4), 2)
    r = O.mlp_shard_fwd(X, W1, W2)
    A = _bf_matmul(X, W1)
    H = np.vectorize(_bf_gelu)(A)
    Z = _bf_matmul(H, W2)
    np.testing.assert_allclose(r["A"], A, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["H"], H, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["Z"], Z, rtol=1e-13, atol=1e-14)


def test_mlp_fwd_brute_force_c1_size():
    wl = tpsynth.WORKLOADS["C1"]
    inp = tpsynth.mlp_inputs(wl)
    r = O.mlp_shard_fwd(inp["X"], inp["W1s"][0], inp["W2s"][0])
    A = _bf_matmul(inp["X"], inp["W1s"][0])
    np.testing.assert_allclose(r["A"], A, rtol=1e-13, atol=1e-13)


def _fd_grad(fun, arr, h=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = arr[idx]
        arr[idx] = old + h
        fp = fun()
        arr[idx] = old - h
        fm = fun()
        arr[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def test_mlp_bwd_matches_finite_differences():
    X, W1, W2, dY = _tiny((3, 4), 3), _tiny((4, 6), 4, 0.7), _tiny((6, 4), 5, 0.7), _tiny((3, 4), 6)
    loss = lambda: float(np.sum(dY * O.mlp_shard_fwd(X, W1, W2)["Z"]))
    g = O.mlp_shard_bwd(X, W1, W2, dY)
    np.testing.assert_allclose(g["dX"], _fd_grad(loss, X), atol=1e-8)
    np.testing.assert_allclose(g["dW1"], _fd_grad(loss, W1), atol=1e-8)
    np.testing.assert_allclose(g["dW2"], _fd_grad(loss, W2), atol=1e-8)


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_mlp_sharding_identity_equal_splits(n):
    # [JY] FFN: GeLU(X W1) W2 = sum_i GeLU(X W1_i) W2_i for a column split of
    # W1 and the matching row split of W2; backward: dX = sum_i dX_i ([HC] 3.4).
    wl = tpsynth.WORKLOADS["C1"]
    inp = tpsynth.mlp_inputs(wl)
    X, W1, W2, dY = inp["X"], inp["W1"], inp["W2"], inp["dY"]
    f = W1.shape[1] // n
    Y = O.mlp_unsharded(X, W1, W2)
    full = O.mlp_unsharded_bwd(X, W1, W2, dY)
    parts = [O.mlp_shard_fwd(X, W1[:, i * f:(i + 1) * f], W2[i * f:(i + 1) * f]) for i in range(n)]
    grads = [O.mlp_shard_bwd(X, W1[:, i * f:(i + 1) * f], W2[i * f:(i + 1) * f], dY) for i in range(n)]
    assert O.max_rel_err(O.shard_reduce([p["Z"] for p in parts]), Y) < 1e-12
    assert O.max_rel_err(O.shard_reduce([g["dX"] for g in grads]), full["dX"]) < 1e-12
    assert O.max_rel_err(np.concatenate([g["dW1"] for g in grads], axis=1), full["dW1"]) < 1e-12
    assert O.max_rel_err(np.concatenate([g["dW2"] for g in grads], axis=0), full["dW2"]) < 1e-12


def test_mlp_sharding_identity_uneven_split():
    # [JY] FFN allows any d_1 + d_2 = d_ff.
    wl = tpsynth.WORKLOADS["C1"]
    inp = tpsynth.mlp_inputs(wl)
    X, W1, W2 = inp["X"], inp["W1"], inp["W2"]
    cuts = [0, 37, 100, 201, 256]
    Zs = [O.mlp_shard_fwd(X, W1[:, a:b], W2[a:b])["Z"] for a, b in zip(cuts[:-1], cuts[1:])]
    assert O.max_rel_err(O.shard_reduce(Zs), O.mlp_unsharded(X, W1, W2)) < 1e-12


def test_mlp_sharding_identity_c2_shape():
    # All 8 shards of the GPT-2-medium-shaped workload, on a sample of 128 rows
    # (rows are independent in this identity).
    wl = tpsynth.WORKLOADS["C2"]
    inp = tpsynth.mlp_inputs(wl)
    X = inp["X"][::64]
    Zs = [O.mlp_shard_fwd(X, inp["W1s"][i], inp["W2s"][i])["Z"] for i in range(8)]
    assert O.max_rel_err(O.shard_reduce(Zs), O.mlp_unsharded(X, inp["W1"], inp["W2"])) < 1e-12


def test_row_split_before_gelu_is_not_a_sharding():
    # [JY] FFN and [BM] (quoting the Megatron paper): splitting W1 by rows and
    # X by columns needs a sum before the GeLU, GeLU(X1A1 + X2A2) != GeLU(X1A1) + GeLU(X2A2).
    assert O.gelu(1.0) + O.gelu(1.0) == pytest.approx(1.6826894921370859, abs=1e-15)
    assert abs(O.gelu(2.0) - 2 * O.gelu(1.0)) > 0.27
    inp = tpsynth.mlp_inputs(tpsynth.WORKLOADS["C1"])
    X, W1 = inp["X"].astype(float), inp["W1"].astype(float)
    k = X.shape[1] // 2
    ref = O.gelu(X @ W1)
    wrong = O.gelu(X[:, :k] @ W1[:k]) + O.gelu(X[:, k:] @ W1[k:])
    right = O.gelu(X[:, :k] @ W1[:k] + X[:, k:] @ W1[k:])
    assert O.max_rel_err(wrong, ref) > 1e-2
    assert O.max_rel_err(right, ref) < 1e-13


# -------------------------------------------------------------------- SwiGLU

def test_swiglu_fwd_brute_force():
    X, W1, W3, W2 = _tiny((3, 4), 10), _tiny((4, 5), 11), _tiny((4, 5), 12), _tiny((5, 4), 13)
    r = O.swiglu_shard_fwd(X, W1, W3, W2)
    G, U = _bf_matmul(X, W1), _bf_matmul(X, W3)
    H = np.vectorize(_bf_swish)(G) * U
    np.testing.assert_allclose(r["G"], G, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["H"], H, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["Z"], _bf_matmul(H, W2), rtol=1e-13, atol=1e-14)


def test_swiglu_bwd_matches_finite_differences():
    X, W1, W3, W2, dY = (_tiny((3, 4), 20), _tiny((4, 5), 21, 0.7), _tiny((4, 5), 22, 0.7),
                         _tiny((5, 4), 23, 0.7), _tiny((3, 4), 24))
    loss = lambda: float(np.sum(dY * O.swiglu_shard_fwd(X, W1, W3, W2)["Z"]))
    g = O.swiglu_shard_bwd(X, W1, W3, W2, dY)
    for name, arr in (("dX", X), ("dW1", W1), ("dW3", W3), ("dW2", W2)):
        np.testing.assert_allclose(g[name], _fd_grad(loss, arr), atol=1e-8, err_msg=name)


@pytest.mark.parametrize("cuts", [[0, 64, 128], [0, 32, 64, 96, 128], [0, 5, 77, 128]])
def test_swiglu_sharding_identity(cuts):
    # [JY] FFN, SwiGLU: Y = sum_i (X W3_i (.) Swish(X W1_i)) W2_i.
    inp = tpsynth.random_swiglu(40, 48, 128, "f32", seed=7, w_std=0.1)
    X, W1, W3, W2, dY = inp["X"], inp["W1"], inp["W3"], inp["W2"], inp["dY"]
    Y = O.swiglu_unsharded(X, W1, W3, W2)
    full = O.swiglu_shard_bwd(X, W1, W3, W2, dY)
    Zs, dXs = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        Zs.append(O.swiglu_shard_fwd(X, W1[:, a:b], W3[:, a:b], W2[a:b])["Z"])
        dXs.append(O.swiglu_shard_bwd(X, W1[:, a:b], W3[:, a:b], W2[a:b], dY)["dX"])
    assert O.max_rel_err(O.shard_reduce(Zs), Y) < 1e-12
    assert O.max_rel_err(O.shard_reduce(dXs), full["dX"]) < 1e-12


# ----------------------------------------------------------------- attention

def _bf_attention_head(Q, K, V, scale, causal=True):
    s = Q.shape[0]
    out = np.zeros_like(V)
    for t in range(s):
        us = range(t + 1) if causal else range(s)
        sc = [math.fsum(Q[t, c] * K[u, c] for c in range(Q.shape[1])) * scale for u in us]
        m = max(sc)
        w = [math.exp(v - m) for v in sc]
        z = math.fsum(w)
        for c in range(V.shape[1]):
            out[t, c] = math.fsum(w[i] * V[u, c] for i, u in enumerate(us)) / z
    return out


def test_attention_brute_force():
    b, s, h, dh, d = 1, 5, 2, 4, 6
    X, Wq, Wk, Wv, Wo = (_tiny((b * s, d), 30), _tiny((d, h * dh), 31), _tiny((d, h * dh), 32),
                         _tiny((d, h * dh), 33), _tiny((h * dh, d), 34))
    r = O.attn_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, h, dh)
    Qf, Kf, Vf = _bf_matmul(X, Wq), _bf_matmul(X, Wk), _bf_matmul(X, Wv)
    heads = []
    for j in range(h):
        sl = slice(j * dh, (j + 1) * dh)
        heads.append(_bf_attention_head(Qf[:, sl], Kf[:, sl], Vf[:, sl], 1 / math.sqrt(dh)))
    Ob = np.concatenate(heads, axis=1)
    np.testing.assert_allclose(r["O"], Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["Z"], _bf_matmul(Ob, Wo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["Q"][0, 1], Qf[:, dh:2 * dh], rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(40)
    s, dh = 9, 4
    Q, K, V = rng.standard_normal((s, dh)), rng.standard_normal((s, dh)), rng.standard_normal((s, dh))
    o = O.attn_core(Q, K, V)
    np.testing.assert_array_equal(o[0], V[0])                      # row 0 sees key 0 only
    o0 = O.attn_core(Q, np.zeros_like(K), V)                       # equal scores
    prefix = np.cumsum(V, axis=0) / np.arange(1, s + 1)[:, None]
    np.testing.assert_allclose(o0, prefix, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(O.attn_core(Q[:1], K[:1], V[:1]), V[:1], rtol=0, atol=0)
    c = 1.7                                                        # scaling Q by c
    np.testing.assert_allclose(O.attn_core(c * Q, K, V), O.attn_core(Q, K, V, scale=c / math.sqrt(dh)),
                               rtol=1e-13, atol=1e-14)
    full = O.attn_core(Q, K, V, causal=False)                      # last row unaffected by the mask
    np.testing.assert_allclose(o[-1], full[-1], rtol=1e-13, atol=1e-14)


def test_attention_shards_concatenate_and_sum_to_unsharded():
    # [JY] Attention: heads may be placed on GPUs one or several at a time;
    # [HC] Figure 3.5: contiguous groups; the W_O row split leaves partial sums.
    n, h_l, dh, b, s, d = 4, 2, 8, 2, 12, 24
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "f32", seed=41, w_std=0.2, n_shards=n)
    full = O.attn_unsharded(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, n * h_l, dh)
    shards = [O.attn_shard_fwd(inp["X"], inp["Wqs"][i], inp["Wks"][i], inp["Wvs"][i], inp["Wos"][i],
                               b, s, h_l, dh) for i in range(n)]
    np.testing.assert_allclose(np.concatenate([r["O"] for r in shards], axis=1), full["O"], rtol=1e-13, atol=1e-14)
    assert O.max_rel_err(O.shard_reduce([r["Z"] for r in shards]), full["Z"]) < 1e-12


def test_online_softmax_tiling_equals_direct_softmax():
    # The GPU kernel streams keys in tiles with a running max and sum; in exact
    # arithmetic this is the direct softmax.  Written here in fp64, tile 3.
    rng = np.random.default_rng(42)
    s, dh, tile = 11, 5, 3
    Q, K, V = rng.standard_normal((s, dh)), rng.standard_normal((s, dh)), rng.standard_normal((s, dh))
    scale = 1 / math.sqrt(dh)
    out = np.zeros((s, dh))
    for t in range(s):
        m, l, acc = -np.inf, 0.0, np.zeros(dh)
        for u0 in range(0, t + 1, tile):
            u1 = min(u0 + tile, t + 1)
            sc = (K[u0:u1] @ Q[t]) * scale
            m_new = max(m, sc.max())
            corr = math.exp(m - m_new) if m > -np.inf else 0.0
            p = np.exp(sc - m_new)
            l = l * corr + p.sum()
            acc = acc * corr + p @ V[u0:u1]
            m = m_new
        out[t] = acc / l
    np.testing.assert_allclose(out, O.attn_core(Q, K, V), rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ GQA

def test_gqa_with_one_group_is_mha():
    b, s, d, h, dh = 2, 7, 12, 3, 4
    inp = tpsynth.random_attn(b, s, d, h, dh, "f32", seed=60, w_std=0.3)
    g = O.attn_gqa_shard_fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, h, h, dh)
    m = O.attn_shard_fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, h, dh)
    for k in ("O", "Z", "L"):
        np.testing.assert_allclose(g[k], m[k], rtol=1e-13, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    # Sharing a K/V head among a group of query heads is the same as giving
    # every query head its own copy of that K/V projection.
    b, s, d, h, hkv, dh = 1, 9, 16, 6, 2, 4
    rng = np.random.default_rng(61)
    X = rng.standard_normal((b * s, d))
    Wq = rng.standard_normal((d, h * dh)) * 0.3
    Wk = rng.standard_normal((d, hkv * dh)) * 0.3
    Wv = rng.standard_normal((d, hkv * dh)) * 0.3
    Wo = rng.standard_normal((h * dh, d)) * 0.3
    rep = lambda W: np.concatenate([W[:, (j // (h // hkv)) * dh:(j // (h // hkv) + 1) * dh] for j in range(h)], axis=1)
    g = O.attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, h, hkv, dh)
    m = O.attn_shard_fwd(X, Wq, rep(Wk), rep(Wv), Wo, b, s, h, dh)
    for k in ("O", "Z", "L"):
        np.testing.assert_allclose(g[k], m[k], rtol=1e-13, atol=1e-14)


def test_gqa_query_rows_match_full():
    b, s, d, h, hkv, dh = 1, 11, 16, 4, 1, 4
    rng = np.random.default_rng(62)
    X = rng.standard_normal((s, d))
    Wq, Wk, Wv = (rng.standard_normal((d, n * dh)) * 0.3 for n in (h, hkv, hkv))
    Wo = rng.standard_normal((h * dh, d)) * 0.3
    full = O.attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, 1, s, h, hkv, dh)
    rows = [0, 3, 10]
    r = O.attn_gqa_query_rows(X, Wq, Wk, Wv, Wo, rows, h, hkv, dh)
    np.testing.assert_allclose(r["O"], full["O"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["Z"], full["Z"][rows], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------- attention backward

@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_matches_finite_differences(causal):
    # The gradients of <dY, Z> with respect to every input, by central
    # differences of the forward definition alone.
    b, s, h, dh, d = 1, 5, 2, 4, 6
    X, Wq, Wk, Wv, Wo = (_tiny((b * s, d), 50), _tiny((d, h * dh), 51, 0.6), _tiny((d, h * dh), 52, 0.6),
                         _tiny((d, h * dh), 53, 0.6), _tiny((h * dh, d), 54, 0.6))
    dY = _tiny((b * s, d), 55)
    loss = lambda: float(np.sum(dY * O.attn_shard_fwd(X, Wq, Wk, Wv, Wo, b, s, h, dh, causal)["Z"]))
    g = O.attn_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b, s, h, dh, causal)
    for name, arr in (("dX", X), ("dWq", Wq), ("dWk", Wk), ("dWv", Wv), ("dWo", Wo)):
        np.testing.assert_allclose(g[name], _fd_grad(loss, arr), atol=2e-8, err_msg=name)


def test_attention_lse_brute_force():
    # L_t = log sum_{u <= t} exp(S[t, u]) written out with math.exp/math.log.
    rng = np.random.default_rng(56)
    s, dh = 7, 3
    Q, K, V = rng.standard_normal((s, dh)), rng.standard_normal((s, dh)), rng.standard_normal((s, dh))
    _, L = O.attn_core_lse(Q, K, V)
    sc = 1 / math.sqrt(dh)
    for t in range(s):
        ref = math.log(math.fsum(math.exp(math.fsum(Q[t, c] * K[u, c] for c in range(dh)) * sc)
                                 for u in range(t + 1)))
        assert abs(L[t] - ref) < 1e-13
    o, _ = O.attn_core_lse(Q, K, V)
    np.testing.assert_allclose(o, O.attn_core(Q, K, V), rtol=1e-14, atol=1e-14)


def test_attention_bwd_special_cases():
    rng = np.random.default_rng(57)
    s, dh = 6, 3
    Q, K, V, dO = (rng.standard_normal((s, dh)) for _ in range(4))
    # One key: the softmax is constant 1, so O = V and only V gets gradient.
    g1 = O.attn_core_bwd(Q[:1], K[:1], V[:1], dO[:1])
    np.testing.assert_array_equal(g1["dV"], dO[:1])
    np.testing.assert_array_equal(g1["dQ"], np.zeros((1, dh)))
    np.testing.assert_array_equal(g1["dK"], np.zeros((1, dh)))
    # K = 0: every allowed key weighs 1/(t+1), so dV_u = sum_{t >= u} dO_t / (t + 1).
    g0 = O.attn_core_bwd(Q, np.zeros_like(K), V, dO)
    w = 1.0 / np.arange(1, s + 1)
    dv = np.array([np.sum(dO[u:] * w[u:, None], axis=0) for u in range(s)])
    np.testing.assert_allclose(g0["dV"], dv, rtol=1e-13, atol=1e-14)
    # Row 0 attends only to key 0 with weight 1: its query gets no gradient.
    g = O.attn_core_bwd(Q, K, V, dO)
    np.testing.assert_allclose(g["dQ"][0], np.zeros(dh), atol=1e-15)
    # Each softmax row's Jacobian sums to zero (sum_u dS[t, u] = 0), so the key
    # gradients cancel: sum_u dK_u = scale * sum_t (sum_u dS[t, u]) Q_t = 0.
    np.testing.assert_allclose(g["dK"].sum(axis=0), np.zeros(dh), atol=1e-13)


def test_attention_bwd_shards_sum_and_concatenate():
    # [HC] 3.4 / [BM] Megatron_f: dX is summed over the head-group shards;
    # the weight gradients are the shards' column (W_Q/W_K/W_V) and row (W_O)
    # slices of the unsharded gradients.
    n, h_l, dh, b, s, d = 3, 2, 4, 2, 6, 12
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "f32", seed=58, w_std=0.3, n_shards=n)
    dY = _tiny((b * s, d), 59)
    full = O.attn_shard_bwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dY, b, s, n * h_l, dh)
    parts = [O.attn_shard_bwd(inp["X"], inp["Wqs"][i], inp["Wks"][i], inp["Wvs"][i], inp["Wos"][i], dY,
                              b, s, h_l, dh) for i in range(n)]
    assert O.max_rel_err(O.shard_reduce([p["dX"] for p in parts]), full["dX"]) < 1e-12
    for k in ("dWq", "dWk", "dWv"):
        np.testing.assert_allclose(np.concatenate([p[k] for p in parts], axis=1), full[k], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([p["dWo"] for p in parts], axis=0), full["dWo"], rtol=1e-12, atol=1e-13)


def test_gqa_bwd_one_group_is_mha_bwd():
    rng = np.random.default_rng(90)
    b, s, d, h, dh = 1, 6, 5, 3, 4
    X = rng.standard_normal((b * s, d))
    Wq, Wk, Wv = (rng.standard_normal((d, h * dh)) * 0.5 for _ in range(3))
    Wo = rng.standard_normal((h * dh, d)) * 0.5
    dY = rng.standard_normal((b * s, d))
    g = O.attn_gqa_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b, s, h, h, dh)
    m = O.attn_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b, s, h, dh)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        np.testing.assert_allclose(g[k], m[k], rtol=1e-12, atol=1e-12)


def test_gqa_bwd_matches_finite_differences_and_repeated_kv_mha():
    """Gradients of <dY, Z> by central differences; and the grouped backward
    equals multi-head attention's with each K/V head's weight columns
    repeated over its group, the repeated copies' gradients summed."""
    rng = np.random.default_rng(91)
    b, s, d, h, hkv, dh = 2, 5, 4, 4, 2, 3
    group = h // hkv
    X = rng.standard_normal((b * s, d))
    Wq = rng.standard_normal((d, h * dh)) * 0.6
    Wk, Wv = (rng.standard_normal((d, hkv * dh)) * 0.6 for _ in range(2))
    Wo = rng.standard_normal((h * dh, d)) * 0.6
    dY = rng.standard_normal((b * s, d))
    g = O.attn_gqa_shard_bwd(X, Wq, Wk, Wv, Wo, dY, b, s, h, hkv, dh)

    def f(X_, Wq_, Wk_, Wv_, Wo_):
        return float((O.attn_gqa_shard_fwd(X_, Wq_, Wk_, Wv_, Wo_, b, s, h, hkv, dh)["Z"] * dY).sum())

    eps = 1e-6
    args = [X, Wq, Wk, Wv, Wo]
    names = ["dX", "dWq", "dWk", "dWv", "dWo"]
    for ai, (r, c) in [(0, (3, 1)), (1, (2, 5)), (2, (1, 4)), (3, (0, 2)), (4, (7, 3))]:
        p, m = [a.copy() for a in args], [a.copy() for a in args]
        p[ai][r, c] += eps
        m[ai][r, c] -= eps
        assert g[names[ai]][r, c] == pytest.approx((f(*p) - f(*m)) / (2 * eps), rel=1e-6, abs=1e-8)

    def rep(W):
        return np.concatenate([W[:, (j // group) * dh:(j // group + 1) * dh] for j in range(h)], axis=1)

    def fold(G):
        return np.concatenate([sum(G[:, (k * group + i) * dh:(k * group + i + 1) * dh] for i in range(group))
                               for k in range(hkv)], axis=1)

    mh = O.attn_shard_bwd(X, Wq, rep(Wk), rep(Wv), Wo, dY, b, s, h, dh)
    np.testing.assert_allclose(g["dX"], mh["dX"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWq"], mh["dWq"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWk"], fold(mh["dWk"]), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dWv"], fold(mh["dWv"]), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------- sequence parallel

def test_reduce_scatter_then_all_gather_is_all_reduce():
    # [HC] Figure 3.2: the all-reduce is a reduce-scatter followed by an
    # all-gather.  The pages' own 4-GPU example: rank r holds [0,1,2,3] + r.
    P = [np.arange(4.0) + r for r in range(4)]
    stripes = [O.reduce_scatter([p[:, None] for p in P], 4, j) for j in range(4)]
    np.testing.assert_array_equal(O.all_gather(stripes)[:, 0], [6, 10, 14, 18])
    rng = np.random.default_rng(63)
    Q = [rng.standard_normal((12, 5)) for _ in range(3)]
    full = O.shard_reduce(Q)
    np.testing.assert_array_equal(O.all_gather([O.reduce_scatter(Q, 3, j) for j in range(3)]), full)
    with pytest.raises(ValueError):
        O.reduce_scatter(Q, 5, 0)                                  # 12 rows over 5 GPUs


def test_layer_norm_brute_force_and_properties():
    rng = np.random.default_rng(64)
    h = rng.standard_normal((3, 7)) * 3 + 1
    g, b = rng.standard_normal(7), rng.standard_normal(7)
    x = O.layer_norm(h, g, b, eps=1e-5)
    for r in range(3):
        mu = math.fsum(h[r]) / 7
        var = math.fsum((v - mu) ** 2 for v in h[r]) / 7
        for c in range(7):
            assert abs(x[r, c] - ((h[r, c] - mu) / math.sqrt(var + 1e-5) * g[c] + b[c])) < 1e-12
    z = O.layer_norm(h, np.ones(7), np.zeros(7), eps=0.0)
    np.testing.assert_allclose(z.mean(axis=1), 0, atol=1e-14)
    np.testing.assert_allclose((z ** 2).mean(axis=1), 1, rtol=1e-13)
    np.testing.assert_allclose(O.layer_norm(np.full((2, 5), 3.0), g[:5], b[:5]), np.tile(b[:5], (2, 1)),
                               atol=1e-12)                         # a constant row gives beta


def test_sp_block_end_definition():
    rng = np.random.default_rng(65)
    n, rows, cols, p = 4, 16, 6, 0.25
    P = [rng.standard_normal((rows, cols)) for _ in range(n)]
    res, g, b, bias = rng.standard_normal((4, cols)), rng.standard_normal(cols), rng.standard_normal(cols), \
        rng.standard_normal(cols)
    keep = (rng.random((4, cols)) >= p).astype(np.float64)
    out = O.sp_block_end(P, n, 2, res, g, b, bias=bias, keep=keep, p_drop=p)
    y = sum(q[8:12] for q in P) + bias
    h = res + y * keep / (1 - p)
    np.testing.assert_allclose(out["h"], h, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["x"], O.layer_norm(h, g, b), rtol=1e-14, atol=1e-14)
    # p = 0 with no mask: dropout is the identity
    out0 = O.sp_block_end(P, n, 0, res, g, b)
    np.testing.assert_allclose(out0["h"], res + sum(q[0:4] for q in P), rtol=1e-14, atol=1e-14)


def test_layer_norm_bwd_matches_finite_differences():
    rng = np.random.default_rng(96)
    h = rng.standard_normal((3, 7)) * 2 + 0.5
    g, b = rng.standard_normal(7), rng.standard_normal(7)
    G = rng.standard_normal((3, 7))
    r = O.layer_norm_bwd(G, h, g)
    L = lambda h_, g_, b_: float((O.layer_norm(h_, g_, b_) * G).sum())
    eps = 1e-6
    for (i, j) in [(0, 0), (1, 3), (2, 6)]:
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        assert r["dh"][i, j] == pytest.approx((L(hp, g, b) - L(hm, g, b)) / (2 * eps), rel=1e-6, abs=1e-9)
    for j in (0, 4):
        gp, gm = g.copy(), g.copy()
        gp[j] += eps
        gm[j] -= eps
        assert r["dgamma"][j] == pytest.approx((L(h, gp, b) - L(h, gm, b)) / (2 * eps), rel=1e-6, abs=1e-9)
        bp, bm = b.copy(), b.copy()
        bp[j] += eps
        bm[j] -= eps
        assert r["dbeta"][j] == pytest.approx((L(h, g, bp) - L(h, g, bm)) / (2 * eps), rel=1e-6, abs=1e-9)
    # a row's input gradient is orthogonal to the constant and to xhat (LayerNorm's invariances)
    np.testing.assert_allclose(r["dh"].sum(axis=1), 0, atol=1e-12)


def test_sp_block_end_bwd_matches_finite_differences():
    """Gradients of <Gx, x> + <Gh, h> through sp_block_end, with Gx the
    reduce-scattered stripe of the shards' summands."""
    rng = np.random.default_rng(97)
    n, rows, cols, index, p = 3, 6, 5, 1, 0.25
    P = rng.standard_normal((n, rows, cols))
    r0, k = O.stripe_rows(rows, n, index)
    res = rng.standard_normal((k, cols))
    g, b, bias = rng.standard_normal(cols), rng.standard_normal(cols), rng.standard_normal(cols)
    keep = (rng.random((k, cols)) > p).astype(np.uint8)
    Gp = rng.standard_normal((n, rows, cols))            # next block's input-gradient summands
    Gh = rng.standard_normal((k, cols))
    Gx = Gp.sum(axis=0)[r0:r0 + k]
    fw = O.sp_block_end(list(P), n, index, res, g, b, bias, keep, p)
    bw = O.sp_block_end_bwd(list(Gp), n, index, fw["h"], g, keep, p, dres=Gh)

    def L(P_, res_, g_, b_, bias_):
        o = O.sp_block_end(list(P_), n, index, res_, g_, b_, bias_, keep, p)
        return float((o["x"] * Gx).sum() + (o["h"] * Gh).sum())

    eps = 1e-6
    for (sh, i, j) in [(0, r0, 0), (2, r0 + 1, 3)]:       # any shard's partial at a stripe row gets dy
        Pp, Pm = P.copy(), P.copy()
        Pp[sh, i, j] += eps
        Pm[sh, i, j] -= eps
        num = (L(Pp, res, g, b, bias) - L(Pm, res, g, b, bias)) / (2 * eps)
        assert bw["dy"][i - r0, j] == pytest.approx(num, rel=1e-6, abs=1e-9)
    for (i, j) in [(0, 2), (1, 4)]:
        rp, rm = res.copy(), res.copy()
        rp[i, j] += eps
        rm[i, j] -= eps
        assert bw["dh"][i, j] == pytest.approx((L(P, rp, g, b, bias) - L(P, rm, g, b, bias)) / (2 * eps),
                                               rel=1e-6, abs=1e-9)
    for j in (1, 3):
        e = np.zeros(cols)
        e[j] = eps
        assert bw["dgamma"][j] == pytest.approx((L(P, res, g + e, b, bias) - L(P, res, g - e, b, bias)) / (2 * eps),
                                                rel=1e-6, abs=1e-9)
        assert bw["dbeta"][j] == pytest.approx((L(P, res, g, b + e, bias) - L(P, res, g, b - e, bias)) / (2 * eps),
                                               rel=1e-6, abs=1e-9)
        assert bw["dbias"][j] == pytest.approx((L(P, res, g, b, bias + e) - L(P, res, g, b, bias - e)) / (2 * eps),
                                               rel=1e-6, abs=1e-9)
    # a partial outside the stripe does not touch this GPU's outputs
    Pp = P.copy()
    Pp[0, 0 if r0 else rows - 1, 0] += 1.0
    assert L(Pp, res, g, b, bias) == pytest.approx(L(P, res, g, b, bias), abs=1e-12)


# -------------------------------------------------------------- shard-reduce

def _read_golden_allreduce():
    ranks, ar, rs = {}, None, {}
    with open(os.path.join(GOLDEN, "allreduce_world4.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            t = line.split()
            if t[0] == "rank":
                ranks[int(t[1])] = [float(v) for v in t[3:]]
            elif t[0] == "allreduce":
                ar = [float(v) for v in t[1:]]
            elif t[0] == "reducescatter":
                rs[int(t[1][4:])] = float(t[2])
    return ranks, ar, rs


def test_shard_reduce_pages_worked_example():
    ranks, ar, rs = _read_golden_allreduce()
    out = O.shard_reduce([ranks[r] for r in range(4)])
    np.testing.assert_array_equal(out, ar)
    for c in range(4):                                # reduce-scatter: column c on rank c
        assert out[c] == rs[c]
    # all-gather of the reduce-scatter pieces rebuilds the all-reduce
    np.testing.assert_array_equal(np.array([rs[c] for c in range(4)]), ar)


def test_shard_reduce_bias_added_once():
    rng = np.random.default_rng(50)
    P = rng.standard_normal((3, 4, 6))
    bias = rng.standard_normal(6)
    out = O.shard_reduce(list(P), bias)
    np.testing.assert_allclose(out - P.sum(axis=0), np.broadcast_to(bias, (4, 6)), atol=1e-14)


def test_shard_range_divisibility():
    assert O.shard_range(4096, 8, 3) == (1536, 512)
    with pytest.raises(ValueError):
        O.shard_range(11008, 3, 0)
    with pytest.raises(ValueError):
        O.shard_range(16, 4, 4)


def test_max_rel_err():
    assert O.max_rel_err([1.0, -2.0], [1.0, -2.0]) == 0.0
    assert O.max_rel_err([1.0, -2.2], [1.0, -2.0]) == pytest.approx(0.1)


# ------------------------------------------------ vocabulary-parallel embedding

def _vocab_case(seed, T=7, d=5, V=24):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((V, d))
    ids = rng.integers(0, V, size=T)
    ids[:4] = [0, V - 1, V // 2, V // 2 - 1]          # both ends and a shard boundary
    return rng, E, ids


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_vocab_embed_equals_one_hot_product(n):
    """[JY] Embedding: the all-reduce of the shards' partials is the lookup in
    the whole table, which is onehot(ids) E."""
    _, E, ids = _vocab_case(60)
    V = E.shape[0]
    shards = [E[i * V // n:(i + 1) * V // n] for i in range(n)]
    onehot = np.zeros((len(ids), V))
    onehot[np.arange(len(ids)), ids] = 1.0
    np.testing.assert_array_equal(O.vocab_embed(ids, shards), onehot @ E)
    # every token's row comes from exactly one shard
    nonzero = np.stack([np.any(O.vocab_embed_shard(ids, shards[i], i * V // n) != 0, axis=1) for i in range(n)])
    np.testing.assert_array_equal(nonzero.sum(axis=0), np.ones(len(ids)))


def test_vocab_embed_shard_brute_force_and_out_of_range_ids():
    """[JY] Implementation (ParallelEmbedding): an id outside the shard's rows
    gives a zero row; an id outside the whole vocabulary is outside every
    shard, so its embedding is zero."""
    _, E, ids = _vocab_case(61)
    ids = np.concatenate([ids, [-1, 24, 1000]])
    start, El = 8, E[8:16]
    y = O.vocab_embed_shard(ids, El, start)
    for t, v in enumerate(ids):
        want = El[v - start] if start <= v < start + 8 else np.zeros(E.shape[1])
        np.testing.assert_array_equal(y[t], want)
    full = O.vocab_embed(ids, [E[0:8], E[8:16], E[16:24]])
    np.testing.assert_array_equal(full[-3:], np.zeros((3, E.shape[1])))


def test_vocab_embed_bwd_one_hot_product_and_finite_differences():
    """dE_local = onehot(ids - start)^T dY over the shard's rows; the gradient
    of <dY, Y_i> with respect to the shard's table; the shards' gradients
    stacked are the whole table's."""
    rng, E, ids = _vocab_case(66, T=9, d=4, V=12)
    ids = np.concatenate([ids, [5, 5, -1, 12]])         # a repeated id and two in no shard
    dY = rng.standard_normal((len(ids), 4))
    n, V = 3, 12
    parts = [O.vocab_embed_shard_bwd(ids, dY, V // n, i * V // n) for i in range(n)]
    onehot = np.zeros((len(ids), V))
    ok = (ids >= 0) & (ids < V)
    onehot[np.nonzero(ok)[0], ids[ok]] = 1.0
    np.testing.assert_allclose(np.concatenate(parts), onehot.T @ dY, rtol=1e-14, atol=1e-14)
    eps = 1e-6
    for (i, r, c) in [(0, 0, 1), (1, 1, 3), (2, 3, 0)]:
        Es = [E[k * V // n:(k + 1) * V // n].copy() for k in range(n)]
        Ep, Em = Es[i].copy(), Es[i].copy()
        Ep[r, c] += eps
        Em[r, c] -= eps
        f = lambda El: float((O.vocab_embed_shard(ids, El, i * V // n) * dY).sum())
        assert parts[i][r, c] == pytest.approx((f(Ep) - f(Em)) / (2 * eps), rel=1e-7, abs=1e-9)


def _ce_brute(X, E, targets):
    out = []
    for t in range(X.shape[0]):
        z = [sum(X[t, k] * E[v, k] for k in range(X.shape[1])) for v in range(E.shape[0])]
        zmax = max(z)
        lse = zmax + math.log(sum(math.exp(zv - zmax) for zv in z))
        out.append((lse - z[targets[t]], lse))
    return np.array(out)


@pytest.mark.parametrize("n", [1, 2, 3, 6])
def test_vocab_ce_brute_force(n):
    """Fused output embedding + cross-entropy ([JY] Embedding) equals
    -log softmax(X E^T)[target] computed with plain loops."""
    rng = np.random.default_rng(62)
    T, d, V = 4, 3, 12
    X, E = rng.standard_normal((T, d)), rng.standard_normal((V, d))
    targets = np.array([0, 11, 5, 6])
    got = O.vocab_ce_fwd(X, [E[i * V // n:(i + 1) * V // n] for i in range(n)], targets)
    ref = _ce_brute(X, E, targets)
    np.testing.assert_allclose(got["loss"], ref[:, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["lse"], ref[:, 1], rtol=1e-12, atol=1e-12)


def test_vocab_ce_closed_forms():
    rng = np.random.default_rng(63)
    T, d, V = 5, 4, 16
    E = rng.standard_normal((V, d))
    targets = rng.integers(0, V, size=T)
    shards = [E[0:4], E[4:8], E[8:12], E[12:16]]
    # zero hidden states: every logit is 0, the loss is log V
    r = O.vocab_ce_fwd(np.zeros((T, d)), shards, targets)
    np.testing.assert_allclose(r["loss"], np.full(T, math.log(V)), rtol=1e-14)
    # one logit 1000 above the rest: the loss of that target vanishes and
    # the shifted log-sum-exp does not overflow
    X = np.zeros((1, d))
    X[0, 0] = 1.0
    Eb = np.zeros((V, d))
    Eb[9, 0] = 1000.0
    r = O.vocab_ce_fwd(X, [Eb[0:8], Eb[8:16]], [9])
    assert abs(r["loss"][0]) < 1e-300 and r["lse"][0] == pytest.approx(1000.0)
    r = O.vocab_ce_fwd(X, [Eb[0:8], Eb[8:16]], [3])
    assert r["loss"][0] == pytest.approx(1000.0)


def test_vocab_ce_shard_count_independence():
    rng = np.random.default_rng(64)
    T, d, V = 6, 8, 48
    X, E = rng.standard_normal((T, d)), rng.standard_normal((V, d))
    targets = rng.integers(0, V, size=T)
    ref = O.vocab_ce_fwd(X, [E], targets)
    for n in (2, 4, 8):
        got = O.vocab_ce_fwd(X, [E[i * V // n:(i + 1) * V // n] for i in range(n)], targets)
        np.testing.assert_allclose(got["loss"], ref["loss"], rtol=1e-13)


def test_vocab_ce_bwd_matches_finite_differences():
    """Gradients of L = sum_t dloss_t loss_t: the shards' dX summands add up
    to dL/dX, and dE_i is the i-th row block of dL/dE."""
    rng = np.random.default_rng(65)
    T, d, V, n = 5, 4, 12, 3
    X, E = rng.standard_normal((T, d)), rng.standard_normal((V, d))
    targets = np.array([0, 11, 4, 7, 3])
    dloss = rng.uniform(0.5, 1.5, size=T)
    shards = [E[i * V // n:(i + 1) * V // n] for i in range(n)]
    lse = O.vocab_ce_fwd(X, shards, targets)["lse"]
    parts = [O.vocab_ce_shard_bwd(X, shards[i], targets, i * V // n, lse, dloss) for i in range(n)]
    dX = sum(p["dX"] for p in parts)
    dE = np.concatenate([p["dE"] for p in parts])

    def L(X_, E_):
        return float((O.vocab_ce_fwd(X_, [E_[i * V // n:(i + 1) * V // n] for i in range(n)], targets)["loss"]
                      * dloss).sum())

    h = 1e-6
    for (t, k) in [(0, 0), (2, 3), (4, 1)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[t, k] += h
        Xm[t, k] -= h
        assert dX[t, k] == pytest.approx((L(Xp, E) - L(Xm, E)) / (2 * h), rel=1e-6, abs=1e-8)
    for (v, k) in [(0, 0), (4, 2), (11, 3), (7, 1)]:
        Ep, Em = E.copy(), E.copy()
        Ep[v, k] += h
        Em[v, k] -= h
        assert dE[v, k] == pytest.approx((L(X, Ep) - L(X, Em)) / (2 * h), rel=1e-6, abs=1e-8)
    # softmax minus one-hot: each token's gradient over the whole vocabulary sums to 0
    dz = np.concatenate([p["dlogits"] for p in parts], axis=1)
    np.testing.assert_allclose(dz.sum(axis=1), np.zeros(T), atol=1e-14)


# --------------------------------------------------------------- input recipe

def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8), 3.0e38],
                    dtype=np.float32)
    r = tpsynth.round_to_bf16(vals)
    np.testing.assert_array_equal(r[:4], np.array([1.0, 1.0 + 2 ** -6, 1.0, -1.0], dtype=np.float32))
    assert np.isfinite(r[4])


def test_workload_shapes():
    W = tpsynth.WORKLOADS
    assert (W["C2"].M, W["C2"].f_local) == (8192, 512)
    assert W["C3"].f_local == 2752 and W["C4"].h_local == 8
    assert (W["C5"].M, W["C5"].d, W["C5"].f_local) == (8192, 8192, 4096)


# --------------------------------------------------------------- error metrics

def test_error_metrics():
    ref = np.array([1.0, -2.0, 1e-6, 0.0])
    # max_rel_err is measured against the tensor's largest entry
    y = ref.copy()
    y[2] += 1e-6                     # doubles a tiny entry
    assert O.max_rel_err(y, ref) == pytest.approx(5e-7)
    # per-element: that entry's error against the floor 1e-3 * ||ref||_inf = 2e-3
    assert O.per_element_rel_err(y, ref) == pytest.approx(1e-6 / 2e-3)
    # an entry above the floor is measured against itself
    z = ref * np.array([1.0, 1.0 + 3e-3, 1.0, 1.0])
    assert O.per_element_rel_err(z, ref) == pytest.approx(3e-3)
    assert O.max_rel_err(z, ref) == pytest.approx(3e-3)
    # a uniform relative error is the same under both metrics
    w = ref * (1 + 1e-4)
    assert O.per_element_rel_err(w, ref) == pytest.approx(1e-4)
    assert O.max_rel_err(ref, ref) == 0.0 and O.per_element_rel_err(ref, ref) == 0.0


def test_per_element_error_of_bf16_rounding_alone():
    """What the per-element figure means for a bf16 path.  Rounding only the
    stored hidden activation H to bf16 (everything else exact, fp64) already
    gives Z = H W2 a per-element error near 1 against the fp64 oracle, while
    its norm-relative error stays far inside the 2e-2 bound: entries of Z
    that cancel to below 1e-3 of its largest carry the rounding error of the
    whole sum.  This is the figure the C5 line reports for Z, dX and the
    weight gradients."""
    import tpsynth
    rng = np.random.default_rng(5)
    M, d, f = 512, 256, 1024
    X = tpsynth.round_to_bf16(rng.standard_normal((M, d)).astype(np.float32)).astype(np.float64)
    W1 = tpsynth.round_to_bf16((0.02 * rng.standard_normal((d, f))).astype(np.float32)).astype(np.float64)
    W2 = tpsynth.round_to_bf16((0.02 * rng.standard_normal((f, d))).astype(np.float32)).astype(np.float64)
    ref = O.mlp_shard_fwd(X, W1, W2)
    Hb = tpsynth.round_to_bf16(ref["H"].astype(np.float32)).astype(np.float64)
    Z = Hb @ W2
    assert O.max_rel_err(Z, ref["Z"]) < 5e-3
    assert O.per_element_rel_err(Z, ref["Z"]) > 0.1
    # the hidden activation itself is one rounding away (2^-9 relative, more
    # only for entries measured against the floor)
    assert O.per_element_rel_err(Hb, ref["H"]) < 1e-2
