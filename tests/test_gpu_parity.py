"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar: max_rel_err = ||gpu - oracle||_inf / ||oracle||_inf <= 2e-2 for bf16
inputs with fp32 accumulation and <= 1e-5 for the all-fp32 path, for every
output tensor.  Inputs are the seeded synthetic ones (tpsynth); the oracle
sees exactly the bf16-rounded values the GPU sees.  Full-size workloads are
checked on sampled rows and columns the oracle computes directly (rows of
the output depend only on rows of X and dY; a subset of the shard's d_ff
columns is itself a smaller shard).
"""
import math
import sys

import numpy as np
import pytest

import oracle as O
import tpsynth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import megatron_tensor_transformer_fwd_amd as m
    m.lib()          # raises if the library is missing: no fallback path exists
    return m


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def empty(shape, dtype):
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")


def check(name, got, ref, dtype):
    err = O.max_rel_err(host(got) if torch.is_tensor(got) else got, ref)
    assert np.isfinite(err) and err <= TOL[dtype], f"{name}: max_rel_err {err:.3e} > {TOL[dtype]}"
    return err


def run_mlp_shard(tp, X, W1, W2, dY, dtype):
    M, d = X.shape
    f = W1.shape[1]
    A, H, Z = empty((M, f), dtype), empty((M, f), dtype), empty((M, d), dtype)
    tp.tp_mlp_fwd(X, W1, W2, A, H, Z)
    out = {"A": A, "H": H, "Z": Z}
    if dY is not None:
        dX = empty((M, d), dtype)
        dW1 = torch.empty((d, f), dtype=torch.float32, device="cuda")
        dW2 = torch.empty((f, d), dtype=torch.float32, device="cuda")
        dt = tp.TP_DT_BF16 if dtype == "bf16" else tp.TP_DT_F32
        ws = torch.empty(tp.tp_mlp_bwd_workspace_bytes(dt, M, d, f), dtype=torch.uint8, device="cuda")
        tp.tp_mlp_bwd(X, W1, W2, A, H, dY, dX, dW1, dW2, ws)
        out.update(dX=dX, dW1=dW1, dW2=dW2)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------- shard-reduce

def test_shard_reduce_pages_worked_example(tp):
    _say("shard_reduce pages example")
    # "Chapter 8: Distributed Training", 8.4.2: ranks r = 0..3 hold [0,1,2,3] + r
    for dtype in ("f32", "bf16"):
        P = dev(np.stack([np.arange(4) + r for r in range(4)]), dtype)
        out = empty((4,), dtype)
        tp.tp_shard_reduce(P, out, 4, 4)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), [6, 10, 14, 18])


@pytest.mark.parametrize("dtype_in,dtype_out,n,numel,stride,bias_len", [
    ("bf16", "bf16", 8, 8192 * 1024, None, 0),        # C2: 8 partials of [8192 x 1024]
    ("bf16", "bf16", 3, 1001, 1008, 7),                # ragged numel, padded stride, bias
    ("f32", "f32", 2, 32 * 64, None, 64),              # C1 size with a row bias
    ("bf16", "f32", 5, 4099, 4101, 0),                 # stride breaks 16-byte alignment
    ("f32", "bf16", 9, 77, None, 0),
])
def test_shard_reduce_random(tp, dtype_in, dtype_out, n, numel, stride, bias_len):
    _say(f"shard_reduce {dtype_in}->{dtype_out} n={n} numel={numel} stride={stride} bias={bias_len}")
    st = stride or numel
    inp = tpsynth.reduce_inputs(n, st, dtype_in, seed=3, bias_len=bias_len)
    P = dev(inp["P"], dtype_in)
    bias = dev(inp["bias"], dtype_in) if bias_len else None
    out = empty((numel,), dtype_out)
    tp.tp_shard_reduce(P, out, n, numel, shard_stride=st, bias=bias)
    torch.cuda.synchronize()
    ref = O.shard_reduce([inp["P"][i, :numel] for i in range(n)], inp["bias"])
    check("out", out, ref, "bf16" if "bf16" in (dtype_in, dtype_out) else "f32")
    out2 = empty((numel,), dtype_out)
    tp.tp_shard_reduce(P, out2, n, numel, shard_stride=st, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "shard-reduce is not bitwise deterministic"


def test_shard_reduce_in_place(tp):
    _say("shard_reduce in place")
    inp = tpsynth.reduce_inputs(4, 4096, "bf16", seed=4)
    P = dev(inp["P"], "bf16")
    tp.tp_shard_reduce(P, P[0], 4, 4096)
    torch.cuda.synchronize()
    check("out", P[0], O.shard_reduce(list(inp["P"])), "bf16")


# ---------------------------------------------------------------- GeLU MLP

def test_mlp_c1_fp32_two_shards(tp):
    _say("mlp C1 fp32, both shards, Z and dX reduces")
    wl = tpsynth.WORKLOADS["C1"]
    inp = tpsynth.mlp_inputs(wl)
    X, dY = dev(inp["X"], "f32"), dev(inp["dY"], "f32")
    Zs, dXs = [], []
    for i in range(wl.n_shards):
        W1, W2 = inp["W1s"][i], inp["W2s"][i]
        out = run_mlp_shard(tp, X, dev(W1, "f32"), dev(W2, "f32"), dY, "f32")
        ref = O.mlp_shard_fwd(inp["X"], W1, W2)
        refb = O.mlp_shard_bwd(inp["X"], W1, W2, inp["dY"])
        for k in ("A", "H", "Z"):
            check(f"{k}_{i}", out[k], ref[k], "f32")
        for k in ("dX", "dW1", "dW2"):
            check(f"{k}_{i}", out[k], refb[k], "f32")
        Zs.append(out["Z"])
        dXs.append(out["dX"])
    M, d = inp["X"].shape
    Zp, dXp = torch.stack(Zs), torch.stack(dXs)
    Z, dX = empty((M, d), "f32"), empty((M, d), "f32")
    tp.tp_shard_reduce(Zp, Z, wl.n_shards, M * d)
    tp.tp_shard_reduce(dXp, dX, wl.n_shards, M * d)
    torch.cuda.synchronize()
    check("Y", Z, O.mlp_unsharded(inp["X"], inp["W1"], inp["W2"]), "f32")
    check("dX", dX, O.mlp_unsharded_bwd(inp["X"], inp["W1"], inp["W2"], inp["dY"])["dX"], "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,d,f", [(300, 136, 200), (1, 8, 8), (520, 264, 392), (64, 64, 128)])
def test_mlp_ragged_shapes(tp, dtype, M, d, f):
    _say(f"mlp ragged {dtype} M={M} d={d} f={f}")
    inp = tpsynth.random_mlp(M, d, f, dtype, seed=M + d + f, w_std=0.05)
    out = run_mlp_shard(tp, dev(inp["X"], dtype), dev(inp["W1"], dtype), dev(inp["W2"], dtype),
                        dev(inp["dY"], dtype), dtype)
    ref = O.mlp_shard_fwd(inp["X"], inp["W1"], inp["W2"])
    refb = O.mlp_shard_bwd(inp["X"], inp["W1"], inp["W2"], inp["dY"])
    for k in ("A", "H", "Z"):
        check(k, out[k], ref[k], dtype)
    for k in ("dX", "dW1", "dW2"):
        check(k, out[k], refb[k], dtype)


def _slice_rel_err(got, ref, axis):
    """The worst slice's ||got - ref||_inf / ||ref||_inf, slices taken along
    `axis` (axis 0: each column over its rows; axis 1: each row)."""
    g = host(got).astype(np.float64)
    return float((np.abs(g - ref).max(axis=axis) / np.abs(ref).max(axis=axis)).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mlp_slices_of_unequal_scale(tp, dtype):
    """W1's columns and W2's rows scaled over three decades (log-spaced 1e-3 .. 1
    along d_ff): A, H and dW1 then have columns, and dW2 rows, from about 1e-3
    to 1 of the tensor's largest.  Each such slice depends only on its own
    weight slice, and each is compared with the oracle against its own largest
    value, so a small slice cannot pass on the tensor's norm alone."""
    M, d, f = 512, 256, 384
    _say(f"mlp slices of unequal scale {dtype} M={M} d={d} f={f}")
    inp = tpsynth.random_mlp(M, d, f, dtype, seed=17, w_std=0.05)
    sc = np.logspace(-3.0, 0.0, f)
    rnd = tpsynth.round_to_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    W1 = rnd((inp["W1"] * sc[None, :]).astype(np.float32))
    W2 = rnd((inp["W2"] * sc[:, None]).astype(np.float32))
    out = run_mlp_shard(tp, dev(inp["X"], dtype), dev(W1, dtype), dev(W2, dtype), dev(inp["dY"], dtype), dtype)
    ref = O.mlp_shard_fwd(inp["X"], W1, W2)
    refb = O.mlp_shard_bwd(inp["X"], W1, W2, inp["dY"])
    for k, r, axis in (("A", ref["A"], 0), ("H", ref["H"], 0), ("dW1", refb["dW1"], 0), ("dW2", refb["dW2"], 1)):
        err = _slice_rel_err(out[k], r, axis)
        assert err <= TOL[dtype], f"{k}: worst slice max_rel_err {err:.3e} > {TOL[dtype]}"
    for k in ("Z", "dX"):
        check(k, out[k], (ref if k == "Z" else refb)[k], dtype)


def test_mlp_row_pitch_limit(tp):
    """d at the ABI's row-pitch limit (2^21 elements): every operand tile spans
    256 rows of 4 MiB, the widest the kernels address with 32-bit offsets
    from a tile's first row.  M 64, f 64, forward and backward, every tensor."""
    M, d, f = 64, 1 << 21, 64
    _say(f"mlp row-pitch limit bf16 M={M} d={d} f={f}")
    rng = np.random.default_rng(99)
    X = tpsynth.normal(rng, (M, d), 1.0, "bf16")
    W1 = tpsynth.normal(rng, (d, f), d ** -0.5, "bf16")
    W2 = tpsynth.normal(rng, (f, d), 0.1, "bf16")
    dY = tpsynth.normal(rng, (M, d), 1.0, "bf16")
    out = run_mlp_shard(tp, dev(X, "bf16"), dev(W1, "bf16"), dev(W2, "bf16"), dev(dY, "bf16"), "bf16")
    ref = O.mlp_shard_fwd(X, W1, W2)
    for k in ("A", "H", "Z"):
        check(k, out[k], ref[k], "bf16")
    refb = O.mlp_shard_bwd(X, W1, W2, dY)
    for k in ("dX", "dW1", "dW2"):
        check(k, out[k], refb[k], "bf16")


def _launch_labels(tp, fn):
    """Run fn() with the library's launch hook armed; the labels of its launches."""
    import bench
    L = tp.lib()
    ev = bench.HipEvents(128)
    assert L.tp_profile_begin(ev.start, ev.stop, ev.n) == 0
    try:
        r = fn()
        torch.cuda.synchronize()
    finally:
        n = L.tp_profile_end()
    labels = [L.tp_profile_label(i).decode() for i in range(n)]
    ev.close()
    return r, labels


def _act_grid(n, lo=-10.0, hi=10.0, seed=0):
    """n x n values spread over [lo, hi] in shuffled order (the activations' tails included)."""
    v = np.linspace(lo, hi, n * n)
    np.random.default_rng(seed).shuffle(v)
    return v.reshape(n, n)


def _as_dtype(a, dtype):
    """The values the device holds: rounded to bf16 (or fp32) on the host."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.float().numpy().astype(np.float64)


def _elementwise(name, got, ref, scale, rtol):
    g = host(got)
    bad = np.abs(g - ref) > rtol * scale
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements off, worst at x-index "
                           f"{np.unravel_index(np.argmax(np.abs(g - ref) / scale), ref.shape)}")


_ACT_RTOL = {"bf16": 2.0 ** -8, "f32": 1e-5}


@pytest.mark.parametrize("n", [64, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gelu_elementwise_tails(tp, dtype, n):
    """GeLU and GeLU' value by value over [-10, 10]: with X = W2 = I the forward
    gives A = W1 and H = GeLU(W1), and the backward's dW1 = X^T dA is
    dA = dY * GeLU'(W1) itself, each rounded once to the output type.  The
    bound is relative to each value (to |dY| (Phi + |x| phi) for GeLU', which
    crosses zero), so the lower tail, where GeLU is tiny, is checked too.
    n = 64 leaves every output tile ragged (the bounds-checked epilogue);
    n = 512 fills whole tiles (the unchecked one)."""
    _say(f"gelu elementwise tails {dtype} n {n}")
    I = np.eye(n)
    W1 = _as_dtype(_act_grid(n, seed=1), dtype)
    dY = _as_dtype(np.random.default_rng(2).standard_normal((n, n)), dtype)
    out = run_mlp_shard(tp, dev(I, dtype), dev(W1, dtype), dev(I, dtype), dev(dY, dtype), dtype)
    rtol = _ACT_RTOL[dtype]
    np.testing.assert_array_equal(host(out["A"]), W1)
    H = O.gelu(W1)
    _elementwise("H", out["H"], H, np.abs(H), rtol)
    _elementwise("Z", out["Z"], H, np.abs(H), rtol)
    phi = np.exp(-0.5 * W1 * W1) / math.sqrt(2 * math.pi)
    cdf = 0.5 * np.vectorize(math.erfc)(-W1 / math.sqrt(2))
    _elementwise("dA (dW1)", out["dW1"], dY * O.gelu_prime(W1), np.abs(dY) * (cdf + np.abs(W1) * phi), rtol)


@pytest.mark.parametrize("n", [64, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swiglu_elementwise_tails(tp, dtype, n):
    """Swish and Swish' value by value: with X = W2 = I, G = W1 and U = W3, so
    H = Swish(W1) * W3, and the weight gradients are dW1 = dG = dY * U * Swish'(G)
    and dW3 = dU = dY * Swish(G) themselves (n as in the GeLU test)."""
    _say(f"swiglu elementwise tails {dtype} n {n}")
    I = np.eye(n)
    W1 = _as_dtype(_act_grid(n, seed=3), dtype)
    W3 = _as_dtype(np.random.default_rng(4).standard_normal((n, n)), dtype)
    dY = _as_dtype(np.random.default_rng(5).standard_normal((n, n)), dtype)
    inp = {"X": I, "W1": W1, "W3": W3, "W2": I, "dY": dY}
    out = run_swiglu(tp, inp, dtype)
    rtol = _ACT_RTOL[dtype]
    H = O.swish(W1) * W3
    _elementwise("H", out["H"], H, np.abs(H), rtol)
    sig = 1.0 / (1.0 + np.exp(-W1))
    dU = dY * O.swish(W1)
    _elementwise("dU (dW3)", out["dW3"], dU, np.abs(dU), rtol)
    dG = dY * W3 * O.swish_prime(W1)
    _elementwise("dG (dW1)", out["dW1"], dG, np.abs(dY * W3) * sig * (1 + np.abs(W1) * (1 - sig)), rtol)


def test_mlp_c2_all_shards_and_reduces(tp):
    _say("mlp C2 bf16, 8 shards + Z/dX shard-reduce")
    wl = tpsynth.WORKLOADS["C2"]
    inp = tpsynth.mlp_inputs(wl)
    M, d = inp["X"].shape
    X, dY = dev(inp["X"], "bf16"), dev(inp["dY"], "bf16")
    Zp = empty((wl.n_shards, M, d), "bf16")
    dXp = empty((wl.n_shards, M, d), "bf16")
    for i in range(wl.n_shards):
        out = run_mlp_shard(tp, X, dev(inp["W1s"][i], "bf16"), dev(inp["W2s"][i], "bf16"), dY, "bf16")
        Zp[i].copy_(out["Z"])
        dXp[i].copy_(out["dX"])
        if i in (0, wl.n_shards - 1):   # every output tensor of two shards, in full
            ref = O.mlp_shard_fwd(inp["X"], inp["W1s"][i], inp["W2s"][i])
            refb = O.mlp_shard_bwd(inp["X"], inp["W1s"][i], inp["W2s"][i], inp["dY"])
            for k in ("A", "H", "Z"):
                check(f"{k}_{i}", out[k], ref[k], "bf16")
            for k in ("dX", "dW1", "dW2"):
                check(f"{k}_{i}", out[k], refb[k], "bf16")
    Z, dX = empty((M, d), "bf16"), empty((M, d), "bf16")
    tp.tp_shard_reduce(Zp, Z, wl.n_shards, M * d)
    tp.tp_shard_reduce(dXp, dX, wl.n_shards, M * d)
    torch.cuda.synchronize()
    check("Y", Z, O.mlp_unsharded(inp["X"], inp["W1"], inp["W2"]), "bf16")
    check("dX", dX, O.mlp_unsharded_bwd(inp["X"], inp["W1"], inp["W2"], inp["dY"])["dX"], "bf16")


def run_mlp_shards(tp, X, W1s, W2s, dY, dtype):
    """Every shard in one call per direction (tp_mlp_fwd_shards / _bwd_shards)."""
    n, d, f = W1s.shape
    M = X.shape[0]
    A, H = empty((n, M, f), dtype), empty((n, M, f), dtype)
    Z, dX = empty((n, M, d), dtype), empty((n, M, d), dtype)
    dW1 = torch.empty((n, d, f), dtype=torch.float32, device="cuda")
    dW2 = torch.empty((n, f, d), dtype=torch.float32, device="cuda")
    dt = tp.TP_DT_BF16 if dtype == "bf16" else tp.TP_DT_F32
    ws = torch.empty(tp.tp_mlp_bwd_shards_workspace_bytes(dt, n, M, d, f), dtype=torch.uint8, device="cuda")
    tp.tp_mlp_fwd_shards(X, W1s, W2s, A, H, Z)
    tp.tp_mlp_bwd_shards(X, W1s, W2s, A, H, dY, dX, dW1, dW2, ws)
    torch.cuda.synchronize()
    return dict(A=A, H=H, Z=Z, dX=dX, dW1=dW1, dW2=dW2)


def test_mlp_c2_shards_in_one_call(tp):
    """C2's 8 shards through the all-shards entry points: every tensor of
    every shard against the oracle, and both shard-reduces against the
    unsharded layer."""
    _say("mlp C2 bf16, all 8 shards per call + Z/dX shard-reduce")
    wl = tpsynth.WORKLOADS["C2"]
    inp = tpsynth.mlp_inputs(wl)
    M, d = inp["X"].shape
    n = wl.n_shards
    W1s = dev(np.stack(inp["W1s"]), "bf16")
    W2s = dev(np.stack(inp["W2s"]), "bf16")
    out = run_mlp_shards(tp, dev(inp["X"], "bf16"), W1s, W2s, dev(inp["dY"], "bf16"), "bf16")
    for i in range(n):
        ref = O.mlp_shard_fwd(inp["X"], inp["W1s"][i], inp["W2s"][i])
        refb = O.mlp_shard_bwd(inp["X"], inp["W1s"][i], inp["W2s"][i], inp["dY"])
        for k in ("A", "H", "Z"):
            check(f"{k}_{i}", out[k][i], ref[k], "bf16")
        for k in ("dX", "dW1", "dW2"):
            check(f"{k}_{i}", out[k][i], refb[k], "bf16")
    Z, dX = empty((M, d), "bf16"), empty((M, d), "bf16")
    tp.tp_shard_reduce(out["Z"], Z, n, M * d)
    tp.tp_shard_reduce(out["dX"], dX, n, M * d)
    torch.cuda.synchronize()
    check("Y", Z, O.mlp_unsharded(inp["X"], inp["W1"], inp["W2"]), "bf16")
    check("dX", dX, O.mlp_unsharded_bwd(inp["X"], inp["W1"], inp["W2"], inp["dY"])["dX"], "bf16")


@pytest.mark.parametrize("dtype,n,M,d,f", [
    ("bf16", 3, 300, 72, 40),       # ragged in every dimension
    ("bf16", 5, 1000, 520, 264),    # several tiles, ragged tails
    ("bf16", 1, 64, 64, 128),
    ("f32", 2, 32, 64, 128),        # C1's shape
    ("f32", 3, 100, 40, 24),
])
def test_mlp_shards_ragged(tp, dtype, n, M, d, f):
    _say(f"mlp all shards per call {dtype} n={n} M={M} d={d} f={f}")
    inp = tpsynth.random_mlp(M, d, n * f, dtype, seed=M + n)
    W1s = np.stack([inp["W1"][:, i * f:(i + 1) * f] for i in range(n)])
    W2s = np.stack([inp["W2"][i * f:(i + 1) * f] for i in range(n)])
    out = run_mlp_shards(tp, dev(inp["X"], dtype), dev(W1s, dtype), dev(W2s, dtype), dev(inp["dY"], dtype), dtype)
    for i in range(n):
        ref = O.mlp_shard_fwd(inp["X"], W1s[i], W2s[i])
        refb = O.mlp_shard_bwd(inp["X"], W1s[i], W2s[i], inp["dY"])
        for k in ("A", "H", "Z"):
            check(f"{k}_{i}", out[k][i], ref[k], dtype)
        for k in ("dX", "dW1", "dW2"):
            check(f"{k}_{i}", out[k][i], refb[k], dtype)
    # the shards' Z sum to the unsharded layer's output
    full = O.mlp_unsharded(inp["X"], inp["W1"], inp["W2"])
    check("sum Z", host(out["Z"]).sum(axis=0), full, dtype)


def test_mlp_shards_f32_beyond_one_launch(tp):
    """fp32 shards whose launch grid would exceed the z limit (64 shards x
    1024 column tiles of f = 65536) run in groups of shards: every tensor of
    the first, a middle and the last shard against the oracle.  W1's columns
    and W2's rows are zero outside 16 positions per shard (the same ones), so
    the 65536-long sums have at most 16 nonzero terms and the fp32 results
    stay within the fp32 tolerance; the positions include both ends of f."""
    n, M, d, f = 64, 8, 8, 65536
    _say(f"mlp all shards per call f32 n={n} M={M} d={d} f={f} (shard groups)")
    rng = np.random.default_rng(7)
    X = rng.standard_normal((M, d)).astype(np.float32)
    dY = rng.standard_normal((M, d)).astype(np.float32)
    W1s = np.zeros((n, d, f), np.float32)
    W2s = np.zeros((n, f, d), np.float32)
    for i in range(n):
        cols = np.unique(np.concatenate([[0, f - 1], rng.choice(f, 14, replace=False)]))
        W1s[i][:, cols] = rng.standard_normal((d, cols.size)).astype(np.float32)
        W2s[i][cols, :] = rng.standard_normal((cols.size, d)).astype(np.float32)
    out = run_mlp_shards(tp, dev(X, "f32"), dev(W1s, "f32"), dev(W2s, "f32"), dev(dY, "f32"), "f32")
    for i in (0, 31, 62, 63):
        ref = O.mlp_shard_fwd(X, W1s[i], W2s[i])
        refb = O.mlp_shard_bwd(X, W1s[i], W2s[i], dY)
        for k in ("A", "H", "Z"):
            check(f"{k}_{i}", out[k][i], ref[k], "f32")
        for k in ("dX", "dW1", "dW2"):
            check(f"{k}_{i}", out[k][i], refb[k], "f32")


def test_mlp_bwd_bitwise_deterministic(tp):
    _say("mlp C2-shard backward twice, bitwise")
    wl = tpsynth.WORKLOADS["C2"]
    inp = tpsynth.mlp_inputs(wl)
    args = (dev(inp["X"], "bf16"), dev(inp["W1s"][3], "bf16"), dev(inp["W2s"][3], "bf16"), dev(inp["dY"], "bf16"))
    a = run_mlp_shard(tp, *args, "bf16")
    b = run_mlp_shard(tp, *args, "bf16")
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n, size=k, replace=False))
    idx[0], idx[-1] = 0, n - 1      # the first and last row/column always
    return np.unique(idx)


def test_mlp_c5_full_size_sampled(tp):
    _say("mlp C5 bf16 full size, sampled rows/cols")
    wl = tpsynth.WORKLOADS["C5"]
    inp = tpsynth.mlp_inputs(wl)
    Xh, W1h, W2h, dYh = inp["X"], inp["W1s"][0], inp["W2s"][0], inp["dY"]
    out = run_mlp_shard(tp, dev(Xh, "bf16"), dev(W1h, "bf16"), dev(W2h, "bf16"), dev(dYh, "bf16"), "bf16")
    rows = _sample(wl.M, 48, 11)
    cols = _sample(wl.f_local, 16, 12)
    ref = O.mlp_shard_fwd(Xh[rows], W1h, W2h)
    for k in ("A", "H", "Z"):
        check(k, host(out[k])[rows], ref[k], "bf16")
    check("dX", host(out["dX"])[rows], O.mlp_shard_bwd(Xh[rows], W1h, W2h, dYh[rows])["dX"], "bf16")
    sub = O.mlp_shard_bwd(Xh, W1h[:, cols], W2h[cols], dYh)      # the columns `cols` as a sub-shard
    check("dW1", host(out["dW1"])[:, cols], sub["dW1"], "bf16")
    check("dW2", host(out["dW2"])[cols], sub["dW2"], "bf16")


# ------------------------------------------------------------------ SwiGLU

def run_swiglu(tp, inp, dtype):
    X, W1, W3, W2, dY = (dev(inp[k], dtype) for k in ("X", "W1", "W3", "W2", "dY"))
    M, d = X.shape
    f = W1.shape[1]
    G, U, H = empty((M, f), dtype), empty((M, f), dtype), empty((M, f), dtype)
    Z = empty((M, d), dtype)
    tp.tp_swiglu_fwd(X, W1, W3, W2, G, U, H, Z)
    dX = empty((M, d), dtype)
    dW1, dW3 = (torch.empty((d, f), dtype=torch.float32, device="cuda") for _ in range(2))
    dW2 = torch.empty((f, d), dtype=torch.float32, device="cuda")
    dt = tp.TP_DT_BF16 if dtype == "bf16" else tp.TP_DT_F32
    ws = torch.empty(tp.tp_swiglu_bwd_workspace_bytes(dt, M, d, f), dtype=torch.uint8, device="cuda")
    tp.tp_swiglu_bwd(X, W1, W3, W2, G, U, H, dY, dX, dW1, dW3, dW2, ws)
    torch.cuda.synchronize()
    return dict(G=G, U=U, H=H, Z=Z, dX=dX, dW1=dW1, dW3=dW3, dW2=dW2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,d,f", [(300, 136, 200), (257, 64, 2752 // 8), (8, 8, 8)])
def test_swiglu_ragged_shapes(tp, dtype, M, d, f):
    _say(f"swiglu ragged {dtype} M={M} d={d} f={f}")
    inp = tpsynth.random_swiglu(M, d, f, dtype, seed=M * 3 + f, w_std=0.05)
    out = run_swiglu(tp, inp, dtype)
    ref = O.swiglu_shard_fwd(inp["X"], inp["W1"], inp["W3"], inp["W2"])
    refb = O.swiglu_shard_bwd(inp["X"], inp["W1"], inp["W3"], inp["W2"], inp["dY"])
    for k in ("G", "U", "H", "Z"):
        check(k, out[k], ref[k], dtype)
    for k in ("dX", "dW1", "dW3", "dW2"):
        check(k, out[k], refb[k], dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swiglu_slices_of_unequal_scale(tp, dtype):
    """W3's columns and W2's rows scaled over three decades along d_ff: U, H,
    dW3 (and dW1, through dG = dH U Swish'(G), over six) have columns, dW2
    rows, of very different size; each slice is compared with the oracle
    against its own largest value."""
    M, d, f = 512, 256, 384
    _say(f"swiglu slices of unequal scale {dtype} M={M} d={d} f={f}")
    inp = tpsynth.random_swiglu(M, d, f, dtype, seed=23, w_std=0.05)
    sc = np.logspace(-3.0, 0.0, f)
    rnd = tpsynth.round_to_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    inp["W3"] = rnd((inp["W3"] * sc[None, :]).astype(np.float32))
    inp["W2"] = rnd((inp["W2"] * sc[:, None]).astype(np.float32))
    out = run_swiglu(tp, inp, dtype)
    ref = O.swiglu_shard_fwd(inp["X"], inp["W1"], inp["W3"], inp["W2"])
    refb = O.swiglu_shard_bwd(inp["X"], inp["W1"], inp["W3"], inp["W2"], inp["dY"])
    for k, r, axis in (("U", ref["U"], 0), ("H", ref["H"], 0), ("dW1", refb["dW1"], 0), ("dW3", refb["dW3"], 0),
                       ("dW2", refb["dW2"], 1)):
        err = _slice_rel_err(out[k], r, axis)
        assert err <= TOL[dtype], f"{k}: worst slice max_rel_err {err:.3e} > {TOL[dtype]}"
    for k in ("G", "Z"):
        check(k, out[k], ref[k], dtype)
    check("dX", out["dX"], refb["dX"], dtype)


def test_swiglu_c3_full_size_sampled(tp):
    """At C3 size dW2 and the SwiGLU' dgrad run as one launch (176 and 352
    tiles of 256 x 256, the dgrad's last column tile ragged): the launch list
    must show it, and both products' outputs are checked."""
    _say("swiglu C3 bf16 full size, sampled rows/cols")
    wl = tpsynth.WORKLOADS["C3"]
    inp = tpsynth.swiglu_inputs(wl)
    out, labels = _launch_labels(tp, lambda: run_swiglu(tp, inp, "bf16"))
    assert "swiglu_bwd.htdy_dswiglu_pair" in labels, labels
    X, W1, W3, W2, dY = (inp[k] for k in ("X", "W1", "W3", "W2", "dY"))
    rows = _sample(wl.M, 48, 21)
    cols = np.unique(np.concatenate([_sample(wl.f_local, 14, 22), [2687, 2688, 2751]]))  # ragged last tile
    ref = O.swiglu_shard_fwd(X[rows], W1, W3, W2)
    for k in ("G", "U", "H", "Z"):
        check(k, host(out[k])[rows], ref[k], "bf16")
    check("dX", host(out["dX"])[rows], O.swiglu_shard_bwd(X[rows], W1, W3, W2, dY[rows])["dX"], "bf16")
    sub = O.swiglu_shard_bwd(X, W1[:, cols], W3[:, cols], W2[cols], dY)
    check("dW1", host(out["dW1"])[:, cols], sub["dW1"], "bf16")
    check("dW3", host(out["dW3"])[:, cols], sub["dW3"], "bf16")
    check("dW2", host(out["dW2"])[cols], sub["dW2"], "bf16")


# --------------------------------------------------------------- attention

def run_attn(tp, inp, b, s, h_l, dh, causal=True, dY=None):
    X, Wq, Wk, Wv, Wo = (dev(inp[k], "bf16") for k in ("X", "Wq", "Wk", "Wv", "Wo"))
    d = X.shape[1]
    Q, K, V = (empty((b, h_l, s, dh), "bf16") for _ in range(3))
    Ob, Z = empty((b * s, h_l * dh), "bf16"), empty((b * s, d), "bf16")
    L = empty((b, h_l, s), "f32")
    tp.tp_attn_shard_fwd(X, Wq, Wk, Wv, Wo, Q, K, V, Ob, Z, b, s, h_l, dh, causal=causal, L=L)
    out = dict(Q=Q, K=K, V=V, O=Ob, Z=Z, L=L)
    if dY is not None:
        dYd = dev(dY, "bf16")
        dX = empty((b * s, d), "bf16")
        dWq, dWk, dWv = (empty((d, h_l * dh), "f32") for _ in range(3))
        dWo = empty((h_l * dh, d), "f32")
        ws = torch.empty(tp.tp_attn_shard_bwd_workspace_bytes(tp.TP_DT_BF16, b, s, d, h_l, dh),
                         dtype=torch.uint8, device="cuda")
        tp.tp_attn_shard_bwd(X, Wq, Wk, Wv, Wo, Q, K, V, Ob, L, dYd, dX, dWq, dWk, dWv, dWo, ws,
                             b, s, h_l, dh, causal=causal)
        out.update(dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dWo=dWo)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("b,s,d,h_l,dh,causal", [
    (2, 200, 64, 2, 128, True),      # ragged sequence (not a multiple of the 128-query tile)
    (1, 64, 136, 3, 64, True),
    (2, 130, 64, 1, 128, False),
    (1, 1, 32, 2, 128, True),        # one token: o = v
    (3, 257, 96, 2, 64, True),
    (1, 900, 64, 1, 128, False),     # 15 key tiles (an odd count), non-causal
    (1, 1000, 64, 2, 128, True),     # 8 query tiles with 2 to 16 key tiles each
    (1, 3000, 64, 2, 128, True),     # long and ragged: up to 47 key tiles, the last one partial
])
def test_attention_small_shapes(tp, b, s, d, h_l, dh, causal):
    _say(f"attention b={b} s={s} d={d} h_l={h_l} dh={dh} causal={causal}")
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "bf16", seed=b * s + dh, w_std=0.1)
    out = run_attn(tp, inp, b, s, h_l, dh, causal)
    ref = O.attn_shard_fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, h_l, dh, causal)
    for k in ("Q", "K", "V", "O", "Z"):
        check(k, out[k], ref[k], "bf16")
    # L is fp32 from bf16 Q, K: an absolute error relative to the score scale
    assert np.abs(host(out["L"]) - ref["L"]).max() < 2e-2 * max(1.0, np.abs(ref["L"]).max())


@pytest.mark.parametrize("b,s,d,h_l,causal", [
    (2, 200, 64, 2, True),           # ragged sequence
    (2, 130, 72, 1, False),
    (1, 1, 32, 2, True),             # one token: only V gets gradient
    (1, 257, 96, 2, True),           # ragged key tile and query chunk
    (1, 384, 64, 1, True),           # several key tiles, query chunks and dQ tiles
])
def test_attention_bwd_small_shapes(tp, b, s, d, h_l, causal):
    dh = 128
    _say(f"attention bwd b={b} s={s} d={d} h_l={h_l} causal={causal}")
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "bf16", seed=7 * s + d, w_std=0.1)
    dY = tpsynth.round_to_bf16(np.random.default_rng(s + 1).standard_normal((b * s, d)).astype(np.float32))
    out = run_attn(tp, inp, b, s, h_l, dh, causal, dY=dY)
    ref = O.attn_shard_bwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dY, b, s, h_l, dh, causal)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        check(k, out[k], ref[k], "bf16")


def test_attention_bwd_deterministic(tp):
    _say("attention bwd bitwise deterministic")
    b, s, d, h_l, dh = 1, 256, 64, 2, 128
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "bf16", seed=3, w_std=0.1)
    dY = tpsynth.round_to_bf16(np.random.default_rng(4).standard_normal((b * s, d)).astype(np.float32))
    a = run_attn(tp, inp, b, s, h_l, dh, True, dY=dY)
    c = run_attn(tp, inp, b, s, h_l, dh, True, dY=dY)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        assert torch.equal(a[k], c[k]), k


def test_attention_shards_sum_to_unsharded(tp):
    _say("attention 4 shards summed == unsharded")
    n, b, s, d, h_l, dh = 4, 1, 96, 64, 1, 64
    inp = tpsynth.random_attn(b, s, d, h_l, dh, "bf16", seed=5, w_std=0.1, n_shards=n)
    X = inp["X"]
    Zp = empty((n, b * s, d), "bf16")
    for i in range(n):
        sh = {"X": X, "Wq": inp["Wqs"][i], "Wk": inp["Wks"][i], "Wv": inp["Wvs"][i], "Wo": inp["Wos"][i]}
        Zp[i].copy_(run_attn(tp, sh, b, s, h_l, dh)["Z"])
    Z = empty((b * s, d), "bf16")
    tp.tp_shard_reduce(Zp, Z, n, b * s * d)
    torch.cuda.synchronize()
    full = O.attn_unsharded(X, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, n * h_l, dh)
    check("Z", Z, full["Z"], "bf16")


def test_attention_c4_full_size_sampled(tp):
    _say("attention C4 bf16 full size, sampled heads and queries")
    wl = tpsynth.WORKLOADS["C4"]
    inp = tpsynth.attn_inputs(wl)
    b, s, h_l, dh = wl.b, wl.s, wl.h_local, wl.d_head
    out = run_attn(tp, inp, b, s, h_l, dh)
    bi = b - 1                                  # one batch row, all heads, all positions
    Xb = inp["X"][bi * s:(bi + 1) * s]
    ref = O.attn_shard_fwd(Xb, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], 1, s, h_l, dh)
    for k in ("Q", "K", "V"):
        check(k, host(out[k])[bi], ref[k][0], "bf16")
    check("O", host(out["O"])[bi * s:(bi + 1) * s], ref["O"], "bf16")
    check("Z", host(out["Z"])[bi * s:(bi + 1) * s], ref["Z"], "bf16")
    rows = _sample(s, 32, 31)                  # batch 0: sampled query rows
    ref0 = O.attn_shard_fwd(inp["X"][:s], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], 1, s, h_l, dh)
    check("O[b0]", host(out["O"])[rows], ref0["O"][rows], "bf16")


def test_attention_bwd_c4_full_size_sampled(tp):
    # C4 shapes: dX for one batch row over all heads; dW for one head over
    # all batch rows (head j's weight gradients depend on head j alone).
    _say("attention bwd C4 bf16 full size: dX of one batch row, dW of one head")
    wl = tpsynth.WORKLOADS["C4"]
    inp = tpsynth.attn_inputs(wl)
    b, s, h_l, dh = wl.b, wl.s, wl.h_local, wl.d_head
    dY = tpsynth.round_to_bf16(np.random.default_rng(44).standard_normal((b * s, wl.d)).astype(np.float32))
    # dX and [dW_Q | dW_K | dW_V] run as one launch at this size
    out, labels = _launch_labels(tp, lambda: run_attn(tp, inp, b, s, h_l, dh, True, dY=dY))
    assert "attn_bwd.wgrad_dx_pair" in labels, labels
    bi = 1
    rows = slice(bi * s, (bi + 1) * s)
    ref = O.attn_shard_bwd(inp["X"][rows], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dY[rows], 1, s, h_l, dh)
    check("dX", host(out["dX"])[rows], ref["dX"], "bf16")
    j = 5
    cols = slice(j * dh, (j + 1) * dh)
    refh = O.attn_shard_bwd(inp["X"], inp["Wq"][:, cols], inp["Wk"][:, cols], inp["Wv"][:, cols],
                            inp["Wo"][cols], dY, b, s, 1, dh)
    for k in ("dWq", "dWk", "dWv"):
        check(k, host(out[k])[:, cols], refh[k], "bf16")
    check("dWo", host(out["dWo"])[cols], refh["dWo"], "bf16")


# ------------------------------------------------------- grouped-query attention

def _growing_rows(X, b, s, rate):
    """X with token t's row scaled by 1 + t / rate (then rounded to bf16):
    queries and keys grow along the sequence, so a row's running max of the
    scaled scores keeps rising from one key tile to the next."""
    f = 1.0 + np.arange(s, dtype=np.float64) / rate
    return tpsynth.round_to_bf16((X.reshape(b, s, -1) * f[None, :, None]).reshape(b * s, -1).astype(np.float32))


def _max_rise_after_first_tile(Q, K, dh):
    """Over every (batch, head, query), the largest rise of the running max of
    the scaled scores in log2 units (the forward's units) after the query's
    first 64-key tile (causal)."""
    sl2 = dh ** -0.5 * math.log2(math.e)
    worst = 0.0
    for bi in range(Q.shape[0]):
        for j in range(Q.shape[1]):
            S = (Q[bi, j] @ K[bi, j].T) * sl2
            S[np.triu_indices(S.shape[0], 1)] = -np.inf
            first = S[:, :64].max(axis=1)
            worst = max(worst, float((S.max(axis=1) - first).max()))
    return worst


@pytest.mark.parametrize("h_l,h_kv", [(2, 2), (4, 2)])
def test_attention_growing_scores(tp, h_l, h_kv):
    """Scores that keep growing along the sequence: the forward subtracts a
    running max that may lag the true one by up to 2^8, and rescales O and
    the sum when a row's max moves past that, mid-stream.  One head per
    workgroup (MHA) and two query heads of a group per workgroup."""
    b, s, d, dh = 1, 512, 64, 128
    _say(f"attention growing scores h_l={h_l} h_kv={h_kv}")
    inp = tpsynth.random_gqa(b, s, d, h_l, h_kv, dh, "bf16", seed=91 + h_l, w_std=0.1)
    # grow by 1 + t/384: a row's max rises up to 14-16 log2 units past its
    # first tile, while the scores stay well enough conditioned for bf16 Q and
    # K (a steeper ramp makes the softmax so peaked that bf16 rounding alone
    # moves O past the tolerance)
    inp["X"] = _growing_rows(inp["X"], b, s, 384.0)
    ref = O.attn_gqa_shard_fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, h_l, h_kv, dh, True)
    group = h_l // h_kv
    Kq = np.repeat(ref["K"], group, axis=1)
    assert _max_rise_after_first_tile(ref["Q"], Kq, dh) > 8.0   # past the lag: rescales happen mid-stream
    if h_kv == h_l:
        out = run_attn(tp, inp, b, s, h_l, dh, True)
    else:
        out = run_gqa(tp, inp, b, s, h_l, h_kv, dh, True)
    for k in ("O", "Z"):
        check(k, out[k], ref[k], "bf16")
    assert np.abs(host(out["L"]) - ref["L"]).max() < 2e-2 * max(1.0, np.abs(ref["L"]).max())


def test_attention_sequence_limit(tp):
    """s at the ABI's sequence limit (2^22 tokens, one head of 128: 1 GiB per
    head of K or V, the most the core's 32-bit key/value offsets address),
    causal; sampled queries across the sequence, O and Z, and L finite."""
    b, s, d, h_l, dh = 1, 1 << 22, 64, 1, 128
    _say(f"attention sequence limit s={s}")
    inp = tpsynth.random_gqa(b, s, d, h_l, h_l, dh, "bf16", seed=100, w_std=0.1)
    out = run_attn(tp, inp, b, s, h_l, dh)
    assert torch.isfinite(out["L"]).all()
    rows = np.unique(np.concatenate([_sample(s, 6, 101), [1 << 21, (1 << 22) - 2]]))
    ref = O.attn_gqa_query_rows(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], rows, h_l, h_l, dh)
    check("O", host(out["O"][torch.from_numpy(rows).cuda()]), ref["O"], "bf16")
    check("Z", host(out["Z"][torch.from_numpy(rows).cuda()]), ref["Z"], "bf16")


def run_gqa(tp, inp, b, s, h_l, h_kv, dh, causal=True):
    X, Wq, Wk, Wv, Wo = (dev(inp[k], "bf16") for k in ("X", "Wq", "Wk", "Wv", "Wo"))
    d = X.shape[1]
    Q = empty((b, h_l, s, dh), "bf16")
    K, V = (empty((b, h_kv, s, dh), "bf16") for _ in range(2))
    Ob, Z = empty((b * s, h_l * dh), "bf16"), empty((b * s, d), "bf16")
    L = empty((b, h_l, s), "f32")
    tp.tp_attn_gqa_shard_fwd(X, Wq, Wk, Wv, Wo, Q, K, V, Ob, Z, b, s, h_l, h_kv, dh, causal=causal, L=L)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, V=V, O=Ob, Z=Z, L=L)


@pytest.mark.parametrize("b,s,d,h_l,h_kv,dh,causal", [
    (2, 200, 64, 4, 2, 128, True),
    (1, 257, 96, 4, 1, 128, True),
    (2, 130, 64, 6, 3, 64, False),
    (1, 64, 72, 16, 1, 128, True),    # the G1 grouping, 16 query heads on one K/V head
    (1, 300, 64, 3, 1, 128, True),    # an odd group: one query head per workgroup
    (1, 200, 64, 4, 2, 128, False),   # two query heads per workgroup, non-causal (every wave on every tile)
    (1, 3000, 64, 4, 2, 128, True),   # two query heads per workgroup, long and ragged
    (1, 256, 2048, 4, 1, 128, True),  # long d: the K/V projection splits K (2 ways) through Z's memory
    (2, 128, 4096, 4, 2, 128, True),  # 4-way split, two K/V heads scattered
])
def test_gqa_small_shapes(tp, b, s, d, h_l, h_kv, dh, causal):
    _say(f"gqa b={b} s={s} d={d} h_l={h_l} h_kv={h_kv} dh={dh} causal={causal}")
    # weights ~ N(0, min(0.1, 1/sqrt(d))^2): scores of order one at every width
    inp = tpsynth.random_gqa(b, s, d, h_l, h_kv, dh, "bf16", seed=s + h_l, w_std=min(0.1, d ** -0.5))
    out = run_gqa(tp, inp, b, s, h_l, h_kv, dh, causal)
    ref = O.attn_gqa_shard_fwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], b, s, h_l, h_kv, dh, causal)
    for k in ("Q", "K", "V", "O", "Z"):
        check(k, out[k], ref[k], "bf16")


def test_gqa_g1_full_size_sampled(tp):
    # G1 (d 16384, 16 query heads on 1 K/V head, b 2, s 4096): sampled query
    # rows of each batch row, every head, against the definition at those rows.
    _say("gqa G1 bf16 full size, sampled queries")
    wl = tpsynth.WORKLOADS["G1"]
    inp = tpsynth.gqa_inputs(wl)
    b, s, h_l, h_kv, dh = wl.b, wl.s, wl.h_local, wl.h_kv_local, wl.d_head
    out = run_gqa(tp, inp, b, s, h_l, h_kv, dh)
    for bi in range(b):
        rows = np.unique(np.concatenate([_sample(s, 12, 70 + bi), [0, s - 1]]))
        Xb = inp["X"][bi * s:(bi + 1) * s]
        ref = O.attn_gqa_query_rows(Xb, inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], rows, h_l, h_kv, dh)
        check(f"O[b{bi}]", host(out["O"])[bi * s + rows], ref["O"], "bf16")
        check(f"Z[b{bi}]", host(out["Z"])[bi * s + rows], ref["Z"], "bf16")


def run_gqa_bwd(tp, inp, fwd, dY, b, s, h_l, h_kv, dh, causal=True):
    X, Wq, Wk, Wv, Wo = (dev(inp[k], "bf16") for k in ("X", "Wq", "Wk", "Wv", "Wo"))
    d = X.shape[1]
    N, Nkv = h_l * dh, h_kv * dh
    dX = empty((b * s, d), "bf16")
    dWq, dWo = empty((d, N), "f32"), empty((N, d), "f32")
    dWk, dWv = empty((d, Nkv), "f32"), empty((d, Nkv), "f32")
    ws = torch.empty(tp.tp_attn_gqa_shard_bwd_workspace_bytes(tp.TP_DT_BF16, b, s, d, h_l, h_kv, dh),
                     dtype=torch.uint8, device="cuda")
    tp.tp_attn_gqa_shard_bwd(X, Wq, Wk, Wv, Wo, fwd["Q"], fwd["K"], fwd["V"], fwd["O"], fwd["L"], dY, dX, dWq,
                             dWk, dWv, dWo, ws, b, s, h_l, h_kv, dh, causal=causal)
    torch.cuda.synchronize()
    return dict(dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dWo=dWo)


@pytest.mark.parametrize("b,s,d,h_l,h_kv,causal", [
    (2, 200, 64, 4, 2, True),
    (1, 257, 96, 4, 1, True),
    (2, 130, 64, 6, 3, False),
    (1, 64, 72, 16, 1, True),     # the G1 grouping
    (1, 96, 64, 3, 3, True),      # one query head per K/V head: the multi-head backward
])
def test_gqa_bwd_small_shapes(tp, b, s, d, h_l, h_kv, causal):
    _say(f"gqa bwd b={b} s={s} d={d} h_l={h_l} h_kv={h_kv} causal={causal}")
    dh = 128
    inp = tpsynth.random_gqa(b, s, d, h_l, h_kv, dh, "bf16", seed=s + 7 * h_l, w_std=0.1)
    dYn = tpsynth.normal(np.random.default_rng(s + 1), (b * s, d), 1.0, "bf16")
    fwd = run_gqa(tp, inp, b, s, h_l, h_kv, dh, causal)
    out = run_gqa_bwd(tp, inp, fwd, dev(dYn, "bf16"), b, s, h_l, h_kv, dh, causal)
    ref = O.attn_gqa_shard_bwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dYn, b, s, h_l, h_kv, dh,
                               causal)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        check(k, out[k], ref[k], "bf16")


def test_gqa_bwd_g1_grouping_long_sequence(tp):
    """The G1 grouping (16 query heads on one K/V head, d_head 128) at s 1024
    and d 2048, every output against the oracle."""
    _say("gqa bwd 16:1 grouping, s 1024, d 2048")
    b, s, d, h_l, h_kv, dh = 1, 1024, 2048, 16, 1, 128
    inp = tpsynth.random_gqa(b, s, d, h_l, h_kv, dh, "bf16", seed=93, w_std=0.01)
    dYn = tpsynth.normal(np.random.default_rng(94), (b * s, d), 1.0, "bf16")
    fwd = run_gqa(tp, inp, b, s, h_l, h_kv, dh)
    out = run_gqa_bwd(tp, inp, fwd, dev(dYn, "bf16"), b, s, h_l, h_kv, dh)
    ref = O.attn_gqa_shard_bwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dYn, b, s, h_l, h_kv, dh)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        check(k, out[k], ref[k], "bf16")


def test_gqa_bwd_g1_full_size(tp):
    """G1 at full size (b 2, s 4096, d 16384, 16 query heads on one K/V head)
    against the oracle, every gradient whole.  Its QKV weight gradient
    ([16384 x 2304], 576 tiles of 256 x 256) runs two whole rounds of tiles and
    splits the last 64 tiles (rows 14336..16383, columns 256..2303) along K,
    finished by the ordered fixup kernel: the launch list must contain that
    fixup, and the rows it writes are also checked on their own (normalised by
    their own largest value, so an error there cannot hide behind larger rows
    elsewhere).  Two runs agree bit for bit."""
    import bench
    _say("gqa bwd G1 full size against the oracle (tail-split weight gradient)")
    wl = tpsynth.WORKLOADS["G1"]
    inp = tpsynth.gqa_inputs(wl)
    b, s, h_l, h_kv, dh = wl.b, wl.s, wl.h_local, wl.h_kv_local, wl.d_head
    dYn = tpsynth.normal(np.random.default_rng(95), (b * s, wl.d), 1.0, "bf16")
    dY = dev(dYn, "bf16")
    fwd = run_gqa(tp, inp, b, s, h_l, h_kv, dh)
    L = tp.lib()
    ev = bench.HipEvents(64)
    assert L.tp_profile_begin(ev.start, ev.stop, ev.n) == 0
    a = run_gqa_bwd(tp, inp, fwd, dY, b, s, h_l, h_kv, dh)
    n = L.tp_profile_end()
    labels = [L.tp_profile_label(i).decode() for i in range(n)]
    ev.close()
    assert "gemm.tail_split" in labels and "gemm.tail_fixup" in labels, labels
    c = run_gqa_bwd(tp, inp, fwd, dY, b, s, h_l, h_kv, dh)
    for k in a:
        assert torch.equal(a[k], c[k]), k
    del c, fwd
    _say("gqa bwd G1 full size: oracle")
    ref = O.attn_gqa_shard_bwd(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], dYn, b, s, h_l, h_kv, dh)
    for k in ("dX", "dWq", "dWk", "dWv", "dWo"):
        check(k, a[k], ref[k], "bf16")
    r0, c0 = 56 * 256, 256          # the tail tiles: m-tiles 56..63, columns 256.. of [dWq | dWk | dWv]
    check("dWq tail", a["dWq"][r0:, c0:], ref["dWq"][r0:, c0:], "bf16")
    check("dWk tail", a["dWk"][r0:], ref["dWk"][r0:], "bf16")
    check("dWv tail", a["dWv"][r0:], ref["dWv"][r0:], "bf16")

