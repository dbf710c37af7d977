"""tp_mlp_bwd_noalloc against tp_mlp_bwd on the GPU: two calls in a row (the
second smaller, so the scratch holds the first call's contents), each
compared bit for bit with the caller-workspace entry point (same kernels and
plan) and with the fp64 oracle at the bf16 bar; the same for fp32; and a
shape whose workspace exceeds the scratch is refused before any launch."""
import numpy as np
import pytest

import oracle as O
import tpsynth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import megatron_tensor_transformer_fwd_amd as m
    m.lib()
    return m


def _case(tp, M, d, f, dtype, seed):
    print(f"[case] mlp_bwd_noalloc M={M} d={d} f={f} {dtype}", flush=True)
    inp = tpsynth.random_mlp(M, d, f, dtype, seed=seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdt).cuda()
    X, W1, W2, dY = (dev(inp[k]) for k in ("X", "W1", "W2", "dY"))
    A, H = (torch.empty((M, f), dtype=tdt, device="cuda") for _ in range(2))
    Z = torch.empty((M, d), dtype=tdt, device="cuda")
    tp.tp_mlp_fwd(X, W1, W2, A, H, Z)
    outs = []
    for noalloc in (False, True):
        dX = torch.full((M, d), float("nan"), dtype=tdt, device="cuda")
        dW1 = torch.full((d, f), float("nan"), device="cuda")
        dW2 = torch.full((f, d), float("nan"), device="cuda")
        if noalloc:
            tp.tp_mlp_bwd_noalloc(X, W1, W2, A, H, dY, dX, dW1, dW2)
        else:
            dt = tp.TP_DT_BF16 if dtype == "bf16" else tp.TP_DT_F32
            ws = torch.empty(tp.tp_mlp_bwd_workspace_bytes(dt, M, d, f), dtype=torch.uint8, device="cuda")
            tp.tp_mlp_bwd(X, W1, W2, A, H, dY, dX, dW1, dW2, ws)
        torch.cuda.synchronize()
        outs.append({"dX": dX, "dW1": dW1, "dW2": dW2})
    ref = O.mlp_shard_bwd(inp["X"], inp["W1"], inp["W2"], inp["dY"])
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for k in ("dX", "dW1", "dW2"):
        assert torch.equal(outs[0][k], outs[1][k]), k
        err = O.max_rel_err(outs[1][k].float().cpu().numpy(), ref[k])
        assert err <= tol, (k, err)


def test_noalloc_matches_workspace_entry_point(tp):
    # C2's shard shape: dA (8 MiB) and the split-K partials of both weight gradients
    _case(tp, 8192, 1024, 512, "bf16", seed=11)
    # then a smaller, ragged one: the scratch still holds the first call's values
    _case(tp, 1000, 256, 384, "bf16", seed=12)
    _case(tp, 96, 64, 128, "f32", seed=13)


def test_noalloc_refuses_oversized_workspace(tp):
    M, d, f = 8192, 8192, 8192       # dA alone is 128 MiB
    assert tp.tp_mlp_bwd_workspace_bytes(tp.TP_DT_BF16, M, d, f) > tp.MLP_BWD_NOALLOC_MAX_WORKSPACE
    bf = torch.bfloat16
    X, dY, dX = (torch.zeros((M, d), dtype=bf, device="cuda") for _ in range(3))
    W1, W2 = torch.zeros((d, f), dtype=bf, device="cuda"), torch.zeros((f, d), dtype=bf, device="cuda")
    A, H = (torch.zeros((M, f), dtype=bf, device="cuda") for _ in range(2))
    dW1, dW2 = torch.zeros((d, f), device="cuda"), torch.zeros((f, d), device="cuda")
    with pytest.raises(tp.TPError) as e:
        tp.tp_mlp_bwd_noalloc(X, W1, W2, A, H, dY, dX, dW1, dW2)
    assert e.value.status == -7 and "allocation-free" in e.value.detail
    torch.cuda.synchronize()
    assert float(dX.abs().max()) == 0.0 and float(dW1.abs().max()) == 0.0     # nothing ran
