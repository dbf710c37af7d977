"""The C ABI without a GPU: every entry point rejects bad arguments with the
documented status before any HIP call.  The addresses passed are fabricated,
so the module runs only on a machine that provably has no GPU (the few calls
whose arguments pass validation then fail at the launch); nothing here
touches a device."""
import ctypes
import os

import pytest

import megatron_tensor_transformer_fwd_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_DIM, E_DIVIS, E_DTYPE, E_ALIGN, E_ALIAS, E_WS, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _no_device_proven() -> bool:
    """True only where this process provably sees no GPU: no /dev/kfd and the
    HIP runtime reports no device.  Anything else (the device node exists, the
    runtime cannot be loaded, or it answers with another error) counts as a
    device that may be present."""
    if os.path.exists("/dev/kfd"):
        return False
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            continue
    else:
        return False
    n = ctypes.c_int(-1)
    rc = hip.hipGetDeviceCount(ctypes.byref(n))
    hip_error_no_device = 100
    return rc == hip_error_no_device or (rc == 0 and n.value == 0)


NO_DEVICE = _no_device_proven()

# Every call below passes fabricated device addresses: validation must refuse
# them on the host, and the few that pass validation fail at the launch for
# want of a device.  On a machine with a GPU such a call would reach a kernel,
# so the whole module runs only where no device is provably present.
pytestmark = [pytest.mark.skipif(not os.path.exists(tp.LIB_PATH), reason="libtpshard.so not built"),
              pytest.mark.skipif(not NO_DEVICE, reason="fabricated device addresses: CPU-only machines")]


def _fails_at_launch(call):
    """A call whose arguments pass validation, made on this module's
    fabricated addresses: with no device it fails at the launch with
    TP_E_HIP (the module runs only where no device is present)."""
    assert NO_DEVICE
    assert call() == E_HIP


BF16, F32 = tp.TP_DT_BF16, tp.TP_DT_F32


# Fake, well separated, 16-byte aligned device addresses: validation never
# dereferences them and every case below fails before any HIP call.
BASE = 1 << 40


def _addrs(n, gap=1 << 32):
    return [BASE + i * gap for i in range(n)]


def _mlp_fwd(**kw):
    X, W1, W2, A, H, Z = _addrs(6)
    args = dict(stream=None, dt=BF16, M=64, d=64, f=128, X=X, W1=W1, W2=W2, A=A, H=H, Z=Z)
    args.update(kw)
    rc = tp.lib().tp_mlp_fwd(*args.values())
    return rc, tp.lib().tp_last_error_detail().decode()


def test_mlp_fwd_validation():
    assert _mlp_fwd(X=None)[0] == E_NULL
    assert _mlp_fwd(H=None)[0] == E_NULL
    assert _mlp_fwd(M=0)[0] == E_DIM
    assert _mlp_fwd(d=-8)[0] == E_DIM
    assert _mlp_fwd(M=(1 << 30) + 1)[0] == E_DIM
    assert _mlp_fwd(d=60)[0] == E_DIVIS
    assert _mlp_fwd(f=130)[0] == E_DIVIS
    assert _mlp_fwd(dt=7)[0] == E_DTYPE
    assert _mlp_fwd(W1=BASE + (1 << 32) + 8)[0] == E_ALIGN
    rc, msg = _mlp_fwd(Z=BASE + 16)          # Z on top of X
    assert rc == E_ALIAS and "Z" in msg and "X" in msg
    assert _mlp_fwd(H=BASE + 7 * (1 << 32), Z=BASE + 7 * (1 << 32) + 64)[0] == E_ALIAS   # H and Z overlap


def _mlp_bwd(**kw):
    ptrs = _addrs(10)
    names = ["X", "W1", "W2", "A", "H", "dY", "dX", "dW1", "dW2", "ws"]
    args = dict(stream=None, dt=BF16, M=64, d=64, f=128)
    args.update(dict(zip(names, ptrs)))
    args["ws_bytes"] = 1 << 30
    args.update(kw)
    return tp.lib().tp_mlp_bwd(*args.values())


def test_mlp_bwd_validation_and_workspace():
    need = tp.tp_mlp_bwd_workspace_bytes(BF16, 64, 64, 128)
    assert need >= 64 * 128 * 2
    assert tp.tp_mlp_bwd_workspace_bytes(F32, 64, 64, 128) >= 64 * 128 * 4
    assert tp.tp_mlp_bwd_workspace_bytes(BF16, 0, 64, 128) == 0
    assert tp.tp_mlp_bwd_workspace_bytes(BF16, 64, 60, 128) == 0
    assert _mlp_bwd(ws_bytes=need - 1) == E_WS
    assert _mlp_bwd(ws=None) in (E_WS, E_NULL)
    assert _mlp_bwd(A=None) == E_NULL
    assert _mlp_bwd(dW1=BASE + 4) == E_ALIGN
    assert _mlp_bwd(dX=BASE + 5 * (1 << 32)) == E_ALIAS       # dX on top of dY
    assert _mlp_bwd(f=12) == E_DIVIS


def _mlp_bwd_noalloc(**kw):
    names = ["X", "W1", "W2", "A", "H", "dY", "dX", "dW1", "dW2"]
    args = dict(stream=None, dt=BF16, M=64, d=64, f=128)
    args.update(dict(zip(names, _addrs(9))))
    args.update(kw)
    rc = tp.lib().tp_mlp_bwd_noalloc(*args.values())
    return rc, tp.lib().tp_last_error_detail().decode()


def test_mlp_bwd_noalloc_validation_and_limit():
    """The allocation-free backward validates like tp_mlp_bwd and refuses
    shapes whose workspace exceeds its 64 MiB scratch before any HIP call."""
    limit = tp.MLP_BWD_NOALLOC_MAX_WORKSPACE
    assert limit == 64 << 20
    # the 8192-token shards of the large (f 4096) and GPT-2-medium (f 512) layers fit
    assert tp.tp_mlp_bwd_workspace_bytes(BF16, 8192, 8192, 4096) <= limit
    assert tp.tp_mlp_bwd_workspace_bytes(BF16, 8192, 1024, 512) <= limit
    for M, d, f in ((8192, 8192, 8192), (16384, 8192, 4096), (8192, 4096, 4104)):
        assert tp.tp_mlp_bwd_workspace_bytes(BF16, M, d, f) > limit
        rc, msg = _mlp_bwd_noalloc(M=M, d=d, f=f)
        assert rc == E_WS and "allocation-free" in msg, msg
    assert _mlp_bwd_noalloc(A=None)[0] == E_NULL
    assert _mlp_bwd_noalloc(dW2=BASE + 8)[0] == E_ALIGN
    assert _mlp_bwd_noalloc(dX=BASE + 5 * (1 << 32))[0] == E_ALIAS     # dX on top of dY
    assert _mlp_bwd_noalloc(f=12)[0] == E_DIVIS
    assert _mlp_bwd_noalloc(dt=7)[0] == E_DTYPE
    assert _mlp_bwd_noalloc(M=0)[0] == E_DIM
    # arguments that pass validation fail only at the scratch lookup or launch
    _fails_at_launch(lambda: _mlp_bwd_noalloc()[0])


def test_mlp_shards_validation():
    """The all-shards entry points: n_shards in [1, 64], the shard-stacked
    extents in the overlap checks, and the workspace."""
    L = tp.lib()
    X, W1s, W2s, A, H, Z, dY, dX, dW1s, dW2s, ws = _addrs(11)
    fwd = lambda **kw: L.tp_mlp_fwd_shards(*dict(dict(stream=None, dt=BF16, n=4, M=64, d=64, f=128, X=X, W1s=W1s,
                                                      W2s=W2s, A=A, H=H, Z=Z), **kw).values())
    assert fwd(n=0) == E_DIM and fwd(n=65) == E_DIM
    assert fwd(W2s=None) == E_NULL and fwd(f=12) == E_DIVIS and fwd(dt=3) == E_DTYPE
    # H holds 4 shards of [64 x 128] bf16 = 64 KiB: a Z starting inside it overlaps
    assert fwd(Z=H + 4 * 64 * 128 * 2 - 16) == E_ALIAS
    _fails_at_launch(lambda: fwd(Z=H + 4 * 64 * 128 * 2))
    need = L.tp_mlp_bwd_shards_workspace_bytes(BF16, 4, 64, 64, 128)
    assert need >= 4 * 64 * 128 * 2
    assert L.tp_mlp_bwd_shards_workspace_bytes(BF16, 0, 64, 64, 128) == 0
    # fp32: the shards run in one launch per product, so the workspace holds every shard's dA
    assert L.tp_mlp_bwd_shards_workspace_bytes(F32, 4, 64, 64, 128) == 4 * 64 * 128 * 4
    bwd = lambda **kw: L.tp_mlp_bwd_shards(*dict(dict(stream=None, dt=BF16, n=4, M=64, d=64, f=128, X=X, W1s=W1s,
                                                      W2s=W2s, A=A, H=H, dY=dY, dX=dX, dW1s=dW1s, dW2s=dW2s, ws=ws,
                                                      ws_bytes=need), **kw).values())
    assert bwd(ws_bytes=need - 1) == E_WS
    assert bwd(dW1s=BASE + 4) == E_ALIGN
    assert bwd(dX=dY + 16) == E_ALIAS
    assert bwd(n=100) == E_DIM
    _fails_at_launch(lambda: bwd())


def test_mlp_bwd_workspace_grows_with_split_k():
    # narrow weight-gradient outputs take a split-K workspace of fp32 partials
    small = tp.tp_mlp_bwd_workspace_bytes(BF16, 8192, 1024, 512)
    assert small >= 8192 * 512 * 2 + 2 * 1024 * 512 * 4


def test_swiglu_validation():
    L = tp.lib()
    p = _addrs(8)
    assert L.tp_swiglu_fwd(None, BF16, 64, 64, 128, *p[:4], p[4], None, p[6], p[7]) == E_NULL   # G without U
    assert L.tp_swiglu_fwd(None, BF16, 64, 64, 124, *p[:4], p[4], p[5], p[6], p[7]) == E_DIVIS
    assert L.tp_swiglu_fwd(None, 3, 64, 64, 128, *p[:4], p[4], p[5], p[6], p[7]) == E_DTYPE
    q = _addrs(17)
    need = tp.tp_swiglu_bwd_workspace_bytes(BF16, 64, 64, 128)
    assert need >= 64 * 256 * 2
    assert L.tp_swiglu_bwd(None, BF16, 64, 64, 128, *q[:12], q[16], need - 16) == E_WS
    assert L.tp_swiglu_bwd(None, BF16, 64, 64, 128, *q[:4], None, *q[5:12], q[16], need) == E_NULL


def _attn(**kw):
    p = _addrs(10)
    args = dict(stream=None, dt=BF16, b=2, s=64, d=64, h_local=2, d_head=128, causal=1, scale=0.0)
    args.update(dict(zip(["X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "Z"], p)))
    args["L"] = None
    args.update(kw)
    return tp.lib().tp_attn_shard_fwd(*args.values())


def _attn_bwd(**kw):
    p = _addrs(22)
    args = dict(stream=None, dt=BF16, b=2, s=64, d=64, h_local=2, d_head=128, causal=1, scale=0.0)
    names = ["X", "Wq", "Wk", "Wv", "Wo", "Q", "K", "V", "O", "L", "dY", "dX", "dWq", "dWk", "dWv", "dWo", "ws"]
    args.update(dict(zip(names, p)))
    args["ws_bytes"] = tp.tp_attn_shard_bwd_workspace_bytes(BF16, 2, 64, 64, 2, 128)
    args.update(kw)
    return tp.lib().tp_attn_shard_bwd(*args.values())


def test_attention_backward_validation():
    need = tp.tp_attn_shard_bwd_workspace_bytes(BF16, 2, 64, 64, 2, 128)
    # dO, [dQ|dK|dV], [Wq|Wk|Wv] and D at least
    assert need >= 128 * 256 * 2 + 128 * 768 * 2 + 64 * 768 * 2 + 2 * 2 * 64 * 4
    assert tp.tp_attn_shard_bwd_workspace_bytes(F32, 2, 64, 64, 2, 128) == 0
    assert _attn_bwd(d_head=64) == E_DIM                 # the backward kernels are written for 128
    assert _attn_bwd(dt=F32) == E_DTYPE
    assert _attn_bwd(L=None) == E_NULL
    assert _attn_bwd(ws_bytes=need - 8) == E_WS
    assert _attn_bwd(ws=None) == E_WS                    # a missing workspace is a workspace error


def test_attention_validation():
    assert _attn(dt=F32) == E_DTYPE
    assert _attn(d_head=96) == E_DIM
    assert _attn(s=0) == E_DIM
    assert _attn(causal=2) == E_DIM
    assert _attn(scale=float("nan")) == E_DIM
    assert _attn(d=60) == E_DIVIS
    assert _attn(O=None) == E_NULL
    assert _attn(Q=BASE + 8) == E_ALIGN
    assert _attn(Z=BASE) == E_ALIAS


def test_shard_reduce_validation():
    L = tp.lib()
    P, out, bias = _addrs(3)
    assert L.tp_shard_reduce(None, BF16, BF16, 0, 16, P, 16, None, 0, out) == E_DIM
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 0, P, 16, None, 0, out) == E_DIM
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 16, P, 8, None, 0, out) == E_DIM       # stride < numel
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 16, P, 16, bias, 0, out) == E_DIM      # bias_len
    assert L.tp_shard_reduce(None, 5, BF16, 4, 16, P, 16, None, 0, out) == E_DTYPE
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 16, None, 16, None, 0, out) == E_NULL
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 16, P + 2, 16, None, 0, out) == E_ALIGN
    assert L.tp_shard_reduce(None, BF16, BF16, 4, 16, P, 16, None, 0, P + 32) == E_ALIAS  # into block 1
    assert L.tp_shard_reduce(None, BF16, F32, 4, 16, P, 16, None, 0, P) == E_ALIAS       # in place, dtypes differ
    assert L.tp_shard_reduce(None, F32, F32, 4, 16, P, 8 + 8, None, 0, P + 16) == E_ALIAS
    # an exactly in-place reduce with out's extent inside block 0 passes validation:
    # only the launch (no device here) can then fail, with TP_E_HIP.
    assert L.tp_last_error_detail() != b""


def test_row_pitch_and_sequence_limits():
    """Sizes the kernels cannot address with 32-bit tile offsets are refused
    on the host: d, f, h_local*d_head above 2^21 and s above 2^22."""
    L = tp.lib()
    fake = ctypes.c_void_p(1 << 20)
    big = (1 << 21) + 8
    rc = L.tp_mlp_fwd(None, 1, 64, big, 64, fake, fake, fake, None, fake, fake)
    assert rc == -2 and b"2^21" in L.tp_last_error_detail()
    rc = L.tp_mlp_fwd(None, 1, 64, 64, big, fake, fake, fake, None, fake, fake)
    assert rc == -2
    assert L.tp_swiglu_bwd_workspace_bytes(1, 64, 64, big) == 0
    rc = L.tp_attn_shard_fwd(None, 1, 1, (1 << 22) + 1, 64, 1, 128, 1, 0.0,
                             fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, None)
    assert rc == -2 and b"2^22" in L.tp_last_error_detail()
    rc = L.tp_attn_shard_fwd(None, 1, 1, 128, 64, (1 << 21) // 128 + 1, 128, 1, 0.0,
                             fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, None)
    assert rc == -2
    # the limits themselves are accepted up to the pointer checks
    rc = L.tp_mlp_fwd(None, 1, 64, 1 << 21, 64, None, fake, fake, None, fake, fake)
    assert rc == -1


def test_gqa_validation():
    L = tp.lib()
    p = _addrs(11)
    # h_kv_local must divide h_local
    assert L.tp_attn_gqa_shard_fwd(None, BF16, 1, 64, 64, 6, 4, 128, 1, 0.0, *p[:10], None) == E_DIVIS
    assert L.tp_attn_gqa_shard_fwd(None, BF16, 1, 64, 64, 4, 0, 128, 1, 0.0, *p[:10], None) == E_DIVIS
    assert L.tp_attn_gqa_shard_fwd(None, BF16, 1, 64, 64, 4, 8, 128, 1, 0.0, *p[:10], None) == E_DIVIS
    assert L.tp_attn_gqa_shard_fwd(None, F32, 1, 64, 64, 4, 2, 128, 1, 0.0, *p[:10], None) == E_DTYPE
    assert L.tp_attn_gqa_shard_fwd(None, BF16, 1, 64, 64, 4, 2, 128, 1, 0.0, None, *p[1:10], None) == E_NULL


def test_sp_reduce_scatter_ln_validation():
    L = tp.lib()
    P, bias, res, keep, g, b, h, x = _addrs(8)

    def rs(dt=BF16, n=4, rows=64, cols=32, index=1, P=P, stride=None, bias=bias, res=res, keep=keep,
           p_drop=0.1, g=g, b=b, eps=1e-5, h=h, x=x):
        stride = rows * cols if stride is None else stride
        return L.tp_sp_reduce_scatter_ln(None, dt, n, rows, cols, index, P, stride, bias, res, keep, p_drop,
                                         g, b, eps, h, x)

    assert rs(dt=7) == E_DTYPE
    assert rs(n=0) == E_DIM
    assert rs(rows=0) == E_DIM
    assert rs(index=4) == E_DIM and rs(index=-1) == E_DIM
    assert rs(rows=66) == E_DIVIS                         # rows % n_shards
    assert rs(cols=36) == E_DIVIS                         # cols % 8
    assert rs(stride=64 * 32 - 8) == E_DIM                # stride < rows*cols
    assert rs(stride=64 * 32 + 4) == E_DIVIS
    assert rs(p_drop=1.0) == E_DIM and rs(p_drop=-0.1) == E_DIM
    assert rs(eps=0.0) == E_DIM and rs(eps=float("nan")) == E_DIM
    assert rs(rows=((1 << 24) + 1) * 4) == E_DIM          # stripe rows beyond 2^24
    for kw in ("P", "res", "g", "b", "h", "x"):
        assert rs(**{kw: None}) == E_NULL, kw
    assert rs(keep=keep + 8) == E_ALIGN
    assert rs(h=res) == E_ALIAS                           # output over the residual
    assert rs(x=h) == E_ALIAS                             # outputs overlap
    assert rs(h=P + 2 * 64 * 32 * 2) == E_ALIAS           # output inside the partials
    # bias and keep are optional; with keep NULL p_drop is not examined.  Such
    # calls pass validation and fail only at the launch (no device here).
    _fails_at_launch(lambda: rs(bias=None, keep=None, p_drop=5.0))


def test_sp_all_gather_validation():
    L = tp.lib()
    s0, s1, s2, s3, full = _addrs(5)
    arr = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    st = arr(s0, s1, s2, s3)
    assert L.tp_sp_all_gather(None, 9, 4, 16, 32, st, full) == E_DTYPE
    assert L.tp_sp_all_gather(None, BF16, 0, 16, 32, st, full) == E_DIM
    assert L.tp_sp_all_gather(None, BF16, 65, 16, 32, arr(*([s0] * 65)), full) == E_DIM
    assert L.tp_sp_all_gather(None, BF16, 4, 0, 32, st, full) == E_DIM
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 36, st, full) == E_DIVIS
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, None, full) == E_NULL
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, st, None) == E_NULL
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, arr(s0, None, s2, s3), full) == E_NULL
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, arr(s0, s1 + 4, s2, s3), full) == E_ALIGN
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, st, full + 2) == E_ALIGN
    stripe = 16 * 32 * 2
    # a stripe that straddles its place in `full` is an overlap ...
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, arr(s0, full + stripe + 16, s2, s3), full) == E_ALIAS
    # ... another stripe's place as well
    assert L.tp_sp_all_gather(None, BF16, 4, 16, 32, arr(s0, full, s2, s3), full) == E_ALIAS
    # exactly in place is accepted (it is not copied); the launch then fails without a device
    _fails_at_launch(lambda: L.tp_sp_all_gather(None, BF16, 4, 16, 32, arr(s0, full + stripe, s2, s3), full))


def test_vocab_validation():
    L = tp.lib()
    ids, E, Y, X, tg, lg, st, loss, lse, dl, dX, dE, ws = _addrs(13)
    # input embedding
    assert L.tp_vocab_embed_fwd(None, 3, 16, 64, 128, 0, ids, E, Y) == E_DTYPE
    assert L.tp_vocab_embed_fwd(None, BF16, 0, 64, 128, 0, ids, E, Y) == E_DIM
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 60, 128, 0, ids, E, Y) == E_DIVIS
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 100, 0, ids, E, Y) == E_DIVIS
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, -1, ids, E, Y) == E_DIM
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, 0, None, E, Y) == E_NULL
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, 0, ids + 4, E, Y) == E_ALIGN
    _fails_at_launch(lambda: L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, 0, ids + 8, E, Y))   # 8 bytes suffice
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, 0, ids, E + 8, Y) == E_ALIGN
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, 128, 0, ids, E, E + 64) == E_ALIAS
    assert L.tp_vocab_embed_fwd(None, BF16, 16, 64, (1 << 21) + 8, 0, ids, E, Y) == E_DIM
    assert L.tp_vocab_embed_fwd(None, BF16, (1 << 24) + 1, 64, 128, 0, ids, E, Y) == E_DIM
    # input embedding backward
    _fails_at_launch(lambda: L.tp_vocab_embed_bwd(None, BF16, 16, 64, 128, 0, ids, Y, E))
    assert L.tp_vocab_embed_bwd(None, BF16, 16, 64, 100, 0, ids, Y, E) == E_DIVIS
    assert L.tp_vocab_embed_bwd(None, BF16, 16, 64, 128, 0, None, Y, E) == E_NULL
    assert L.tp_vocab_embed_bwd(None, BF16, 16, 64, 128, 0, ids, Y, Y + 64) == E_ALIAS
    assert L.tp_vocab_embed_bwd(None, BF16, 16, 64, 128, 0, ids + 4, Y, E) == E_ALIGN
    # fused output embedding + cross-entropy
    fws = L.tp_vocab_ce_fwd_workspace_bytes(BF16, 16, 64, 128)
    assert fws >= 16 * 8 and L.tp_vocab_ce_fwd_workspace_bytes(F32, 16, 64, 128) == 0
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, tg, lg, None, ws, fws) == E_NULL
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, None, lg, st, ws, fws) == E_NULL
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, tg, lg, lg + 16, ws, fws) == E_ALIAS
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, tg, X, st, ws, fws) == E_ALIAS
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, tg, lg, st, None, 0) == E_WS
    assert L.tp_vocab_ce_fwd(None, BF16, 16, 64, 128, 0, X, E, tg, lg, st, ws, fws - 1) == E_WS
    _fails_at_launch(lambda: L.tp_vocab_ce_fwd(None, F32, 16, 64, 128, 0, X, E, tg, lg, st, None, 0))   # fp32: no workspace
    assert L.tp_vocab_ce_combine(None, 0, 16, st, 48, loss, lse) == E_DIM
    assert L.tp_vocab_ce_combine(None, 4, 16, st, 40, loss, lse) == E_DIM       # stride < 3 * n_tokens
    assert L.tp_vocab_ce_combine(None, 4, 16, st, 48, loss, loss) == E_ALIAS
    assert L.tp_vocab_ce_combine(None, 4, 16, st + 2, 48, loss, lse) == E_ALIGN
    _fails_at_launch(lambda: L.tp_vocab_ce_combine(None, 4, 16, st + 4, 49, loss + 12, lse + 4))
    assert L.tp_vocab_ce_combine(None, 4, 16, st, 48, st + 64, lse) == E_ALIAS
    need = L.tp_vocab_ce_bwd_workspace_bytes(BF16, 16, 64, 128)
    assert need >= 16 * 128 * 2
    assert L.tp_vocab_ce_bwd_workspace_bytes(BF16, 16, 64, 100) == 0
    args = [X, E, tg, lg, lse, dl, dX, dE]
    assert L.tp_vocab_ce_bwd(None, BF16, 16, 64, 128, 0, *args, None, 0) == E_WS
    assert L.tp_vocab_ce_bwd(None, BF16, 16, 64, 128, 0, *args, ws, need - 1) == E_WS
    assert L.tp_vocab_ce_bwd(None, BF16, 16, 64, 128, 0, *args[:6], X, dE, ws, need) == E_ALIAS
    assert L.tp_vocab_ce_bwd(None, BF16, 16, 64, 128, 0, *args[:7], None, ws, need) == E_NULL


def test_gqa_backward_validation():
    L = tp.lib()
    p = _addrs(17)
    ws = p[16]
    need = L.tp_attn_gqa_shard_bwd_workspace_bytes(BF16, 1, 64, 64, 4, 2, 128)
    assert need > 0
    assert L.tp_attn_gqa_shard_bwd_workspace_bytes(BF16, 1, 64, 64, 4, 3, 128) == 0
    args = p[:16]
    assert L.tp_attn_gqa_shard_bwd(None, BF16, 1, 64, 64, 4, 3, 128, 1, 0.0, *args, ws, need) == E_DIVIS
    assert L.tp_attn_gqa_shard_bwd(None, BF16, 1, 64, 64, 4, 2, 64, 1, 0.0, *args, ws, need) == E_DIM
    assert L.tp_attn_gqa_shard_bwd(None, F32, 1, 64, 64, 4, 2, 128, 1, 0.0, *args, ws, need) == E_DTYPE
    assert L.tp_attn_gqa_shard_bwd(None, BF16, 1, 64, 64, 4, 2, 128, 1, 0.0, *args, None, 0) == E_WS
    assert L.tp_attn_gqa_shard_bwd(None, BF16, 1, 64, 64, 4, 2, 128, 1, 0.0, *args, ws, need - 1) == E_WS
    assert L.tp_attn_gqa_shard_bwd(None, BF16, 1, 64, 64, 4, 2, 128, 1, 0.0, None, *args[1:], ws, need) == E_NULL
    # one group is the multi-head backward: same workspace
    assert (L.tp_attn_gqa_shard_bwd_workspace_bytes(BF16, 2, 96, 64, 4, 4, 128)
            == L.tp_attn_shard_bwd_workspace_bytes(BF16, 2, 96, 64, 4, 128))


def test_sp_ln_bwd_validation():
    L = tp.lib()
    P, h, g, keep, dres, dh, dy, dg, db, dbi, ws = _addrs(11)
    need = L.tp_sp_ln_bwd_workspace_bytes(BF16, 4, 64, 32)
    assert need > 0
    assert L.tp_sp_ln_bwd_workspace_bytes(BF16, 4, 66, 32) == 0
    assert L.tp_sp_ln_bwd_workspace_bytes(BF16, 4, 64, 16392) == 0     # rows kept in registers: <= 16384

    def bw(dt=BF16, n=4, rows=64, cols=32, index=1, P=P, stride=None, h=h, g=g, eps=1e-5, keep=keep, p=0.1,
           dres=dres, dh=dh, dy=dy, dg=dg, db=db, dbi=dbi, ws=ws, wsb=None):
        stride = rows * cols if stride is None else stride
        return L.tp_sp_ln_bwd_reduce_scatter(None, dt, n, rows, cols, index, P, stride, h, g, eps, keep, p, dres,
                                             dh, dy, dg, db, dbi, ws, need if wsb is None else wsb)

    assert bw(dt=9) == E_DTYPE
    assert bw(rows=66) == E_DIVIS and bw(cols=36) == E_DIVIS
    assert bw(cols=16392) == E_DIM and bw(index=4) == E_DIM and bw(p=1.0) == E_DIM and bw(eps=0.0) == E_DIM
    assert bw(stride=64 * 32 - 8) == E_DIM
    for kw in ("P", "h", "g", "dh", "dy", "dg", "db"):
        assert bw(**{kw: None}) == E_NULL, kw
    assert bw(ws=None) == E_WS and bw(wsb=need - 1) == E_WS
    assert bw(dh=h) == E_ALIAS and bw(dy=dh) == E_ALIAS
    assert bw(dg=dg + 2) == E_ALIGN
    _fails_at_launch(lambda: bw(dg=dg + 4, dbi=None, dres=None, keep=None, p=3.0))      # 4-byte fp32 arrays; optional inputs
