"""GPU parity of the backward entry points against the CPU fp64 oracle, element
by element, at small and ragged sizes (several tiles, partial tiles in M, N
and K, K-split weight gradients with a ragged last slice), plus the edge
cases: M = 0, M = 1, k = 1, no bias, gradient accumulation, in-place dA,
guard bands around every output, run-to-run determinism of both variants.

Inputs are seeded draws (X, W, b, V, dZ and, for the per-step entry points,
G, Y and dA themselves); expected values come from the oracle only, and the
element-wise bounds (tests/_helpers.py) from the float32 / bf16 error model.
"""
import numpy as np
import pytest

from _helpers import (act_grad_bound, assert_within, backward_terms, f64, from_dev, gemm_bound,
                      grad_g_bound, rel_fro, say, to_dev, U32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_transformer_mlp_amd as tpm
    tpm.lib()
    return tpm


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def _draw(stream, shape, std, dtype, seed):
    from tensor_transformer_mlp_amd import inputs
    return inputs.draw(stream, shape, std, dtype, seed=seed)


def _guarded(torch, shape, dtype, fill, pad=64):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


def _guards_ok(torch, buf, pad, fill_nan=True):
    test = torch.isnan if fill_nan else torch.isinf
    return bool(torch.all(test(buf[:pad]))) and bool(torch.all(test(buf[-pad:])))


def _tdt(torch, dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


SAVE_CASES = [(1, 64, 128, "bf16"), (9, 200, 136, "bf16"), (257, 520, 392, "bf16"), (300, 64, 8, "bf16"),
              (512, 384, 512, "bf16"), (8, 64, 128, "f32"), (65, 200, 136, "f32")]


@pytest.mark.parametrize("M,H,Fk,dtype", SAVE_CASES)
def test_col_gelu_save_parity(tpm, orc, M, H, Fk, dtype):
    import torch
    say("col_gelu_save M=%d H=%d Fk=%d %s" % (M, H, Fk, dtype))
    k, i = 3, 2
    X = _draw(0, (M, H), 1.0, dtype, M + 1)
    W = _draw(1, (H, Fk * k), 0.05, dtype, H + 2)
    b = _draw(2, (Fk * k,), 0.05, dtype, Fk + 3)
    Wi = np.ascontiguousarray(W[:, i * Fk:(i + 1) * Fk])
    bi = np.ascontiguousarray(b[i * Fk:(i + 1) * Fk])
    tdt = _tdt(torch, dtype)
    pad = 64
    by, Y = _guarded(torch, (M, Fk), tdt, float("nan"), pad)
    bg, G = _guarded(torch, (M, Fk), tdt, float("nan"), pad)
    tpm.tp_mlp_col_gelu_save(to_dev(X), to_dev(Wi), to_dev(bi), Y_i=Y, G_i=G)
    Y2 = tpm.tp_mlp_col_gelu(to_dev(X), to_dev(Wi), to_dev(bi))
    torch.cuda.synchronize()
    assert _guards_ok(torch, by, pad) and _guards_ok(torch, bg, pad)
    assert torch.equal(Y, Y2), "training-mode Y differs from the inference column step"
    t = backward_terms(orc, X, Wi, bi, np.zeros((Fk, H)), np.zeros((M, H)), dtype)
    Yr = orc.col_gelu(X, W, b, k, i)
    Gr = orc.col_gelu_grad(X, W, b, k, i)
    assert_within(f64(from_dev(Y)), Yr, t["tolY"], "Y_i")
    S = np.abs(f64(X)) @ np.abs(f64(Wi)) + np.abs(f64(bi))[None, :]
    assert_within(f64(from_dev(G)), Gr, grad_g_bound(S, Gr, H, dtype), "G_i")
    assert rel_fro(f64(from_dev(G)), Gr) <= (1e-2 if dtype == "bf16" else 1e-5)


ACT_CASES = [(1, 128, 64, "bf16"), (9, 200, 136, "bf16"), (129, 72, 264, "bf16"), (257, 520, 392, "bf16"),
             (512, 256, 768, "bf16"), (300, 8, 64, "bf16"), (8, 64, 128, "f32"), (65, 136, 200, "f32")]


@pytest.mark.parametrize("M,H,Fk,dtype", ACT_CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_grad_act_parity(tpm, orc, M, H, Fk, dtype, inplace):
    import torch
    say("grad_act M=%d H=%d Fk=%d %s inplace=%s" % (M, H, Fk, dtype, inplace))
    k, i = 2, 1
    dZ = _draw(4, (M, H), 1.0, dtype, M + 5)
    V = _draw(3, (Fk * k, H), 0.05, dtype, H + 6)
    Gh = _draw(0, (M, Fk), 0.6, dtype, Fk + 7)
    Vi = np.ascontiguousarray(V[i * Fk:(i + 1) * Fk])
    tdt = _tdt(torch, dtype)
    pad = 64
    bg, G = _guarded(torch, (M, Fk), tdt, float("nan"), pad)
    G.copy_(to_dev(Gh))
    if inplace:
        dA, bd = G, bg
    else:
        bd, dA = _guarded(torch, (M, Fk), tdt, float("nan"), pad)
    tpm.tp_mlp_grad_act(to_dev(dZ), to_dev(Vi), G, dA_i=dA)
    torch.cuda.synchronize()
    assert _guards_ok(torch, bd, pad)
    if not inplace:
        assert torch.equal(G, to_dev(Gh)), "G_i was modified"
    dAr = orc.act_grad(dZ, V, Gh, k, i)
    dY = orc.act_grad(dZ, V, np.ones((M, Fk)), k, i)
    errdY = 2 * (H + 2) * U32 * (np.abs(f64(dZ)) @ np.abs(f64(Vi)).T)
    bound = act_grad_bound(dY, f64(Gh), errdY, 0.0, dtype)
    got = f64(from_dev(dA))
    assert_within(got, dAr, bound, "dA_i")
    assert rel_fro(got, dAr) <= (1e-2 if dtype == "bf16" else 1e-5)


# (M, Fk, H, dtype): M is the contraction length of the weight gradients; the
# large-M cases take the K-split path (with a ragged last slice for M % 32 != 0).
WGRAD_CASES = [(1, 128, 64, "bf16"), (9, 136, 200, "bf16"), (131, 264, 72, "bf16"), (257, 392, 520, "bf16"),
               (4100, 136, 200, "bf16"), (8192, 256, 256, "bf16"), (3000, 128, 128, "bf16"),
               (8, 128, 64, "f32"), (65, 136, 200, "f32"), (5000, 72, 64, "f32")]


@pytest.mark.parametrize("M,Fk,H,dtype", WGRAD_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_grad_row_weight_parity(tpm, orc, M, Fk, H, dtype, accumulate):
    import torch
    say("grad_row_weight M=%d Fk=%d H=%d %s acc=%s" % (M, Fk, H, dtype, accumulate))
    Y = _draw(0, (M, Fk), 0.5, dtype, M + 8)
    dZ = _draw(4, (M, H), 1.0, dtype, H + 9)
    pad = 64
    if accumulate:
        D0 = _draw(3, (Fk, H), 1.0, "f32", Fk + 10)
        buf, dV = _guarded(torch, (Fk, H), torch.float32, float("inf"), pad)
        dV.copy_(torch.from_numpy(D0))
    else:
        buf, dV = _guarded(torch, (Fk, H), torch.float32, float("nan"), pad)
    tpm.tp_mlp_grad_row_weight(to_dev(Y), to_dev(dZ), dV_i=dV, accumulate=accumulate)
    torch.cuda.synchronize()
    assert _guards_ok(torch, buf, pad, fill_nan=not accumulate)
    ref = orc.row_weight_grad(Y, dZ)
    bound = gemm_bound(f64(Y).T, f64(dZ), M)
    if accumulate:
        ref = ref + f64(D0)
        bound = bound + 2 * U32 * (np.abs(ref) + bound)
    got = f64(from_dev(dV))
    assert_within(got, ref, bound, "dV_i")
    assert rel_fro(got, ref) <= 1e-5


@pytest.mark.parametrize("M,Fk,H,dtype", WGRAD_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_grad_col_weight_parity(tpm, orc, M, Fk, H, dtype, accumulate):
    import torch
    say("grad_col_weight M=%d H=%d Fk=%d %s acc=%s" % (M, H, Fk, dtype, accumulate))
    X = _draw(0, (M, H), 1.0, dtype, M + 11)
    dA = _draw(4, (M, Fk), 0.1, dtype, Fk + 12)
    pad = 64
    fill = float("inf") if accumulate else float("nan")
    bw, dW = _guarded(torch, (H, Fk), torch.float32, fill, pad)
    bb, db = _guarded(torch, (Fk,), torch.float32, fill, pad)
    if accumulate:
        W0 = _draw(1, (H, Fk), 1.0, "f32", H + 13)
        b0 = _draw(2, (Fk,), 1.0, "f32", Fk + 14)
        dW.copy_(torch.from_numpy(W0))
        db.copy_(torch.from_numpy(b0))
    tpm.tp_mlp_grad_col_weight(to_dev(X), to_dev(dA), dW_i=dW, db_i=db, accumulate=accumulate)
    torch.cuda.synchronize()
    assert _guards_ok(torch, bw, pad, fill_nan=not accumulate)
    assert _guards_ok(torch, bb, pad, fill_nan=not accumulate)
    rW, rb = orc.col_weight_grad(X, dA)
    boundW = gemm_bound(f64(X).T, f64(dA), M)
    boundb = 2 * (M + 2) * U32 * np.abs(f64(dA)).sum(axis=0) + 1e-30
    if accumulate:
        rW, rb = rW + f64(W0), rb + f64(b0)
        boundW = boundW + 2 * U32 * (np.abs(rW) + boundW)
        boundb = boundb + 2 * U32 * (np.abs(rb) + boundb)
    assert_within(f64(from_dev(dW)), rW, boundW, "dW_i")
    assert_within(f64(from_dev(db)), rb, boundb, "db_i")
    assert rel_fro(f64(from_dev(dW)), rW) <= 1e-5


INPUT_CASES = [(1, 128, 64, "bf16"), (9, 136, 200, "bf16"), (129, 264, 72, "bf16"), (257, 392, 520, "bf16"),
               (512, 512, 384, "bf16"), (300, 64, 8, "bf16"), (8, 128, 64, "f32"), (65, 136, 200, "f32")]


@pytest.mark.parametrize("M,Fk,H,dtype", INPUT_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_grad_input_partial_parity(tpm, orc, M, Fk, H, dtype, accumulate):
    import torch
    say("grad_input_partial M=%d Fk=%d H=%d %s acc=%s" % (M, Fk, H, dtype, accumulate))
    k, i = 2, 0
    dA = _draw(4, (M, Fk), 0.1, dtype, M + 15)
    W = _draw(1, (H, Fk * k), 0.05, dtype, H + 16)
    Wi = np.ascontiguousarray(W[:, i * Fk:(i + 1) * Fk])
    pad = 64
    if accumulate:
        X0 = _draw(3, (M, H), 1.0, "f32", M + 17)
        buf, dX = _guarded(torch, (M, H), torch.float32, float("inf"), pad)
        dX.copy_(torch.from_numpy(X0))
    else:
        buf, dX = _guarded(torch, (M, H), torch.float32, float("nan"), pad)
    tpm.tp_mlp_grad_input_partial(to_dev(dA), to_dev(Wi), dX_i=dX, accumulate=accumulate)
    torch.cuda.synchronize()
    assert _guards_ok(torch, buf, pad, fill_nan=not accumulate)
    ref = orc.input_grad_partial(dA, W, k, i)
    bound = gemm_bound(f64(dA), f64(Wi).T, Fk)
    if accumulate:
        ref = ref + f64(X0)
        bound = bound + 2 * U32 * (np.abs(ref) + bound)
    got = f64(from_dev(dX))
    assert_within(got, ref, bound, "dX_i")
    assert rel_fro(got, ref) <= 1e-5


def backward_bounds(orc, X, W, b, V, dZ, k, dtype, fused=False):
    """Element-wise bounds of the whole backward (small shapes, all entries).
    dX: each shard's Fk products then the k partials (literal), or one float32
    sum through all F products (fused)."""
    M, H = X.shape
    F = W.shape[1]
    Fk = F // k
    bW, bb, bV = np.zeros((H, F)), np.zeros(F), np.zeros((F, H))
    bX = np.zeros((M, H))
    absX = np.abs(f64(X))
    for i in range(k):
        sl = slice(i * Fk, (i + 1) * Fk)
        t = backward_terms(orc, X, W[:, sl], None if b is None else b[sl], V[sl], dZ, dtype)
        bV[sl] = gemm_bound(t["Y"].T, f64(dZ), M, ea=t["tolY"].T)
        bW[:, sl] = gemm_bound(f64(X).T, t["dA"], M, eb=t["errdA"])
        bb[sl] = t["errdA"].sum(axis=0) + 2 * (M + 2) * U32 * (np.abs(t["dA"]) + t["errdA"]).sum(axis=0)
        part = gemm_bound(t["dA"], f64(W[:, sl]).T, F if fused else Fk, ea=t["errdA"])
        bX += part + (k + 2) * U32 * ((np.abs(t["dA"]) + t["errdA"]) @ np.abs(f64(W[:, sl])).T)
    del absX
    return bX + 1e-30, bW + 1e-30, bb + 1e-30, bV + 1e-30


BWD_CASES = [
    # M, H, F, k, dtype, bias
    (8, 64, 256, 2, "f32", True), (1, 64, 256, 2, "f32", True), (33, 72, 288, 3, "f32", False),
    (8, 64, 256, 2, "bf16", True), (1, 64, 256, 4, "bf16", True), (131, 136, 544, 4, "bf16", True),
    (40, 64, 512, 64, "bf16", True), (257, 200, 800, 1, "bf16", False), (300, 96, 384, 8, "bf16", True),
    (512, 256, 1024, 4, "bf16", True), (2100, 128, 512, 2, "bf16", True),
]


@pytest.mark.parametrize("M,H,F,k,dtype,bias", BWD_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_shard_backward_parity(tpm, orc, M, H, F, k, dtype, bias, fused):
    import torch
    say("shard_backward M=%d H=%d F=%d k=%d %s bias=%s fused=%s" % (M, H, F, k, dtype, bias, fused))
    from tensor_transformer_mlp_amd import inputs
    seed = M + H + F + k
    X = _draw(0, (M, H), 1.0, dtype, seed)
    W = _draw(1, (H, F), 0.05, dtype, seed)
    b = _draw(2, (F,), 0.05, dtype, seed) if bias else None
    V = _draw(3, (F, H), 0.05, dtype, seed)
    dZ = _draw(4, (M, H), 1.0, dtype, seed)
    Ws, bs, Vs = inputs.shard_slices(W, b if bias else np.zeros(F, W.dtype), V, k)
    Fk = F // k
    pad = 64
    bx, dX = _guarded(torch, (M, H), torch.float32, float("nan"), pad)
    gW = [_guarded(torch, (H, Fk), torch.float32, float("nan"), pad) for _ in range(k)]
    gV = [_guarded(torch, (Fk, H), torch.float32, float("nan"), pad) for _ in range(k)]
    gb = [_guarded(torch, (Fk,), torch.float32, float("nan"), pad) for _ in range(k)]
    tpm.tp_mlp_shard_backward(to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs] if bias else None,
                              [to_dev(v) for v in Vs], to_dev(dZ), dX=dX, dW=[t for _, t in gW],
                              db=[t for _, t in gb] if bias else None, dV=[t for _, t in gV], fused=fused)
    torch.cuda.synchronize()
    for buf, _ in [(bx, None)] + gW + gV + (gb if bias else []):
        assert _guards_ok(torch, buf, pad)
    rX, rW, rb, rV = orc.backward(X, W, b, V, dZ, k)
    bX, bW, bb, bV = backward_bounds(orc, X, W, b, V, dZ, k, dtype, fused=fused)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    gotX = f64(from_dev(dX))
    gotW = np.concatenate([f64(from_dev(t)) for _, t in gW], axis=1)
    gotV = np.concatenate([f64(from_dev(t)) for _, t in gV], axis=0)
    assert_within(gotX, rX, bX, "dX")
    assert_within(gotW, rW, bW, "dW")
    assert_within(gotV, rV, bV, "dV")
    for got, ref in ((gotX, rX), (gotW, rW), (gotV, rV)):
        assert rel_fro(got, ref) <= tol
    if bias:
        gotb = np.concatenate([f64(from_dev(t)) for _, t in gb])
        assert_within(gotb, rb, bb, "db")
        assert rel_fro(gotb, rb) <= tol


def _bwd_args(tpm, M, H, F, k, dtype, seed):
    from tensor_transformer_mlp_amd import inputs
    X = _draw(0, (M, H), 1.0, dtype, seed)
    W = _draw(1, (H, F), 0.05, dtype, seed)
    b = _draw(2, (F,), 0.05, dtype, seed)
    V = _draw(3, (F, H), 0.05, dtype, seed)
    dZ = _draw(4, (M, H), 1.0, dtype, seed)
    Ws, bs, Vs = inputs.shard_slices(W, b, V, k)
    return (to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs],
            to_dev(dZ))


def test_backward_fused_and_literal_deterministic(tpm):
    """Each variant gives the same bits on every run; the parameter gradients
    do not involve the dX sum and are equal across the variants bit for bit;
    the two dX (the same sum, rounded in different places) agree to float32
    rounding."""
    import torch
    args = _bwd_args(tpm, 2100, 136, 1088, 8, "bf16", 5)
    say("backward fused vs literal")
    r1 = tpm.tp_mlp_shard_backward(*args, fused=False)
    r2 = tpm.tp_mlp_shard_backward(*args, fused=True)
    r3 = tpm.tp_mlp_shard_backward(*args, fused=False)
    r4 = tpm.tp_mlp_shard_backward(*args, fused=True)
    torch.cuda.synchronize()
    for a, b_, c, d in zip(r1, r2, r3, r4):
        if isinstance(a, list):
            for x, y, z, u in zip(a, b_, c, d):
                assert torch.equal(x, y) and torch.equal(x, z) and torch.equal(y, u)
        else:
            assert torch.equal(a, c) and torch.equal(b_, d)
            assert float(torch.linalg.vector_norm((a - b_).double())) <= 1e-5 * float(
                torch.linalg.vector_norm(a.double()))


def test_backward_gradient_accumulation(tpm):
    """TP_GRAD_ACCUMULATE adds this call's parameter gradients to the given ones
    (dX is overwritten): two accumulating calls from zero give about twice one
    plain call."""
    import torch
    args = _bwd_args(tpm, 300, 64, 512, 4, "bf16", 6)
    say("backward gradient accumulation")
    dX1, dW1, db1, dV1 = tpm.tp_mlp_shard_backward(*args)
    dW = [torch.zeros_like(t) for t in dW1]
    db = [torch.zeros_like(t) for t in db1]
    dV = [torch.zeros_like(t) for t in dV1]
    for _ in range(2):
        dX2, _, _, _ = tpm.tp_mlp_shard_backward(*args, dW=dW, db=db, dV=dV, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dX1, dX2)
    for one, two in zip(dW1 + db1 + dV1, dW + db + dV):
        assert torch.allclose(two, 2 * one, rtol=1e-6, atol=1e-7)


def test_backward_empty_and_single_row(tpm, orc):
    import torch
    H, F, k = 64, 256, 2
    args = _bwd_args(tpm, 5, H, F, k, "f32", 7)
    X, Ws, bs, Vs, dZ = args
    say("backward M=0")
    dW = [torch.full((H, F // k), float("nan"), device="cuda") for _ in range(k)]
    db = [torch.full((F // k,), float("nan"), device="cuda") for _ in range(k)]
    dV = [torch.full((F // k, H), float("nan"), device="cuda") for _ in range(k)]
    dX0, dW0, db0, dV0 = tpm.tp_mlp_shard_backward(X[:0], Ws, bs, Vs, dZ[:0], dW=dW, db=db, dV=dV)
    torch.cuda.synchronize()
    assert dX0.shape == (0, H)
    for t in dW0 + db0 + dV0:
        assert not bool(torch.any(t != 0)), "empty batch must give zero parameter gradients"
    say("backward M=1")
    dX1, dW1, db1, dV1 = tpm.tp_mlp_shard_backward(X[:1], Ws, bs, Vs, dZ[:1])
    torch.cuda.synchronize()
    Xh, dZh = from_dev(X[:1]), from_dev(dZ[:1])
    Wh = np.concatenate([from_dev(w) for w in Ws], axis=1)
    bh = np.concatenate([from_dev(x) for x in bs])
    Vh = np.concatenate([from_dev(v) for v in Vs], axis=0)
    rX, rW, rb, rV = orc.backward(Xh, Wh, bh, Vh, dZh, k)
    assert rel_fro(from_dev(dX1), rX) <= 1e-5
    assert rel_fro(np.concatenate([from_dev(t) for t in dW1], axis=1), rW) <= 1e-5
    assert rel_fro(np.concatenate([from_dev(t) for t in db1]), rb) <= 1e-5
    assert rel_fro(np.concatenate([from_dev(t) for t in dV1], axis=0), rV) <= 1e-5


@pytest.mark.parametrize("M,H,F,k,fused", [(4096, 256, 1024, 4, False), (4100, 136, 544, 4, True),
                                           (8192, 768, 3072, 4, False)])
def test_backward_transposed_weights_equal_steps(tpm, M, H, F, k, fused):
    """From M = 4096 tokens (bf16) the whole backward multiplies by V_i^T and
    W_i^T through transposed copies of the weights on the GEMM's NN path; the
    step entry points read the weights as transposes (NT).  Both accumulate
    every output element over K in the same order: equal bit for bit (the
    fused dX against the steps' shard sum, the literal one against partials
    + reduce)."""
    import torch
    say("backward transposed weights M=%d H=%d F=%d k=%d fused=%s" % (M, H, F, k, fused))
    X, Ws, bs, Vs, dZ = _bwd_args(tpm, M, H, F, k, "bf16", 11)
    dX, dW, db, dV = tpm.tp_mlp_shard_backward(X, Ws, bs, Vs, dZ, fused=fused)
    Fk = F // k
    Y = [torch.empty(M, Fk, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    G = [torch.empty(M, Fk, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    tpm.tp_mlp_col_gelu_shards(X, Ws, bs, Y, G)
    dA = [torch.empty_like(g) for g in G]
    tpm.tp_mlp_grad_act_shards(dZ, Vs, G, dA)
    dV2 = [torch.empty(Fk, H, device="cuda") for _ in range(k)]
    tpm.tp_mlp_grad_row_weight_shards(Y, dZ, dV2)
    dW2 = [torch.empty(H, Fk, device="cuda") for _ in range(k)]
    db2 = [torch.empty(Fk, device="cuda") for _ in range(k)]
    tpm.tp_mlp_grad_col_weight_shards(X, dA, dW2, db2)
    if fused:
        dX2 = torch.empty(M, H, device="cuda")
        tpm.tp_mlp_grad_input_shards(dA, Ws, [dX2], sum_shards=True)
    else:
        dXp = [torch.empty(M, H, device="cuda") for _ in range(k)]
        tpm.tp_mlp_grad_input_shards(dA, Ws, dXp)
        dX2 = tpm.tp_shard_reduce(dXp)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2)
    for i in range(k):
        assert torch.equal(dW[i], dW2[i]) and torch.equal(db[i], db2[i]), ("dW/db", i)
        assert torch.equal(dV[i], dV2[i]), ("dV", i)
