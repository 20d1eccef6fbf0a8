"""GPU parity at seeded random shapes: the block forward and backward (M any
size, H and F/k any multiple of 8, 1 to 6 shards, both element types, both
variants of the shard sum; a few bf16 backward cases with M >= 4096, the path
through transposed weights), the SwiGLU column step, and the attention kernel
(random sequence lengths, head counts, widths 64 and 128, causal or not).
Every output element within the oracle's bound and the relative Frobenius
bar.  The shapes land on mixes of whole and partial tiles (in M, N, K and in
query and key blocks) that the fixed cases do not name one by one.
"""
import numpy as np
import pytest

from _helpers import assert_within, col_bound, f64, forward_bound, from_dev, rel_fro, say, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261202):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        M = int(rng.randint(1, 1500))
        H = 8 * int(rng.randint(1, 81))
        Fk = 8 * int(rng.randint(1, 81))
        k = int(rng.randint(1, 7))
        dtype = "f32" if rng.rand() < 0.25 else "bf16"
        if M * H * Fk * k > 200_000_000:  # keep each oracle call around a second
            continue
        out.append((M, H, Fk, k, dtype))
    return out


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


@pytest.mark.parametrize("M,H,Fk,k,dtype", _cases())
def test_random_shape_forward(tpm, orc, M, H, Fk, k, dtype):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("random forward M=%d H=%d Fk=%d k=%d %s" % (M, H, Fk, k, dtype))
    F = Fk * k
    inp = inputs.make_custom(M, H, F, dtype, std=0.05, seed=M * 131 + H * 7 + Fk + k)
    X, W, b, V = inp["X"], inp["W"], inp["b"], inp["V"]
    Ws, bs, Vs = inputs.shard_slices(W, b, V, k)
    args = (to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs])
    Zl = tpm.tp_mlp_shard_forward(*args, fused=False)
    Zf = tpm.tp_mlp_shard_forward(*args, fused=True)
    torch.cuda.synchronize()
    Zg = f64(from_dev(Zl))
    Zgf = f64(from_dev(Zf))
    assert np.all(np.isfinite(Zg)) and np.all(np.isfinite(Zgf))
    Zr = orc.forward(X, W, b, V, k)
    X64, W64, b64, V64 = f64(X), f64(W), f64(b), f64(V)
    A = np.concatenate([orc.col_preact(X, W, b, k, i) for i in range(k)], axis=1)
    Y = np.concatenate([orc.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
    tolY = np.concatenate([col_bound(X64, W64[:, i * Fk:(i + 1) * Fk], b64[i * Fk:(i + 1) * Fk],
                                     A[:, i * Fk:(i + 1) * Fk], Y[:, i * Fk:(i + 1) * Fk], dtype)
                           for i in range(k)], axis=1)
    assert_within(Zg, Zr, forward_bound(tolY, Y, V64, k), "Z")
    assert_within(Zgf, Zr, forward_bound(tolY, Y, V64, k, fused=True), "Z (fused)")
    assert rel_fro(Zg, Zr) <= (1e-2 if dtype == "bf16" else 1e-5)
    assert rel_fro(Zgf, Zr) <= (1e-2 if dtype == "bf16" else 1e-5)


def _bwd_cases(n=12, seed=20261203):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        M = int(rng.randint(1, 1200))
        H = 8 * int(rng.randint(1, 49))
        Fk = 8 * int(rng.randint(1, 49))
        k = int(rng.randint(1, 5))
        dtype = "f32" if rng.rand() < 0.25 else "bf16"
        bias = bool(rng.rand() < 0.75)
        if M * H * Fk * k > 40_000_000:
            continue
        out.append((M, H, Fk, k, dtype, bias))
    return out


def _bwd_big_m_cases(n=4, seed=20261206):
    """bf16 with M >= 4096: the whole backward's path through transposed
    weight copies (narrow H and F/k keep the oracle quick)."""
    rng = np.random.RandomState(seed)
    return [(int(rng.randint(4096, 6500)), 8 * int(rng.randint(1, 13)), 8 * int(rng.randint(1, 13)),
             int(rng.randint(1, 4)), "bf16", bool(rng.rand() < 0.7)) for _ in range(n)]


@pytest.mark.parametrize("M,H,Fk,k,dtype,bias", _bwd_cases() + _bwd_big_m_cases())
def test_random_shape_backward(tpm, orc, M, H, Fk, k, dtype, bias):
    """The block backward (dX, dW_i, db_i, dV_i) at seeded random shapes,
    both variants within the oracle's element bounds (their parameter
    gradients equal bit for bit)."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    from test_gpu_backward import backward_bounds
    say("random backward M=%d H=%d Fk=%d k=%d %s bias=%s" % (M, H, Fk, k, dtype, bias))
    F = Fk * k
    seed = M * 17 + H + Fk * 3 + k
    X = inputs.draw(0, (M, H), 1.0, dtype, seed=seed)
    W = inputs.draw(1, (H, F), 0.05, dtype, seed=seed)
    b = inputs.draw(2, (F,), 0.05, dtype, seed=seed) if bias else None
    V = inputs.draw(3, (F, H), 0.05, dtype, seed=seed)
    dZ = inputs.draw(4, (M, H), 1.0, dtype, seed=seed)
    Ws, bs, Vs = inputs.shard_slices(W, b if bias else np.zeros(F, W.dtype), V, k)
    dev_args = (to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs] if bias else None,
                [to_dev(v) for v in Vs], to_dev(dZ))
    outs = []
    for fused in (False, True):
        dX = torch.empty(M, H, device="cuda")
        dW = [torch.empty(H, Fk, device="cuda") for _ in range(k)]
        dV = [torch.empty(Fk, H, device="cuda") for _ in range(k)]
        db = [torch.empty(Fk, device="cuda") for _ in range(k)] if bias else None
        tpm.tp_mlp_shard_backward(*dev_args, dX=dX, dW=dW, db=db, dV=dV, fused=fused)
        outs.append((dX, dW, db, dV))
    torch.cuda.synchronize()
    (dX, dW, db, dV), (dX2, dW2, db2, dV2) = outs
    assert all(torch.equal(x, y) for x, y in zip(dW + dV + (db or []), dW2 + dV2 + (db2 or [])))
    rX, rW, rb, rV = orc.backward(X, W, b, V, dZ, k)
    bX, bW, bb, bV = backward_bounds(orc, X, W, b, V, dZ, k, dtype)
    bXf = backward_bounds(orc, X, W, b, V, dZ, k, dtype, fused=True)[0]
    assert_within(f64(from_dev(dX2)), rX, bXf, "dX (fused)")
    gotW = np.concatenate([f64(from_dev(t)) for t in dW], axis=1)
    gotV = np.concatenate([f64(from_dev(t)) for t in dV], axis=0)
    assert_within(f64(from_dev(dX)), rX, bX, "dX")
    assert_within(gotW, rW, bW, "dW")
    assert_within(gotV, rV, bV, "dV")
    tol = 1e-2 if dtype == "bf16" else 1e-5
    for got, ref in ((f64(from_dev(dX)), rX), (gotW, rW), (gotV, rV)):
        assert rel_fro(got, ref) <= tol
    if bias:
        gotb = np.concatenate([f64(from_dev(t)) for t in db])
        assert_within(gotb, rb, bb, "db")


def _swiglu_cases(n=12, seed=20261204):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        M = int(rng.randint(1, 1500))
        H = 8 * int(rng.randint(1, 81))
        Fk = 8 * int(rng.randint(1, 81))
        dtype = "f32" if rng.rand() < 0.25 else "bf16"
        if M * H * Fk > 60_000_000:
            continue
        out.append((M, H, Fk, dtype))
    return out


@pytest.mark.parametrize("M,H,Fk,dtype", _swiglu_cases())
def test_random_shape_swiglu_col(tpm, orc, M, H, Fk, dtype):
    """The SwiGLU column step (two weights, SiLU(X Wg) * (X Wu)) at seeded
    random shapes, within the oracle's element bounds."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    from _helpers import swiglu_bound
    say("random swiglu_col M=%d H=%d Fk=%d %s" % (M, H, Fk, dtype))
    inp = inputs.make_swiglu(M=M, H=H, F=Fk, dtype=dtype, std=0.05, seed=M * 3 + H + Fk)
    X, Wg, Wu = inp["X"], inp["Wg"], inp["Wu"]
    Y = tpm.tp_swiglu_col(to_dev(X), to_dev(Wg), to_dev(Wu))
    torch.cuda.synchronize()
    Yg = f64(from_dev(Y))
    Yr = orc.swiglu_col(X, Wg, Wu, 1, 0)
    X64 = f64(X)
    G, U = X64 @ f64(Wg), X64 @ f64(Wu)
    assert_within(Yg, Yr, swiglu_bound(X64, f64(Wg), f64(Wu), G, U, Yr, dtype), "Y")
    assert rel_fro(Yg, Yr) <= (1e-2 if dtype == "bf16" else 1e-5)


def _attn_cases(n=12, seed=20261205):
    rng = np.random.RandomState(seed)
    out = []
    while len(out) < n:
        B = int(rng.randint(1, 4))
        S = int(rng.randint(1, 700))
        heads = int(rng.randint(1, 4))
        d = 64 if rng.rand() < 0.5 else 128
        causal = bool(rng.rand() < 0.7)
        std = float(rng.choice([0.5, 1.0, 2.0]))
        out.append((B, S, heads, d, causal, std))
    return out


@pytest.mark.parametrize("B,S,heads,d,causal,std", _attn_cases())
def test_random_shape_attention_core(tpm, orc, B, S, heads, d, causal, std):
    """The attention kernel at seeded random sequence lengths, head counts and
    widths, causal or not, within the oracle's element bounds."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    from _helpers import attn_core_bound
    say("random attn_core B=%d S=%d heads=%d d=%d causal=%s std=%g" % (B, S, heads, d, causal, std))
    Hk = heads * d
    qkv = inputs.draw(inputs.STREAM_X, (B * S, 3 * Hk), std, "bf16", seed=B * 7919 + S * 13 + heads + d)
    A = torch.full((B * S, Hk), float("nan"), dtype=torch.bfloat16, device="cuda")
    tpm.tp_attn_core_shards([to_dev(qkv)], [A], B, S, heads, d, causal=causal)
    torch.cuda.synchronize()
    Ag = f64(from_dev(A))
    assert np.all(np.isfinite(Ag))
    Ar = orc.attn_core(qkv, B, S, heads, d, causal)
    assert_within(Ag, Ar, attn_core_bound(f64(qkv), Ar, B, S, heads, d, causal), "A")
    assert rel_fro(Ag, Ar) <= 1e-2
