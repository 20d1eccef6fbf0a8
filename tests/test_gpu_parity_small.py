"""GPU parity of every entry point against the CPU fp64 oracle at small and
ragged sizes (several tiles plus partial tiles in M, N and K), element by
element, plus the edge cases: M = 0, M = 1, k = 1, the largest shard count,
no bias, NaN-prefilled outputs and guard bands around every output.
"""
import numpy as np
import pytest

from _helpers import (assert_within, col_bound, f64, forward_bound, from_dev, rel_fro,
                      row_bound, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_transformer_mlp_amd as tpm
    tpm.lib()  # raises if the library is not built
    return tpm


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def _inputs(M, H, F, dtype, seed, std=0.05):
    from tensor_transformer_mlp_amd import inputs
    return inputs.make_custom(M, H, F, dtype, std=std, seed=seed)


def _guarded(torch, shape, dtype, fill, pad=64):
    """A tensor view with `pad` canary elements on each side."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


COL_CASES = [
    # M, H, Fk, dtype
    (1, 64, 128, "bf16"), (7, 64, 128, "bf16"), (9, 200, 136, "bf16"), (129, 72, 264, "bf16"),
    (257, 520, 392, "bf16"), (300, 64, 8, "bf16"), (64, 8, 64, "bf16"),
    (1, 64, 128, "f32"), (8, 64, 128, "f32"), (65, 200, 136, "f32"), (257, 72, 264, "f32"),
    (130, 8, 8, "f32"),
    # interior shapes (whole 256x256 / 256x128 tiles, K % 128 == 0): direct-to-LDS kernel
    (256, 128, 256, "bf16"), (512, 384, 512, "bf16"), (768, 256, 384, "bf16"),
]


@pytest.mark.parametrize("M,H,Fk,dtype", COL_CASES)
def test_col_gelu_parity(tpm, orc, M, H, Fk, dtype):
    import torch
    say("col_gelu M=%d H=%d Fk=%d %s" % (M, H, Fk, dtype))
    k = 3
    inp = _inputs(M, H, Fk * k, dtype, seed=M * 7 + H)
    X, W, b = inp["X"], inp["W"], inp["b"]
    i = 1
    Wi = np.ascontiguousarray(W[:, i * Fk:(i + 1) * Fk])
    bi = np.ascontiguousarray(b[i * Fk:(i + 1) * Fk])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pad = 64
    buf, Y = _guarded(torch, (M, Fk), tdt, float("nan"), pad)
    tpm.tp_mlp_col_gelu(to_dev(X), to_dev(Wi), to_dev(bi), Y_i=Y)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Yg = f64(from_dev(Y))
    assert np.all(np.isfinite(Yg))
    A = orc.col_preact(X, W, b, k, i)
    Yr = orc.col_gelu(X, W, b, k, i)
    bound = col_bound(f64(X), f64(Wi), f64(bi), A, Yr, dtype)
    assert_within(Yg, Yr, bound, "Y_i")
    assert rel_fro(Yg, Yr) <= (1e-2 if dtype == "bf16" else 1e-5)


ROW_CASES = [
    (1, 128, 64, "bf16"), (9, 136, 200, "bf16"), (129, 264, 72, "bf16"), (257, 392, 520, "bf16"),
    (300, 8, 64, "bf16"), (8, 128, 64, "f32"), (65, 136, 200, "f32"), (257, 264, 72, "f32"),
    (256, 128, 256, "bf16"), (512, 512, 384, "bf16"), (768, 384, 256, "bf16"),
]


@pytest.mark.parametrize("M,Fk,H,dtype", ROW_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_row_partial_parity(tpm, orc, M, Fk, H, dtype, accumulate):
    import torch
    say("row_partial M=%d Fk=%d H=%d %s acc=%s" % (M, Fk, H, dtype, accumulate))
    k = 2
    inp = _inputs(M, H, Fk * k, dtype, seed=M * 5 + Fk)
    V = inp["V"]
    # Y_i with the magnitude of GeLU outputs: draw from the X stream
    from tensor_transformer_mlp_amd import inputs
    Y = inputs.draw(0, (M, Fk), 0.5, dtype, seed=M + 11)
    i = 1
    Vi = np.ascontiguousarray(V[i * Fk:(i + 1) * Fk])
    pad = 64
    if accumulate:
        Z0 = inputs.draw(3, (M, H), 1.0, "f32", seed=M + 13)
        buf, Z = _guarded(torch, (M, H), torch.float32, float("inf"), pad)
        Z.copy_(torch.from_numpy(Z0))
    else:
        buf, Z = _guarded(torch, (M, H), torch.float32, float("nan"), pad)
    tpm.tp_mlp_row_partial(to_dev(Y), to_dev(Vi), Z_i=Z, accumulate=accumulate)
    torch.cuda.synchronize()
    fill_ok = (lambda t: bool(torch.all(torch.isinf(t)))) if accumulate else (lambda t: bool(torch.all(torch.isnan(t))))
    assert fill_ok(buf[:pad]) and fill_ok(buf[-pad:])
    Zg = f64(from_dev(Z))
    Zr = orc.row_partial(Y, V, k, i)
    bound = row_bound(f64(Y), f64(Vi))
    if accumulate:
        Zr = Zr + f64(Z0)
        bound = bound + 2 * 2.0 ** -24 * np.abs(Zr)
    assert_within(Zg, Zr, bound, "Z_i")
    assert rel_fro(Zg, Zr) <= 1e-5


@pytest.mark.parametrize("k,n", [(1, 1000), (2, 4096), (3, 1003), (4, 65536), (8, 12345), (16, 777),
                                 (64, 2048)])
@pytest.mark.parametrize("inplace", [False, True])
def test_shard_reduce_parity(tpm, orc, k, n, inplace):
    import torch
    say("shard_reduce k=%d n=%d inplace=%s" % (k, n, inplace))
    from tensor_transformer_mlp_amd import inputs
    parts_h = [inputs.draw(3, (n,), 1.0, "f32", seed=100 + j) for j in range(k)]
    parts = [torch.from_numpy(p).cuda() for p in parts_h]
    pad = 32
    if inplace:
        Z = parts[0]
        tpm.tp_shard_reduce(parts, Z=Z)
    else:
        buf, Z = _guarded(torch, (n,), torch.float32, float("nan"), pad)
        tpm.tp_shard_reduce(parts, Z=Z)
    torch.cuda.synchronize()
    if not inplace:
        assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Zg = from_dev(Z).astype(np.float64)
    ref = orc.shard_reduce(parts_h)
    # float32 left-to-right sum, exactly as the kernel must do it
    s = parts_h[0].copy()
    for p in parts_h[1:]:
        s = (s + p).astype(np.float32)
    assert np.array_equal(from_dev(Z), s)
    bound = (k + 1) * 2.0 ** -24 * orc.shard_reduce([np.abs(p) for p in parts_h]) + 1e-30
    assert_within(Zg, ref, bound, "Z")


FWD_CASES = [
    # M, H, F, k, dtype
    (8, 64, 256, 2, "f32"), (1, 64, 256, 2, "f32"), (33, 72, 288, 3, "f32"), (16, 64, 256, 1, "f32"),
    (8, 64, 256, 2, "bf16"), (1, 64, 256, 4, "bf16"), (131, 136, 544, 4, "bf16"), (64, 64, 512, 16, "bf16"),
    (40, 64, 512, 64, "bf16"), (257, 200, 800, 1, "bf16"), (300, 96, 384, 8, "bf16"),
    (512, 256, 1024, 4, "bf16"), (256, 384, 1536, 3, "bf16"),
]


@pytest.mark.parametrize("M,H,F,k,dtype", FWD_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_shard_forward_parity(tpm, orc, M, H, F, k, dtype, fused):
    import torch
    say("shard_forward M=%d H=%d F=%d k=%d %s fused=%s" % (M, H, F, k, dtype, fused))
    from tensor_transformer_mlp_amd import inputs
    inp = _inputs(M, H, F, dtype, seed=M + H + F + k, std=0.05)
    X, W, b, V = inp["X"], inp["W"], inp["b"], inp["V"]
    Ws, bs, Vs = inputs.shard_slices(W, b, V, k)
    pad = 64
    buf, Z = _guarded(torch, (M, H), torch.float32, float("nan"), pad)
    tpm.tp_mlp_shard_forward(to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs],
                             [to_dev(v) for v in Vs], Z=Z, fused=fused)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Zg = f64(from_dev(Z))
    assert np.all(np.isfinite(Zg))
    Zr = orc.forward(X, W, b, V, k)
    Fk = F // k
    X64, W64, b64, V64 = f64(X), f64(W), f64(b), f64(V)
    A = np.concatenate([orc.col_preact(X, W, b, k, i) for i in range(k)], axis=1)
    Y = np.concatenate([orc.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
    tolY = np.concatenate([col_bound(X64, W64[:, i * Fk:(i + 1) * Fk], b64[i * Fk:(i + 1) * Fk],
                                     A[:, i * Fk:(i + 1) * Fk], Y[:, i * Fk:(i + 1) * Fk], dtype)
                           for i in range(k)], axis=1)
    bound = forward_bound(tolY, Y, V64, k, fused=fused)
    assert_within(Zg, Zr, bound, "Z")
    assert rel_fro(Zg, Zr) <= (1e-2 if dtype == "bf16" else 1e-5)


def test_fused_and_literal_deterministic(tpm):
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F, k = 300, 136, 1088, 8
    inp = _inputs(M, H, F, "bf16", seed=5)
    Ws, bs, Vs = inputs.shard_slices(inp["W"], inp["b"], inp["V"], k)
    args = (to_dev(inp["X"]), [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs])
    say("fused vs literal M=%d H=%d F=%d k=%d" % (M, H, F, k))
    Z1 = tpm.tp_mlp_shard_forward(*args, fused=False)
    Z2 = tpm.tp_mlp_shard_forward(*args, fused=True)
    Z3 = tpm.tp_mlp_shard_forward(*args, fused=False)
    Z4 = tpm.tp_mlp_shard_forward(*args, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z3) and torch.equal(Z2, Z4)
    # the same sum, rounded in different places
    assert rel_fro(from_dev(Z2), from_dev(Z1)) <= 1e-5


def test_no_bias_and_empty(tpm, orc):
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F, k = 17, 64, 256, 2
    inp = _inputs(M, H, F, "f32", seed=9)
    Ws, bs, Vs = inputs.shard_slices(inp["W"], inp["b"], inp["V"], k)
    say("no-bias forward")
    Z = tpm.tp_mlp_shard_forward(to_dev(inp["X"]), [to_dev(w) for w in Ws], None, [to_dev(v) for v in Vs])
    torch.cuda.synchronize()
    Zr = orc.forward(inp["X"], inp["W"], None, inp["V"], k)
    assert rel_fro(from_dev(Z), Zr) <= 1e-5
    # M == 0: nothing to do, nothing written
    say("empty forward")
    X0 = torch.empty(0, H, device="cuda")
    Z0 = tpm.tp_mlp_shard_forward(X0, [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs])
    Y0 = tpm.tp_mlp_col_gelu(X0, to_dev(Ws[0]), to_dev(bs[0]))
    torch.cuda.synchronize()
    assert Z0.shape == (0, H) and Y0.shape == (0, F // k)


def test_k_invariance_gpu(tpm):
    """Same full W, b, V at k = 1, 2, 4, 8: the float32 results agree to the
    accumulation-order bound (they differ only in where partial sums split)."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F = 96, 64, 512
    inp = _inputs(M, H, F, "f32", seed=21)
    Zs = []
    for k in (1, 2, 4, 8):
        say("k-invariance k=%d" % k)
        Ws, bs, Vs = inputs.shard_slices(inp["W"], inp["b"], inp["V"], k)
        Zs.append(from_dev(tpm.tp_mlp_shard_forward(to_dev(inp["X"]), [to_dev(w) for w in Ws],
                                                     [to_dev(x) for x in bs], [to_dev(v) for v in Vs])))
    torch.cuda.synchronize()
    for Z in Zs[1:]:
        assert rel_fro(Z, Zs[0]) <= 1e-6
