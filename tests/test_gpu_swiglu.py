"""GPU parity of the SwiGLU block (tp_swiglu_col, tp_swiglu_col_shards,
tp_swiglu_shard_forward) against the CPU fp64 oracle, element by element,
at small and ragged sizes (several tiles plus partial tiles in M, Fk and H,
H not a multiple of 32), at the workload sizes on sampled rows, plus the
edge cases (M = 0, M = 1, k = 1, 16 shards in one launch, guard bands, the
fp32 path), the batched == single-shard bit-identity and both variants of
the shard sum.  The exact gate and up pre-activations for the bounds are
plain float64 products of the same inputs; expected values come from the
oracle.
"""
import numpy as np
import pytest

from _helpers import (U32, assert_within, f64, forward_bound, from_dev, rel_fro, say, swiglu_bound,
                      tile_rows, to_dev)

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


def _inputs(M, H, F, dtype, seed, std=0.05):
    from tensor_transformer_mlp_amd import inputs
    return inputs.make_swiglu(M=M, H=H, F=F, dtype=dtype, std=std, seed=seed)


def _guarded(torch, shape, dtype, pad=64):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


COL_CASES = [
    # M, H, Fk, dtype
    (1, 64, 128, "bf16"), (7, 64, 136, "bf16"), (129, 72, 264, "bf16"), (257, 520, 392, "bf16"),
    (300, 64, 8, "bf16"), (64, 8, 64, "bf16"), (512, 256, 512, "bf16"), (1024, 768, 768, "bf16"),
    (96, 200, 96, "bf16"),
    (1, 64, 128, "f32"), (65, 200, 136, "f32"), (130, 8, 8, "f32"),
]


@pytest.mark.parametrize("M,H,Fk,dtype", COL_CASES)
def test_swiglu_col_parity(tpm, orc, M, H, Fk, dtype):
    import torch
    say("swiglu_col M=%d H=%d Fk=%d %s" % (M, H, Fk, dtype))
    k = 3
    inp = _inputs(M, H, Fk * k, dtype, seed=M * 7 + H)
    X, Wg, Wu = inp["X"], inp["Wg"], inp["Wu"]
    i = 2
    Wgi = np.ascontiguousarray(Wg[:, i * Fk:(i + 1) * Fk])
    Wui = np.ascontiguousarray(Wu[:, i * Fk:(i + 1) * Fk])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pad = 64
    buf, Y = _guarded(torch, (M, Fk), tdt, pad)
    tpm.tp_swiglu_col(to_dev(X), to_dev(Wgi), to_dev(Wui), Y_i=Y)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Yg = f64(from_dev(Y))
    assert np.all(np.isfinite(Yg))
    Yr = orc.swiglu_col(X, Wg, Wu, k, i)
    X64 = f64(X)
    G, U = X64 @ f64(Wgi), X64 @ f64(Wui)
    assert_within(Yg, Yr, swiglu_bound(X64, f64(Wgi), f64(Wui), G, U, Yr, dtype), "Y_i")
    assert rel_fro(Yg, Yr) <= (1e-2 if dtype == "bf16" else 1e-5)


def test_swiglu_col_shards_equal_single(tpm):
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F, n = 300, 136, 16 * 136, 16
    say("swiglu_col_shards n=%d M=%d H=%d Fk=%d" % (n, M, H, F // n))
    inp = _inputs(M, H, F, "bf16", seed=3)
    X = to_dev(inp["X"])
    Wg = [to_dev(w) for w in inputs.col_slices(inp["Wg"], n)]
    Wu = [to_dev(w) for w in inputs.col_slices(inp["Wu"], n)]
    Fk = F // n
    Yb = [torch.empty(M, Fk, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tpm.tp_swiglu_col_shards(X, Wg, Wu, Yb)
    for i in range(n):
        Ys = tpm.tp_swiglu_col(X, Wg[i], Wu[i])
        torch.cuda.synchronize()
        assert torch.equal(Ys, Yb[i]), i


FWD_CASES = [
    # M, H, F, k, dtype
    (8, 64, 256, 2, "f32"), (96, 72, 408, 3, "bf16"), (256, 128, 1024, 4, "bf16"),
    (33, 136, 272, 1, "bf16"), (64, 64, 512, 8, "bf16"), (160, 200, 1600, 10, "bf16"),
    (17, 64, 1024, 16, "f32"),
]


@pytest.mark.parametrize("M,H,F,k,dtype", FWD_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_swiglu_shard_forward_parity(tpm, orc, M, H, F, k, dtype, fused):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("swiglu_shard_forward M=%d H=%d F=%d k=%d %s fused=%s" % (M, H, F, k, dtype, fused))
    inp = _inputs(M, H, F, dtype, seed=M + H + F + k)
    X, Wg, Wu, V = inp["X"], inp["Wg"], inp["Wu"], inp["V"]
    Wgs, Wus = inputs.col_slices(Wg, k), inputs.col_slices(Wu, k)
    Fk = F // k
    Vs = [np.ascontiguousarray(V[i * Fk:(i + 1) * Fk]) for i in range(k)]
    pad = 64
    buf, Z = _guarded(torch, (M, H), torch.float32, pad)
    tpm.tp_swiglu_shard_forward(to_dev(X), [to_dev(w) for w in Wgs], [to_dev(w) for w in Wus],
                                [to_dev(v) for v in Vs], Z=Z, fused=fused)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Zg = f64(from_dev(Z))
    assert np.all(np.isfinite(Zg))
    Zr = orc.swiglu_forward(X, Wg, Wu, V, k)
    X64 = f64(X)
    G, U = X64 @ f64(Wg), X64 @ f64(Wu)
    Y = np.concatenate([orc.swiglu_col(X, Wg, Wu, k, i) for i in range(k)], axis=1)
    tolY = swiglu_bound(X64, f64(Wg), f64(Wu), G, U, Y, dtype)
    assert_within(Zg, Zr, forward_bound(tolY, Y, f64(V), k, fused=fused), "Z")
    assert rel_fro(Zg, Zr) <= (1e-2 if dtype == "bf16" else 1e-5)


def test_swiglu_fused_and_literal_and_empty(tpm):
    """Both variants deterministic; the same Z up to float32 rounding of the
    shard sum; M = 0 is a no-op."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F, k = 300, 136, 1088, 8
    say("swiglu fused vs literal M=%d H=%d F=%d k=%d" % (M, H, F, k))
    inp = _inputs(M, H, F, "bf16", seed=5)
    Fk = F // k
    args = (to_dev(inp["X"]), [to_dev(w) for w in inputs.col_slices(inp["Wg"], k)],
            [to_dev(w) for w in inputs.col_slices(inp["Wu"], k)],
            [to_dev(np.ascontiguousarray(inp["V"][i * Fk:(i + 1) * Fk])) for i in range(k)])
    Z1 = tpm.tp_swiglu_shard_forward(*args, fused=False)
    Z2 = tpm.tp_swiglu_shard_forward(*args, fused=True)
    Z3 = tpm.tp_swiglu_shard_forward(*args, fused=False)
    Z4 = tpm.tp_swiglu_shard_forward(*args, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z3) and torch.equal(Z2, Z4)
    assert rel_fro(from_dev(Z2), from_dev(Z1)) <= 1e-5
    say("swiglu M=0")
    X0 = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    Z0 = tpm.tp_swiglu_shard_forward(X0, *args[1:])
    Y0 = tpm.tp_swiglu_col(X0, args[1][0], args[2][0])
    torch.cuda.synchronize()
    assert Z0.numel() == 0 and Y0.numel() == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "gpt2_small", "llama7b", "gpt3_175b", "long_seq"])
def test_swiglu_workload_tile_rows(tpm, orc, name):
    """Full-size SwiGLU forward in the benchmark's launch configuration, both
    variants; rows covering every 256-row tile of the output (all rows of the
    tiny workload) against the oracle, element by element with the SwiGLU
    bound through V."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    w = inputs.WORKLOADS[name]
    say("workload swiglu %s M=%d H=%d F=%d k=%d" % (name, w.M, w.H, w.F, w.k))
    inp = inputs.make_swiglu(w)
    X, Wg, Wu, V = inp["X"], inp["Wg"], inp["Wu"], inp["V"]
    Fk, k = w.Fk, w.k
    args = (to_dev(X), [to_dev(x) for x in inputs.col_slices(Wg, k)], [to_dev(x) for x in inputs.col_slices(Wu, k)],
            [to_dev(np.ascontiguousarray(V[i * Fk:(i + 1) * Fk])) for i in range(k)])
    Zl = tpm.tp_swiglu_shard_forward(*args, fused=False)
    Zf = tpm.tp_swiglu_shard_forward(*args, fused=True)
    torch.cuda.synchronize()
    del args
    rows = np.arange(w.M) if w.M <= 64 else tile_rows(w.M)
    rows_t = torch.from_numpy(rows).cuda()
    Zr = orc.swiglu_forward_rows(X, Wg, Wu, V, k, rows)
    X64 = f64(X[rows])
    Wg64, Wu64, V64 = f64(Wg), f64(Wu), f64(V)
    G, U = X64 @ Wg64, X64 @ Wu64
    Y = np.concatenate([orc.swiglu_col(X[rows], Wg, Wu, k, i) for i in range(k)], axis=1)
    tolY = swiglu_bound(X64, Wg64, Wu64, G, U, Y, w.dtype)
    tol = 1e-2 if w.dtype == "bf16" else 1e-5
    for label, fused, Zd in (("literal", False, Zl), ("fused", True, Zf)):
        Zg = f64(from_dev(Zd.index_select(0, rows_t)))
        assert np.all(np.isfinite(Zg))
        assert_within(Zg, Zr, forward_bound(tolY, Y, V64, k, fused=fused), "%s Z (%s)" % (name, label))
        err = rel_fro(Zg, Zr)
        say("  %s: rel_fro on %d rows covering every row tile = %.3e (%s)" % (name, rows.size, err, label))
        assert err <= tol
