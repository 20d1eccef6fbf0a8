"""GPU parity of the sequence-parallel reduce-scatter with the residual
(tp_sp_reduce_scatter) and of the sequence-parallel block forward
(tp_mlp_shard_forward_sp) against the CPU fp64 oracle, element by element,
at small and ragged sizes and at the workload sizes, plus bit-exact checks
against the same float32 additions done by torch, and the edge cases: M = 0,
one row per rank, k = 1, the largest part and rank counts, no residual,
bf16 output, separate block buffers and guard bands around the output.

Error model: the kernel sums n parts and the residual in float32, so
|O - O_exact| <= (n + 1) u32 (|R| + sum |P_i|) before the output rounding;
a bf16 output adds at most half an ulp, 2^-8 |O| (8 significant bits).
"""
import numpy as np
import pytest

from _helpers import (U16, U32, assert_within, col_bound, f64, forward_bound, from_dev, rel_fro, say,
                      to_dev)

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


def _guarded(torch, shape, dtype, pad=64):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


def _torch_sum(torch, parts, R):
    """The kernel's float32 additions, done by torch: ((P0 + P1) + ...) then R + s."""
    s = parts[0].clone()
    for p in parts[1:]:
        s = s + p
    return s if R is None else R.float() + s


SP_CASES = [
    # M, H, k, nparts, residual dtype (None: no residual), output dtype
    (8, 64, 2, 2, "bf16", "f32"), (12, 72, 4, 4, "f32", "f32"), (16, 8, 8, 8, "bf16", "bf16"),
    (300, 200, 3, 5, "bf16", "f32"), (1024, 768, 4, 4, "bf16", "bf16"), (4, 16, 4, 1, None, "f32"),
    (6, 24, 1, 3, "f32", "bf16"), (128, 64, 64, 2, "bf16", "f32"), (8, 32, 2, 64, "f32", "f32"),
    (8192, 768, 4, 4, "bf16", "f32"), (2048, 1032, 8, 8, "bf16", "bf16"),
]


@pytest.mark.parametrize("M,H,k,nparts,rdt,odt", SP_CASES)
def test_sp_reduce_scatter_parity(tpm, orc, M, H, k, nparts, rdt, odt):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("sp_reduce_scatter M=%d H=%d k=%d nparts=%d R=%s out=%s" % (M, H, k, nparts, rdt, odt))
    parts = [inputs.draw(3, (M, H), 1.0, "f32", seed=1000 + 17 * i + M) for i in range(nparts)]
    R = inputs.draw(0, (M, H), 1.0, rdt, seed=77 + M) if rdt else None
    pd = [to_dev(p) for p in parts]
    Rd = to_dev(R) if R is not None else None
    tdt = torch.bfloat16 if odt == "bf16" else torch.float32
    pad = 64
    buf, O = _guarded(torch, (M, H), tdt, pad)
    tpm.tp_sp_reduce_scatter(pd, k, R=Rd, O=O, out_dtype=tdt)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    # bit-exact: the same float32 additions in the same order (and the same rounding to bf16)
    ref32 = _torch_sum(torch, pd, Rd)
    assert torch.equal(O, ref32.to(tdt))
    # against the oracle, block by block
    blocks = orc.sp_reduce_scatter(parts, R, k)
    Og = f64(from_dev(O))
    Mb = M // k
    S = sum(np.abs(f64(p)) for p in parts) + (np.abs(f64(R)) if R is not None else 0.0)
    err32 = (nparts + 1) * U32 * S
    for r in range(k):
        ref = blocks[r]
        e = err32[r * Mb:(r + 1) * Mb]
        bound = e + (U16 * (np.abs(ref) + e) if odt == "bf16" else 0.0) + 1e-30
        assert_within(Og[r * Mb:(r + 1) * Mb], ref, bound, "O[%d]" % r)


def test_sp_separate_blocks_and_empty(tpm, orc):
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, k = 96, 48, 3
    say("sp_reduce_scatter separate blocks M=%d H=%d k=%d" % (M, H, k))
    parts = [inputs.draw(3, (M, H), 1.0, "f32", seed=s) for s in (5, 6)]
    R = inputs.draw(0, (M, H), 1.0, "bf16", seed=8)
    blocks = [torch.full((M // k, H), float("nan"), device="cuda") for _ in range(k)]
    tpm.tp_sp_reduce_scatter([to_dev(p) for p in parts], k, R=to_dev(R), O=blocks)
    torch.cuda.synchronize()
    ref = orc.sp_reduce_scatter(parts, R, k)
    for r in range(k):
        assert rel_fro(from_dev(blocks[r]), ref[r]) <= 1e-6
    # M == 0: nothing launched, nothing written
    say("sp_reduce_scatter M=0")
    e = torch.empty(0, H, device="cuda")
    out = tpm.tp_sp_reduce_scatter([e, e], 2, R=e)
    torch.cuda.synchronize()
    assert out.numel() == 0


SPF_CASES = [
    # M, H, F, k, dtype, out dtype
    (8, 64, 256, 2, "f32", "f32"),     # the tiny fp32 configuration's shapes
    (96, 72, 408, 3, "bf16", "f32"), (256, 128, 1024, 4, "bf16", "bf16"), (64, 64, 512, 8, "bf16", "f32"),
    (33, 136, 272, 1, "bf16", "f32"), (160, 64, 256, 16, "f32", "bf16"),
]


@pytest.mark.parametrize("M,H,F,k,dtype,odt", SPF_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_shard_forward_sp_parity(tpm, orc, M, H, F, k, dtype, odt, fused):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("shard_forward_sp M=%d H=%d F=%d k=%d %s out=%s fused=%s" % (M, H, F, k, dtype, odt, fused))
    inp = inputs.make_custom(M, H, F, dtype, std=0.05, seed=M + 3 * H + k)
    X, W, b, V = inp["X"], inp["W"], inp["b"], inp["V"]
    Ws, bs, Vs = inputs.shard_slices(W, b, V, k)
    args = (to_dev(X), [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs])
    tdt = torch.bfloat16 if odt == "bf16" else torch.float32
    pad = 64
    buf, O = _guarded(torch, (M, H), tdt, pad)
    tpm.tp_mlp_shard_forward_sp(*args, O=O, out_dtype=tdt, fused=fused)
    Z = tpm.tp_mlp_shard_forward(*args, fused=fused)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    # the blocks are X + Z of the all-reduce forward, bit for bit
    assert torch.equal(O, (args[0].float() + Z).to(tdt))
    # against the oracle
    Og = f64(from_dev(O))
    assert np.all(np.isfinite(Og))
    ref = np.concatenate(orc.sp_forward(X, W, b, V, k), axis=0)
    Fk = F // k
    X64, W64, b64, V64 = f64(X), f64(W), f64(b), f64(V)
    A = np.concatenate([orc.col_preact(X, W, b, k, i) for i in range(k)], axis=1)
    Y = np.concatenate([orc.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
    tolY = np.concatenate([col_bound(X64, W64[:, i * Fk:(i + 1) * Fk], b64[i * Fk:(i + 1) * Fk],
                                     A[:, i * Fk:(i + 1) * Fk], Y[:, i * Fk:(i + 1) * Fk], dtype)
                           for i in range(k)], axis=1)
    e = forward_bound(tolY, Y, V64, k, fused=fused) + 2 * U32 * (np.abs(X64) + np.abs(ref))
    bound = e + (U16 * (np.abs(ref) + e) if odt == "bf16" else 0.0)
    assert_within(Og, ref, bound, "O")
    assert rel_fro(Og, ref) <= (1e-2 if dtype == "bf16" or odt == "bf16" else 1e-5)


def test_shard_forward_sp_fused_and_literal(tpm):
    """Both variants deterministic; the same blocks up to float32 rounding of
    the shard sum."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    M, H, F, k = 512, 136, 2176, 8
    say("shard_forward_sp fused vs literal M=%d H=%d F=%d k=%d" % (M, H, F, k))
    inp = inputs.make_custom(M, H, F, "bf16", std=0.05, seed=21)
    Ws, bs, Vs = inputs.shard_slices(inp["W"], inp["b"], inp["V"], k)
    args = (to_dev(inp["X"]), [to_dev(w) for w in Ws], [to_dev(x) for x in bs], [to_dev(v) for v in Vs])
    O1 = tpm.tp_mlp_shard_forward_sp(*args, fused=False)
    O2 = tpm.tp_mlp_shard_forward_sp(*args, fused=True)
    O3 = tpm.tp_mlp_shard_forward_sp(*args, fused=False)
    O4 = tpm.tp_mlp_shard_forward_sp(*args, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O3) and torch.equal(O2, O4)
    assert rel_fro(from_dev(O2), from_dev(O1)) <= 1e-5


@pytest.mark.parametrize("name", ["tiny", "gpt2_small", "llama7b", "gpt3_175b", "long_seq"])
def test_workload_sp_sampled_rows(tpm, orc, name):
    """Full-size sequence-parallel forward in the benchmark's launch
    configuration; sampled rows of every rank's block against the oracle."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    w = inputs.WORKLOADS[name]
    say("workload sp %s M=%d H=%d F=%d k=%d" % (name, w.M, w.H, w.F, w.k))
    inp = inputs.make_inputs(w)
    X, W, b, V = inp["X"], inp["W"], inp["b"], inp["V"]
    Ws, bs, Vs = inputs.shard_slices(W, b, V, w.k)
    Xd = to_dev(X)
    O = tpm.tp_mlp_shard_forward_sp(Xd, [to_dev(x) for x in Ws], [to_dev(x) for x in bs],
                                    [to_dev(x) for x in Vs])
    torch.cuda.synchronize()
    Mb = w.M // w.k
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([r * Mb + rng.choice(Mb, min(2, Mb), replace=False) for r in range(w.k)]))
    Og = f64(from_dev(O[torch.from_numpy(rows).cuda()]))
    ref = orc.sp_forward_rows(X, W, b, V, w.k, rows)
    tol = 1e-2 if w.dtype == "bf16" else 1e-5
    assert rel_fro(Og, ref) <= tol
    # the residual is there: O - X is the MLP output, of a different scale than X
    assert rel_fro(Og - f64(X[rows]), ref - f64(X[rows])) <= tol
