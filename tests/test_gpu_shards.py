"""GPU checks of the batched (*_shards) entry points: a batch of n shards in one
launch gives bit-identical results to n single-shard calls; the shard sum
(TP_SUM_SHARDS) is the unsplit GEMM of the shards side by side, [Y_0 ...
Y_{n-1}] [V_0; ...; V_{n-1}] (the row-parallel identity of "千亿参数模型如何拆分到多张
GPU上训练", 方案二): in bf16 with Fk a multiple of 32 it equals the single GEMM over
the concatenated operands bit for bit, it agrees with the materialised
partials followed by tp_shard_reduce within the float32 accumulation bound,
and a batch split over several calls (TP_ACCUMULATE) gives the same bits as
one call.  In float32 the sum runs shard by shard and equals partials +
reduce bit for bit.  Covers grouped tiles, ragged shapes, the ragged-K
variant and both dtypes; the single-shard calls themselves are checked
against the oracle in test_gpu_parity_small.py and test_gpu_backward.py.
"""
import numpy as np
import pytest

from _helpers import U32, assert_within, f64, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_transformer_mlp_amd as tpm
    tpm.lib()
    return tpm


def _draw(stream, shape, std, dtype, seed):
    from tensor_transformer_mlp_amd import inputs
    return to_dev(inputs.draw(stream, shape, std, dtype, seed=seed))


CASES = [(257, 200, 136, 3, "bf16"), (512, 256, 384, 4, "bf16"), (8192, 768, 768, 4, "bf16"),
         (300, 72, 40, 5, "bf16"), (65, 136, 200, 3, "f32"), (1, 64, 128, 2, "bf16")]


@pytest.mark.parametrize("M,H,Fk,n,dtype", CASES)
def test_forward_shards_bitwise(tpm, M, H, Fk, n, dtype):
    import torch
    say("forward shards M=%d H=%d Fk=%d n=%d %s" % (M, H, Fk, n, dtype))
    X = _draw(0, (M, H), 1.0, dtype, M)
    W = [_draw(1, (H, Fk), 0.05, dtype, 10 + i) for i in range(n)]
    b = [_draw(2, (Fk,), 0.05, dtype, 20 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, dtype, 30 + i) for i in range(n)]
    tdt = X.dtype
    Yb = [torch.empty(M, Fk, dtype=tdt, device="cuda") for _ in range(n)]
    Gb = [torch.empty(M, Fk, dtype=tdt, device="cuda") for _ in range(n)]
    tpm.tp_mlp_col_gelu_shards(X, W, b, Yb, Gb)
    Yb2 = [torch.empty(M, Fk, dtype=tdt, device="cuda") for _ in range(n)]
    tpm.tp_mlp_col_gelu_shards(X, W, b, Yb2)
    Pb = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Yb, V, Pb)
    Zs = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Yb, V, [Zs], sum_shards=True)
    torch.cuda.synchronize()
    for i in range(n):
        Y1, G1 = tpm.tp_mlp_col_gelu_save(X, W[i], b[i])
        P1 = tpm.tp_mlp_row_partial(Yb[i], V[i])
        torch.cuda.synchronize()
        assert torch.equal(Y1, Yb[i]) and torch.equal(G1, Gb[i]) and torch.equal(Y1, Yb2[i]), i
        assert torch.equal(P1, Pb[i]), i
    Zr = tpm.tp_shard_reduce(Pb)
    torch.cuda.synchronize()
    _check_sum(tpm, torch, Zs, Zr, Yb, V, dtype, Fk, transposed=False)


@pytest.mark.parametrize("M,H,Fk,n,dtype", CASES)
def test_backward_shards_bitwise(tpm, M, H, Fk, n, dtype):
    import torch
    say("backward shards M=%d H=%d Fk=%d n=%d %s" % (M, H, Fk, n, dtype))
    X = _draw(0, (M, H), 1.0, dtype, M + 1)
    dZ = _draw(4, (M, H), 1.0, dtype, M + 2)
    V = [_draw(3, (Fk, H), 0.05, dtype, 40 + i) for i in range(n)]
    W = [_draw(1, (H, Fk), 0.05, dtype, 50 + i) for i in range(n)]
    G = [_draw(0, (M, Fk), 0.6, dtype, 60 + i) for i in range(n)]
    Y = [_draw(0, (M, Fk), 0.5, dtype, 70 + i) for i in range(n)]
    dA = [torch.empty_like(G[0]) for _ in range(n)]
    tpm.tp_mlp_grad_act_shards(dZ, V, G, dA)
    dV = [torch.empty(Fk, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_grad_row_weight_shards(Y, dZ, dV)
    dW = [torch.empty(H, Fk, device="cuda") for _ in range(n)]
    db = [torch.empty(Fk, device="cuda") for _ in range(n)]
    tpm.tp_mlp_grad_col_weight_shards(X, dA, dW, db)
    dXp = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_grad_input_shards(dA, W, dXp)
    dXs = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_grad_input_shards(dA, W, [dXs], sum_shards=True)
    torch.cuda.synchronize()
    for i in range(n):
        a1 = tpm.tp_mlp_grad_act(dZ, V[i], G[i])
        v1 = tpm.tp_mlp_grad_row_weight(Y[i], dZ)
        w1, b1 = tpm.tp_mlp_grad_col_weight(X, dA[i])
        x1 = tpm.tp_mlp_grad_input_partial(dA[i], W[i])
        torch.cuda.synchronize()
        assert torch.equal(a1, dA[i]), ("dA", i)
        assert torch.equal(w1, dW[i]) and torch.equal(b1, db[i]), ("dW/db", i)
        assert torch.equal(x1, dXp[i]), ("dX", i)
        assert torch.equal(v1, dV[i]), ("dV", i)
    dXr = tpm.tp_shard_reduce(dXp)
    torch.cuda.synchronize()
    _check_sum(tpm, torch, dXs, dXr, dA, W, dtype, Fk, transposed=True)


def _check_sum(tpm, torch, Zs, Zr, A, B, dtype, Fk, transposed):
    """Zs: the shard sum of A_i B_i (B_i^T when transposed); Zr: partials +
    tp_shard_reduce.  float32: equal bit for bit.  bf16: within the float32
    accumulation bound of both orders, and, when Fk is a multiple of 32, equal
    bit for bit to one GEMM over the concatenated operands."""
    if dtype == "f32":
        assert torch.equal(Zs, Zr), "float32 shard sum differs from partials + reduce"
        return
    n = len(A)
    Acat = torch.cat(A, dim=1).contiguous()
    Bcat = torch.cat(B, dim=1 if transposed else 0).contiguous()
    a64 = np.abs(f64(from_dev(Acat)))
    b64 = np.abs(f64(from_dev(Bcat)))
    mag = a64 @ (b64.T if transposed else b64)
    bound = 2 * (n * Fk + n + 4) * U32 * 2 * mag + 1e-30
    assert_within(f64(from_dev(Zs)), f64(from_dev(Zr)), bound, "shard sum vs partials + reduce")
    if Fk % 32 == 0:
        Zu = (tpm.tp_mlp_grad_input_partial(Acat, Bcat) if transposed else tpm.tp_mlp_row_partial(Acat, Bcat))
        torch.cuda.synchronize()
        assert torch.equal(Zs, Zu), "shard sum differs from the GEMM over the concatenated shards"


def test_sum_shards_accumulate_continues_the_order(tpm):
    """Two batches, the second with TP_ACCUMULATE, give the bits of one batch
    (the accumulator of the second starts at the first's float32 result),
    and agree with partials + reduce within the accumulation bound."""
    import torch
    M, H, Fk, n = 300, 136, 264, 6
    say("sum across two batches")
    Y = [_draw(0, (M, Fk), 0.5, "bf16", 80 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, "bf16", 90 + i) for i in range(n)]
    Z = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y[:4], V[:4], [Z], sum_shards=True)
    tpm.tp_mlp_row_partial_shards(Y[4:], V[4:], [Z], sum_shards=True, accumulate=True)
    Z1 = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y, V, [Z1], sum_shards=True)
    P = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Y, V, P)
    Zr = tpm.tp_shard_reduce(P)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z1)
    _check_sum(tpm, torch, Z, Zr, Y, V, "bf16", Fk, transposed=False)


@pytest.mark.timeout(300)
def test_large_sum(tpm):
    """A sum whose output fills the chip many times over (256 x 256 tiles, K
    through both shards) equals the GEMM over the concatenated shards bit for
    bit, and partials + reduce within the accumulation bound."""
    import torch
    M, H, Fk, n = 16384, 4096, 512, 2
    say("large sum M=%d H=%d" % (M, H))
    Y = [_draw(0, (M, Fk), 0.5, "bf16", 100 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, "bf16", 110 + i) for i in range(n)]
    Z = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y, V, [Z], sum_shards=True)
    P = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Y, V, P)
    Zr = tpm.tp_shard_reduce(P)
    torch.cuda.synchronize()
    _check_sum(tpm, torch, Z, Zr, Y, V, "bf16", Fk, transposed=False)
