"""GPU checks of the batched (*_shards) entry points: a batch of n shards in one
launch gives bit-identical results to n single-shard calls, and the
shard-order sum (TP_SUM_SHARDS) is bit-identical to the materialised partials
followed by tp_shard_reduce.  Covers grouped tiles, ragged shapes, the
ragged-K variant, both dtypes and the sequential path taken by very large
sums; the single-shard calls themselves are checked against the oracle in
test_gpu_parity_small.py and test_gpu_backward.py.
"""
import numpy as np
import pytest

from _helpers import say, to_dev

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
    assert torch.equal(Zr, Zs), "shard-order sum differs from partials + reduce"


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
    assert torch.equal(dXr, dXs)


def test_sum_shards_accumulate_continues_the_order(tpm):
    """Two batches, the second with TP_ACCUMULATE, equal one left-to-right sum."""
    import torch
    M, H, Fk, n = 300, 136, 264, 6
    say("sum across two batches")
    Y = [_draw(0, (M, Fk), 0.5, "bf16", 80 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, "bf16", 90 + i) for i in range(n)]
    Z = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y[:4], V[:4], [Z], sum_shards=True)
    tpm.tp_mlp_row_partial_shards(Y[4:], V[4:], [Z], sum_shards=True, accumulate=True)
    P = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Y, V, P)
    Zr = tpm.tp_shard_reduce(P)
    torch.cuda.synchronize()
    assert torch.equal(Z, Zr)


@pytest.mark.timeout(300)
def test_large_sum_sequential_path(tpm):
    """A sum whose per-shard GEMM fills the chip many times over runs shard by
    shard with the 256x256 tile; still bit-identical to partials + reduce."""
    import torch
    M, H, Fk, n = 16384, 4096, 512, 2
    say("large sequential sum M=%d H=%d" % (M, H))
    Y = [_draw(0, (M, Fk), 0.5, "bf16", 100 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, "bf16", 110 + i) for i in range(n)]
    Z = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y, V, [Z], sum_shards=True)
    P = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Y, V, P)
    Zr = tpm.tp_shard_reduce(P)
    torch.cuda.synchronize()
    assert torch.equal(Z, Zr)
