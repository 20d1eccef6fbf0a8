"""GPU parity of the block forward at seeded random shapes (M any size, H and
F/k any multiple of 8, 1 to 6 shards, both element types), literal and fused:
every output element within the oracle's bound, the relative Frobenius bar,
and the two variants bit-identical.  The shapes land on every mix of whole
and partial tiles in M, N and K that the fixed cases do not name one by one.
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
    assert torch.equal(Zl, Zf), "fused and literal forward differ"
    Zg = f64(from_dev(Zl))
    assert np.all(np.isfinite(Zg))
    Zr = orc.forward(X, W, b, V, k)
    X64, W64, b64, V64 = f64(X), f64(W), f64(b), f64(V)
    A = np.concatenate([orc.col_preact(X, W, b, k, i) for i in range(k)], axis=1)
    Y = np.concatenate([orc.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
    tolY = np.concatenate([col_bound(X64, W64[:, i * Fk:(i + 1) * Fk], b64[i * Fk:(i + 1) * Fk],
                                     A[:, i * Fk:(i + 1) * Fk], Y[:, i * Fk:(i + 1) * Fk], dtype)
                           for i in range(k)], axis=1)
    assert_within(Zg, Zr, forward_bound(tolY, Y, V64, k), "Z")
    assert rel_fro(Zg, Zr) <= (1e-2 if dtype == "bf16" else 1e-5)
