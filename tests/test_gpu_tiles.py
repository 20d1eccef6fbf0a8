"""GPU checks of the tile table hooks: the column step, the row step and the
row step with the shard sum give the same results, bit for bit, with every
tile of the bf16 GEMM's table that can run them (each output element is
accumulated over K in the same order whatever the tile), and tiles that are
not compiled for a step are refused.  The default path itself is checked
against the oracle in test_gpu_parity_small.py and test_gpu_workloads.py.
"""
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


def _draw(stream, shape, std, seed):
    from tensor_transformer_mlp_amd import inputs
    return to_dev(inputs.draw(stream, shape, std, "bf16", seed=seed))


# (M, H, Fk, n): gpt2_small's four shards, ragged M over several tiles, and
# K = H = 200 (only the ragged-K tile runs the column step; the row step's
# K = Fk = 136 likewise)
CASES = [(8192, 768, 768, 4), (1000, 768, 512, 2), (513, 256, 384, 3), (300, 200, 136, 2)]


@pytest.mark.parametrize("M,H,Fk,n", CASES)
def test_every_tile_bitwise(tpm, M, H, Fk, n):
    import torch
    say("tiles M=%d H=%d Fk=%d n=%d" % (M, H, Fk, n))
    X = _draw(0, (M, H), 1.0, M)
    W = [_draw(1, (H, Fk), 0.05, 10 + i) for i in range(n)]
    b = [_draw(2, (Fk,), 0.05, 20 + i) for i in range(n)]
    V = [_draw(3, (Fk, H), 0.05, 30 + i) for i in range(n)]
    Y0 = [torch.empty(M, Fk, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tpm.tp_mlp_col_gelu_shards(X, W, b, Y0)
    P0 = [torch.empty(M, H, device="cuda") for _ in range(n)]
    tpm.tp_mlp_row_partial_shards(Y0, V, P0)
    S0 = torch.empty(M, H, device="cuda")
    tpm.tp_mlp_row_partial_shards(Y0, V, [S0], sum_shards=True)
    torch.cuda.synchronize()
    ran = {"col": [], "row": [], "sum": []}
    for t, shape in enumerate(tpm.tp_gemm_tiles()):
        Y = [torch.full((M, Fk), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        try:
            tpm.tp_mlp_col_gelu_shards_tile(t, X, W, b, Y)
            torch.cuda.synchronize()
            assert all(torch.equal(Y[i], Y0[i]) for i in range(n)), ("col", t, shape)
            ran["col"].append(t)
        except tpm.TpMlpError as e:
            assert e.code == -2 and H % 32, (t, e)
        P = [torch.full((M, H), float("nan"), device="cuda") for _ in range(n)]
        try:
            tpm.tp_mlp_row_partial_shards_tile(t, Y0, V, P)
            torch.cuda.synchronize()
            assert all(torch.equal(P[i], P0[i]) for i in range(n)), ("row", t, shape)
            ran["row"].append(t)
        except tpm.TpMlpError as e:
            assert e.code == -2 and Fk % 32, (t, e)
        S = torch.full((M, H), float("nan"), device="cuda")
        try:
            tpm.tp_mlp_row_partial_shards_tile(t, Y0, V, [S], sum_shards=True)
            torch.cuda.synchronize()
            assert torch.equal(S, S0), ("sum", t, shape)
            ran["sum"].append(t)
        except tpm.TpMlpError as e:
            assert e.code == -2 and Fk % 32, (t, e)
    say("  ran col %s row %s sum %s" % (ran["col"], ran["row"], ran["sum"]))
    # every tile runs an aligned K; the ragged-K variant exists for one tile
    count = len(tpm.tp_gemm_tiles())
    assert len(ran["col"]) == (count if H % 32 == 0 else 1)
    assert len(ran["row"]) == (count if Fk % 32 == 0 else 1)
    assert tpm.tp_mlp_step_tile(0, n, M, H, Fk) in ran["col"]
    assert tpm.tp_mlp_step_tile(1, n, M, H, Fk) in ran["row"]
    assert tpm.tp_mlp_step_tile(2, n, M, H, Fk) in ran["sum"]
