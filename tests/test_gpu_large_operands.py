"""Operands past 4 GiB: one layer whose X and dZ (4.9 GB of bf16 each), Y_i
(4.9 GB) and float32 Z and partials (9.8 GB each) hold elements at byte
offsets past 2^31, 2^32 and 2^33, with a ragged M (a multiple of no tile),
through the forward (both variants) and the backward, against the CPU fp64
oracle.

The GEMMs address an operand from a 64-bit base that advances stage by
stage, with 32-bit offsets only inside one stage of one tile, and the
epilogues and the shard reduce index their outputs with 64-bit offsets;
here every one of them runs at sizes where a 32-bit byte offset into the
whole operand would wrap.  The layer is the column-parallel then
row-parallel MLP of "千亿参数模型如何拆分到多张GPU上训练" (张量并行, 方案一 and
方案二) with two shards.

Inputs: X, dZ ~ N(0, 1) and W, b, V ~ N(0, 0.02) from the seeded
counter-based generator of the input module, which draws any row on its own
from its counter offset, so the host regenerates the rows the oracle needs
instead of holding the whole operand.  Checked: Z on rows covering every
256-row block of the output plus the rows on both sides of each 2^31-,
2^32- and 2^33-byte boundary of X, Y_i and Z; the backward with a dZ that
is zero but on those boundary rows and one row of every 4096-row block: dX
on all M rows (exactly zero where dZ is) and dW, db and dV on sampled
columns.
"""
from types import SimpleNamespace

import numpy as np
import pytest

from _helpers import (U32, assert_within, backward_terms, check_forward_rows, f64, from_dev,
                      gemm_bound, rel_fro, say, tile_rows, to_dev)

pytestmark = pytest.mark.gpu

M, H, F, K_SHARDS = 600_037, 4096, 8192, 2
FK = F // K_SHARDS
STD = 0.02
SEED = 4242
CHUNK = 65536  # rows per host-generated chunk
TOL = 1e-2


def _boundary_rows():
    """The rows on both sides of every 2^31-, 2^32- and 2^33-byte boundary of
    X and dZ (bf16, H wide), Y_i (bf16, F/k wide) and Z and the partials
    (float32, H wide), and the last rows."""
    rows = {0, M - 2, M - 1}
    for row_bytes in (2 * H, 2 * FK, 4 * H):
        for p in (31, 32, 33):
            r = (1 << p) // row_bytes
            if r < M:
                rows.update({r - 1, r})
    return np.array(sorted(rows))


def _draw_dev(stream, cols, std):
    """The M x cols bf16 operand of `stream`, generated in chunks straight
    into device memory."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    out = torch.empty(M, cols, dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, CHUNK):
        r1 = min(M, r0 + CHUNK)
        out[r0:r1].copy_(to_dev(inputs.draw(stream, (r1 - r0, cols), std, "bf16", seed=SEED, first=r0 * cols)))
    return out


def _host_rows(stream, cols, std, rows):
    from tensor_transformer_mlp_amd import inputs
    return np.stack([inputs.draw(stream, (cols,), std, "bf16", seed=SEED, first=int(r) * cols) for r in rows])


def _params():
    from tensor_transformer_mlp_amd import inputs
    W = inputs.draw(inputs.STREAM_W, (H, F), STD, "bf16", seed=SEED)
    b = inputs.draw(inputs.STREAM_B, (F,), STD, "bf16", seed=SEED)
    V = inputs.draw(inputs.STREAM_V, (F, H), STD, "bf16", seed=SEED)
    return W, b, V


def _shards(W, b, V):
    Ws = [to_dev(np.ascontiguousarray(W[:, i * FK:(i + 1) * FK])) for i in range(K_SHARDS)]
    bs = [to_dev(np.ascontiguousarray(b[i * FK:(i + 1) * FK])) for i in range(K_SHARDS)]
    Vs = [to_dev(np.ascontiguousarray(V[i * FK:(i + 1) * FK])) for i in range(K_SHARDS)]
    return Ws, bs, Vs


@pytest.fixture(scope="module")
def xd():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_amd import inputs
    say("operands past 4 GiB: M=%d H=%d F=%d k=%d bf16, drawing X" % (M, H, F, K_SHARDS))
    X = _draw_dev(inputs.STREAM_X, H, 1.0)
    yield X
    del X
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_forward_operands_past_4gib(xd):
    import torch
    import tensor_transformer_mlp_amd as tpm
    from tensor_transformer_mlp_amd import inputs

    W, b, V = _params()
    Ws, bs, Vs = _shards(W, b, V)
    say("  forward literal, fused")
    Zl = tpm.tp_mlp_shard_forward(xd, Ws, bs, Vs, fused=False)
    Zf = tpm.tp_mlp_shard_forward(xd, Ws, bs, Vs, fused=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Zl).all()) and bool(torch.isfinite(Zf).all())
    rows = np.union1d(tile_rows(M, per_tile=1), _boundary_rows())
    rows_t = torch.from_numpy(rows).to("cuda")
    got = {"literal": (False, from_dev(Zl.index_select(0, rows_t))),
           "fused": (True, from_dev(Zf.index_select(0, rows_t)))}
    del Zl, Zf, rows_t
    torch.cuda.empty_cache()

    say("  oracle forward on %d rows" % rows.size)
    Xr = _host_rows(inputs.STREAM_X, H, 1.0, rows)
    pos = np.arange(rows.size)  # positions in Xr and in the gathered outputs
    variants = {lb: (fused, lambda rr, g=g: g[rr]) for lb, (fused, g) in got.items()}
    w = SimpleNamespace(k=K_SHARDS, H=H, dtype="bf16")
    errs = check_forward_rows("past 4 GiB", w, Xr, W, b, V, variants, pos)
    for lb, err in errs.items():
        say("  rel_fro over %d rows = %.3e (bar %.0e), %s" % (rows.size, err, TOL, lb))
        assert err <= TOL, lb


def _dz_rows():
    """The rows where the backward's dZ is drawn (zero elsewhere): the boundary
    rows and one row of every 4096-row block, at offsets that move through
    the blocks."""
    rows = set(int(r) for r in _boundary_rows())
    for t in range((M + 4095) // 4096):
        r = t * 4096 + (t * 97 + 13) % 4096
        if r < M:
            rows.add(r)
    return np.array(sorted(rows))


@pytest.mark.timeout(600)
def test_backward_operands_past_4gib(xd):
    """dZ is zero but for the rows R of _dz_rows(), so dY, dA and dX vanish
    exactly outside R and the parameter gradients, sums over all M rows, equal
    the oracle's sums over R exactly (a zero term adds nothing in float64),
    while every GEMM still walks all M rows.  Checked: dX is exactly zero on
    every row outside R, dX on R against the oracle, and dW, db and dV on
    sampled columns."""
    import torch
    import oracle
    import tensor_transformer_mlp_amd as tpm
    from tensor_transformer_mlp_amd import inputs

    W, b, V = _params()
    Ws, bs, Vs = _shards(W, b, V)
    rows = _dz_rows()
    rows_t = torch.from_numpy(rows).to("cuda")
    dZr = _host_rows(inputs.STREAM_DZ, H, 1.0, rows)
    say("  dZ on %d rows; backward literal, fused" % rows.size)
    dZd = torch.zeros(M, H, dtype=torch.bfloat16, device="cuda")
    dZd[rows_t] = to_dev(dZr)
    r1 = tpm.tp_mlp_shard_backward(xd, Ws, bs, Vs, dZd, fused=False)
    rf = tpm.tp_mlp_shard_backward(xd, Ws, bs, Vs, dZd, fused=True)
    torch.cuda.synchronize()
    same = all(torch.equal(a, c) for g1, g2 in zip(r1[1:], rf[1:]) for a, c in zip(g1, g2))
    assert same, "parameter gradients of the literal and fused variants differ"
    outside = torch.ones(M, dtype=torch.bool, device="cuda")
    outside[rows_t] = False
    for label, dX in (("literal", r1[0]), ("fused", rf[0])):
        nz = int(torch.count_nonzero(dX[outside]))
        assert nz == 0, "%s dX: %d nonzero elements on rows where dZ is zero" % (label, nz)
    cols = np.array([0, 1, FK - 1, FK, FK + 517, F - 1])
    dXr = from_dev(r1[0].index_select(0, rows_t)).astype(np.float64)
    dXfr = from_dev(rf[0].index_select(0, rows_t)).astype(np.float64)
    gW = np.stack([from_dev(r1[1][c // FK][:, c % FK]) for c in cols]).astype(np.float64)
    gb = np.array([from_dev(r1[2][c // FK][c % FK:c % FK + 1])[0] for c in cols], dtype=np.float64)
    gV = np.stack([from_dev(r1[3][c // FK][c % FK]) for c in cols]).astype(np.float64)
    del r1, rf, dZd, rows_t, outside
    torch.cuda.empty_cache()

    # dX on R: every shard's dA_i on those rows.
    say("  oracle dX on %d rows" % rows.size)
    Xr = _host_rows(inputs.STREAM_X, H, 1.0, rows)
    ref = oracle.backward_rows(Xr, W, b, V, dZr, K_SHARDS)
    bound = np.zeros_like(ref)
    boundf = np.zeros_like(ref)
    for i in range(K_SHARDS):
        sl = slice(i * FK, (i + 1) * FK)
        t = backward_terms(oracle, Xr, W[:, sl], b[sl], V[sl], dZr, "bf16")
        Wi64 = f64(W[:, sl])
        bound += gemm_bound(t["dA"], Wi64.T, FK, ea=t["errdA"])
        bound += (K_SHARDS + 2) * U32 * ((np.abs(t["dA"]) + t["errdA"]) @ np.abs(Wi64).T)
        boundf += gemm_bound(t["dA"], Wi64.T, F, ea=t["errdA"])
    assert_within(dXr, ref, bound, "past 4 GiB dX")
    assert_within(dXfr, ref, boundf, "past 4 GiB dX (fused)")
    for label, got in (("literal", dXr), ("fused", dXfr)):
        err = rel_fro(got, ref)
        say("  dX rel_fro on %d rows = %.3e (bar %.0e), %s" % (rows.size, err, TOL, label))
        assert err <= TOL

    # Parameter gradients on sampled columns: the GPU sums all M rows (M terms
    # in the float32 accumulation bound), the oracle the rows of R.
    say("  oracle dW, db, dV on %d columns" % cols.size)
    rW, rb, rV = oracle.backward_cols(Xr, W, b, V, dZr, cols)
    t = backward_terms(oracle, Xr, W[:, cols], b[cols], V[cols], dZr, "bf16")
    X64, dZ64 = f64(Xr), f64(dZr)
    bW = gemm_bound(t["dA"].T, X64, M, ea=t["errdA"].T)
    bb = t["errdA"].sum(axis=0) + 2 * (M + 2) * U32 * (np.abs(t["dA"]) + t["errdA"]).sum(axis=0) + 1e-30
    bV = gemm_bound(t["Y"].T, dZ64, M, ea=t["tolY"].T)
    assert_within(gW, rW, bW, "past 4 GiB dW columns")
    assert_within(gb, rb, bb, "past 4 GiB db")
    assert_within(gV, rV, bV, "past 4 GiB dV rows")
    for nm, g, r in (("dW", gW, rW), ("db", gb, rb), ("dV", gV, rV)):
        err = rel_fro(g, r)
        say("  %s rel_fro on sampled columns = %.3e" % (nm, err))
        assert err <= TOL
