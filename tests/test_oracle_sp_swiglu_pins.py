"""Pins for the oracle's sequence-parallel reduce-scatter and SwiGLU variant,
checked against things other than the oracle itself.

Sequence parallelism (the all-reduce as reduce-scatter + all-gather,
"大模型分布式训练四维并行：DDP、ZeRO、张量、流水线与上下文" §2.1; the sequence split of
the block's non-TP region, "AI大模型分布式训练：张量并行与流水线并行深度实践" §4.2; the
residual x + mlp(x) of the TransformerBlock, §3.4 of the same page):
* a hand-worked split of small integers (rank r gets rows [r M/k, (r+1) M/k),
  the residual is added once);
* the all-gather of the blocks equals the residual plus the all-reduce of the
  parts (the ring identity), against the separately pinned shard_reduce;
* residual-only and residual-free cases; row locality (a block depends on its
  own rows only); k = 1 and one row per rank;
* the whole sequence-parallel forward against X + the pinned forward, and the
  gathered result is the same for every k.

SwiGLU (gate/up column-parallel, down row-parallel: §6.1 of the page above;
"大模型分布式优化技术（一）" §5.1 and §3.3), Y_i = SiLU(X Wg_i) * (X Wu_i):
* SiLU closed forms: SiLU(0) = 0, SiLU(x) - SiLU(-x) = x, sigma(+-1), the
  asymptotes, the minimum at x = -1 - W(1/e) with value -W(1/e) (Lambert W),
  and a 50-digit grid;
* exact rational brute force on tiny dyadic inputs with 50-digit exp;
* a one-element case that tells gate from up;
* the column-split and row-split identities, k-invariance, zero gate / zero
  up / zero V, and an independent numpy float64 implementation.
"""
import random
from fractions import Fraction

import mpmath
import numpy as np
import pytest

mpmath.mp.dps = 50


# ---------------------------------------------------------------------------
# Sequence-parallel reduce-scatter with the residual.

def test_sp_hand_worked(oracle_mod):
    P0 = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=np.float64)
    P1 = 10 * P0
    R = 100 * P0
    out = oracle_mod.sp_reduce_scatter([P0, P1], R, 2)
    assert len(out) == 2
    np.testing.assert_array_equal(out[0], [[111, 222], [333, 444]])
    np.testing.assert_array_equal(out[1], [[555, 666], [777, 888]])
    # four ranks: one row each
    out4 = oracle_mod.sp_reduce_scatter([P0, P1], R, 4)
    for r in range(4):
        np.testing.assert_array_equal(out4[r], [[111 * (2 * r + 1), 222 * (r + 1)]])
    # without the residual
    out_nr = oracle_mod.sp_reduce_scatter([P0, P1], None, 2)
    np.testing.assert_array_equal(out_nr[1], [[55, 66], [77, 88]])


@pytest.mark.parametrize("M,H,k,nparts,seed", [(8, 16, 2, 2, 0), (12, 8, 4, 4, 1), (16, 24, 8, 8, 2),
                                               (6, 5, 3, 1, 3), (9, 7, 1, 3, 4), (5, 3, 5, 2, 5)])
def test_sp_gather_is_residual_plus_allreduce(oracle_mod, M, H, k, nparts, seed):
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal((M, H)) for _ in range(nparts)]
    R = rng.standard_normal((M, H))
    blocks = oracle_mod.sp_reduce_scatter(parts, R, k)
    assert [b.shape for b in blocks] == [(M // k, H)] * k
    gathered = np.concatenate(blocks, axis=0)
    # same summation order as the all-reduce, then one addition of R
    np.testing.assert_array_equal(gathered, R + oracle_mod.shard_reduce(parts))
    # residual-free blocks are the all-reduce's row blocks
    free = np.concatenate(oracle_mod.sp_reduce_scatter(parts, None, k), axis=0)
    np.testing.assert_array_equal(free, oracle_mod.shard_reduce(parts))
    # residual only
    zeros = [np.zeros((M, H)) for _ in range(nparts)]
    np.testing.assert_array_equal(np.concatenate(oracle_mod.sp_reduce_scatter(zeros, R, k), axis=0), R)


def test_sp_small_integers_exact(oracle_mod):
    rng = random.Random(7)
    M, H, k, n = 6, 4, 3, 3
    parts = [[[rng.randint(-50, 50) for _ in range(H)] for _ in range(M)] for _ in range(n)]
    R = [[rng.randint(-50, 50) for _ in range(H)] for _ in range(M)]
    blocks = oracle_mod.sp_reduce_scatter([np.array(p, dtype=np.float64) for p in parts],
                                          np.array(R, dtype=np.float64), k)
    Mb = M // k
    for r in range(k):
        for m in range(Mb):
            for c in range(H):
                row = r * Mb + m
                assert blocks[r][m, c] == R[row][c] + sum(p[row][c] for p in parts)


def test_sp_row_locality(oracle_mod):
    rng = np.random.default_rng(11)
    M, H, k = 12, 6, 3
    parts = [rng.standard_normal((M, H)) for _ in range(2)]
    R = rng.standard_normal((M, H))
    base = oracle_mod.sp_reduce_scatter(parts, R, k)
    Mb = M // k
    for r in range(k):
        # change every row outside block r: block r is unchanged
        p2 = [p.copy() for p in parts]
        R2 = R.copy()
        outside = [m for m in range(M) if not r * Mb <= m < (r + 1) * Mb]
        for p in p2:
            p[outside] += 3.0
        R2[outside] -= 5.0
        np.testing.assert_array_equal(oracle_mod.sp_reduce_scatter(p2, R2, k)[r], base[r])
        # change one row inside: only that row of block r moves
        p3 = [p.copy() for p in parts]
        p3[1][r * Mb + 1] += 1.0
        got = oracle_mod.sp_reduce_scatter(p3, R, k)[r]
        diff = np.nonzero(np.any(got != base[r], axis=1))[0]
        assert diff.tolist() == [1]


def test_sp_rejects_ragged_split(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.sp_reduce_scatter([np.zeros((6, 2))], None, 4)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_sp_forward_is_residual_plus_forward(oracle_mod, k):
    rng = np.random.default_rng(20 + k)
    M, H, F = 8, 16, 32
    X = rng.standard_normal((M, H))
    W = rng.standard_normal((H, F)) * 0.3
    b = rng.standard_normal(F) * 0.1
    V = rng.standard_normal((F, H)) * 0.3
    blocks = oracle_mod.sp_forward(X, W, b, V, k)
    g = np.concatenate(blocks, axis=0)
    ref = X + oracle_mod.forward(X, W, b, V, 1)
    assert np.max(np.abs(g - ref)) <= 1e-13 * np.max(np.abs(ref))
    # rows version (any rows, in the gathered index space)
    rows = [7, 0, 3]
    np.testing.assert_allclose(oracle_mod.sp_forward_rows(X, W, b, V, k, rows), g[rows], rtol=0, atol=1e-13)
    # V = 0: the block output is the residual alone
    g0 = np.concatenate(oracle_mod.sp_forward(X, W, b, np.zeros_like(V), k), axis=0)
    np.testing.assert_array_equal(g0, X)


# ---------------------------------------------------------------------------
# SwiGLU.

def test_silu_closed_form(oracle_mod):
    s = oracle_mod.silu_scalar
    assert s(0.0) == 0.0
    assert abs(s(1.0) - 0.7310585786300049) <= 2e-16       # sigma(1)
    assert abs(s(-1.0) - (-0.2689414213699951)) <= 2e-16   # -sigma(-1)
    for x in np.linspace(-30, 30, 301):
        # sigma(x) + sigma(-x) = 1
        assert abs((s(x) - s(-x)) - x) <= 4e-16 * max(1.0, abs(x))
    assert s(800.0) == 800.0
    assert s(-800.0) == 0.0
    # minimum: d/dx x sigma(x) = 0 at x* = -1 - W(1/e), with value -W(1/e)
    w = float(mpmath.lambertw(1 / mpmath.e).real)
    xstar = -1.0 - w
    assert abs(s(xstar) - (-w)) <= 2e-16
    assert s(xstar - 1e-4) > s(xstar) and s(xstar + 1e-4) > s(xstar)
    xs = np.linspace(-1.4, -1.1, 30001)
    assert abs(xs[int(np.argmin(oracle_mod.silu(xs)))] - xstar) < 2e-5
    # 50-digit grid
    grid = np.concatenate([np.linspace(-40, 40, 1601), [1e-300, -1e-300, 1e-9, -1e-9]])
    for x, y in zip(grid, oracle_mod.silu(grid)):
        xm = mpmath.mpf(float(x))
        ref = xm / (1 + mpmath.exp(-xm))
        assert abs(y - float(ref)) <= 4e-16 * abs(float(ref)) * (1 + abs(float(x))) + 1e-320, x


def _dyadic(rng, shape, num_range, denom):
    return [[Fraction(rng.randint(-num_range, num_range), denom) for _ in range(shape[1])]
            for _ in range(shape[0])]


def _np(a):
    return np.array([[float(x) for x in r] for r in a])


def _mp(f):
    return mpmath.mpf(f.numerator) / f.denominator


@pytest.mark.parametrize("M,H,F,k,seed", [(1, 1, 1, 1, 0), (2, 3, 4, 2, 1), (3, 5, 12, 3, 2),
                                          (4, 8, 16, 4, 3), (2, 4, 8, 1, 4)])
def test_swiglu_brute_force_tiny(oracle_mod, M, H, F, k, seed):
    rng = random.Random(100 + seed)
    X = _dyadic(rng, (M, H), 12, 4)
    Wg = _dyadic(rng, (H, F), 8, 8)
    Wu = _dyadic(rng, (H, F), 8, 8)
    V = _dyadic(rng, (F, H), 16, 16)
    Fk = F // k
    Y = [[None] * F for _ in range(M)]
    for m in range(M):
        for c in range(F):
            g = sum((X[m][h] * Wg[h][c] for h in range(H)), Fraction(0))
            u = sum((X[m][h] * Wu[h][c] for h in range(H)), Fraction(0))
            gm = _mp(g)
            Y[m][c] = gm / (1 + mpmath.exp(-gm)) * _mp(u)
    Xn, Wgn, Wun, Vn = map(_np, (X, Wg, Wu, V))
    for i in range(k):
        Yo = oracle_mod.swiglu_col(Xn, Wgn, Wun, k, i)
        for m in range(M):
            for j in range(Fk):
                ref = float(Y[m][i * Fk + j])
                assert abs(Yo[m, j] - ref) <= 1e-14 * abs(ref) + 1e-300, (i, m, j)
    Zo = oracle_mod.swiglu_forward(Xn, Wgn, Wun, Vn, k)
    absY = np.abs(np.array([[float(v) for v in r] for r in Y]))
    scale = absY @ np.abs(Vn)
    for m in range(M):
        for n in range(H):
            ref = sum((Y[m][c] * _mp(V[c][n]) for c in range(F)), mpmath.mpf(0))
            assert abs(Zo[m, n] - float(ref)) <= 1e-14 * scale[m, n] + 1e-300, (m, n)


def test_swiglu_gate_and_up_are_not_interchangeable(oracle_mod):
    X = np.array([[1.0]])
    Wg = np.array([[2.0]])
    Wu = np.array([[3.0]])
    V = np.array([[1.0]])
    y = oracle_mod.swiglu_col(X, Wg, Wu, 1, 0)[0, 0]
    assert abs(y - 3 * 2 / (1 + np.exp(-2.0))) <= 1e-15 * 6      # SiLU(2) * 3 = 5.2847...
    assert abs(y - 2 * 3 / (1 + np.exp(-3.0))) > 0.4              # not SiLU(3) * 2 = 5.7153...
    assert oracle_mod.swiglu_forward(X, Wg, Wu, V, 1)[0, 0] == y


@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_splits_and_k_invariance(oracle_mod, seed):
    rng = np.random.default_rng(300 + seed)
    M, H, F = 6, 16, 32
    X = rng.standard_normal((M, H))
    Wg = rng.standard_normal((H, F)) * 0.3
    Wu = rng.standard_normal((H, F)) * 0.3
    V = rng.standard_normal((F, H)) * 0.3
    Yfull = oracle_mod.swiglu_col(X, Wg, Wu, 1, 0)
    Zs = {}
    for k in (1, 2, 4, 8):
        # column split: the shards side by side are the unsplit Y, bit for bit
        Ycat = np.concatenate([oracle_mod.swiglu_col(X, Wg, Wu, k, i) for i in range(k)], axis=1)
        np.testing.assert_array_equal(Ycat, Yfull)
        Zs[k] = oracle_mod.swiglu_forward(X, Wg, Wu, V, k)
    # row split: sum_i Y_i V_i = Y V
    ref = Yfull @ V
    scale = np.abs(Yfull) @ np.abs(V)
    for k, Z in Zs.items():
        assert np.all(np.abs(Z - ref) <= 1e-14 * scale + 1e-300), k
    # independent float64 implementation
    A, U = X @ Wg, X @ Wu
    Znp = (A / (1.0 + np.exp(-A)) * U) @ V
    assert np.all(np.abs(Zs[4] - Znp) <= 1e-13 * scale + 1e-300)
    # rows version
    np.testing.assert_array_equal(oracle_mod.swiglu_forward_rows(X, Wg, Wu, V, 4, [5, 1]), Zs[4][[5, 1]])


def test_swiglu_special_cases(oracle_mod):
    rng = np.random.default_rng(9)
    M, H, F = 4, 8, 16
    X = rng.standard_normal((M, H))
    Wg = rng.standard_normal((H, F))
    Wu = rng.standard_normal((H, F))
    V = rng.standard_normal((F, H))
    assert np.all(oracle_mod.swiglu_forward(X, Wg, np.zeros_like(Wu), V, 2) == 0)   # up = 0
    assert np.all(oracle_mod.swiglu_forward(X, np.zeros_like(Wg), Wu, V, 2) == 0)   # SiLU(0) = 0
    assert np.all(oracle_mod.swiglu_forward(X, Wg, Wu, np.zeros_like(V), 2) == 0)
    # a large positive gate passes the up projection through: SiLU(g) = g
    Y = oracle_mod.swiglu_col(np.ones((1, 1)), np.full((1, 2), 50.0), np.array([[2.0, -3.0]]), 1, 0)
    np.testing.assert_array_equal(Y, [[100.0, -150.0]])
