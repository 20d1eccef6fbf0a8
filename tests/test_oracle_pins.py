"""Pins for the CPU fp64 oracle, checked against things other than itself.

* Brute force on tiny inputs: dyadic X, W, b, V make every GEMM sum exact in
  rational arithmetic (fractions.Fraction); GeLU is evaluated at 50 digits with
  mpmath.  A dropped bias, a sign error, a transposed operand, a wrong shard
  offset or the tanh GeLU approximation all fail these.
* The column-split identity [X W_0 | ... | X W_{k-1}] = X W and the row-split
  identity sum_i Y_i V_i = [Y_0 ... Y_{k-1}] V (the column and row splits of
  "千亿参数模型如何拆分到多张GPU上训练", 张量并行 section; "大模型分布式并行策略详解：
  TP、DP、PP、CP、EP核心原理与实战" §4.1).
* GeLU's closed form: GeLU(x) = x Phi(x), GeLU(0) = 0, GeLU(x) - GeLU(-x) = x,
  GeLU(+-1) from the standard normal CDF, the asymptotes.
* Special cases that reduce to library routines (W = 0, X = 0, V = 0) and a
  cross-check against numpy float64 matmul with math.erf.
* Structural invariants: row independence, exact scaling by 2.
"""
import math
import random
from fractions import Fraction

import mpmath
import numpy as np
import pytest

mpmath.mp.dps = 50


def _exact_forward(X, W, b, V, k):
    """Exact-rational GEMMs, 50-digit GeLU; returns (Y blocks, Z) as mpf."""
    M, H = len(X), len(X[0])
    F = len(W[0])
    Fk = F // k
    Z = [[mpmath.mpf(0)] * H for _ in range(M)]
    Ys = []
    for i in range(k):
        Yi = []
        for m in range(M):
            row = []
            for j in range(Fk):
                col = i * Fk + j
                a = sum((X[m][h] * W[h][col] for h in range(H)), Fraction(0)) + b[col]
                a = mpmath.mpf(a.numerator) / a.denominator
                row.append(a * (1 + mpmath.erf(a / mpmath.sqrt(2))) / 2)
            Yi.append(row)
        Ys.append(Yi)
        for m in range(M):
            for n in range(H):
                s = mpmath.mpf(0)
                for j in range(Fk):
                    vj = V[i * Fk + j][n]
                    s += Yi[m][j] * (mpmath.mpf(vj.numerator) / vj.denominator)
                Z[m][n] += s
    return Ys, Z


def _dyadic(rng, shape, num_range, denom):
    if len(shape) == 1:
        return [Fraction(rng.randint(-num_range, num_range), denom) for _ in range(shape[0])]
    return [[Fraction(rng.randint(-num_range, num_range), denom) for _ in range(shape[1])]
            for _ in range(shape[0])]


def _to_np(a):
    return np.array([[float(x) for x in r] for r in a]) if isinstance(a[0], list) else \
        np.array([float(x) for x in a])


@pytest.mark.parametrize("M,H,F,k,seed", [(1, 1, 1, 1, 0), (2, 3, 4, 2, 1), (3, 5, 12, 3, 2),
                                          (4, 8, 16, 4, 3), (2, 7, 6, 6, 4), (4, 4, 16, 1, 5)])
def test_brute_force_tiny(oracle_mod, M, H, F, k, seed):
    rng = random.Random(seed)
    X = _dyadic(rng, (M, H), 12, 4)      # values in [-3, 3]
    W = _dyadic(rng, (H, F), 8, 8)
    b = _dyadic(rng, (F,), 8, 8)
    V = _dyadic(rng, (F, H), 16, 16)
    Ys, Zx = _exact_forward(X, W, b, V, k)
    Xn, Wn, bn, Vn = map(_to_np, (X, W, b, V))
    # per-shard column step
    for i in range(k):
        Yo = oracle_mod.col_gelu(Xn, Wn, bn, k, i)
        for m in range(M):
            for j in range(F // k):
                ref = Ys[i][m][j]
                # relative error grows with the conditioning of Phi at negative x (~x^2)
                assert abs(Yo[m, j] - float(ref)) <= 1e-14 * abs(float(ref)) + 1e-300, (i, m, j)
        # row step from the exact Y_i (rounded once to double)
        Yi = np.array([[float(v) for v in r] for r in Ys[i]])
        Zi = oracle_mod.row_partial(Yi, Vn, k, i)
        assert Zi.shape == (M, H)
    Zo = oracle_mod.forward(Xn, Wn, bn, Vn, k)
    scale = np.abs(np.concatenate([np.array([[float(v) for v in r] for r in Y]) for Y in Ys], axis=1)) @ np.abs(Vn)
    for m in range(M):
        for n in range(H):
            assert abs(Zo[m, n] - float(Zx[m][n])) <= 1e-14 * scale[m, n] + 1e-300, (m, n)


def test_brute_force_catches_tanh_gelu(oracle_mod):
    """The tanh approximation of GeLU differs from erf-GeLU by ~1e-4 here; the
    oracle must match erf-GeLU to 1e-15, so it cannot be the tanh form."""
    xs = [-3.0, -1.5, -0.75, 0.5, 1.25, 2.5]
    for x in xs:
        exact = mpmath.mpf(x) * (1 + mpmath.erf(mpmath.mpf(x) / mpmath.sqrt(2))) / 2
        tanh_form = 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
        got = oracle_mod.gelu_scalar(x)
        assert abs(got - float(exact)) <= 4e-16 * (2 + x * x) * abs(float(exact))
        assert abs(tanh_form - float(exact)) > 1e-6 or abs(x) < 0.1


def test_gelu_closed_form(oracle_mod):
    g = oracle_mod.gelu_scalar
    assert g(0.0) == 0.0
    # Phi(1) and Phi(-1) from the standard normal distribution
    assert abs(g(1.0) - 0.8413447460685429) <= 2e-16
    assert abs(g(-1.0) - (-0.15865525393145707)) <= 2e-16
    # GeLU(x) - GeLU(-x) = x since Phi(x) + Phi(-x) = 1
    for x in np.linspace(-8, 8, 161):
        assert abs((g(x) - g(-x)) - x) <= 4e-16 * max(1.0, abs(x))
    # asymptotes
    assert g(40.0) == 40.0
    assert g(-40.0) == 0.0 or abs(g(-40.0)) < 1e-300
    # grid against 50-digit mpmath
    xs = np.concatenate([np.linspace(-10, 10, 2001), [1e-300, -1e-300, 1e-8, -1e-8, 0.5, -0.5]])
    ys = oracle_mod.gelu(xs)
    for x, y in zip(xs, ys):
        xm = mpmath.mpf(float(x))
        ref = xm * (1 + mpmath.erf(xm / mpmath.sqrt(2))) / 2
        assert abs(y - float(ref)) <= 4e-16 * (2 + x * x) * abs(float(ref)) + 1e-320, x


def test_gelu_is_not_relu_or_sigmoid_form(oracle_mod):
    g = oracle_mod.gelu_scalar
    # GeLU has its minimum near x = -0.7518 with value ~ -0.16997
    xs = np.linspace(-1.5, 0, 15001)
    ys = oracle_mod.gelu(xs)
    i = int(np.argmin(ys))
    assert abs(xs[i] - (-0.7518)) < 2e-4
    assert abs(ys[i] - (-0.16997)) < 1e-5
    assert g(2.0) != max(2.0, 0.0)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("M,H,F", [(5, 16, 32), (9, 24, 48)])
def test_column_split_concatenation_bitwise(oracle_mod, M, H, F):
    X, W, b = _rand((M, H), 1), _rand((H, F), 2, 0.1), _rand((F,), 3, 0.1)
    full_A = oracle_mod.col_preact(X, W, b, 1, 0)
    full_Y = oracle_mod.col_gelu(X, W, b, 1, 0)
    for k in (2, 4, 8):
        A = np.concatenate([oracle_mod.col_preact(X, W, b, k, i) for i in range(k)], axis=1)
        Y = np.concatenate([oracle_mod.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
        assert np.array_equal(A, full_A)
        assert np.array_equal(Y, full_Y)
    # and X W + b is the numpy product to rounding
    assert np.allclose(full_A, X @ W + b, rtol=1e-13, atol=1e-13)


def test_row_split_identity(oracle_mod):
    M, H, F = 7, 16, 64
    Y, V = _rand((M, F), 4), _rand((F, H), 5, 0.1)
    for k in (1, 2, 4, 8):
        Fk = F // k
        parts = [oracle_mod.row_partial(np.ascontiguousarray(Y[:, i * Fk:(i + 1) * Fk]), V, k, i)
                 for i in range(k)]
        Z = oracle_mod.shard_reduce(parts)
        ref = Y @ V
        assert np.max(np.abs(Z - ref)) <= 1e-13 * np.max(np.abs(Y) @ np.abs(V))
    # exact on small integers
    rng = np.random.default_rng(6)
    Yi = rng.integers(-8, 9, size=(M, F)).astype(np.float64)
    Vi = rng.integers(-8, 9, size=(F, H)).astype(np.float64)
    parts = [oracle_mod.row_partial(np.ascontiguousarray(Yi[:, i * 16:(i + 1) * 16]), Vi, 4, i)
             for i in range(4)]
    assert np.array_equal(oracle_mod.shard_reduce(parts), Yi @ Vi)


def test_k_invariance(oracle_mod):
    M, H, F = 6, 32, 128
    X, W, b, V = _rand((M, H), 7), _rand((H, F), 8, 0.2), _rand((F,), 9, 0.2), _rand((F, H), 10, 0.2)
    Z1 = oracle_mod.forward(X, W, b, V, 1)
    for k in (2, 4, 8, 16):
        Zk = oracle_mod.forward(X, W, b, V, k)
        assert np.max(np.abs(Zk - Z1)) <= 1e-13 * np.max(np.abs(Z1))


def test_forward_equals_steps(oracle_mod):
    """The fused per-row forward equals col_gelu -> row_partial -> shard_reduce."""
    M, H, F, k = 5, 24, 96, 4
    X, W, b, V = _rand((M, H), 11), _rand((H, F), 12, 0.2), _rand((F,), 13, 0.2), _rand((F, H), 14, 0.2)
    parts = [oracle_mod.row_partial(oracle_mod.col_gelu(X, W, b, k, i), V, k, i) for i in range(k)]
    assert np.array_equal(oracle_mod.shard_reduce(parts), oracle_mod.forward(X, W, b, V, k))


def test_special_cases(oracle_mod):
    M, H, F, k = 4, 16, 64, 4
    X, W, b, V = _rand((M, H), 15), _rand((H, F), 16, 0.3), _rand((F,), 17, 0.3), _rand((F, H), 18, 0.3)
    gb = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in b])
    # W = 0: Y_i = GeLU(b_i) on every row
    for i in range(k):
        Y = oracle_mod.col_gelu(X, np.zeros_like(W), b, k, i)
        assert np.allclose(Y, np.broadcast_to(gb[i * 16:(i + 1) * 16], Y.shape), rtol=1e-15, atol=0)
    # X = 0: Z = GeLU(b) V on every row (a vector-matrix product)
    Z = oracle_mod.forward(np.zeros_like(X), W, b, V, k)
    assert np.allclose(Z, np.broadcast_to(gb @ V, Z.shape), rtol=1e-13, atol=1e-15)
    # V = 0: Z = 0
    assert not np.any(oracle_mod.forward(X, W, b, np.zeros_like(V), k))
    # no bias: same as zero bias
    assert np.array_equal(oracle_mod.forward(X, W, None, V, k), oracle_mod.forward(X, W, np.zeros(F), V, k))


@pytest.mark.parametrize("M,H,F,k", [(8, 64, 256, 2), (33, 48, 192, 3)])
def test_against_numpy_float64(oracle_mod, M, H, F, k):
    X, W, b, V = _rand((M, H), 19), _rand((H, F), 20, 0.1), _rand((F,), 21, 0.1), _rand((F, H), 22, 0.1)
    A = X @ W + b
    Y = A * 0.5 * (1 + np.vectorize(math.erf)(A / math.sqrt(2)))
    ref = Y @ V
    Z = oracle_mod.forward(X, W, b, V, k)
    assert np.max(np.abs(Z - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_row_independence_and_scaling(oracle_mod):
    M, H, F, k = 10, 16, 64, 4
    X, W, b, V = _rand((M, H), 23), _rand((H, F), 24, 0.3), _rand((F,), 25, 0.3), _rand((F, H), 26, 0.3)
    Z = oracle_mod.forward(X, W, b, V, k)
    perm = np.random.default_rng(0).permutation(M)
    assert np.array_equal(oracle_mod.forward(X[perm], W, b, V, k), Z[perm])
    rows = [9, 0, 3, 3]
    assert np.array_equal(oracle_mod.forward_rows(X, W, b, V, k, rows), Z[rows])
    assert np.array_equal(oracle_mod.forward(X, W, b, 2 * V, k), 2 * Z)


def test_bf16_widening(oracle_mod):
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F81, 0x7F7F, 0x0001], dtype=np.uint16)
    w = oracle_mod.widen(bits)
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == 0.0 and math.copysign(1, w[3]) < 0
    assert w[4] == 1.0 + 2.0 ** -7
    assert w[5] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert w[6] == 2.0 ** -133


def test_pages_shapes(oracle_mod):
    """Shapes the pages state: W is (H, 4H), V is (4H, H), the MLP's single
    all-reduce carries a (B, S, H) message; their GPT-3 175B and 13B examples."""
    import json, os
    here = os.path.dirname(os.path.abspath(__file__))
    g = json.load(open(os.path.join(here, "golden", "pages_shapes.json")))
    B, S, H = 2, 3, 8
    F = 4 * H
    k = 4
    X, W, b, V = _rand((B * S, H), 27), _rand((H, F), 28, 0.2), _rand((F,), 29, 0.2), _rand((F, H), 30, 0.2)
    parts = [oracle_mod.row_partial(oracle_mod.col_gelu(X, W, b, k, i), V, k, i) for i in range(k)]
    assert all(p.shape == (B * S, H) for p in parts)          # each partial is the message
    assert oracle_mod.col_gelu(X, W, b, k, 0).shape == (B * S, F // k)
    e = g["gpt3_tp_comm_example"]
    total = e["allreduces_per_layer"] * e["L"] * e["B"] * e["S"] * e["H"] * e["bytes_per_element"]
    assert abs(total / 1e9 - e["stated_total_GB"]) < 0.05
    e = g["megatron_13b_example"]
    per = e["S"] * e["H"] * e["bytes_per_element"]
    assert abs(per / 2 ** 20 - e["stated_per_allreduce_MB"]) < 0.5
    assert abs(2 * e["layers"] * per / 2 ** 20 - e["stated_total_MB"]) < 20
