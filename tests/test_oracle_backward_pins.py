"""Pins for the CPU fp64 oracle's backward pass, checked against things other
than itself.

* 50-digit numerical differentiation of the forward: the loss
  L = sum(Z * dZ) is evaluated with mpmath at 50 significant digits (the
  forward itself is pinned by brute force in test_oracle_pins.py) and every
  gradient entry of the oracle is compared with a central difference whose
  error is far below float64 rounding.  A wrong sign, a dropped term of
  GeLU' = Phi + x phi, a transposed operand, a wrong shard offset or a missing
  bias gradient all fail this.
* float64 autograd of an independent implementation (torch matmul +
  torch.nn.functional.gelu with the erf form) on random inputs.
* GeLU' closed forms: GeLU'(0) = 1/2, GeLU'(x) + GeLU'(-x) = 1 (because
  GeLU(x) - GeLU(-x) = x), Phi + x phi against mpmath's ncdf/npdf, the
  numerical derivative of the oracle's own GeLU.
* Structure: a column of ones in X makes that row of dW equal to db; the
  gradients are linear in dZ (exact scaling by 2); dZ = 0 and V = 0 reduce to
  zeros and to Y^T dZ; the gradients do not depend on the shard count; the
  per-step functions agree with numpy float64 matmul; the sampled-row and
  sampled-column variants agree with the full backward bit for bit.
"""
import math

import mpmath
import numpy as np
import pytest

mpmath.mp.dps = 50


def _rand(rng, *shape, scale=0.5):
    return rng.standard_normal(shape) * scale


def _mp_loss(X, W, b, V, dZ, k):
    """L = sum(Z * dZ) in 50-digit arithmetic, Z the forward by shards."""
    M, H = len(X), len(X[0])
    F = len(W[0])
    Fk = F // k
    L = mpmath.mpf(0)
    for i in range(k):
        for m in range(M):
            y = []
            for j in range(Fk):
                c = i * Fk + j
                a = mpmath.fsum(X[m][h] * W[h][c] for h in range(H))
                if b is not None:
                    a += b[c]
                y.append(a * (1 + mpmath.erf(a / mpmath.sqrt(2))) / 2)
            for n in range(H):
                z = mpmath.fsum(y[j] * V[i * Fk + j][n] for j in range(Fk))
                L += z * dZ[m][n]
    return L


def _to_mp(a):
    if a is None:
        return None
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 1:
        return [mpmath.mpf(float(v)) for v in a]
    return [[mpmath.mpf(float(v)) for v in row] for row in a]


def _fd_grads(X, W, b, V, dZ, k, h=mpmath.mpf("1e-15")):
    """Central differences of the 50-digit loss for every parameter entry."""
    P = {"X": _to_mp(X), "W": _to_mp(W), "b": _to_mp(b), "V": _to_mp(V)}
    dZm = _to_mp(dZ)
    out = {}
    for name, arr in P.items():
        if arr is None:
            continue
        shape = np.asarray({"X": X, "W": W, "b": b, "V": V}[name]).shape
        g = np.empty(shape)
        for idx in np.ndindex(*shape):
            def setv(v):
                if len(idx) == 1:
                    arr[idx[0]] = v
                else:
                    arr[idx[0]][idx[1]] = v
            orig = arr[idx[0]] if len(idx) == 1 else arr[idx[0]][idx[1]]
            setv(orig + h)
            lp = _mp_loss(P["X"], P["W"], P["b"], P["V"], dZm, k)
            setv(orig - h)
            lm = _mp_loss(P["X"], P["W"], P["b"], P["V"], dZm, k)
            setv(orig)
            g[idx] = float((lp - lm) / (2 * h))
        out[name] = g
    return out


@pytest.mark.parametrize("M,H,F,k,seed,bias", [(2, 3, 4, 2, 1, True), (3, 2, 6, 3, 2, True),
                                               (1, 4, 4, 1, 3, False), (2, 2, 8, 4, 4, True)])
def test_backward_matches_50_digit_numerical_derivative(oracle_mod, M, H, F, k, seed, bias):
    rng = np.random.default_rng(seed)
    X, W, V, dZ = _rand(rng, M, H, scale=1.0), _rand(rng, H, F), _rand(rng, F, H), _rand(rng, M, H)
    b = _rand(rng, F) if bias else None
    dX, dW, db, dV = oracle_mod.backward(X, W, b, V, dZ, k)
    fd = _fd_grads(X, W, b, V, dZ, k)
    for name, got in (("X", dX), ("W", dW), ("V", dV)) + ((("b", db),) if bias else ()):
        ref = fd[name]
        scale = max(1.0, float(np.max(np.abs(ref))))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * scale, err_msg=name)


def test_numerical_derivative_catches_tanh_gelu_grad(oracle_mod):
    """The pin above separates the erf GeLU' from the derivative of the tanh
    approximation (whose gradients differ by ~1e-4 at these inputs)."""
    x = np.linspace(-3, 3, 61)
    c = math.sqrt(2 / math.pi)
    u = c * (x + 0.044715 * x ** 3)
    tanh_grad = 0.5 * (1 + np.tanh(u)) + 0.5 * x * (1 - np.tanh(u) ** 2) * c * (1 + 3 * 0.044715 * x ** 2)
    g = oracle_mod.gelu_grad(x)
    assert np.max(np.abs(g - tanh_grad)) > 1e-4
    exact = np.array([float(mpmath.ncdf(v) + v * mpmath.npdf(v)) for v in x])
    assert np.max(np.abs(g - exact)) < 1e-15


def test_gelu_grad_closed_form(oracle_mod):
    assert oracle_mod.gelu_grad_scalar(0.0) == 0.5
    # Phi(1) + phi(1) from the standard normal tables
    assert abs(oracle_mod.gelu_grad_scalar(1.0) - (0.8413447460685429 + 0.24197072451914337)) < 2e-16
    x = np.concatenate([np.linspace(-9, 9, 721), [1e-8, -1e-8, 37.0, -37.0]])
    g = oracle_mod.gelu_grad(x)
    gm = oracle_mod.gelu_grad(-x)
    assert np.max(np.abs(g + gm - 1.0)) < 4e-16
    exact = np.array([float(mpmath.ncdf(v) + v * mpmath.npdf(v)) for v in x])
    assert np.max(np.abs(g - exact)) < 2e-16 * np.max(np.abs(exact)) * 8
    # asymptotes
    assert oracle_mod.gelu_grad_scalar(37.0) == 1.0
    assert abs(oracle_mod.gelu_grad_scalar(-37.0)) < 1e-290
    # the derivative of the oracle's own GeLU
    h = 1e-5
    xs = np.linspace(-6, 6, 97)
    num = (oracle_mod.gelu(xs + h) - oracle_mod.gelu(xs - h)) / (2 * h)
    assert np.max(np.abs(num - oracle_mod.gelu_grad(xs))) < 1e-9


@pytest.mark.parametrize("M,H,F,k,bias", [(17, 24, 32, 4, True), (5, 8, 64, 8, False), (33, 16, 16, 1, True)])
def test_backward_against_torch_float64_autograd(oracle_mod, M, H, F, k, bias):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(M * 100 + F)
    X, W, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F, H), _rand(rng, M, H)
    b = _rand(rng, F) if bias else None
    tX, tW, tV = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (X, W, V))
    tb = torch.tensor(b, dtype=torch.float64, requires_grad=True) if bias else None
    Fk = F // k
    Z = torch.zeros(M, H, dtype=torch.float64)
    for i in range(k):
        A = tX @ tW[:, i * Fk:(i + 1) * Fk]
        if bias:
            A = A + tb[i * Fk:(i + 1) * Fk]
        Z = Z + torch.nn.functional.gelu(A, approximate="none") @ tV[i * Fk:(i + 1) * Fk]
    (Z * torch.tensor(dZ)).sum().backward()
    dX, dW, db, dV = oracle_mod.backward(X, W, b, V, dZ, k)
    for got, ref in ((dX, tX.grad), (dW, tW.grad), (dV, tV.grad)) + (((db, tb.grad),) if bias else ()):
        ref = ref.numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_ones_column_makes_dW_row_equal_db(oracle_mod):
    rng = np.random.default_rng(7)
    M, H, F, k = 40, 8, 24, 3
    X, W, b, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H), _rand(rng, M, H)
    X[:, 3] = 1.0
    _, dW, db, _ = oracle_mod.backward(X, W, b, V, dZ, k)
    np.testing.assert_array_equal(dW[3], db)


def test_linear_in_dZ_and_special_cases(oracle_mod):
    rng = np.random.default_rng(8)
    M, H, F, k = 9, 8, 16, 2
    X, W, b, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H), _rand(rng, M, H)
    g1 = oracle_mod.backward(X, W, b, V, dZ, k)
    g2 = oracle_mod.backward(X, W, b, V, 2.0 * dZ, k)
    for a, c in zip(g1, g2):
        np.testing.assert_array_equal(2.0 * a, c)
    for a in oracle_mod.backward(X, W, b, V, np.zeros_like(dZ), k):
        assert not np.any(a)
    dX, dW, db, dV = oracle_mod.backward(X, W, b, np.zeros_like(V), dZ, k)
    assert not np.any(dX) and not np.any(dW) and not np.any(db)
    Y = np.concatenate([oracle_mod.col_gelu(X, W, b, k, i) for i in range(k)], axis=1)
    np.testing.assert_allclose(dV, Y.T @ dZ, rtol=1e-13, atol=1e-15)


def test_shard_count_invariance(oracle_mod):
    rng = np.random.default_rng(9)
    M, H, F = 12, 16, 32
    X, W, b, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H), _rand(rng, M, H)
    ref = oracle_mod.backward(X, W, b, V, dZ, 1)
    for k in (2, 4, 8):
        dX, dW, db, dV = oracle_mod.backward(X, W, b, V, dZ, k)
        np.testing.assert_array_equal(dW, ref[1])
        np.testing.assert_array_equal(db, ref[2])
        np.testing.assert_array_equal(dV, ref[3])
        np.testing.assert_allclose(dX, ref[0], rtol=1e-13, atol=1e-14)


def test_steps_against_numpy_matmul(oracle_mod):
    rng = np.random.default_rng(10)
    M, H, F, k, i = 13, 24, 40, 5, 3
    Fk = F // k
    X, W, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F, H), _rand(rng, M, H)
    G = rng.uniform(-0.2, 1.2, (M, Fk))
    Y = _rand(rng, M, Fk)
    dA = _rand(rng, M, Fk)
    Vi, Wi = V[i * Fk:(i + 1) * Fk], W[:, i * Fk:(i + 1) * Fk]
    tol = dict(rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle_mod.act_grad(dZ, V, G, k, i), (dZ @ Vi.T) * G, **tol)
    np.testing.assert_allclose(oracle_mod.row_weight_grad(Y, dZ), Y.T @ dZ, **tol)
    dW, db = oracle_mod.col_weight_grad(X, dA)
    np.testing.assert_allclose(dW, X.T @ dA, **tol)
    np.testing.assert_allclose(db, dA.sum(axis=0), **tol)
    np.testing.assert_allclose(oracle_mod.input_grad_partial(dA, W, k, i), dA @ Wi.T, **tol)
    A = oracle_mod.col_preact(X, W, None, k, i)
    np.testing.assert_array_equal(oracle_mod.col_gelu_grad(X, W, None, k, i), oracle_mod.gelu_grad(A))


def test_sampled_variants_equal_full_backward(oracle_mod):
    rng = np.random.default_rng(11)
    M, H, F, k = 21, 16, 48, 3
    X, W, b, V, dZ = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H), _rand(rng, M, H)
    dX, dW, db, dV = oracle_mod.backward(X, W, b, V, dZ, k)
    rows = [0, 5, 20, 7]
    np.testing.assert_array_equal(oracle_mod.backward_rows(X, W, b, V, dZ, k, rows), dX[rows])
    np.testing.assert_array_equal(oracle_mod.backward_rows(X, W, b, V, dZ, k), dX)
    cols = [0, 15, 16, 47, 30]
    dWc, dbc, dVc = oracle_mod.backward_cols(X, W, b, V, dZ, cols)
    np.testing.assert_array_equal(dWc, dW[:, cols].T)
    np.testing.assert_array_equal(dbc, db[cols])
    np.testing.assert_array_equal(dVc, dV[cols])
    dWc, dbc, dVc = oracle_mod.backward_cols(X, W, None, V, dZ, cols)
    _, dW0, _, dV0 = oracle_mod.backward(X, W, None, V, dZ, k)
    np.testing.assert_array_equal(dWc, dW0[:, cols].T)
    np.testing.assert_array_equal(dVc, dV0[cols])


def test_bf16_inputs_widen_exactly(oracle_mod):
    """bf16 bit patterns are widened exactly: the backward of the widened
    float64 arrays is the same computation."""
    rng = np.random.default_rng(12)
    M, H, F, k = 6, 8, 16, 2
    arrs = [_rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H), _rand(rng, M, H)]
    bits = [(a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for a in arrs]
    wide = [oracle_mod.widen(x) for x in bits]
    g1 = oracle_mod.backward(*bits[:4], bits[4], k)
    g2 = oracle_mod.backward(*wide[:4], wide[4], k)
    for a, c in zip(g1, g2):
        np.testing.assert_array_equal(a, c)
