"""Pins for the oracle's tensor-parallel attention block, checked against
things other than the oracle itself (heads split over the shards, Q/K/V
column-parallel, output projection row-parallel: "AI大模型分布式训练：张量并行与流水线
并行深度实践" §2.3; "千亿参数模型如何拆分到多张GPU上训练" 注意力层的切分; "大模型分布式并行
策略详解：TP、DP、PP、CP、EP核心原理与实战" §4.2):

* exact-rational projections and 50-digit softmax on tiny dyadic inputs (a
  wrong scale, a missing bias, a transposed score, a wrong head offset or a
  mask off by one all fail it);
* closed forms: one visible key gives its value; a zero query attends
  uniformly (the mean of the visible values); two keys with a known score
  difference give the logistic weights, which pins the 1/sqrt(d) scale;
* structure: causality (later rows change nothing before them), sequence
  independence, key-permutation invariance without the mask;
* the head split (shards' heads side by side are the unsplit heads, bit for
  bit), the row split of the output projection, k-invariance, the sampled-row
  variant, and an independent numpy float64 implementation.
"""
import random
from fractions import Fraction

import mpmath
import numpy as np
import pytest

mpmath.mp.dps = 50


def _rand(rng, M, H, std=0.3):
    X = rng.standard_normal((M, H))
    Ws = [rng.standard_normal((H, H)) * std for _ in range(4)]
    bs = [rng.standard_normal(H) * 0.1 for _ in range(3)]
    return X, Ws, bs


def _numpy_attention(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, causal):
    M, H = X.shape
    d = H // nh
    q = (X @ Wq + bq).reshape(M // S, S, nh, d).transpose(0, 2, 1, 3)
    k = (X @ Wk + bk).reshape(M // S, S, nh, d).transpose(0, 2, 1, 3)
    v = (X @ Wv + bv).reshape(M // S, S, nh, d).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) / np.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((S, S), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    a = (p @ v).transpose(0, 2, 1, 3).reshape(M, H)
    return a @ Wo


@pytest.mark.parametrize("B,S,H,nh,k,causal,seed", [(1, 1, 2, 1, 1, True, 0), (1, 3, 4, 2, 2, True, 1),
                                                     (2, 3, 4, 2, 1, False, 2), (1, 4, 6, 3, 3, True, 3),
                                                     (2, 2, 8, 4, 2, False, 4)])
def test_attention_brute_force_tiny(oracle_mod, B, S, H, nh, k, causal, seed):
    rng = random.Random(seed)
    M, d = B * S, H // nh
    dy = lambda r, c, n, q: [[Fraction(rng.randint(-n, n), q) for _ in range(c)] for _ in range(r)]
    X = dy(M, H, 8, 4)
    Wq, Wk, Wv, Wo = dy(H, H, 8, 8), dy(H, H, 8, 8), dy(H, H, 8, 8), dy(H, H, 8, 8)
    bq, bk, bv = dy(1, H, 4, 8)[0], dy(1, H, 4, 8)[0], dy(1, H, 4, 8)[0]
    mp = lambda f: mpmath.mpf(f.numerator) / f.denominator

    def proj(W, bvec):
        return [[sum((X[m][h] * W[h][c] for h in range(H)), Fraction(0)) + bvec[c] for c in range(H)]
                for m in range(M)]
    Q, K, V = proj(Wq, bq), proj(Wk, bk), proj(Wv, bv)
    A = [[mpmath.mpf(0)] * H for _ in range(M)]
    for b in range(B):
        for t in range(S):
            m = b * S + t
            for h in range(nh):
                cols = range(h * d, (h + 1) * d)
                keys = range(t + 1) if causal else range(S)
                sc = [mp(sum((Q[m][c] * K[b * S + j][c] for c in cols), Fraction(0))) / mpmath.sqrt(d)
                      for j in keys]
                mx = max(sc)
                e = [mpmath.exp(x - mx) for x in sc]
                tot = sum(e)
                for c in cols:
                    A[m][c] = sum((e[n] / tot * mp(V[b * S + j][c]) for n, j in enumerate(keys)), mpmath.mpf(0))
    Zx = [[sum((A[m][c] * mp(Wo[c][e]) for c in range(H)), mpmath.mpf(0)) for e in range(H)] for m in range(M)]
    npf = lambda a: np.array([[float(x) for x in r] for r in a])
    Xn, Wqn, Wkn, Wvn, Won = map(npf, (X, Wq, Wk, Wv, Wo))
    bqn, bkn, bvn = (np.array([float(x) for x in v]) for v in (bq, bk, bv))
    # per shard: the projection is exact, the attention output within 1e-14
    hk, Hk = nh // k, (nh // k) * d
    for i in range(k):
        qkv = oracle_mod.attn_qkv(Xn, Wqn, Wkn, Wvn, bqn, bkn, bvn, nh, k, i)
        for m in range(M):
            for c in range(Hk):
                assert qkv[m, c] == float(Q[m][i * Hk + c])
                assert qkv[m, Hk + c] == float(K[m][i * Hk + c])
                assert qkv[m, 2 * Hk + c] == float(V[m][i * Hk + c])
        Ai = oracle_mod.attn_core(qkv, B, S, hk, d, causal)
        scale = np.abs(npf(V)).max() + 1e-300
        for m in range(M):
            for c in range(Hk):
                assert abs(Ai[m, c] - float(A[m][i * Hk + c])) <= 1e-14 * scale, (i, m, c)
    Z = oracle_mod.attn_forward(Xn, Wqn, Wkn, Wvn, bqn, bkn, bvn, Won, nh, S, k, causal)
    zs = np.abs(npf([[float(x) for x in r] for r in A])) @ np.abs(Won) + 1e-300
    for m in range(M):
        for e in range(H):
            assert abs(Z[m, e] - float(Zx[m][e])) <= 1e-14 * zs[m, e], (m, e)


def test_attention_closed_forms(oracle_mod):
    rng = np.random.default_rng(1)
    B, S, hk, d = 2, 5, 2, 4
    Hk = hk * d
    QKV = rng.standard_normal((B * S, 3 * Hk))
    V = QKV[:, 2 * Hk:]
    # causal position 0 sees only itself: its output is its own value
    A = oracle_mod.attn_core(QKV, B, S, hk, d, True)
    for b in range(B):
        np.testing.assert_allclose(A[b * S], V[b * S], rtol=0, atol=1e-15)
    # S = 1: the only key, with or without the mask
    A1 = oracle_mod.attn_core(QKV[:1], 1, 1, hk, d, False)
    np.testing.assert_allclose(A1[0], V[0], rtol=0, atol=1e-15)
    # a zero query attends uniformly: the mean of the visible values
    Q0 = QKV.copy()
    Q0[:, :Hk] = 0.0
    Ac = oracle_mod.attn_core(Q0, B, S, hk, d, True)
    An = oracle_mod.attn_core(Q0, B, S, hk, d, False)
    for b in range(B):
        for t in range(S):
            vis = V[b * S:b * S + t + 1]
            np.testing.assert_allclose(Ac[b * S + t], vis.mean(axis=0), rtol=0, atol=1e-14)
            np.testing.assert_allclose(An[b * S + t], V[b * S:(b + 1) * S].mean(axis=0), rtol=0, atol=1e-14)
    # two keys, one head, d = 4: q = (1,0,0,0), k0 = (2,0,0,0), k1 = 0 give
    # scores 2/sqrt(4) = 1 and 0, so p0 = e / (e + 1)
    q = np.zeros((2, 12))
    q[1, 0] = 1.0            # query of position 1
    q[0, 4] = 2.0            # key of position 0
    q[0, 8:12] = [1, 2, 3, 4]
    q[1, 8:12] = [-1, 0, 1, 0]
    A2 = oracle_mod.attn_core(q, 1, 2, 1, 4, True)
    p0 = np.e / (np.e + 1.0)
    np.testing.assert_allclose(A2[1], p0 * np.array([1, 2, 3, 4.]) + (1 - p0) * np.array([-1, 0, 1, 0.]),
                               rtol=0, atol=1e-15)


def test_attention_structure(oracle_mod):
    rng = np.random.default_rng(2)
    B, S, H, nh, k = 3, 6, 8, 2, 2
    X, (Wq, Wk, Wv, Wo), (bq, bk, bv) = _rand(rng, B * S, H)
    Z = oracle_mod.attn_forward(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, k, True)
    # causality: changing rows after position t of sequence 1 changes nothing up to t
    t = 2
    X2 = X.copy()
    X2[S + t + 1:2 * S] += 1.0
    Z2 = oracle_mod.attn_forward(X2, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, k, True)
    np.testing.assert_array_equal(Z2[:S + t + 1], Z[:S + t + 1])
    assert np.abs(Z2[S + t + 1:2 * S] - Z[S + t + 1:2 * S]).max() > 1e-3
    np.testing.assert_array_equal(Z2[2 * S:], Z[2 * S:])           # other sequences untouched
    # without the mask: permuting a sequence's rows permutes its outputs
    Zn = oracle_mod.attn_forward(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, k, False)
    perm = np.array([4, 0, 5, 2, 1, 3])
    Xp = X.copy()
    Xp[S:2 * S] = X[S + perm]
    Zp = oracle_mod.attn_forward(Xp, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, k, False)
    np.testing.assert_allclose(Zp[S:2 * S], Zn[S + perm], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_splits_and_numpy(oracle_mod, causal):
    rng = np.random.default_rng(3 + causal)
    B, S, H, nh = 2, 7, 16, 8
    X, (Wq, Wk, Wv, Wo), (bq, bk, bv) = _rand(rng, B * S, H)
    d = H // nh
    # head split: the shards' heads side by side are the unsplit heads, bit for bit
    A1 = oracle_mod.attn_core(oracle_mod.attn_qkv(X, Wq, Wk, Wv, bq, bk, bv, nh, 1, 0), B, S, nh, d, causal)
    Zs = {}
    for k in (1, 2, 4, 8):
        hk = nh // k
        Ak = np.concatenate([oracle_mod.attn_core(oracle_mod.attn_qkv(X, Wq, Wk, Wv, bq, bk, bv, nh, k, i),
                                                  B, S, hk, d, causal) for i in range(k)], axis=1)
        np.testing.assert_array_equal(Ak, A1)
        Zs[k] = oracle_mod.attn_forward(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, k, causal)
    ref = A1 @ Wo                                                 # row split of the output projection
    scale = np.abs(A1) @ np.abs(Wo)
    for k, Z in Zs.items():
        assert np.all(np.abs(Z - ref) <= 1e-14 * scale + 1e-300), k
    Znp = _numpy_attention(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, causal)
    assert np.all(np.abs(Zs[2] - Znp) <= 1e-12 * scale + 1e-300)
    rows = [0, 6, 7, 13, 3]
    np.testing.assert_allclose(oracle_mod.attn_forward_rows(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh, S, 4, rows, causal),
                               Zs[4][rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_core_rows(oracle_mod, causal):
    """The rows-only evaluation of the attention core equals the whole-output
    one on the same rows bit for bit (the same per-row evaluation, pinned
    above), and an independent numpy softmax attention of those rows to
    1e-12; rows from both sequences, first, middle and last positions."""
    rng = np.random.default_rng(11 + causal)
    B, S, hk, d = 2, 37, 3, 8
    Hk = hk * d
    qkv = rng.standard_normal((B * S, 3 * Hk)) * 1.5
    rows = np.array([0, 1, 17, 36, 37, 38, 55, 73])
    full = oracle_mod.attn_core(qkv, B, S, hk, d, causal)
    got = oracle_mod.attn_core_rows(qkv, B, S, hk, d, rows, causal)
    np.testing.assert_array_equal(got, full[rows])
    for r, m in enumerate(rows):
        b, t = divmod(int(m), S)
        n = t + 1 if causal else S
        for h in range(hk):
            q = qkv[m, h * d:(h + 1) * d]
            K = qkv[b * S:b * S + n, Hk + h * d:Hk + (h + 1) * d]
            V = qkv[b * S:b * S + n, 2 * Hk + h * d:2 * Hk + (h + 1) * d]
            s = K @ q / np.sqrt(d)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ V
            np.testing.assert_allclose(got[r, h * d:(h + 1) * d], ref, rtol=0, atol=1e-12)
    assert oracle_mod.attn_core_rows(qkv, B, S, hk, d, np.array([], dtype=np.int64), causal).shape == (0, Hk)
    with pytest.raises(IndexError):
        oracle_mod.attn_core_rows(qkv, B, S, hk, d, [B * S], causal)
