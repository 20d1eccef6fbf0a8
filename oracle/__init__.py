"""CPU fp64 oracle for the tensor-parallel MLP shard forward and backward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package imports nothing from the product path.

The arithmetic is in ``tp_mlp_oracle.c`` (plain fp64 loops in the order of the
definition, OpenMP over output rows).  This wrapper only widens inputs exactly
to float64 and marshals pointers.  Input arrays may be float64, float32, or
uint16 holding bfloat16 bit patterns; bf16 widening puts the 16 bits in the
top half of a float32, which is exact.

Definition (cited passages in the C file's header):
  W_i = W[:, i*Fk:(i+1)*Fk], b_i = b[i*Fk:(i+1)*Fk], V_i = V[i*Fk:(i+1)*Fk, :]
  Y_i = GeLU(X W_i + b_i),  GeLU(x) = x/2 (1 + erf(x/sqrt 2))
  Z_i = Y_i V_i,  Z = sum_i Z_i  (shard order).
Backward for dZ = dL/dZ (chain rule through the same steps):
  G_i = GeLU'(A_i) = Phi(A_i) + A_i phi(A_i),  dA_i = (dZ V_i^T) * G_i,
  dV_i = Y_i^T dZ,  dW_i = X^T dA_i,  db_i = colsum(dA_i),
  dX = sum_i dA_i W_i^T.

Sequence parallelism: the all-reduce becomes a reduce-scatter over row
blocks of the sequence, with the block's residual added to each block:
  O_r = X[r Mb:(r+1) Mb] + (sum_i Z_i)[r Mb:(r+1) Mb],  Mb = M / k.
SwiGLU variant (no biases):
  Y_i = SiLU(X Wg_i) * (X Wu_i),  SiLU(x) = x / (1 + exp(-x)),  Z = sum_i Y_i V_i.

Tensor-parallel attention (heads split over the k shards, hk = n_heads / k
per shard, d = H / n_heads, Hk = hk d):
  QKV_i = X [Wq_i | Wk_i | Wv_i] + [bq_i | bk_i | bv_i]   (column blocks i)
  per head: softmax(q k^T / sqrt d, causal or not, within each sequence) v
  A_i = heads side by side,  Z = sum_i A_i Wo_i  (Wo_i = rows block i of Wo).

Every forward function here is pinned by tests/test_oracle_pins.py (brute
force in exact rational arithmetic with 50-digit erf, the column-split and
row-split identities, GeLU closed forms, special cases that reduce to library
routines, row independence and exact scaling); every backward function by
tests/test_oracle_backward_pins.py (50-digit numerical differentiation of the
exact forward, float64 autograd of an independent implementation, GeLU' closed
forms, the ones-column identity between db and dW, k-invariance, linearity);
the sequence-parallel and SwiGLU functions by tests/test_oracle_sp_swiglu_pins.py
(exact small-integer sums and a hand-worked block split, the all-gather of the
blocks against the all-reduce, residual-only and zero-residual cases, row
locality; SiLU closed forms and 50-digit values, exact rational brute force,
gate/up asymmetry, the column- and row-split identities and k-invariance, an
independent numpy implementation); the attention functions by
tests/test_oracle_attn_pins.py (exact-rational projections with 50-digit
softmax on tiny inputs, one key gives v, a zero query gives the mean of the
visible values, two-key closed forms with the 1/sqrt(d) scale, causality,
sequence independence, key permutation invariance without the mask, the
head split and row split identities, k-invariance, an independent numpy
implementation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tp_mlp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _source_sha256() -> str:
    import hashlib
    return hashlib.sha256(open(_SRC, "rb").read()).hexdigest()


def build_oracle(force: bool = True) -> str:
    """Compile liboracle.so with gcc and OpenMP (called by the build step only,
    before anything touches the GPU); the source's SHA-256 is compiled in."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               '-DORACLE_SOURCE_SHA256="%s"' % _source_sha256(), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("oracle/liboracle.so is not built: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_source_sha256.restype = ctypes.c_char_p
        if lib.oracle_source_sha256().decode() != _source_sha256():
            raise RuntimeError("oracle/liboracle.so was built from another version of tp_mlp_oracle.c: "
                               "run __graft_entry__.build() again")
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_gelu_array.argtypes = [vp, i64, vp]
        lib.oracle_col_preact.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_col_gelu.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_row_partial.argtypes = [vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_shard_reduce.argtypes = [vp, ci, i64, vp]
        lib.oracle_forward_rows.argtypes = [vp, vp, vp, vp, i64, i64, ci, vp, i64, vp]
        lib.oracle_max_threads.restype = ci
        lib.oracle_sp_reduce_scatter.argtypes = [vp, ci, vp, ci, i64, i64, vp]
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu_array.argtypes = [vp, i64, vp]
        lib.oracle_swiglu_col.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_swiglu_forward_rows.argtypes = [vp, vp, vp, vp, i64, i64, ci, vp, i64, vp]
        lib.oracle_attn_qkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, ci, ci, vp]
        lib.oracle_attn_core.argtypes = [vp, i64, i64, ci, i64, ci, vp]
        lib.oracle_attn_core_rows.argtypes = [vp, i64, ci, i64, ci, vp, i64, vp]
        lib.oracle_attn_forward_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, ci, ci, vp, i64,
                                                 vp]
        lib.oracle_gelu_grad.argtypes = [ctypes.c_double]
        lib.oracle_gelu_grad.restype = ctypes.c_double
        lib.oracle_gelu_grad_array.argtypes = [vp, i64, vp]
        lib.oracle_col_gelu_grad.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_act_grad.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_row_weight_grad.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.oracle_col_weight_grad.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        lib.oracle_input_grad_partial.argtypes = [vp, vp, i64, i64, i64, ci, ci, vp]
        lib.oracle_backward_rows.argtypes = [vp, vp, vp, vp, vp, i64, i64, ci, vp, i64, vp]
        lib.oracle_backward_cols.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp]
        for f in (lib.oracle_gelu_array, lib.oracle_col_preact, lib.oracle_col_gelu,
                  lib.oracle_row_partial, lib.oracle_shard_reduce, lib.oracle_forward_rows,
                  lib.oracle_gelu_grad_array, lib.oracle_col_gelu_grad, lib.oracle_act_grad,
                  lib.oracle_row_weight_grad, lib.oracle_col_weight_grad,
                  lib.oracle_input_grad_partial, lib.oracle_backward_rows, lib.oracle_backward_cols,
                  lib.oracle_sp_reduce_scatter, lib.oracle_silu_array, lib.oracle_swiglu_col,
                  lib.oracle_swiglu_forward_rows, lib.oracle_attn_qkv, lib.oracle_attn_core,
                  lib.oracle_attn_core_rows,
                  lib.oracle_attn_forward_rows):
            f.restype = None
        _lib = lib
    return _lib


def widen(a) -> np.ndarray:
    """Exact float64 copy of a float64/float32 array or of bf16 bits in uint16."""
    a = np.asarray(a)
    if a.dtype == np.float64:
        return np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise TypeError("oracle inputs must be float64, float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _p(a):
    return a.ctypes.data if a is not None else None


def max_threads() -> int:
    return int(_L().oracle_max_threads())


def gelu_scalar(x: float) -> float:
    return float(_L().oracle_gelu(float(x)))


def gelu(x) -> np.ndarray:
    x = widen(x)
    y = np.empty_like(x)
    _L().oracle_gelu_array(_p(x), x.size, _p(y))
    return y


def _check_shard(F: int, k: int, i: int):
    if k < 1 or F % k:
        raise ValueError("k must be >= 1 and divide F")
    if not 0 <= i < k:
        raise ValueError("shard index out of range")


def col_preact(X, W, b, k: int, i: int) -> np.ndarray:
    """A_i = X W_i + b_i, float64 [M, F/k].  b may be None."""
    X, W = widen(X), widen(W)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H
    _check_shard(F, k, i)
    A = np.empty((M, F // k))
    _L().oracle_col_preact(_p(X), _p(W), _p(b), M, H, F, k, i, _p(A))
    return A


def col_gelu(X, W, b, k: int, i: int) -> np.ndarray:
    """Y_i = GeLU(X W_i + b_i), float64 [M, F/k]."""
    X, W = widen(X), widen(W)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H
    _check_shard(F, k, i)
    Y = np.empty((M, F // k))
    _L().oracle_col_gelu(_p(X), _p(W), _p(b), M, H, F, k, i, _p(Y))
    return Y


def row_partial(Yi, V, k: int, i: int) -> np.ndarray:
    """Z_i = Y_i V_i with V the full [F, H] matrix, float64 [M, H]."""
    Yi, V = widen(Yi), widen(V)
    F, H = V.shape
    _check_shard(F, k, i)
    M, Fk = Yi.shape
    assert Fk == F // k
    Z = np.empty((M, H))
    _L().oracle_row_partial(_p(Yi), _p(V), M, F, H, k, i, _p(Z))
    return Z


def shard_reduce(parts) -> np.ndarray:
    """Z = parts[0] + ... + parts[k-1] (float64, left to right)."""
    ws = [np.ascontiguousarray(widen(p)).reshape(-1) for p in parts]
    n = ws[0].size
    assert all(w.size == n for w in ws)
    ptrs = (ctypes.c_void_p * len(ws))(*[w.ctypes.data for w in ws])
    Z = np.empty(n)
    _L().oracle_shard_reduce(ptrs, len(ws), n, _p(Z))
    return Z.reshape(np.asarray(parts[0]).shape)


def forward_rows(X, W, b, V, k: int, rows=None) -> np.ndarray:
    """Z[rows, :] of the whole forward, float64 [len(rows), H] (all rows if None)."""
    X, W, V = widen(X), widen(W), widen(V)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H and V.shape == (F, H)
    _check_shard(F, k, 0)
    if rows is None:
        r = None
        nrows = M
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row index out of range")
        nrows = r.size
    Z = np.empty((nrows, H))
    if nrows:
        _L().oracle_forward_rows(_p(X), _p(W), _p(b), _p(V), H, F, k, _p(r), nrows, _p(Z))
    return Z


def forward(X, W, b, V, k: int) -> np.ndarray:
    """Z = sum_i GeLU(X W_i + b_i) V_i, float64 [M, H]."""
    return forward_rows(X, W, b, V, k, None)


# ---------------------------------------------------------------------------
# Backward.

def gelu_grad_scalar(x: float) -> float:
    return float(_L().oracle_gelu_grad(float(x)))


def gelu_grad(x) -> np.ndarray:
    """GeLU'(x) = Phi(x) + x phi(x), float64."""
    x = widen(x)
    g = np.empty_like(x)
    _L().oracle_gelu_grad_array(_p(x), x.size, _p(g))
    return g


def col_gelu_grad(X, W, b, k: int, i: int) -> np.ndarray:
    """G_i = GeLU'(X W_i + b_i), float64 [M, F/k]."""
    X, W = widen(X), widen(W)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H
    _check_shard(F, k, i)
    G = np.empty((M, F // k))
    _L().oracle_col_gelu_grad(_p(X), _p(W), _p(b), M, H, F, k, i, _p(G))
    return G


def act_grad(dZ, V, Gi, k: int, i: int) -> np.ndarray:
    """dA_i = (dZ V_i^T) * G_i with V the full [F, H] matrix, float64 [M, F/k]."""
    dZ, V, Gi = widen(dZ), widen(V), widen(Gi)
    F, H = V.shape
    _check_shard(F, k, i)
    M = dZ.shape[0]
    assert dZ.shape == (M, H) and Gi.shape == (M, F // k)
    dA = np.empty((M, F // k))
    _L().oracle_act_grad(_p(dZ), _p(V), _p(Gi), M, F, H, k, i, _p(dA))
    return dA


def row_weight_grad(Yi, dZ) -> np.ndarray:
    """dV_i = Y_i^T dZ, float64 [Fk, H]."""
    Yi, dZ = widen(Yi), widen(dZ)
    M, Fk = Yi.shape
    H = dZ.shape[1]
    assert dZ.shape[0] == M
    dV = np.empty((Fk, H))
    _L().oracle_row_weight_grad(_p(Yi), _p(dZ), M, Fk, H, _p(dV))
    return dV


def col_weight_grad(X, dAi):
    """(dW_i, db_i) = (X^T dA_i, colsum dA_i), float64 [H, Fk] and [Fk]."""
    X, dAi = widen(X), widen(dAi)
    M, H = X.shape
    Fk = dAi.shape[1]
    assert dAi.shape[0] == M
    dW = np.empty((H, Fk))
    db = np.empty(Fk)
    _L().oracle_col_weight_grad(_p(X), _p(dAi), M, H, Fk, _p(dW), _p(db))
    return dW, db


def input_grad_partial(dAi, W, k: int, i: int) -> np.ndarray:
    """dX_i = dA_i W_i^T with W the full [H, F] matrix, float64 [M, H]."""
    dAi, W = widen(dAi), widen(W)
    H, F = W.shape
    _check_shard(F, k, i)
    M = dAi.shape[0]
    assert dAi.shape == (M, F // k)
    dX = np.empty((M, H))
    _L().oracle_input_grad_partial(_p(dAi), _p(W), M, H, F, k, i, _p(dX))
    return dX


def backward_rows(X, W, b, V, dZ, k: int, rows=None) -> np.ndarray:
    """dX[rows, :] of the whole backward, float64 (all rows if None)."""
    X, W, V, dZ = widen(X), widen(W), widen(V), widen(dZ)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H and V.shape == (F, H) and dZ.shape == (M, H)
    _check_shard(F, k, 0)
    if rows is None:
        r, nrows = None, M
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row index out of range")
        nrows = r.size
    dX = np.empty((nrows, H))
    if nrows:
        _L().oracle_backward_rows(_p(X), _p(W), _p(b), _p(V), _p(dZ), H, F, k, _p(r), nrows, _p(dX))
    return dX


def backward_cols(X, W, b, V, dZ, cols):
    """Parameter gradients of columns `cols` of the full F: (dW[:, cols].T,
    db[cols], dV[cols, :]), float64 [n, H], [n], [n, H]."""
    X, W, V, dZ = widen(X), widen(W), widen(V), widen(dZ)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    assert W.shape[0] == H and V.shape == (F, H) and dZ.shape == (M, H)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if c.size and (c.min() < 0 or c.max() >= F):
        raise IndexError("column index out of range")
    n = c.size
    dWc, dbc, dVc = np.empty((n, H)), np.empty(n), np.empty((n, H))
    if n:
        _L().oracle_backward_cols(_p(X), _p(W), _p(b), _p(V), _p(dZ), M, H, F, _p(c), n, _p(dWc),
                                  _p(dbc), _p(dVc))
    return dWc, dbc, dVc


def backward(X, W, b, V, dZ, k: int):
    """The whole backward by shards, in the order of the steps:
    returns (dX [M, H], dW [H, F], db [F], dV [F, H]), float64."""
    X, W, V, dZ = widen(X), widen(W), widen(V), widen(dZ)
    b = widen(b) if b is not None else None
    M, H = X.shape
    F = W.shape[1]
    _check_shard(F, k, 0)
    Fk = F // k
    dW, db, dV = np.empty((H, F)), np.empty(F), np.empty((F, H))
    parts = []
    for i in range(k):
        Yi = col_gelu(X, W, b, k, i)
        Gi = col_gelu_grad(X, W, b, k, i)
        dAi = act_grad(dZ, V, Gi, k, i)
        dV[i * Fk:(i + 1) * Fk] = row_weight_grad(Yi, dZ)
        dWi, dbi = col_weight_grad(X, dAi)
        dW[:, i * Fk:(i + 1) * Fk] = dWi
        db[i * Fk:(i + 1) * Fk] = dbi
        parts.append(input_grad_partial(dAi, W, k, i))
    dX = shard_reduce(parts)
    return dX, dW, db, dV


# ---------------------------------------------------------------------------
# Sequence parallelism.

def sp_reduce_scatter(parts, R, k: int):
    """Blocks O_r = R[r Mb:(r+1) Mb] + (parts[0] + ... )[r Mb:(r+1) Mb] for
    r < k, Mb = M / k; float64 [Mb, H] each.  R may be None (no residual)."""
    ws = [np.ascontiguousarray(widen(p)) for p in parts]
    if not ws:
        raise ValueError("need at least one part")
    M, H = ws[0].shape
    assert all(w.shape == (M, H) for w in ws)
    if k < 1 or M % k:
        raise ValueError("k must be >= 1 and divide M")
    R64 = np.ascontiguousarray(widen(R)) if R is not None else None
    if R64 is not None:
        assert R64.shape == (M, H)
    outs = [np.empty((M // k, H)) for _ in range(k)]
    pp = (ctypes.c_void_p * len(ws))(*[w.ctypes.data for w in ws])
    po = (ctypes.c_void_p * k)(*[o.ctypes.data for o in outs])
    if M:
        _L().oracle_sp_reduce_scatter(pp, len(ws), _p(R64), k, M, H, po)
    return outs


def sp_forward(X, W, b, V, k: int):
    """Sequence-parallel block output: the k blocks of X + sum_i Z_i."""
    X64 = widen(X)
    parts = [row_partial(col_gelu(X64, W, b, k, i), V, k, i) for i in range(k)]
    return sp_reduce_scatter(parts, X64, k)


def sp_forward_rows(X, W, b, V, k: int, rows) -> np.ndarray:
    """Rows `rows` (indices into the gathered [M, H]) of the blocks' union,
    X[rows] + Z[rows], float64."""
    X64 = widen(X)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    Z = forward_rows(X64, W, b, V, k, r)
    return sp_reduce_scatter([Z], X64[r], 1)[0]


# ---------------------------------------------------------------------------
# SwiGLU.

def silu_scalar(x: float) -> float:
    return float(_L().oracle_silu(float(x)))


def silu(x) -> np.ndarray:
    x = widen(x)
    y = np.empty_like(x)
    _L().oracle_silu_array(_p(x), x.size, _p(y))
    return y


def swiglu_col(X, Wg, Wu, k: int, i: int) -> np.ndarray:
    """Y_i = SiLU(X Wg_i) * (X Wu_i), float64 [M, F/k]."""
    X, Wg, Wu = widen(X), widen(Wg), widen(Wu)
    M, H = X.shape
    F = Wg.shape[1]
    assert Wg.shape == (H, F) and Wu.shape == (H, F)
    _check_shard(F, k, i)
    Y = np.empty((M, F // k))
    _L().oracle_swiglu_col(_p(X), _p(Wg), _p(Wu), M, H, F, k, i, _p(Y))
    return Y


def swiglu_forward_rows(X, Wg, Wu, V, k: int, rows=None) -> np.ndarray:
    """Z[rows, :] of the SwiGLU forward, float64 (all rows if None)."""
    X, Wg, Wu, V = widen(X), widen(Wg), widen(Wu), widen(V)
    M, H = X.shape
    F = Wg.shape[1]
    assert Wg.shape == (H, F) and Wu.shape == (H, F) and V.shape == (F, H)
    _check_shard(F, k, 0)
    if rows is None:
        r, nrows = None, M
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row index out of range")
        nrows = r.size
    Z = np.empty((nrows, H))
    if nrows:
        _L().oracle_swiglu_forward_rows(_p(X), _p(Wg), _p(Wu), _p(V), H, F, k, _p(r), nrows, _p(Z))
    return Z


def swiglu_forward(X, Wg, Wu, V, k: int) -> np.ndarray:
    """Z = sum_i (SiLU(X Wg_i) * (X Wu_i)) V_i, float64 [M, H]."""
    return swiglu_forward_rows(X, Wg, Wu, V, k, None)


# ---------------------------------------------------------------------------
# Tensor-parallel attention.

def _attn_dims(H: int, nh: int, k: int):
    if nh < 1 or H % nh or nh % k:
        raise ValueError("n_heads must divide H and k must divide n_heads")
    d = H // nh
    return d, nh // k, (nh // k) * d


def attn_qkv(X, Wq, Wk, Wv, bq, bk, bv, nh: int, k: int, i: int) -> np.ndarray:
    """[q | k | v] of shard i: float64 [M, 3 Hk]; biases may be None."""
    X, Wq, Wk, Wv = widen(X), widen(Wq), widen(Wk), widen(Wv)
    bq, bk, bv = [widen(x) if x is not None else None for x in (bq, bk, bv)]
    M, H = X.shape
    assert Wq.shape == Wk.shape == Wv.shape == (H, H)
    d, hk, Hk = _attn_dims(H, nh, k)
    if not 0 <= i < k:
        raise ValueError("shard index out of range")
    out = np.empty((M, 3 * Hk))
    if M:
        _L().oracle_attn_qkv(_p(X), _p(Wq), _p(Wk), _p(Wv), _p(bq), _p(bk), _p(bv), M, H, nh, k, i, _p(out))
    return out


def attn_core(QKV, B: int, S: int, hk: int, d: int, causal: bool = True) -> np.ndarray:
    """The shard's heads' attention outputs side by side, float64 [B S, hk d]."""
    Q = np.ascontiguousarray(widen(QKV))
    assert Q.shape == (B * S, 3 * hk * d)
    A = np.empty((B * S, hk * d))
    if B * S:
        _L().oracle_attn_core(_p(Q), B, S, hk, d, 1 if causal else 0, _p(A))
    return A


def attn_core_rows(QKV, B: int, S: int, hk: int, d: int, rows, causal: bool = True) -> np.ndarray:
    """Rows `rows` (indices into [B S]) of attn_core's output, float64
    [len(rows), hk d]: each query row evaluated on its own (a row at position t
    of its sequence needs keys 0..t, or the whole sequence without the mask)."""
    Q = np.ascontiguousarray(widen(QKV))
    assert Q.shape == (B * S, 3 * hk * d)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= B * S):
        raise IndexError("row index out of range")
    A = np.empty((r.size, hk * d))
    if r.size:
        _L().oracle_attn_core_rows(_p(Q), S, hk, d, 1 if causal else 0, _p(r), r.size, _p(A))
    return A


def attn_forward_rows(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh: int, S: int, k: int, rows,
                      causal: bool = True) -> np.ndarray:
    """Z[rows, :] of the whole attention block, float64 (rows index X = [B S, H])."""
    X, Wq, Wk, Wv, Wo = widen(X), widen(Wq), widen(Wk), widen(Wv), widen(Wo)
    bq, bk, bv = [widen(x) if x is not None else None for x in (bq, bk, bv)]
    M, H = X.shape
    _attn_dims(H, nh, k)
    if S < 1 or M % S:
        raise ValueError("S must divide M")
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= M):
        raise IndexError("row index out of range")
    Z = np.empty((r.size, H))
    if r.size:
        _L().oracle_attn_forward_rows(_p(X), _p(Wq), _p(Wk), _p(Wv), _p(bq), _p(bk), _p(bv), _p(Wo), S, H, nh, k,
                                      1 if causal else 0, _p(r), r.size, _p(Z))
    return Z


def attn_forward(X, Wq, Wk, Wv, bq, bk, bv, Wo, nh: int, S: int, k: int, causal: bool = True) -> np.ndarray:
    """The attention block by shards, in the order of the steps: float64 [M, H]."""
    X64 = widen(X)
    M, H = X64.shape
    d, hk, Hk = _attn_dims(H, nh, k)
    Wo64 = widen(Wo)
    parts = []
    for i in range(k):
        A = attn_core(attn_qkv(X64, Wq, Wk, Wv, bq, bk, bv, nh, k, i), M // S, S, hk, d, causal)
        Woi = np.ascontiguousarray(Wo64[i * Hk:(i + 1) * Hk])
        # Z_i = A_i Wo_i: the row-parallel partial of the MLP oracle with one shard
        parts.append(row_partial(A, Woi, 1, 0))
    return shard_reduce(parts)
