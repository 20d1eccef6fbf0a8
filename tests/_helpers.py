"""Shared helpers for the GPU parity tests: host<->device copies and the
element-wise error bounds the comparisons use.

Error model (u = unit roundoff: 2^-24 for float32, 2^-8 for bfloat16):

* column step, per element of Y_i:
    |Y_gpu - Y| <= u_out |Y| + 1.13 * 2 (K + 2) u32 S + 8 u32 (2 + a^2) |Y| + 2e-7 |a|
  with S = |X| |W_i| + |b_i| (the sum of absolute terms of the pre-activation
  a), 1.13 >= max |GeLU'|, (2 + a^2) the conditioning of Phi(a) for negative a,
  u_out = 2^-8 when Y is stored as bf16 (0 for float32), and 2e-7 |a| the
  error of the kernel's erfc approximation (absolute error <= 1.5e-7 in erfc,
  i.e. <= 0.75e-7 in Phi, times |a|, plus its float32 evaluation).
* row step from the GPU's own Y_i:  |Z_gpu - Z| <= 2 (K + 2) u32 (|Y_i| |V_i|).
* whole forward:  |Z_gpu - Z| <= tolY |V| + 2 (Fk + k + 4) u32 (|Y| |V|), with
  tolY the column-step bound of every shard, side by side.
"""
from __future__ import annotations

import sys

import numpy as np

U32 = 2.0 ** -24
U16 = 2.0 ** -8
GELU_LIP = 1.13


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    raise TypeError(a.dtype)


def from_dev(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.contiguous().cpu().numpy()
    raise TypeError(t.dtype)


def f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den else float(np.linalg.norm(got))


def col_bound(X64, Wi64, bi64, A, Y, dtype: str):
    """Element-wise bound for Y_i (see module docstring)."""
    K = X64.shape[1]
    S = np.abs(X64) @ np.abs(Wi64)
    if bi64 is not None:
        S = S + np.abs(bi64)[None, :]
    u_out = U16 if dtype == "bf16" else 0.0
    absY = np.abs(Y)
    return ((1 + u_out) * (GELU_LIP * 2 * (K + 2) * U32 * S + 8 * U32 * (2 + A * A) * absY
                           + 2e-7 * np.abs(A)) + u_out * absY + 1e-30)


def row_bound(Y64, Vi64):
    K = Y64.shape[1]
    return 2 * (K + 2) * U32 * (np.abs(Y64) @ np.abs(Vi64)) + 1e-30


def forward_bound(tolY, Y64, V64, k: int):
    """tolY, Y64: [rows, F] (all shards side by side); V64: [F, H]."""
    Fk = Y64.shape[1] // k
    return (tolY + 2 * (Fk + k + 4) * U32 * np.abs(Y64)) @ np.abs(V64) + 1e-30


def assert_within(got, ref, bound, what: str, max_report: int = 5):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= bound)  # also catches NaN
    if bad.any():
        idx = np.argwhere(bad)[:max_report]
        lines = ["%s: %d of %d elements outside the bound" % (what, int(bad.sum()), bad.size)]
        for ix in idx:
            t = tuple(ix)
            lines.append("  at %s: got %.9g ref %.9g err %.3g bound %.3g" % (t, got[t], ref[t], err[t], bound[t]))
        raise AssertionError("\n".join(lines))
