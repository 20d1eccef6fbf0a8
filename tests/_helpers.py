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
* whole forward:  |Z_gpu - Z| <= tolY |V| + 2 (T + 4) u32 (|Y| |V|), with
  tolY the column-step bound of every shard, side by side, and T the number
  of float32 additions per output: Fk + k for the literal variant (each
  shard's Fk products, then the k partials), F for the fused one (one running
  sum through every shard's products).

Backward (dY = dZ V_i^T, dA = dY * G, G = GeLU'(A)):

* G_i from the training-mode column step:
    |G_gpu - G| <= u_out |G| + (1 + u_out) (0.8 errA + 5e-7),
  errA = 2 (K + 2) u32 S the pre-activation's accumulation bound, 0.8 >=
  max |GeLU''| = 2 phi(0), and 5e-7 the absolute error of the float32 GeLU'
  evaluation (0.75e-7 from the erfc approximation, a few float32 roundings of
  Phi <= 1 and of x phi(x) <= 0.25).
* dA_i = round(float32(dY) * G_used): with errdY = 2 (H + 2) u32 |dZ| |V_i|^T
  and errG the error of the G the kernel used,
    |dA_gpu - dA| <= u_out |dA| + (1 + u_out) (errdY |G| + |dY| errG
                     + errdY errG + u32 |dY| |G|).
* SwiGLU column step, per element of Y_i = SiLU(g) u with g = X Wg_i,
  u = X Wu_i accumulated in float32 (errors e_g, e_u <= 2 (K + 2) u32 S_g, S_u):
    |Y_gpu - Y| <= u_out |Y| + (1 + u_out) (1.1 |u| e_g + |SiLU(g)| e_u + 1.1 e_g e_u
                                            + (4 + 2 |g|) u32 |Y|)
  with 1.1 >= max |SiLU'| and (4 + 2 |g|) u32 the relative error of the
  float32 SiLU (the exponential's argument rounding grows with |g|).
* attention of one head from given bf16 q, k, v (exact inputs): with
  p_tj the exact softmax weights and W_t = sum_j p_tj |v_j|,
    |A_gpu - A| <= 1.5 u16 W_t + 1.01 u16 |A| + 2^-16 W_t
  (the probabilities are rounded to bf16 for the products with V, and the
  normaliser sums the same rounded values, so the output is a weighted mean
  whose weights each moved by at most one bf16 rounding; the output is
  rounded to bf16, and the float32 scores, exp2 and sums add far less; the
  weights are taken against a reference maximum that may trail the running
  one, so a weight can reach 2^8, which changes none of these relative
  terms).  On long sequences the
  float32 sums over n keys add up to 4 (n + 2) u32 W_t (the weighted sum and
  the normaliser, n terms each) and the float32 scores move each weight by
  up to 2 e_s with e_s = 2 (d + 2) u32 max_j (|q| . |k_j|) / sqrt d; the
  rows-only bound (attn_rows_bound) adds both terms.  From the block's inputs the
  scores also carry the projection's error: |ds_tj| <= e_s = 2 u16 (|q| . |k|)
  / sqrt(d) + the GEMMs' accumulation bound, which moves each output by at
  most 2 max_j e_s W_t; the value's rounding adds u16 W_t.
* a float32 GEMM over K terms of operands with errors e_a, e_b:
    |C_gpu - C| <= e_a^T |b| + |a|^T e_b + 2 (K + 2) u32 (|a| + e_a)^T (|b| + e_b).
"""
from __future__ import annotations

import sys

import numpy as np

U32 = 2.0 ** -24
U16 = 2.0 ** -8
GELU_LIP = 1.13


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_initialised() -> bool:
    """True once this process has initialised the GPU: from then on it must not
    start another program (a child interpreter or a compiler)."""
    if "torch" not in sys.modules:
        return False
    import torch
    return bool(torch.cuda.is_initialized())


def tile_rows(M, tile=256, per_tile=2):
    """Rows that cover every `tile`-row block of the output: per block,
    `per_tile` rows at offsets that move through the block from one block to
    the next, plus the first and the last row."""
    rows = {0, M - 1}
    for t in range((M + tile - 1) // tile):
        for j in range(per_tile):
            r = t * tile + (t * 37 + j * (tile // per_tile) + 11) % tile
            if r < M:
                rows.add(r)
    return np.array(sorted(rows))


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


def forward_bound(tolY, Y64, V64, k: int, fused: bool = False, absV=None):
    """tolY, Y64: [rows, F] (all shards side by side); V64: [F, H].  The
    literal variant sums each shard's Fk products and then the k partials;
    the fused one carries one float32 sum through all F products."""
    F = Y64.shape[1]
    terms = F if fused else F // k + k
    aV = np.abs(V64) if absV is None else absV
    return (tolY + 2 * (terms + 4) * U32 * np.abs(Y64)) @ aV + 1e-30


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


GELU2_MAX = 0.8
G_EVAL = 5e-7


def grad_g_bound(S, G, K: int, dtype: str):
    """Bound on the GPU's G = GeLU'(A); S = |X| |W_i| + |b_i|, K = H."""
    u_out = U16 if dtype == "bf16" else 0.0
    errA = 2 * (K + 2) * U32 * S
    return u_out * np.abs(G) + (1 + u_out) * (GELU2_MAX * errA + G_EVAL) + 1e-30


def act_grad_bound(dY, G, errdY, errG, dtype: str):
    u_out = U16 if dtype == "bf16" else 0.0
    aY, aG = np.abs(dY), np.abs(G)
    return (u_out * aY * aG + (1 + u_out) * (errdY * aG + aY * errG + errdY * errG + U32 * aY * aG)
            + 1e-30)


def gemm_bound(a, b, K: int, ea=None, eb=None):
    """Bound of a float32-accumulated a @ b (K terms) with operand errors ea, eb."""
    aa, ab = np.abs(a), np.abs(b)
    out = 0.0
    if ea is not None:
        out = out + ea @ ab
        aa = aa + ea
    if eb is not None:
        out = out + np.abs(a) @ eb
        ab = ab + eb
    return out + 2 * (K + 2) * U32 * (aa @ ab) + 1e-30


def backward_terms(orc, Xr, Wc, bc, Vc, dZr, dtype: str):
    """Magnitudes and error bounds of the backward's intermediates, for the
    bounds only (expected values come from the oracle), for rows Xr of X and
    columns Wc of W (bc of b, rows Vc of V): a dict with float64 A, Y, G, dY,
    dA and the GPU-error bounds tolY (Y), errG (G) and errdA (dA)."""
    X64, W64, V64, dZ64 = f64(Xr), f64(Wc), f64(Vc), f64(dZr)
    b64 = f64(bc) if bc is not None else None
    H = X64.shape[1]
    A = X64 @ W64 + (b64[None, :] if b64 is not None else 0.0)
    S = np.abs(X64) @ np.abs(W64) + (np.abs(b64)[None, :] if b64 is not None else 0.0)
    Y = orc.gelu(A)
    G = orc.gelu_grad(A)
    dY = dZ64 @ V64.T
    errdY = 2 * (H + 2) * U32 * (np.abs(dZ64) @ np.abs(V64).T)
    u_out = U16 if dtype == "bf16" else 0.0
    tolY = ((1 + u_out) * (GELU_LIP * 2 * (H + 2) * U32 * S + 8 * U32 * (2 + A * A) * np.abs(Y)
                           + 2e-7 * np.abs(A)) + u_out * np.abs(Y) + 1e-30)
    errG = grad_g_bound(S, G, H, dtype)
    errdA = act_grad_bound(dY, G, errdY, errG, dtype)
    return dict(A=A, Y=Y, G=G, dY=dY, dA=dY * G, tolY=tolY, errG=errG, errdA=errdA)


SILU_LIP = 1.1


def swiglu_bound(X64, Wg64, Wu64, G, U, Y, dtype: str):
    """Element-wise bound for the SwiGLU Y_i (see module docstring); G, U the
    exact gate and up pre-activations, Y the exact output."""
    K = X64.shape[1]
    aX = np.abs(X64)
    eg = 2 * (K + 2) * U32 * (aX @ np.abs(Wg64))
    eu = 2 * (K + 2) * U32 * (aX @ np.abs(Wu64))
    s = G / (1.0 + np.exp(-G))
    u_out = U16 if dtype == "bf16" else 0.0
    aY = np.abs(Y)
    return (u_out * aY + (1 + u_out) * (SILU_LIP * np.abs(U) * eg + np.abs(s) * eu + SILU_LIP * eg * eu
                                        + (4 + 2 * np.abs(G)) * U32 * aY) + 1e-30)


def attn_weights(qkv64, B: int, S: int, hk: int, d: int, causal: bool):
    """float64 softmax weights P [B, hk, S, S] of a shard's heads (for bounds only)."""
    Hk = hk * d
    q = qkv64[:, :Hk].reshape(B, S, hk, d).transpose(0, 2, 1, 3)
    k = qkv64[:, Hk:2 * Hk].reshape(B, S, hk, d).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) / np.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((S, S), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def attn_core_bound(qkv64, A, B: int, S: int, hk: int, d: int, causal: bool, e_s=None):
    """Element-wise bound for the GPU attention A [B S, hk d] from exact q, k, v
    (see the module docstring); e_s [B, hk, S] adds the score-error term."""
    Hk = hk * d
    P = attn_weights(qkv64, B, S, hk, d, causal)
    v = np.abs(qkv64[:, 2 * Hk:]).reshape(B, S, hk, d).transpose(0, 2, 1, 3)
    W = (P @ v).transpose(0, 2, 1, 3).reshape(B * S, Hk)          # sum_j p_tj |v_j|
    bound = 1.5 * U16 * W + 1.01 * U16 * np.abs(A) + 2.0 ** -16 * W
    if e_s is not None:
        es = np.repeat(e_s.transpose(0, 2, 1).reshape(B * S, hk), d, axis=1)
        bound = bound + 2 * es * W + U16 * W
    return bound + 1e-30


def attn_rows_bound(qkv64, rows, S: int, hk: int, d: int, A, causal: bool = True):
    """Element-wise bound for rows `rows` (indices into [B S]) of the GPU
    attention A from exact q, k, v (see the module docstring): the per-row
    softmax weights are evaluated here in float64 for the bound only."""
    Hk = hk * d
    out = np.empty_like(A)
    for r, m in enumerate(np.asarray(rows)):
        b, t = divmod(int(m), S)
        n = t + 1 if causal else S
        base = b * S
        for h in range(hk):
            q = qkv64[m, h * d:(h + 1) * d]
            K = qkv64[base:base + n, Hk + h * d:Hk + (h + 1) * d]
            aV = np.abs(qkv64[base:base + n, 2 * Hk + h * d:2 * Hk + (h + 1) * d])
            s = K @ q / np.sqrt(d)
            p = np.exp(s - s.max())
            p /= p.sum()
            W = p @ aV
            e_s = 2 * (d + 2) * U32 * float((np.abs(K) @ np.abs(q)).max()) / np.sqrt(d)
            a = np.abs(A[r, h * d:(h + 1) * d])
            out[r, h * d:(h + 1) * d] = ((1.5 * U16 + 2.0 ** -16 + 4 * (n + 2) * U32 + 2 * e_s) * W
                                         + 1.01 * U16 * a)
    return out + 1e-30


def attn_score_err(qkv64, B: int, S: int, hk: int, d: int, H: int, X64=None, Wq=None, Wk=None):
    """max_j of the score error bound e_s [B, hk, S] for bf16 q and k computed
    by a float32 GEMM over H terms (|X| |W| the GEMM's absolute terms)."""
    Hk = hk * d
    aq = np.abs(qkv64[:, :Hk]).reshape(B, S, hk, d).transpose(0, 2, 1, 3)
    ak = np.abs(qkv64[:, Hk:2 * Hk]).reshape(B, S, hk, d).transpose(0, 2, 1, 3)
    e = 2 * U16 * (aq @ ak.transpose(0, 1, 3, 2)) / np.sqrt(d)
    if X64 is not None:
        gq = 2 * (H + 2) * U32 * (np.abs(X64) @ np.abs(Wq))
        gk = 2 * (H + 2) * U32 * (np.abs(X64) @ np.abs(Wk))
        gq = gq.reshape(B, S, hk, d).transpose(0, 2, 1, 3)
        gk = gk.reshape(B, S, hk, d).transpose(0, 2, 1, 3)
        e = e + ((gq @ ak.transpose(0, 1, 3, 2)) + (aq @ gk.transpose(0, 1, 3, 2))) / np.sqrt(d)
    return e.max(axis=-1)


def check_forward_rows(name, w, X, W, b, V, variants, rows, block=512):
    """Compare the GPU's Z on `rows` with the oracle's forward, element by
    element against forward_bound, in blocks of rows.  `variants` maps a label
    to (fused, Zg_of) with Zg_of(row_indices) -> float32 numpy rows.  Returns
    each variant's relative Frobenius error over all the rows compared."""
    import oracle
    W64, b64, V64 = f64(W), f64(b), f64(V)
    aW, aV = np.abs(W64), np.abs(V64)
    k = w.k
    num = {lb: 0.0 for lb in variants}
    den = 0.0
    for r0 in range(0, rows.size, block):
        rr = rows[r0:r0 + block]
        X64r = f64(X[rr])
        Zr = oracle.forward_rows(X64r, W64, b64, V64, k)     # expected values: the oracle
        # bound (magnitudes only): the column step's bound per shard, through V
        A = X64r @ W64 + b64[None, :]
        Y = oracle.gelu(A)
        S = np.abs(X64r) @ aW + np.abs(b64)[None, :]
        u_out = 2.0 ** -8 if w.dtype == "bf16" else 0.0
        tolY = ((1 + u_out) * (1.13 * 2 * (w.H + 2) * 2.0 ** -24 * S + 8 * 2.0 ** -24 * (2 + A * A) * np.abs(Y)
                               + 2e-7 * np.abs(A)) + u_out * np.abs(Y) + 1e-30)
        del A, S
        den += float(np.sum(Zr ** 2))
        for lb, (fused, Zg_of) in variants.items():
            Zg = Zg_of(rr).astype(np.float64)
            bound = forward_bound(tolY, Y, V64, k, fused=fused, absV=aV)
            assert_within(Zg, Zr, bound, "%s Z rows %d..%d (%s)" % (name, rr[0], rr[-1], lb))
            num[lb] += float(np.sum((Zg - Zr) ** 2))
        del tolY, Y
    return {lb: (num[lb] / den) ** 0.5 if den else num[lb] ** 0.5 for lb in variants}
