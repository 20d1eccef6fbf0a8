"""Host-side checks of the C ABI that need no GPU.

The library must load and export every function include/tp_mlp.h (the product
interface) and include/tp_mlp_dev.h (the tile-measurement hooks) declare, and
every argument error must be reported before any HIP call (so these calls are
safe without a device: fake, aligned, non-NULL pointers are never touched).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp.h")
DEV_HEADER = os.path.join(ROOT, "include", "tp_mlp_dev.h")


@pytest.fixture(scope="module")
def L():
    import tensor_transformer_mlp_amd as tpm
    return tpm.lib()   # built by __graft_entry__.build(); raises if it is not


def _declared(path=None):
    if path is None:
        return _declared(HEADER) | _declared(DEV_HEADER)
    text = open(path).read()
    return set(re.findall(r"^(?:int|size_t|const char\s*\*)\s*(tp_\w+)\s*\(", text, re.M))


def _header_constants():
    text = open(HEADER).read()
    out = {}
    for name, val in re.findall(r"^#define\s+(TP_\w+)\s+\(?(-?\d+)u?\)?", text, re.M):
        out[name] = int(val)
    return out


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert names == {"tp_mlp_col_gelu", "tp_mlp_row_partial", "tp_shard_reduce",
                     "tp_mlp_workspace_bytes", "tp_mlp_shard_forward", "tp_status_string",
                     "tp_mlp_version", "tp_mlp_col_gelu_save", "tp_mlp_grad_act",
                     "tp_mlp_grad_weight_workspace_bytes", "tp_mlp_grad_row_weight",
                     "tp_mlp_grad_col_weight", "tp_mlp_grad_input_partial",
                     "tp_mlp_backward_workspace_bytes", "tp_mlp_shard_backward",
                     "tp_mlp_col_gelu_shards", "tp_mlp_row_partial_shards", "tp_mlp_grad_act_shards",
                     "tp_mlp_grad_weight_workspace_bytes_shards", "tp_mlp_grad_row_weight_shards",
                     "tp_mlp_grad_col_weight_shards", "tp_mlp_grad_input_shards",
                     "tp_sp_reduce_scatter", "tp_mlp_sp_workspace_bytes", "tp_mlp_shard_forward_sp",
                     "tp_swiglu_col", "tp_swiglu_col_shards", "tp_swiglu_shard_forward",
                     "tp_attn_qkv_shards", "tp_attn_core_shards", "tp_attn_workspace_bytes",
                     "tp_attn_shard_forward", "tp_gemm_tiles", "tp_mlp_step_tile",
                     "tp_mlp_col_gelu_shards_tile", "tp_mlp_row_partial_shards_tile",
                     "tp_attn_core_shards_variant", "tp_mlp_shard_forward_noalloc"}
    for n in names:
        assert hasattr(L, n), n
    # the measurement hooks live in the dev header only
    assert _declared(DEV_HEADER) == {"tp_gemm_tiles", "tp_mlp_step_tile", "tp_mlp_col_gelu_shards_tile",
                                     "tp_mlp_row_partial_shards_tile", "tp_attn_core_shards_variant"}
    assert not _declared(HEADER) & _declared(DEV_HEADER)


def test_python_constants_match_header():
    import tensor_transformer_mlp_amd as tpm
    c = _header_constants()
    for n in ("TP_F32", "TP_BF16", "TP_ACCUMULATE", "TP_FUSED_ACCUM", "TP_GRAD_ACCUMULATE",
              "TP_SUM_SHARDS", "TP_MAX_SHARDS", "TP_MAX_BATCH", "TP_CAUSAL"):
        assert getattr(tpm, n) == c[n], n
    text = open(HEADER).read()
    assert re.search(r"#define TP_NOALLOC_SCRATCH_BYTES \(128u << 20\)", text)
    assert tpm.TP_NOALLOC_SCRATCH_BYTES == 128 << 20


def test_status_strings(L):
    import tensor_transformer_mlp_amd as tpm
    c = _header_constants()
    seen = set()
    for n, v in c.items():
        if n.startswith("TP_ERR_") or n == "TP_OK":
            s = tpm.tp_status_string(v)
            assert s and s != "unknown status"
            seen.add(s)
    assert tpm.tp_status_string(12345) == "unknown status"
    assert len(seen) == 9
    assert tpm.tp_mlp_version() >= 100


P = 0x10000  # fake aligned device addresses; never dereferenced by a rejected call


def _p(i):
    return ctypes.c_void_p(P * (i + 1))


def test_col_gelu_errors(L):
    c = _header_constants()
    f = L.tp_mlp_col_gelu
    ok_args = lambda: [_p(0), _p(1), _p(2), _p(3), 16, 64, 128, 1, None]
    a = ok_args(); a[7] = 7
    assert f(*a) == c["TP_ERR_DTYPE"]
    for idx, val in [(5, 60), (5, 0), (6, 12), (6, 0), (4, -1), (5, -8), (5, (1 << 22) + 8),
                     (6, (1 << 22) + 8), (4, 1 << 31)]:
        a = ok_args(); a[idx] = val
        assert f(*a) == c["TP_ERR_SHAPE"], (idx, val)
    for idx in (0, 1, 3):
        a = ok_args(); a[idx] = None
        assert f(*a) == c["TP_ERR_NULL"], idx
    for idx in (0, 1, 2, 3):
        a = ok_args(); a[idx] = ctypes.c_void_p(P * (idx + 1) + 8)
        assert f(*a) == c["TP_ERR_ALIGN"], idx
    a = ok_args(); a[3] = _p(0)  # Y overlaps X
    assert f(*a) == c["TP_ERR_ALIAS"]
    # M == 0 is a valid no-op, even with NULL pointers
    a = ok_args(); a[4] = 0; a[0] = None; a[3] = None
    assert f(*a) == c["TP_OK"]


def test_row_partial_errors(L):
    c = _header_constants()
    f = L.tp_mlp_row_partial
    ok_args = lambda: [_p(0), _p(1), _p(2), 16, 128, 64, 1, 0, None]
    a = ok_args(); a[7] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = ok_args(); a[6] = -1
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = ok_args(); a[4] = 100
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok_args(); a[2] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok_args(); a[2] = ctypes.c_void_p(P * 3 + 4)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok_args(); a[2] = ctypes.c_void_p(P * 2 + 16)  # Z inside V
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok_args(); a[3] = 0
    assert f(*a) == c["TP_OK"]


def test_shard_reduce_errors(L):
    c = _header_constants()
    f = L.tp_shard_reduce
    parts = (ctypes.c_void_p * 4)(P, 2 * P, 3 * P, 4 * P)
    assert f(parts, 0, _p(9), 64, None) == c["TP_ERR_SHAPE"]
    assert f(parts, 65, _p(9), 64, None) == c["TP_ERR_SHAPE"]
    assert f(parts, 4, _p(9), -1, None) == c["TP_ERR_SHAPE"]
    assert f(parts, 4, None, 64, None) == c["TP_ERR_NULL"]
    assert f(None, 4, _p(9), 64, None) == c["TP_ERR_NULL"]
    bad = (ctypes.c_void_p * 4)(P, None, 3 * P, 4 * P)
    assert f(bad, 4, _p(9), 64, None) == c["TP_ERR_NULL"]
    bad = (ctypes.c_void_p * 4)(P, 2 * P + 4, 3 * P, 4 * P)
    assert f(bad, 4, _p(9), 64, None) == c["TP_ERR_ALIGN"]
    # Z may be parts[0] but no other partial
    assert f(parts, 4, ctypes.c_void_p(2 * P), 64, None) == c["TP_ERR_ALIAS"]
    assert f(parts, 4, ctypes.c_void_p(2 * P + 16), 64, None) == c["TP_ERR_ALIAS"]
    assert f(parts, 4, _p(9), 0, None) == c["TP_OK"]


def test_workspace_bytes(L):
    f = L.tp_mlp_workspace_bytes
    # one Y buffer per shard of a batch of min(k, 16) shards (M*Fk*elt rounded
    # to 256), plus (k-1) fp32 partials of M*H unless fused
    assert f(4, 8192, 768, 768, 1, 0) == 4 * 8192 * 768 * 2 + 3 * 8192 * 768 * 4
    assert f(4, 8192, 768, 768, 1, 1) == 4 * 8192 * 768 * 2
    assert f(2, 8, 64, 128, 0, 0) == 2 * 8 * 128 * 4 + 8 * 64 * 4
    assert f(1, 3, 8, 8, 1, 0) == 256
    assert f(2, 3, 8, 8, 1, 0) == 2 * 256 + 256
    assert f(64, 3, 8, 8, 1, 1) == 16 * 256
    assert f(0, 8, 64, 128, 0, 0) == 0
    assert f(2, 8, 60, 128, 0, 0) == 0
    assert f(2, 8, 64, 128, 5, 0) == 0
    assert f(2, 8, 64, 128, 0, 4) == 0
    assert f(2, 0, 64, 128, 0, 0) == 0
    big = f(8, 32768, 8192, 4096, 1, 0)
    assert big == 8 * 32768 * 4096 * 2 + 7 * 32768 * 8192 * 4


def test_shard_forward_errors(L):
    c = _header_constants()
    f = L.tp_mlp_shard_forward
    k = 2
    W = (ctypes.c_void_p * k)(10 * P, 11 * P)
    V = (ctypes.c_void_p * k)(12 * P, 13 * P)
    b = (ctypes.c_void_p * k)(14 * P, 15 * P)
    need = L.tp_mlp_workspace_bytes(k, 8, 64, 128, 1, 0)
    ws = ctypes.c_void_p(1 << 40)
    Z = ctypes.c_void_p(1 << 41)
    X = ctypes.c_void_p(1 << 42)
    base = lambda: [X, W, b, V, k, 8, 64, 128, 1, ws, need, Z, 0, None]
    a = base(); a[12] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = base(); a[4] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[4] = 65
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[10] = need - 1
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[9] = None
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[1] = (ctypes.c_void_p * k)(10 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[2] = (ctypes.c_void_p * k)(14 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[3] = (ctypes.c_void_p * k)(12 * P + 2, 13 * P)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = base(); a[11] = ctypes.c_void_p((1 << 40) + 256)  # Z inside the workspace
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[8] = 3
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = base(); a[5] = 0
    assert f(*a) == c["TP_OK"]


def test_binding_rejects_cpu_tensors(L):
    import torch
    import tensor_transformer_mlp_amd as tpm
    X = torch.zeros(4, 64)
    W = torch.zeros(64, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        tpm.tp_mlp_col_gelu(X, W, None, Y_i=torch.zeros(4, 128))


def test_col_gelu_save_errors(L):
    c = _header_constants()
    f = L.tp_mlp_col_gelu_save
    ok_args = lambda: [_p(0), _p(1), _p(2), _p(3), _p(4), 16, 64, 128, 1, None]
    a = ok_args(); a[8] = 2
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = ok_args(); a[6] = 20
    assert f(*a) == c["TP_ERR_SHAPE"]
    for idx in (0, 1, 3, 4):
        a = ok_args(); a[idx] = None
        assert f(*a) == c["TP_ERR_NULL"], idx
    a = ok_args(); a[4] = ctypes.c_void_p(P * 5 + 8)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok_args(); a[4] = _p(3)  # G == Y
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok_args(); a[4] = _p(1)  # G overlaps W_i
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok_args(); a[5] = 0
    assert f(*a) == c["TP_OK"]


def test_grad_act_errors(L):
    c = _header_constants()
    f = L.tp_mlp_grad_act
    ok_args = lambda: [_p(0), _p(1), _p(2), _p(3), 16, 64, 128, 1, None]
    a = ok_args(); a[7] = 5
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = ok_args(); a[5] = 7
    assert f(*a) == c["TP_ERR_SHAPE"]
    for idx in range(4):
        a = ok_args(); a[idx] = None
        assert f(*a) == c["TP_ERR_NULL"], idx
    a = ok_args(); a[3] = ctypes.c_void_p(P * 4 + 2)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok_args(); a[3] = _p(0)  # dA overlaps dZ
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok_args(); a[3] = ctypes.c_void_p(P * 3 + 64)  # dA partly over G (not in place)
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok_args(); a[4] = 0
    assert f(*a) == c["TP_OK"]


def test_grad_weight_errors(L):
    c = _header_constants()
    need = L.tp_mlp_grad_weight_workspace_bytes(16, 64, 128, 1)
    ws = ctypes.c_void_p(1 << 40)
    f = L.tp_mlp_grad_row_weight  # (Y_i, dZ, dV_i, M, Fk, H, dtype, ws, ws_bytes, flags, stream)
    ok = lambda: [_p(0), _p(1), _p(2), 16, 128, 64, 1, ws, need, 0, None]
    a = ok(); a[9] = 1  # TP_ACCUMULATE is not a weight-gradient flag
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[6] = 3
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = ok(); a[4] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[2] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok(); a[2] = ctypes.c_void_p(P * 3 + 4)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok(); a[2] = _p(1)
    assert f(*a) == c["TP_ERR_ALIAS"]
    if need:
        a = ok(); a[8] = need - 1
        assert f(*a) == c["TP_ERR_WORKSPACE"]
    g = L.tp_mlp_grad_col_weight  # (X, dA_i, dW_i, db_i, M, H, Fk, dtype, ws, ws_bytes, flags, stream)
    ok = lambda: [_p(0), _p(1), _p(2), _p(3), 16, 64, 128, 1, ws, need, 2, None]
    a = ok(); a[10] = 3
    assert f is not g and g(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[3] = ctypes.c_void_p(P * 4 + 8)
    assert g(*a) == c["TP_ERR_ALIGN"]
    a = ok(); a[3] = ctypes.c_void_p(P * 3 + 16)  # db inside dW
    assert g(*a) == c["TP_ERR_ALIAS"]
    assert need > 0  # the column-sum partials
    a = ok(); a[8] = ctypes.c_void_p(P * 2)  # workspace over dA
    assert g(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[0] = None
    assert g(*a) == c["TP_ERR_NULL"]


def test_grad_input_partial_errors(L):
    c = _header_constants()
    f = L.tp_mlp_grad_input_partial  # (dA_i, W_i, dX_i, M, Fk, H, dtype, flags, stream)
    ok = lambda: [_p(0), _p(1), _p(2), 16, 128, 64, 1, 0, None]
    a = ok(); a[7] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[5] = 4
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[1] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok(); a[2] = _p(0)
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[3] = 0
    assert f(*a) == c["TP_OK"]


def test_backward_workspace_bytes(L):
    f = L.tp_mlp_backward_workspace_bytes
    gw = L.tp_mlp_grad_weight_workspace_bytes
    for (k, M, H, Fk, dt) in [(4, 8192, 768, 768, 1), (8, 8192, 4096, 2048, 1), (2, 40, 64, 128, 0),
                              (1, 3, 8, 8, 1), (20, 64, 64, 64, 1)]:
        e = 2 if dt == 1 else 4
        G = min(k, 16)
        act = -(-M * Fk * e // 256) * 256
        part = -(-M * H * 4 // 256) * 256
        lit = f(k, M, H, Fk, dt, 0)
        fused = f(k, M, H, Fk, dt, 1)
        assert lit - fused == (k - 1) * part
        assert f(k, M, H, Fk, dt, 3) == fused
        # two activation buffers per shard of a batch, then the weight-gradient
        # workspace of the batch, which covers at least the single-shard one
        assert fused >= 2 * G * act + gw(M, H, Fk, dt)
        assert (fused - 2 * G * act) % 256 == 0
        # bf16 with M >= 4096: transposed copies of W_i and V_i for the shards of a batch
        tw = 2 * G * (-(-H * Fk * 2 // 256) * 256) if dt == 1 and M >= 4096 else 0
        assert fused == 2 * G * act + L.tp_mlp_grad_weight_workspace_bytes_shards(G, M, H, Fk, dt) + tw
    assert gw(8192, 768, 768, 1) >= 768 * 4
    assert f(0, 8, 64, 128, 0, 0) == 0
    assert f(2, 8, 60, 128, 0, 0) == 0
    assert f(2, 8, 64, 128, 0, 4) == 0
    assert gw(8, 64, 128, 7) == 0
    assert f(2, 0, 64, 128, 0, 0) == 0


def test_shard_backward_errors(L):
    c = _header_constants()
    f = L.tp_mlp_shard_backward
    k = 2
    arr = lambda *xs: (ctypes.c_void_p * k)(*xs)
    W, V, b = arr(10 * P, 11 * P), arr(12 * P, 13 * P), arr(14 * P, 15 * P)
    dW, dV, db = arr(20 * P, 21 * P), arr(22 * P, 23 * P), arr(24 * P, 25 * P)
    need = L.tp_mlp_backward_workspace_bytes(k, 8, 64, 128, 1, 0)
    ws, dX, X, dZ = (ctypes.c_void_p(1 << s) for s in (40, 41, 42, 43))
    base = lambda: [X, W, b, V, dZ, k, 8, 64, 128, 1, ws, need, dX, dW, db, dV, 0, None]
    a = base(); a[16] = 4
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = base(); a[5] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[7] = 12
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[11] = need - 1
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[13] = arr(20 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[14] = arr(24 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[4] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[15] = arr(22 * P + 4, 23 * P)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = base(); a[15] = arr(22 * P, 22 * P)  # two shards' dV on one buffer
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[13] = arr(20 * P, 10 * P)  # dW[1] over W[0]
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[12] = ctypes.c_void_p((1 << 40) + 512)  # dX inside the workspace
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[9] = 2
    assert f(*a) == c["TP_ERR_DTYPE"]


def test_shards_entry_point_errors(L):
    c = _header_constants()
    arr = lambda *xs: (ctypes.c_void_p * len(xs))(*xs)
    X = ctypes.c_void_p(1 << 40)
    W, b, Y, G = arr(10 * P, 11 * P), arr(12 * P, 13 * P), arr(14 * P, 15 * P), arr(16 * P, 17 * P)
    f = L.tp_mlp_col_gelu_shards  # (X, W, b, Y, G, n, M, H, Fk, dtype, stream)
    ok = lambda: [X, W, b, Y, G, 2, 16, 64, 128, 1, None]
    a = ok(); a[5] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[5] = c["TP_MAX_BATCH"] + 1
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[3] = arr(14 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok(); a[4] = arr(16 * P, 17 * P + 4)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok(); a[3] = arr(14 * P, 14 * P)  # two shards write one Y
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[4] = arr(16 * P, 11 * P)  # G[1] over W[1]
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[6] = 0
    assert f(*a) == c["TP_OK"]
    r = L.tp_mlp_row_partial_shards  # (Y, V, Z, n, M, Fk, H, dtype, flags, stream)
    Z = arr(20 * P, None)
    ok = lambda: [Y, W, arr(20 * P, 21 * P), 2, 16, 128, 64, 1, 0, None]
    a = ok(); a[8] = 8
    assert r(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[2] = Z  # Z[1] needed without TP_SUM_SHARDS
    assert r(*a) == c["TP_ERR_NULL"]
    a = ok(); a[2] = arr(20 * P, 20 * P)
    assert r(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[4] = 0
    assert r(*a) == c["TP_OK"]
    # the single-shard call rejects the batch-only flag
    assert L.tp_mlp_row_partial(_p(0), _p(1), _p(2), 16, 128, 64, 1, c["TP_SUM_SHARDS"], None) == c["TP_ERR_FLAGS"]
    g = L.tp_mlp_grad_act_shards  # (dZ, V, G, dA, n, M, H, Fk, dtype, stream)
    ok = lambda: [X, W, G, arr(16 * P, 17 * P), 2, 16, 64, 128, 1, None]  # in place
    a = ok(); a[3] = arr(17 * P, 16 * P)  # dA[0] over G[1]: not in place
    assert g(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[1] = None
    assert g(*a) == c["TP_ERR_NULL"]
    w = L.tp_mlp_grad_weight_workspace_bytes_shards
    assert w(0, 16, 64, 128, 1) == 0 and w(17, 16, 64, 128, 1) == 0
    assert w(1, 8192, 768, 768, 1) == L.tp_mlp_grad_weight_workspace_bytes(8192, 768, 768, 1)
    assert w(4, 8192, 768, 768, 1) >= w(1, 8192, 768, 768, 1)
    d = L.tp_mlp_grad_input_shards  # (dA, W, dX, n, M, Fk, H, dtype, flags, stream)
    ok = lambda: [Y, W, Z, 2, 16, 128, 64, 1, c["TP_SUM_SHARDS"], None]
    a = ok(); a[8] = 16
    assert d(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[2] = arr(11 * P, None)  # dX[0] over W[1]
    assert d(*a) == c["TP_ERR_ALIAS"]


def test_sp_reduce_scatter_errors(L):
    c = _header_constants()
    f = L.tp_sp_reduce_scatter
    parts = (ctypes.c_void_p * 2)(P, 2 * P)
    O = (ctypes.c_void_p * 4)(20 * P, 21 * P, 22 * P, 23 * P)
    R = ctypes.c_void_p(30 * P)
    base = lambda: [parts, 2, R, 1, O, 0, 4, 64, 64, None]
    a = base(); a[3] = 2
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = base(); a[5] = -1
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = base(); a[1] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[1] = 65
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[6] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[7] = 66            # k = 4 does not divide M
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[8] = 60            # H % 8
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[0] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[4] = (ctypes.c_void_p * 4)(20 * P, None, 22 * P, 23 * P)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[4] = (ctypes.c_void_p * 4)(20 * P, 21 * P + 8, 22 * P, 23 * P)
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = base(); a[2] = ctypes.c_void_p(30 * P + 4)
    assert f(*a) == c["TP_ERR_ALIGN"]
    # an output block inside a part, inside R, or over another block
    a = base(); a[4] = (ctypes.c_void_p * 4)(20 * P, P + 1024, 22 * P, 23 * P)
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[4] = (ctypes.c_void_p * 4)(20 * P, 21 * P, 30 * P + 16, 23 * P)
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[4] = (ctypes.c_void_p * 4)(20 * P, 20 * P + 256, 22 * P, 23 * P)
    assert f(*a) == c["TP_ERR_ALIAS"]
    # blocks side by side (the gathered layout) do not overlap: 16 rows x 64 x 4 bytes each
    a = base(); a[4] = (ctypes.c_void_p * 4)(*[20 * P + r * 16 * 64 * 4 for r in range(4)])
    a[7] = 0                          # M == 0: a no-op after the checks
    assert f(*a) == c["TP_OK"]
    a = base(); a[7] = 0
    assert f(*a) == c["TP_OK"]


def test_sp_workspace_bytes(L):
    f = L.tp_mlp_sp_workspace_bytes
    # one Y per shard of a batch plus k fp32 partials (1 when fused)
    assert f(4, 8192, 768, 768, 1, 0) == 4 * 8192 * 768 * 2 + 4 * 8192 * 768 * 4
    assert f(4, 8192, 768, 768, 1, 1) == 4 * 8192 * 768 * 2 + 8192 * 768 * 4
    assert f(2, 8, 64, 128, 0, 0) == 2 * 8 * 128 * 4 + 2 * 8 * 64 * 4
    assert f(4, 6, 64, 128, 0, 0) == 0      # k does not divide M
    assert f(4, 0, 64, 128, 0, 0) == 0
    assert f(4, 8, 64, 128, 0, 2) == 0
    assert f(4, 8, 64, 128, 7, 0) == 0


def test_shard_forward_sp_errors(L):
    c = _header_constants()
    f = L.tp_mlp_shard_forward_sp
    k = 2
    W = (ctypes.c_void_p * k)(10 * P, 11 * P)
    V = (ctypes.c_void_p * k)(12 * P, 13 * P)
    b = (ctypes.c_void_p * k)(14 * P, 15 * P)
    O = (ctypes.c_void_p * k)(1 << 41, (1 << 41) + 4 * 64 * 4)
    need = L.tp_mlp_sp_workspace_bytes(k, 8, 64, 128, 1, 0)
    ws = ctypes.c_void_p(1 << 40)
    X = ctypes.c_void_p(1 << 42)
    base = lambda: [X, W, b, V, k, 8, 64, 128, 1, ws, need, O, 0, 0, None]
    a = base(); a[13] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = base(); a[12] = 5
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = base(); a[5] = 9              # k does not divide M
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[10] = need - 1
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[11] = (ctypes.c_void_p * k)(1 << 41, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[11] = (ctypes.c_void_p * k)(1 << 41, (1 << 41) + 16)
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[11] = (ctypes.c_void_p * k)(1 << 41, (1 << 40) + 512)   # block inside the workspace
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[11] = (ctypes.c_void_p * k)((1 << 42) + 64, (1 << 41))  # block over X
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[5] = 0
    assert f(*a) == c["TP_OK"]


def test_swiglu_errors(L):
    c = _header_constants()
    f = L.tp_swiglu_col
    X, Wg, Wu, Y = _p(0), _p(1), _p(2), _p(3)
    assert f(X, Wg, Wu, Y, 8, 64, 128, 2, None) == c["TP_ERR_DTYPE"]
    assert f(X, Wg, Wu, Y, 8, 60, 128, 1, None) == c["TP_ERR_SHAPE"]
    assert f(X, None, Wu, Y, 8, 64, 128, 1, None) == c["TP_ERR_NULL"]
    assert f(X, Wg, None, Y, 8, 64, 128, 1, None) == c["TP_ERR_NULL"]
    assert f(X, Wg, ctypes.c_void_p(3 * P + 8), Y, 8, 64, 128, 1, None) == c["TP_ERR_ALIGN"]
    assert f(X, Wg, Wu, ctypes.c_void_p(2 * P + 64), 8, 64, 128, 1, None) == c["TP_ERR_ALIAS"]  # Y over Wu
    assert f(X, Wg, Wu, Y, 0, 64, 128, 1, None) == c["TP_OK"]
    fs = L.tp_swiglu_col_shards
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    assert fs(X, arr(P, 2 * P), arr(3 * P, 4 * P), arr(5 * P, 6 * P), 0, 8, 64, 128, 1, None) == c["TP_ERR_SHAPE"]
    assert fs(X, arr(P, 2 * P), arr(3 * P, 4 * P), arr(5 * P, 5 * P + 16), 2, 8, 64, 128, 1, None) == \
        c["TP_ERR_ALIAS"]
    ff = L.tp_swiglu_shard_forward
    k = 2
    need = L.tp_mlp_workspace_bytes(k, 8, 64, 128, 1, 0)
    ws, Z = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41)
    base = lambda: [ctypes.c_void_p(1 << 42), arr(10 * P, 11 * P), arr(12 * P, 13 * P), arr(14 * P, 15 * P), k, 8,
                    64, 128, 1, ws, need, Z, 0, None]
    a = base(); a[12] = 2
    assert ff(*a) == c["TP_ERR_FLAGS"]
    a = base(); a[10] = need - 1
    assert ff(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[2] = arr(12 * P, None)
    assert ff(*a) == c["TP_ERR_NULL"]
    a = base(); a[11] = ctypes.c_void_p(12 * P + 256)      # Z over an up weight
    assert ff(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[5] = 0
    assert ff(*a) == c["TP_OK"]


def test_attention_errors(L):
    c = _header_constants()
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    core = L.tp_attn_core_shards
    qkv, A = arr(P, 2 * P), arr(3 * P, 4 * P)
    # B=1, S=8, 2 heads of 64
    assert core(qkv, A, 2, 1, 8, 2, 64, 0, 8, None) == c["TP_ERR_DTYPE"]        # fp32 attention
    assert core(qkv, A, 2, 1, 8, 2, 96, 1, 8, None) == c["TP_ERR_SHAPE"]        # head_dim
    assert core(qkv, A, 2, 1, 8, 2, 64, 1, 16, None) == c["TP_ERR_FLAGS"]
    assert core(qkv, A, 0, 1, 8, 2, 64, 1, 8, None) == c["TP_ERR_SHAPE"]
    assert core(arr(P, None), A, 2, 1, 8, 2, 64, 1, 8, None) == c["TP_ERR_NULL"]
    assert core(qkv, arr(3 * P, 4 * P + 8), 2, 1, 8, 2, 64, 1, 8, None) == c["TP_ERR_ALIGN"]
    assert core(qkv, arr(3 * P, P + 64), 2, 1, 8, 2, 64, 1, 8, None) == c["TP_ERR_ALIAS"]   # A over QKV
    assert core(qkv, A, 2, 1, 0, 2, 64, 1, 8, None) == c["TP_OK"]
    ws_f = L.tp_attn_workspace_bytes
    # k = 4, B = 8, S = 1024, H = 768, 12 heads: per batch shard QKV [M, 576] and A [M, 192] bf16,
    # plus 3 fp32 partials [M, 768]
    M = 8 * 1024
    assert ws_f(4, 8, 1024, 768, 12, 1, 8) == 4 * (M * 576 * 2 + M * 192 * 2) + 3 * M * 768 * 4
    assert ws_f(4, 8, 1024, 768, 12, 1, 9) == 4 * (M * 576 * 2 + M * 192 * 2)
    assert ws_f(4, 8, 1024, 768, 10, 1, 8) == 0       # 768 / 10 is not a head width
    assert ws_f(5, 8, 1024, 768, 12, 1, 8) == 0       # 5 does not divide 12
    assert ws_f(4, 8, 1024, 768, 12, 0, 8) == 0       # fp32
    f = L.tp_attn_shard_forward
    k = 2
    need = ws_f(k, 1, 64, 256, 4, 1, 8)
    ws, Z, X = ctypes.c_void_p(1 << 40), ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42)
    base = lambda: [X, arr(10 * P, 11 * P), arr(12 * P, 13 * P), arr(14 * P, 15 * P), k, 1, 64, 256, 4, 1, ws,
                    need, Z, 8, None]
    a = base(); a[13] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = base(); a[8] = 3
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = base(); a[9] = 0
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = base(); a[11] = need - 1
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    a = base(); a[3] = arr(14 * P, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = base(); a[12] = ctypes.c_void_p(14 * P + 64)   # Z over an output weight
    assert f(*a) == c["TP_ERR_ALIAS"]
    a = base(); a[6] = 0
    assert f(*a) == c["TP_OK"]


def test_tile_table_and_choice(L):
    import tensor_transformer_mlp_amd as tpm
    tiles = tpm.tp_gemm_tiles()
    assert len(tiles) == L.tp_gemm_tiles(-1, None) >= 2
    for t in tiles:
        assert t["bm"] in (128, 256) and t["bn"] in (128, 256, 384)
        assert t["waves"] in (4, 8) and 3 <= t["stages"] <= 6
        # LDS: the stages of one workgroup fit the 160 KB of a CU
        assert t["stages"] * (t["bm"] + t["bn"]) * 64 <= 160 * 1024
    info = (ctypes.c_int * 4)(7, 7, 7, 7)
    assert L.tp_gemm_tiles(len(tiles), info) == len(tiles) and list(info) == [7, 7, 7, 7]
    big = [i for i, t in enumerate(tiles) if t["bm"] == t["bn"] == 256]
    # the choices the tile rule documents: 4 gpt2_small shards (768 workgroups of
    # 128 x 256) and 8 llama7b shards (256 x 256, at least two rounds of the CUs)
    for step in (0, 1, 2):
        t = tpm.tp_mlp_step_tile(step, 4, 8192, 768, 768)
        assert (tiles[t]["bm"], tiles[t]["bn"]) == (128, 256), step
    # with 3 stages (two workgroups per CU) for the 768 workgroups of the
    # per-shard steps, 4 for the shard sum's one 8192 x 768 GEMM (192 tiles,
    # one workgroup per CU)
    assert tiles[tpm.tp_mlp_step_tile(0, 4, 8192, 768, 768)]["stages"] == 3
    assert tiles[tpm.tp_mlp_step_tile(1, 4, 8192, 768, 768)]["stages"] == 3
    assert tiles[tpm.tp_mlp_step_tile(2, 4, 8192, 768, 768)]["stages"] == 4
    assert tpm.tp_mlp_step_tile(0, 8, 8192, 4096, 2048) in big
    assert tpm.tp_mlp_step_tile(1, 8, 8192, 4096, 2048) in big
    # a group sum is one GEMM of the output's size (K through every shard):
    # llama7b's 8192 x 4096 output is two rounds of 256 x 256 tiles, and so on
    assert tpm.tp_mlp_step_tile(2, 8, 8192, 4096, 2048) in big
    assert tpm.tp_mlp_step_tile(2, 8, 32768, 8192, 4096) in big
    # gpt3_175b's shard sum: 1.5 rounds of 256 x 256 tiles, two whole rounds
    # of 128 x 384 ones; its per-shard steps fill 6 and 12 rounds of 256 x 256
    t = tpm.tp_mlp_step_tile(2, 8, 2048, 12288, 6144)
    assert (tiles[t]["bm"], tiles[t]["bn"]) == (128, 384)
    assert tpm.tp_mlp_step_tile(0, 8, 2048, 12288, 6144) in big
    assert tpm.tp_mlp_step_tile(1, 8, 2048, 12288, 6144) in big
    # K = H not a multiple of 32: the ragged-K tile for any shape
    assert len({tpm.tp_mlp_step_tile(0, n, M, 200, 512) for n in (1, 4) for M in (64, 8192)}) == 1


def test_tile_hook_errors(L):
    c = _header_constants()
    st = L.tp_mlp_step_tile
    assert st(3, 4, 64, 64, 64) == c["TP_ERR_SHAPE"]
    assert st(0, 0, 64, 64, 64) == c["TP_ERR_SHAPE"]
    assert st(0, 17, 64, 64, 64) == c["TP_ERR_SHAPE"]
    assert st(1, 4, 64, 60, 64) == c["TP_ERR_SHAPE"]
    count = L.tp_gemm_tiles(-1, None)
    arr = lambda *xs: (ctypes.c_void_p * len(xs))(*xs)
    col = L.tp_mlp_col_gelu_shards_tile
    X = _p(0)
    W, b, Y = arr(P * 2, P * 3), arr(P * 4, P * 5), arr(P * 6, P * 7)
    ok = lambda: [0, X, W, b, Y, 2, 64, 256, 128, None]
    for bad in (-1, count, 1000):
        a = ok(); a[0] = bad
        assert col(*a) == c["TP_ERR_SHAPE"], bad
    a = ok(); a[7] = 200          # K = H = 200: only the ragged-K tile runs
    ragged = L.tp_mlp_step_tile(0, 2, 64, 200, 128)
    for t in range(count):
        if t != ragged:
            a[0] = t
            assert col(*a) == c["TP_ERR_SHAPE"], t
    a = ok(); a[1] = None
    assert col(*a) == c["TP_ERR_NULL"]
    a = ok(); a[4] = arr(P * 6, P * 2)    # Y[1] over W[0]
    assert col(*a) == c["TP_ERR_ALIAS"]
    a = ok(); a[6] = 0
    assert col(*a) == c["TP_OK"]
    row = L.tp_mlp_row_partial_shards_tile
    Yr, V, Z = arr(P * 2, P * 3), arr(P * 4, P * 5), arr(P * 6, P * 7)
    okr = lambda: [0, Yr, V, Z, 2, 64, 128, 256, 0, None]
    a = okr(); a[8] = 8
    assert row(*a) == c["TP_ERR_FLAGS"]
    a = okr(); a[0] = count
    assert row(*a) == c["TP_ERR_SHAPE"]
    a = okr(); a[3] = arr(None, P * 7)
    assert row(*a) == c["TP_ERR_NULL"]
    a = okr(); a[5] = 0
    assert row(*a) == c["TP_OK"]
    att = L.tp_attn_core_shards_variant
    Q, A = arr(P * 2, P * 3), arr(P * 4, P * 5)
    oka = lambda: [0, Q, A, 2, 1, 64, 2, 64, c["TP_BF16"], c["TP_CAUSAL"], None]
    for bad in (-1, 2, 100):
        a = oka(); a[0] = bad
        assert att(*a) == c["TP_ERR_SHAPE"], bad
    a = oka(); a[7] = 96
    assert att(*a) == c["TP_ERR_SHAPE"]
    a = oka(); a[9] = 4
    assert att(*a) == c["TP_ERR_FLAGS"]
    a = oka(); a[2] = arr(P * 4, None)
    assert att(*a) == c["TP_ERR_NULL"]
    a = oka(); a[2] = arr(P * 4, P * 2)   # A[1] over QKV[0]
    assert att(*a) == c["TP_ERR_ALIAS"]
    for v in (0, 1):
        a = oka(); a[0] = v; a[5] = 0
        assert att(*a) == c["TP_OK"]


def test_library_binds_torchs_hip_runtime():
    """lib() loads PyTorch before libtpmlp.so, so that the process has one HIP
    runtime (torch's) and the library's launches share torch's memory and
    streams; loaded first, the library would bind a second runtime and every
    launch would fail.  Checked in a fresh interpreter (no GPU is touched)."""
    import subprocess
    import sys
    from _helpers import gpu_initialised
    if gpu_initialised():
        pytest.skip("this process has initialised the GPU: it must not start a child interpreter")
    code = ("import os, sys, tensor_transformer_mlp_amd as t; t.lib(); import torch; "
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; "
            "d = os.path.realpath(os.path.join(os.path.dirname(torch.__file__), 'lib')); "
            "print(sorted(libs)); "
            "assert libs and all(os.path.realpath(p).startswith(d) for p in libs), libs")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_noalloc_forward_errors(L):
    """tp_mlp_shard_forward_noalloc rejects bad arguments, and shapes whose
    intermediates exceed the static scratch array, before any HIP call."""
    c = _header_constants()
    f = L.tp_mlp_shard_forward_noalloc
    arr = lambda *xs: (ctypes.c_void_p * len(xs))(*xs)
    W, V, b = arr(P * 2, P * 3), arr(P * 4, P * 5), arr(P * 6, P * 7)
    # X, W, b, V, k, M, H, Fk, dtype, Z, flags, stream
    ok = lambda: [P, W, b, V, 2, 64, 128, 256, c["TP_BF16"], P * 8, 0, None]
    a = ok(); a[8] = 7
    assert f(*a) == c["TP_ERR_DTYPE"]
    a = ok(); a[10] = 2
    assert f(*a) == c["TP_ERR_FLAGS"]
    a = ok(); a[4] = 0
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[6] = 60
    assert f(*a) == c["TP_ERR_SHAPE"]
    a = ok(); a[9] = None
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok(); a[1] = arr(P * 2, None)
    assert f(*a) == c["TP_ERR_NULL"]
    a = ok(); a[0] = P + 8
    assert f(*a) == c["TP_ERR_ALIGN"]
    a = ok(); a[5] = 0                      # M == 0: nothing to do
    assert f(*a) == c["TP_OK"]
    a = ok(); a[9] = P                      # Z over X
    assert f(*a) == c["TP_ERR_ALIAS"]
    # one shard's Y_i [32768, 4096] bf16 (268 MB) exceeds the 128 MiB array
    a = ok(); a[5], a[6], a[7] = 32768, 64, 4096
    assert f(*a) == c["TP_ERR_WORKSPACE"]
    # literal: 7 float32 partials [8192, 1024] (235 MB) do not fit; fused fits
    big = [P, arr(*[P * (10 + i) for i in range(8)]), None, arr(*[P * (30 + i) for i in range(8)]), 8,
           8192, 1024, 1024, c["TP_BF16"], P * 60, 0, None]
    assert f(*big) == c["TP_ERR_WORKSPACE"]
