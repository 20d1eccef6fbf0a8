"""MI355X (gfx950) tensor-parallel MLP shard forward and backward.

Python binding of libtpmlp.so (C ABI in include/tp_mlp.h).  The functions have
the C names and only marshal arguments: PyTorch supplies device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is not built, or a tensor is not
on the GPU, the call raises.

    Y_i = GeLU(X W_i + b_i)      tp_mlp_col_gelu
    Z_i = Y_i V_i                tp_mlp_row_partial
    Z   = sum_i Z_i              tp_shard_reduce
    all of the above, k shards   tp_mlp_shard_forward

Backward (dZ = dL/dZ):

    Y_i, G_i = GeLU(A_i), GeLU'(A_i)   tp_mlp_col_gelu_save
    dA_i = (dZ V_i^T) * G_i            tp_mlp_grad_act
    dV_i = Y_i^T dZ                    tp_mlp_grad_row_weight
    dW_i = X^T dA_i, db_i = colsum     tp_mlp_grad_col_weight
    dX_i = dA_i W_i^T                  tp_mlp_grad_input_partial
    all of the above, k shards, + dX   tp_mlp_shard_backward

Sequence parallelism (the all-reduce as a reduce-scatter over row blocks,
with the residual X added):

    O_r = X[rows of r] + sum_i Z_i[rows of r]   tp_sp_reduce_scatter
    the whole block, k shards                   tp_mlp_shard_forward_sp

SwiGLU block (Y_i = SiLU(X Wg_i) * (X Wu_i), no biases):

    Y_i                          tp_swiglu_col (tp_swiglu_col_shards)
    the whole block, k shards    tp_swiglu_shard_forward

Tensor-parallel attention (heads split over the shards):

    QKV_i = X Wqkv_i + bqkv_i          tp_attn_qkv_shards
    A_i = softmax(q k^T / sqrt d) v    tp_attn_core_shards (causal or not)
    Z = sum_i A_i Wo_i, k shards       tp_attn_shard_forward

Every per-step call has a *_shards form that runs the step for up to
TP_MAX_BATCH shards in one launch (what the k-shard calls do inside).
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

__all__ = [
    "TP_F32", "TP_BF16", "TP_ACCUMULATE", "TP_FUSED_ACCUM", "TP_MAX_SHARDS", "TpMlpError",
    "lib", "tp_status_string", "tp_mlp_version", "tp_mlp_col_gelu", "tp_mlp_row_partial",
    "tp_shard_reduce", "tp_mlp_workspace_bytes", "tp_mlp_shard_forward", "TP_GRAD_ACCUMULATE",
    "tp_mlp_col_gelu_save", "tp_mlp_grad_act", "tp_mlp_grad_weight_workspace_bytes",
    "tp_mlp_grad_row_weight", "tp_mlp_grad_col_weight", "tp_mlp_grad_input_partial",
    "tp_mlp_backward_workspace_bytes", "tp_mlp_shard_backward", "TP_SUM_SHARDS", "TP_MAX_BATCH",
    "tp_mlp_col_gelu_shards", "tp_mlp_row_partial_shards", "tp_mlp_grad_act_shards",
    "tp_mlp_grad_weight_workspace_bytes_shards", "tp_mlp_grad_row_weight_shards",
    "tp_mlp_grad_col_weight_shards", "tp_mlp_grad_input_shards",
    "tp_sp_reduce_scatter", "tp_mlp_sp_workspace_bytes", "tp_mlp_shard_forward_sp",
    "tp_swiglu_col", "tp_swiglu_col_shards", "tp_swiglu_shard_forward", "TP_CAUSAL",
    "tp_attn_qkv_shards", "tp_attn_core_shards", "tp_attn_workspace_bytes", "tp_attn_shard_forward",
    "tp_gemm_tiles", "tp_mlp_step_tile", "tp_mlp_col_gelu_shards_tile", "tp_mlp_row_partial_shards_tile",
    "tp_attn_core_shards_variant", "tp_mlp_shard_forward_noalloc", "TP_NOALLOC_SCRATCH_BYTES",
]

TP_F32 = 0
TP_BF16 = 1
TP_ACCUMULATE = 1
TP_FUSED_ACCUM = 1
TP_GRAD_ACCUMULATE = 2
TP_SUM_SHARDS = 4
TP_CAUSAL = 8
TP_MAX_SHARDS = 64
TP_MAX_BATCH = 16
TP_NOALLOC_SCRATCH_BYTES = 128 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpmlp.so")
_lib = None


class TpMlpError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (status %d)" % (where, tp_status_string(code), code))


def lib() -> ctypes.CDLL:
    """The loaded libtpmlp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtpmlp.so is not built (run `python -m tensor_transformer_mlp_amd.build`"
                               " or __graft_entry__.build()); there is no fallback path")
        # PyTorch first: its HIP runtime must be the process's one, so that the
        # library's launches and torch's allocations and streams share it
        # (loaded the other way round, the library's libamdhip64 would be
        # bound first and every launch would fail).
        _torch()
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci, cu, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
        L.tp_status_string.argtypes = [ci]
        L.tp_status_string.restype = ctypes.c_char_p
        L.tp_mlp_version.argtypes = []
        L.tp_mlp_version.restype = ci
        L.tp_mlp_col_gelu.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp]
        L.tp_mlp_col_gelu.restype = ci
        L.tp_mlp_row_partial.argtypes = [vp, vp, vp, i64, i64, i64, ci, cu, vp]
        L.tp_mlp_row_partial.restype = ci
        L.tp_shard_reduce.argtypes = [vp, ci, vp, i64, vp]
        L.tp_shard_reduce.restype = ci
        L.tp_mlp_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, cu]
        L.tp_mlp_workspace_bytes.restype = sz
        L.tp_mlp_shard_forward.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, vp, cu, vp]
        L.tp_mlp_shard_forward.restype = ci
        L.tp_mlp_shard_forward_noalloc.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, cu, vp]
        L.tp_mlp_shard_forward_noalloc.restype = ci
        L.tp_mlp_col_gelu_save.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, vp]
        L.tp_mlp_col_gelu_save.restype = ci
        L.tp_mlp_grad_act.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp]
        L.tp_mlp_grad_act.restype = ci
        L.tp_mlp_grad_weight_workspace_bytes.argtypes = [i64, i64, i64, ci]
        L.tp_mlp_grad_weight_workspace_bytes.restype = sz
        L.tp_mlp_grad_row_weight.argtypes = [vp, vp, vp, i64, i64, i64, ci, vp, sz, cu, vp]
        L.tp_mlp_grad_row_weight.restype = ci
        L.tp_mlp_grad_col_weight.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, sz, cu, vp]
        L.tp_mlp_grad_col_weight.restype = ci
        L.tp_mlp_grad_input_partial.argtypes = [vp, vp, vp, i64, i64, i64, ci, cu, vp]
        L.tp_mlp_grad_input_partial.restype = ci
        L.tp_mlp_backward_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, cu]
        L.tp_mlp_backward_workspace_bytes.restype = sz
        L.tp_mlp_shard_backward.argtypes = [vp, vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, vp, vp,
                                            vp, vp, cu, vp]
        L.tp_mlp_shard_backward.restype = ci
        L.tp_mlp_col_gelu_shards.argtypes = [vp, vp, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.tp_mlp_row_partial_shards.argtypes = [vp, vp, vp, ci, i64, i64, i64, ci, cu, vp]
        L.tp_mlp_grad_act_shards.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.tp_mlp_grad_weight_workspace_bytes_shards.argtypes = [ci, i64, i64, i64, ci]
        L.tp_mlp_grad_weight_workspace_bytes_shards.restype = sz
        L.tp_mlp_grad_row_weight_shards.argtypes = [vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, cu, vp]
        L.tp_mlp_grad_col_weight_shards.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, cu, vp]
        L.tp_mlp_grad_input_shards.argtypes = [vp, vp, vp, ci, i64, i64, i64, ci, cu, vp]
        L.tp_sp_reduce_scatter.argtypes = [vp, ci, vp, ci, vp, ci, ci, i64, i64, vp]
        L.tp_sp_reduce_scatter.restype = ci
        L.tp_mlp_sp_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, cu]
        L.tp_mlp_sp_workspace_bytes.restype = sz
        L.tp_mlp_shard_forward_sp.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, vp, ci, cu, vp]
        L.tp_mlp_shard_forward_sp.restype = ci
        L.tp_swiglu_col.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp]
        L.tp_swiglu_col.restype = ci
        L.tp_swiglu_col_shards.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.tp_swiglu_col_shards.restype = ci
        L.tp_swiglu_shard_forward.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp, sz, vp, cu, vp]
        L.tp_swiglu_shard_forward.restype = ci
        L.tp_attn_qkv_shards.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, vp]
        L.tp_attn_qkv_shards.restype = ci
        L.tp_attn_core_shards.argtypes = [vp, vp, ci, i64, i64, ci, ci, ci, cu, vp]
        L.tp_attn_core_shards.restype = ci
        L.tp_attn_core_shards_variant.argtypes = [ci, vp, vp, ci, i64, i64, ci, ci, ci, cu, vp]
        L.tp_attn_core_shards_variant.restype = ci
        L.tp_attn_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ci, cu]
        L.tp_attn_workspace_bytes.restype = sz
        L.tp_attn_shard_forward.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, ci, ci, vp, sz, vp, cu, vp]
        L.tp_attn_shard_forward.restype = ci
        L.tp_gemm_tiles.argtypes = [ci, ctypes.POINTER(ci)]
        L.tp_gemm_tiles.restype = ci
        L.tp_mlp_step_tile.argtypes = [ci, ci, i64, i64, i64]
        L.tp_mlp_step_tile.restype = ci
        L.tp_mlp_col_gelu_shards_tile.argtypes = [ci, vp, vp, vp, vp, ci, i64, i64, i64, vp]
        L.tp_mlp_col_gelu_shards_tile.restype = ci
        L.tp_mlp_row_partial_shards_tile.argtypes = [ci, vp, vp, vp, ci, i64, i64, i64, cu, vp]
        L.tp_mlp_row_partial_shards_tile.restype = ci
        for f in (L.tp_mlp_col_gelu_shards, L.tp_mlp_row_partial_shards, L.tp_mlp_grad_act_shards,
                  L.tp_mlp_grad_row_weight_shards, L.tp_mlp_grad_col_weight_shards, L.tp_mlp_grad_input_shards):
            f.restype = ci
        _lib = L
    return _lib


def tp_status_string(code: int) -> str:
    return lib().tp_status_string(int(code)).decode()


def tp_mlp_version() -> int:
    return int(lib().tp_mlp_version())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError("tensors must be torch.bfloat16 or torch.float32, got %s" % (t.dtype,))


def _dev(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_caller_stream(fn):
    """Run ``fn`` with its ``stream`` argument (when one is given) made torch's
    current stream.  Every tensor the binding allocates on the caller's behalf
    (outputs, workspaces) then belongs to the stream its kernels run on, so
    torch's caching allocator never hands such a block to other work while
    those kernels may still read or write it."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = kwargs["stream"] if "stream" in kwargs else (args[pos] if len(args) > pos else None)
        if stream is None:
            return fn(*args, **kwargs)
        with _torch().cuda.stream(stream):
            return fn(*args, **kwargs)

    return wrapper


def _check(code: int, where: str):
    if code != 0:
        raise TpMlpError(code, where)


@_on_caller_stream
def tp_mlp_col_gelu(X, W_i, b_i=None, Y_i=None, stream=None):
    """Y_i = GeLU(X W_i + b_i); X [..., H], W_i [H, Fk], b_i [Fk] or None."""
    torch = _torch()
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W_i.shape[-1]
    dt = _dtype_code(X)
    if W_i.dtype != X.dtype or (b_i is not None and b_i.dtype != X.dtype):
        raise TypeError("X, W_i and b_i must share one dtype")
    if tuple(W_i.shape) != (H, Fk) or (b_i is not None and tuple(b_i.shape) != (Fk,)):
        raise ValueError("shape mismatch: X %s, W_i %s, b_i %s" % (tuple(X.shape), tuple(W_i.shape),
                                                                  None if b_i is None else tuple(b_i.shape)))
    if Y_i is None:
        Y_i = torch.empty(*X.shape[:-1], Fk, dtype=X.dtype, device=X.device)
    elif Y_i.dtype != X.dtype or Y_i.numel() != M * Fk:
        raise ValueError("Y_i must be %s with %d elements" % (X.dtype, M * Fk))
    _check(lib().tp_mlp_col_gelu(_dev(X, "X"), _dev(W_i, "W_i"), _dev(b_i, "b_i"), _dev(Y_i, "Y_i"),
                                 M, H, Fk, dt, _stream(stream)), "tp_mlp_col_gelu")
    return Y_i


@_on_caller_stream
def tp_mlp_row_partial(Y_i, V_i, Z_i=None, accumulate: bool = False, stream=None):
    """Z_i = Y_i V_i (float32), or Z_i += Y_i V_i with accumulate=True."""
    torch = _torch()
    Fk = Y_i.shape[-1]
    M = Y_i.numel() // Fk if Fk else 0
    H = V_i.shape[-1]
    dt = _dtype_code(Y_i)
    if V_i.dtype != Y_i.dtype:
        raise TypeError("Y_i and V_i must share one dtype")
    if tuple(V_i.shape) != (Fk, H):
        raise ValueError("shape mismatch: Y_i %s, V_i %s" % (tuple(Y_i.shape), tuple(V_i.shape)))
    if Z_i is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing Z_i")
        Z_i = torch.empty(*Y_i.shape[:-1], H, dtype=torch.float32, device=Y_i.device)
    elif Z_i.dtype != torch.float32 or Z_i.numel() != M * H:
        raise ValueError("Z_i must be float32 with %d elements" % (M * H))
    _check(lib().tp_mlp_row_partial(_dev(Y_i, "Y_i"), _dev(V_i, "V_i"), _dev(Z_i, "Z_i"), M, Fk, H,
                                    dt, TP_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_row_partial")
    return Z_i


@_on_caller_stream
def tp_shard_reduce(parts, Z=None, stream=None):
    """Z = parts[0] + parts[1] + ... (float32, left to right).  Z may be parts[0]."""
    torch = _torch()
    k = len(parts)
    if k < 1:
        raise ValueError("need at least one partial")
    n = parts[0].numel()
    for p in parts:
        if p.dtype != torch.float32 or p.numel() != n:
            raise ValueError("partials must be float32 tensors of one size")
    if Z is None:
        Z = torch.empty_like(parts[0])
    elif Z.dtype != torch.float32 or Z.numel() != n:
        raise ValueError("Z must be float32 with %d elements" % n)
    ptrs = (ctypes.c_void_p * k)(*[_dev(p, "parts[%d]" % i) for i, p in enumerate(parts)])
    _check(lib().tp_shard_reduce(ptrs, k, _dev(Z, "Z"), n, _stream(stream)), "tp_shard_reduce")
    return Z


def tp_mlp_workspace_bytes(k: int, M: int, H: int, Fk: int, dtype: int, flags: int = 0) -> int:
    return int(lib().tp_mlp_workspace_bytes(k, M, H, Fk, dtype, flags))


@_on_caller_stream
def tp_mlp_shard_forward(X, W, b, V, Z=None, workspace=None, fused: bool = False, stream=None):
    """Z = sum_i GeLU(X W[i] + b[i]) V[i] over the k shards in the lists W, b, V.

    ``b`` may be None (no bias).  ``workspace`` is a uint8 GPU tensor of at
    least tp_mlp_workspace_bytes(...) bytes; it is allocated if None.
    """
    torch = _torch()
    k = len(W)
    if k < 1 or len(V) != k or (b is not None and len(b) != k):
        raise ValueError("W, V (and b) must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    dt = _dtype_code(X)
    for i in range(k):
        if tuple(W[i].shape) != (H, Fk) or tuple(V[i].shape) != (Fk, H) or \
                (b is not None and tuple(b[i].shape) != (Fk,)):
            raise ValueError("shard %d has the wrong shape" % i)
        if W[i].dtype != X.dtype or V[i].dtype != X.dtype or (b is not None and b[i].dtype != X.dtype):
            raise TypeError("shard %d has the wrong dtype" % i)
    flags = TP_FUSED_ACCUM if fused else 0
    need = tp_mlp_workspace_bytes(k, M, H, Fk, dt, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    if Z is None:
        Z = torch.empty(*X.shape[:-1], H, dtype=torch.float32, device=X.device)
    elif Z.dtype != torch.float32 or Z.numel() != M * H:
        raise ValueError("Z must be float32 with %d elements" % (M * H))
    Wp = (ctypes.c_void_p * k)(*[_dev(w, "W[%d]" % i) for i, w in enumerate(W)])
    Vp = (ctypes.c_void_p * k)(*[_dev(v, "V[%d]" % i) for i, v in enumerate(V)])
    bp = None if b is None else (ctypes.c_void_p * k)(*[_dev(x, "b[%d]" % i) for i, x in enumerate(b)])
    _check(lib().tp_mlp_shard_forward(_dev(X, "X"), Wp, bp, Vp, k, M, H, Fk, dt,
                                      _dev(workspace, "workspace"), workspace.numel(), _dev(Z, "Z"),
                                      flags, _stream(stream)), "tp_mlp_shard_forward")
    return Z



@_on_caller_stream
def tp_mlp_shard_forward_noalloc(X, W, b, V, Z=None, fused: bool = False, stream=None):
    """tp_mlp_shard_forward without a workspace: the library keeps the
    intermediates in its static device scratch array (TP_NOALLOC_SCRATCH_BYTES
    per GPU) and the call allocates no device memory (only Z, when it is not
    given, is allocated here before the call).  Calls that overlap in time on
    one GPU share that array and must be ordered by the caller."""
    torch = _torch()
    k = len(W)
    if k < 1 or len(V) != k or (b is not None and len(b) != k):
        raise ValueError("W, V (and b) must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    dt = _dtype_code(X)
    if Z is None:
        Z = torch.empty(*X.shape[:-1], H, dtype=torch.float32, device=X.device)
    elif Z.dtype != torch.float32 or Z.numel() != M * H:
        raise ValueError("Z must be float32 with %d elements" % (M * H))
    Wp = (ctypes.c_void_p * k)(*[_dev(w, "W[%d]" % i) for i, w in enumerate(W)])
    Vp = (ctypes.c_void_p * k)(*[_dev(v, "V[%d]" % i) for i, v in enumerate(V)])
    bp = None if b is None else (ctypes.c_void_p * k)(*[_dev(x, "b[%d]" % i) for i, x in enumerate(b)])
    _check(lib().tp_mlp_shard_forward_noalloc(_dev(X, "X"), Wp, bp, Vp, k, M, H, Fk, dt, _dev(Z, "Z"),
                                              TP_FUSED_ACCUM if fused else 0, _stream(stream)),
           "tp_mlp_shard_forward_noalloc")
    return Z

def _same_dtype(where, ref, *ts):
    for t in ts:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError("%s: every operand must be %s" % (where, ref.dtype))


def _out(t, shape, dtype, device, name):
    torch = _torch()
    n = 1
    for d in shape:
        n *= d
    if t is None:
        return torch.empty(*shape, dtype=dtype, device=device)
    if t.dtype != dtype or t.numel() != n:
        raise ValueError("%s must be %s with %d elements" % (name, dtype, n))
    return t


def _workspace(t, need, device):
    torch = _torch()
    if t is None:
        t = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return t


@_on_caller_stream
def tp_mlp_col_gelu_save(X, W_i, b_i=None, Y_i=None, G_i=None, stream=None):
    """Y_i = GeLU(A_i), G_i = GeLU'(A_i) with A_i = X W_i + b_i.  Returns (Y_i, G_i)."""
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W_i.shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_mlp_col_gelu_save", X, W_i, b_i)
    if tuple(W_i.shape) != (H, Fk) or (b_i is not None and tuple(b_i.shape) != (Fk,)):
        raise ValueError("shape mismatch: X %s, W_i %s" % (tuple(X.shape), tuple(W_i.shape)))
    Y_i = _out(Y_i, (M, Fk), X.dtype, X.device, "Y_i")
    G_i = _out(G_i, (M, Fk), X.dtype, X.device, "G_i")
    _check(lib().tp_mlp_col_gelu_save(_dev(X, "X"), _dev(W_i, "W_i"), _dev(b_i, "b_i"), _dev(Y_i, "Y_i"),
                                      _dev(G_i, "G_i"), M, H, Fk, dt, _stream(stream)),
           "tp_mlp_col_gelu_save")
    return Y_i, G_i


@_on_caller_stream
def tp_mlp_grad_act(dZ, V_i, G_i, dA_i=None, stream=None):
    """dA_i = (dZ V_i^T) * G_i; dA_i may be G_i (in place)."""
    H = dZ.shape[-1]
    M = dZ.numel() // H if H else 0
    Fk = V_i.shape[0]
    dt = _dtype_code(dZ)
    _same_dtype("tp_mlp_grad_act", dZ, V_i, G_i, dA_i)
    if tuple(V_i.shape) != (Fk, H) or G_i.numel() != M * Fk:
        raise ValueError("shape mismatch: dZ %s, V_i %s, G_i %s" % (tuple(dZ.shape), tuple(V_i.shape),
                                                                   tuple(G_i.shape)))
    dA_i = _out(dA_i, (M, Fk), dZ.dtype, dZ.device, "dA_i")
    _check(lib().tp_mlp_grad_act(_dev(dZ, "dZ"), _dev(V_i, "V_i"), _dev(G_i, "G_i"), _dev(dA_i, "dA_i"),
                                 M, H, Fk, dt, _stream(stream)), "tp_mlp_grad_act")
    return dA_i


def tp_mlp_grad_weight_workspace_bytes(M: int, H: int, Fk: int, dtype: int) -> int:
    return int(lib().tp_mlp_grad_weight_workspace_bytes(M, H, Fk, dtype))


@_on_caller_stream
def tp_mlp_grad_row_weight(Y_i, dZ, dV_i=None, workspace=None, accumulate: bool = False, stream=None):
    """dV_i = Y_i^T dZ (float32), or dV_i += ... with accumulate=True."""
    torch = _torch()
    Fk = Y_i.shape[-1]
    M = Y_i.numel() // Fk if Fk else 0
    H = dZ.shape[-1]
    dt = _dtype_code(Y_i)
    _same_dtype("tp_mlp_grad_row_weight", Y_i, dZ)
    if dZ.numel() != M * H:
        raise ValueError("shape mismatch: Y_i %s, dZ %s" % (tuple(Y_i.shape), tuple(dZ.shape)))
    if dV_i is None and accumulate:
        raise ValueError("accumulate=True needs an existing dV_i")
    dV_i = _out(dV_i, (Fk, H), torch.float32, Y_i.device, "dV_i")
    need = tp_mlp_grad_weight_workspace_bytes(M, H, Fk, dt)
    workspace = _workspace(workspace, need, Y_i.device)
    _check(lib().tp_mlp_grad_row_weight(_dev(Y_i, "Y_i"), _dev(dZ, "dZ"), _dev(dV_i, "dV_i"), M, Fk, H, dt,
                                        _dev(workspace, "workspace"), workspace.numel(),
                                        TP_GRAD_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_grad_row_weight")
    return dV_i


@_on_caller_stream
def tp_mlp_grad_col_weight(X, dA_i, dW_i=None, db_i=None, want_db: bool = True, workspace=None,
                           accumulate: bool = False, stream=None):
    """dW_i = X^T dA_i and db_i = sum over rows of dA_i (float32).  Returns (dW_i, db_i)."""
    torch = _torch()
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = dA_i.shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_mlp_grad_col_weight", X, dA_i)
    if dA_i.numel() != M * Fk:
        raise ValueError("shape mismatch: X %s, dA_i %s" % (tuple(X.shape), tuple(dA_i.shape)))
    if accumulate and (dW_i is None or (want_db and db_i is None)):
        raise ValueError("accumulate=True needs existing dW_i (and db_i)")
    dW_i = _out(dW_i, (H, Fk), torch.float32, X.device, "dW_i")
    if want_db:
        db_i = _out(db_i, (Fk,), torch.float32, X.device, "db_i")
    need = tp_mlp_grad_weight_workspace_bytes(M, H, Fk, dt)
    workspace = _workspace(workspace, need, X.device)
    _check(lib().tp_mlp_grad_col_weight(_dev(X, "X"), _dev(dA_i, "dA_i"), _dev(dW_i, "dW_i"),
                                        _dev(db_i, "db_i") if want_db else None, M, H, Fk, dt,
                                        _dev(workspace, "workspace"), workspace.numel(),
                                        TP_GRAD_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_grad_col_weight")
    return dW_i, (db_i if want_db else None)


@_on_caller_stream
def tp_mlp_grad_input_partial(dA_i, W_i, dX_i=None, accumulate: bool = False, stream=None):
    """dX_i = dA_i W_i^T (float32), or dX_i += ... with accumulate=True."""
    torch = _torch()
    Fk = dA_i.shape[-1]
    M = dA_i.numel() // Fk if Fk else 0
    H = W_i.shape[0]
    dt = _dtype_code(dA_i)
    _same_dtype("tp_mlp_grad_input_partial", dA_i, W_i)
    if tuple(W_i.shape) != (H, Fk):
        raise ValueError("shape mismatch: dA_i %s, W_i %s" % (tuple(dA_i.shape), tuple(W_i.shape)))
    if dX_i is None and accumulate:
        raise ValueError("accumulate=True needs an existing dX_i")
    dX_i = _out(dX_i, (M, H), torch.float32, dA_i.device, "dX_i")
    _check(lib().tp_mlp_grad_input_partial(_dev(dA_i, "dA_i"), _dev(W_i, "W_i"), _dev(dX_i, "dX_i"), M, Fk,
                                           H, dt, TP_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_grad_input_partial")
    return dX_i


def tp_mlp_backward_workspace_bytes(k: int, M: int, H: int, Fk: int, dtype: int, flags: int = 0) -> int:
    return int(lib().tp_mlp_backward_workspace_bytes(k, M, H, Fk, dtype, flags))


@_on_caller_stream
def tp_mlp_shard_backward(X, W, b, V, dZ, dX=None, dW=None, db=None, dV=None, want_db: bool = True,
                          workspace=None, fused: bool = False, accumulate: bool = False, stream=None):
    """Gradients of Z = sum_i GeLU(X W[i] + b[i]) V[i] for dZ = dL/dZ.

    Returns (dX, dW, db, dV): dX [M, H] and per-shard lists dW[i] [H, Fk],
    db[i] [Fk] (None when b is None or want_db is False) and dV[i] [Fk, H], all
    float32.  ``fused`` folds the dX shard sum into the GEMMs; ``accumulate``
    adds into the given dW, db, dV.
    """
    torch = _torch()
    k = len(W)
    if k < 1 or len(V) != k or (b is not None and len(b) != k):
        raise ValueError("W, V (and b) must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_mlp_shard_backward", X, dZ, *W, *V, *(b or []))
    if dZ.numel() != M * H:
        raise ValueError("dZ must have %d elements" % (M * H))
    for i in range(k):
        if tuple(W[i].shape) != (H, Fk) or tuple(V[i].shape) != (Fk, H) or \
                (b is not None and tuple(b[i].shape) != (Fk,)):
            raise ValueError("shard %d has the wrong shape" % i)
    want_db = want_db and b is not None
    if accumulate and (dW is None or dV is None or (want_db and db is None)):
        raise ValueError("accumulate=True needs existing dW, dV (and db)")
    dX = _out(dX, (M, H), torch.float32, X.device, "dX")
    dW = [_out(None if dW is None else dW[i], (H, Fk), torch.float32, X.device, "dW[%d]" % i) for i in range(k)]
    dV = [_out(None if dV is None else dV[i], (Fk, H), torch.float32, X.device, "dV[%d]" % i) for i in range(k)]
    if want_db:
        db = [_out(None if db is None else db[i], (Fk,), torch.float32, X.device, "db[%d]" % i) for i in range(k)]
    else:
        db = None
    flags = (TP_FUSED_ACCUM if fused else 0) | (TP_GRAD_ACCUMULATE if accumulate else 0)
    need = tp_mlp_backward_workspace_bytes(k, M, H, Fk, dt, flags)
    workspace = _workspace(workspace, need, X.device)
    arr = lambda ts, name: (ctypes.c_void_p * k)(*[_dev(t, "%s[%d]" % (name, i)) for i, t in enumerate(ts)])
    _check(lib().tp_mlp_shard_backward(_dev(X, "X"), arr(W, "W"), None if b is None else arr(b, "b"), arr(V, "V"),
                                       _dev(dZ, "dZ"), k, M, H, Fk, dt, _dev(workspace, "workspace"),
                                       workspace.numel(), _dev(dX, "dX"), arr(dW, "dW"),
                                       None if db is None else arr(db, "db"), arr(dV, "dV"), flags,
                                       _stream(stream)), "tp_mlp_shard_backward")
    return dX, dW, db, dV


# ---------------------------------------------------------------------------
# Batched steps: one launch for n <= TP_MAX_BATCH shards.

def _ptrs(ts, name, allow_none=False):
    if ts is None:
        return None
    vals = []
    for i, t in enumerate(ts):
        if t is None and allow_none:
            vals.append(None)
        else:
            vals.append(_dev(t, "%s[%d]" % (name, i)))
    return (ctypes.c_void_p * len(vals))(*vals)


def _batch_n(n):
    if not 1 <= n <= TP_MAX_BATCH:
        raise ValueError("a batch holds 1..%d shards, got %d" % (TP_MAX_BATCH, n))
    return n


@_on_caller_stream
def tp_mlp_col_gelu_shards(X, W, b, Y, G=None, stream=None):
    """Y[i] = GeLU(X W[i] + b[i]) (and G[i] = GeLU'(.) when G is given) for
    every shard i of the lists, in one launch; b may be None."""
    n = _batch_n(len(W))
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    _check(lib().tp_mlp_col_gelu_shards(_dev(X, "X"), _ptrs(W, "W"), _ptrs(b, "b"), _ptrs(Y, "Y"),
                                        _ptrs(G, "G"), n, M, H, Fk, _dtype_code(X), _stream(stream)),
           "tp_mlp_col_gelu_shards")
    return Y, G


@_on_caller_stream
def tp_mlp_row_partial_shards(Y, V, Z, sum_shards=False, accumulate=False, stream=None):
    """Z[i] (+)= Y[i] V[i] for every shard, or Z[0] (+)= sum_i Y[i] V[i] in shard
    order with sum_shards=True (Z may then hold just Z[0])."""
    n = _batch_n(len(Y))
    Fk = Y[0].shape[-1]
    M = Y[0].numel() // Fk if Fk else 0
    H = V[0].shape[-1]
    Zl = list(Z) + [None] * (n - len(Z)) if sum_shards else list(Z)
    flags = (TP_SUM_SHARDS if sum_shards else 0) | (TP_ACCUMULATE if accumulate else 0)
    _check(lib().tp_mlp_row_partial_shards(_ptrs(Y, "Y"), _ptrs(V, "V"), _ptrs(Zl, "Z", allow_none=True), n,
                                           M, Fk, H, _dtype_code(Y[0]), flags, _stream(stream)),
           "tp_mlp_row_partial_shards")
    return Z


@_on_caller_stream
def tp_mlp_grad_act_shards(dZ, V, G, dA, stream=None):
    """dA[i] = (dZ V[i]^T) * G[i] for every shard (dA[i] may be G[i])."""
    n = _batch_n(len(V))
    H = dZ.shape[-1]
    M = dZ.numel() // H if H else 0
    Fk = V[0].shape[0]
    _check(lib().tp_mlp_grad_act_shards(_dev(dZ, "dZ"), _ptrs(V, "V"), _ptrs(G, "G"), _ptrs(dA, "dA"), n, M, H,
                                        Fk, _dtype_code(dZ), _stream(stream)), "tp_mlp_grad_act_shards")
    return dA


def tp_mlp_grad_weight_workspace_bytes_shards(n: int, M: int, H: int, Fk: int, dtype: int) -> int:
    return int(lib().tp_mlp_grad_weight_workspace_bytes_shards(n, M, H, Fk, dtype))


@_on_caller_stream
def tp_mlp_grad_row_weight_shards(Y, dZ, dV, workspace=None, accumulate=False, stream=None):
    """dV[i] (+)= Y[i]^T dZ for every shard."""
    n = _batch_n(len(Y))
    Fk = Y[0].shape[-1]
    M = Y[0].numel() // Fk if Fk else 0
    H = dZ.shape[-1]
    dt = _dtype_code(dZ)
    workspace = _workspace(workspace, tp_mlp_grad_weight_workspace_bytes_shards(n, M, H, Fk, dt), dZ.device)
    _check(lib().tp_mlp_grad_row_weight_shards(_ptrs(Y, "Y"), _dev(dZ, "dZ"), _ptrs(dV, "dV"), n, M, Fk, H, dt,
                                               _dev(workspace, "workspace"), workspace.numel(),
                                               TP_GRAD_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_grad_row_weight_shards")
    return dV


@_on_caller_stream
def tp_mlp_grad_col_weight_shards(X, dA, dW, db=None, workspace=None, accumulate=False, stream=None):
    """dW[i] (+)= X^T dA[i] and db[i] (+)= colsum(dA[i]) for every shard."""
    n = _batch_n(len(dA))
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = dA[0].shape[-1]
    dt = _dtype_code(X)
    workspace = _workspace(workspace, tp_mlp_grad_weight_workspace_bytes_shards(n, M, H, Fk, dt), X.device)
    _check(lib().tp_mlp_grad_col_weight_shards(_dev(X, "X"), _ptrs(dA, "dA"), _ptrs(dW, "dW"), _ptrs(db, "db"),
                                               n, M, H, Fk, dt, _dev(workspace, "workspace"), workspace.numel(),
                                               TP_GRAD_ACCUMULATE if accumulate else 0, _stream(stream)),
           "tp_mlp_grad_col_weight_shards")
    return dW, db


@_on_caller_stream
def tp_mlp_grad_input_shards(dA, W, dX, sum_shards=False, accumulate=False, stream=None):
    """dX[i] (+)= dA[i] W[i]^T for every shard, or the shard-order sum into dX[0]."""
    n = _batch_n(len(dA))
    Fk = dA[0].shape[-1]
    M = dA[0].numel() // Fk if Fk else 0
    H = W[0].shape[0]
    dXl = list(dX) + [None] * (n - len(dX)) if sum_shards else list(dX)
    flags = (TP_SUM_SHARDS if sum_shards else 0) | (TP_ACCUMULATE if accumulate else 0)
    _check(lib().tp_mlp_grad_input_shards(_ptrs(dA, "dA"), _ptrs(W, "W"), _ptrs(dXl, "dX", allow_none=True), n,
                                          M, Fk, H, _dtype_code(dA[0]), flags, _stream(stream)),
           "tp_mlp_grad_input_shards")
    return dX


# ---------------------------------------------------------------------------
# Sequence parallelism.

def _sp_blocks(O, k, Mb, H, dtype, device):
    """k output blocks [Mb, H]: a list of tensors, or views of one [k Mb, H] tensor."""
    torch = _torch()
    if O is None:
        O = torch.empty(k * Mb, H, dtype=dtype, device=device)
    if isinstance(O, (list, tuple)):
        if len(O) != k:
            raise ValueError("need k = %d output blocks" % k)
        blocks = list(O)
    else:
        if O.dtype != dtype or O.numel() != k * Mb * H or not O.is_contiguous():
            raise ValueError("O must be a contiguous %s tensor of %d elements" % (dtype, k * Mb * H))
        blocks = [O.view(k * Mb, H)[r * Mb:(r + 1) * Mb] for r in range(k)]
    for r, t in enumerate(blocks):
        if t.dtype != dtype or t.numel() != Mb * H:
            raise ValueError("block %d must be %s with %d elements" % (r, dtype, Mb * H))
    return O, blocks


@_on_caller_stream
def tp_sp_reduce_scatter(parts, k: int, R=None, O=None, out_dtype=None, stream=None):
    """Blocks O_r = R[rows of r] + sum_i parts[i][rows of r] for the k ranks.

    ``parts``: float32 [M, H] tensors; ``R``: [M, H] bf16/float32 or None;
    ``O``: None (a new [M, H] tensor), one [M, H] tensor (the gathered
    blocks) or a list of k [M/k, H] tensors.  ``out_dtype`` defaults to
    float32.  Returns O.
    """
    torch = _torch()
    if not parts:
        raise ValueError("need at least one partial")
    M, H = parts[0].shape[0], parts[0].shape[-1]
    for p in parts:
        if p.dtype != torch.float32 or tuple(p.shape) != (M, H):
            raise ValueError("partials must be float32 [M, H] tensors of one shape")
    if R is not None and tuple(R.shape) != (M, H):
        raise ValueError("R must be [M, H]")
    if k < 1 or M % k:
        raise ValueError("k must divide M")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    O, blocks = _sp_blocks(O, k, M // k, H, out_dtype, parts[0].device)
    pp = (ctypes.c_void_p * len(parts))(*[_dev(p, "parts[%d]" % i) for i, p in enumerate(parts)])
    po = (ctypes.c_void_p * k)(*[_dev(t, "O[%d]" % r) for r, t in enumerate(blocks)])
    _check(lib().tp_sp_reduce_scatter(pp, len(parts), _dev(R, "R"), _dtype_code(R) if R is not None else TP_F32,
                                      po, TP_BF16 if out_dtype == torch.bfloat16 else TP_F32, k, M, H,
                                      _stream(stream)), "tp_sp_reduce_scatter")
    return O


def tp_mlp_sp_workspace_bytes(k: int, M: int, H: int, Fk: int, dtype: int, flags: int = 0) -> int:
    return int(lib().tp_mlp_sp_workspace_bytes(k, M, H, Fk, dtype, flags))


@_on_caller_stream
def tp_mlp_shard_forward_sp(X, W, b, V, O=None, out_dtype=None, workspace=None, fused: bool = False,
                            stream=None):
    """Sequence-parallel block forward: O_r = X[rows of r] + Z[rows of r] with
    Z = sum_i GeLU(X W[i] + b[i]) V[i]; O as for tp_sp_reduce_scatter."""
    torch = _torch()
    k = len(W)
    if k < 1 or len(V) != k or (b is not None and len(b) != k):
        raise ValueError("W, V (and b) must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_mlp_shard_forward_sp", X, *W, *V, *(b or []))
    for i in range(k):
        if tuple(W[i].shape) != (H, Fk) or tuple(V[i].shape) != (Fk, H) or \
                (b is not None and tuple(b[i].shape) != (Fk,)):
            raise ValueError("shard %d has the wrong shape" % i)
    if M % k:
        raise ValueError("k must divide M")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    O, blocks = _sp_blocks(O, k, M // k, H, out_dtype, X.device)
    flags = TP_FUSED_ACCUM if fused else 0
    need = tp_mlp_sp_workspace_bytes(k, M, H, Fk, dt, flags)
    workspace = _workspace(workspace, need, X.device)
    Wp = (ctypes.c_void_p * k)(*[_dev(w, "W[%d]" % i) for i, w in enumerate(W)])
    Vp = (ctypes.c_void_p * k)(*[_dev(v, "V[%d]" % i) for i, v in enumerate(V)])
    bp = None if b is None else (ctypes.c_void_p * k)(*[_dev(x, "b[%d]" % i) for i, x in enumerate(b)])
    po = (ctypes.c_void_p * k)(*[_dev(t, "O[%d]" % r) for r, t in enumerate(blocks)])
    _check(lib().tp_mlp_shard_forward_sp(_dev(X, "X"), Wp, bp, Vp, k, M, H, Fk, dt,
                                         _dev(workspace, "workspace"), workspace.numel(), po,
                                         TP_BF16 if out_dtype == torch.bfloat16 else TP_F32, flags,
                                         _stream(stream)), "tp_mlp_shard_forward_sp")
    return O


# ---------------------------------------------------------------------------
# SwiGLU block.

@_on_caller_stream
def tp_swiglu_col(X, Wg_i, Wu_i, Y_i=None, stream=None):
    """Y_i = SiLU(X Wg_i) * (X Wu_i); X [..., H], Wg_i and Wu_i [H, Fk]."""
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = Wg_i.shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_swiglu_col", X, Wg_i, Wu_i, Y_i)
    if tuple(Wg_i.shape) != (H, Fk) or tuple(Wu_i.shape) != (H, Fk):
        raise ValueError("shape mismatch: X %s, Wg_i %s, Wu_i %s" % (tuple(X.shape), tuple(Wg_i.shape),
                                                                    tuple(Wu_i.shape)))
    Y_i = _out(Y_i, (M, Fk), X.dtype, X.device, "Y_i")
    _check(lib().tp_swiglu_col(_dev(X, "X"), _dev(Wg_i, "Wg_i"), _dev(Wu_i, "Wu_i"), _dev(Y_i, "Y_i"), M, H, Fk,
                               dt, _stream(stream)), "tp_swiglu_col")
    return Y_i


@_on_caller_stream
def tp_swiglu_col_shards(X, Wg, Wu, Y, stream=None):
    """tp_swiglu_col for the n shards of the lists Wg, Wu, Y in one launch."""
    n = len(Wg)
    if n < 1 or len(Wu) != n or len(Y) != n:
        raise ValueError("Wg, Wu and Y must hold the same number n >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = Wg[0].shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_swiglu_col_shards", X, *Wg, *Wu, *Y)
    for i in range(n):
        if tuple(Wg[i].shape) != (H, Fk) or tuple(Wu[i].shape) != (H, Fk) or Y[i].numel() != M * Fk:
            raise ValueError("shard %d has the wrong shape" % i)
    arr = lambda ts, nm: (ctypes.c_void_p * n)(*[_dev(t, "%s[%d]" % (nm, i)) for i, t in enumerate(ts)])
    _check(lib().tp_swiglu_col_shards(_dev(X, "X"), arr(Wg, "Wg"), arr(Wu, "Wu"), arr(Y, "Y"), n, M, H, Fk, dt,
                                      _stream(stream)), "tp_swiglu_col_shards")
    return Y


@_on_caller_stream
def tp_swiglu_shard_forward(X, Wg, Wu, V, Z=None, workspace=None, fused: bool = False, stream=None):
    """Z = sum_i (SiLU(X Wg[i]) * (X Wu[i])) V[i] over the k shards."""
    torch = _torch()
    k = len(Wg)
    if k < 1 or len(Wu) != k or len(V) != k:
        raise ValueError("Wg, Wu and V must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = Wg[0].shape[-1]
    dt = _dtype_code(X)
    _same_dtype("tp_swiglu_shard_forward", X, *Wg, *Wu, *V)
    for i in range(k):
        if tuple(Wg[i].shape) != (H, Fk) or tuple(Wu[i].shape) != (H, Fk) or tuple(V[i].shape) != (Fk, H):
            raise ValueError("shard %d has the wrong shape" % i)
    flags = TP_FUSED_ACCUM if fused else 0
    need = tp_mlp_workspace_bytes(k, M, H, Fk, dt, flags)
    workspace = _workspace(workspace, need, X.device)
    Z = _out(Z, (M, H), torch.float32, X.device, "Z")
    arr = lambda ts, nm: (ctypes.c_void_p * k)(*[_dev(t, "%s[%d]" % (nm, i)) for i, t in enumerate(ts)])
    _check(lib().tp_swiglu_shard_forward(_dev(X, "X"), arr(Wg, "Wg"), arr(Wu, "Wu"), arr(V, "V"), k, M, H, Fk, dt,
                                         _dev(workspace, "workspace"), workspace.numel(), _dev(Z, "Z"), flags,
                                         _stream(stream)), "tp_swiglu_shard_forward")
    return Z


# ---------------------------------------------------------------------------
# Tensor-parallel attention.

@_on_caller_stream
def tp_attn_qkv_shards(X, Wqkv, bqkv, QKV, stream=None):
    """QKV[i] = X Wqkv[i] + bqkv[i] for the n shards (bqkv may be None)."""
    n = len(Wqkv)
    if n < 1 or len(QKV) != n or (bqkv is not None and len(bqkv) != n):
        raise ValueError("Wqkv, QKV (and bqkv) must hold the same number n >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    N3 = Wqkv[0].shape[-1]
    if N3 % 3:
        raise ValueError("Wqkv must have 3 Hk columns")
    _same_dtype("tp_attn_qkv_shards", X, *Wqkv, *QKV, *(bqkv or []))
    for i in range(n):
        if tuple(Wqkv[i].shape) != (H, N3) or QKV[i].numel() != M * N3 or \
                (bqkv is not None and tuple(bqkv[i].shape) != (N3,)):
            raise ValueError("shard %d has the wrong shape" % i)
    _check(lib().tp_attn_qkv_shards(_dev(X, "X"), _ptrs(Wqkv, "Wqkv"), None if bqkv is None else _ptrs(bqkv, "bqkv"),
                                    _ptrs(QKV, "QKV"), n, M, H, N3 // 3, _dtype_code(X), _stream(stream)),
           "tp_attn_qkv_shards")
    return QKV


@_on_caller_stream
def tp_attn_core_shards(QKV, A, B: int, S: int, heads: int, head_dim: int, causal: bool = True, stream=None):
    """A[i] = the attention of shard i's heads from its projection QKV[i]."""
    return _attn_core(-1, QKV, A, B, S, heads, head_dim, causal, stream)


@_on_caller_stream
def tp_attn_core_shards_variant(variant: int, QKV, A, B: int, S: int, heads: int, head_dim: int,
                                causal: bool = True, stream=None):
    """tp_attn_core_shards with attention kernel `variant` (0: one query group per wave, 1: two; a
    measurement hook)."""
    return _attn_core(variant, QKV, A, B, S, heads, head_dim, causal, stream)


def _attn_core(variant, QKV, A, B, S, heads, head_dim, causal, stream):
    n = len(QKV)
    if n < 1 or len(A) != n:
        raise ValueError("QKV and A must hold the same number n >= 1 of shards")
    Hk = heads * head_dim
    for i in range(n):
        if QKV[i].numel() != B * S * 3 * Hk or A[i].numel() != B * S * Hk:
            raise ValueError("shard %d has the wrong size" % i)
    _same_dtype("tp_attn_core_shards", QKV[0], *QKV, *A)
    flags = TP_CAUSAL if causal else 0
    if variant < 0:
        st = lib().tp_attn_core_shards(_ptrs(QKV, "QKV"), _ptrs(A, "A"), n, B, S, heads, head_dim,
                                       _dtype_code(QKV[0]), flags, _stream(stream))
    else:
        st = lib().tp_attn_core_shards_variant(variant, _ptrs(QKV, "QKV"), _ptrs(A, "A"), n, B, S, heads,
                                               head_dim, _dtype_code(QKV[0]), flags, _stream(stream))
    _check(st, "tp_attn_core_shards" if variant < 0 else "tp_attn_core_shards_variant")
    return A


def tp_attn_workspace_bytes(k: int, B: int, S: int, H: int, n_heads: int, dtype: int, flags: int = 0) -> int:
    return int(lib().tp_attn_workspace_bytes(k, B, S, H, n_heads, dtype, flags))


@_on_caller_stream
def tp_attn_shard_forward(X, Wqkv, bqkv, Wo, B: int, S: int, n_heads: int, Z=None, workspace=None,
                          fused: bool = False, causal: bool = True, stream=None):
    """Z = sum_i A_i Wo[i] over the k shards of the attention block; X [B S, H]."""
    torch = _torch()
    k = len(Wqkv)
    if k < 1 or len(Wo) != k or (bqkv is not None and len(bqkv) != k):
        raise ValueError("Wqkv, Wo (and bqkv) must hold the same number k >= 1 of shards")
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    if M != B * S:
        raise ValueError("X must hold B S rows")
    dt = _dtype_code(X)
    _same_dtype("tp_attn_shard_forward", X, *Wqkv, *Wo, *(bqkv or []))
    flags = (TP_FUSED_ACCUM if fused else 0) | (TP_CAUSAL if causal else 0)
    need = tp_attn_workspace_bytes(k, B, S, H, n_heads, dt, flags)
    workspace = _workspace(workspace, need, X.device)
    Z = _out(Z, (M, H), torch.float32, X.device, "Z")
    _check(lib().tp_attn_shard_forward(_dev(X, "X"), _ptrs(Wqkv, "Wqkv"), None if bqkv is None else _ptrs(bqkv, "bqkv"),
                                       _ptrs(Wo, "Wo"), k, B, S, H, n_heads, dt, _dev(workspace, "workspace"),
                                       workspace.numel(), _dev(Z, "Z"), flags, _stream(stream)),
           "tp_attn_shard_forward")
    return Z


# Tile table of the bf16 GEMM (measurement of the tile choice).

def tp_gemm_tiles():
    """The bf16 GEMM's tiles: a list of {"bm", "bn", "waves", "stages"}, index = tile id."""
    L = lib()
    count = L.tp_gemm_tiles(-1, None)
    out = []
    for t in range(count):
        info = (ctypes.c_int * 4)()
        L.tp_gemm_tiles(t, info)
        out.append({"bm": info[0], "bn": info[1], "waves": info[2], "stages": info[3]})
    return out


def tp_mlp_step_tile(step: int, n: int, M: int, H: int, Fk: int) -> int:
    """The tile the bf16 step runs with: step 0 column (bias + GeLU), 1 row
    partials, 2 row with the shard sum; n shards of M x H x Fk."""
    r = lib().tp_mlp_step_tile(step, n, M, H, Fk)
    _check(min(r, 0), "tp_mlp_step_tile")
    return r


@_on_caller_stream
def tp_mlp_col_gelu_shards_tile(tile, X, W, b, Y, stream=None):
    """tp_mlp_col_gelu_shards (bf16, no G) with tile `tile` of tp_gemm_tiles()."""
    n = _batch_n(len(W))
    H = X.shape[-1]
    M = X.numel() // H if H else 0
    Fk = W[0].shape[-1]
    _check(lib().tp_mlp_col_gelu_shards_tile(tile, _dev(X, "X"), _ptrs(W, "W"), _ptrs(b, "b"), _ptrs(Y, "Y"),
                                             n, M, H, Fk, _stream(stream)), "tp_mlp_col_gelu_shards_tile")
    return Y


@_on_caller_stream
def tp_mlp_row_partial_shards_tile(tile, Y, V, Z, sum_shards=False, accumulate=False, stream=None):
    """tp_mlp_row_partial_shards (bf16) with tile `tile` of tp_gemm_tiles()."""
    n = _batch_n(len(Y))
    Fk = Y[0].shape[-1]
    M = Y[0].numel() // Fk if Fk else 0
    H = V[0].shape[-1]
    Zl = list(Z) + [None] * (n - len(Z)) if sum_shards else list(Z)
    flags = (TP_SUM_SHARDS if sum_shards else 0) | (TP_ACCUMULATE if accumulate else 0)
    _check(lib().tp_mlp_row_partial_shards_tile(tile, _ptrs(Y, "Y"), _ptrs(V, "V"), _ptrs(Zl, "Z", allow_none=True),
                                                n, M, Fk, H, flags, _stream(stream)),
           "tp_mlp_row_partial_shards_tile")
    return Z
