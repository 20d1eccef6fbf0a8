"""Seeded synthetic inputs for the tensor-parallel MLP shard forward.

This module draws numbers and lays them out; it holds none of the MLP's
arithmetic.  The GPU path and the CPU oracle are both fed from it, so they see
bit-identical inputs.  Draws come from ``csrc/synth_inputs.c`` (counter-based
Philox4x64-10 plus Box-Muller, OpenMP), built with gcc into ``libtpsynth.so``.

Workloads (the shapes of the MLP block on the pages: the first linear layer
W is (H, 4H) and the second V is (4H, H), "大模型分布式并行策略详解：TP、DP、PP、CP、EP
核心原理与实战" §4.1; weights laid out ``[in, out]`` and X as ``[batch, seq,
hidden]`` as in the ColumnParallelLinear / RowParallelLinear classes of
"AI大模型分布式训练：张量并行与流水线并行深度实践" §2.1-2.2):

=============  ===========  =====  =====  ==  =====  =====  =======
name           B x S = M    H      F      k   F/k    dtype  std
=============  ===========  =====  =====  ==  =====  =====  =======
tiny           1x8 = 8      64     256    2   128    f32    0.02
gpt2_small     8x1024       768    3072   4   768    bf16   0.02
llama7b        4x2048       4096   16384  8   2048   bf16   0.02
gpt3_175b      1x2048       12288  49152  8   6144   bf16   0.006
long_seq       1x32768      8192   32768  8   4096   bf16   0.01
=============  ===========  =====  =====  ==  =====  =====  =======

X ~ N(0, 1); W, b, V ~ N(0, std) (the second parameter is the standard
deviation).  For the backward, the gradient of the block output is
dZ ~ N(0, 1) (the gradient of L = sum(Z * R) for a standard normal R).
Streams: X = 0, W = 1, b = 2, V = 3, dZ = 4 under base seed 42.  The full
W, b and V are drawn first and shards are slices of them, so the same weights
serve every shard count k.  bf16 workloads store the float32 draw rounded to
nearest-even bfloat16 (as raw uint16 bit patterns on the host).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth_inputs.c")
_LIB_PATH = os.path.join(_HERE, "libtpsynth.so")

STREAM_X, STREAM_W, STREAM_B, STREAM_V, STREAM_DZ, STREAM_WU = 0, 1, 2, 3, 4, 5
# attention block: Wq, Wk, Wv, Wo, bq, bk, bv
STREAM_WQ, STREAM_WK, STREAM_WV, STREAM_WO, STREAM_BQ, STREAM_BK, STREAM_BV = 6, 7, 8, 9, 10, 11, 12
BASE_SEED = 42


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    F: int
    k: int
    dtype: str  # "f32" or "bf16"
    std: float

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def Fk(self) -> int:
        return self.F // self.k

    @property
    def flop(self) -> int:
        """Two GEMMs of 2*M*H*(F/k) per shard, k shards: 4*M*H*F."""
        return 4 * self.M * self.H * self.F

    @property
    def heads(self) -> int:
        """Attention heads of the model the shape is taken from: 64-wide heads
        for the GPT-2-small width, 128-wide above (GPT-2 small: 12 heads; 7B:
        32; GPT-3 175B: 96; the long-sequence layer: 64)."""
        return self.H // (64 if self.H <= 1024 else 128)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "S": self.S, "M": self.M, "H": self.H,
                "F": self.F, "k": self.k, "Fk": self.Fk, "dtype": self.dtype,
                "init_std": self.std}


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 8, 64, 256, 2, "f32", 0.02),
        Workload("gpt2_small", 8, 1024, 768, 3072, 4, "bf16", 0.02),
        Workload("llama7b", 4, 2048, 4096, 16384, 8, "bf16", 0.02),
        Workload("gpt3_175b", 1, 2048, 12288, 49152, 8, "bf16", 0.006),
        Workload("long_seq", 1, 32768, 8192, 32768, 8, "bf16", 0.01),
    ]
}


def _source_sha256() -> str:
    import hashlib
    return hashlib.sha256(open(_SRC, "rb").read()).hexdigest()


def build_synth(force: bool = True) -> str:
    """Compile libtpsynth.so with gcc (host code only; called by the build step,
    before anything touches the GPU); the source's SHA-256 is compiled in."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               '-DSYNTH_SOURCE_SHA256="%s"' % _source_sha256(), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _synth():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libtpsynth.so is not built: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_source_sha256.restype = ctypes.c_char_p
        if lib.synth_source_sha256().decode() != _source_sha256():
            raise RuntimeError("libtpsynth.so was built from another version of synth_inputs.c: "
                               "run __graft_entry__.build() again")
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_philox4x64.argtypes = [vp, vp, ctypes.c_int, vp]
        lib.synth_normal_f64.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_normal_f32.argtypes = [u64, u64, i64, i64, dbl, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, i64, dbl, vp]
        lib.synth_round_bf16.argtypes = [vp, i64, vp]
        for f in (lib.synth_philox4x64, lib.synth_normal_f64, lib.synth_normal_f32,
                  lib.synth_normal_bf16, lib.synth_round_bf16):
            f.restype = None
        _lib = lib
    return _lib


def philox4x64(ctr, key, rounds: int = 10) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    kk = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    _synth().synth_philox4x64(c.ctypes.data, kk.ctypes.data, rounds, out.ctypes.data)
    return out


def normal_f64(stream: int, n: int, first: int = 0, seed: int = BASE_SEED) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _synth().synth_normal_f64(seed, stream, first, n, out.ctypes.data)
    return out


def draw(stream: int, shape, std: float, dtype: str, seed: int = BASE_SEED, first: int = 0) -> np.ndarray:
    """N(0, std) of ``shape``: float32 array, or uint16 bf16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        if n:
            _synth().synth_normal_f32(seed, stream, first, n, float(std), out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        if n:
            _synth().synth_normal_bf16(seed, stream, first, n, float(std), out.ctypes.data)
    else:
        raise ValueError("dtype must be 'f32' or 'bf16', got %r" % (dtype,))
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (round to nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        _synth().synth_round_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: Workload, seed: int = BASE_SEED, M: int | None = None) -> dict:
    """Full X[M,H], W[H,F], b[F], V[F,H] for a workload (host numpy arrays).

    ``M`` overrides the row count (rows are a prefix of the same X stream).
    """
    M = w.M if M is None else M
    return {
        "X": draw(STREAM_X, (M, w.H), 1.0, w.dtype, seed),
        "W": draw(STREAM_W, (w.H, w.F), w.std, w.dtype, seed),
        "b": draw(STREAM_B, (w.F,), w.std, w.dtype, seed),
        "V": draw(STREAM_V, (w.F, w.H), w.std, w.dtype, seed),
    }


def make_custom(M: int, H: int, F: int, dtype: str, std: float = 0.02, x_std: float = 1.0,
                seed: int = BASE_SEED) -> dict:
    """Inputs of an arbitrary shape from the same four streams."""
    return {
        "X": draw(STREAM_X, (M, H), x_std, dtype, seed),
        "W": draw(STREAM_W, (H, F), std, dtype, seed),
        "b": draw(STREAM_B, (F,), std, dtype, seed),
        "V": draw(STREAM_V, (F, H), std, dtype, seed),
    }


def make_swiglu(w: Workload | None = None, seed: int = BASE_SEED, M: int | None = None, H: int | None = None,
                F: int | None = None, dtype: str | None = None, std: float | None = None) -> dict:
    """Inputs of the SwiGLU block: X[M,H], gate Wg[H,F] (the W stream), up
    Wu[H,F] (its own stream) and V[F,H], for a workload or a custom shape."""
    M = M if M is not None else w.M
    H = H if H is not None else w.H
    F = F if F is not None else w.F
    dtype = dtype if dtype is not None else w.dtype
    std = std if std is not None else w.std
    return {
        "X": draw(STREAM_X, (M, H), 1.0, dtype, seed),
        "Wg": draw(STREAM_W, (H, F), std, dtype, seed),
        "Wu": draw(STREAM_WU, (H, F), std, dtype, seed),
        "V": draw(STREAM_V, (F, H), std, dtype, seed),
    }


def make_attention(w: Workload | None = None, seed: int = BASE_SEED, M: int | None = None,
                   H: int | None = None, dtype: str | None = None, std: float | None = None) -> dict:
    """Inputs of the attention block: X[M,H], Wq, Wk, Wv, Wo [H,H] and biases
    bq, bk, bv [H], each from its own stream."""
    M = M if M is not None else w.M
    H = H if H is not None else w.H
    dtype = dtype if dtype is not None else w.dtype
    std = std if std is not None else w.std
    out = {"X": draw(STREAM_X, (M, H), 1.0, dtype, seed)}
    for name, st in (("Wq", STREAM_WQ), ("Wk", STREAM_WK), ("Wv", STREAM_WV), ("Wo", STREAM_WO)):
        out[name] = draw(st, (H, H), std, dtype, seed)
    for name, st in (("bq", STREAM_BQ), ("bk", STREAM_BK), ("bv", STREAM_BV)):
        out[name] = draw(st, (H,), std, dtype, seed)
    return out


def qkv_shards(Wq, Wk, Wv, bq, bk, bv, n_heads: int, k: int):
    """Per-shard projection weights [Wq_i | Wk_i | Wv_i] [H, 3 Hk] and biases
    [bq_i | bk_i | bv_i] (columns of the shard's heads side by side; data
    placement only).  Biases may be None."""
    H = Wq.shape[0]
    if n_heads % k or H % n_heads:
        raise ValueError("k must divide n_heads, n_heads must divide H")
    Hk = H // n_heads * (n_heads // k)
    Ws, bs = [], []
    for i in range(k):
        sl = slice(i * Hk, (i + 1) * Hk)
        Ws.append(np.ascontiguousarray(np.concatenate([Wq[:, sl], Wk[:, sl], Wv[:, sl]], axis=1)))
        if bq is not None:
            bs.append(np.ascontiguousarray(np.concatenate([bq[sl], bk[sl], bv[sl]])))
    return Ws, (bs if bq is not None else None)


def col_slices(W: np.ndarray, k: int):
    """Contiguous column blocks W_i = W[:, i*Fk:(i+1)*Fk] (data placement only)."""
    F = W.shape[1]
    if F % k:
        raise ValueError("k must divide F")
    Fk = F // k
    return [np.ascontiguousarray(W[:, i * Fk:(i + 1) * Fk]) for i in range(k)]


def shard_slices(W: np.ndarray, b: np.ndarray, V: np.ndarray, k: int):
    """Contiguous per-shard copies: W_i = W[:, i*Fk:(i+1)*Fk], b_i, V_i = V[i*Fk:(i+1)*Fk, :].

    Shard i owns the i-th block of columns of W (entries of b, rows of V), in
    index order, as in the column split W = [W_1, W_2] and the row split of V on
    "千亿参数模型如何拆分到多张GPU上训练" (张量并行 section).  This is data
    placement only (what each GPU of a TP group would hold).
    """
    F = W.shape[1]
    if F % k:
        raise ValueError("k must divide F")
    Fk = F // k
    Ws = [np.ascontiguousarray(W[:, i * Fk:(i + 1) * Fk]) for i in range(k)]
    bs = [np.ascontiguousarray(b[i * Fk:(i + 1) * Fk]) for i in range(k)]
    Vs = [np.ascontiguousarray(V[i * Fk:(i + 1) * Fk, :]) for i in range(k)]
    return Ws, bs, Vs
