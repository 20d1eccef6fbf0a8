"""GPU parity of the tensor-parallel attention block (tp_attn_qkv_shards,
tp_attn_core_shards, tp_attn_shard_forward) against the CPU fp64 oracle,
element by element: the attention kernel from given bf16 projections at
small and ragged sizes (sequences shorter than a key block, not a multiple
of the 128-query block, head widths 64 and 128, causal or not, several heads
and shards per launch; scores rising along the keys, so that the kernel's
reference maximum is raised late), the projection GEMM with its bias epilogue, and the
whole block at small sizes and at the workload sizes on sampled rows; plus
batched == single-shard bit-identity, both variants of the shard sum and M = 0.
Bounds: tests/_helpers.py (the softmax weights for them are an independent
float64 computation; expected values come from the oracle).
"""
import numpy as np
import pytest

from _helpers import (U32, assert_within, attn_core_bound, attn_rows_bound, attn_score_err, f64, from_dev,
                      gemm_bound, rel_fro, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tpm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_transformer_mlp_amd as tpm
    tpm.lib()
    return tpm


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def _guarded(torch, shape, dtype, pad=64):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


CORE_CASES = [
    # B, S, heads, d, causal, score std
    (1, 1, 1, 64, True, 1.0), (1, 7, 1, 64, True, 1.0), (2, 64, 2, 64, False, 1.0), (1, 100, 3, 64, True, 1.5),
    (2, 129, 1, 128, True, 1.0), (1, 256, 2, 128, False, 1.0), (3, 300, 2, 128, True, 2.0),
    (1, 1024, 3, 64, True, 1.0), (1, 200, 4, 128, True, 3.0), (2, 65, 2, 64, False, 2.0),
]


@pytest.mark.parametrize("B,S,heads,d,causal,std", CORE_CASES)
def test_attn_core_parity(tpm, orc, B, S, heads, d, causal, std):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("attn_core B=%d S=%d heads=%d d=%d causal=%s std=%g" % (B, S, heads, d, causal, std))
    Hk = heads * d
    M = B * S
    qkv = inputs.draw(inputs.STREAM_X, (M, 3 * Hk), std, "bf16", seed=B * 1000 + S + heads + d)
    pad = 64
    buf, A = _guarded(torch, (M, Hk), torch.bfloat16, pad)
    tpm.tp_attn_core_shards([to_dev(qkv)], [A], B, S, heads, d, causal=causal)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Ag = f64(from_dev(A))
    assert np.all(np.isfinite(Ag))
    Ar = orc.attn_core(qkv, B, S, heads, d, causal)
    assert_within(Ag, Ar, attn_core_bound(f64(qkv), Ar, B, S, heads, d, causal), "A")
    assert rel_fro(Ag, Ar) <= 1e-2


def test_attn_core_shards_equal_single(tpm):
    import torch
    from tensor_transformer_mlp_amd import inputs
    B, S, heads, d, n = 2, 300, 2, 128, 5
    say("attn_core_shards n=%d B=%d S=%d" % (n, B, S))
    Hk = heads * d
    qkvs = [to_dev(inputs.draw(inputs.STREAM_X, (B * S, 3 * Hk), 1.0, "bf16", seed=40 + i)) for i in range(n)]
    A = [torch.empty(B * S, Hk, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tpm.tp_attn_core_shards(qkvs, A, B, S, heads, d)
    for i in range(n):
        Ai = torch.empty_like(A[i])
        tpm.tp_attn_core_shards([qkvs[i]], [Ai], B, S, heads, d)
        torch.cuda.synchronize()
        assert torch.equal(Ai, A[i]), i


# Grids of at least 4096 workgroups of 256 queries (ceil(S / 256) x shards x
# sequences x heads) run two 32-query groups per wave; the same shards one at a
# time run one group per wave.
WIDE_CASES = [
    # shards, B, S, heads, d, causal
    (8, 16, 384, 16, 64, True), (8, 16, 300, 16, 64, False), (16, 8, 1000, 8, 128, True),
]


@pytest.mark.parametrize("G,B,S,heads,d,causal", WIDE_CASES)
def test_attn_core_wide_grid(tpm, orc, G, B, S, heads, d, causal):
    """The two-group kernel (a wide batch) equals the one-group kernel (each
    shard alone) bit for bit, and shard 0's first sequence passes the oracle
    bounds."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    assert -(-S // 256) * G * B * heads >= 4096 and -(-S // 256) * B * heads < 4096
    say("attn_core wide grid G=%d B=%d S=%d heads=%d d=%d causal=%s" % (G, B, S, heads, d, causal))
    Hk = heads * d
    qkv_h = [inputs.draw(inputs.STREAM_X, (B * S, 3 * Hk), 1.0, "bf16", seed=70 + i) for i in range(G)]
    qkvs = [to_dev(q) for q in qkv_h]
    A = [torch.full((B * S, Hk), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(G)]
    tpm.tp_attn_core_shards(qkvs, A, B, S, heads, d, causal=causal)
    for i in range(G):
        Ai = torch.full_like(A[i], float("nan"))
        tpm.tp_attn_core_shards([qkvs[i]], [Ai], B, S, heads, d, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(Ai, A[i]), i
    A0 = f64(from_dev(A[0][:S]))
    q0 = qkv_h[0][:S]
    Ar = orc.attn_core(q0, 1, S, heads, d, causal)
    assert np.all(np.isfinite(A0))
    assert_within(A0, Ar, attn_core_bound(f64(q0), Ar, 1, S, heads, d, causal), "A")
    assert rel_fro(A0, Ar) <= 1e-2


VARIANT_CASES = CORE_CASES + [
    # B, S, heads, d, causal, score std: several 256-query blocks, ragged tails
    (1, 511, 2, 128, True, 1.0), (2, 777, 1, 128, False, 1.0), (1, 1300, 2, 64, True, 2.0),
    (3, 257, 3, 64, False, 1.0), (1, 2048, 1, 128, True, 1.0), (2, 33, 2, 128, True, 1.0),
]


@pytest.mark.parametrize("B,S,heads,d,causal,std", VARIANT_CASES)
def test_attn_core_variants_identical(tpm, orc, B, S, heads, d, causal, std):
    """Both attention kernels (one and two query groups per wave), chosen
    through the measurement hook at shapes where the library would pick
    either, give the same bits, write nothing outside A, and the two-group
    kernel passes the oracle bounds element by element."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("attn_core variants B=%d S=%d heads=%d d=%d causal=%s" % (B, S, heads, d, causal))
    Hk = heads * d
    M = B * S
    n = 2
    qkv_h = [inputs.draw(inputs.STREAM_X, (M, 3 * Hk), std, "bf16", seed=B * 777 + S + heads + d + i)
             for i in range(n)]
    qkvs = [to_dev(q) for q in qkv_h]
    pad = 64
    outs = {}
    for v in (0, 1):
        bufs, As = zip(*[_guarded(torch, (M, Hk), torch.bfloat16, pad) for _ in range(n)])
        tpm.tp_attn_core_shards_variant(v, qkvs, list(As), B, S, heads, d, causal=causal)
        torch.cuda.synchronize()
        for buf in bufs:
            assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:]))), v
        outs[v] = As
    for v in (1,):
        for i in range(n):
            assert torch.equal(outs[v][i], outs[0][i]), (v, i)
    Ag = f64(from_dev(outs[1][1]))
    assert np.all(np.isfinite(Ag))
    Ar = orc.attn_core(qkv_h[1], B, S, heads, d, causal)
    assert_within(Ag, Ar, attn_core_bound(f64(qkv_h[1]), Ar, B, S, heads, d, causal), "A")
    assert rel_fro(Ag, Ar) <= 1e-2


def _shard_inputs(inp, n_heads, k):
    from tensor_transformer_mlp_amd import inputs
    Wqkv, bqkv = inputs.qkv_shards(inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], n_heads, k)
    H = inp["Wo"].shape[0]
    Hk = H // k
    Wo = [np.ascontiguousarray(inp["Wo"][i * Hk:(i + 1) * Hk]) for i in range(k)]
    return Wqkv, bqkv, Wo


GROW_CASES = [
    # B, S, heads, d, causal, score growth per 64 keys (base 2) for the queries with c = 1
    (1, 512, 2, 128, True, 10.0), (2, 300, 1, 64, False, 16.0), (1, 640, 3, 128, False, 6.0),
]


def _growing_qkv(B, S, heads, d, ramp, seed):
    """bf16 projections whose scores rise along the keys at a rate that
    differs per query: k_j[0] = a j (j the key's position in its sequence)
    and q_t[0] = c_t in [-1, 1), spread over every 32 queries, so that in
    base 2 the score of query t grows by about c_t ramp per 64 keys; the
    other entries are N(0, 1)."""
    from tensor_transformer_mlp_amd import inputs
    Hk = heads * d
    x = f64(inputs.draw(inputs.STREAM_X, (B * S, 3 * Hk), 1.0, "bf16", seed=seed)).astype(np.float32)
    pos = np.tile(np.arange(S), B).astype(np.float32)
    c = ((np.arange(B * S) * 37) % 64).astype(np.float32) / 32.0 - 1.0
    a = ramp * np.sqrt(d) / (64.0 * np.log2(np.e))
    for h in range(heads):
        x[:, Hk + h * d] = a * pos
        x[:, h * d] = c
    return inputs.round_bf16(x)


@pytest.mark.parametrize("B,S,heads,d,causal,ramp", GROW_CASES)
def test_attn_core_growing_scores(tpm, orc, B, S, heads, d, causal, ramp):
    """Scores that keep rising along the keys for some queries of a wave and
    fall for others: the kernel's reference maximum has to be raised on late
    key blocks for some lanes and not for others (partial rescales of
    accumulators that already hold many blocks), and between raises the
    weights grow up to 2^8.  Every row, both kernel variants, against the
    oracle; the rows bound includes the float32 score error, which grows
    with the scores here."""
    import torch
    say("attn_core growing scores B=%d S=%d heads=%d d=%d causal=%s ramp=%g" % (B, S, heads, d, causal, ramp))
    qkv = _growing_qkv(B, S, heads, d, ramp, seed=3000 + S + d)
    q64 = f64(qkv)
    Hk, M = heads * d, B * S
    ref = orc.attn_core(qkv, B, S, heads, d, causal)
    rows = np.arange(M)
    bound = attn_rows_bound(q64, rows, S, heads, d, ref, causal)
    outs = []
    for v in (0, 1):
        A = torch.empty(M, Hk, dtype=torch.bfloat16, device="cuda")
        tpm.tp_attn_core_shards_variant(v, [to_dev(qkv)], [A], B, S, heads, d, causal=causal)
        torch.cuda.synchronize()
        got = f64(from_dev(A))
        assert np.all(np.isfinite(got))
        assert_within(got, ref, bound, "A (variant %d)" % v)
        say("  variant %d: rel_fro %.3e" % (v, rel_fro(got, ref)))
        outs.append(got)
    assert np.array_equal(outs[0], outs[1])


def test_attn_qkv_parity(tpm, orc):
    import torch
    from tensor_transformer_mlp_amd import inputs
    B, S, H, nh, k = 2, 100, 256, 4, 2
    say("attn_qkv B=%d S=%d H=%d heads=%d k=%d" % (B, S, H, nh, k))
    inp = inputs.make_attention(M=B * S, H=H, dtype="bf16", std=0.05, seed=3)
    Wqkv, bqkv, _ = _shard_inputs(inp, nh, k)
    Hk = H // k
    QKV = [torch.empty(B * S, 3 * Hk, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    tpm.tp_attn_qkv_shards(to_dev(inp["X"]), [to_dev(w) for w in Wqkv], [to_dev(x) for x in bqkv], QKV)
    torch.cuda.synchronize()
    X64 = f64(inp["X"])
    for i in range(k):
        ref = orc.attn_qkv(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], nh, k, i)
        got = f64(from_dev(QKV[i]))
        bound = gemm_bound(X64, f64(Wqkv[i]), H) + 2.0 ** -8 * np.abs(ref) + 2 * U32 * np.abs(f64(bqkv[i]))[None, :]
        assert_within(got, ref, bound, "QKV[%d]" % i)


FWD_CASES = [
    # B, S, H, n_heads, k, causal
    (1, 64, 256, 4, 2, True), (2, 100, 256, 4, 4, True), (1, 130, 512, 4, 2, False), (2, 48, 768, 12, 4, True),
    (1, 200, 512, 4, 1, True),
]


@pytest.mark.parametrize("B,S,H,nh,k,causal", FWD_CASES)
@pytest.mark.parametrize("fused", [False, True])
def test_attn_shard_forward_parity(tpm, orc, B, S, H, nh, k, causal, fused):
    import torch
    from tensor_transformer_mlp_amd import inputs
    say("attn_shard_forward B=%d S=%d H=%d heads=%d k=%d causal=%s fused=%s" % (B, S, H, nh, k, causal, fused))
    inp = inputs.make_attention(M=B * S, H=H, dtype="bf16", std=0.05, seed=B + S + H + k)
    Wqkv, bqkv, Wo = _shard_inputs(inp, nh, k)
    pad = 64
    buf, Z = _guarded(torch, (B * S, H), torch.float32, pad)
    tpm.tp_attn_shard_forward(to_dev(inp["X"]), [to_dev(w) for w in Wqkv], [to_dev(x) for x in bqkv],
                              [to_dev(w) for w in Wo], B, S, nh, Z=Z, fused=fused, causal=causal)
    torch.cuda.synchronize()
    assert bool(torch.all(torch.isnan(buf[:pad]))) and bool(torch.all(torch.isnan(buf[-pad:])))
    Zg = f64(from_dev(Z))
    assert np.all(np.isfinite(Zg))
    Zr = orc.attn_forward(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], inp["Wo"],
                          nh, S, k, causal)
    # bound: per shard, the attention bound with the projection's score and
    # value errors, through the output projection
    d, hk, Hk = H // nh, nh // k, H // k
    X64 = f64(inp["X"])
    bound = np.zeros_like(Zr)
    for i in range(k):
        qkv = orc.attn_qkv(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], nh, k, i)
        A = orc.attn_core(qkv, B, S, hk, d, causal)
        sl = slice(i * Hk, (i + 1) * Hk)
        es = attn_score_err(qkv, B, S, hk, d, H, X64, f64(inp["Wq"])[:, sl], f64(inp["Wk"])[:, sl])
        eA = attn_core_bound(qkv, A, B, S, hk, d, causal, e_s=es)
        bound += gemm_bound(A, f64(Wo[i]), H if fused else Hk, ea=eA)
    bound += 2 * (k + 2) * U32 * np.abs(Zr)
    assert_within(Zg, Zr, bound, "Z")
    assert rel_fro(Zg, Zr) <= 1e-2


def test_attn_fused_and_literal_and_empty(tpm):
    """Both variants deterministic; the same Z up to float32 rounding of the
    shard sum; M = 0 is a no-op."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    B, S, H, nh, k = 2, 200, 512, 4, 4
    say("attn fused vs literal B=%d S=%d H=%d k=%d" % (B, S, H, k))
    inp = inputs.make_attention(M=B * S, H=H, dtype="bf16", std=0.05, seed=8)
    Wqkv, bqkv, Wo = _shard_inputs(inp, nh, k)
    args = (to_dev(inp["X"]), [to_dev(w) for w in Wqkv], [to_dev(x) for x in bqkv], [to_dev(w) for w in Wo])
    Z1 = tpm.tp_attn_shard_forward(*args, B, S, nh, fused=False)
    Z2 = tpm.tp_attn_shard_forward(*args, B, S, nh, fused=True)
    Z3 = tpm.tp_attn_shard_forward(*args, B, S, nh, fused=False)
    Z4 = tpm.tp_attn_shard_forward(*args, B, S, nh, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z3) and torch.equal(Z2, Z4)
    assert rel_fro(from_dev(Z2), from_dev(Z1)) <= 1e-5
    say("attn M=0")
    X0 = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    Z0 = tpm.tp_attn_shard_forward(X0, *args[1:], 0, S, nh)
    torch.cuda.synchronize()
    assert Z0.numel() == 0


@pytest.mark.parametrize("name", ["gpt2_small", "llama7b", "gpt3_175b", "long_seq"])
def test_attn_workload_sampled_rows(tpm, orc, name):
    """Full-size causal attention block (the workload's B, S, H and heads) in
    the benchmark's launch configuration; sampled rows at several positions
    of several sequences against the oracle (a row at position t needs only
    the t + 1 rows before it)."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    w = inputs.WORKLOADS[name]
    nh = w.heads
    say("workload attention %s B=%d S=%d H=%d heads=%d k=%d" % (name, w.B, w.S, w.H, nh, w.k))
    inp = inputs.make_attention(w)
    Wqkv, bqkv, Wo = _shard_inputs(inp, nh, w.k)
    Z = tpm.tp_attn_shard_forward(to_dev(inp["X"]), [to_dev(x) for x in Wqkv], [to_dev(x) for x in bqkv],
                                  [to_dev(x) for x in Wo], w.B, w.S, nh)
    torch.cuda.synchronize()
    # the oracle projects t + 1 rows for a row at position t: keep t small on the widest layers
    pos = [0, 1, 63, 64, 127, 128, 200] if w.H <= 4096 else [0, 1, 17, 40]
    rows = np.array(sorted({(r % w.B) * w.S + t for r, t in enumerate(pos)}))
    Zg = f64(from_dev(Z[torch.from_numpy(rows).cuda()]))
    Zr = orc.attn_forward_rows(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["bq"], inp["bk"], inp["bv"], inp["Wo"],
                               nh, w.S, w.k, rows, True)
    assert np.all(np.isfinite(Zg))
    assert rel_fro(Zg, Zr) <= 1e-2
    for j in range(len(rows)):
        assert rel_fro(Zg[j], Zr[j]) <= 2e-2, rows[j]


def _late_positions(S):
    """Query positions that reach deep into a sequence: the first key blocks,
    both halves of the first 256-query blocks (the wide-grid kernel's two
    query groups per wave), the middle, and the last positions before and
    after 32-, 64- and 128-row block boundaries."""
    pos = {0, 1, 31, 32, 63, 64, 127, 128, 160, 191, 192, 224, 255, 256,
           S // 2 - 1, S // 2, S // 2 + 100, S - 257, S - 256, S - 129, S - 128, S - 100, S - 65, S - 64,
           S - 33, S - 32, S - 2, S - 1}
    return sorted(p for p in pos if 0 <= p < S)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["gpt2_small", "llama7b", "gpt3_175b", "long_seq"])
def test_attn_core_late_queries(tpm, orc, name):
    """The attention kernel at the workloads' full sequence lengths (S = 1024,
    2048, 2048 and 32768), every shard of the workload in one launch (the
    benchmark's launch configuration: the long-sequence one runs the wide-grid
    kernel with two query groups per wave), from given bf16 projections drawn
    on the host; query rows deep into the sequences, every head of every
    shard, against the oracle's rows-only attention, element by element."""
    import torch
    from tensor_transformer_mlp_amd import inputs
    w = inputs.WORKLOADS[name]
    nh, k = w.heads, w.k
    hk, d = nh // k, w.H // nh
    Hk, M, S = hk * d, w.M, w.S
    n = min(k, tpm.TP_MAX_BATCH)
    say("attn_core late queries %s: B=%d S=%d heads/shard=%d d=%d shards=%d" % (name, w.B, S, hk, d, n))
    qkv_h = [inputs.draw(inputs.STREAM_X, (M, 3 * Hk), 1.0, "bf16", seed=2000 + i) for i in range(n)]
    QKV = [to_dev(x) for x in qkv_h]
    A = [torch.empty(M, Hk, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    tpm.tp_attn_core_shards(QKV, A, w.B, S, hk, d, causal=True)
    torch.cuda.synchronize()
    pos = _late_positions(S)
    seqs = sorted({0, w.B - 1})
    rows = np.array([b * S + t for b in seqs for t in pos])
    rows_t = torch.from_numpy(rows).cuda()
    for i in range(n):
        q64 = f64(qkv_h[i])
        ref = orc.attn_core_rows(q64, w.B, S, hk, d, rows, True)
        got = f64(from_dev(A[i].index_select(0, rows_t)))
        assert np.all(np.isfinite(got))
        assert_within(got, ref, attn_rows_bound(q64, rows, S, hk, d, ref, True), "%s shard %d A" % (name, i))
        err = rel_fro(got, ref)
        say("  %s shard %d: rel_fro on %d late rows = %.3e" % (name, i, rows.size, err))
        assert err <= 1e-2
        del q64
