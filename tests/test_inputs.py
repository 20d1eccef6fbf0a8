"""Checks of the seeded synthetic input generator (no MLP arithmetic here)."""
import numpy as np
import pytest
import torch


def test_philox_matches_numpy(inputs_mod):
    # numpy's Philox advances its counter before producing a block, so block
    # counter c corresponds to numpy's state counter c - 1.
    for c0, key in [(0, (0, 0)), (5, (7, 9)), (2 ** 40 + 3, (42, 3)), (2 ** 64 - 2, (2 ** 64 - 1, 1))]:
        mine = inputs_mod.philox4x64([c0 + 1, 0, 0, 0], key)
        ref = np.random.Philox(counter=np.array([c0, 0, 0, 0], dtype=np.uint64),
                              key=np.array(key, dtype=np.uint64)).random_raw(4)
        assert np.array_equal(mine, ref)


def test_normals_statistics(inputs_mod):
    z = inputs_mod.normal_f64(1, 2_000_000)
    assert abs(z.mean()) < 3e-3
    assert abs(z.std() - 1) < 3e-3
    assert abs(np.mean(z ** 3)) < 1e-2
    assert abs(np.mean(z ** 4) - 3) < 3e-2
    # independent streams are uncorrelated
    z2 = inputs_mod.normal_f64(2, 2_000_000)
    assert abs(np.corrcoef(z, z2)[0, 1]) < 3e-3


def test_slices_are_position_independent(inputs_mod):
    full = inputs_mod.normal_f64(3, 1001)
    for first, n in [(0, 1), (1, 7), (3, 500), (998, 3)]:
        assert np.array_equal(inputs_mod.normal_f64(3, n, first=first), full[first:first + n])
    a = inputs_mod.draw(1, (37,), 0.5, "bf16")
    b = inputs_mod.draw(1, (20,), 0.5, "bf16", first=17)
    assert np.array_equal(a[17:], b)


def test_bf16_rounding_matches_torch(inputs_mod):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # keep finite values only, plus ties and boundary cases
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    specials = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                         3.3895314e38, 1e-40, -1e-40, 2 ** -126], dtype=np.float32)
    f = np.concatenate([f, specials])
    mine = inputs_mod.round_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_draw_is_round_of_f32_draw(inputs_mod):
    a32 = inputs_mod.draw(2, (64, 33), 0.02, "f32")
    a16 = inputs_mod.draw(2, (64, 33), 0.02, "bf16")
    assert np.array_equal(inputs_mod.round_bf16(a32), a16)
    assert abs(a32.std() - 0.02) < 2e-3


def test_workloads_and_shards(inputs_mod):
    W = inputs_mod.WORKLOADS
    assert [w.name for w in W.values()] == ["tiny", "gpt2_small", "llama7b", "gpt3_175b", "long_seq"]
    for w in W.values():
        assert w.F == 4 * w.H and w.F % w.k == 0 and w.H % 8 == 0 and w.Fk % 8 == 0
    assert W["gpt3_175b"].flop == 4 * 2048 * 12288 * 49152
    inp = inputs_mod.make_inputs(W["tiny"])
    assert inp["X"].shape == (8, 64) and inp["X"].dtype == np.float32
    Ws, bs, Vs = inputs_mod.shard_slices(inp["W"], inp["b"], inp["V"], 2)
    assert Ws[1].shape == (64, 128) and Vs[1].shape == (128, 64) and bs[1].shape == (128,)
    assert np.array_equal(Ws[1], inp["W"][:, 128:]) and np.array_equal(Vs[0], inp["V"][:128])
    # deterministic
    assert np.array_equal(inputs_mod.make_inputs(W["tiny"])["V"], inp["V"])
    with pytest.raises(ValueError):
        inputs_mod.shard_slices(inp["W"], inp["b"], inp["V"], 3)
