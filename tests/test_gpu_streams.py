"""The binding on a caller's stream: every tensor the binding allocates on the
caller's behalf (outputs and workspaces) must belong to the stream its kernels
run on.  The forward and the backward are queued on a side stream held back by
a spin kernel, while the current stream allocates blocks of the workspaces'
sizes and fills them with NaN; the results must equal, bit for bit, those of
the same calls on the current stream."""
import numpy as np
import pytest

from _helpers import say, to_dev

pytestmark = pytest.mark.gpu


def test_side_stream_forward_backward():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_transformer_mlp_amd as tpm
    from tensor_transformer_mlp_amd import inputs
    w = inputs.Workload("streams", 2, 1024, 768, 3072, 4, "bf16", 0.02)
    say("side-stream forward and backward M=%d H=%d F=%d k=%d" % (w.M, w.H, w.F, w.k))
    inp = inputs.make_inputs(w)
    Ws, bs, Vs = inputs.shard_slices(inp["W"], inp["b"], inp["V"], w.k)
    X = to_dev(inp["X"])
    Ws, bs, Vs = [to_dev(x) for x in Ws], [to_dev(x) for x in bs], [to_dev(x) for x in Vs]
    dZ = to_dev(inputs.draw(inputs.STREAM_DZ, (w.M, w.H), 1.0, w.dtype))
    sizes = []
    for fused in (False, True):
        sizes.append(tpm.tp_mlp_workspace_bytes(w.k, w.M, w.H, w.Fk, tpm.TP_BF16, tpm.TP_FUSED_ACCUM if fused else 0))
        sizes.append(tpm.tp_mlp_backward_workspace_bytes(w.k, w.M, w.H, w.Fk, tpm.TP_BF16,
                                                         tpm.TP_FUSED_ACCUM if fused else 0))
    for fused in (False, True):
        ref_z = tpm.tp_mlp_shard_forward(X, Ws, bs, Vs, fused=fused)
        ref_b = tpm.tp_mlp_shard_backward(X, Ws, bs, Vs, dZ, fused=fused)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            torch.cuda._sleep(100_000_000)     # the side stream's kernels start well after the host returns
        z = tpm.tp_mlp_shard_forward(X, Ws, bs, Vs, fused=fused, stream=side)
        b = tpm.tp_mlp_shard_backward(X, Ws, bs, Vs, dZ, fused=fused, stream=side)
        # the current stream takes blocks of the workspaces' sizes and writes them
        junk = [torch.full((max(n, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda") for n in sizes]
        junk += [torch.full((max(n, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda") for n in sizes]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        assert torch.equal(z, ref_z), "forward on a side stream differs (fused=%s)" % fused
        assert torch.equal(b[0], ref_b[0]), "dX on a side stream differs (fused=%s)" % fused
        for g1, g2 in zip(b[1:], ref_b[1:]):
            assert all(torch.equal(x, y) for x, y in zip(g1, g2)), "parameter gradients differ (fused=%s)" % fused
    assert np.isfinite(float(z.abs().max()))
