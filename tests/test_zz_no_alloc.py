"""moe_layer_forward_noalloc (the layer on the library's static scratch, no
allocation) against moe_layer_forward with a caller workspace: same inputs,
two calls in a row, the second with fewer tokens, and the size limit."""
import pytest

torch = pytest.importorskip("torch")

from mixture_experts_layer_19_amd import binding as B
from mixture_experts_layer_19_amd import inputs as I
from mixture_experts_layer_19_amd.layer import to_device

from _gpu import device_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "hy3_decode", "w4a8_decode"])
def test_noalloc_matches_forward(name):
    w = I.workload(name)
    lay = device_layer(w)
    for T in (w.T, 5):                  # the second call is smaller
        xg, _ = I.x_input(w, T)
        xd = to_device(xg)
        print("[noalloc] %s T=%d" % (name, T), flush=True)
        ref = lay.forward(xd).clone()
        out = torch.full_like(ref, float("nan"))
        B.moe_layer_forward_noalloc(lay.ctx, lay.desc, lay.weights, xd, T, out)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: bit-identical output
        assert torch.equal(out, ref), name


def test_noalloc_rejects_more_tokens_than_the_scratch_holds():
    w = I.workload("hy3_decode", T=600)       # needs more than 64 MiB
    lay = device_layer(w)
    assert B.moe_workspace_bytes(lay.desc, w.T, B.MOE_WS_LAYER) > B.MOE_NOALLOC_SCRATCH_BYTES
    xd = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    out = torch.full((w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward_noalloc(lay.ctx, lay.desc, lay.weights, xd, w.T, out)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)              # nothing was enqueued
