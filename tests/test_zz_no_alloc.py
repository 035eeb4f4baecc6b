"""The no-allocation forward (strata_moe_forward_noalloc, through the C ABI)
against the ordinary forward of the same layer: bitwise the same y and
routing outputs, on two calls in a row (the second with fewer tokens, so it
reuses a scratch that still holds the first call's buffers), on int4 (with
the scaled fp16 copy of x), NVFP4 with a gated shared expert, and MXFP4 layers.
Then the refusals: a T whose buffers exceed the static scratch, a budgeted
layer, and kernel timing on."""
import numpy as np
import pytest

from synth import CONFIGS, make_layer, make_tokens

from gpu_util import to_dev, y_bits

pytestmark = pytest.mark.gpu

LAYERS = {
    "int4": CONFIGS["qwen3_30b_a3b"].scaled(hidden=1024, ffn=256, num_experts=32),
    "nvfp4_shared": CONFIGS["e256_nvfp4"].scaled(hidden=1024, ffn=256, num_experts=64, shared_gate=True),
    "mxfp4_shared": CONFIGS["e512_mxfp4"].scaled(hidden=1024, ffn=256, num_experts=64),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _routing_equal(a, b):
    for k in ("logits", "idx", "w", "counts", "offsets", "perm"):
        assert np.array_equal(a[k].cpu().numpy().view(np.uint32), b[k].cpu().numpy().view(np.uint32)), k


@pytest.mark.parametrize("name", list(LAYERS))
def test_noalloc_forward_equals_forward(torch_cuda, name):
    import expert_paged_quantized_amd as epq
    cfg = LAYERS[name]
    lw = make_layer(cfg, seed=cfg.seed + 90)
    layer = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=512)
    for i, T in enumerate((300, 5, 1)):
        print(f"[noalloc] {name} call {i} T={T}", flush=True)
        x = to_dev(make_tokens(cfg, T, step=i, seed=cfg.seed + 90))
        y_ref, d_ref = layer.forward(x, dbg=True)
        y_na = torch_cuda.full_like(y_ref, float("nan"))
        y_na, d_na = layer.forward_noalloc(x, y=y_na, dbg=True)
        torch_cuda.cuda.synchronize()
        assert np.array_equal(y_bits(y_na), y_bits(y_ref)), f"{name} T={T}: y differs"
        _routing_equal(d_na, d_ref)
    layer.close()


def test_noalloc_refusals(torch_cuda):
    import expert_paged_quantized_amd as epq
    from expert_paged_quantized_amd import _capi
    cfg = CONFIGS["qwen3_30b_a3b"].scaled(hidden=2048, ffn=512, num_experts=8, top_k=2, budget_frac=0.5)
    lw = make_layer(cfg, seed=5)
    layer = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=4096)
    x = to_dev(make_tokens(cfg, 4096, seed=5))
    with pytest.raises(epq.StrataError) as ei:   # about 22 KB per token: 4096 do not fit 64 MiB
        layer.forward_noalloc(x)
    assert ei.value.status == _capi.E_INVALID and "at most" in str(ei.value)
    y = layer.forward_noalloc(x[:1000])          # within the scratch
    assert np.array_equal(y_bits(y), y_bits(layer.forward(x[:1000])))
    layer.set_timing(True)
    with pytest.raises(epq.StrataError) as ei:
        layer.forward_noalloc(x[:8])
    assert ei.value.status == _capi.E_UNSUPPORTED
    layer.set_timing(False)
    layer.close()
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=64)
    with pytest.raises(epq.StrataError) as ei:
        paged.forward_noalloc(x[:8])
    assert ei.value.status == _capi.E_UNSUPPORTED and "budget" in str(ei.value)
    paged.close()
    torch_cuda.cuda.synchronize()
