"""GPU parity at the layer's limits, through the C ABI: the largest expert
count and top-k the descriptor admits (E = 1024, k = 32, with a 5% budget so
that forwards stream in many waves) and a 16,384-token prompt on the
Qwen3-30B-A3B-shaped layer (many token tiles per expert, 256 rank blocks)."""
import numpy as np
import pytest

from oracle import moe as om
from synth import CONFIGS, make_layer, make_tokens

from gpu_util import assert_routing_equal, assert_y_close, check_sampled, to_dev, y_bits, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("quant,router,zipf", [("int4_g64", "softmax", 1.1), ("mxfp4_g32", "sigmoid", None)])
def test_max_experts_and_top_k(torch_cuda, quant, router, zipf):
    import expert_paged_quantized_amd as epq
    cfg = CONFIGS["e896_top16_mxfp4"].scaled(name="e1024_top32", index=40, num_experts=1024, top_k=32,
                                             hidden=512, ffn=128, quant=quant, router=router, zipf_s=zipf,
                                             budget_frac=0.05)
    lw = make_layer(cfg)
    res = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=300)
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=300)
    for i, T in enumerate((1, 5, 8, 64, 300)):
        print(f"[limits] E=1024 k=32 {quant} T={T}", flush=True)
        x = make_tokens(cfg, T, step=i)
        y, dbg = res.forward(to_dev(x), dbg=True)
        if T <= 64:
            ref = om.moe_forward(lw, x)
            assert_routing_equal(dbg, ref, T, cfg.num_experts, cfg.top_k, f"E=1024 T={T}")
            assert_y_close(y_to_f64(y), ref["y"], f"E=1024 T={T}")
        else:
            sample = [0, 7, 150, T - 1]
            check_sampled(lw, res, x, sample, f"E=1024 T={T}")
        assert np.array_equal(y_bits(paged.forward(to_dev(x))), y_bits(y)), f"E=1024 T={T}: paged != resident"
    st = paged.stats()
    assert st["waves"] > st["forwards"] and st["misses"] > 0
    res.close()
    paged.close()


def test_long_prompt_qwen3_shape(torch_cuda):
    import expert_paged_quantized_amd as epq
    cfg = CONFIGS["qwen3_30b_a3b"]
    lw = make_layer(cfg)
    T = 16384
    res = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=T)
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=T)
    x = make_tokens(cfg, T, step=9000)
    sample = [0, 1, 4095, 8191, 12000, T - 2, T - 1]
    print(f"[limits] qwen3 T={T}", flush=True)
    y = check_sampled(lw, res, x, sample, f"qwen3 T={T}")
    assert np.array_equal(y_bits(paged.forward(to_dev(x))), y_bits(y)), "T=16384: paged != resident"
    res.close()
    paged.close()
