"""Decode at 5 to 8 tokens, where each expert's rows are cut into tiles of at
most 4: a router bias sends every token to the same k experts, so each of
them (and the shared expert) holds all T rows and takes two tiles.  y against
the oracle, routing bitwise, and a budgeted layer (paged, both engines, and
the hybrid host path) bitwise the all-resident one."""
import dataclasses

import numpy as np
import pytest

from oracle import moe as om
from synth import CONFIGS, make_layer, make_tokens

from gpu_util import assert_routing_equal, assert_y_close, to_dev, y_bits, y_to_f64

pytestmark = pytest.mark.gpu

LAYERS = {
    # int4 g64 softmax (Zipf bias replaced), int4 g64 sigmoid with a shared
    # expert, MXFP4 with a shared expert
    "qwen_hot": CONFIGS["qwen3_30b_a3b"].scaled(hidden=1024, ffn=256, num_experts=32, budget_frac=0.25),
    "glm_hot": CONFIGS["glm45_air"].scaled(hidden=1024, ffn=320, num_experts=16, top_k=4, budget_frac=0.2),
    "e512_hot": CONFIGS["e512_mxfp4"].scaled(hidden=1024, ffn=256, num_experts=64, budget_frac=0.18),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def hot_layer(name):
    cfg = LAYERS[name]
    lw = make_layer(cfg, seed=cfg.seed + 90)
    bias = np.zeros(cfg.num_experts, np.float32)
    bias[[3 * j + 1 for j in range(cfg.top_k)]] = 64.0  # the same k experts win for every token
    return dataclasses.replace(lw, router_bias=bias)


@pytest.mark.parametrize("name", list(LAYERS))
def test_tiles_of_four_rows_match_oracle_and_paged(torch_cuda, name):
    import expert_paged_quantized_amd as epq
    lw = hot_layer(name)
    cfg = lw.cfg
    res = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=8)
    paged = {p: epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=8, pager=p) for p in ("kernel", "dma")}
    hyb = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=8, hybrid=True, host_threads=4)
    for i, T in enumerate((5, 6, 7, 8, 1, 8)):
        print(f"[tiles4] {name} T={T}", flush=True)
        x = make_tokens(cfg, T, step=40 + i, seed=cfg.seed + 90)
        xd = to_dev(x)
        y, dbg = res.forward(xd, dbg=True)
        ref = om.moe_forward(lw, x)
        assert_routing_equal(dbg, ref, T, cfg.num_experts, cfg.top_k, f"{name} T={T}")
        # every token chose the biased experts: each holds all T rows
        assert sorted(np.nonzero(ref["counts"])[0].tolist()) == [3 * j + 1 for j in range(cfg.top_k)]
        assert (ref["counts"][ref["counts"] > 0] == T).all()
        assert_y_close(y_to_f64(y), ref["y"], f"{name} T={T}")
        for p, layer in paged.items():
            assert np.array_equal(y_bits(layer.forward(xd)), y_bits(y)), f"{name} T={T} paged ({p}) != resident"
        yh = hyb.forward(xd)
        assert_y_close(y_to_f64(yh), ref["y"], f"{name} T={T} hybrid")
    for layer in [res, hyb, *paged.values()]:
        layer.close()
