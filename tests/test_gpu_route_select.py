"""Small-batch routing of wide layers, where a token's top-k is found by a
search for its k-th largest selection key (not k rounds of one-wave picks):
indices, weights, counts and the permutation bitwise against the oracle at
T = 1 .. 16, with exact ties among the logits (a zero router matrix and a
bias with repeated values, positive and negative, so that more experts share
the k-th value than are still needed and the lower ids must win) and with
random logits."""
import dataclasses

import numpy as np
import pytest

from oracle import moe as om
from synth import CONFIGS, make_layer, make_tokens
from synth.workloads import WIDE_CONFIGS

from gpu_util import assert_routing_equal, assert_y_close, to_dev, y_to_f64

pytestmark = pytest.mark.gpu

LAYERS = {
    "e512_k10": CONFIGS["e512_mxfp4"].scaled(hidden=512, ffn=128),
    "e896_k16": WIDE_CONFIGS["e896_top16_mxfp4"].scaled(hidden=512, ffn=128),
    "e1024_k32": WIDE_CONFIGS["e896_top16_mxfp4"].scaled(hidden=512, ffn=128, num_experts=1024, top_k=32),
    "e200_k7_sigmoid": CONFIGS["glm45_air"].scaled(hidden=512, ffn=128, num_experts=200, top_k=7),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def tied_layer(cfg, seed):
    lw = make_layer(cfg, seed=seed)
    e = np.arange(cfg.num_experts)
    # values -1.5 .. 1.5 in steps of 0.5, each shared by ~E/7 experts
    bias = ((e * 5) % 7 - 3).astype(np.float32) * 0.5
    return dataclasses.replace(lw, router_w=np.zeros_like(lw.router_w), router_bias=bias)


@pytest.mark.parametrize("name", list(LAYERS))
@pytest.mark.parametrize("tied", [True, False])
def test_small_batch_selection_matches_oracle(torch_cuda, name, tied):
    import expert_paged_quantized_amd as epq
    cfg = LAYERS[name]
    lw = tied_layer(cfg, cfg.seed + 70) if tied else make_layer(cfg, seed=cfg.seed + 71)
    layer = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=16)
    for i, T in enumerate((1, 2, 3, 5, 8, 16)):
        print(f"[select] {name} tied={tied} T={T}", flush=True)
        x = make_tokens(cfg, T, step=60 + i, seed=cfg.seed + 70)
        y, dbg = layer.forward(to_dev(x), dbg=True)
        ref = om.moe_forward(lw, x)
        assert_routing_equal(dbg, ref, T, cfg.num_experts, cfg.top_k, f"{name} tied={tied} T={T}")
        if tied:
            # the top value 1.5 is shared by every expert e with 5e = 6 (mod 7): the lowest ids win
            top = [e for e in range(cfg.num_experts) if (e * 5) % 7 == 6][: cfg.top_k]
            assert list(ref["idx"][0][: len(top)]) == top
        assert_y_close(y_to_f64(y), ref["y"], f"{name} tied={tied} T={T}")
    layer.close()
