"""Full-size parity of the five measured layer configurations, in the launch
configuration the benchmark times (the configured expert budget, LRU paging).

At these sizes the oracle checks sampled outputs one by one:
  * router logits of sampled tokens: bitwise against the fixed-order oracle;
  * for all tokens: top-k, weights, counts, offsets and permutation equal the
    oracle's selection / grouping applied to the GPU logits (integer work,
    bitwise), so routing is checked everywhere once the logits are;
  * y of sampled tokens against the oracle forward of those tokens;
  * the budgeted (paged) output equals the all-resident output bitwise.
"""
import numpy as np
import pytest

from oracle import moe as om
from synth import CONFIG_ORDER, CONFIGS, FORMAT_ORDER, WIDE_ORDER, make_layer, make_tokens

from gpu_util import W_ABS, assert_y_close, to_dev, y_bits, y_to_f64

pytestmark = pytest.mark.gpu


def _check(lw, layer, x, sample, what):
    import torch
    cfg = lw.cfg
    T = x.shape[0]
    y, dbg = layer.forward(to_dev(x), dbg=True)
    torch.cuda.synchronize()
    lg = dbg["logits"].cpu().numpy()
    ref_l = om.router_logits_fp32(x[sample], lw.router_w, lw.router_bias)
    assert np.array_equal(lg[sample].view(np.uint32), ref_l.view(np.uint32)), f"{what}: sampled logits"
    idx = om.select_topk(lg, cfg.top_k)
    assert np.array_equal(dbg["idx"].cpu().numpy(), idx), f"{what}: idx"
    w = om.routing_weights(lg, idx, cfg.router)
    assert np.abs(dbg["w"].cpu().numpy() - w).max() <= W_ABS, f"{what}: w"
    counts, offsets, perm, pos = om.permute(idx, cfg.num_experts)
    assert np.array_equal(dbg["counts"].cpu().numpy(), counts), f"{what}: counts"
    assert np.array_equal(dbg["offsets"].cpu().numpy(), offsets), f"{what}: offsets"
    assert np.array_equal(dbg["perm"].cpu().numpy(), perm), f"{what}: perm"
    ref = om.moe_forward(lw, x, tokens=sample)
    assert np.array_equal(ref["idx"], idx[sample])
    assert_y_close(y_to_f64(y)[sample], ref["y"], what)
    return y


@pytest.mark.parametrize("name", CONFIG_ORDER + WIDE_ORDER + FORMAT_ORDER)
def test_fullsize_config(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_paged_quantized_amd as epq
    cfg = CONFIGS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    lw = make_layer(cfg)
    Tmax = max(cfg.prefill_T, max(cfg.decode_T))
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=Tmax)
    resident = epq.MoELayer.from_weights(lw, budget=cfg.num_experts, max_tokens=Tmax)
    rng = np.random.default_rng(5)
    for step, T in enumerate((cfg.prefill_T,) + tuple(cfg.decode_T)):
        print(f"[fullsize] {name} T={T}", flush=True)
        x = make_tokens(cfg, T, step=step)
        sample = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=min(T, 4))]))
        y = _check(lw, paged, x, sample, f"{name} T={T}")
        y_r = resident.forward(to_dev(x))
        assert np.array_equal(y_bits(y), y_bits(y_r)), f"{name} T={T}: paged != resident"
    st = paged.stats()
    print(f"[fullsize] {name} stats {st}", flush=True)
    paged.close()
    resident.close()
