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

from gpu_util import check_sampled as _check, to_dev, y_bits

pytestmark = pytest.mark.gpu


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
