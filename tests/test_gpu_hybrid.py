"""Hybrid decode through the C ABI: in a decode forward (T <= 8) of a budgeted
layer the resident experts run on the GPU and the others on host threads
from the pinned store ("Strata, Explained", section 2; the `hybrid` policy
value of the "Documentation" page).  y must meet the layer's tolerance
against the oracle (the host computes in fp32 with its own summation order,
so it is not bitwise the resident y), the counters must equal the residency
model fed with the same needed sets, repeated runs must give the same bits,
and the number of host threads must not change any bit.  Prefill forwards of
the same layer page as usual."""
import numpy as np
import pytest

from oracle import moe as om
from oracle.residency import ResidencyModel
from synth import CONFIGS, make_layer, make_tokens

from gpu_util import assert_y_close, to_dev, y_bits, y_to_f64

pytestmark = pytest.mark.gpu

LAYERS = {
    "int4_zipf": CONFIGS["qwen3_30b_a3b"].scaled(hidden=1024, ffn=256, num_experts=32, budget_frac=0.25),
    "int4_sigmoid_gated": CONFIGS["glm45_air"].scaled(hidden=1024, ffn=320, num_experts=16, top_k=4,
                                                      budget_frac=0.2, shared_gate=True),
    "int4_g128": CONFIGS["e256_int4g128"].scaled(hidden=1024, ffn=256, num_experts=32, budget_frac=0.25),
    "mxfp4_shared": CONFIGS["e512_mxfp4"].scaled(hidden=1024, ffn=256, num_experts=64, budget_frac=0.18),
    "nvfp4_shared": CONFIGS["e256_nvfp4"].scaled(hidden=1024, ffn=256, num_experts=64),
}
TS = [1, 3, 300, 1, 8, 2, 1, 5, 257, 1, 4, 1]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(lw, xs, threads=0):
    import expert_paged_quantized_amd as epq
    cfg = lw.cfg
    layer = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=512, policy="lfu", prefetch=1,
                                      hybrid=True, host_threads=threads)
    ys, needs = [], []
    for x in xs:
        y, dbg = layer.forward(to_dev(x), dbg=True)
        ys.append(y_bits(y))
        needs.append(np.nonzero(dbg["counts"].cpu().numpy())[0].tolist())
    st = layer.stats()
    layer.close()
    return ys, needs, st


@pytest.mark.parametrize("name", list(LAYERS))
def test_hybrid_decode_matches_oracle_and_model(torch_cuda, name):
    cfg = LAYERS[name]
    lw = make_layer(cfg, seed=cfg.seed + 80)
    xs = [make_tokens(cfg, T, step=i, seed=cfg.seed + 80) for i, T in enumerate(TS)]
    print(f"[hybrid] {name}", flush=True)
    ys, needs, st = _run(lw, xs)
    model = ResidencyModel(cfg.num_experts, cfg.budget, "lfu", cfg.expert_bytes(), prefetch=1)
    for i, (x, T) in enumerate(zip(xs, TS)):
        ref = om.moe_forward(lw, x)
        assert_y_close(om.bf16_to_f64(ys[i]), ref["y"], f"{name} step {i} T={T}")
        assert needs[i] == np.nonzero(ref["counts"])[0].tolist()
        if T <= 8:
            model.forward_hybrid(needs[i])
        else:
            model.forward(needs[i])
    want = model.stats()
    for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident", "prefetched",
              "prefetch_hits", "host_experts"):
        assert st[k] == want[k], (k, st[k], want[k])
    assert st["host_experts"] > 0, "no expert went to the host"
    # the same sequence again, and with one host thread: the same bits
    ys2, _, _ = _run(lw, xs)
    ys1, _, _ = _run(lw, xs, threads=1)
    for i in range(len(TS)):
        assert np.array_equal(ys2[i], ys[i]), f"{name} step {i}: repeat differs"
        assert np.array_equal(ys1[i], ys[i]), f"{name} step {i}: one host thread differs"


def test_hybrid_prefill_is_bitwise_the_paged_prefill(torch_cuda):
    """A forward with T > 8 of a hybrid layer is an ordinary paged forward."""
    import expert_paged_quantized_amd as epq
    cfg = LAYERS["int4_zipf"]
    lw = make_layer(cfg, seed=cfg.seed + 81)
    a = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=512, hybrid=True)
    b = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=512)
    for i, T in enumerate((300, 9, 129)):
        x = to_dev(make_tokens(cfg, T, step=50 + i, seed=cfg.seed + 81))
        assert np.array_equal(y_bits(a.forward(x)), y_bits(b.forward(x)))
    assert a.stats()["host_experts"] == 0
    a.close()
    b.close()


# hybrid prefill: a needed expert that is not resident and has at most R
# tokens is computed on the host in a forward of more than 8 tokens
PREFILL_LAYERS = {
    "int4_zipf": (LAYERS["int4_zipf"], 4, [300, 129, 1, 257, 64, 3, 96]),
    "int4_sigmoid_gated": (LAYERS["int4_sigmoid_gated"], 2, [40, 17, 2, 33]),
    "mxfp4_shared": (LAYERS["mxfp4_shared"], 3, [300, 1, 120, 200]),
    "nvfp4_shared": (LAYERS["nvfp4_shared"], 8, [250, 64, 4]),
    # down GEMM split in two K planes (ffn 6144): host rows fill plane 0, zero plane 1
    "int4_ksplit": (CONFIGS["mixtral"].scaled(hidden=512, ffn=6144, num_experts=8, top_k=2, budget_frac=0.375),
                    4, [12, 20, 9, 1, 16]),
}


def _run_prefill(lw, xs, R, threads=0):
    import expert_paged_quantized_amd as epq
    cfg = lw.cfg
    layer = epq.MoELayer.from_weights(lw, budget=cfg.budget, max_tokens=512, policy="lfu", prefetch=1,
                                      hybrid=True, host_threads=threads, hybrid_rows=R)
    ys, counts = [], []
    for x in xs:
        y, dbg = layer.forward(to_dev(x), dbg=True)
        ys.append(y_bits(y))
        counts.append(dbg["counts"].cpu().numpy())
    st = layer.stats()
    layer.close()
    return ys, counts, st


@pytest.mark.parametrize("name", list(PREFILL_LAYERS))
def test_hybrid_prefill_matches_oracle_and_model(torch_cuda, name):
    cfg, R, Ts = PREFILL_LAYERS[name]
    lw = make_layer(cfg, seed=cfg.seed + 90)
    xs = [make_tokens(cfg, T, step=i, seed=cfg.seed + 90) for i, T in enumerate(Ts)]
    print(f"[hybrid prefill] {name} R={R}", flush=True)
    ys, counts, st = _run_prefill(lw, xs, R)
    model = ResidencyModel(cfg.num_experts, cfg.budget, "lfu", cfg.expert_bytes(), prefetch=1)
    for i, (x, T) in enumerate(zip(xs, Ts)):
        ref = om.moe_forward(lw, x)
        assert_y_close(om.bf16_to_f64(ys[i]), ref["y"], f"{name} step {i} T={T}")
        assert counts[i].tolist() == np.asarray(ref["counts"]).tolist()
        need = np.nonzero(counts[i])[0].tolist()
        if T <= 8:
            model.forward_hybrid(need)
        else:
            model.forward_split(need, {e: int(counts[i][e]) for e in need}, host_rows=R)
    want = model.stats()
    for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident", "prefetched",
              "prefetch_hits", "host_experts"):
        assert st[k] == want[k], (k, st[k], want[k])
    assert st["host_experts"] > 0, "no expert went to the host"
    # the same sequence again, and with one host thread: the same bits
    ys2, _, _ = _run_prefill(lw, xs, R)
    ys1, _, _ = _run_prefill(lw, xs, R, threads=1)
    for i in range(len(Ts)):
        assert np.array_equal(ys2[i], ys[i]), f"{name} step {i}: repeat differs"
        assert np.array_equal(ys1[i], ys[i]), f"{name} step {i}: one host thread differs"
