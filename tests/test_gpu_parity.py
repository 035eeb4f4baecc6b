"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Reduced-size layers keep every structural feature of the five measured
configurations (int4 g64 and MXFP4 g32, softmax and sigmoid routers, Zipf
logit bias, a shared expert, partial weight blocks, prefill token tiles with
ragged tails, decode T <= 8) at sizes the oracle finishes in seconds.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import moe as om
from oracle.residency import ResidencyModel
from synth import CONFIGS, make_layer, make_tokens

from gpu_util import assert_routing_equal, assert_y_close, to_dev, y_bits, y_to_f64

pytestmark = pytest.mark.gpu

SMALL = {
    # name: (config, Ts)
    "tiny": (CONFIGS["tiny"], (1, 2, 5, 8, 16)),
    "mixtral_s": (CONFIGS["mixtral"].scaled(hidden=1024, ffn=512), (1, 3, 257)),
    "qwen_s": (CONFIGS["qwen3_30b_a3b"].scaled(hidden=1024, ffn=256, num_experts=32), (1, 8, 300)),
    "glm_s": (CONFIGS["glm45_air"].scaled(hidden=1024, ffn=320, num_experts=16, top_k=4, budget_frac=0.2),
              (1, 2, 4, 8, 300)),
    "e512_s": (CONFIGS["e512_mxfp4"].scaled(hidden=1024, ffn=256, num_experts=64, budget_frac=0.18),
               (1, 2, 3, 8, 333)),
    # wider routing at the full expert counts (top-16 of 896, top-6 of 256)
    "e896_s": (CONFIGS["e896_top16_mxfp4"].scaled(hidden=512, ffn=128, budget_frac=0.1), (1, 3, 8, 300)),
    "e256_s": (CONFIGS["e256_top6_fp4"].scaled(hidden=1024, ffn=256), (1, 4, 333)),
    # more 4-bit formats: int4 group-128, NVFP4 (with a shared expert)
    "g128_s": (CONFIGS["e256_int4g128"].scaled(hidden=1024, ffn=256, num_experts=32, budget_frac=0.25),
               (1, 2, 6, 300)),
    "nvfp4_s": (CONFIGS["e256_nvfp4"].scaled(hidden=1024, ffn=256, num_experts=64), (1, 3, 8, 333)),
    # a long down-projection reduction (F = 8192: the prefill down GEMM splits
    # K in two partial-sum planes), int4 group-64 and group-128
    "longk_s": (CONFIGS["mixtral"].scaled(hidden=512, ffn=8192), (1, 3, 257)),
    "longk_g128_s": (CONFIGS["e256_int4g128"].scaled(hidden=512, ffn=8192, num_experts=8, top_k=2,
                                                       budget_frac=0.5), (1, 200)),
    # a gated shared expert (its output weighted by sigmoid(x . w_s)) in three formats
    "glm_gate_s": (CONFIGS["glm45_air"].scaled(hidden=1024, ffn=320, num_experts=16, top_k=4, budget_frac=0.2,
                                               shared_gate=True), (1, 3, 8, 300)),
    "e512_gate_s": (CONFIGS["e512_mxfp4"].scaled(hidden=1024, ffn=256, num_experts=64, budget_frac=0.18,
                                                 shared_gate=True), (1, 5, 333)),
    "nvfp4_gate_s": (CONFIGS["e256_nvfp4"].scaled(hidden=1024, ffn=256, num_experts=64, shared_gate=True),
                     (2, 8, 129)),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


_layers = {}


def _get(name):
    if name not in _layers:
        cfg, Ts = SMALL[name]
        _layers[name] = make_layer(cfg, seed=cfg.seed + 50)
    return _layers[name]


def _mk(lw, budget=None, max_tokens=512):
    import expert_paged_quantized_amd as epq
    return epq.MoELayer.from_weights(lw, budget=budget, max_tokens=max_tokens)


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_matches_oracle_all_resident(torch_cuda, name):
    lw = _get(name)
    cfg = lw.cfg
    layer = _mk(lw, budget=cfg.num_experts)
    for i, T in enumerate(SMALL[name][1]):
        print(f"[parity] {name} T={T}", flush=True)
        x = make_tokens(cfg, T, step=i, seed=cfg.seed + 50)
        y, dbg = layer.forward(to_dev(x), dbg=True)
        ref = om.moe_forward(lw, x)
        assert_routing_equal(dbg, ref, T, cfg.num_experts, cfg.top_k, f"{name} T={T}")
        assert_y_close(y_to_f64(y), ref["y"], f"{name} T={T}")
    layer.close()


@pytest.mark.parametrize("name", ["qwen_s", "glm_s", "e512_s", "mixtral_s", "e896_s", "g128_s", "nvfp4_s",
                                  "longk_s", "longk_g128_s", "glm_gate_s", "e512_gate_s"])
@pytest.mark.parametrize("policy", ["lru", "lfu"])
@pytest.mark.parametrize("pager", ["kernel", "dma"])
def test_paged_output_is_bitwise_the_resident_output(torch_cuda, name, policy, pager):
    """Budgeted (paged, waves) vs all-resident, with either paging engine:
    identical y bits; counters equal the residency model fed with the oracle's
    needed sets."""
    lw = _get(name)
    cfg = lw.cfg
    res = _mk(lw, budget=cfg.num_experts)
    import expert_paged_quantized_amd as epq
    paged = epq.MoELayer.from_weights(lw, budget=cfg.budget, policy=policy, max_tokens=512, pager=pager)
    model = ResidencyModel(cfg.num_experts, cfg.budget, policy, cfg.expert_bytes())
    Ts = [1, 300, 1, 2, 8, 1, 257, 4, 1, 1, 5, 3]
    for i, T in enumerate(Ts):
        print(f"[paged] {name} {policy} {pager} step={i} T={T}", flush=True)
        x = make_tokens(cfg, T, step=100 + i, seed=cfg.seed + 50)
        xd = to_dev(x)
        y_r = res.forward(xd)
        y_p, dbg = paged.forward(xd, dbg=True)
        assert np.array_equal(y_bits(y_p), y_bits(y_r)), f"{name} step {i}: paged != resident"
        model.forward(np.nonzero(dbg["counts"].cpu().numpy())[0].tolist())
    st, want = paged.stats(), model.stats()
    for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
              "resident_bytes"):
        assert st[k] == want[k], (k, st[k], want[k])
    assert st["budget"] == cfg.budget
    assert st["pager"] == {"kernel": 1, "dma": 2}[pager]
    assert st["misses"] > 0 and st["waves"] > len(Ts)  # paging and waves were exercised
    rs = res.stats()
    assert rs["forwards"] == len(Ts) and rs["misses"] == 0 and rs["hits"] == want["hits"] + want["misses"]
    res.close()
    paged.close()


def test_all_resident_forward_replays_from_a_graph(torch_cuda):
    """An all-resident forward captured into a HIP graph: every replay (with
    eager forwards and synchronisations between replays) gives the eager
    forward's bits for the input it finds in x; a budgeted layer refuses."""
    torch = torch_cuda
    import expert_paged_quantized_amd as epq
    lw = _get("glm_s")
    cfg = lw.cfg
    layer = _mk(lw, budget=cfg.num_experts)
    for T in (1, 4, 8, 300):
        print(f"[graph] T={T}", flush=True)
        xs = [to_dev(make_tokens(cfg, T, step=400 + 10 * T + i, seed=cfg.seed + 50)) for i in range(4)]
        x_static = xs[0].clone()
        y_static = torch.empty_like(x_static)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer.forward(x_static, y=y_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(x_static, y=y_static)
        for i, x in enumerate(xs):
            x_static.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            y_eager = layer.forward(x)
            torch.cuda.synchronize()
            assert np.array_equal(y_bits(y_static), y_bits(y_eager)), f"T={T} replay {i} differs from eager"
        del g
    paged = _mk(lw, budget=cfg.budget)
    x = to_dev(make_tokens(cfg, 1, step=499, seed=cfg.seed + 50))
    g = torch.cuda.CUDAGraph()
    with pytest.raises(epq.StrataError) as ei:
        with torch.cuda.graph(g):
            paged.forward(x)
    assert ei.value.status == 2  # E_UNSUPPORTED
    torch.cuda.synchronize()
    y_p, y_r = paged.forward(x), layer.forward(x)
    assert np.array_equal(y_bits(y_p), y_bits(y_r))  # both layers still usable
    layer.close()
    paged.close()


def test_auto_pager_picks_the_kernel_for_small_records(torch_cuda):
    """pager="auto" pages records of at most 8 MiB with the page-in kernel."""
    lw = _get("qwen_s")
    import expert_paged_quantized_amd as epq
    layer = epq.MoELayer.from_weights(lw, budget=lw.cfg.budget, max_tokens=64)
    assert lw.cfg.expert_bytes() <= 8 << 20 and layer.stats()["pager"] == 1
    layer.close()


@pytest.mark.parametrize("name", ["qwen_s", "glm_s", "e512_s", "nvfp4_s"])
def test_warm_policy_prefetch_and_profiles_only_reorder_work(torch_cuda, name):
    """WARM (decayed scores) with prefetch, a warm start from a profile and a
    run-time profile load between forwards: y is bitwise the resident y, and
    counters and scores equal the residency model's."""
    lw = _get(name)
    cfg = lw.cfg
    E, B = cfg.num_experts, cfg.budget
    P = max(1, B // 2)
    rng = np.random.default_rng(cfg.seed + 90)
    prof0 = rng.integers(0, 6 * 65536, size=E).astype(np.uint64)
    prof1 = rng.integers(0, 6 * 65536, size=E).astype(np.uint64)
    res = _mk(lw, budget=E)
    import expert_paged_quantized_amd as epq
    paged = epq.MoELayer.from_weights(lw, budget=B, policy="warm", decay_shift=2, prefetch=P,
                                      profile=prof0, max_tokens=512)
    model = ResidencyModel(E, B, "warm", cfg.expert_bytes(), decay_shift=2, prefetch=P,
                           profile=prof0.tolist())
    Ts = [1, 1, 300, 1, 2, 8, 1, 257, 4, 1, 1, 5, 3, 1, 1]
    for i, T in enumerate(Ts):
        if i == 6:
            paged.load_profile(prof1)
            model.load_profile(prof1.tolist())
        print(f"[warm] {name} step={i} T={T}", flush=True)
        x = make_tokens(cfg, T, step=400 + i, seed=cfg.seed + 50)
        xd = to_dev(x)
        y_r = res.forward(xd)
        y_p, dbg = paged.forward(xd, dbg=True)
        assert np.array_equal(y_bits(y_p), y_bits(y_r)), f"{name} step {i}: paged != resident"
        model.forward(np.nonzero(dbg["counts"].cpu().numpy())[0].tolist())
    st, want = paged.stats(), model.stats()
    for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
              "resident_bytes", "prefetched", "prefetch_hits"):
        assert st[k] == want[k], (k, st[k], want[k])
    assert st["policy"] == 3 and st["decay_shift"] == 2 and st["prefetch"] == P
    assert paged.save_profile().tolist() == model.profile()
    assert st["prefetched"] > 0 and st["misses"] > 0
    res.close()
    paged.close()


def test_budget_one_thrashes_but_matches(torch_cuda):
    lw = _get("glm_s")
    cfg = lw.cfg
    res = _mk(lw, budget=cfg.num_experts)
    one = _mk(lw, budget=1)
    for i, T in enumerate([1, 40, 3]):
        x = to_dev(make_tokens(cfg, T, step=200 + i, seed=7))
        assert np.array_equal(y_bits(one.forward(x)), y_bits(res.forward(x)))
    assert one.stats()["waves"] >= 4


def test_repeat_runs_are_bitwise_identical(torch_cuda):
    lw = _get("e512_s")
    layer = _mk(lw, budget=lw.cfg.budget)
    x = to_dev(make_tokens(lw.cfg, 333, step=5, seed=9))
    y0 = y_bits(layer.forward(x))
    for _ in range(3):
        assert np.array_equal(y_bits(layer.forward(x)), y0)


def test_forward_on_a_side_stream(torch_cuda):
    torch = torch_cuda
    lw = _get("qwen_s")
    layer = _mk(lw, budget=lw.cfg.budget)
    x = to_dev(make_tokens(lw.cfg, 64, step=1, seed=3))
    y0 = y_bits(layer.forward(x))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = layer.forward(x, stream=s)
    s.synchronize()
    assert np.array_equal(y_bits(y1), y0)


def test_degenerate_routing_all_tokens_one_expert(torch_cuda):
    """A +1e4 bias on one expert: every token picks it first (one huge segment,
    many tiles) and the remaining picks follow the tie-free logits."""
    lw = make_layer(CONFIGS["qwen3_30b_a3b"].scaled(hidden=512, ffn=128, num_experts=16, top_k=2), seed=31)
    lw.router_bias = np.zeros(16, np.float32)
    lw.router_bias[5] = 1e4
    layer = _mk(lw, budget=4)
    x = make_tokens(lw.cfg, 400, seed=31)
    y, dbg = layer.forward(to_dev(x), dbg=True)
    ref = om.moe_forward(lw, x)
    assert_routing_equal(dbg, ref, 400, 16, 2, "one-expert")
    assert ref["counts"][5] == 400
    assert_y_close(y_to_f64(y), ref["y"], "one-expert")


def test_equal_logits_tie_break_on_gpu(torch_cuda):
    """All-zero router weights: every logit is +0 (or the bias), ties go to the lower id."""
    lw = make_layer(CONFIGS["tiny"].scaled(num_experts=8, top_k=3, ffn=128), seed=32)
    lw.router_w = np.zeros_like(lw.router_w)
    layer = _mk(lw, budget=8)
    x = make_tokens(lw.cfg, 20, seed=32)
    y, dbg = layer.forward(to_dev(x), dbg=True)
    ref = om.moe_forward(lw, x)
    assert_routing_equal(dbg, ref, 20, 8, 3, "ties")
    assert np.array_equal(ref["idx"], np.tile([0, 1, 2], (20, 1)))
    assert_y_close(y_to_f64(y), ref["y"], "ties")


def test_zero_tokens_and_errors(torch_cuda):
    torch = torch_cuda
    import expert_paged_quantized_amd as epq
    lw = _get("tiny")
    layer = _mk(lw, budget=4, max_tokens=16)
    x = to_dev(make_tokens(lw.cfg, 16, seed=1))
    before = layer.stats()["forwards"]
    layer.forward(x[:0])
    assert layer.stats()["forwards"] == before
    with pytest.raises(epq.StrataError) as ei:
        big = to_dev(make_tokens(lw.cfg, 17, seed=1))
        layer.forward(big)
    assert ei.value.status == 1
    with pytest.raises(epq.StrataError):  # y aliases x
        layer.forward(x, y=x)


def test_copy_failure_poisons_the_handle(torch_cuda, monkeypatch):
    import expert_paged_quantized_amd as epq
    lw = _get("glm_s")
    layer = _mk(lw, budget=2)
    x = to_dev(make_tokens(lw.cfg, 50, seed=2))
    monkeypatch.setenv("STRATA_FAULT", "h2d")
    with pytest.raises(epq.StrataError) as ei:
        layer.forward(x)
    assert ei.value.status == 5
    monkeypatch.delenv("STRATA_FAULT")
    with pytest.raises(epq.StrataError) as ei:
        layer.forward(x)
    assert ei.value.status == 6
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("fault", ["hostalloc", "devalloc"])
def test_allocation_failures_are_reported(torch_cuda, monkeypatch, fault):
    import expert_paged_quantized_amd as epq
    monkeypatch.setenv("STRATA_FAULT", fault)
    with pytest.raises(epq.StrataError) as ei:
        _mk(_get("tiny"), budget=2)
    assert ei.value.status == 4


def test_device_memory_holds_no_widened_copy(torch_cuda):
    lw = _get("e512_s")
    cfg = lw.cfg
    layer = _mk(lw, budget=cfg.budget, max_tokens=64)
    m = layer.memory()
    eb = cfg.expert_bytes()
    stride = (eb + 255) // 256 * 256
    assert m["slot_pool"] == cfg.budget * stride
    assert m["shared"] == stride
    # prepack keeps the byte count; records sit at the 256-byte slot stride
    assert m["host_store"] == cfg.num_experts * stride and stride - eb < 256
    assert m["device_total"] == m["slot_pool"] + m["shared"] + m["router"] + m["workspace"]
    widened = cfg.num_experts * 3 * cfg.hidden * cfg.ffn * 2
    assert m["device_total"] < widened / 2
    st = layer.stats()
    assert st["expert_bytes"] == eb and st["resident_bytes"] == cfg.budget * eb
