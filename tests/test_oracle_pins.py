"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-packed block, the bit
definition of a format, a closed form, a hand-derived fp32 rounding case or a
brute-force enumeration on a tiny input.
"""
import math
import os
from collections import OrderedDict

import numpy as np
import pytest

import oracle
from oracle import moe as om
from oracle.residency import LFU, LRU, ResidencyModel
from synth import (CONFIGS, f32_to_bf16_bits, make_layer, make_tokens, quantize_int4, quantize_int4_g64,
                   quantize_nvfp4_g16,
                   quantize_mxfp4_g32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(v):
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def pack(q):
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------------------
# P-1 int4 group-64 affine, hand-packed
# ----------------------------------------------------------------------------
def test_p1_int4_hand_packed_block():
    # one row, two groups; codes 0..15 repeated, written byte by byte by hand:
    # byte i holds element 2i (low nibble) and 2i+1 (high nibble)
    q = np.array([i % 16 for i in range(128)])
    codes = np.zeros((1, 64), np.uint8)
    for i in range(64):
        codes[0, i] = q[2 * i] + 16 * q[2 * i + 1]
    scales = np.array([[0x3F00, 0x4000]], np.uint16)   # bf16 0.5 and 2.0
    biases = np.array([[0xC080, 0x3F80]], np.uint16)   # bf16 -4.0 and 1.0
    w = om.dequant_int4_g64(codes, scales, biases)
    expect = np.concatenate([0.5 * q[:64] - 4.0, 2.0 * q[64:] + 1.0])
    assert np.array_equal(w[0], expect)
    # the low nibble is the even element
    assert w[0, 0] == -4.0 and w[0, 1] == -3.5


def test_p1_int4_group128_hand_packed_block():
    # one row, two groups of 128: the scale/bias index is k // 128
    q = np.array([(i * 7) % 16 for i in range(256)])
    codes = np.zeros((1, 128), np.uint8)
    for i in range(128):
        codes[0, i] = q[2 * i] + 16 * q[2 * i + 1]
    scales = np.array([[0x3E80, 0x4040]], np.uint16)   # bf16 0.25 and 3.0
    biases = np.array([[0xBF80, 0x4100]], np.uint16)   # bf16 -1.0 and 8.0
    w = om.dequant_int4_g128(codes, scales, biases)
    expect = np.concatenate([0.25 * q[:128] - 1.0, 3.0 * q[128:] + 8.0])
    assert np.array_equal(w[0], expect)
    # a group-64 reading of the same bytes would differ at element 64
    assert w[0, 64] == 0.25 * q[64] - 1.0


# ----------------------------------------------------------------------------
# P-2b NVFP4: E4M3 value table (OCP FP8), NaN refused, a hand-packed block
# ----------------------------------------------------------------------------
def _golden_e4m3():
    vals = {}
    with open(os.path.join(GOLDEN, "e4m3_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    return vals


def test_p2_e4m3_table():
    g = _golden_e4m3()
    assert len(g) >= 15
    for b, v in g.items():
        got = float(om.e4m3_value(b))
        assert got == v and np.signbit(got) == np.signbit(v), (hex(b), got, v)


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
def test_p2_e4m3_nan_is_refused(bad):
    with pytest.raises(ValueError):
        om.e4m3_value(np.array([0x38, bad]))
    codes = np.zeros((1, 16), np.uint8)
    with pytest.raises(ValueError):
        om.dequant_nvfp4_g16(codes, np.array([[0x38, bad]], np.uint8), 1.0)


def test_p2_nvfp4_hand_packed_block():
    # one row, two blocks of 16: codes 0..15 in both; block scales 1.0 (0x38)
    # and 0.015625 (0x08, the smallest normal); matrix scale 0.5
    e2m1 = {c: float(v) for c, v in _golden_e2m1().items()}
    q = np.array([i % 16 for i in range(32)])
    codes = np.zeros((1, 16), np.uint8)
    for i in range(16):
        codes[0, i] = q[2 * i] + 16 * q[2 * i + 1]
    w = om.dequant_nvfp4_g16(codes, np.array([[0x38, 0x08]], np.uint8), np.float32(0.5))
    expect = np.array([e2m1[c] * (1.0 if i < 16 else 0.015625) * 0.5 for i, c in enumerate(q)])
    assert np.array_equal(w[0], expect)
    with pytest.raises(ValueError):
        om.dequant_nvfp4_g16(codes, np.array([[0x38, 0x08]], np.uint8), 0.0)


# ----------------------------------------------------------------------------
# P-2 MXFP4: E2M1 value table, E8M0 as a bf16 exponent field, admission
# ----------------------------------------------------------------------------
def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def test_p2_e2m1_codes_match_ocp_table():
    table = _golden_e2m1()
    got = om.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == table[c]
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, table[c]) or table[c] == 0.0


def test_p2_e8m0_is_a_bf16_exponent_field():
    # an E8M0 byte s placed in the exponent field of a bf16 with zero mantissa
    for s in range(1, 255):
        bits = np.array([s << 7], np.uint16)
        assert om.e8m0_value(s) == om.bf16_to_f64(bits)[0]
    for s in (0, 255):
        with pytest.raises(ValueError):
            om.e8m0_value(np.array([s]))


def test_p2_mxfp4_block_scaling_and_groups():
    table = _golden_e2m1()
    codes16 = np.arange(16)
    q = np.concatenate([codes16, codes16, codes16, codes16])  # 64 elements, 2 groups
    codes = pack(q)[None, :]
    for s0, s1 in [(127, 127), (128, 126), (130, 120)]:
        w = om.dequant_mxfp4_g32(codes, np.array([[s0, s1]], np.uint8))[0]
        exp = np.array([table[int(c)] for c in q])
        exp[:32] *= 2.0 ** (s0 - 127)
        exp[32:] *= 2.0 ** (s1 - 127)
        assert np.array_equal(w, exp)
    for bad in (0, 255):
        with pytest.raises(ValueError):
            om.dequant_mxfp4_g32(codes, np.array([[127, bad]], np.uint8))


# ----------------------------------------------------------------------------
# P-3 quantise -> pack -> dequant round trip on exactly representable values
# ----------------------------------------------------------------------------
def test_p3_int4_round_trip():
    rng = np.random.default_rng(3)
    N, K = 8, 256
    s = np.float32(2.0) ** rng.integers(-8, -2, size=(N, K // 64)).astype(np.float32)
    b = -np.float32(8.0) * s
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::64] = 0   # every group reaches min and max
    q[:, 1::64] = 15
    w = (q.reshape(N, K // 64, 64) * s[..., None] + b[..., None]).reshape(N, K).astype(np.float32)
    codes, sb, bb = quantize_int4_g64(w)
    assert np.array_equal(om.dequant_int4_g64(codes, sb, bb), w.astype(np.float64))


def test_p3_int4_group128_round_trip():
    rng = np.random.default_rng(31)
    N, K = 6, 512
    s = np.float32(2.0) ** rng.integers(-8, -2, size=(N, K // 128)).astype(np.float32)
    b = -np.float32(4.0) * s
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::128] = 0
    q[:, 1::128] = 15
    w = (q.reshape(N, K // 128, 128) * s[..., None] + b[..., None]).reshape(N, K).astype(np.float32)
    codes, sb, bb = quantize_int4(w, 128)
    assert sb.shape == (N, K // 128)
    assert np.array_equal(om.dequant_int4_g128(codes, sb, bb), w.astype(np.float64))


def test_p3_nvfp4_round_trip():
    # values on the NVFP4 grid whose matrix amax is 6 * 448 * g and whose every
    # block holds a +-6 code, so the recipe recovers scales and codes exactly
    rng = np.random.default_rng(32)
    e2m1 = np.array([_golden_e2m1()[c] for c in range(16)])
    g = np.float32(2.0 ** -10)
    N, K = 4, 64
    c = rng.integers(0, 16, size=(N, K))
    c[:, ::16] = 7
    sc = rng.integers(0x20, 0x7E, size=(N, K // 16))
    sc[0, 0] = 0x7E   # 448: sets the matrix amax
    sval = om.e4m3_value(sc)
    w = (e2m1[c].reshape(N, K // 16, 16) * sval[..., None]).reshape(N, K) * float(g)
    codes, s2, g2 = quantize_nvfp4_g16(w.astype(np.float32))
    assert g2 == g and np.array_equal(s2, sc.astype(np.uint8))
    assert np.array_equal(om.dequant_nvfp4_g16(codes, s2, g2), w)


def test_p3_mxfp4_round_trip():
    rng = np.random.default_rng(4)
    table = np.array([_golden_e2m1()[c] for c in range(16)])
    N, K = 8, 128
    c = rng.integers(0, 16, size=(N, K))
    c[:, ::32] = 7   # every group holds a +6 so the shared exponent is exact
    e = rng.integers(100, 150, size=(N, K // 32))
    w = (table[c].reshape(N, K // 32, 32) * np.exp2(e - 127.0)[..., None]).reshape(N, K)
    codes, sc = quantize_mxfp4_g32(w.astype(np.float32))
    assert np.array_equal(sc, e.astype(np.uint8))
    assert np.array_equal(om.dequant_mxfp4_g32(codes, sc), w)


# ----------------------------------------------------------------------------
# P-4 router logits: fp64 bound, exact integer case, hand-derived order cases
# ----------------------------------------------------------------------------
def test_p4_router_close_to_fp64():
    rng = np.random.default_rng(5)
    T, E, H = 5, 7, 1024
    x = bf(rng.standard_normal((T, H)))
    w = bf(rng.standard_normal((E, H)) / 32)
    l = om.router_logits_fp32(x, w)
    x64, w64 = om.bf16_to_f64(x), om.bf16_to_f64(w)
    exact = x64 @ w64.T
    bound = H * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T)
    assert np.all(np.abs(l - exact) <= bound)


def test_p4_router_small_integers_exact():
    rng = np.random.default_rng(6)
    T, E, H = 3, 4, 1024
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-8, 9, size=(E, H))
    l = om.router_logits_fp32(bf(xi), bf(wi))
    for t in range(T):
        for e in range(E):
            assert l[t, e] == sum(int(a) * int(b) for a, b in zip(xi[t], wi[e]))


def _one_row(vals: dict, H=512):
    x = np.zeros((1, H), np.float32)
    for h, v in vals.items():
        x[0, h] = v
    return bf(x), bf(np.ones((1, H), np.float32))


def test_p4_lane_sums_run_in_h_order_within_a_lane():
    # h = 0, 1, 2 are v = 0, 1, 2 of lane 0 (h = (c*64 + L)*8 + v):
    # ((0 + 2^24) + 1) rounds to 2^24 (tie to even), minus 2^24 gives 0.
    # The exact sum, or any order that puts them in different lanes, gives 1.
    x, w = _one_row({0: 2.0 ** 24, 1: 1.0, 2: -2.0 ** 24})
    assert om.router_logits_fp32(x, w)[0, 0] == 0.0


def test_p4_butterfly_folds_offset_32_first():
    # lane 0 = 2^24, lane 1 = 1, lane 33 = 1 (h = 8*L).  Offset 32 first makes
    # lane 1 = 2 before it meets lane 0, so the result is 2^24 + 2 exactly.
    # A sequential lane sum or a fold starting at offset 1 gives 2^24.
    x, w = _one_row({0: 2.0 ** 24, 8: 1.0, 264: 1.0})
    assert om.router_logits_fp32(x, w)[0, 0] == 2.0 ** 24 + 2


def test_p4_bias_is_added_after_the_fold():
    # lane 0 terms 2^24 then -2^24 cancel to 0; bias 1 added last gives 1.
    # Starting lane 0 from the bias would give (1 + 2^24) - 2^24 = 0.
    x, w = _one_row({0: 2.0 ** 24, 1: -2.0 ** 24})
    l = om.router_logits_fp32(x, w, bias=np.array([1.0], np.float32))
    assert l[0, 0] == 1.0


def test_p4_chunks_follow_lanes():
    # h = 512 is chunk 1 of lane 0 (not lane 64); h = 520 is chunk 1 of lane 1.
    # lane 0: 2^24 (c=0) + 1 (c=1) -> 2^24; lane 1: 1 (c=1); lane 33: 1 (c=0).
    # fold: offset 32 gives lane 1 = 2, then lane 0 = 2^24 + 2.
    x, w = _one_row({0: 2.0 ** 24, 512: 1.0, 520: 1.0, 264: 1.0}, H=1024)
    assert om.router_logits_fp32(x, w)[0, 0] == 2.0 ** 24 + 2


# ----------------------------------------------------------------------------
# P-5 / P-6 top-k selection and weights
# ----------------------------------------------------------------------------
def test_p5_topk_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float32)  # many ties
        if rng.random() < 0.3:
            l[0, rng.integers(0, E)] = -0.0
        got = om.select_topk(l, k)[0].tolist()
        want = sorted(range(E), key=lambda e: (-float(l[0, e]), e))[:k]
        assert got == want


def test_p5_all_equal_logits():
    for k in (2, 8):
        l = np.zeros((3, 16), np.float32)
        idx = om.select_topk(l, k)
        assert np.array_equal(idx, np.tile(np.arange(k), (3, 1)))
        for router in ("softmax", "sigmoid"):
            assert np.all(om.routing_weights(l, idx, router) == 1.0 / k)


def test_p6_softmax_k2_is_logistic_and_weights_sum_to_one():
    rng = np.random.default_rng(8)
    l = rng.standard_normal((50, 6)).astype(np.float32)
    idx = om.select_topk(l, 2)
    w = om.routing_weights(l, idx, "softmax")
    for t in range(50):
        d = float(l[t, idx[t, 0]]) - float(l[t, idx[t, 1]])
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(-d))) < 1e-15
    for router in ("softmax", "sigmoid"):
        for k in (1, 3, 6):
            idx = om.select_topk(l, k)
            ws = om.routing_weights(l, idx, router)
            assert np.all(np.abs(ws.sum(axis=1) - 1.0) <= k * 2.0 ** -52)
            assert np.all(np.diff(ws, axis=1) <= 0)  # rank order is weight order


def test_p6_sigmoid_closed_forms():
    l = np.array([[0.0, 0.0, -50.0], [60.0, 0.0, -60.0]], np.float32)
    idx = om.select_topk(l, 2)
    w = om.routing_weights(l, idx, "sigmoid")
    assert np.allclose(w[0], [0.5, 0.5], rtol=0, atol=1e-16)
    # sigma(60) = 1 - ~1e-26, sigma(0) = 1/2 -> weights 2/3, 1/3
    assert abs(w[1, 0] - 2.0 / 3.0) < 1e-15 and abs(w[1, 1] - 1.0 / 3.0) < 1e-15


# ----------------------------------------------------------------------------
# P-7 permutation, brute force
# ----------------------------------------------------------------------------
def test_p7_permutation_brute_force():
    rng = np.random.default_rng(9)
    for _ in range(50):
        T, E = int(rng.integers(1, 40)), int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, pos = om.permute(idx, E)
        want = []
        for e in range(E):
            for t in range(T):
                if e in idx[t].tolist():
                    want.append(t)
        assert perm.tolist() == want
        assert counts.sum() == T * k and offsets[-1] == T * k
        for t in range(T):
            for j in range(k):
                r = pos[t, j]
                assert perm[r] == t and offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]
    with pytest.raises(ValueError):
        om.permute(np.array([[1, 1]]), 4)


# ----------------------------------------------------------------------------
# P-9 expert FFN closed forms
# ----------------------------------------------------------------------------
def test_p9_swiglu_scalar_closed_form():
    one = np.ones((1, 1))
    # gate goes through silu, up multiplies: silu(1) * 2 = 2 / (1 + e^-1)
    o = om.expert_ffn(one, np.array([[1.0]]), np.array([[2.0]]), np.array([[1.0]]))
    assert abs(o[0, 0] - 2.0 / (1.0 + math.exp(-1.0))) < 1e-15
    o = om.expert_ffn(one, np.array([[-1.0]]), np.array([[1.0]]), np.array([[3.0]]))
    assert abs(o[0, 0] - 3.0 * (-1.0 / (1.0 + math.e))) < 1e-15


def test_p9_one_hot_input_selects_columns():
    rng = np.random.default_rng(10)
    n = 16  # square so that a transposed operand would still type-check
    wg, wu, wd = (rng.standard_normal((n, n)) for _ in range(3))
    for h in (0, 5, 15):
        x = np.zeros((1, n))
        x[0, h] = 1.0
        g, u = wg[:, h], wu[:, h]
        a = np.array([gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
        want = np.array([sum(wd[r, f] * a[f] for f in range(n)) for r in range(n)])
        assert np.allclose(om.expert_ffn(x, wg, wu, wd)[0], want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# P-8 / P-10 / P-13 whole-layer invariants
# ----------------------------------------------------------------------------
def _tiny(**kw):
    base = CONFIGS["tiny"].scaled(ffn=128, num_experts=4, top_k=2)
    return base.scaled(**kw)


def _loop_ffn(x, wg, wu, wd):
    """Per-element loops with math.fsum: an implementation independent of numpy matmul."""
    F, H = wg.shape
    g = [math.fsum(wg[f, h] * x[h] for h in range(H)) for f in range(F)]
    u = [math.fsum(wu[f, h] * x[h] for h in range(H)) for f in range(F)]
    a = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return np.array([math.fsum(wd[r, f] * a[f] for f in range(F)) for r in range(H)])


@pytest.mark.parametrize("router,shared,quant", [("softmax", 0, "int4_g64"),
                                                  ("sigmoid", 1, "int4_g64"),
                                                  ("softmax", 1, "mxfp4_g32"),
                                                  ("sigmoid", 0, "int4_g128"),
                                                  ("softmax", 1, "nvfp4_g16")])
def test_p8_isolation_per_expert(router, shared, quant):
    cfg = _tiny(router=router, num_shared=shared, quant=quant)
    layer = make_layer(cfg, seed=11)
    x = make_tokens(cfg, 2, seed=11)
    x64 = om.bf16_to_f64(x)
    dq = lambda m: om.dequant_qmat(quant, m)
    sh = None
    if shared:
        g, u, d = layer.shared()
        sh = [_loop_ffn(x64[t], dq(g), dq(u), dq(d)) for t in range(2)]
    for e in range(cfg.num_experts):
        layer.router_bias = np.full(cfg.num_experts, -1e4, np.float32)
        layer.router_bias[e] = 1e4
        out = om.moe_forward(layer, x)
        assert np.all(out["idx"][:, 0] == e)
        assert np.all(out["w"][:, 0] == 1.0) and np.all(out["w"][:, 1:] == 0.0)
        g, u, d = layer.expert(e)
        for t in range(2):
            want = _loop_ffn(x64[t], dq(g), dq(u), dq(d))
            if shared:
                want = want + sh[t]
            assert np.allclose(out["y"][t], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("router,shared", [("softmax", 0), ("sigmoid", 1)])
def test_p8_mixed_routing_combine(router, shared):
    # generic routing: y[t] = sum_j w[t,j] * expert_{idx[t,j]}(x[t]) (+ shared),
    # with the experts evaluated by per-element loops
    cfg = _tiny(router=router, num_shared=shared, num_experts=6, top_k=3)
    layer = make_layer(cfg, seed=16)
    x = make_tokens(cfg, 4, seed=16)
    x64 = om.bf16_to_f64(x)
    out = om.moe_forward(layer, x)
    dq = lambda m: om.dequant_qmat(cfg.quant, m)
    for t in range(4):
        want = np.zeros(cfg.hidden)
        for j in range(3):
            g, u, d = layer.expert(int(out["idx"][t, j]))
            want += out["w"][t, j] * _loop_ffn(x64[t], dq(g), dq(u), dq(d))
        if shared:
            g, u, d = layer.shared()
            want += _loop_ffn(x64[t], dq(g), dq(u), dq(d))
        assert np.allclose(out["y"][t], want, rtol=1e-12, atol=1e-12)
    assert 0.0 < out["w"][:, 1:].min()


# ----------------------------------------------------------------------------
# P-14 gated shared expert: y = routed + sigmoid(x . w_s) * shared
# ----------------------------------------------------------------------------
def _gated(quant="int4_g64", seed=21):
    cfg = _tiny(router="sigmoid", num_shared=1, quant=quant).scaled(shared_gate=True)
    return cfg, make_layer(cfg, seed=seed)


@pytest.mark.parametrize("quant", ["int4_g64", "mxfp4_g32", "nvfp4_g16"])
def test_p14_gate_of_zero_halves_the_shared_expert(quant):
    """w_s = 0: the gate logit is exactly 0 and sigmoid(0) = 1/2, so the gated
    output is the ungated one minus half the shared expert's output, whose
    value comes from per-element loops."""
    cfg, layer = _gated(quant)
    x = make_tokens(cfg, 3, seed=21)
    layer.shared_gate_w = np.zeros(cfg.hidden, np.uint16)
    gated = om.moe_forward(layer, x)
    gw = layer.shared_gate_w
    layer.shared_gate_w = None
    plain = om.moe_forward(layer, x)
    layer.shared_gate_w = gw
    x64 = om.bf16_to_f64(x)
    dq = lambda m: om.dequant_qmat(quant, m)
    g, u, d = layer.shared()
    for t in range(3):
        sh = _loop_ffn(x64[t], dq(g), dq(u), dq(d))
        assert np.allclose(gated["y"][t], plain["y"][t] - 0.5 * sh, rtol=1e-12, atol=1e-12)


def test_p14_gate_weight_closed_form():
    """x = 1 everywhere and w_s with one entry 2.0 (all exact): logit 2, weight
    1 / (1 + e^-2); with the entry -2.0 the weight is 1 / (1 + e^2)."""
    cfg, layer = _gated()
    x = bf(np.ones((2, cfg.hidden)))
    for v, want in ((2.0, 1.0 / (1.0 + math.exp(-2.0))), (-2.0, 1.0 / (1.0 + math.exp(2.0)))):
        ws = np.zeros(cfg.hidden, np.float32)
        ws[37] = v
        layer.shared_gate_w = bf(ws)
        assert np.all(om.shared_gate_weight(x, layer.shared_gate_w) == want)
        out = om.moe_forward(layer, x, want_rows=True)
        assert np.all(out["shared_w"] == want)


def test_p14_saturated_gate_keeps_or_drops_the_shared_expert():
    """w_s = +-c x (a large multiple of the token's own direction): the weight
    saturates to 1 (the ungated layer) or to 0 (routed experts only, from
    per-element loops): the gate scales the shared expert, not the routed sum."""
    cfg, layer = _gated(seed=22)
    x = make_tokens(cfg, 1, seed=22)
    x64 = om.bf16_to_f64(x)
    gw = layer.shared_gate_w
    layer.shared_gate_w = None
    plain = om.moe_forward(layer, x)
    for sign in (1.0, -1.0):
        layer.shared_gate_w = bf(sign * 64.0 * x64[0])
        out = om.moe_forward(layer, x)
        if sign > 0:
            assert np.array_equal(out["y"], plain["y"])
        else:
            dq = lambda m: om.dequant_qmat(cfg.quant, m)
            want = np.zeros(cfg.hidden)
            for j in range(cfg.top_k):
                g, u, d = layer.expert(int(out["idx"][0, j]))
                want += out["w"][0, j] * _loop_ffn(x64[0], dq(g), dq(u), dq(d))
            assert np.allclose(out["y"][0], want, rtol=1e-12, atol=1e-12)
    layer.shared_gate_w = gw


def test_p10_identical_experts_make_routing_irrelevant():
    cfg = _tiny(num_experts=6, top_k=3)
    layer = make_layer(cfg, seed=12)
    for m in (layer.gate, layer.up, layer.down):
        m.codes[:] = m.codes[0]
        m.scales[:] = m.scales[0]
        m.biases[:] = m.biases[0]
    x = make_tokens(cfg, 9, seed=12)
    out = om.moe_forward(layer, x)
    g, u, d = layer.expert(0)
    dq = lambda m: om.dequant_qmat(cfg.quant, m)
    want = om.expert_ffn(om.bf16_to_f64(x), dq(g), dq(u), dq(d))
    assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-12)
    assert len(set(out["idx"].reshape(-1).tolist())) > 1


def test_p13_relabelling_experts():
    cfg = _tiny(num_experts=8, top_k=3)
    layer = make_layer(cfg, seed=13)
    x = make_tokens(cfg, 11, seed=13)
    base = om.moe_forward(layer, x)
    pi = np.random.default_rng(13).permutation(cfg.num_experts)  # new id of old expert e is pi[e]
    inv = np.argsort(pi)
    layer.router_w = layer.router_w[inv]
    layer.router_bias = None
    for m in (layer.gate, layer.up, layer.down):
        m.codes, m.scales, m.biases = m.codes[inv], m.scales[inv], m.biases[inv]
    out = om.moe_forward(layer, x)
    assert np.array_equal(out["idx"], pi[base["idx"]])
    assert np.array_equal(out["y"], base["y"])


def test_generator_keeps_outputs_in_the_bf16_error_budget():
    # |y| stays small, so bf16 rounding of y alone uses a fraction of the
    # 2e-2 max-abs / 5e-3 relative-L2 tolerance
    cfg = _tiny(num_experts=8, top_k=2, hidden=1024, ffn=256)
    layer = make_layer(cfg, seed=14)
    y = om.moe_forward(layer, make_tokens(cfg, 32, seed=14))["y"]
    assert np.abs(y).max() < 4.0
    yb = om.bf16_to_f64(f32_to_bf16_bits(y.astype(np.float32)))
    assert np.linalg.norm(yb - y) / np.linalg.norm(y) < 2e-3


# ----------------------------------------------------------------------------
# P-11 residency model
# ----------------------------------------------------------------------------
def _ordered_dict_lru(E, B, trace):
    """Textbook LRU on an OrderedDict (front = least recent); only for traces
    whose needed sets fit in one wave.  Same-call uses are refreshed in
    ascending id so ties break toward the lower id."""
    od = OrderedDict((e, None) for e in range(B))
    hits = misses = ev = 0
    for needed in trace:
        N = sorted(set(needed))
        hit = [e for e in N if e in od]
        miss = [e for e in N if e not in od]
        hits += len(hit)
        misses += len(miss)
        pinned = set(hit)
        for e in miss:
            victim = next(x for x in od if x not in pinned)
            del od[victim]
            ev += 1
            od[e] = None
            pinned.add(e)
        for e in N:
            od.move_to_end(e)
    return hits, misses, ev, set(od)


def test_p11_lru_matches_ordered_dict():
    rng = np.random.default_rng(15)
    for _ in range(30):
        E = int(rng.integers(4, 40))
        B = int(rng.integers(2, E + 1))
        trace = [rng.choice(E, size=int(rng.integers(1, B + 1)), replace=False).tolist()
                 for _ in range(60)]
        m = ResidencyModel(E, B, LRU, expert_bytes=10)
        for n in trace:
            m.forward(n)
        h, mi, ev, res = _ordered_dict_lru(E, B, trace)
        st = m.stats()
        assert (st["hits"], st["misses"], st["evictions"]) == (h, mi, ev)
        assert set(m.resident()) == res
        assert st["bytes_h2d"] == 10 * mi and st["waves"] == len(trace)


def test_p11_hand_worked_waves_and_lfu():
    # E=6, B=2; slots hold experts 0,1.  Need {0,3,4,5}: hit 0, misses 3,4,5.
    # More than B experts: no pin (floor(2/4) = 0), S = 2 streaming slots,
    # waves of 1; a miss may not evict the current or the previous wave.
    m = ResidencyModel(6, 2, LRU)
    plan = m.forward([5, 3, 0, 4])
    # [0] hit in slot 0; [3] may not take 0's slot -> evicts 1 (slot 1);
    # [4] may not take 3's -> evicts 0 (slot 0); [5] may not take 4's -> evicts 3
    assert plan == [[(0, 0, False)], [(3, 1, True)], [(4, 0, True)], [(5, 1, True)]]
    st = m.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == (1, 3, 3, 4)
    # LFU keeps the frequently used expert 0 over the recently used expert 2
    m = ResidencyModel(4, 2, LFU)
    m.forward([0])
    m.forward([0])
    m.forward([2])      # evicts 1 (use_count 0)
    m.forward([3])      # candidates 0 (count 2) and 2 (count 1): evicts 2
    assert set(m.resident()) == {0, 3}


def test_p11_streaming_forward_keeps_the_pinned_hot_expert():
    # E=10, B=4, LRU: slots hold 0..3; f1 {2} makes expert 2 the most recent.
    # f2 needs 0..7 (> B): pin floor(4/4) = 1 hit with the largest key -> 2;
    # S = 3 streaming slots, waves of 1, victims outside {current, previous, 2}
    # (keys are the values before f2's update: 2 has last_use 1, others 0):
    #   [4]: candidates 0, 1 -> 0 (slot 0)   [5]: candidates 1, 3 -> 1 (slot 1)
    #   [6]: candidates 3, 4 -> 3 (slot 3)   [7]: candidates 4, 5 -> 4 (slot 0)
    m = ResidencyModel(10, 4, LRU)
    m.forward([2])
    plan = m.forward(list(range(8)))
    assert plan == [[(0, 0, False)], [(1, 1, False)], [(2, 2, False)], [(3, 3, False)],
                    [(4, 0, True)], [(5, 1, True)], [(6, 3, True)], [(7, 0, True)]]
    assert m.resident() == {7: 0, 5: 1, 2: 2, 6: 3}
    st = m.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == (5, 4, 4, 9)
    # a forward that fits (N <= B) is one wave with no pin: {2, 8} -> evicts the
    # smallest key among 7, 5, 6 (all last_use 2) = 5
    assert m.forward([2, 8]) == [[(2, 2, False), (8, 1, True)]]


def test_p11_misses_stream_coldest_first():
    # E=6, B=2, LFU from the profile [0, 0, 5U, U, 3U, 0]: create keeps the two
    # largest scores resident (2 in slot 0, 4 in slot 1).  f1 needs {0,1,3,5}:
    # all misses, ordered by increasing key (score, last_use, id):
    # 0 (0,0,0), 1 (0,0,1), 5 (0,0,5), 3 (U,0,3) -- not ascending by id.
    # N > B: no pin (floor(2/4) = 0), S = 2, waves of 1; a page may not evict
    # the current or the previous wave:
    #   [0]: candidates 2 (5U), 4 (3U) -> 4 (slot 1)
    #   [1]: candidates 2 (0 is the previous wave) -> 2 (slot 0)
    #   [5]: candidates 0 (1 is the previous wave) -> slot 1
    #   [3]: candidates 1 (5 is the previous wave) -> slot 0
    U_ = 65536
    m = ResidencyModel(6, 2, LFU, profile=[0, 0, 5 * U_, U_, 3 * U_, 0])
    assert m.resident() == {2: 0, 4: 1}
    plan = m.forward([0, 1, 3, 5])
    assert plan == [[(0, 1, True)], [(1, 0, True)], [(5, 1, True)], [(3, 0, True)]]
    assert m.resident() == {3: 0, 5: 1}
    st = m.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["waves"]) == (0, 4, 4, 4)


def test_p11_model_rejects_bad_budgets():
    with pytest.raises(ValueError):
        ResidencyModel(4, 0)
    with pytest.raises(ValueError):
        ResidencyModel(4, 5)


# ----------------------------------------------------------------------------
# P-11b frequency decay, prefetch and expert profiles (hand-worked traces;
# U = one use = 65536)
# ----------------------------------------------------------------------------
U = 65536


def test_p11c_hybrid_forwards_hand_worked():
    """E = 5, B = 2, LFU, prefetch 1.  Create: slots [0, 1].
    hybrid {2}: no hit; 2 on the host; scores e2 = 1U; prefetch pairs the best
      non-resident (e2) with the coldest resident (e0: key (0, 0, 0)) and
      pages it into slot 0 (an eviction and a prefetch).
    hybrid {2, 3}: hit e2 (slot 0; a prefetch hit), 3 on the host; scores e2 =
      2U, e3 = 1U; prefetch pages e3 over e1 (slot 1).
    plain {4}: a miss; victims outside the wave: e3 (1U) before e2 (2U):
      e4 takes slot 1."""
    m = ResidencyModel(5, 2, LFU, expert_bytes=10, prefetch=1)
    assert m.forward_hybrid([2]) == ([], [2])
    assert m.resident() == {2: 0, 1: 1}
    assert m.forward_hybrid([3, 2]) == ([(2, 0)], [3])
    assert m.resident() == {2: 0, 3: 1}
    assert m.forward([4]) == [[(4, 1, True)]]
    st = m.stats()
    assert (st["forwards"], st["hits"], st["host_experts"], st["misses"], st["evictions"], st["prefetched"],
            st["prefetch_hits"], st["bytes_h2d"], st["waves"]) == (3, 1, 2, 1, 3, 2, 1, 30, 3)


def test_p11c_hybrid_without_prefetch_moves_no_slot():
    m = ResidencyModel(8, 3, LRU, expert_bytes=7)
    for need in ([5, 6], [0, 7], [1, 2, 3, 4]):
        m.forward_hybrid(need)
    assert m.resident() == {0: 0, 1: 1, 2: 2}
    st = m.stats()
    assert st["misses"] == st["evictions"] == st["bytes_h2d"] == 0
    # hits: e0 (second forward), e1 and e2 (third); on the host: 5, 6, 7, 3, 4
    assert st["hits"] == 3 and st["host_experts"] == 5 and st["waves"] == 3
    # the uses still count: a plain forward now evicts the least recent (e0,
    # used in the second forward, before e1 and e2 of the third)
    assert m.forward([6]) == [[(6, 0, True)]]


def test_p11d_hybrid_prefill_split_hand_worked():
    """E = 8, B = 2, LRU, row limit 2.  Create: slots [0, 1].
    {0: 5 rows, 1: 4, 3: 1, 5: 3}: hits 0, 1; e3 (1 row, not resident) to the
      host; e5 (3 rows) is a miss.  Order [0, 1, 5] is longer than B, so
      floor(B/4) = 0 hits are pinned, S = 2, W = 1, previous wave kept: waves
      [0], [1], [5]; e5 may evict neither e5 (current) nor e1 (previous):
      e0's slot 0.
    {3: 2 rows, 5: 9}: e5 hits slot 0; e3 (2 rows, not resident) to the host.
    {6: 1 row}: all on the host; no wave runs an expert, one is counted.
    {1: 1 row}: e1 is resident (slot 1): a hit, whatever its rows."""
    m = ResidencyModel(8, 2, LRU, expert_bytes=10)
    rows = {0: 5, 1: 4, 3: 1, 5: 3}
    plan, host = m.forward_split([0, 1, 3, 5], rows, host_rows=2)
    assert plan == [[(0, 0, False)], [(1, 1, False)], [(5, 0, True)]] and host == [3]
    assert m.resident() == {5: 0, 1: 1}
    assert m.forward_split([3, 5], {3: 2, 5: 9}, host_rows=2) == ([[(5, 0, False)]], [3])
    assert m.forward_split([6], {6: 1}, host_rows=2) == ([], [6])
    assert m.forward_split([1], {1: 1}, host_rows=2) == ([[(1, 1, False)]], [])
    st = m.stats()
    assert (st["forwards"], st["hits"], st["misses"], st["evictions"], st["host_experts"], st["waves"],
            st["bytes_h2d"]) == (4, 4, 1, 1, 3, 6, 10)
    # every needed expert counts as used: LRU last uses are 1 (e0), 4 (e1),
    # 2 (e3), 2 (e5), 3 (e6), so a plain forward needing e7 evicts e5
    assert m.forward([7]) == [[(7, 0, True)]]


def test_p11d_row_limit_zero_is_the_plain_forward():
    a, b = ResidencyModel(16, 4, LFU, expert_bytes=3), ResidencyModel(16, 4, LFU, expert_bytes=3)
    rng = np.random.default_rng(7)
    for _ in range(30):
        need = sorted(set(rng.integers(0, 16, size=6).tolist()))
        rows = {e: int(rng.integers(1, 5)) for e in need}
        assert a.forward(need) == b.forward_split(need, rows, host_rows=0)[0]
    assert a.stats() == b.stats()


def test_p11b_decay_changes_the_victim():
    # E=3, B=2 (slots hold 0 and 1).  Expert 0 is used three times, expert 2
    # twice later, then expert 1 is needed.  Scores under WARM d=1, by hand:
    #   f1..f3 {0}: s0 = U, 1.5U, 1.75U          (decay halves, then +U)
    #   f4 {2}: miss, evicts 1 (score 0);  s0 = 0.875U, s2 = U
    #   f5 {2}: hit;                       s0 = 0.4375U = 28672, s2 = 1.5U = 98304
    #   f6 {1}: miss; WARM evicts 0 (28672 < 98304), LFU evicts 2 (3U > 2U).
    trace = [[0], [0], [0], [2], [2], [1]]
    m = ResidencyModel(3, 2, "warm", decay_shift=1)
    for n in trace[:5]:
        m.forward(n)
    assert m.profile() == [28672, 0, 98304]
    assert m.forward([1]) == [[(1, 0, True)]]       # expert 0 sat in slot 0
    m = ResidencyModel(3, 2, LFU)
    for n in trace[:5]:
        m.forward(n)
    assert m.profile() == [3 * U, 0, 2 * U]
    assert m.forward([1]) == [[(1, 1, True)]]       # expert 2 sat in slot 1
    # decay rounds the loss down: 5 - (5 >> 2) = 4, 5 - (5 >> 1) = 3, and a
    # score of 1 never decays (1 >> d = 0 for d >= 1)
    m = ResidencyModel(3, 1, "warm", decay_shift=2, profile=[5, 1, 0])
    m.forward([2])
    assert m.profile() == [4, 1, U]
    m = ResidencyModel(3, 1, "warm", decay_shift=1, profile=[5, 1, 0])
    m.forward([2])
    assert m.profile() == [3, 1, U]


def test_p11b_prefetch_restores_the_hot_expert():
    # E=3, B=2, LFU, prefetch 1.  {0,1} three times (s0 = s1 = 3U, last_use 3);
    # f4 {2}: miss evicts 0 (key (3U,3,0) < (3U,3,1)) into slot 0; s2 = U.
    # Prefetch: candidate 0 rank (3U,3) > smallest resident 2 rank (U,4):
    # 0 is paged back into slot 0.  f5 {0} is then a hit from the prefetch.
    m = ResidencyModel(3, 2, LFU, expert_bytes=10, prefetch=1)
    for _ in range(3):
        m.forward([0, 1])
    assert m.forward([2]) == [[(2, 0, True)]]
    assert m.resident() == {0: 0, 1: 1}
    assert m.forward([0]) == [[(0, 0, False)]]
    st = m.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["prefetched"], st["prefetch_hits"],
            st["bytes_h2d"]) == (7, 1, 2, 1, 1, 20)
    # without prefetch the same trace misses on f5
    m = ResidencyModel(3, 2, LFU, expert_bytes=10)
    for n in [[0, 1]] * 3 + [[2], [0]]:
        m.forward(n)
    st = m.stats()
    assert (st["hits"], st["misses"], st["prefetched"]) == (6, 2, 0)
    # equal ranks never swap: after f1 {2} (evicts 0) the non-residents 0 and
    # 3 have rank (0, 0), the same as resident 1, so nothing is paged ahead
    m = ResidencyModel(4, 2, LFU, prefetch=2)
    m.forward([2])
    assert m.resident() == {2: 0, 1: 1} and m.stats()["prefetched"] == 0


def test_p11b_profile_warm_start_and_reload():
    # profile [5, 0, 9U, 9U, 1], B=2: wanted = {2, 3}; slots 0,1 freed, 2 -> slot 0,
    # 3 -> slot 1, nothing counted at create
    prof = [5, 0, 9 * U, 9 * U, 1]
    m = ResidencyModel(5, 2, "warm", expert_bytes=7, decay_shift=2, profile=prof)
    assert m.resident() == {2: 0, 3: 1}
    assert m.stats()["prefetched"] == 0 and m.stats()["bytes_h2d"] == 0
    assert m.forward([2]) == [[(2, 0, False)]]
    # d=2: s2 = 9U - 9U/4 + U = 507904; s3 = 442368; s0 = 5 - 1 = 4; s4 = 1
    assert m.profile() == [4, 0, 507904, 442368, 1]
    # run-time load [0,0,0,0,100]: wanted = {4, 0} (ties to the lower id);
    # both residents leave, 0 -> slot 0, 4 -> slot 1; two prefetches, two evictions
    m.load_profile([0, 0, 0, 0, 100])
    assert m.resident() == {0: 0, 4: 1}
    st = m.stats()
    assert (st["prefetched"], st["evictions"], st["bytes_h2d"]) == (2, 2, 14)
    m.forward([4])
    assert m.stats()["prefetch_hits"] == 1
    # a zero profile keeps the default slots; a wrong length or huge score is refused
    assert ResidencyModel(5, 2, LFU, profile=[0] * 5).resident() == {0: 0, 1: 1}
    with pytest.raises(ValueError):
        ResidencyModel(5, 2, LFU, profile=[0] * 4)
    with pytest.raises(ValueError):
        ResidencyModel(5, 2, LFU, profile=[0, 0, 0, 0, 1 << 63])
    with pytest.raises(ValueError):
        ResidencyModel(5, 2, "warm")                 # warm needs a decay
    with pytest.raises(ValueError):
        ResidencyModel(5, 2, LRU, decay_shift=3)     # decay is warm only
    with pytest.raises(ValueError):
        ResidencyModel(5, 2, LRU, prefetch=3)        # prefetch above B


def test_p11b_full_prefetch_keeps_the_top_ranked_set():
    """With prefetch = B, after every forward no non-resident outranks a
    resident (ranks compared without ids); brute force over random traces."""
    rng = np.random.default_rng(33)
    for policy, d in ((LFU, 0), ("warm", 1), ("warm", 5), (LRU, 0)):
        for _ in range(20):
            E = int(rng.integers(3, 24))
            B = int(rng.integers(1, E))
            m = ResidencyModel(E, B, policy, decay_shift=d, prefetch=B)
            p = 1.0 / np.arange(1, E + 1) ** 1.2
            for _ in range(40):
                n = rng.choice(E, size=int(rng.integers(1, E + 1)), replace=False, p=p / p.sum())
                m.forward(n.tolist())
                res = m.resident()
                rank = (lambda e: (m.last_use[e],)) if policy == LRU else \
                    (lambda e: (m.score[e], m.last_use[e]))
                inside = min(rank(e) for e in res)
                outside = [rank(e) for e in range(E) if e not in res]
                assert not outside or max(outside) <= inside


def test_p11b_decay_is_exponential_forgetting():
    """An expert used once and then never again follows
    s_{n+1} = s_n - floor(s_n / 2**d): the loss is rounded down, so s_n lies
    between U (1 - 2**-d)**n and that plus n."""
    for d in (1, 3, 6):
        m = ResidencyModel(2, 1, "warm", decay_shift=d)
        m.forward([1])
        for n in range(1, 60):
            m.forward([0])
            exact = U * (1 - 2.0 ** -d) ** n
            assert exact - 1e-9 <= m.score[1] <= exact + n
