"""Seeded synthetic workloads for the routed 4-bit MoE FFN layer.

This module only draws random numbers and encodes them into the packed byte
formats the layer consumes.  It holds none of the layer's forward arithmetic
(no router, no dequantisation, no expert FFN, no combine): both the CPU oracle
and the HIP path are fed from here and neither is imported by this file.

Shapes follow the five layer configurations the work is measured on
(a tiny correctness layer, a Mixtral-8x7B-shaped layer, a Qwen3-30B-A3B-shaped
layer, a GLM-4.5-Air-shaped layer and a 512-expert MXFP4 layer).  The pages
describe these model families only by their expert counts and top-k
(strata.amperor.ai landing page "% of experts hot" lines; the Medium tutorial
section 2: 512 experts, 10 routed + 1 shared), so the value distributions are
a stated recipe, not data:

* activations x ~ N(0, 1), rounded to bf16 (round-to-nearest-even);
* router weights Wr ~ N(0, 1/H) in bf16, so logits are roughly N(0, 1);
* a Zipf(s) logit bias b_e = -s * ln(rank_e), rank a random permutation of
  1..E, for the configurations whose routing is Zipf-skewed;
* expert weights Wg, Wu ~ N(0, 1/H), Wd ~ N(0, 0.25/F);
* int4 group-64 affine encoding: per group scale = (max - min) / 15 and
  bias = min, both rounded to bf16, code = clamp(rint((w - bias)/scale), 0, 15);
* MXFP4 encoding (OCP MX v1.0 recommended conversion): E8M0 exponent
  floor(log2(amax)) - 2 + 127 clamped to [1, 254], E2M1 round-to-nearest-even
  with saturation at +-6;
* int4 group-128: as group-64 with groups of 128;
* NVFP4 encoding (the published two-level recipe): fp32 matrix scale
  amax / (6 * 448), E4M3 block scale per 16 rounded to nearest, E2M1 codes.

Packing (the layout the C ABI takes, row-major [out, in], quantised along in):
codes u8 [rows, in/2] with element 2i in the low nibble of byte i.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

INT4 = "int4_g64"
INT4_G128 = "int4_g128"
MXFP4 = "mxfp4_g32"
NVFP4 = "nvfp4_g16"
AFFINE = (INT4, INT4_G128)
SOFTMAX = "softmax"
SIGMOID = "sigmoid"


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int
    hidden: int
    ffn: int
    num_experts: int
    top_k: int
    num_shared: int
    quant: str
    router: str
    zipf_s: Optional[float]
    budget_frac: float
    decode_T: tuple
    prefill_T: int
    shared_gate: bool = False  # the shared expert's output is scaled by sigmoid(x . w_s)

    @property
    def group(self) -> int:
        return {INT4: 64, INT4_G128: 128, MXFP4: 32, NVFP4: 16}[self.quant]

    @property
    def budget(self) -> int:
        # budget rounding: max(1, floor(p * E))
        return max(1, int(math.floor(self.budget_frac * self.num_experts + 1e-9)))

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def expert_bytes(self) -> int:
        """Packed bytes of one expert (gate + up + down: codes, scales, biases)."""
        H, F, G = self.hidden, self.ffn, self.group
        if self.quant in AFFINE:
            per = lambda n, k: n * k // 2 + 2 * (n * (k // G)) * 2
        else:
            per = lambda n, k: n * k // 2 + n * (k // G)
        extra = 3 * 4 if self.quant == NVFP4 else 0  # one fp32 scale per matrix
        return 2 * per(F, H) + per(H, F) + extra

    def scaled(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig("tiny", 0, 512, 1024, 8, 2, 0, INT4, SOFTMAX, None, 1.0, (16,), 16),
    "mixtral": LayerConfig("mixtral", 1, 4096, 14336, 8, 2, 0, INT4, SOFTMAX, None, 0.5, (1,), 512),
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", 2, 2048, 768, 128, 8, 0, INT4, SOFTMAX, 1.1, 0.25,
                                 (1,), 1180),
    "glm45_air": LayerConfig("glm45_air", 3, 4096, 1408, 128, 8, 1, INT4, SIGMOID, None, 0.09,
                             (1, 2, 4, 8), 1180),
    "e512_mxfp4": LayerConfig("e512_mxfp4", 4, 2048, 512, 512, 10, 1, MXFP4, SOFTMAX, 1.1, 0.18,
                              (1,), 4096),
}
CONFIG_ORDER = ["tiny", "mixtral", "qwen3_30b_a3b", "glm45_air", "e512_mxfp4"]

# Wider routing (the ro99/strata README model table lists an 896-expert top-16
# MXFP4 model and 256-expert top-6 FP4 models; it gives no hidden or expert
# sizes, so those, the router kind and the budgets here are choices of this
# recipe, not the pages').
WIDE_CONFIGS = {
    "e896_top16_mxfp4": LayerConfig("e896_top16_mxfp4", 5, 2048, 512, 896, 16, 0, MXFP4, SOFTMAX, 1.1,
                                    0.18, (1,), 2048),
    "e256_top6_fp4": LayerConfig("e256_top6_fp4", 6, 4096, 1024, 256, 6, 0, MXFP4, SIGMOID, None, 0.25,
                                 (1,), 1180),
}
WIDE_ORDER = ["e896_top16_mxfp4", "e256_top6_fp4"]
CONFIGS.update(WIDE_CONFIGS)

# More 4-bit formats (the same table: a 256-expert top-8 model in INT4
# group-128 W4A16, and a 256-expert + 1 shared top-10 model in NVFP4 or
# MXFP4).  Again H, F, router kind, bias and budgets are this recipe's choices.
FORMAT_CONFIGS = {
    "e256_int4g128": LayerConfig("e256_int4g128", 7, 2048, 1024, 256, 8, 0, INT4_G128, SIGMOID, None,
                                 0.1, (1,), 1180),
    "e256_nvfp4": LayerConfig("e256_nvfp4", 8, 2048, 512, 256, 10, 1, NVFP4, SOFTMAX, 1.1, 0.18,
                              (1,), 2048),
}
FORMAT_ORDER = ["e256_int4g128", "e256_nvfp4"]
CONFIGS.update(FORMAT_CONFIGS)


# ----------------------------------------------------------------------------
# bf16 helpers (encoding only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# quantisers (encode float weights into the packed formats)
# ----------------------------------------------------------------------------
def _pack_nibbles(q: np.ndarray) -> np.ndarray:
    """q uint8 [..., K] with values 0..15 -> u8 [..., K/2]; element 2i low nibble."""
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def quantize_int4(w: np.ndarray, group: int):
    """w float32 [N, K] -> (codes u8 [N,K/2], scales bf16 bits [N,K/G], biases bf16 bits [N,K/G])."""
    N, K = w.shape
    g = w.reshape(N, K // group, group).astype(np.float32)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    s_bits = f32_to_bf16_bits((mx - mn) / np.float32(15.0))
    b_bits = f32_to_bf16_bits(mn)
    s = bf16_bits_to_f32(s_bits)[..., None]
    b = bf16_bits_to_f32(b_bits)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - b) / np.where(s > 0, s, 1)), 0)
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(N, K)
    return _pack_nibbles(q), s_bits, b_bits


def quantize_int4_g64(w: np.ndarray):
    return quantize_int4(w, 64)


# E2M1 magnitudes in code order (sign is bit 3); used here only to encode.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto the E2M1 grid, saturating at 6; returns 4-bit codes."""
    a = np.abs(v)
    # midpoints between consecutive grid values; at a tie the even code
    # (mantissa bit 0: codes 0, 2, 4, 6) wins
    mids = ((_E2M1_GRID[:-1] + _E2M1_GRID[1:]) / 2.0).astype(a.dtype)
    code = np.searchsorted(mids, a, side="left")  # a == mid -> lower code
    tie = a == mids[np.minimum(code, 6)]
    code = code + (tie & (code % 2 == 1))
    code = np.minimum(code, 7).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8)
    return code | (sign << 3)


def quantize_mxfp4_g32(w: np.ndarray):
    """w float32 [N, K] -> (codes u8 [N,K/2], e8m0 scales u8 [N,K/32])."""
    N, K = w.shape
    g = w.reshape(N, K // 32, 32)
    amax = np.abs(g).max(axis=2).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1e-300))) - 2 + 127
    e = np.clip(e, 1, 254).astype(np.int32)
    # division by a power of two is exact, in float32 as in float64 (normal range)
    scaled = g.astype(np.float64) / np.exp2(e - 127.0)[..., None]
    codes = _e2m1_encode(scaled).reshape(N, K)
    return _pack_nibbles(codes), e.astype(np.uint8)


# E4M3 (OCP FP8, bias 7) magnitudes of the 127 non-NaN non-negative codes, in
# code order; used here only to encode scales.
_E4M3_GRID = np.array([(m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
                       for e in range(16) for m in range(8)][:127], dtype=np.float64)


def _e4m3_encode_pos(v: np.ndarray) -> np.ndarray:
    """Non-negative values -> E4M3 codes, round to nearest (ties to even code),
    saturating at 448 (code 0x7E)."""
    mids = (_E4M3_GRID[:-1] + _E4M3_GRID[1:]) / 2.0
    code = np.searchsorted(mids, v, side="left")
    tie = v == mids[np.minimum(code, 125)]
    code = code + (tie & (code % 2 == 1))
    return np.minimum(code, 126).astype(np.uint8)


def quantize_nvfp4_g16(w: np.ndarray):
    """w float32 [N, K] -> (codes u8 [N,K/2], E4M3 scales u8 [N,K/16], fp32 matrix scale).

    The usual two-level recipe: matrix scale g = amax / (6 * 448); block scale =
    E4M3(amax_block / (6 * g)); codes = E2M1(w / (block scale * g)), RNE."""
    N, K = w.shape
    amax = float(np.abs(w).max())
    g = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blk = w.reshape(N, K // 16, 16).astype(np.float64)
    bmax = np.abs(blk).max(axis=2)
    sc = _e4m3_encode_pos(bmax / (6.0 * float(g)))
    sval = _E4M3_GRID[sc]
    with np.errstate(divide="ignore", invalid="ignore"):
        scaled = np.where(sval[..., None] > 0, blk / (sval[..., None] * float(g)), 0.0)
    codes = _e2m1_encode(scaled).reshape(N, K)
    return _pack_nibbles(codes), sc, g


# ----------------------------------------------------------------------------
# layer weights
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class QMat:
    codes: np.ndarray
    scales: np.ndarray
    biases: Optional[np.ndarray]
    global_scale: Optional[np.ndarray] = None  # NVFP4: fp32 per matrix ([E] for a stack)


@dataclasses.dataclass
class LayerWeights:
    cfg: LayerConfig
    router_w: np.ndarray            # uint16 bf16 bits [E, H]
    router_bias: Optional[np.ndarray]  # float32 [E] or None
    gate: QMat                      # stacked over E
    up: QMat
    down: QMat
    sh_gate: Optional[QMat] = None
    sh_up: Optional[QMat] = None
    sh_down: Optional[QMat] = None
    shared_gate_w: Optional[np.ndarray] = None  # uint16 bf16 bits [H]: the shared expert's gate row

    def expert(self, e: int):
        """(gate, up, down) QMats of routed expert e (views)."""
        def sl(m):
            return QMat(m.codes[e], m.scales[e], None if m.biases is None else m.biases[e],
                        None if m.global_scale is None else m.global_scale[e])
        return sl(self.gate), sl(self.up), sl(self.down)

    def shared(self):
        def sl(m):
            return QMat(m.codes[0], m.scales[0], None if m.biases is None else m.biases[0],
                        None if m.global_scale is None else m.global_scale[0])
        return sl(self.sh_gate), sl(self.sh_up), sl(self.sh_down)


def _quant(cfg: LayerConfig, w: np.ndarray) -> QMat:
    if cfg.quant in AFFINE:
        c, s, b = quantize_int4(w, cfg.group)
        return QMat(c, s, b)
    if cfg.quant == NVFP4:
        c, s, g = quantize_nvfp4_g16(w)
        return QMat(c, s, None, np.float32(g))
    c, s = quantize_mxfp4_g32(w)
    return QMat(c, s, None)


def _alloc_stack(cfg: LayerConfig, n_exp: int, rows: int, cols: int) -> QMat:
    G = cfg.group
    codes = np.empty((n_exp, rows, cols // 2), np.uint8)
    if cfg.quant in AFFINE:
        return QMat(codes, np.empty((n_exp, rows, cols // G), np.uint16),
                    np.empty((n_exp, rows, cols // G), np.uint16))
    if cfg.quant == NVFP4:
        return QMat(codes, np.empty((n_exp, rows, cols // G), np.uint8), None,
                    np.empty((n_exp,), np.float32))
    return QMat(codes, np.empty((n_exp, rows, cols // G), np.uint8), None)


def _store(dst: QMat, e: int, src: QMat):
    dst.codes[e] = src.codes
    dst.scales[e] = src.scales
    if dst.biases is not None:
        dst.biases[e] = src.biases
    if dst.global_scale is not None:
        dst.global_scale[e] = src.global_scale


def _gen_expert(cfg: LayerConfig, seed: int, e: int):
    """One expert's (gate, up, down) from its own stream, so experts generate in parallel."""
    H, F = cfg.hidden, cfg.ffn
    rng = np.random.default_rng([seed, 104729, e])
    sg, sd = np.float32(1.0 / math.sqrt(H)), np.float32(math.sqrt(0.25 / F))
    g = _quant(cfg, rng.standard_normal((F, H), dtype=np.float32) * sg)
    u = _quant(cfg, rng.standard_normal((F, H), dtype=np.float32) * sg)
    d = _quant(cfg, rng.standard_normal((H, F), dtype=np.float32) * sd)
    return g, u, d


def _gen_experts(cfg: LayerConfig, seed: int, first: int, n_exp: int, threads: int):
    H, F = cfg.hidden, cfg.ffn
    gate = _alloc_stack(cfg, n_exp, F, H)
    up = _alloc_stack(cfg, n_exp, F, H)
    down = _alloc_stack(cfg, n_exp, H, F)

    def one(i):
        g, u, d = _gen_expert(cfg, seed, first + i)
        _store(gate, i, g)
        _store(up, i, u)
        _store(down, i, d)

    if threads > 1 and n_exp > 1:
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(n_exp)))
    else:
        for i in range(n_exp):
            one(i)
    return gate, up, down


def make_layer(cfg: LayerConfig, seed: Optional[int] = None, threads: Optional[int] = None) -> LayerWeights:
    """Seeded synthetic layer weights for `cfg` (deterministic in seed, whatever the thread count).

    Routed expert e draws from the stream (seed, 104729, e); the shared expert
    from (seed, 104729, E); a shared-expert gate row w_s ~ N(0, 1/H) in bf16
    from (seed, 4241)."""
    seed = cfg.seed if seed is None else seed
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    rng = np.random.default_rng(seed)
    H, E = cfg.hidden, cfg.num_experts
    router_w = f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32)
                                * np.float32(1.0 / math.sqrt(H)))
    bias = None
    if cfg.zipf_s is not None:
        rank = 1 + rng.permutation(E)
        bias = (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    gate, up, down = _gen_experts(cfg, seed, 0, E, threads)
    lw = LayerWeights(cfg, router_w, bias, gate, up, down)
    if cfg.num_shared:
        lw.sh_gate, lw.sh_up, lw.sh_down = _gen_experts(cfg, seed, E, 1, 1)
        if cfg.shared_gate:
            g = np.random.default_rng([seed, 4241])
            lw.shared_gate_w = f32_to_bf16_bits(g.standard_normal(H, dtype=np.float32)
                                                * np.float32(1.0 / math.sqrt(H)))
    return lw


def make_tokens(cfg: LayerConfig, T: int, step: int = 0, seed: Optional[int] = None,
                topic: Optional[int] = None, strength: float = 1.0) -> np.ndarray:
    """Activations x ~ N(0,1) in bf16 bits, uint16 [T, H]; one stream per step.

    With `topic`, every token also carries `strength` times a fixed N(0,1)
    direction drawn from (seed, 31337, topic): a stand-in for one kind of
    work, which moves the router's preferred experts (a topic shift moves the
    hot set)."""
    base = cfg.seed if seed is None else seed
    rng = np.random.default_rng([base, 7919, step])
    x = rng.standard_normal((T, cfg.hidden), dtype=np.float32)
    if topic is not None:
        v = np.random.default_rng([base, 31337, topic]).standard_normal(cfg.hidden, dtype=np.float32)
        x = x + np.float32(strength) * v
    return f32_to_bf16_bits(x)
