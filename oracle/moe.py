"""Plain CPU definition of one routed 4-bit MoE FFN layer (test infrastructure only).

Sources, cited by page title and section:

* "Documentation" (strata.amperor.ai docs), Signature: a layer keeps a budget
  of resident experts; everything else is streamed.  Budgets do not change the
  result, so nothing here models them.
* ro99/strata README (C++20/CUDA engine), precision paragraph: MXFP4 packs two
  E2M1 codes per byte with one E8M0 exponent per group of 32 and is read as
  such; an E8M0 byte is placed in a bf16 exponent field, so bytes 0 and 255
  (+0 and +inf there) are refused when the checkpoint is admitted.
* Same README, its list of enforced rules: the router's arithmetic, the expert
  count and k are the checkpoint's; prediction changes the order of work only,
  never its numbers.
* "Strata, Explained" (Medium tutorial), section 2: a 512-expert layer runs
  10 routed experts plus 1 shared expert per token.

Where the pages are silent the readings below are taken (each is listed in the
design notes of the repository):

R2  router logit l[t,e] = sum_h x[t,h]*Wr[e,h] in fp32, summed in one fixed
    order: 64 lanes; lane L accumulates h = (c*64 + L)*8 + v for chunk
    c = 0..H/512-1 and v = 0..7 in increasing (c, v) from +0 with a fused
    multiply-add (the bf16 x bf16 product is exact in fp32, so this is one
    rounding per term); the 64 partials are then folded pairwise with offsets
    32, 16, 8, 4, 2, 1 (p[L] += p[L+o]) and lane 0 is the sum; an optional
    fp32 bias is added last.
R3  top-k by (logit descending, expert id ascending), -0 == +0.
R4  weights: softmax restricted to the selected logits, or sigmoid of each
    selected logit divided by their sum; no epsilon, no scaling.
R5  tokens grouped by expert, ascending expert id, ascending token within one.
R6  nibble 2i of a row is the low nibble of byte i.  int4: w = s*q + b with
    bf16 s, b per 64 (or 128) along the input dim.  MXFP4: E2M1 value times
    2^(e-127).  NVFP4 (named, not defined, in the ro99/strata README model
    table; taken as the published format): E2M1 value times an E4M3 (OCP FP8,
    bias 7) scale per 16 inputs times one fp32 scale per matrix; E4M3 NaN
    bytes (0x7F, 0xFF) are refused like E8M0 0/255.
R7  expert: g = Wg x, u = Wu x, a = silu(g)*u, o = Wd a; the shared expert is
    the same FFN with weight 1, or, for a layer that carries a shared-expert
    gate row w_s (the ro99/strata README's model table lists shared experts
    beside routed ones without saying how they are weighted, so the gated
    form is a reading), with weight sigmoid(l_s), l_s = x . w_s formed in fp32
    in the R2 order like a router logit.
R8  y[t] = sum_j w[t,j] o_j + g_t shared(x[t]), j ascending, shared last
    (g_t = 1 without a gate).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# decoding of stored numbers
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): the bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """u8 [N, K/2] -> int [N, K]; element 2i is the low nibble of byte i (R6)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


def dequant_int4_affine(codes, scales, biases, group) -> np.ndarray:
    """int4 affine: w[n,k] = s[n,k//G] * q[n,k] + b[n,k//G] (R6), fp64 [N, K]."""
    q = _unpack_nibbles(codes).astype(np.float64)
    N, K = q.shape
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    assert s.shape == (N, K // group) and b.shape == (N, K // group)
    return (q.reshape(N, K // group, group) * s[..., None] + b[..., None]).reshape(N, K)


def dequant_int4_g64(codes, scales, biases) -> np.ndarray:
    return dequant_int4_affine(codes, scales, biases, 64)


def dequant_int4_g128(codes, scales, biases) -> np.ndarray:
    return dequant_int4_affine(codes, scales, biases, 128)


def e2m1_value(code) -> np.ndarray:
    """E2M1 from its bits: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    ex = (c >> 1) & 3
    man = c & 1
    mag = np.where(ex == 0, man * 0.5, np.exp2(ex - 1.0) * (1.0 + man * 0.5))
    return sign * mag


def e8m0_value(s) -> np.ndarray:
    """E8M0 byte as an exponent field: 2^(s-127); bytes 0 and 255 are refused
    (ro99/strata README, precision paragraph)."""
    s = np.asarray(s, dtype=np.int64)
    if np.any((s == 0) | (s == 255)):
        raise ValueError("E8M0 scale byte 0 or 255: checkpoint fails admission")
    return np.exp2(s - 127.0)


def dequant_mxfp4_g32(codes, scales) -> np.ndarray:
    """MXFP4: w[n,k] = e2m1(code[n,k]) * 2^(s[n,k//32]-127), fp64 [N, K]."""
    v = e2m1_value(_unpack_nibbles(codes))
    N, K = v.shape
    sc = e8m0_value(scales)
    assert sc.shape == (N, K // 32)
    return (v.reshape(N, K // 32, 32) * sc[..., None]).reshape(N, K)


def e4m3_value(b) -> np.ndarray:
    """OCP FP8 E4M3 from its bits: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN
    and is refused (a scale must be a number), there is no infinity."""
    b = np.asarray(b, dtype=np.int64)
    if np.any((b & 0x7F) == 0x7F):
        raise ValueError("E4M3 scale byte is NaN: checkpoint fails admission")
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    ex = (b >> 3) & 15
    man = b & 7
    mag = np.where(ex == 0, man * 2.0 ** -9, np.exp2(ex - 7.0) * (1.0 + man / 8.0))
    return sign * mag


def dequant_nvfp4_g16(codes, scales, global_scale) -> np.ndarray:
    """NVFP4: w[n,k] = e2m1(code[n,k]) * e4m3(s[n,k//16]) * g, fp64 [N, K]."""
    v = e2m1_value(_unpack_nibbles(codes))
    N, K = v.shape
    sc = e4m3_value(scales)
    assert sc.shape == (N, K // 16)
    g = float(np.float32(global_scale))
    if not np.isfinite(g) or g <= 0:
        raise ValueError("NVFP4 matrix scale must be finite and positive")
    return (v.reshape(N, K // 16, 16) * sc[..., None]).reshape(N, K) * g


def dequant_qmat(quant: str, m) -> np.ndarray:
    """Dequantise one packed matrix object with .codes/.scales/.biases
    (and .global_scale for NVFP4)."""
    if quant == "int4_g64":
        return dequant_int4_g64(m.codes, m.scales, m.biases)
    if quant == "int4_g128":
        return dequant_int4_g128(m.codes, m.scales, m.biases)
    if quant == "mxfp4_g32":
        return dequant_mxfp4_g32(m.codes, m.scales)
    if quant == "nvfp4_g16":
        return dequant_nvfp4_g16(m.codes, m.scales, m.global_scale)
    raise ValueError(f"unknown quant {quant!r}")


# ----------------------------------------------------------------------------
# router (R2..R4)
# ----------------------------------------------------------------------------
def router_logits_fp32(x_bits, wr_bits, bias=None) -> np.ndarray:
    """fp32 router logits [T, E] in the fixed summation order R2.

    Each step adds one exact bf16*bf16 product to a lane partial with one fp32
    rounding (numpy's float32 product is exact whenever it is zero or at least
    2^-126 in magnitude, which is checked up front, so mul-then-add here equals
    a fused multiply-add)."""
    x = bf16_to_f32(x_bits)
    w = bf16_to_f32(wr_bits)
    T, H = x.shape
    E = w.shape[0]
    if H % 512:
        raise ValueError("hidden size must be a multiple of 512 for the router order")
    C = H // 512
    ax, aw = np.abs(x[x != 0]), np.abs(w[w != 0])
    if ax.size and aw.size and float(ax.min()) * float(aw.min()) < 2.0 ** -126:
        raise ValueError("a router product may fall below the fp32 normal range: outside the contract")
    xr = x.reshape(T, C, 64, 8)
    wrr = w.reshape(E, C, 64, 8)
    p = np.zeros((T, E, 64), dtype=np.float32)
    for c in range(C):
        for v in range(8):
            p = p + xr[:, None, c, :, v] * wrr[None, :, c, :, v]
    o = 32
    while o >= 1:
        p[:, :, :o] = p[:, :, :o] + p[:, :, o:2 * o]
        o //= 2
    logits = p[:, :, 0].copy()
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32)[None, :]
    return logits


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """idx [T, k] int32: the k largest logits per row, ties to the lower expert id (R3)."""
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    if not np.all(np.isfinite(l)):
        raise ValueError("non-finite logits are outside the contract")
    ids = np.broadcast_to(np.arange(E), (T, E))
    neg = -(l.astype(np.float64)) + 0.0  # +0.0 folds -0 into +0
    order = np.lexsort((ids, neg), axis=1)
    return order[:, :k].astype(np.int32)


def routing_weights(logits: np.ndarray, idx: np.ndarray, router: str) -> np.ndarray:
    """w [T, k] fp64 from the fp32 logits of the selected experts (R4)."""
    sel = np.take_along_axis(np.asarray(logits, np.float32), idx, axis=1).astype(np.float64)
    if router == "softmax":
        z = np.exp(sel - sel[:, :1])
        return z / z.sum(axis=1, keepdims=True)
    if router == "sigmoid":
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-sel))
        return sg / sg.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown router {router!r}")


# ----------------------------------------------------------------------------
# permutation (R5)
# ----------------------------------------------------------------------------
def permute(idx: np.ndarray, num_experts: int):
    """counts[E], offsets[E+1], perm[T*k] (token ids grouped by expert, ascending
    token inside an expert) and pos[T,k] (row of (t, idx[t,j]) in perm)."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    flat_j = np.tile(np.arange(k), T)
    for t in range(T):
        if len(set(idx[t].tolist())) != k:
            raise ValueError("a token selected one expert twice")
    counts = np.bincount(flat_e, minlength=num_experts).astype(np.int32)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.lexsort((flat_t, flat_e))  # by expert, then token
    perm = flat_t[order].astype(np.int32)
    pos = np.empty((T, k), dtype=np.int32)
    pos[flat_t[order], flat_j[order]] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, perm, pos


# ----------------------------------------------------------------------------
# experts and combine (R7, R8)
# ----------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert on rows of x (fp64): o = Wd (silu(Wg x) * (Wu x))."""
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


def moe_forward(layer, x_bits, tokens=None, want_rows=False) -> dict:
    """Forward of the whole layer for the bf16 activations `x_bits` [T, H].

    `layer` provides: cfg (top_k, router, quant, num_experts, num_shared),
    router_w, router_bias, expert(e) -> (gate, up, down) and shared().
    `tokens` optionally restricts the expert/combine part to a subset of token
    rows (routing is still returned for those rows only)."""
    cfg = layer.cfg
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if tokens is not None:
        x_bits = x_bits[np.asarray(tokens)]
    T = x_bits.shape[0]
    logits = router_logits_fp32(x_bits, layer.router_w, layer.router_bias)
    idx = select_topk(logits, cfg.top_k)
    w = routing_weights(logits, idx, cfg.router)
    counts, offsets, perm, pos = permute(idx, cfg.num_experts)
    x = bf16_to_f64(x_bits)
    o = np.zeros((T * cfg.top_k, cfg.hidden), dtype=np.float64)
    for e in np.nonzero(counts)[0]:
        rows = slice(offsets[e], offsets[e + 1])
        g, u, d = layer.expert(int(e))
        o[rows] = expert_ffn(x[perm[rows]], dequant_qmat(cfg.quant, g),
                             dequant_qmat(cfg.quant, u), dequant_qmat(cfg.quant, d))
    y = np.zeros((T, cfg.hidden), dtype=np.float64)
    for j in range(cfg.top_k):
        y += w[:, j:j + 1] * o[pos[:, j]]
    shared = None
    shared_w = None
    if cfg.num_shared:
        g, u, d = layer.shared()
        shared = expert_ffn(x, dequant_qmat(cfg.quant, g), dequant_qmat(cfg.quant, u),
                            dequant_qmat(cfg.quant, d))
        gate_w = getattr(layer, "shared_gate_w", None)
        if gate_w is None:
            y += shared
        else:
            shared_w = shared_gate_weight(x_bits, gate_w)
            y += shared_w[:, None] * shared
    out = dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, pos=pos, y=y)
    if want_rows:
        out["o"] = o
        out["shared"] = shared
        out["shared_w"] = shared_w
    return out


def shared_gate_weight(x_bits, gate_w_bits) -> np.ndarray:
    """Weight of the shared expert per token, fp64 [T]: sigmoid of the fp32
    gate logit x . w_s, formed in the R2 order (R7)."""
    l = router_logits_fp32(x_bits, np.asarray(gate_w_bits, dtype=np.uint16)[None, :])[:, 0]
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
