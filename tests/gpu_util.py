"""Helpers shared by the GPU tests (torch only moves bytes here)."""
import numpy as np

import oracle
from oracle import moe as om

Y_MAX_ABS = 2e-2     # max |y_gpu - y_oracle|
Y_REL_L2 = 5e-3      # ||y_gpu - y_oracle||_2 / ||y_oracle||_2
W_ABS = 1e-5       # routing weights (fp32 on the GPU vs fp64 oracle from the same logits)


def to_dev(x_bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(device)


def y_to_f64(y):
    import torch
    return om.bf16_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))


def y_bits(y):
    import torch
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_y_close(y_gpu64, y_ref, what=""):
    d = np.abs(y_gpu64 - y_ref)
    rel = np.linalg.norm(y_gpu64 - y_ref) / max(np.linalg.norm(y_ref), 1e-30)
    assert np.abs(y_ref).max() <= 4.0, f"{what}: generator left the bf16 error budget (max|y|)"
    assert d.max() <= Y_MAX_ABS and rel <= Y_REL_L2, f"{what}: max|dy|={d.max():.3g} relL2={rel:.3g}"
    return float(d.max()), float(rel)


def assert_routing_equal(dbg, ref, T, E, k, what=""):
    """Bitwise routing: logits, idx, counts, offsets, perm; weights within W_ABS."""
    import torch
    torch.cuda.synchronize()
    lg = dbg["logits"].cpu().numpy()
    assert np.array_equal(lg.view(np.uint32), ref["logits"].astype(np.float32).view(np.uint32)), \
        f"{what}: logits differ at {np.argwhere(lg.view(np.uint32) != ref['logits'].view(np.uint32))[:5]}"
    assert np.array_equal(dbg["idx"].cpu().numpy(), ref["idx"]), f"{what}: idx"
    assert np.array_equal(dbg["counts"].cpu().numpy(), ref["counts"]), f"{what}: counts"
    assert np.array_equal(dbg["offsets"].cpu().numpy(), ref["offsets"]), f"{what}: offsets"
    assert np.array_equal(dbg["perm"].cpu().numpy(), ref["perm"]), f"{what}: perm"
    dw = np.abs(dbg["w"].cpu().numpy().astype(np.float64) - ref["w"]).max()
    assert dw <= W_ABS, f"{what}: routing weights off by {dw}"


def check_sampled(lw, layer, x, sample, what):
    """One forward at any size: sampled logits bitwise, all routing against
    the oracle's selection / grouping of the GPU logits, sampled y against
    the oracle forward of those tokens.  Returns y."""
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
