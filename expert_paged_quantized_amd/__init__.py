"""Routed 4-bit MoE FFN layer under an expert budget, for AMD MI355X (gfx950).

Python binding of libstrata_moe.so: argument marshalling only.  Every step of
a forward (router, top-k, permute, expert GEMMs, combine, paging) runs in the
HIP library; PyTorch only provides device memory and the stream.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _capi
from ._capi import StrataError, check, lib

__all__ = ["MoELayer", "StrataError", "measure_h2d", "measure_hbm_read", "replay_residency", "lib"]

_QUANT = {"int4_g64": _capi.Q_INT4_G64, "mxfp4_g32": _capi.Q_MXFP4_G32,
          "int4_g128": _capi.Q_INT4_G128, "nvfp4_g16": _capi.Q_NVFP4_G16}
_ROUTER = {"softmax": _capi.R_SOFTMAX, "sigmoid": _capi.R_SIGMOID}
_POLICY = {"lru": _capi.P_LRU, "lfu": _capi.P_LFU, "warm": _capi.P_WARM}
_PAGER = {"auto": _capi.PAGER_AUTO, "kernel": _capi.PAGER_KERNEL, "dma": _capi.PAGER_DMA}


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _qmat(m, keep):
    if m is None:
        return _capi.QMat(None, None, None, None)
    gs = getattr(m, "global_scale", None)
    arrs = [np.ascontiguousarray(m.codes), np.ascontiguousarray(m.scales),
            None if m.biases is None else np.ascontiguousarray(m.biases),
            None if gs is None else np.ascontiguousarray(np.atleast_1d(gs), dtype=np.float32)]
    keep.extend(a for a in arrs if a is not None)
    return _capi.QMat(*[None if a is None else a.ctypes.data for a in arrs])


class MoELayer:
    """One MoE FFN layer held by the HIP library.

    Weights are host numpy arrays in the C ABI layout (objects with .codes,
    .scales, .biases per matrix, stacked over experts); they are copied into the
    library's pinned store at construction and may be dropped afterwards."""

    def __init__(self, *, hidden, ffn, num_experts, top_k, num_shared, quant, router, budget,
                 max_tokens, router_w, router_bias, gate, up, down, sh_gate=None, sh_up=None,
                 sh_down=None, policy="lru", decay_shift=0, prefetch=0, profile=None, device=-1,
                 pager="auto", shared_gate_w=None, hybrid=False, host_threads=0, hybrid_rows=0):
        self.hidden, self.ffn, self.num_experts, self.top_k = hidden, ffn, num_experts, top_k
        self.num_shared, self.max_tokens = num_shared, max_tokens
        keep = []
        rw = np.ascontiguousarray(router_w, dtype=np.uint16)
        rb = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
        keep += [rw] + ([rb] if rb is not None else [])
        d = _capi.Desc()
        d.hidden, d.ffn, d.num_experts, d.top_k, d.num_shared = hidden, ffn, num_experts, top_k, num_shared
        d.quant = _QUANT[quant] if isinstance(quant, str) else quant
        d.router = _ROUTER[router] if isinstance(router, str) else router
        d.policy = _POLICY[policy] if isinstance(policy, str) else policy
        d.expert_budget, d.max_tokens, d.device = budget, max_tokens, device
        d.decay_shift, d.prefetch = decay_shift, prefetch
        d.pager = _PAGER[pager] if isinstance(pager, str) else pager
        d.hybrid, d.host_threads, d.hybrid_rows = int(bool(hybrid)), host_threads, hybrid_rows
        if profile is not None:
            prof = _profile_array(profile, num_experts)
            keep.append(prof)
            d.expert_profile = prof.ctypes.data
        d.router_w, d.router_bias = rw.ctypes.data, (None if rb is None else rb.ctypes.data)
        d.gate, d.up, d.down = _qmat(gate, keep), _qmat(up, keep), _qmat(down, keep)
        d.sh_gate, d.sh_up, d.sh_down = _qmat(sh_gate, keep), _qmat(sh_up, keep), _qmat(sh_down, keep)
        if shared_gate_w is not None:
            gw = np.ascontiguousarray(shared_gate_w, dtype=np.uint16)
            keep.append(gw)
            d.shared_gate_w = gw.ctypes.data
        h = ctypes.c_void_p()
        check(lib().strata_moe_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h

    @classmethod
    def from_weights(cls, lw, budget=None, policy="lru", max_tokens=None, device=-1, decay_shift=0,
                     prefetch=0, profile=None, pager="auto", hybrid=False, host_threads=0, hybrid_rows=0):
        """Builds a layer from a weights object with .cfg and the packed arrays."""
        c = lw.cfg
        return cls(hidden=c.hidden, ffn=c.ffn, num_experts=c.num_experts, top_k=c.top_k,
                   num_shared=c.num_shared, quant=c.quant, router=c.router,
                   budget=c.budget if budget is None else budget,
                   max_tokens=max(c.prefill_T, max(c.decode_T)) if max_tokens is None else max_tokens,
                   router_w=lw.router_w, router_bias=lw.router_bias, gate=lw.gate, up=lw.up,
                   down=lw.down, sh_gate=lw.sh_gate, sh_up=lw.sh_up, sh_down=lw.sh_down,
                   policy=policy, decay_shift=decay_shift, prefetch=prefetch, profile=profile,
                   device=device, pager=pager, shared_gate_w=getattr(lw, "shared_gate_w", None),
                   hybrid=hybrid, host_threads=host_threads, hybrid_rows=hybrid_rows)

    # ------------------------------------------------------------------
    def forward(self, x, y=None, stream=None, dbg=False):
        """x: torch bf16 [T, H] on the layer's GPU.  Returns y (bf16 [T, H]) or,
        with dbg=True, (y, dict of routing tensors)."""
        return self._forward(lib().strata_moe_forward, x, y, stream, dbg)

    def forward_noalloc(self, x, y=None, stream=None, dbg=False):
        """The same forward on the library's static device scratch
        (strata_moe_forward_noalloc): no device allocation by the library.
        Pass y (and the dbg tensors are allocated here by torch) if the
        caller itself must not allocate."""
        return self._forward(lib().strata_moe_forward_noalloc, x, y, stream, dbg)

    def _forward(self, fn, x, y, stream, dbg):
        import torch
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.hidden:
            raise ValueError("x must be bf16 [T, hidden]")
        x = x.contiguous()
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        d = None
        out = None
        if dbg:
            dev = x.device
            E, k = self.num_experts, self.top_k
            out = dict(logits=torch.empty((T, E), dtype=torch.float32, device=dev),
                       idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                       w=torch.empty((T, k), dtype=torch.float32, device=dev),
                       counts=torch.empty((E,), dtype=torch.int32, device=dev),
                       offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                       perm=torch.empty((T * k,), dtype=torch.int32, device=dev))
            d = _capi.RouteDbg(out["logits"].data_ptr(), out["idx"].data_ptr(), out["w"].data_ptr(),
                               out["counts"].data_ptr(), out["offsets"].data_ptr(),
                               out["perm"].data_ptr())
        check(fn(self._h, ctypes.c_void_p(x.data_ptr()), T, ctypes.c_void_p(y.data_ptr()),
                 ctypes.c_void_p(stream.cuda_stream), ctypes.byref(d) if d is not None else None))
        return (y, out) if dbg else y

    __call__ = forward

    def stats(self) -> dict:
        s = _capi.CacheStats()
        check(lib().strata_expert_cache_stats(self._h, ctypes.byref(s)))
        return s.as_dict()

    def save_profile(self) -> np.ndarray:
        """The learned per-expert frequency scores, uint64 [E] (one use = 65536)."""
        out = np.zeros(self.num_experts, dtype=np.uint64)
        check(lib().strata_expert_profile_save(self._h, out.ctypes.data, self.num_experts))
        return out

    def load_profile(self, profile):
        """Sets the scores and pages the profile's hottest experts in, ahead of need."""
        prof = _profile_array(profile, self.num_experts)
        check(lib().strata_expert_profile_load(self._h, prof.ctypes.data, self.num_experts))

    def memory(self) -> dict:
        m = _capi.MemoryInfo()
        check(lib().strata_moe_memory(self._h, ctypes.byref(m)))
        return m.as_dict()

    def set_timing(self, enable: bool):
        check(lib().strata_moe_set_timing(self._h, 1 if enable else 0))

    def timing(self) -> dict:
        t = _capi.Timing()
        check(lib().strata_moe_timing(self._h, ctypes.byref(t)))
        return {name: (t.ms[i], t.launches[i]) for i, name in enumerate(_capi.KERNEL_CLASSES)}

    def close(self):
        if getattr(self, "_h", None):
            lib().strata_moe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def measure_h2d(device=-1, nbytes=256 << 20, iters=3) -> float:
    """Pinned host -> device copy rate in GB/s (the paging link)."""
    g = ctypes.c_double()
    check(lib().strata_measure_h2d(device, nbytes, iters, ctypes.byref(g)))
    return g.value


def measure_hbm_read(device=-1, nbytes=1 << 30, iters=5) -> float:
    """HBM read ceiling in GB/s: best of `iters` streaming-read passes over `nbytes`."""
    g = ctypes.c_double()
    check(lib().strata_measure_hbm_read(device, nbytes, iters, ctypes.byref(g)))
    return g.value


def _profile_array(profile, num_experts):
    prof = np.ascontiguousarray(profile, dtype=np.uint64)
    if prof.shape != (num_experts,):
        raise ValueError(f"profile must have shape ({num_experts},)")
    return prof


def replay_residency(num_experts, budget, trace, policy="lru", expert_bytes=0, want_slots=False,
                     decay_shift=0, prefetch=0, profile=None, hybrid=None, rows=None, host_rows=0):
    """Dry-run of the residency policy on a trace of needed-expert lists (host
    only); `hybrid` optionally flags the hybrid decode forwards of the trace;
    host_rows > 0 replays the other forwards as hybrid prefills with that row
    limit, `rows` then giving each needed expert's token count (a list per
    forward, parallel to the trace).  Returns the counters, plus "slots"
    (want_slots) and the final "scores"."""
    lens = np.array([len(n) for n in trace], dtype=np.int32)
    nrows = None if rows is None else np.array([r for rr in rows for r in rr], dtype=np.int32)
    hyb = None if hybrid is None else np.ascontiguousarray(hybrid, dtype=np.int32)
    flat = np.array([e for n in trace for e in n], dtype=np.int32)
    slots = np.full(max(1, flat.size), -1, dtype=np.int32) if want_slots else None
    scores = np.zeros(max(1, num_experts), dtype=np.uint64)
    prof = None if profile is None else _profile_array(profile, num_experts)
    s = _capi.CacheStats()
    check(lib().strata_residency_replay(num_experts, budget, _POLICY.get(policy, policy), decay_shift,
                                        prefetch, None if prof is None else prof.ctypes.data,
                                        expert_bytes, len(trace), _ptr(lens),
                                        _ptr(flat if flat.size else np.zeros(1, np.int32)),
                                        _ptr(hyb), _ptr(nrows), host_rows, _ptr(slots), scores.ctypes.data,
                                        ctypes.byref(s)))
    res = s.as_dict()
    if want_slots:
        res["slots"] = slots[:flat.size]
    res["scores"] = scores[:num_experts]
    return res
