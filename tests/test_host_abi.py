"""Host-side checks of the C ABI library: symbols, descriptor validation and
admission errors (all decided before any HIP call), and the residency manager
through the dry-run planner against the residency model."""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_paged_quantized_amd as epq
from expert_paged_quantized_amd import _capi
from oracle.residency import LFU, LRU, WARM, ResidencyModel
from synth import CONFIGS, make_layer

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "strata_moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(strata_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "strata_moe_create" in names and "strata_moe_forward" in names
    assert "strata_expert_cache_stats" in names
    L = epq.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_capi.EXPORTS)


_QCODE = {"int4_g64": 1, "mxfp4_g32": 2, "int4_g128": 3, "nvfp4_g16": 4}


def _desc_from(lw, **over):
    c = lw.cfg
    keep = []
    d = _capi.Desc()
    d.hidden, d.ffn, d.num_experts, d.top_k, d.num_shared = c.hidden, c.ffn, c.num_experts, c.top_k, c.num_shared
    d.quant = _QCODE[c.quant]
    d.router = 1 if c.router == "softmax" else 2
    d.policy, d.expert_budget, d.max_tokens, d.device = 1, c.budget, 16, -1
    keep.append(lw.router_w)
    d.router_w = lw.router_w.ctypes.data
    d.router_bias = None
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        m = getattr(lw, name)
        if m is None:
            setattr(d, name, _capi.QMat(None, None, None))
        else:
            gs = None
            if m.global_scale is not None:
                gs = np.ascontiguousarray(np.atleast_1d(m.global_scale), dtype=np.float32)
                keep.append(gs)
            setattr(d, name, _capi.QMat(m.codes.ctypes.data, m.scales.ctypes.data,
                                        None if m.biases is None else m.biases.ctypes.data,
                                        None if gs is None else gs.ctypes.data))
    for k, v in over.items():
        setattr(d, k, v)
    return d, keep


def _create_status(d):
    h = ctypes.c_void_p()
    st = epq.lib().strata_moe_create(ctypes.byref(d), ctypes.byref(h))
    if st == 0:
        epq.lib().strata_moe_destroy(h)
    return st, epq.lib().strata_last_error().decode()


@pytest.fixture(scope="module")
def tiny_int4():
    return make_layer(CONFIGS["tiny"].scaled(ffn=128, num_experts=4, top_k=2, budget_frac=0.5), seed=1)


@pytest.fixture(scope="module")
def tiny_fp4():
    return make_layer(CONFIGS["tiny"].scaled(ffn=128, num_experts=4, top_k=2, quant="mxfp4_g32",
                                             num_shared=1, budget_frac=0.5), seed=2)


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 0, _capi.E_INVALID),
    ("hidden", 768, _capi.E_UNSUPPORTED),      # not a multiple of 512
    ("ffn", 96, _capi.E_UNSUPPORTED),          # not a multiple of 64
    ("top_k", 5, _capi.E_INVALID),             # k > E
    ("top_k", 0, _capi.E_INVALID),
    ("expert_budget", 0, _capi.E_INVALID),
    ("expert_budget", 5, _capi.E_INVALID),     # budget > E
    ("num_shared", 2, _capi.E_UNSUPPORTED),
    ("quant", 7, _capi.E_INVALID),
    ("router", 0, _capi.E_INVALID),
    ("policy", 9, _capi.E_INVALID),
    ("policy", 3, _capi.E_INVALID),            # WARM without a decay_shift
    ("decay_shift", 2, _capi.E_INVALID),       # decay on LRU
    ("prefetch", 3, _capi.E_INVALID),          # prefetch > budget (2)
    ("prefetch", -1, _capi.E_INVALID),
    ("pager", 3, _capi.E_INVALID),
    ("pager", -1, _capi.E_INVALID),
    ("max_tokens", 0, _capi.E_INVALID),
    ("num_experts", 2000, _capi.E_UNSUPPORTED),
    ("router_w", None, _capi.E_INVALID),
    ("hybrid", 2, _capi.E_INVALID),
    ("host_threads", -1, _capi.E_INVALID),
    ("hybrid_rows", 2, _capi.E_INVALID),       # a row limit without hybrid
    ("hybrid_rows", -1, _capi.E_INVALID),
])
def test_invalid_descriptors(tiny_int4, field, value, status):
    d, keep = _desc_from(tiny_int4, **{field: value})
    st, msg = _create_status(d)
    assert st == status, msg
    assert msg


def test_null_arguments():
    L = epq.lib()
    h = ctypes.c_void_p()
    assert L.strata_moe_create(None, ctypes.byref(h)) == _capi.E_INVALID
    assert L.strata_moe_forward(None, None, 1, None, None, None) == _capi.E_INVALID
    s = _capi.CacheStats()
    assert L.strata_expert_cache_stats(None, ctypes.byref(s)) == _capi.E_INVALID
    L.strata_moe_destroy(None)  # ignored


def test_int4_requires_biases_and_mxfp4_refuses_them(tiny_int4, tiny_fp4):
    d, keep = _desc_from(tiny_int4)
    d.gate = _capi.QMat(d.gate.codes, d.gate.scales, None)
    assert _create_status(d)[0] == _capi.E_INVALID
    d, keep = _desc_from(tiny_fp4)
    d.up = _capi.QMat(d.up.codes, d.up.scales, d.up.codes)
    assert _create_status(d)[0] == _capi.E_INVALID


def test_shared_gate_needs_a_shared_expert(tiny_int4):
    gw = np.zeros(tiny_int4.cfg.hidden, np.uint16)
    d, keep = _desc_from(tiny_int4, shared_gate_w=gw.ctypes.data)
    st, msg = _create_status(d)
    assert st == _capi.E_INVALID and "shared_gate_w" in msg


def test_shared_weights_must_match_num_shared(tiny_fp4):
    d, keep = _desc_from(tiny_fp4, num_shared=0)
    assert _create_status(d)[0] == _capi.E_INVALID


@pytest.mark.parametrize("bad", [0, 255])
@pytest.mark.parametrize("which", ["gate", "down", "sh_up"])
def test_e8m0_admission_refuses_0_and_255(tiny_fp4, bad, which):
    lw = tiny_fp4
    m = getattr(lw, which)
    saved = m.scales.copy()
    try:
        m.scales.reshape(-1)[m.scales.size // 2] = bad
        d, keep = _desc_from(lw)
        st, msg = _create_status(d)
        assert st == _capi.E_BAD_SCALE, msg
        assert "E8M0" in msg
    finally:
        m.scales[...] = saved


def _bf16_times_pow2(bits, k):
    """bf16 bit patterns times 2^k (exact for normal values that stay normal)."""
    b = bits.astype(np.int32)
    e = (b >> 7) & 0xFF
    nz = e > 0
    assert np.all(e[nz] + k > 0) and np.all(e[nz] + k < 255)
    b[nz] += k << 7
    return b.astype(np.uint16)


@pytest.mark.parametrize("k", [-30, 20])
def test_int4_scales_outside_the_fp16_range_are_admitted(tiny_int4, k):
    """bf16 scales and biases far below or above fp16's range are stored with
    one power-of-two rescaling per matrix, not refused."""
    lw = tiny_int4
    saved = [(m, m.scales.copy(), m.biases.copy()) for m in (lw.gate, lw.up, lw.down)]
    try:
        for m, s, b in saved:
            m.scales[...] = _bf16_times_pow2(s, k)
            m.biases[...] = _bf16_times_pow2(b, k)
        d, keep = _desc_from(lw)
        st, msg = _create_status(d)
        # admission passes; without a GPU the first HIP call then fails
        assert st in (_capi.OK, _capi.E_HIP), msg
    finally:
        for m, s, b in saved:
            m.scales[...] = s
            m.biases[...] = b


def test_int4_scales_spanning_more_than_fp16_are_refused(tiny_int4):
    lw = tiny_int4
    saved = lw.up.scales.copy()
    try:
        # bf16 ~1.2e-38 beside scales near 1e-2 in the same matrix: no single
        # power of two brings both into fp16 exactly
        lw.up.scales.reshape(-1)[3] = 0x0081
        d, keep = _desc_from(lw)
        st, msg = _create_status(d)
        assert st == _capi.E_UNSUPPORTED and "span" in msg and "up" in msg, msg
    finally:
        lw.up.scales[...] = saved


@pytest.mark.parametrize("bad", [0x7FC0, 0x7F80, 0xFF80])
def test_int4_nan_or_infinite_scale_fails_admission(tiny_int4, bad):
    lw = tiny_int4
    saved = lw.down.biases.copy()
    try:
        lw.down.biases.reshape(-1)[5] = bad
        d, keep = _desc_from(lw)
        st, msg = _create_status(d)
        assert st == _capi.E_BAD_SCALE and "finite" in msg, msg
    finally:
        lw.down.biases[...] = saved


# ----------------------------------------------------------------------------
# residency manager (C++) through the dry-run planner vs. the residency model
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("policy", [LRU, LFU])
def test_residency_replay_matches_model(policy):
    rng = np.random.default_rng(21)
    for trial in range(40):
        E = int(rng.integers(2, 64))
        B = int(rng.integers(1, E + 1))
        trace = []
        for _ in range(int(rng.integers(1, 40))):
            n = int(rng.integers(1, E + 1))
            # Zipf-ish popularity so hits and waves both occur
            p = 1.0 / np.arange(1, E + 1) ** 1.1
            p = p[rng.permutation(E)]
            trace.append(rng.choice(E, size=n, replace=False, p=p / p.sum()).tolist())
        m = ResidencyModel(E, B, policy, expert_bytes=1000)
        want_slots = []
        for n in trace:
            for wave in m.forward(n):
                want_slots += [s for (_, s, _) in wave]
        got = epq.replay_residency(E, B, trace, policy=policy, expert_bytes=1000, want_slots=True)
        st = m.stats()
        for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
                  "resident_bytes"):
            assert got[k] == st[k], (trial, k)
        assert got["slots"].tolist() == want_slots


def test_residency_replay_rejects_bad_arguments():
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 0, [[0]])
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[7]])
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], policy=WARM)               # no decay
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], policy=LFU, decay_shift=2)
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], policy=WARM, decay_shift=25)
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], prefetch=3)
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], profile=[0, 0, 0, (1 << 62) + 1])


@pytest.mark.parametrize("policy,d", [(LRU, 0), (LFU, 0), (WARM, 1), (WARM, 4)])
def test_residency_replay_with_decay_prefetch_and_profile_matches_model(policy, d):
    """The C++ manager (decayed scores, prefetch pairing, warm start from a
    profile) against the residency model: every counter, every slot and the
    final scores agree."""
    rng = np.random.default_rng(77 + d)
    for trial in range(40):
        E = int(rng.integers(2, 48))
        B = int(rng.integers(1, E + 1))
        P = int(rng.integers(0, B + 1))
        prof = None
        if trial % 3 == 0:
            prof = rng.integers(0, 8 * 65536, size=E).astype(np.uint64)
            prof[rng.integers(0, E)] = prof[0]           # a tie in the warm set
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[rng.permutation(E)]
        trace = []
        for f in range(int(rng.integers(1, 50))):
            if f == 25:                                   # the workload shifts
                p = p[rng.permutation(E)]
            n = int(rng.integers(1, E + 1))
            trace.append(rng.choice(E, size=n, replace=False, p=p / p.sum()).tolist())
        m = ResidencyModel(E, B, policy, expert_bytes=1000, decay_shift=d, prefetch=P,
                           profile=None if prof is None else prof.tolist())
        want_slots = []
        for n in trace:
            for wave in m.forward(n):
                want_slots += [s for (_, s, _) in wave]
        got = epq.replay_residency(E, B, trace, policy=policy, expert_bytes=1000, want_slots=True,
                                   decay_shift=d, prefetch=P, profile=prof)
        st = m.stats()
        for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
                  "resident_bytes", "prefetched", "prefetch_hits"):
            assert got[k] == st[k], (trial, k, got[k], st[k])
        assert got["slots"].tolist() == want_slots, trial
        assert got["scores"].tolist() == m.profile(), trial


@pytest.mark.parametrize("policy,d,P", [(LRU, 0, 0), (LFU, 0, 2), (WARM, 3, 1)])
def test_residency_replay_with_hybrid_forwards_matches_model(policy, d, P):
    """Traces mixing hybrid decode forwards (hits from slots, the rest on the
    host, nothing paged) with plain forwards: the C++ manager and the model
    agree on every counter, slot (-1 for a host expert) and score."""
    rng = np.random.default_rng(5 + d + P)
    for trial in range(30):
        E = int(rng.integers(2, 40))
        B = int(rng.integers(1, E + 1))
        P_ = min(P, B)
        trace, flags = [], []
        for f in range(int(rng.integers(1, 40))):
            n = int(rng.integers(1, E + 1))
            trace.append(rng.choice(E, size=n, replace=False).tolist())
            flags.append(int(rng.random() < 0.6))
        m = ResidencyModel(E, B, policy, expert_bytes=100, decay_shift=d, prefetch=P_)
        want = []
        for n, h in zip(trace, flags):
            if h:
                hits, host = m.forward_hybrid(n)
                slot = dict(hits)
                want += [slot.get(e, -1) for e in sorted(set(n))]
            else:
                for wave in m.forward(n):
                    want += [s for (_, s, _) in wave]
        got = epq.replay_residency(E, B, trace, policy=policy, expert_bytes=100, want_slots=True,
                                   decay_shift=d, prefetch=P_, hybrid=flags)
        st = m.stats()
        for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
                  "prefetched", "prefetch_hits", "host_experts"):
            assert got[k] == st[k], (trial, k, got[k], st[k])
        assert got["slots"].tolist() == want, trial
        assert got["scores"].tolist() == m.profile(), trial


def test_hybrid_rows_above_eight_is_refused(tiny_int4):
    d, keep = _desc_from(tiny_int4, hybrid=1, hybrid_rows=9)
    st, msg = _create_status(d)
    assert st == _capi.E_INVALID and "hybrid_rows" in msg


@pytest.mark.parametrize("policy,d,P,R", [(LRU, 0, 0, 2), (LFU, 0, 2, 4), (WARM, 3, 1, 8)])
def test_residency_replay_with_hybrid_prefills_matches_model(policy, d, P, R):
    """Traces of hybrid prefills (a needed expert that is not resident and has
    at most R rows goes to the host) mixed with hybrid decode forwards: the C++
    manager and the model agree on every counter, slot (-1 for a host expert,
    listed after the forward's run order) and score."""
    rng = np.random.default_rng(11 + d + P + R)
    for trial in range(30):
        E = int(rng.integers(2, 40))
        B = int(rng.integers(1, E + 1))
        P_ = min(P, B)
        trace, rows, flags = [], [], []
        for f in range(int(rng.integers(1, 40))):
            n = int(rng.integers(1, E + 1))
            need = rng.choice(E, size=n, replace=False).tolist()
            trace.append(need)
            rows.append([int(rng.integers(1, 2 * R + 2)) for _ in need])
            flags.append(int(rng.random() < 0.25))
        m = ResidencyModel(E, B, policy, expert_bytes=100, decay_shift=d, prefetch=P_)
        want = []
        for n, r, h in zip(trace, rows, flags):
            if h:
                hits, host = m.forward_hybrid(n)
                slot = dict(hits)
                want += [slot.get(e, -1) for e in sorted(set(n))]
            else:
                plan, host = m.forward_split(n, dict(zip(n, r)), host_rows=R)
                for wave in plan:
                    want += [s for (_, s, _) in wave]
                want += [-1] * len(host)
        got = epq.replay_residency(E, B, trace, policy=policy, expert_bytes=100, want_slots=True,
                                   decay_shift=d, prefetch=P_, hybrid=flags, rows=rows, host_rows=R)
        st = m.stats()
        for k in ("forwards", "hits", "misses", "evictions", "bytes_h2d", "waves", "resident",
                  "prefetched", "prefetch_hits", "host_experts"):
            assert got[k] == st[k], (trial, k, got[k], st[k])
        assert got["slots"].tolist() == want, trial
        assert got["scores"].tolist() == m.profile(), trial


def test_residency_replay_rejects_bad_row_limits():
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], host_rows=2)                  # no rows
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], rows=[[1]], host_rows=9)
    with pytest.raises(epq.StrataError):
        epq.replay_residency(4, 2, [[0]], rows=[[0]], host_rows=2)      # a count below 1


def test_ctypes_mirrors_match_the_c_struct_sizes(tmp_path):
    """Compiles the header with gcc and compares sizeof/offsetof of every struct
    the binding passes by pointer with the ctypes declarations."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    structs = {"strata_moe_desc": _capi.Desc, "strata_qmat": _capi.QMat,
               "strata_route_dbg": _capi.RouteDbg, "strata_cache_stats": _capi.CacheStats,
               "strata_memory_info": _capi.MemoryInfo, "strata_timing": _capi.Timing}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "sizes.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.split("\n") if l)
    for cname, py in structs.items():
        assert int(out[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(out[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


# ----------------------------------------------------------------------------
# more 4-bit formats: int4 group-128 and NVFP4 admission
# ----------------------------------------------------------------------------
@pytest.fixture(scope="module")
def tiny_g128():
    return make_layer(CONFIGS["tiny"].scaled(ffn=128, num_experts=4, top_k=2, quant="int4_g128",
                                             budget_frac=0.5), seed=3)


@pytest.fixture(scope="module")
def tiny_nvfp4():
    return make_layer(CONFIGS["tiny"].scaled(ffn=128, num_experts=4, top_k=2, quant="nvfp4_g16",
                                             num_shared=1, budget_frac=0.5), seed=4)


def test_int4_group128_ffn_must_be_a_multiple_of_128(tiny_g128):
    d, keep = _desc_from(tiny_g128, ffn=192)
    assert _create_status(d)[0] == _capi.E_UNSUPPORTED


def test_int4_group128_needs_biases(tiny_g128):
    d, keep = _desc_from(tiny_g128)
    d.gate = _capi.QMat(d.gate.codes, d.gate.scales, None, None)
    assert _create_status(d)[0] == _capi.E_INVALID


def test_nvfp4_needs_matrix_scales_and_refuses_biases(tiny_nvfp4):
    d, keep = _desc_from(tiny_nvfp4)
    d.up = _capi.QMat(d.up.codes, d.up.scales, None, None)
    assert _create_status(d)[0] == _capi.E_INVALID
    d, keep = _desc_from(tiny_nvfp4)
    d.down = _capi.QMat(d.down.codes, d.down.scales, d.down.codes, d.down.global_scale)
    assert _create_status(d)[0] == _capi.E_INVALID


def test_matrix_scale_is_refused_for_other_formats(tiny_int4):
    d, keep = _desc_from(tiny_int4)
    g = np.ones(4, np.float32)
    d.gate = _capi.QMat(d.gate.codes, d.gate.scales, d.gate.biases, g.ctypes.data)
    assert _create_status(d)[0] == _capi.E_INVALID


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
@pytest.mark.parametrize("which", ["gate", "down", "sh_up"])
def test_e4m3_nan_scale_is_refused(tiny_nvfp4, bad, which):
    m = getattr(tiny_nvfp4, which)
    saved = m.scales.copy()
    try:
        m.scales.reshape(-1)[m.scales.size // 3] = bad
        d, keep = _desc_from(tiny_nvfp4)
        st, msg = _create_status(d)
        assert st == _capi.E_BAD_SCALE and "E4M3" in msg
    finally:
        m.scales[...] = saved


@pytest.mark.parametrize("value", [0.0, -1.0, float("inf"), float("nan")])
def test_nvfp4_matrix_scale_must_be_finite_and_positive(tiny_nvfp4, value):
    m = tiny_nvfp4.up
    saved = m.global_scale.copy()
    try:
        m.global_scale[1] = value
        d, keep = _desc_from(tiny_nvfp4)
        assert _create_status(d)[0] == _capi.E_BAD_SCALE
    finally:
        m.global_scale[...] = saved
