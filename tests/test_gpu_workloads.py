"""Full-size workloads on the GPU, every output element checked against the fp64 oracle.

Each workload runs at its full shape in the launch configuration the
benchmark uses; the oracle then recomputes every (sequence, head) unit from
exact host copies of the same inputs and the whole output tensors are
compared. Tolerance as for the small cases: max|gpu - oracle| / max|oracle|
<= 2e-2 (bf16), 1e-4 (fp32), for o and for the final state separately (and
for every gradient of the backward passes). The packed batch is streamed one
sequence at a time so that the host copies stay bounded.
"""

import numpy as np
import pytest
import torch

import oracle
import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import WORKLOADS, make_channel_gates, make_gates, workload_inputs
from helpers import TOL, rel_err, rms_rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def f64(t):
    return None if t is None else t.detach().to("cpu").to(torch.float64).numpy()


class MaxErr:
    """Running max|x - ref| and max|ref| over pieces of one tensor."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, x, ref):
        self.num = max(self.num, float(np.abs(np.asarray(x) - ref).max(initial=0.0)))
        self.den = max(self.den, float(np.abs(ref).max(initial=0.0)))

    @property
    def err(self):
        return self.num / self.den if self.den > 0 else self.num


def report(name, pairs, tol):
    """Print and check whole-tensor errors; pairs = [(label, gpu, ref), ...]."""
    parts = []
    for label, x, ref in pairs:
        e, r = rel_err(x, ref), rms_rel(x, ref)
        parts.append(f"{label} max {e:.3e} rms {r:.3e}")
        assert e <= tol, f"{name}: {label} error {e} > {tol}"
    print(f"  {name}: " + ", ".join(parts) + f" (tol {tol})", flush=True)


def run_dense(w, cp_groups=1, seed=2):
    print(f"[case] {w.name} full size, cp_groups={cp_groups}", flush=True)
    inputs = workload_inputs(w, seed=seed, device=DEV)
    q, k, v, beta, S0 = inputs
    o, Sf = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=cp_groups)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    return inputs, o, Sf


def oracle_dense(inputs):
    q, k, v, beta, S0 = inputs
    return oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))


def test_tiny_f32_full():
    w = WORKLOADS["tiny_f32"]
    inputs, o, Sf = run_dense(w)
    ro, rs = oracle_dense(inputs)
    report(w.name, [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.float32])


def test_layer_b8_h16_t4096_every_unit():
    w = WORKLOADS["layer_b8_h16_t4096"]
    inputs, o, Sf = run_dense(w)
    ro, rs = oracle_dense(inputs)
    report(f"{w.name} all {w.B * w.H} units", [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.bfloat16])


@pytest.mark.parametrize("cp_groups", [1, 0])
def test_chunks128_b4_h16_t8192_every_unit(cp_groups):
    w = WORKLOADS["chunks128_b4_h16_t8192"]
    inputs, o, Sf = run_dense(w, cp_groups=cp_groups)
    assert inputs[4] is not None  # non-zero initial state
    ro, rs = oracle_dense(inputs)
    report(f"{w.name} all {w.B * w.H} units, cp_groups={cp_groups}",
           [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.bfloat16])


_LONG = {}


def long_case():
    """Inputs and oracle outputs of the long-context workload, computed once."""
    if not _LONG:
        w = WORKLOADS["long_b1_h16_t131072"]
        inputs = workload_inputs(w, seed=2, device=DEV)
        print(f"[case] {w.name}: oracle over all {w.H} heads", flush=True)
        _LONG["inputs"] = inputs
        _LONG["ref"] = oracle_dense(inputs)
    return _LONG["inputs"], _LONG["ref"]


@pytest.mark.parametrize("cp_groups", [1, 0, 16])
def test_long_b1_h16_t131072_every_head(cp_groups):
    w = WORKLOADS["long_b1_h16_t131072"]
    inputs, (ro, rs) = long_case()
    q, k, v, beta, S0 = inputs
    print(f"[case] {w.name} full size, cp_groups={cp_groups}", flush=True)
    o, Sf = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=cp_groups)
    torch.cuda.synchronize()
    if cp_groups == 0:
        assert dn.deltanet_pick_cp_groups(w.B, w.H, w.T, w.dk, w.dv) > 1
    report(f"{w.name} all {w.H} heads, cp_groups={cp_groups}", [("o", f64(o), ro), ("S_final", f64(Sf), rs)],
           TOL[torch.bfloat16])


def test_varlen_n64_h32_every_sequence_and_head():
    w = WORKLOADS["varlen_n64_h32"]
    print(f"[case] {w.name} full size", flush=True)
    q, k, v, beta, cu, S0, lengths = workload_inputs(w, seed=2, device=DEV)
    order = dn.longest_first_order(cu)
    o, Sf = dn.deltanet_fwd_varlen(q, k, v, beta, cu, S0, seq_order=order)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    cu_h = cu.cpu().numpy().astype(np.int64)
    eo, es = MaxErr(), MaxErr()
    for n in range(w.N):
        a, b = int(cu_h[n]), int(cu_h[n + 1])
        # one sequence as a batch of one: the oracle runs its H heads in parallel
        sl = lambda x: f64(x[a:b].unsqueeze(0))
        ro, rs = oracle.deltanet_fwd(sl(q), sl(k), sl(v), sl(beta), None)
        eo.add(f64(o[a:b]), ro[0])
        es.add(f64(Sf[n]), rs[0])
    tol = TOL[torch.bfloat16]
    print(f"  {w.name}: all {w.N} sequences x {w.H} heads ({int(cu_h[-1])} tokens), "
          f"err o={eo.err:.3e} S={es.err:.3e} (tol {tol})", flush=True)
    assert eo.err <= tol and es.err <= tol


def test_gated_layer_b8_h16_t4096_every_unit():
    # Gated DeltaNet at the benchmark's full shape and launch configuration
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, gated", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = make_gates((w.B, w.T, w.H), seed=2, device=DEV)
    o, Sf = dn.deltanet_gated_fwd(q, k, v, beta, g, S0)
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g))
    report(f"gated {w.name} all units", [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.bfloat16])


def test_gated_long_context_parallel_every_head():
    w = WORKLOADS["long_b1_h16_t131072"]
    print(f"[case] {w.name} full size, gated, cp auto", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=4, device=DEV)
    g = make_gates((w.B, w.T, w.H), seed=4, device=DEV)
    o, Sf = dn.deltanet_gated_fwd(q, k, v, beta, g, S0, cp_groups=0)
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g))
    report(f"gated {w.name} all heads, cp auto", [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.bfloat16])


def test_bwd_layer_b8_h16_t4096_every_unit():
    # the backward pass at the benchmark's full shape, every unit against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, backward", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=DEV, dtype=torch.float32).to(v.dtype)
    out = dn.deltanet_bwd(q, k, v, beta, dO, S0)
    torch.cuda.synchronize()
    ref = oracle.deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(dO))
    names = ("dq", "dk", "dv", "dbeta", "dS0")
    report(f"bwd {w.name} all units", [(n, f64(x), r) for n, x, r in zip(names, out, ref)], 2e-2)


def test_bwd_long_b1_h16_t131072_context_parallel_every_head():
    # the backward at the long-context shape with the library's group count,
    # every head against the oracle's reverse mode
    w = WORKLOADS["long_b1_h16_t131072"]
    G = dn.deltanet_pick_cp_groups(w.B, w.H, w.T, w.dk, w.dv)
    print(f"[case] {w.name} full size, backward, cp_groups=0 ({G} groups)", flush=True)
    assert G > 1
    q, k, v, beta, S0 = workload_inputs(w, seed=5, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(11)
    dO = torch.randn(v.shape, generator=g, device=DEV, dtype=torch.float32).to(v.dtype)
    dSf = torch.randn((w.B, w.H, w.dv, w.dk), generator=g, device=DEV, dtype=torch.float32) * 0.1
    out = dn.deltanet_bwd(q, k, v, beta, dO, S0, dSf, cp_groups=0)
    torch.cuda.synchronize()
    ref = oracle.deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(dO), f64(S0), f64(dSf))
    names = ("dq", "dk", "dv", "dbeta", "dS0")
    report(f"bwd {w.name} all heads, cp_groups=0", [(n, f64(x), r) for n, x, r in zip(names, out, ref)], 2e-2)


def test_gated_bwd_layer_b8_h16_t4096_every_unit():
    # the Gated DeltaNet backward at the benchmark's full shape, in the launch
    # configuration bench.py times, every unit against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, gated backward", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=3, device=DEV)
    gl = make_gates((w.B, w.T, w.H), seed=7, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=DEV, dtype=torch.float32).to(v.dtype)
    out = dn.deltanet_gated_bwd(q, k, v, beta, gl, dO, S0)
    torch.cuda.synchronize()
    ref = oracle.gated_deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(gl), f64(dO))
    names = ("dq", "dk", "dv", "dbeta", "dg", "dS0")
    report(f"gated bwd {w.name} all units", [(n, f64(x), r) for n, x, r in zip(names, out, ref)], 2e-2)


def test_gdp_bwd_layer_b8_h16_t4096_every_unit():
    # the GDP backward (n_h = 2) at the benchmark's full shape, inputs drawn
    # as bench.py's variant draws them, every unit against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    nh = 2
    print(f"[case] {w.name} full size, gdp backward n_h={nh}", flush=True)
    from chunkwise_delta_rule_amd.synth import make_inputs
    B, H, T = w.B, w.H, w.T
    q, _, _, _, _ = make_inputs(B, H, T, w.dk, w.dv, seed=6, device=DEV)
    _, k, v, beta, _ = make_inputs(B, H, T * nh, w.dk, w.dv, seed=7, device=DEV)
    k, v, beta = k.view(B, T, nh, H, w.dk), v.view(B, T, nh, H, w.dv), beta.view(B, T, nh, H)
    gl = make_gates((B, T, H), seed=6, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(9)
    dO = torch.randn((B, T, H, w.dv), generator=gen, device=DEV, dtype=torch.float32).to(q.dtype)
    out = dn.deltanet_gdp_bwd(q, k, v, beta, gl, dO)
    torch.cuda.synchronize()
    ref = oracle.gdp_bwd(f64(q), f64(k), f64(v), f64(beta), f64(gl), nh, f64(dO))
    names = ("dq", "dk", "dv", "dbeta", "dg", "dS0")
    report(f"gdp bwd {w.name} all units", [(n, f64(x), r) for n, x, r in zip(names, out, ref)], 2e-2)


def test_kda_layer_b8_h16_t4096_every_unit():
    # KDA at the benchmark's full shape, every unit against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, kda", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = make_channel_gates((w.B, w.T, w.H, w.dk), seed=2, device=DEV)
    o, Sf = dn.deltanet_kda_fwd(q, k, v, beta, g, S0)
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g))
    report(f"kda {w.name} all units", [("o", f64(o), ro), ("S_final", f64(Sf), rs)], TOL[torch.bfloat16])
