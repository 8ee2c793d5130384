"""Full-size workloads on the GPU, checked against the fp64 oracle on sampled units.

Each workload runs at its full shape in the launch configuration the
benchmark uses; the oracle then recomputes a sample of (sequence, head)
units from exact host copies of their inputs. Tolerance as for the small
cases: max|gpu - oracle| / max|oracle| <= 2e-2 (bf16), 1e-4 (fp32), for o and
for the final state. Properties that hold at any size (finite outputs,
context-parallel == serial within tolerance on every head) are checked on
the whole tensors.
"""

import numpy as np
import pytest
import torch

import oracle
import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import WORKLOADS, make_channel_gates, make_gates, workload_inputs
from helpers import TOL, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_dense_sample(w, inputs, o, Sf, units):
    q, k, v, beta, S0 = inputs
    sel = lambda x, b, h: f64(x[b:b + 1, :, h:h + 1])
    ro_all, rs_all, go_all, gs_all = [], [], [], []
    args = [[], [], [], [], []]
    for b, h in units:
        args[0].append(sel(q, b, h))
        args[1].append(sel(k, b, h))
        args[2].append(sel(v, b, h))
        args[3].append(f64(beta[b:b + 1, :, h:h + 1]))
        args[4].append(None if S0 is None else f64(S0[b:b + 1, h:h + 1]))
    # one oracle call over the sampled units (stacked as a batch) runs them in parallel
    cat = lambda xs: np.concatenate(xs, axis=0)
    ro, rs = oracle.deltanet_fwd(cat(args[0]), cat(args[1]), cat(args[2]), cat(args[3]),
                                 None if S0 is None else cat(args[4]))
    for i, (b, h) in enumerate(units):
        go_all.append(f64(o[b, :, h]))
        gs_all.append(f64(Sf[b, h]))
        ro_all.append(ro[i, :, 0])
        rs_all.append(rs[i, 0])
    eo = rel_err(np.stack(go_all), np.stack(ro_all))
    es = rel_err(np.stack(gs_all), np.stack(rs_all))
    tol = TOL[q.dtype]
    print(f"  {w.name}: sampled {len(units)} units, err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


def run_dense(w, cp_groups=1, seed=2):
    print(f"[case] {w.name} full size, cp_groups={cp_groups}", flush=True)
    inputs = workload_inputs(w, seed=seed, device=DEV)
    q, k, v, beta, S0 = inputs
    o, Sf = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=cp_groups)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    return inputs, o, Sf


def test_tiny_f32_full():
    w = WORKLOADS["tiny_f32"]
    inputs, o, Sf = run_dense(w)
    check_dense_sample(w, inputs, o, Sf, [(0, 0)])


def test_layer_b8_h16_t4096_sampled():
    w = WORKLOADS["layer_b8_h16_t4096"]
    inputs, o, Sf = run_dense(w)
    check_dense_sample(w, inputs, o, Sf, [(0, 0), (1, 5), (3, 15), (5, 8), (7, 3), (7, 15)])


def test_chunks128_b4_h16_t8192_sampled():
    w = WORKLOADS["chunks128_b4_h16_t8192"]
    inputs, o, Sf = run_dense(w)
    assert inputs[4] is not None  # non-zero initial state
    check_dense_sample(w, inputs, o, Sf, [(0, 0), (1, 7), (2, 12), (3, 15)])


@pytest.mark.parametrize("cp_groups", [1, 0])
def test_long_b1_h16_t131072_sampled(cp_groups):
    w = WORKLOADS["long_b1_h16_t131072"]
    inputs, o, Sf = run_dense(w, cp_groups=cp_groups)
    check_dense_sample(w, inputs, o, Sf, [(0, 3), (0, 12)])


def test_long_context_parallel_equals_serial_on_every_head():
    w = WORKLOADS["long_b1_h16_t131072"]
    q, k, v, beta, S0 = workload_inputs(w, seed=3, device=DEV)
    o1, s1 = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=1)
    oc, sc = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=0)
    torch.cuda.synchronize()
    groups = dn.deltanet_pick_cp_groups(w.B, w.H, w.T, w.dk, w.dv)
    assert groups > 1
    for h in range(w.H):
        eo = rel_err(f64(oc[0, :, h]), f64(o1[0, :, h]))
        es = rel_err(f64(sc[0, h]), f64(s1[0, h]))
        assert eo <= 2e-2 and es <= 2e-2, (h, eo, es)


def test_varlen_n64_h32_sampled():
    w = WORKLOADS["varlen_n64_h32"]
    print(f"[case] {w.name} full size", flush=True)
    q, k, v, beta, cu, S0, lengths = workload_inputs(w, seed=2, device=DEV)
    order = dn.longest_first_order(cu)
    o, Sf = dn.deltanet_fwd_varlen(q, k, v, beta, cu, S0, seq_order=order)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    cu_h = cu.cpu().numpy().astype(np.int64)
    lens = np.diff(cu_h)
    # the longest and shortest sequences and two in between, two heads each
    by_len = np.argsort(lens)
    seqs = [int(by_len[-1]), int(by_len[0]), int(by_len[len(by_len) // 2]), 17]
    heads = [0, 31, 9, 20]
    go, gs, ro, rs = [], [], [], []
    for n, h in zip(seqs, heads):
        a, b = int(cu_h[n]), int(cu_h[n + 1])
        sel = lambda x: f64(x[a:b, h:h + 1])
        o_ref, s_ref = oracle.deltanet_fwd_varlen(sel(q), sel(k), sel(v), f64(beta[a:b, h:h + 1]),
                                                  np.array([0, b - a]))
        go.append(f64(o[a:b, h]).ravel())
        ro.append(o_ref[:, 0].ravel())
        gs.append(f64(Sf[n, h]))
        rs.append(s_ref[0, 0])
    eo = rel_err(np.concatenate(go), np.concatenate(ro))
    es = rel_err(np.stack(gs), np.stack(rs))
    print(f"  varlen: sampled units {list(zip(seqs, heads))} lengths {[int(lens[n]) for n in seqs]} "
          f"err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def test_gated_layer_b8_h16_t4096_sampled():
    # Gated DeltaNet at the benchmark's full shape and launch configuration
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, gated", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = make_gates((w.B, w.T, w.H), seed=2, device=DEV)
    o, Sf = dn.deltanet_gated_fwd(q, k, v, beta, g, S0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    units = [(0, 0), (2, 9), (6, 15)]
    sel = lambda x, b, h: f64(x[b:b + 1, :, h:h + 1])
    cat = lambda xs: np.concatenate(xs, axis=0)
    ro, rs = oracle.gated_deltanet_fwd(*(cat([sel(x, b, h) for b, h in units]) for x in (q, k, v, beta, g)))
    eo = rel_err(np.stack([f64(o[b, :, h]) for b, h in units]), ro[:, :, 0])
    es = rel_err(np.stack([f64(Sf[b, h]) for b, h in units]), rs[:, 0])
    print(f"  gated {w.name}: sampled {len(units)} units, err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= TOL[q.dtype] and es <= TOL[q.dtype]


def test_gated_long_context_parallel_sampled():
    w = WORKLOADS["long_b1_h16_t131072"]
    print(f"[case] {w.name} full size, gated, cp auto", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=4, device=DEV)
    g = make_gates((w.B, w.T, w.H), seed=4, device=DEV)
    o, Sf = dn.deltanet_gated_fwd(q, k, v, beta, g, S0, cp_groups=0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    h = 6
    sel = lambda x: f64(x[:, :, h:h + 1])
    ro, rs = oracle.gated_deltanet_fwd(sel(q), sel(k), sel(v), sel(beta), sel(g))
    eo = rel_err(f64(o[0, :, h]), ro[0, :, 0])
    es = rel_err(f64(Sf[0, h]), rs[0, 0])
    print(f"  gated {w.name} head {h}: err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def test_bwd_layer_b8_h16_t4096_sampled():
    # the backward pass at the benchmark's full shape, sampled units against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, backward", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=DEV, dtype=torch.float32).to(v.dtype)
    out = dn.deltanet_bwd(q, k, v, beta, dO, S0)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(x).all()) for x in out)
    units = [(0, 0), (5, 11)]
    sel = lambda x, b, h: f64(x[b:b + 1, :, h:h + 1])
    cat = lambda xs: np.concatenate(xs, axis=0)
    ref = oracle.deltanet_bwd(*(cat([sel(x, b, h) for b, h in units]) for x in (q, k, v, beta, dO)))
    for name, i, gi in (("dq", 0, out[0]), ("dk", 1, out[1]), ("dv", 2, out[2])):
        e = rel_err(np.stack([f64(gi[b, :, h]) for b, h in units]), ref[i][:, :, 0])
        print(f"  {name} err {e:.3e}", flush=True)
        assert e <= 2e-2
    eb = rel_err(np.stack([f64(out[3][b, :, h]) for b, h in units]), ref[3][:, :, 0])
    es = rel_err(np.stack([f64(out[4][b, h]) for b, h in units]), ref[4][:, 0])
    print(f"  dbeta err {eb:.3e} dS0 err {es:.3e}", flush=True)
    assert eb <= 2e-2 and es <= 2e-2


def test_gated_bwd_layer_b8_h16_t4096_sampled():
    # the Gated DeltaNet backward at the benchmark's full shape, in the launch
    # configuration bench.py times, sampled units against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, gated backward", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=3, device=DEV)
    gl = make_gates((w.B, w.T, w.H), seed=7, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(9)
    dO = torch.randn(v.shape, generator=g, device=DEV, dtype=torch.float32).to(v.dtype)
    out = dn.deltanet_gated_bwd(q, k, v, beta, gl, dO, S0)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(x).all()) for x in out)
    units = [(0, 3), (7, 15)]
    sel = lambda x, b, h: f64(x[b:b + 1, :, h:h + 1])
    cat = lambda xs: np.concatenate(xs, axis=0)
    ref = oracle.gated_deltanet_bwd(*(cat([sel(x, b, h) for b, h in units]) for x in (q, k, v, beta, gl, dO)))
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2), ("dbeta", 3), ("dg", 4)):
        e = rel_err(np.stack([f64(out[i][b, :, h]) for b, h in units]), ref[i][:, :, 0])
        print(f"  {name} err {e:.3e}", flush=True)
        assert e <= 2e-2
    es = rel_err(np.stack([f64(out[5][b, h]) for b, h in units]), ref[5][:, 0])
    print(f"  dS0 err {es:.3e}", flush=True)
    assert es <= 2e-2


def test_gdp_bwd_layer_b8_h16_t4096_sampled():
    # the GDP backward (n_h = 2) at the benchmark's full shape, inputs drawn
    # as bench.py's variant draws them, sampled units against the oracle
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
    assert all(bool(torch.isfinite(x).all()) for x in out)
    units = [(2, 5)]
    for b, h in units:
        ref = oracle.gdp_bwd(f64(q[b:b + 1, :, h:h + 1]), f64(k[b:b + 1, :, :, h:h + 1]),
                             f64(v[b:b + 1, :, :, h:h + 1]), f64(beta[b:b + 1, :, :, h:h + 1]),
                             f64(gl[b:b + 1, :, h:h + 1]), nh, f64(dO[b:b + 1, :, h:h + 1]))
        mine = [f64(out[0][b:b + 1, :, h:h + 1]), f64(out[1][b:b + 1, :, :, h:h + 1]),
                f64(out[2][b:b + 1, :, :, h:h + 1]), f64(out[3][b:b + 1, :, :, h:h + 1]),
                f64(out[4][b:b + 1, :, h:h + 1]), f64(out[5][b:b + 1, h:h + 1])]
        errs = [rel_err(x, r) for x, r in zip(mine, ref)]
        print("  unit ({}, {}) err ".format(b, h) + " ".join(f"{e:.3e}" for e in errs), flush=True)
        assert max(errs) <= 2e-2


def test_kda_layer_b8_h16_t4096_sampled():
    # KDA at the benchmark's full shape, sampled units against the oracle
    w = WORKLOADS["layer_b8_h16_t4096"]
    print(f"[case] {w.name} full size, kda", flush=True)
    q, k, v, beta, S0 = workload_inputs(w, seed=2, device=DEV)
    g = make_channel_gates((w.B, w.T, w.H, w.dk), seed=2, device=DEV)
    o, Sf = dn.deltanet_kda_fwd(q, k, v, beta, g, S0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(Sf).all())
    units = [(1, 1), (6, 14)]
    sel = lambda x, b, h: f64(x[b:b + 1, :, h:h + 1])
    cat = lambda xs: np.concatenate(xs, axis=0)
    ro, rs = oracle.kda_fwd(*(cat([sel(x, b, h) for b, h in units]) for x in (q, k, v, beta, g)))
    eo = rel_err(np.stack([f64(o[b, :, h]) for b, h in units]), ro[:, :, 0])
    es = rel_err(np.stack([f64(Sf[b, h]) for b, h in units]), rs[:, 0])
    print(f"  kda {w.name}: err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2
