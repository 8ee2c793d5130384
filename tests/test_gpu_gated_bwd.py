"""Gated DeltaNet backward through the C-ABI vs the fp64 oracle's reverse mode.

The oracle (``oracle.gated_deltanet_bwd``) applies the chain rule to the
token-serial gated recurrence and is pinned by finite differences, the
no-decay reduction and the pure-decay closed form; the library runs the same
three passes as the ungated backward with the decay factors applied. Cases:
every (dk, dv), ragged lengths and chunk boundaries, strong and mild decay,
initial state and final-state gradient present or absent, no decay against
the ungated backward, the empty sequence, packed sequences, and the
context-parallel backward (deltanet_gated_bwd_cp) over several group counts
and decay strengths. Metric:
max|gpu - oracle| / max|oracle| per gradient tensor.
"""

import numpy as np
import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import (deltanet_bwd, deltanet_gated_bwd, deltanet_gated_bwd_varlen,
                                      longest_first_order)
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs, make_varlen_inputs
from helpers import f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BWD = 2e-2  # as for the ungated backward
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dS0")


def run_gbwd(B, H, T, dk, dv, seed, s0=True, dsf=True, mu=2.0, cp_groups=1):
    print(f"[case] gated bwd B={B} H={H} T={T} dk={dk} dv={dv} s0={s0} dSf={dsf} mu={mu} cp={cp_groups}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=seed, s0_std=0.3 if s0 else 0.0)
    gl = make_gates((B, T, H), seed=seed + 2, mu=mu)
    gen = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    dSf = torch.randn((B, H, dv, dk), generator=gen) * 0.1 if dsf else None
    d = [x.to(DEV) for x in (q, k, v, beta, gl, dO)]
    out = deltanet_gated_bwd(*d, None if S0 is None else S0.to(DEV), None if dSf is None else dSf.to(DEV),
                             cp_groups=cp_groups)
    torch.cuda.synchronize()
    ref = oracle.gated_deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(gl), f64(dO), f64(S0), f64(dSf))
    errs = [rel_err(f64(x), r) for x, r in zip(out, ref)]
    print("  err " + " ".join(f"{n}={e:.3e}" for n, e in zip(NAMES, errs)), flush=True)
    return errs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_gated_bwd_shapes_ragged(dk, dv):
    errs = run_gbwd(2, 2, 200, dk, dv, seed=600 + dk + dv)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_gated_bwd_lengths(T):
    errs = run_gbwd(1, 2, T, 128, 128, seed=610 + T)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("mu", [-1.0, 0.0, 5.0])
def test_gated_bwd_decay_strength(mu):
    # mu = -1: a = sigmoid(N(-1, 1)), most tokens keep under half the state;
    # mu = 5: almost no decay
    errs = run_gbwd(1, 2, 256, 128, 128, seed=620, mu=mu)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("dk,dv,G,mu", [(128, 128, 2, 2.0), (128, 128, 5, -1.0), (128, 128, 7, 5.0),
                                         (64, 64, 3, 2.0), (64, 128, 4, 0.0), (128, 64, 3, -1.0)])
def test_gated_bwd_context_parallel(dk, dv, G, mu):
    # deltanet_gated_bwd_cp: the chains split into G groups (ragged last group)
    errs = run_gbwd(2, 3, 7 * 64 + 21, dk, dv, seed=640 + G + dk, mu=mu, cp_groups=G)
    assert max(errs) <= TOL_BWD


def test_gated_bwd_context_parallel_without_states():
    errs = run_gbwd(1, 2, 6 * 64 + 1, 128, 128, seed=650, s0=False, dsf=False, cp_groups=6)
    assert max(errs) <= TOL_BWD


def test_gated_bwd_without_s0_and_final_gradient():
    errs = run_gbwd(2, 3, 150, 128, 128, seed=630, s0=False, dsf=False)
    assert max(errs) <= TOL_BWD


def test_gated_bwd_no_decay_matches_ungated():
    # g = 0: the gated gradients of q, k, v, beta and S0 are the ungated ones
    B, H, T, dk, dv = 2, 2, 190, 128, 128
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=640, s0_std=0.3)
    gen = torch.Generator().manual_seed(641)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    dSf = torch.randn((B, H, dv, dk), generator=gen) * 0.1
    d = [x.to(DEV) for x in (q, k, v, beta)]
    z = torch.zeros((B, T, H), device=DEV)
    gout = deltanet_gated_bwd(*d, z, dO.to(DEV), S0.to(DEV), dSf.to(DEV))
    uout = deltanet_bwd(*d, dO.to(DEV), S0.to(DEV), dSf.to(DEV))
    torch.cuda.synchronize()
    pairs = [(gout[i], uout[i]) for i in range(4)] + [(gout[5], uout[4])]
    errs = [rel_err(f64(a), f64(b)) for a, b in pairs]
    print("[case] gated bwd g=0 vs ungated: " + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= 1e-2


def test_gated_bwd_empty_sequence():
    S0 = torch.randn(1, 2, 64, 64, device=DEV)
    dSf = torch.randn(1, 2, 64, 64, device=DEV)
    z = torch.empty(1, 0, 2, 64, device=DEV, dtype=torch.bfloat16)
    b = torch.empty(1, 0, 2, device=DEV, dtype=torch.bfloat16)
    gz = torch.empty(1, 0, 2, device=DEV)
    out = deltanet_gated_bwd(z, z, z, b, gz, z, S0, dSf)
    torch.cuda.synchronize()
    assert torch.equal(out[5], dSf) and out[4].numel() == 0


@pytest.mark.parametrize("order", ["given", "longest_first"])
def test_gated_bwd_varlen(order):
    lengths = [0, 1, 63, 64, 65, 200, 130, 7]
    H, dk, dv = 2, 128, 128
    print(f"[case] gated bwd varlen {lengths} order={order}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, H, dk, dv, seed=650, s0_std=0.3)
    gl = make_gates((q.shape[0], H), seed=652, mu=1.0)
    gen = torch.Generator().manual_seed(651)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    dSf = torch.randn((len(lengths), H, dv, dk), generator=gen) * 0.1
    d = [x.to(DEV) for x in (q, k, v, beta, gl, dO)]
    cud = cu.to(DEV)
    so = longest_first_order(cud) if order == "longest_first" else None
    out = deltanet_gated_bwd_varlen(*d, cud, S0.to(DEV), dSf.to(DEV), seq_order=so)
    torch.cuda.synchronize()
    got = [f64(x) for x in out]
    worst = 0.0
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = [f64(x)[None, a:b] for x in (q, k, v, beta, gl, dO)]
        ref = oracle.gated_deltanet_bwd(*sl, f64(S0)[n:n + 1], f64(dSf)[n:n + 1])
        mine = [got[i][None, a:b] for i in range(5)] + [got[5][n:n + 1]]
        errs = [rel_err(x, r) for x, r in zip(mine, ref)] if L > 0 else [rel_err(mine[5], ref[5])]
        worst = max(worst, max(errs))
        assert max(errs) <= TOL_BWD, (n, L, errs)
    print(f"  worst err {worst:.3e}", flush=True)


def test_gated_bwd_varlen_d64_no_state():
    lengths = [100, 1, 64]
    H = 3
    q, k, v, beta, cu, _ = make_varlen_inputs(lengths, H, 64, 64, seed=660)
    gl = make_gates((q.shape[0], H), seed=662)
    gen = torch.Generator().manual_seed(661)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    d = [x.to(DEV) for x in (q, k, v, beta, gl, dO)]
    out = deltanet_gated_bwd_varlen(*d, cu.to(DEV))
    torch.cuda.synchronize()
    got = [f64(x) for x in out]
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = [f64(x)[None, a:b] for x in (q, k, v, beta, gl, dO)]
        ref = oracle.gated_deltanet_bwd(*sl, None, None)
        mine = [got[i][None, a:b] for i in range(5)] + [got[5][n:n + 1]]
        errs = [rel_err(x, r) for x, r in zip(mine, ref)]
        print(f"[case] gated bwd varlen d64 seq {n}: " + " ".join(f"{e:.2e}" for e in errs), flush=True)
        assert max(errs) <= TOL_BWD, (n, errs)


def test_gated_bwd_near_reset_decays():
    # a few g = -80 (the state is all but erased there), as in the forward's reset test
    B, H, T, dk, dv = 1, 2, 200, 128, 128
    print("[case] gated bwd near-reset decays", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=670, s0_std=0.3)
    gl = make_gates((B, T, H), seed=671)
    gl[0, 30, 0] = -80.0
    gl[0, 64, 1] = -80.0
    gl[0, 150, :] = -80.0
    gen = torch.Generator().manual_seed(672)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    dSf = torch.randn((B, H, dv, dk), generator=gen) * 0.1
    d = [x.to(DEV) for x in (q, k, v, beta, gl, dO)]
    out = deltanet_gated_bwd(*d, S0.to(DEV), dSf.to(DEV))
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(x).all()) for x in out)
    ref = oracle.gated_deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(gl), f64(dO), f64(S0), f64(dSf))
    errs = [rel_err(f64(x), r) for x, r in zip(out, ref)]
    print("  err " + " ".join(f"{n}={e:.3e}" for n, e in zip(NAMES, errs)), flush=True)
    assert max(errs) <= TOL_BWD
