"""Gated Delta Product backward through the C-ABI vs the fp64 oracle.

The oracle (``oracle.gdp_bwd``) is the gated reverse mode over the virtual
sequence of "Linear Attention, Visualized", "GDP as GDN over a virtual
sequence", pinned by central differences of the token-by-token GDP forward.
The library runs the gated backward passes over the virtual sequence, reading
queries, decays and output gradients at the real tokens and writing dq and dg
there. Cases: n_h = 2 and 3, every (dk, dv) among them, ragged virtual
lengths, with and without S0 and dS_final, and n_h = 1 against
deltanet_gated_bwd. Metric: max|gpu - oracle| / max|oracle| per gradient.
"""

import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import deltanet_gated_bwd, deltanet_gdp_bwd
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs
from helpers import f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BWD = 2e-2  # as for the other backward paths
NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dS0")


def gdp_inputs(B, H, T, nh, dk, dv, seed, s0_std=0.0):
    # the substep tensors come from a virtual-length draw, reshaped [B, T, nh, H, d]
    q, _, _, _, S0 = make_inputs(B, H, T, dk, dv, seed=seed, s0_std=s0_std)
    _, k, v, beta, _ = make_inputs(B, H, T * nh, dk, dv, seed=seed + 1)
    k = k.reshape(B, T, nh, H, dk)
    v = v.reshape(B, T, nh, H, dv)
    beta = beta.reshape(B, T, nh, H)
    g = make_gates((B, T, H), seed=seed)
    return q, k, v, beta, g, S0


@pytest.mark.parametrize("dk,dv,nh,T,s0,dsf", [
    (128, 128, 2, 150, True, True),
    (64, 128, 3, 77, True, False),
    (128, 64, 2, 200, False, True),
    (64, 64, 3, 43, False, False),
    (128, 128, 4, 33, True, True),
])
def test_gdp_bwd_parity(dk, dv, nh, T, s0, dsf):
    print(f"[case] gdp bwd dk={dk} dv={dv} n_h={nh} T={T} s0={s0} dSf={dsf}", flush=True)
    B, H = 2, 2
    q, k, v, beta, g, S0 = gdp_inputs(B, H, T, nh, dk, dv, seed=700 + T, s0_std=0.3 if s0 else 0.0)
    gen = torch.Generator().manual_seed(701 + T)
    dO = torch.randn((B, T, H, dv), generator=gen).to(torch.bfloat16)
    dSf = torch.randn((B, H, dv, dk), generator=gen) * 0.1 if dsf else None
    d = [x.to(DEV) for x in (q, k, v, beta, g, dO)]
    out = deltanet_gdp_bwd(*d, None if S0 is None else S0.to(DEV), None if dSf is None else dSf.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gdp_bwd(f64(q), f64(k), f64(v), f64(beta), f64(g), nh, f64(dO), f64(S0), f64(dSf))
    errs = [rel_err(f64(x), r) for x, r in zip(out, ref)]
    print("  err " + " ".join(f"{n}={e:.3e}" for n, e in zip(NAMES, errs)), flush=True)
    assert max(errs) <= TOL_BWD


def test_gdp_bwd_one_substep_matches_gated_bwd():
    B, H, T = 2, 2, 130
    q, k, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=720, s0_std=0.3)
    g = make_gates((B, T, H), seed=720)
    gen = torch.Generator().manual_seed(721)
    dO = torch.randn(v.shape, generator=gen).to(torch.bfloat16)
    d = [x.to(DEV) for x in (q, k, v, beta, g, dO)]
    a = deltanet_gdp_bwd(d[0], d[1][:, :, None], d[2][:, :, None], d[3][:, :, None], d[4], d[5], S0.to(DEV))
    b = deltanet_gated_bwd(*d, S0.to(DEV))
    torch.cuda.synchronize()
    same = [torch.equal(a[0], b[0]), torch.equal(a[1][:, :, 0], b[1]), torch.equal(a[2][:, :, 0], b[2]),
            torch.equal(a[3][:, :, 0], b[3]), torch.equal(a[4], b[4]), torch.equal(a[5], b[5])]
    print(f"[case] gdp bwd n_h=1 vs gated bwd: identical {same}", flush=True)
    assert all(same)
