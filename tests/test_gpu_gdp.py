"""Gated Delta Product through the C-ABI vs the fp64 oracle.

The oracle runs the substep recurrence of "Linear Attention, Visualized",
"Gated Delta Product (GDP)" token by token (``oracle.gdp_fwd``); the library
runs the chunkwise Gated DeltaNet kernels over the virtual sequence, reading
queries and decays and writing outputs at the real tokens. Cases: both
dtypes, n_h = 2 and 3, ragged virtual lengths, a non-zero initial state,
context parallelism, and n_h = 1 against deltanet_gated_fwd. Bar as for the
other forward paths.
"""

import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import deltanet_gated_fwd, deltanet_gdp_fwd
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gdp_inputs(B, H, T, nh, dk, dv, dtype, seed, s0_std=0.0):
    # the substep tensors come from a virtual-length draw, reshaped [B, T, nh, H, d]
    q, _, _, _, S0 = make_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, s0_std=s0_std)
    _, k, v, beta, _ = make_inputs(B, H, T * nh, dk, dv, dtype=dtype, seed=seed + 1)
    k = k.reshape(B, T, nh, H, dk)
    v = v.reshape(B, T, nh, H, dv)
    beta = beta.reshape(B, T, nh, H)
    g = make_gates((B, T, H), seed=seed)
    return q, k, v, beta, g, S0


@pytest.mark.parametrize("dtype,dk,dv,nh,T,cp", [
    ("bf16", 128, 128, 2, 150, 1),
    ("bf16", 64, 128, 3, 77, 1),
    ("bf16", 128, 64, 2, 200, 3),
    ("bf16", 128, 128, 2, 300, 3),
    ("f32", 64, 64, 2, 90, 1),
    ("f32", 64, 128, 3, 70, 2),
])
def test_gdp_parity(dtype, dk, dv, nh, T, cp):
    print(f"[case] gdp {dtype} dk={dk} dv={dv} n_h={nh} T={T} cp={cp}", flush=True)
    B, H = 2, 3
    q, k, v, beta, g, S0 = gdp_inputs(B, H, T, nh, dk, dv, dtype, seed=300 + T, s0_std=0.3)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o, Sf = deltanet_gdp_fwd(*d, S0.to(DEV), cp_groups=cp)
    torch.cuda.synchronize()
    ro, rs = oracle.gdp_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), nh, f64(S0))
    eo, es = rel_err(f64(o), ro), rel_err(f64(Sf), rs)
    tol = TOL[q.dtype]
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


def test_gdp_one_substep_matches_gated_deltanet():
    B, H, T = 2, 2, 130
    q, k, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=310, s0_std=0.3)
    g = make_gates((B, T, H), seed=310)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o1, s1 = deltanet_gdp_fwd(d[0], d[1][:, :, None], d[2][:, :, None], d[3][:, :, None], d[4], S0.to(DEV))
    o2, s2 = deltanet_gated_fwd(*d, S0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
