"""Backward pass through the C-ABI vs the fp64 oracle's reverse mode.

The oracle (``oracle.deltanet_bwd``) applies the chain rule to the
token-serial recurrence and is pinned by finite differences; the library runs
three passes (forward chain keeping per-chunk states, reverse state-gradient
chain, chunk-parallel finish). Cases: every (dk, dv), ragged lengths, chunk
boundaries, initial state and final-state gradient present or absent, the
empty sequence, packed sequences (varlen) against the oracle per sequence, and
the context-parallel backward (deltanet_bwd_cp) over several group counts. Metric: max|gpu - oracle| / max|oracle| per gradient tensor.
"""

import numpy as np
import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import deltanet_bwd, deltanet_bwd_varlen, longest_first_order
from chunkwise_delta_rule_amd.synth import make_inputs, make_varlen_inputs
from helpers import f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BWD = 2e-2  # as for the bf16 forward; measured errors are 1e-3 .. 7e-3


def run_bwd(B, H, T, dk, dv, seed, s0=True, dsf=True, cp_groups=1):
    print(f"[case] bwd B={B} H={H} T={T} dk={dk} dv={dv} s0={s0} dSf={dsf} cp={cp_groups}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=seed, s0_std=0.3 if s0 else 0.0)
    g = torch.Generator().manual_seed(seed + 1)
    dO = torch.randn(v.shape, generator=g).to(torch.bfloat16)
    dSf = torch.randn((B, H, dv, dk), generator=g) * 0.1 if dsf else None
    d = [x.to(DEV) for x in (q, k, v, beta, dO)]
    out = deltanet_bwd(d[0], d[1], d[2], d[3], d[4], None if S0 is None else S0.to(DEV),
                       None if dSf is None else dSf.to(DEV), cp_groups=cp_groups)
    torch.cuda.synchronize()
    ref = oracle.deltanet_bwd(f64(q), f64(k), f64(v), f64(beta), f64(dO), f64(S0), f64(dSf))
    errs = [rel_err(f64(x), r) for x, r in zip(out, ref)]
    print("  err dq={:.3e} dk={:.3e} dv={:.3e} dbeta={:.3e} dS0={:.3e}".format(*errs), flush=True)
    return errs


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bwd_shapes_ragged(dk, dv):
    errs = run_bwd(2, 2, 200, dk, dv, seed=400 + dk + dv)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_bwd_lengths(T):
    errs = run_bwd(1, 2, T, 128, 128, seed=410 + T)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("dk,dv,G", [(128, 128, 2), (128, 128, 3), (128, 128, 7), (64, 64, 4), (64, 128, 3),
                                      (128, 64, 5)])
def test_bwd_context_parallel(dk, dv, G):
    # deltanet_bwd_cp: the chains split into G groups (ragged last group)
    errs = run_bwd(2, 3, 7 * 64 + 21, dk, dv, seed=430 + G + dk, cp_groups=G)
    assert max(errs) <= TOL_BWD


@pytest.mark.parametrize("s0,dsf", [(False, False), (True, False), (False, True)])
def test_bwd_context_parallel_optional_states(s0, dsf):
    errs = run_bwd(1, 2, 6 * 64 + 1, 128, 128, seed=440, s0=s0, dsf=dsf, cp_groups=6)
    assert max(errs) <= TOL_BWD


def test_bwd_context_parallel_matches_serial_closely():
    q, k, v, beta, S0 = make_inputs(1, 2, 2000, 128, 128, seed=450, s0_std=0.2)
    g = torch.Generator().manual_seed(451)
    dO = torch.randn(v.shape, generator=g).to(torch.bfloat16)
    dSf = torch.randn((1, 2, 128, 128), generator=g) * 0.1
    d = [x.to(DEV) for x in (q, k, v, beta, dO, S0, dSf)]
    a = deltanet_bwd(*d)
    b = deltanet_bwd(*d, cp_groups=4)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert rel_err(f64(y), f64(x)) < 2e-2


def test_bwd_without_s0_and_final_gradient():
    errs = run_bwd(2, 3, 150, 128, 128, seed=420, s0=False, dsf=False)
    assert max(errs) <= TOL_BWD


def test_bwd_empty_sequence():
    S0 = torch.randn(1, 2, 64, 64, device=DEV)
    dSf = torch.randn(1, 2, 64, 64, device=DEV)
    z = torch.empty(1, 0, 2, 64, device=DEV, dtype=torch.bfloat16)
    b = torch.empty(1, 0, 2, device=DEV, dtype=torch.bfloat16)
    out = deltanet_bwd(z, z, z, b, z, S0, dSf)
    out0 = deltanet_bwd(z, z, z, b, z, S0, None)
    torch.cuda.synchronize()
    assert torch.equal(out[4], dSf) and bool((out0[4] == 0).all())


@pytest.mark.parametrize("order", ["given", "longest_first"])
def test_bwd_varlen(order):
    # packed sequences (the state and its gradient restart at each one): every
    # sequence's gradients against the oracle's reverse mode over that sequence
    lengths = [0, 1, 63, 64, 65, 200, 130, 7]
    H, dk, dv = 2, 128, 128
    print(f"[case] bwd varlen {lengths} order={order}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, H, dk, dv, seed=430, s0_std=0.3)
    g = torch.Generator().manual_seed(431)
    dO = torch.randn(v.shape, generator=g).to(torch.bfloat16)
    dSf = torch.randn((len(lengths), H, dv, dk), generator=g) * 0.1
    d = [x.to(DEV) for x in (q, k, v, beta, dO)]
    cud = cu.to(DEV)
    so = longest_first_order(cud) if order == "longest_first" else None
    out = deltanet_bwd_varlen(d[0], d[1], d[2], d[3], d[4], cud, S0.to(DEV), dSf.to(DEV), seq_order=so)
    torch.cuda.synchronize()
    got = [f64(x) for x in out]
    worst = 0.0
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = [f64(x)[None, a:b] for x in (q, k, v, beta, dO)]
        ref = oracle.deltanet_bwd(*sl[:4], sl[4], f64(S0)[n:n + 1], f64(dSf)[n:n + 1])
        mine = [got[0][None, a:b], got[1][None, a:b], got[2][None, a:b], got[3][None, a:b], got[4][n:n + 1]]
        errs = [rel_err(x, r) for x, r in zip(mine, ref)] if L > 0 else [rel_err(mine[4], ref[4])]
        worst = max(worst, max(errs))
        assert max(errs) <= TOL_BWD, (n, L, errs)
    print(f"  worst err {worst:.3e}", flush=True)


def test_bwd_varlen_d64_no_state():
    # dk = dv = 64, no initial state and no final-state gradient
    lengths = [100, 1, 64]
    H = 3
    q, k, v, beta, cu, _ = make_varlen_inputs(lengths, H, 64, 64, seed=440)
    g = torch.Generator().manual_seed(441)
    dO = torch.randn(v.shape, generator=g).to(torch.bfloat16)
    d = [x.to(DEV) for x in (q, k, v, beta, dO)]
    out = deltanet_bwd_varlen(*d, cu.to(DEV))
    torch.cuda.synchronize()
    got = [f64(x) for x in out]
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = [f64(x)[None, a:b] for x in (q, k, v, beta, dO)]
        ref = oracle.deltanet_bwd(*sl[:4], sl[4], None, None)
        mine = [got[0][None, a:b], got[1][None, a:b], got[2][None, a:b], got[3][None, a:b], got[4][n:n + 1]]
        errs = [rel_err(x, r) for x, r in zip(mine, ref)]
        print(f"[case] bwd varlen d64 seq {n}: " + " ".join(f"{e:.2e}" for e in errs), flush=True)
        assert max(errs) <= TOL_BWD, (n, errs)
