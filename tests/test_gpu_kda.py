"""Kimi Delta Attention forward through the C-ABI vs the fp64 oracle.

The oracle runs the KDA token recurrence of "Linear Attention, Visualized"
("Kimi Delta Attention (KDA)": per-channel decay, then the delta rule) token
by token; the library runs that section's per-chunk algorithm on 16-token
sub-chunks. Cases: every (dk, dv), ragged lengths around chunk and sub-chunk
boundaries, initial state, weak, strong and absent decay, decay equal
across channels against the Gated DeltaNet kernel, packed sequences
(varlen) against the oracle per sequence, and context parallelism (group
transitions, composition, per-group outputs). Bar: max|gpu - oracle| /
max|oracle| within 2e-2 (bf16 operands), for o and for the final state.
"""

import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import (deltanet_gated_fwd, deltanet_kda_fwd, deltanet_kda_fwd_varlen,
                                      longest_first_order)
from chunkwise_delta_rule_amd.synth import make_channel_gates, make_inputs, make_varlen_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_kda(B, H, T, dk, dv, seed, s0_std=0.3, mu=2.0):
    print(f"[case] kda B={B} H={H} T={T} dk={dk} dv={dv} mu={mu}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=seed, s0_std=s0_std)
    g = make_channel_gates((B, T, H, dk), seed=seed, mu=mu)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o, Sf = deltanet_kda_fwd(*d, None if S0 is None else S0.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(f64(o), ro), rel_err(f64(Sf), rs)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    return eo, es


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_kda_shapes_ragged(dk, dv):
    eo, es = run_kda(2, 2, 200, dk, dv, seed=500 + dk + dv)
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("T", [1, 15, 16, 17, 64, 65, 130])
def test_kda_lengths(T):
    eo, es = run_kda(1, 2, T, 128, 128, seed=510 + T)
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("mu", [-1.0, 6.0])
def test_kda_strong_and_weak_decay(mu):
    eo, es = run_kda(1, 2, 150, 128, 128, seed=520, mu=mu)
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_kda_equal_channels_matches_gated_deltanet():
    B, H, T = 1, 2, 140
    q, k, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=530, s0_std=0.3)
    gs = make_channel_gates((B, T, H, 1), seed=530).expand(B, T, H, 128).contiguous()
    d = [x.to(DEV) for x in (q, k, v, beta)]
    o1, s1 = deltanet_kda_fwd(*d, gs.to(DEV), S0.to(DEV))
    o2, s2 = deltanet_gated_fwd(*d, gs[..., 0].contiguous().to(DEV), S0.to(DEV))
    torch.cuda.synchronize()
    assert rel_err(f64(o1), f64(o2)) < 2e-2 and rel_err(f64(s1), f64(s2)) < 2e-2


@pytest.mark.parametrize("order", ["given", "longest_first"])
def test_kda_varlen(order):
    # packed sequences, the state starting afresh at each one: every sequence
    # against the oracle's KDA recurrence over that sequence alone
    lengths = [0, 1, 15, 16, 17, 64, 65, 200, 130, 7]
    H, dk, dv = 3, 128, 128
    print(f"[case] kda varlen {lengths} order={order}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, H, dk, dv, seed=330, s0_std=0.3)
    g = make_channel_gates((1, sum(lengths), H, dk), seed=330)[0]
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    cud = cu.to(DEV)
    so = longest_first_order(cud) if order == "longest_first" else None
    o, Sf = deltanet_kda_fwd_varlen(*d, cud, S0.to(DEV), seq_order=so)
    torch.cuda.synchronize()
    o64, s64 = f64(o), f64(Sf)
    worst = 0.0
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = [f64(x)[None, a:b] for x in (q, k, v, beta, g)]
        ro, rs = oracle.kda_fwd(*sl, f64(S0)[n:n + 1])
        es = rel_err(s64[n:n + 1], rs)
        eo = rel_err(o64[None, a:b], ro) if L > 0 else 0.0
        worst = max(worst, eo, es)
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16], (n, L, eo, es)
    print(f"  worst err {worst:.3e}", flush=True)


@pytest.mark.parametrize("G", [2, 5, 8, 0])
def test_kda_context_parallel(G):
    # one long sequence per head split into G groups (0: the library's choice):
    # transitions from the identity, composition, then every group from its start
    B, H, T, dk, dv = 1, 2, 1000, 128, 128
    print(f"[case] kda context parallel T={T} G={G}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, seed=340 + G, s0_std=0.3)
    g = make_channel_gates((B, T, H, dk), seed=340 + G)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o, Sf = deltanet_kda_fwd(*d, S0.to(DEV), cp_groups=G)
    os_, Ss = deltanet_kda_fwd(*d, S0.to(DEV), cp_groups=1)
    torch.cuda.synchronize()
    ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    eo, es = rel_err(f64(o), ro), rel_err(f64(Sf), rs)
    print(f"  err o={eo:.3e} S={es:.3e}; vs serial o={rel_err(f64(o), f64(os_)):.3e}", flush=True)
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
    assert rel_err(f64(o), f64(os_)) <= TOL[torch.bfloat16]


def test_kda_context_parallel_shapes():
    for dk, dv in [(64, 64), (64, 128), (128, 64)]:
        q, k, v, beta, S0 = make_inputs(2, 1, 300, dk, dv, seed=350 + dk + dv, s0_std=0.3)
        g = make_channel_gates((2, 300, 1, dk), seed=350 + dk + dv)
        d = [x.to(DEV) for x in (q, k, v, beta, g)]
        o, Sf = deltanet_kda_fwd(*d, S0.to(DEV), cp_groups=3)
        torch.cuda.synchronize()
        ro, rs = oracle.kda_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
        eo, es = rel_err(f64(o), ro), rel_err(f64(Sf), rs)
        print(f"[case] kda cp dk={dk} dv={dv}: err o={eo:.3e} S={es:.3e}", flush=True)
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_kda_varlen_small_heads():
    # dk = dv = 64, one head per sequence, a single very short and a long one
    lengths = [3, 130, 64]
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, 1, 64, 64, seed=360, s0_std=0.3)
    g = make_channel_gates((1, sum(lengths), 1, 64), seed=360)[0]
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o, Sf = deltanet_kda_fwd_varlen(*d, cu.to(DEV), S0.to(DEV))
    torch.cuda.synchronize()
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        ro, rs = oracle.kda_fwd(*[f64(x)[None, a:b] for x in (q, k, v, beta, g)], f64(S0)[n:n + 1])
        eo, es = rel_err(f64(o)[None, a:b], ro), rel_err(f64(Sf)[n:n + 1], rs)
        print(f"[case] kda varlen d64 seq {n}: err o={eo:.3e} S={es:.3e}", flush=True)
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
