"""Gated DeltaNet: HIP path vs the fp64 oracle, element by element, through the C-ABI.

The oracle is the token-serial recurrence of "Linear Attention, Visualized",
"Gated DeltaNet (GDN)" (a_t = exp(g_t) decays the previous state before the
correction). Cases: every supported (dk, dv) and dtype, ragged tails, zero and
non-zero initial states, weak, strong and absent decay, a near-reset token,
context-parallel group counts and packed varlen batches. Bar as for DeltaNet:
max|gpu - oracle| / max|oracle| within 2e-2 (bf16) or 1e-4 (fp32), for o and
for the final state separately.
"""

import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import (deltanet_fwd, deltanet_gated_fwd, deltanet_gated_fwd_varlen,
                                      longest_first_order)
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs, make_varlen_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gated(B, H, T, dk, dv, dtype="bf16", seed=0, s0_std=0.0, cp_groups=1, mu=2.0, edit_g=None):
    print(f"[case] gated B={B} H={H} T={T} dk={dk} dv={dv} {dtype} seed={seed} s0={s0_std} "
          f"cp={cp_groups} mu={mu}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, s0_std=s0_std)
    g = make_gates((B, T, H), seed=seed, mu=mu)
    if edit_g is not None:
        edit_g(g)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    dS0 = None if S0 is None else S0.to(DEV)
    o, Sf = deltanet_gated_fwd(*d, dS0, cp_groups=cp_groups)
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(g), f64(S0))
    return f64(o), f64(Sf), ro, rs, q.dtype


def assert_close(o, Sf, ro, rs, dt):
    tol = TOL[dt]
    eo, es = rel_err(o, ro), rel_err(Sf, rs)
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol, f"o error {eo}"
    assert es <= tol, f"S_final error {es}"


@pytest.mark.parametrize("dv", [64, 128])
def test_gated_fp32_ragged(dv):
    assert_close(*run_gated(2, 2, 150, 64, dv, dtype="f32", seed=101, s0_std=0.5))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_gated_bf16_shapes_ragged(dk, dv):
    assert_close(*run_gated(2, 3, 200, dk, dv, seed=102, s0_std=0.5))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_gated_lengths_around_chunk_boundaries(T):
    assert_close(*run_gated(1, 2, T, 128, 128, seed=110 + T, s0_std=0.3))


@pytest.mark.parametrize("mu,dtype", [(-1.0, "bf16"), (6.0, "bf16"), (-1.0, "f32")])
def test_gated_strong_and_weak_decay(mu, dtype):
    # mu = -1: a averages about 0.3, a chunk decays by ~e^-90 end to end (factors
    # underflow); mu = 6: a close to 1
    dk = 64 if dtype == "f32" else 128
    assert_close(*run_gated(1, 2, 260, dk, 128, dtype=dtype, seed=103, s0_std=0.5, mu=mu))


def test_gated_no_decay_matches_deltanet():
    q, k, v, beta, S0 = make_inputs(1, 2, 300, 128, 128, seed=104, s0_std=0.3)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    g = torch.zeros(1, 300, 2, device=DEV)
    og, sg = deltanet_gated_fwd(*d, g, S0.to(DEV))
    o, s = deltanet_fwd(*d, S0.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    assert_close(f64(og), f64(sg), ro, rs, torch.bfloat16)
    assert rel_err(f64(og), f64(o)) < 1e-2 and rel_err(f64(sg), f64(s)) < 1e-2


def test_gated_near_reset_token():
    # a = e^-80 at token 150 forgets (almost) everything before it
    def edit(g):
        g[:, 150] = -80.0
    assert_close(*run_gated(1, 2, 260, 128, 128, seed=105, s0_std=0.5, edit_g=edit))


def test_gated_deterministic():
    q, k, v, beta, S0 = make_inputs(2, 2, 333, 128, 128, seed=106, s0_std=0.1)
    g = make_gates((2, 333, 2), seed=106)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    a = deltanet_gated_fwd(*d, S0.to(DEV))
    b = deltanet_gated_fwd(*d, S0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("G", [2, 3, 0])
def test_gated_context_parallel_groups(G):
    assert_close(*run_gated(1, 2, 7 * 64 + 20, 128, 128, seed=120 + G, s0_std=0.3, cp_groups=G))


@pytest.mark.parametrize("mu", [-1.0, 5.0])
def test_gated_context_parallel_decay_strength(mu):
    # strong (mu = -1) and weak decay through the 128-row transitions, 3 units of 5 groups
    assert_close(*run_gated(1, 3, 9 * 64 + 7, 128, 128, seed=130, s0_std=0.3, cp_groups=5, mu=mu))


def test_gated_context_parallel_fp32():
    assert_close(*run_gated(1, 1, 6 * 64 + 9, 64, 64, dtype="f32", seed=125, s0_std=0.3, cp_groups=3))


@pytest.mark.parametrize("order", ["natural", "longest_first"])
def test_gated_varlen(order):
    lengths = [0, 1, 63, 64, 65, 300, 130, 7]
    print(f"[case] gated varlen {lengths} order={order}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, 3, 128, 128, seed=130, s0_std=0.3)
    g = make_gates((q.shape[0], 3), seed=130)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    cud = cu.to(DEV)
    so = longest_first_order(cud) if order == "longest_first" else None
    o, Sf = deltanet_gated_fwd_varlen(*d, cud, S0.to(DEV), seq_order=so)
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), f64(g),
                                              cu.numpy(), f64(S0))
    assert_close(f64(o), f64(Sf), ro, rs, torch.bfloat16)


def test_gated_varlen_fp32():
    lengths = [70, 5, 128]
    q, k, v, beta, cu, _ = make_varlen_inputs(lengths, 2, 64, 128, dtype="f32", seed=131)
    g = make_gates((q.shape[0], 2), seed=131)
    d = [x.to(DEV) for x in (q, k, v, beta, g)]
    o, Sf = deltanet_gated_fwd_varlen(*d, cu.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.gated_deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), f64(g), cu.numpy())
    assert_close(f64(o), f64(Sf), ro, rs, torch.float32)
