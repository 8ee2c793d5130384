"""HIP path vs the fp64 oracle, element by element, through the C-ABI.

Small cases cover several chunks, ragged tails, every supported (dk, dv) and
dtype, zero and non-zero initial states, degenerate inputs, context-parallel
group counts and packed varlen batches. Bar: max|gpu - oracle| / max|oracle|
within 2e-2 (bf16) or 1e-4 (fp32), for o and for the final state separately.
"""

import numpy as np
import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import deltanet_fwd, deltanet_fwd_varlen, longest_first_order
from chunkwise_delta_rule_amd.synth import make_inputs, make_varlen_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_dense(B, H, T, dk, dv, dtype="bf16", seed=0, s0_std=0.0, cp_groups=1, beta_zero=None):
    print(f"[case] dense B={B} H={H} T={T} dk={dk} dv={dv} {dtype} seed={seed} "
          f"s0={s0_std} cp={cp_groups}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, dtype=dtype, seed=seed, s0_std=s0_std)
    if beta_zero is not None:
        beta[:, beta_zero] = 0
    dq, dk_, dv_, db = (x.to(DEV) for x in (q, k, v, beta))
    dS0 = None if S0 is None else S0.to(DEV)
    o, Sf = deltanet_fwd(dq, dk_, dv_, db, dS0, cp_groups=cp_groups)
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    return f64(o), f64(Sf), ro, rs, q.dtype


def assert_close(o, Sf, ro, rs, dt):
    tol = TOL[dt]
    eo, es = rel_err(o, ro), rel_err(Sf, rs)
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol, f"o error {eo}"
    assert es <= tol, f"S_final error {es}"


def test_tiny_fp32_workload():
    # B=1, H=1, T=256, d=64, fp32, zero initial state
    assert_close(*run_dense(1, 1, 256, 64, 64, dtype="f32", seed=1))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_bf16_shapes_ragged(dk, dv):
    assert_close(*run_dense(2, 3, 200, dk, dv, seed=2, s0_std=0.5))


@pytest.mark.parametrize("dv", [64, 128])
def test_fp32_shapes_ragged(dv):
    assert_close(*run_dense(2, 2, 150, 64, dv, dtype="f32", seed=3, s0_std=0.5))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 129])
def test_lengths_around_chunk_boundaries(T):
    assert_close(*run_dense(1, 2, T, 128, 128, seed=10 + T, s0_std=0.3))


def test_zero_length_copies_state():
    S0 = torch.randn(2, 3, 128, 128, device=DEV)
    z = torch.empty(2, 0, 3, 128, device=DEV, dtype=torch.bfloat16)
    o, Sf = deltanet_fwd(z, z, z, torch.empty(2, 0, 3, device=DEV, dtype=torch.bfloat16), S0)
    torch.cuda.synchronize()
    assert torch.equal(Sf, S0)


def test_beta_zero_tokens():
    # some tokens write nothing (beta = 0), including a whole leading chunk
    assert_close(*run_dense(1, 2, 300, 128, 128, seed=5, s0_std=0.5,
                            beta_zero=list(range(0, 64)) + [100, 101, 250]))


def test_final_state_optional_and_no_s0():
    q, k, v, beta, _ = make_inputs(2, 2, 130, 128, 128, seed=6)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    o1, s1 = deltanet_fwd(*d, None)
    o2, s2 = deltanet_fwd(*d, None, output_final_state=False)
    torch.cuda.synchronize()
    assert s2 is None and torch.equal(o1, o2)


def test_resume_from_final_state():
    # [0, T1) then [T1, T) from the returned state equals one pass (up to rounding)
    q, k, v, beta, S0 = make_inputs(2, 2, 320, 128, 128, seed=7, s0_std=0.2)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    t1 = 192
    o_a, s_a = deltanet_fwd(*(x[:, :t1].contiguous() for x in d), S0.to(DEV))
    o_b, s_b = deltanet_fwd(*(x[:, t1:].contiguous() for x in d), s_a)
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    o = np.concatenate([f64(o_a), f64(o_b)], axis=1)
    assert_close(o, f64(s_b), ro, rs, torch.bfloat16)


def test_deterministic():
    q, k, v, beta, S0 = make_inputs(2, 4, 333, 128, 128, seed=8, s0_std=0.1)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    a = deltanet_fwd(*d, S0.to(DEV))
    b = deltanet_fwd(*d, S0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("G", [2, 3, 7, 0])
def test_context_parallel_groups(G):
    assert_close(*run_dense(1, 2, 7 * 64 + 20, 128, 128, seed=20 + G, s0_std=0.3, cp_groups=G))


@pytest.mark.parametrize("B,H,T,G", [(2, 3, 9 * 64 + 5, 5), (1, 5, 5 * 64 + 1, 6), (3, 1, 2 * 64, 2), (2, 7, 1500, 0)])
def test_context_parallel_128_row_transitions(B, H, T, G):
    # dk = dv = 128: the transitions run as 128-row tiles. Unit counts
    # B H (G - 1) off the block map's groups of 8; one chunk per group (T =
    # 5 x 64 + 1 in 6 groups: the last group holds one token); two groups;
    # the automatic count (3 groups of 8 chunks here)
    assert_close(*run_dense(B, H, T, 128, 128, seed=40 + G, s0_std=0.3, cp_groups=G))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_context_parallel_shapes(dk, dv):
    assert_close(*run_dense(2, 1, 5 * 64 + 1, dk, dv, seed=30, s0_std=0.3, cp_groups=3))


def test_context_parallel_fp32():
    assert_close(*run_dense(1, 1, 6 * 64, 64, 64, dtype="f32", seed=31, s0_std=0.3, cp_groups=3))


def test_context_parallel_matches_serial_closely():
    q, k, v, beta, S0 = make_inputs(1, 2, 1024, 128, 128, seed=32, s0_std=0.2)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    o1, s1 = deltanet_fwd(*d, S0.to(DEV), cp_groups=1)
    o4, s4 = deltanet_fwd(*d, S0.to(DEV), cp_groups=4)
    torch.cuda.synchronize()
    assert rel_err(f64(o4), f64(o1)) < 2e-2 and rel_err(f64(s4), f64(s1)) < 2e-2


@pytest.mark.parametrize("order", ["natural", "longest_first"])
def test_varlen(order):
    lengths = [0, 1, 63, 64, 65, 300, 130, 7]
    print(f"[case] varlen {lengths} order={order}", flush=True)
    q, k, v, beta, cu, S0 = make_varlen_inputs(lengths, 3, 128, 128, seed=40, s0_std=0.3)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    cud = cu.to(DEV)
    so = longest_first_order(cud) if order == "longest_first" else None
    o, Sf = deltanet_fwd_varlen(*d, cud, S0.to(DEV), seq_order=so)
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), cu.numpy(), f64(S0))
    assert_close(f64(o), f64(Sf), ro, rs, torch.bfloat16)


def test_varlen_fp32_no_s0():
    lengths = [70, 5, 128]
    q, k, v, beta, cu, _ = make_varlen_inputs(lengths, 2, 64, 128, dtype="f32", seed=41)
    d = [x.to(DEV) for x in (q, k, v, beta)]
    o, Sf = deltanet_fwd_varlen(*d, cu.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd_varlen(f64(q), f64(k), f64(v), f64(beta), cu.numpy())
    assert_close(f64(o), f64(Sf), ro, rs, torch.float32)
