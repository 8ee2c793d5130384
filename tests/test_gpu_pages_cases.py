"""The pages' own cases through the HIP path, plus the degenerate key patterns.

* "Linear Attention, Visualized" (Haoran Zhang), DeltaNet > "The triangular
  correction system" and "Compact the transition product with WY": the
  three-token chunk worked by hand in ``tests/golden/three_token_chunk.json``
  (exact fractions). Zero-padded to dk = dv = 64 (zero key, query and value
  channels carry nothing), run through the fp32 and the bf16 kernels, alone
  and placed so that it straddles a chunk boundary behind identity tokens
  (k = 0, beta = 0). Compared with the exact values.
* Same page, DeltaNet > "An intuitive example": the Alice/Bob memory of
  ``tests/golden/alice_bob.json``, written with beta = 1/2, 1 (exact
  replacement) and 1/4. Compared with the exact values.
* beta = 1 with q = k: each token replaces the value stored along its own key
  (same section), so o_t = v_t at every token whatever came before; checked
  against that and against the oracle.
* Repeated keys (a token reusing an earlier key of the same chunk), collinear
  keys (-k, k/2) and keys of non-unit norm, against the oracle.

Bar: max|gpu - reference| / max|reference| <= 1e-4 (fp32 inputs) or 2e-2
(bf16 inputs), o and the final state separately.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from chunkwise_delta_rule_amd import deltanet_fwd
from chunkwise_delta_rule_amd.synth import make_inputs
from helpers import TOL, f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def frac_array(rows):
    return np.array([[float(Fraction(x)) for x in r] for r in rows], dtype=np.float64)


def padded(x, T, d, at=0):
    """Rows of x (t x small d) at tokens at..at+t of a [1, T, 1, d] zero tensor."""
    out = np.zeros((1, T, 1, d))
    out[0, at:at + x.shape[0], 0, :x.shape[1]] = x
    return out


def run(q, k, v, beta, S0, dtype):
    dt = DTYPES[dtype]
    t = lambda x: torch.from_numpy(x).to(dt).to(DEV).contiguous()
    s0 = None if S0 is None else torch.from_numpy(S0).to(torch.float32).to(DEV).contiguous()
    o, Sf = deltanet_fwd(t(q), t(k), t(v), t(beta), s0)
    torch.cuda.synchronize()
    return f64(o), f64(Sf)


def check(name, o, Sf, ro, rs, dtype):
    tol = TOL[DTYPES[dtype]]
    eo, es = rel_err(o, ro), rel_err(Sf, rs)
    print(f"  {name} [{dtype}]: err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("at", [0, 62])
def test_golden_three_token_chunk(dtype, at):
    gold = json.load(open(os.path.join(GOLDEN, "three_token_chunk.json")))
    print(f"[case] three-token chunk at token {at}, {dtype}", flush=True)
    k = frac_array(gold["inputs"]["k"])
    v = frac_array(gold["inputs"]["v"])
    q = frac_array(gold["inputs"]["q"])
    b = np.array([float(Fraction(x)) for x in gold["inputs"]["beta"]])
    d = 64
    T = at + 3
    beta = np.zeros((1, T, 1))
    beta[0, at:at + 3, 0] = b
    o, Sf = run(padded(q, T, d, at), padded(k, T, d, at), padded(v, T, d, at), beta, None, dtype)
    ro = padded(frac_array(gold["expected"]["o"]), T, d, at)[0, :, 0]
    rs = np.zeros((d, d))
    rs[:2, :2] = frac_array(gold["expected"]["S_final"])
    check("three-token chunk", o[0, :, 0], Sf[0, 0], ro, rs, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [0, 1, 2])
def test_golden_alice_bob(dtype, case):
    gold = json.load(open(os.path.join(GOLDEN, "alice_bob.json")))
    c = gold["cases"][case]
    print(f"[case] Alice/Bob beta={c['beta']} {dtype}", flush=True)
    d = 64
    S0 = np.zeros((1, 1, d, d))
    S0[0, 0, :3, :2] = frac_array(gold["S0"])
    e2 = np.array([[0.0, 1.0]])
    office = np.array([[0.0, 0.0, 1.0]])
    beta = np.full((1, 1, 1), float(Fraction(c["beta"])))
    o, Sf = run(padded(e2, 1, d), padded(e2, 1, d), padded(office, 1, d), beta, S0, dtype)
    ro = np.zeros(d)
    ro[:3] = [float(Fraction(x)) for x in c["o_bob"]]
    rs = np.zeros((d, d))
    rs[:3, :2] = frac_array(c["S_final"])
    check("Alice/Bob", o[0, 0, 0], Sf[0, 0], ro, rs, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_one_replaces_the_value_under_its_key(dtype):
    # q = k and beta = 1: every read returns the value just written
    B, H, T = 2, 3, 200
    dk = dv = 64 if dtype == "f32" else 128
    print(f"[case] beta = 1, q = k, {dtype} B={B} H={H} T={T} d={dk}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, dtype=dtype, seed=61, s0_std=0.5)
    beta = torch.ones_like(beta)
    q = k.clone()
    args = [x.to(DEV) for x in (q, k, v, beta)]
    o, Sf = deltanet_fwd(*args, S0.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    check("beta = 1 vs oracle", f64(o), f64(Sf), ro, rs, dtype)
    # the replacement property itself: exact for unit keys, so the bound is
    # the tolerance plus the keys' rounding from unit norm
    n2 = (f64(k) ** 2).sum(-1)
    slack = float(np.abs(1 - n2).max()) * 4
    e = rel_err(f64(o), f64(v))
    print(f"  o vs v: {e:.3e} (bound {TOL[DTYPES[dtype]] + slack:.3e})", flush=True)
    assert e <= TOL[DTYPES[dtype]] + slack


def keys_with_structure(B, T, H, d, seed):
    """Unit keys in which, inside every chunk of 64, token 5 repeats token 2,
    token 9 is minus token 2, token 20 is token 7 halved, token 33 repeats
    token 32 and token 63 repeats token 0 of the same chunk."""
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, T, H, d), generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    for c0 in range(0, T, 64):
        for dst, src, s in ((5, 2, 1.0), (9, 2, -1.0), (20, 7, 0.5), (33, 32, 1.0), (63, 0, 1.0)):
            if c0 + dst < T:
                k[:, c0 + dst] = s * k[:, c0 + src]
    return k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeated_and_collinear_keys_in_a_chunk(dtype):
    B, H, T = 2, 2, 64 * 3 + 37
    dk = dv = 64 if dtype == "f32" else 128
    print(f"[case] repeated/collinear keys, {dtype} T={T}", flush=True)
    q, _, v, beta, S0 = make_inputs(B, H, T, dk, dv, dtype=dtype, seed=62, s0_std=0.3)
    k = keys_with_structure(B, T, H, dk, 63).to(DTYPES[dtype])
    # a beta = 1 token repeating an earlier key of its chunk, too
    beta[:, 33] = 1
    args = [x.to(DEV) for x in (q, k, v, beta)]
    o, Sf = deltanet_fwd(*args, S0.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    check("repeated/collinear keys", f64(o), f64(Sf), ro, rs, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_non_unit_keys_and_queries(dtype):
    # norms in [0.25, 1.4]; with beta <= 1 the factor 1 - beta |k|^2 stays in
    # [-0.96, 1], so the recurrence stays bounded
    B, H, T = 2, 2, 64 * 2 + 50
    dk = dv = 64 if dtype == "f32" else 128
    print(f"[case] non-unit keys, {dtype} T={T}", flush=True)
    q, k, v, beta, S0 = make_inputs(B, H, T, dk, dv, dtype="f32", seed=64, s0_std=0.3)
    g = torch.Generator().manual_seed(65)
    k = k * (0.25 + 1.15 * torch.rand((B, T, H, 1), generator=g))
    q = q * (0.25 + 2.0 * torch.rand((B, T, H, 1), generator=g))
    dt = DTYPES[dtype]
    q, k, v, beta = (x.to(dt) for x in (q, k, v, beta))
    args = [x.to(DEV) for x in (q, k, v, beta)]
    o, Sf = deltanet_fwd(*args, S0.to(DEV))
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    check("non-unit keys", f64(o), f64(Sf), ro, rs, dtype)


@pytest.mark.parametrize("cp_groups", [2, 3])
def test_beta_one_and_repeated_keys_context_parallel(cp_groups):
    # the same degenerate keys through the context-parallel path
    B, H, T = 1, 2, 64 * 6 + 11
    print(f"[case] repeated keys + beta = 1, cp_groups={cp_groups}", flush=True)
    q, _, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=66, s0_std=0.3)
    k = keys_with_structure(B, T, H, 128, 67).to(torch.bfloat16)
    beta[:, ::7] = 1
    args = [x.to(DEV) for x in (q, k, v, beta)]
    o, Sf = deltanet_fwd(*args, S0.to(DEV), cp_groups=cp_groups)
    torch.cuda.synchronize()
    ro, rs = oracle.deltanet_fwd(f64(q), f64(k), f64(v), f64(beta), f64(S0))
    check(f"cp={cp_groups} degenerate keys", f64(o), f64(Sf), ro, rs, "bf16")
