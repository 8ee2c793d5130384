"""deltanet_fwd_noalloc (context-parallel workspace in the library's fixed
per-device array) against deltanet_fwd (caller's workspace) through the C-ABI,
on consecutive calls that reuse the array: the long-context shape with the
library's group count (about 25 MB of the 32 MiB array), then a smaller input
with a forced group count, then a serial call. The same kernels run in the
same plan on the same inputs, so the outputs must agree bit for bit; the
oracle's tolerance (2e-2 relative, bf16) is checked as well."""

import pytest
import torch

import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import make_inputs
from helpers import f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_deltanet_fwd(order):
    cases = [(1, 16, 131072, 0), (2, 3, 1000, 3), (2, 2, 300, 1)]
    for i, (B, H, T, cp) in enumerate(cases):
        G = cp if cp > 0 else dn.deltanet_pick_cp_groups(B, H, T, 128, 128)
        need = dn.deltanet_workspace_bytes(B, H, T, 128, 128, 64, G)
        print(f"[case] noalloc call {i}: B={B} H={H} T={T} cp_groups={cp} (G={G}, scratch {need} B)", flush=True)
        assert need <= 32 << 20
        q, k, v, beta, S0 = make_inputs(B, H, T, 128, 128, seed=70 + i, device=DEV, s0_std=0.1)
        o_ref, s_ref = dn.deltanet_fwd(q, k, v, beta, S0, cp_groups=cp)
        o = torch.full_like(o_ref, float("nan"))
        sf = torch.full_like(s_ref, float("nan"))
        dn.deltanet_fwd_noalloc(q, k, v, beta, S0, o=o, S_final=sf, cp_groups=cp)
        torch.cuda.synchronize()
        eo, es = rel_err(f64(o), f64(o_ref)), rel_err(f64(sf), f64(s_ref))
        print(f"  err vs deltanet_fwd o={eo:.3e} S={es:.3e}; bitwise equal: "
              f"{torch.equal(o, o_ref) and torch.equal(sf, s_ref)}", flush=True)
        assert eo <= 2e-2 and es <= 2e-2
        assert torch.equal(o, o_ref) and torch.equal(sf, s_ref)
