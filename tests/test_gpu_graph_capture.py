"""The context-parallel forward captured into a HIP graph and replayed.

At dk = dv = 128 with three or more groups the forward runs group 0 beside
the transitions of the other groups on a second stream of the library; while
the caller's stream is being captured it runs the same launches one after
another on that stream instead. The captured call is replayed several times,
with eager work (the outputs overwritten with NaN) and a synchronisation
between replays, and every replay must equal the eager call bit for bit (the
same kernels on the same inputs), and the eager call must match the oracle
on sampled heads to the bf16 bar of the other parity tests.
"""

import pytest
import torch

import oracle
import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs
from helpers import f64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("gated", [False, True])
def test_cp_forward_graph_replays_match_eager(gated):
    B, H, T, d = 1, 16, 16384, 128
    G = dn.deltanet_pick_cp_groups(B, H, T, d, d)
    print(f"[case] graph capture gated={gated} B={B} H={H} T={T} cp_groups=0 ({G} groups)", flush=True)
    assert G >= 3
    q, k, v, beta, S0 = make_inputs(B, H, T, d, d, seed=91, device=DEV, s0_std=0.1)
    g = make_gates((B, T, H), seed=91, device=DEV) if gated else None
    ws = torch.empty(dn.deltanet_workspace_bytes(B, H, T, d, d, 64, 0), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(v)
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)

    def call():
        if gated:
            return dn.deltanet_gated_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf, cp_groups=0, workspace=ws)
        return dn.deltanet_fwd(q, k, v, beta, S0, o=o, S_final=Sf, cp_groups=0, workspace=ws)

    call()  # eager, with the second stream
    torch.cuda.synchronize()
    o_ref, s_ref = o.clone(), Sf.clone()
    heads = [0, 7, 15]
    sl = lambda x: x[:, :, heads]
    if gated:
        ro, rs = oracle.gated_deltanet_fwd(f64(sl(q)), f64(sl(k)), f64(sl(v)), f64(sl(beta)), f64(sl(g)),
                                           f64(S0[:, heads]))
    else:
        ro, rs = oracle.deltanet_fwd(f64(sl(q)), f64(sl(k)), f64(sl(v)), f64(sl(beta)), f64(S0[:, heads]))
    eo, es = rel_err(f64(sl(o_ref)), ro), rel_err(f64(s_ref[:, heads]), rs)
    print(f"  eager vs oracle (heads {heads}): o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        o.fill_(float("nan"))
        Sf.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(Sf, s_ref)
        print(f"  replay {r}: bitwise equal to the eager call: {same}", flush=True)
        assert same
    # the eager path still works after a capture
    call()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(Sf, s_ref)
