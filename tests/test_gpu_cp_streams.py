"""Stream ordering of the context-parallel forward that uses a second stream.

At dk = dv = 128 with three or more groups, deltanet_fwd and
deltanet_gated_fwd fork part of the call onto a second stream of the library
and join it back. These tests check, on the GPU, that the call stays ordered
on the caller's stream: inputs written on that stream just before the call
are the ones the forked work reads, outputs read on that stream just after
the call are complete, and calls from two host threads on two streams at
once (the fork and join events are shared, under a lock) give the results of
the same calls made one at a time.
"""

import threading

import pytest
import torch

import chunkwise_delta_rule_amd as dn
from chunkwise_delta_rule_amd.synth import make_gates, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, H, T, D = 1, 16, 16384, 128


def inputs(seed, gated):
    q, k, v, beta, S0 = make_inputs(B, H, T, D, D, seed=seed, device=DEV, s0_std=0.1)
    g = make_gates((B, T, H), seed=seed, device=DEV) if gated else None
    return q, k, v, beta, g, S0


def fwd(x, o, Sf, ws):
    q, k, v, beta, g, S0 = x
    if g is not None:
        return dn.deltanet_gated_fwd(q, k, v, beta, g, S0, o=o, S_final=Sf, cp_groups=0, workspace=ws)
    return dn.deltanet_fwd(q, k, v, beta, S0, o=o, S_final=Sf, cp_groups=0, workspace=ws)


def buffers():
    ws = torch.empty(dn.deltanet_workspace_bytes(B, H, T, D, D, 64, 0), dtype=torch.uint8, device=DEV)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=DEV)
    Sf = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    return o, Sf, ws


@pytest.mark.parametrize("gated", [False, True])
def test_inputs_written_just_before_and_outputs_read_just_after(gated):
    G = dn.deltanet_pick_cp_groups(B, H, T, D, D)
    print(f"[case] stream ordering gated={gated} B={B} H={H} T={T} ({G} groups)", flush=True)
    assert G >= 3
    x = inputs(31, gated)
    o, Sf, ws = buffers()
    fwd(x, o, Sf, ws)
    torch.cuda.synchronize()
    o_ref, s_ref = o.clone(), Sf.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # the call's inputs hold other values until a copy on s, enqueued just
    # before the call, restores them; its outputs are copied on s just after
    q, k, v, beta, g, S0 = x
    live = [t.clone() for t in (q, k, v, beta)]
    with torch.cuda.stream(s):
        for t in live:
            t.fill_(0.5)
        torch.cuda._sleep(2_000_000)  # keeps s busy, so a fork that does not wait for it reads 0.5s
        for t, src in zip(live, (q, k, v, beta)):
            t.copy_(src)
        o.fill_(float("nan"))
        Sf.fill_(float("nan"))
        fwd((live[0], live[1], live[2], live[3], g, S0), o, Sf, ws)
        o_after, s_after = o.clone(), Sf.clone()
    torch.cuda.synchronize()
    same = torch.equal(o_after, o_ref) and torch.equal(s_after, s_ref)
    print(f"  outputs on the caller's stream equal the reference call: {same}", flush=True)
    assert same


@pytest.mark.parametrize("gated", [False, True])
def test_two_host_threads_on_two_streams(gated):
    print(f"[case] two host threads gated={gated} B={B} H={H} T={T}", flush=True)
    xs = [inputs(41 + i, gated) for i in range(2)]
    bufs = [buffers() for _ in range(2)]
    refs = []
    for x, (o, Sf, ws) in zip(xs, bufs):
        fwd(x, o, Sf, ws)
        torch.cuda.synchronize()
        refs.append((o.clone(), Sf.clone()))
    streams = [torch.cuda.Stream() for _ in range(2)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    errors = []
    results = [[] for _ in range(2)]

    def worker(i):
        try:
            torch.cuda.set_device(0)
            o, Sf, ws = bufs[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(4):
                    o.fill_(float("nan"))
                    Sf.fill_(float("nan"))
                    fwd(xs[i], o, Sf, ws)
                    results[i].append((o.clone(), Sf.clone()))
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 4
        ok = all(torch.equal(a, refs[i][0]) and torch.equal(b, refs[i][1]) for a, b in results[i])
        print(f"  thread {i}: 4 calls equal to its one-at-a-time call: {ok}", flush=True)
        assert ok
