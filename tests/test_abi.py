"""C-ABI checks that need no GPU: exports, status strings, workspace sizing and
argument validation (every rejected call returns before anything touches the
device)."""

import ctypes
import os
import re

import pytest

import chunkwise_delta_rule_amd as dn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltanet.h")

DN_OK, DN_ERR_INVALID, DN_ERR_UNSUPPORTED, DN_ERR_WORKSPACE, DN_ERR_HIP = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(deltanet_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dn.load_library()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"deltanet_fwd", "deltanet_fwd_varlen", "deltanet_gated_fwd",
                          "deltanet_gated_fwd_varlen", "deltanet_gdp_fwd", "deltanet_decode_step",
                          "deltanet_kda_fwd", "deltanet_kda_fwd_varlen", "deltanet_kda_decode_step",
                          "deltanet_bwd", "deltanet_bwd_varlen", "deltanet_bwd_varlen_workspace_bytes",
                          "deltanet_workspace_bytes",
                          "deltanet_pick_cp_groups", "deltanet_status_string"}
    raw = ctypes.CDLL(dn.library_path())
    for n in names:
        assert hasattr(raw, n), f"{n} declared in deltanet.h but not exported"


def test_status_strings(lib):
    for code in (DN_OK, DN_ERR_INVALID, DN_ERR_UNSUPPORTED, DN_ERR_WORKSPACE, DN_ERR_HIP):
        s = dn.deltanet_status_string(code)
        assert s and s != "unknown status"
    assert dn.deltanet_status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    assert dn.deltanet_workspace_bytes(8, 16, 4096, 128, 128, 64, 1) == 0
    # G = 4 groups over 64 chunks: per (b,h,g) P (dk^2) + Q and S (dv*dk each), fp32
    assert dn.deltanet_workspace_bytes(2, 3, 4096, 128, 64, 64, 4) == 2 * 3 * 4 * (
        128 * 128 + 2 * 64 * 128) * 4
    # group count is clamped to the chunk count (3 chunks here)
    assert dn.deltanet_workspace_bytes(1, 1, 150, 64, 64, 64, 10) == 3 * (64 * 64 + 2 * 64 * 64) * 4
    # 5 chunks, 3 requested -> 2 chunks per group -> 3 groups
    assert dn.deltanet_workspace_bytes(1, 1, 5 * 64, 64, 64, 64, 3) == 3 * (3 * 64 * 64) * 4
    # 5 chunks, 4 requested -> 2 chunks per group -> 3 groups (no empty group)
    assert dn.deltanet_workspace_bytes(1, 1, 5 * 64, 64, 64, 64, 4) == 3 * (3 * 64 * 64) * 4
    assert dn.deltanet_workspace_bytes(1, 1, 64, 96, 64, 64, 2) == 0  # unsupported dk
    assert dn.deltanet_workspace_bytes(0, 1, 64, 64, 64, 64, 2) == 0  # invalid B


FAKE = 1 << 20  # an aligned non-NULL address; never dereferenced on these paths


def call_fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, o=FAKE, S_final=None, B=1, H=1, T=128,
             dk=64, dv=64, chunk=64, dtype=1, cp_groups=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.deltanet_fwd(vp(a["q"]) if a["q"] else None, vp(a["k"]) if a["k"] else None,
                            vp(a["v"]) if a["v"] else None, vp(a["beta"]) if a["beta"] else None,
                            vp(a["S0"]) if a["S0"] else None, vp(a["o"]) if a["o"] else None,
                            vp(a["S_final"]) if a["S_final"] else None, a["B"], a["H"], a["T"],
                            a["dk"], a["dv"], a["chunk"], a["dtype"], a["cp_groups"],
                            vp(a["ws"]) if a["ws"] else None, a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=32), DN_ERR_UNSUPPORTED),
    (dict(dk=96), DN_ERR_UNSUPPORTED),
    (dict(dv=256), DN_ERR_UNSUPPORTED),
    (dict(dtype=0, dk=128), DN_ERR_UNSUPPORTED),
    (dict(dtype=7), DN_ERR_INVALID),
    (dict(B=0), DN_ERR_INVALID),
    (dict(H=-1), DN_ERR_INVALID),
    (dict(T=-5), DN_ERR_INVALID),
    (dict(dk=0), DN_ERR_INVALID),
    (dict(q=None), DN_ERR_INVALID),
    (dict(beta=None), DN_ERR_INVALID),
    (dict(o=None), DN_ERR_INVALID),
    (dict(k=FAKE + 8), DN_ERR_INVALID),
    (dict(S0=FAKE + 4), DN_ERR_INVALID),
    (dict(S_final=FAKE + 2), DN_ERR_INVALID),
    (dict(beta=FAKE + 1), DN_ERR_INVALID),
    (dict(cp_groups=-1), DN_ERR_INVALID),
    (dict(cp_groups=2), DN_ERR_WORKSPACE),
    (dict(cp_groups=2, ws=FAKE, ws_bytes=16), DN_ERR_WORKSPACE),
    (dict(cp_groups=2, ws=FAKE + 8, ws_bytes=1 << 30), DN_ERR_WORKSPACE),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert call_fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), DN_ERR_INVALID),
    (dict(cu=None), DN_ERR_INVALID),
    (dict(chunk=16), DN_ERR_UNSUPPORTED),
    (dict(order=FAKE + 2), DN_ERR_INVALID),
    (dict(q=None), DN_ERR_INVALID),
    (dict(dtype=0, dk=128), DN_ERR_UNSUPPORTED),
])
def test_varlen_rejects_bad_arguments(lib, kw, status):
    a = dict(q=FAKE, cu=FAKE, order=None, N=2, total_T=100, dk=64, dv=64, chunk=64, dtype=1)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_fwd_varlen(vp(a["q"]) if a["q"] else None, vp(FAKE), vp(FAKE), vp(FAKE),
                                 None, vp(FAKE), None, vp(a["cu"]) if a["cu"] else None,
                                 vp(a["order"]) if a["order"] else None, a["N"], a["total_T"], 2,
                                 a["dk"], a["dv"], a["chunk"], a["dtype"], None)
    assert st == status


def call_gated(lib, g=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, S0=None, o=FAKE, S_final=None, B=1, H=1, T=128,
             dk=64, dv=64, chunk=64, dtype=1, cp_groups=1, ws=None, ws_bytes=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.deltanet_gated_fwd(vp(a["q"]) if a["q"] else None, vp(a["k"]), vp(a["v"]), vp(a["beta"]),
                                  vp(g) if g else None, None, vp(a["o"]) if a["o"] else None, None,
                                  a["B"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"],
                                  a["cp_groups"], vp(a["ws"]) if a["ws"] else None, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), DN_ERR_INVALID),
    (dict(g=FAKE + 2), DN_ERR_INVALID),
    (dict(q=None), DN_ERR_INVALID),
    (dict(chunk=32), DN_ERR_UNSUPPORTED),
    (dict(dtype=0, dk=128), DN_ERR_UNSUPPORTED),
    (dict(cp_groups=2), DN_ERR_WORKSPACE),
])
def test_gated_fwd_rejects_bad_arguments(lib, kw, status):
    assert call_gated(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), DN_ERR_INVALID),
    (dict(g=FAKE + 1), DN_ERR_INVALID),
    (dict(N=0), DN_ERR_INVALID),
    (dict(chunk=16), DN_ERR_UNSUPPORTED),
])
def test_gated_varlen_rejects_bad_arguments(lib, kw, status):
    a = dict(g=FAKE, N=2, chunk=64)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_gated_fwd_varlen(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                       vp(a["g"]) if a["g"] else None, None, vp(FAKE), None,
                                       vp(FAKE), None, a["N"], 100, 2, 64, 64, a["chunk"], 1, None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), DN_ERR_INVALID),
    (dict(dk=96), DN_ERR_UNSUPPORTED),
    (dict(dv=32), DN_ERR_UNSUPPORTED),
    (dict(dtype=3), DN_ERR_INVALID),
    (dict(S=None), DN_ERR_INVALID),
    (dict(S=FAKE + 8), DN_ERR_INVALID),
    (dict(q=FAKE + 2), DN_ERR_INVALID),
    (dict(g=FAKE + 2), DN_ERR_INVALID),
    (dict(o=None), DN_ERR_INVALID),
])
def test_decode_step_rejects_bad_arguments(lib, kw, status):
    a = dict(q=FAKE, g=None, S=FAKE, o=FAKE, B=2, H=2, dk=128, dv=128, dtype=1)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_decode_step(vp(a["q"]), vp(FAKE), vp(FAKE), vp(FAKE), vp(a["g"]) if a["g"] else None,
                                  vp(a["S"]) if a["S"] else None, vp(a["o"]) if a["o"] else None,
                                  a["B"], a["H"], a["dk"], a["dv"], a["dtype"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), DN_ERR_INVALID),
    (dict(N=0), DN_ERR_INVALID),
    (dict(cu=FAKE + 2), DN_ERR_INVALID),
    (dict(dtype=0), DN_ERR_UNSUPPORTED),
    (dict(dk=96), DN_ERR_UNSUPPORTED),
    (dict(ws_bytes=0), DN_ERR_WORKSPACE),
])
def test_bwd_varlen_rejects_bad_arguments(lib, kw, status):
    a = dict(cu=FAKE, N=3, T=200, dk=128, dtype=1, ws_bytes=1 << 40)
    a.update(kw)
    vp = ctypes.c_void_p
    ptrs = [vp(FAKE)] * 12
    st = lib.deltanet_bwd_varlen(*ptrs, vp(a["cu"]) if a["cu"] else None, None, a["N"], a["T"], 2, a["dk"], 128,
                                 64, a["dtype"], vp(FAKE) if a["ws_bytes"] else None, a["ws_bytes"], None)
    if kw.get("ws_bytes", 1) == 0 or status != DN_ERR_WORKSPACE:
        assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(cp=-1), DN_ERR_INVALID),
    (dict(cp=2), DN_ERR_WORKSPACE),        # context parallelism needs a workspace
    (dict(g=None), DN_ERR_INVALID),
    (dict(g=FAKE + 8), DN_ERR_INVALID),
    (dict(dtype=0), DN_ERR_UNSUPPORTED),
])
def test_kda_fwd_rejects_bad_arguments(lib, kw, status):
    a = dict(cp=1, g=FAKE, dtype=1)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_kda_fwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(a["g"]) if a["g"] else None, None,
                              vp(FAKE), None, 1, 2, 4096, 128, 128, 64, a["dtype"], a["cp"], None, 0, None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), DN_ERR_INVALID),        # the decays are required when tokens are present
    (dict(dg=None), DN_ERR_INVALID),       # and so is their gradient
    (dict(g=FAKE + 2), DN_ERR_INVALID),    # fp32, 4-byte aligned
    (dict(B=0), DN_ERR_INVALID),
    (dict(dtype=0), DN_ERR_UNSUPPORTED),
    (dict(dk=96), DN_ERR_UNSUPPORTED),
    (dict(ws_bytes=0), DN_ERR_WORKSPACE),
])
def test_gated_bwd_rejects_bad_arguments(lib, kw, status):
    a = dict(g=FAKE, dg=FAKE, B=2, dk=128, dtype=1, ws_bytes=0)
    a.update(kw)
    vp = ctypes.c_void_p
    opt = lambda x: vp(x) if x else None
    st = lib.deltanet_gated_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), opt(a["g"]), None, vp(FAKE), None,
                                vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), opt(a["dg"]), None, a["B"], 2, 200, a["dk"],
                                128, 64, a["dtype"], None, a["ws_bytes"], None)
    assert st == status


def test_bwd_workspace_sizes(lib):
    # per chunk slot, DeltaNet: the state entering the chunk and the gradient of
    # the state leaving it (bf16 each), then T^T (64 x 64 bf16); gated: the state
    # entering the chunk (bf16), per value tile dP, dT (64 x 64), dQ, dK (64 x dk)
    # (bf16) and 256 floats of decay terms (fp32), then T^T
    for dk, dv in [(128, 128), (64, 64), (64, 128), (128, 64)]:
        plain = 2 * dv * dk * 2 + 64 * 64 * 2
        gated = dv * dk * 2 + (dv // 64) * ((2 * 64 * 64 + 2 * 64 * dk) * 2 + 256 * 4) + 64 * 64 * 2
        slots = 2 * 3 * 4  # B = 2, H = 3, T = 200 -> 4 chunks
        assert lib.deltanet_bwd_workspace_bytes(2, 3, 200, dk, dv, 64) == slots * plain
        assert lib.deltanet_gated_bwd_workspace_bytes(2, 3, 200, dk, dv, 64) == slots * gated
        vslots = (200 // 64 + 3) * 2  # N = 3, total 200 tokens, H = 2; + 4 offsets, padded to 16 bytes
        assert lib.deltanet_bwd_varlen_workspace_bytes(3, 200, 2, dk, dv, 64) == vslots * plain + 16
        assert lib.deltanet_gated_bwd_varlen_workspace_bytes(3, 200, 2, dk, dv, 64) == vslots * gated + 16
    assert lib.deltanet_gated_bwd_workspace_bytes(2, 3, 200, 96, 128, 64) == 0
    assert lib.deltanet_bwd_workspace_bytes(2, 3, 200, 96, 128, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(nh=0), DN_ERR_INVALID),
    (dict(g=None), DN_ERR_INVALID),
    (dict(T=1 << 29, nh=4), DN_ERR_UNSUPPORTED),  # the virtual length must stay under 2^30
    (dict(dtype=0), DN_ERR_UNSUPPORTED),
    (dict(ws_bytes=0), DN_ERR_WORKSPACE),
])
def test_gdp_bwd_rejects_bad_arguments(lib, kw, status):
    a = dict(g=FAKE, nh=2, T=100, dtype=1, ws_bytes=0)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_gdp_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(a["g"]) if a["g"] else None, None,
                              vp(FAKE), None, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, 2, 2, a["T"],
                              a["nh"], 128, 128, 64, a["dtype"], None, a["ws_bytes"], None)
    assert st == status


def test_gdp_bwd_workspace_is_gated_over_the_virtual_length(lib):
    assert (lib.deltanet_gdp_bwd_workspace_bytes(2, 3, 100, 3, 128, 64, 64)
            == lib.deltanet_gated_bwd_workspace_bytes(2, 3, 300, 128, 64, 64))
    assert lib.deltanet_gdp_bwd_workspace_bytes(2, 3, 100, 0, 128, 64, 64) == 0


def test_bwd_varlen_workspace_bound(lib):
    # chunk slots are bounded by total_T / 64 + N per head, whatever the lengths
    one = lib.deltanet_bwd_varlen_workspace_bytes(1, 64, 1, 128, 128, 64)  # 2 slots + the offsets
    slot = (one - 16) // 2
    assert slot == lib.deltanet_bwd_workspace_bytes(1, 1, 64, 128, 128, 64)
    assert lib.deltanet_bwd_varlen_workspace_bytes(3, 200, 2, 128, 128, 64) == (200 // 64 + 3) * 2 * slot + 16
    assert lib.deltanet_bwd_varlen_workspace_bytes(0, 200, 2, 128, 128, 64) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), DN_ERR_INVALID),        # the per-channel decays are required
    (dict(g=FAKE + 8), DN_ERR_INVALID),    # and 16-byte aligned
    (dict(B=0), DN_ERR_INVALID),
    (dict(dk=96), DN_ERR_UNSUPPORTED),
    (dict(S=FAKE + 8), DN_ERR_INVALID),
    (dict(o=None), DN_ERR_INVALID),
])
def test_kda_decode_step_rejects_bad_arguments(lib, kw, status):
    a = dict(g=FAKE, S=FAKE, o=FAKE, B=2, H=2, dk=128, dv=128)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_kda_decode_step(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(a["g"]) if a["g"] else None,
                                      vp(a["S"]) if a["S"] else None, vp(a["o"]) if a["o"] else None,
                                      a["B"], a["H"], a["dk"], a["dv"], 1, None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(nh=0), DN_ERR_INVALID),
    (dict(g=None), DN_ERR_INVALID),
    (dict(T=1 << 28, nh=8), DN_ERR_UNSUPPORTED),
    (dict(chunk=32), DN_ERR_UNSUPPORTED),
    (dict(cp_groups=2), DN_ERR_WORKSPACE),
])
def test_gdp_rejects_bad_arguments(lib, kw, status):
    a = dict(g=FAKE, T=100, nh=2, chunk=64, cp_groups=1)
    a.update(kw)
    vp = ctypes.c_void_p
    st = lib.deltanet_gdp_fwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(a["g"]) if a["g"] else None,
                              None, vp(FAKE), None, 1, 2, a["T"], a["nh"], 64, 64, a["chunk"], 1,
                              a["cp_groups"], None, 0, None)
    assert st == status


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises((ValueError, TypeError)):
        dn.deltanet_fwd(x, x, x, torch.zeros(1, 4, 1))


def test_noalloc_rejects_a_workspace_beyond_its_array(lib):
    # 8 x 16 heads of T = 131072 in 16 groups need 403 MB of workspace, more than
    # the fixed 32 MiB array: refused before anything touches the device
    vp = ctypes.c_void_p
    need = dn.deltanet_workspace_bytes(8, 16, 131072, 128, 128, 64, 16)
    assert need > 32 << 20
    st = lib.deltanet_fwd_noalloc(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), None, 8, 16, 131072,
                                  128, 128, 64, 1, 16, None)
    assert st == DN_ERR_WORKSPACE
    # invalid shapes keep the forward's own status
    st = lib.deltanet_fwd_noalloc(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), None, 1, 1, 128,
                                  96, 128, 64, 1, 1, None)
    assert st == DN_ERR_UNSUPPORTED
    st = lib.deltanet_fwd_noalloc(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), None, 1, 1, 128,
                                  128, 128, 32, 1, 1, None)
    assert st == DN_ERR_UNSUPPORTED


def prototype(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    return [" ".join(p.split()) for p in m.group(1).split(",")]


def test_bwd_cp_workspace_sizes(lib):
    # deltanet_bwd's workspace plus, per (sequence, head, group), P_g^T (dk^2)
    # and two dv x dk matrices, fp32; one group needs nothing more
    for dk, dv in [(128, 128), (64, 128), (128, 64)]:
        serial = dn.deltanet_bwd_workspace_bytes(2, 3, 1000, dk, dv)
        assert dn.deltanet_bwd_cp_workspace_bytes(2, 3, 1000, dk, dv, 64, 1) == serial
        # 16 chunks in 4 groups of 4
        assert dn.deltanet_bwd_cp_workspace_bytes(2, 3, 1000, dk, dv, 64, 4) == serial + 2 * 3 * 4 * (
            dk * dk + 2 * dv * dk) * 4
        G = dn.deltanet_pick_cp_groups(1, 2, 131072, dk, dv, 64)
        assert G > 1
        # at dk = dv = 128 the forward's choice may hold one group more than the
        # backward's (its group 0 runs beside the transitions)
        choices = (G, G - 1) if (dk, dv) == (128, 128) else (G,)
        assert dn.deltanet_bwd_cp_workspace_bytes(1, 2, 131072, dk, dv, 64, 0) in [
            dn.deltanet_bwd_workspace_bytes(1, 2, 131072, dk, dv) + 2 * c * (dk * dk + 2 * dv * dk) * 4
            for c in choices]
        gated = dn.deltanet_gated_bwd_workspace_bytes(2, 3, 1000, dk, dv)
        assert dn.deltanet_gated_bwd_cp_workspace_bytes(2, 3, 1000, dk, dv, 64, 1) == gated
        assert dn.deltanet_gated_bwd_cp_workspace_bytes(2, 3, 1000, dk, dv, 64, 4) == gated + 2 * 3 * 4 * (
            dk * dk + 2 * dv * dk) * 4
    assert lib.deltanet_bwd_cp_workspace_bytes(2, 3, 1000, 128, 128, 64, -1) == 0
    assert lib.deltanet_gated_bwd_cp_workspace_bytes(2, 3, 1000, 128, 128, 64, -1) == 0
    assert lib.deltanet_bwd_cp_workspace_bytes(2, 3, 1000, 96, 128, 64, 2) == 0


def test_boundary_signatures_as_documented():
    # the departures from the proposed boundary that the design notes list
    fwd = prototype("deltanet_fwd")
    assert fwd[:7] == ["const void *q", "const void *k", "const void *v", "const void *beta", "const float *S0",
                       "void *o", "float *S_final"]
    assert "int dtype" in fwd and "int cp_groups" in fwd and "void *workspace" in fwd
    var = prototype("deltanet_fwd_varlen")
    assert "const int32_t *cu_seqlens" in var and "const int32_t *seq_order" in var
    assert not any("workspace" in p for p in var)
    assert "int dtype" in var
    assert not any("dn_dtype_t" in p for name in ("deltanet_fwd", "deltanet_fwd_varlen", "deltanet_gated_fwd")
                   for p in prototype(name))
