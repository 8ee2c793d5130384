"""DeltaNet chunkwise-parallel forward pass for AMD MI355X (gfx950).

A thin ctypes binding over the C-ABI of ``include/deltanet.h``
(``libdeltanet.so``, built in-tree by ``python -m chunkwise_delta_rule_amd.build``).
This module only checks and marshals arguments: every step of the forward
pass runs in the library's HIP kernels. PyTorch provides device memory and
the current stream. There is no fallback: if the library is missing or the
tensors are not on a GPU the calls raise.

The method (the state S is dv x dk, read after the write):
    S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
evaluated chunkwise with chunk 64 ("Linear Attention, Visualized", Haoran
Zhang, DeltaNet > "Complete per-chunk algorithm"), optionally with
context parallelism over chunk groups ("Context Parallelism for DeltaNet").
The gated variant (same page, "Gated DeltaNet (GDN)") multiplies the
previous state by a per-token decay a_t = exp(g_t) first:
    S_t = a_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["deltanet_fwd", "deltanet_fwd_noalloc", "deltanet_fwd_varlen", "deltanet_gated_fwd", "deltanet_gated_fwd_varlen",
           "deltanet_gdp_fwd", "deltanet_kda_fwd", "deltanet_kda_fwd_varlen", "deltanet_decode_step", "deltanet_kda_decode_step", "deltanet_bwd", "deltanet_bwd_workspace_bytes",
           "deltanet_bwd_cp_workspace_bytes", "deltanet_gated_bwd_cp_workspace_bytes",
           "deltanet_bwd_varlen", "deltanet_bwd_varlen_workspace_bytes", "deltanet_gated_bwd",
           "deltanet_gated_bwd_workspace_bytes", "deltanet_gated_bwd_varlen",
           "deltanet_gated_bwd_varlen_workspace_bytes", "deltanet_gdp_bwd", "deltanet_gdp_bwd_workspace_bytes",
           "deltanet_workspace_bytes",
           "deltanet_pick_cp_groups", "deltanet_status_string", "longest_first_order",
           "library_path", "load_library", "DeltaNetError", "DN_F32", "DN_BF16"]

DN_F32 = 0
DN_BF16 = 1
_DTYPE_CODE = {torch.float32: DN_F32, torch.bfloat16: DN_BF16}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdeltanet.so"
_lib = None


class DeltaNetError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {deltanet_status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library(path: str | None = None):
    """Load libdeltanet.so and declare its signatures (no GPU call is made)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m chunkwise_delta_rule_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.deltanet_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_fwd.restype = i
    lib.deltanet_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.deltanet_fwd_varlen.restype = i
    lib.deltanet_gated_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gated_fwd.restype = i
    lib.deltanet_gated_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.deltanet_gated_fwd_varlen.restype = i
    lib.deltanet_gdp_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gdp_fwd.restype = i
    lib.deltanet_kda_fwd.argtypes = [vp] * 8 + [i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_kda_fwd.restype = i
    lib.deltanet_kda_fwd_varlen.argtypes = [vp] * 10 + [i, i, i, i, i, i, i, vp]
    lib.deltanet_kda_fwd_varlen.restype = i
    lib.deltanet_bwd.argtypes = [vp] * 12 + [i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_bwd.restype = i
    lib.deltanet_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.deltanet_bwd_workspace_bytes.restype = sz
    lib.deltanet_bwd_cp.argtypes = [vp] * 12 + [i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_bwd_cp.restype = i
    lib.deltanet_bwd_cp_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_bwd_cp_workspace_bytes.restype = sz
    lib.deltanet_bwd_varlen.argtypes = [vp] * 14 + [i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_bwd_varlen.restype = i
    lib.deltanet_bwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.deltanet_bwd_varlen_workspace_bytes.restype = sz
    lib.deltanet_gated_bwd.argtypes = [vp] * 14 + [i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gated_bwd.restype = i
    lib.deltanet_gated_bwd_cp.argtypes = [vp] * 14 + [i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gated_bwd_cp.restype = i
    lib.deltanet_gated_bwd_cp_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_gated_bwd_cp_workspace_bytes.restype = sz
    lib.deltanet_gated_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.deltanet_gated_bwd_workspace_bytes.restype = sz
    lib.deltanet_gated_bwd_varlen.argtypes = [vp] * 16 + [i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gated_bwd_varlen.restype = i
    lib.deltanet_gated_bwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.deltanet_gated_bwd_varlen_workspace_bytes.restype = sz
    lib.deltanet_gdp_bwd.argtypes = [vp] * 14 + [i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.deltanet_gdp_bwd.restype = i
    lib.deltanet_gdp_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_gdp_bwd_workspace_bytes.restype = sz
    lib.deltanet_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.deltanet_decode_step.restype = i
    lib.deltanet_kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.deltanet_kda_decode_step.restype = i
    lib.deltanet_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    lib.deltanet_fwd_noalloc.restype = i
    lib.deltanet_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.deltanet_workspace_bytes.restype = sz
    lib.deltanet_pick_cp_groups.argtypes = [i, i, i, i, i, i]
    lib.deltanet_pick_cp_groups.restype = i
    lib.deltanet_status_string.argtypes = [i]
    lib.deltanet_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def deltanet_status_string(status: int) -> str:
    return load_library().deltanet_status_string(int(status)).decode()


def deltanet_workspace_bytes(B, H, T, dk, dv, chunk=64, cp_groups=1) -> int:
    return int(load_library().deltanet_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups))


def deltanet_pick_cp_groups(B, H, T, dk, dv, chunk=64) -> int:
    st = load_library().deltanet_pick_cp_groups(B, H, T, dk, dv, chunk)
    if st < 0:
        raise DeltaNetError(st, "deltanet_pick_cp_groups")
    return st


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, device, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd(q, k, v, beta, g, S0, chunk, cp_groups, o, S_final, output_final_state, workspace, stream):
    lib = load_library()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, dk]")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(beta, "beta", dt, dev, (B, T, H))
    if g is not None:
        _check(g, "g", torch.float32, dev, (B, T, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, T, H, dv))
    if output_final_state and S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    need = int(lib.deltanet_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        if g is None:
            st = lib.deltanet_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o),
                                  _ptr(S_final), B, H, T, dk, dv, chunk, _DTYPE_CODE[dt], cp_groups,
                                  _ptr(workspace), ws_bytes, _stream_handle(stream))
        else:
            st = lib.deltanet_gated_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0),
                                        _ptr(o), _ptr(S_final), B, H, T, dk, dv, chunk,
                                        _DTYPE_CODE[dt], cp_groups, _ptr(workspace), ws_bytes,
                                        _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_fwd" if g is None else "deltanet_gated_fwd")
    return o, S_final


def deltanet_fwd(q, k, v, beta, S0=None, *, chunk: int = 64, cp_groups: int = 1, o=None,
                 S_final=None, output_final_state: bool = True, workspace=None, stream=None):
    """Forward pass over [B, T, H, d] inputs (C-ABI ``deltanet_fwd``).

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H] (same dtype, fp32 or bf16);
    S0: [B,H,dv,dk] fp32 or None. Returns (o, S_final); S_final is None when
    ``output_final_state`` is False. ``cp_groups``: 1 serial, 0 library's
    choice, G > 1 forced. Preallocated ``o``/``S_final``/``workspace`` are used
    when given (workspace: a uint8 CUDA tensor of at least
    ``deltanet_workspace_bytes`` bytes).
    """
    return _fwd(q, k, v, beta, None, S0, chunk, cp_groups, o, S_final, output_final_state,
                workspace, stream)


def deltanet_fwd_noalloc(q, k, v, beta, S0=None, *, o, S_final=None, chunk: int = 64, cp_groups: int = 1,
                         stream=None):
    """``deltanet_fwd`` through the C-ABI ``deltanet_fwd_noalloc``: the
    context-parallel workspace is the library's fixed per-device array, and
    neither the library nor this wrapper allocates (o, and S_final when
    wanted, are the caller's). Returns (o, S_final)."""
    lib = load_library()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, dk]")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(beta, "beta", dt, dev, (B, T, H))
    _check(o, "o", dt, dev, (B, T, H, dv))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    with torch.cuda.device(dev):
        st = lib.deltanet_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final),
                                      B, H, T, dk, dv, chunk, _DTYPE_CODE[dt], cp_groups, _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_fwd_noalloc")
    return o, S_final


def deltanet_gated_fwd(q, k, v, beta, g, S0=None, *, chunk: int = 64, cp_groups: int = 1, o=None,
                       S_final=None, output_final_state: bool = True, workspace=None, stream=None):
    """Gated DeltaNet forward (C-ABI ``deltanet_gated_fwd``).

    As ``deltanet_fwd``, plus g: [B,T,H] float32, the natural logarithm of
    each token's decay a_t.
    """
    if g is None:
        raise ValueError("g is required")
    return _fwd(q, k, v, beta, g, S0, chunk, cp_groups, o, S_final, output_final_state,
                workspace, stream)


def longest_first_order(cu_seqlens) -> torch.Tensor:
    """Permutation of sequence indices by decreasing length (ties by index).

    Computed on the host (a device ``cu_seqlens`` is copied back, which
    synchronises); returns an int32 tensor on the device of ``cu_seqlens``.
    """
    cu = cu_seqlens.detach().to("cpu", torch.int64)
    lens = cu[1:] - cu[:-1]
    order = sorted(range(lens.numel()), key=lambda n: (-int(lens[n]), n))
    return torch.tensor(order, dtype=torch.int32, device=cu_seqlens.device)


def deltanet_gdp_fwd(q, k, v, beta, g, S0=None, *, chunk: int = 64, cp_groups: int = 1, o=None,
                     S_final=None, output_final_state: bool = True, workspace=None, stream=None):
    """Gated Delta Product forward (C-ABI ``deltanet_gdp_fwd``).

    q: [B,T,H,dk]; k: [B,T,n_h,H,dk]; v: [B,T,n_h,H,dv]; beta: [B,T,n_h,H];
    g: [B,T,H] float32 log decays; S0: [B,H,dv,dk] fp32 or None. Returns
    (o [B,T,H,dv], S_final).
    """
    lib = load_library()
    if k.dim() != 5:
        raise ValueError("k must be [B, T, n_h, H, dk]")
    B, T, nh, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, nh, H, dk))
    _check(v, "v", dt, dev, (B, T, nh, H, dv))
    _check(beta, "beta", dt, dev, (B, T, nh, H))
    _check(g, "g", torch.float32, dev, (B, T, H))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, T, H, dv))
    if output_final_state and S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    need = int(lib.deltanet_workspace_bytes(B, H, T * nh, dk, dv, chunk, cp_groups))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.deltanet_gdp_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                  _ptr(S_final), B, H, T, nh, dk, dv, chunk, _DTYPE_CODE[dt],
                                  cp_groups, _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_gdp_fwd")
    return o, S_final


def _fwd_varlen(q, k, v, beta, g, cu_seqlens, S0, seq_order, chunk, o, S_final,
                output_final_state, stream):
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [T, H, dk]")
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    N = cu_seqlens.numel() - 1
    _check(q, "q", dt, dev, (T, H, dk))
    _check(k, "k", dt, dev, (T, H, dk))
    _check(v, "v", dt, dev, (T, H, dv))
    _check(beta, "beta", dt, dev, (T, H))
    if g is not None:
        _check(g, "g", torch.float32, dev, (T, H))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (N + 1,))
    if seq_order is not None:
        _check(seq_order, "seq_order", torch.int32, dev, (N,))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (N, H, dv, dk))
    if o is None:
        o = torch.empty((T, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (T, H, dv))
    if output_final_state and S_final is None:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (N, H, dv, dk))
    with torch.cuda.device(dev):
        if g is None:
            st = lib.deltanet_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o),
                                         _ptr(S_final), _ptr(cu_seqlens), _ptr(seq_order), N, T, H,
                                         dk, dv, chunk, _DTYPE_CODE[dt], _stream_handle(stream))
        else:
            st = lib.deltanet_gated_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                               _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens),
                                               _ptr(seq_order), N, T, H, dk, dv, chunk,
                                               _DTYPE_CODE[dt], _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_fwd_varlen" if g is None else "deltanet_gated_fwd_varlen")
    return o, S_final


def deltanet_fwd_varlen(q, k, v, beta, cu_seqlens, S0=None, *, seq_order=None, chunk: int = 64,
                        o=None, S_final=None, output_final_state: bool = True, stream=None):
    """Forward pass over packed sequences (C-ABI ``deltanet_fwd_varlen``).

    q, k: [T,H,dk]; v: [T,H,dv]; beta: [T,H]; cu_seqlens: int32 [N+1] on the
    device; S0: [N,H,dv,dk] fp32 or None; seq_order: int32 [N] device
    permutation (scheduling order only) or None.
    """
    return _fwd_varlen(q, k, v, beta, None, cu_seqlens, S0, seq_order, chunk, o, S_final,
                       output_final_state, stream)


def deltanet_gated_fwd_varlen(q, k, v, beta, g, cu_seqlens, S0=None, *, seq_order=None,
                              chunk: int = 64, o=None, S_final=None,
                              output_final_state: bool = True, stream=None):
    """Gated DeltaNet over packed sequences (C-ABI ``deltanet_gated_fwd_varlen``).

    As ``deltanet_fwd_varlen``, plus g: [T,H] float32 log decays.
    """
    if g is None:
        raise ValueError("g is required")
    return _fwd_varlen(q, k, v, beta, g, cu_seqlens, S0, seq_order, chunk, o, S_final,
                       output_final_state, stream)


def deltanet_decode_step(q, k, v, beta, S, g=None, *, o=None, stream=None):
    """One decode step in place (C-ABI ``deltanet_decode_step``).

    q, k: [B,H,dk]; v: [B,H,dv]; beta: [B,H] (same dtype, fp32 or bf16);
    S: [B,H,dv,dk] fp32, updated in place; g: [B,H] fp32 log decays (Gated
    DeltaNet) or None. Returns o [B,H,dv].
    """
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [B, H, dk]")
    B, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _check(q, "q", dt, dev, (B, H, dk))
    _check(k, "k", dt, dev, (B, H, dk))
    _check(v, "v", dt, dev, (B, H, dv))
    _check(beta, "beta", dt, dev, (B, H))
    _check(S, "S", torch.float32, dev, (B, H, dv, dk))
    if g is not None:
        _check(g, "g", torch.float32, dev, (B, H))
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, H, dv))
    with torch.cuda.device(dev):
        st = lib.deltanet_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S),
                                      _ptr(o), B, H, dk, dv, _DTYPE_CODE[dt],
                                      _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_decode_step")
    return o


def deltanet_kda_fwd_varlen(q, k, v, beta, g, cu_seqlens, S0=None, *, seq_order=None, chunk: int = 64,
                            o=None, S_final=None, output_final_state: bool = True, stream=None):
    """Kimi Delta Attention over packed sequences (C-ABI ``deltanet_kda_fwd_varlen``).

    As ``deltanet_fwd_varlen`` (bf16), plus g: [T,H,dk] float32 per-channel
    log decays.
    """
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [T, H, dk]")
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_kda_fwd_varlen takes bfloat16 inputs")
    N = cu_seqlens.numel() - 1
    _check(q, "q", dt, dev, (T, H, dk))
    _check(k, "k", dt, dev, (T, H, dk))
    _check(v, "v", dt, dev, (T, H, dv))
    _check(beta, "beta", dt, dev, (T, H))
    _check(g, "g", torch.float32, dev, (T, H, dk))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (N + 1,))
    if seq_order is not None:
        _check(seq_order, "seq_order", torch.int32, dev, (N,))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (N, H, dv, dk))
    if o is None:
        o = torch.empty((T, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (T, H, dv))
    if output_final_state and S_final is None:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (N, H, dv, dk))
    with torch.cuda.device(dev):
        st = lib.deltanet_kda_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                         _ptr(S_final), _ptr(cu_seqlens), _ptr(seq_order), N, T, H, dk, dv,
                                         chunk, _DTYPE_CODE[dt], _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_kda_fwd_varlen")
    return o, S_final


def deltanet_kda_decode_step(q, k, v, beta, S, g, *, o=None, stream=None):
    """One Kimi Delta Attention decode step in place (C-ABI
    ``deltanet_kda_decode_step``).

    q, k: [B,H,dk]; v: [B,H,dv]; beta: [B,H] (same dtype, fp32 or bf16);
    S: [B,H,dv,dk] fp32, updated in place; g: [B,H,dk] fp32 per-channel log
    decays. Returns o [B,H,dv].
    """
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [B, H, dk]")
    B, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"unsupported dtype {dt}")
    _check(q, "q", dt, dev, (B, H, dk))
    _check(k, "k", dt, dev, (B, H, dk))
    _check(v, "v", dt, dev, (B, H, dv))
    _check(beta, "beta", dt, dev, (B, H))
    _check(S, "S", torch.float32, dev, (B, H, dv, dk))
    _check(g, "g", torch.float32, dev, (B, H, dk))
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, H, dv))
    with torch.cuda.device(dev):
        st = lib.deltanet_kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S),
                                          _ptr(o), B, H, dk, dv, _DTYPE_CODE[dt],
                                          _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_kda_decode_step")
    return o


def deltanet_bwd_workspace_bytes(B, H, T, dk, dv, chunk=64) -> int:
    return int(load_library().deltanet_bwd_workspace_bytes(B, H, T, dk, dv, chunk))


def deltanet_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk=64, cp_groups=0) -> int:
    return int(load_library().deltanet_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups))


def deltanet_gated_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk=64, cp_groups=0) -> int:
    return int(load_library().deltanet_gated_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups))


def deltanet_bwd(q, k, v, beta, dO, S0=None, dS_final=None, *, chunk: int = 64, cp_groups: int = 1,
                 workspace=None, want_dS0: bool = True, stream=None):
    """Backward of ``deltanet_fwd`` (C-ABI ``deltanet_bwd``, bf16 only; with
    ``cp_groups`` other than 1, ``deltanet_bwd_cp``: 0 the library's group
    count, G > 1 forced).

    q, k: [B,T,H,dk]; v, dO: [B,T,H,dv]; beta: [B,T,H] (bf16); S0, dS_final:
    [B,H,dv,dk] fp32 or None. Returns (dq, dk, dv, dbeta, dS0 or None).
    """
    lib = load_library()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, dk]")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_bwd supports bfloat16 inputs only")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(beta, "beta", dt, dev, (B, T, H))
    _check(dO, "dO", dt, dev, (B, T, H, dv))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, dev, (B, H, dv, dk))
    dq, dkk, dvv, db = (torch.empty_like(x) for x in (q, k, v, beta))
    dS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    cp = cp_groups != 1
    need = int(lib.deltanet_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups) if cp
               else lib.deltanet_bwd_workspace_bytes(B, H, T, dk, dv, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        if cp:
            st = lib.deltanet_bwd_cp(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_final),
                                     _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dS0), B, H, T, dk, dv, chunk,
                                     DN_BF16, cp_groups, _ptr(workspace), ws_bytes, _stream_handle(stream))
        else:
            st = lib.deltanet_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_final),
                                  _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dS0), B, H, T, dk, dv, chunk,
                                  DN_BF16, _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_bwd_cp" if cp else "deltanet_bwd")
    return dq, dkk, dvv, db, dS0


def deltanet_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk=64) -> int:
    return int(load_library().deltanet_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk))


def deltanet_bwd_varlen(q, k, v, beta, dO, cu_seqlens, S0=None, dS_final=None, *, seq_order=None,
                        chunk: int = 64, workspace=None, want_dS0: bool = True, stream=None):
    """Backward of ``deltanet_fwd_varlen`` (C-ABI ``deltanet_bwd_varlen``, bf16 only).

    q, k: [T,H,dk]; v, dO: [T,H,dv]; beta: [T,H] (bf16); cu_seqlens: [N+1]
    int32; S0, dS_final: [N,H,dv,dk] fp32 or None. Returns (dq, dk, dv, dbeta,
    dS0 or None).
    """
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [T, H, dk]")
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_bwd_varlen supports bfloat16 inputs only")
    N = cu_seqlens.numel() - 1
    _check(q, "q", dt, dev, (T, H, dk))
    _check(k, "k", dt, dev, (T, H, dk))
    _check(v, "v", dt, dev, (T, H, dv))
    _check(beta, "beta", dt, dev, (T, H))
    _check(dO, "dO", dt, dev, (T, H, dv))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (N + 1,))
    if seq_order is not None:
        _check(seq_order, "seq_order", torch.int32, dev, (N,))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (N, H, dv, dk))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, dev, (N, H, dv, dk))
    dq, dkk, dvv, db = (torch.empty_like(x) for x in (q, k, v, beta))
    dS0 = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    need = int(lib.deltanet_bwd_varlen_workspace_bytes(N, T, H, dk, dv, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.deltanet_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_final),
                                     _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dS0), _ptr(cu_seqlens),
                                     _ptr(seq_order), N, T, H, dk, dv, chunk, DN_BF16, _ptr(workspace), ws_bytes,
                                     _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_bwd_varlen")
    return dq, dkk, dvv, db, dS0


def deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, chunk=64) -> int:
    return int(load_library().deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, chunk))


def deltanet_gated_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk=64) -> int:
    return int(load_library().deltanet_gated_bwd_varlen_workspace_bytes(N, total_T, H, dk, dv, chunk))


def deltanet_gated_bwd(q, k, v, beta, g, dO, S0=None, dS_final=None, *, chunk: int = 64, cp_groups: int = 1,
                       workspace=None, want_dS0: bool = True, stream=None):
    """Backward of ``deltanet_gated_fwd`` (C-ABI ``deltanet_gated_bwd``, bf16 only;
    with ``cp_groups`` other than 1, ``deltanet_gated_bwd_cp``).

    q, k: [B,T,H,dk]; v, dO: [B,T,H,dv]; beta: [B,T,H] (bf16); g: [B,T,H]
    fp32 log decays; S0, dS_final: [B,H,dv,dk] fp32 or None. Returns (dq, dk,
    dv, dbeta, dg, dS0 or None).
    """
    lib = load_library()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, dk]")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_gated_bwd supports bfloat16 inputs only")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(beta, "beta", dt, dev, (B, T, H))
    _check(g, "g", torch.float32, dev, (B, T, H))
    _check(dO, "dO", dt, dev, (B, T, H, dv))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, dev, (B, H, dv, dk))
    dq, dkk, dvv, db = (torch.empty_like(x) for x in (q, k, v, beta))
    dg = torch.empty_like(g)
    dS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    cp = cp_groups != 1
    need = int(lib.deltanet_gated_bwd_cp_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups) if cp
               else lib.deltanet_gated_bwd_workspace_bytes(B, H, T, dk, dv, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        if cp:
            st = lib.deltanet_gated_bwd_cp(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO),
                                           _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg),
                                           _ptr(dS0), B, H, T, dk, dv, chunk, DN_BF16, cp_groups, _ptr(workspace),
                                           ws_bytes, _stream_handle(stream))
        else:
            st = lib.deltanet_gated_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO),
                                        _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg), _ptr(dS0),
                                        B, H, T, dk, dv, chunk, DN_BF16, _ptr(workspace), ws_bytes,
                                        _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_gated_bwd_cp" if cp else "deltanet_gated_bwd")
    return dq, dkk, dvv, db, dg, dS0


def deltanet_gated_bwd_varlen(q, k, v, beta, g, dO, cu_seqlens, S0=None, dS_final=None, *, seq_order=None,
                              chunk: int = 64, workspace=None, want_dS0: bool = True, stream=None):
    """Backward of ``deltanet_gated_fwd_varlen`` (C-ABI ``deltanet_gated_bwd_varlen``, bf16 only).

    q, k: [T,H,dk]; v, dO: [T,H,dv]; beta: [T,H] (bf16); g: [T,H] fp32;
    cu_seqlens: [N+1] int32; S0, dS_final: [N,H,dv,dk] fp32 or None. Returns
    (dq, dk, dv, dbeta, dg, dS0 or None).
    """
    lib = load_library()
    if k.dim() != 3:
        raise ValueError("k must be [T, H, dk]")
    T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_gated_bwd_varlen supports bfloat16 inputs only")
    N = cu_seqlens.numel() - 1
    _check(q, "q", dt, dev, (T, H, dk))
    _check(k, "k", dt, dev, (T, H, dk))
    _check(v, "v", dt, dev, (T, H, dv))
    _check(beta, "beta", dt, dev, (T, H))
    _check(g, "g", torch.float32, dev, (T, H))
    _check(dO, "dO", dt, dev, (T, H, dv))
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev, (N + 1,))
    if seq_order is not None:
        _check(seq_order, "seq_order", torch.int32, dev, (N,))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (N, H, dv, dk))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, dev, (N, H, dv, dk))
    dq, dkk, dvv, db = (torch.empty_like(x) for x in (q, k, v, beta))
    dg = torch.empty_like(g)
    dS0 = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    need = int(lib.deltanet_gated_bwd_varlen_workspace_bytes(N, T, H, dk, dv, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.deltanet_gated_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO),
                                           _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg),
                                           _ptr(dS0), _ptr(cu_seqlens), _ptr(seq_order), N, T, H, dk, dv, chunk,
                                           DN_BF16, _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_gated_bwd_varlen")
    return dq, dkk, dvv, db, dg, dS0


def deltanet_gdp_bwd_workspace_bytes(B, H, T, n_h, dk, dv, chunk=64) -> int:
    return int(load_library().deltanet_gdp_bwd_workspace_bytes(B, H, T, n_h, dk, dv, chunk))


def deltanet_gdp_bwd(q, k, v, beta, g, dO, S0=None, dS_final=None, *, chunk: int = 64, workspace=None,
                     want_dS0: bool = True, stream=None):
    """Backward of ``deltanet_gdp_fwd`` (C-ABI ``deltanet_gdp_bwd``, bf16 only).

    q: [B,T,H,dk]; k: [B,T,n_h,H,dk]; v: [B,T,n_h,H,dv]; beta: [B,T,n_h,H]
    (bf16); g: [B,T,H] fp32; dO: [B,T,H,dv]; S0, dS_final: [B,H,dv,dk] fp32
    or None. Returns (dq, dk, dv, dbeta, dg, dS0 or None) in the layouts of
    the inputs.
    """
    lib = load_library()
    if k.dim() != 5:
        raise ValueError("k must be [B, T, n_h, H, dk]")
    B, T, n_h, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_gdp_bwd supports bfloat16 inputs only")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, n_h, H, dk))
    _check(v, "v", dt, dev, (B, T, n_h, H, dv))
    _check(beta, "beta", dt, dev, (B, T, n_h, H))
    _check(g, "g", torch.float32, dev, (B, T, H))
    _check(dO, "dO", dt, dev, (B, T, H, dv))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if dS_final is not None:
        _check(dS_final, "dS_final", torch.float32, dev, (B, H, dv, dk))
    dq, dkk, dvv, db = (torch.empty_like(x) for x in (q, k, v, beta))
    dg = torch.empty_like(g)
    dS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    need = int(lib.deltanet_gdp_bwd_workspace_bytes(B, H, T, n_h, dk, dv, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.deltanet_gdp_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO),
                                  _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg), _ptr(dS0),
                                  B, H, T, n_h, dk, dv, chunk, DN_BF16, _ptr(workspace), ws_bytes,
                                  _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_gdp_bwd")
    return dq, dkk, dvv, db, dg, dS0


def deltanet_kda_fwd(q, k, v, beta, g, S0=None, *, chunk: int = 64, cp_groups: int = 1, o=None,
                     S_final=None, output_final_state: bool = True, workspace=None, stream=None):
    """Kimi Delta Attention forward (C-ABI ``deltanet_kda_fwd``, bf16 only).

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; g: [B,T,H,dk] float32
    per-channel log decays; S0: [B,H,dv,dk] fp32 or None. ``cp_groups`` as in
    ``deltanet_fwd`` (context parallelism). Returns (o, S_final).
    """
    lib = load_library()
    if k.dim() != 4:
        raise ValueError("k must be [B, T, H, dk]")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    if dt != torch.bfloat16:
        raise TypeError("deltanet_kda_fwd supports bfloat16 inputs only")
    _check(q, "q", dt, dev, (B, T, H, dk))
    _check(k, "k", dt, dev, (B, T, H, dk))
    _check(v, "v", dt, dev, (B, T, H, dv))
    _check(beta, "beta", dt, dev, (B, T, H))
    _check(g, "g", torch.float32, dev, (B, T, H, dk))
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(o, "o", dt, dev, (B, T, H, dv))
    if output_final_state and S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _check(S_final, "S_final", torch.float32, dev, (B, H, dv, dk))
    need = int(lib.deltanet_workspace_bytes(B, H, T, dk, dv, chunk, cp_groups))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.deltanet_kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o),
                                  _ptr(S_final), B, H, T, dk, dv, chunk, DN_BF16, cp_groups, _ptr(workspace),
                                  ws_bytes, _stream_handle(stream))
    if st != 0:
        raise DeltaNetError(st, "deltanet_kda_fwd")
    return o, S_final
