"""fp64 CPU oracle for the DeltaNet chunkwise-parallel forward pass.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or link anything in this
package. The HIP library never uses it, and it shares no code, header, table
or constant with the HIP library: the two meet only in the seeded input
generators (``chunkwise_delta_rule_amd.synth``), which hold none of the
method's arithmetic.

Sources (page titles as published; "p3" below is "Linear Attention, Visualized"
by Haoran Zhang, "p1" is "Context Parallelism for DeltaNet" by yywangcs):

* ``deltanet_fwd`` / ``deltanet_fwd_varlen`` -- the definition: the
  token-serial recurrence of p3 "DeltaNet" > "Recurrent form", in fp64, in C
  (``deltanet_oracle.c``), OpenMP over independent (sequence, head) units.
* ``chunked_fwd`` -- p3 "DeltaNet" > "Chunkwise algorithm" > "Complete
  per-chunk algorithm", with the triangular system solved by forward
  substitution row by row (p3 "Solving for U").
* ``full_sequence_fwd`` -- p3 "The triangular correction system" and
  "Parallel output": U = (I + BL)^-1 BV, O = (QK^T . M) U  (zero initial state).
* ``householder_states`` / ``exact_states`` -- the state as explicit products
  of generalized Householder transitions, p3 "One chunk as an affine
  recurrence" (A = I - beta k k^T, X = beta k^T v), in fp64 and in exact
  rationals.
* ``chunk_factors`` -- T, W, U of one chunk (p3 "Compact the transition
  product with WY", "Compact the local writes").
* ``cp_group_transition`` / ``cp_compose`` -- the affine map of a group of
  chunks and its composition (p3 "One chunk as an affine recurrence"; p1
  sections 2-3, context parallelism).
* ``gated_deltanet_fwd`` / ``gated_deltanet_fwd_varlen`` -- the Gated
  DeltaNet definition: p3 "Gated DeltaNet (GDN)" token recurrence, in C
  (the decay a_t = exp(g_t) multiplies the previous state before the
  correction); ``gated_chunked_fwd`` -- that section's "Complete per-chunk
  algorithm"; ``householder_states``, ``exact_states`` and
  ``cp_group_transition`` take the decays as an optional argument.
* ``kda_fwd`` -- Kimi Delta Attention token by token (p3 "Kimi Delta
  Attention (KDA)": decay per key channel, then the delta rule), in C;
  ``kda_chunked_fwd`` -- that section's complete per-chunk algorithm.
* ``deltanet_bwd`` -- the backward pass: reverse mode of the token-serial
  recurrence in fp64 (C), with the states recomputed from checkpoints.
* ``gdp_fwd`` -- Gated Delta Product token by token with its substeps (p3
  "Gated Delta Product (GDP)"); ``gdp_virtual_sequence`` -- the mapping of p3
  "GDP as GDN over a virtual sequence".

Convention (p1 section 2): the state S is dv x dk and acts on column vectors:
S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t. The
formulas of p3, written for a dk x dv state acting on row vectors, map onto it
by transposing S.

Layouts: q, k [B, T, H, dk]; v, o [B, T, H, dv]; beta, g [B, T, H];
S0, S_final [B, H, dv, dk]. Every function takes and returns float64 numpy
arrays (exact_states works on ``fractions.Fraction``).

Pins: every function here is checked in ``tests/test_oracle.py`` against
closed forms, hand-derived values of the pages' worked examples
(``tests/golden/``), exact rational brute force, invariants and agreement
between the independent forms above, and against planted mistakes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "deltanet_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_deltanet.so")
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", src, "-o", out, "-lm"]
        subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH):
    """Load (building if needed) the C oracle library."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if path == _LIB_PATH:
        override = os.environ.get("DELTANET_ORACLE_LIB")
        if override:
            # a separately built copy of the same source (the sanitizer test's build)
            lib = ctypes.CDLL(override)
            _declare(lib)
            _lib = lib
            return lib
        build()
    lib = ctypes.CDLL(path)
    _declare(lib)
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _declare(lib):
    """Argument and result types of the C oracle's exports."""
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_deltanet_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_deltanet_fwd.restype = ctypes.c_int
    lib.oracle_deltanet_fwd_varlen.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                               ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int]
    lib.oracle_deltanet_fwd_varlen.restype = ctypes.c_int
    lib.oracle_gated_deltanet_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
    lib.oracle_gated_deltanet_fwd.restype = ctypes.c_int
    lib.oracle_gated_deltanet_fwd_varlen.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                                     ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     ctypes.c_int]
    lib.oracle_gated_deltanet_fwd_varlen.restype = ctypes.c_int
    lib.oracle_deltanet_bwd.argtypes = [dp] * 12 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                    ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_deltanet_bwd.restype = ctypes.c_int
    lib.oracle_gated_deltanet_bwd.argtypes = [dp] * 14 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                          ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_gated_deltanet_bwd.restype = ctypes.c_int
    lib.oracle_kda_fwd.argtypes = [dp] * 8 + [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
    lib.oracle_kda_fwd.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return load().oracle_max_threads()


# ---------------------------------------------------------------------------
# The definition: token-serial recurrence (C, fp64)
# ---------------------------------------------------------------------------

def deltanet_fwd(q, k, v, beta, S0=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 forward. Returns (o [B,T,H,dv], S_final [B,H,dv,dk]).

    p3 "DeltaNet" > "Recurrent form" (transposed state, p1 section 2).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape and v.shape[:3] == (B, T, H) and beta.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    o = np.empty((B, T, H, dv))
    Sf = np.empty((B, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_deltanet_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(o),
                                 _ptr(Sf), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_deltanet_fwd failed with {rc}")
    return o, Sf


def deltanet_fwd_varlen(q, k, v, beta, cu_seqlens, S0=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 forward over packed sequences.

    q, k: [T, H, dk] (or [1, T, H, dk]); v: [T, H, dv]; beta: [T, H];
    cu_seqlens: [N+1] non-decreasing token offsets; S0: [N, H, dv, dk] or None.
    Returns (o [T, H, dv], S_final [N, H, dv, dk]). The state restarts at each
    sequence start.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    if k.ndim == 4:
        q, k, v, beta = q[0], k[0], v[0], beta[0]
    T, H, dk = k.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    S0 = None if S0 is None else _f64(S0)
    o = np.empty((T, H, dv))
    Sf = np.empty((N, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_deltanet_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0),
                                        _ptr(o), _ptr(Sf),
                                        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                        N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_deltanet_fwd_varlen failed with {rc}")
    return o, Sf


def gated_deltanet_fwd(q, k, v, beta, g, S0=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 Gated DeltaNet forward. Returns (o, S_final).

    p3 "Gated DeltaNet (GDN)", token recurrence (transposed state):
    S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t,
    with a_t = exp(g_t); g has the layout of beta, [B, T, H].
    """
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape and v.shape[:3] == (B, T, H)
    assert beta.shape == (B, T, H) and g.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    o = np.empty((B, T, H, dv))
    Sf = np.empty((B, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_gated_deltanet_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0),
                                       _ptr(o), _ptr(Sf), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gated_deltanet_fwd failed with {rc}")
    return o, Sf


def gated_deltanet_fwd_varlen(q, k, v, beta, g, cu_seqlens, S0=None, nthreads: int = 0,
                              lib=None):
    """Token-serial fp64 Gated DeltaNet over packed sequences (g: [T, H])."""
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    if k.ndim == 4:
        q, k, v, beta, g = q[0], k[0], v[0], beta[0], g[0]
    T, H, dk = k.shape
    dv = v.shape[-1]
    assert g.shape == (T, H)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    S0 = None if S0 is None else _f64(S0)
    o = np.empty((T, H, dv))
    Sf = np.empty((N, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_gated_deltanet_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
                                              _ptr(S0), _ptr(o), _ptr(Sf),
                                              cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                              N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gated_deltanet_fwd_varlen failed with {rc}")
    return o, Sf


def kda_fwd(q, k, v, beta, g, S0=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 Kimi Delta Attention (KDA) forward.

    p3 "Kimi Delta Attention (KDA)" (transposed state): the state decays per
    key channel, S <- S Diag(exp(g_t)), then the delta-rule correction
    applies; g: [B,T,H,dk]. Returns (o [B,T,H,dv], S_final [B,H,dv,dk]).
    """
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert g.shape == k.shape and beta.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    o = np.empty((B, T, H, dv))
    Sf = np.empty((B, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(o), _ptr(Sf),
                            B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_kda_fwd failed with {rc}")
    return o, Sf


def kda_chunked_unit(q, k, v, beta, a, S, C):
    """One unit of KDA, chunk size C, in the page's order and notation.

    p3 "Kimi Delta Attention (KDA)" > "Complete per-chunk algorithm" (state
    transposed): per chunk, with lambda[i:j] the elementwise product of the
    decay vectors a_i .. a_j (ones when i > j),
        <-q_l = lambda[1:l] * q_l, <-k_l = lambda[1:l] * k_l, ->k_l = lambda[l+1:C] * k_l,
        A[l, m] = q_l . (lambda[m+1:l] * k_m) for m <= l,
        L[l, m] = k_l . (lambda[m+1:l] * k_m) for m < l,
        (I + B L) T = B,  U = T V,  <-W = T <-K,  Z = U - <-W S^T,
        O = <-Q S^T + A Z,  S <- S Diag(lambda[1:C]) + Z^T ->K.
    a: [L, dk] decays (not logarithms).
    """
    Ltot, dk = k.shape
    o = np.zeros((Ltot, v.shape[1]))
    S = np.array(S, dtype=np.float64, copy=True)
    for c0 in range(0, Ltot, C):
        Kr, Qr, Vr, br, ar = k[c0:c0 + C], q[c0:c0 + C], v[c0:c0 + C], beta[c0:c0 + C], a[c0:c0 + C]
        n = Kr.shape[0]

        def lam(i, j):  # 1-based inclusive elementwise product a_i ... a_j
            return np.prod(ar[i - 1:j], axis=0) if i <= j else np.ones(dk)

        Qb = np.stack([lam(1, l) * Qr[l - 1] for l in range(1, n + 1)])
        Kb = np.stack([lam(1, l) * Kr[l - 1] for l in range(1, n + 1)])
        Kf = np.stack([lam(l + 1, n) * Kr[l - 1] for l in range(1, n + 1)])
        Am = np.zeros((n, n))
        Lm = np.zeros((n, n))
        for l in range(1, n + 1):
            for m in range(1, l + 1):
                wk = lam(m + 1, l) * Kr[m - 1]
                Am[l - 1, m - 1] = Qr[l - 1] @ wk
                if m < l:
                    Lm[l - 1, m - 1] = Kr[l - 1] @ wk
        T = forward_substitution_T(Lm, br)
        U = T @ Vr
        Wb = T @ Kb
        Z = U - Wb @ S.T
        o[c0:c0 + C] = Qb @ S.T + Am @ Z
        S = S * lam(1, n)[None, :] + Z.T @ Kf
    return o, S


def kda_chunked_fwd(q, k, v, beta, g, S0=None, chunk: int = 64):
    """Chunked fp64 KDA over [B,T,H,*] inputs (g: [B,T,H,dk] log decays)."""
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else _f64(S0)[b, h]
            o[b, :, h], Sf[b, h] = kda_chunked_unit(q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h],
                                                    np.exp(g[b, :, h]), S, chunk)
    return o, Sf


def deltanet_bwd(q, k, v, beta, dO, S0=None, dS_final=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 backward of DeltaNet (reverse mode of the recurrence).

    Upstream gradients dO [B,T,H,dv] of o and dS_final [B,H,dv,dk] of the final
    state (None: zero). Returns (dq, dk, dv, dbeta, dS0). The pages give no
    backward pass; this is the chain rule on p3 DeltaNet > "Recurrent form"
    (transposed state), written out in ``deltanet_oracle.c``.
    """
    q, k, v, beta, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(dO)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S0 = None if S0 is None else _f64(S0)
    dS_final = None if dS_final is None else _f64(dS_final)
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    db = np.empty_like(beta)
    dS0 = np.empty((B, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_deltanet_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S0), _ptr(dO),
                                 _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dS0),
                                 B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_deltanet_bwd failed with {rc}")
    return dq, dkk, dvv, db, dS0


def gated_deltanet_bwd(q, k, v, beta, g, dO, S0=None, dS_final=None, nthreads: int = 0, lib=None):
    """Token-serial fp64 backward of Gated DeltaNet (reverse mode of the gated recurrence).

    Inputs as ``gated_deltanet_fwd`` (g [B,T,H]: log decays) plus the upstream
    gradients dO [B,T,H,dv] and dS_final [B,H,dv,dk] (None: zero). Returns
    (dq, dk, dv, dbeta, dg, dS0). The pages give no backward pass; this is the
    chain rule on p3 "Gated DeltaNet (GDN)" (transposed state), written out in
    ``deltanet_oracle.c``.
    """
    q, k, v, beta, g, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g), _f64(dO)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert g.shape == beta.shape
    S0 = None if S0 is None else _f64(S0)
    dS_final = None if dS_final is None else _f64(dS_final)
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    db, dg = np.empty_like(beta), np.empty_like(g)
    dS0 = np.empty((B, H, dv, dk))
    lib = lib or load()
    rc = lib.oracle_gated_deltanet_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(S0), _ptr(dO),
                                       _ptr(dS_final), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(db), _ptr(dg),
                                       _ptr(dS0), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gated_deltanet_bwd failed with {rc}")
    return dq, dkk, dvv, db, dg, dS0


def gdp_bwd(q, k, v, beta, g, n_h, dO, S0=None, dS_final=None, lib=None):
    """Gated Delta Product backward, fp64: the reverse mode of the gated
    recurrence over the virtual sequence that p3 "GDP as GDN over a virtual
    sequence" defines (n_h substeps per real token; the decay sits on the first
    substep, the query and the output on the last).

    Shapes as ``gdp_fwd`` plus dO [B,T,H,dv] and dS_final [B,H,dv,dk] (None:
    zero). Returns (dq [B,T,H,dk], dk [B,T,n_h,H,dk], dv [B,T,n_h,H,dv],
    dbeta [B,T,n_h,H], dg [B,T,H], dS0).
    """
    q, k, v, beta, g, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g), _f64(dO)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    TV = T * n_h
    qv = np.zeros((B, T, n_h, H, dk))
    qv[:, :, n_h - 1] = q
    gv = np.zeros((B, T, n_h, H))
    gv[:, :, 0] = g
    dOv = np.zeros((B, T, n_h, H, dv))
    dOv[:, :, n_h - 1] = dO
    flat = lambda x: x.reshape((B, TV) + x.shape[3:])
    dqv, dkv, dvv, dbv, dgv, dS0 = gated_deltanet_bwd(flat(qv), flat(k), flat(v), flat(beta), flat(gv), flat(dOv),
                                                      S0, dS_final, lib=lib)
    unflat = lambda x: x.reshape((B, T, n_h) + x.shape[2:])
    return (unflat(dqv)[:, :, n_h - 1], unflat(dkv), unflat(dvv), unflat(dbv), unflat(dgv)[:, :, 0], dS0)


def gdp_fwd(q, k, v, beta, g, n_h, S0=None):
    """Gated Delta Product forward, fp64, token by token (numpy; small cases).

    p3 "Gated Delta Product (GDP)": for each real token t, the previous state
    decays once, S_{t,0} = a_t S_{t-1} (a_t = exp(g_t)); then n_h generalized
    Householder substeps follow in order, S_{t,j} = S_{t,j-1}(I - b_{t,j}
    k_{t,j} k_{t,j}^T) + b_{t,j} v_{t,j} k_{t,j}^T (state transposed, p1
    section 2); the query reads the state after the last substep,
    o_t = S_{t,n_h} q_t.

    q: [B,T,H,dk]; k: [B,T,n_h,H,dk]; v: [B,T,n_h,H,dv]; beta: [B,T,n_h,H];
    g: [B,T,H]; S0: [B,H,dv,dk] or None. Returns (o [B,T,H,dv], S_final).
    """
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, n_h, H, dk) and v.shape == (B, T, n_h, H, dv)
    assert beta.shape == (B, T, n_h, H) and g.shape == (B, T, H)
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else _f64(S0)[b, h].copy()
            for t in range(T):
                S = np.exp(g[b, t, h]) * S
                for j in range(n_h):
                    kk, vv, bb = k[b, t, j, h], v[b, t, j, h], beta[b, t, j, h]
                    S = S - bb * np.outer(S @ kk, kk) + bb * np.outer(vv, kk)
                o[b, t, h] = S @ q[b, t, h]
            Sf[b, h] = S
    return o, Sf


def gdp_virtual_sequence(q, k, v, beta, g, n_h):
    """The virtual sequence of p3 "GDP as GDN over a virtual sequence".

    Real token t and substep j become virtual step m = n_h t + j (0-based):
    k, v, beta move over unchanged; the decay sits on the first substep
    (g = g_t for j = 0, else 0, i.e. a = 1); the query sits on the last
    (q_t for j = n_h - 1, else zero). Returns q, k, v, beta, g of shapes
    [B, T n_h, H, *].
    """
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    qv = np.zeros((B, T, n_h, H, dk))
    qv[:, :, n_h - 1] = q
    gv = np.zeros((B, T, n_h, H))
    gv[:, :, 0] = g
    Tv = T * n_h
    return (qv.reshape(B, Tv, H, dk), k.reshape(B, Tv, H, dk), v.reshape(B, Tv, H, dv),
            beta.reshape(B, Tv, H), gv.reshape(B, Tv, H))


# ---------------------------------------------------------------------------
# Chunked form (numpy, fp64): p3 "Complete per-chunk algorithm"
# ---------------------------------------------------------------------------

def forward_substitution_T(Lr, b):
    """Solve (I + diag(b) Lr) T = diag(b) for T, one row at a time.

    p3 "Solving for U": A = I + BL is unit lower triangular, so row i of the
    solution needs only rows j < i. Row i: T_i = b_i e_i - b_i sum_{j<i} Lr[i,j] T_j.
    """
    n = Lr.shape[0]
    T = np.zeros((n, n))
    for i in range(n):
        row = np.zeros(n)
        row[i] = b[i]
        if i:
            row -= b[i] * (Lr[i, :i] @ T[:i])
        T[i] = row
    return T


def chunk_factors(Kr, Vr, br):
    """T, W, U of one chunk (p3 "Complete per-chunk algorithm", first four lines).

    L = (K K^T) . M^-  (strictly lower), (I + B L) T = B, W = T K, U = T V.
    """
    Lr = np.tril(Kr @ Kr.T, -1)
    T = forward_substitution_T(Lr, br)
    return T, T @ Kr, T @ Vr


def chunked_unit(q, k, v, beta, S, C):
    """One (sequence, head) unit, chunk size C; the last chunk may be partial.

    q, k [L, dk]; v [L, dv]; beta [L]; S [dv, dk] (initial state).
    Per chunk (p3's formulas with the state transposed):
        Z = U - W S^T;  O = Q S^T + ((Q K^T) . M_c) Z;  S <- S + Z^T K.
    """
    L = k.shape[0]
    o = np.zeros((L, v.shape[1]))
    S = np.array(S, dtype=np.float64, copy=True)
    for c0 in range(0, L, C):
        Kr, Qr, Vr, br = k[c0:c0 + C], q[c0:c0 + C], v[c0:c0 + C], beta[c0:c0 + C]
        _, W, U = chunk_factors(Kr, Vr, br)
        Z = U - W @ S.T
        o[c0:c0 + C] = Qr @ S.T + np.tril(Qr @ Kr.T) @ Z
        S = S + Z.T @ Kr
    return o, S


def chunked_fwd(q, k, v, beta, S0=None, chunk: int = 64):
    """Chunked fp64 forward over [B,T,H,*] inputs. Returns (o, S_final)."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else _f64(S0)[b, h]
            o[b, :, h], Sf[b, h] = chunked_unit(q[b, :, h], k[b, :, h], v[b, :, h],
                                                beta[b, :, h], S, chunk)
    return o, Sf


def gated_chunked_unit(q, k, v, beta, a, S, C):
    """One unit of Gated DeltaNet, chunk size C, the last chunk may be partial.

    p3 "Gated DeltaNet (GDN)" > "Complete per-chunk algorithm", in the page's
    order and notation, with the state transposed. Within a chunk (1-based
    positions l, i):
        lambda[i:j] = a_i a_{i+1} ... a_j  (1 when i > j)
        Gamma[l, i] = lambda[i+1:l] for i <= l, else 0
        <-q_l = lambda[1:l] q_l,  <-k_l = lambda[1:l] k_l,  ->k_l = lambda[l+1:C] k_l
        L = (K K^T . Gamma) strictly lower,  (I + B L) T = B
        U = T V,  <-W = T <-K,  Z = U - <-W S^T
        O = <-Q S^T + (Q K^T . Gamma) Z,  S <- lambda[1:C] S + Z^T ->K
    a: [L] decays (not logarithms). C of a partial last chunk is its length.
    """
    Ltot = k.shape[0]
    o = np.zeros((Ltot, v.shape[1]))
    S = np.array(S, dtype=np.float64, copy=True)
    for c0 in range(0, Ltot, C):
        Kr, Qr, Vr, br, ar = k[c0:c0 + C], q[c0:c0 + C], v[c0:c0 + C], beta[c0:c0 + C], a[c0:c0 + C]
        n = Kr.shape[0]

        def lam(i, j):  # 1-based inclusive product a_i ... a_j
            return float(np.prod(ar[i - 1:j])) if i <= j else 1.0

        Gam = np.zeros((n, n))
        for l in range(1, n + 1):
            for i in range(1, l + 1):
                Gam[l - 1, i - 1] = lam(i + 1, l)
        left = np.array([lam(1, l) for l in range(1, n + 1)])
        right = np.array([lam(l + 1, n) for l in range(1, n + 1)])
        Lr = np.tril(Kr @ Kr.T * Gam, -1)
        T = forward_substitution_T(Lr, br)
        U = T @ Vr
        W_left = T @ (left[:, None] * Kr)
        Z = U - W_left @ S.T
        o[c0:c0 + C] = (left[:, None] * Qr) @ S.T + (Qr @ Kr.T * Gam) @ Z
        S = lam(1, n) * S + Z.T @ (right[:, None] * Kr)
    return o, S


def gated_chunked_fwd(q, k, v, beta, g, S0=None, chunk: int = 64):
    """Chunked fp64 Gated DeltaNet over [B,T,H,*] inputs (g = log a). Returns (o, S_final)."""
    q, k, v, beta, g = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else _f64(S0)[b, h]
            o[b, :, h], Sf[b, h] = gated_chunked_unit(q[b, :, h], k[b, :, h], v[b, :, h],
                                                      beta[b, :, h], np.exp(g[b, :, h]), S, chunk)
    return o, Sf


# ---------------------------------------------------------------------------
# Full-sequence triangular system (zero initial state)
# ---------------------------------------------------------------------------

def full_sequence_unit(q, k, v, beta):
    """p3 "The triangular correction system" + "Parallel output", one unit.

    L = (K K^T) . M^-, (I + B L) U = B V (solved by a library triangular solve),
    O = ((Q K^T) . M) U, and the final state S^T = K^T U  (S = U^T K).
    """
    from scipy.linalg import solve_triangular
    n = k.shape[0]
    Lf = np.tril(k @ k.T, -1)
    A = np.eye(n) + beta[:, None] * Lf
    U = solve_triangular(A, beta[:, None] * v, lower=True, unit_diagonal=True)
    O = np.tril(q @ k.T) @ U
    return O, U.T @ k


def full_sequence_fwd(q, k, v, beta):
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            o[b, :, h], Sf[b, h] = full_sequence_unit(q[b, :, h], k[b, :, h], v[b, :, h],
                                                      beta[b, :, h])
    return o, Sf


# ---------------------------------------------------------------------------
# Explicit transition products (brute force)
# ---------------------------------------------------------------------------

def householder_states(k, v, beta, S0, a=None):
    """All states S_1..S_L of one unit from explicit d x d transition products.

    p3 "One chunk as an affine recurrence": each token applies the affine map
    S -> S A_t + X_t with A_t = I - beta_t k_t k_t^T and X_t = beta_t v_t k_t^T
    (state transposed). Unrolled:
        S_t = S0 A_1 ... A_t + sum_{i<=t} X_i A_{i+1} ... A_t.
    With decays a (p3 "Gated DeltaNet (GDN)"), A_t = a_t (I - beta_t k_t k_t^T).
    Each S_t is rebuilt from scratch from these products (O(t^2) matrix
    products per state), so no state is carried from one t to the next.
    """
    L, dk = k.shape
    av = np.ones(L) if a is None else np.asarray(a, dtype=np.float64)
    A = [av[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(L)]
    X = [beta[t] * np.outer(v[t], k[t]) for t in range(L)]
    states = []
    for t in range(L):
        P = np.eye(dk)
        for s in range(t + 1):
            P = P @ A[s]
        St = S0 @ P
        for i in range(t + 1):
            Pi = np.eye(dk)
            for s in range(i + 1, t + 1):
                Pi = Pi @ A[s]
            St = St + X[i] @ Pi
        states.append(St)
    return states


def householder_unit(q, k, v, beta, S0, a=None):
    """(o, S_final) of one unit from ``householder_states``; o_t = S_t q_t."""
    states = householder_states(k, v, beta, S0, a)
    o = np.stack([states[t] @ q[t] for t in range(len(states))]) if states else \
        np.zeros((0, v.shape[1]))
    return o, (states[-1] if states else np.array(S0, dtype=np.float64))


def _fmat(rows, cols, val=0):
    return [[Fraction(val) for _ in range(cols)] for _ in range(rows)]


def _fmatmul(A, Bm):
    n, m, p = len(A), len(Bm), len(Bm[0])
    return [[sum((A[i][j] * Bm[j][c] for j in range(m)), Fraction(0)) for c in range(p)]
            for i in range(n)]


def _fadd(A, Bm):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, Bm)]


def exact_states(k, v, beta, S0, a=None):
    """``householder_states`` in exact rational arithmetic (fractions.Fraction).

    k: L lists of dk Fractions; v: L lists of dv; beta: L Fractions;
    S0: dv x dk nested lists; a: L Fractions (decays) or None.
    Returns the list of exact states S_1..S_L.
    """
    L, dk = len(k), len(k[0])
    av = [Fraction(1)] * L if a is None else list(a)
    dv = len(v[0])
    A, X = [], []
    for t in range(L):
        At = _fmat(dk, dk)
        Xt = _fmat(dv, dk)
        for i in range(dk):
            for j in range(dk):
                At[i][j] = av[t] * ((Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j])
        for i in range(dv):
            for j in range(dk):
                Xt[i][j] = beta[t] * v[t][i] * k[t][j]
        A.append(At)
        X.append(Xt)
    ident = [[Fraction(1) if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
    states = []
    for t in range(L):
        P = ident
        for s in range(t + 1):
            P = _fmatmul(P, A[s])
        St = _fmatmul(S0, P)
        for i in range(t + 1):
            Pi = ident
            for s in range(i + 1, t + 1):
                Pi = _fmatmul(Pi, A[s])
            St = _fadd(St, _fmatmul(X[i], Pi))
        states.append(St)
    return states


# ---------------------------------------------------------------------------
# Context parallelism: affine group transitions and their composition
# ---------------------------------------------------------------------------

def cp_group_transition(k, v, beta, a=None):
    """Affine map of a token range of one unit: S_end = S_start P + Q.

    P = A_1 A_2 ... A_L (ordered products of the transitions, dk x dk) and
    Q = sum_i X_i A_{i+1} ... A_L (the state reached from a zero start, dv x dk).
    Both are built as explicit d x d matrix products, composing the per-token
    affine maps (A_t, X_t) one after another: (P, Q) <- (P A_t, Q A_t + X_t)
    (p3 "One chunk as an affine recurrence"; p1 section 3 splits the chunk
    chain into groups that are processed independently). With decays a,
    A_t = a_t (I - beta_t k_t k_t^T) (p3 "Gated DeltaNet (GDN)").
    """
    L, dk = k.shape
    dv = v.shape[1]
    av = np.ones(L) if a is None else np.asarray(a, dtype=np.float64)
    P = np.eye(dk)
    Q = np.zeros((dv, dk))
    for t in range(L):
        At = av[t] * (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
        P = P @ At
        Q = Q @ At + beta[t] * np.outer(v[t], k[t])
    return P, Q


def cp_compose(S0, Ps, Qs):
    """Boundary states of consecutive groups: S_{g+1} = S_g P_g + Q_g.

    Returns the list [S_0, S_1, ..., S_G] (S_0 = S0 is the start of group 0).
    """
    out = [np.array(S0, dtype=np.float64)]
    for P, Q in zip(Ps, Qs):
        out.append(out[-1] @ P + Q)
    return out
