"""TEST INFRASTRUCTURE ONLY: the CPU oracle for the KDA forward prefill.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It shares no code with the GPU library and never imports
it. Everything here is fp64 on the host, written for a reader to check by eye.

Sources (the pages):
  [P1] "feat(kda/sm90): FlashKDA prefill port + intracard-CP prefill", cuLA
       pull request #103 -- commit summary (K1 prepares decayed q/k, beta and
       the WY inverse; K2 runs the inter-chunk recurrence; CHUNK=16, D=128,
       forward only; intracard CP: K1 once, pre_scan, merge, segment-K2,
       bit-identical to serial) and description (FLA-compatible API, varlen,
       initial/final state).
  [P3] "fix(cake_kda): support non-aligned recurrent prefill head counts",
       FlashInfer pull request #4351 -- description, correctness section
       (bf16 output plus the complete final state, atol = rtol = 1e-2).

Functions
  recurrent    per-token recurrence, numpy (the definition; small cases)
  recurrent_c  the same recurrence in plain C with OpenMP (kda_oracle.c)
  dense        one sequence and head as a single dense block: the WY form
               with C = T, pairwise decays taken directly (independent pin)
  chunked      the chunked WY algebra with CHUNK=16, returning the K1
               quantities per chunk (decayed q/k, WY-transformed keys and
               values, masked q-k Gram, chunk decay) and the K2 results
  decode_step  one token per sequence, the state advanced by one step, in
               the matrix form (I - beta k k^T) Diag(exp g) S + beta k v^T
  gva_expand   grouped value heads: the q/k heads each value head reads

Every function takes fp64-convertible arrays (numpy, or torch tensors of any
float dtype; bf16/fp32 values upcast exactly) in the packed token-major
layout q, k, g: [Tt, H, dk]; v: [Tt, H, dv]; beta: [Tt, H];
states [N, H, dk, dv] (rows are key channels, because o_t = S_t^T q_t).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_C_SRC = os.path.join(_HERE, "kda_oracle.c")
_C_LIB = os.path.join(_HERE, "libkda_oracle.so")


def to_f64(x):
    """Upcast a numpy array or torch tensor (any float dtype) to fp64 numpy."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor, possibly bf16 or on a device
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _cu(cu_seqlens, Tt):
    if cu_seqlens is None:
        return np.array([0, Tt], dtype=np.int64)
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().to("cpu").numpy()
    return np.asarray(cu_seqlens, dtype=np.int64)


# ---------------------------------------------------------------------------
# The definition: per-token recurrence (numpy)
# ---------------------------------------------------------------------------
def recurrent(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0):
    """Per-token KDA recurrence in fp64: the definition.

    The pages name the method and its chunked two-kernel form ([P1] commit
    summary) but print no equation for it; this is the published Kimi Delta
    Attention rule (a gated delta rule with per-key-channel decay), in the
    orientation that tests/golden/hand_two_tokens.txt pins by hand.

    For each sequence and head, token by token:
      S <- Diag(exp g_t) S;  e = v_t - S^T k_t;  S <- S + beta_t k_t e^T;
      o_t = scale * S^T q_t.
    Returns (o [Tt,H,dv], final_state [N,H,dk,dv]).
    """
    q, k, v, g, beta = map(to_f64, (q, k, v, g, beta))
    Tt, H, dk = k.shape
    dv = v.shape[-1]
    cu = _cu(cu_seqlens, Tt)
    n = len(cu) - 1
    s0 = to_f64(initial_state)
    o = np.zeros((Tt, H, dv))
    sT = np.zeros((n, H, dk, dv))
    for i in range(n):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else s0[i, h].copy()
            for t in range(cu[i], cu[i + 1]):
                S = np.exp(g[t, h])[:, None] * S
                e = v[t, h] - S.T @ k[t, h]
                S = S + beta[t, h] * np.outer(k[t, h], e)
                o[t, h] = scale * (S.T @ q[t, h])
            sT[i, h] = S
    return o, sT


# ---------------------------------------------------------------------------
# The same recurrence in plain C (fast enough for full-size samples)
# ---------------------------------------------------------------------------
def build_c(force=False):
    """Compile kda_oracle.c into oracle/libkda_oracle.so with gcc -O2 -fopenmp."""
    if not force and os.path.exists(_C_LIB) and os.path.getmtime(_C_LIB) >= os.path.getmtime(_C_SRC):
        return _C_LIB
    tmp = _C_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _C_SRC, "-lm"])
    os.replace(tmp, _C_LIB)
    return _C_LIB


_c_handle = None


def _c():
    global _c_handle
    if _c_handle is None:
        lib = ctypes.CDLL(build_c())
        P = ctypes.c_void_p
        lib.kda_oracle_recurrent.argtypes = [
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            P, P, P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_int32, ctypes.c_int32]
        lib.kda_oracle_recurrent.restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _c_handle = lib
    return _c_handle


def c_max_threads():
    return _c().kda_oracle_max_threads()


def recurrent_c(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0,
                col_block=32, n_threads=0, heads=None):
    """The per-token recurrence through kda_oracle.c (same definition as
    `recurrent`, OpenMP over (sequence, head, value-column block)).

    heads: optional list of head indices to evaluate (the other heads' outputs
    are left zero); used to time a bounded sample of a large workload.
    """
    q, k, v, g, beta = map(to_f64, (q, k, v, g, beta))
    s0 = to_f64(initial_state)
    if heads is not None:
        heads = list(heads)
        q, k, v, g, beta = (x[:, heads] for x in (q, k, v, g, beta))
        if s0 is not None:
            s0 = s0[:, heads]
    Tt, H, dk = k.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(_cu(cu_seqlens, Tt), dtype=np.int32)
    n = len(cu) - 1
    q, k, v, g, beta = (np.ascontiguousarray(x) for x in (q, k, v, g, beta))
    if s0 is not None:
        s0 = np.ascontiguousarray(s0)
    o = np.zeros((Tt, H, dv))
    sT = np.zeros((n, H, dk, dv))
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a is not None else None
    rc = _c().kda_oracle_recurrent(Tt, H, dk, dv, n, ptr(cu), ptr(q), ptr(k), ptr(v), ptr(g),
                                   ptr(beta), float(scale), ptr(s0), ptr(o), ptr(sT),
                                   int(col_block), int(n_threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrent failed with code %d" % rc)
    return o, sT


# ---------------------------------------------------------------------------
# Dense single-block form (independent formulation, for pinning)
# ---------------------------------------------------------------------------
def _forward_substitute(L, B):
    """Solve (I + L) X = B for strictly lower-triangular L, row by row."""
    X = np.zeros_like(B)
    for r in range(B.shape[0]):
        X[r] = B[r] - L[r, :r] @ X[:r]
    return X


def dense(q, k, v, g, beta, s0=None, scale=1.0):
    """One sequence, one head, as a single block of all T tokens.

    Inputs q, k, g [T, dk]; v [T, dv]; beta [T]; s0 [dk, dv] or None.
    With G_r the cumulative log-decay through token r (per key channel),
    the rescaled state P_r = Diag(exp G_r)^-1 S_r obeys
    P_r = P_{r-1} + (k_r exp(-G_r)) u_r^T with
    u_r = beta_r (v_r - P_{r-1}^T (k_r exp(G_r))). Stacking the rows gives
    (I + L) U = diag(beta) (V - (K exp G) S0), L = strict-lower(diag(beta) A),
    A[r,i] = sum_d k_rd k_id exp(G_rd - G_id); the outputs are
    O = (Q exp G) S0 + tril(B) U with B[r,i] = sum_d q_rd k_id exp(G_rd - G_id)
    and S_T = Diag(exp G_T) S0 + (K exp(G_T - G))^T U. The pairwise decay
    factors exp(G_r - G_i) are formed directly (no factorisation).
    Returns (o [T, dv], S_T [dk, dv]).
    """
    q, k, v, g, beta = map(to_f64, (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[-1]
    S0 = np.zeros((dk, dv)) if s0 is None else to_f64(s0)
    if T == 0:
        return np.zeros((0, dv)), S0.copy()
    G = np.cumsum(g, axis=0)
    D = np.exp(G[:, None, :] - G[None, :, :])            # D[r, i, d] = exp(G_rd - G_id)
    A = np.einsum("rd,id,rid->ri", k, k, D)
    B = np.einsum("rd,id,rid->ri", q, k, D)
    L = np.tril(beta[:, None] * A, -1)
    U = _forward_substitute(L, beta[:, None] * (v - (k * np.exp(G)) @ S0))
    o = (q * np.exp(G)) @ S0 + np.tril(B) @ U
    ST = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1][None, :] - G)).T @ U
    return scale * o, ST


# ---------------------------------------------------------------------------
# Chunked WY form (CHUNK = 16): K1 quantities and K2 recurrence
# ---------------------------------------------------------------------------
def chunk_k1(q, k, v, g, beta):
    """K1 for one chunk of n <= C rows of one head ([P1] commit summary:
    decayed q/k, beta and the WY inverse).

    Inputs q, k, g [n, dk]; v [n, dv]; beta [n]. Returns a dict:
      G    in-chunk cumulative log-decay [n, dk]
      Qt   q * exp(G)                    (decayed queries)
      Kt   k * exp(G_C - G)              (keys decayed to the chunk end)
      A_kk strictly-lower k-k Gram with pairwise decay, A_qk lower (incl.
           diagonal) q-k Gram with pairwise decay
      Tinv (I + strict-lower(diag(beta) A_kk))^-1  (the WY inverse)
      W    Tinv diag(beta) (k * exp(G))
      U    Tinv diag(beta) v                        (U-tilde)
      gC   exp(G_C), G_C the cumulative decay at the chunk's last row.
    """
    n, dk = k.shape
    G = np.cumsum(g, axis=0)
    GC = G[-1]
    D = np.exp(G[:, None, :] - G[None, :, :])
    A_kk = np.tril(np.einsum("rd,id,rid->ri", k, k, D), -1)
    A_qk = np.tril(np.einsum("rd,id,rid->ri", q, k, D))
    L = beta[:, None] * A_kk
    Tinv = _forward_substitute(L, np.eye(n))
    return dict(
        G=G, Qt=q * np.exp(G), Kt=k * np.exp(GC[None, :] - G), A_kk=A_kk, A_qk=A_qk,
        Tinv=Tinv, W=Tinv @ (beta[:, None] * (k * np.exp(G))), U=Tinv @ (beta[:, None] * v),
        gC=np.exp(GC))


def chunk_k2(S, k1):
    """K2 for one chunk, from the chunk-start state S [dk, dv]:
    U = U~ - W S;  O = Qt S + A_qk U;  S_next = Diag(gC) S + Kt^T U."""
    U = k1["U"] - k1["W"] @ S
    O = k1["Qt"] @ S + k1["A_qk"] @ U
    S_next = k1["gC"][:, None] * S + k1["Kt"].T @ U
    return O, S_next


def chunked(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0, chunk=16,
            intermediates=False):
    """Chunked prefill in fp64: every sequence cut into chunks of `chunk` rows
    (the last may be shorter), K1 per chunk, then K2 chunk by chunk.

    Returns (o, final_state) or, with intermediates=True,
    (o, final_state, records) where records[(seq, chunk_index, head)] is the
    K1 dict of that chunk (tail chunks keep their true row count).
    """
    q, k, v, g, beta = map(to_f64, (q, k, v, g, beta))
    Tt, H, dk = k.shape
    dv = v.shape[-1]
    cu = _cu(cu_seqlens, Tt)
    n = len(cu) - 1
    s0 = to_f64(initial_state)
    o = np.zeros((Tt, H, dv))
    sT = np.zeros((n, H, dk, dv))
    recs = {}
    for i in range(n):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else s0[i, h].copy()
            for c, t0 in enumerate(range(cu[i], cu[i + 1], chunk)):
                t1 = min(t0 + chunk, cu[i + 1])
                k1 = chunk_k1(q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], g[t0:t1, h], beta[t0:t1, h])
                O, S = chunk_k2(S, k1)
                o[t0:t1, h] = scale * O
                if intermediates:
                    recs[(i, c, h)] = k1
            sT[i, h] = S
    if intermediates:
        return o, sT, recs
    return o, sT


def segment_summary(k1_list, dk, dv):
    """Affine summary of a run of chunks (the CP pre_scan quantities of [P1]'s
    commit summary): the state map S_end = M S_start + B, with B the end state
    from S_start = 0 and M the end state from S_start = I with U~ := 0."""
    B = np.zeros((dk, dv))
    M = np.eye(dk)
    for k1 in k1_list:
        _, B = chunk_k2(B, k1)
        M = k1["gC"][:, None] * M - k1["Kt"].T @ (k1["W"] @ M)
    return M, B


# ---------------------------------------------------------------------------
# Decode: one new token per sequence, the state advanced by one step
# ---------------------------------------------------------------------------
def decode_step(q, k, v, g, beta, state, scale=1.0):
    """One decode step for a batch of N sequences, each receiving one token.

    "feat(cake_kda): share recurrent prefill kernels across SM100 family"
    (FlashInfer pull request #4313, its AOT registration notes) keeps a KDA
    decode entry beside the prefill; the step is the recurrence of [P1]'s
    commit summary for a single token, written here in its matrix form:
      S' = (I - beta k k^T) Diag(exp g) S + beta k v^T,   o = scale S'^T q.
    Inputs q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H]; state [N, H, dk, dv]
    (rows are key channels). Returns (o [N, H, dv], new_state); the input
    state is not modified.
    """
    q, k, v, g, beta, S = map(to_f64, (q, k, v, g, beta, state))
    N, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    S_new = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            kk = k[n, h]
            P = np.eye(dk) - beta[n, h] * np.outer(kk, kk)
            S1 = P @ (np.diag(np.exp(g[n, h])) @ S[n, h]) + beta[n, h] * np.outer(kk, v[n, h])
            S_new[n, h] = S1
            o[n, h] = scale * (S1.T @ q[n, h])
    return o, S_new


# ---------------------------------------------------------------------------
# Grouped value heads (GVA): fewer q/k heads than value heads
# ---------------------------------------------------------------------------
def gva_expand(q, k, H):
    """q, k with Hk heads -> the [.., H, dk] q, k that the H value heads read.

    [P1]'s reviewer notes restrict the prefill to num_kv_heads ==
    num_qk_heads and name grouped value heads (GVA) as a follow-up. Read
    here as the grouped layout: H = G * Hk value heads, value head h (its v,
    g, beta, state and output) reads q/k head floor(h / G), so each q/k head
    serves G consecutive value heads. Every other function then runs
    unchanged on the expanded q, k.
    """
    q, k = to_f64(q), to_f64(k)
    Hk = k.shape[-2]
    if H % Hk:
        raise ValueError("value heads %d not a multiple of q/k heads %d" % (H, Hk))
    G = H // Hk
    return np.repeat(q, G, axis=-2), np.repeat(k, G, axis=-2)
