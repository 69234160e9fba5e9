"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin is a closed form, an invariant of the recurrence, an independent
formulation, or a hand-derived example, chosen so that a plausible mistake in
the oracle (order of decay and write, transposed state, dropped beta, wrong
sign, decay on the wrong axis, missing scale, wrong chunk carry) fails at
least one of them; test_planted_mistakes_are_caught checks exactly that.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(7)


def rand_case(lengths, H=2, dk=8, dv=8, s0=True, g_scale=1.0, seed=0):
    r = np.random.default_rng(seed)
    Tt = sum(lengths)
    q = r.standard_normal((Tt, H, dk))
    k = r.standard_normal((Tt, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((Tt, H, dv))
    g = -np.logaddexp(0.0, g_scale * r.standard_normal((Tt, H, dk)))  # -softplus
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((Tt, H))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    S0 = 0.1 * r.standard_normal((len(lengths), H, dk, dv)) if s0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, initial_state=S0)


def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *nums = line.split()
                vals[key] = np.array([float(x) for x in nums])
    return vals


def golden_inputs():
    gv = load_golden("hand_two_tokens.txt")
    sh = lambda a: a.reshape(2, 1, 2)
    return dict(q=sh(gv["q"]), k=sh(gv["k"]), v=sh(gv["v"]), g=sh(gv["g"]),
                beta=gv["beta"].reshape(2, 1), cu_seqlens=[0, 2],
                initial_state=gv["S0"].reshape(1, 1, 2, 2)), gv


IMPLS = {
    "recurrent": lambda c, scale=1.0: ref.recurrent(**c, scale=scale),
    "recurrent_c": lambda c, scale=1.0: ref.recurrent_c(**c, scale=scale),
    "chunked16": lambda c, scale=1.0: ref.chunked(**c, scale=scale),
    "chunked4": lambda c, scale=1.0: ref.chunked(**c, scale=scale, chunk=4),
}


def run_dense(c, scale=1.0):
    """Run the dense single-block form sequence by sequence and head by head."""
    q, k, v, g, beta = (np.asarray(c[x], dtype=np.float64) for x in ("q", "k", "v", "g", "beta"))
    cu = np.asarray(c["cu_seqlens"])
    S0 = c["initial_state"]
    Tt, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((Tt, H, dv))
    sT = np.zeros((len(cu) - 1, H, dk, dv))
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        for h in range(H):
            o[a:b, h], sT[i, h] = ref.dense(q[a:b, h], k[a:b, h], v[a:b, h], g[a:b, h],
                                            beta[a:b, h], None if S0 is None else S0[i, h], scale)
    return o, sT


IMPLS["dense"] = run_dense


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_golden_hand_example(impl):
    c, gv = golden_inputs()
    o, sT = IMPLS[impl](c)
    np.testing.assert_allclose(o.reshape(-1), gv["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sT.reshape(-1), gv["ST"], rtol=0, atol=1e-12)
    o_half, _ = IMPLS[impl](c, scale=0.5)
    np.testing.assert_allclose(o_half.reshape(-1), 0.5 * gv["o"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,dk,dv", [(1, 8, 8), (5, 8, 4), (17, 8, 8), (40, 16, 8), (24, 128, 128)])
def test_dense_matches_recurrent(T, dk, dv):
    c = rand_case([T], H=1, dk=dk, dv=dv, seed=T + dk)
    o1, s1 = ref.recurrent(**c)
    o2, s2 = run_dense(c)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_beta_zero_is_pure_decay(impl):
    """beta = 0: o_t = S0^T (q_t * exp G_t), S_T = Diag(exp G_T) S0, G the
    cumulative decay over the whole sequence."""
    c = rand_case([23, 9], H=2, dk=8, dv=6, seed=3)
    c["beta"] = np.zeros_like(c["beta"])
    o, sT = IMPLS[impl](c)
    cu = c["cu_seqlens"]
    for i in range(2):
        for h in range(2):
            G = np.cumsum(c["g"][cu[i]:cu[i + 1], h], axis=0)
            S0 = c["initial_state"][i, h]
            np.testing.assert_allclose(o[cu[i]:cu[i + 1], h],
                                       (c["q"][cu[i]:cu[i + 1], h] * np.exp(G)) @ S0,
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sT[i, h], np.exp(G[-1])[:, None] * S0, rtol=1e-12, atol=1e-13)
    c["initial_state"] = None
    o, sT = IMPLS[impl](c)
    assert np.all(o == 0) and np.all(sT == 0)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_delta_rule_overwrite(impl):
    """g = 0, beta = 1, |k| = 1: the write makes S_t^T k_t = v_t, so q_t = k_t
    reads back v_t exactly."""
    c = rand_case([19], H=2, dk=8, dv=5, seed=11)
    c["g"] = np.zeros_like(c["g"])
    c["beta"] = np.ones_like(c["beta"])
    c["q"] = c["k"].copy()
    o, _ = IMPLS[impl](c)
    np.testing.assert_allclose(o, c["v"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_orthonormal_keys_replace_rows(impl):
    """g = 0, beta = 1, k_t = e_{pi(t)}: row pi(t) of the state becomes v_t
    (the last write to a row wins); other rows keep S0."""
    dk, dv = 8, 5
    pi = [3, 0, 6, 3, 1, 7, 0]
    c = rand_case([len(pi)], H=1, dk=dk, dv=dv, seed=5)
    c["g"] = np.zeros_like(c["g"])
    c["beta"] = np.ones_like(c["beta"])
    c["k"] = np.zeros_like(c["k"])
    for t, p in enumerate(pi):
        c["k"][t, 0, p] = 1.0
    _, sT = IMPLS[impl](c)
    expect = c["initial_state"][0, 0].copy()
    for t, p in enumerate(pi):
        expect[p] = c["v"][t, 0]
    np.testing.assert_allclose(sT[0, 0], expect, rtol=0, atol=1e-13)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_read_only_state(impl):
    """g = 0, beta = 0: the state never changes, o_t = S0^T q_t."""
    c = rand_case([13], H=2, dk=8, dv=8, seed=2)
    c["g"] = np.zeros_like(c["g"])
    c["beta"] = np.zeros_like(c["beta"])
    o, sT = IMPLS[impl](c)
    np.testing.assert_allclose(sT, c["initial_state"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[:, 0], c["q"][:, 0] @ c["initial_state"][0, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("split", [1, 7, 16, 21])
def test_carry_equivalence(impl, split):
    """run([a; b], S0) == run(b, run(a, S0).final) -- the final state is the
    resume point of a prefill cut at any token."""
    c = rand_case([37], H=2, dk=8, dv=8, seed=split)
    o_all, s_all = IMPLS[impl](c)
    ca = {x: c[x][:split] for x in ("q", "k", "v", "g", "beta")}
    cb = {x: c[x][split:] for x in ("q", "k", "v", "g", "beta")}
    oa, sa = IMPLS[impl](dict(ca, cu_seqlens=[0, split], initial_state=c["initial_state"]))
    ob, sb = IMPLS[impl](dict(cb, cu_seqlens=[0, 37 - split], initial_state=sa))
    np.testing.assert_allclose(np.concatenate([oa, ob]), o_all, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sb, s_all, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_varlen_packing(impl):
    """A packed batch equals its sequences run one by one (incl. empty ones)."""
    lengths = [5, 0, 17, 1, 33]
    c = rand_case(lengths, H=2, dk=8, dv=4, seed=9)
    o, sT = IMPLS[impl](c)
    cu = c["cu_seqlens"]
    for i in range(len(lengths)):
        sl = slice(cu[i], cu[i + 1])
        ci = {x: c[x][sl] for x in ("q", "k", "v", "g", "beta")}
        oi, si = IMPLS[impl](dict(ci, cu_seqlens=[0, lengths[i]],
                                  initial_state=c["initial_state"][i:i + 1]))
        np.testing.assert_allclose(o[sl], oi, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(sT[i:i + 1], si, rtol=1e-13, atol=1e-14)
    assert np.array_equal(sT[1], c["initial_state"][1])  # empty sequence: final = initial


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_head_permutation_and_column_independence(impl):
    c = rand_case([21], H=3, dk=8, dv=6, seed=4)
    o, sT = IMPLS[impl](c)
    perm = [2, 0, 1]
    cp = {x: c[x][:, perm] for x in ("q", "k", "v", "g", "beta")}
    op, sp = IMPLS[impl](dict(cp, cu_seqlens=c["cu_seqlens"], initial_state=c["initial_state"][:, perm]))
    np.testing.assert_allclose(op, o[:, perm], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sp, sT[:, perm], rtol=1e-14, atol=1e-15)
    # value column j of o and S depends only on v[:, :, j] and S0[..., j]
    c2 = dict(c)
    c2["v"] = c["v"].copy()
    c2["v"][:, :, 1:] = 0.0
    c2["initial_state"] = c["initial_state"].copy()
    c2["initial_state"][..., 1:] = 0.0
    o2, s2 = IMPLS[impl](c2)
    np.testing.assert_allclose(o2[..., 0], o[..., 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2[..., 0], sT[..., 0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("impl", sorted(IMPLS))
def test_linearity_in_values_and_state(impl):
    c = rand_case([18], H=1, dk=8, dv=8, seed=6)
    ca, cb = dict(c), dict(c)
    r = np.random.default_rng(1)
    cb["v"] = r.standard_normal(c["v"].shape)
    cb["initial_state"] = r.standard_normal(c["initial_state"].shape)
    cs = dict(c)
    cs["v"] = 2.0 * ca["v"] - 3.0 * cb["v"]
    cs["initial_state"] = 2.0 * ca["initial_state"] - 3.0 * cb["initial_state"]
    oa, sa = IMPLS[impl](ca)
    ob, sb = IMPLS[impl](cb)
    os_, ss = IMPLS[impl](cs)
    np.testing.assert_allclose(os_, 2 * oa - 3 * ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ss, 2 * sa - 3 * sb, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("lengths", [[3], [16], [33], [32, 3], [35, 48, 1, 17]])
def test_chunked_matches_recurrent_with_tails(lengths):
    c = rand_case(lengths, H=2, dk=16, dv=8, seed=len(lengths) + sum(lengths))
    o1, s1 = ref.recurrent(**c)
    o2, s2 = ref.chunked(**c)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-12, atol=1e-12)


def test_c_oracle_full_width():
    """The C recurrence at D = 128 with several column blocks, vs the dense form."""
    c = rand_case([29, 40], H=2, dk=128, dv=128, seed=12)
    o1, s1 = ref.recurrent_c(**c, col_block=32)
    o2, s2 = run_dense(c)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-11, atol=1e-12)
    o3, s3 = ref.recurrent_c(**c, col_block=128, heads=[1])
    np.testing.assert_allclose(o3[:, 0], o1[:, 1], rtol=1e-13, atol=1e-14)


def test_wy_inverse_is_an_inverse():
    """K1's WY inverse times (I + strict-lower(diag(beta) A_kk)) is I, and the
    chunk quantities reproduce the dense form on one full chunk."""
    c = rand_case([16], H=1, dk=16, dv=8, seed=21)
    sl = lambda x: c[x][:, 0]
    k1 = ref.chunk_k1(sl("q"), sl("k"), sl("v"), sl("g"), sl("beta"))
    L = c["beta"][:, 0][:, None] * k1["A_kk"]
    np.testing.assert_allclose(k1["Tinv"] @ (np.eye(16) + L), np.eye(16), atol=1e-13)
    assert np.all(np.triu(k1["A_kk"]) == 0) and np.all(np.triu(k1["A_qk"], 1) == 0)
    O, S = ref.chunk_k2(c["initial_state"][0, 0], k1)
    od, sd = ref.dense(sl("q"), sl("k"), sl("v"), sl("g"), sl("beta"), c["initial_state"][0, 0])
    np.testing.assert_allclose(O, od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, sd, rtol=1e-12, atol=1e-13)


def test_segment_summary_composes():
    """The CP summary (M, B) of a run of chunks maps any start state to the
    end state: S_end = M S_start + B."""
    c = rand_case([80], H=1, dk=16, dv=8, seed=31)
    _, _, recs = ref.chunked(**c, intermediates=True)
    k1s = [recs[(0, j, 0)] for j in range(5)]
    M, B = ref.segment_summary(k1s, 16, 8)
    _, sT = ref.recurrent(**c)
    np.testing.assert_allclose(M @ c["initial_state"][0, 0] + B, sT[0, 0], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# planted mistakes: each mutated copy of the oracle must fail some pin above
# ---------------------------------------------------------------------------
def _mutant(kind):
    def run(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        Tt, H, dk = k.shape
        dv = v.shape[-1]
        cu = np.asarray(cu_seqlens if cu_seqlens is not None else [0, Tt])
        o = np.zeros((Tt, H, dv))
        sT = np.zeros((len(cu) - 1, H, dk, dv))
        for i in range(len(cu) - 1):
            for h in range(H):
                S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[i, h], dtype=float)
                for t in range(cu[i], cu[i + 1]):
                    gam = np.exp(-g[t, h] if kind == "decay_sign" else g[t, h])
                    if kind != "decay_after":
                        S = S * np.resize(gam, dv)[None, :] if kind == "decay_axis" else gam[:, None] * S
                    e = v[t, h] + (S.T @ k[t, h] if kind == "residual_sign" else -(S.T @ k[t, h]))
                    b = 1.0 if kind == "drop_beta" else beta[t, h]
                    S_new = S + b * np.outer(k[t, h], e)
                    if kind == "decay_after":
                        S_new = gam[:, None] * S_new
                    read = S if kind == "read_before_write" else S_new
                    o[t, h] = (1.0 if kind == "drop_scale" else scale) * (
                        np.resize(read @ np.resize(q[t, h], dv), dv) if kind == "transpose_read" else read.T @ q[t, h])
                    S = S_new
                sT[i, h] = S
        return o, sT
    return run


MUTANTS = ["decay_after", "decay_sign", "decay_axis", "residual_sign", "drop_beta",
           "read_before_write", "transpose_read", "drop_scale"]


def _pins_pass(impl):
    """The impl-parametrised pins of this file, as one boolean battery."""
    failures = 0
    for test in (test_golden_hand_example, test_beta_zero_is_pure_decay, test_delta_rule_overwrite,
                 test_orthonormal_keys_replace_rows, test_read_only_state):
        try:
            test("_under_test")
        except AssertionError:
            failures += 1
    try:
        c = rand_case([24], H=1, dk=8, dv=8, seed=24)
        o1, s1 = IMPLS["_under_test"](c)
        o2, s2 = run_dense(c)
        np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s1, s2, rtol=1e-11, atol=1e-12)
    except AssertionError:
        failures += 1
    return failures == 0


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistakes_are_caught(kind):
    IMPLS["_under_test"] = lambda c, scale=1.0: _mutant(kind)(**c, scale=scale)
    try:
        assert not _pins_pass("_under_test"), "planted mistake %r went unnoticed" % kind
    finally:
        del IMPLS["_under_test"]


def test_unmutated_copy_passes_battery():
    IMPLS["_under_test"] = lambda c, scale=1.0: _mutant("none")(**c, scale=scale)
    try:
        assert _pins_pass("_under_test")
    finally:
        del IMPLS["_under_test"]


CHUNK_MUTANTS = {
    "aqk_strict": lambda d: dict(d, A_qk=np.tril(d["A_qk"], -1)),
    "kt_undecayed": lambda d: dict(d, Kt=d["Kt"] / np.exp(d["G"][-1][None, :] - d["G"])),
    "gc_first_row": lambda d: dict(d, gC=np.exp(d["G"][0])),
    "no_wy_inverse": lambda d: dict(d, W=d["W"] * 0 + (np.linalg.inv(d["Tinv"]) @ d["W"])),
}


@pytest.mark.parametrize("kind", sorted(CHUNK_MUTANTS))
def test_planted_chunk_mistakes_are_caught(kind, monkeypatch):
    real = ref.chunk_k1
    monkeypatch.setattr(ref, "chunk_k1", lambda *a: CHUNK_MUTANTS[kind](real(*a)))
    c = rand_case([35], H=1, dk=16, dv=8, seed=40)
    o1, s1 = ref.recurrent(**c)
    o2, s2 = ref.chunked(**c)
    assert not (np.allclose(o1, o2, rtol=1e-9, atol=1e-10) and np.allclose(s1, s2, rtol=1e-9, atol=1e-10))


# ---------------------------------------------------------------------------
# decode step (one token per sequence, matrix form of the update)
# ---------------------------------------------------------------------------
def _decode_tokens(step, c):
    """Feed each sequence of a packed case through `step` one token at a time
    (all sequences advance together; shorter ones stop early)."""
    q, k, v, g, beta = (np.asarray(c[x], dtype=np.float64) for x in ("q", "k", "v", "g", "beta"))
    cu = np.asarray(c["cu_seqlens"])
    n = len(cu) - 1
    H, dk, dv = k.shape[1], k.shape[2], v.shape[2]
    S = np.zeros((n, H, dk, dv)) if c["initial_state"] is None else np.array(c["initial_state"], dtype=float)
    o = np.zeros((cu[-1], H, dv))
    for t in range(int(np.max(np.diff(cu))) if n else 0):
        live = [i for i in range(n) if cu[i] + t < cu[i + 1]]
        rows = [cu[i] + t for i in live]
        ot, St = step(q[rows], k[rows], v[rows], g[rows], beta[rows], S[live])
        o[rows] = ot
        S[live] = St
    return o, S


def test_decode_golden_hand_example():
    c, gv = golden_inputs()
    o, sT = _decode_tokens(ref.decode_step, c)
    np.testing.assert_allclose(o.reshape(-1), gv["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sT.reshape(-1), gv["ST"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("lengths,dk,dv", [([1], 8, 8), ([5, 1, 9], 8, 4), ([12, 7], 16, 16), ([3], 128, 128)])
def test_decode_matches_recurrent(lengths, dk, dv):
    """The matrix form, stepped token by token, equals the residual form of
    the recurrence over whole sequences (two different algebraic forms)."""
    c = rand_case(lengths, H=3, dk=dk, dv=dv, seed=sum(lengths) + dk)
    o1, s1 = ref.recurrent(**c)
    o2, s2 = _decode_tokens(ref.decode_step, c)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-11, atol=1e-12)


def test_decode_closed_forms():
    r = np.random.default_rng(11)
    N, H, dk, dv = 4, 2, 8, 6
    q, k = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v, g = r.standard_normal((N, H, dv)), -r.random((N, H, dk))
    beta, S = r.random((N, H)), r.standard_normal((N, H, dk, dv))
    # beta = 0: pure per-key-channel decay
    o, S1 = ref.decode_step(q, k, v, g, np.zeros((N, H)), S, scale=0.5)
    np.testing.assert_allclose(S1, np.exp(g)[..., None] * S, rtol=1e-13, atol=0)
    np.testing.assert_allclose(o, 0.5 * np.einsum("nhkv,nhk->nhv", np.exp(g)[..., None] * S, q), rtol=1e-12)
    # zero state: S' = beta k v^T, o = scale beta (q.k) v
    o, S1 = ref.decode_step(q, k, v, g, beta, np.zeros_like(S), scale=2.0)
    np.testing.assert_allclose(S1, beta[..., None, None] * k[..., :, None] * v[..., None, :], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o, 2.0 * (beta * np.einsum("nhk,nhk->nh", q, k))[..., None] * v, rtol=1e-12, atol=1e-14)
    # g = 0, beta = 1, |k| = 1: the new state maps k to v exactly
    _, S1 = ref.decode_step(q, k, v, np.zeros_like(g), np.ones((N, H)), S)
    np.testing.assert_allclose(np.einsum("nhkv,nhk->nhv", S1, k), v, rtol=1e-12, atol=1e-12)


DECODE_MUTANTS = {
    # decay applied after the projection instead of before it
    "decay_after": lambda P, Dg, S, w: Dg @ (P @ S) + w,
    # projection skipped (plain additive update)
    "no_projection": lambda P, Dg, S, w: Dg @ S + w,
    # state decayed along the value axis
    "decay_axis": lambda P, Dg, S, w: P @ (S @ Dg[:S.shape[1], :S.shape[1]]) + w,
}


@pytest.mark.parametrize("kind", sorted(DECODE_MUTANTS))
def test_planted_decode_mistakes_are_caught(kind):
    def step(q, k, v, g, beta, S):
        N, H, dk = k.shape
        o, S_new = np.zeros((N, H, v.shape[-1])), np.zeros_like(S)
        for n in range(N):
            for h in range(H):
                P = np.eye(dk) - beta[n, h] * np.outer(k[n, h], k[n, h])
                S_new[n, h] = DECODE_MUTANTS[kind](P, np.diag(np.exp(g[n, h])), S[n, h],
                                                   beta[n, h] * np.outer(k[n, h], v[n, h]))
                o[n, h] = S_new[n, h].T @ q[n, h]
        return o, S_new
    c, gv = golden_inputs()
    o, sT = _decode_tokens(step, c)
    golden_ok = np.allclose(o.reshape(-1), gv["o"], atol=1e-9) and np.allclose(sT.reshape(-1), gv["ST"], atol=1e-9)
    c = rand_case([6, 3], H=2, dk=8, dv=8, seed=5)
    o1, s1 = ref.recurrent(**c)
    o2, s2 = _decode_tokens(step, c)
    rec_ok = np.allclose(o1, o2, rtol=1e-9, atol=1e-10) and np.allclose(s1, s2, rtol=1e-9, atol=1e-10)
    assert not (golden_ok and rec_ok), "planted decode mistake %r went unnoticed" % kind


# ---------------------------------------------------------------------------
# grouped value heads: the head mapping
# ---------------------------------------------------------------------------
def _gva_case(Hk, G, seed):
    """Value heads of one group share v, g, beta and S0, so only the q/k head
    they read can tell them apart."""
    c = rand_case([9, 4], H=Hk, dk=8, dv=8, seed=seed)
    rep = lambda x, axis: np.repeat(x, G, axis=axis)
    return dict(q=c["q"], k=c["k"], v=rep(c["v"], 1), g=rep(c["g"], 1), beta=rep(c["beta"], 1),
                cu_seqlens=c["cu_seqlens"], initial_state=rep(c["initial_state"], 1))


def _gva_run(c, expand):
    H = c["v"].shape[1]
    q, k = expand(c["q"], c["k"], H)
    return ref.recurrent(q, k, c["v"], c["g"], c["beta"], c["cu_seqlens"], c["initial_state"])


def _gva_pins_pass(expand):
    c = _gva_case(3, 4, seed=12)
    o, sT = _gva_run(c, expand)
    # value heads 4j .. 4j+3 form one group: identical results inside it ...
    same = all(np.allclose(o[:, 4 * j], o[:, 4 * j + i]) and np.allclose(sT[:, 4 * j], sT[:, 4 * j + i])
               for j in range(3) for i in range(1, 4))
    # ... and each equals the plain single-head run of its q/k head
    plain_o, plain_s = ref.recurrent(c["q"], c["k"], c["v"][:, ::4], c["g"][:, ::4], c["beta"][:, ::4],
                                     c["cu_seqlens"], c["initial_state"][:, ::4])
    return same and np.allclose(o[:, ::4], plain_o, rtol=1e-12, atol=1e-13) and np.allclose(
        sT[:, ::4], plain_s, rtol=1e-12, atol=1e-13)


def test_gva_grouping_pins():
    assert _gva_pins_pass(ref.gva_expand)
    c = rand_case([5], H=4, dk=8, dv=8, seed=3)
    q, k = ref.gva_expand(c["q"], c["k"], 4)  # one value head per q/k head: unchanged
    assert np.array_equal(q, c["q"]) and np.array_equal(k, c["k"])
    with pytest.raises(ValueError):
        ref.gva_expand(c["q"], c["k"], 6)


def test_planted_gva_mapping_is_caught():
    # value head h reading q/k head h mod Hk (interleaved groups) instead of floor(h / G)
    interleaved = lambda q, k, H: (np.tile(q, (1, H // q.shape[1], 1)), np.tile(k, (1, H // k.shape[1], 1)))
    assert not _gva_pins_pass(interleaved)
