"""GPU parity of the HIP prefill against the fp64 CPU oracle.

Bar: bf16 output and the complete fp32 final state within atol = rtol = 1e-2
of the oracle (the correctness gate of "fix(cake_kda): support non-aligned
recurrent prefill head counts", FlashInfer pull request #4351, description),
and bitwise equality where the arithmetic is identical by construction:
intracard CP vs serial ("feat(kda/sm90): FlashKDA prefill port +
intracard-CP prefill", cuLA pull request #103, commit summary and tests),
packing, head permutation, chunk-aligned carry, repetition.
All calls go through the C ABI (libkda.so) via the ctypes binding.
"""
import os

os.environ.setdefault("KDA_DEBUG_POISON", "1")  # NaN-filled workspace catches uninitialised reads

import numpy as np
import pytest
import torch

import kda_chunked_delta_amd as kda
from kda_inputs import draw, workload
from oracle import reference as ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = dict(atol=1e-2, rtol=1e-2)


def say(*a):
    print(*a, flush=True)


def assert_close(name, gpu, expect, atol=1e-2, rtol=1e-2):
    g = gpu.double().cpu().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, dtype=np.float64)
    e = np.asarray(expect, dtype=np.float64)
    assert g.shape == e.shape, (name, g.shape, e.shape)
    bad = np.abs(g - e) > atol + rtol * np.abs(e)
    err = np.abs(g - e)
    say("  %-14s max|err| %.3e  max rel-to-tol %.3f" % (name, err.max() if err.size else 0.0,
                                                        (err / (atol + rtol * np.abs(e))).max() if err.size else 0.0))
    if bad.any() or not np.isfinite(g).all():
        idx = np.unravel_index(np.argmax(np.where(np.isfinite(g), err, np.inf)), g.shape)
        raise AssertionError("%s: %d elements out of tolerance; worst at %s: gpu %r oracle %r"
                             % (name, int(bad.sum()) + int((~np.isfinite(g)).sum()), idx, g[idx], e[idx]))


def run(d, mode=False, s0="given", final=True, plan=None, scale=1.0):
    init = d["initial_state"] if s0 == "given" else None
    o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=init,
                       output_final_state=final, use_intracard_cp=mode, plan=plan, scale=scale)
    torch.cuda.synchronize()
    return o, s


def oracle(d, s0="given", scale=1.0, heads=None):
    init = d["initial_state"] if s0 == "given" else None
    return ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens_host"], init,
                           scale=scale, heads=heads)


@pytest.mark.parametrize("name", ["t64_h1", "h12_2x32", "h12_2x33", "h12_32_3"])
def test_small_workloads_match_oracle(name):
    say("case", name)
    d = workload(name, device=DEV)
    o, s = run(d)
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


@pytest.mark.parametrize("lengths", [[1], [15], [16], [17], [0, 5, 0, 31, 48, 0], [3, 100, 257]])
def test_short_and_ragged_lengths(lengths):
    say("case lengths", lengths)
    d = draw(lengths, 5, seed=sum(lengths) + 11, state_std=0.1, device=DEV)
    o, s = run(d)
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


@pytest.mark.parametrize("s0,final", [("given", True), ("given", False), (None, True), (None, False)])
def test_state_in_out_combinations(s0, final):
    say("case s0", s0, "final", final)
    d = workload("h12_2x33", device=DEV)
    o, s = run(d, s0=s0, final=final)
    o_ref, s_ref = oracle(d, s0=s0)
    assert_close("out", o, o_ref)
    if final:
        assert_close("final_state", s, s_ref)
    else:
        assert s is None


def test_in_place_state_update():
    d = workload("h12_32_3", device=DEV)
    o_ref, s_ref = oracle(d)
    st = d["initial_state"].clone()
    o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert_close("out", o, o_ref)
    assert_close("final_state", st, s_ref)


def test_zero_state_equals_no_state():
    d = workload("h12_2x33", device=DEV)
    o1, s1 = run(d, s0=None)
    d2 = dict(d, initial_state=torch.zeros_like(d["initial_state"]))
    o2, s2 = run(d2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_scale():
    d = workload("h12_2x32", device=DEV)
    o, _ = run(d, scale=0.5)
    o_ref, _ = oracle(d, scale=0.5)
    assert_close("out(scale=0.5)", o, o_ref)


# ---------------------------------------------------------------------------
# K1 records against the chunked fp64 oracle
# ---------------------------------------------------------------------------
def decode_records(rec):
    """uint8 [KDA_RECORD_BYTES] record -> dict of fp32 numpy arrays (layout of include/kda.h)."""
    r = rec.cpu().numpy()
    bf = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    lanes = np.arange(64)
    g, i = lanes // 16, lanes % 16
    out = {}
    for name, off in (("Qt", 0), ("X", 4096)):
        a = bf(r[off:off + 4096].view(np.uint16).reshape(4, 64, 8))
        x = np.zeros((16, 128), np.float32)
        for p in range(4):
            for j in range(8):
                x[i, 32 * p + 16 * (j // 4) + 4 * g + j % 4] = a[p, :, j]
        out[name] = x
    # Kt: lane l's fragment sits in slot (l & 0x33) | ((((l >> 2) + (l >> 4)) & 3) << 2)
    slot = (lanes & 0x33) | ((((lanes >> 2) + (lanes >> 4)) & 3) << 2)
    a = bf(r[8192:12288].view(np.uint16).reshape(8, 64, 4))[:, slot, :]
    x = np.zeros((16, 128), np.float32)
    for t in range(8):
        for j in range(4):
            x[4 * g + j, 16 * t + i] = a[t, :, j]
    out["Kt"] = x
    a = bf(r[12288:12800].view(np.uint16).reshape(64, 4))
    x = np.zeros((16, 16), np.float32)
    for j in range(4):
        x[i, 4 * g + j] = a[:, j]
    out["A_qk"] = x
    # exp(G_C): channel c = 16t + 4g + j at position 32g + 4t + j
    gcp = r[12800:13312].view(np.float32)
    c = np.arange(128)
    out["gC"] = gcp[32 * ((c >> 2) & 3) + 4 * (c >> 4) + (c & 3)].copy()
    t = bf(r[13312:14336].view(np.uint16).reshape(2, 64, 4)).astype(np.float64)
    x = np.zeros((16, 16))
    for j in range(4):
        x[i, 4 * g + j] = t[0, :, j] + t[1, :, j]
    out["Tb"] = x
    return out


@pytest.mark.parametrize("lengths", [[16], [33, 3], [64, 21]])
def test_k1_records_match_chunked_oracle(lengths):
    """Each record field against the fp64 chunked oracle's K1 of that chunk:
    X = k exp(G) and T' = Tinv diag(beta) are formed from its G and Tinv."""
    say("case lengths", lengths)
    H = 3
    d = draw(lengths, H, seed=77 + sum(lengths), state_std=None, device=DEV)
    p = kda.plan(d["cu_seqlens_host"], H, device=DEV)
    recs = kda.k1_records(d["q"], d["k"], d["v"], d["g"], d["beta"], p)
    torch.cuda.synchronize()
    _, _, ks = ref.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens_host"], None,
                           intermediates=True)
    k64, b64 = (ref.to_f64(d[n]) for n in ("k", "beta"))
    cu = d["cu_seqlens_host"]
    gidx = 0
    for i, L in enumerate(lengths):
        for c in range((L + 15) // 16):
            t0 = cu[i] + 16 * c
            for h in range(H):
                got = decode_records(recs[h, gidx])
                exp = ks[(i, c, h)]
                n = exp["Qt"].shape[0]
                want = dict(Qt=exp["Qt"], Kt=exp["Kt"], X=k64[t0:t0 + n, h] * np.exp(exp["G"]))
                for key in ("Qt", "X", "Kt"):
                    assert_close("%s[%d,%d,%d]" % (key, i, c, h), got[key][:n], want[key])
                    assert np.all(got[key][n:] == 0), "%s rows past the tail must be zero" % key
                aq = np.zeros((16, 16))
                aq[:n, :n] = exp["A_qk"]
                assert_close("A_qk", got["A_qk"], aq)
                tb = exp["Tinv"] * b64[t0:t0 + n, h][None, :]
                assert_close("T'", got["Tb"][:n, :n], tb)
                assert np.all(got["Tb"][n:, :] == 0) and np.all(got["Tb"][:, n:] == 0)
                assert_close("gC", got["gC"], exp["gC"], atol=1e-6, rtol=1e-5)
            gidx += 1


# ---------------------------------------------------------------------------
# bitwise properties of the serial path
# ---------------------------------------------------------------------------
def test_chunk_aligned_carry_is_bitwise():
    """run([a; b]) == run(b, run(a).final) bitwise when |a| is a multiple of 16."""
    d = draw([160], 4, seed=5, state_std=0.1, device=DEV)
    o, s = run(d)
    cut = 96
    sl = lambda x, a, b: x[a:b].contiguous()
    da = dict(d, q=sl(d["q"], 0, cut), k=sl(d["k"], 0, cut), v=sl(d["v"], 0, cut), g=sl(d["g"], 0, cut),
              beta=sl(d["beta"], 0, cut), cu_seqlens=None, cu_seqlens_host=[0, cut])
    oa, sa = run(da)
    db = dict(d, q=sl(d["q"], cut, 160), k=sl(d["k"], cut, 160), v=sl(d["v"], cut, 160),
              g=sl(d["g"], cut, 160), beta=sl(d["beta"], cut, 160), cu_seqlens=None,
              cu_seqlens_host=[0, 160 - cut], initial_state=sa)
    ob, sb = run(db)
    assert torch.equal(torch.cat([oa, ob]), o)
    assert torch.equal(sb, s)


def test_varlen_packing_is_bitwise():
    lengths = [40, 7, 130]
    d = draw(lengths, 6, seed=8, state_std=0.1, device=DEV)
    o, s = run(d)
    cu = d["cu_seqlens_host"]
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        di = dict(d, q=d["q"][a:b].contiguous(), k=d["k"][a:b].contiguous(), v=d["v"][a:b].contiguous(),
                  g=d["g"][a:b].contiguous(), beta=d["beta"][a:b].contiguous(), cu_seqlens=None,
                  cu_seqlens_host=[0, b - a], initial_state=d["initial_state"][i:i + 1].contiguous())
        oi, si = run(di)
        assert torch.equal(oi, o[a:b]) and torch.equal(si, s[i:i + 1])


def test_head_permutation_is_bitwise():
    d = draw([70, 33], 5, seed=9, state_std=0.1, device=DEV)
    o, s = run(d)
    perm = torch.tensor([3, 0, 4, 1, 2], device=DEV)
    dp = dict(d)
    for key in ("q", "k", "v", "g", "beta"):
        dp[key] = d[key].index_select(1, perm).contiguous()
    dp["initial_state"] = d["initial_state"].index_select(1, perm).contiguous()
    op, sp = run(dp)
    assert torch.equal(op, o.index_select(1, perm)) and torch.equal(sp, s.index_select(1, perm))


@pytest.mark.parametrize("form", ["serial", "split", "warm_cp", "cp"])
def test_repeated_runs_are_bitwise_deterministic(form):
    """Repeated runs are bitwise equal in every plan form (fixed reduction
    orders everywhere; no atomics in any result)."""
    d = draw([600, 77], 4, seed=10, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    plan = {"serial": None,
            "split": lambda: kda.plan_split(cu, 4, [20, 0], 12, device=DEV),
            "warm_cp": lambda: kda.plan_warm_cp(cu, 4, 16, 12, device=DEV),
            "cp": lambda: kda.plan_segments(cu, 4, 8, device=DEV)}[form]
    p = plan() if plan else None
    o0, s0 = run(d, plan=p)
    for _ in range(20):
        o, s = run(d, plan=p)
        assert torch.equal(o, o0) and torch.equal(s, s0)


# ---------------------------------------------------------------------------
# intracard CP
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seg_chunks,lengths", [(2, [200]), (3, [100, 35, 260]), (8, [1000, 20])])
def test_forced_cp_accuracy(seg_chunks, lengths):
    say("case seg_chunks", seg_chunks, "lengths", lengths)
    d = draw(lengths, 4, seed=seg_chunks * 100 + len(lengths), state_std=0.1, device=DEV)
    p = kda.plan_segments(d["cu_seqlens_host"], 4, seg_chunks, device=DEV)
    assert p.info()["uses_cp"] == 1
    o, s = run(d, plan=p)
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


def test_forced_cp_in_place_state():
    d = draw([400, 50], 3, seed=3, state_std=0.1, device=DEV)
    o_ref, s_ref = oracle(d)
    p = kda.plan_segments(d["cu_seqlens_host"], 3, 4, device=DEV)
    st = d["initial_state"].clone()
    o, _ = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=st, final_state=st, plan=p)
    torch.cuda.synchronize()
    assert_close("out", o, o_ref)
    assert_close("final_state", st, s_ref)


def test_cp_bitwise_on_long_sequence_and_oracle():
    """One 65536-token sequence, 8 heads: the auto plan splits it; the result
    must equal the serial path bitwise and the oracle within 1e-2."""
    say("case long65536_h8")
    d = workload("long65536_h8", device=DEV)
    p_auto = kda.plan(d["cu_seqlens_host"], 8, "auto", device=DEV)
    assert p_auto.info()["uses_cp"] == 1
    say("  auto plan: warm-start CP %d (segments of %d chunks)" % (p_auto.info()["warm_cp"],
                                                                 p_auto.info()["warm_cp_seg_chunks"]))
    o_ser, s_ser = run(d, mode=False)
    o_cp, s_cp = run(d, plan=p_auto)
    assert torch.equal(o_cp, o_ser), "CP output differs from serial"
    assert torch.equal(s_cp, s_ser), "CP final state differs from serial"
    o_ref, s_ref = oracle(d)
    assert_close("out", o_cp, o_ref)
    assert_close("final_state", s_cp, s_ref)


def test_padded_batch_cp_paths_are_bitwise_serial():
    """Equal-length batches passed as [B, T, H, 128] (no cu_seqlens) run
    through every CP form: the segmented pipeline forced, AUTO, and warm-start
    CP forced; each equals the packed serial result bit for bit (the cuLA
    pull request's reviewer notes list CP on padded B > 1 as a limitation)."""
    B, T, H = 3, 2048, 2
    d = draw([T] * B, H, seed=54, state_std=0.1, device=DEV)
    o_ser, s_ser = run(d, mode=False)
    as4 = lambda x: x.view(B, T, *x.shape[1:])
    q, k, v, g, beta = (as4(d[n]) for n in ("q", "k", "v", "g", "beta"))
    cu = [i * T for i in range(B + 1)]
    for label, kw in (("cp on", dict(use_intracard_cp=True)), ("auto", dict(use_intracard_cp="auto")),
                      ("warm-start cp", dict(plan=kda.plan_warm_cp(cu, H, 32, 12, device=DEV)))):
        o, s = kda.prefill(q, k, v, g, beta, initial_state=d["initial_state"], output_final_state=True, **kw)
        torch.cuda.synchronize()
        assert o.shape == (B, T, H, 128), label
        assert torch.equal(o.reshape(B * T, H, 128), o_ser) and torch.equal(s, s_ser), label
    assert kda.plan(cu, H, True, device=DEV).info()["n_cp_seqs"] == B


def test_long_sequence_segmented_cp_is_bitwise_serial():
    """The segmented CP pipeline alone (forced) on the 65536-token workload:
    bitwise the serial result."""
    d = workload("long65536_h8", device=DEV)
    p = kda.plan_segments(d["cu_seqlens_host"], 8, 64, device=DEV)
    assert p.info()["warm_cp"] == 0
    o_ser, s_ser = run(d, mode=False)
    o_cp, s_cp = run(d, plan=p)
    assert torch.equal(o_cp, o_ser) and torch.equal(s_cp, s_ser)


def test_materialized_k1_paths_are_bitwise_equal_to_fused(monkeypatch):
    """The two-kernel form (K1 writes records once; K2, pre_scan read them)
    runs the same arithmetic as the fused form: serial and CP results match
    the fused serial path bitwise."""
    d = draw([1500, 300, 2100], 4, seed=21, state_std=0.1, device=DEV)
    o_ref, s_ref = run(d, mode=False)
    monkeypatch.setenv("KDA_MATERIALIZE_K1", "1")
    p_ser = kda.plan(d["cu_seqlens_host"], 4, False, device=DEV)
    p_cp = kda.plan_segments(d["cu_seqlens_host"], 4, 64, device=DEV)
    monkeypatch.delenv("KDA_MATERIALIZE_K1")
    assert p_ser.info()["k1_materialized"] == 1 and p_cp.info()["k1_materialized"] == 1
    o1, s1 = run(d, plan=p_ser)
    assert torch.equal(o1, o_ref) and torch.equal(s1, s_ref)
    o2, s2 = run(d, plan=p_cp)
    assert torch.equal(o2, o_ref) and torch.equal(s2, s_ref)


def test_cp_weak_decay_within_tolerance():
    """With weak decay the carried state is not forgotten inside a segment, so
    CP equals serial only within rounding; both match the oracle."""
    d = draw([4096], 2, seed=12, state_std=0.1, device=DEV)
    d["g"] = d["g"] * 0.05
    p = kda.plan_segments(d["cu_seqlens_host"], 2, 64, device=DEV)
    o_cp, s_cp = run(d, plan=p)
    o_ser, s_ser = run(d)
    o_ref, s_ref = oracle(d)
    assert_close("out(cp)", o_cp, o_ref)
    assert_close("final(cp)", s_cp, s_ref)
    assert_close("out(serial)", o_ser, o_ref)


def test_cp_merge_long_live_run():
    """One run of 63 live transfers (64 segments of 4 chunks under very weak
    decay): the merge chains 63 steps, each reading its transfer M in the
    operand order the K1 pass stores it in, with its 16-byte quad-transposed
    stores; outputs and final states match the oracle within 1e-2."""
    d = draw([4096], 2, seed=23, state_std=0.1, device=DEV)
    d["g"] = d["g"] * 0.02
    say("case: 4096 tokens, H=2, 64 segments of 4 chunks, g x 0.02")
    p = kda.plan_segments(d["cu_seqlens_host"], 2, 4, device=DEV)
    info = p.info()
    assert info["uses_cp"] == 1 and info["n_prescan"] == 63, info
    o_cp, s_cp = run(d, plan=p)
    o_ref, s_ref = oracle(d)
    assert_close("out(cp)", o_cp, o_ref)
    assert_close("final(cp)", s_cp, s_ref)


def test_cp_merge_runs_starting_mid_sequence():
    """Decay that alternates by region: strong (g x 4) where a segment's
    transfer vanishes, weak (g x 0.05) where it survives. The merge then has
    runs of live transfers that start after segment 0 (from the B of a
    segment whose transfer vanished) and end at a vanished transfer or at
    the last summary, with odd and even lengths. CP matches the oracle and
    the serial path within 1e-2; in place as well."""
    seg = 8  # chunks per segment
    regions = [(5, 4.0), (10, 0.05), (5, 4.0), (7, 0.05), (2, 4.0), (11, 0.05)]  # (segments, g scale)
    n_seg = sum(r[0] for r in regions)
    T = n_seg * seg * 16
    say("case: %d segments of %d chunks, regions %s" % (n_seg, seg, regions))
    d = draw([T], 2, seed=91, state_std=0.1, device=DEV)
    scale = torch.cat([torch.full((n * seg * 16,), f, dtype=torch.float32) for n, f in regions]).to(DEV)
    d["g"] = d["g"] * scale[:, None, None]
    cu = d["cu_seqlens_host"]
    p = kda.plan_segments(cu, 2, seg, device=DEV)
    assert p.info()["uses_cp"] == 1
    o_cp, s_cp = run(d, plan=p)
    o_ser, s_ser = run(d)
    o_ref, s_ref = oracle(d)
    assert_close("out(cp)", o_cp, o_ref)
    assert_close("final(cp)", s_cp, s_ref)
    assert_close("out(cp vs serial)", o_cp, o_ser.double().cpu().numpy())
    st = d["initial_state"].clone()
    o_in, _ = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                          cu_seqlens_host=cu, initial_state=st, final_state=st, plan=p)
    torch.cuda.synchronize()
    assert torch.equal(o_in, o_cp) and torch.equal(st, s_cp), "in-place CP differs from out-of-place CP"


def test_cp_transfer_with_vanished_and_live_tiles():
    """A transfer whose 16-column tiles differ: keys are zero on channels
    0..15 (no delta-rule mixing into or out of them) and those channels
    decay strongly (g x 4), the rest weakly (g x 0.05). Tile 0 of every
    segment's transfer then underflows to exactly zero while the other seven
    live, so the merge reads a transfer with a tile that vanished. The same
    plan first runs a weak-decay batch that leaves every tile of the
    workspace's transfers nonzero, so a vanished tile that were not written
    as zeros would corrupt the carries. CP matches the oracle within 1e-2."""
    seg, n_seg = 8, 6
    T = seg * n_seg * 16
    d = draw([T], 2, seed=17, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    p = kda.plan_segments(cu, 2, seg, device=DEV)
    assert p.info()["uses_cp"] == 1
    weak = dict(d)
    weak["g"] = d["g"] * 0.05
    run(weak, plan=p)  # every transfer tile live
    mixed = dict(d)
    k = d["k"].clone()
    k[:, :, :16] = 0
    mixed["k"] = k
    chan = torch.full((128,), 0.05, dtype=torch.float32, device=DEV)
    chan[:16] = 4.0
    mixed["g"] = d["g"] * chan
    say("case: %d segments of %d chunks, keys zero and decay x4 on channels 0..15" % (n_seg, seg))
    o_cp, s_cp = run(mixed, plan=p)
    o_ref, s_ref = oracle(mixed)
    assert_close("out(cp)", o_cp, o_ref)
    assert_close("final(cp)", s_cp, s_ref)


def test_steep_in_chunk_decay_matches_oracle(monkeypatch):
    """Decay steps of e^-40 at rows 0 and 8 of every chunk, on the key
    channels of two of the eight K1 wavefronts of the second sequence: the
    in-chunk decay there (e^-80) is past what the chunk-start factoring of
    the Grams can hold, so those wavefronts factor about row 7, while the
    rows between the steps still interact fully. The other channels and the
    first sequence keep ordinary decay. Fused serial, materialised K1 and
    forced CP all match the oracle."""
    d = draw([40, 70], 3, seed=31, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    g = d["g"].clone()
    t = torch.arange(cu[1], cu[2], device=DEV)
    steep = ((t - cu[1]) % 8 == 0)
    rows = t[steep]
    g[cu[1]:cu[2], :, 16:32] = -0.01
    g[cu[1]:cu[2], :, 96:112] = -0.02
    for c0, c1 in ((16, 32), (96, 112)):
        g[rows, :, c0:c1] = -40.0
    d["g"] = g
    o_ref, s_ref = oracle(d)
    o, s = run(d)
    assert_close("out(fused)", o, o_ref)
    assert_close("final(fused)", s, s_ref)
    monkeypatch.setenv("KDA_MATERIALIZE_K1", "1")
    p_ser = kda.plan(cu, 3, False, device=DEV)
    monkeypatch.delenv("KDA_MATERIALIZE_K1")
    o1, s1 = run(d, plan=p_ser)
    assert torch.equal(o1, o) and torch.equal(s1, s), "materialised K1 differs from fused"
    p_cp = kda.plan_segments(cu, 3, 2, device=DEV)
    o2, s2 = run(d, plan=p_cp)
    assert_close("out(cp)", o2, o_ref)
    assert_close("final(cp)", s2, s_ref)


def test_extreme_in_chunk_decay_stays_finite(monkeypatch):
    """Decays beyond what either factoring of the Grams holds in fp32: tokens
    with g = -100 (e^-100) at rows 3 and 5 of two chunks on some channels, a
    token with g = -200 on every channel of one head, and tokens with g = -inf
    (a reset of those channels) at rows 7, 13 and 9. Such chunks are taken
    with each token's log-decay floored at about e^-10.7, which changes the
    carried-in state's contribution by at most that factor. Outputs and final
    states stay finite and match the oracle; fused serial, materialised K1 and
    forced CP agree."""
    d = draw([200, 77], 6, seed=123, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    g = d["g"].clone()
    g[3, :, :40] = -100.0
    g[21, :, 64:] = -100.0
    g[40, 2, :] = -200.0
    g[55, :, 64:] = float("-inf")
    g[77, :, 16:48] = float("-inf")
    g[cu[1] + 9, :, :] = float("-inf")
    d["g"] = g
    o_ref, s_ref = oracle(d)
    assert np.isfinite(o_ref).all() and np.isfinite(s_ref).all()
    o, s = run(d)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    assert_close("out(fused)", o, o_ref)
    assert_close("final(fused)", s, s_ref)
    monkeypatch.setenv("KDA_MATERIALIZE_K1", "1")
    p_ser = kda.plan(cu, 6, False, device=DEV)
    monkeypatch.delenv("KDA_MATERIALIZE_K1")
    o1, s1 = run(d, plan=p_ser)
    assert torch.equal(o1, o) and torch.equal(s1, s), "materialised K1 differs from fused"
    p_cp = kda.plan_segments(cu, 6, 3, device=DEV)
    o2, s2 = run(d, plan=p_cp)
    assert_close("out(cp)", o2, o_ref)
    assert_close("final(cp)", s2, s_ref)


# ---------------------------------------------------------------------------
# warm-start splits (intracard CP inside the fused kernel)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lengths,split,warm", [([300, 520], [10, 15], 8), ([1000, 40, 700], [30, 0, 8], 8),
                                                ([250], [5], 4), ([161, 33], [10, 0], 10)])
def test_split_plan_is_bitwise_serial(lengths, split, warm):
    """Under the workloads' decay the warm-up transfer vanishes, so the
    warm-start segment's state from zero is its carry: output and final state
    equal the unsplit serial path bit for bit, and the oracle within 1e-2."""
    say("case lengths", lengths, "split", split, "warm", warm)
    d = draw(lengths, 4, seed=sum(lengths) + 3, state_std=0.1, device=DEV)
    p = kda.plan_split(d["cu_seqlens_host"], 4, split, warm, device=DEV)
    info = p.info()
    assert info["n_split_seqs"] == sum(1 for x in split if x) and info["split_warm_chunks"] == warm
    assert sorted(u["warm_chunks"] for u in p.units())[-1] == warm
    o_ser, s_ser = run(d, mode=False)
    o, s = run(d, plan=p)
    assert torch.equal(o, o_ser), "split output differs from serial"
    assert torch.equal(s, s_ser), "split final state differs from serial"
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


def test_split_plan_weak_decay_reruns_exactly():
    """With weak decay the warm-up transfer does not vanish; the fix-up
    launch reruns the warm-start segment from the first segment's end state,
    so the result is still the serial path's, bit for bit."""
    d = draw([900, 300], 3, seed=41, state_std=0.1, device=DEV)
    d["g"] = d["g"] * 0.05
    p = kda.plan_split(d["cu_seqlens_host"], 3, [30, 9], 8, device=DEV)
    o_ser, s_ser = run(d, mode=False)
    o, s = run(d, plan=p)
    assert torch.equal(o, o_ser) and torch.equal(s, s_ser)
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_split_plan_state_variants(g_scale):
    """In place (final state over the initial state), no initial state, no
    final state: each equals the serial path's result."""
    d = draw([600, 20], 3, seed=43, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    cu = d["cu_seqlens_host"]
    p = kda.plan_split(cu, 3, [20, 0], 8, device=DEV)
    o_ser, s_ser = run(d, mode=False)
    st = d["initial_state"].clone()
    o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=cu, initial_state=st, final_state=st, plan=p)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ser) and torch.equal(st, s_ser), "in place"
    o0, s0 = run(d, mode=False, s0=None)
    o1, s1 = run(d, plan=p, s0=None)
    assert torch.equal(o1, o0) and torch.equal(s1, s0), "no initial state"
    o2, _ = run(d, plan=p, final=False)
    assert torch.equal(o2, o_ser), "no final state"


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_split_plans_in_place_calls_in_a_row(g_scale):
    """In place, each call's fix-up launch publishes (or reruns) the
    warm-start segments after every unit has read its initial state. Five
    calls in a row, alternating two split plans of different pairs on one
    stream (so one arena), all equal the serial path bit for bit."""
    d = draw([640, 400], 4, seed=53, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    cu = d["cu_seqlens_host"]
    p1 = kda.plan_split(cu, 4, [20, 12], 8, device=DEV)
    p2 = kda.plan_split(cu, 4, [0, 13], 8, device=DEV)
    o_ser, s_ser = run(d, mode=False)
    for i in range(5):
        for p in (p1, p2):
            say("call", i, "split sequences", p.info()["n_split_seqs"], "g_scale", g_scale)
            st = d["initial_state"].clone()
            o, _ = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                               cu_seqlens_host=cu, initial_state=st, final_state=st, plan=p)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ser) and torch.equal(st, s_ser), f"call {i}"


# ---------------------------------------------------------------------------
# warm-start CP (all segments in the fused launch, segmented pipeline as fallback)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("aliased", [False, True])
def test_warm_cp_is_bitwise_serial(aliased):
    """Under the workloads' decay every warm-up transfer vanishes, the
    fallback stays unarmed, and the result is the serial path's bit for
    bit (in place too), and the oracle's within 1e-2."""
    d = draw([3000, 900, 40, 0], 4, seed=51, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    p = kda.plan_warm_cp(cu, 4, 32, 12, device=DEV)
    info = p.info()
    assert info["warm_cp"] == 1 and info["warm_cp_seg_chunks"] == 32 and info["n_warm_segments"] >= 5
    o_ser, s_ser = run(d, mode=False)
    if aliased:
        st = d["initial_state"].clone()
        o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                           cu_seqlens_host=cu, initial_state=st, final_state=st, plan=p)
        torch.cuda.synchronize()
    else:
        o, s = run(d, plan=p)
    assert torch.equal(o, o_ser), "warm-start CP output differs from serial"
    assert torch.equal(s, s_ser), "warm-start CP final state differs from serial"
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


@pytest.mark.parametrize("aliased", [False, True])
def test_warm_cp_weak_decay_is_the_cp_result(aliased):
    """Weak decay: warm-up transfers survive, the fallback is armed, and the
    result is that of the segmented CP plan with the same segments, bit for
    bit, within 1e-2 of the oracle."""
    d = draw([2500, 300], 3, seed=52, state_std=0.1, device=DEV)
    d["g"] = d["g"] * 0.05
    cu = d["cu_seqlens_host"]
    p = kda.plan_warm_cp(cu, 3, 32, 12, device=DEV)
    o_cp, s_cp = run(d, plan=kda.plan_segments(cu, 3, 32, device=DEV))
    if aliased:
        st = d["initial_state"].clone()
        o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                           cu_seqlens_host=cu, initial_state=st, final_state=st, plan=p)
        torch.cuda.synchronize()
    else:
        o, s = run(d, plan=p)
    assert torch.equal(o, o_cp) and torch.equal(s, s_cp), "armed fallback differs from the CP plan"
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_graph_replay_of_warm_cp(g_scale):
    """Warm-start CP captured in a HIP graph: every replay, with eager work
    between replays, equals the eager result (fallback unarmed or armed)."""
    d = draw([1500, 100], 4, seed=53, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    cu_h = d["cu_seqlens_host"]
    p = kda.plan_warm_cp(cu_h, 4, 24, 12, device=DEV)
    cu = p.cu_device()
    o_buf = torch.empty_like(d["q"])
    s_buf = torch.empty_like(d["initial_state"])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    o_e, s_e = run(d, plan=p)
    for trial in range(3):
        o_buf.zero_()
        s_buf.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_buf, o_e) and torch.equal(s_buf, s_e), "replay %d differs from eager" % trial
        run(d, mode=False)  # eager work between replays


def _launches(fn):
    """Names of the library's launches during fn()."""
    ctx = kda.context(DEV)
    ctx.set_timing(True)
    try:
        r = fn()
        torch.cuda.synchronize()
        names = set(ctx.timing())
    finally:
        ctx.set_timing(False)
    return r, names


@pytest.mark.parametrize("kind", ["split", "warm_cp"])
def test_speculation_turns_off_after_it_fails(kind):
    """Weak decay: the first call speculates, fails and stays exact; once its
    outcome has reached the host, the plan runs its exact path (the batch
    unsplit, or the segmented pipeline), with the same bits."""
    d = draw([1200, 300], 3, seed=81, state_std=0.1, device=DEV)
    d["g"] = d["g"] * 0.05
    cu = d["cu_seqlens_host"]
    if kind == "split":
        p = kda.plan_split(cu, 3, [30, 0], 12, device=DEV)
        ref_o, ref_s = run(d, mode=False)
        spec_name, exact_name = "fused_split", "fused_serial"
    else:
        p = kda.plan_warm_cp(cu, 3, 24, 12, device=DEV)
        ref_o, ref_s = run(d, plan=kda.plan_segments(cu, 3, 24, device=DEV))
        spec_name, exact_name = "fused_warm_cp", "k2_segment"
    (o1, s1), n1 = _launches(lambda: run(d, plan=p))
    assert spec_name in n1 and p.info()["speculation_off"] == 0
    (o2, s2), n2 = _launches(lambda: run(d, plan=p))
    assert spec_name not in n2 and exact_name in n2, n2
    assert p.info()["speculation_off"] == 1
    for o, s in ((o1, s1), (o2, s2)):
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


def test_speculation_stays_on_while_it_holds():
    d = draw([1200, 300], 3, seed=82, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    p = kda.plan_split(cu, 3, [30, 0], 12, device=DEV)
    o_ser, s_ser = run(d, mode=False)
    for _ in range(3):
        (o, s), names = _launches(lambda: run(d, plan=p))
        assert "fused_split" in names and torch.equal(o, o_ser) and torch.equal(s, s_ser)
    assert p.info()["speculation_off"] == 0


def test_split_plan_validation():
    d = draw([100], 2, seed=1, device=DEV)
    cu = d["cu_seqlens_host"]
    for split, warm in (([3], 8), ([7], 8), ([0], 0)):
        with pytest.raises(kda.KDAError):
            kda.plan_split(cu, 2, split, warm, device=DEV)
    for seg, warm in ((8, 0), (4, 8), (0, 1)):
        with pytest.raises(kda.KDAError):
            kda.plan_warm_cp(cu, 2, seg, warm, device=DEV)


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def test_headline_varlen_h32_full_parity():
    say("case varlen8_h32 (auto plan, as benchmarked)")
    d = workload("varlen8_h32", device=DEV)
    p = kda.plan(d["cu_seqlens_host"], 32, "auto", device=DEV)
    say("  plan: %d warm-start splits" % p.info()["n_split_seqs"])
    o, s = run(d, mode="auto")
    o_ser, s_ser = run(d, mode=False)
    assert torch.equal(o, o_ser) and torch.equal(s, s_ser), "auto plan differs from serial"
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


def test_batch16_h64_sampled_parity():
    say("case batch16x8192_h64 (sampled sequences and heads)")
    d = workload("batch16x8192_h64", device=DEV)
    o, s = run(d, mode="auto", s0=None)
    heads = [0, 17, 63]
    for i in (0, 9, 15):
        a, b = i * 8192, (i + 1) * 8192
        sub = {key: d[key][a:b, heads].contiguous() for key in ("q", "k", "v", "g", "beta")}
        o_ref, s_ref = ref.recurrent_c(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], [0, 8192])
        assert_close("out[seq %d]" % i, o[a:b, heads], o_ref)
        assert_close("final[seq %d]" % i, s[i:i + 1, heads], s_ref)


# ---------------------------------------------------------------------------
# runtime behaviour
# ---------------------------------------------------------------------------
def test_graph_replay_picks_up_changed_beta():
    d = workload("h12_2x33", device=DEV)
    run(d)  # grow the arena outside capture
    o_buf = torch.empty_like(d["q"])
    s_buf = torch.empty_like(d["initial_state"])
    p = kda.plan(d["cu_seqlens_host"], 12, device=DEV)
    cu = p.cu_device()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm the side stream's arena
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens_host"],
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens_host"],
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    for trial in range(3):
        d["beta"].copy_(torch.sigmoid(torch.randn(d["beta"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(trial))))
        graph.replay()
        torch.cuda.synchronize()
        o_e, s_e = run(d)
        assert torch.equal(o_buf, o_e) and torch.equal(s_buf, s_e), "replay %d differs from eager" % trial
    o_ref, s_ref = oracle(d)
    assert_close("out(replay)", o_buf, o_ref)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_graph_replay_of_a_warm_start_split(g_scale):
    """A split plan (main and fix-up launches) captured in a HIP graph: each
    replay, with eager work between replays, equals the eager result, under
    the workloads' decay (segments stand) and weak decay (fix-up reruns)."""
    d = draw([600, 150], 4, seed=71, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    cu_h = d["cu_seqlens_host"]
    p = kda.plan_split(cu_h, 4, [20, 0], 12, device=DEV)
    cu = p.cu_device()
    o_buf = torch.empty_like(d["q"])
    s_buf = torch.empty_like(d["initial_state"])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # grow the side stream's arena outside capture
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    o_ser, s_ser = run(d, mode=False)
    for trial in range(3):
        o_buf.zero_()
        s_buf.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_buf, o_ser) and torch.equal(s_buf, s_ser), "replay %d differs from serial" % trial
        run(d, plan=p)  # eager work between replays


def test_arena_reuse_across_shape_changes():
    big = draw([3000, 1000], 8, seed=1, state_std=0.1, device=DEV)
    small = draw([40], 2, seed=2, state_std=0.1, device=DEV)
    ob1, sb1 = run(big)
    os1, ss1 = run(small)
    ob2, sb2 = run(big)
    os2, ss2 = run(small)
    assert torch.equal(ob1, ob2) and torch.equal(sb1, sb2)
    assert torch.equal(os1, os2) and torch.equal(ss1, ss2)
    o_ref, s_ref = oracle(small)
    assert_close("out(small)", os2, o_ref)


def test_validation_errors_reach_python():
    """Every check runs on the host before any launch."""
    d = workload("h12_2x32", device=DEV)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    with pytest.raises(kda.KDAError) as e:
        kda.prefill(*args, cu_seqlens=d["cu_seqlens"], cu_seqlens_host=d["cu_seqlens_host"], out=d["q"])
    assert e.value.status == 3
    # a final state that partly overlaps the initial state
    st = d["initial_state"]
    buf = torch.zeros(st.numel() + 4096, device=DEV)
    init = buf[:st.numel()].view(st.shape)
    init.copy_(st)
    bad_final = buf[4096:].view(st.shape)
    with pytest.raises(kda.KDAError) as e:
        kda.prefill(*args, cu_seqlens=d["cu_seqlens"], cu_seqlens_host=d["cu_seqlens_host"],
                    initial_state=init, final_state=bad_final)
    assert e.value.status == 3 and "partially overlaps" in str(e.value)
    with pytest.raises(ValueError):
        kda.prefill(d["q"], d["k"], d["v"], d["g"].to(torch.bfloat16), d["beta"], cu_seqlens=d["cu_seqlens"])
    # tables that do not describe the packed tokens exactly
    Tt = d["q"].shape[0]
    for cu in ([0, 32, Tt - 1], [0, 40, 32, Tt], [1, 32, Tt], [0, 32, Tt + 16], [0]):
        with pytest.raises(ValueError, match="cu_seqlens"):
            kda.prefill(*args, cu_seqlens=cu)
    with pytest.raises(ValueError, match="int32 CUDA tensor"):
        kda.prefill(*args, cu_seqlens=torch.tensor([0, Tt], dtype=torch.int32, device=DEV),
                    cu_seqlens_host=d["cu_seqlens_host"])
    # a plan built for other heads or other sequences
    for cu_p, H_p in (([0, 32, 64], 8), ([0, 30, 64], 12), ([0, 64], 12)):
        p_other = kda.plan(cu_p, H_p, device=DEV)
        with pytest.raises(ValueError, match="plan"):
            kda.prefill(*args, cu_seqlens=d["cu_seqlens"], cu_seqlens_host=d["cu_seqlens_host"], plan=p_other)


@pytest.mark.parametrize("name", ["t64_h1", "h12_32_3", "h12_2x33"])
def test_c_abi_kda_prefill_entry(name):
    """kda_prefill itself (the entry without options), called through ctypes
    with raw device pointers and the current stream, against the oracle and
    bitwise against the binding's call."""
    import ctypes
    say("case", name)
    d = workload(name, device=DEV)
    cu_h, H = d["cu_seqlens_host"], d["H"]
    N = len(cu_h) - 1
    L = kda.lib()
    ctx = kda.context(DEV)
    p = kda.plan(cu_h, H, device=DEV)
    o = torch.full_like(d["v"], float("nan"))
    s = torch.full((N, H, 128, 128), float("nan"), device=DEV)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = L.kda_prefill(ctx.handle, p.handle, ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["g"]), ptr(d["beta"]),
                       ptr(d["cu_seqlens"]), 1.0, ptr(d["initial_state"]), ptr(s), ptr(o),
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.kda_last_error().decode()
    torch.cuda.synchronize()
    o_ref, s_ref = oracle(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)
    o_b, s_b = run(d, plan=p)
    assert torch.equal(o, o_b) and torch.equal(s, s_b)


def test_graph_replay_survives_arena_growth_and_plan_release():
    """A graph captured with a split plan (which uses the stream's workspace
    arena) is replayed after (a) an uncaptured call with a far larger plan on
    the same stream has grown that arena and (b) the caller has dropped its
    reference to the captured plan. Each replay equals the eager result."""
    import gc
    d = draw([600, 150], 4, seed=71, state_std=0.1, device=DEV)
    cu_h = d["cu_seqlens_host"]
    p = kda.plan_split(cu_h, 4, [20, 0], 12, device=DEV)
    cu = p.cu_device()
    o_buf = torch.empty_like(d["q"])
    s_buf = torch.empty_like(d["initial_state"])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, cu_seqlens_host=cu_h,
                    initial_state=d["initial_state"], final_state=s_buf, out=o_buf, plan=p)
    small_ws = p.info()["workspace_bytes"]
    del p
    gc.collect()
    # a segmented plan on the same stream needs far more workspace: the arena grows
    big = draw([3000, 1000], 8, seed=5, state_std=0.1, device=DEV)
    p_big = kda.plan_segments(big["cu_seqlens_host"], 8, 64, device=DEV)
    assert p_big.info()["workspace_bytes"] > 4 * small_ws + (1 << 20)
    with torch.cuda.stream(stream):
        o_big, s_big = kda.prefill(big["q"], big["k"], big["v"], big["g"], big["beta"],
                                   cu_seqlens_host=big["cu_seqlens_host"], initial_state=big["initial_state"],
                                   output_final_state=True, plan=p_big)
    torch.cuda.current_stream().wait_stream(stream)
    o_ser, s_ser = run(d, mode=False)
    for trial in range(3):
        o_buf.zero_()
        s_buf.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_buf, o_ser) and torch.equal(s_buf, s_ser), "replay %d differs from serial" % trial
        with torch.cuda.stream(stream):  # eager work on the capture stream between replays
            kda.prefill(big["q"], big["k"], big["v"], big["g"], big["beta"],
                        cu_seqlens_host=big["cu_seqlens_host"], initial_state=big["initial_state"],
                        output_final_state=True, plan=p_big)
        torch.cuda.synchronize()
    o_ref, s_ref = oracle(big)
    assert_close("out(big)", o_big, o_ref)
