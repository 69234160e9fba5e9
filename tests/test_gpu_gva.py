"""GPU parity with grouped value heads (GVA): q and k with Hk heads serve
H = G * Hk value heads, value head h reading q/k head h // G. The oracle
expands q and k to the value heads (oracle.reference.gva_expand) and runs its
recurrence. Bar as everywhere: atol = rtol = 1e-2 on the bf16 output and the
complete fp32 state, bitwise equality between the serial and CP paths.
All calls go through the C ABI (libkda.so) via the ctypes binding."""
import numpy as np
import pytest
import torch

import kda_chunked_delta_amd as kda
from kda_inputs import draw, draw_decode
from oracle import reference as ref

from test_gpu_parity import DEV, assert_close, say

pytestmark = pytest.mark.gpu


def oracle_gva(d):
    H = d["v"].shape[1]
    q, k = ref.gva_expand(d["q"], d["k"], H)
    return ref.recurrent_c(q, k, d["v"], d["g"], d["beta"], d["cu_seqlens_host"], d["initial_state"])


@pytest.mark.parametrize("lengths,Hk,H", [([33, 100, 1], 2, 8), ([64, 17], 3, 6), ([50], 1, 4), ([40, 0, 9], 4, 4)])
def test_gva_prefill_matches_oracle(lengths, Hk, H):
    say("case gva prefill lengths", lengths, "Hk", Hk, "H", H)
    d = draw(lengths, H, seed=sum(lengths) + 10 * Hk, state_std=0.1, device=DEV, qk_heads=Hk)
    o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=d["initial_state"],
                       output_final_state=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_gva(d)
    assert_close("out", o, o_ref)
    assert_close("final_state", s, s_ref)


def test_gva_cp_is_bitwise_equal_to_serial():
    lengths, Hk, H = [3000, 700], 2, 4
    say("case gva cp vs serial", lengths)
    d = draw(lengths, H, seed=5, state_std=0.1, device=DEV, qk_heads=Hk)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    kw = dict(cu_seqlens=d["cu_seqlens"], cu_seqlens_host=d["cu_seqlens_host"],
              initial_state=d["initial_state"], output_final_state=True)
    o1, s1 = kda.prefill(*args, use_intracard_cp=False, **kw)
    cp = kda.plan_segments(d["cu_seqlens_host"], H, 64, device=DEV)
    assert cp.info()["uses_cp"]
    o2, s2 = kda.prefill(*args, plan=cp, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle_gva(d)
    assert_close("out", o1, o_ref)
    assert_close("final_state", s1, s_ref)


def test_gva_decode_matches_oracle():
    N, Hk, H = 6, 3, 12
    say("case gva decode N=%d Hk=%d H=%d" % (N, Hk, H))
    d = draw_decode(N, H, seed=21, state_std=0.1, device=DEV, qk_heads=Hk)
    state = d["state"].clone()
    o = kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    q, k = ref.gva_expand(d["q"], d["k"], H)
    o_ref, s_ref = ref.decode_step(q, k, d["v"], d["g"], d["beta"], d["state"])
    assert_close("out", o, o_ref)
    assert_close("state", state, s_ref)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_gva_warm_start_split_is_bitwise_equal_to_serial(g_scale):
    """Grouped value heads on a warm-start split plan: the segment stands or
    is rerun by the fix-up, and either way equals serial bit for bit."""
    lengths, Hk, H = [600, 200], 2, 8
    say("case GVA split", lengths, Hk, H, "g x", g_scale)
    d = draw(lengths, H, seed=61, state_std=0.1, device=DEV, qk_heads=Hk)
    d["g"] = d["g"] * g_scale
    o1, s1 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                         cu_seqlens_host=d["cu_seqlens_host"], initial_state=d["initial_state"],
                         output_final_state=True)
    p = kda.plan_split(d["cu_seqlens_host"], H, [18, 0], 12, device=DEV)
    o2, s2 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                         cu_seqlens_host=d["cu_seqlens_host"], initial_state=d["initial_state"],
                         output_final_state=True, plan=p)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = oracle_gva(d)
    assert_close("out", o2, o_ref)
    assert_close("final_state", s2, s_ref)


def test_gva_warm_start_cp_is_bitwise_equal_to_serial():
    lengths, Hk, H = [1200, 50], 2, 6
    d = draw(lengths, H, seed=62, state_std=0.1, device=DEV, qk_heads=Hk)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    kw = dict(cu_seqlens=d["cu_seqlens"], cu_seqlens_host=d["cu_seqlens_host"],
              initial_state=d["initial_state"], output_final_state=True)
    o1, s1 = kda.prefill(*args, **kw)
    o2, s2 = kda.prefill(*args, plan=kda.plan_warm_cp(d["cu_seqlens_host"], H, 24, 12, device=DEV), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
