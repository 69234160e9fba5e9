"""GPU tests of the bf16 beta and bf16 state options of kda_prefill_ex.

bf16 beta is widened exactly, so results must equal, bit for bit, those of the
fp32 path on the widened beta; a bf16 initial state is read exactly and the
state is carried in fp32, so the output must equal the fp32 path's on the
widened state and the bf16 final state must be its fp32 final state rounded to
nearest even. Against the oracle the usual bar holds (atol = rtol = 1e-2).
All calls go through the C ABI (libkda.so) via the ctypes binding."""
import pytest
import torch

import kda_chunked_delta_amd as kda
from kda_inputs import draw
from oracle import reference as ref

from test_gpu_parity import DEV, assert_close, say

pytestmark = pytest.mark.gpu


def run(d, beta, s0, plan=None, final=None):
    o, s = kda.prefill(d["q"], d["k"], d["v"], d["g"], beta, cu_seqlens=d["cu_seqlens"],
                       cu_seqlens_host=d["cu_seqlens_host"], initial_state=s0, output_final_state=True,
                       final_state=final, plan=plan)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("lengths,H", [([33, 100, 1], 4), ([17, 0, 64], 12)])
def test_bf16_beta_is_the_widened_fp32_path(lengths, H):
    say("case bf16 beta", lengths, H)
    d = draw(lengths, H, seed=sum(lengths) + 3, state_std=0.1, device=DEV)
    b16 = d["beta"].to(torch.bfloat16)
    o1, s1 = run(d, b16, d["initial_state"])
    o2, s2 = run(d, b16.float(), d["initial_state"])
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], b16, d["cu_seqlens_host"], d["initial_state"])
    assert_close("out", o1, o_ref)
    assert_close("final_state", s1, s_ref)


@pytest.mark.parametrize("lengths,H", [([33, 100, 1], 4), ([300, 47], 8)])
def test_bf16_states(lengths, H):
    say("case bf16 states", lengths, H)
    d = draw(lengths, H, seed=sum(lengths) + 5, state_std=0.1, device=DEV)
    s0_16 = d["initial_state"].to(torch.bfloat16)
    o1, s1 = run(d, d["beta"], s0_16)
    assert s1.dtype == torch.bfloat16
    o2, s2 = run(d, d["beta"], s0_16.float())
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2.to(torch.bfloat16))
    o_ref, s_ref = ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens_host"], s0_16)
    assert_close("out", o1, o_ref)
    assert_close("final_state", s1, s_ref)
    # in place, and with no initial state
    st = s0_16.clone()
    o3, s3 = run(d, d["beta"], st, final=st)
    assert s3.data_ptr() == st.data_ptr() and torch.equal(st, s1) and torch.equal(o3, o1)
    o4, s4 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                         cu_seqlens_host=d["cu_seqlens_host"], output_final_state=True, state_dtype=torch.bfloat16)
    o5, s5 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                         cu_seqlens_host=d["cu_seqlens_host"], output_final_state=True)
    torch.cuda.synchronize()
    assert s4.dtype == torch.bfloat16 and torch.equal(o4, o5) and torch.equal(s4, s5.to(torch.bfloat16))


def test_bf16_options_on_the_cp_path():
    """Forced CP with bf16 beta and bf16 states: bitwise the serial result."""
    lengths, H = [3000, 700], 4
    say("case bf16 beta + states, CP vs serial", lengths)
    d = draw(lengths, H, seed=77, state_std=0.1, device=DEV)
    b16, s0_16 = d["beta"].to(torch.bfloat16), d["initial_state"].to(torch.bfloat16)
    o1, s1 = run(d, b16, s0_16)
    cp = kda.plan_segments(d["cu_seqlens_host"], H, 64, device=DEV)
    assert cp.info()["uses_cp"]
    o2, s2 = run(d, b16, s0_16, plan=cp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    o_ref, s_ref = ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], b16, d["cu_seqlens_host"], s0_16)
    assert_close("out", o1, o_ref)
    assert_close("final_state", s1, s_ref)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_bf16_options_on_warm_start_splits(g_scale):
    """Warm-start splits with bf16 beta and bf16 states, not aliased and in
    place, under the workloads' decay (the segment stands) and weak decay
    (the fix-up reruns it): bitwise the serial result."""
    lengths, H = [700, 300], 4
    say("case bf16 beta + states, split vs serial, g x", g_scale)
    d = draw(lengths, H, seed=78, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    b16, s0_16 = d["beta"].to(torch.bfloat16), d["initial_state"].to(torch.bfloat16)
    o1, s1 = run(d, b16, s0_16)
    sp = kda.plan_split(d["cu_seqlens_host"], H, [20, 12], 12, device=DEV)
    o2, s2 = run(d, b16, s0_16, plan=sp)
    assert s2.dtype == torch.bfloat16
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    st = s0_16.clone()
    o3, s3 = run(d, b16, st, plan=sp, final=st)
    assert s3.data_ptr() == st.data_ptr() and torch.equal(o3, o1) and torch.equal(st, s1)


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_bf16_options_on_warm_start_cp(g_scale):
    """Warm-start CP with bf16 beta and bf16 states: the serial result under
    the workloads' decay, the segmented CP result under weak decay."""
    lengths, H = [1600, 90], 4
    say("case bf16 beta + states, warm-start CP, g x", g_scale)
    d = draw(lengths, H, seed=79, state_std=0.1, device=DEV)
    d["g"] = d["g"] * g_scale
    b16, s0_16 = d["beta"].to(torch.bfloat16), d["initial_state"].to(torch.bfloat16)
    cu = d["cu_seqlens_host"]
    ref_plan = None if g_scale == 1.0 else kda.plan_segments(cu, H, 32, device=DEV)
    o1, s1 = run(d, b16, s0_16, plan=ref_plan)
    wp = kda.plan_warm_cp(cu, H, 32, 12, device=DEV)
    o2, s2 = run(d, b16, s0_16, plan=wp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
