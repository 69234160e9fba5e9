"""kda_prefill_noalloc, the entry point for callers that cannot allocate: its
workspace is the library's static per-device scratch instead of a per-stream
arena. Its results must be bitwise those of kda_prefill_ex with the same plan
(the same kernels run on the same inputs), call after call, with the scratch
keeping the previous call's contents. Calls go through the C ABI (ctypes)."""
import ctypes

import pytest
import torch

import kda_chunked_delta_amd as kda
from kda_inputs import draw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def call(entry, d, plan, s0, sT, out, beta=None, state_bf16=False):
    L = kda.lib()
    ctx = kda.context(DEV)
    beta = d["beta"] if beta is None else beta
    opts = kda.PrefillOpts(0, int(beta.dtype == torch.bfloat16), int(state_bf16))
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = getattr(L, entry)(ctx.handle, plan.handle, ctypes.byref(opts), ptr(d["q"]), ptr(d["k"]), ptr(d["v"]),
                           ptr(d["g"]), ptr(beta), ptr(plan.cu_device()), 1.0, ptr(s0), ptr(sT), ptr(out),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, L.kda_last_error().decode()


def both(d, plan, in_place=False, beta=None):
    """(out, final) of kda_prefill_ex and of kda_prefill_noalloc."""
    res = []
    for entry in ("kda_prefill_ex", "kda_prefill_noalloc"):
        out = torch.full_like(d["v"], float("nan"))
        if in_place:
            s0 = d["initial_state"].clone()
            sT = s0
        else:
            s0 = d["initial_state"]
            sT = torch.full_like(s0, float("nan"))
        st, msg = call(entry, d, plan, s0, sT, out, beta=beta)
        assert st == 0, (entry, msg)
        torch.cuda.synchronize()
        res.append((out, sT))
    return res


def test_scratch_size_is_stated():
    assert kda.lib().kda_noalloc_scratch_bytes() == 32 << 20


@pytest.mark.parametrize("g_scale", [1.0, 0.05])
def test_noalloc_equals_prefill_ex_on_two_calls_in_a_row(g_scale):
    """A split plan (carries, end states and flags in the workspace), then a
    smaller split plan with a bf16 beta (which is widened into the
    workspace too), then the first again with the state updated in place.
    Under weak decay (g x 0.05) the warm-start segments are rerun from their
    carries, which the scratch holds."""
    big = draw([1000, 700, 300], 8, seed=91, state_std=0.1, device=DEV)
    small = draw([200, 64], 4, seed=92, state_std=0.1, device=DEV)
    for d in (big, small):
        d["g"].mul_(g_scale)
    p_big = kda.plan_split(big["cu_seqlens_host"], 8, [30, 20, 0], 12, device=DEV)
    p_small = kda.plan_split(small["cu_seqlens_host"], 4, [6, 0], 4, device=DEV)
    assert 0 < p_small.info()["workspace_bytes"] < p_big.info()["workspace_bytes"] < 32 << 20
    say("case split plans, g_scale", g_scale)
    (o_ex, s_ex), (o_na, s_na) = both(big, p_big)
    assert torch.equal(o_ex, o_na) and torch.equal(s_ex, s_na)
    (o_ex, s_ex), (o_na, s_na) = both(small, p_small, beta=small["beta"].to(torch.bfloat16))
    assert torch.equal(o_ex, o_na) and torch.equal(s_ex, s_na)
    (o_ex, s_ex), (o_na, s_na) = both(big, p_big, in_place=True)
    assert torch.equal(o_ex, o_na) and torch.equal(s_ex, s_na)


def test_noalloc_serial_and_forced_cp_plans():
    """A serial plan (no workspace) and a forced-CP plan small enough for the
    scratch (K1 records, summaries and carries in it)."""
    d = draw([900, 33, 0, 250], 6, seed=93, state_std=0.1, device=DEV)
    cu_h = d["cu_seqlens_host"]
    for p in (kda.plan(cu_h, 6, device=DEV), kda.plan_segments(cu_h, 6, 8, device=DEV)):
        say("case plan", p.info()["uses_cp"], p.info()["workspace_bytes"])
        assert p.info()["workspace_bytes"] < 32 << 20
        (o_ex, s_ex), (o_na, s_na) = both(d, p)
        assert torch.equal(o_ex, o_na) and torch.equal(s_ex, s_na)


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    d = draw([8192], 8, seed=94, state_std=0.1, device=DEV)
    p = kda.plan_segments(d["cu_seqlens_host"], 8, 64, device=DEV)
    assert p.info()["workspace_bytes"] > 32 << 20
    out = torch.full_like(d["v"], float("nan"))
    st, msg = call("kda_prefill_noalloc", d, p, d["initial_state"], None, out)
    torch.cuda.synchronize()
    assert st == 1 and "static scratch" in msg
    assert torch.isnan(out.float()).all()  # nothing was launched


def test_noalloc_through_the_binding():
    d = draw([300, 47], 4, seed=95, state_std=0.1, device=DEV)
    cu_h = d["cu_seqlens_host"]
    p = kda.plan_split(cu_h, 4, [8, 0], 4, device=DEV)
    o1, s1 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens_host=cu_h,
                         initial_state=d["initial_state"], output_final_state=True, plan=p)
    o2, s2 = kda.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens_host=cu_h,
                         initial_state=d["initial_state"], output_final_state=True, plan=p, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
