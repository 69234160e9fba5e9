"""GPU parity of the HIP decode step against the fp64 CPU oracle.

The step advances each sequence's fp32 state by one token, in place. Bar: the
bf16 output and the complete fp32 state within atol = rtol = 1e-2 of the
oracle (the correctness gate of "fix(cake_kda): support non-aligned recurrent
prefill head counts", FlashInfer pull request #4351, description); several
steps in a row must agree with the oracle's prefill over the same tokens, and
a decode step after the GPU prefill must continue it. All calls go through the
C ABI (libkda.so) via the ctypes binding.
"""
import numpy as np
import pytest
import torch

import kda_chunked_delta_amd as kda
from kda_inputs import decode_workload, draw, draw_decode
from oracle import reference as ref

from test_gpu_parity import DEV, assert_close, say

pytestmark = pytest.mark.gpu


def decode_gpu(d, scale=1.0):
    state = d["state"].clone()
    o = kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], state, scale=scale)
    torch.cuda.synchronize()
    return o, state


@pytest.mark.parametrize("N,H", [(1, 1), (3, 5), (7, 12), (64, 32)])
def test_decode_matches_oracle(N, H):
    say("case decode N=%d H=%d" % (N, H))
    d = draw_decode(N, H, seed=100 + N * H, state_std=0.1, device=DEV)
    o, s = decode_gpu(d, scale=0.75)
    o_ref, s_ref = ref.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], scale=0.75)
    assert_close("out", o, o_ref)
    assert_close("state", s, s_ref)


def test_decode_strong_decay_and_large_state():
    say("case decode strong decay, state N(0, 1)")
    d = draw_decode(16, 8, seed=7, state_std=1.0, g_scale=2.0, device=DEV)
    o, s = decode_gpu(d)
    o_ref, s_ref = ref.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    assert_close("out", o, o_ref)
    assert_close("state", s, s_ref)


def test_decode_zero_state_and_empty_batch():
    say("case decode zero state; N = 0")
    d = draw_decode(5, 3, seed=9, state_std=None, device=DEV)
    o, s = decode_gpu(d)
    o_ref, s_ref = ref.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    assert_close("out", o, o_ref)
    assert_close("state", s, s_ref)
    e = draw_decode(0, 3, seed=9, device=DEV)
    o = kda.decode(e["q"], e["k"], e["v"], e["g"], e["beta"], e["state"])
    torch.cuda.synchronize()
    assert o.shape == (0, 3, 128)


def test_decode_steps_match_oracle_prefill():
    """T decode steps on the GPU == the oracle's recurrence over the T tokens."""
    N, H, T = 5, 4, 24
    say("case decode %d steps N=%d H=%d" % (T, N, H))
    d = draw([T] * N, H, seed=31, state_std=0.1, device=DEV)
    state = d["initial_state"].clone()
    per_seq = lambda x, t: x.view(N, T, *x.shape[1:])[:, t].contiguous()
    outs = []
    for t in range(T):
        outs.append(kda.decode(per_seq(d["q"], t), per_seq(d["k"], t), per_seq(d["v"], t),
                               per_seq(d["g"], t), per_seq(d["beta"], t), state))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1).reshape(N * T, H, 128)
    o_ref, s_ref = ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens_host"],
                                   d["initial_state"])
    assert_close("out", o, o_ref)
    assert_close("state", state, s_ref)


def test_decode_continues_gpu_prefill():
    """GPU prefill of each sequence but its last token, then one GPU decode
    step with the last tokens == the oracle over whole sequences."""
    lengths, H = [1, 17, 40, 2], 6
    say("case prefill + decode lengths", lengths)
    d = draw(lengths, H, seed=47, state_std=0.1, device=DEV)
    cu = d["cu_seqlens_host"]
    head = torch.cat([torch.arange(cu[i], cu[i + 1] - 1) for i in range(len(lengths))]).to(DEV)
    last = torch.tensor([cu[i + 1] - 1 for i in range(len(lengths))], device=DEV)
    cu_head = [0]
    for L in lengths:
        cu_head.append(cu_head[-1] + L - 1)
    pick = lambda x, idx: x.index_select(0, idx).contiguous()
    state = d["initial_state"].clone()
    o_head, _ = kda.prefill(pick(d["q"], head), pick(d["k"], head), pick(d["v"], head), pick(d["g"], head),
                            pick(d["beta"], head), cu_seqlens=cu_head, initial_state=state,
                            final_state=state)
    o_last = kda.decode(pick(d["q"], last), pick(d["k"], last), pick(d["v"], last), pick(d["g"], last),
                        pick(d["beta"], last), state)
    torch.cuda.synchronize()
    o_ref, s_ref = ref.recurrent_c(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"])
    assert_close("out_prefix", o_head, o_ref[head.cpu().numpy()])
    assert_close("out_last", o_last, o_ref[last.cpu().numpy()])
    assert_close("state", state, s_ref)


def test_decode_is_bitwise_repeatable_and_accepts_4d():
    say("case decode repeatability, [N, 1, H, 128] inputs")
    d = draw_decode(9, 7, seed=3, device=DEV)
    o1, s1 = decode_gpu(d)
    o2, s2 = decode_gpu(d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    state = d["state"].clone()
    u = lambda x: x.unsqueeze(1)
    o4 = kda.decode(u(d["q"]), u(d["k"]), u(d["v"]), u(d["g"]), u(d["beta"]), state)
    torch.cuda.synchronize()
    assert o4.shape == (9, 1, 7, 128)
    assert torch.equal(o4.squeeze(1), o1) and torch.equal(state, s1)


def test_decode_full_size_sampled():
    """The benchmark's decode batch (256 sequences x 32 heads), in the launch
    configuration the benchmark times, checked on 48 sampled (sequence, head)
    pairs."""
    say("case decode_n256_h32 sampled")
    d = decode_workload("decode_n256_h32", device=DEV)
    o, s = decode_gpu(d)
    rng = np.random.default_rng(5)
    pairs = [(int(n), int(h)) for n, h in zip(rng.integers(0, d["N"], 48), rng.integers(0, d["H"], 48))]
    pairs += [(0, 0), (d["N"] - 1, d["H"] - 1)]
    ns = torch.tensor([p[0] for p in pairs])
    hs = torch.tensor([p[1] for p in pairs])
    sub = lambda x: x.cpu()[ns, hs].unsqueeze(1)
    o_ref, s_ref = ref.decode_step(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["beta"]),
                                   sub(d["state"]))
    assert_close("out", o.cpu()[ns, hs], o_ref[:, 0])
    assert_close("state", s.cpu()[ns, hs], s_ref[:, 0])


def test_decode_with_a_state_pool_and_slot_table():
    """Sequences address a pool of states through a slot table; a slot of -1
    or past the pool skips its sequence (zero output, no state touched)."""
    N, H, n_slots = 6, 4, 9
    say("case decode slots N=%d H=%d pool=%d" % (N, H, n_slots))
    d = draw_decode(N, H, seed=61, state_std=0.1, device=DEV)
    pool = 0.1 * torch.randn(n_slots, H, 128, 128, generator=torch.Generator(device=DEV).manual_seed(62),
                             device=DEV)
    slots = torch.tensor([7, 2, -1, 0, 9, 4], dtype=torch.int32, device=DEV)
    before = pool.clone()
    o = kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, slots=slots)
    torch.cuda.synchronize()
    live = [n for n, s in enumerate(slots.tolist()) if 0 <= s < n_slots]
    idx = torch.tensor(live)
    sl = slots.cpu()[idx].long()
    sub = lambda x: x.cpu()[idx]
    o_ref, s_ref = ref.decode_step(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["g"]), sub(d["beta"]),
                                   before.cpu()[sl])
    assert_close("out", o.cpu()[idx], o_ref)
    assert_close("state", pool.cpu()[sl], s_ref)
    skipped = [n for n in range(N) if n not in live]
    assert torch.count_nonzero(o[skipped]) == 0
    untouched = [s for s in range(n_slots) if s not in sl.tolist()]
    assert torch.equal(pool[untouched], before[untouched])
