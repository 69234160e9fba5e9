"""Seeded synthetic inputs for the KDA forward prefill.

This module only draws random tensors with the workloads' shapes and value
distributions; it holds none of the method's arithmetic, so both the GPU
library's tests and the CPU oracle may consume what it produces.

Recipe (per workload seed s): sequence lengths drawn first by a CPU
torch.Generator seeded with s, so a workload's batch structure is the same on
every device; then one torch.Generator on the generating device, seeded with
s, draws in this order q, k, v, g, beta, initial state:
  q, k  : randn fp32, L2-normalised per (token, head) over D, rounded to bf16
  v     : randn, rounded to bf16
  g     : -softplus(g_scale * randn) fp32 log-decay per key channel
  beta  : sigmoid(randn) fp32
  S0    : state_std * randn fp32, shape [N, H, D, D], or None
"N(0, s)" is read as s * randn (a standard deviation).
Decode inputs (draw_decode) follow the same recipe for one token per
sequence: q, k, v, g, beta shaped [N, H, D] / [N, H], then the state
[N, H, D, D].
Tensor values differ between a CPU and a GPU generator; the oracle always
evaluates the exact tensors the library consumed, so parity does not depend
on where the inputs were drawn.
"""
from __future__ import annotations

import torch

D = 128

# name -> (seed, description, spec)
WORKLOADS = {
    # one sequence of 64 tokens, one head, zero initial state
    "t64_h1": dict(seed=1000, lengths=[64], H=1, state_std=None, g_scale=1.0),
    # twelve (non-multiple-of-eight) heads, two equal sequences of 32 tokens
    "h12_2x32": dict(seed=1001, lengths=[32, 32], H=12, state_std=0.1, g_scale=1.0),
    # twelve heads, two sequences of 33 tokens: two chunks plus a one-token tail
    "h12_2x33": dict(seed=1001, lengths=[33, 33], H=12, state_std=0.1, g_scale=1.0),
    # twelve heads, packed varlen cu_seqlens = [0, 32, 35]
    "h12_32_3": dict(seed=1001, lengths=[32, 3], H=12, state_std=0.1, g_scale=1.0),
    # eight sequences with lengths uniform in [512, 4096], 32 heads (headline)
    "varlen8_h32": dict(seed=1002, lengths=("uniform", 8, 512, 4096), H=32, state_std=0.1,
                        g_scale=1.0),
    # one 65536-token sequence, 8 heads (few heads: needs intracard CP)
    "long65536_h8": dict(seed=1003, lengths=[65536], H=8, state_std=0.1, g_scale=1.0),
    # 16 sequences of 8192 tokens, 64 heads, stronger decay, zero initial state
    "batch16x8192_h64": dict(seed=1004, lengths=[8192] * 16, H=64, state_std=None,
                             g_scale=2.0),
}


def draw(lengths, H, *, seed, state_std=0.1, g_scale=1.0, device="cpu", D=D, qk_heads=None):
    """Draw one packed-varlen input set.

    lengths: list of sequence lengths, or ("uniform", n, lo, hi) for n lengths
    drawn uniformly from [lo, hi] inclusive by a CPU generator seeded with seed.
    Returns a dict with q, k, v (bf16), g, beta (fp32), cu_seqlens (int32, on
    the device), cu_seqlens_host (python list), initial_state (fp32 or None).
    qk_heads: q and k get that many heads instead of H (grouped value heads).
    """
    if isinstance(lengths, tuple) and lengths[0] == "uniform":
        _, n, lo, hi = lengths
        lgen = torch.Generator(device="cpu")
        lgen.manual_seed(int(seed))
        lengths = torch.randint(lo, hi + 1, (n,), generator=lgen).tolist()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    lengths = [int(x) for x in lengths]
    Tt = sum(lengths)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit_rows(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    Hk = H if qk_heads is None else qk_heads
    q = unit_rows(normal(Tt, Hk, D)).to(torch.bfloat16)
    k = unit_rows(normal(Tt, Hk, D)).to(torch.bfloat16)
    v = normal(Tt, H, D).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(g_scale * normal(Tt, H, D))
    beta = torch.sigmoid(normal(Tt, H))
    s0 = None
    if state_std is not None:
        s0 = state_std * normal(len(lengths), H, D, D)
    return dict(q=q, k=k, v=v, g=g, beta=beta,
                cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
                cu_seqlens_host=cu, initial_state=s0, H=H, lengths=lengths)


# name -> spec of a decode batch (one token per sequence)
DECODE_WORKLOADS = {
    # 256 sequences x 32 heads, state N(0, 0.1): a serving-size decode batch
    "decode_n256_h32": dict(seed=1005, N=256, H=32, state_std=0.1, g_scale=1.0),
}


def draw_decode(N, H, *, seed, state_std=0.1, g_scale=1.0, device="cpu", D=D, qk_heads=None):
    """One decode batch: q, k, v (bf16) [N, H, D], g (fp32) [N, H, D],
    beta (fp32) [N, H], state (fp32) [N, H, D, D] (zeros if state_std is None)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit_rows(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)

    Hk = H if qk_heads is None else qk_heads
    q = unit_rows(normal(N, Hk, D)).to(torch.bfloat16)
    k = unit_rows(normal(N, Hk, D)).to(torch.bfloat16)
    v = normal(N, H, D).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(g_scale * normal(N, H, D))
    beta = torch.sigmoid(normal(N, H))
    if state_std is None:
        state = torch.zeros(N, H, D, D, device=device, dtype=torch.float32)
    else:
        state = state_std * normal(N, H, D, D)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state=state, N=N, H=H)


def decode_workload(name, device="cpu"):
    """Inputs of a named decode batch (see DECODE_WORKLOADS)."""
    spec = dict(DECODE_WORKLOADS[name])
    out = draw_decode(spec.pop("N"), spec.pop("H"), seed=spec.pop("seed"), device=device, **spec)
    out["name"] = name
    return out


def workload(name, device="cpu"):
    """Inputs of a named workload (see WORKLOADS)."""
    spec = dict(WORKLOADS[name])
    seed = spec.pop("seed")
    lengths = spec.pop("lengths")
    H = spec.pop("H")
    out = draw(lengths, H, seed=seed, device=device, **spec)
    out["name"] = name
    return out
