"""Host-side tests of the C-ABI library (no GPU needed): exported symbols,
the planner and argument validation. No compute entry point is called."""
import ctypes
import os
import re

import pytest

import kda_chunked_delta_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kda_create", "kda_destroy", "kda_plan_prefill", "kda_prefill", "kda_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(kda_lib):
    lib = ctypes.CDLL(kda.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, "declared in include/kda.h but not exported: %s" % missing


def test_record_size_matches_header(kda_lib):
    m = re.search(r"#define KDA_RECORD_BYTES (\d+)", open(HEADER).read())
    assert int(m.group(1)) == kda.RECORD_BYTES


def test_version(kda_lib):
    assert b"gfx950" in kda_lib.kda_version()


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------
def cu_of(lengths):
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    return cu


def test_serial_plan_orders_longest_first(kda_lib):
    lengths = [100, 4096, 17, 0, 2000]
    p = kda.plan_host(cu_of(lengths), H=4, n_cus=256)
    info = p.info()
    assert info["uses_cp"] == 0
    assert info["total_chunks"] == sum((L + 15) // 16 for L in lengths)
    units = p.units()
    assert sorted(u["seq"] for u in units) == list(range(len(lengths)))
    chunks = [u["n_chunks"] for u in units]
    assert chunks == sorted(chunks, reverse=True)
    assert all(u["n_segments"] == 1 for u in units)
    # the fused serial path needs no workspace
    assert info["k1_materialized"] == 0 and info["workspace_bytes"] == 0


def test_materialized_plan_sizes_records(kda_lib, monkeypatch):
    monkeypatch.setenv("KDA_MATERIALIZE_K1", "1")
    info = kda.plan_host(cu_of([100, 4096]), H=4, n_cus=256).info()
    # one record per (chunk, head)
    assert info["k1_materialized"] == 1
    assert info["workspace_bytes"] >= info["total_chunks"] * 4 * kda.RECORD_BYTES


def test_auto_plan_splits_few_head_long_sequence(kda_lib):
    """One 65536-token sequence with 8 heads: AUTO picks warm-start CP (all
    segments in the fused launch), keeping the segmented pipeline, with its
    own segment table, as the fallback."""
    p = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp="auto")
    info = p.info()
    assert info["uses_cp"] == 1 and info["n_cp_seqs"] == 1
    assert info["warm_cp"] == 1 and info["split_warm_chunks"] >= 1
    S, W = info["warm_cp_seg_chunks"], info["split_warm_chunks"]
    units = p.units()
    segs = sorted((u["chunk0"], u["n_chunks"], u["warm_chunks"]) for u in units)
    # chunk-aligned, contiguous, covering all 4096 chunks; every segment but
    # the first warms up, and none starts before its warm-up
    pos = 0
    for c0, n, w in segs:
        assert c0 == pos and n >= 1 and n <= S
        assert w == (W if c0 > 0 else 0) and c0 >= w
        pos += n
    assert pos == 4096
    # speculation slots: every warm-start segment (the last one included)
    assert info["n_warm_segments"] == len(segs) - 1
    # the fallback's segmented tables: pre_scan over all but the last segment
    assert info["n_prescan"] >= 1 and info["k1_materialized"] == 1
    assert 0 < info["est_warm_cp_us"] < info["est_cp_us"] < info["est_serial_us"]
    # forced CP stays the segmented pipeline alone
    forced = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=True).info()
    assert forced["uses_cp"] == 1 and forced["warm_cp"] == 0


def test_auto_plan_declines_saturated_and_short(kda_lib):
    # batch x heads already fills the machine
    assert kda.plan_host(cu_of([8192] * 16), H=64, n_cus=256, use_intracard_cp="auto").info()["uses_cp"] == 0
    # sequences too short to split
    assert kda.plan_host(cu_of([512] * 4), H=2, n_cus=256, use_intracard_cp="auto").info()["uses_cp"] == 0
    # off means off
    assert kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=False).info()["uses_cp"] == 0


def test_plan_depends_on_cu_count(kda_lib):
    small = kda.plan_host([0, 32768], H=16, n_cus=32, use_intracard_cp="auto").info()
    big = kda.plan_host([0, 32768], H=16, n_cus=256, use_intracard_cp="auto").info()
    assert big["n_units"] >= small["n_units"]
    assert big["n_cus"] == 256 and small["n_cus"] == 32


def test_ragged_batch_splits_only_long_sequences(kda_lib):
    lengths = [32768, 300, 50, 20000]
    p = kda.plan_host(cu_of(lengths), H=4, n_cus=256, use_intracard_cp=True)
    units = p.units()
    by_seq = {}
    for u in units:
        by_seq.setdefault(u["seq"], []).append(u)
    assert len(by_seq[1]) == 1 and len(by_seq[2]) == 1
    assert len(by_seq[0]) > 1


def headline_lengths():
    # the headline workload's lengths: 8 uniform in [512, 4096], CPU generator, seed 1002
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(1002)
    return torch.randint(512, 4097, (8,), generator=g).tolist()


def test_auto_plan_splits_the_tail_of_one_round(kda_lib):
    """Eight sequences x 32 heads fill 256 CUs once; the longest chains set
    the time, so AUTO runs the longest sequences as a first segment plus a
    warm-start segment."""
    lengths = headline_lengths()
    nch = [(L + 15) // 16 for L in lengths]
    p = kda.plan_host(cu_of(lengths), H=32, n_cus=256, use_intracard_cp="auto")
    info = p.info()
    assert info["uses_cp"] == 0 and info["k1_materialized"] == 0
    assert info["n_split_seqs"] >= 1 and info["split_warm_chunks"] >= 1
    W, WW = info["split_warm_chunks"], info["split_warm_work"]
    # the warm-up counted at its cost: W chunks, each advancing two states
    assert W < WW < 2 * W
    by_seq = {}
    for u in p.units():
        by_seq.setdefault(u["seq"], []).append(u)
    n_split = 0
    for i, us in by_seq.items():
        us.sort(key=lambda u: u["chunk0"])
        assert sum(u["n_chunks"] for u in us) == nch[i]
        if len(us) == 2:
            n_split += 1
            first, second = us
            assert first["chunk0"] == 0 and first["warm_chunks"] == 0
            assert second["chunk0"] == first["n_chunks"] >= W and second["warm_chunks"] == W
        else:
            assert len(us) == 1 and us[0]["warm_chunks"] == 0
    assert n_split == info["n_split_seqs"]
    # the split sequences are the longest ones
    split_seqs = [i for i, us in by_seq.items() if len(us) == 2]
    assert min(nch[i] for i in split_seqs) >= max(nch[i] for i in by_seq if i not in split_seqs)
    # carry, end state and flags of each warm-start segment
    assert info["workspace_bytes"] >= n_split * 32 * 2 * 128 * 128 * 4
    # the warm-start segments run longest-first with their warm-up counted
    work = [u["n_chunks"] + (WW if u["warm_chunks"] else 0) for u in p.units()]
    assert work == sorted(work, reverse=True)


def _fused_model_us(work, n_cus):
    """The planner's fused-kernel schedule model: units start longest first,
    one per CU, and every running unit advances one chunk per interval, the
    interval rising with the fraction of busy CUs (1.21 us alone, 1.60 us with
    all busy, piecewise linear through the measured shape)."""
    import heapq
    xs = [0.0, 0.125, 0.25, 0.5, 0.75, 1.0]
    ys = [0.0, 0.046, 0.061, 0.096, 0.47, 1.0]

    def interval(busy):
        x = min(1.0, max(0.0, busy / n_cus))
        i = 0
        while i < 4 and x > xs[i + 1]:
            i += 1
        return 1.21 + 0.39 * (ys[i] + (ys[i + 1] - ys[i]) * (x - xs[i]) / (xs[i + 1] - xs[i]))

    work = sorted(work, reverse=True)
    heap, nxt, prog, t = [], 0, 0.0, 0.0
    while nxt < len(work) and len(heap) < n_cus:
        heapq.heappush(heap, float(work[nxt]))
        nxt += 1
    while heap:
        f = heap[0]
        t += (f - prog) * interval(len(heap))
        prog = f
        while heap and heap[0] <= prog:
            heapq.heappop(heap)
        while nxt < len(work) and len(heap) < n_cus:
            heapq.heappush(heap, prog + work[nxt])
            nxt += 1
    return t


def test_split_search_is_at_least_the_uniform_grid(kda_lib):
    """The split search starts from the grid of uniform fractions (the k
    longest sequences split at the same fraction f) and only moves split
    points while the modelled time falls: its estimate is the model's time
    of the plan's own units, and no grid point models faster."""
    lengths = headline_lengths()
    nch = [(L + 15) // 16 for L in lengths]
    H, n_cus = 32, 256
    p = kda.plan_host(cu_of(lengths), H=H, n_cus=n_cus, use_intracard_cp="auto")
    info = p.info()
    W, WW = info["split_warm_chunks"], info["split_warm_work"]
    work = [u["n_chunks"] + (WW if u["warm_chunks"] else 0) for u in p.units()] * H
    t_plan = _fused_model_us(work, n_cus)
    assert abs(info["est_split_us"] - (t_plan + 5.0)) < 1e-3
    order = sorted(range(len(nch)), key=lambda i: -nch[i])
    best_grid = 1e300
    for k in range(1, len(nch) + 1):
        for fi in range(6, 13):
            f = 0.05 * fi
            units = list(nch)
            ok = True
            for i in order[:k]:
                a = int(round(nch[i] * f + 1e-9))
                if a < W or nch[i] - a < 1 or nch[i] < 4 * W:
                    ok = False
                    break
                units[i] = a
                units.append(nch[i] - a + WW)
            if not ok:
                break
            best_grid = min(best_grid, _fused_model_us(units * H, n_cus))
    assert t_plan <= best_grid + 1e-6


def test_auto_plan_splits_nothing_else(kda_lib, monkeypatch):
    # several rounds of units smooth the tail
    assert kda.plan_host(cu_of([8192] * 16), H=64, n_cus=256, use_intracard_cp="auto").info()["n_split_seqs"] == 0
    # off means off; CP plans segment instead
    assert kda.plan_host(cu_of(headline_lengths()), H=32, n_cus=256).info()["n_split_seqs"] == 0
    assert kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp="auto").info()["n_split_seqs"] == 0
    # short sequences
    assert kda.plan_host(cu_of([100, 64]), H=2, n_cus=256, use_intracard_cp="auto").info()["n_split_seqs"] == 0
    # the fused kernel is the only one that runs warm-start segments
    monkeypatch.setenv("KDA_MATERIALIZE_K1", "1")
    assert kda.plan_host(cu_of(headline_lengths()), H=32, n_cus=256,
                         use_intracard_cp="auto").info()["n_split_seqs"] == 0


def test_split_warm_chunks_is_env_overridable(kda_lib, monkeypatch):
    monkeypatch.setenv("KDA_SPLIT_WARM_CHUNKS", "12")
    info = kda.plan_host(cu_of(headline_lengths()), H=32, n_cus=256, use_intracard_cp="auto").info()
    assert info["n_split_seqs"] == 0 or info["split_warm_chunks"] == 12


def test_forced_cp_segment_length_follows_the_measured_sweep(kda_lib, monkeypatch):
    """One 65536-token sequence with 8 heads on 256 CUs: the segmented model
    picks 128-chunk segments (one workgroup per CU), which measured fastest
    of 32, 48, 64, 128 and 256 chunks under both strong and weak decay. K2
    streams the records at the same rate with one or two workgroups per CU,
    so it is priced by the longer of one unit's chain and the HBM stream;
    with a slower chain step (its constant overridden) the chain term wins
    and the model prefers 64-chunk segments."""
    info = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=True).info()
    assert info["uses_cp"] == 1 and info["warm_cp"] == 0
    assert info["max_unit_chunks"] == 128 and info["n_units"] == 32
    monkeypatch.setenv("KDA_CP_REC_CHUNK_US_ALONE", "3.0")
    slow_chain = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=True).info()
    assert slow_chain["max_unit_chunks"] == 64 and slow_chain["est_cp_us"] > info["est_cp_us"]


def test_planner_constants_are_env_overridable(kda_lib, monkeypatch):
    base = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=True).info()
    monkeypatch.setenv("KDA_CP_MIN_SEG_CHUNKS", "1024")
    big = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp=True).info()
    assert big["max_unit_chunks"] >= 1024 > base["max_unit_chunks"]


@pytest.mark.parametrize("cu,H,err", [
    ([1, 5], 2, "cu_seqlens[0]"),
    ([0, 5, 3], 2, "decreases"),
    ([0, 5], 0, "H must be"),
])
def test_plan_rejects_bad_input(kda_lib, cu, H, err):
    with pytest.raises(kda.KDAError, match=re.escape(err)) as e:
        kda.plan_host(cu, H=H, n_cus=256)
    assert e.value.status == 1


def test_plan_rejects_other_head_dims(kda_lib):
    arr = (ctypes.c_int32 * 2)(0, 16)
    h = ctypes.c_void_p()
    st = kda_lib.kda_plan_prefill_host(256, arr, 1, 2, 64, 64, 0, ctypes.byref(h))
    assert st == 2 and b"128" in kda_lib.kda_last_error()


# ---------------------------------------------------------------------------
# validation (addresses only; never dereferenced)
# ---------------------------------------------------------------------------
class FakeBuffers:
    def __init__(self, Tt, H, N):
        act = Tt * H * 128 * 2
        self.size = dict(act=act, g=Tt * H * 128 * 4, beta=Tt * H * 4, state=N * H * 128 * 128 * 4,
                         cu=(N + 1) * 4)
        base = 1 << 40
        self.addr = {}
        for name, kind in (("q", "act"), ("k", "act"), ("v", "act"), ("g", "g"), ("beta", "beta"),
                           ("cu", "cu"), ("s0", "state"), ("sT", "state"), ("out", "act")):
            self.addr[name] = base
            base += (self.size[kind] + 4096) // 256 * 256

    def call(self, lib, plan, **over):
        a = dict(self.addr)
        a.update(over)
        P = lambda x: ctypes.c_void_p(x) if x else None
        return lib.kda_prefill_validate(plan.handle, P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]),
                                        P(a["beta"]), P(a["cu"]), ctypes.c_float(a.get("scale", 1.0)),
                                        P(a["s0"]), P(a["sT"]), P(a["out"]))


@pytest.fixture
def setup(kda_lib):
    p = kda.plan_host([0, 40, 100], H=3, n_cus=256)
    return kda_lib, p, FakeBuffers(100, 3, 2)


def test_validate_accepts_good_call(setup):
    lib, p, fb = setup
    assert fb.call(lib, p) == 0
    assert fb.call(lib, p, s0=0) == 0                      # no initial state
    assert fb.call(lib, p, sT=0) == 0                      # no final state
    assert fb.call(lib, p, s0=0, sT=0) == 0                # neither
    assert fb.call(lib, p, sT=fb.addr["s0"]) == 0          # in place


def test_validate_rejects_aliasing(setup):
    lib, p, fb = setup
    assert fb.call(lib, p, out=fb.addr["q"]) == 3
    assert fb.call(lib, p, out=fb.addr["v"] + 256) == 3
    assert fb.call(lib, p, sT=fb.addr["s0"] + 4096) == 3   # partial state overlap
    assert b"partially overlaps" in lib.kda_last_error()
    assert fb.call(lib, p, sT=fb.addr["g"]) == 3
    assert fb.call(lib, p, out=fb.addr["sT"]) == 3


def test_validate_rejects_null_and_misaligned(setup):
    lib, p, fb = setup
    assert fb.call(lib, p, q=0) == 1
    assert fb.call(lib, p, cu=0) == 1
    assert fb.call(lib, p, k=fb.addr["k"] + 8) == 1
    assert b"aligned" in lib.kda_last_error()
    assert fb.call(lib, p, scale=float("nan")) == 1


def test_host_plan_cannot_execute(setup):
    lib, p, fb = setup
    # kda_prefill needs a context; with a NULL context it fails before any HIP call
    P = lambda x: ctypes.c_void_p(x)
    a = fb.addr
    st = lib.kda_prefill(None, p.handle, P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                         P(a["cu"]), ctypes.c_float(1.0), P(a["s0"]), P(a["sT"]), P(a["out"]), None)
    assert st == 1 and b"ctx" in lib.kda_last_error()


# ---------------------------------------------------------------------------
# decode validation (addresses only; never dereferenced)
# ---------------------------------------------------------------------------
def decode_validate(lib, N, H, over=None, dk=128, dv=128, Hk=None):
    NH, Hk = N * H, H if Hk is None else Hk
    size = dict(q=N * Hk * 256, k=N * Hk * 256, v=NH * 256, g=NH * 512, beta=NH * 4, state=NH * 65536, out=NH * 256)
    base, addr = 1 << 40, {}
    for name in ("q", "k", "v", "g", "beta", "state", "out"):
        addr[name] = base
        base += (size[name] + 4096) // 256 * 256
    addr.update(over or {})
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.kda_decode_validate(N, H, Hk, dk, dv, P(addr["q"]), P(addr["k"]), P(addr["v"]), P(addr["g"]),
                                   P(addr["beta"]), ctypes.c_float(addr.get("scale", 1.0)), P(addr["state"]),
                                   P(addr["out"])), addr


def test_decode_validate(kda_lib):
    lib = kda_lib
    st, a = decode_validate(lib, 64, 12)
    assert st == 0
    assert decode_validate(lib, 0, 12, dict(q=0, state=0))[0] == 0        # empty batch: nothing to check
    assert decode_validate(lib, 4, 2, dk=64)[0] == 2
    assert decode_validate(lib, -1, 2)[0] == 1
    assert decode_validate(lib, 4, 0)[0] == 1
    assert decode_validate(lib, 4, 2, dict(state=0))[0] == 1
    assert decode_validate(lib, 4, 2, dict(scale=float("inf")))[0] == 1
    assert decode_validate(lib, 4, 2, dict(g=a["g"] + 8))[0] == 1
    assert b"aligned" in lib.kda_last_error()
    _, a = decode_validate(lib, 4, 2)
    assert decode_validate(lib, 4, 2, dict(out=a["q"]))[0] == 3
    assert decode_validate(lib, 4, 2, dict(state=a["beta"]))[0] == 3
    assert decode_validate(lib, 4, 2, dict(out=a["state"] + 1024))[0] == 3
    # grouped value heads: 12 value heads over 4 q/k heads; 5 does not divide 12
    assert decode_validate(lib, 4, 12, Hk=4)[0] == 0
    assert decode_validate(lib, 4, 12, Hk=5)[0] == 1
    assert decode_validate(lib, 4, 12, Hk=0)[0] == 1


def test_decode_needs_context(kda_lib):
    _, a = decode_validate(kda_lib, 4, 2)
    P = lambda x: ctypes.c_void_p(x)
    st = kda_lib.kda_decode(None, 4, 2, 2, 128, 128, P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]),
                            ctypes.c_float(1.0), P(a["state"]), P(a["out"]), None)
    assert st == 1 and b"ctx" in kda_lib.kda_last_error()


def test_prefill_ex_validate(kda_lib):
    """kda_prefill_ex_validate sizes q/k by the q/k head count, beta and the
    states by their dtypes."""
    lib = kda_lib
    p = kda.plan_host([0, 40, 100], H=6, n_cus=256)
    fb = FakeBuffers(100, 6, 2)
    a = dict(fb.addr)
    P = lambda x: ctypes.c_void_p(x) if x else None

    def call(Hk, beta16=0, state16=0, **o):
        b = dict(a, **o)
        opts = kda.PrefillOpts(Hk, beta16, state16)
        return lib.kda_prefill_ex_validate(
            p.handle, ctypes.byref(opts), *(P(b[n]) for n in ("q", "k", "v", "g", "beta", "cu")),
            ctypes.c_float(1.0), P(b["s0"]), P(b["sT"]), P(b["out"]))
    assert call(6) == 0 and call(3) == 0 and call(2) == 0 and call(1) == 0 and call(0) == 0
    assert call(4) == 1 and b"multiple" in lib.kda_last_error()
    assert call(-1) == 1
    assert lib.kda_prefill_ex_validate(p.handle, None, *(P(a[n]) for n in ("q", "k", "v", "g", "beta", "cu")),
                                       ctypes.c_float(1.0), P(a["s0"]), P(a["sT"]), P(a["out"])) == 0
    # q sized for 2 q/k heads still may not overlap out
    assert call(2, q=a["out"] + 256) == 3
    # bf16 beta needs only 2-byte alignment; fp32 beta 4
    assert call(6, beta16=1, beta=a["beta"] + 2) == 0
    assert call(6, beta=a["beta"] + 2) == 1
    # a bf16 state is half the bytes: a final state right behind a bf16 initial state is disjoint
    half = 2 * 6 * 128 * 128 * 2
    assert call(6, state16=1, sT=a["s0"] + half) == 0
    assert call(6, state16=0, sT=a["s0"] + half) == 3


def test_decode_slots_validate(kda_lib):
    lib = kda_lib
    N, H, n_slots = 4, 2, 10
    base, addr = 1 << 40, {}
    size = dict(q=N * H * 256, k=N * H * 256, v=N * H * 256, g=N * H * 512, beta=N * H * 4,
                state=n_slots * H * 65536, slots=N * 4, out=N * H * 256)
    for name in ("q", "k", "v", "g", "beta", "state", "slots", "out"):
        addr[name] = base
        base += (size[name] + 4096) // 256 * 256
    P = lambda x: ctypes.c_void_p(x) if x else None

    def call(ns=n_slots, **o):
        a = dict(addr, **o)
        return lib.kda_decode_slots_validate(N, H, H, 128, 128, P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]),
                                             P(a["beta"]), ctypes.c_float(1.0), P(a["state"]), ns, P(a["slots"]),
                                             P(a["out"]))
    assert call() == 0
    assert call(ns=-1) == 1
    assert call(slots=0) == 1 and b"without a slot table" in lib.kda_last_error()   # n_slots != N
    assert call(ns=N, slots=0) == 0
    assert call(slots=addr["slots"] + 2) == 1
    assert call(slots=addr["state"] + 4096) == 3      # the table may not live inside the pool
    assert call(out=addr["state"] + 65536 * 9) == 3


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before
    touching any device."""
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_plan_workspace_bytes(kda_lib, monkeypatch):
    p = kda.plan_host([0, 65536], H=8, n_cus=256, use_intracard_cp="auto")
    info = p.info()
    assert info["uses_cp"] and info["workspace_bytes"] > 0
    assert kda_lib.kda_plan_workspace_bytes(p.handle) == info["workspace_bytes"]
    assert kda_lib.kda_plan_workspace_bytes(None) == 0
    serial = kda.plan_host([0, 100, 300], H=4, n_cus=256)
    assert kda_lib.kda_plan_workspace_bytes(serial.handle) == 0
