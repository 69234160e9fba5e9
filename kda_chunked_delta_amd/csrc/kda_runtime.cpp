// Host runtime of the KDA forward-prefill library: context, planner, per-stream
// workspace arena, argument validation and kernel dispatch behind the C ABI of
// include/kda.h.
//
// Structure follows "feat(kda/sm90): FlashKDA prefill port + intracard-CP
// prefill" (cuLA pull request #103): the planner returns the plan the executor
// runs and a trivial plan means serial (reviewer notes); the executor makes no
// decisions; the workspace arena is reused across calls (description). The
// review thread of that pull request found a race when scratch buffers are
// shared across streams, so arenas here are keyed by stream.
#include "kda.h"

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kda_launch.h"
#include "kda_decode_launch.h"

using namespace kda;

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status hip_fail(hipError_t e, const char* what) {
    return fail(KDA_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per-device addresses of the static scratch of kda_prefill_noalloc, each
// looked up once, with its device current.
hipError_t device_scratch(int device, void** out) {
    static std::mutex mu;
    static std::unordered_map<int, void*> addr;
    std::lock_guard<std::mutex> lk(mu);
    auto it = addr.find(device);
    if (it != addr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = static_scratch_address(&ptr);
    if (prev >= 0 && prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess) return e;
    addr[device] = ptr;
    *out = ptr;
    return hipSuccess;
}

double env_double(const char* name, double dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    char* e = nullptr;
    const double v = strtod(s, &e);
    return (e && *e == 0 && std::isfinite(v) && v > 0) ? v : dflt;
}

// Planner cost model, in microseconds. The constants were fitted on MI355X
// from per-kernel timings of this library's kernels (environment-
// overridable, as the pull request's planner constants are):
//   fused      one chunk step of a fused serial workgroup (one per CU)
//   k1         K1 of one (chunk, head) with its record written and both
//              pre_scan summaries advanced (B, and the transfer M while any
//              tile of it lives), per CU, at full load; priced at weak
//              decay, where the transfer lives through the whole segment
//              (the worst case)
//   rec        one chunk step of a K2 workgroup over materialised records
//   merge      one segment step of the carry merge (weak decay: the worst
//              case; under decay the transfers vanish and it costs little)
//   launch     one kernel launch
struct PlannerConsts {
    double fused_us, k1_us, rec_us, merge_us, launch_us;
    double k1_alone_us;   // K1 with few CUs busy (k1_us: all busy)
    double rec_alone_us;  // K2 over records, one workgroup's chunk step (rec_us: per CU, HBM-bound)
    int min_seg_chunks;  // shortest segment the planner will form
    // fused kernel interval per chunk against the fraction of busy CUs:
    // alone_us with few busy, full_us with all busy, in between the shape
    // measured on MI355X (the shader clock falls as more CUs work)
    double alone_us, full_us;
    int split_warm;      // warm-up chunks of a warm-start segment
    // a warm-up chunk's cost in the schedule model, in main-chunk intervals
    // (both states, the transfer and the state from zero, advance in it)
    double warm_cost;
};

PlannerConsts planner_consts() {
    PlannerConsts c;
    // fitted at steady clocks on the 65536-token, 8-head workload with
    // segments of 64, 96, 128, 160, 192 and 256 chunks (512 .. 128
    // workgroups) under weak decay (g x 0.05): K1 with both summaries 250,
    // 331, 237, 276, 317 and 369 us, the merge 2.3 us per segment step while
    // the transfers live, segment-K2 150, 185, 154, 170, 184 and 229 us. And
    // on the fused kernel's interval with few CUs busy.
    c.fused_us = env_double("KDA_CP_FUSED_CHUNK_US", 1.21);
    c.k1_us = env_double("KDA_CP_K1_CHUNK_US", 1.85);
    c.k1_alone_us = env_double("KDA_CP_K1_CHUNK_US_ALONE", 1.44);
    c.rec_us = env_double("KDA_CP_REC_CHUNK_US", 1.16);
    c.rec_alone_us = env_double("KDA_CP_REC_CHUNK_US_ALONE", 0.89);
    c.merge_us = env_double("KDA_CP_MERGE_SEG_US", 2.3);
    c.launch_us = env_double("KDA_CP_LAUNCH_US", 5.0);
    c.min_seg_chunks = (int)env_double("KDA_CP_MIN_SEG_CHUNKS", 64.0);
    c.alone_us = env_double("KDA_FUSED_CHUNK_US_ALONE", 1.21);
    c.full_us = env_double("KDA_FUSED_CHUNK_US_FULL", 1.60);
    c.split_warm = (int)env_double("KDA_SPLIT_WARM_CHUNKS", 12.0);
    // fitted on the plans it yields: with 1.0, 1.2 and 1.6 the searched
    // split plan of the 8-sequence, 32-head batch ran 0.2597, 0.2601 and
    // 0.2545 ms (a warm-up interval itself takes about as long as a main
    // one; the factor also stands for what the schedule model leaves out)
    c.warm_cost = env_double("KDA_SPLIT_WARM_COST", 1.6);
    return c;
}

// The warm-up of W chunks in chunk intervals.
int warm_work(int W, const PlannerConsts& pc) { return W > 0 ? (int)std::lround(pc.warm_cost * W) : 0; }

// Interval of the fused kernel per chunk with `busy` of n_cus CUs working.
double fused_interval_us(int busy, int n_cus, const PlannerConsts& pc) {
    static const double xs[] = {0.0, 0.125, 0.25, 0.5, 0.75, 1.0};
    // measured at steady clocks: 1.21, 1.23, 1.23, 1.25, 1.39 and 1.60 us
    // per chunk with 8, 32, 64, 128, 192 and 256 of 256 CUs busy
    static const double ys[] = {0.0, 0.046, 0.061, 0.096, 0.47, 1.0};
    const double x = std::min(1.0, std::max(0.0, (double)busy / n_cus));
    int i = 0;
    while (i < 4 && x > xs[i + 1]) ++i;
    const double phi = ys[i] + (ys[i + 1] - ys[i]) * (x - xs[i]) / (xs[i + 1] - xs[i]);
    return pc.alone_us + (pc.full_us - pc.alone_us) * phi;
}

// Time of the fused kernel over work units of the given chunk counts,
// started longest first on n_cus CUs (one workgroup per CU), every running
// unit advancing one chunk per interval at the current occupancy. With
// copies > 1, `work` is one of `copies` identical groups of units (the heads
// of a batch) and the group runs on n_cus / copies CUs: the same timeline as
// all groups together, since identical units start and finish together.
double simulate_fused_us(std::vector<int> work, int n_cus, const PlannerConsts& pc, int copies = 1) {
    std::sort(work.begin(), work.end(), std::greater<int>());
    const int slots = n_cus / copies;
    std::vector<double> heap;  // finish progress of running units (min-heap)
    auto cmp = std::greater<double>();
    size_t next = 0;
    double progress = 0.0, t = 0.0;
    while (next < work.size() && (int)heap.size() < slots) {
        heap.push_back((double)work[next++]);
        std::push_heap(heap.begin(), heap.end(), cmp);
    }
    while (!heap.empty()) {
        const double f = heap.front();
        t += (f - progress) * fused_interval_us((int)heap.size() * copies, n_cus, pc);
        progress = f;
        while (!heap.empty() && heap.front() <= progress) {
            std::pop_heap(heap.begin(), heap.end(), cmp);
            heap.pop_back();
        }
        while (next < work.size() && (int)heap.size() < slots) {
            heap.push_back(progress + work[next++]);
            std::push_heap(heap.begin(), heap.end(), cmp);
        }
    }
    return t;
}

}  // namespace

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
struct kda_plan {
    kda_plan_info info{};
    std::vector<int32_t> cu;            // host copy of cu_seqlens
    std::vector<ChunkDesc> chunks;      // K1 items (global chunk order)
    std::vector<UnitDesc> units;        // K2 units, launch order
    std::vector<MergeDesc> merges;      // CP merge items
    std::vector<UnitDesc> fixups;       // warm-start segments, as rerun from their carry
    std::vector<UnitDesc> cp_units;     // warm-start CP: the segmented fallback's K2 units
    std::vector<UnitDesc> alt_units;    // split plans: the batch unsplit (the exact path)
    std::vector<UnitDesc> k1_units;     // segmented pipeline: K1 with the B summaries, one per K2 unit
    std::vector<MergeSeg> merge_segs;   // segmented pipeline: one merge workgroup row per segment
    // workspace layout (byte offsets into the arena)
    size_t off_rec = 0, off_b = 0, off_m = 0, off_mlive = 0, off_carry = 0;
    size_t off_spec_states = 0, off_spec_flags = 0, off_gate = 0;
    // device copy of the tables
    int device = -1;
    void* dev_tables = nullptr;
    size_t dev_off_chunks = 0, dev_off_units = 0, dev_off_merges = 0, dev_off_fixups = 0;
    size_t dev_off_cp_units = 0, dev_off_alt_units = 0, dev_off_k1_units = 0, dev_off_merge_segs = 0;
    // Speculation feedback, outside graph capture: a speculative call (the
    // first, then every 64th) copies its outcome (split plans: the speculation
    // flags; warm-start CP: the gate) into pinned host memory and records an
    // event; a later call
    // that finds the copy complete and a failure in it turns speculation off
    // for this plan, which then runs its exact path (unsplit serial, or the
    // segmented pipeline ungated). Results are the same bits either way.
    mutable std::mutex spec_mu;
    mutable int32_t* spec_host = nullptr;
    mutable size_t spec_words = 0;
    mutable hipEvent_t spec_event = nullptr;
    mutable bool spec_pending = false;
    mutable bool spec_off = false;
    mutable uint64_t spec_calls = 0;  // the outcome is copied on the first call and every 64th
};

namespace {

// Serial estimate (fused kernel, one (sequence, head) workgroup per CU):
// the longest sequence, or the total work spread over the CUs, whichever is
// larger.
double est_serial(const std::vector<int>& nch, int H, int n_cus, const PlannerConsts& pc) {
    long long tot = 0;
    int mx = 0;
    for (int n : nch) { tot += n; mx = std::max(mx, n); }
    return pc.fused_us * std::max((double)mx, std::ceil((double)tot * H / n_cus)) + pc.launch_us;
}

// Segmented estimate for segment length `seg` (chunks): K1 materialised for
// every chunk, with both pre_scan summaries of every segment but the last of
// each split sequence, a serial merge over segments, then K2 over all units.
// K1 and the merge are priced at weak decay, where no transfer vanishes (the
// worst case).
double est_cp(const std::vector<int>& nch, int H, int n_cus, int seg, const PlannerConsts& pc) {
    long long tot = 0;
    int longest_unit = 0, max_segs = 0;
    std::vector<int> k1_work;  // K1 units of one head
    for (int n : nch) {
        tot += n;
        const int s = (n > seg) ? (n + seg - 1) / seg : 1;
        for (int j = 0; j < s; ++j) k1_work.push_back(std::min(seg, n - j * seg));
        if (s > 1) {
            max_segs = std::max(max_segs, s);
            longest_unit = std::max(longest_unit, seg);
        } else {
            longest_unit = std::max(longest_unit, n);
        }
    }
    if (max_segs == 0) return 1e300;
    // K1 runs the fused kernel's body (with the record writes) one workgroup
    // per CU: its schedule in the fused kernel's model, at K1's own interval
    PlannerConsts k1c = pc;
    k1c.alone_us = pc.k1_alone_us;
    k1c.full_us = pc.k1_us;
    const bool grouped = H <= n_cus && n_cus % H == 0;
    if (!grouped) {
        const std::vector<int> one = k1_work;
        for (int h = 1; h < H; ++h) k1_work.insert(k1_work.end(), one.begin(), one.end());
    }
    const double t_k1 = simulate_fused_us(k1_work, n_cus, k1c, grouped ? H : 1);
    const double t_merge = pc.merge_us * (max_segs - 1);
    // K2: the longest unit's chain, or the HBM stream over the CUs
    const double t_k2 = std::max(pc.rec_alone_us * longest_unit, pc.rec_us * std::ceil((double)tot * H / n_cus));
    return t_k1 + t_merge + t_k2 + 3 * pc.launch_us;
}

// Fused work of each unit when sequence i is split at chunk split[i]
// (0: not split): the first segment runs split[i] chunks, the warm-start
// segment the rest plus the warm-up's work.
std::vector<int> split_work(const std::vector<int>& nch, const std::vector<int>& split, int H, int warm) {
    std::vector<int> w;
    w.reserve(nch.size() * H * 2);
    for (size_t i = 0; i < nch.size(); ++i) {
        const int a = split[i];
        for (int h = 0; h < H; ++h) {
            if (a > 0) {
                w.push_back(a);
                w.push_back(nch[i] - a + warm);
            } else {
                w.push_back(nch[i]);
            }
        }
    }
    return w;
}

// Warm-start split search. First a grid: the k longest sequences split at
// the same fraction f of their chunks. Then, from the best few grid points,
// a coordinate descent that moves each split sequence's split point over a
// set of fractions, one sequence at a time, while the simulated time falls
// (a split's two pieces can then pair with different units in the
// schedule). Only for batches of at most a few rounds of units, where the
// longest chains make the tail. When H divides the CU count the simulation
// runs one head's units on its share of the CUs.
double best_split(const std::vector<int>& nch, int H, int n_cus, const PlannerConsts& pc,
                  std::vector<int>& split_out) {
    const int n = (int)nch.size();
    split_out.assign(n, 0);
    const int W = pc.split_warm;
    if ((long long)n * H > 4LL * n_cus || W < 1) return 1e300;
    const bool grouped = H <= n_cus && n_cus % H == 0;
    auto cost = [&](const std::vector<int>& sp) {
        return grouped ? simulate_fused_us(split_work(nch, sp, 1, warm_work(W, pc)), n_cus, pc, H)
                       : simulate_fused_us(split_work(nch, sp, H, warm_work(W, pc)), n_cus, pc);
    };
    auto valid = [&](int i, int a) { return a >= W && nch[i] - a >= 1 && nch[i] >= 4 * W; };
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return nch[x] > nch[y]; });
    std::vector<std::pair<double, std::vector<int>>> grid;
    std::vector<int> split(n, 0);
    for (int k = 1; k <= std::min(n, 8); ++k) {
        for (int fi = 6; fi <= 12; ++fi) {
            const double f = 0.05 * fi;
            std::fill(split.begin(), split.end(), 0);
            bool ok = true;
            for (int j = 0; j < k; ++j) {
                const int i = order[j];
                const int a = (int)std::lround(nch[i] * f);
                if (!valid(i, a)) { ok = false; break; }
                split[i] = a;
            }
            if (!ok) break;
            grid.emplace_back(cost(split), split);
        }
    }
    if (grid.empty()) return 1e300;
    std::stable_sort(grid.begin(), grid.end(),
                     [](const std::pair<double, std::vector<int>>& x, const std::pair<double, std::vector<int>>& y) {
                         return x.first < y.first;
                     });
    double best = grid[0].first;
    split_out = grid[0].second;
    static const double fracs[] = {0.25, 0.35, 0.45, 0.55, 0.65, 0.75};
    const size_t seeds = std::min<size_t>(grid.size(), 8);
    // grid and descent together simulate at most 64K units, so planning a
    // batch of many sequences stays cheap (the grid alone reaches that at
    // the largest shapes considered, n * H = 4 CUs' worth)
    const long long units_per_sim = (long long)(n + 8) * (grouped ? 1 : H);
    long long budget = 64 * 1024 - (long long)grid.size() * units_per_sim;
    for (size_t g = 0; g < seeds && budget > 0; ++g) {
        std::vector<int> cur = grid[g].second;
        double ct = grid[g].first;
        for (int sweep = 0; sweep < 3 && budget > 0; ++sweep) {
            bool improved = false;
            for (int i = 0; i < n && budget > 0; ++i) {
                if (cur[i] == 0) continue;
                for (double f : fracs) {
                    const int a = (int)std::lround(nch[i] * f);
                    if (a == cur[i] || !valid(i, a)) continue;
                    const int keep = cur[i];
                    cur[i] = a;
                    budget -= units_per_sim;
                    const double t = cost(cur);
                    if (t < ct - 1e-9) {
                        ct = t;
                        improved = true;
                    } else {
                        cur[i] = keep;
                    }
                }
            }
            if (!improved) break;
        }
        if (ct < best) {
            best = ct;
            split_out = cur;
        }
    }
    return best + pc.launch_us;
}

// seg_chunks > 0 forces that segment length on every longer sequence;
// force_split (per sequence, 0 = none) forces warm-start splits with
// force_warm warm-up chunks.
kda_status build_plan(int32_t n_cus, const int32_t* cu_host, int32_t n_seqs, int32_t H,
                      int32_t dk, int32_t dv, kda_cp_mode mode, int32_t seg_chunks,
                      kda_plan** out, const int32_t* force_split = nullptr, int32_t force_warm = 0,
                      int32_t force_warm_cp_seg = 0) {
    if (!out) return fail(KDA_ERR_INVALID, "kda_plan_prefill: out is NULL");
    *out = nullptr;
    if (dk != 128 || dv != 128)
        return fail(KDA_ERR_UNSUPPORTED, "kda_plan_prefill: dk = dv = 128 required (got dk=%d dv=%d)",
                    dk, dv);
    if (H < 1) return fail(KDA_ERR_INVALID, "kda_plan_prefill: H must be >= 1 (got %d)", H);
    if (n_seqs < 1) return fail(KDA_ERR_INVALID, "kda_plan_prefill: n_seqs must be >= 1 (got %d)", n_seqs);
    if (!cu_host) return fail(KDA_ERR_INVALID, "kda_plan_prefill: cu_seqlens_host is NULL");
    if (n_cus < 1) return fail(KDA_ERR_INVALID, "kda_plan_prefill: n_cus must be >= 1 (got %d)", n_cus);
    if (mode != KDA_CP_OFF && mode != KDA_CP_ON && mode != KDA_CP_AUTO)
        return fail(KDA_ERR_INVALID, "kda_plan_prefill: unknown cp mode %d", (int)mode);
    if (cu_host[0] != 0)
        return fail(KDA_ERR_INVALID, "kda_plan_prefill: cu_seqlens[0] must be 0 (got %d)", cu_host[0]);
    for (int i = 0; i < n_seqs; ++i)
        if (cu_host[i + 1] < cu_host[i])
            return fail(KDA_ERR_INVALID, "kda_plan_prefill: cu_seqlens decreases at index %d (%d -> %d)",
                        i, cu_host[i], cu_host[i + 1]);

    const PlannerConsts pc = planner_consts();
    kda_plan* p = new kda_plan();
    p->cu.assign(cu_host, cu_host + n_seqs + 1);
    std::vector<int> nch(n_seqs), chunk_base(n_seqs);
    long long total_chunks = 0;
    for (int i = 0; i < n_seqs; ++i) {
        const int L = cu_host[i + 1] - cu_host[i];
        nch[i] = (L + kChunk - 1) / kChunk;
        chunk_base[i] = (int)total_chunks;
        total_chunks += nch[i];
    }
    if (total_chunks > (1LL << 30)) {
        delete p;
        return fail(KDA_ERR_INVALID, "kda_plan_prefill: too many chunks (%lld)", total_chunks);
    }
    p->chunks.reserve(total_chunks);
    for (int i = 0; i < n_seqs; ++i)
        for (int c = 0; c < nch[i]; ++c) p->chunks.push_back(ChunkDesc{i, c});

    // segment length decision
    const double t_serial = est_serial(nch, H, n_cus, pc);
    double t_cp = 1e300;
    int seg = 0;
    if (seg_chunks > 0) {
        seg = seg_chunks;
        t_cp = est_cp(nch, H, n_cus, seg, pc);
    } else if (mode != KDA_CP_OFF) {
        const int mx = *std::max_element(nch.begin(), nch.end());
        for (int s = std::max(1, pc.min_seg_chunks); s < mx; s *= 2) {
            const double t = est_cp(nch, H, n_cus, s, pc);
            if (t < t_cp) { t_cp = t; seg = s; }
        }
        if (mode == KDA_CP_AUTO && !(t_cp < 0.9 * t_serial)) seg = 0;
    }
    // warm-start splits (fused serial path only)
    const bool materialize_env = env_double("KDA_MATERIALIZE_K1", 0.0) > 0.5;
    std::vector<int> split(n_seqs, 0);
    int warm = pc.split_warm;
    double t_split = 1e300, t_sim_serial = -1.0;
    if (force_split) {
        warm = force_warm;
        for (int i = 0; i < n_seqs; ++i) split[i] = force_split[i];
        t_split = simulate_fused_us(split_work(nch, split, H, warm_work(warm, pc)), n_cus, pc) + pc.launch_us;
    } else if (mode == KDA_CP_AUTO && seg == 0 && !materialize_env) {
        t_sim_serial = simulate_fused_us(split_work(nch, split, H, 0), n_cus, pc);
        std::vector<int> cand;
        t_split = best_split(nch, H, n_cus, pc, cand);
        if (t_split < 0.97 * t_sim_serial) split = cand;
    }
    int n_split = 0;
    for (int i = 0; i < n_seqs; ++i) n_split += split[i] > 0;
    // warm-start CP: every segment of the segmented plan runs in the fused
    // kernel (segments after the first as warm-start segments), and the
    // segmented pipeline is kept as a fallback, armed on the device only if
    // a warm-up transfer survives
    int wseg = 0;
    double t_wcp = 1e300;
    if (force_warm_cp_seg > 0) {
        wseg = force_warm_cp_seg;
        warm = force_warm;
        seg = force_warm_cp_seg;
    } else if (mode == KDA_CP_AUTO && seg > 0 && !materialize_env && pc.split_warm >= 1) {
        std::vector<int> cands;
        const int mx = *std::max_element(nch.begin(), nch.end());
        for (int b = 16; b <= mx; b *= 2)
            for (int s : {b, b + b / 2})
                if (s >= 2 * pc.split_warm && s < mx) cands.push_back(s);
        for (int s : cands) {
            std::vector<int> work;
            for (int i = 0; i < n_seqs; ++i)
                for (int h = 0; h < H; ++h)
                    for (int c0 = 0; c0 < std::max(nch[i], 1); c0 += s)
                        work.push_back(std::min(s, nch[i] - c0) + (c0 > 0 ? warm_work(pc.split_warm, pc) : 0));
            const double t = simulate_fused_us(work, n_cus, pc) + 6 * pc.launch_us;
            if (t < t_wcp) { t_wcp = t; wseg = s; }
        }
        if (!(t_wcp < 0.8 * t_cp)) wseg = 0;
        else warm = pc.split_warm;
    }

    // units
    int n_cp_seqs = 0, n_prescan = 0, n_carry = 0;
    std::vector<int> order(n_seqs);
    for (int i = 0; i < n_seqs; ++i) order[i] = i;
    int n_spec = 0;
    for (int i : order) {
        if (split[i] > 0) {
            // first segment from the initial state, writing its end state to a
            // carry slot; warm-start segment from its warm-up; the fix-up
            // table reruns the latter from that carry if its warm-up transfer
            // did not vanish
            const int a = split[i], carry = n_carry++, spec = n_spec++;
            p->units.push_back(UnitDesc{i, 0, a, chunk_base[i], -1, 0, 0, 2, 0, -1, carry, -1});
            p->units.push_back(UnitDesc{i, a, nch[i] - a, chunk_base[i] + a, -1, 1, 1, 2, warm, spec, -1, -1});
            p->fixups.push_back(UnitDesc{i, a, nch[i] - a, chunk_base[i] + a, carry, 1, 1, 2, 0, spec, -1, -1});
            continue;
        }
        const int s = (seg > 0 && nch[i] > seg) ? (nch[i] + seg - 1) / seg : 1;
        if (s == 1) {
            p->units.push_back(UnitDesc{i, 0, nch[i], chunk_base[i], -1, 1, 0, 1, 0, -1, -1, -1});
            p->k1_units.push_back(UnitDesc{i, 0, nch[i], chunk_base[i], -1, 0, 0, 1, 0, -1, -1, -1});
            continue;
        }
        MergeDesc md{i, s, n_carry, n_prescan};
        for (int j = 0; j < s; ++j) p->merge_segs.push_back(MergeSeg{(int32_t)p->merges.size(), j});
        p->merges.push_back(md);
        for (int j = 0; j < s; ++j) {
            const int c0 = j * seg, n = std::min(seg, nch[i] - c0);
            // segment j starts from carry j, or from B_{j-1} itself when the
            // transfer of segment j - 1 vanished
            p->units.push_back(UnitDesc{i, c0, n, chunk_base[i] + c0, n_carry + j, j == s - 1, j, s, 0, -1, -1,
                                        j > 0 ? n_prescan + j - 1 : -1});
            // K1 of its chunks, and (but for the last segment) its B summary
            p->k1_units.push_back(UnitDesc{i, c0, n, chunk_base[i] + c0, -1, 0, j, s, 0, -1,
                                           j < s - 1 ? n_prescan + j : -1, -1});
        }
        n_cp_seqs++;
        n_prescan += s - 1;
        n_carry += s;
    }
    int n_wspec = 0;
    if (wseg > 0) {
        // the classic tables above are the fallback; the fused launch runs
        // the warm-start segments
        p->cp_units.swap(p->units);
        for (int i = 0; i < n_seqs; ++i) {
            const int ns = nch[i] > 0 ? (nch[i] + wseg - 1) / wseg : 1;
            for (int j = 0; j < ns; ++j) {
                const int c0 = j * wseg, n = std::min(wseg, nch[i] - c0);
                const bool last = j == ns - 1;
                const int spec = (j > 0 || last) ? n_wspec++ : -1;
                // the last segment's end state is the final state; a warm-start
                // one leaves it in spec_states when the final state aliases
                // the initial state (published by the gated fix-up launch)
                p->units.push_back(UnitDesc{i, c0, std::max(n, 0), chunk_base[i] + c0, -1, last ? 1 : 0, j, ns,
                                            j > 0 ? warm : 0, spec, -1, -1});
                if (last)
                    p->fixups.push_back(UnitDesc{i, c0, n, chunk_base[i] + c0, -1, 1, j, ns, 0, spec, -1, -1});
            }
        }
        std::stable_sort(p->cp_units.begin(), p->cp_units.end(),
                         [](const UnitDesc& a, const UnitDesc& b) { return a.n_chunks > b.n_chunks; });
    }
    if (n_split > 0) {
        for (int i = 0; i < n_seqs; ++i)
            p->alt_units.push_back(UnitDesc{i, 0, nch[i], chunk_base[i], -1, 1, 0, 1, 0, -1, -1, -1});
        std::stable_sort(p->alt_units.begin(), p->alt_units.end(),
                         [](const UnitDesc& a, const UnitDesc& b) { return a.n_chunks > b.n_chunks; });
    }
    // longest chains first (a warm-start segment's warm-up counted at its cost)
    std::stable_sort(p->units.begin(), p->units.end(), [&](const UnitDesc& a, const UnitDesc& b) {
        return a.n_chunks + warm_work(a.warm, pc) > b.n_chunks + warm_work(b.warm, pc);
    });
    std::stable_sort(p->k1_units.begin(), p->k1_units.end(),
                     [](const UnitDesc& a, const UnitDesc& b) { return a.n_chunks > b.n_chunks; });

    // workspace layout
    // CP plans always materialise K1 (K1 once, then pre_scan and segment-K2
    // read its records); serial plans run the fused kernel unless asked not to.
    const bool materialize = n_cp_seqs > 0 || wseg > 0 || (materialize_env && n_split == 0);
    size_t off = 0;
    p->off_rec = off;
    if (materialize) off = align_up(off + (size_t)total_chunks * H * kRecBytes, 256);
    p->off_b = off;
    off = align_up(off + (size_t)n_prescan * H * kStateBytes, 256);
    p->off_m = off;
    off = align_up(off + (size_t)n_prescan * H * kStateBytes, 256);
    p->off_mlive = off;
    off = align_up(off + (size_t)n_prescan * H * 8 * sizeof(int32_t), 256);
    p->off_carry = off;
    off = align_up(off + (size_t)n_carry * H * kStateBytes, 256);
    const int n_spec_slots = std::max(n_spec, n_wspec);
    p->off_spec_states = off;
    off = align_up(off + (size_t)n_spec_slots * H * kStateBytes, 256);
    p->off_spec_flags = off;
    off = align_up(off + (size_t)n_spec_slots * H * 8 * sizeof(int32_t), 256);
    p->off_gate = off;
    if (wseg > 0) off = align_up(off + sizeof(int32_t), 256);

    kda_plan_info& in = p->info;
    in.n_seqs = n_seqs;
    in.H = H;
    in.dk = dk;
    in.dv = dv;
    in.total_tokens = cu_host[n_seqs];
    in.total_chunks = (int32_t)total_chunks;
    in.uses_cp = n_cp_seqs > 0;
    in.n_units = (int32_t)p->units.size();
    in.n_cp_seqs = n_cp_seqs;
    in.n_prescan = n_prescan;
    in.n_carry_slots = n_carry;
    in.max_unit_chunks = 0;
    for (const auto& u : p->units) in.max_unit_chunks = std::max(in.max_unit_chunks, u.n_chunks);
    in.n_cus = n_cus;
    in.workspace_bytes = off;
    in.est_serial_us = t_serial;
    in.est_cp_us = t_cp < 1e299 ? t_cp : -1.0;
    in.k1_materialized = materialize ? 1 : 0;
    in.n_split_seqs = n_split;
    in.split_warm_chunks = (n_split > 0 || wseg > 0) ? warm : 0;
    in.est_split_us = t_split < 1e299 ? t_split : -1.0;
    in.warm_cp = wseg > 0 ? 1 : 0;
    in.warm_cp_seg_chunks = wseg;
    in.n_warm_segments = n_wspec;
    in.est_warm_cp_us = t_wcp < 1e299 ? t_wcp : -1.0;
    in.split_warm_work = in.split_warm_chunks > 0 ? warm_work(in.split_warm_chunks, pc) : 0;
    if (wseg > 0) {
        in.n_units = (int32_t)p->units.size();
        in.max_unit_chunks = 0;
        for (const auto& u : p->units) in.max_unit_chunks = std::max(in.max_unit_chunks, u.n_chunks);
    }
    *out = p;
    return KDA_OK;
}

kda_status upload_plan(kda_plan* p, int device) {
    size_t off = 0;
    p->dev_off_chunks = off;
    off = align_up(off + p->chunks.size() * sizeof(ChunkDesc), 256);
    p->dev_off_units = off;
    off = align_up(off + p->units.size() * sizeof(UnitDesc), 256);
    p->dev_off_merges = off;
    off = align_up(off + p->merges.size() * sizeof(MergeDesc), 256);
    p->dev_off_fixups = off;
    off = align_up(off + p->fixups.size() * sizeof(UnitDesc), 256);
    p->dev_off_cp_units = off;
    off = align_up(off + p->cp_units.size() * sizeof(UnitDesc), 256);
    p->dev_off_alt_units = off;
    off = align_up(off + p->alt_units.size() * sizeof(UnitDesc), 256);
    p->dev_off_k1_units = off;
    off = align_up(off + p->k1_units.size() * sizeof(UnitDesc), 256);
    p->dev_off_merge_segs = off;
    off = align_up(off + p->merge_segs.size() * sizeof(MergeSeg), 256);
    std::vector<uint8_t> host(off, 0);
    if (!p->chunks.empty()) memcpy(&host[p->dev_off_chunks], p->chunks.data(), p->chunks.size() * sizeof(ChunkDesc));
    if (!p->units.empty()) memcpy(&host[p->dev_off_units], p->units.data(), p->units.size() * sizeof(UnitDesc));
    if (!p->merges.empty()) memcpy(&host[p->dev_off_merges], p->merges.data(), p->merges.size() * sizeof(MergeDesc));
    if (!p->fixups.empty()) memcpy(&host[p->dev_off_fixups], p->fixups.data(), p->fixups.size() * sizeof(UnitDesc));
    if (!p->cp_units.empty())
        memcpy(&host[p->dev_off_cp_units], p->cp_units.data(), p->cp_units.size() * sizeof(UnitDesc));
    if (!p->alt_units.empty())
        memcpy(&host[p->dev_off_alt_units], p->alt_units.data(), p->alt_units.size() * sizeof(UnitDesc));
    if (!p->k1_units.empty())
        memcpy(&host[p->dev_off_k1_units], p->k1_units.data(), p->k1_units.size() * sizeof(UnitDesc));
    if (!p->merge_segs.empty())
        memcpy(&host[p->dev_off_merge_segs], p->merge_segs.data(), p->merge_segs.size() * sizeof(MergeSeg));
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* d = nullptr;
    e = hipMalloc(&d, off);
    if (e == hipSuccess) e = hipMemcpy(d, host.data(), off, hipMemcpyHostToDevice);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        if (d) (void)hipFree(d);
        return hip_fail(e, "kda_plan_prefill: uploading plan tables");
    }
    p->dev_tables = d;
    p->device = device;
    return KDA_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

// ---------------------------------------------------------------------------
// context and arena
// ---------------------------------------------------------------------------
struct Arena {
    void* ptr = nullptr;
    size_t bytes = 0;
    // A call captured into a graph bakes this address into the graph, which
    // may be replayed at any time after: such memory is never freed before
    // kda_destroy (growing or evicting the arena retires it instead).
    bool captured = false;
};

struct TimedLaunch {
    const char* name;
    hipEvent_t beg, end;
};

struct kda_ctx {
    int device = 0;
    int n_cus = 0;
    hipDeviceProp_t prop{};
    std::mutex mu;
    std::unordered_map<hipStream_t, Arena> arenas;
    std::vector<void*> retired;  // arena memory that served a graph capture, freed in kda_destroy
    void* scratch = nullptr;     // this device's copy of the static scratch (kda_prefill_noalloc)
    bool poison = false;
    bool timing = false;
    std::vector<TimedLaunch> events;  // pool, reused across calls
    int n_timed = 0;
};

static const size_t kMaxArenas = 16;
static const int kMaxTimedLaunches = 4096;

// Run `launch` on `stream`; while the context's timing is on, bracket it with
// a pair of HIP events from the context's pool (ctx->mu held by the caller).
template <class F>
static hipError_t timed_launch(kda_ctx* ctx, hipStream_t stream, const char* name, F&& launch) {
    if (!ctx->timing) return launch();
    if (ctx->n_timed >= kMaxTimedLaunches) return launch();  // log full: run untimed
    if ((int)ctx->events.size() <= ctx->n_timed) {
        TimedLaunch t{name, nullptr, nullptr};
        hipError_t ee = hipEventCreate(&t.beg);
        if (ee == hipSuccess) ee = hipEventCreate(&t.end);
        if (ee != hipSuccess) return ee;
        ctx->events.push_back(t);
    }
    TimedLaunch& t = ctx->events[ctx->n_timed++];
    t.name = name;
    hipError_t ee = hipEventRecord(t.beg, stream);
    if (ee == hipSuccess) ee = launch();
    if (ee == hipSuccess) ee = hipEventRecord(t.end, stream);
    return ee;
}

extern "C" {

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_version(void) { return "kda-mi355x 0.1.0 (gfx950)"; }

kda_status kda_create(int device, kda_ctx** out) {
    if (!out) return fail(KDA_ERR_INVALID, "kda_create: out is NULL");
    *out = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= n)
        return fail(KDA_ERR_INVALID, "kda_create: device %d out of range (%d devices)", device, n);
    kda_ctx* c = new kda_ctx();
    c->device = device;
    e = hipGetDeviceProperties(&c->prop, device);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "hipGetDeviceProperties");
    }
    c->n_cus = c->prop.multiProcessorCount;
    // the device address of the static scratch, looked up once per device
    // with that device current
    e = device_scratch(device, &c->scratch);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "hipGetSymbolAddress (static scratch)");
    }
    const char* pz = getenv("KDA_DEBUG_POISON");
    c->poison = pz && *pz && strcmp(pz, "0") != 0;
    *out = c;
    return KDA_OK;
}

void kda_destroy(kda_ctx* c) {
    if (!c) return;
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
    for (auto& kv : c->arenas)
        if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    for (void* ptr : c->retired) (void)hipFree(ptr);
    for (auto& t : c->events) {
        (void)hipEventDestroy(t.beg);
        (void)hipEventDestroy(t.end);
    }
    if (prev >= 0) (void)hipSetDevice(prev);
    delete c;
}

kda_status kda_plan_prefill_host(int32_t n_cus, const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t H,
                                 int32_t dk, int32_t dv, kda_cp_mode mode, kda_plan** out) {
    return build_plan(n_cus, cu_seqlens_host, n_seqs, H, dk, dv, mode, 0, out);
}

kda_status kda_plan_prefill(kda_ctx* ctx, const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t H,
                            int32_t dk, int32_t dv, kda_cp_mode mode, kda_plan** out) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_plan_prefill: ctx is NULL");
    kda_status st = build_plan(ctx->n_cus, cu_seqlens_host, n_seqs, H, dk, dv, mode, 0, out);
    if (st != KDA_OK) return st;
    st = upload_plan(*out, ctx->device);
    if (st != KDA_OK) {
        delete *out;
        *out = nullptr;
    }
    return st;
}

kda_status kda_plan_prefill_segments(kda_ctx* ctx, const int32_t* cu_seqlens_host, int32_t n_seqs,
                                     int32_t H, int32_t dk, int32_t dv, int32_t seg_chunks,
                                     kda_plan** out) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_plan_prefill_segments: ctx is NULL");
    if (seg_chunks < 1)
        return fail(KDA_ERR_INVALID, "kda_plan_prefill_segments: seg_chunks must be >= 1 (got %d)", seg_chunks);
    kda_status st = build_plan(ctx->n_cus, cu_seqlens_host, n_seqs, H, dk, dv, KDA_CP_ON, seg_chunks, out);
    if (st != KDA_OK) return st;
    st = upload_plan(*out, ctx->device);
    if (st != KDA_OK) {
        delete *out;
        *out = nullptr;
    }
    return st;
}

kda_status kda_plan_prefill_split(kda_ctx* ctx, const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t H,
                                  int32_t dk, int32_t dv, const int32_t* split_chunk, int32_t warm_chunks,
                                  kda_plan** out) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_plan_prefill_split: ctx is NULL");
    if (!out) return fail(KDA_ERR_INVALID, "kda_plan_prefill_split: out is NULL");
    *out = nullptr;
    if (!split_chunk || !cu_seqlens_host || n_seqs < 1)
        return fail(KDA_ERR_INVALID, "kda_plan_prefill_split: split_chunk, cu_seqlens_host and n_seqs >= 1 required");
    if (warm_chunks < 1) return fail(KDA_ERR_INVALID, "kda_plan_prefill_split: warm_chunks must be >= 1 (got %d)",
                                     warm_chunks);
    for (int i = 0; i < n_seqs; ++i) {
        const int L = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
        const int nch = L > 0 ? (L + kChunk - 1) / kChunk : 0;
        const int a = split_chunk[i];
        if (a != 0 && (a < warm_chunks || a >= nch))
            return fail(KDA_ERR_INVALID, "kda_plan_prefill_split: sequence %d (%d chunks): split chunk %d must be 0 "
                                         "or in [warm_chunks=%d, chunks)", i, nch, a, warm_chunks);
    }
    kda_status st = build_plan(ctx->n_cus, cu_seqlens_host, n_seqs, H, dk, dv, KDA_CP_OFF, 0, out, split_chunk,
                               warm_chunks);
    if (st != KDA_OK) return st;
    st = upload_plan(*out, ctx->device);
    if (st != KDA_OK) {
        delete *out;
        *out = nullptr;
    }
    return st;
}

kda_status kda_plan_prefill_warm_cp(kda_ctx* ctx, const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t H,
                                    int32_t dk, int32_t dv, int32_t seg_chunks, int32_t warm_chunks,
                                    kda_plan** out) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_plan_prefill_warm_cp: ctx is NULL");
    if (seg_chunks < 1 || warm_chunks < 1 || warm_chunks > seg_chunks)
        return fail(KDA_ERR_INVALID, "kda_plan_prefill_warm_cp: need 1 <= warm_chunks <= seg_chunks (got %d, %d)",
                    warm_chunks, seg_chunks);
    kda_status st = build_plan(ctx->n_cus, cu_seqlens_host, n_seqs, H, dk, dv, KDA_CP_ON, seg_chunks, out, nullptr,
                               warm_chunks, seg_chunks);
    if (st != KDA_OK) return st;
    st = upload_plan(*out, ctx->device);
    if (st != KDA_OK) {
        delete *out;
        *out = nullptr;
    }
    return st;
}

void kda_plan_destroy(kda_plan* p) {
    if (!p) return;
    if (p->dev_tables || p->spec_event || p->spec_host) {
        int prev = -1;
        (void)hipGetDevice(&prev);
        (void)hipSetDevice(p->device);
        if (p->spec_event) {
            (void)hipEventSynchronize(p->spec_event);  // the last copy into spec_host has landed
            (void)hipEventDestroy(p->spec_event);
        }
        if (p->spec_host) (void)hipHostFree(p->spec_host);
        if (p->dev_tables) (void)hipFree(p->dev_tables);
        if (prev >= 0) (void)hipSetDevice(prev);
    }
    delete p;
}

size_t kda_plan_workspace_bytes(const kda_plan* p) { return p ? p->info.workspace_bytes : 0; }

kda_status kda_plan_get_info(const kda_plan* p, kda_plan_info* info) {
    if (!p || !info) return fail(KDA_ERR_INVALID, "kda_plan_get_info: NULL argument");
    *info = p->info;
    std::lock_guard<std::mutex> sl(p->spec_mu);
    info->speculation_off = p->spec_off ? 1 : 0;
    return KDA_OK;
}

kda_status kda_plan_get_units(const kda_plan* p, kda_unit_info* units, int32_t max_units) {
    if (!p || (!units && max_units > 0)) return fail(KDA_ERR_INVALID, "kda_plan_get_units: NULL argument");
    const int n = std::min<int>(max_units, (int)p->units.size());
    for (int i = 0; i < n; ++i) {
        const UnitDesc& u = p->units[i];
        units[i] = kda_unit_info{u.seq, u.chunk0, u.n_chunks, u.segment, u.n_segments, u.warm};
    }
    return KDA_OK;
}

kda_status kda_prefill_ex_validate(const kda_plan* p, const kda_prefill_opts* opts, const void* q, const void* k,
                                   const void* v, const float* g, const void* beta, const int32_t* cu_dev,
                                   float scale, const void* s0, const void* sT, const void* out) {
    if (!p) return fail(KDA_ERR_INVALID, "kda_prefill: plan is NULL");
    const kda_plan_info& in = p->info;
    const int32_t qk_heads = (opts && opts->qk_heads > 0) ? opts->qk_heads : in.H;
    const bool beta16 = opts && opts->beta_bf16, state16 = opts && opts->state_bf16;
    if (opts && opts->qk_heads < 0)
        return fail(KDA_ERR_INVALID, "kda_prefill: qk_heads must be >= 0 (got %d)", opts->qk_heads);
    if (in.H % qk_heads != 0)
        return fail(KDA_ERR_INVALID, "kda_prefill: the plan's %d value heads are not a multiple of %d q/k heads",
                    in.H, qk_heads);
    const size_t Tt = (size_t)in.total_tokens, H = (size_t)in.H, N = (size_t)in.n_seqs;
    const size_t n_act = Tt * H * 128 * 2, n_g = Tt * H * 128 * 4, n_beta = Tt * H * (beta16 ? 2 : 4);
    const size_t n_qk = Tt * (size_t)qk_heads * 128 * 2;
    const size_t n_state = N * H * 128 * 128 * (state16 ? 2 : 4), n_cu = (N + 1) * 4;
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID, "kda_prefill: scale is not finite");
    if (!cu_dev) return fail(KDA_ERR_INVALID, "kda_prefill: cu_seqlens is NULL");
    if (Tt > 0) {
        const void* need[] = {q, k, v, g, beta, out};
        const char* names[] = {"q", "k", "v", "g", "beta", "out"};
        for (int i = 0; i < 6; ++i) {
            if (!need[i]) return fail(KDA_ERR_INVALID, "kda_prefill: %s is NULL", names[i]);
            const int al = i == 4 ? (beta16 ? 2 : 4) : 16;
            if ((uintptr_t)need[i] % al)
                return fail(KDA_ERR_INVALID, "kda_prefill: %s is not %d-byte aligned", names[i], al);
        }
    }
    if ((uintptr_t)cu_dev % 4) return fail(KDA_ERR_INVALID, "kda_prefill: cu_seqlens is not 4-byte aligned");
    if (s0 && (uintptr_t)s0 % 16) return fail(KDA_ERR_INVALID, "kda_prefill: initial_state is not 16-byte aligned");
    if (sT && (uintptr_t)sT % 16) return fail(KDA_ERR_INVALID, "kda_prefill: final_state is not 16-byte aligned");
    // out may not overlap anything
    struct B { const void* p; size_t n; const char* name; };
    const B ins[] = {{q, n_qk, "q"}, {k, n_qk, "k"}, {v, n_act, "v"}, {g, n_g, "g"},
                     {beta, n_beta, "beta"}, {cu_dev, n_cu, "cu_seqlens"}};
    for (const B& b : ins) {
        if (overlap(out, n_act, b.p, b.n))
            return fail(KDA_ERR_ALIAS, "kda_prefill: out overlaps %s", b.name);
        if (overlap(sT, n_state, b.p, b.n))
            return fail(KDA_ERR_ALIAS, "kda_prefill: final_state overlaps %s", b.name);
    }
    if (overlap(out, n_act, s0, n_state)) return fail(KDA_ERR_ALIAS, "kda_prefill: out overlaps initial_state");
    if (overlap(out, n_act, sT, n_state)) return fail(KDA_ERR_ALIAS, "kda_prefill: out overlaps final_state");
    if (s0 && sT && s0 != sT && overlap(s0, n_state, sT, n_state))
        return fail(KDA_ERR_ALIAS, "kda_prefill: final_state partially overlaps initial_state "
                                   "(must be the same buffer or disjoint)");
    return KDA_OK;
}

kda_status kda_prefill_validate(const kda_plan* p, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const int32_t* cu_dev, float scale,
                                const float* s0, const float* sT, const void* out) {
    return kda_prefill_ex_validate(p, nullptr, q, k, v, g, beta, cu_dev, scale, s0, sT, out);
}

kda_status kda_set_timing(kda_ctx* ctx, int enable) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_set_timing: ctx is NULL");
    std::lock_guard<std::mutex> lk(ctx->mu);
    ctx->timing = enable != 0;
    ctx->n_timed = 0;
    return KDA_OK;
}

int32_t kda_get_timing(kda_ctx* ctx, const char** names, double* total_ms, int32_t* launches, int32_t max) {
    if (!ctx) {
        fail(KDA_ERR_INVALID, "kda_get_timing: ctx is NULL");
        return -1;
    }
    std::lock_guard<std::mutex> lk(ctx->mu);
    std::vector<const char*> order;
    std::vector<double> tot;
    std::vector<int32_t> cnt;
    for (int i = 0; i < ctx->n_timed; ++i) {
        TimedLaunch& t = ctx->events[i];
        hipError_t e = hipEventSynchronize(t.end);
        float v = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&v, t.beg, t.end);
        if (e != hipSuccess) {
            ctx->n_timed = 0;
            hip_fail(e, "kda_get_timing");
            return -1;
        }
        size_t j = 0;
        while (j < order.size() && strcmp(order[j], t.name) != 0) ++j;
        if (j == order.size()) {
            order.push_back(t.name);
            tot.push_back(0.0);
            cnt.push_back(0);
        }
        tot[j] += v;
        cnt[j] += 1;
    }
    ctx->n_timed = 0;
    const int n = std::min((int)order.size(), (int)max);
    for (int i = 0; i < n; ++i) {
        if (names) names[i] = order[i];
        if (total_ms) total_ms[i] = tot[i];
        if (launches) launches[i] = cnt[i];
    }
    return n;
}

kda_status kda_prefill(kda_ctx* ctx, const kda_plan* p, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const int32_t* cu_dev, float scale,
                       const float* s0, float* sT, void* out, hipStream_t stream) {
    return kda_prefill_ex(ctx, p, nullptr, q, k, v, g, beta, cu_dev, scale, s0, sT, out, stream);
}

}  // extern "C"

namespace {

// A fixed workspace given instead of the stream's arena: the call then
// allocates nothing, synchronises nothing and leaves no event behind.
struct FixedWorkspace {
    uint8_t* ptr;
    size_t bytes;
};

kda_status prefill_impl(kda_ctx* ctx, const kda_plan* p, const kda_prefill_opts* opts, const void* q,
                        const void* k, const void* v, const float* g, const void* beta, const int32_t* cu_dev,
                        float scale, const void* s0, void* sT, void* out, hipStream_t stream,
                        const FixedWorkspace* fixed) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_prefill: ctx is NULL");
    kda_status st = kda_prefill_ex_validate(p, opts, q, k, v, g, beta, cu_dev, scale, s0, sT, out);
    if (st != KDA_OK) return st;
    if (!p->dev_tables)
        return fail(KDA_ERR_INVALID, "kda_prefill: plan has no device tables (built by kda_plan_prefill_host?)");
    if (p->device != ctx->device)
        return fail(KDA_ERR_INVALID, "kda_prefill: plan is for device %d, context for device %d", p->device,
                    ctx->device);

    std::lock_guard<std::mutex> lk(ctx->mu);
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (prev != ctx->device && (e = hipSetDevice(ctx->device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    struct Restore {
        int prev, cur;
        ~Restore() { if (prev >= 0 && prev != cur) (void)hipSetDevice(prev); }
    } restore{prev, ctx->device};

    // workspace arena of this stream
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    const int32_t qk_heads = (opts && opts->qk_heads > 0) ? opts->qk_heads : p->info.H;
    const bool beta16 = opts && opts->beta_bf16, state16 = opts && opts->state_bf16;
    // a bf16 beta is widened to fp32 into the arena, after the plan's part
    const size_t off_beta = align_up(p->info.workspace_bytes, 256);
    const size_t n_beta = (size_t)p->info.total_tokens * p->info.H;
    const size_t need = beta16 ? off_beta + n_beta * 4 : p->info.workspace_bytes;
    // A plan that needs no workspace touches no arena (nor allocates, nor
    // synchronises), also on a stream seen for the first time.
    uint8_t* ws = nullptr;
    if (fixed) {
        if (need > fixed->bytes)
            return fail(KDA_ERR_INVALID, "kda_prefill_noalloc: this plan needs %zu bytes of workspace, more than the "
                                         "%zu bytes of static scratch (a serial plan needs none)", need, fixed->bytes);
        ws = fixed->ptr;
    } else if (need > 0) {
        auto it = ctx->arenas.find(stream);
        if (it == ctx->arenas.end() || it->second.bytes < need) {
            if (cap != hipStreamCaptureStatusNone)
                return fail(KDA_ERR_CAPTURE, "kda_prefill: the workspace arena of this stream must grow to %zu bytes, "
                                             "which is not allowed while the stream is capturing; run once uncaptured "
                                             "first", need);
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
            // memory that a captured graph may still use is retired, not freed
            auto release = [&](Arena& a) {
                if (!a.ptr) return;
                if (a.captured) ctx->retired.push_back(a.ptr);
                else (void)hipFree(a.ptr);
                a.ptr = nullptr;
                a.bytes = 0;
                a.captured = false;
            };
            if (it == ctx->arenas.end() && ctx->arenas.size() >= kMaxArenas) {
                // evict one arena (the device is idle after the synchronise)
                auto victim = ctx->arenas.begin();
                release(victim->second);
                ctx->arenas.erase(victim);
            }
            Arena& a = ctx->arenas[stream];
            release(a);
            const size_t bytes = align_up(need + need / 8, 1 << 20);
            e = hipMalloc(&a.ptr, bytes);
            if (e != hipSuccess) {
                a.ptr = nullptr;
                return hip_fail(e, "hipMalloc (workspace arena)");
            }
            a.bytes = bytes;
            if (ctx->poison) {
                e = hipMemset(a.ptr, 0xff, bytes);  // NaN in both bf16 and fp32
                if (e != hipSuccess) return hip_fail(e, "hipMemset (poison)");
            }
            it = ctx->arenas.find(stream);
        }
        if (cap != hipStreamCaptureStatusNone) it->second.captured = true;
        ws = (uint8_t*)it->second.ptr;
    }

    const uint8_t* tabs = (const uint8_t*)p->dev_tables;
    CommonArgs c{};
    c.q = (const uint16_t*)q;
    c.k = (const uint16_t*)k;
    c.v = (const uint16_t*)v;
    c.g = g;
    c.beta = beta16 ? (const float*)(ws + off_beta) : (const float*)beta;
    c.cu = cu_dev;
    c.Tt = p->info.total_tokens;
    c.H = p->info.H;
    c.Hk = qk_heads;
    c.group = p->info.H / qk_heads;
    c.n_seqs = p->info.n_seqs;
    c.total_chunks = p->info.total_chunks;
    c.rec = ws + p->off_rec;

    // the fixed-workspace form records no timing events (creating one may allocate)
    auto timed = [&](const char* name, auto&& launch) -> hipError_t {
        if (fixed) return launch();
        return timed_launch(ctx, stream, name, launch);
    };

    if (beta16) {
        e = timed("beta_to_f32", [&] {
            return launch_beta_to_f32((const uint16_t*)beta, (float*)(ws + off_beta), (int64_t)n_beta, stream);
        });
        if (e != hipSuccess) return hip_fail(e, "beta_to_f32 launch");
    }
    // speculation feedback from an earlier call of this plan (never under capture)
    const bool capturing = cap != hipStreamCaptureStatusNone;
    const bool speculative = p->info.warm_cp || p->info.n_split_seqs > 0;
    bool spec_off = false;
    if (speculative) {
        std::lock_guard<std::mutex> sl(p->spec_mu);
        if (p->spec_pending && !capturing && hipEventQuery(p->spec_event) == hipSuccess) {
            p->spec_pending = false;
            for (size_t i = 0; i < p->spec_words && !p->spec_off; ++i) p->spec_off = p->spec_host[i] != 0;
        }
        spec_off = p->spec_off;
    }
    // after a speculative call: copy its outcome back without waiting for it
    // (on a plan's first call and every 64th, so the copy costs little)
    auto report = [&](const int32_t* dev_words, size_t n_words) -> hipError_t {
        // (the copy needs pinned host memory, allocated on first use)
        if (capturing || fixed || n_words == 0) return hipSuccess;
        std::lock_guard<std::mutex> sl(p->spec_mu);
        if (p->spec_calls++ % 64 != 0 || p->spec_pending) return hipSuccess;
        hipError_t err = hipSuccess;
        if (!p->spec_host) {
            err = hipHostMalloc((void**)&p->spec_host, n_words * sizeof(int32_t), hipHostMallocDefault);
            if (err != hipSuccess) { p->spec_host = nullptr; return err; }
            p->spec_words = n_words;
            err = hipEventCreateWithFlags(&p->spec_event, hipEventDisableTiming);
            if (err != hipSuccess) { p->spec_event = nullptr; return err; }
        }
        err = hipMemcpyAsync(p->spec_host, dev_words, p->spec_words * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
        if (err == hipSuccess) err = hipEventRecord(p->spec_event, stream);
        if (err == hipSuccess) p->spec_pending = true;
        return err;
    };
    // The segmented pipeline. CP plans: K1 writes the records of every chunk
    // and each segment's pre_scan summaries (B, the update from zero, and the
    // transfer M, the update from the identity with V := 0) in one launch,
    // the merge forms the carries, and K2 runs every unit over the records. A serial plan with
    // materialised K1 runs K1 alone and then K2. cc.gate gates every launch
    // when set (the fallback of warm-start CP); with gate_flags, the first
    // launch reduces those flags into the gate word cc.gate points to.
    auto segmented = [&](const CommonArgs& cc, const UnitDesc* k2_units, int32_t n_k2_units,
                         const char* k2_name, const int32_t* gate_flags, int64_t n_gate_flags) -> kda_status {
        const bool cp = !p->merges.empty();
        float* b_seg = (float*)(ws + p->off_b);
        int32_t* m_live = (int32_t*)(ws + p->off_mlive);
        if (cp) {
            K2Args kb{};
            kb.c = cc;
            if (gate_flags) kb.c.gate = nullptr;  // this launch computes the gate
            kb.units = (const UnitDesc*)(tabs + p->dev_off_k1_units);
            kb.n_units = (int32_t)p->k1_units.size();
            kb.carries = b_seg;  // the B summaries go to their pre_scan slots
            kb.m_out = (float*)(ws + p->off_m);  // and the transfers to theirs
            kb.m_live_out = m_live;
            kb.scale = scale;
            kb.spec_final_direct = 1;
            kb.gate_flags = gate_flags;
            kb.n_gate_flags = n_gate_flags;
            kb.gate_out = const_cast<int32_t*>(cc.gate);
            e = timed("k1_bsum", [&] { return launch_k1_bsum(kb, stream); });
            if (e != hipSuccess) return hip_fail(e, "k1_bsum launch");
        } else {
            K1Args k1{cc, (const ChunkDesc*)(tabs + p->dev_off_chunks), gate_flags, n_gate_flags,
                      const_cast<int32_t*>(cc.gate)};
            if (gate_flags) k1.c.gate = nullptr;  // the K1 launch computes the gate
            e = timed("k1_prepare", [&] { return launch_k1_prepare(k1, stream); });
            if (e != hipSuccess) return hip_fail(e, "k1_prepare launch");
        }
        if (gate_flags && (e = report(cc.gate, 1)) != hipSuccess) return hip_fail(e, "speculation feedback");
        if (cp) {
            MergeArgs ma{cc, (const MergeDesc*)(tabs + p->dev_off_merges),
                         (const MergeSeg*)(tabs + p->dev_off_merge_segs), (int32_t)p->merge_segs.size(), s0, b_seg,
                         (const float*)(ws + p->off_m), (float*)(ws + p->off_carry), state16 ? 1 : 0, m_live};
            e = timed("cp_merge", [&] { return launch_cp_merge(ma, stream); });
            if (e != hipSuccess) return hip_fail(e, "cp_merge launch");
        }
        K2Args kc{cc, k2_units, n_k2_units, s0, sT, (float*)(ws + p->off_carry), (uint16_t*)out, scale,
                  state16 ? 1 : 0, nullptr, nullptr, 0, 0, b_seg, m_live};
        e = timed(k2_name, [&] { return launch_k2_recur(kc, stream); });
        if (e != hipSuccess) return hip_fail(e, "k2 launch");
        return KDA_OK;
    };
    const UnitDesc* cp_units = (const UnitDesc*)(tabs + p->dev_off_cp_units);
    if (p->info.warm_cp && spec_off)  // the exact path of a warm-start CP plan: the pipeline alone
        return segmented(c, cp_units, (int32_t)p->cp_units.size(), "k2_segment", nullptr, 0);
    if (p->info.n_split_seqs > 0 && spec_off) {
        // the exact path of a split plan: the batch unsplit
        K2Args ks{c, (const UnitDesc*)(tabs + p->dev_off_alt_units), (int32_t)p->alt_units.size(), s0, sT,
                  (float*)(ws + p->off_carry), (uint16_t*)out, scale, state16 ? 1 : 0, nullptr, nullptr, 0, 1};
        e = timed("fused_serial", [&] { return launch_fused(ks, stream); });
        if (e != hipSuccess) return hip_fail(e, "fused launch");
        return KDA_OK;
    }
    if (p->info.warm_cp) {
        // warm-start CP: all segments in one fused launch; the segmented
        // pipeline runs only if the flag reduction arms its gate
        const bool direct = !(sT && s0 && sT == s0);
        int32_t* gate = (int32_t*)(ws + p->off_gate);
        K2Args kw{c, (const UnitDesc*)(tabs + p->dev_off_units), (int32_t)p->units.size(), s0, sT,
                  (float*)(ws + p->off_carry), (uint16_t*)out, scale, state16 ? 1 : 0,
                  (int32_t*)(ws + p->off_spec_flags), (float*)(ws + p->off_spec_states), 0, direct ? 1 : 0};
        e = timed("fused_warm_cp", [&] { return launch_fused(kw, stream); });
        if (e != hipSuccess) return hip_fail(e, "warm-start CP launch");
        CommonArgs cg = c;
        cg.gate = gate;
        const kda_status st2 = segmented(cg, cp_units, (int32_t)p->cp_units.size(), "k2_segment", kw.spec_flags,
                                         (int64_t)p->info.n_warm_segments * p->info.H * 8);
        if (st2 != KDA_OK) return st2;
        if (!direct && !p->fixups.empty()) {
            // publish the final states the warm-start launch left in scratch
            K2Args kf = kw;
            kf.c = cg;
            kf.units = (const UnitDesc*)(tabs + p->dev_off_fixups);
            kf.n_units = (int32_t)p->fixups.size();
            kf.fixup = 1;
            e = timed("publish_final", [&] { return launch_fused(kf, stream); });
            if (e != hipSuccess) return hip_fail(e, "publish launch");
        }
        return KDA_OK;
    }
    const bool mat = p->info.k1_materialized != 0;
    if (mat)  // segmented CP, or the two-kernel serial form (no pre_scan, no merge)
        return segmented(c, (const UnitDesc*)(tabs + p->dev_off_units), (int32_t)p->units.size(),
                         p->info.uses_cp ? "k2_segment" : "k2_recur", nullptr, 0);
    K2Args ka{c, (const UnitDesc*)(tabs + p->dev_off_units), (int32_t)p->units.size(), s0, sT,
              (float*)(ws + p->off_carry), (uint16_t*)out, scale, state16 ? 1 : 0,
              (int32_t*)(ws + p->off_spec_flags), (float*)(ws + p->off_spec_states), 0, 0};
    // a final state that aliases the initial state is published by the fix-up
    // launch, after every unit has read its initial state
    ka.spec_final_direct = (sT && s0 && sT == s0) ? 0 : 1;
    const bool split = p->info.n_split_seqs > 0;
    e = timed(split ? "fused_split" : "fused_serial", [&] { return launch_fused(ka, stream); });
    if (e != hipSuccess) return hip_fail(e, "k2 launch");
    if (split) {
        // warm-start segments: keep (and publish the end state of) each one
        // whose warm-up transfer vanished, rerun the others from their carry
        K2Args kf = ka;
        kf.units = (const UnitDesc*)(tabs + p->dev_off_fixups);
        kf.n_units = (int32_t)p->fixups.size();
        kf.fixup = 1;
        e = timed("fused_fixup", [&] { return launch_fused(kf, stream); });
        if (e != hipSuccess) return hip_fail(e, "fix-up launch");
        if ((e = report(ka.spec_flags, p->fixups.size() * (size_t)p->info.H * 8)) != hipSuccess)
            return hip_fail(e, "speculation feedback");
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_ex(kda_ctx* ctx, const kda_plan* p, const kda_prefill_opts* opts, const void* q,
                          const void* k, const void* v, const float* g, const void* beta, const int32_t* cu_dev,
                          float scale, const void* s0, void* sT, void* out, hipStream_t stream) {
    return prefill_impl(ctx, p, opts, q, k, v, g, beta, cu_dev, scale, s0, sT, out, stream, nullptr);
}

kda_status kda_prefill_noalloc(kda_ctx* ctx, const kda_plan* p, const kda_prefill_opts* opts, const void* q,
                               const void* k, const void* v, const float* g, const void* beta,
                               const int32_t* cu_dev, float scale, const void* s0, void* sT, void* out,
                               hipStream_t stream) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_prefill_noalloc: ctx is NULL");
    if (!ctx->scratch)
        return fail(KDA_ERR_HIP, "kda_prefill_noalloc: the static scratch of device %d has no address", ctx->device);
    const FixedWorkspace fw{(uint8_t*)ctx->scratch, static_scratch_bytes()};
    return prefill_impl(ctx, p, opts, q, k, v, g, beta, cu_dev, scale, s0, sT, out, stream, &fw);
}

size_t kda_noalloc_scratch_bytes(void) { return static_scratch_bytes(); }

kda_status kda_decode_slots_validate(int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                                     const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, float scale, const float* state, int32_t n_slots,
                                     const int32_t* slots, const void* out) {
    if (dk != 128 || dv != 128)
        return fail(KDA_ERR_UNSUPPORTED, "kda_decode: dk = dv = 128 required (got dk=%d dv=%d)", dk, dv);
    if (n_seqs < 0 || H < 1)
        return fail(KDA_ERR_INVALID, "kda_decode: n_seqs must be >= 0 and H >= 1 (got n_seqs=%d H=%d)", n_seqs, H);
    if (qk_heads < 1 || H % qk_heads != 0)
        return fail(KDA_ERR_INVALID, "kda_decode: %d value heads are not a multiple of %d q/k heads", H, qk_heads);
    if (n_slots < 0) return fail(KDA_ERR_INVALID, "kda_decode: n_slots must be >= 0 (got %d)", n_slots);
    if (!slots && n_slots != n_seqs)
        return fail(KDA_ERR_INVALID, "kda_decode: without a slot table the state holds n_seqs = %d states, "
                                     "not %d", n_seqs, n_slots);
    if ((int64_t)n_seqs * H * 2 > (int64_t)INT32_MAX)
        return fail(KDA_ERR_INVALID, "kda_decode: n_seqs * H too large (%lld)", (long long)n_seqs * H);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID, "kda_decode: scale is not finite");
    if (n_seqs == 0) return KDA_OK;
    const size_t NH = (size_t)n_seqs * H;
    const size_t n_act = NH * 128 * 2, n_g = NH * 128 * 4, n_beta = NH * 4;
    const size_t n_state = (size_t)n_slots * H * kStateBytes, n_slot_tab = (size_t)n_seqs * 4;
    const size_t n_qk = (size_t)n_seqs * qk_heads * 128 * 2;
    const void* need[] = {q, k, v, g, beta, out};
    const char* names[] = {"q", "k", "v", "g", "beta", "out"};
    for (int i = 0; i < 6; ++i) {
        if (!need[i]) return fail(KDA_ERR_INVALID, "kda_decode: %s is NULL", names[i]);
        const int al = i == 4 ? 4 : 16;
        if ((uintptr_t)need[i] % al)
            return fail(KDA_ERR_INVALID, "kda_decode: %s is not %d-byte aligned", names[i], al);
    }
    if (n_slots > 0 && !state) return fail(KDA_ERR_INVALID, "kda_decode: state is NULL");
    if (state && (uintptr_t)state % 16) return fail(KDA_ERR_INVALID, "kda_decode: state is not 16-byte aligned");
    if (slots && (uintptr_t)slots % 4) return fail(KDA_ERR_INVALID, "kda_decode: slots is not 4-byte aligned");
    struct B { const void* p; size_t n; const char* name; };
    const B ins[] = {{q, n_qk, "q"}, {k, n_qk, "k"}, {v, n_act, "v"}, {g, n_g, "g"}, {beta, n_beta, "beta"},
                     {slots, n_slot_tab, "slots"}};
    for (const B& b : ins) {
        if (overlap(out, n_act, b.p, b.n)) return fail(KDA_ERR_ALIAS, "kda_decode: out overlaps %s", b.name);
        if (overlap(state, n_state, b.p, b.n)) return fail(KDA_ERR_ALIAS, "kda_decode: state overlaps %s", b.name);
    }
    if (overlap(out, n_act, state, n_state)) return fail(KDA_ERR_ALIAS, "kda_decode: out overlaps state");
    return KDA_OK;
}

kda_status kda_decode_validate(int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                               const void* q, const void* k, const void* v, const float* g, const float* beta,
                               float scale, const float* state, const void* out) {
    if (n_seqs > 0 && !state) return fail(KDA_ERR_INVALID, "kda_decode: state is NULL");
    return kda_decode_slots_validate(n_seqs, H, qk_heads, dk, dv, q, k, v, g, beta, scale, state, n_seqs, nullptr,
                                     out);
}

kda_status kda_decode_slots(kda_ctx* ctx, int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                            const void* q, const void* k, const void* v, const float* g, const float* beta,
                            float scale, float* state, int32_t n_slots, const int32_t* slots, void* out,
                            hipStream_t stream) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_decode: ctx is NULL");
    kda_status st = kda_decode_slots_validate(n_seqs, H, qk_heads, dk, dv, q, k, v, g, beta, scale, state, n_slots,
                                              slots, out);
    if (st != KDA_OK || n_seqs == 0) return st;
    std::lock_guard<std::mutex> lk(ctx->mu);
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (prev != ctx->device && (e = hipSetDevice(ctx->device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    DecodeArgs a{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, beta, state, (uint16_t*)out,
                 n_seqs, H, qk_heads, H / qk_heads, scale, slots, n_slots};
    e = timed_launch(ctx, stream, "decode", [&] { return launch_decode(a, stream); });
    if (prev >= 0 && prev != ctx->device) (void)hipSetDevice(prev);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return KDA_OK;
}

kda_status kda_decode(kda_ctx* ctx, int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                      const void* q, const void* k, const void* v, const float* g, const float* beta, float scale,
                      float* state, void* out, hipStream_t stream) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_decode: ctx is NULL");
    if (n_seqs > 0 && !state) return fail(KDA_ERR_INVALID, "kda_decode: state is NULL");
    return kda_decode_slots(ctx, n_seqs, H, qk_heads, dk, dv, q, k, v, g, beta, scale, state, n_seqs, nullptr, out,
                            stream);
}

kda_status kda_debug_k1_records(kda_ctx* ctx, const kda_plan* p, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, const int32_t* cu_dev,
                                void* records, hipStream_t stream) {
    if (!ctx) return fail(KDA_ERR_INVALID, "kda_debug_k1_records: ctx is NULL");
    if (!records && p && p->info.total_chunks > 0)
        return fail(KDA_ERR_INVALID, "kda_debug_k1_records: records is NULL");
    // the prefill checks, with records standing in for out
    kda_status st = kda_prefill_validate(p, q, k, v, g, beta, cu_dev, 1.0f, nullptr, nullptr, records);
    if (st != KDA_OK) return st;
    if (!p->dev_tables || p->device != ctx->device)
        return fail(KDA_ERR_INVALID, "kda_debug_k1_records: plan not executable on this context");
    CommonArgs c{};
    c.q = (const uint16_t*)q;
    c.k = (const uint16_t*)k;
    c.v = (const uint16_t*)v;
    c.g = g;
    c.beta = beta;
    c.cu = cu_dev;
    c.Tt = p->info.total_tokens;
    c.H = p->info.H;
    c.Hk = p->info.H;
    c.group = 1;
    c.n_seqs = p->info.n_seqs;
    c.total_chunks = p->info.total_chunks;
    c.rec = (uint8_t*)records;
    K1Args k1{c, (const ChunkDesc*)((const uint8_t*)p->dev_tables + p->dev_off_chunks)};
    const hipError_t e = launch_k1_prepare(k1, stream);
    if (e != hipSuccess) return hip_fail(e, "k1_prepare launch");
    return KDA_OK;
}

}  // extern "C"
