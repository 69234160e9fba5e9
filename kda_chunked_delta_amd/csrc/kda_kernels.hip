// HIP kernels of the KDA forward prefill for gfx950: K1 (chunk preparation),
// K2 (inter-chunk recurrence, serial or per CP segment), and the intracard
// context-parallel pre_scan and merge named in the commit summary of
// "feat(kda/sm90): FlashKDA prefill port + intracard-CP prefill" (cuLA pull
// request #103): K1 once, pre_scan, merge of segment carries, segment-K2.
#include "kda_device.hpp"
#include "kda_launch.h"

namespace kda {

static_assert(REC_HBM_BYTES == kRecBytes, "record size differs between host and device");

namespace {

// Sequence bounds from the device cu_seqlens, clamped into [0, Tt] so that an
// inconsistent table can never address outside the inputs.
__device__ __forceinline__ void seq_bounds(const CommonArgs& c, int seq, int64_t& beg,
                                           int64_t& end) {
    int64_t b = c.cu[seq], e = c.cu[seq + 1];
    b = b < 0 ? 0 : (b > c.Tt ? c.Tt : b);
    e = e < b ? b : (e > c.Tt ? c.Tt : e);
    beg = b;
    end = e;
}

// A uniform byte offset that the compiler treats as opaque (no strength
// reduction of the addresses built on it across loop iterations).
__device__ __forceinline__ int ring_off(int off) { return __builtin_amdgcn_readfirstlane(off); }

__device__ __forceinline__ int rows_of(int64_t tok, int64_t end) {
    const int64_t n = end - tok;
    return n <= 0 ? 0 : (n >= CH ? CH : (int)n);
}

// The input rows of V for K2 over materialised records (the HBM records
// carry no V): the unit's first token row of head h, the bytes per token
// row, and the tokens of the sequence from that row on.
struct VRows {
    const uint8_t* base;
    uint32_t stride;
    int rem;
};

// K2's record prefetch through registers: the 896 vectors of an HBM record,
// up to two per thread, and the chunk's 16 value rows, one 16-byte granule per
// thread of wavefronts 0..3 (row tid >> 4, granule tid & 15). Wavefronts
// 4..7 issue the same load over an empty range (no memory access), so that
// every load is unconditional; rows past the sequence read as zeros. In LDS
// a stage holds the record and, after it, the chunk's V block.
constexpr int K2_STAGE_BYTES = REC_BYTES + VBLK_BYTES;
struct K2Prefetch {
    static constexpr int N = (REC_HBM_VEC + 511) / 512;
    u32x4 r[N];
    u32x4 vr;
    __device__ __forceinline__ void load(const uint8_t* __restrict__ src, const VRows& v, int ci) {
        const u32x4* s = (const u32x4*)src;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int i = threadIdx.x + j * 512;
            if (i < REC_HBM_VEC) r[j] = __builtin_nontemporal_load(s + i);
        }
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t bytes = wave < 4 ? (uint32_t)chunk_rows(v.rem, ci) * v.stride : 0u;
        const int off = (int)((threadIdx.x >> 4) & 15) * (int)v.stride + (int)(threadIdx.x & 15) * 16;
        vr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            chunk_rsrc(v.base + (size_t)ci * CH * v.stride, bytes), off, 0, BUF_POLICY));
    }
    __device__ __forceinline__ void store(uint8_t* dst) const {
        u32x4* d = (u32x4*)dst;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int i = threadIdx.x + j * 512;
            if (i < REC_HBM_VEC) d[i] = r[j];
        }
        if (threadIdx.x < 256) *(u32x4*)(dst + REC_BYTES + vblk_off(threadIdx.x >> 4, threadIdx.x & 15)) = vr;
    }
};

// Stream nc materialised records (starting at rb) and the chunks' value rows
// through a double-buffered LDS stage; both are fetched two chunks ahead.
// step(ci, rec) runs once per chunk with the record (and its V block) in
// LDS, by every thread.
template <class Step>
__device__ __forceinline__ void record_loop(const uint8_t* __restrict__ rb, const VRows& v, int nc,
                                            uint8_t (*recs)[K2_STAGE_BYTES], Step&& step) {
    K2Prefetch p0, p1;
    if (nc > 0) p0.load(rb, v, 0);
    if (nc > 1) p1.load(rb + REC_HBM_BYTES, v, 1);
    if (nc > 0) p0.store(recs[0]);
    lds_barrier();
    for (int ci = 0; ci < nc; ci += 2) {
        if (ci + 2 < nc) p0.load(rb + (size_t)(ci + 2) * REC_HBM_BYTES, v, ci + 2);
        step(ci, recs[0]);
        if (ci + 1 < nc) p1.store(recs[1]);
        lds_barrier();
        if (ci + 1 < nc) {
            if (ci + 3 < nc) p1.load(rb + (size_t)(ci + 3) * REC_HBM_BYTES, v, ci + 3);
            step(ci + 1, recs[1]);
            if (ci + 2 < nc) p0.store(recs[0]);
            lds_barrier();
        }
    }
}

// Make every register of x live here: its loads complete before this point,
// so no wait for them is left inside the chunk loop that follows (where it
// would also wait for the prefetches issued there).
template <int NT>
__device__ __forceinline__ void settle(const f32x4 (&S)[8][NT]) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) asm volatile("" ::"v"(S[t][n]));
}

// State tiles of value columns 16(n0 + n) .. +15 (see chain_step).
template <int NT>
__device__ __forceinline__ void load_state(const float* sin, f32x4 (&S)[8][NT], int n0, int gg, int m) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                S[t][n][vv] = sin ? sin[(16 * t + 4 * gg + vv) * D + 16 * (n0 + n) + m] : 0.f;
    settle(S);
}

template <int NT>
__device__ __forceinline__ void store_state(float* so, const f32x4 (&S)[8][NT], int n0, int gg, int m) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                so[(16 * t + 4 * gg + vv) * D + 16 * (n0 + n) + m] = S[t][n][vv];
}

// The transfer M in HBM, in the order the CP merge reads it as its MFMA A
// operand. The merge's wavefront t forms carry rows 16t..16t+15; in its
// product lane (gg, m) (lane = 16 gg + m) takes, at MFMA step q, key index
// merge_k(gg, q), from M's row 16t + m. The lane's 32 entries lie in two runs
// of 16 keys, so that the 64 lanes of each carry read fall on distinct LDS
// banks. The stored order puts the entries one lane reads for steps
// 4j..4j+3 in 16 consecutive bytes and the 64 lanes' in one 1 KiB block:
// each of the merge's operand loads then reads 1 KiB of consecutive memory.
__device__ __forceinline__ int merge_k(int gg, int q) { return (q < 16 ? 0 : 48) + 16 * gg + q; }
__device__ __forceinline__ int m_operand_index(int i, int k) {
    const int q = (k & 15) | ((k >> 2) & 16);  // merge_k(gg, q) == k
    const int gg = (k >> 4) & 3;
    return (((i >> 4) * 8 + (q >> 2)) * 64 + 16 * gg + (i & 15)) * 4 + (q & 3);
}
// A 4x4 block held by a lane quad (lane c of the quad: column c, rows 0..3)
// transposed: lane c then holds row c (columns 0..3). Two butterfly stages
// swap lane bit 0 with register bit 0, then lane bit 1 with register bit 1;
// in each a lane sends its partner the two entries that belong there.
__device__ __forceinline__ f32x4 quad_transpose_f32(f32x4 x, int lane) {
    const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
    float s0 = b0 ? x[0] : x[1], s1 = b0 ? x[2] : x[3];
    s0 = __builtin_amdgcn_update_dpp(0.0f, s0, 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
    s1 = __builtin_amdgcn_update_dpp(0.0f, s1, 0xB1, 0xF, 0xF, true);
    x = f32x4{b0 ? s0 : x[0], b0 ? x[1] : s0, b0 ? s1 : x[2], b0 ? x[3] : s1};
    float t0 = b1 ? x[0] : x[2], t1 = b1 ? x[1] : x[3];
    t0 = __builtin_amdgcn_update_dpp(0.0f, t0, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
    t1 = __builtin_amdgcn_update_dpp(0.0f, t1, 0x4E, 0xF, 0xF, true);
    return f32x4{b1 ? t0 : x[0], b1 ? t1 : x[1], b1 ? x[2] : t0, b1 ? x[3] : t1};
}
// A wavefront's tiles of M (store_state's layout: value columns 16 n0 ..
// 16 n0 + 15) written in that order, or zeros in their place. After a quad
// transpose, lane 4a + c holds the entries of M row 16t + 4 gg + c at keys
// 16 n0 + 4a .. + 3, which are 16 consecutive bytes of the stored order: one
// 16-byte store per tile (row tile t lies 2048 floats further on: eight
// 1 KiB operand blocks per 16 rows).
__device__ __forceinline__ float* transfer_base(float* mo, int n0, int gg, int m) {
    return mo + m_operand_index(4 * gg + (m & 3), 16 * n0 + (m & ~3));
}
__device__ __forceinline__ void store_transfer(float* mo, const f32x4 (&S)[8][1], int n0, int gg, int m) {
    float* b = transfer_base(mo, n0, gg, m);
#pragma unroll
    for (int t = 0; t < 8; ++t) *(f32x4*)(b + t * 2048) = quad_transpose_f32(S[t][0], m & 3);
}
__device__ __forceinline__ void zero_transfer(float* mo, int n0, int gg, int m) {
    float* b = transfer_base(mo, n0, gg, m);
#pragma unroll
    for (int t = 0; t < 8; ++t) *(f32x4*)(b + t * 2048) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// load_state and store_state for a bf16 state (loaded exactly; stored
// rounded to nearest even).
template <int NT>
__device__ __forceinline__ void load_state_bf16(const uint16_t* sin, f32x4 (&S)[8][NT], int n0, int gg, int m) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                S[t][n][vv] = bf16_lo(sin[(16 * t + 4 * gg + vv) * D + 16 * (n0 + n) + m]);
    settle(S);
}

template <int NT>
__device__ __forceinline__ void store_state_bf16(uint16_t* so, const f32x4 (&S)[8][NT], int n0, int gg, int m) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                so[(16 * t + 4 * gg + vv) * D + 16 * (n0 + n) + m] = (uint16_t)pack_bf16(S[t][n][vv], 0.f);
}

// Whether any element of the wavefront's state tile is nonzero (-0 counts
// as zero); the result is uniform over the wavefront.
template <int NT>
__device__ __forceinline__ bool tile_nonzero(const f32x4 (&S)[8][NT]) {
    uint32_t acc = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) acc |= __float_as_uint(S[t][n][vv]);
    return __builtin_amdgcn_ballot_w64((acc & 0x7fffffffu) != 0u) != 0;
}

template <int NT>
__device__ __forceinline__ void identity_state(f32x4 (&S)[8][NT], int n0, int gg, int m) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv)
                S[t][n][vv] = (16 * t + 4 * gg + vv == 16 * (n0 + n) + m) ? 1.f : 0.f;
}

// Output rows of one chunk: oacc[v] is o[token m][16 n + 4gg + v].
__device__ __forceinline__ void store_output(const K2Args& a, int h, int64_t tk, int nrows,
                                             const f32x4& oacc, int n, int gg, int m) {
    // a buffer store whose range ends with row nrows - 1 of head h: the
    // lanes of rows past the end are dropped without a branch
    const uint32_t rowb = (uint32_t)a.c.H * (D * 2);
    const uint32_t n_out = nrows > 0 ? (uint32_t)(nrows - 1) * rowb + D * 2 : 0u;
    u32x2 w;
    w.x = pack_bf16(a.scale * oacc[0], a.scale * oacc[1]);
    w.y = pack_bf16(a.scale * oacc[2], a.scale * oacc[3]);
    __builtin_amdgcn_raw_buffer_store_b64(
        __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t, w),
        chunk_rsrc(a.out + ((size_t)tk * a.c.H + h) * D, n_out),
        (int)((uint32_t)m * rowb + (16 * n + 4 * gg) * 2), 0, 0);
}

// Start state of a unit: its carry (fp32, CP segments), else the caller's
// initial state (fp32 or bf16), else zeros.
template <int NT>
__device__ __forceinline__ void load_unit_state(const K2Args& a, const UnitDesc& u, int h, f32x4 (&S)[8][NT],
                                                int n0, int gg, int m) {
    const size_t off = ((size_t)u.seq * a.c.H + h) * (D * D);
    if (u.b_slot >= 0) {
        // a CP segment whose predecessor's transfer vanished starts from that
        // segment's B summary (its carry, bit for bit)
        const size_t so = (size_t)u.b_slot * a.c.H + h;
        const int32_t* fl = a.m_live + so * 8;
        int live = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) live |= fl[j];
        if (!live) {
            load_state(a.b_seg + so * (D * D), S, n0, gg, m);
            return;
        }
    }
    if (u.in_slot >= 0)
        load_state(a.carries + ((size_t)u.in_slot * a.c.H + h) * (D * D), S, n0, gg, m);
    else if (a.s0 && a.state_bf16)
        load_state_bf16((const uint16_t*)a.s0 + off, S, n0, gg, m);
    else
        load_state(a.s0 ? (const float*)a.s0 + off : nullptr, S, n0, gg, m);
}

// Final state of a unit, if it writes one (fp32 or bf16).
template <int NT>
__device__ __forceinline__ void store_unit_state(const K2Args& a, const UnitDesc& u, int h,
                                                 const f32x4 (&S)[8][NT], int n0, int gg, int m) {
    if (!u.write_final || !a.sT) return;
    const size_t off = ((size_t)u.seq * a.c.H + h) * (D * D);
    if (a.state_bf16) store_state_bf16((uint16_t*)a.sT + off, S, n0, gg, m);
    else store_state((float*)a.sT + off, S, n0, gg, m);
}

}  // namespace

// ---------------------------------------------------------------------------
// K1 (materialised form): one workgroup of 8 wavefronts per (chunk, head),
// head fastest (a gated launch caps the grid and strides over the items).
// The rows are loaded whole and
// staged through LDS as in the fused kernel; the staging area overlays the
// record and scratch, which are written only after every wavefront has read
// its phase-1 fragments.
// ---------------------------------------------------------------------------
constexpr int K1P_LDS = REC_BYTES + K1_BYTES + N_WAVE_T * K1_LBYTES;
static_assert(STG_BYTES <= K1P_LDS, "staging overlays the record area");

template <bool GVA>
__global__ __launch_bounds__(512) void kda_k1_prepare(K1Args a) {
    if (a.c.gate && *a.c.gate == 0) return;  // fallback not armed
    if (a.gate_flags) {
        int32_t acc = 0;
        for (int64_t i = threadIdx.x; i < a.n_gate_flags; i += blockDim.x) acc |= a.gate_flags[i];
        const int armed = __syncthreads_or(acc != 0);
        if (blockIdx.x == 0 && threadIdx.x == 0) a.gate_out[0] = armed;
        if (!armed) return;  // fallback not armed
    }
    __shared__ __align__(16) uint8_t lds[K1P_LDS];
    uint8_t* rec = lds;
    uint8_t* scr = lds + REC_BYTES;
    float* lw = (float*)(lds + REC_BYTES + K1_BYTES);
    uint8_t* stg = lds;
    const int H = a.c.H;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const RowLaneOffsets lo = row_lane_offsets(H, a.c.Hk, wave, lane);
    // (chunk, head) items, head fastest; one per workgroup, or a stride over
    // them when the grid is capped
    const int64_t n_items = (int64_t)a.c.total_chunks * H;
    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int h = (int)(item % H);
        const int gc = (int)(item / H);
        const ChunkDesc cd = a.chunks[gc];
        int64_t beg, end;
        seq_bounds(a.c, cd.seq, beg, end);
        const int64_t tok0 = beg + (int64_t)CH * cd.chunk;
        const RowStreams rs = row_streams(a.c.q, a.c.k, a.c.v, a.c.g, a.c.beta, H, a.c.Hk, tok0, h, h / a.c.group,
                                          wave);
        RowChunk rc;
        const int nr = rows_of(tok0, end);
        k1_load_chunk<GVA>(rs, 0, nr, nr, lo, rc, wave);
        k1_stage(rc, wave, lane, lo, stg, (float*)(stg + STG_B));
        lds_barrier();
        RawChunk raw;
        k1_read_staged(stg, (const float*)(stg + STG_B), lane, lo, raw);
        lds_barrier();  // the staging area is free again
        k1_phase1<false>(raw, wave, lane, rec, scr, (float*)(scr + K1_BETA));
        lds_barrier();
        k1_phase2(wave, lane, rec, scr, lw);
        lds_barrier();
        u32x4* dst = (u32x4*)(a.c.rec + ((size_t)h * a.c.total_chunks + gc) * REC_HBM_BYTES);
        const u32x4* src = (const u32x4*)rec;
        for (int i = threadIdx.x; i < REC_HBM_VEC; i += 512) dst[i] = src[i];
        lds_barrier();  // the record is read before the next item stages over it
    }
}

// ---------------------------------------------------------------------------
// Fused K1 + K2 (the serial path): one workgroup of 16 wavefronts per (unit,
// head), software-pipelined with one barrier per chunk. In the interval that
// ends with barrier i:
//   - wavefronts 0..7 hold the state (wavefront w: value columns
//     16w..16w+15, in MFMA accumulators for the whole unit), advance it over
//     chunk i and store that chunk's output. Four of them (fused_t_role)
//     also form four rows each of T' of chunk i+1 from the shared L^T;
//     wavefront WAVE_QK forms A_qk of chunk i+2 and L of chunk i+2, once,
//     into the shared L^T;
//   - wavefronts 8 + w issue the direct-to-LDS load of the g rows of chunk
//     i+6 (and, every other interval, of two chunks' V blocks), run K1
//     phase 1 of chunk i+3 (key channels 16w..16w+15) from the staged rows,
//     stage the q and k rows of chunk i+4 that they loaded two intervals
//     earlier, and issue the register loads of those rows of chunk i+6
//     (into the register set just staged). Issuing the direct-to-LDS loads
//     first spreads the loads over the interval.
// Each SIMD holds two state wavefronts and two K1 wavefronts. Records and the
// staged g rows live in 4-deep LDS rings (a g slot is written by the loads
// issued three intervals before it is read, and read once), the V blocks in
// a 5-deep one; K1 scratch, the shared L^T and the staged q, k rows in 2-deep
// ones. The staged q, k rows and the K1 scratch (without their betas) lie in the first 64 KiB, so
// that every K1 access to them is a per-lane base plus an immediate offset;
// the K1 loop is unrolled over the two slots of those rings. A g slot is
// complete once the compiler's wait for the same chunk's register loads,
// issued after it, returns (loads complete in order), which comes before
// the barrier that precedes its read. Both roles run three start-up
// intervals and then the same even number of intervals, after one start-up barrier: the trailing K1 work on
// chunks past the end reads zeros (a buffer load of a chunk with no rows
// touches no memory) and fills slots nobody reads, so the K1 loop body is
// unconditional and the compiler's wait for a register set covers only that
// set's loads.
// ---------------------------------------------------------------------------
constexpr int F_STG = 0;                              // 2 staged chunks (q, k rows)
constexpr int F_SCR = F_STG + 2 * FSTG_NB;            // 2 K1 scratch areas (Gram factors)
constexpr int F_LB = F_SCR + 2 * K1_NB;               // 2 shared L^T + beta
constexpr int F_BETA = F_LB + 2 * LB_BYTES;           // betas: 2 staged [16], 2 scratch [16]
constexpr int F_GR = (F_BETA + 256 + 255) / 256 * 256;  // 4 staged g chunks (direct-to-LDS)
constexpr int F_VR = F_GR + 4 * GRING_BYTES;          // 5 V blocks (direct-to-LDS)
constexpr int F_REC = F_VR + 5 * VBLK_BYTES;          // 4 records
constexpr int F_MFL = F_REC + 4 * REC_BYTES;          // K1 pass: flags of the 8 transfer tiles
constexpr int FUSED_LDS = F_MFL + 32;
static_assert(F_LB <= 65536, "the K1 rings fit the immediate-offset range of LDS instructions");
static_assert(FUSED_LDS <= 160 * 1024, "fused kernel LDS");

// GVA: q/k heads differ from the value heads (value head h reads q/k head
// h / group); the plain instance keeps the q/k loads on v's offsets.
// BSUM: the K1 pass of the segmented CP pipeline, with pre_scan. Every chunk
// record formed in LDS is also written to the workspace (records
// [H][total_chunks]), and the state wavefronts of a unit with out_slot >= 0
// run, without output, the state update from zero, whose end state (the
// segment's B summary) goes to carries[out_slot] (the host points carries at
// the summaries), and beside it the update from the identity with V := 0
// (the transfer M, to m_out[out_slot]) until it vanishes.
template <bool GVA, bool BSUM>
__device__ __forceinline__ void fused_body(const K2Args& a) {
    if constexpr (BSUM) {
        if (a.c.gate && *a.c.gate == 0) return;  // fallback not armed
        if (a.gate_flags) {
            int32_t acc = 0;
            for (int64_t i = threadIdx.x; i < a.n_gate_flags; i += blockDim.x) acc |= a.gate_flags[i];
            const int armed = __syncthreads_or(acc != 0);
            if (blockIdx.x == 0 && threadIdx.x == 0) a.gate_out[0] = armed;
            if (!armed) return;  // fallback not armed
        }
    }
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* recs = smem + F_REC;              // 4 records
    uint8_t* scrs = smem + F_SCR;              // 2 K1 scratch areas
    uint8_t* lbs = smem + F_LB;                // 2 shared L^T + beta
    uint8_t* stgs = smem + F_STG;              // 2 staged chunks
    uint8_t* grs = smem + F_GR;                // 4 staged g chunks
    uint8_t* vrs = smem + F_VR;                // 5 V blocks
    float* stg_betas = (float*)(smem + F_BETA);          // [2][16]
    float* scr_betas = (float*)(smem + F_BETA + 128);    // [2][16]
    const int H = a.c.H;
    // workgroups go round-robin to the 8 XCDs by index: within a unit, index
    // w lands on XCD w % 8, which takes heads (w % 8) * H/8 + w / 8 (when H is
    // a multiple of 8), so each XCD reads H/8 adjacent heads of every row
    int h = blockIdx.x % H;
    if ((H & 7) == 0) h = (h & 7) * (H >> 3) + (h >> 3);
    const UnitDesc u = a.units[blockIdx.x / H];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gg = lane >> 4, m = lane & 15;
    // uniform by construction; said explicitly so that buffer descriptors
    // built from it stay scalar
    const int w8 = __builtin_amdgcn_readfirstlane(wave & 7);
    int64_t beg, end;
    seq_bounds(a.c, u.seq, beg, end);
    if (a.fixup) {
        // fix-up launch over warm-start segments: the segment stands as
        // computed when every tile of its warm-up transfer was exactly zero.
        // With a gate (warm-start CP), the gate says whether any warm-up
        // transfer of the plan survived; the segmented pipeline then
        // recomputes everything, and this launch only publishes final states
        // otherwise.
        int live = 0;
        if (a.c.gate) {
            live = *a.c.gate;
        } else {
            const int32_t* fl = a.spec_flags + ((size_t)u.spec * H + h) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) live |= fl[j];
        }
        if (a.c.gate && live) return;
        if (!live) {
            if (!a.spec_final_direct && u.write_final && a.sT) {
                const float* src = a.spec_states + ((size_t)u.spec * H + h) * (D * D);
                const size_t off = ((size_t)u.seq * H + h) * (D * D);
                for (int i = threadIdx.x; i < D * D; i += blockDim.x) {
                    if (a.state_bf16) ((uint16_t*)a.sT)[off + i] = (uint16_t)pack_bf16(src[i], 0.f);
                    else ((float*)a.sT)[off + i] = src[i];
                }
            }
            return;
        }
    }
    const int64_t tok0 = beg + (int64_t)CH * u.chunk0;
    const int nc = u.n_chunks;
    // A warm-start segment runs `warm` chunks before its own: steps 0 .. W-1
    // are chunks chunk0-W .. chunk0-1, over which the state wavefronts form
    // the transfer and the state from zero side by side, and step W + c is
    // chunk chunk0 + c.
    const int W = BSUM ? 0 : u.warm;  // the K1 pass of the pipeline has no warm-start units
    const int n_steps = nc + W;
    // barrier intervals: -3, -2, -1, then 0 .. n_main - 1 (even)
    const int n_main = (n_steps + 1) & ~1;
    if (wave < 8) {
        // state wavefronts
        f32x4 S[8][1];
        if (W > 0) identity_state(S, w8, gg, m);
        else load_unit_state(a, u, h, S, w8, gg, m);
        // a unit with a speculation slot but no warm-up has nothing to
        // speculate on: its flags read "vanished"
        if (W == 0 && u.spec >= 0 && !a.fixup && lane == 0) a.spec_flags[((size_t)u.spec * H + h) * 8 + w8] = 0;
        lds_barrier();  // start-up: the first chunk is staged
        const int rem = (int)(end - tok0);
        // K1 pass: whether this wavefront's tile of the transfer lives, and
        // every tile's flag (written when its wavefront leaves the transfer)
        bool m_nz = true;
        volatile int32_t* m_flags = (volatile int32_t*)(smem + F_MFL);
        // the record of chunk c is complete in its interval (its T' was
        // formed in the previous one) and its slot is overwritten after the
        // next barrier: the state wavefronts other than WAVE_QK (whose phase-2
        // role is the heaviest) copy it out then, two 16-byte vectors per
        // thread
        static_assert(REC_HBM_VEC == 2 * 7 * 64 && WAVE_QK < 8, "seven wavefronts copy a record out");
        auto copy_out = [&](int c, const uint8_t* rec) __attribute__((always_inline)) {
            u32x4* dst = (u32x4*)(a.c.rec + ((size_t)h * a.c.total_chunks + u.rec_chunk0 + c) * REC_HBM_BYTES);
            const u32x4* src = (const u32x4*)rec;
            const int v0 = (w8 < WAVE_QK ? w8 : w8 - 1) * 64 + lane, v1 = v0 + 7 * 64;
            const u32x4 x0 = src[v0];
            const u32x4 x1 = src[v1];
            dst[v0] = x0;
            dst[v1] = x1;
        };
        // the V block of step i (5-slot ring)
        auto vblk = [&](int i) __attribute__((always_inline)) { return vrs + ring_off((i % 5) * VBLK_BYTES); };
        auto step = [&](int c, int i, auto role) __attribute__((always_inline)) {
            const uint8_t* rec = recs + ring_off((i % 4) * REC_BYTES);
            if constexpr (BSUM) {
                f32x4 unused[1];
                if (u.out_slot >= 0) chain_step<1, true, false, !BSUM>(rec, vblk(i), S, w8, lane, unused);
                if constexpr (decltype(role)::value != 2) copy_out(c, rec);
            } else {
                f32x4 oacc[1];
                chain_step<1, true, true, !BSUM>(rec, vblk(i), S, w8, lane, oacc);
                store_output(a, h, tok0 + (int64_t)CH * c, chunk_rows(rem, c), oacc[0], w8, gg, m);
            }
        };
        // one loop per phase-2 role (0: none, 1: rows 4 w8.. of T', 2: A_qk and
        // L), so that each loop body is one block in which phase 2 of later
        // chunks (independent of the chain) interleaves with the chain over chunk i
        auto run = [&](auto role) __attribute__((always_inline)) {
            constexpr int R = decltype(role)::value;
            auto gram = [&](int c) __attribute__((always_inline)) {  // A_qk and L of chunk c
                if constexpr (R == 2) {
                    const uint8_t* scr = scrs + ring_off((c & 1) * K1_NB);
                    const float* scr_b = (const float*)((const uint8_t*)scr_betas + ring_off((c & 1) * 64));
                    float* lb = (float*)(lbs + ring_off((c & 1) * LB_BYTES));
                    k1_grams(lane, recs + ring_off((c % 4) * REC_BYTES), scr, scr_b, lb, lb + LB_BETA / 4);
                }
            };
            auto solve = [&](int c) __attribute__((always_inline)) {  // rows of T' of chunk c
                if constexpr (R == 1) {
                    const float* lb = (const float*)(lbs + ring_off((c & 1) * LB_BYTES));
                    k1_tsolve(lane, fused_t_block(w8), recs + ring_off((c % 4) * REC_BYTES), lb, lb + LB_BETA / 4);
                }
            };
            lds_barrier();  // interval -3: phase 1 of chunk 0
            gram(0);
            lds_barrier();  // interval -2
            gram(1);
            solve(0);
            lds_barrier();  // interval -1
            if (W > 0) {
                // the transfer M (S, from the identity, V := 0) and the state
                // from zero (Z) over the same warm-up records, each with the
                // arithmetic of its own chain (pre_scan's M and B chains)
                f32x4 Z[8][1];
#pragma unroll
                for (int t = 0; t < 8; ++t) Z[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int i = 0; i < W; ++i) {
                    gram(i + 2);
                    solve(i + 1);
                    // the role's work first: interleaved with the two states'
                    // step it does not fit the registers
                    __builtin_amdgcn_sched_barrier(0);
                    chain_step_warm<!BSUM>(recs + ring_off((i % 4) * REC_BYTES), vblk(i), S, Z, w8, lane);
                    lds_barrier();
                }
                const bool live = tile_nonzero(S);
                if (lane == 0) a.spec_flags[((size_t)u.spec * H + h) * 8 + w8] = live ? 1 : 0;
#pragma unroll
                for (int t = 0; t < 8; ++t) S[t][0] = Z[t][0];
            }
            int i0 = W;
            if constexpr (BSUM) {
                if (u.out_slot >= 0 && a.m_out) {
                    // the segment's transfer M (from the identity, V := 0)
                    // beside its B summary, over the same records, each with
                    // the arithmetic of its own chain. A tile of M that is
                    // exactly zero stays zero (its columns evolve on their
                    // own), so every 4 chunks a wavefront whose tile vanished
                    // leaves M and continues with B alone.
                    f32x4 M[8][1];
                    identity_state(M, w8, gg, m);
                    bool live = true;
                    while (live && i0 < n_steps) {
                        gram(i0 + 2);
                        solve(i0 + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        const uint8_t* rec = recs + ring_off((i0 % 4) * REC_BYTES);
                        chain_step_warm<!BSUM>(rec, vblk(i0), M, S, w8, lane);
                        if constexpr (R != 2) {
                            __builtin_amdgcn_sched_barrier(0);
                            copy_out(i0 - W, rec);
                        }
                        lds_barrier();
                        ++i0;
                        if ((i0 & 3) == 0) live = tile_nonzero(M);
                    }
                    const bool nz = tile_nonzero(M);
                    if (lane == 0) {
                        a.m_live_out[((size_t)u.out_slot * H + h) * 8 + w8] = nz ? 1 : 0;
                        m_flags[w8] = nz ? 1 : 0;
                    }
                    m_nz = nz;
                    if (nz) store_transfer(a.m_out + ((size_t)u.out_slot * H + h) * (D * D), M, w8, gg, m);
                }
            }
            for (int i = i0; i < n_steps; ++i) {
                gram(i + 2);
                solve(i + 1);
                step(i - W, i, role);
                lds_barrier();
            }
            for (int i = n_steps; i < n_main; ++i) lds_barrier();
        };
        if (fused_t_role(w8)) run(std::integral_constant<int, 1>{});
        else if (w8 == WAVE_QK) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 0>{});
        if constexpr (BSUM) {
            if (u.out_slot >= 0 && a.m_out) {
                // the merge reads every tile of M once any flag is set: a tile
                // that vanished is stored as zeros when another one lives
                lds_barrier();  // the last, after every tile's flag
                int any = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) any |= m_flags[j];
                if (!m_nz && any) zero_transfer(a.m_out + ((size_t)u.out_slot * H + h) * (D * D), w8, gg, m);
            }
        }
        if (u.out_slot >= 0) store_state(a.carries + ((size_t)u.out_slot * H + h) * (D * D), S, w8, gg, m);
        if (u.spec >= 0 && !a.fixup && !a.spec_final_direct) {
            if (u.write_final) store_state(a.spec_states + ((size_t)u.spec * H + h) * (D * D), S, w8, gg, m);
        } else {
            store_unit_state(a, u, h, S, w8, gg, m);
        }
    } else {
        // K1 wavefronts: chunk c is loaded into register set c & 1
        RowChunkF r0, r1;
        const RowLaneOffsets lo = row_lane_offsets(H, a.c.Hk, w8, lane);
        const uint32_t g_off = g_dma_off(H, w8, lane);
        const uint32_t v_off = v_dma_off(H, w8 & 3, lane);
        // rows from the first chunk the unit runs (its warm-up, if any)
        const int64_t tok_k1 = tok0 - (int64_t)CH * W;
        const RowStreams rs = row_streams(a.c.q, a.c.k, a.c.v, a.c.g, a.c.beta, H, a.c.Hk, tok_k1, h,
                                          h / a.c.group, w8);
        // tokens of the unit from that chunk on (sequences are < 2^31 tokens):
        // its rows end with its last chunk, so the loads issued ahead for the
        // chunks after it (the loop's tail) read zeros and touch no memory
        const int64_t unit_end = tok0 + (int64_t)CH * nc < end ? tok0 + (int64_t)CH * nc : end;
        const int rem = (int)(unit_end - tok_k1);
        // step i -> chunk i from tok_k1. The warm-up chunks form no output
        // and read no q: its rows read as zeros, and no record field that
        // the warm-up uses depends on them.
        auto load_g = [&](int i) __attribute__((always_inline)) {
            k1_load_g_dma(rs, i, chunk_rows(rem, i), g_off, w8, grs + (i & 3) * GRING_BYTES);
        };
        // the V block of step i: block w8 & 3, by the wavefronts with
        // (w8 >> 2) = i - 3 - (the odd interval that issues it), see below
        auto load_v = [&](int i) __attribute__((always_inline)) {
            k1_load_v_dma(rs, i, chunk_rows(rem, i), v_off, w8 & 3, vrs + ring_off((i % 5) * VBLK_BYTES));
        };
        auto load_rows = [&](RowChunkF& rc, int i) __attribute__((always_inline)) {
            const int nr = chunk_rows(rem, i);
            k1_load_rows_f<GVA>(rs, i, nr, i >= W ? nr : 0, lo, rc, w8);
        };
        auto load = [&](RowChunkF& rc, int i) __attribute__((always_inline)) {
            load_g(i);
            load_rows(rc, i);
        };
        // the staging and scratch slots are compile-time constants: chunk c
        // uses slot c & 1 of both rings
        auto stage = [&](RowChunkF& rc, auto slot) __attribute__((always_inline)) {
            constexpr int S = decltype(slot)::value;
            // the register set is read only from here on (see below)
            asm volatile("" : "+v"(rc.qk), "+v"(rc.b));
            k1_stage_f(rc, w8, lane, lo, stgs + S * FSTG_NB, stg_betas + 16 * S);
        };
        // interval i works on chunk i + 3 (staging and scratch slot R = (i + 3) & 1)
        // and stages chunk i + 4 (slot 1 - R)
        auto interval = [&](int i, RowChunkF& rc, auto rslot) __attribute__((always_inline)) {
            constexpr int R = decltype(rslot)::value;
            // Phase 1 reads LDS only after the barrier that ends the previous
            // interval, and the staging of rc waits for its loads there too:
            // the empty redefinitions keep the compiler from hoisting
            // either above that barrier.
            // the g rows of chunk i + 6 first: their slot was last read in
            // the previous interval
            load_g(i + 6);
            // Every other interval (i odd: slot R = 0), the V blocks of
            // steps i + 3 (wavefronts 8..11) and i + 4 (12..15). A V block
            // is read by the state wavefronts in the interval of its step,
            // so five are live in interval i: i .. i + 4 (slot (i + 4) % 5
            // was last read in interval i - 1). Like the g rows, it is
            // complete once the wait for this interval's register loads,
            // issued after it, returns (two intervals on, before the
            // barrier that precedes its read).
            if constexpr (R == 0) load_v(i + 3 + (w8 >> 2));
            RawChunk raw;
            k1_read_staged_f(stgs + R * FSTG_NB, stg_betas + 16 * R, grs + ((i + 3) & 3) * GRING_BYTES, lane, lo, raw);
            // the record slot as an opaque uniform offset, so every record
            // access of the phase is one per-lane base plus immediate offsets
            k1_phase1<!BSUM>(raw, w8, lane, recs + ring_off(((i + 3) % 4) * REC_BYTES), scrs + R * K1_NB,
                      scr_betas + 16 * R);
            stage(rc, std::integral_constant<int, 1 - R>{});
            load_rows(rc, i + 6);
            lds_barrier();
        };
        using Z = std::integral_constant<int, 0>;
        using O = std::integral_constant<int, 1>;
        load(r0, 0);
        load(r1, 1);
        stage(r0, Z{});
        load(r0, 2);
        lds_barrier();  // start-up: chunk 0 staged
        interval(-3, r1, Z{});
        interval(-2, r0, O{});
        interval(-1, r1, Z{});
        for (int i = 0; i < n_main; i += 2) {
            interval(i, r0, O{});
            interval(i + 1, r1, Z{});
        }
        if constexpr (BSUM) {
            if (u.out_slot >= 0 && a.m_out) lds_barrier();  // the transfer flags' barrier
        }
    }
}

template <bool GVA>
__global__ __launch_bounds__(1024) void kda_fused(K2Args a) {
    fused_body<GVA, false>(a);
}

// The fix-up and publish launches (a.fixup): the same body under a symbol of
// its own, so that kernel traces and statistics tell them from the main launch.
template <bool GVA>
__global__ __launch_bounds__(1024) void kda_fused_fixup(K2Args a) {
    fused_body<GVA, false>(a);
}

// K1 of the segmented CP pipeline with pre_scan: the records of every chunk,
// written once, and each segment's B and M summaries.
template <bool GVA>
__global__ __launch_bounds__(1024) void kda_k1_bsum(K2Args a) {
    fused_body<GVA, true>(a);
}

// ---------------------------------------------------------------------------
// K2 over materialised K1 records (two-kernel serial form and CP segment-K2):
// one workgroup of 8 wavefronts per (unit, head), wavefront w on value
// columns 16w..16w+15.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void kda_k2_recur(K2Args a) {
    if (a.c.gate && *a.c.gate == 0) return;  // fallback not armed
    __shared__ __align__(16) uint8_t recs[2][K2_STAGE_BYTES];
    const int H = a.c.H;
    const int h = blockIdx.x % H;
    const UnitDesc u = a.units[blockIdx.x / H];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gg = lane >> 4, m = lane & 15;
    int64_t beg, end;
    seq_bounds(a.c, u.seq, beg, end);
    const int64_t tok0 = beg + (int64_t)CH * u.chunk0;
    f32x4 S[8][1];
    load_unit_state(a, u, h, S, wave, gg, m);
    const uint8_t* rb = a.c.rec + ((size_t)h * a.c.total_chunks + u.rec_chunk0) * REC_HBM_BYTES;
    const int rem = (int)(end - tok0);
    const VRows vrows{(const uint8_t*)a.c.v + ((size_t)tok0 * H + h) * (D * 2), (uint32_t)H * (D * 2), rem};
    record_loop(rb, vrows, u.n_chunks, recs, [&](int ci, const uint8_t* r) {
        f32x4 oacc[1];
        chain_step<1, true, true, false>(r, r + REC_BYTES, S, wave, lane, oacc);
        store_output(a, h, tok0 + (int64_t)CH * ci, chunk_rows(rem, ci), oacc[0], wave, gg, m);
    });
    store_unit_state(a, u, h, S, wave, gg, m);
}

// ---------------------------------------------------------------------------
// CP merge: carry_0 = S0 (or 0); carry_{s+1} = M_s carry_s + B_s, in segment
// order, on fp32 MFMA. Where M_s vanished (every tile exactly zero), carry_{s+1}
// is B_s itself and depends on nothing before it, so the carries fall into
// runs, each started by such a segment (or by segment 0) and continued over
// the following live transfers. One workgroup of 8 wavefronts per (segment,
// head, 16-column value tile); the workgroup of a segment that starts a run
// computes the run, the others return at once. A segment whose predecessor's
// transfer vanished takes its start state from B directly (segment-K2 reads
// it), so only carry_0 and the carries after live transfers are written.
// Carry_0 is always written, so that segment-K2 never reads initial_state
// while another segment writes final_state in place. Wavefront t owns carry
// rows 16t..16t+15, and each step splits its 32 MFMAs over two accumulators.
// The run's length is found before its first step, so the steps test no
// flag, and the summaries of each step load while the step before it runs.
// In the product M carry, lane group gg of MFMA step q takes key index
// merge_k(gg, q), and M comes in that operand order (m_operand_index), so
// each of a step's eight M loads per wavefront reads 1 KiB of consecutive
// memory; with the carry's LDS rows padded to MERGE_CST floats the 64 lanes
// of each carry read fall on distinct banks. The carry is double-buffered in
// LDS, so a step needs one barrier.
// ---------------------------------------------------------------------------
constexpr int MERGE_CST = 17;
struct MergeOperands {
    f32x4 m[8];  // M_s[16 wave + m][merge_k(gg, 4j) .. + 3], j = 0..7 (m_operand_index order)
    f32x4 b;     // B_s[16 wave + 4 gg + v][16 vt + m], v = 0..3
};

__global__ __launch_bounds__(512, 4) void kda_cp_merge(MergeArgs a) {
    if (a.c.gate && *a.c.gate == 0) return;  // fallback not armed
    __shared__ float carry[2][D][MERGE_CST];
    __shared__ int32_t run_end;
    const int H = a.c.H;
    const int vt = blockIdx.x & 7;
    const int h = (blockIdx.x >> 3) % H;
    const MergeSeg sg = a.segs[(blockIdx.x >> 3) / H];
    const MergeDesc it = a.items[sg.item];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gg = lane >> 4, m = lane & 15;
    const int n_sum = it.n_segments - 1;  // summaries (segments 0 .. n-2)
    auto flags = [&](int j) __attribute__((always_inline)) {
        const int32_t* fl = a.m_live + ((size_t)(it.prescan0 + j) * H + h) * 8;
        int32_t any = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) any |= fl[k];
        return any;
    };
    const int s0 = sg.seg;
    // a segment after a live transfer lies inside a run started earlier
    if (s0 > 0 && __builtin_amdgcn_readfirstlane(flags(s0 - 1)) != 0) return;
    // a run of this segment alone has nothing to compute (segment-K2 reads
    // B_{s0-1} itself)
    const bool live0 = s0 < n_sum && __builtin_amdgcn_readfirstlane(flags(s0)) != 0;
    if (s0 > 0 && !live0) return;
    // the run: transfers s0 .. run_end - 1 are live (the first vanished one,
    // or the last summary, ends it), so its length is known before the
    // first step and the steps need no flag of their own
    if (tid == 0) run_end = live0 ? n_sum : s0;
    __syncthreads();
    if (live0)
        for (int j = s0 + 1 + tid; j < n_sum; j += 512)
            if (flags(j) == 0) atomicMin(&run_end, j);
    if (s0 == 0) {
        const size_t s0_off = ((size_t)it.seq * H + h) * (D * D);
        const float* si = (a.s0 && !a.state_bf16) ? (const float*)a.s0 + s0_off : nullptr;
        const uint16_t* sih = (a.s0 && a.state_bf16) ? (const uint16_t*)a.s0 + s0_off : nullptr;
        float* c0 = a.carries + ((size_t)it.carry0 * H + h) * (D * D);
        for (int i = tid; i < D * 16; i += 512) {
            const int row = i >> 4, col = i & 15;
            const float val = si ? si[row * D + 16 * vt + col] : (sih ? bf16_lo(sih[row * D + 16 * vt + col]) : 0.f);
            carry[0][row][col] = val;
            c0[row * D + 16 * vt + col] = val;
        }
    } else {
        // the run starts from B_{s0-1}
        const float* B = a.b_seg + ((size_t)(it.prescan0 + s0 - 1) * H + h) * (D * D);
        for (int i = tid; i < D * 16; i += 512) {
            const int row = i >> 4, col = i & 15;
            carry[0][row][col] = B[row * D + 16 * vt + col];
        }
    }
    __syncthreads();
    const int n_run = __builtin_amdgcn_readfirstlane(run_end - s0);
    // summaries of step s (transfer s0 + s; clamped to the run's last, so
    // every load is valid and unconditional)
    auto load = [&](int s, MergeOperands& x) __attribute__((always_inline)) {
        const int jj = s0 + (s < n_run ? s : n_run - 1);
        const size_t sum_off = ((size_t)(it.prescan0 + jj) * H + h) * (D * D);
        const float* M = a.m_seg + sum_off;
        const float* B = a.b_seg + sum_off;
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) x.b[vv] = B[(16 * wave + 4 * gg + vv) * D + 16 * vt + m];
        const __amdgpu_buffer_rsrc_t mr = chunk_rsrc(M, (uint32_t)(D * D * 4));
#pragma unroll
        for (int k = 0; k < 8; ++k)
            x.m[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                mr, (int)(((wave * 8 + k) * 64 + lane) * 16), 0, 0));
    };
    // carry_{s0+s+1} = M carry + B
    auto step = [&](int s, MergeOperands& x) __attribute__((always_inline)) {
        // the operands are read only from here on (keeps their wait here)
        asm volatile("" : "+v"(x.m[0]), "+v"(x.m[1]), "+v"(x.m[2]), "+v"(x.m[3]), "+v"(x.m[4]),
                     "+v"(x.m[5]), "+v"(x.m[6]), "+v"(x.m[7]), "+v"(x.b));
        // the carry operands of the products, 16 at a time, each half read
        // before its first product: one wait per half, not one per product
        const float(*cur)[MERGE_CST] = carry[s & 1];
        f32x4 acc0 = x.b, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 32; hh += 16) {
            float cb[16];
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) cb[qq] = cur[merge_k(gg, hh + qq)][m];
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) asm volatile("" : "+v"(cb[qq]));
#pragma unroll
            for (int qq = 0; qq < 16; qq += 2) {
                acc0 = mfma_f32_k4(x.m[(hh + qq) >> 2][qq & 3], cb[qq], acc0);
                acc1 = mfma_f32_k4(x.m[(hh + qq) >> 2][(qq & 3) + 1], cb[qq + 1], acc1);
            }
        }
        const f32x4 acc = acc0 + acc1;
        float(*nxt)[MERGE_CST] = carry[(s + 1) & 1];
        float* cn = a.carries + ((size_t)(it.carry0 + s0 + s + 1) * H + h) * (D * D);
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            nxt[16 * wave + 4 * gg + vv][m] = acc[vv];
            cn[(16 * wave + 4 * gg + vv) * D + 16 * vt + m] = acc[vv];
        }
        // orders the LDS carry only (no wait for the global stores or the
        // summaries in flight)
        lds_barrier();
    };
    if (n_run <= 0) return;
    // two operand sets in flight: a step's summaries load a step ahead of
    // the step before it (deeper rings measured slower: the compiler then
    // waits for every load at the loop head)
    MergeOperands xa, xb;
    load(0, xa);
    load(1, xb);
    for (int s = 0; s < n_run; s += 2) {
        step(s, xa);
        load(s + 2, xa);
        if (s + 1 >= n_run) break;
        step(s + 1, xb);
        load(s + 3, xb);
    }
}

// ---------------------------------------------------------------------------
// Static scratch of the no-allocation prefill (kda_prefill_noalloc): the
// workspace of a call that may not allocate, one copy per device, held until
// the process ends. Host code must never pass the array's name to a kernel
// (on the host it is only a stand-in): the runtime looks up each device's
// address with hipGetSymbolAddress, once, and passes that.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch_address(void** ptr) { return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch)); }

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {
hipError_t launch_fused_any(const K2Args& a, hipStream_t s, bool bsum) {
    const long long n = (long long)a.n_units * a.c.H;
    if (n <= 0) return hipSuccess;
    static const hipError_t attr = [] {
        const void* fns[] = {(const void*)kda_fused<false>, (const void*)kda_fused<true>,
                             (const void*)kda_fused_fixup<false>, (const void*)kda_fused_fixup<true>,
                             (const void*)kda_k1_bsum<false>, (const void*)kda_k1_bsum<true>};
        for (const void* f : fns) {
            const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, FUSED_LDS);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    const dim3 grid((unsigned)n), block(1024);
    if (bsum) {
        if (a.c.group > 1) hipLaunchKernelGGL(kda_k1_bsum<true>, grid, block, FUSED_LDS, s, a);
        else hipLaunchKernelGGL(kda_k1_bsum<false>, grid, block, FUSED_LDS, s, a);
    } else if (a.fixup) {
        if (a.c.group > 1) hipLaunchKernelGGL(kda_fused_fixup<true>, grid, block, FUSED_LDS, s, a);
        else hipLaunchKernelGGL(kda_fused_fixup<false>, grid, block, FUSED_LDS, s, a);
    } else {
        if (a.c.group > 1) hipLaunchKernelGGL(kda_fused<true>, grid, block, FUSED_LDS, s, a);
        else hipLaunchKernelGGL(kda_fused<false>, grid, block, FUSED_LDS, s, a);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_fused(const K2Args& a, hipStream_t s) { return launch_fused_any(a, s, false); }

hipError_t launch_k1_bsum(const K2Args& a, hipStream_t s) { return launch_fused_any(a, s, true); }

// bf16 beta -> fp32 beta (exact), for callers that keep beta in bf16.
__global__ __launch_bounds__(256) void kda_beta_to_f32(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                                       int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = bf16_lo(src[i]);
}

hipError_t launch_beta_to_f32(const uint16_t* src, float* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(kda_beta_to_f32, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_k1_prepare(const K1Args& a, hipStream_t s) {
    long long n = (long long)a.c.total_chunks * a.c.H;
    if (n <= 0) return hipSuccess;
    // a gated launch is usually empty: a capped grid that strides over the
    // items costs little to dispatch when every workgroup returns at once
    if ((a.c.gate || a.gate_flags) && n > 2048) n = 2048;
    if (a.c.group > 1) hipLaunchKernelGGL(kda_k1_prepare<true>, dim3((unsigned)n), dim3(512), 0, s, a);
    else hipLaunchKernelGGL(kda_k1_prepare<false>, dim3((unsigned)n), dim3(512), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_k2_recur(const K2Args& a, hipStream_t s) {
    const long long n = (long long)a.n_units * a.c.H;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(kda_k2_recur, dim3((unsigned)n), dim3(512), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cp_merge(const MergeArgs& a, hipStream_t s) {
    const long long n = (long long)a.n_segs * a.c.H * 8;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(kda_cp_merge, dim3((unsigned)n), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
