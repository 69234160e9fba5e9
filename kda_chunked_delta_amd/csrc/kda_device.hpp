// Device building blocks of the KDA forward prefill for gfx950 (CDNA4).
//
// The chunked form follows the commit summary of "feat(kda/sm90): FlashKDA
// prefill port + intracard-CP prefill" (cuLA pull request #103): K1 prepares,
// per 16-token chunk, the decayed q/k, beta and the WY inverse; K2 runs the
// inter-chunk recurrence over a 128 x 128 fp32 state per head. The per-chunk
// algebra, for a chunk of rows r = 0..15 with start state S0, in-chunk
// cumulative log-decay G_r (per key channel) and G_C = G at the last row:
//   A_kk[r,i] = sum_d k_rd k_id exp(G_rd - G_id)   (i < r)
//   A_qk[r,i] = sum_d q_rd k_id exp(G_rd - G_id)   (i <= r)
//   L  = strict-lower(diag(beta) A_kk),   T' = (I + L)^-1 diag(beta)
//   X  = k * exp G,   Qt = q * exp G,   Kt = k * exp(G_C - G)
//   U  = T' (V - X S0)
//   O  = Qt S0 + A_qk U,   S_next = Diag(exp G_C) S0 + Kt^T U
// U is the WY form U~ - W S0 with W = T' X and U~ = T' V regrouped, so K1
// never forms W or U~ and K2 applies T' to the 16 x 16 tile V - X S0.
// All matrix products run on bf16 MFMA with fp32 accumulation; the state and
// the decays stay fp32, and T' is formed in fp32 and applied as a hi/lo pair
// of bf16 MFMA operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

constexpr int D = 128;   // head dimension (dk = dv)
constexpr int CH = 16;   // chunk length

// ---------------------------------------------------------------------------
// K1 -> K2 chunk record: everything K2 needs for one (chunk, head), in the
// order in which each wavefront lane reads its MFMA fragments. Lane l has
// group gg = l >> 4 and index m = l & 15; dkperm(p, gg, j) =
// 32p + 16(j >> 2) + 4gg + (j & 3) is the key-channel order of one 16x16x32
// MFMA step, chosen so the fp32 state, held in 16x16 accumulator tiles,
// feeds the next MFMA as an operand without any shuffle.
//   REC_Q  : Qt fragments [p 4][lane 64][8 bf16]: Qt[m][dkperm(p, gg, j)]
//   REC_X  : X fragments, same layout as REC_Q
//   REC_KT : Kt^T fragments [t 8][slot 64][4 bf16]: lane l's fragment
//            Kt[4gg + j][16t + m] in slot kv_slot(l) (materialised records,
//            and the LDS records of the K1 pass of the segmented pipeline);
//            the fused kernel keeps them in LDS as 4-channel row segments
//            instead: slot kv_store_slot(a, 4b + c) holds
//            Kt[4a + b][16t + 4c + j], and lane l reads slot kv_load_slot(l)
//            with a transposing load
//   REC_AQK: A_qk fragment [lane 64][4 bf16]: A_qk[m][4gg + j] (masked i <= r)
//   REC_GC : exp(G_C) [128] fp32, channel c = 16t + 4gg + v at position
//            32gg + 4t + v: lane (gg, m) of a state wavefront reads the pair
//            at 2 * lane, which holds channels 16(m >> 1) + 4gg + 2(m & 1) + 0..1
//   REC_T  : T' fragments, hi then lo [2][lane 64][4 bf16]: T'[m][4gg + j]
// A record holds no V: the chunk's value rows are a copy of the input, and
// they reach LDS as a V block of their own (VBLK_*), straight from memory.
// HBM holds the same bytes when K1 is materialised.
// ---------------------------------------------------------------------------
constexpr int REC_Q = 0;
constexpr int REC_X = 4096;
constexpr int REC_KT = 8192;
constexpr int REC_AQK = 12288;
constexpr int REC_GC = 12800;
constexpr int REC_T = 13312;
constexpr int REC_BYTES = 14336;
constexpr int REC_HBM_BYTES = REC_BYTES;
constexpr int REC_HBM_VEC = REC_HBM_BYTES / 16;  // 896 16-byte vectors

// V block of one chunk (LDS only): its 16 value rows (256 bytes each) in four
// 1 KiB blocks of four rows. Granule gi (16 bytes, columns 8gi .. 8gi + 7)
// of row 4b + r sits at granule position 16r + (gi ^ (2r + 8(b & 1))) of
// block b. A state lane l = 16gg + 4r + c loads, with the transposing load,
// the 8-byte segment of row 4gg + r and columns 16n + 4c .. + 3 of value
// tile n, and so receives its 16x16x16 B fragment V[4gg + j][16n + m]. Per
// half-wavefront the 16 granules a tile's load touches sit at distinct
// positions modulo 16 (no bank conflict); the writers store whole 1 KiB
// blocks.
constexpr int VBLK_BYTES = 4096;
__device__ __forceinline__ int vblk_off(int row, int gi) {
    const int b = row >> 2, r = row & 3;
    return 1024 * b + 16 * (16 * r + (gi ^ (2 * r + 8 * (b & 1))));
}
__device__ __forceinline__ int vblk_load_off(int lane, int n) {
    const int c = lane & 3;
    return vblk_off(4 * (lane >> 4) + ((lane >> 2) & 3), 2 * n + (c >> 1)) + 8 * (c & 1);
}

// K1 scratch of one chunk (LDS only), from phase 1 to phase 2:
//   K1_KA, K1_QA: the Gram row factors k exp(G - G_ref), q exp(G - G_ref) as
//                 fragments in the REC_Q layout, with G_ref = 0 (the chunk
//                 start) or G_7 (see k1_phase1)
//   K1_KB       : the column factor k exp(G_ref - G), each 16x16x32 fragment
//                 split into halves: K-step p holds at p * 1024 + 8 l the
//                 first half of lane l's fragment (from wavefront 2p) and at
//                 p * 1024 + 512 + 8 l the second (from wavefront 2p + 1), so
//                 that each wavefront writes 512 contiguous bytes
//   K1_BETA     : beta of the chunk's 16 rows, fp32
constexpr int K1_KA = 0;
constexpr int K1_KB = 4096;
constexpr int K1_QA = 8192;
constexpr int K1_BETA = 12288;
constexpr int K1_BYTES = K1_BETA + 64;
constexpr int K1_NB = K1_BETA;  // the Gram factors alone (beta kept elsewhere by the fused kernel)
// per T' wavefront, private LDS: L^T as fp32 [16][K1_LSTRIDE] (a 20-float row
// stride puts the 16 lanes of each b128 phase on distinct banks)
constexpr int K1_LSTRIDE = 20;
constexpr int K1_LBYTES = 16 * K1_LSTRIDE * 4;
// L^T shared by the fused kernel's T' wavefronts: K1_LBYTES of L^T, then
// beta of the chunk's 16 rows
constexpr int LB_BETA = K1_LBYTES;
constexpr int LB_BYTES = K1_LBYTES + 64;

// Phase-2 roles: wavefronts 0..3 (one per SIMD) each form four rows of T',
// wavefront WAVE_QK forms A_qk (and, in the fused kernel, L for the others).
constexpr int N_WAVE_T = 4;
constexpr int WAVE_QK = 5;

// The fused kernel's T' wavefronts among its state wavefronts 0..7. State
// wavefront w runs on SIMD w % 4 beside state wavefront w ^ 4 and two K1
// wavefronts, so the T' role of WAVE_QK's SIMD partner (1) goes to wavefront
// 6 instead: WAVE_QK's SIMD then carries the Gram role alone (measured 1-3%
// faster on every fused workload than T' on wavefronts 0..3).
// fused_t_role(w): wavefront w forms T' rows; fused_t_block(w): which block
// of four rows it forms (meaningful only where fused_t_role(w) holds).
__device__ __forceinline__ bool fused_t_role(int w) {
    static_assert(WAVE_QK == 5, "the T' wavefronts avoid WAVE_QK's SIMD");
    return w == 0 || w == 2 || w == 3 || w == 6;
}
__device__ __forceinline__ int fused_t_block(int w) { return w == 6 ? 1 : w; }

constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (round to nearest even), one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{pack_bf16(a, b), pack_bf16(c, d)};
}
__device__ __forceinline__ u32x2 pack4(const f32x4& x) { return pack4(x[0], x[1], x[2], x[3]); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// D(16x16) += A(16x32) B(32x16), bf16 in, fp32 accumulate.
// A: lane holds A[m][8gg + j]; B: lane holds B[8gg + j][m]; C: lane holds C[4gg + v][m].
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D(16x16) += A(16x16) B(16x16), bf16 in; A: A[m][4gg + j], B: B[4gg + j][m].
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// D(16x16) += A(16x4) B(4x16), fp32; A: A[m][gg], B: B[gg][m].
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroup barrier that waits only for this wavefront's LDS traffic, so
// global loads issued earlier (prefetch of later chunks) stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// x from lane (m - n) of the same 16-lane row, 0 for m < n (DPP row shift;
// folds into the consuming add).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x110 + N, 0xF, 0xF, true);
}
// x from lane K of the same 16-lane row (DPP row broadcast; folds into the
// consuming multiply).
template <int K>
__device__ __forceinline__ float row_newbcast(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x150 + K, 0xF, 0xF, true);
}

// 4 x 4 transpose of 16-bit elements across the four lanes of a quad: lane j
// holds elements x[0..3] as (x0 | x1 << 16, x2 | x3 << 16); afterwards it
// holds element j of lanes 0..3, in lane order. First the 2 x 2 blocks of
// dwords move between lanes j and j ^ 2, then each 2 x 2 block of halves is
// transposed between lanes j and j ^ 1 (DPP quad permutes and a byte
// permute).
__device__ __forceinline__ u32x2 quad_transpose16(u32x2 x, int lane) {
    const bool hi = (lane & 2) != 0;
    const uint32_t send = hi ? x.x : x.y;
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    const uint32_t y0 = hi ? recv : x.x;
    const uint32_t y1 = hi ? x.y : recv;
    const uint32_t p0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)y0, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)y1, 0xB1, 0xF, 0xF, false);
    // even lane: own low half, then the partner's; odd lane: the partner's
    // high half, then its own (v_perm_b32: bytes 0-3 from the second
    // operand, 4-7 from the first)
    const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
    return u32x2{__builtin_amdgcn_perm(p0, y0, sel), __builtin_amdgcn_perm(p1, y1, sel)};
}

// Slot of lane l's 8-byte Kt^T fragment in the fragment layout: lane
// l = 16g + 4a + j sits in slot 16g + 4((a + g) & 3) + j. The reads stay one
// contiguous 512-byte tile (each half-wavefront's 32 reads on distinct
// banks; two tiles per paired load), and the stores that K1 writes them with
// (lane (gg, 4a + j) -> fragment of lane 16a + 4gg + j, after a quad
// transpose) put each group of 16 lanes on 16 distinct 8-byte slots of a
// 128-byte bank row, so neither side has a bank conflict.
__device__ __forceinline__ int kv_slot(int l) { return (l & 0x33) | ((((l >> 2) + (l >> 4)) & 3) << 2); }

// Kt in the row-segment layout: K1 lane (gg, m) holds token m, channels 4gg .. 4gg + 3 of
// a tile, an 8-byte row segment, and stores it untransposed in slot
// kv_store_slot(gg, m). gfx950's transposing LDS load (ds_read_b64_tr_b16)
// works on groups of 16 lanes: lane 4r + c of a group loads row segment
// (r, c) of a 4 x 16 block of 16-bit elements, and lane i then receives
// column i of the block (its element i & 3 from the segments of lanes
// 4r + (i >> 2), r = 0..3; checked on the GPU with an in-bounds probe). A
// state lane l = 16gg + 4r + c therefore loads the segment of token 4gg + r
// and channels 4c .. 4c + 3, and receives tokens 4gg .. 4gg + 3 of channel
// m: its 16x16x16 MFMA fragment. Slots rotate the segment index by gg, so
// the loads of a 16-lane group stay in one 128-byte row (no bank conflict)
// and each group of 16 stores (fixed gg, m = 0..15) covers 16 distinct
// 8-byte positions of a 128-byte bank row (none either).
__device__ __forceinline__ int kv_store_slot(int gg, int m) {
    return 16 * (m >> 2) + 4 * (m & 3) + ((gg + (m >> 2)) & 3);
}
__device__ __forceinline__ int kv_load_slot(int l) { return (l & 0x3C) | (((l & 3) + (l >> 4)) & 3); }

// The transposing 8-byte LDS load (p: an LDS address).
__device__ __forceinline__ u32x2 lds_load_tr16(const uint8_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// Lane `lane`'s Kt^T fragment of tile t of a record: from the row-segment
// layout by a transposing load (KT_TR), else from the fragment layout. The
// fragment layout is the one records have in HBM: it serves two tiles per
// paired load, which the two-state steps of the segmented pipeline's K1
// pass need (with the transposing load its loads serialise, one per tile,
// and that pass ran 30% slower under weak decay); the fused kernel saves the
// quad transpose in K1 with the row segments.
template <bool KT_TR>
__device__ __forceinline__ u32x2 kt_frag(const uint8_t* rec, int t, int lane) {
    if constexpr (KT_TR) return lds_load_tr16(rec + REC_KT + t * 512 + kv_load_slot(lane) * 8);
    else return *(const u32x2*)(rec + REC_KT + t * 512 + kv_slot(lane) * 8);
}

// ---------------------------------------------------------------------------
// K1, phase 1 (8 wavefronts). Wavefront w owns key channels and value
// columns 16w..16w+15; lane (gg, m) holds token m of the chunk and channels
// 16w + 4gg + j, j = 0..3. Rows past nrows are zero (k = q = v = 0, g = 0,
// beta = 0), which leaves them inert.
// ---------------------------------------------------------------------------
struct RawChunk {
    u32x2 q, k;
    f32x4 g;
    float b;
};

// Buffer descriptor over [base, base + bytes): raw (unstrided) addressing,
// 32-bit data format. A load whose byte range ends past `bytes` returns
// zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of the input loads: default. (The streaming hint keeps a line
// out of L1 although the four wavefronts that read its quarters want it
// there, and measured slower.)
constexpr int BUF_POLICY = 0;

// ---------------------------------------------------------------------------
// Row-coalesced K1 input path (both K1 kernels). A per-lane load of phase 1's
// layout touches 16 rows with 32-64 bytes each and four wavefronts fetch
// every line; measured, that runs at about a third of the rate of whole-row
// loads. So the wavefronts load whole rows into registers (RowChunk):
// wavefront w rows 2w and 2w + 1 of g, and 16 bytes per lane of rows
// 4w .. 4w + 3 of q (w < 4) or of k (w >= 4) (measured 1-1.5% faster than
// two rows per wavefront of each). They write the rows to an LDS staging
// area, and after the next barrier each wavefront reads its phase-1
// fragments from there. (The fused kernel loads g straight into LDS
// instead.) K1 does not read v: the value rows are not part of a record.
// Staging of one chunk: rows in order; the 16-byte granules of row r are
// XOR-swizzled with r & 15, so both the row writes and phase 1's column
// reads (16 rows, one granule each) spread over all banks.
// ---------------------------------------------------------------------------
constexpr int STG_Q = 0;       // q  [16][256 B]
constexpr int STG_K = 4096;    // k  [16][256 B]
constexpr int STG_G = 8192;    // g  [16][512 B]
constexpr int STG_B = 16384;   // beta [16] fp32
constexpr int STG_BYTES = 16448;
constexpr int STG_NB = STG_B;  // the staged rows alone (beta kept elsewhere by the fused kernel)

// Staging byte offset of byte `byte` of row r of a 256-byte (bf16) row.
__device__ __forceinline__ int stg_act_off(int r, int byte) {
    return r * 256 + ((((byte >> 4) ^ r) & 15) << 4) + (byte & 15);
}
// Staging byte offset of byte `byte` of row r of a 512-byte (fp32) row.
__device__ __forceinline__ int stg_g_off(int r, int byte) {
    const int c = byte >> 4;
    return r * 512 + (((c & 16) | ((c ^ r) & 15)) << 4) + (byte & 15);
}

struct RowChunk {
    u32x4 qk;       // wavefronts 0-3: 16 bytes of q row 4w + (lane >> 4) at byte 16 (lane & 15); 4-7: of k
    f32x4 g;        // 16 bytes of row 2w + (lane >> 5) of g at byte 16 (lane & 31)
    float b;        // beta of row lane & 15 (wavefront 0 only)
};

// Per-lane constants of the row path of wavefront w.
struct RowLaneOffsets {
    uint32_t qk, g, beta;  // global byte offsets from the chunk's first row (qk: of q or k)
    int st_g;              // staging offset of the g row write
    int st_qk;             // staging offset of the q or k write (its tensor's area included)
    int rd_act, rd_g;      // staging offsets of phase 1's reads (q and k; g)
};

// H value heads (v, g, beta rows), Hk q/k heads (q, k rows)
__device__ __forceinline__ RowLaneOffsets row_lane_offsets(int H, int Hk, int wave, int lane) {
    const int r = 2 * wave + (lane >> 5), gg = lane >> 4, m = lane & 15;
    RowLaneOffsets o;
    const int r4 = 4 * (wave & 3) + (lane >> 4);
    o.qk = (uint32_t)r4 * (uint32_t)Hk * (D * 2) + (lane & 15) * 16;
    o.st_qk = (wave < 4 ? STG_Q : STG_K) + stg_act_off(r4, (lane & 15) * 16);
    o.g = (uint32_t)r * (uint32_t)H * (D * 4) + (lane & 31) * 16;
    o.beta = (uint32_t)m * (uint32_t)H * 4;
    o.st_g = stg_g_off(r, (lane & 31) * 16);
    o.rd_act = stg_act_off(m, 32 * wave + 8 * gg);
    o.rd_g = stg_g_off(m, 64 * wave + 16 * gg);
    return o;
}

// Row streams of one (unit, head): the first chunk's row bases and the bytes
// per token row of each tensor (all uniform). st_b is 0 on the wavefronts
// that do not read beta (every wavefront but 0), which makes their beta
// range empty.
struct RowStreams {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const uint8_t* g;
    const uint8_t* b;
    uint32_t st_qk, st_act, st_g, st_b;
};

// H value heads (v, g, beta rows), Hk q/k heads (value head h reads q/k
// head hq); the unit's first token is tok0.
__device__ __forceinline__ RowStreams row_streams(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                  const float* g, const float* beta, int H, int Hk, int64_t tok0,
                                                  int h, int hq, int wave) {
    RowStreams r;
    const int64_t crow = tok0 * H + h, crow_qk = tok0 * Hk + hq;
    r.q = (const uint8_t*)q + crow_qk * (D * 2);
    r.k = (const uint8_t*)k + crow_qk * (D * 2);
    r.v = (const uint8_t*)v + crow * (D * 2);
    r.g = (const uint8_t*)g + crow * (D * 4);
    r.b = (const uint8_t*)beta + crow * 4;
    r.st_qk = (uint32_t)Hk * (D * 2);
    r.st_act = (uint32_t)H * (D * 2);
    r.st_g = (uint32_t)H * (D * 4);
    r.st_b = wave == 0 ? (uint32_t)H * 4 : 0u;
    return r;
}

// Loads of chunk ci of the streams with nrows (0..16) valid rows. Each range
// covers nrows whole token rows, so the lanes of rows past them, and every
// lane when nrows = 0, read zeros and touch no memory. nrows_q (0 or nrows)
// is the rows of q alone: 0 where the chunk's use needs no q (a warm-up
// chunk), which then reads zeros for it. GVA = false: q/k heads are the
// value heads, and q/k share v's offsets and ranges.
template <bool GVA>
__device__ __forceinline__ void k1_load_chunk(const RowStreams& rs, int ci, int nrows, int nrows_q,
                                              const RowLaneOffsets& lo, RowChunk& rc, int wave) {
    const size_t c_act = (size_t)ci * (CH * (size_t)rs.st_act);
    size_t c_qk = c_act;
    uint32_t st_qk = rs.st_act;
    if constexpr (GVA) {
        c_qk = (size_t)ci * (CH * (size_t)rs.st_qk);
        st_qk = rs.st_qk;
    }
    // wavefronts 0-3 load q, 4-7 k (uniform per wavefront)
    const bool is_q = wave < 4;
    const uint8_t* qkb = (is_q ? rs.q : rs.k) + c_qk;
    const uint32_t n_qk = (uint32_t)(is_q ? nrows_q : nrows) * st_qk;
    rc.qk = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(chunk_rsrc(qkb, n_qk), (int)lo.qk, 0,
                                                                           BUF_POLICY));
    // g rows are twice as long as v rows, beta rows 1/64 of them
    rc.g = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
        chunk_rsrc(rs.g + 2 * c_act, (uint32_t)nrows * rs.st_g), (int)lo.g, 0, BUF_POLICY));
    rc.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        chunk_rsrc(rs.b + (c_act >> 6), (uint32_t)nrows * rs.st_b), (int)lo.beta, 0, BUF_POLICY));
}

// Valid rows of chunk ci when rem tokens of the sequence start at the unit's
// first token: clamp(rem - 16 ci, 0, 16), in 32-bit arithmetic. Written as
// scalar min/max so that the buffer ranges built on it stay in SGPRs (the
// compiler would otherwise pick the vector v_med3_i32, and every load would
// then need a waterfall loop over its descriptor). Both instructions write
// SCC, which the compiler must not keep live across them (a 64-bit address
// add split around them would lose its carry): hence the clobber.
__device__ __forceinline__ int chunk_rows(int rem, int ci) {
    int n = rem - CH * ci;
    asm("s_max_i32 %0, %0, 0\n\ts_min_i32 %0, %0, %1" : "+s"(n) : "i"(CH) : "scc");
    return n;
}

// Write a loaded RowChunk to the staging area stg (rows) and stg_b (the 16
// betas; stg + STG_B where the layout keeps them together).
__device__ __forceinline__ void k1_stage(const RowChunk& rc, int wave, int lane, const RowLaneOffsets& lo,
                                         uint8_t* stg, float* stg_b) {
    *(u32x4*)(stg + lo.st_qk) = rc.qk;
    *(f32x4*)(stg + STG_G + lo.st_g) = rc.g;
    if (wave == 0 && lane < 16) stg_b[lane] = rc.b;
}

// Phase 1's fragments of wavefront w from a staged chunk.
__device__ __forceinline__ void k1_read_staged(const uint8_t* stg, const float* stg_b, int lane,
                                               const RowLaneOffsets& lo, RawChunk& raw) {
    raw.q = *(const u32x2*)(stg + STG_Q + lo.rd_act);
    raw.k = *(const u32x2*)(stg + STG_K + lo.rd_act);
    raw.g = *(const f32x4*)(stg + STG_G + lo.rd_g);
    raw.b = stg_b[lane & 15];
}

// The fused kernel's row path: q and k as above, staged through registers
// into slots of FSTG_NB bytes; g goes from memory straight into a ring of
// LDS slots of GRING_BYTES (one per chunk, the staged layout of STG_G) by
// direct-to-LDS buffer loads, so the K1 wavefronts neither hold nor stage
// it. Lane l of wavefront w loads the 16-byte granule that the staged
// layout puts at slot l & 31 of row 2w + (l >> 5): a direct-to-LDS load
// writes lane l's 16 bytes at the wavefront's LDS base + 16 l (lanes
// past the descriptor's range write zeros). The value rows go the same way
// into V blocks (VBLK_*) that the state wavefronts read: lane l of a K1
// wavefront with w & 3 = b loads granule (l & 15) ^ (2r + 8(b & 1)) of row
// 4b + r, r = l >> 4, into block b.
constexpr int FSTG_NB = STG_G;      // q, k [16][256 B] each
constexpr int GRING_BYTES = 8192;   // g [16][512 B]

struct RowChunkF {
    u32x4 qk;  // as RowChunk
    float b;
};

// Global byte offset (from the chunk's first v row) of lane `lane`'s
// direct-to-LDS v granule in a K1 wavefront that loads block b.
__device__ __forceinline__ uint32_t v_dma_off(int H, int b, int lane) {
    const int r = lane >> 4;
    const int gi = (lane & 15) ^ (2 * r + 8 * (b & 1));
    return (uint32_t)(4 * b + r) * (uint32_t)H * (D * 2) + gi * 16;
}

// Block b of the V block of chunk ci into vblk, by one direct-to-LDS load.
__device__ __forceinline__ void k1_load_v_dma(const RowStreams& rs, int ci, int nrows, uint32_t v_off, int b,
                                              uint8_t* vblk) {
    const size_t c_act = (size_t)ci * (CH * (size_t)rs.st_act);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(chunk_rsrc(rs.v + c_act, (uint32_t)nrows * rs.st_act),
                                             (__attribute__((address_space(3))) void*)(vblk + 1024 * b), 16,
                                             (int)v_off, 0, 0, BUF_POLICY);
    __builtin_amdgcn_sched_barrier(0);
}

// Global byte offset (from the chunk's first g row) of lane `lane`'s
// direct-to-LDS g granule in wavefront w.
__device__ __forceinline__ uint32_t g_dma_off(int H, int wave, int lane) {
    const int r = 2 * wave + (lane >> 5), sl = lane & 31;
    const int c = (sl & 16) | ((sl ^ r) & 15);
    return (uint32_t)r * (uint32_t)H * (D * 4) + c * 16;
}

// The g rows of chunk ci into their LDS slot. Issued before the chunk's
// register loads (k1_load_rows_f), so that the compiler's wait for those
// also covers it (loads complete in order).
__device__ __forceinline__ void k1_load_g_dma(const RowStreams& rs, int ci, int nrows, uint32_t g_off, int wave,
                                              uint8_t* gslot) {
    const size_t c_act = (size_t)ci * (CH * (size_t)rs.st_act);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        chunk_rsrc(rs.g + 2 * c_act, (uint32_t)nrows * rs.st_g),
        (__attribute__((address_space(3))) void*)(gslot + 2 * wave * (D * 4)), 16, (int)g_off, 0, 0, BUF_POLICY);
    __builtin_amdgcn_sched_barrier(0);
}

// The q or k and beta rows of chunk ci into a register set.
template <bool GVA>
__device__ __forceinline__ void k1_load_rows_f(const RowStreams& rs, int ci, int nrows, int nrows_q,
                                               const RowLaneOffsets& lo, RowChunkF& rc, int wave) {
    const size_t c_act = (size_t)ci * (CH * (size_t)rs.st_act);
    size_t c_qk = c_act;
    uint32_t st_qk = rs.st_act;
    if constexpr (GVA) {
        c_qk = (size_t)ci * (CH * (size_t)rs.st_qk);
        st_qk = rs.st_qk;
    }
    const bool is_q = wave < 4;
    const uint8_t* qkb = (is_q ? rs.q : rs.k) + c_qk;
    const uint32_t n_qk = (uint32_t)(is_q ? nrows_q : nrows) * st_qk;
    rc.qk = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(chunk_rsrc(qkb, n_qk), (int)lo.qk, 0,
                                                                           BUF_POLICY));
    rc.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
        chunk_rsrc(rs.b + (c_act >> 6), (uint32_t)nrows * rs.st_b), (int)lo.beta, 0, BUF_POLICY));
}

__device__ __forceinline__ void k1_stage_f(const RowChunkF& rc, int wave, int lane, const RowLaneOffsets& lo,
                                           uint8_t* stg, float* stg_b) {
    *(u32x4*)(stg + lo.st_qk) = rc.qk;
    if (wave == 0 && lane < 16) stg_b[lane] = rc.b;
}

__device__ __forceinline__ void k1_read_staged_f(const uint8_t* stg, const float* stg_b, const uint8_t* gslot,
                                                 int lane, const RowLaneOffsets& lo, RawChunk& raw) {
    raw.q = *(const u32x2*)(stg + STG_Q + lo.rd_act);
    raw.k = *(const u32x2*)(stg + STG_K + lo.rd_act);
    raw.g = *(const f32x4*)(gslot + lo.rd_g);
    raw.b = stg_b[lane & 15];
}

// Largest |G| (log2 units) for which phase 1 factors the decays about the
// chunk start: exp(G) and exp(-G) are then normal fp32 and bf16 values, and
// the unmasked Gram terms exp(G_r - G_i) (i <= r) are at most 1.
constexpr float G_FACTOR0_MAX = 100.0f;
// Largest |G - G_7| (log2 units) the row-7 factors exp(G - G_7), exp(G_7 - G)
// take as normal fp32 values.
constexpr float G_SPAN_MAX = 126.0f;
// Floor on one token's log2-decay for the rare chunk whose in-chunk decay
// exceeds even the row-7 range (a token decaying beyond about e^-87, or g =
// -inf): with it, no token's decay exceeds 2^-15.5 (about e^-10.7), and 8
// tokens span at most 124. The flooring changes a carried-in state's
// contribution by at most that factor, against the exact decay of such a
// token, which is smaller still.
constexpr float G_TOKEN_FLOOR = 15.5f;

// scr_b: the chunk's 16 betas (scr + K1_BETA where the layout keeps them
// together)
template <bool KT_TR>
__device__ __forceinline__ void k1_phase1(const RawChunk& raw, int wave, int lane, uint8_t* rec,
                                          uint8_t* scr, float* scr_b) {
    const int gg = lane >> 4, m = lane & 15;
    // in-chunk cumulative log2-decay per channel: inclusive scan over the tokens
    float G[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x = raw.g[j] * LOG2E;
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
        G[j] = x;
    }
    const float qf[4] = {bf16_lo(raw.q.x), bf16_hi(raw.q.x), bf16_lo(raw.q.y), bf16_hi(raw.q.y)};
    const float kf[4] = {bf16_lo(raw.k.x), bf16_hi(raw.k.x), bf16_lo(raw.k.y), bf16_hi(raw.k.y)};
    // The Grams need k_r k_i exp(G_r - G_i) (and q_r k_i ...) as a product of
    // a row factor and a column factor. Factored about the chunk start, the
    // row factors are the chain's own operands X = k exp(G) and
    // Qt = q exp(G), and the column factor is k exp(-G): two exponentials
    // and four products per element. That needs |G| within G_FACTOR0_MAX
    // over the wavefront's channels; otherwise (decay beyond about e^-69
    // inside one chunk) the wavefront factors about row 7 instead, which
    // only needs |G - G_7| within the fp32 exponent range. The choice is
    // uniform per wavefront and per chunk, and a function of g alone.
    const float amax = fmaxf(fmaxf(fabsf(G[0]), fabsf(G[1])), fmaxf(fabsf(G[2]), fabsf(G[3])));
    const bool about_row7 = __builtin_amdgcn_ballot_w64(!(amax <= G_FACTOR0_MAX)) != 0;
    float gam[4];  // exp(G)
    u32x2 pka, pkb, pqa, pqt, pxk, pkt;
    if (!about_row7) {
        f32x4 kb, qt, xk, kt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gam[j] = exp2_hw(G[j]);
            const float ig = exp2_hw(-G[j]);
            qt[j] = qf[j] * gam[j];
            xk[j] = kf[j] * gam[j];
            kb[j] = kf[j] * ig;
            kt[j] = kb[j] * row_newbcast<15>(gam[j]);  // k exp(G_C - G)
        }
        pqt = pack4(qt);
        pxk = pack4(xk);
        pkb = pack4(kb);
        pkt = pack4(kt);
        pka = pxk;
        pqa = pqt;
    } else {
        // The row-7 factors need |G - G_7| within G_SPAN_MAX; a chunk beyond
        // that (the check also catches NaN, from g = -inf) is scanned again
        // with each token's log-decay floored at -G_TOKEN_FLOOR. The choice is
        // again uniform per wavefront and chunk, and a function of g alone.
        bool wide = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) wide |= !(fabsf(G[j] - row_newbcast<7>(G[j])) <= G_SPAN_MAX);
        if (__builtin_amdgcn_ballot_w64(wide) != 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x = fmaxf(raw.g[j] * LOG2E, -G_TOKEN_FLOOR);
                x += row_shr<1>(x);
                x += row_shr<2>(x);
                x += row_shr<4>(x);
                x += row_shr<8>(x);
                G[j] = x;
            }
        }
        // E = exp(G - G_7), F = exp(G_7 - G)
        float E[4], F[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float g7 = row_newbcast<7>(G[j]);
            E[j] = exp2_hw(G[j] - g7);
            F[j] = exp2_hw(g7 - G[j]);
            gam[j] = exp2_hw(G[j]);
        }
        f32x4 ka, kb, qa, qt, xk, kt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ka[j] = kf[j] * E[j];
            kb[j] = kf[j] * F[j];
            qa[j] = qf[j] * E[j];
            qt[j] = qf[j] * gam[j];
            xk[j] = kf[j] * gam[j];
            kt[j] = kb[j] * row_newbcast<15>(E[j]);  // k exp(G_C - G)
        }
        pka = pack4(ka);
        pkb = pack4(kb);
        pqa = pack4(qa);
        pqt = pack4(qt);
        pxk = pack4(xk);
        pkt = pack4(kt);
    }
    // fragments in the REC_Q layout: half (wave & 1) of K-step (wave >> 1);
    // K1_KB in its split-half layout
    const int fo = (wave >> 1) * 1024 + lane * 16 + (wave & 1) * 8;
    *(u32x2*)(scr + K1_KA + fo) = pka;
    *(u32x2*)(scr + K1_QA + fo) = pqa;
    *(u32x2*)(scr + K1_KB + (wave >> 1) * 1024 + (wave & 1) * 512 + lane * 8) = pkb;
    *(u32x2*)(rec + REC_Q + fo) = pqt;
    *(u32x2*)(rec + REC_X + fo) = pxk;
    if constexpr (KT_TR) {
        // Kt of tile `wave`: the lane's row segment, untransposed (the state
        // wavefronts transpose it as they load it)
        *(u32x2*)(rec + REC_KT + wave * 512 + kv_store_slot(gg, m) * 8) = pkt;
    } else {
        // Kt^T: element (token m, channel 16 wave + 4gg + j) -> tile wave,
        // lane (m >> 2) * 16 + 4gg + j, element m & 3. The four lanes of a
        // quad (m = 4a .. 4a + 3) hold a 4 x 4 block of it (tokens x
        // channels); after a 16-bit transpose inside the quad, lane
        // (gg, 4a + j) holds channel 4gg + j for tokens 4a .. 4a + 3: the
        // whole 8-byte fragment of lane 16a + 4gg + j, one store to its slot.
        const int dl = 16 * (m >> 2) + 4 * gg + (m & 3);
        *(u32x2*)(rec + REC_KT + wave * 512 + kv_slot(dl) * 8) = quad_transpose16(pkt, lane);
    }
    // exp(G_C): the last row holds the chunk total (rows past nrows add 0)
    if (m == 15) *(f32x4*)(rec + REC_GC + (32 * gg + 4 * wave) * 4) = f32x4{gam[0], gam[1], gam[2], gam[3]};
    if (wave == 0 && gg == 0) scr_b[m] = raw.b;
}

// ---------------------------------------------------------------------------
// K1, phase 2 (after a barrier that publishes phase 1). L =
// strict-lower(diag(beta) A_kk) and the masked A_qk are Grams over all 128
// channels on MFMA from the phase-1 fragments; rows of T' = (I + L)^-1
// diag(beta) follow by a substitution over 15 dependent steps, each one
// DPP-broadcast multiply-subtract. In the materialised K1 kernel, wavefront
// s < 4 forms its own copy of L in a private 1 KiB and rows 4s + gg of T'
// (so phase 2 needs no barrier of its own), and wavefront WAVE_QK forms
// A_qk. The fused kernel forms L once, a stage earlier (k1_lkk), and runs
// only the substitution on the T' wavefronts (k1_tsolve).
// ---------------------------------------------------------------------------
// The Gram operands of K-step p for lane `lane`: the column factor from its
// split-half layout, and a row factor (K1_KA or K1_QA).
__device__ __forceinline__ u32x4 gram_kb(const uint8_t* scr, int p, int lane) {
    const u32x2 lo = *(const u32x2*)(scr + K1_KB + p * 1024 + lane * 8);
    const u32x2 hi = *(const u32x2*)(scr + K1_KB + p * 1024 + 512 + lane * 8);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}
__device__ __forceinline__ u32x4 gram_row(const uint8_t* scr, int off, int p, int lane) {
    return *(const u32x4*)(scr + off + p * 1024 + lane * 16);
}

// L = strict-lower(diag(beta) A_kk) from A_kk (lane: A_kk[4gg + v][m]),
// stored transposed (lt[c * K1_LSTRIDE + r] = L[r][c]), so that lane (gg, i)
// of a reader finds column i of L in row i of lt. With lbeta, the chunk's
// beta is copied beside it.
__device__ __forceinline__ void k1_store_l(int lane, const f32x4& a, const float* scr_b, float* lt, float* lbeta) {
    const int gg = lane >> 4, m = lane & 15;
    const f32x4 br = *(const f32x4*)(scr_b + 4 * gg);
    f32x4 l;
#pragma unroll
    for (int v = 0; v < 4; ++v) l[v] = (m < 4 * gg + v) ? br[v] * a[v] : 0.f;
    *(f32x4*)(lt + m * K1_LSTRIDE + 4 * gg) = l;
    if (lbeta && gg == 0) lbeta[m] = scr_b[m];
}

// L from the phase-1 Gram factors (see k1_store_l): A_kk = KA KB^T over the
// 128 channels, lane holding A_kk[4gg + v][m].
__device__ __forceinline__ void k1_lkk(int lane, const uint8_t* scr, const float* scr_b, float* lt, float* lbeta) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) a = mfma_k32(gram_row(scr, K1_KA, p, lane), gram_kb(scr, p, lane), a);
    k1_store_l(lane, a, scr_b, lt, lbeta);
}

// Rows 4 s4 .. 4 s4 + 3 of T' = (I + L)^-1 diag(beta) from L^T (as k1_lkk
// stores it) and beta, to the record.
__device__ __forceinline__ void k1_tsolve(int lane, int s4, uint8_t* rec, const float* lt, const float* beta) {
    const int gg = lane >> 4, m = lane & 15;
    float lc[16];  // lc[K] = L[K][m]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x4 c = *(const f32x4*)(lt + m * K1_LSTRIDE + 4 * q);
#pragma unroll
        for (int v = 0; v < 4; ++v) lc[4 * q + v] = c[v];
    }
    // Rows of T = (I + L)^-1 are independent: T[r][c] = [r = c] -
    // sum_{K > c} T[r][K] L[K][c]. Row r = 4 s4 + gg lives in 16-lane row gg,
    // column i in lane i; for K = 15..1, T[r][K] is final and is broadcast
    // along the row to update the columns c < K (L[K][c] = 0 for c >= K).
    float t = (4 * s4 + gg == m) ? 1.f : 0.f;
    auto step = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        t -= lc[K] * row_newbcast<K>(t);
    };
    step(std::integral_constant<int, 15>{}); step(std::integral_constant<int, 14>{});
    step(std::integral_constant<int, 13>{}); step(std::integral_constant<int, 12>{});
    step(std::integral_constant<int, 11>{}); step(std::integral_constant<int, 10>{});
    step(std::integral_constant<int, 9>{});  step(std::integral_constant<int, 8>{});
    step(std::integral_constant<int, 7>{});  step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 5>{});  step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 3>{});  step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 1>{});
    // T'[r][i] = T[r][i] beta_i, split into bf16 hi + lo, to the A-fragment
    // layout T'[m'][4gg' + j] at lane (gg', m') = (i >> 2, r), j = i & 3
    const float tb = t * beta[m];
    const uint32_t th = pack_bf16(tb, tb);
    const uint32_t tl = pack_bf16(tb - bf16_lo(th), tb - bf16_lo(th));
    uint8_t* td = rec + REC_T + ((16 * (m >> 2) + 4 * s4 + gg) * 4 + (m & 3)) * 2;
    *(uint16_t*)(td + 0) = (uint16_t)th;
    *(uint16_t*)(td + 512) = (uint16_t)tl;
}

// Both halves on one wavefront, through its private lw (1 KiB).
__device__ __forceinline__ void k1_phase2_t(int lane, int s4, uint8_t* rec, const uint8_t* scr, float* lw) {
    k1_lkk(lane, scr, (const float*)(scr + K1_BETA), lw, nullptr);
    k1_tsolve(lane, s4, rec, lw, (const float*)(scr + K1_BETA));
}

// A_qk^T = (k exp(G_ref - G)) (q exp(G - G_ref))^T, masked (i <= r), to the
// record: lane holds A_qk[m][4gg + v]. kb: the column-factor fragments.
__device__ __forceinline__ void k1_aqk(int lane, uint8_t* rec, const uint8_t* scr, const u32x4 (&kb)[4]) {
    const int gg = lane >> 4, m = lane & 15;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) a = mfma_k32(kb[p], gram_row(scr, K1_QA, p, lane), a);
#pragma unroll
    for (int v = 0; v < 4; ++v) a[v] = (4 * gg + v <= m) ? a[v] : 0.f;
    *(u32x2*)(rec + REC_AQK + lane * 8) = pack4(a);
}

__device__ __forceinline__ void k1_phase2_qk(int lane, uint8_t* rec, const uint8_t* scr) {
    u32x4 kb[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) kb[p] = gram_kb(scr, p, lane);
    k1_aqk(lane, rec, scr, kb);
}

// Both Grams of a chunk on one wavefront (the fused kernel's WAVE_QK): A_qk
// to the record and L to the shared lt (with beta at lbeta), reading the
// column factor once.
__device__ __forceinline__ void k1_grams(int lane, uint8_t* rec, const uint8_t* scr, const float* scr_b, float* lt,
                                         float* lbeta) {
    u32x4 kb[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) kb[p] = gram_kb(scr, p, lane);
    k1_aqk(lane, rec, scr, kb);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) a = mfma_k32(gram_row(scr, K1_KA, p, lane), kb[p], a);
    k1_store_l(lane, a, scr_b, lt, lbeta);
}

// Phase 2 by role; other wavefronts have nothing to do in it. lw is the
// N_WAVE_T * K1_LBYTES of LDS that the T' wavefronts use privately.
__device__ __forceinline__ void k1_phase2(int wave, int lane, uint8_t* rec, const uint8_t* scr, float* lw) {
    if (wave < N_WAVE_T) k1_phase2_t(lane, wave, rec, scr, lw + wave * (K1_LBYTES / 4));
    else if (wave == WAVE_QK) k1_phase2_qk(lane, rec, scr);
}

// ---------------------------------------------------------------------------
// K2 chain step: one wavefront advances NT value-column tiles n0..n0+NT-1 of
// the state (16 columns each) over one chunk record held in LDS, with the
// chunk's V block vb (VBLK_* layout; unused without V).
// State tile S[t][n] holds S[16t + 4gg + v][16(n0 + n) + m], v = 0..3.
// WITH_V = false runs the same update with V := 0 (the segment transfer of
// the CP pre_scan). WITH_OUT also forms O^T = S0^T Qt^T + U^T A_qk^T, whose
// accumulator oacc[n][v] is o[token m][16(n0 + n) + 4gg + v].
// The arithmetic of a tile is identical in every instantiation.
// ---------------------------------------------------------------------------
template <int NT, bool WITH_V, bool WITH_OUT, bool KT_TR>
__device__ __forceinline__ void chain_step(const uint8_t* rec, const uint8_t* vb, f32x4 (&S)[8][NT], int n0,
                                           int lane, f32x4 (&oacc)[NT]) {
    const int gg = lane >> 4;
    // bf16 copy of the chunk-start state, as K=32 operands
    u32x4 Sb[4][NT];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            Sb[p][n].x = pack_bf16(S[2 * p][n][0], S[2 * p][n][1]);
            Sb[p][n].y = pack_bf16(S[2 * p][n][2], S[2 * p][n][3]);
            Sb[p][n].z = pack_bf16(S[2 * p + 1][n][0], S[2 * p + 1][n][1]);
            Sb[p][n].w = pack_bf16(S[2 * p + 1][n][2], S[2 * p + 1][n][3]);
        }
    // P = X S0
    f32x4 P[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) P[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4 xf = *(const u32x4*)(rec + REC_X + p * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < NT; ++n) P[n] = mfma_k32(xf, Sb[p][n], P[n]);
    }
    // U = T' (V - P): hi and lo halves of T'
    const u32x2 th = *(const u32x2*)(rec + REC_T + lane * 8);
    const u32x2 tl = *(const u32x2*)(rec + REC_T + 512 + lane * 8);
    u32x2 Ub[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        f32x4 r;
        if constexpr (WITH_V) {
            const u32x2 vw = lds_load_tr16(vb + vblk_load_off(lane, n0 + n));
            r[0] = bf16_lo(vw.x) - P[n][0];
            r[1] = bf16_hi(vw.x) - P[n][1];
            r[2] = bf16_lo(vw.y) - P[n][2];
            r[3] = bf16_hi(vw.y) - P[n][3];
        } else {
            r = -P[n];
        }
        const u32x2 rb = pack4(r);
        f32x4 u = mfma_k16(th, rb, f32x4{0.f, 0.f, 0.f, 0.f});
        u = mfma_k16(tl, rb, u);
        Ub[n] = pack4(u);
    }
    // O^T = S0^T Qt^T + U^T A_qk^T
    if constexpr (WITH_OUT) {
        const u32x2 aq = *(const u32x2*)(rec + REC_AQK + lane * 8);
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 qf = *(const u32x4*)(rec + REC_Q + p * 1024 + lane * 16);
#pragma unroll
            for (int n = 0; n < NT; ++n) oacc[n] = mfma_k32(Sb[p][n], qf, oacc[n]);
        }
        // A_qk U goes to a fresh 16x16x16 accumulator and is added with VALU.
        // Chaining it onto oacc (a 16x16x32 accumulator handed straight to the
        // 16x16x16 shape as its C operand) was seen to lose the last 16x16x32
        // contribution in two of the four output rows.
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[n] += mfma_k16(Ub[n], aq, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // S_next = Diag(exp G_C) S0 + Kt^T U. Lane (gg, m) holds exp(G_C) of
    // channels 16(m >> 1) + 4gg + 2(m & 1) + 0..1; row 4gg + v of tile t
    // takes it from lane 2t + (v >> 1) of its 16-lane row (a DPP broadcast
    // folded into the multiply), so the wavefront reads 512 bytes instead
    // of 32 values per lane.
    const f32x2 gcp = *(const f32x2*)(rec + REC_GC + lane * 8);
    auto decay = [&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        const f32x4 gcv = {row_newbcast<2 * t>(gcp[0]), row_newbcast<2 * t>(gcp[1]),
                           row_newbcast<2 * t + 1>(gcp[0]), row_newbcast<2 * t + 1>(gcp[1])};
        const u32x2 kt = kt_frag<KT_TR>(rec, t, lane);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            S[t][n] = gcv * S[t][n];
            S[t][n] = mfma_k16(kt, Ub[n], S[t][n]);
        }
    };
    decay(std::integral_constant<int, 0>{}); decay(std::integral_constant<int, 1>{});
    decay(std::integral_constant<int, 2>{}); decay(std::integral_constant<int, 3>{});
    decay(std::integral_constant<int, 4>{}); decay(std::integral_constant<int, 5>{});
    decay(std::integral_constant<int, 6>{}); decay(std::integral_constant<int, 7>{});
}

// The warm-up step of a warm-start segment: the transfer M (V := 0) and the
// state from zero Z (with V from the V block vb) over the same record,
// each tile's arithmetic exactly that of chain_step<1, false, false> and
// chain_step<1, true, false>. The record's operands are read once for both,
// and each bf16 operand of a state is packed just before its one use (no
// output is formed), so the two states fit the registers beside the step.
template <bool KT_TR>
__device__ __forceinline__ void chain_step_warm(const uint8_t* rec, const uint8_t* vb, f32x4 (&M)[8][1],
                                                f32x4 (&Z)[8][1], int n0, int lane) {
    f32x4 pm = {0.f, 0.f, 0.f, 0.f}, pz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4 xf = *(const u32x4*)(rec + REC_X + p * 1024 + lane * 16);
        u32x4 sm, sz;
        sm.x = pack_bf16(M[2 * p][0][0], M[2 * p][0][1]);
        sm.y = pack_bf16(M[2 * p][0][2], M[2 * p][0][3]);
        sm.z = pack_bf16(M[2 * p + 1][0][0], M[2 * p + 1][0][1]);
        sm.w = pack_bf16(M[2 * p + 1][0][2], M[2 * p + 1][0][3]);
        sz.x = pack_bf16(Z[2 * p][0][0], Z[2 * p][0][1]);
        sz.y = pack_bf16(Z[2 * p][0][2], Z[2 * p][0][3]);
        sz.z = pack_bf16(Z[2 * p + 1][0][0], Z[2 * p + 1][0][1]);
        sz.w = pack_bf16(Z[2 * p + 1][0][2], Z[2 * p + 1][0][3]);
        pm = mfma_k32(xf, sm, pm);
        pz = mfma_k32(xf, sz, pz);
    }
    const u32x2 th = *(const u32x2*)(rec + REC_T + lane * 8);
    const u32x2 tl = *(const u32x2*)(rec + REC_T + 512 + lane * 8);
    const u32x2 vw = lds_load_tr16(vb + vblk_load_off(lane, n0));
    f32x4 rz;
    rz[0] = bf16_lo(vw.x) - pz[0];
    rz[1] = bf16_hi(vw.x) - pz[1];
    rz[2] = bf16_lo(vw.y) - pz[2];
    rz[3] = bf16_hi(vw.y) - pz[3];
    const u32x2 rbm = pack4(-pm), rbz = pack4(rz);
    f32x4 um = mfma_k16(th, rbm, f32x4{0.f, 0.f, 0.f, 0.f});
    f32x4 uz = mfma_k16(th, rbz, f32x4{0.f, 0.f, 0.f, 0.f});
    um = mfma_k16(tl, rbm, um);
    uz = mfma_k16(tl, rbz, uz);
    const u32x2 ubm = pack4(um), ubz = pack4(uz);
    const f32x2 gcp = *(const f32x2*)(rec + REC_GC + lane * 8);
    auto decay = [&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        const f32x4 gcv = {row_newbcast<2 * t>(gcp[0]), row_newbcast<2 * t>(gcp[1]),
                           row_newbcast<2 * t + 1>(gcp[0]), row_newbcast<2 * t + 1>(gcp[1])};
        const u32x2 kt = kt_frag<KT_TR>(rec, t, lane);
        M[t][0] = gcv * M[t][0];
        M[t][0] = mfma_k16(kt, ubm, M[t][0]);
        Z[t][0] = gcv * Z[t][0];
        Z[t][0] = mfma_k16(kt, ubz, Z[t][0]);
    };
    decay(std::integral_constant<int, 0>{}); decay(std::integral_constant<int, 1>{});
    decay(std::integral_constant<int, 2>{}); decay(std::integral_constant<int, 3>{});
    decay(std::integral_constant<int, 4>{}); decay(std::integral_constant<int, 5>{});
    decay(std::integral_constant<int, 6>{}); decay(std::integral_constant<int, 7>{});
}

}  // namespace kda
