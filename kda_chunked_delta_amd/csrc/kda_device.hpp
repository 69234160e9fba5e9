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
//   L  = strict-lower(diag(beta) A_kk)
//   W  = (I + L)^-1 diag(beta) (k * exp G),   U~ = (I + L)^-1 diag(beta) v
//   Qt = q * exp G,   Kt = k * exp(G_C - G)
//   U  = U~ - W S0;   O = Qt S0 + A_qk U;   S_next = Diag(exp G_C) S0 + Kt^T U
// All matrix products run on bf16 MFMA with fp32 accumulation; the state
// and the decays stay fp32, and the WY inverse is formed in fp32 and applied
// as a hi/lo pair of bf16 MFMA operands.
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
//   REC_W  : W fragments, same layout as REC_Q
//   REC_KT : Kt^T fragments [t 8][lane 64][4 bf16]: Kt[4gg + j][16t + m]
//   REC_U  : U~ in accumulator layout [n 8][lane 64][4 bf16]: U~[4gg + j][16n + m]
//   REC_AQK: A_qk^T fragment [lane 64][4 bf16]: A_qk[m][4gg + j] (masked i <= r)
//   REC_GC : exp(G_C) [128] fp32
// The same bytes are used in LDS and, when K1 is materialised, in HBM.
// ---------------------------------------------------------------------------
constexpr int REC_Q = 0;
constexpr int REC_W = 4096;
constexpr int REC_KT = 8192;
constexpr int REC_U = 12288;
constexpr int REC_AQK = 16384;
constexpr int REC_GC = 16896;
constexpr int REC_BYTES = 17408;
constexpr int REC_VEC = REC_BYTES / 16;  // 1088 16-byte vectors

// K1 scratch of one chunk (LDS only), shared between its two phases:
//   K1_XCT : X = beta k exp(G) (bf16) in Kt^T fragment layout: X[4gg + j][16t + m]
//   K1_YCT : Y = beta v (bf16), same layout
//   K1_GP  : partial Grams fp32 [wavefront 8][A_kk, A_qk][lane 64][4] over its 16 channels
//   K1_BETA: beta of the chunk's 16 rows, fp32
constexpr int K1_XCT = 0;
constexpr int K1_YCT = 4096;
constexpr int K1_GP = 8192;
constexpr int K1_BETA = 8192 + 16384;
constexpr int K1_BYTES = K1_BETA + 64;
constexpr int K1_LBYTES = 1024;  // per phase-2 wavefront: L as fp32 [16][16]

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
// fp32 -> bf16 bits in the low half.
__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16(x, x) & 0xffffu; }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{pack_bf16(a, b), pack_bf16(c, d)};
}

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

// x from lane (m - n) of the same 16-lane row, 0 for m < n (DPP row shift).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x110 + N, 0xF, 0xF, false);
}
// x from lane I of the same 16-lane row (swizzle broadcast).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (I << 5)));
}
// x from the same lane index m of 16-lane row R, in every row (two permlane swaps).
template <int R>
__device__ __forceinline__ float rows_from(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t pr = (R & 1) ? s16[1] : s16[0];  // rows (R & 2), (R & 2) + 1 now hold row R
    const auto s32 = __builtin_amdgcn_permlane32_swap(pr, pr, false, false);
    return __uint_as_float((R & 2) ? s32[1] : s32[0]);
}

// ---------------------------------------------------------------------------
// K1, phase 1 (8 wavefronts). Wavefront p (0..7) owns key channels 16p..16p+15
// and value columns 16p..16p+15; lane (gg, m) holds token m of the chunk and
// channels 16p + 4gg + j, j = 0..3. Rows past nrows are zero (k = q = v = 0,
// g = 0, beta = 0), which leaves them inert.
// ---------------------------------------------------------------------------
struct RawChunk {
    u32x2 q, k, v;
    f32x4 g;
    float b;
};

__device__ __forceinline__ void k1_load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                        const uint16_t* __restrict__ v, const float* __restrict__ g,
                                        const float* __restrict__ beta, int H, int h, int64_t tok0,
                                        int nrows, int wave, int lane, RawChunk& raw) {
    const int gg = lane >> 4, m = lane & 15;
    raw.q = u32x2{0u, 0u};
    raw.k = raw.q;
    raw.v = raw.q;
    raw.g = f32x4{0.f, 0.f, 0.f, 0.f};
    raw.b = 0.f;
    if (m < nrows) {
        const size_t row = (size_t)(tok0 + m) * H + h;
        const size_t off = row * D + 16 * wave + 4 * gg;
        raw.q = __builtin_nontemporal_load((const u32x2*)(q + off));
        raw.k = __builtin_nontemporal_load((const u32x2*)(k + off));
        raw.v = __builtin_nontemporal_load((const u32x2*)(v + off));
        raw.g = __builtin_nontemporal_load((const f32x4*)(g + off));
        raw.b = beta[row];
    }
}

__device__ __forceinline__ void k1_phase1(const RawChunk& raw, int wave, int lane, uint8_t* rec,
                                          uint8_t* ws) {
    const int gg = lane >> 4, m = lane & 15;
    // in-chunk cumulative log-decay per channel: inclusive scan over the tokens
    float G[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x = raw.g[j];
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
        G[j] = x;
    }
    // decays relative to the reference row 7: E = exp(G - G_7), F = exp(G_7 - G)
    float E[4], F[4], c7[4], e15[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float g7 = row_bcast<7>(G[j]);
        E[j] = __expf(G[j] - g7);
        F[j] = __expf(g7 - G[j]);
        c7[j] = __expf(g7);  // exp(G_7)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) e15[j] = row_bcast<15>(E[j]);  // exp(G_C - G_7)
    const float qf[4] = {bf16_lo(raw.q.x), bf16_hi(raw.q.x), bf16_lo(raw.q.y), bf16_hi(raw.q.y)};
    const float kf[4] = {bf16_lo(raw.k.x), bf16_hi(raw.k.x), bf16_lo(raw.k.y), bf16_hi(raw.k.y)};
    const float vf[4] = {bf16_lo(raw.v.x), bf16_hi(raw.v.x), bf16_lo(raw.v.y), bf16_hi(raw.v.y)};
    float ka[4], kb[4], qa[4], qt[4], kt[4], X[4], Y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float gam = E[j] * c7[j];  // exp(G_r)
        const float kc = F[j] * e15[j];  // exp(G_C - G_r)
        ka[j] = kf[j] * E[j];
        kb[j] = kf[j] * F[j];
        qa[j] = qf[j] * E[j];
        qt[j] = qf[j] * gam;
        kt[j] = kf[j] * kc;
        X[j] = raw.b * (kf[j] * gam);
        Y[j] = raw.b * vf[j];
    }
    // partial Grams over this wavefront's 16 channels (A: token m, B: token m)
    const u32x2 fa = pack4(ka[0], ka[1], ka[2], ka[3]);
    const u32x2 fb = pack4(kb[0], kb[1], kb[2], kb[3]);
    const u32x2 fq = pack4(qa[0], qa[1], qa[2], qa[3]);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 pkk = mfma_k16(fa, fb, zero);
    const f32x4 pqk = mfma_k16(fq, fb, zero);
    *(f32x4*)(ws + K1_GP + ((wave * 2 + 0) * 64 + lane) * 16) = pkk;
    *(f32x4*)(ws + K1_GP + ((wave * 2 + 1) * 64 + lane) * 16) = pqk;
    // Qt: half (wave & 1) of K-step (wave >> 1)
    *(u32x2*)(rec + REC_Q + (wave >> 1) * 1024 + lane * 16 + (wave & 1) * 8) = pack4(qt[0], qt[1], qt[2], qt[3]);
    // Kt^T, X, Y: element (token m, channel 16 wave + 4gg + j) -> tile wave,
    // lane (m >> 2) * 16 + 4gg + j, slot m & 3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int o = wave * 512 + ((m >> 2) * 16 + 4 * gg + j) * 8 + (m & 3) * 2;
        *(uint16_t*)(rec + REC_KT + o) = (uint16_t)bf16_bits(kt[j]);
        *(uint16_t*)(ws + K1_XCT + o) = (uint16_t)bf16_bits(X[j]);
        *(uint16_t*)(ws + K1_YCT + o) = (uint16_t)bf16_bits(Y[j]);
    }
    if (m == 0)
        *(f32x4*)(rec + REC_GC + (16 * wave + 4 * gg) * 4) =
            f32x4{c7[0] * e15[0], c7[1] * e15[1], c7[2] * e15[2], c7[3] * e15[3]};
    if (wave == 0 && gg == 0) *(float*)(ws + K1_BETA + 4 * m) = raw.b;
}

// ---------------------------------------------------------------------------
// K1, phase 2 (4 wavefronts, after a barrier that publishes phase 1): the
// Grams, L = strict-lower(diag(beta) A_kk), the WY inverse T = (I + L)^-1
// and the WY-transformed keys and values of tiles 2w, 2w+1. Each wavefront
// forms T itself (no further barrier); lw is its private 1 KiB of LDS.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void k1_phase2(int w, int lane, uint8_t* rec, const uint8_t* ws, float* lw) {
    const int gg = lane >> 4, m = lane & 15;
    f32x4 akk = *(const f32x4*)(ws + K1_GP + (0 * 64 + lane) * 16);
    f32x4 aqk = *(const f32x4*)(ws + K1_GP + (1 * 64 + lane) * 16);
#pragma unroll
    for (int p = 1; p < 8; ++p) {
        akk += *(const f32x4*)(ws + K1_GP + ((p * 2 + 0) * 64 + lane) * 16);
        aqk += *(const f32x4*)(ws + K1_GP + ((p * 2 + 1) * 64 + lane) * 16);
    }
    // lane holds rows r = 4gg + v, column m
    const f32x4 b4 = *(const f32x4*)(ws + K1_BETA + 16 * gg);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 4 * gg + v;
        const float lv = b4[v] * akk[v];
        lw[r * 16 + m] = (m < r) ? lv : 0.f;
    }
    if (w == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 4 * gg + v;
            const float val = (m <= r) ? aqk[v] : 0.f;
            *(uint16_t*)(rec + REC_AQK + ((m >> 2) * 16 + r) * 8 + (m & 3) * 2) = (uint16_t)bf16_bits(val);
        }
    }
    // T^T = (I + L^T)^-1 by back substitution; lane holds T^T[4gg + v][m].
    // Row k is final once rows k+1..15 are applied; L[k][i] = 0 for i >= k.
    float tt[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) tt[v] = (4 * gg + v == m) ? 1.f : 0.f;
    auto step = [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        const f32x4 lk = *(const f32x4*)(lw + K * 16 + 4 * gg);  // L[K][4gg .. 4gg+3]
        const float rowk = rows_from<(K >> 2)>(tt[K & 3]);         // T^T[K][m]
#pragma unroll
        for (int v = 0; v < 4; ++v) tt[v] = __builtin_fmaf(-lk[v], rowk, tt[v]);
    };
    step(std::integral_constant<int, 15>{}); step(std::integral_constant<int, 14>{});
    step(std::integral_constant<int, 13>{}); step(std::integral_constant<int, 12>{});
    step(std::integral_constant<int, 11>{}); step(std::integral_constant<int, 10>{});
    step(std::integral_constant<int, 9>{});  step(std::integral_constant<int, 8>{});
    step(std::integral_constant<int, 7>{});  step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 5>{});  step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 3>{});  step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 1>{});
    // hi/lo bf16 split of T^T: B operand of W^T = X^T T^T and A operand of U~ = T Y
    const u32x2 th = pack4(tt[0], tt[1], tt[2], tt[3]);
    const u32x2 tl = pack4(tt[0] - bf16_lo(th.x), tt[1] - bf16_hi(th.x), tt[2] - bf16_lo(th.y),
                           tt[3] - bf16_hi(th.y));
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
        const int n = 2 * w + nn;
        // W^T tile n: lane (gg, m) gets W[m][16n + 4gg + v]
        const u32x2 xf = *(const u32x2*)(ws + K1_XCT + n * 512 + lane * 8);
        f32x4 wt = mfma_k16(xf, th, zero);
        wt = mfma_k16(xf, tl, wt);
        *(u32x2*)(rec + REC_W + (n >> 1) * 1024 + lane * 16 + (n & 1) * 8) = pack4(wt[0], wt[1], wt[2], wt[3]);
        // U~ tile n: lane (gg, m) gets U~[4gg + v][16n + m]
        const u32x2 yf = *(const u32x2*)(ws + K1_YCT + n * 512 + lane * 8);
        f32x4 ut = mfma_k16(th, yf, zero);
        ut = mfma_k16(tl, yf, ut);
        *(u32x2*)(rec + REC_U + n * 512 + lane * 8) = pack4(ut[0], ut[1], ut[2], ut[3]);
    }
}

// ---------------------------------------------------------------------------
// K2 chain step: one wavefront advances its 128 x 32 slice of the state
// (value-column tiles wcol, wcol + 1) over one chunk record held in LDS.
// State tile S[t][n] holds S[16t + 4gg + v][16(wcol + n) + m], v = 0..3.
// WITH_U = false runs the same update with U~ := 0 (the segment transfer of
// the CP pre_scan). WITH_OUT also forms O^T = S0^T Qt^T + U^T A_qk^T, whose
// accumulator oacc[n][v] is o[token m][16(wcol + n) + 4gg + v].
// The state-update arithmetic is identical in every instantiation.
// ---------------------------------------------------------------------------
template <bool WITH_U, bool WITH_OUT>
__device__ __forceinline__ void chain_step(const uint8_t* rec, f32x4 (&S)[8][2], int wcol,
                                           int lane, f32x4 (&oacc)[2]) {
    const int gg = lane >> 4;
    // bf16 copy of the chunk-start state, as K=32 operands
    u32x4 Sb[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            Sb[p][n].x = pack_bf16(S[2 * p][n][0], S[2 * p][n][1]);
            Sb[p][n].y = pack_bf16(S[2 * p][n][2], S[2 * p][n][3]);
            Sb[p][n].z = pack_bf16(S[2 * p + 1][n][0], S[2 * p + 1][n][1]);
            Sb[p][n].w = pack_bf16(S[2 * p + 1][n][2], S[2 * p + 1][n][3]);
        }
    // W S0
    f32x4 ws[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4 wf = *(const u32x4*)(rec + REC_W + p * 1024 + lane * 16);
#pragma unroll
        for (int n = 0; n < 2; ++n) ws[n] = mfma_k32(wf, Sb[p][n], ws[n]);
    }
    // U = U~ - W S0 (fp32), bf16 operand copy
    u32x2 Ub[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        f32x4 u;
        if constexpr (WITH_U) {
            const u32x2 uw = *(const u32x2*)(rec + REC_U + (wcol + n) * 512 + lane * 8);
            u[0] = bf16_lo(uw.x) - ws[n][0];
            u[1] = bf16_hi(uw.x) - ws[n][1];
            u[2] = bf16_lo(uw.y) - ws[n][2];
            u[3] = bf16_hi(uw.y) - ws[n][3];
        } else {
            u = -ws[n];
        }
        Ub[n].x = pack_bf16(u[0], u[1]);
        Ub[n].y = pack_bf16(u[2], u[3]);
    }
    // O^T = S0^T Qt^T + U^T A_qk^T
    if constexpr (WITH_OUT) {
        const u32x2 aq = *(const u32x2*)(rec + REC_AQK + lane * 8);
#pragma unroll
        for (int n = 0; n < 2; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 qf = *(const u32x4*)(rec + REC_Q + p * 1024 + lane * 16);
#pragma unroll
            for (int n = 0; n < 2; ++n) oacc[n] = mfma_k32(Sb[p][n], qf, oacc[n]);
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) oacc[n] = mfma_k16(Ub[n], aq, oacc[n]);
    }
    // S_next = Diag(exp G_C) S0 + Kt^T U
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const f32x4 gcv = *(const f32x4*)(rec + REC_GC + (16 * t + 4 * gg) * 4);
        const u32x2 kt = *(const u32x2*)(rec + REC_KT + t * 512 + lane * 8);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            S[t][n] = gcv * S[t][n];
            S[t][n] = mfma_k16(kt, Ub[n], S[t][n]);
        }
    }
}

}  // namespace kda
