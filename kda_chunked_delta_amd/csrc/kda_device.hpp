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
// All matrix products run on bf16 MFMA with fp32 accumulation; the state,
// the decays and the WY solve stay fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int D = 128;   // head dimension (dk = dv)
constexpr int CH = 16;   // chunk length

// ---------------------------------------------------------------------------
// K1 -> K2 chunk record: everything K2 needs for one (chunk, head). Layouts
// are chosen so that K1 writes and K2's MFMA fragment reads are both free of
// heavy LDS bank conflicts (all bf16 unless noted):
//   REC_Q  : Qt[token r][channel c], row-major 256 B rows, 16-byte chunks of a
//            row XOR-swizzled by the row: byte r*256 + (((c>>3) ^ r) << 4) + 2(c&7)
//   REC_W  : W, same layout as REC_Q
//   REC_KT : Kt column-major: byte 32c + 2r holds Kt[r][c]
//   REC_U  : U~ column-major: byte 32c + 2r holds U~[r][c]
//   REC_AQK: A_qk^T fragment [lane 64][4]: A_qk[m][4gg + j] (masked i <= r)
//   REC_GC : exp(G_C) [128] fp32
// Lane l of a wavefront has group gg = l >> 4 and index m = l & 15.
// ---------------------------------------------------------------------------
constexpr int REC_Q = 0;
constexpr int REC_W = 4096;
constexpr int REC_KT = 8192;
constexpr int REC_U = 12288;
constexpr int REC_AQK = 16384;
constexpr int REC_GC = 16896;
constexpr int REC_BYTES = 17408;
constexpr int REC_VEC = REC_BYTES / 16;  // 1088 16-byte vectors

// byte offset of element (row r, channel c) in a swizzled row-major block
__host__ __device__ constexpr int swz(int r, int c) { return r * 256 + ((((c >> 3) ^ r) & 15) << 4) + 2 * (c & 7); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// ---------------------------------------------------------------------------
// K1: one chunk of one head, 256 threads, result written to an LDS record.
// ---------------------------------------------------------------------------
struct __align__(16) K1Smem {
    float G[CH][D];          // raw g, then in-chunk cumulative log-decay
    float XY[CH][2 * D];     // right-hand sides: beta*k*exp(G) | beta*v
    uint16_t qa[CH][D + 8];  // Gram operands (bf16), rows padded
    uint16_t ka[CH][D + 8];
    uint16_t kb[CH][D + 8];
    uint16_t kt[CH * D];     // Kt = k * exp(G_C - G), swizzled row-major (transposed later)
    float L[CH][CH];         // strict-lower(diag(beta) A_kk)
    float eref[D];           // exp(G_ref), G_ref = G at row 7
    float ecr[D];            // exp(G_C - G_ref)
    float gc[D];             // exp(G_C)
    float beta[CH];
};

// Workgroup barrier that waits only for this wavefront's LDS traffic, so
// global loads issued earlier (prefetch of later chunks) stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw inputs of one chunk held by K1 thread tid < 256: row r = tid >> 4,
// channels 8c..8c+7 with c = tid & 15 (16-byte loads). Rows at or beyond
// nrows are zero (k = q = v = 0, g = 0, beta = 0), which leaves them inert.
struct RawChunk {
    u32x4 q8, k8, v8;
    f32x4 ga, gb;
    float br;
};

__device__ __forceinline__ void k1_load(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                        const uint16_t* __restrict__ v, const float* __restrict__ g,
                                        const float* __restrict__ beta, int H, int h, int64_t tok0,
                                        int nrows, RawChunk& raw) {
    const int tid = threadIdx.x;
    const int r = (tid >> 4) & 15, c = tid & 15;
    raw.q8 = u32x4{0u, 0u, 0u, 0u};
    raw.k8 = raw.q8;
    raw.v8 = raw.q8;
    raw.ga = f32x4{0.f, 0.f, 0.f, 0.f};
    raw.gb = raw.ga;
    raw.br = 0.f;
    if (tid < 256 && r < nrows) {
        const size_t row = (size_t)(tok0 + r) * H + h;
        const size_t off = row * D + 8 * c;
        raw.q8 = __builtin_nontemporal_load((const u32x4*)(q + off));
        raw.k8 = __builtin_nontemporal_load((const u32x4*)(k + off));
        raw.v8 = __builtin_nontemporal_load((const u32x4*)(v + off));
        raw.ga = __builtin_nontemporal_load((const f32x4*)(g + off));
        raw.gb = __builtin_nontemporal_load((const f32x4*)(g + off + 4));
        raw.br = beta[row];
    }
}

// K1 on one chunk of one head: threads 0..255 compute, every thread of the
// workgroup (any multiple of 64 threads >= 256) must call it, since it holds
// workgroup barriers. The record is complete in `rec` (LDS) on return.
__device__ __forceinline__ void k1_compute(const RawChunk& raw, K1Smem& sm, uint8_t* rec) {
    const int tid = threadIdx.x;
    const bool act = tid < 256;
    const int r = (tid >> 4) & 15, c = tid & 15;
    if (act) {
        *(f32x4*)&sm.G[r][8 * c] = raw.ga;
        *(f32x4*)&sm.G[r][8 * c + 4] = raw.gb;
        if (c == 0) sm.beta[r] = raw.br;
    }
    lds_barrier();

    // -- in-chunk cumulative sum per key channel, per-channel decays -------
    if (tid < D) {
        float gv[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) gv[i] = sm.G[i][tid];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            acc += gv[i];
            gv[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) sm.G[i][tid] = gv[i];
        sm.eref[tid] = __expf(gv[7]);
        sm.ecr[tid] = __expf(gv[15] - gv[7]);
        sm.gc[tid] = __expf(gv[15]);
    }
    lds_barrier();

    // -- decayed operands (thread: row r, channels 8c..8c+7) ---------------
    if (act) {
        const float br = raw.br;
        const uint32_t qw[4] = {raw.q8.x, raw.q8.y, raw.q8.z, raw.q8.w};
        const uint32_t kw[4] = {raw.k8.x, raw.k8.y, raw.k8.z, raw.k8.w};
        const uint32_t vw[4] = {raw.v8.x, raw.v8.y, raw.v8.z, raw.v8.w};
        float qt[8], kt[8], qa[8], ka[8], kb[8], X[8], Y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * c + e;
            const float qf = (e & 1) ? bf16_hi(qw[e >> 1]) : bf16_lo(qw[e >> 1]);
            const float kf = (e & 1) ? bf16_hi(kw[e >> 1]) : bf16_lo(kw[e >> 1]);
            const float vf = (e & 1) ? bf16_hi(vw[e >> 1]) : bf16_lo(vw[e >> 1]);
            const float Gd = sm.G[r][d], Gref = sm.G[7][d];
            const float E = __expf(Gd - Gref);    // exp(G_r - G_ref)
            const float F = __expf(Gref - Gd);    // exp(G_ref - G_r)
            const float gam = E * sm.eref[d];     // exp(G_r)
            const float kc = F * sm.ecr[d];       // exp(G_C - G_r)
            qa[e] = qf * E;
            ka[e] = kf * E;
            kb[e] = kf * F;
            qt[e] = qf * gam;
            kt[e] = kf * kc;
            X[e] = br * (kf * gam);
            Y[e] = br * vf;
        }
        u32x4 wqa, wka, wkb;
        wqa.x = pack_bf16(qa[0], qa[1]); wqa.y = pack_bf16(qa[2], qa[3]);
        wqa.z = pack_bf16(qa[4], qa[5]); wqa.w = pack_bf16(qa[6], qa[7]);
        wka.x = pack_bf16(ka[0], ka[1]); wka.y = pack_bf16(ka[2], ka[3]);
        wka.z = pack_bf16(ka[4], ka[5]); wka.w = pack_bf16(ka[6], ka[7]);
        wkb.x = pack_bf16(kb[0], kb[1]); wkb.y = pack_bf16(kb[2], kb[3]);
        wkb.z = pack_bf16(kb[4], kb[5]); wkb.w = pack_bf16(kb[6], kb[7]);
        *(u32x4*)&sm.qa[r][8 * c] = wqa;
        *(u32x4*)&sm.ka[r][8 * c] = wka;
        *(u32x4*)&sm.kb[r][8 * c] = wkb;
        *(f32x4*)&sm.XY[r][8 * c] = f32x4{X[0], X[1], X[2], X[3]};
        *(f32x4*)&sm.XY[r][8 * c + 4] = f32x4{X[4], X[5], X[6], X[7]};
        *(f32x4*)&sm.XY[r][D + 8 * c] = f32x4{Y[0], Y[1], Y[2], Y[3]};
        *(f32x4*)&sm.XY[r][D + 8 * c + 4] = f32x4{Y[4], Y[5], Y[6], Y[7]};
        u32x4 wqt, wkt;
        wqt.x = pack_bf16(qt[0], qt[1]); wqt.y = pack_bf16(qt[2], qt[3]);
        wqt.z = pack_bf16(qt[4], qt[5]); wqt.w = pack_bf16(qt[6], qt[7]);
        wkt.x = pack_bf16(kt[0], kt[1]); wkt.y = pack_bf16(kt[2], kt[3]);
        wkt.z = pack_bf16(kt[4], kt[5]); wkt.w = pack_bf16(kt[6], kt[7]);
        *(u32x4*)(rec + REC_Q + swz(r, 8 * c)) = wqt;
        *(u32x4*)((uint8_t*)sm.kt + swz(r, 8 * c)) = wkt;
        if (r == 0) {
            *(f32x4*)(rec + REC_GC + 32 * c) = *(const f32x4*)&sm.gc[8 * c];
            *(f32x4*)(rec + REC_GC + 32 * c + 16) = *(const f32x4*)&sm.gc[8 * c + 4];
        }
    }
    lds_barrier();

    // -- Grams on MFMA: wave 0 A_kk -> L, wave 1 A_qk -> record ------------
    {
        const int wave = tid >> 6, lane = tid & 63, gg = lane >> 4, m = lane & 15;
        if (wave < 2) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const u32x4 a = wave == 0 ? *(const u32x4*)&sm.ka[m][32 * p + 8 * gg]
                                          : *(const u32x4*)&sm.qa[m][32 * p + 8 * gg];
                const u32x4 b = *(const u32x4*)&sm.kb[m][32 * p + 8 * gg];
                acc = mfma_k32(a, b, acc);
            }
            // acc[vv] = Gram[row 4gg + vv][col m]
            if (wave == 0) {
                const f32x4 b4 = *(const f32x4*)&sm.beta[4 * gg];
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int rr = 4 * gg + vv;
                    const float lv = b4[vv] * acc[vv];
                    sm.L[rr][m] = (m < rr) ? lv : 0.f;
                }
            } else {
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int rr = 4 * gg + vv;
                    const float val = (m <= rr) ? acc[vv] : 0.f;
                    *(uint16_t*)(rec + REC_AQK + ((m >> 2) * 16 + rr) * 8 + (m & 3) * 2) =
                        (uint16_t)bf16_bits(val);
                }
            }
        }
    }
    lds_barrier();

    // -- WY inverse applied by forward substitution, one column per thread --
    if (act) {
        const int col = tid;  // 0..127: column of W, 128..255: column of U~
        float x[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) x[i] = sm.XY[i][col];
        // row rr of L is read one row ahead of its use
        f32x4 lnext[4], lcur[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) lnext[q4] = *(const f32x4*)&sm.L[1][4 * q4];
#pragma unroll
        for (int rr = 1; rr < CH; ++rr) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) lcur[q4] = lnext[q4];
            if (rr + 1 < CH) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    if (4 * q4 < rr + 1) lnext[q4] = *(const f32x4*)&sm.L[rr + 1][4 * q4];
            }
            float acc = x[rr];
#pragma unroll
            for (int i = 0; i < rr; ++i) acc = __builtin_fmaf(-lcur[i >> 2][i & 3], x[i], acc);
            x[rr] = acc;
        }
        if (col < D) {
            // W row-major (swizzled), one column per thread
#pragma unroll
            for (int rr = 0; rr < CH; ++rr)
                *(uint16_t*)(rec + REC_W + swz(rr, col)) = (uint16_t)bf16_bits(x[rr]);
            // Kt: transpose column `col` of the row-major scratch into column-major
            uint32_t kw[8];
#pragma unroll
            for (int rr = 0; rr < CH; rr += 2) {
                const uint32_t lo = *(const uint16_t*)((const uint8_t*)sm.kt + swz(rr, col));
                const uint32_t hi = *(const uint16_t*)((const uint8_t*)sm.kt + swz(rr + 1, col));
                kw[rr >> 1] = lo | (hi << 16);
            }
            *(u32x4*)(rec + REC_KT + 32 * col) = u32x4{kw[0], kw[1], kw[2], kw[3]};
            *(u32x4*)(rec + REC_KT + 32 * col + 16) = u32x4{kw[4], kw[5], kw[6], kw[7]};
        } else {
            // U~ column-major, one column per thread
            const int j = col - D;
            u32x4 w0, w1;
            w0.x = pack_bf16(x[0], x[1]);   w0.y = pack_bf16(x[2], x[3]);
            w0.z = pack_bf16(x[4], x[5]);   w0.w = pack_bf16(x[6], x[7]);
            w1.x = pack_bf16(x[8], x[9]);   w1.y = pack_bf16(x[10], x[11]);
            w1.z = pack_bf16(x[12], x[13]); w1.w = pack_bf16(x[14], x[15]);
            *(u32x4*)(rec + REC_U + 32 * j) = w0;
            *(u32x4*)(rec + REC_U + 32 * j + 16) = w1;
        }
    }
    lds_barrier();
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
    const int m = lane & 15;
    // fragment of a swizzled row-major block: row m, channels dkperm(p, gg, 0..7)
    auto row_frag = [&](int base, int p) {
        const u32x2 a0 = *(const u32x2*)(rec + base + swz(m, 32 * p + 4 * gg));
        const u32x2 a1 = *(const u32x2*)(rec + base + swz(m, 32 * p + 16 + 4 * gg));
        return u32x4{a0.x, a0.y, a1.x, a1.y};
    };
    // W S0
    f32x4 ws[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4 wf = row_frag(REC_W, p);
#pragma unroll
        for (int n = 0; n < 2; ++n) ws[n] = mfma_k32(wf, Sb[p][n], ws[n]);
    }
    // U = U~ - W S0 (fp32), bf16 operand copy
    u32x2 Ub[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        f32x4 u;
        if constexpr (WITH_U) {
            const u32x2 uw = *(const u32x2*)(rec + REC_U + 32 * (16 * (wcol + n) + m) + 8 * gg);
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
            const u32x4 qf = row_frag(REC_Q, p);
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
        const u32x2 kt = *(const u32x2*)(rec + REC_KT + 32 * (16 * t + m) + 8 * gg);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            S[t][n] = gcv * S[t][n];
            S[t][n] = mfma_k16(kt, Ub[n], S[t][n]);
        }
    }
}

}  // namespace kda
