// KDA decode step on gfx950 (CDNA4): one new token per sequence, the fp32
// state advanced in place.
//
// The step is the per-token recurrence of "feat(kda/sm90): FlashKDA prefill
// port + intracard-CP prefill" (cuLA pull request #103, commit summary) for a
// single token; "feat(cake_kda): share recurrent prefill kernels across SM100
// family" (FlashInfer pull request #4313, AOT registration notes) keeps such a
// decode entry beside the prefill. With d_r = exp(g_r) per key channel r and
// value column j, the update S' = (I - beta k k^T) Diag(d) S + beta k v^T and
// the output o = scale S'^T q expand to
//   a_j = sum_r (k_r d_r) S_rj          (S^T k after the decay)
//   b_j = sum_r (q_r d_r) S_rj          (S^T q after the decay)
//   e_j = v_j - a_j
//   S'_rj = d_r S_rj + (beta k_r) e_j
//   o_j = scale (b_j + beta (q . k) e_j)
// so both column sums come out of one pass over the state, which is read once
// and written once. The step is bound by HBM bandwidth: 2 x 64 KiB of state
// per (sequence, head) against 1.3 KiB of token data.
//
// With grouped value heads, value head h reads q/k head h / group. With a
// slot table, sequence n reads and writes the state of pool slot slots[n]
// (continuous batching keeps a pool of states and a table per step).
//
//
// Launch: one workgroup of 256 threads per (sequence, head, 64-column tile),
// the two tiles of one (sequence, head) adjacent in the grid. Thread t owns
// the four columns 4 (t & 15) .. +3 of its tile and the rows (t >> 4) + 16 i,
// i = 0..7, held in registers between the two passes; one load instruction of
// a wavefront covers four whole 256-byte row segments. Every sum runs in a
// fixed order, so results are bitwise reproducible.
//
// When the batch's states are larger than half the 256 MiB last-level cache
// (MALL), the state is read and written with the nontemporal hint: it cannot
// stay cached until the next step anyway, and the hinted stream ran 10%
// faster, at the rate of a hinted plain copy of the same bytes. Smaller
// batches keep the default policy, under which back-to-back steps find their
// states in the MALL.
#include "kda_decode_launch.h"

namespace kda {
namespace {

constexpr int DEC_COLS = 64;                          // value columns per workgroup
constexpr int DEC_TILES = 128 / DEC_COLS;             // tiles per (sequence, head)
constexpr int DEC_THREADS = 256;
constexpr int DEC_CG = DEC_COLS / 4;                  // 4-column groups per tile (16)
constexpr int DEC_ROWSETS = DEC_THREADS / DEC_CG;     // 16
constexpr int DEC_ROWS = 128 / DEC_ROWSETS;           // rows per thread (8)
constexpr float DEC_LOG2E = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t x) { return __uint_as_float(x << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m, 64); }

template <bool NT>
__device__ __forceinline__ f32x4 load_state(const f32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void store_state(f32x4* p, f32x4 x) {
    if constexpr (NT) __builtin_nontemporal_store(x, p);
    else *p = x;
}

template <bool NT>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode_step(DecodeArgs a) {
    __shared__ float s_d[128], s_kd[128], s_qd[128], s_bk[128];
    __shared__ float s_qk[2];
    __shared__ f32x4 s_red[2][DEC_THREADS / 64][DEC_CG];  // [a | b][wave][column group]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x % DEC_TILES;
    const int64_t nh = blockIdx.x / DEC_TILES;  // n * H + h
    const int64_t n = nh / a.H;
    const int h = (int)(nh % a.H);
    // q/k row of the value head's group: n * Hk + h / group
    const int64_t nq = n * a.Hk + h / a.group;
    const int cg = tid % DEC_CG, rs = tid / DEC_CG;
    const int col = tile * DEC_COLS + 4 * cg;
    // state slot of sequence n; a sequence whose slot is outside the pool is
    // skipped: zero output, no state touched
    const int64_t slot = a.slots ? (int64_t)a.slots[n] : n;
    if (slot < 0 || slot >= a.n_slots) {
        if (rs == 0) *(uint2*)(a.out + nh * 128 + col) = uint2{0u, 0u};
        return;
    }
    const int64_t sh = slot * a.H + h;  // state row of (slot, head)
    const float beta = a.beta[nh];

    // the thread's state rows: issued first, they stream while the token's
    // per-row factors are formed
    f32x4* st = (f32x4*)(a.state + sh * (128 * 128) + col);
    f32x4 s[DEC_ROWS];
#pragma unroll
    for (int i = 0; i < DEC_ROWS; ++i) s[i] = load_state<NT>(st + (rs + DEC_ROWSETS * i) * (128 / 4));
    const uint2 vb = *(const uint2*)(a.v + nh * 128 + col);
    const f32x4 vv = {bf16_bits_to_f32(vb.x & 0xffffu), bf16_bits_to_f32(vb.x >> 16),
                      bf16_bits_to_f32(vb.y & 0xffffu), bf16_bits_to_f32(vb.y >> 16)};

    if (tid < 128) {
        const float kr = bf16_bits_to_f32(a.k[nq * 128 + tid]);
        const float qr = bf16_bits_to_f32(a.q[nq * 128 + tid]);
        const float d = __builtin_amdgcn_exp2f(a.g[nh * 128 + tid] * DEC_LOG2E);
        s_d[tid] = d;
        s_kd[tid] = kr * d;
        s_qd[tid] = qr * d;
        s_bk[tid] = beta * kr;
        float p = qr * kr;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) p = xor_sum(p, m);
        if (lane == 0) s_qk[wave] = p;
    }
    __syncthreads();

    // column sums over the thread's rows, then over the four row sets of the
    // wavefront (lanes 16 apart), then over the wavefronts
    f32x4 ca = {0.f, 0.f, 0.f, 0.f}, cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DEC_ROWS; ++i) {
        const int r = rs + DEC_ROWSETS * i;
        const float kd = s_kd[r], qd = s_qd[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ca[j] = __builtin_fmaf(kd, s[i][j], ca[j]);
            cb[j] = __builtin_fmaf(qd, s[i][j], cb[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ca[j] = xor_sum(xor_sum(ca[j], 16), 32);
        cb[j] = xor_sum(xor_sum(cb[j], 16), 32);
    }
    if (lane < DEC_CG) {
        s_red[0][wave][cg] = ca;
        s_red[1][wave][cg] = cb;
    }
    __syncthreads();
    f32x4 A = s_red[0][0][cg], B = s_red[1][0][cg];
#pragma unroll
    for (int w = 1; w < DEC_THREADS / 64; ++w) {
        A += s_red[0][w][cg];
        B += s_red[1][w][cg];
    }
    const f32x4 e = vv - A;

#pragma unroll
    for (int i = 0; i < DEC_ROWS; ++i) {
        const int r = rs + DEC_ROWSETS * i;
        const float d = s_d[r], bk = s_bk[r];
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = __builtin_fmaf(d, s[i][j], bk * e[j]);
        store_state<NT>(st + r * (128 / 4), o);
    }
    if (rs == 0) {
        const float bqk = beta * (s_qk[0] + s_qk[1]);
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = a.scale * __builtin_fmaf(bqk, e[j], B[j]);
        *(uint2*)(a.out + nh * 128 + col) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int64_t blocks = (int64_t)a.n_seqs * a.H * DEC_TILES;
    if (blocks == 0) return hipSuccess;
    const bool nt = (size_t)a.n_seqs * a.H * (128 * 128 * 4) > ((size_t)128 << 20);
    if (nt) hipLaunchKernelGGL(kda_decode_step<true>, dim3((unsigned)blocks), dim3(DEC_THREADS), 0, s, a);
    else hipLaunchKernelGGL(kda_decode_step<false>, dim3((unsigned)blocks), dim3(DEC_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
