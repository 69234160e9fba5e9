/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA forward prefill and decode library.
 *
 * Operation. Kimi Delta Attention (KDA) forward prefill: for every packed
 * sequence and head, the gated delta rule with per-key-channel decay
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = scale * S_t^T q_t,
 * computed in chunked form as the two kernels named in the commit summary of
 * "feat(kda/sm90): FlashKDA prefill port + intracard-CP prefill" (cuLA pull
 * request #103): K1 prepares decayed q/k, beta and the WY inverse per 16-token
 * chunk, K2 runs the inter-chunk recurrence (CHUNK = 16, D = 128, forward
 * only). The same commit summary defines the intracard context-parallel mode
 * (K1 once, then pre_scan, merge of segment carries, segment-K2; bit-identical
 * to serial), and its description the FLA-compatible prefill API with varlen
 * packing, initial/final state and a workspace arena reused across calls; its
 * reviewer notes say the planner returns the plan the executor runs, a trivial
 * plan meaning serial.
 *
 * Conventions shared by every entry point:
 *  - Packed token-major layouts, contiguous, row-major:
 *      q, k, out : bf16 [Tt, H, 128]      v : bf16 [Tt, H, 128]
 *      g         : fp32 [Tt, H, 128]  raw per-token log-decay (g <= 0 expected;
 *                  the in-chunk cumulative sum is taken by the library)
 *      beta      : fp32 [Tt, H]
 *      states    : fp32 [N, H, 128 (key channel), 128 (value channel)]
 *      cu_seqlens: int32 [N + 1], 0 = cu[0] <= cu[1] <= ... <= cu[N] = Tt
 *    Device pointers must be 16-byte aligned (beta: 4-byte aligned).
 *  - Ownership: the caller owns every tensor, stream and plan. The context
 *    owns only its workspace arenas (one per stream), which it frees in
 *    kda_destroy.
 *  - Errors: every check runs on the host before any launch, so nothing is
 *    written on error. Functions return a kda_status; kda_last_error() gives
 *    a message for the calling thread's most recent failure.
 *  - Asynchrony: kda_prefill only enqueues work on `stream` and never
 *    synchronises, except when it must grow the stream's workspace arena (a
 *    device synchronise, refused with KDA_ERR_CAPTURE while the stream is
 *    being captured into a graph). A plan whose workspace is 0 bytes touches
 *    no arena at all. "feat(cake_kda): share recurrent prefill kernels across
 *    SM100 family" (FlashInfer pull request #4313, review threads) asks that
 *    a captured call do no host preparation.
 *  - Graph capture: a captured call bakes into the graph the plan's device
 *    tables and the address of the stream's workspace arena. The plan must
 *    outlive every graph captured with it. Arena memory that served a capture
 *    is never freed before kda_destroy: growing or evicting such an arena
 *    retires the old memory instead, so a graph replayed after an uncaptured
 *    call with a larger plan on the same stream still finds its workspace
 *    (with the contents the replay itself writes).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID = 1,     /* bad shape, size, pointer, alignment or argument */
    KDA_ERR_UNSUPPORTED = 2, /* a head dimension other than 128 */
    KDA_ERR_ALIAS = 3,       /* forbidden overlap between buffers */
    KDA_ERR_CAPTURE = 4,     /* would allocate or synchronise during graph capture */
    KDA_ERR_HIP = 5          /* a HIP runtime call failed */
} kda_status;

/* Intracard context parallelism (the use_intracard_cp switch of the cuLA pull
 * request's description): off, forced on, or decided by the planner. */
typedef enum { KDA_CP_OFF = 0, KDA_CP_ON = 1, KDA_CP_AUTO = 2 } kda_cp_mode;

typedef struct kda_ctx kda_ctx;
typedef struct kda_plan kda_plan;

/* Summary of a plan, for inspection and tests. */
typedef struct {
    int32_t n_seqs, H, dk, dv;
    int64_t total_tokens;
    int32_t total_chunks;      /* sum over sequences of ceil(L_i / 16) */
    int32_t uses_cp;           /* 0 = trivial plan (serial), 1 = segmented */
    int32_t n_units;           /* K2 work units (sequences or segments) */
    int32_t n_cp_seqs;         /* sequences split into more than one segment */
    int32_t n_prescan;         /* segments that get a pre_scan summary */
    int32_t n_carry_slots;     /* carries kept for segmented sequences */
    int32_t max_unit_chunks;   /* longest serial chain of the plan, in chunks */
    int32_t n_cus;             /* compute units the plan was made for */
    size_t  workspace_bytes;   /* arena bytes kda_prefill needs for this plan */
    double  est_serial_us;     /* planner's cost estimate of the serial path */
    double  est_cp_us;         /* planner's cost estimate of the segmented path */
    int32_t k1_materialized;   /* 1: K1 writes chunk records to the workspace once and
                                  K2 / pre_scan read them (always so for segmented
                                  plans, and for serial plans made with
                                  KDA_MATERIALIZE_K1=1 in the environment); 0: serial
                                  plan whose fused kernel recomputes K1 per chunk in LDS
                                  (the default for serial plans) */
    int32_t n_split_seqs;      /* sequences run as a first segment plus a warm-start
                                  segment (see kda_plan_prefill_split); AUTO plans
                                  choose these when the longest sequences would
                                  otherwise leave the compute units idle at the end */
    int32_t split_warm_chunks; /* warm-up chunks of each warm-start segment */
    double  est_split_us;      /* planner's estimate of the split plan (-1: none) */
    int32_t warm_cp;           /* 1: warm-start CP (see kda_plan_prefill_warm_cp) */
    int32_t warm_cp_seg_chunks;/* its segment length in chunks */
    int32_t n_warm_segments;   /* its speculation slots (warm-start and last segments) */
    double  est_warm_cp_us;    /* planner's estimate of warm-start CP (-1: none) */
    int32_t speculation_off;   /* 1 once an earlier call of this split or warm-start CP plan
                                  found that speculation failed: later calls outside graph
                                  capture run the plan's exact path (the batch unsplit, or
                                  the segmented pipeline), which gives the same bits */
    int32_t split_warm_work;   /* the warm-up's cost in chunk intervals as the planner
                                  counts it (a warm-start segment of n chunks costs
                                  n + split_warm_work): its W chunks each form two
                                  states, the transfer and the state from zero */
} kda_plan_info;

/* One K2 work unit of a plan (a whole sequence, or one segment of it). */
typedef struct {
    int32_t seq;          /* sequence index */
    int32_t chunk0;       /* first chunk of the unit within its sequence */
    int32_t n_chunks;     /* chunks in the unit (0 for an empty sequence) */
    int32_t segment;      /* segment index within its sequence (0 if serial) */
    int32_t n_segments;   /* segments of its sequence (1 if serial) */
    int32_t warm_chunks;  /* warm-up chunks run before chunk0 (warm-start segment), else 0 */
} kda_unit_info;

/* Create a context on HIP device `device`: caches the device properties
 * (compute-unit count) once. The review thread of "feat(cake_kda): share
 * recurrent prefill kernels across SM100 family" (FlashInfer pull request
 * #4313) asks that device properties be cached rather than queried on every
 * launch; the compute-unit count is also what the planner of "feat(kda/sm90):
 * FlashKDA prefill port + intracard-CP prefill" (cuLA pull request #103,
 * description) sizes its decision by. `out` receives the context, owned by
 * the caller until kda_destroy. Returns KDA_ERR_INVALID for a NULL `out` or a
 * device index out of range, KDA_ERR_HIP if the device is unusable. */
kda_status kda_create(int device, kda_ctx **out);

/* Wait for the device, then free every workspace arena (including memory
 * retired after serving a graph capture) and the context. The arena is the
 * workspace reused across calls of the cuLA pull request's description; it
 * lives as long as its context. NULL is a no-op. The caller must not destroy a
 * context while another thread uses it. */
void kda_destroy(kda_ctx *ctx);

/* Message of the calling thread's most recent failure ("" if none); the
 * pointer stays valid until that thread's next failing call. A review thread
 * of "feat(cake_kda): share recurrent prefill kernels across SM100 family"
 * (FlashInfer pull request #4313) asks that an unsupported call be rejected
 * by a check rather than crash; every check here fails with a message. */
const char *kda_last_error(void);

/* Library version string. */
const char *kda_version(void);

/* Build the plan for one packed batch: chunk table, K2 work units ordered
 * longest chain first, and -- when `mode` asks for it, or AUTO predicts a win
 * for the device's compute-unit count -- chunk-aligned segments for intracard
 * CP. ON always gives the segmented pipeline (kda_plan_prefill_segments). AUTO
 * may instead give warm-start CP (kda_plan_prefill_warm_cp) for few-head long
 * sequences, or warm-start splits of the longest sequences of a batch that
 * fills the compute units about once (kda_plan_prefill_split). Both speculate
 * that the decay forgets a segment's carry within its warm-up, and stay exact
 * when it does not, at a cost. OFF never segments.
 * cu_seqlens_host: host int32 [n_seqs + 1]. dk and dv must be 128.
 * The plan keeps its tables in device memory of ctx's device (uploaded here,
 * synchronously; do not call while a stream of that device is being
 * captured). The caller frees it with kda_plan_destroy. */
kda_status kda_plan_prefill(kda_ctx *ctx, const int32_t *cu_seqlens_host, int32_t n_seqs,
                            int32_t H, int32_t dk, int32_t dv, kda_cp_mode mode,
                            kda_plan **out);

/* The same planning for an explicit compute-unit count, host only (no device
 * tables; such a plan can be inspected but not executed). Needs no GPU. */
kda_status kda_plan_prefill_host(int32_t n_cus, const int32_t *cu_seqlens_host, int32_t n_seqs,
                                 int32_t H, int32_t dk, int32_t dv, kda_cp_mode mode,
                                 kda_plan **out);

/* A segmented plan with an explicit segment length: every sequence longer
 * than seg_chunks chunks is cut into chunk-aligned segments of seg_chunks
 * chunks (the last may be shorter) and run through pre_scan, merge and
 * segment-K2 -- the forced-CP mode of the cuLA pull request's tests. Device
 * tables are uploaded as in kda_plan_prefill. */
kda_status kda_plan_prefill_segments(kda_ctx *ctx, const int32_t *cu_seqlens_host, int32_t n_seqs,
                                     int32_t H, int32_t dk, int32_t dv, int32_t seg_chunks,
                                     kda_plan **out);

/* A plan that splits sequence i at chunk split_chunk[i] (0: not split) into
 * two segments run side by side in the fused serial kernel, the intracard
 * context parallelism of "feat(kda/sm90): FlashKDA prefill port +
 * intracard-CP prefill" (cuLA pull request #103, description) without its
 * separate pre_scan and merge passes. The first segment runs from the initial
 * state. The second, a warm-start segment, first runs the warm_chunks chunks
 * before its start, advancing two states over them: the transfer M from the
 * identity with V := 0, and the state B from zero. Where every tile of M is
 * exactly zero, B is
 * its carry, exactly as the CP merge takes it; otherwise a fix-up launch
 * reruns the segment from the first segment's end state. Either way the
 * result equals the unsplit serial path's bit for bit wherever the CP
 * path's does. split_chunk[i] must be 0 or in [warm_chunks, chunks of
 * sequence i), and warm_chunks >= 1; otherwise KDA_ERR_INVALID and no plan.
 * AUTO plans (kda_plan_prefill) pick such splits themselves.
 * Device tables are uploaded as in kda_plan_prefill. */
kda_status kda_plan_prefill_split(kda_ctx *ctx, const int32_t *cu_seqlens_host, int32_t n_seqs,
                                  int32_t H, int32_t dk, int32_t dv, const int32_t *split_chunk,
                                  int32_t warm_chunks, kda_plan **out);

/* Warm-start CP: every sequence longer than seg_chunks chunks is cut into
 * chunk-aligned segments of seg_chunks, and all segments run side by side in
 * one fused launch, each after the first as a warm-start segment with
 * warm_chunks warm-up chunks (see kda_plan_prefill_split). The segmented CP
 * pipeline of kda_plan_prefill_segments with the same segment length is kept
 * as the fallback. A flag reduction on the device arms it only if some
 * warm-up transfer did not vanish; it then recomputes every output and
 * final state. With the fallback unarmed, the result equals the serial
 * path's bit for bit wherever the CP path's does; armed, it is the CP path's
 * result. No host synchronisation is involved, so a captured graph replays
 * either way. AUTO plans choose this for few-head long sequences when the
 * planner predicts a win over the segmented path. 1 <= warm_chunks <=
 * seg_chunks, else KDA_ERR_INVALID. The plan's workspace includes the
 * fallback's (the K1 records of every chunk). Device tables are uploaded as
 * in kda_plan_prefill. */
kda_status kda_plan_prefill_warm_cp(kda_ctx *ctx, const int32_t *cu_seqlens_host, int32_t n_seqs,
                                    int32_t H, int32_t dk, int32_t dv, int32_t seg_chunks,
                                    int32_t warm_chunks, kda_plan **out);

void kda_plan_destroy(kda_plan *plan);

/* Bytes of the per-stream workspace arena that kda_prefill needs for this
 * plan (0 for NULL), so that a caller can warm the arena up before graph
 * capture. kda_prefill_ex with a bf16 beta needs 4 * Tt * H bytes more,
 * after this much rounded up to 256. The workspace holds the scratch of the
 * intracard CP pipeline (K1 records, the b_seg / m_seg summaries and the
 * carries named in the cuLA pull request's review thread), which the arena
 * reuses across calls (its description). */
size_t kda_plan_workspace_bytes(const kda_plan *plan);

/* Plan summary; returns KDA_ERR_INVALID for NULL arguments. */
kda_status kda_plan_get_info(const kda_plan *plan, kda_plan_info *info);

/* Copy up to `max_units` unit descriptors, in launch order. */
kda_status kda_plan_get_units(const kda_plan *plan, kda_unit_info *units, int32_t max_units);

/* Check a prefill call's arguments against the plan without launching
 * anything (the same checks kda_prefill runs first). Pointers are compared as
 * addresses only and never dereferenced. Needs no GPU. */
kda_status kda_prefill_validate(const kda_plan *plan, const void *q, const void *k,
                                const void *v, const float *g, const float *beta,
                                const int32_t *cu_seqlens_dev, float scale,
                                const float *initial_state, const float *final_state,
                                const void *out);

/* Run the forward prefill described by `plan` on `stream`.
 *   q, k, v, out : bf16 [Tt, H, 128] (device)
 *   g, beta      : fp32 [Tt, H, 128], [Tt, H] (device)
 *   cu_seqlens_dev: int32 [N + 1] (device), the same values the plan was
 *                  built from
 *   scale        : multiplies every output (1.0 for the plain recurrence)
 *   initial_state: fp32 [N, H, 128, 128] or NULL (zero state)
 *   final_state  : fp32 [N, H, 128, 128] or NULL (not written); may equal
 *                  initial_state (updated in place) but may not partly
 *                  overlap it; may not overlap any input or out
 *   out          : may not overlap any input or state
 * Serial plans launch one fused K1+K2 kernel (or K1 then K2 when the plan
 * materialises K1); segmented plans launch pre_scan, merge and segment-K2
 * (preceded by K1 when it is materialised). Every form runs the same K1 and
 * K2 arithmetic, so their results are bitwise equal. Results of a segmented plan are
 * bitwise equal to the serial plan's whenever the carried-in state is
 * forgotten within a segment (strong decay); otherwise equal within fp32
 * rounding. */
kda_status kda_prefill(kda_ctx *ctx, const kda_plan *plan, const void *q, const void *k,
                       const void *v, const float *g, const float *beta,
                       const int32_t *cu_seqlens_dev, float scale, const float *initial_state,
                       float *final_state, void *out, hipStream_t stream);

/* Decode step: each of n_seqs sequences receives one new token, and its state
 * is advanced by one step of the recurrence, in place:
 *   S' = (I - beta k k^T) Diag(exp g) S + beta k v^T,   o = scale S'^T q.
 * This is the single-token case of the recurrence in the commit summary of
 * "feat(kda/sm90): FlashKDA prefill port + intracard-CP prefill" (cuLA pull
 * request #103); "feat(cake_kda): share recurrent prefill kernels across
 * SM100 family" (FlashInfer pull request #4313, AOT registration notes) keeps
 * a KDA decode entry of this kind beside the prefill.
 *   q, k         : bf16 [n_seqs, qk_heads, 128] (device, 16-byte aligned); H
 *                  must be a multiple of qk_heads, and value head h reads q/k
 *                  head h / (H / qk_heads) (grouped value heads, as in
 *                  kda_prefill_opts; qk_heads = H is the plain case)
 *   v, out       : bf16 [n_seqs, H, 128] (device, 16-byte aligned)
 *   g            : fp32 [n_seqs, H, 128] raw log-decay (device, 16-byte aligned)
 *   beta         : fp32 [n_seqs, H] (device, 4-byte aligned)
 *   state        : fp32 [n_seqs, H, 128, 128] (device, 16-byte aligned), read
 *                  and overwritten with the advanced state; may not overlap
 *                  any input or out
 *   out          : may not overlap any input or state
 * dk and dv must be 128. n_seqs = 0 is a no-op. One kernel launch on `stream`,
 * no allocation, no synchronisation; results are bitwise reproducible. The
 * step reads and writes each (sequence, head) state once. */
kda_status kda_decode(kda_ctx *ctx, int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                      const void *q, const void *k, const void *v, const float *g, const float *beta,
                      float scale, float *state, void *out, hipStream_t stream);

/* kda_decode over a pool of states: sequence n reads and advances state
 * slot slots[n] of state [n_slots, H, 128, 128] (a continuous-batching
 * engine keeps such a pool and a slot table per step). slots: device int32
 * [n_seqs], 4-byte aligned. A sequence whose slot is outside [0, n_slots)
 * (for instance -1 for a padded entry) is skipped: its output is zero and no
 * state is touched. Two sequences may not share a slot (their updates would
 * race). slots = NULL with n_slots = n_seqs is kda_decode. */
kda_status kda_decode_slots(kda_ctx *ctx, int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                            const void *q, const void *k, const void *v, const float *g, const float *beta,
                            float scale, float *state, int32_t n_slots, const int32_t *slots, void *out,
                            hipStream_t stream);

/* The argument checks of kda_decode_slots (addresses only; needs no GPU). */
kda_status kda_decode_slots_validate(int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                                     const void *q, const void *k, const void *v, const float *g,
                                     const float *beta, float scale, const float *state, int32_t n_slots,
                                     const int32_t *slots, const void *out);

/* The argument checks of kda_decode, without launching anything. Pointers are
 * compared as addresses only and never dereferenced. Needs no GPU. */
kda_status kda_decode_validate(int32_t n_seqs, int32_t H, int32_t qk_heads, int32_t dk, int32_t dv,
                               const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float scale, const float *state, const void *out);

/* Options of kda_prefill_ex. A zeroed struct (or NULL) gives kda_prefill. */
typedef struct {
    /* Grouped value heads (GVA): q and k have qk_heads heads while v, g,
     * beta, the states and out have the plan's H heads, H a multiple of
     * qk_heads; value head h reads q/k head h / (H / qk_heads), so each q/k
     * head serves that many consecutive value heads. 0 means H (no grouping).
     * The reviewer notes of "feat(kda/sm90): FlashKDA prefill port +
     * intracard-CP prefill" (cuLA pull request #103) restrict that prefill to
     * num_kv_heads == num_qk_heads and name GVA as its follow-up. */
    int32_t qk_heads;
    /* 1: beta is bf16 [Tt, H] (2-byte aligned). It is widened to fp32 in the
     * stream's workspace arena by one extra launch; the results are then
     * bitwise those of kda_prefill on that fp32 beta. The FlashInfer KDA
     * facade of "fix(cake_kda): support non-aligned recurrent prefill head
     * counts" (pull request #4351, description) keeps beta in bf16. */
    int32_t beta_bf16;
    /* 1: initial_state and final_state are bf16 [N, H, 128, 128]; the state
     * is read exactly, carried in fp32 and rounded to nearest even once, when
     * the final state is written. The same facade allocates its returned
     * final state in bf16 (review thread of FlashInfer pull request #4313). */
    int32_t state_bf16;
} kda_prefill_opts;

/* kda_prefill with options (grouped value heads, bf16 beta, bf16 states).
 *   q, k : bf16 [Tt, qk_heads, 128] (device)
 *   beta : fp32 [Tt, H], or bf16 with beta_bf16
 *   initial_state, final_state : fp32 [N, H, 128, 128], or bf16 with
 *          state_bf16 (device, 16-byte aligned)
 * everything else as in kda_prefill. Errors as kda_prefill, plus
 * KDA_ERR_INVALID when H is not a multiple of qk_heads. */
kda_status kda_prefill_ex(kda_ctx *ctx, const kda_plan *plan, const kda_prefill_opts *opts, const void *q,
                          const void *k, const void *v, const float *g, const void *beta,
                          const int32_t *cu_seqlens_dev, float scale, const void *initial_state,
                          void *final_state, void *out, hipStream_t stream);

/* The argument checks of kda_prefill_ex, without launching anything
 * (addresses only, never dereferenced; needs no GPU). */
kda_status kda_prefill_ex_validate(const kda_plan *plan, const kda_prefill_opts *opts, const void *q,
                                   const void *k, const void *v, const float *g, const void *beta,
                                   const int32_t *cu_seqlens_dev, float scale, const void *initial_state,
                                   const void *final_state, const void *out);

/* kda_prefill_ex for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc. The call
 * allocates nothing and synchronises nothing: its workspace is a static
 * device array of kda_noalloc_scratch_bytes() bytes (32 MiB) that each GPU
 * the library runs on holds from the first kda_create on it until the
 * process ends (its address is looked up once per device, in kda_create).
 * Arguments, results and errors are those of kda_prefill_ex, and the
 * results are bitwise those of kda_prefill_ex with the same plan. A plan
 * whose workspace (kda_plan_workspace_bytes, plus 4 * Tt * H bytes after it,
 * rounded up to 256, for a bf16 beta) exceeds the static array is refused
 * with KDA_ERR_INVALID before any launch. Serial plans need no workspace;
 * warm-start split plans need 128 KiB per (split sequence, head); the
 * segmented and warm-start CP plans of long sequences usually exceed it. The
 * speculation feedback of split and warm-start CP plans is not collected by
 * this call (it needs pinned host memory), and no per-kernel timing is
 * recorded. Every call on one GPU shares that GPU's array and leaves it
 * holding its own intermediates; nothing in it needs clearing between calls,
 * but calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race on it. */
kda_status kda_prefill_noalloc(kda_ctx *ctx, const kda_plan *plan, const kda_prefill_opts *opts, const void *q,
                               const void *k, const void *v, const float *g, const void *beta,
                               const int32_t *cu_seqlens_dev, float scale, const void *initial_state,
                               void *final_state, void *out, hipStream_t stream);

/* Bytes of the static scratch of kda_prefill_noalloc (32 MiB). */
size_t kda_noalloc_scratch_bytes(void);

/* K1 alone, for inspection and tests: write every chunk record of the plan
 * into `records` (device, total_chunks * H * KDA_RECORD_BYTES bytes, record
 * of (chunk c, head h) at index h * total_chunks + c; layout in
 * KDA_RECORD_* below). Arguments as in kda_prefill. */
#define KDA_RECORD_BYTES 14336
/* Record layout: the order in which a 64-wide wavefront reads its MFMA
 * fragments (bf16 unless noted). Lane l has g = l / 16, i = l % 16;
 * dkperm(p, g, j) = 32p + 16(j / 4) + 4g + j % 4. r = token row 0..15 of the
 * chunk (rows past the end of a short chunk are zero), c = channel.
 *   [0, 4096)      Qt = q * exp(G): [p 4][lane 64][j 8] = Qt[i][dkperm(p, g, j)]
 *   [4096, 8192)   X = k * exp(G): same layout as Qt
 *   [8192, 12288)  Kt = k * exp(G_C - G): [t 8][slot 64][j 4]; slot s(l) holds
 *                  lane l's Kt[4g + j][16t + i], s(l) = (l & 0x33) | ((((l >> 2) + (l >> 4)) & 3) << 2)
 *   [12288, 12800) A_qk (lower incl. diagonal): [lane 64][j 4] = A_qk[i][4g + j]
 *   [12800, 13312) exp(G_C): fp32 [128], channel 16t + 4g + j at position 32g + 4t + j
 *   [13312, 14336) T' = (I + L)^-1 diag(beta), L = strict-lower(diag(beta) A_kk),
 *                  as a bf16 pair hi + lo: [2][lane 64][j 4] = T'[i][4g + j]
 * K2 forms U = T' (V - X S) (= U~ - W S in WY terms), then O = Qt S + A_qk U
 * and S <- Diag(exp G_C) S + Kt^T U. A record holds no copy of V: K2 reads
 * the chunk's value rows from v itself.
 */
kda_status kda_debug_k1_records(kda_ctx *ctx, const kda_plan *plan, const void *q, const void *k,
                                const void *v, const float *g, const float *beta,
                                const int32_t *cu_seqlens_dev, void *records, hipStream_t stream);

/* Per-kernel timing of kda_prefill and kda_decode calls on this context: while enabled,
 * every call records HIP events around each of its launches on its stream.
 * kda_get_timing waits for all recorded events, and returns, per kernel name
 * (in order of first launch), the summed elapsed milliseconds and the number
 * of launches since the previous kda_get_timing or kda_set_timing call; it
 * then clears the log. Returns the number of names (<= max), or -1 on error. */
kda_status kda_set_timing(kda_ctx *ctx, int enable);
int32_t kda_get_timing(kda_ctx *ctx, const char **names, double *total_ms, int32_t *launches,
                       int32_t max);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
