// Internal interface between the host runtime (kda_runtime.cpp) and the
// kernels (kda_kernels.hip): plan-table entry types, kernel parameter blocks
// and launchers. Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// K1 work item: one chunk (a sequence's local chunk index).
struct ChunkDesc {
    int32_t seq;
    int32_t chunk;  // local chunk index within the sequence
};

// K2 work unit: a whole sequence (serial) or one segment of it (CP).
struct UnitDesc {
    int32_t seq;
    int32_t chunk0;      // first local chunk of the unit
    int32_t n_chunks;    // chunks to run (may be 0: state copy only)
    int32_t rec_chunk0;  // global index of the unit's first chunk record
    int32_t in_slot;     // -1: initial_state[seq] (or zero); >= 0: carries[in_slot]
    int32_t write_final; // 1: write final_state[seq] at the end
    int32_t segment;     // segment index within the sequence
    int32_t n_segments;  // segments of the sequence
    // Warm-start segment (fused kernel only): the unit first runs the `warm`
    // chunks before chunk0, advancing over them both the transfer M (from the
    // identity, V := 0) and the state from zero, and then continues from that
    // state as if it were its carry. spec >= 0 names its slot of
    // speculation flags and end state; out_slot >= 0 makes a unit write its
    // end state to carries[out_slot] as well.
    int32_t warm;
    int32_t spec;
    int32_t out_slot;
    // CP segment-K2: the pre_scan summary slot of the previous segment (-1:
    // none). When that segment's transfer vanished (all its tiles exactly
    // zero), the unit starts from that segment's B summary, which is then its
    // carry bit for bit, and the merge writes no carry for it.
    int32_t b_slot;
};

// CP merge item: one segmented sequence.
struct MergeDesc {
    int32_t seq;
    int32_t n_segments;
    int32_t carry0;    // carries slot of segment 0 (segments use carry0 + s)
    int32_t prescan0;  // summary slot of segment 0 (segments 0..n-2)
};

// One segment of a merge item: the merge runs one workgroup per (segment,
// head, 16-column tile); only segments that start a run of live transfers
// compute.
struct MergeSeg {
    int32_t item;  // index into the merge items
    int32_t seg;   // segment index within the sequence
};

struct CommonArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const int32_t* cu;  // device cu_seqlens [n_seqs + 1]
    int64_t Tt;
    int32_t H;       // value heads (v, g, beta, states, out)
    int32_t Hk;      // q/k heads; H = group * Hk
    int32_t group;   // value heads per q/k head (value head h reads q/k head h / group)
    int32_t n_seqs;
    int32_t total_chunks;
    uint8_t* rec;  // K1 records [H][total_chunks][REC_BYTES]
    // When set, a kernel of the segmented pipeline does nothing unless
    // *gate != 0 (the fallback of a warm-start CP plan: armed by the flag
    // reduction when a warm-up transfer did not vanish).
    const int32_t* gate;
};

struct K2Args {
    CommonArgs c;
    const UnitDesc* units;
    int32_t n_units;
    const void* s0;      // may be null; fp32, or bf16 when state_bf16
    void* sT;            // may be null; fp32, or bf16 when state_bf16
    float* carries;      // [slots][H][128][128] fp32: read by in_slot, written by out_slot
    uint16_t* out;
    float scale;
    int32_t state_bf16;  // initial and final states are bf16
    // Warm-start segments: per (spec slot, head), one flag per 16-column tile
    // of the warm-up transfer (1 when that tile of M is not exactly zero)
    // and the segment's end state.
    int32_t* spec_flags;  // [spec slots][H][8]
    float* spec_states;   // [spec slots][H][128][128] fp32
    // Fix-up launch over warm-start segments: a unit whose warm-up transfer
    // was exactly zero copies its end state to the final state and stops;
    // any other reruns from its carry.
    int32_t fixup;
    // the warm-start segments write the final state themselves (it does not
    // alias the initial state, which other units may still read); else they
    // leave their end state in spec_states for the fix-up launch to publish
    int32_t spec_final_direct;
    // CP segment-K2 (units with b_slot >= 0): the pre_scan B summaries and
    // the per-tile flags of the transfers
    const float* b_seg;
    const int32_t* m_live;
    // K1 with the B summaries (the fused kernel's record-writing instance):
    // with gate_flags, every workgroup first ORs those n_gate_flags flags,
    // workgroup 0 writes the result to gate_out, and all return if none is
    // set (the first launch of warm-start CP's fallback)
    const int32_t* gate_flags;
    int64_t n_gate_flags;
    int32_t* gate_out;
    // K1 with the B summaries also forms each summarised segment's transfer M
    // (the update from S = I with V := 0) into m_out[out_slot], one flag per
    // 16-column tile into m_live_out (0: that tile is exactly zero). M is
    // stored only when some tile lives, a vanished tile then as zeros.
    float* m_out;
    int32_t* m_live_out;
};

struct MergeArgs {
    CommonArgs c;
    const MergeDesc* items;
    const MergeSeg* segs;
    int32_t n_segs;
    const void* s0;      // fp32, or bf16 when state_bf16
    const float* b_seg;
    const float* m_seg;
    float* carries;  // [slots][H][128][128]
    int32_t state_bf16;
    const int32_t* m_live;  // [slots][H][8]: 0 when that 16-column tile of M is exactly zero
};

struct K1Args {
    CommonArgs c;
    const ChunkDesc* chunks;
    // Gate from flags (the first launch of warm-start CP's fallback): every
    // workgroup ORs the n_gate_flags speculation flags and returns if none is
    // set; workgroup 0 writes the result to gate_out for the later launches.
    const int32_t* gate_flags;
    int64_t n_gate_flags;
    int32_t* gate_out;
};

hipError_t launch_k1_prepare(const K1Args& a, hipStream_t s);
hipError_t launch_beta_to_f32(const uint16_t* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_fused(const K2Args& a, hipStream_t s);
hipError_t launch_k2_recur(const K2Args& a, hipStream_t s);
hipError_t launch_k1_bsum(const K2Args& a, hipStream_t s);
hipError_t launch_cp_merge(const MergeArgs& a, hipStream_t s);

// The static scratch of the no-allocation prefill: its size, and its device
// address on the current device (hipGetSymbolAddress, in the source file that
// defines it).
size_t static_scratch_bytes();
hipError_t static_scratch_address(void** ptr);


constexpr int kChunk = 16;                      // tokens per chunk
constexpr size_t kRecBytes = 14336;            // bytes of one K1 chunk record in HBM (no V)
constexpr size_t kStateBytes = 128 * 128 * 4;  // one (sequence, head) state

}  // namespace kda
