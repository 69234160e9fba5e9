// Internal interface between the host runtime (kda_runtime.cpp) and the
// decode kernel (kda_decode.hip). Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Decode step: one token per sequence, state [n_seqs][H][128][128] in place.
struct DecodeArgs {
    const uint16_t* q;     // [n_seqs][Hk][128] bf16
    const uint16_t* k;
    const uint16_t* v;
    const float* g;        // [n_seqs][H][128]
    const float* beta;     // [n_seqs][H]
    float* state;          // [n_seqs][H][128][128], read and written
    uint16_t* out;         // [n_seqs][H][128] bf16 (v too)
    int32_t n_seqs;
    int32_t H;             // value heads
    int32_t Hk;            // q/k heads; value head h reads q/k head h / group
    int32_t group;
    float scale;
    const int32_t* slots;  // null: sequence n uses state[n]; else state[slots[n]], skipped when
                           // slots[n] is outside [0, n_slots)
    int32_t n_slots;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace kda
