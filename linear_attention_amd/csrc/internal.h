// Internal interface between the C-ABI front end (argument checks) and the
// HIP launchers. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "lightning.h"

namespace lt {

// One prefill launch: `units` independent sequences x `heads` heads.
// Fixed-length batches leave cu_seqlens NULL and use seqlen; packed batches
// pass cu_seqlens (device int32, units + 1 entries) and total_tokens.
struct PrefillArgs {
    const void *q, *k, *v;
    const float *slopes;
    void *o;
    const float *state_in;
    float *state_out;
    const int *cu_seqlens;
    long long seqlen;
    long long total_tokens;
    int units;
    int heads;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *slopes;
    float *state;
    void *o;
    int batch;
    int heads;
};

// Head dimension the kernels are built for.
constexpr int kHeadDim = 128;
// Value columns per prefill workgroup; a head's columns split over this many
// independent workgroups.
constexpr int kValueSlices = 4;

hipError_t launch_prefill(const PrefillArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                          hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                         hipStream_t stream);

}  // namespace lt
