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

// How a bf16 prefill is cut into workgroups. Each (unit, head) sequence is
// split into `segments` consecutive pieces of `seg_len` tokens (the last may be
// shorter), one workgroup each. With more than one segment, a pre-pass over
// `sub` equal pieces of every segment but the last computes the state each
// piece contributes; segment g then starts from the decayed sum of everything
// before it. All lengths are multiples of the 64-token sub-block.
// With value_slices == 4 the head is instead split into four 32-column value
// slices (one workgroup each, no segments, no workspace).
struct PrefillPlan {
    int segments;
    int sub;
    long long seg_len;
    size_t workspace;  // bytes: per (unit, head), (1 + (segments-1)*sub) fp32 d x d states
    int value_slices;  // 1 = whole head per workgroup, 4 = value-slice workgroups
};

PrefillPlan plan_prefill(long long units, long long seqlen, int heads, lt_dtype in_dtype,
                         bool varlen);

// fp32 inputs: one workgroup per (unit, head, 32-column value slice).
hipError_t launch_prefill_slices(const PrefillArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                                 hipStream_t stream);
// bf16 inputs: one 8-wave workgroup per (unit, head, segment) or per
// (unit, head, value slice).
hipError_t launch_prefill_heads(const PrefillArgs &a, const PrefillPlan &plan, void *workspace,
                                lt_dtype out_dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                         hipStream_t stream);

}  // namespace lt
