// Internal interface between the C-ABI front end (argument checks) and the
// HIP launchers. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "lightning.h"

namespace lt {

// One prefill launch: `units` independent sequences x `heads` heads.
// Fixed-length batches leave cu_seqlens NULL and use seqlen; packed batches
// pass cu_seqlens (device int32, units + 1 entries), total_tokens, and in
// seqlen the length of their longest sequence (the plan's upper bound).
// Optional epilogue after O = O_intra + O_inter: with gate != nullptr the
// kernels write y = o / sqrt(mean_d(o^2) + eps) * norm_weight[h] * sigmoid(g)
// per (token, head) instead of o; gate has o's shape in the input dtype,
// norm_weight is fp32 [heads, d].
struct NormGate {
    const void *gate = nullptr;
    const float *norm_weight = nullptr;
    float eps = 0.f;
};

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
    NormGate ng;
    // state_in holds S_0 transposed ([units, heads, d_value, d_key]); the
    // backward pass's dQ = forward(dO, V, K) carries S_0^T.
    bool state_in_t = false;
};

// Decode: state is [batch, heads, d, d], or with slot_ids != nullptr a pool
// [num_slots, heads, d, d] in which sequence b uses entry slot_ids[b] (an id
// outside [0, num_slots) marks a padding row: zero output, no state access).
struct DecodeArgs {
    const void *q, *k, *v;
    const float *slopes;
    float *state;
    void *o;
    int batch;
    int heads;
    NormGate ng;
    const int *slot_ids = nullptr;
    int num_slots = 0;
    // Workgroup order: workgroup (b, h) serves sequence (b * seq_stride) % batch,
    // a bijection (seq_stride is coprime with batch) that keeps the states of
    // workgroups running at the same time far apart in memory.
    int seq_stride = 1;
};

// Head dimension the kernels are built for.
constexpr int kHeadDim = 128;
// Value columns per prefill workgroup; a head's columns split over this many
// independent workgroups.
constexpr int kValueSlices = 4;

// How a bf16 prefill is cut into workgroups. Each (unit, head) sequence is
// split into `segments` consecutive pieces of `seg_len` tokens (the last may be
// shorter), one workgroup each. With more than one segment, the first
// (segments-1)*seg_len tokens are also cut into `pieces` pre-pass pieces of
// `piece_len` tokens (the last may be shorter); the pre-pass computes the state
// each piece contributes (and, for a piece that straddles a segment boundary,
// the part before the boundary), and the workgroup of segment g sums those
// before its start into its start state. Heads whose memory ends within a
// segment skip the pre-pass and take warm-up ranges (tiles.h). seg_len and
// piece_len are multiples of 128 tokens (two 64-token sub-blocks).
// With value_slices == 4 the head is instead split into four 32-column value
// slices (one workgroup each, no segments, no workspace).
struct PrefillPlan {
    int segments = 1;
    long long seg_len = 0;
    int pieces = 0;
    long long piece_len = 0;
    size_t workspace = 0;  // bytes: per (unit, head), prefill_states(...) fp32 d x d states
    int value_slices = 1;  // 1 = whole head per workgroup, 4 = value-slice workgroups
    // A segmented plan was wanted but even its coarsest pre-pass pieces need
    // more workspace than allowed (this plan is then the one without segments).
    bool workspace_short = false;
};

// fp32 d x d states per (unit, head) in the workspace of a segmented plan:
// one per piece, one partial state per segment boundary, one carried-in state
// per segment.
constexpr long long prefill_states(int segments, int pieces) { return pieces + (long long)segments; }

// HIP keeps the last error of any runtime call until it is read. Launchers
// clear it first, so the check after a launch reports that launch only and not
// an error some earlier call (the caller's, say) left behind.
inline void clear_pending_error() { (void)hipGetLastError(); }

// prepass_wgs: pre-pass workgroups to aim for (sets the piece length).
// max_workspace: bytes the plan may use; when the preferred pieces need more,
// the pieces are made longer (fewer states) until they fit. Without any fit the
// plan has no segments (value slices; whole heads for the caller to choose) and
// workspace_short set.
PrefillPlan plan_prefill(long long units, long long seqlen, int heads, lt_dtype in_dtype,
                         bool varlen, long long prepass_wgs, size_t max_workspace);

// The no-allocation entry point's scratch: the device address of this device's
// copy of a fixed static array, looked up once per device (hipGetSymbolAddress
// with the stream's device current) and kept until the process ends.
hipError_t noalloc_scratch(hipStream_t stream, void **ptr, size_t *bytes);

// Each kernel source's code object, loaded on the current device (the HIP
// runtime otherwise loads it at the first launch of one of its kernels): a
// query of one of its kernels' attributes forces the load.
hipError_t load_prefill_heads_code();
hipError_t load_prefill_slices_code();
hipError_t load_decode_code();
hipError_t load_backward_code();
hipError_t load_softmax_code();

// Backward of a fixed-length bf16 prefill (gradients of
// l = sum dout . o + <d_state_out, S_final>): dk, dv and d_state_in from one
// reverse pass; dq is the forward operator on (dout, v, k) with S_0^T.
struct BackwardArgs {
    const void *q, *k, *v, *dout;  // [units * seqlen, heads, d] bf16
    const float *slopes;
    const float *d_state_out;      // [units, heads, d, d] or null (zero)
    void *dk, *dv;                 // [units * seqlen, heads, d], OutT
    float *d_state_in;             // [units, heads, d, d] or null (not written)
    long long seqlen;
    int units;
    int heads;
};
// With a segmented plan (segments > 1, workspace of plan.workspace bytes) the
// reverse pass is split like the forward, in mirrored token order: segments
// and pre-pass pieces are counted from the end of each sequence.
hipError_t launch_backward_kv(const BackwardArgs &a, const PrefillPlan &plan, void *workspace,
                              lt_dtype out_dtype, hipStream_t stream);

// Softmax attention with grouped K/V heads and partial RoPE (the hybrid's
// other layer type). q [batch, seqlen, q_heads, d], k, v [batch, seqlen,
// kv_heads, d] bf16; o [batch, seqlen, q_heads, d]. Token t at position
// pos0 + t; rope on the first rope_dims features (a multiple of 32).
struct SoftmaxArgs {
    const void *q, *k, *v;
    void *o;
    int batch;
    long long seqlen;
    long long pos0;
    int q_heads, kv_heads;
    int rope_dims;
    double log2_base;
    float scale;
};
// workspace: rope(k), batch * seqlen * kv_heads * d bf16
hipError_t launch_softmax_prefill(const SoftmaxArgs &a, void *workspace, lt_dtype out_dtype,
                                  hipStream_t stream);

// One decode step of the softmax layer over a KV cache. q [batch, q_heads, d],
// k_new, v_new [batch, kv_heads, d], caches [batch, capacity, kv_heads, d]
// holding rope(k) and v, lengths [batch] int32 on the device (the new token's
// position; outside [0, capacity) marks a padding row).
struct SoftmaxDecodeArgs {
    const void *q, *k_new, *v_new;
    void *k_cache, *v_cache;
    const int *lengths;
    void *o;
    int batch;
    long long capacity;
    int q_heads, kv_heads;
    int rope_dims;
    double log2_base;
    float scale;
};
// Key splits per (sequence, K/V head): each split is one wave's range of
// chunk keys (a multiple of 32); splits > 1 needs a workspace of
// softmax_decode_workspace(batch, q_heads, splits) bytes.
struct SoftmaxDecodePlan {
    int splits = 1;
    long long chunk = 0;
};
inline long long softmax_decode_workspace(int batch, int q_heads, int splits) {
    return splits > 1 ? (long long)batch * q_heads * splits * 132 * 4 : 0;
}
hipError_t launch_softmax_decode(const SoftmaxDecodeArgs &a, const SoftmaxDecodePlan &plan,
                                 float *workspace, lt_dtype out_dtype, hipStream_t stream);

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
