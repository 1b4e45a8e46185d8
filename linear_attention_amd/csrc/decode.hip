// Lightning Attention decode step for gfx950 (MI355X).
//
// One token per sequence reads and rewrites that sequence's fixed d x d fp32
// state per head (MiniMax Signal Lab · M1, §03: the next step reads the carried
// state directly instead of rescanning history; §04: the state does not grow):
//     S <- e^{-s} S + k^T v ;   o = q S
// The output reads the updated state, as the per-token form of §03 does (the
// block diagonal D_ii = 1 lets a token see its own key). Optionally the output
// is normalised and gated before it is stored (the step after the sum in the
// §03 data-flow figure).
//
// With slot ids, the states live in a pool and sequence b uses entry
// slot_ids[b] (§04: each concurrent sequence keeps its own fixed state).
//
// The step is a pure HBM stream: 64 KiB of state read and 64 KiB written per
// (sequence, head) for about 5 * 128^2 flops, 0.62 flop per byte. Design:
//  * one 256-thread workgroup per (sequence, head); thread t owns value
//    columns 4*(t%32)..+3 of rows (t/32) + 8i, i = 0..15, so every row is one
//    fully coalesced 512-byte transaction of float4 loads/stores;
//  * all 16 state loads of a thread are issued before anything waits on them
//    (64 KiB in flight per workgroup);
//  * state loads and stores carry the non-temporal hint: a batch's states
//    (1 GiB at 256 sequences x 64 heads) are streamed once per step;
//  * workgroups visit sequences in a strided order (b * P mod batch, P near
//    0.618 * batch), so the states being streamed at any moment are spread
//    over the whole tensor: 0.357 ms per step on the 256 x 64 batch against
//    0.380 ms in sequence order;
//  * q.S is reduced in registers, across the two row groups of a wave with a
//    lane shuffle, then across the four waves through 2 KiB of LDS.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

namespace lt {
namespace {

constexpr int D = kHeadDim;
constexpr int NT = 256;
constexpr int ROWS_PER_THREAD = D / (NT / 32);  // 16
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float load_in(const float *p, long long i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t *p, long long i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 stream_load(const float *p) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void stream_store(float *p, float4 x) {
    __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4 *>(p));
}

__device__ __forceinline__ void store4(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }
__device__ __forceinline__ void store4(__bf16 *p, float4 x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 y;
    y[0] = static_cast<__bf16>(x.x);
    y[1] = static_cast<__bf16>(x.y);
    y[2] = static_cast<__bf16>(x.z);
    y[3] = static_cast<__bf16>(x.w);
    *reinterpret_cast<bf16x4 *>(p) = y;
}

__device__ __forceinline__ float4 load4_in(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4_in(const uint16_t *p) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}
__device__ __forceinline__ float sigmoid(float g) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g * LOG2E));
}

// NG: write y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g) instead of o.
template <typename G, typename OutT, bool NG>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
    __shared__ float qs[D], ks[D];
    __shared__ float4 part[4][D / 4];

    // sequence * heads + head, sequences visited in a strided order
    const int h = blockIdx.x % a.heads;
    const int unit = (int)(((long long)(blockIdx.x / a.heads) * a.seq_stride) % a.batch) * a.heads + h;
    const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5;
    long long su = unit;  // state entry of this (sequence, head)
    if (a.slot_ids) {
        const int slot = a.slot_ids[unit / a.heads];
        if (slot < 0 || slot >= a.num_slots) {  // padding row (uniform per workgroup)
            if (tid < 32) store4(static_cast<OutT *>(a.o) + (long long)unit * D + 4 * tid,
                                 make_float4(0.f, 0.f, 0.f, 0.f));
            return;
        }
        su = (long long)slot * a.heads + h;
    }
    float *st = a.state + su * D * D;

    float4 s[ROWS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < ROWS_PER_THREAD; ++i)
        s[i] = stream_load(st + (rg + 8 * i) * D + 4 * cg);

    const G *q = static_cast<const G *>(a.q) + (long long)unit * D;
    const G *k = static_cast<const G *>(a.k) + (long long)unit * D;
    const G *v = static_cast<const G *>(a.v) + (long long)unit * D;
    if (tid < D) {
        qs[tid] = load_in(q, tid);
        ks[tid] = load_in(k, tid);
    }
    const float4 v4 = make_float4(load_in(v, 4 * cg), load_in(v, 4 * cg + 1),
                                  load_in(v, 4 * cg + 2), load_in(v, 4 * cg + 3));
    const float lam = exp2f(-a.slopes[h] * LOG2E);
    float4 gate4 = make_float4(0.f, 0.f, 0.f, 0.f), w4 = gate4;
    if (NG && tid < 32) {
        gate4 = load4_in(static_cast<const G *>(a.ng.gate) + (long long)unit * D + 4 * tid);
        w4 = *reinterpret_cast<const float4 *>(a.ng.norm_weight + h * D + 4 * tid);
    }
    __syncthreads();

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < ROWS_PER_THREAD; ++i) {
        const int r = rg + 8 * i;
        const float kr = ks[r], qr = qs[r];
        float4 x = s[i];
        x.x = lam * x.x + kr * v4.x;
        x.y = lam * x.y + kr * v4.y;
        x.z = lam * x.z + kr * v4.z;
        x.w = lam * x.w + kr * v4.w;
        stream_store(st + r * D + 4 * cg, x);
        acc.x += qr * x.x;
        acc.y += qr * x.y;
        acc.z += qr * x.z;
        acc.w += qr * x.w;
    }
    // lanes l and l^32 of a wave hold row groups 2w and 2w+1 of the same columns
    acc.x += __shfl_xor(acc.x, 32);
    acc.y += __shfl_xor(acc.y, 32);
    acc.z += __shfl_xor(acc.z, 32);
    acc.w += __shfl_xor(acc.w, 32);
    const int w = tid >> 6;
    if ((tid & 63) < 32) part[w][cg] = acc;
    __syncthreads();
    if (tid < 32) {
        float4 o = part[0][tid];
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            o.x += part[j][tid].x;
            o.y += part[j][tid].y;
            o.z += part[j][tid].z;
            o.w += part[j][tid].w;
        }
        if constexpr (NG) {
            float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
            for (int m = 16; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / D) + a.ng.eps);
            o = make_float4(o.x * inv * w4.x * sigmoid(gate4.x), o.y * inv * w4.y * sigmoid(gate4.y),
                            o.z * inv * w4.z * sigmoid(gate4.z), o.w * inv * w4.w * sigmoid(gate4.w));
        }
        store4(static_cast<OutT *>(a.o) + (long long)unit * D + 4 * tid, o);
    }
}

template <typename G, typename OutT>
hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    clear_pending_error();
    const long long units = (long long)a.batch * a.heads;
    if (a.ng.gate)
        hipLaunchKernelGGL((decode_kernel<G, OutT, true>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<G, OutT, false>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t load_decode_code() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&decode_kernel<uint16_t, float, false>));
}

hipError_t launch_decode(const DecodeArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                         hipStream_t stream) {
    if (in_dtype == LT_BF16)
        return out_dtype == LT_F32 ? launch<uint16_t, float>(a, stream)
                                   : launch<uint16_t, __bf16>(a, stream);
    return out_dtype == LT_F32 ? launch<float, float>(a, stream) : launch<float, __bf16>(a, stream);
}

}  // namespace lt
