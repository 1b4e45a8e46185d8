// Device-side building blocks shared by the bf16 prefill kernels (forward and
// backward) on gfx950: tile shapes, LDS layouts, MFMA operand loads, streaming
// HBM access, register staging of 64-token sub-blocks, the state update and the
// staged full-row output stores. Internal; included by .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

namespace lt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int D = kHeadDim;  // 128
constexpr int C = 64;        // tokens per sub-block
constexpr int NT = 512;      // 8 waves
constexpr int PW = C;        // width of the P tile
constexpr float LOG2E = 1.4426950408889634f;

static_assert(D == 128 && C == 64, "tile shapes are fixed below");

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Masked, decayed scores. A score of key j for query i is multiplied by
// D_ij = e^{-s(i-j)} for i >= j and is 0 for i < j. The product uses the
// legacy multiply (v_mul_legacy_f32: 0 times anything, NaN and Inf included,
// is 0), so a NaN or Inf score from a non-finite q or k never reaches a query
// that cannot see that key, while every visible entry keeps a factor of at
// least 2^-126 (a decay that underflows contributes below 1e-38 instead of
// 0), through which a NaN or Inf still propagates as in the exact operator.
__device__ __forceinline__ float masked_decay(int diff, float s2) {
    return diff >= 0 ? fmaxf(fast_exp2(-s2 * (float)diff), 0x1p-126f) : 0.f;
}
extern "C" __device__ float lt_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");
__device__ __forceinline__ float mask_mul(float score, float decay) { return lt_fmul_legacy(score, decay); }

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tile layouts. Tiles are row-major without padding; bank conflicts are
// avoided by permuting the 16-byte chunks of each row. For a 128-wide bf16 tile
// (16 chunks per 256-byte row) chunk c of row r is stored at c ^ swz(r) with
// swz(r) = ((r & 3) << 2) | ((r >> 2) & 3), a bijection on the 16 rows of any
// aligned 16-row group (16-byte operand reads of 16 consecutive rows hit 64
// distinct banks) that also sends the chunk pairs read by one transposing read
// (4 consecutive rows x 2 adjacent chunks) to 4 disjoint pairs (8-byte reads of
// a 32-lane half-wave hit 64 distinct banks).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct L128 {  // [rows][128] bf16
    static constexpr int kPitch = 128;
    __device__ static int off(int row, int col) {
        return row * 128 + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
    }
};
struct LP {  // P tile [64][64] bf16: 8 chunks per 128-byte row, two rows per bank line
    static constexpr int kPitch = PW;
    __device__ static int off(int row, int col) {
        return row * PW + ((((col >> 3) ^ ((row >> 1) & 7)) << 3) | (col & 7));
    }
};
template <int PITCH>
struct LPad {  // narrow tiles: plain padded rows
    static constexpr int kPitch = PITCH;
    __device__ static int off(int row, int col) { return row * PITCH + col; }
};

// MFMA operand (32x32x16, bf16) from an LDS tile whose rows are the operand
// rows: lane l reads row row0 + (l % 32), contraction slots k0 + 8*(l / 32)..+7.
template <class L>
__device__ __forceinline__ bf16x8 ld_op(const __bf16 *t, int row0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(t + L::off(row0 + (lane & 31), k0 + 8 * (lane >> 5)));
}

// MFMA operand whose rows are the COLUMNS of an LDS tile and whose contraction
// runs down the tile rows: lane l gets tile[k0 + 8*(l/32) + e][c0 + (l % 32)],
// e = 0..7. ds_read_b64_tr_b16 lets each 16-lane group load a 4x16 block (lanes
// 4r..4r+3 give row r) and hands lane i column i.
template <class L>
__device__ __forceinline__ bf16x8 ld_op_t(const __bf16 *t, int c0, int k0, int lane) {
    const int li = lane & 15, grp = lane >> 4;
    // k0 (a multiple of 16 at every call) enters as a whole number of rows:
    // each layout's row swizzle repeats every 16 rows, so k0 * kPitch is a plain
    // offset, which the compiler folds into the read's immediate field instead
    // of holding one address register per k0 (15 fewer in the main prefill
    // loop; the norm-gate variant's spill reloads left its loop)
    const int r = 8 * (grp >> 1) + (li >> 2), col = c0 + 16 * (grp & 1) + 4 * (li & 3);
    const __bf16 *p = t + k0 * L::kPitch;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + L::off(r, col)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + L::off(r + 4, col)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Streaming HBM access. q, k, v are read once and o is written once, so loads
// and stores carry the non-temporal hint; measured on this kernel's access
// pattern (256-byte row pieces at a 16 KiB token stride) it lifts the k, v
// read rate from 2.4 to 5.7 TB/s and the q, k, v + o pattern from 5.2 to
// 5.8 TB/s. State and workspace traffic keeps the default policy.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The streams live in device memory. Their accesses go through global-address-
// space pointers: a generic pointer that the compiler cannot trace back to a
// kernel argument (one read back from LDS, as the piece loops do) would get
// flat loads and stores instead, and on this GPU a flat access counts against
// the LDS wait counter too, so every wait for an LDS operand would also wait
// for the sub-block prefetches in flight.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T *global_view(T *p) {
    return (__attribute__((address_space(1))) T *)p;
}
__device__ __forceinline__ uint4 stream_load16(const uint16_t *p) {
    const u32x4 x = __builtin_nontemporal_load(global_view(reinterpret_cast<const u32x4 *>(p)));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 stream_load8(const uint16_t *p) {
    const u32x2 x = __builtin_nontemporal_load(global_view(reinterpret_cast<const u32x2 *>(p)));
    return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void stream_store(float *p, float4 x) {
    __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, global_view(reinterpret_cast<f32x4 *>(p)));
}
template <class V>
__device__ __forceinline__ void stream_store_bits(__bf16 *p, const V &x) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "16- or 8-byte stores");
    if constexpr (sizeof(V) == 16) {
        u32x4 b;
        __builtin_memcpy(&b, &x, 16);
        __builtin_nontemporal_store(b, global_view(reinterpret_cast<u32x4 *>(p)));
    } else {
        u32x2 b;
        __builtin_memcpy(&b, &x, 8);
        __builtin_nontemporal_store(b, global_view(reinterpret_cast<u32x2 *>(p)));
    }
}

__device__ __forceinline__ uint4 keep_if(bool keep, uint4 x) {
    return make_uint4(keep ? x.x : 0u, keep ? x.y : 0u, keep ? x.z : 0u, keep ? x.w : 0u);
}

// 8 bf16 (in a uint4) scaled by f, rounded back to bf16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 x, float f) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16) * f;
        const float hi = __uint_as_float(w[i] & 0xffff0000u) * f;
        const __bf16 blo = static_cast<__bf16>(lo), bhi = static_cast<__bf16>(hi);
        uint16_t ulo, uhi;
        __builtin_memcpy(&ulo, &blo, 2);
        __builtin_memcpy(&uhi, &bhi, 2);
        r[i] = (uint32_t)ulo | ((uint32_t)uhi << 16);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Register staging of one sub-block: thread t holds tokens (t/16) + 32i,
// i = 0, 1, elements 8*(t%16)..+7 of q, k and v. Loads are unconditional with
// rows clamped into [0, m), so their number never depends on m; rows >= m are
// zeroed when written to LDS.
template <bool WITH_Q>
struct Stage {
    uint4 q[2], k[2], v[2];

    __device__ void load(const uint16_t *qg, const uint16_t *kg, const uint16_t *vg, int ts, int m,
                         int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const int row = (t < m ? t : m - 1) * ts + 8 * seg;
            if (WITH_Q) q[i] = stream_load16(qg + row);
            k[i] = stream_load16(kg + row);
            v[i] = stream_load16(vg + row);
        }
    }

    // Writes Q, K, V row-major and V ⊙ d_k (d_k[t] = e^{-s(m-1-t)}, 0 for t >= m);
    // without Q (the pre-pass) only K and V ⊙ d_k. FULL: m == C (no masking).
    template <bool FULL>
    __device__ void store(__bf16 *Qs, __bf16 *Ks, __bf16 *Vs, __bf16 *Vds, int m, float s2,
                          int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const bool in = FULL || t < m;
            const int off = L128::off(t, 8 * seg);
            if (WITH_Q) *reinterpret_cast<uint4 *>(Qs + off) = keep_if(in, q[i]);
            *reinterpret_cast<uint4 *>(Ks + off) = keep_if(in, k[i]);
            const uint4 vv = keep_if(in, v[i]);
            if (WITH_Q) *reinterpret_cast<uint4 *>(Vs + off) = vv;  // the pre-pass needs only V ⊙ d_k
            const float dk = in ? fast_exp2(-s2 * (float)((FULL ? C : m) - 1 - t)) : 0.f;
            *reinterpret_cast<uint4 *>(Vds + off) = scale_bf16x8(vv, dk);
        }
    }
};

// Wave roles (w = wave index, h = lane / 32, r32 = lane % 32):
//   qh = w / 4, cq = w % 4
//   output block   O[32qh + r32][32cq + 8(v/4) + 4h + v%4]           (as O^T)
//   state blocks   S[64qh + 32db + 8(v/4) + 4h + v%4][32cq + r32], db = 0, 1
// so the state block layout equals the accumulator layout of
// mma(K^T rows, (V ⊙ d_k)^T rows).

// S <- e^{-s m} S + K^T (V ⊙ d_k) for this wave's two state blocks.
__device__ __forceinline__ void state_update(f32x16 (&S)[2], const __bf16 *Ks, const __bf16 *Vds,
                                             float bd, int qh, int cq, int lane) {
#pragma unroll
    for (int db = 0; db < 2; ++db) S[db] *= bd;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 b = ld_op_t<L128>(Vds, 32 * cq, 16 * ks, lane);
#pragma unroll
        for (int db = 0; db < 2; ++db)
            S[db] = mma(ld_op_t<L128>(Ks, 64 * qh + 32 * db, 16 * ks, lane), b, S[db]);
    }
}

// Writes the wave's state blocks as bf16 S^T rows (value column major).
__device__ __forceinline__ void write_state_t(__bf16 *Sts, const f32x16 (&S)[2], int qh, int cq,
                                              int lane) {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int gv = 0; gv < 4; ++gv) {
            bf16x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = static_cast<__bf16>(S[db][4 * gv + r]);
            *reinterpret_cast<bf16x4 *>(Sts + L128::off(32 * cq + r32, 64 * qh + 32 * db + 8 * gv + 4 * h)) = x;
        }
}

// Output tile staging. Each wave writes its 32x32 fp32 output block into an
// LDS tile Os[64][128]; the workgroup then stores whole output rows (512 B in
// fp32) with consecutive lanes on consecutive addresses. Stored straight from
// the MFMA accumulator layout, a row would arrive in 32-byte pieces from four
// instructions, which measured at under 60% of the HBM throughput of full-row
// stores for this access pattern.
// Staged output tile: fp32 [64][128], 4-float chunks of row r permuted by
// r & 15 (writes of 16 rows of one chunk and reads of one whole row are both
// conflict-free).
__device__ __forceinline__ int ooff(int row, int col) {
    return row * D + ((((col >> 2) ^ (row & 15)) << 2) | (col & 3));
}

__device__ __forceinline__ void stage_out(float *Os, const f32x16 &o, int qh, int cq, int lane) {
    const int r32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int gv = 0; gv < 4; ++gv)
        *reinterpret_cast<float4 *>(Os + ooff(32 * qh + r32, 32 * cq + 8 * gv + 4 * hf)) =
            make_float4(o[4 * gv], o[4 * gv + 1], o[4 * gv + 2], o[4 * gv + 3]);
}

// Stores rows [0, m) of the staged tile to out (row r at out + r * ts).
template <bool FULL>
__device__ __forceinline__ void store_rows(float *out, long long ts, const float *Os, int m, int tid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
        const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
        if (FULL || row < m) stream_store(out + row * ts + col, x);
    }
}
template <bool FULL>
__device__ __forceinline__ void store_rows(__bf16 *out, long long ts, const float *Os, int m, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = (tid >> 4) + 32 * j, col = 8 * (tid & 15);
        const float4 x0 = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
        const float4 x1 = *reinterpret_cast<const float4 *>(Os + ooff(row, col + 4));
        const bf16x8 y = {static_cast<__bf16>(x0.x), static_cast<__bf16>(x0.y), static_cast<__bf16>(x0.z),
                          static_cast<__bf16>(x0.w), static_cast<__bf16>(x1.x), static_cast<__bf16>(x1.y),
                          static_cast<__bf16>(x1.z), static_cast<__bf16>(x1.w)};
        if (FULL || row < m) stream_store_bits(out + row * ts + col, y);
    }
}

struct SeqRange {
    long long start, len;
};

__device__ __forceinline__ SeqRange sequence_of(const PrefillArgs &a, int n) {
    if (a.cu_seqlens) {
        const long long T = a.total_tokens;
        long long lo = a.cu_seqlens[n], hi = a.cu_seqlens[n + 1];
        lo = lo < 0 ? 0 : (lo > T ? T : lo);
        hi = hi < lo ? lo : (hi > T ? T : hi);
        return {lo, hi - lo};
    }
    return {(long long)n * a.seqlen, a.seqlen};
}

// ---------------------------------------------------------------------------
// Segmented plans. Sequence (unit, head) is cut into `segments` segments of
// seg_len tokens; the first covered = (segments-1)*seg_len tokens are cut again
// into `pieces` pre-pass pieces of piece_len tokens (piece_len <= seg_len; both
// multiples of 128, so every piece and part of a piece is an even number of
// 64-token sub-blocks). Workspace per (unit, head), fp32 d x d states:
//   [P_0 .. P_{pieces-1}]       state of each piece's tokens from a zero state
//   [B_1 .. B_{segments-1}]     for a boundary inside a piece: the state of that
//                               piece's tokens before the boundary
//   [F]                         the final state of an in-place call
// (pairs on the warm-up route use slot 0 of theirs for the records of their
// ranges' non-finite end states, and F). The workgroups of a segment combine
// its start state from the P and B states themselves (combine_start).
// A state of tokens [t0, t1) from zero is sum_t e^{-s(t1-1-t)} k_t^T v_t, and
// states compose as S(t2) = e^{-s(t2-t1)} S(t1) + state of [t1, t2).
// Warm-up ranges. A range of a sequence that starts at token t0 > 0 computes
// its carried-in state from the last W tokens before t0 (from a zero state;
// from S_0 when the sequence starts within them), by state-only steps. A term
// of the state t tokens old carries the factor e^{-s t}, below 2^-kFixExp of
// its own scale once t > kFixExp / s2 (s2 = s log2 e): with W past that, what
// the window leaves out is under 2^-16 of its scale, 2^7 below the bf16
// rounding of the state operand of every inter-block product (the path's
// dominant error; in o the window changes a row by at most about 1e-5 relative
// on unit-variance inputs). W is rounded up to whole pairs of 64-token sub-blocks
// (with pieces starting at multiples of 128 tokens every warm-up is then an
// even number of sub-blocks, which the main kernels' warm-up steps rely on); a
// head whose W is shorter than a segment takes this route, the others the
// pre-pass. The backward's reverse pass does the same in mirrored token order
// (its carry composes like the forward state; see backward.hip).
constexpr float kFixExp = 16.f;
__device__ __forceinline__ long long warm_len(float s2) {
    if (!(s2 > 0.f)) return 1LL << 62;  // no decay (or NaN): never forgets
    const float t = kFixExp / s2;
    if (!(t < 1.0e15f)) return 1LL << 62;
    return ((long long)t + 128) / 128 * 128;
}

// Lengths of the sequences of a launch: packed (cu_seqlens, every boundary
// clamped into [0, total]) or all of one length.
struct SeqLens {
    const int *cu;
    long long total, seqlen;
    __device__ long long len(int n) const {
        if (!cu) return seqlen;
        long long lo = cu[n], hi = cu[n + 1];
        lo = lo < 0 ? 0 : (lo > total ? total : lo);
        hi = hi < lo ? lo : (hi > total ? total : hi);
        return hi - lo;
    }
};

// The plan is cut on the longest sequence (packed batches: the caller's
// max_seqlen); a sequence of `len` tokens uses its first used(len) segments
// (at least one, which also carries a zero-length sequence's state), and its
// pre-pass pieces cover the first covered(len) of its tokens. Workgroups of the
// other segments and pieces exit at once.
struct Segmented {
    int segments, pieces;
    long long seg_len, piece_len;
    __device__ int used(long long len) const {
        const long long g = (len + seg_len - 1) / seg_len;
        return g < 1 ? 1 : (g > segments ? segments : (int)g);
    }
    __device__ long long covered(long long len) const { return (long long)(used(len) - 1) * seg_len; }
    __device__ float *unit(float *ws, int uh) const {
        return ws + (size_t)uh * (size_t)(pieces + segments) * D * D;
    }
    __device__ static float *slot(float *u, long long i) { return u + (size_t)i * D * D; }
    __device__ float *piece_state(float *u, int j) const { return slot(u, j); }
    __device__ int partial_slot(int g) const { return pieces + g - 1; }
    __device__ float *partial(float *u, int g) const { return slot(u, partial_slot(g)); }
    __device__ float *final_state(float *u) const { return slot(u, pieces + segments - 1); }
};

__device__ __forceinline__ bool nonfinite(float x) {
    return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

// A 64-bit value that is the same in every lane, kept in scalar registers.
__device__ __forceinline__ long long uniform64(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}
// The same for a pointer and a float.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    return reinterpret_cast<T *>(uniform64((long long)reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ float uniformf(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
// x, opaque to the optimiser: nothing computed from it moves out of the loop
// that computes it.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Heads whose segments start from states combined from the pre-pass's; the
// others take warm-up ranges.
__device__ __forceinline__ bool takes_prepass(const Segmented &sp, float s2) {
    return !(warm_len(s2) < sp.seg_len);
}

// Warm-up route records, in slot 0 of each warm pair's workspace unit, reset by
// the pre-pass kernel (reset_records) before the main kernel runs. A range that ends at token t
// inside its pair and leaves a NaN or Inf in entry (r, c) of its end state
// (forward: S; backward: the carry R, t counted in mirrored order) records
//   ints [0, D)            per column c, the earliest such t (kNoCut: none);
//   ints [D, D + D*D/32)   one bit per state entry: non-finite in some such end
//                          state;
//   ints [kRecRowCut, +D)  per row r, the earliest such t (backward only);
//   int kFineCounter       (first warm pair only) the next fine chunk to hand out.
constexpr int kRecColCut = 0, kRecEntBad = D, kRecRowCut = D + D * D / 32, kRecInts = 2 * D + D * D / 32;
constexpr int kFineCounter = 1024;
constexpr int kNoCut = 0x7fffffff;
static_assert(kRecInts <= kFineCounter, "warm records");
__device__ __forceinline__ int *warm_records(const Segmented &sp, float *ws, int uh) {
    return reinterpret_cast<int *>(Segmented::slot(sp.unit(ws, uh), 0));
}
// Every thread of a workgroup of nt threads.
__device__ inline void reset_records(int *rec, int nt) {
    for (int i = threadIdx.x; i < kRecInts; i += nt) rec[i] = i < kRecEntBad || i >= kRecRowCut ? kNoCut : 0;
    if (threadIdx.x == 0) rec[kFineCounter] = 0;
}
// The finishing passes' NaN, and the float4 elements of a d x d state per
// thread of a workgroup.
__device__ __forceinline__ void poison(float *p) { *p = __builtin_nanf(""); }
__device__ __forceinline__ void poison(__bf16 *p) { *reinterpret_cast<uint16_t *>(p) = 0x7fc0; }
constexpr int kStateF4 = D * D / (4 * NT);
static_assert(kStateF4 * 4 * NT == D * D, "state elements per thread");

// Segmented plans have fewer than 256 (sequence, head) pairs.
constexpr int kMaxPairs = 256;

// The heads of a segmented plan split by route (each wave computes the same
// lists: 64 heads at a time by ballot, in head order).
struct Routes {
    int npre, nwarm;
};
__device__ inline Routes split_heads(const float *slopes, int heads, const Segmented &sp, short *pre,
                                     short *warm, bool write) {
    const int lane = threadIdx.x & 63;
    Routes r{0, 0};
    for (int h0 = 0; h0 < heads; h0 += 64) {
        const int h = h0 + lane;
        const bool in = h < heads;
        const bool p = in && takes_prepass(sp, slopes[in ? h : 0] * LOG2E);
        const unsigned long long bp = __ballot(p), bw = __ballot(in && !p);
        if (write) {
            const int below = lane ? __popcll(bp & (~0ull >> (64 - lane))) : 0;
            const int belw = lane ? __popcll(bw & (~0ull >> (64 - lane))) : 0;
            if (p) pre[r.npre + below] = (short)h;
            if (in && !p) warm[r.nwarm + belw] = (short)h;
        }
        r.npre += __popcll(bp);
        r.nwarm += __popcll(bw);
    }
    return r;
}

// Work of a workgroup of a segmented plan. The (unit, head) pairs of heads on
// the pre-pass route take `segments` workgroups each, one per segment: the
// first npre * units * segments workgroups, pair i of them (i / segments) the
// i-th such pair in (unit, head) order. The other pairs (the warm-up route, see
// warm_len) share the remaining workgroups in two phases.
//  * Fine chunks: about kFineFrac of the warm-up route's tokens, taken from the
//    end of the pairs whose warm-up is at most kFineWarm tokens (256 or 512
//    when fewer than kFinePairs pairs qualify at 128), nf chunks of
//    kFineChunk tokens (the forward's; the backward's kernel passes its own) from each such pair that is long enough (at most half
//    its tokens). A workgroup that has finished its range takes the next
//    chunk from a counter; chunk c is chunk c / Q of the (c % Q)-th of the Q
//    such pairs, so the chunks in flight at any time spread over the heads
//    (the rows of one head sit at the same offset of every token's row, and
//    many workgroups on a few heads stream far slower). Which chunk a
//    workgroup gets depends on timing, but where the chunks are cut does not,
//    so the result does not either; the chunks absorb the differences in speed
//    between workgroups that a static split cannot foresee (on the M1 layer
//    one head in four streams about 15% slower than the others, the same
//    heads on every call).
//  * Ranges: the rest of each pair's tokens ("bulk") is cut into ranges of
//    equal cost, one per workgroup; a range may end in one pair and go on in
//    the next. An output token costs 1 and a warm-up token warm_cost(); pair j
//    (the j-th warm pair in (unit, head) order, with B_j bulk tokens) costs
//        C_j = B_j + warm_cost * min(W_j, B_j) * B_j / T0,
//    its bulk plus the warm-ups of the about B_j / T0 cuts inside it (T0: the
//    bulk tokens per workgroup), spread evenly over its tokens; that balances
//    the ranges to first order. A workgroup's range is [r T, (r+1) T) of the
//    prefix sums of C (T = sum C / workgroups), mapped onto each pair's tokens
//    linearly and cut at multiples of 128 tokens, so neighbours agree on every
//    cut and every warm-up is an even number of 64-token sub-blocks.
// A piece that ends inside its pair with a NaN or Inf in its end state records
// them in the pair's records (warm_records), from which the finishing pass
// restores them in the later tokens.
constexpr double kFineFrac = 0.15;
constexpr long long kFineWarm = 128, kFineChunk = 768;
constexpr int kFinePairs = 16;
static_assert(kFineChunk % 128 == 0, "pieces start at multiples of 128 tokens");
struct WarmCut {
    const double *cpre;  // [nwarm pairs + 1] prefix sums of C
    double T;
    __device__ long long cut(int j, double c, long long len) const {
        const double a = cpre[j], b = cpre[j + 1];
        if (c <= a) return 0;
        if (c >= b) return len;
        long long x = (long long)((c - a) / (b - a) * (double)len) / 128 * 128;
        return x < 0 ? 0 : (x > len ? len : x);
    }
};

// Warm-route bookkeeping of a workgroup.
struct PlanState {
    double T;   // cost per workgroup
    int rl;     // this workgroup's range, counted from the first warm workgroup
    int next;   // the next pair of its range to visit (pw: none)
    int npre, nwarm, pw;
    int last;   // the last workgroup (takes every pair left)
    int nfine;     // fine chunks in all (nq pairs x nf chunks)
    int nq, nf;
    long long chunk;  // tokens per fine chunk
    int *counter;     // the fine-chunk counter
};

// Wave 0 of a workgroup computes the warm-up route's plan into LDS: cpre (the
// prefix sums of the ranges' costs, see WarmCut), bulk (each pair's bulk
// tokens), qlist and fq (the pairs that give fine chunks, their count and the
// chunks per pair). Warm pair j (j < pw < 256) is head heads_warm[j % nwarm] of
// unit j / nwarm; nwg workgroups share the ranges; a warm-up token costs wcost
// output tokens; fine chunks hold `chunk` tokens (a multiple of 128). Lane l takes pairs 4l .. 4l+3. Every workgroup computes the
// same plan (the same fp64 operations on the same inputs).
__device__ inline void warm_plan(const SeqLens &lens, const float *slopes, const short *heads_warm, int nwarm, int pw,
                                 double nwg, double wcost, long long chunk, double *cpre, long long *bulk, short *qlist,
                                 int *fq) {
    const int lane0 = threadIdx.x & 63;
    long long L[4], Wt[4], nf[4];
    double lsum = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * lane0 + i;
        L[i] = 0;
        Wt[i] = 0;
        if (j < pw) {
            L[i] = lens.len(j / nwarm);
            Wt[i] = warm_len(slopes[heads_warm[j % nwarm]] * LOG2E);
        }
        lsum += (double)L[i];
    }
    for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
    // fine chunks: kFineFrac of all warm tokens, nf from each pair that
    // qualifies (at first count) and holds at least 2 nf chunks
    // (capped at half the longest such pair, so that a large fraction
    // does not leave every pair out)
    // The pairs' warm-up bound is kFineWarm, doubled (at most twice) while
    // fewer than kFinePairs pairs would qualify: chunks from a few heads stream
    // slowly (M1 layer with its slopes scaled by 0.1: one head of 64 qualifies).
    long long fwarm = kFineWarm;
    for (int step = 0; step < 2; ++step) {
        int n = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) n += Wt[i] <= fwarm && L[i] >= 2 * chunk;
        for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
        if (n >= kFinePairs) break;
        fwarm *= 2;
    }
    int nq0 = 0;
    long long lmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (Wt[i] <= fwarm && L[i] >= 2 * chunk) {
            ++nq0;
            lmax = L[i] > lmax ? L[i] : lmax;
        }
    for (int o = 32; o >= 1; o >>= 1) {
        nq0 += __shfl_xor(nq0, o);
        const long long y = __shfl_xor(lmax, o);
        lmax = y > lmax ? y : lmax;
    }
    long long nfw = nq0 > 0 ? (long long)(kFineFrac * lsum / ((double)nq0 * (double)chunk)) : 0;
    if (nfw > lmax / (2 * chunk)) nfw = lmax / (2 * chunk);
    double bsum = 0.0;
    int nrun = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool q = nfw > 0 && Wt[i] <= fwarm && L[i] >= 2 * nfw * chunk;
        nf[i] = q ? nfw : 0;
        // bulk: the tokens before the first fine chunk (a multiple of 128)
        const long long b = q ? (L[i] - nfw * chunk) / 128 * 128 : L[i];
        const int j = 4 * lane0 + i;
        if (j < pw) bulk[j] = b;
        L[i] = b;
        bsum += (double)b;
        nrun += q;
    }
    for (int o = 32; o >= 1; o >>= 1) bsum += __shfl_xor(bsum, o);
    const double t0 = bsum / nwg;  // bulk tokens per workgroup
    double c[4], run = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double bl = (double)L[i], wl = Wt[i] < L[i] ? (double)Wt[i] : bl;
        c[i] = L[i] > 0 ? bl + wcost * wl * (bl / t0) : 0.0;
        run += c[i];
    }
    double incl = run;  // inclusive scans of the lanes' sums
    int fincl = nrun;
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o);
        const int fy = __shfl_up(fincl, o);
        if (lane0 >= o) {
            incl += y;
            fincl += fy;
        }
    }
    double acc = incl - run;
    int facc = fincl - nrun;  // qualifying pairs before this lane's
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * lane0 + i;
        if (j < pw) cpre[j] = acc;
        if (nf[i] > 0) qlist[facc++] = (short)j;
        acc += c[i];
    }
    if (lane0 == 63) {
        cpre[pw] = incl;
        fq[0] = fincl;
        fq[1] = (int)nfw;
    }
}

// Thread 0: the bookkeeping of warm workgroup rl (counted from the first warm
// workgroup) of nwg = pw * segments, from the plan above; `counter` is the
// fine-chunk counter.
__device__ inline void warm_plan_state(PlanState &ps, const double *cpre, const int *fq, int pw, int segments, int rl,
                                       long long chunk, int *counter) {
    ps.chunk = chunk;
    ps.rl = rl;
    ps.T = cpre[pw] / ((double)pw * segments);
    ps.last = rl + 1 == pw * segments;
    // the first warm pair this range reaches: the first j with cpre[j + 1] > rl T
    const double c0 = (double)rl * ps.T;
    int lo = 0, hi = pw;
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (cpre[mid + 1] > c0) hi = mid; else lo = mid + 1;
    }
    ps.next = lo;
    ps.nq = fq[0];
    ps.nf = fq[1];
    ps.nfine = ps.nq * ps.nf;
    ps.counter = counter;
}

// Tokens of segment g of a sequence of `seqlen` tokens (0 past its end).
__device__ __forceinline__ long long seg_len_at(const Segmented &sp, long long seqlen, int g) {
    const long long rest = seqlen - (long long)g * sp.seg_len;
    return rest < 0 ? 0 : (rest < sp.seg_len ? rest : sp.seg_len);
}

// A workgroup's next piece: tokens [t0, t1) of pair (sequence n, head h), of a
// sequence of len tokens (the backward counts them in mirrored order).
struct PieceRange {
    int n, h;  // n < 0: no more pieces
    int kind;  // 0 the whole pair (no segments), 1 segment g of a pre-pass pair, 2 a warm-route piece
    int g;
    long long t0, t1, len;
};
// Thread 0 walks its workgroup's plan: mode 0 (no segments; by_rank, if given,
// maps workgroup slots to sequences), 1 (a pre-pass pair's segment) or 2 (its
// range of bulk tokens, then fine chunks while any are left); k counts the
// pieces taken so far.
__device__ inline PieceRange next_range(const SeqLens &lens, int heads, const Segmented &sp, int mode, int k,
                                        PlanState &ps, const short *heads_pre, const short *heads_warm,
                                        const double *cpre, const long long *bulk, const short *qlist,
                                        const int *by_rank) {
    PieceRange r{-1, 0, 0, 0, 0, 0, 0};
    if (mode == 0) {
        if (k > 0) return r;
        r.n = blockIdx.x / heads;
        if (by_rank) r.n = by_rank[r.n];
        r.h = blockIdx.x % heads;
        r.len = r.t1 = lens.len(r.n);
        return r;
    }
    if (mode == 1) {
        if (k > 0) return r;
        const int i = blockIdx.x / sp.segments, g = blockIdx.x % sp.segments;
        const int n = i / ps.npre;
        const long long len = lens.len(n);
        if (g >= sp.used(len)) return r;
        r.n = n;
        r.h = heads_pre[i % ps.npre];
        r.kind = 1;
        r.g = g;
        r.len = len;
        r.t0 = (long long)g * sp.seg_len;
        r.t1 = r.t0 + seg_len_at(sp, len, g);
        return r;
    }
    // this workgroup's range of bulk tokens
    const WarmCut wc{cpre, ps.T};
    const double c0 = (double)ps.rl * ps.T, c1 = (double)(ps.rl + 1) * ps.T;
    while (ps.next < ps.pw) {
        const int j = ps.next;
        const long long b = bulk[j];
        const long long t0 = wc.cut(j, c0, b);
        const long long t1 = ps.last ? b : wc.cut(j, c1, b);
        ps.next = ps.last || cpre[j + 1] < c1 ? j + 1 : ps.pw;  // the range goes on into the next pair
        if (t1 <= t0) continue;
        r.n = j / ps.nwarm;
        r.h = heads_warm[j % ps.nwarm];
        r.kind = 2;
        r.len = lens.len(r.n);
        r.t0 = t0;
        r.t1 = t1;
        return r;
    }
    // then fine chunks, while any are left
    if (ps.nfine > 0) {
        const int c = atomicAdd(ps.counter, 1);
        if (c >= ps.nfine) {
            ps.nfine = 0;
            return r;
        }
        const int j = qlist[c % ps.nq], i = c / ps.nq;
        r.n = j / ps.nwarm;
        r.h = heads_warm[j % ps.nwarm];
        r.kind = 2;
        r.len = lens.len(r.n);
        r.t0 = bulk[j] + (long long)i * ps.chunk;
        r.t1 = i + 1 == ps.nf ? r.len : r.t0 + ps.chunk;
    }
    return r;
}

// Pre-pass grouping. The plan cuts the first G-1 segments of every head into
// many short pieces, which is right when few heads take the pre-pass; when
// many do, a workgroup takes k consecutive pieces of a head (writing one state,
// in the slot of the group's last piece), so that about kPrepassActive
// workgroups work and the segments' combines walk fewer, larger states. Every
// kernel derives k with this function from the count of pre-pass heads that
// split_heads gives it. A group never exceeds one segment, so it holds at most
// one segment boundary strictly inside.
// 256: the pre-pass kernel fits one workgroup per CU, so with 512 the second
// half ran in a second round (M1 layer, slopes x1e-5: 0.659 -> 0.639 ms per
// call at 256; x0.1: 0.613 -> 0.610 ms).
constexpr int kPrepassActive = 256;
__device__ inline int prepass_group_of(int npre, int units, const Segmented &sp) {
    long long k = ((long long)units * npre * sp.pieces + kPrepassActive - 1) / kPrepassActive;
    const long long kmax = sp.seg_len / sp.piece_len;
    if (k > kmax) k = kmax;
    return k < 1 ? 1 : (int)k;
}

// Start state of segment g >= 1 of a pair on the pre-pass route, in each
// thread's accumulator blocks S (wave w: rows 64(w/4).., columns 32(w%4)..;
// entry (db, v) at row 64(w/4) + 32db + 8(v/4) + 4(lane/32) + v%4, column
// 32(w%4) + lane%32, as the pre-pass stores its states), which hold the first
// state S_0 on entry: the pre-pass group states (kg pieces each; the last group
// ends at `covered`) combined in order,
//   S <- e^{-s len_j} S + P_j,
// over the groups that end at or before b = g seg_len, then, if b falls inside
// the next group j, S <- e^{-s(b - start_j)} S + B_g. A group never exceeds one
// segment, so the group holding b is the one whose partial state is B_g. The
// states are loaded kCombineBatch at a time ahead of their updates (more keep
// too many registers live in the main kernels, which then spill).
constexpr int kCombineBatch = 2;
__device__ inline void combine_start(f32x16 (&S)[2], const Segmented &sp, float *u, int g, int kg,
                                     long long covered, float s2, int qh, int cq, int lane) {
    const long long b = (long long)g * sp.seg_len, glen = (long long)kg * sp.piece_len;
    const int nfull = (int)(b / glen);                  // groups 0 .. nfull-1 end at or before b
    const int n = nfull + ((long long)nfull * glen < b);  // and the part of group nfull before b
    const int base = (64 * qh + 4 * (lane >> 5)) * D + 32 * cq + (lane & 31);
    auto src = [&](int j) {
        // group nfull ends at covered = b on the last segment (a whole group),
        // else b is strictly inside it (its partial state B_g)
        const int lp = (j + 1) * kg - 1 < sp.pieces - 1 ? (j + 1) * kg - 1 : sp.pieces - 1;
        return j < nfull || covered <= b ? sp.piece_state(u, lp) : sp.partial(u, g);
    };
    for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
        float x[kCombineBatch][32];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const float *p = src(j0 + i < n ? j0 + i : n - 1);
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) x[i][16 * db + v] = p[base + (32 * db + 8 * (v >> 2) + (v & 3)) * D];
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const int j = j0 + i;
            if (j >= n) break;
            const float f = fast_exp2(-s2 * (float)(j < nfull ? glen : b - (long long)j * glen));
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[db][v] = f * S[db][v] + x[i][16 * db + v];
        }
    }
}

}  // namespace
}  // namespace lt
