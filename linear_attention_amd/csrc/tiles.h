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

__device__ __forceinline__ uint4 stream_load16(const uint16_t *p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 stream_load8(const uint16_t *p) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void stream_store(float *p, float4 x) {
    __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4 *>(p));
}
template <class V>
__device__ __forceinline__ void stream_store_bits(__bf16 *p, const V &x) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "16- or 8-byte stores");
    if constexpr (sizeof(V) == 16) {
        u32x4 b;
        __builtin_memcpy(&b, &x, 16);
        __builtin_nontemporal_store(b, reinterpret_cast<u32x4 *>(p));
    } else {
        u32x2 b;
        __builtin_memcpy(&b, &x, 8);
        __builtin_nontemporal_store(b, reinterpret_cast<u32x2 *>(p));
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
//   [S_0 .. S_{segments-1}]     state at the start of each segment
// (pairs on the forward's warm-up route use slots 0 .. segments + 1 of theirs
// instead: end states and flags of warm ranges, and an in-place final state).
// A state of tokens [t0, t1) from zero is sum_t e^{-s(t1-1-t)} k_t^T v_t, and
// states compose as S(t2) = e^{-s(t2-t1)} S(t1) + state of [t1, t2).
// Local-start segments (the reverse pass of the backward). A segment that
// starts from a zero state instead of its true start state S_in misses, at its token t (t = 0, 1, ...), the term
// e^{-s(t+1)} q_t S_in. With s2 = s log2(e) that factor is below 2^-kFixExp once
// t + 1 > kFixExp / s2: a correction pass adds the term to the first
// fix_len = min(segment, kFixExp / s2) tokens and leaves the rest: past them
// the term is below 2^-24 of its own scale at the segment start, the unit
// roundoff of fp32 (and 2^15 times below the rounding of the bf16 operands
// every product of the path already carries). A head takes this
// route when its decay cuts the term off inside the segment and re-reading q
// and o for fix_len tokens costs at most twice the HBM traffic of the pre-pass
// re-read of the whole segment's k and v:
//   fix_len < seg_len  and  fix_len (256 + 256 osz) <= 2 * 512 seg_len
// (osz: bytes per output element; q read once, o read and written). The factor
// 2 is measured: the pre-pass of the few heads that still need it runs far
// below the bandwidth the correction pass reaches, and the pre-pass and combine
// launches are dependent steps ahead of the main kernel (M1 layer, 64 heads,
// 32,768 tokens, with a 2^-32 cutoff: with factor 1, 57 heads correct and 7
// take the pre-pass, 0.574 ms; with factor 2 all 64 correct, 0.557 ms).
constexpr float kFixExp = 24.f;
__device__ __forceinline__ long long fix_len(float s2, long long seg_len) {
    const float t = kFixExp / s2;
    return t >= (float)seg_len ? seg_len : (long long)t;
}
__device__ __forceinline__ bool fix_head(float s2, long long seg_len, int osz) {
    if (osz <= 0 || !(s2 > 0.f)) return false;
    const long long n = fix_len(s2, seg_len);
    return n < seg_len && n * (1 + osz) <= 4 * seg_len;
}

// Warm-up segments (the forward). A range of a sequence that starts at token
// t0 > 0 computes its carried-in state from the last W tokens before t0 (from a
// zero state; from S_0 when the sequence starts within them), by state-only
// steps: the terms older than W tokens are below 2^-kFixExp of their scale, as
// with the correction above, but no output needs a second pass. W is rounded up
// to whole pairs of 64-token sub-blocks (with pieces starting at multiples of
// 128 tokens every warm-up is then an even number of sub-blocks, which the main
// kernel's warm-up steps rely on); a head whose W is shorter than a segment
// takes this route, the others the pre-pass.
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
    int fix_osz = 0;    // local-start segments with a correction pass (the backward): output element size
    bool warm = false;  // warm-up segments (the forward): see warm_len
    __device__ int used(long long len) const {
        const long long g = (len + seg_len - 1) / seg_len;
        return g < 1 ? 1 : (g > segments ? segments : (int)g);
    }
    __device__ long long covered(long long len) const { return (long long)(used(len) - 1) * seg_len; }
    __device__ float *unit(float *ws, int uh) const {
        return ws + (size_t)uh * (size_t)(pieces + 2 * segments - 1) * D * D;
    }
    __device__ static float *slot(float *u, long long i) { return u + (size_t)i * D * D; }
    __device__ float *piece_state(float *u, int j) const { return slot(u, j); }
    __device__ int partial_slot(int g) const { return pieces + g - 1; }
    __device__ float *partial(float *u, int g) const { return slot(u, partial_slot(g)); }
    __device__ float *start_state(float *u, int g) const { return slot(u, pieces + segments - 1 + g); }
};

// Non-finite carried-in states (local-start segments). The correction's cutoff
// is sound only for a finite S_in: e^{-s(t+1)} q_t S_in is then below 2^-24 of
// its scale past fix_len tokens, but a NaN or Inf in S_in reaches every later
// token of the exact operator. So the main pass flags each local-start segment whose end
// state E_g holds a NaN or Inf, and the correction pass treats the whole of
// segment g as "first tokens" when any of E_0 .. E_{g-1} is flagged (S_in(g)
// is then non-finite). The flags of E_g (g <= segments - 2) sit in the slot
// of the partial state B_{g+1}, which heads on local starts never use: one int
// per wave of the segment's workgroup.
__device__ __forceinline__ bool nonfinite(float x) {
    return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}
__device__ __forceinline__ int *end_flags(const Segmented &sp, float *u, int g) {
    return reinterpret_cast<int *>(sp.partial(u, g + 1));
}
// Wave w's flag of its accumulator blocks of E_g.
__device__ __forceinline__ void flag_end_state(int *flags, const f32x16 (&S)[2], int w, int lane) {
    bool bad = false;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) bad |= nonfinite(S[db][v]);
    const bool any = __ballot(bad) != 0;
    if (lane == 0) flags[w] = any ? 1 : 0;
}
// S_in(g) non-finite: some E_j, j < g, flagged.
__device__ __forceinline__ bool start_poisoned(const Segmented &sp, float *u, int g) {
    int bad = 0;
    for (int j = 0; j < g; ++j) {
        const int *f = end_flags(sp, u, j);
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) bad |= f[w];
    }
    return bad != 0;
}

// Correction passes: (unit, head, segment g >= 1) pairs of a segmented plan
// (fewer than 256), and the final-state slices (4 elements per thread).
constexpr int kFixMaxPairs = 256;                  // segmented plans have fewer (unit, head, g >= 1) pairs
constexpr int kFinalSlices = D * D / (4 * NT);     // 4 state elements per thread

// A 64-bit value that is the same in every lane, kept in scalar registers.
__device__ __forceinline__ long long uniform64(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// Heads whose segments start from states the pre-pass and combine compute; the
// others take local-start segments (the backward) or warm-up segments (the
// forward).
__device__ __forceinline__ bool takes_prepass(const Segmented &sp, float s2) {
    if (sp.warm) return !(warm_len(s2) < sp.seg_len);
    return !fix_head(s2, sp.seg_len, sp.fix_osz);
}

// Warm-up route records, in slot 0 of each warm pair's workspace unit, reset by
// the combine pass before the main kernel runs:
//   ints [0, D)           per value column c, the earliest token t at which a
//                         range ending at t left a non-finite end state with a
//                         NaN or Inf in column c (kNoCut: none);
//   ints [D, D + D*D/32)  one bit per state entry: non-finite in some such end
//                         state;
//   int kFineCounter      (first warm pair only) the next fine chunk to hand out.
// Slot 1 holds the pair's final state on in-place calls.
constexpr int kRecColCut = 0, kRecEntBad = D, kRecInts = D + D * D / 32, kFineCounter = 1024;
constexpr int kNoCut = 0x7fffffff;
static_assert(kRecInts <= kFineCounter, "warm records");
__device__ __forceinline__ int *warm_records(const Segmented &sp, float *ws, int uh) {
    return reinterpret_cast<int *>(Segmented::slot(sp.unit(ws, uh), 0));
}

// Tokens of segment g of a sequence of `seqlen` tokens (0 past its end).
__device__ __forceinline__ long long seg_len_at(const Segmented &sp, long long seqlen, int g) {
    const long long rest = seqlen - (long long)g * sp.seg_len;
    return rest < 0 ? 0 : (rest < sp.seg_len ? rest : sp.seg_len);
}

// Pre-pass grouping. The plan cuts the first G-1 segments of every head into
// many short pieces, which is right when few heads take the pre-pass; when
// many do, a workgroup takes k consecutive pieces of a head (writing one state,
// in the slot of the group's last piece), so that about kPrepassActive
// workgroups work and the combine walks fewer, larger states. Every kernel
// derives k from the slopes with this function (each wave counts the heads on
// the pre-pass itself, 64 at a time by ballot, so no barrier is needed). A
// group never exceeds one segment, so it holds at most one segment boundary
// strictly inside.
constexpr int kPrepassActive = 512;
__device__ inline int prepass_group_of(int npre, int units, const Segmented &sp) {
    long long k = ((long long)units * npre * sp.pieces + kPrepassActive - 1) / kPrepassActive;
    const long long kmax = sp.seg_len / sp.piece_len;
    if (k > kmax) k = kmax;
    return k < 1 ? 1 : (int)k;
}
__device__ inline int prepass_group(const float *slopes, int heads, int units, const Segmented &sp) {
    const int lane = threadIdx.x & 63;
    int npre = 0;
    for (int h0 = 0; h0 < heads; h0 += 64) {
        const int h = h0 + lane;
        npre += __popcll(__ballot(h < heads && takes_prepass(sp, slopes[h < heads ? h : 0] * LOG2E)));
    }
    return prepass_group_of(__builtin_amdgcn_readfirstlane(npre), units, sp);
}

// Combine pass: the state at every segment start, S_0 being the first state
// (the carried-in state, or zero). Workgroup (unit, head, 1024-element slice) walks the pieces
// (groups of pieces, above) in order with 4 elements per thread:
//   acc <- e^{-s len_j} acc + P_j,
// and at each boundary b_g: S_g = acc if b_g ends group j, or
// e^{-s(b_g - start_j)} acc + B_g if it falls inside group j.
constexpr int kCombineThreads = 256;
constexpr int kCombineSlices = D * D / (4 * kCombineThreads);

// s0: [units, heads, d, d] first state (null: zero); s0_t: given transposed.
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *slopes, int heads,
                                                                   const float *s0, bool s0_t,
                                                                   Segmented sp, SeqLens sl, float *ws) {
    const int uh = blockIdx.x / kCombineSlices;
    const int e = 4 * ((blockIdx.x % kCombineSlices) * kCombineThreads + threadIdx.x);
    const int h = uh % heads;
    const float s2 = slopes[h] * LOG2E;
    if (!takes_prepass(sp, s2)) {  // local-start or warm-up segments: no pre-pass states
        if (sp.warm && blockIdx.x % kCombineSlices == 0) {  // reset the warm-up route's records
            int *rec = warm_records(sp, ws, uh);
            for (int i = threadIdx.x; i < kRecInts; i += kCombineThreads) rec[i] = i < kRecEntBad ? kNoCut : 0;
            if (threadIdx.x == 0) rec[kFineCounter] = 0;
        }
        return;
    }
    float *u = sp.unit(ws, uh);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s0) {
        const float *si = s0 + (size_t)uh * D * D;
        if (s0_t) {  // element (r, c) at c * D + r
            const int r = e / D, c = e % D;
            acc = make_float4(si[c * D + r], si[(c + 1) * D + r], si[(c + 2) * D + r], si[(c + 3) * D + r]);
        } else {
            acc = *reinterpret_cast<const float4 *>(si + e);
        }
    }
    *reinterpret_cast<float4 *>(sp.start_state(u, 0) + e) = acc;
    const long long covered = sp.covered(sl.len(uh / heads));
    const int kg = prepass_group(slopes, heads, (int)(gridDim.x / kCombineSlices) / heads, sp);
    const int groups = (int)((covered + kg * sp.piece_len - 1) / (kg * sp.piece_len));
    auto last_piece = [&](int j) { return (j + 1) * kg - 1 < sp.pieces - 1 ? (j + 1) * kg - 1 : sp.pieces - 1; };
    // the group states are independent loads: issue a batch of them ahead of
    // the sequential accumulation (this kernel never writes piece slots)
    constexpr int kBatch = 8;
    for (int j0 = 0; j0 < groups; j0 += kBatch) {
        float4 pj[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (j0 + i < groups) pj[i] = *reinterpret_cast<const float4 *>(sp.piece_state(u, last_piece(j0 + i)) + e);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int j = j0 + i;
            if (j >= groups) break;
            const long long t0 = (long long)j * kg * sp.piece_len;
            const long long t1 = t0 + kg * sp.piece_len < covered ? t0 + kg * sp.piece_len : covered;
            const int gb = (int)(t0 / sp.seg_len) + 1;
            const long long b = gb * sp.seg_len;
            if (b < t1) {
                const float f = fast_exp2(-s2 * (float)(b - t0));
                const float4 p = *reinterpret_cast<const float4 *>(sp.partial(u, gb) + e);
                *reinterpret_cast<float4 *>(sp.start_state(u, gb) + e) =
                    make_float4(f * acc.x + p.x, f * acc.y + p.y, f * acc.z + p.z, f * acc.w + p.w);
            }
            const float f = fast_exp2(-s2 * (float)(t1 - t0));
            const float4 p = pj[i];
            acc = make_float4(f * acc.x + p.x, f * acc.y + p.y, f * acc.z + p.z, f * acc.w + p.w);
            if (t1 % sp.seg_len == 0)
                *reinterpret_cast<float4 *>(sp.start_state(u, (int)(t1 / sp.seg_len)) + e) = acc;
        }
    }
}

}  // namespace
}  // namespace lt
