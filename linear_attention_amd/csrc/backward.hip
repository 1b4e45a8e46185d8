// Lightning Attention backward for bf16 inputs on gfx950 (MI355X): dK, dV and
// the gradient of the carried-in state, in one reverse pass per (sequence, head).
//
// Gradients of l = sum_t dO_t . o_t + <dS, S_final> (the reverse-mode
// derivative of the per-token form of MiniMax Signal Lab · M1, §03; the pages
// give no backward). With G_t = q_t^T dO_t + e^{-s} G_{t+1} (G_L adds dS):
//   dk_t = G_t v_t,  dv_t = G_t^T k_t,  dS_0 = e^{-s} G_1.
// In blocks of m tokens (positions i = 1..m) walked from the last to the
// first, with R the carry from the right (R = dS for the last block):
//   dV = [(K Q^T) ⊙ D^T] dO + diag(d_r) K R,     d_r[i] = e^{-s(m-i)}
//   dK = [(V dO^T) ⊙ D^T] Q + diag(d_r) V R^T
//   R <- e^{-s m} R + (Q ⊙ d_q)^T dO,            d_q[i] = e^{-s i}
// (D as in the forward; D^T keeps i' >= i). dQ is the forward operator on
// (dO, V, K) with S_0^T and is computed by the forward kernels.
//
// gfx950 design, mirroring the forward kernel (tiles.h):
//  * one 8-wave workgroup per (sequence, head); R lives in the MFMA
//    accumulators of the eight waves (wave w: rows 64(w/4).., columns
//    32(w%4)..) and, once per sub-block, in LDS as bf16 R^T;
//  * waves 0..5 compute the six nonzero 32x32 blocks of A = (K Q^T) ⊙ D^T and
//    B = (V dO^T) ⊙ D^T, stored transposed; wave w then produces the dV^T and
//    dK^T blocks (rows 32(w%4).., tokens 32(w/4)..): the inter product
//    (R^T K^T, R V^T) scaled by d_r, plus the intra product (dO^T A^T, Q^T B^T);
//  * the R update is the forward state update with (Q ⊙ d_q, dO) in place of
//    (K, V ⊙ d_k);
//  * sub-blocks are anchored at the end of the sequence (a short block, if
//    any, comes last and covers the first tokens);
//  * long sequences with few (sequence, head) pairs are cut into segments
//    counted from the end, with a reverse pre-pass and the forward's combine
//    kernel (see rev_piece_kernel);
//  * dV and dK are staged through LDS (in the R^T buffer and the K, V tiles,
//    free by then) and leave as whole rows; four barriers per sub-block.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "tiles.h"

namespace lt {
namespace {

// Padded row-major LDS tiles (pitch 136 for 128-wide tiles, 72 for the 64-wide
// score tiles): 16 consecutive rows start 4 banks apart, so 16-byte operand
// reads are conflict-free, and addresses stay affine in the contraction step
// (the XOR-swizzled layouts of the forward would need an address register per
// unrolled read, more than this kernel's register budget allows).
constexpr int PT = D + 8;   // pitch of the 128-wide tiles
constexpr int PS = PW + 8;  // pitch of the score tiles
using LT = LPad<PT>;
using LS = LPad<PS>;

// R^T (bf16) as the forward writes S^T, in the padded layout.
__device__ __forceinline__ void write_rt(__bf16 *Rts, const f32x16 (&R)[2], int qh, int cq, int lane) {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int gv = 0; gv < 4; ++gv) {
            bf16x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = static_cast<__bf16>(R[db][4 * gv + r]);
            *reinterpret_cast<bf16x4 *>(Rts + LT::off(32 * cq + r32, 64 * qh + 32 * db + 8 * gv + 4 * h)) = x;
        }
}

// R <- bd R + X^T Y over the sub-block (the forward's state_update, padded layout).
__device__ __forceinline__ void carry_update(f32x16 (&R)[2], const __bf16 *X, const __bf16 *Y, float bd,
                                             int qh, int cq, int lane) {
#pragma unroll
    for (int db = 0; db < 2; ++db) R[db] *= bd;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 b = ld_op_t<LT>(Y, 32 * cq, 16 * ks, lane);
#pragma unroll
        for (int db = 0; db < 2; ++db)
            R[db] = mma(ld_op_t<LT>(X, 64 * qh + 32 * db, 16 * ks, lane), b, R[db]);
    }
}

// Staged fp32 output tile [64][128] (pitch 132 floats) and its full-row stores.
constexpr int PO = D + 4;
__device__ __forceinline__ void stage_rows(float *Os, const f32x16 &o, int qh, int cq, int lane) {
    const int r32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int gv = 0; gv < 4; ++gv)
        *reinterpret_cast<float4 *>(Os + (32 * qh + r32) * PO + 32 * cq + 8 * gv + 4 * hf) =
            make_float4(o[4 * gv], o[4 * gv + 1], o[4 * gv + 2], o[4 * gv + 3]);
}
template <bool FULL>
__device__ __forceinline__ void put_rows(float *out, long long ts, const float *Os, int m, int tid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
        const float4 x = *reinterpret_cast<const float4 *>(Os + row * PO + col);
        if (FULL || row < m) stream_store(out + row * ts + col, x);
    }
}
template <bool FULL>
__device__ __forceinline__ void put_rows(__bf16 *out, long long ts, const float *Os, int m, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = (tid >> 4) + 32 * j, col = 8 * (tid & 15);
        const float4 x0 = *reinterpret_cast<const float4 *>(Os + row * PO + col);
        const float4 x1 = *reinterpret_cast<const float4 *>(Os + row * PO + col + 4);
        const bf16x8 y = {static_cast<__bf16>(x0.x), static_cast<__bf16>(x0.y), static_cast<__bf16>(x0.z),
                          static_cast<__bf16>(x0.w), static_cast<__bf16>(x1.x), static_cast<__bf16>(x1.y),
                          static_cast<__bf16>(x1.z), static_cast<__bf16>(x1.w)};
        if (FULL || row < m) stream_store_bits(out + row * ts + col, y);
    }
}

// Register staging of one sub-block for the backward: q, k, v and dO (layout
// as Stage: tokens (t/16) + 32i, elements 8(t%16)..; rows clamped into [0, m)).
struct BwdStage {
    uint4 q[2], k[2], v[2], g[2];

    __device__ void load(const uint16_t *qg, const uint16_t *kg, const uint16_t *vg,
                         const uint16_t *gg, int ts, int m, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const int row = (t < m ? t : m - 1) * ts + 8 * seg;
            q[i] = stream_load16(qg + row);
            k[i] = stream_load16(kg + row);
            v[i] = stream_load16(vg + row);
            g[i] = stream_load16(gg + row);
        }
    }

    // Q, K, V, dO row-major, and Q ⊙ d_q with d_q[t] = e^{-s(t+1)} (0 for t >= m).
    template <bool FULL>
    __device__ void store(__bf16 *Qs, __bf16 *Ks, __bf16 *Vs, __bf16 *Gs, __bf16 *Qds, int m,
                          float s2, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const bool in = FULL || t < m;
            const int off = LT::off(t, 8 * seg);
            const uint4 qq = keep_if(in, q[i]);
            *reinterpret_cast<uint4 *>(Qs + off) = qq;
            *reinterpret_cast<uint4 *>(Ks + off) = keep_if(in, k[i]);
            *reinterpret_cast<uint4 *>(Vs + off) = keep_if(in, v[i]);
            *reinterpret_cast<uint4 *>(Gs + off) = keep_if(in, g[i]);
            const float dq = in ? fast_exp2(-s2 * (float)(t + 1)) : 0.f;
            *reinterpret_cast<uint4 *>(Qds + off) = scale_bf16x8(qq, dq);
        }
    }
};

// ---------------------------------------------------------------------------
// Long sequences with few (sequence, head) pairs are split as in the forward,
// in mirrored token order (position t' = L - 1 - t): segment g covers real
// tokens [L - (g+1) seg_len, L - g seg_len) (the last one starts at 0), and the
// first (segments-1) segments from the end are cut into pre-pass pieces. In
// these coordinates the carry R composes exactly like the forward state, with
// dS in place of S_0, so the forward's combine kernel gives every segment its
// starting carry. A piece's contribution, from zero at its real end p1 back to
// its real start p0, is sum_i e^{-s(i - p0 + 1)} q_i^T dO_i: the carry update
// over the piece's sub-blocks walked backward.
struct RevStage {
    uint4 q[2], g[2];

    __device__ void load(const uint16_t *qg, const uint16_t *gg, int ts, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = ((tid >> 4) + 32 * i) * ts + 8 * seg;
            q[i] = stream_load16(qg + row);
            g[i] = stream_load16(gg + row);
        }
    }
    // Q ⊙ d_q (d_q[t] = e^{-s(t+1)}) and dO, full sub-blocks only
    __device__ void store(__bf16 *Qds, __bf16 *Gs, float s2, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const int off = L128::off(t, 8 * seg);
            *reinterpret_cast<uint4 *>(Qds + off) = scale_bf16x8(q[i], fast_exp2(-s2 * (float)(t + 1)));
            *reinterpret_cast<uint4 *>(Gs + off) = g[i];
        }
    }
};

__global__ __launch_bounds__(NT, 2) void rev_piece_kernel(BackwardArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Qds[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Gs[C * D];

    // groups of kgr pieces, numbered as in the forward pre-pass
    const int kgr = prepass_group(a.slopes, a.heads, a.units, sp);
    const int gph = (sp.pieces + kgr - 1) / kgr;
    if ((int)blockIdx.x >= a.units * a.heads * gph) return;
    const int j = (blockIdx.x % gph) * kgr;
    const int uh = blockIdx.x / gph;
    const int h = uh % a.heads, n = uh / a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    const float s2 = a.slopes[h] * LOG2E;
    if (!takes_prepass(sp, s2)) return;  // local-start segments: no pre-pass
    const int jl = j + kgr - 1 < sp.pieces - 1 ? j + kgr - 1 : sp.pieces - 1;
    // mirrored range [t0, t1) = real tokens [L - t1, L - t0)
    const long long L = a.seqlen;
    const long long t0 = j * sp.piece_len;
    const long long covered = sp.covered(L);
    const long long t1 = t0 + kgr * sp.piece_len < covered ? t0 + kgr * sp.piece_len : covered;
    const int ts = a.heads * D;
    const long long seq = (long long)n * L * a.heads;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + (seq + h) * (long long)D;
    const uint16_t *gg = static_cast<const uint16_t *>(a.dout) + (seq + h) * (long long)D;
    float *u = sp.unit(ws, uh);

    f32x16 R[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) R[db][v] = 0.f;
    auto store_state = [&](int slot) {
        asm volatile("" : "+s"(slot));
        float *dst = Segmented::slot(u, slot);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                dst[(64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + 32 * cq + r32] = R[db][v];
    };

    // sub-block k covers real tokens [L - t0 - 64(k+1), L - t0 - 64k)
    const long long nch = (t1 - t0) / C;  // even, >= 2
    const float bd = fast_exp2(-s2 * (float)C);
    RevStage st0, st1;
    auto prefetch = [&](RevStage &st, long long k) {
        // past the piece one row is read again (row stride 0; ignored), so the
        // count of loads stays fixed without a whole sub-block of traffic
        const bool in = k < nch;
        const long long kk = in ? k : nch - 1;
        const long long off = (L - t0 - C * (kk + 1)) * (long long)ts;
        st.load(qg + off, gg + off, in ? ts : 0, tid);
    };
    auto step = [&](long long k, RevStage &st) {
        __syncthreads();
        st.store(Qds, Gs, s2, tid);
        prefetch(st, k + 2);
        __syncthreads();
        state_update(R, Qds, Gs, bd, qh, cq, lane);
    };
    auto run = [&](long long k0, long long k1) {
        for (long long k = k0; k < k1; k += 2) {
            step(k, st0);
            step(k + 1, st1);
        }
    };
    prefetch(st0, 0);
    prefetch(st1, 1);
    const int gb = (int)(t0 / sp.seg_len) + 1;  // first mirrored segment boundary after t0
    const long long b = gb * sp.seg_len;
    const long long cb = b < t1 ? (b - t0) / C : nch;
    run(0, cb);
    store_state(b < t1 ? sp.partial_slot(gb) : jl);
    run(cb, nch);
    store_state(jl);
}

template <typename OutT>
__global__ __launch_bounds__(NT) void bwd_kv_kernel(BackwardArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * PT];
    __shared__ __attribute__((aligned(16))) __bf16 KVs[2][C * PT];  // K, V; dK staging (fp32)
    __shared__ __attribute__((aligned(16))) __bf16 Gs[C * PT];      // dO
    __shared__ __attribute__((aligned(16))) __bf16 Qds[C * PT];     // Q ⊙ d_q
    __shared__ __attribute__((aligned(16))) __bf16 Rts[D * PT];     // R^T; dV staging (fp32)
    __shared__ __attribute__((aligned(16))) __bf16 Ats[C * PS];     // A^T: [i'][i]
    __shared__ __attribute__((aligned(16))) __bf16 Bts[C * PS];     // B^T: [i'][i]
    static_assert(sizeof(float) * C * PO <= sizeof(__bf16) * D * PT, "dV staging fits R^T");
    static_assert(sizeof(float) * C * PO <= 2 * sizeof(__bf16) * C * PT, "dK staging fits K, V");
    __bf16 *Ks = KVs[0], *Vs = KVs[1];

    const int g = blockIdx.x % sp.segments;  // mirrored segment (0 = the end of the sequence)
    const int uh = blockIdx.x / sp.segments;
    const int h = uh % a.heads, n = uh / a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    // real tokens [seg_lo, seg_hi) of this segment
    const long long L = a.seqlen;
    const long long seg_hi = L - g * sp.seg_len;
    const long long seg_lo = seg_hi - sp.seg_len > 0 && g + 1 < sp.segments ? seg_hi - sp.seg_len : 0;
    const long long len = seg_hi - seg_lo;
    const int ts = a.heads * D;
    const long long base = (((long long)n * L + seg_lo) * a.heads + h) * (long long)D;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + base;
    const uint16_t *gg = static_cast<const uint16_t *>(a.dout) + base;
    OutT *dkg = static_cast<OutT *>(a.dk) + base;
    OutT *dvg = static_cast<OutT *>(a.dv) + base;
    const float s2 = a.slopes[h] * LOG2E;

    // ---- carry from the right of the sequence: dS (or zero)
    f32x16 R[2];
    auto sidx = [&](int db, int v) {
        return (64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + 32 * cq + r32;
    };
    // local-start segments: segment 0 (the sequence end) starts from dS, the
    // others from zero (the correction pass adds their carried-in term)
    const bool fix = sp.segments > 1 && fix_head(s2, sp.seg_len, sp.fix_osz);
    const float *r_in = sp.segments > 1 && !fix
                            ? sp.start_state(sp.unit(ws, uh), g)
                            : ((sp.segments == 1 || g == 0) && a.d_state_out ? a.d_state_out + (size_t)uh * D * D
                                                                              : nullptr);
    if (r_in) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) R[db][v] = r_in[sidx(db, v)];
    } else {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) R[db][v] = 0.f;
    }
    write_rt(Rts, R, qh, cq, lane);

    // score blocks: waves 0..2 A, waves 3..5 B; block (I, I') in {(0,0), (0,1), (1,1)}
    const bool scorer = w < 6;
    const int blk = w % 3;
    const int sI = blk == 2 ? 1 : 0, sJ = blk == 0 ? 0 : 1;  // rows i in 32sI.., columns i' in 32sJ..

    // Sub-blocks are anchored at the end of the sequence: step p < nfull covers
    // tokens [len - 64(p+1), len - 64p); a short first block [0, len mod 64),
    // if any, is the last step (the block form holds for any partition).
    const long long nfull = len / C;
    const int head_len = (int)(len - nfull * C);
    const long long nsteps = nfull + (head_len > 0);
    auto step_start = [&](long long p) { return p < nfull ? len - C * (p + 1) : 0; };
    auto step_len = [&](long long p) { return p < nfull ? C : head_len; };
    // sub-block of step p is staged in st[p % 2], loaded two steps ahead
    BwdStage st0, st1;
    auto prefetch = [&](BwdStage &st, long long p) {
        // past the start one row is read again (row stride 0; ignored), so the
        // count of loads stays fixed without a whole sub-block of traffic
        const bool in = p < nsteps;
        const long long pp = in ? p : nsteps - 1;
        const long long off = step_start(pp) * (long long)ts;
        st.load(qg + off, kg + off, vg + off, gg + off, in ? ts : 0, in ? step_len(pp) : C, tid);
    };
    if (nsteps > 0) {
        prefetch(st0, 0);
        prefetch(st1, 1);
    }

    auto step = [&](long long p, int m, auto full, BwdStage &st) {
        constexpr bool FULL = decltype(full)::value;
        const long long t0 = step_start(p);
        st.template store<FULL>(Qs, Ks, Vs, Gs, Qds, m, s2, tid);
        prefetch(st, p + 2);
        __syncthreads();  // (B) tiles and R^T visible

        if (scorer) {
            // A^T or B^T block: C[i][i'] = x_i . y_i' masked to i' >= i and decayed,
            // stored as [i'][i]
            const __bf16 *X = w < 3 ? Ks : Vs;
            const __bf16 *Y = w < 3 ? Qs : Gs;
            __bf16 *T = w < 3 ? Ats : Bts;
            f32x16 sc;
#pragma unroll
            for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                sc = mma(ld_op<LT>(X, 32 * sI, 16 * ks, lane), ld_op<LT>(Y, 32 * sJ, 16 * ks, lane), sc);
            // decay of C[i][i'], e^{-s(i' - i)} for i' >= i, recomputed every step
            // from an opaque copy of the lane: kept across the loop these 16
            // values were spilled, and each reload waited for every load in
            // flight, the prefetch of the sub-blocks ahead included
            int lo = lane;
            asm volatile("" : "+v"(lo));
            float dscore[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int diff = (32 * sJ + (lo & 31)) - (32 * sI + 8 * (v >> 2) + 4 * (lo >> 5) + (v & 3));
                dscore[v] = masked_decay(diff, s2);
            }
#pragma unroll
            for (int gv = 0; gv < 4; ++gv) {
                bf16x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[r] = static_cast<__bf16>(mask_mul(sc[4 * gv + r], dscore[4 * gv + r]));
                *reinterpret_cast<bf16x4 *>(T + LS::off(32 * sJ + r32, 32 * sI + 8 * gv + 4 * hf)) = pv;
            }
        }

        // inter products, scaled per token i = 32 qh + r32 by d_r[i] = e^{-s(m-1-i)}
        f32x16 dv, dk;
#pragma unroll
        for (int v = 0; v < 16; ++v) dv[v] = dk[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            dv = mma(ld_op<LT>(Rts, 32 * cq, 16 * ks, lane), ld_op<LT>(Ks, 32 * qh, 16 * ks, lane), dv);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            dk = mma(ld_op_t<LT>(Rts, 32 * cq, 16 * ks, lane), ld_op<LT>(Vs, 32 * qh, 16 * ks, lane), dk);
        const int ti = 32 * qh + r32;
        const float dr = ti < m ? fast_exp2(-s2 * (float)(m - 1 - ti)) : 0.f;
        dv *= dr;
        dk *= dr;

        // R <- e^{-s m} R + (Q ⊙ d_q)^T dO
        carry_update(R, Qds, Gs, fast_exp2(-s2 * (float)m), qh, cq, lane);
        __syncthreads();  // (C) A^T, B^T visible; reads of R^T, K, V, Q ⊙ d_q done

        // intra products over i' >= 32 qh
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
            if (ks < 2 * qh) continue;
            dv = mma(ld_op_t<LT>(Gs, 32 * cq, 16 * ks, lane), ld_op_t<LS>(Ats, 32 * qh, 16 * ks, lane), dv);
        }
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
            if (ks < 2 * qh) continue;
            dk = mma(ld_op_t<LT>(Qs, 32 * cq, 16 * ks, lane), ld_op_t<LS>(Bts, 32 * qh, 16 * ks, lane), dk);
        }
        float *dVs = reinterpret_cast<float *>(Rts);
        float *dKs = reinterpret_cast<float *>(KVs[0]);
        stage_rows(dVs, dv, qh, cq, lane);
        stage_rows(dKs, dk, qh, cq, lane);
        __syncthreads();  // (D) dV, dK staged
        put_rows<FULL>(dvg + t0 * (long long)ts, ts, dVs, m, tid);
        put_rows<FULL>(dkg + t0 * (long long)ts, ts, dKs, m, tid);
        __syncthreads();  // (E) staging read; R^T and the next tiles may be written
        write_rt(Rts, R, qh, cq, lane);
    };
    long long p = 0;
    for (; p + 1 < nfull; p += 2) {
        step(p, C, std::true_type{}, st0);
        step(p + 1, C, std::true_type{}, st1);
    }
    if (p < nfull) step(p++, C, std::true_type{}, st0);
    if (head_len > 0) {  // staged in st[nfull % 2]
        if (nfull & 1)
            step(p, head_len, std::false_type{}, st1);
        else
            step(p, head_len, std::false_type{}, st0);
    }

    if (fix) {  // end carry of this local-start segment, for the chain
        float *u = sp.unit(ws, uh);
        float *dst = sp.start_state(u, g);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[sidx(db, v)] = R[db][v];
        if (g + 1 < sp.segments) flag_end_state(end_flags(sp, u, g), R, w, lane);
    } else if (a.d_state_in && g == sp.segments - 1) {  // the segment holding token 0
        float *dst = a.d_state_in + (size_t)uh * D * D;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[sidx(db, v)] = R[db][v];
    }
}

// Reverse pass on local-start segments. Mirrored segment g >= 1 started from a
// zero carry instead of R_in(g), so token t of it, n = seg_hi - 1 - t tokens
// before its right end, misses e^{-s n} R_in in its gradient of S_t:
//   dv_t += e^{-s n} k_t R_in,    dk_t += e^{-s n} v_t R_in^T,
// added here for n <= kFixExp / s2 (past that the factor is below the fp32
// unit roundoff, 2^-24), in 64-token chunks counted from the right end. As in
// the forward correction, the chunks of all (unit, head, segment) pairs are
// numbered in pair order and cut into equal contiguous ranges, consecutive
// ranges on one XCD; a workgroup forms R_in(g) itself from the end carries E_j
// the main pass left (R_in(1) = E_0, R_in(j+1) = e^{-s len_j} R_in(j) + E_j)
// and loads the next chunk's rows before the current chunk's products, which
// take R_in^T (bf16, LDS) as the operand of the dv term and, through the
// transposing read, R_in for the dk term. The first `nfinal` workgroups write
// d_state_in, the final carry, of each local-start head.
constexpr int kRevFixWorkgroups = 256;  // one per CU (98 KB of LDS); a multiple of 8 (XCDs)

// Rows a thread adds to (loaded ahead of the products): fp32 rows (t/32) + 16j,
// 4 columns at 4(t%32); bf16 rows (t/16) + 32j, 8 columns at 8(t%16). `out`
// points at chunk row rlo; rows below rlo read that row and are not stored.
template <typename OutT>
struct RowsFrom;
template <>
struct RowsFrom<float> {
    uint4 y[4];
    __device__ void load(const float *out, int ts, int rlo, int tid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j;
            y[j] = *reinterpret_cast<const uint4 *>(out + (unsigned)((row > rlo ? row - rlo : 0) * ts + 4 * (tid & 31)));
        }
    }
    __device__ void add_store(float *out, int ts, const float *Os, int rlo, int tid) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
            const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
            if (row >= rlo)
                *reinterpret_cast<float4 *>(out + (unsigned)((row - rlo) * ts + col)) =
                    make_float4(__uint_as_float(y[j].x) + x.x, __uint_as_float(y[j].y) + x.y,
                                __uint_as_float(y[j].z) + x.z, __uint_as_float(y[j].w) + x.w);
        }
    }
};
template <>
struct RowsFrom<__bf16> {
    uint4 y[2];
    __device__ void load(const __bf16 *out, int ts, int rlo, int tid) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 4) + 32 * j;
            y[j] = *reinterpret_cast<const uint4 *>(out + (unsigned)((row > rlo ? row - rlo : 0) * ts + 8 * (tid & 15)));
        }
    }
    __device__ void add_store(__bf16 *out, int ts, const float *Os, int rlo, int tid) const {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 4) + 32 * j, col = 8 * (tid & 15);
            const float4 x0 = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
            const float4 x1 = *reinterpret_cast<const float4 *>(Os + ooff(row, col + 4));
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const uint32_t wv[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
            uint32_t r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 lo = static_cast<__bf16>(__uint_as_float(wv[i] << 16) + xs[2 * i]);
                const __bf16 hi = static_cast<__bf16>(__uint_as_float(wv[i] & 0xffff0000u) + xs[2 * i + 1]);
                uint16_t ulo, uhi;
                __builtin_memcpy(&ulo, &lo, 2);
                __builtin_memcpy(&uhi, &hi, 2);
                r[i] = (uint32_t)ulo | ((uint32_t)uhi << 16);
            }
            if (row >= rlo)
                *reinterpret_cast<uint4 *>(out + (unsigned)((row - rlo) * ts + col)) = make_uint4(r[0], r[1], r[2], r[3]);
        }
    }
};

template <typename OutT>
__global__ __launch_bounds__(NT) void rev_fix_kernel(BackwardArgs a, Segmented sp, float *ws, int nfinal) {
    __shared__ __attribute__((aligned(16))) __bf16 Rt[D * D];  // R_in^T
    __shared__ __attribute__((aligned(16))) __bf16 Kt[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[C * D];
    __shared__ __attribute__((aligned(16))) float Os[C * D];
    __shared__ long long first[kFixMaxPairs + 1];  // first chunk number of each pair
    __shared__ long long prows[kFixMaxPairs];       // rows corrected in each pair

    const int tid = threadIdx.x;
    const long long L = a.seqlen;
    if ((int)blockIdx.x < nfinal) {  // d_state_in of a local-start head
        const int uh = blockIdx.x / kFinalSlices;
        const float s2 = a.slopes[uh % a.heads] * LOG2E;
        if (!fix_head(s2, sp.seg_len, sp.fix_osz)) return;
        const int e = 4 * ((blockIdx.x % kFinalSlices) * NT + tid);
        float *u = sp.unit(ws, uh);
        float4 acc = *reinterpret_cast<const float4 *>(sp.start_state(u, 0) + e);
        for (int g = 1; g < sp.segments; ++g) {
            const float f = fast_exp2(-s2 * (float)seg_len_at(sp, L, g));
            const float4 x = *reinterpret_cast<const float4 *>(sp.start_state(u, g) + e);
            acc = make_float4(f * acc.x + x.x, f * acc.y + x.y, f * acc.z + x.z, f * acc.w + x.w);
        }
        *reinterpret_cast<float4 *>(a.d_state_in + (size_t)uh * D * D + e) = acc;
        return;
    }

    // rows and chunks per pair (the whole segment when its carried-in carry is
    // non-finite), then the chunks' prefix sums
    const int gs = sp.segments - 1;
    const int pairs = a.units * a.heads * gs;
    long long x = 0;
    if (tid < pairs) {
        const int g = 1 + tid % gs, uh = tid / gs;
        const float s2 = a.slopes[uh % a.heads] * LOG2E;
        long long rows = 0;
        if (fix_head(s2, sp.seg_len, sp.fix_osz)) {
            const long long len = seg_len_at(sp, L, g), fl = fix_len(s2, sp.seg_len) + 1;  // n = 0 .. fix_len
            rows = start_poisoned(sp, sp.unit(ws, uh), g) || fl > len ? len : fl;
        }
        prows[tid] = rows;
        x = (rows + C - 1) / C;
    }
    for (int off = 1; off < kFixMaxPairs; off <<= 1) {
        if (tid < kFixMaxPairs) first[tid + 1] = x;
        __syncthreads();
        if (tid < kFixMaxPairs && tid >= off) x += first[tid + 1 - off];
        __syncthreads();
    }
    if (tid < kFixMaxPairs) first[tid + 1] = x;
    if (tid == 0) first[0] = 0;
    __syncthreads();

    const long long total = uniform64(first[pairs]);
    const int nwg = gridDim.x - nfinal;
    const int r = (int)(blockIdx.x % 8) * (nwg / 8) + (int)(blockIdx.x - nfinal) / 8;
    const long long j0 = total * r / nwg, j1 = total * (r + 1) / nwg;
    if (j0 >= j1) return;

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3;
    const int ts = a.heads * D;
    struct Chunk {
        const uint16_t *k, *v;
        OutT *dk, *dv;
        long long seg_hi, tlo;
        int rlo, pair, uh, g;
        float s2;
    };
    int p = 0;
    auto chunk_at = [&](long long j) {
        while (first[p + 1] <= j) ++p;
        p = __builtin_amdgcn_readfirstlane(p);
        Chunk c;
        c.pair = p;
        c.uh = p / gs;
        c.g = 1 + p % gs;
        const int h = c.uh % a.heads, n = c.uh / a.heads;
        c.s2 = a.slopes[h] * LOG2E;
        const long long T = uniform64(prows[p]);
        c.seg_hi = L - (long long)c.g * sp.seg_len;
        const long long ci = uniform64(j - first[p]);
        c.tlo = c.seg_hi - C * (ci + 1);
        c.rlo = (int)(c.seg_hi - T - c.tlo > 0 ? c.seg_hi - T - c.tlo : 0);
        // rows below rlo are never touched: the base is the chunk's first
        // corrected row, and row offsets are taken relative to it
        const long long off = (((long long)n * L + c.tlo + c.rlo) * a.heads + h) * (long long)D;
        c.k = static_cast<const uint16_t *>(a.k) + off;
        c.v = static_cast<const uint16_t *>(a.v) + off;
        c.dk = static_cast<OutT *>(a.dk) + off;
        c.dv = static_cast<OutT *>(a.dv) + off;
        return c;
    };
    // loads of a chunk: k, v rows and the dv, dk rows (row r of the chunk at
    // offset (r - rlo) from the base; rows below rlo read row rlo)
    struct Loads {
        uint4 kx[2], vx[2];
        RowsFrom<OutT> dvr, dkr;
    };
    auto load = [&](const Chunk &c, Loads &l, int th) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = (th >> 4) + 32 * i;
            const unsigned o = (unsigned)((rr > c.rlo ? rr - c.rlo : 0) * ts + 8 * (th & 15));
            l.kx[i] = stream_load16(c.k + o);
            l.vx[i] = stream_load16(c.v + o);
        }
        l.dvr.load(c.dv, ts, c.rlo, th);
        l.dkr.load(c.dk, ts, c.rlo, th);
    };
    Chunk cur = chunk_at(j0);
    Loads la;
    load(cur, la, tid);
    int loaded = -1;
    for (long long j = j0; j < j1; ++j) {
        if (j > j0) __syncthreads();  // the previous chunk's reads of Kt, Vt, Os done
        int tl = tid;
        asm volatile("" : "+v"(tl));  // lane offsets recomputed per chunk (not spilled)
        const int ln = tl & 63;
        Chunk nxt = cur;
        Loads lb = la;
        if (j + 1 < j1) {
            nxt = chunk_at(j + 1);
            load(nxt, lb, tl);
        }
        if (cur.pair != loaded) {  // R_in(g)^T as bf16 (the last reads of Rt ended before a barrier)
            const int c = tl & (D - 1), kq = tl >> 7;
            float *u = sp.unit(ws, cur.uh);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float acc[4][4];
                {
                    const float *e = sp.start_state(u, 0) + (4 * kq + 64 * half) * D + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) acc[i][rr] = e[(16 * i + rr) * D];
                }
                for (int g = 1; g < cur.g; ++g) {
                    const float f = fast_exp2(-cur.s2 * (float)seg_len_at(sp, L, g));
                    const float *e = sp.start_state(u, g) + (4 * kq + 64 * half) * D + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) acc[i][rr] = f * acc[i][rr] + e[(16 * i + rr) * D];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x4 y;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) y[rr] = static_cast<__bf16>(acc[i][rr]);
                    *reinterpret_cast<bf16x4 *>(Rt + L128::off(c, 4 * (kq + 4 * i) + 64 * half)) = y;
                }
            }
            loaded = cur.pair;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = (tl >> 4) + 32 * i;
            *reinterpret_cast<uint4 *>(Kt + L128::off(rr, 8 * (tl & 15))) = keep_if(rr >= cur.rlo, la.kx[i]);
            *reinterpret_cast<uint4 *>(Vt + L128::off(rr, 8 * (tl & 15))) = keep_if(rr >= cur.rlo, la.vx[i]);
        }
        __syncthreads();  // K, V tiles and R_in^T visible
        f32x16 odv, odk;
#pragma unroll
        for (int v = 0; v < 16; ++v) odv[v] = odk[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            odv = mma(ld_op<L128>(Rt, 32 * cq, 16 * ks, ln), ld_op<L128>(Kt, 32 * qh, 16 * ks, ln), odv);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            odk = mma(ld_op_t<L128>(Rt, 32 * cq, 16 * ks, ln), ld_op<L128>(Vt, 32 * qh, 16 * ks, ln), odk);
        const float f = fast_exp2(-cur.s2 * (float)(cur.seg_hi - 1 - (cur.tlo + 32 * qh + (ln & 31))));
        odv *= f;
        odk *= f;
        stage_out(Os, odv, qh, cq, ln);
        __syncthreads();  // dv rows staged
        la.dvr.add_store(cur.dv, ts, Os, cur.rlo, tl);
        __syncthreads();  // Os read
        stage_out(Os, odk, qh, cq, ln);
        __syncthreads();  // dk rows staged
        la.dkr.add_store(cur.dk, ts, Os, cur.rlo, tl);
        cur = nxt;
        la = lb;
    }
}

template <typename OutT>
hipError_t launch(const BackwardArgs &a, const PrefillPlan &p, void *workspace, hipStream_t stream) {
    clear_pending_error();
    const long long uh = (long long)a.units * a.heads;
    float *ws = static_cast<float *>(workspace);
    const bool seg = p.segments > 1 && p.value_slices == 1;
    // heads may take local-start segments (fix_head's rule). The correction moves
    // k, v once and dk, dv read and written, 512 (1 + sizeof(OutT)) B per token,
    // against the reverse pre-pass's q, dO re-read, 512 B per token. fix_head
    // weighs a correction token at 256 (1 + osz) B; osz = 1 + sizeof(OutT) counts
    // it at 60-67% of that traffic, because the reverse pre-pass of the few heads
    // that would still need it runs far below the correction's bandwidth (M1
    // layer: with the exact weight the 3 slowest-decay heads take the pre-pass,
    // 1.430 ms per call; with this one all 64 heads correct, 1.418 ms)
    const int fix_osz = seg ? 1 + (int)sizeof(OutT) : 0;
    const Segmented sp = seg ? Segmented{p.segments, p.pieces, p.seg_len, p.piece_len, fix_osz}
                             : Segmented{1, 0, a.seqlen, 0};
    if (seg) {
        hipLaunchKernelGGL(rev_piece_kernel, dim3((unsigned)(uh * p.pieces)), dim3(NT), 0, stream, a,
                           sp, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(uh * kCombineSlices)), dim3(kCombineThreads),
                           0, stream, a.slopes, a.heads, a.d_state_out, false, sp,
                           SeqLens{nullptr, (long long)a.units * a.seqlen, a.seqlen}, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_kv_kernel<OutT>), dim3((unsigned)(uh * sp.segments)), dim3(NT), 0, stream,
                       a, sp, ws);
    if (!fix_osz) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (uh * (sp.segments - 1) > kFixMaxPairs) return hipErrorInvalidValue;  // not a segmented plan
    const int nfinal = a.d_state_in ? (int)(uh * kFinalSlices) : 0;
    hipLaunchKernelGGL((rev_fix_kernel<OutT>), dim3((unsigned)(nfinal + kRevFixWorkgroups)), dim3(NT), 0, stream,
                       a, sp, ws, nfinal);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_kv(const BackwardArgs &a, const PrefillPlan &plan, void *workspace,
                              lt_dtype out_dtype, hipStream_t stream) {
    return out_dtype == LT_F32 ? launch<float>(a, plan, workspace, stream)
                               : launch<__bf16>(a, plan, workspace, stream);
}

}  // namespace lt
