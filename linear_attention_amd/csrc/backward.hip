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
//  * long sequences with few (sequence, head) pairs are split like the
//    forward's, counted from the end (see rev_piece_kernel);
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
// tokens [L - (g+1) seg_len, L - g seg_len) (the last one starts at 0). In
// these coordinates the carry R composes exactly like the forward state, with
// dS in place of S_0, so the forward's two routes carry over:
//  * pre-pass heads: the first (segments-1) segments from the end are cut into
//    pieces; a piece's contribution, from zero at its real end p1 back to its
//    real start p0, is sum_i e^{-s(i - p0 + 1)} q_i^T dO_i (the carry update
//    over the piece's sub-blocks walked backward), and each segment's
//    workgroup combines its starting carry from them (combine_start);
//  * the other heads: warm-up ranges balanced by cost, then fine chunks (the
//    forward's plan, tiles.h), each rebuilding its starting carry by carry-only
//    steps over the q, dO rows of the W tokens after its real end (from zero;
//    from dS when the window reaches the end of the sequence).
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
    // Q ⊙ d_q (d_q[t] = e^{-s(t+1)}) and dO in layout Lay, full sub-blocks only
    template <typename Lay>
    __device__ void store(__bf16 *Qds, __bf16 *Gs, float s2, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const int off = Lay::off(t, 8 * seg);
            *reinterpret_cast<uint4 *>(Qds + off) = scale_bf16x8(q[i], fast_exp2(-s2 * (float)(t + 1)));
            *reinterpret_cast<uint4 *>(Gs + off) = g[i];
        }
    }
};

__global__ __launch_bounds__(NT, 2) void rev_piece_kernel(BackwardArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Qds[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Gs[C * D];
    __shared__ short heads_pre[kMaxPairs], heads_warm[kMaxPairs];

    // workgroup b < units * heads first resets the records of pair b if that
    // pair takes warm-up ranges
    if ((int)blockIdx.x < a.units * a.heads && !takes_prepass(sp, a.slopes[blockIdx.x % a.heads] * LOG2E))
        reset_records(warm_records(sp, ws, blockIdx.x), NT);

    // groups of kgr pieces, numbered as in the forward pre-pass: workgroup b
    // takes group b % gph of the (b / gph)-th pre-pass pair (the launch is
    // sized for at most kPrepassActive + units * heads working workgroups)
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Routes rt = split_heads(a.slopes, a.heads, sp, heads_pre, heads_warm, w == 0);
    if (rt.npre == 0) return;  // every head on warm-up ranges
    const int kgr = prepass_group_of(rt.npre, a.units, sp);
    const int gph = (sp.pieces + kgr - 1) / kgr;
    if ((int)blockIdx.x >= a.units * rt.npre * gph) return;
    __syncthreads();  // wave 0's head lists are visible
    const int j = (blockIdx.x % gph) * kgr;
    const int i = blockIdx.x / gph;
    const int n = i / rt.npre, h = heads_pre[i % rt.npre];
    const int uh = n * a.heads + h;
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    const float s2 = a.slopes[h] * LOG2E;
    const int jl = j + kgr - 1 < sp.pieces - 1 ? j + kgr - 1 : sp.pieces - 1;
    // mirrored range [t0, t1) = real tokens [L - t1, L - t0)
    const long long L = a.seqlen;
    const long long t0 = j * sp.piece_len;
    const long long covered = sp.covered(L);
    if (t0 >= covered) return;
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
        st.store<L128>(Qds, Gs, s2, tid);
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

// Warm-up cost of a token against an output token of the reverse pass. By
// bytes a warm-up token moves its q and dO rows (2 x 256 B) against the q, k,
// v, dO rows and the dk, dv rows of an output token; the warm-up's steps run
// below the streaming rate by the forward's factor.
// Tokens per fine chunk of the reverse pass.
constexpr long long kBwdFineChunk = 768;
static_assert(kBwdFineChunk % 128 == 0, "pieces start at multiples of 128 tokens");

template <typename OutT>
__device__ constexpr double bwd_warm_cost() {
    return 1.25 * 512.0 / (1024.0 + 256.0 * sizeof(OutT));
}

// A workgroup's current piece (thread 0 lays it out for the others): rows of
// the piece's first real token, the warm-up's rows (those of the real token
// just past the piece), its length, the carried-in carry and where the end
// carry goes.
struct BwdPiece {
    const uint16_t *q, *k, *v, *g;
    void *dk, *dv;
    const uint16_t *qw, *gw;
    const float *r_in;    // carried-in carry (nullptr: zero)
    float *dst;           // end == 1: d_state_in
    int *rec;             // end == 2: the pair's records
    float *u;             // comb_g > 0: the pair's workspace unit
    long long covered;    // comb_g > 0: the pair's pre-pass tokens
    long long len, warm;  // tokens of the piece; warm-up tokens (whole sub-blocks)
    float s2;
    int ts;
    int uh;   // -1: no more pieces
    int cut;  // end == 2: the mirrored token the piece ends at
    int end;  // 0 nothing, 1 d_state_in, 2 records if the end carry is non-finite
    int comb_g;  // > 0: mirrored segment comb_g of a pre-pass pair, whose start carry the piece combines
    int kg;      // comb_g > 0: pre-pass pieces per group
};

template <typename OutT>
__device__ BwdPiece next_bwd_piece(const BackwardArgs &a, const Segmented &sp, float *ws, int mode, int k,
                                   PlanState &ps, const short *heads_pre, const short *heads_warm,
                                   const double *cpre, const long long *bulk, const short *qlist) {
    const long long L = a.seqlen;
    const PieceRange r = next_range(SeqLens{nullptr, (long long)a.units * L, L}, a.heads, sp, mode, k, ps,
                                    heads_pre, heads_warm, cpre, bulk, qlist, nullptr);
    BwdPiece p{};
    p.uh = -1;
    if (r.n < 0) return p;
    p.uh = r.n * a.heads + r.h;
    p.ts = a.heads * D;
    p.s2 = a.slopes[r.h] * LOG2E;
    // mirrored [t0, t1) = real [L - t1, L - t0)
    const long long row0 = (((long long)r.n * L + (L - r.t1)) * a.heads + r.h) * (long long)D;
    const long long roww = (((long long)r.n * L + (L - r.t0)) * a.heads + r.h) * (long long)D;
    p.q = static_cast<const uint16_t *>(a.q) + row0;
    p.k = static_cast<const uint16_t *>(a.k) + row0;
    p.v = static_cast<const uint16_t *>(a.v) + row0;
    p.g = static_cast<const uint16_t *>(a.dout) + row0;
    p.dk = static_cast<OutT *>(a.dk) + row0;
    p.dv = static_cast<OutT *>(a.dv) + row0;
    p.qw = static_cast<const uint16_t *>(a.q) + roww;
    p.gw = static_cast<const uint16_t *>(a.dout) + roww;
    p.len = r.t1 - r.t0;
    const size_t sb = (size_t)p.uh * D * D;
    const float *ds = a.d_state_out ? a.d_state_out + sb : nullptr;
    if (r.kind == 0) {
        p.r_in = ds;
    } else if (r.kind == 1) {  // dS, then the combine of the pieces after the segment
        p.r_in = ds;
        p.u = sp.unit(ws, p.uh);
        p.comb_g = r.g;
        p.kg = prepass_group_of(ps.npre, a.units, sp);
        p.covered = sp.covered(L);
    } else {
        const long long wl = warm_len(p.s2);
        const long long t0w = r.t0 > wl ? r.t0 - wl : 0;
        p.warm = r.t0 - t0w;
        if (t0w == 0) p.r_in = ds;  // the warm-up starts at the end of the sequence: exact
    }
    if (r.kind == 2 && r.t1 < L) {
        p.rec = warm_records(sp, ws, p.uh);
        p.cut = (int)r.t1;
        p.end = 2;
    } else if (r.t1 >= L && a.d_state_in) {
        p.dst = a.d_state_in + sb;
        p.end = 1;
    }
    return p;
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
    __shared__ double cpre[kMaxPairs + 1];
    __shared__ long long bulk[kMaxPairs];
    __shared__ short qlist[kMaxPairs];  // pairs that give fine chunks
    __shared__ int fq[2];               // their count, chunks per pair
    __shared__ short heads_pre[kMaxPairs], heads_warm[kMaxPairs];
    __shared__ PlanState ps;
    __shared__ BwdPiece pc;
    __shared__ __attribute__((aligned(16))) unsigned char args_lds[sizeof(BackwardArgs)];
    __shared__ __attribute__((aligned(16))) unsigned char sp_lds[sizeof(Segmented)];
    __shared__ float *ws_lds;
    __bf16 *Ks = KVs[0], *Vs = KVs[1];

    const int segments = sp.segments;
    // thread indices of the set-up (each piece recomputes its own, below)
    const int t0id = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t0id >> 6);
    if (t0id == 0) {
        *reinterpret_cast<BackwardArgs *>(args_lds) = a;
        *reinterpret_cast<Segmented *>(sp_lds) = sp;
        ws_lds = ws;
    }

    // ---- this workgroup's work: pieces (pair uh, mirrored tokens [t0, t1)),
    // each starting from dS (combined with the pre-pass's carries of the later
    // tokens on the pre-pass route), zero, and a warm-up
    int mode = 0;  // 0: one pair, whole (no segments); 1: one pre-pass segment; 2: warm ranges
    if (segments > 1) {
        const Routes rt = split_heads(a.slopes, a.heads, sp, heads_pre, heads_warm, w == 0);
        __syncthreads();  // wave 0's head lists are visible
        const long long pre_wgs = (long long)a.units * rt.npre * segments;
        mode = (long long)blockIdx.x < pre_wgs ? 1 : 2;
        const int pw = a.units * rt.nwarm;  // warm pairs
        if (mode == 2 && w == 0)
            warm_plan(SeqLens{nullptr, (long long)a.units * a.seqlen, a.seqlen}, a.slopes, heads_warm, rt.nwarm,
                      pw, (double)pw * segments, bwd_warm_cost<OutT>(), kBwdFineChunk, cpre, bulk, qlist, fq);
        __syncthreads();  // cpre, bulk, qlist and fq are visible
        if (t0id == 0) {
            ps.npre = rt.npre;
            ps.nwarm = rt.nwarm;
            ps.pw = pw;
            if (mode == 2)
                warm_plan_state(ps, cpre, fq, pw, segments, (int)((long long)blockIdx.x - pre_wgs), kBwdFineChunk,
                                warm_records(sp, ws, heads_warm[0]) + kFineCounter);  // in the first warm pair's records
        }
    }

    // ---- the pieces
    f32x16 R[2];
    for (int k = 0;; ++k) {
        // the thread index is made opaque once per piece (lane-dependent
        // addresses are recomputed in each piece instead of staying in
        // registers through every piece's warm-up and set-up)
        const int tid = opaque((int)threadIdx.x), lane = tid & 63;
        const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;
        auto sidx = [&](int db, int v) {
            return (64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + 32 * cq + r32;
        };
        __syncthreads();  // the previous piece is done with the tiles, R^T and pc
        if (tid == 0)
            pc = next_bwd_piece<OutT>(*reinterpret_cast<const BackwardArgs *>(args_lds),
                                      *reinterpret_cast<const Segmented *>(sp_lds), ws_lds, mode, k, ps, heads_pre,
                                      heads_warm, cpre, bulk, qlist);
        __syncthreads();
        const int uh = __builtin_amdgcn_readfirstlane(pc.uh);
        if (uh < 0) break;
        const int ts = __builtin_amdgcn_readfirstlane(pc.ts);
        const float s2 = uniformf(pc.s2);
        const float *r_in = uniform_ptr(pc.r_in);
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
        const int comb_g = __builtin_amdgcn_readfirstlane(pc.comb_g);
        if (comb_g > 0)
            combine_start(R, *reinterpret_cast<const Segmented *>(sp_lds), uniform_ptr(pc.u), comb_g,
                          __builtin_amdgcn_readfirstlane(pc.kg), uniform64(pc.covered), s2, qh, cq, lane);
        const long long len = uniform64(pc.len), warm = uniform64(pc.warm);
        const uint16_t *qg = uniform_ptr(pc.q), *kg = uniform_ptr(pc.k), *vg = uniform_ptr(pc.v);
        const uint16_t *gg = uniform_ptr(pc.g);
        OutT *dkg = static_cast<OutT *>(uniform_ptr(pc.dk));
        OutT *dvg = static_cast<OutT *>(uniform_ptr(pc.dv));

        // score blocks: waves 0..2 A, waves 3..5 B; block (I, I') in {(0,0), (0,1), (1,1)}
        const bool scorer = w < 6;
        const int blk = w % 3;
        const int sI = blk == 2 ? 1 : 0, sJ = blk == 0 ? 0 : 1;  // rows i in 32sI.., columns i' in 32sJ..

        // Sub-blocks are anchored at the real end of the piece: step p < nfull
        // covers tokens [len - 64(p+1), len - 64p); a short first block
        // [0, len mod 64), if any, is the last step (only the piece that holds
        // token 0 has one; the block form holds for any partition).
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
        if (warm > 0) {
            // carry-only steps over the warm-up rows, from the last of them
            // down (an even number of whole sub-blocks), with their own stages
            const uint16_t *qw = uniform_ptr(pc.qw), *gw = uniform_ptr(pc.gw);
            const long long nw = warm / C;
            const float bdw = fast_exp2(-s2 * (float)C);
            RevStage w0, w1;
            auto wpre = [&](RevStage &st, long long c) {
                const long long off = (warm - C * (c + 1)) * (long long)ts;
                st.load(qw + off, gw + off, ts, tid);
            };
            auto wstep = [&](RevStage &st, auto &&issue) {
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                st.store<LT>(Qds, Gs, s2, tid);
                issue();
                __syncthreads();
                carry_update(R, Qds, Gs, bdw, qh, cq, lane);
            };
            wpre(w0, 0);
            wpre(w1, 1);
            long long c = 0;
            for (; c + 2 < nw; c += 2) {
                wstep(w0, [&] { wpre(w0, c + 2); });
                wstep(w1, [&] { wpre(w1, c + 3); });
            }
            // the last two warm-up steps issue the first two sub-blocks' loads
            wstep(w0, [&] { prefetch(st0, 0); });
            wstep(w1, [&] { prefetch(st1, 1); });
            __syncthreads();  // the last warm-up reads of Qds, Gs are done
        } else if (nsteps > 0) {
            prefetch(st0, 0);
            prefetch(st1, 1);
        }
        write_rt(Rts, R, qh, cq, lane);

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

        // the end carry (pc is unchanged until the next piece)
        const int end = __builtin_amdgcn_readfirstlane(pc.end);
        if (end == 1) {  // the piece holds token 0: d_state_in
            float *dst = uniform_ptr(pc.dst);
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) dst[sidx(db, v)] = R[db][v];
        } else if (end == 2) {  // a warm piece ending inside its pair: record a NaN or Inf
            bool bad = false;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) bad |= nonfinite(R[db][v]);
            if (bad) {  // rare: entry (r, c) of R poisons dk column r and dv column c
                int *rec = pc.rec;
                const int cut = pc.cut;
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (nonfinite(R[db][v])) {
                            const int e = sidx(db, v);
                            atomicOr(reinterpret_cast<unsigned *>(rec + kRecEntBad) + (e >> 5), 1u << (e & 31));
                            atomicMin(rec + kRecRowCut + e / D, cut);
                        }
                atomicMin(rec + kRecColCut + 32 * cq + r32, cut);  // every entry of this thread is in that column
            }
        }
    }
}

// Finishing pass of the reverse pass's warm-up route: one workgroup per (unit,
// head) pair; pairs on the pre-pass route exit at once. A piece that starts
// inside its pair builds its carry from a window of the tokens after it, so it
// cannot see a NaN or Inf from beyond that window. In exact arithmetic an entry
// (r, c) of the carry that is non-finite at some token stays non-finite at
// every earlier token, and with it dk column r and dv column c of those tokens
// and entry (r, c) of d_state_in. The pieces that ended inside the pair
// recorded where their end carries held one (mirrored token t, per row and per
// column, and the entries); this pass puts NaN in dk column r of every real
// token below L - (earliest t of row r), likewise in dv by column, and in each
// flagged entry of d_state_in (the piece holding token 0 has written it).
template <typename OutT>
__global__ __launch_bounds__(NT) void bwd_finish_kernel(BackwardArgs a, Segmented sp, float *ws) {
    __shared__ int cuts[2 * D];  // [0, D): dv column c; [D, 2D): dk column r
    __shared__ int mincut;
    const int tid = threadIdx.x;
    const int uh = blockIdx.x, h = uh % a.heads, n = uh / a.heads;
    if (takes_prepass(sp, a.slopes[h] * LOG2E)) return;
    const int *rec = warm_records(sp, ws, uh);
    if (tid == 0) mincut = kNoCut;
    __syncthreads();
    if (tid < 2 * D) {
        cuts[tid] = rec[tid < D ? kRecColCut + tid : kRecRowCut + (tid - D)];
        atomicMin(&mincut, cuts[tid]);
    }
    __syncthreads();
    const int first = mincut;
    if (first == kNoCut) return;
    const long long L = a.seqlen;
    // real rows t < L - cut; 32 threads per row (4 columns each), NT / 32 rows at a time
    const int col = 4 * (tid & 31);
    long long vtop[4], ktop[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        vtop[x] = L - cuts[col + x];
        ktop[x] = L - cuts[D + col + x];
    }
    OutT *dk = static_cast<OutT *>(a.dk), *dv = static_cast<OutT *>(a.dv);
    for (long long t = tid >> 5; t < L - first; t += NT / 32) {
        const long long off = (((long long)n * L + t) * a.heads + h) * (long long)D + col;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (t < ktop[x]) poison(dk + off + x);
            if (t < vtop[x]) poison(dv + off + x);
        }
    }
    if (a.d_state_in) {
        const unsigned *bad = reinterpret_cast<const unsigned *>(rec + kRecEntBad);
        float4 *dst = reinterpret_cast<float4 *>(a.d_state_in + (size_t)uh * D * D);
#pragma unroll
        for (int j = 0; j < kStateF4; ++j) {
            const int f = tid + NT * j;
            const unsigned b = (bad[f >> 3] >> (4 * (f & 7))) & 0xfu;  // entries 4f .. 4f+3
            if (b) {
                float4 x = dst[f];
                if (b & 1) x.x = __builtin_nanf("");
                if (b & 2) x.y = __builtin_nanf("");
                if (b & 4) x.z = __builtin_nanf("");
                if (b & 8) x.w = __builtin_nanf("");
                dst[f] = x;
            }
        }
    }
}

template <typename OutT>
hipError_t launch(const BackwardArgs &a, const PrefillPlan &p, void *workspace, hipStream_t stream) {
    clear_pending_error();
    const long long uh = (long long)a.units * a.heads;
    float *ws = static_cast<float *>(workspace);
    const bool seg = p.segments > 1 && p.value_slices == 1;
    const Segmented sp = seg ? Segmented{p.segments, p.pieces, p.seg_len, p.piece_len} : Segmented{1, 0, a.seqlen, 0};
    if (seg) {
        // the kernels' per-plan tables hold every pair and workgroup of a segmented plan
        if (uh >= kMaxPairs) return hipErrorInvalidValue;
        // working pre-pass workgroups: at most kPrepassActive + uh (see rev_piece_kernel)
        const long long pre = uh * p.pieces < kPrepassActive + uh ? uh * p.pieces : kPrepassActive + uh;
        hipLaunchKernelGGL(rev_piece_kernel, dim3((unsigned)pre), dim3(NT), 0, stream, a, sp, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_kv_kernel<OutT>), dim3((unsigned)(uh * sp.segments)), dim3(NT), 0, stream,
                       a, sp, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !seg) return e;
    hipLaunchKernelGGL((bwd_finish_kernel<OutT>), dim3((unsigned)uh), dim3(NT), 0, stream, a, sp, ws);
    return hipGetLastError();
}

}  // namespace

hipError_t load_backward_code() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&bwd_kv_kernel<float>));
}

hipError_t launch_backward_kv(const BackwardArgs &a, const PrefillPlan &plan, void *workspace,
                              lt_dtype out_dtype, hipStream_t stream) {
    return out_dtype == LT_F32 ? launch<float>(a, plan, workspace, stream)
                               : launch<__bf16>(a, plan, workspace, stream);
}

}  // namespace lt
